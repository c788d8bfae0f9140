"""Device probes of assumptions the kernels are built on (tests/probes/):
the lane layout of the gfx950 LDS transpose read through the library's
helpers, and the streaming kernels behind the quoted HBM ceilings."""
from __future__ import annotations

import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.join(os.path.dirname(os.path.abspath(__file__)), "probes"))

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def probes():
    import torch
    assert torch.cuda.is_available(), "needs a GPU"
    from ceilings import load
    return load()


def test_lds_transpose_read_lane_layout(probes):
    """ld_tr over tr_addr: lane (g, l16) receives rows 4g .. 4g+3 of column
    16 (g mod 4) + l16; tr_frag_s: rows 8g .. 8g+7 of column 32 + l16, from a
    tile whose element (r, c) holds r * 64 + c (row stride 72 elements)."""
    import torch
    out = torch.zeros(64 * 12, dtype=torch.int16, device="cuda")
    assert probes.gla_probe_tr16(out.data_ptr(), torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.float16).astype(np.int64).reshape(64, 12)
    want = np.zeros((64, 12), dtype=np.int64)
    for lane in range(64):
        g, l16 = lane >> 4, lane & 15
        for e in range(4):
            want[lane, e] = (4 * g + e) * 64 + 16 * (g & 3) + l16
        for e in range(8):
            want[lane, 4 + e] = (8 * g + e) * 64 + 32 + l16
    bad = np.argwhere(got != want)
    for lane in sorted(set(bad[:, 0].tolist()))[:4]:
        print(f"[tr16] lane {lane}: got {got[lane].tolist()} want {want[lane].tolist()}", flush=True)
    assert bad.size == 0, f"lane layout differs at (lane, element) {bad[:4].tolist()}"


def test_streaming_probes_compute_what_they_read(probes):
    """The copy probe copies; the read and gather probes' per-thread sums
    match a host evaluation of the same access pattern (small sizes)."""
    import torch
    rng = np.random.default_rng(5)
    st = torch.cuda.current_stream().cuda_stream
    blocks = 3
    words = rng.integers(0, 2**32, size=4 * 4096, dtype=np.uint64).astype(np.uint32)
    src = torch.from_numpy(words.view(np.int32)).cuda()
    dst = torch.zeros_like(src)
    sink = torch.zeros(blocks * 512, dtype=torch.int32, device="cuda")
    assert probes.gla_probe_copy(src.data_ptr(), dst.data_ptr(), words.nbytes, blocks, st) == 0
    assert probes.gla_probe_read(src.data_ptr(), words.nbytes, sink.data_ptr(), blocks, st) == 0
    torch.cuda.synchronize()
    assert torch.equal(src, dst)
    v = words.reshape(-1, 4).astype(np.uint64).sum(axis=1) & 0xFFFFFFFF
    want = np.zeros(blocks * 512, dtype=np.uint64)
    for i, x in enumerate(v):
        want[i % (blocks * 512)] ^= x
    assert np.array_equal(sink.cpu().numpy().view(np.uint32).astype(np.uint64), want)

    side = 12
    rows = rng.integers(0, 2**32, size=(side * side, 8, 4), dtype=np.uint64).astype(np.uint32)
    gsrc = torch.from_numpy(rows.reshape(-1).view(np.int32)).cuda()
    assert probes.gla_probe_gather(gsrc.data_ptr(), side, sink.data_ptr(), blocks, st) == 0
    torch.cuda.synchronize()
    want = np.zeros(blocks * 512, dtype=np.uint64)
    npass = (side * side + 63) // 64
    for b in range(blocks):
        for tid in range(512):
            lane, wave = tid & 63, tid >> 6
            g, l16, h = lane >> 4, lane & 15, wave & 1
            acc = 0
            for blk in range(b, npass, blocks):
                t = (blk * 4 + (wave >> 1)) * 16 + l16
                if t < side * side:
                    row = (t % side) * side + t // side
                    acc ^= int(rows[row, 4 * h + g].astype(np.uint64).sum()) & 0xFFFFFFFF
            want[b * 512 + tid] = acc
    assert np.array_equal(sink.cpu().numpy().view(np.uint32).astype(np.uint64), want)


def test_flag_handoff_policies_the_exchange_uses(probes):
    """The segment exchange's cache policies see each other's flags: sc1
    stores and sc1 loads between workgroups on one XCD and on two, and
    default-policy stores read by sc1 loads on one XCD (the flags of
    XCD-local plans); every handoff arrives within the bounded wait.  (On an
    8-XCD device workgroups 0 and 8 share an XCD and 0 and 1 do not, under
    turn-by-turn dispatch.)"""
    import torch
    from ceilings import handoff
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for consumer, ss, ls in ((8, 1, 1), (1, 1, 1), (8, 0, 1)):
        rec = handoff(probes, consumer, ss, ls, iters=200)
        print(f"[handoff] {rec}", flush=True)
        assert rec["handoffs"] == 200 and not rec["ran_out"], rec
        if cus == 256:
            same = rec["xcc"][0] == rec["xcc"][1]
            assert same == (consumer == 8), rec
