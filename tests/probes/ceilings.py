"""Practical HBM ceilings of one MI355X for the roofline discussion: a
16-byte-per-lane streaming read, a read + write copy and the kernels'
row-gather pattern (tests/probes/gla_probes.hip), each over buffers larger
than the 256 MB last-level cache, timed with HIP events on the launch stream
over repeated launches; and the latency of the segment exchange's flag
handoff between two workgroups on one XCD or on two, for each store / load
cache policy (sc1 or default).  Prints one JSON line.

Usage (repo root): ``python tests/probes/ceilings.py [--reps N]``.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)
from build import LIB  # noqa: E402


def load():
    if not os.path.exists(LIB):
        raise RuntimeError(f"{LIB} is missing: build it with python tests/probes/build.py")
    h = ctypes.CDLL(LIB)
    vp, sz, ci = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    h.gla_probe_tr16.argtypes = [vp, vp]
    h.gla_probe_read.argtypes = [vp, sz, vp, ci, vp]
    h.gla_probe_copy.argtypes = [vp, vp, sz, ci, vp]
    h.gla_probe_gather.argtypes = [vp, ci, vp, ci, vp]
    h.gla_probe_handoff.argtypes = [vp, ci, ci, ci, ci, vp, vp]
    for f in (h.gla_probe_tr16, h.gla_probe_read, h.gla_probe_copy, h.gla_probe_gather, h.gla_probe_handoff):
        f.restype = ci
    return h


def handoff(h, consumer, store_sc1, load_sc1, iters=500):
    """One flag handoff probe: producer workgroup 0, consumer `consumer`.
    Returns a dict with the one-way latency in microseconds (the producer's
    loop time over 2 iters handoffs) or the number of handoffs seen before a
    bounded wait ran out, and the XCC_IDs of the two workgroups."""
    import torch
    words = torch.zeros(64, dtype=torch.int32, device="cuda")
    out = torch.zeros(6, dtype=torch.int64, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    assert h.gla_probe_handoff(words.data_ptr(), iters, consumer, store_sc1, load_sc1, out.data_ptr(), st) == 0
    torch.cuda.synchronize()
    ticks, done, xp, xc, tp, tc = out.cpu().tolist()
    rec = {"consumer": consumer, "store": "sc1" if store_sc1 else "default",
           "load": "sc1" if load_sc1 else "default", "xcc": [xp, xc], "handoffs": done,
           "ran_out": bool(tp or tc)}
    if done == iters and not (tp or tc):
        rec["one_way_us"] = round(ticks * 0.01 / (2 * iters), 3)
    return rec


def main():
    import torch
    ap = argparse.ArgumentParser()
    ap.add_argument("--reps", type=int, default=20)
    ap.add_argument("--mib", type=int, default=1024, help="read / copy buffer size")
    ap.add_argument("--side", type=int, default=2048, help="gather grid side (rows of 128 bytes)")
    args = ap.parse_args()
    h = load()
    dev = torch.device("cuda:0")
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    blocks = 8 * cus
    st = torch.cuda.current_stream(dev)
    n = args.mib << 20
    src = torch.ones(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    rows = args.side * args.side
    gsrc = torch.ones(rows * 128, dtype=torch.uint8, device=dev)
    sink = torch.empty(blocks * 512, dtype=torch.int32, device=dev)

    def timed(launch, nbytes):
        for _ in range(3):
            assert launch() == 0
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record(st)
        for _ in range(args.reps):
            assert launch() == 0
        t1.record(st)
        torch.cuda.synchronize()
        us = t0.elapsed_time(t1) * 1000.0 / args.reps
        return {"us_per_launch": round(us, 2), "tb_per_s": round(nbytes / us * 1e-6, 3)}

    s = st.cuda_stream
    out = {
        "device": torch.cuda.get_device_name(dev), "cus": cus, "blocks": blocks, "threads": 512,
        "read_16B_per_lane": timed(lambda: h.gla_probe_read(src.data_ptr(), n, sink.data_ptr(), blocks, s), n),
        "copy_16B_per_lane": timed(lambda: h.gla_probe_copy(src.data_ptr(), dst.data_ptr(), n, blocks, s), 2 * n),
        "row_gather_16x64B": timed(lambda: h.gla_probe_gather(gsrc.data_ptr(), args.side, sink.data_ptr(),
                                                               blocks, s), rows * 128),
        "bytes": {"read": n, "copy": 2 * n, "gather": rows * 128},
        "flag_handoff": [handoff(h, c, ss, ls) for c in (8, 1) for ss, ls in ((1, 1), (0, 1), (1, 0), (0, 0))],
        "peak_tb_per_s": 8.0,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
