"""Shared helpers for the GPU parity tests: run the HIP path through the C ABI
binding and compare it with the CPU oracle on the same seeded inputs."""
from __future__ import annotations

import numpy as np

import oracle
from recurrent_vision_backbone_key_amd import gla

# Tolerances: max |gpu - oracle| <= TOL * max |oracle| (binary16 storage: 2e-3,
# binary32 storage: 1e-5).
TOL = {"f16": 2e-3, "f32": 1e-5}


def to_dev(x, torch):
    return None if x is None else torch.from_numpy(np.ascontiguousarray(x)).cuda()


def run_gpu(x, direction, H, W, chunk, torch, eps=1e-6, segment_chunks=0, out=None, tau=16.0,
            algorithm=gla.ALGO_AUTO):
    d = {n: to_dev(x[n], torch) for n in ("q", "k", "v", "z", "r", "w")}
    B, L, NH, dk = x["q"].shape
    opts = gla.make_opts(B, NH, dk, x["v"].shape[3],
                         gla.F16 if x["q"].dtype == np.float16 else gla.F32,
                         segment_chunks=segment_chunks, algorithm=algorithm)
    need = gla.workspace_size(direction, H, W, chunk, opts)
    # a garbage-filled workspace cleared by the library's own init call
    ws = torch.full((max(need, 16),), 0xA5, dtype=torch.uint8, device="cuda")
    gla.workspace_init(ws)
    y = gla.fwd(d["q"], d["k"], d["v"], d["z"], direction, H, W, chunk=chunk, r=d["r"],
                norm_weight=d["w"], eps=eps, out=out, tau=tau, segment_chunks=segment_chunks,
                workspace=ws, algorithm=algorithm)
    torch.cuda.synchronize()
    # the workspace's error word (sticky until the next init) through the
    # library's own status call, whichever algorithm the plan picked
    if need:
        err = gla.workspace_status(ws)
        assert err == 0, f"kernel error bits set in the workspace: {err:#x}"
    return y.cpu().numpy()


def run_oracle(x, direction, H, W, eps=1e-6, units=None, tau=16.0):
    return oracle.fwd(x["q"], x["k"], x["v"], x["z"], direction, H, W, r=x["r"], w=x["w"],
                      eps=eps, units=units, tau=tau)


def rel_err(got, ref, mask=None):
    got = got.astype(np.float64)
    if mask is not None:
        got, ref = got[mask], ref[mask]
    return float(np.max(np.abs(got - ref)) / max(float(np.max(np.abs(ref))), 1e-300))


def unit_mask(shape, units):
    """Boolean mask of the [B, L, NH, d] rows that belong to (b*NH + h) units."""
    B, L, NH, d = shape
    m = np.zeros((B, L, NH, d), dtype=bool)
    for u in range(*units):
        m[u // NH, :, u % NH, :] = True
    return m


def report(name, got, ref):
    err = rel_err(got, ref)
    print(f"[parity] {name}: max|err|/max|ref| = {err:.3e}", flush=True)
    return err
