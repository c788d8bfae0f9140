"""Seeded synthetic inputs and the workload table.

This module holds no arithmetic of the method: it only draws random arrays
with the shapes and distributions of the workloads and casts them to the
storage dtype.  Both the oracle side and the HIP side of every parity test
consume exactly the arrays produced here.

Workloads (shapes follow the GTR pages: a 640 px frame at stride 16 is a
40x40 patch grid of 1.6K tokens, 1280 px is 80x80, and the long-sequence
kernel point is 16.4K tokens; head dim 64 and 6 heads as in the GTR-L/X
backbone table).  No dataset or trained weight is involved.
"""
from __future__ import annotations

import numpy as np

L2R, R2L, T2B, B2T = 0, 1, 2, 3

# name -> spec.  z = (mean, std) of the gate logits.  dirs: the direction of
# each call in order.  gated: whether the fused output gate (r, w) is used.
WORKLOADS = {
    "tiny": dict(index=1, B=1, NH=1, H=8, W=8, dk=16, dv=16, dtype="f32", z=(0.0, 1.0),
                 chunk=16, dirs=(L2R,), gated=False),
    "frame640": dict(index=2, B=1, NH=6, H=40, W=40, dk=64, dv=64, dtype="f16", z=(0.0, 1.0),
                     chunk=64, dirs=(L2R, R2L, T2B, B2T), gated=False),
    "batch640_gated": dict(index=3, B=8, NH=6, H=40, W=40, dk=64, dv=64, dtype="f16",
                           z=(0.0, 1.0), chunk=64, dirs=(L2R, R2L, T2B, B2T), gated=True),
    "frame1280_gated": dict(index=4, B=1, NH=12, H=80, W=80, dk=64, dv=64, dtype="f16",
                            z=(0.0, 1.5), chunk=64, dirs=(L2R, R2L, T2B, B2T), gated=True),
    "stack16k_gated": dict(index=5, B=2, NH=12, H=128, W=128, dk=128, dv=128, dtype="f16",
                           z=(2.0, 1.0), chunk=64, dirs=(L2R, R2L, T2B, B2T) * 3, gated=True),
}

# The retention gate's logits computed in the library from the block input
# (x W1 W2 + b, rank 16; d_model = NH * dk = 384 as in a 6-head, 64-dim
# backbone stage) instead of read as z: the 640 px frame and batch shapes.
GATE_PROJ = {
    "frame640_gateproj": dict(index=6, B=1, NH=6, H=40, W=40, dk=64, dv=64, dtype="f16",
                              z=(0.0, 1.0), chunk=64, dirs=(L2R, R2L, T2B, B2T), gated=False,
                              gate_proj=dict(d_model=384, rank=16)),
    "batch640_gateproj": dict(index=7, B=8, NH=6, H=40, W=40, dk=64, dv=64, dtype="f16",
                              z=(0.0, 1.0), chunk=64, dirs=(L2R, R2L, T2B, B2T), gated=True,
                              gate_proj=dict(d_model=384, rank=16)),
}
WORKLOADS.update(GATE_PROJ)

# The Spatial SwiGLU core on the same grids: hidden width 4 x 384 = 1536
# (expansion 4 of a 384-wide block) and 6 x 384 = 2304 (expansion 6).
SSWIGLU = {
    "sswiglu640": dict(index=20, kind="sswiglu", B=8, H=40, W=40, C=1536, dtype="f16"),
    "sswiglu640_x6": dict(index=21, kind="sswiglu", B=8, H=40, W=40, C=2304, dtype="f16"),
    "sswiglu1280": dict(index=22, kind="sswiglu", B=1, H=80, W=80, C=1536, dtype="f16"),
}
WORKLOADS.update(SSWIGLU)

# Length and batch sweep at the pages' own kernel points (16x16 = 256 tokens,
# the 1.6K frame, 128x128 = 16.4K tokens) at d = 64 with 6 heads, plus a tail
# grid (42x42 = 1764 tokens, not a multiple of the 64-token chunk); the four
# directions per step, ungated as in the pages' kernel comparison.
SWEEP = {}
for _i, (_h, _w, _b) in enumerate(((16, 16, 1), (16, 16, 8), (40, 40, 1), (40, 40, 8),
                                   (42, 42, 1), (42, 42, 8), (128, 128, 1), (128, 128, 8))):
    SWEEP[f"sweep{_h}x{_w}_b{_b}"] = dict(index=10 + _i, B=_b, NH=6, H=_h, W=_w, dk=64, dv=64,
                                          dtype="f16", z=(0.0, 1.0), chunk=64,
                                          dirs=(L2R, R2L, T2B, B2T), gated=False)
WORKLOADS.update(SWEEP)

# Backward of the ungated forward at the batch shape (8 images, 40 x 40
# patches, 6 heads of 64): the four directions per step.
BWD = {
    "bwd640": dict(index=23, kind="bwd", B=8, NH=6, H=40, W=40, dk=64, dv=64, dtype="f16",
                   z=(0.0, 1.0), chunk=64, dirs=(L2R, R2L, T2B, B2T), gated=False),
    # the same through the output gate (the batch640_gated forward's backward)
    "bwd640_gated": dict(index=24, kind="bwd", B=8, NH=6, H=40, W=40, dk=64, dv=64,
                         dtype="f16", z=(0.0, 1.0), chunk=64, dirs=(L2R, R2L, T2B, B2T),
                         gated=True),
    # the 12-block stack's shape through the output gate (d = 128: four d = 64
    # quarters per call)
    "bwd16k_gated": dict(index=25, kind="bwd", B=2, NH=12, H=128, W=128, dk=128, dv=128,
                         dtype="f16", z=(2.0, 1.0), chunk=64, dirs=(L2R, R2L, T2B, B2T),
                         gated=True),
    # the gate projection's backward at the gated batch's shapes (12800 tokens,
    # d_model 384, 6 heads of 64, rank 16)
    "gateproj_bwd640": dict(index=26, kind="proj_bwd", B=8, NH=6, H=40, W=40, dk=64, dv=64,
                            dtype="f16", d_model=384, rank=16),
}
WORKLOADS.update(BWD)

EPS = 1e-6
TAU = 16.0


def np_dtype(name: str):
    return {"f16": np.float16, "f32": np.float32}[name]


def tokens_per_call(spec) -> int:
    return spec["B"] * spec["NH"] * spec["H"] * spec["W"]


def make_inputs(B, NH, H, W, dk, dv, dtype="f16", z=(0.0, 1.0), gated=False, seed=0,
                q_std=1.0):
    """Draw q, k, v, z, r, w in that fixed order from PCG64(seed).

    q, k, v, r ~ N(0, 1) drawn in float64 and rounded to ``dtype`` (numpy's
    cast rounds to nearest even); z ~ N(z_mean, z_std) kept in float32;
    w ~ U(0.5, 1.5) float32.  r and w are None unless ``gated``.
    """
    rng = np.random.default_rng(seed)
    L = H * W
    dt = np_dtype(dtype)
    q = (rng.standard_normal((B, L, NH, dk)) * q_std).astype(dt)
    k = rng.standard_normal((B, L, NH, dk)).astype(dt)
    v = rng.standard_normal((B, L, NH, dv)).astype(dt)
    zz = (z[0] + z[1] * rng.standard_normal((B, L, NH, dk))).astype(np.float32)
    r = w = None
    if gated:
        r = rng.standard_normal((B, L, NH, dv)).astype(dt)
        w = rng.uniform(0.5, 1.5, size=(dv,)).astype(np.float32)
    return dict(q=q, k=k, v=v, z=zz, r=r, w=w)


def make_bwd_inputs(B, NH, H, W, d, dtype="f16", z=(0.0, 1.0), seed=0, dout_seed=None,
                    gated=False):
    """Operands of the backward: q, k, v, z (and r, w if ``gated``) as
    :func:`make_inputs` with PCG64(seed), then dout ~ N(0, 1) [B, L, NH, d]
    rounded to ``dtype`` from PCG64(dout_seed), by default seed + 1 (dL/do,
    or dL/du when gated)."""
    x = make_inputs(B, NH, H, W, d, d, dtype, z=z, gated=gated, seed=seed)
    rng = np.random.default_rng(seed + 1 if dout_seed is None else dout_seed)
    x["dout"] = rng.standard_normal((B, H * W, NH, d)).astype(np_dtype(dtype))
    return x


def make_bwd_inputs_device(B, NH, H, W, d, dtype="f16", z=(0.0, 1.0), seed=0, device="cuda",
                           gated=False):
    """Same distributions as :func:`make_bwd_inputs`, drawn on the device with
    seeded torch generators (timing inputs)."""
    import torch

    x = make_inputs_device(B, NH, H, W, d, d, dtype, z=z, gated=gated, seed=seed, device=device)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed + 1)
    dt = {"f16": torch.float16, "f32": torch.float32}[dtype]
    x["dout"] = torch.randn((B, H * W, NH, d), generator=gen, device=device,
                            dtype=torch.float32).to(dt)
    return x


def make_gate_proj_inputs(B, L, NH, dk, d_model, rank=16, dtype="f16", seed=0):
    """Draw the retention gate's low-rank projection inputs from PCG64(seed),
    in the order x, w1, w2, bias.

    x ~ N(0, 1) [B, L, d_model] and w1 ~ N(0, 1/d_model) [rank, d_model]
    rounded to ``dtype``; w2 ~ N(0, 1/rank) [NH*dk, rank] and
    bias ~ U(-1/sqrt(rank), 1/sqrt(rank)) [NH*dk] in float32.  With these
    scales x W1 W2 is about N(0, 1), the gate-logit distribution of the
    other workloads.
    """
    rng = np.random.default_rng(seed)
    dt = np_dtype(dtype)
    x = rng.standard_normal((B, L, d_model)).astype(dt)
    w1 = (rng.standard_normal((rank, d_model)) / np.sqrt(d_model)).astype(dt)
    w2 = (rng.standard_normal((NH * dk, rank)) / np.sqrt(rank)).astype(np.float32)
    lim = 1.0 / np.sqrt(rank)
    bias = rng.uniform(-lim, lim, size=(NH * dk,)).astype(np.float32)
    return dict(x=x, w1=w1, w2=w2, bias=bias)


def workload_inputs(name: str, call: int = 0, **overrides):
    """Inputs of call ``call`` of a named workload; seed = 1000*index + call."""
    spec = dict(WORKLOADS[name])
    spec.update(overrides)
    if spec.get("kind") == "bwd":
        # output gradient from its own stream (seed + 500)
        return make_bwd_inputs(spec["B"], spec["NH"], spec["H"], spec["W"], spec["dk"],
                               spec["dtype"], spec["z"], seed=1000 * spec["index"] + call,
                               dout_seed=1000 * spec["index"] + 500 + call,
                               gated=spec["gated"])
    x = make_inputs(spec["B"], spec["NH"], spec["H"], spec["W"], spec["dk"], spec["dv"],
                    spec["dtype"], spec["z"], spec["gated"], seed=1000 * spec["index"] + call)
    gp = spec.get("gate_proj")
    if gp:
        # projection operands from their own stream (seed + 500); z is unused
        x.update(make_gate_proj_inputs(spec["B"], spec["H"] * spec["W"], spec["NH"], spec["dk"],
                                       gp["d_model"], gp["rank"], spec["dtype"],
                                       seed=1000 * spec["index"] + 500 + call))
    return x


def make_inputs_device(B, NH, H, W, dk, dv, dtype="f16", z=(0.0, 1.0), gated=False, seed=0,
                       device="cuda"):
    """Same distributions as :func:`make_inputs`, drawn on the device with a
    seeded torch generator (for large timing inputs; parity tests use the
    numpy generator)."""
    import torch

    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    L = H * W
    dt = {"f16": torch.float16, "f32": torch.float32}[dtype]

    def normal(shape, mean=0.0, std=1.0):
        return (torch.randn(shape, generator=gen, device=device, dtype=torch.float32) * std
                + mean)

    q = normal((B, L, NH, dk)).to(dt)
    k = normal((B, L, NH, dk)).to(dt)
    v = normal((B, L, NH, dv)).to(dt)
    zz = normal((B, L, NH, dk), z[0], z[1])
    r = w = None
    if gated:
        r = normal((B, L, NH, dv)).to(dt)
        w = torch.rand((dv,), generator=gen, device=device, dtype=torch.float32) + 0.5
    return dict(q=q, k=k, v=v, z=zz, r=r, w=w)


def make_gate_proj_inputs_device(B, L, NH, dk, d_model, rank=16, dtype="f16", seed=0,
                                 device="cuda"):
    """Same distributions as :func:`make_gate_proj_inputs`, drawn on the device
    with a seeded torch generator (timing inputs)."""
    import torch

    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    dt = {"f16": torch.float16, "f32": torch.float32}[dtype]

    def normal(shape, std=1.0):
        return torch.randn(shape, generator=gen, device=device, dtype=torch.float32) * std

    x = normal((B, L, d_model)).to(dt)
    w1 = normal((rank, d_model), d_model ** -0.5).to(dt)
    w2 = normal((NH * dk, rank), rank ** -0.5)
    lim = rank ** -0.5
    bias = (torch.rand((NH * dk,), generator=gen, device=device, dtype=torch.float32) * 2 - 1) * lim
    return dict(x=x, w1=w1, w2=w2, bias=bias)


def make_sswiglu_inputs(B, H, W, C, dtype="f16", bias=True, seed=0):
    """Draw the Spatial SwiGLU core's operands from PCG64(seed), in the order
    gate, value, weight, bias.

    gate, value ~ N(0, 1) [B, H*W, C] rounded to ``dtype`` (the two branch
    projections of the block input); weight, bias ~ U(-1/3, 1/3) float32
    ([C, 3, 3] and [C]; the default initialisation range of a depthwise 3x3
    convolution, fan-in 9).
    """
    rng = np.random.default_rng(seed)
    dt = np_dtype(dtype)
    a = rng.standard_normal((B, H * W, C)).astype(dt)
    v = rng.standard_normal((B, H * W, C)).astype(dt)
    w = rng.uniform(-1.0 / 3.0, 1.0 / 3.0, size=(C, 3, 3)).astype(np.float32)
    b = rng.uniform(-1.0 / 3.0, 1.0 / 3.0, size=(C,)).astype(np.float32) if bias else None
    return dict(a=a, v=v, w=w, b=b)
