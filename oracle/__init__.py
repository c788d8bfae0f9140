"""CPU oracle for key-only gated linear attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the HIP
implementation in ``recurrent_vision_backbone_key_amd`` and never imports it.

Seven references, each written from its definition ("GTR: Gated Token
Recurrence for Efficient Dense Prediction", paper Section 2.1):

* :func:`fwd` -- the token-by-token fp64 recurrence in plain C
  (``gla_oracle.c``), OpenMP over the (batch, head) units;
* :func:`gate_logits` -- the low-rank gate logits z = (x W1) W2 + b of
  the retention gate (same section), plain C loops in fp64;
* :func:`gate_proj_bwd` -- the gradients of x, W1, W2, b of those logits
  (the chain rule of a product of matrices), numpy fp64 matrix products;
* :func:`spatial_swiglu` (with :func:`dwconv3x3`, :func:`silu`) -- the
  Spatial SwiGLU core SiLU(a) (.) (3x3 depthwise convolution of v + b)
  (same section), numpy fp64 shifted sums;
* :func:`bwd` -- the gradients of q, k, v, z of the ungated forward (the
  recurrence differentiated, run backwards along the scan), fp64 C;
* :func:`bwd_gated` -- the same through the output gate (dr, dw and the
  gradient entering the ungated backward, from the epilogue's derivative),
  fp64 C;
* :func:`closed_form_fwd` -- the O(L^2) unrolled sum
  ``o_t = scale * sum_{s<=t} (q_t (.) prod_{j=s+1..t} gamma_j (.) k_s) v_s``
  in numpy fp64 with explicit per-pair gate sums, for tiny inputs.  Its scan
  orders are built from array flips and grid transposes, not from the C
  code's index formula.

Every function's pins (closed forms, special cases, invariants) are the
``tests/test_oracle*.py`` tests.  No function here is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_BUILD_DIR = os.path.join(_HERE, "_build")
LIB_PATH = os.path.join(_BUILD_DIR, "libgla_oracle.so")
SOURCE = os.path.join(_HERE, "gla_oracle.c")

L2R, R2L, T2B, B2T = 0, 1, 2, 3
DIRS = (L2R, R2L, T2B, B2T)
DIR_NAMES = {L2R: "L2R", R2L: "R2L", T2B: "T2B", B2T: "B2T"}

_lib = None


def build(force: bool = True) -> str:
    """Compile gla_oracle.c with gcc (fp64, no fast-math, no FMA contraction)."""
    if not force and os.path.exists(LIB_PATH):
        return LIB_PATH
    os.makedirs(_BUILD_DIR, exist_ok=True)
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp",
           "-ffp-contract=off", "-fno-fast-math", "-Wall", "-o", tmp, SOURCE, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        build()
    lib = ctypes.CDLL(LIB_PATH)
    lib.gla_oracle_fwd.restype = ctypes.c_int
    lib.gla_oracle_fwd.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_int, ctypes.c_int,
        ctypes.c_double, ctypes.c_double, ctypes.c_double,
        ctypes.c_long, ctypes.c_long, ctypes.c_void_p]
    lib.gla_oracle_fwd_zd.restype = ctypes.c_int
    lib.gla_oracle_fwd_zd.argtypes = lib.gla_oracle_fwd.argtypes
    lib.gla_oracle_gate_logits.restype = ctypes.c_int
    lib.gla_oracle_gate_logits.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
        ctypes.c_long, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.gla_oracle_bwd.restype = ctypes.c_int
    lib.gla_oracle_bwd.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
        ctypes.c_void_p, ctypes.c_int,
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_int, ctypes.c_double, ctypes.c_double, ctypes.c_long, ctypes.c_long,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.gla_oracle_half_to_double.restype = ctypes.c_double
    lib.gla_oracle_half_to_double.argtypes = [ctypes.c_uint16]
    lib.gla_oracle_scan_token.restype = ctypes.c_long
    lib.gla_oracle_scan_token.argtypes = [ctypes.c_int, ctypes.c_long, ctypes.c_long,
                                          ctypes.c_long]
    _lib = lib
    return lib


def half_to_double(bits: int) -> float:
    return _load().gla_oracle_half_to_double(bits)


def scan_token(direction: int, i: int, H: int, W: int) -> int:
    return _load().gla_oracle_scan_token(direction, i, H, W)


def _ptr(a):
    return None if a is None else a.ctypes.data


def fwd(q, k, v, z, direction, H, W, r=None, w=None, tau=16.0, scale=None,
        eps=1e-6, units=None, threads=None):
    """fp64 recurrence.  q, k: [B, L, NH, dk]; v, r: [B, L, NH, dv] (float16 or
    float32 arrays, read exactly as stored); z: [B, L, NH, dk] float32, or
    float64 (used as is, e.g. from :func:`gate_logits`); w: [dv] float32 or
    None.  Returns float64 [B, L, NH, dv].

    ``units=(u0, u1)`` restricts the work to (batch*NH + head) units in
    [u0, u1); other rows of the result are NaN.
    """
    lib = _load()
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    z64 = np.asarray(z).dtype == np.float64
    z = np.ascontiguousarray(z, dtype=np.float64 if z64 else np.float32)
    dtype = _storage_code(q)
    for name, a in (("k", k), ("v", v)) + ((("r", r),) if r is not None else ()):
        if a.dtype != q.dtype:
            raise TypeError(f"{name} must have q's dtype")
    B, L, NH, dk = q.shape
    dv = v.shape[3]
    if L != H * W or k.shape != q.shape or z.shape != q.shape or v.shape[:3] != q.shape[:3]:
        raise ValueError("shape mismatch")
    if r is not None:
        r = np.ascontiguousarray(r)
        if r.shape != v.shape:
            raise ValueError("r shape mismatch")
    if w is not None:
        w = np.ascontiguousarray(w, dtype=np.float32)
        if w.shape != (dv,):
            raise ValueError("w must have shape [dv]")
    if scale is None:
        scale = 1.0 / math.sqrt(dk)
    u0, u1 = (0, B * NH) if units is None else units
    out = np.full((B, L, NH, dv), np.nan, dtype=np.float64)
    old = os.environ.get("OMP_NUM_THREADS")
    if threads is not None:
        os.environ["OMP_NUM_THREADS"] = str(threads)
    try:
        entry = lib.gla_oracle_fwd_zd if z64 else lib.gla_oracle_fwd
        rc = entry(_ptr(q), _ptr(k), _ptr(v), _ptr(z), _ptr(r), _ptr(w), dtype,
                   B, NH, H, W, dk, dv, direction, float(tau), float(scale),
                   float(eps), u0, u1, _ptr(out))
    finally:
        if threads is not None:
            if old is None:
                os.environ.pop("OMP_NUM_THREADS", None)
            else:
                os.environ["OMP_NUM_THREADS"] = old
    if rc != 0:
        raise RuntimeError(f"gla_oracle_fwd failed with status {rc}")
    return out


def _storage_code(a):
    if a.dtype == np.float16:
        return 0
    if a.dtype == np.float32:
        return 1
    if a.dtype == np.float64:
        return 2
    raise TypeError("inputs must be float16, float32 or float64")


def bwd(q, k, v, z, dout, direction, H, W, tau=16.0, scale=None, units=None, threads=None):
    """Gradients (dq, dk, dv, dz) of the ungated forward for output gradient
    dout ([B, L, NH, dv], q's dtype), fp64 reverse recurrence (paper Section
    2.1 recurrence, differentiated).  q, k, v, dout: float16/32/64 read as
    stored; z: float32 or float64.  Returns four float64 arrays shaped like
    q, k, v, z (rows of units outside ``units`` are NaN)."""
    lib = _load()
    q, k, v, dout = (np.ascontiguousarray(a) for a in (q, k, v, dout))
    z64 = np.asarray(z).dtype == np.float64
    z = np.ascontiguousarray(z, dtype=np.float64 if z64 else np.float32)
    dtype = _storage_code(q)
    for name, a in (("k", k), ("v", v), ("dout", dout)):
        if a.dtype != q.dtype:
            raise TypeError(f"{name} must have q's dtype")
    B, L, NH, dk = q.shape
    dv = v.shape[3]
    if L != H * W or k.shape != q.shape or z.shape != q.shape or dout.shape != v.shape:
        raise ValueError("shape mismatch")
    if scale is None:
        scale = 1.0 / math.sqrt(dk)
    u0, u1 = (0, B * NH) if units is None else units
    outs = [np.full(a.shape, np.nan, dtype=np.float64) for a in (q, k, v, z)]
    old = os.environ.get("OMP_NUM_THREADS")
    if threads is not None:
        os.environ["OMP_NUM_THREADS"] = str(threads)
    try:
        rc = lib.gla_oracle_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(z), 2 if z64 else 1, _ptr(dout),
                                dtype, B, NH, H, W, dk, dv, direction, float(tau), float(scale),
                                u0, u1, *[_ptr(o) for o in outs])
    finally:
        if threads is not None:
            if old is None:
                os.environ.pop("OMP_NUM_THREADS", None)
            else:
                os.environ["OMP_NUM_THREADS"] = old
    if rc != 0:
        raise RuntimeError(f"gla_oracle_bwd failed with status {rc}")
    return tuple(outs)


def bwd_gated(q, k, v, z, r, w, du, direction, H, W, tau=16.0, scale=None, eps=1e-6,
              units=None, threads=None):
    """Gradients of the gated forward u = SiLU(r) (.) w (.) o / sqrt(mean(o^2) + eps)
    (paper Section 2.1, output-gate paragraph) for du = dL/du: returns
    (dq, dk, dv, dz, dr, dw) in float64, dw summed over every (batch, token,
    head) row (one weight vector shared by the heads; w None means ones).

    o is the fp64 ungated forward; with rho = (mean_j o_j^2 + eps)^(-1/2) and
    g = du (.) SiLU(r) (.) w per row:
        do = rho g - (rho^3 / dv) o sum_j(g_j o_j)
        dr = du (.) w (.) o rho (.) SiLU'(r),  SiLU'(x) = s(x) (1 + x (1 - s(x)))
        dw = sum_rows du (.) SiLU(r) (.) o rho
    and dq, dk, dv, dz are the ungated backward's for dout = do."""
    o = fwd(q, k, v, z, direction, H, W, tau=tau, scale=scale, units=units, threads=threads)
    dv_ = v.shape[3]
    r64 = np.asarray(r, dtype=np.float64)
    du64 = np.asarray(du, dtype=np.float64)
    w64 = np.ones(dv_) if w is None else np.asarray(w, dtype=np.float64)
    rho = 1.0 / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)
    sr = silu(r64)
    g = du64 * sr * w64
    do = rho * g - (rho ** 3 / dv_) * o * np.sum(g * o, axis=-1, keepdims=True)
    sig = 1.0 / (1.0 + np.exp(-r64))
    dr = du64 * w64 * o * rho * sig * (1.0 + r64 * (1.0 - sig))
    dw = np.sum(du64 * sr * o * rho, axis=(0, 1, 2))
    q64, k64, v64 = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    z64 = np.asarray(z, dtype=np.float64)
    dq, dk, dvv, dz = bwd(q64, k64, v64, z64, do, direction, H, W, tau=tau, scale=scale,
                          units=units, threads=threads)
    return dq, dk, dvv, dz, dr, dw


def gate_logits(x, w1, w2, bias, heads, threads=None):
    """Low-rank gate logits z = (x W1) W2 + b in fp64 (paper Section 2.1,
    retention gate).  x: [B, L, d_model] float16 or float32; w1: [rank, d_model]
    with x's dtype (W1 transposed); w2: [heads*dk, rank] float32 (W2
    transposed, head h owns rows h*dk .. h*dk+dk-1); bias: [heads*dk] float32
    or None.  Returns float64 [B, L, heads, dk].
    """
    lib = _load()
    x = np.ascontiguousarray(x)
    w1 = np.ascontiguousarray(w1)
    w2 = np.ascontiguousarray(w2, dtype=np.float32)
    if x.dtype == np.float16:
        dtype = 0
    elif x.dtype == np.float32:
        dtype = 1
    else:
        raise TypeError("x must be float16 or float32")
    if w1.dtype != x.dtype:
        raise TypeError("w1 must have x's dtype")
    B, L, d_model = x.shape
    rank = w1.shape[0]
    nout = w2.shape[0]
    if w1.shape != (rank, d_model) or w2.shape != (nout, rank) or nout % heads:
        raise ValueError("shape mismatch")
    if bias is not None:
        bias = np.ascontiguousarray(bias, dtype=np.float32)
        if bias.shape != (nout,):
            raise ValueError("bias must have shape [heads*dk]")
    z = np.empty((B, L, heads, nout // heads), dtype=np.float64)
    old = os.environ.get("OMP_NUM_THREADS")
    if threads is not None:
        os.environ["OMP_NUM_THREADS"] = str(threads)
    try:
        rc = lib.gla_oracle_gate_logits(_ptr(x), _ptr(w1), _ptr(w2), _ptr(bias), dtype,
                                        B * L, d_model, rank, nout, _ptr(z))
    finally:
        if threads is not None:
            if old is None:
                os.environ.pop("OMP_NUM_THREADS", None)
            else:
                os.environ["OMP_NUM_THREADS"] = old
    if rc != 0:
        raise RuntimeError(f"gla_oracle_gate_logits failed with status {rc}")
    return z


def gate_proj_bwd(x, w1, w2, dz):
    """Gradients of the gate logits z = (x W1) W2 + b (paper Section 2.1,
    retention gate; storage as in :func:`gate_logits`: w1 [rank, d_model] is
    W1 transposed, w2 [nout, rank] is W2 transposed) for dz = dL/dz, in fp64.
    x: [B, L, d_model] or [tokens, d_model]; dz: [B, L, heads, dk] or
    [tokens, nout].  With hp = x W1 (rank values per token) and
    dhp = dz W2^T, the chain rule of the two products gives, on the stored
    arrays: dx = dhp w1, dw1 = dhp^T x, dw2 = dz^T hp, db = sum_t dz.
    Returns (dx shaped like x, dw1 [rank, d_model], dw2 [nout, rank],
    db [nout]), all float64."""
    x64 = np.asarray(x, dtype=np.float64)
    shape = x64.shape
    d_model = shape[-1]
    x64 = x64.reshape(-1, d_model)
    w1_64 = np.asarray(w1, dtype=np.float64)
    w2_64 = np.asarray(w2, dtype=np.float64)
    nout, rank = w2_64.shape
    dz64 = np.asarray(dz, dtype=np.float64).reshape(x64.shape[0], nout)
    if w1_64.shape != (rank, d_model):
        raise ValueError("shape mismatch")
    hp = x64 @ w1_64.T          # [tokens, rank]
    dhp = dz64 @ w2_64          # [tokens, rank]
    dx = dhp @ w1_64            # [tokens, d_model]
    dw1 = dhp.T @ x64           # [rank, d_model]
    dw2 = dz64.T @ hp           # [nout, rank]
    db = dz64.sum(axis=0)       # [nout]
    return dx.reshape(shape), dw1, dw2, db


# ---------------------------------------------------------------------------
# Spatial SwiGLU core (paper Section 2.1, Spatial SwiGLU paragraph), numpy fp64.
# ---------------------------------------------------------------------------

def silu(x):
    """SiLU(x) = x / (1 + e^{-x}) in fp64."""
    x = np.asarray(x, dtype=np.float64)
    return x / (1.0 + np.exp(-x))


def dwconv3x3(value, H, W, weight, bias=None):
    """3x3 depthwise convolution of the value branch on the H x W patch grid.

    value: [B, L, C] (L = H*W, token t = h*W + w), any float dtype, read as
    stored; weight: [C, 3, 3]; bias: [C] or None.  Cross-correlation with zero
    padding of one token on every side (a depthwise Conv2d with padding 1):
        y[h, w, c] = b[c] + sum_{i, j in 0..2} weight[c, i, j] * v[h + i - 1, w + j - 1, c]
    written as nine shifted adds of the zero-padded grid.  Returns fp64 [B, L, C].
    """
    v = np.asarray(value, dtype=np.float64)
    B, L, C = v.shape
    if L != H * W:
        raise ValueError("L must be H*W")
    w = np.asarray(weight, dtype=np.float64)
    if w.shape != (C, 3, 3):
        raise ValueError("weight must be [C, 3, 3]")
    grid = v.reshape(B, H, W, C)
    padded = np.zeros((B, H + 2, W + 2, C))
    padded[:, 1:H + 1, 1:W + 1, :] = grid
    out = np.zeros((B, H, W, C))
    for i in range(3):
        for j in range(3):
            out += w[:, i, j] * padded[:, i:i + H, j:j + W, :]
    if bias is not None:
        out += np.asarray(bias, dtype=np.float64)
    return out.reshape(B, L, C)


def spatial_swiglu(gate, value, H, W, weight, bias=None):
    """h = SiLU(gate) (.) dwconv3x3(value): the gating branch stays tokenwise,
    the value branch is mixed over the 3x3 grid neighbourhood.  gate, value:
    [B, L, C] as stored.  Returns fp64 [B, L, C]."""
    return silu(gate) * dwconv3x3(value, H, W, weight, bias)


# ---------------------------------------------------------------------------
# Independent O(L^2) closed form (numpy fp64), tiny inputs only.
# ---------------------------------------------------------------------------

def to_scan_order(x, direction, H, W):
    """Token-ordered [L, ...] -> scan-ordered [L, ...] by flips and transposes."""
    rest = x.shape[1:]
    if direction == L2R:
        return x
    if direction == R2L:
        return x[::-1]
    cols = x.reshape((H, W) + rest).swapaxes(0, 1).reshape((H * W,) + rest)
    return cols if direction == T2B else cols[::-1]


def from_scan_order(y, direction, H, W):
    """Inverse of :func:`to_scan_order`."""
    rest = y.shape[1:]
    if direction == L2R:
        return y
    if direction == R2L:
        return y[::-1]
    if direction == B2T:
        y = y[::-1]
    return y.reshape((W, H) + rest).swapaxes(0, 1).reshape((H * W,) + rest)


def closed_form_fwd(q, k, v, z, direction, H, W, r=None, w=None, tau=16.0, scale=None,
                    eps=1e-6):
    """Unrolled sum over s <= t with gamma products formed per pair.

    log gamma_j = log(sigmoid(z_j)) / tau = -logaddexp(0, -z_j) / tau, and the
    decay between key s and query t is exp(sum_{j=s+1..t} log gamma_j).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    z = np.asarray(z, dtype=np.float64)
    B, L, NH, dk = q.shape
    dv = v.shape[3]
    if scale is None:
        scale = 1.0 / math.sqrt(dk)
    out = np.empty((B, L, NH, dv))
    for b in range(B):
        for h in range(NH):
            Qs = to_scan_order(q[b, :, h, :], direction, H, W)
            Ks = to_scan_order(k[b, :, h, :], direction, H, W)
            Vs = to_scan_order(v[b, :, h, :], direction, H, W)
            lg = -np.logaddexp(0.0, -to_scan_order(z[b, :, h, :], direction, H, W)) / tau
            Os = np.zeros((L, dv))
            for t in range(L):
                for s in range(t + 1):
                    decay = np.exp(lg[s + 1:t + 1].sum(axis=0)) if t > s else np.ones(dk)
                    Os[t] += np.dot(Qs[t] * decay, Ks[s]) * Vs[s]
            Os *= scale
            if r is not None:
                Rs = to_scan_order(np.asarray(r, dtype=np.float64)[b, :, h, :], direction, H, W)
                wv = np.ones(dv) if w is None else np.asarray(w, dtype=np.float64)
                rms = np.sqrt((Os * Os).mean(axis=1, keepdims=True) + eps)
                Os = (Rs / (1.0 + np.exp(-Rs))) * wv * Os / rms
            out[b, :, h, :] = from_scan_order(Os, direction, H, W)
    return out
