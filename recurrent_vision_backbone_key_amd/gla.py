"""Python binding of the C ABI in include/gla.h (argument marshalling only).

Every step of the forward pass runs in the HIP kernels of ``libgla.so``;
PyTorch only provides device memory and the current stream.  There is no
fallback: a missing library raises.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "_lib", "libgla.so")

L2R, R2L, T2B, B2T = 0, 1, 2, 3
F16, F32 = 0, 1
ALGO_AUTO, ALGO_SINGLE_PASS, ALGO_THREE_PASS = 0, 1, 2
STATUS = {0: "GLA_OK", 1: "GLA_EINVAL", 2: "GLA_EUNSUPPORTED", 3: "GLA_EWORKSPACE", 4: "GLA_EHIP",
          5: "GLA_EKERNEL", 6: "GLA_ESCRATCH"}
NOALLOC_SCRATCH_BYTES = 64 << 20  # include/gla.h: GLA_NOALLOC_SCRATCH_BYTES
# error-word bits (include/gla.h: GLA_WS_ERR_*)
WS_ERR_WAIT, WS_ERR_TICKET, WS_ERR_INIT = 1, 2, 4
EXPORTS = ("gla_fwd", "gla_fwd_noalloc", "gla_workspace_size", "gla_workspace_init", "gla_workspace_status",
           "gla_gate_logits", "gla_gate_proj_bwd", "gla_gate_proj_bwd_workspace_size",
           "gla_fwd_gate_proj", "gla_workspace_size_gate_proj", "gla_spatial_swiglu",
           "gla_bwd", "gla_bwd_workspace_size", "gla_bwd_gated", "gla_bwd_gated_workspace_size",
           "gla_status_str", "gla_abi_version")


class GlaOpts(ctypes.Structure):
    """Mirror of ``gla_opts`` (include/gla.h)."""
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("heads", ctypes.c_int32),
        ("dk", ctypes.c_int32),
        ("dv", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("tau", ctypes.c_float),
        ("scale", ctypes.c_float),
        ("eps", ctypes.c_float),
        ("norm_weight", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("stream", ctypes.c_void_p),
        ("segment_chunks", ctypes.c_int32),
        ("algorithm", ctypes.c_int32),
    ]


class GlaGateProj(ctypes.Structure):
    """Mirror of ``gla_gate_proj`` (include/gla.h)."""
    _fields_ = [
        ("x", ctypes.c_void_p),
        ("w1", ctypes.c_void_p),
        ("w2", ctypes.c_void_p),
        ("bias", ctypes.c_void_p),
        ("d_model", ctypes.c_int32),
        ("rank", ctypes.c_int32),
    ]


class GlaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


_lib = None


def lib():
    """The loaded libgla.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m recurrent_vision_backbone_key_amd.build` (no fallback exists)")
        # torch first: its bundled HIP runtime carries the same soname as the
        # system one libgla.so links against, so loading torch first makes the
        # library bind to torch's runtime; loaded the other way round, the
        # process would hold two HIP runtimes and torch's would see no GPU
        _torch()
        h = ctypes.CDLL(LIB_PATH)
        h.gla_fwd.restype = ctypes.c_int
        h.gla_fwd.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int] * 4 + \
            [ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(GlaOpts)]
        h.gla_fwd_noalloc.restype = ctypes.c_int
        h.gla_fwd_noalloc.argtypes = h.gla_fwd.argtypes
        h.gla_workspace_size.restype = ctypes.c_size_t
        h.gla_workspace_size.argtypes = [ctypes.c_int] * 4 + [ctypes.POINTER(GlaOpts)]
        h.gla_workspace_init.restype = ctypes.c_int
        h.gla_workspace_init.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        h.gla_workspace_status.restype = ctypes.c_int
        h.gla_workspace_status.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                           ctypes.POINTER(ctypes.c_uint32)]
        h.gla_gate_logits.restype = ctypes.c_int
        h.gla_gate_logits.argtypes = [ctypes.POINTER(GlaGateProj)] + [ctypes.c_int] * 5 + \
            [ctypes.c_void_p, ctypes.c_void_p]
        h.gla_gate_proj_bwd.restype = ctypes.c_int
        h.gla_gate_proj_bwd.argtypes = [ctypes.POINTER(GlaGateProj)] + [ctypes.c_int] * 3 + \
            [ctypes.c_void_p] * 6 + [ctypes.c_size_t, ctypes.c_void_p]
        h.gla_gate_proj_bwd_workspace_size.restype = ctypes.c_size_t
        h.gla_gate_proj_bwd_workspace_size.argtypes = [ctypes.POINTER(GlaGateProj), ctypes.c_int,
                                                       ctypes.c_int]
        h.gla_fwd_gate_proj.restype = ctypes.c_int
        h.gla_fwd_gate_proj.argtypes = [ctypes.c_void_p] * 3 + [ctypes.POINTER(GlaGateProj)] + \
            [ctypes.c_int] * 4 + [ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(GlaOpts)]
        h.gla_workspace_size_gate_proj.restype = ctypes.c_size_t
        h.gla_workspace_size_gate_proj.argtypes = [ctypes.c_int] * 4 + \
            [ctypes.POINTER(GlaGateProj), ctypes.POINTER(GlaOpts)]
        h.gla_spatial_swiglu.restype = ctypes.c_int
        h.gla_spatial_swiglu.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                         ctypes.c_void_p, ctypes.c_void_p] + [ctypes.c_int] * 5 + \
            [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
        h.gla_bwd.restype = ctypes.c_int
        h.gla_bwd.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int] * 3 + [ctypes.c_void_p] * 4 + \
            [ctypes.POINTER(GlaOpts)]
        h.gla_bwd_workspace_size.restype = ctypes.c_size_t
        h.gla_bwd_workspace_size.argtypes = [ctypes.c_int] * 3 + [ctypes.POINTER(GlaOpts)]
        h.gla_bwd_gated.restype = ctypes.c_int
        h.gla_bwd_gated.argtypes = [ctypes.c_void_p] * 6 + [ctypes.c_int] * 3 + \
            [ctypes.c_void_p] * 6 + [ctypes.POINTER(GlaOpts)]
        h.gla_bwd_gated_workspace_size.restype = ctypes.c_size_t
        h.gla_bwd_gated_workspace_size.argtypes = [ctypes.c_int] * 3 + [ctypes.POINTER(GlaOpts)]
        h.gla_status_str.restype = ctypes.c_char_p
        h.gla_status_str.argtypes = [ctypes.c_int]
        h.gla_abi_version.restype = ctypes.c_int
        h.gla_abi_version.argtypes = []
        _lib = h
    return _lib


def status_str(status: int) -> str:
    return lib().gla_status_str(status).decode()


def abi_version() -> int:
    return lib().gla_abi_version()


def make_opts(batch, heads, dk, dv, dtype, tau=16.0, scale=None, eps=1e-6, norm_weight=0,
              workspace=0, workspace_bytes=0, stream=0, segment_chunks=0,
              algorithm=ALGO_AUTO) -> GlaOpts:
    return GlaOpts(batch, heads, dk, dv, dtype, float(tau),
                   0.0 if scale is None else float(scale), float(eps),
                   norm_weight or None, workspace or None, workspace_bytes, stream or None,
                   segment_chunks, algorithm)


def workspace_size(direction, H, W, chunk, opts: GlaOpts) -> int:
    return lib().gla_workspace_size(direction, H, W, chunk, ctypes.byref(opts))


def workspace_init(workspace, stream=None):
    """Initialise a device workspace tensor (include/gla.h: gla_workspace_init)."""
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(workspace.device).cuda_stream
    nbytes = workspace.numel() * workspace.element_size()
    st = lib().gla_workspace_init(workspace.data_ptr(), nbytes & ~3, stream)
    if st != 0:
        raise GlaError(st, f"gla_workspace_init failed: {status_str(st)}")


def workspace_status(workspace, stream=None) -> int:
    """Error bits a kernel left in a forward workspace (include/gla.h:
    gla_workspace_status; waits for the stream).  Returns 0 when none; a
    nonzero word means the library has re-initialised the workspace."""
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(workspace.device).cuda_stream
    nbytes = workspace.numel() * workspace.element_size()
    bits = ctypes.c_uint32(0)
    st = lib().gla_workspace_status(workspace.data_ptr(), nbytes & ~3, stream, ctypes.byref(bits))
    if st not in (0, 5):
        raise GlaError(st, f"gla_workspace_status failed: {status_str(st)}")
    return int(bits.value)


def new_workspace(direction, H, W, chunk, opts: GlaOpts, device):
    """An initialised workspace tensor sized for these arguments (or None)."""
    torch = _torch()
    need = workspace_size(direction, H, W, chunk, opts)
    if not need:
        return None
    ws = torch.empty(need, dtype=torch.uint8, device=device)
    workspace_init(ws)
    return ws


# Workspaces the binding keeps for calls that pass none: one per (device,
# stream), grown when a call needs more and initialised once when allocated;
# every completed call leaves it ready for the next, so a call allocates
# nothing once the workspace is large enough.  Calls on one stream are ordered,
# so they may share it.
_ws_cache = {}


def cached_workspace(need, device, stream):
    """An initialised workspace of at least `need` bytes for (device, stream)."""
    torch = _torch()
    key = (str(device), int(stream or 0))
    ws = _ws_cache.get(key)
    if ws is None or ws.numel() < need:
        ws = torch.empty(max(need, 1 << 20), dtype=torch.uint8, device=device)
        workspace_init(ws, stream)
        _ws_cache[key] = ws
    return ws


def _torch():
    import torch
    return torch


def fwd(q, k, v, z, direction, H, W, chunk=64, r=None, norm_weight=None, eps=1e-6, out=None,
        tau=16.0, scale=None, segment_chunks=0, workspace=None, stream=None,
        algorithm=ALGO_AUTO):
    """Chunkwise key-only GLA forward (include/gla.h: gla_fwd) on CUDA tensors.

    q, k, z: [B, L, NH, dk]; v, r: [B, L, NH, dv]; q, k, v, r float16 or float32,
    z float32, norm_weight [dv] float32.  Returns out [B, L, NH, dv] in q's dtype.
    """
    torch = _torch()
    B, L, NH, dk = q.shape
    dv = v.shape[3]
    if q.dtype == torch.float16:
        dtype = F16
    elif q.dtype == torch.float32:
        dtype = F32
    else:
        raise TypeError("q must be float16 or float32")
    for name, t in (("q", q), ("k", k), ("v", v), ("z", z), ("r", r), ("norm_weight", norm_weight)):
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous device tensor")
    if z.dtype != torch.float32 or (norm_weight is not None and norm_weight.dtype != torch.float32):
        raise TypeError("gate logits and norm_weight must be float32")
    for name, t in (("k", k), ("v", v), ("r", r)):
        if t is not None and t.dtype != q.dtype:
            raise TypeError(f"{name} must have q's dtype")
    if out is None:
        out = torch.empty((B, L, NH, dv), dtype=q.dtype, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    opts = make_opts(B, NH, dk, dv, dtype, tau, scale, eps,
                     norm_weight.data_ptr() if norm_weight is not None else 0,
                     stream=stream, segment_chunks=segment_chunks, algorithm=algorithm)
    need = workspace_size(direction, H, W, chunk, opts)
    if need:
        # a workspace passed in must have been initialised once
        # (workspace_init); without one the binding's own is used
        if workspace is None:
            workspace = cached_workspace(need, q.device, stream)
        opts.workspace = workspace.data_ptr()
        opts.workspace_bytes = workspace.numel() * workspace.element_size()
    st = lib().gla_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), z.data_ptr(), direction, H, W,
                       chunk, out.data_ptr(), r.data_ptr() if r is not None else None,
                       ctypes.byref(opts))
    if st != 0:
        raise GlaError(st, f"gla_fwd failed: {status_str(st)}")
    return out


def fwd_noalloc(q, k, v, z, direction, H, W, chunk=64, r=None, norm_weight=None, eps=1e-6,
                out=None, tau=16.0, scale=None, segment_chunks=0, stream=None,
                algorithm=ALGO_AUTO):
    """gla_fwd without a workspace (include/gla.h: gla_fwd_noalloc): the
    library's own fixed scratch array holds the exchange; ``out`` must be
    given for a call that allocates nothing at all.  Shapes as :func:`fwd`."""
    torch = _torch()
    B, L, NH, dk = q.shape
    dv = v.shape[3]
    dtype = F16 if q.dtype == torch.float16 else F32 if q.dtype == torch.float32 else None
    if dtype is None:
        raise TypeError("q must be float16 or float32")
    for name, t in (("q", q), ("k", k), ("v", v), ("z", z), ("r", r), ("norm_weight", norm_weight)):
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous device tensor")
    if z.dtype != torch.float32 or (norm_weight is not None and norm_weight.dtype != torch.float32):
        raise TypeError("gate logits and norm_weight must be float32")
    for name, t in (("k", k), ("v", v), ("r", r)):
        if t is not None and t.dtype != q.dtype:
            raise TypeError(f"{name} must have q's dtype")
    if out is None:
        out = torch.empty((B, L, NH, dv), dtype=q.dtype, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    opts = make_opts(B, NH, dk, dv, dtype, tau, scale, eps,
                     norm_weight.data_ptr() if norm_weight is not None else 0,
                     stream=stream, segment_chunks=segment_chunks, algorithm=algorithm)
    st = lib().gla_fwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), z.data_ptr(), direction,
                               H, W, chunk, out.data_ptr(),
                               r.data_ptr() if r is not None else None, ctypes.byref(opts))
    if st != 0:
        raise GlaError(st, f"gla_fwd_noalloc failed: {status_str(st)}")
    return out


def bwd_workspace_size(direction, H, W, opts: GlaOpts) -> int:
    return lib().gla_bwd_workspace_size(direction, H, W, ctypes.byref(opts))


def bwd(q, k, v, z, dout, direction, H, W, tau=16.0, scale=None, grads=None, workspace=None,
        stream=None):
    """Gradients of the ungated forward (include/gla.h: gla_bwd) on CUDA tensors.

    q, k, z: [B, L, NH, d]; v, dout: [B, L, NH, d]; q, k, v, dout float16 or
    float32, z float32.  Returns (dq, dk, dv, dz): dq, dk, dv in q's dtype, dz
    float32.  ``grads`` may supply the four output tensors.
    """
    torch = _torch()
    B, L, NH, dk = q.shape
    dv = v.shape[3]
    if q.dtype == torch.float16:
        dtype = F16
    elif q.dtype == torch.float32:
        dtype = F32
    else:
        raise TypeError("q must be float16 or float32")
    for name, t in (("q", q), ("k", k), ("v", v), ("z", z), ("dout", dout)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
    if z.dtype != torch.float32:
        raise TypeError("gate logits must be float32")
    for name, t in (("k", k), ("v", v), ("dout", dout)):
        if t.dtype != q.dtype:
            raise TypeError(f"{name} must have q's dtype")
    if grads is None:
        grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v),
                 torch.empty(z.shape, dtype=torch.float32, device=q.device))
    dq, dk_, dv_, dz = grads
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    opts = make_opts(B, NH, dk, dv, dtype, tau, scale, stream=stream)
    need = bwd_workspace_size(direction, H, W, opts)
    if need:
        if workspace is None:
            workspace = cached_workspace(need, q.device, stream)
        opts.workspace = workspace.data_ptr()
        opts.workspace_bytes = workspace.numel() * workspace.element_size()
    st = lib().gla_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), z.data_ptr(), dout.data_ptr(),
                       direction, H, W, dq.data_ptr(), dk_.data_ptr(), dv_.data_ptr(),
                       dz.data_ptr(), ctypes.byref(opts))
    if st != 0:
        raise GlaError(st, f"gla_bwd failed: {status_str(st)}")
    return dq, dk_, dv_, dz


def bwd_gated_workspace_size(direction, H, W, opts: GlaOpts) -> int:
    return lib().gla_bwd_gated_workspace_size(direction, H, W, ctypes.byref(opts))


def bwd_gated(q, k, v, z, r, dout, direction, H, W, norm_weight=None, eps=1e-6, tau=16.0,
              scale=None, grads=None, want_dw=True, workspace=None, stream=None):
    """Gradients of the gated forward (include/gla.h: gla_bwd_gated) on CUDA
    tensors: dout = dL/du for u = SiLU(r) * w * RMSNorm(o).  Returns
    (dq, dk, dv, dz, dr, dw); dq, dk, dv, dr in q's dtype, dz float32, dw
    float32 [dv] (None unless want_dw).  ``grads`` may supply the six outputs."""
    torch = _torch()
    B, L, NH, dk = q.shape
    dv = v.shape[3]
    if q.dtype == torch.float16:
        dtype = F16
    elif q.dtype == torch.float32:
        dtype = F32
    else:
        raise TypeError("q must be float16 or float32")
    for name, t in (("q", q), ("k", k), ("v", v), ("z", z), ("r", r), ("dout", dout),
                    ("norm_weight", norm_weight)):
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous device tensor")
    if z.dtype != torch.float32 or (norm_weight is not None and norm_weight.dtype != torch.float32):
        raise TypeError("gate logits and norm_weight must be float32")
    for name, t in (("k", k), ("v", v), ("r", r), ("dout", dout)):
        if t.dtype != q.dtype:
            raise TypeError(f"{name} must have q's dtype")
    if grads is None:
        grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v),
                 torch.empty(z.shape, dtype=torch.float32, device=q.device), torch.empty_like(r),
                 torch.empty((dv,), dtype=torch.float32, device=q.device) if want_dw else None)
    dq, dk_, dv_, dz, dr, dw = grads
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    opts = make_opts(B, NH, dk, dv, dtype, tau, scale, eps,
                     norm_weight.data_ptr() if norm_weight is not None else 0, stream=stream)
    need = bwd_gated_workspace_size(direction, H, W, opts)
    if need:
        if workspace is None:
            workspace = cached_workspace(need, q.device, stream)
        opts.workspace = workspace.data_ptr()
        opts.workspace_bytes = workspace.numel() * workspace.element_size()
    st = lib().gla_bwd_gated(q.data_ptr(), k.data_ptr(), v.data_ptr(), z.data_ptr(), r.data_ptr(),
                             dout.data_ptr(), direction, H, W, dq.data_ptr(), dk_.data_ptr(),
                             dv_.data_ptr(), dz.data_ptr(), dr.data_ptr(),
                             dw.data_ptr() if dw is not None else None, ctypes.byref(opts))
    if st != 0:
        raise GlaError(st, f"gla_bwd_gated failed: {status_str(st)}")
    return dq, dk_, dv_, dz, dr, dw


def make_gate(x, w1, w2, bias=None) -> GlaGateProj:
    """``gla_gate_proj`` over device tensors x [B, L, d_model], w1 [rank, d_model]
    (x's dtype), w2 [NH*dk, rank] and bias [NH*dk] (float32)."""
    torch = _torch()
    for name, t in (("x", x), ("w1", w1), ("w2", w2), ("bias", bias)):
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous device tensor")
    if w1.dtype != x.dtype:
        raise TypeError("w1 must have x's dtype")
    if w2.dtype != torch.float32 or (bias is not None and bias.dtype != torch.float32):
        raise TypeError("w2 and bias must be float32")
    rank, d_model = w1.shape
    if x.shape[-1] != d_model or w2.shape[1] != rank:
        raise ValueError("gate projection shapes do not match")
    return GlaGateProj(x.data_ptr(), w1.data_ptr(), w2.data_ptr(),
                       bias.data_ptr() if bias is not None else None, d_model, rank)


def gate_logits(x, w1, w2, bias, heads, out=None, stream=None):
    """Gate logits z = (x W1) W2 + b (include/gla.h: gla_gate_logits).
    x: [B, L, d_model] float16/float32; returns z [B, L, heads, dk] float32."""
    torch = _torch()
    B, L, _ = x.shape
    nout = w2.shape[0]
    if nout % heads:
        raise ValueError("w2 rows must be heads * dk")
    dk = nout // heads
    dtype = F16 if x.dtype == torch.float16 else F32 if x.dtype == torch.float32 else None
    if dtype is None:
        raise TypeError("x must be float16 or float32")
    gate = make_gate(x, w1, w2, bias)
    if out is None:
        out = torch.empty((B, L, heads, dk), dtype=torch.float32, device=x.device)
    if stream is None:
        stream = torch.cuda.current_stream(x.device).cuda_stream
    st = lib().gla_gate_logits(ctypes.byref(gate), B, L, heads, dk, dtype, out.data_ptr(), stream)
    if st != 0:
        raise GlaError(st, f"gla_gate_logits failed: {status_str(st)}")
    return out


def gate_proj_bwd_workspace_size(gate: GlaGateProj, tokens, nout) -> int:
    return lib().gla_gate_proj_bwd_workspace_size(ctypes.byref(gate), tokens, nout)


def gate_proj_bwd(x, w1, w2, dz, grads=None, workspace=None, stream=None):
    """Gradients of the gate projection (include/gla.h: gla_gate_proj_bwd).
    x: [B, L, d_model] float16/float32, w1 [rank, d_model] (x's dtype),
    w2 [nout, rank] float32, dz: [B, L, heads, dk] or [B, L, nout] float32.
    Returns (dx like x, dw1 [rank, d_model] float32, dw2 [nout, rank] float32,
    db [nout] float32)."""
    torch = _torch()
    B, L, d_model = x.shape
    nout = w2.shape[0]
    if dz.dtype != torch.float32 or dz.numel() != B * L * nout:
        raise ValueError("dz must be float32 with B * L * nout elements")
    dtype = F16 if x.dtype == torch.float16 else F32 if x.dtype == torch.float32 else None
    if dtype is None:
        raise TypeError("x must be float16 or float32")
    for name, t in (("x", x), ("w1", w1), ("w2", w2), ("dz", dz)):
        if not (t.is_cuda and t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous device tensor")
    gate = make_gate(x, w1, w2, None)
    if grads is None:
        grads = (torch.empty_like(x), torch.empty(w1.shape, dtype=torch.float32, device=x.device),
                 torch.empty(w2.shape, dtype=torch.float32, device=x.device),
                 torch.empty((nout,), dtype=torch.float32, device=x.device))
    dx, dw1, dw2, db = grads
    need = gate_proj_bwd_workspace_size(gate, B * L, nout)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
    if stream is None:
        stream = torch.cuda.current_stream(x.device).cuda_stream
    st = lib().gla_gate_proj_bwd(ctypes.byref(gate), B * L, nout, dtype, dz.data_ptr(), dx.data_ptr(),
                                 dw1.data_ptr(), dw2.data_ptr(), db.data_ptr(), workspace.data_ptr(),
                                 workspace.numel(), stream)
    if st != 0:
        raise GlaError(st, f"gla_gate_proj_bwd failed: {status_str(st)}")
    return dx, dw1, dw2, db


def workspace_size_gate_proj(direction, H, W, chunk, gate: GlaGateProj, opts: GlaOpts) -> int:
    return lib().gla_workspace_size_gate_proj(direction, H, W, chunk, ctypes.byref(gate),
                                              ctypes.byref(opts))


def fwd_gate_proj(q, k, v, x, w1, w2, bias, direction, H, W, chunk=64, r=None,
                  norm_weight=None, eps=1e-6, out=None, tau=16.0, scale=None, segment_chunks=0,
                  workspace=None, stream=None, algorithm=ALGO_AUTO):
    """gla_fwd with the gate logits projected from x in the library
    (include/gla.h: gla_fwd_gate_proj).  q, k: [B, L, NH, dk]; v, r:
    [B, L, NH, dv]; x: [B, L, d_model] and w1: [rank, d_model] in q's dtype;
    w2: [NH*dk, rank], bias: [NH*dk] float32 (or None)."""
    torch = _torch()
    B, L, NH, dk = q.shape
    dv = v.shape[3]
    if q.dtype == torch.float16:
        dtype = F16
    elif q.dtype == torch.float32:
        dtype = F32
    else:
        raise TypeError("q must be float16 or float32")
    for name, t in (("q", q), ("k", k), ("v", v), ("r", r), ("norm_weight", norm_weight)):
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous device tensor")
    for name, t in (("k", k), ("v", v), ("r", r), ("x", x)):
        if t is not None and t.dtype != q.dtype:
            raise TypeError(f"{name} must have q's dtype")
    if tuple(x.shape[:2]) != (B, L) or w2.shape[0] != NH * dk:
        raise ValueError("x must be [B, L, d_model] and w2 [NH*dk, rank]")
    gate = make_gate(x, w1, w2, bias)
    if out is None:
        out = torch.empty((B, L, NH, dv), dtype=q.dtype, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    opts = make_opts(B, NH, dk, dv, dtype, tau, scale, eps,
                     norm_weight.data_ptr() if norm_weight is not None else 0,
                     stream=stream, segment_chunks=segment_chunks, algorithm=algorithm)
    need = workspace_size_gate_proj(direction, H, W, chunk, gate, opts)
    if need:
        if workspace is None:
            workspace = cached_workspace(need, q.device, stream)
        opts.workspace = workspace.data_ptr()
        opts.workspace_bytes = workspace.numel() * workspace.element_size()
    st = lib().gla_fwd_gate_proj(q.data_ptr(), k.data_ptr(), v.data_ptr(), ctypes.byref(gate),
                                 direction, H, W, chunk, out.data_ptr(),
                                 r.data_ptr() if r is not None else None, ctypes.byref(opts))
    if st != 0:
        raise GlaError(st, f"gla_fwd_gate_proj failed: {status_str(st)}")
    return out


def spatial_swiglu(gate, value, H, W, conv_w, conv_b=None, out=None, stream=None):
    """Spatial SwiGLU core (include/gla.h: gla_spatial_swiglu):
    out = SiLU(gate) * (3x3 depthwise conv of value on the H x W grid + conv_b).
    gate, value: [B, H*W, C] float16/float32 (row strides taken from the
    tensors: views of one [B, H*W, 2C] tensor work); conv_w [C, 3, 3] and
    conv_b [C] float32.  Returns out [B, H*W, C] in gate's dtype."""
    torch = _torch()
    B, L, C = gate.shape
    if tuple(value.shape) != (B, L, C) or L != H * W:
        raise ValueError("gate and value must be [B, H*W, C]")
    if value.dtype != gate.dtype:
        raise TypeError("value must have gate's dtype")
    dtype = F16 if gate.dtype == torch.float16 else F32 if gate.dtype == torch.float32 else None
    if dtype is None:
        raise TypeError("gate must be float16 or float32")
    for name, t in (("gate", gate), ("value", value)):
        if not t.is_cuda or t.stride(2) != 1 or t.stride(0) != t.stride(1) * L:
            raise ValueError(f"{name} must be a device tensor with unit channel stride and "
                             "uniform token stride")
    if gate.stride(1) != value.stride(1):
        raise ValueError("gate and value must share a row stride")
    for name, t in (("conv_w", conv_w), ("conv_b", conv_b)):
        if t is not None and (not t.is_cuda or not t.is_contiguous() or t.dtype != torch.float32):
            raise ValueError(f"{name} must be a contiguous float32 device tensor")
    if out is None:
        out = torch.empty((B, L, C), dtype=gate.dtype, device=gate.device)
    if stream is None:
        stream = torch.cuda.current_stream(gate.device).cuda_stream
    st = lib().gla_spatial_swiglu(gate.data_ptr(), value.data_ptr(), gate.stride(1),
                                  conv_w.data_ptr(), conv_b.data_ptr() if conv_b is not None else None,
                                  B, H, W, C, dtype, out.data_ptr(), out.stride(1), stream)
    if st != 0:
        raise GlaError(st, f"gla_spatial_swiglu failed: {status_str(st)}")
    return out
