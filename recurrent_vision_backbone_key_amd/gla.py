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
STATUS = {0: "GLA_OK", 1: "GLA_EINVAL", 2: "GLA_EUNSUPPORTED", 3: "GLA_EWORKSPACE", 4: "GLA_EHIP"}
EXPORTS = ("gla_fwd", "gla_workspace_size", "gla_workspace_init", "gla_status_str",
           "gla_abi_version")


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
        h = ctypes.CDLL(LIB_PATH)
        h.gla_fwd.restype = ctypes.c_int
        h.gla_fwd.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int] * 4 + \
            [ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(GlaOpts)]
        h.gla_workspace_size.restype = ctypes.c_size_t
        h.gla_workspace_size.argtypes = [ctypes.c_int] * 4 + [ctypes.POINTER(GlaOpts)]
        h.gla_workspace_init.restype = ctypes.c_int
        h.gla_workspace_init.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
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
    """Clear a device workspace tensor (include/gla.h: gla_workspace_init)."""
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(workspace.device).cuda_stream
    nbytes = workspace.numel() * workspace.element_size()
    st = lib().gla_workspace_init(workspace.data_ptr(), nbytes & ~3, stream)
    if st != 0:
        raise GlaError(st, f"gla_workspace_init failed: {status_str(st)}")


def new_workspace(direction, H, W, chunk, opts: GlaOpts, device):
    """A cleared workspace tensor sized for these arguments (or None)."""
    torch = _torch()
    need = workspace_size(direction, H, W, chunk, opts)
    if not need:
        return None
    return torch.zeros(need, dtype=torch.uint8, device=device)


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
        # a workspace passed in must have been cleared once (workspace_init);
        # one allocated here starts cleared
        if workspace is None or workspace.numel() * workspace.element_size() < need:
            workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)
        opts.workspace = workspace.data_ptr()
        opts.workspace_bytes = workspace.numel() * workspace.element_size()
    st = lib().gla_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), z.data_ptr(), direction, H, W,
                       chunk, out.data_ptr(), r.data_ptr() if r is not None else None,
                       ctypes.byref(opts))
    if st != 0:
        raise GlaError(st, f"gla_fwd failed: {status_str(st)}")
    return out
