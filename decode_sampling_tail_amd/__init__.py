"""Python binding of the decode-tail HIP library (libtail.so).

Argument marshalling only: every step of the tail runs in the library's HIP
kernels.  Tensors must be contiguous CUDA (HIP) tensors on one device; the
calls enqueue on torch's current stream of that device and never
synchronize.  There is no CPU fallback: if the library is not built, loading
it raises.

The names mirror the C entry points in include/tail.h:
rmsnorm, lm_head, rmsnorm_lm_head, topk (tail_topk, or tail_topk_ex with its
options), sample, forward, workspace_size, status_string.  ``page=True``
selects TAIL_PAGE_PRECISION (bf16 GEMM input, top-k over the bf16 logit
mirror); ``nan_fold=True`` selects TAIL_NAN_FOLD.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtail.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = 0, 1, 2, 3, 4
F32, F16, BF16 = 0, 1, 2
EMIT_LOGITS, ZERO_PAD, DEFERRED_RMS, PAGE_PRECISION, NAN_FOLD = 1, 2, 4, 8, 16
K_MAX, GBS_MAX, H_MAX = 1024, 4096, 65536

EXPORTS = ("tail_rmsnorm", "tail_lm_head", "tail_rmsnorm_lm_head", "tail_topk", "tail_topk_ex",
           "tail_sample", "tail_forward", "tail_workspace_size", "tail_status_string")

_lib = None


class TailError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {status_string(status)} (status {status})")


def lib() -> ctypes.CDLL:
    """The loaded libtail.so with typed entry points (raises if not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run `python -m decode_sampling_tail_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i, u, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_uint, ctypes.c_float, ctypes.c_size_t
        L.tail_rmsnorm.argtypes = [vp, i, vp, i, i, i, f, u, vp, vp, vp]
        L.tail_lm_head.argtypes = [vp, vp, vp, i, i, i, i, u, vp, vp, sz, vp]
        L.tail_rmsnorm_lm_head.argtypes = [vp, i, vp, vp, i, i, i, i, f, u, vp, vp, vp, sz, vp]
        L.tail_topk.argtypes = [vp, i, i, i, vp, vp, vp, sz, vp]
        L.tail_topk_ex.argtypes = [vp, i, i, i, u, vp, vp, vp, vp, sz, vp]
        L.tail_sample.argtypes = [vp, vp, i, i, vp, i, vp, vp]
        L.tail_forward.argtypes = [vp, i, vp, vp, i, i, i, i, i, f, u, vp, i, vp, vp, vp, vp, vp, sz, vp]
        L.tail_workspace_size.argtypes = [i, i, i, i, i, u]
        L.tail_workspace_size.restype = sz
        L.tail_status_string.argtypes = [i]
        L.tail_status_string.restype = ctypes.c_char_p
        for name in ("tail_rmsnorm", "tail_lm_head", "tail_rmsnorm_lm_head", "tail_topk",
                     "tail_topk_ex", "tail_sample", "tail_forward"):
            getattr(L, name).restype = i
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().tail_status_string(int(status)).decode()


def workspace_size(gbs: int, H: int, H_u: int, V: int, k: int, flags: int) -> int:
    return int(lib().tail_workspace_size(gbs, H, H_u, V, k, flags))


# ----------------------------------------------------------------- marshalling
def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t):
    if not t.is_cuda:
        raise ValueError("decode_sampling_tail_amd needs GPU tensors")
    if not t.is_contiguous():
        raise ValueError("decode_sampling_tail_amd needs contiguous tensors")
    return t.device


def _stream(device):
    return ctypes.c_void_p(_torch().cuda.current_stream(device).cuda_stream)


def _hidden_dtype(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.float16:
        return F16
    if t.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return BF16
    raise ValueError(f"hidden dtype {t.dtype} is not fp32, fp16 or bf16")


def _weight(t):
    torch = _torch()
    if t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise ValueError("the lm_head weight must be bf16 (or its raw 16-bit pattern)")
    return t


def _call(name, *args):
    st = getattr(lib(), name)(*args)
    if st != OK:
        raise TailError(name, st)


def _flags(zero_pad=False, deferred=False, emit=False, page=False, nan_fold=False) -> int:
    return ((ZERO_PAD if zero_pad else 0) | (DEFERRED_RMS if deferred else 0) |
            (EMIT_LOGITS if emit else 0) | (PAGE_PRECISION if page else 0) |
            (NAN_FOLD if nan_fold else 0))


def rmsnorm(hidden, gamma, H_u=None, eps=1e-5, zero_pad=False, deferred=False, out_y=None, out_r=None,
            page=False):
    """tail_rmsnorm: returns (y [gbs,H] fp32, r [gbs] fp32)."""
    torch = _torch()
    dev = _dev(hidden)
    gbs, H = hidden.shape
    H_u = H if H_u is None else H_u
    y = out_y if out_y is not None else torch.empty((gbs, H), dtype=torch.float32, device=dev)
    r = out_r if out_r is not None else torch.empty((gbs,), dtype=torch.float32, device=dev)
    _call("tail_rmsnorm", _ptr(hidden), _hidden_dtype(hidden), _ptr(gamma), gbs, H, H_u, eps,
          _flags(zero_pad, deferred, page=page), _ptr(y), _ptr(r), _stream(dev))
    return y, r


def lm_head(y, w_t, H_u=None, zero_pad=False, row_scale=None, out=None, ws=None, page=False):
    """tail_lm_head: logits [gbs,V] fp32 = row_scale * (y @ W)."""
    torch = _torch()
    dev = _dev(y)
    gbs, H = y.shape
    V = w_t.shape[1]
    H_u = H if H_u is None else H_u
    logits = out if out is not None else torch.empty((gbs, V), dtype=torch.float32, device=dev)
    if ws is None:
        n = workspace_size(gbs, H, H_u, V, 1, _flags(zero_pad, emit=True, page=page))
        ws = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
    _call("tail_lm_head", _ptr(y), _ptr(_weight(w_t)), _ptr(row_scale), gbs, H, H_u, V,
          _flags(zero_pad, page=page), _ptr(logits), _ptr(ws), ws.numel(), _stream(dev))
    return logits


def rmsnorm_lm_head(hidden, gamma, w_t, H_u=None, eps=1e-5, zero_pad=False, deferred=True, out=None,
                    out_r=None, ws=None, page=False):
    """tail_rmsnorm_lm_head: (logits [gbs,V] fp32, r [gbs] fp32)."""
    torch = _torch()
    dev = _dev(hidden)
    gbs, H = hidden.shape
    V = w_t.shape[1]
    H_u = H if H_u is None else H_u
    flags = _flags(zero_pad, deferred, page=page)
    logits = out if out is not None else torch.empty((gbs, V), dtype=torch.float32, device=dev)
    r = out_r if out_r is not None else torch.empty((gbs,), dtype=torch.float32, device=dev)
    if ws is None:
        n = workspace_size(gbs, H, H_u, V, 1, flags | EMIT_LOGITS)
        ws = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
    _call("tail_rmsnorm_lm_head", _ptr(hidden), _hidden_dtype(hidden), _ptr(gamma), _ptr(_weight(w_t)),
          gbs, H, H_u, V, eps, flags, _ptr(logits), _ptr(r), _ptr(ws), ws.numel(), _stream(dev))
    return logits, r


def topk(logits, k, out_vals=None, out_idx=None, ws=None, mirror=False, nan_fold=False, taps=None):
    """tail_topk, or tail_topk_ex when mirror (rank the bf16 rounding of the
    logits), nan_fold (NaN ranks as -inf) or taps ([gbs, 4] int32 tensor for
    the stage-1 diagnostics, as raw u32) is given: (vals [gbs,k] fp32
    descending, idx [gbs,k] int32)."""
    torch = _torch()
    dev = _dev(logits)
    gbs, V = logits.shape
    vals = out_vals if out_vals is not None else torch.empty((gbs, k), dtype=torch.float32, device=dev)
    idx = out_idx if out_idx is not None else torch.empty((gbs, k), dtype=torch.int32, device=dev)
    if ws is None:
        ws = torch.empty(max(workspace_size(gbs, 1, 1, V, k, EMIT_LOGITS), 1), dtype=torch.uint8, device=dev)
    if mirror or nan_fold or taps is not None:
        flags = (PAGE_PRECISION if mirror else 0) | (NAN_FOLD if nan_fold else 0)
        _call("tail_topk_ex", _ptr(logits), gbs, V, k, flags, _ptr(vals), _ptr(idx), _ptr(taps),
              _ptr(ws), ws.numel(), _stream(dev))
    else:
        _call("tail_topk", _ptr(logits), gbs, V, k, _ptr(vals), _ptr(idx), _ptr(ws), ws.numel(),
              _stream(dev))
    return vals, idx


def sample(vals, idx, params, out=None):
    """tail_sample: tokens [gbs] int32 from [gbs,3|4] params."""
    torch = _torch()
    dev = _dev(vals)
    gbs, k = vals.shape
    tokens = out if out is not None else torch.empty((gbs,), dtype=torch.int32, device=dev)
    _call("tail_sample", _ptr(vals), _ptr(idx), gbs, k, _ptr(params), params.shape[1], _ptr(tokens),
          _stream(dev))
    return tokens


class Forward:
    """Preallocated outputs and workspace for repeated tail_forward calls on
    fixed shapes (what a decode loop or a benchmark wants)."""

    def __init__(self, gbs, H, V, k=256, H_u=None, eps=1e-5, zero_pad=False, deferred=True,
                 emit_logits=True, device="cuda", page=False, nan_fold=False):
        torch = _torch()
        self.gbs, self.H, self.V, self.k = gbs, H, V, k
        self.H_u = H if H_u is None else H_u
        self.eps = eps
        self.flags = _flags(zero_pad, deferred, emit_logits, page, nan_fold)
        self.device = torch.device(device)
        dev = self.device
        self.logits = torch.empty((gbs, V), dtype=torch.float32, device=dev) if emit_logits else None
        self.vals = torch.empty((gbs, k), dtype=torch.float32, device=dev)
        self.idx = torch.empty((gbs, k), dtype=torch.int32, device=dev)
        self.tokens = torch.empty((gbs,), dtype=torch.int32, device=dev)
        n = workspace_size(gbs, H, self.H_u, V, k, self.flags)
        if n == 0:
            raise TailError("tail_workspace_size", ERR_INVALID_ARG)
        self.ws = torch.empty(n, dtype=torch.uint8, device=dev)

    def __call__(self, hidden, gamma, w_t, params=None):
        _dev(hidden)
        _call("tail_forward", _ptr(hidden), _hidden_dtype(hidden), _ptr(gamma), _ptr(_weight(w_t)),
              self.gbs, self.H, self.H_u, self.V, self.k, self.eps, self.flags, _ptr(params),
              0 if params is None else params.shape[1], _ptr(self.logits), _ptr(self.vals),
              _ptr(self.idx), _ptr(self.tokens if params is not None else None), _ptr(self.ws),
              self.ws.numel(), _stream(self.device))
        return dict(logits=self.logits, vals=self.vals, idx=self.idx,
                    tokens=self.tokens if params is not None else None)


def forward(hidden, gamma, w_t, k=256, H_u=None, eps=1e-5, zero_pad=False, deferred=True,
            emit_logits=True, params=None, page=False):
    """tail_forward with freshly allocated outputs; returns a dict of tensors."""
    gbs, H = hidden.shape
    f = Forward(gbs, H, w_t.shape[1], k, H_u, eps, zero_pad, deferred, emit_logits, hidden.device,
                page)
    return f(hidden, gamma, w_t, params)
