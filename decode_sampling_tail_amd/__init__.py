"""Python binding of the decode-tail HIP library (libtail.so).

Argument marshalling only: every step of the tail runs in the library's HIP
kernels.  Tensors must be contiguous CUDA (HIP) tensors on one device, of the
dtypes and shapes each call documents; every tensor argument (inputs,
outputs and workspace) is checked before the call and a mismatch raises
ValueError, so no kernel is handed a pointer of the wrong kind.  The calls
enqueue on torch's current stream of that device and never synchronize.  There is no CPU fallback: if the library is not built, loading
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

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP, ERR_SCRATCH_LIMIT = 0, 1, 2, 3, 4, 5
SCRATCH_BYTES = 64 << 20  # the static scratch of tail_forward_noalloc
F32, F16, BF16 = 0, 1, 2
EMIT_LOGITS, ZERO_PAD, DEFERRED_RMS, PAGE_PRECISION, NAN_FOLD = 1, 2, 4, 8, 16
K_MAX, GBS_MAX, H_MAX = 1024, 4096, 65536

EXPORTS = ("tail_rmsnorm", "tail_lm_head", "tail_rmsnorm_lm_head", "tail_topk", "tail_topk_ex",
           "tail_sample", "tail_forward", "tail_forward_noalloc", "tail_workspace_size",
           "tail_status_string")

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
        L.tail_forward_noalloc.argtypes = [vp, i, vp, vp, i, i, i, i, i, f, u, vp, i, vp, vp, vp, vp, vp]
        L.tail_workspace_size.argtypes = [i, i, i, i, i, u]
        L.tail_workspace_size.restype = sz
        L.tail_status_string.argtypes = [i]
        L.tail_status_string.restype = ctypes.c_char_p
        for name in ("tail_rmsnorm", "tail_lm_head", "tail_rmsnorm_lm_head", "tail_topk",
                     "tail_topk_ex", "tail_sample", "tail_forward", "tail_forward_noalloc"):
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


def _dev(t, name="tensor"):
    """The device of a tensor argument that must live on a GPU, contiguous."""
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (got one on {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.device


def _check(t, name, dev, dtypes, shape=None, optional=False):
    """Validate one tensor argument before any launch: on `dev`, contiguous,
    one of `dtypes`, and of `shape` (None entries match any size).  A tensor
    on another device, of another dtype or shape would hand the kernels a
    pointer to memory of another kind or size."""
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    d = _dev(t, name)
    if d != dev:
        raise ValueError(f"{name} is on {d}, the call's tensors are on {dev}")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}; expected one of {tuple(dtypes)}")
    if shape is not None:
        if t.dim() != len(shape) or any(e is not None and int(n) != int(e)
                                        for n, e in zip(t.shape, shape)):
            raise ValueError(f"{name} has shape {tuple(t.shape)}; expected "
                             f"{tuple('*' if e is None else e for e in shape)}")
    return t


def _f32():
    return (_torch().float32,)


def _i32():
    return (_torch().int32,)


def _u8():
    return (_torch().uint8,)


def _bf16_bits():
    torch = _torch()
    return (torch.bfloat16, torch.int16, torch.uint16)


def _hidden_dtypes():
    torch = _torch()
    return (torch.float32, torch.float16, torch.bfloat16, torch.int16, torch.uint16)


def _check_2d(t, name):
    _dev(t, name)
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D (got shape {tuple(t.shape)})")
    return t.shape


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
    gbs, H = _check_2d(hidden, "hidden")
    dev = _check(hidden, "hidden", hidden.device, _hidden_dtypes()).device
    _check(gamma, "gamma", dev, _f32(), (H,))
    H_u = H if H_u is None else H_u
    y = out_y if out_y is not None else torch.empty((gbs, H), dtype=torch.float32, device=dev)
    r = out_r if out_r is not None else torch.empty((gbs,), dtype=torch.float32, device=dev)
    _check(y, "out_y", dev, _f32(), (gbs, H))
    _check(r, "out_r", dev, _f32(), (gbs,))
    _call("tail_rmsnorm", _ptr(hidden), _hidden_dtype(hidden), _ptr(gamma), gbs, H, H_u, eps,
          _flags(zero_pad, deferred, page=page), _ptr(y), _ptr(r), _stream(dev))
    return y, r


def lm_head(y, w_t, H_u=None, zero_pad=False, row_scale=None, out=None, ws=None, page=False):
    """tail_lm_head: logits [gbs,V] fp32 = row_scale * (y @ W)."""
    torch = _torch()
    gbs, H = _check_2d(y, "y")
    dev = _check(y, "y", y.device, _f32()).device
    _, V = _check_2d(w_t, "w_t")
    _check(w_t, "w_t", dev, _bf16_bits(), (H, V))
    _check(row_scale, "row_scale", dev, _f32(), (gbs,), optional=True)
    H_u = H if H_u is None else H_u
    logits = out if out is not None else torch.empty((gbs, V), dtype=torch.float32, device=dev)
    _check(logits, "out", dev, _f32(), (gbs, V))
    if ws is None:
        n = workspace_size(gbs, H, H_u, V, 1, _flags(zero_pad, emit=True, page=page))
        ws = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
    _check(ws, "ws", dev, _u8(), (None,))
    _call("tail_lm_head", _ptr(y), _ptr(w_t), _ptr(row_scale), gbs, H, H_u, V,
          _flags(zero_pad, page=page), _ptr(logits), _ptr(ws), ws.numel(), _stream(dev))
    return logits


def rmsnorm_lm_head(hidden, gamma, w_t, H_u=None, eps=1e-5, zero_pad=False, deferred=True, out=None,
                    out_r=None, ws=None, page=False):
    """tail_rmsnorm_lm_head: (logits [gbs,V] fp32, r [gbs] fp32)."""
    torch = _torch()
    gbs, H = _check_2d(hidden, "hidden")
    dev = _check(hidden, "hidden", hidden.device, _hidden_dtypes()).device
    _check(gamma, "gamma", dev, _f32(), (H,))
    _, V = _check_2d(w_t, "w_t")
    _check(w_t, "w_t", dev, _bf16_bits(), (H, V))
    H_u = H if H_u is None else H_u
    flags = _flags(zero_pad, deferred, page=page)
    logits = out if out is not None else torch.empty((gbs, V), dtype=torch.float32, device=dev)
    r = out_r if out_r is not None else torch.empty((gbs,), dtype=torch.float32, device=dev)
    _check(logits, "out", dev, _f32(), (gbs, V))
    _check(r, "out_r", dev, _f32(), (gbs,))
    if ws is None:
        n = workspace_size(gbs, H, H_u, V, 1, flags | EMIT_LOGITS)
        ws = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
    _check(ws, "ws", dev, _u8(), (None,))
    _call("tail_rmsnorm_lm_head", _ptr(hidden), _hidden_dtype(hidden), _ptr(gamma), _ptr(w_t),
          gbs, H, H_u, V, eps, flags, _ptr(logits), _ptr(r), _ptr(ws), ws.numel(), _stream(dev))
    return logits, r


def topk(logits, k, out_vals=None, out_idx=None, ws=None, mirror=False, nan_fold=False, taps=None):
    """tail_topk, or tail_topk_ex when mirror (rank the bf16 rounding of the
    logits), nan_fold (NaN ranks as -inf) or taps ([gbs, 4] int32 tensor for
    the stage-1 diagnostics, as raw u32) is given: (vals [gbs,k] fp32
    descending, idx [gbs,k] int32)."""
    torch = _torch()
    gbs, V = _check_2d(logits, "logits")
    dev = _check(logits, "logits", logits.device, _f32()).device
    vals = out_vals if out_vals is not None else torch.empty((gbs, k), dtype=torch.float32, device=dev)
    idx = out_idx if out_idx is not None else torch.empty((gbs, k), dtype=torch.int32, device=dev)
    _check(vals, "out_vals", dev, _f32(), (gbs, k))
    _check(idx, "out_idx", dev, _i32(), (gbs, k))
    _check(taps, "taps", dev, (torch.int32, torch.uint32), (gbs, 4), optional=True)
    if ws is None:
        ws = torch.empty(max(workspace_size(gbs, 1, 1, V, k, EMIT_LOGITS), 1), dtype=torch.uint8, device=dev)
    _check(ws, "ws", dev, _u8(), (None,))
    if mirror or nan_fold or taps is not None:
        flags = (PAGE_PRECISION if mirror else 0) | (NAN_FOLD if nan_fold else 0)
        _call("tail_topk_ex", _ptr(logits), gbs, V, k, flags, _ptr(vals), _ptr(idx), _ptr(taps),
              _ptr(ws), ws.numel(), _stream(dev))
    else:
        _call("tail_topk", _ptr(logits), gbs, V, k, _ptr(vals), _ptr(idx), _ptr(ws), ws.numel(),
              _stream(dev))
    return vals, idx


def _check_params(params, dev, gbs):
    _check_2d(params, "params")
    return _check(params, "params", dev, _f32(), (gbs, None))


def sample(vals, idx, params, out=None):
    """tail_sample: tokens [gbs] int32 from [gbs,3|4] params."""
    torch = _torch()
    gbs, k = _check_2d(vals, "vals")
    dev = _check(vals, "vals", vals.device, _f32()).device
    _check(idx, "idx", dev, _i32(), (gbs, k))
    _check_params(params, dev, gbs)
    tokens = out if out is not None else torch.empty((gbs,), dtype=torch.int32, device=dev)
    _check(tokens, "out", dev, _i32(), (gbs,))
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
        if self.device.type == "cuda" and self.device.index is None:
            self.device = torch.device("cuda", torch.cuda.current_device())
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
        dev = self.device
        _check(hidden, "hidden", dev, _hidden_dtypes(), (self.gbs, self.H))
        _check(gamma, "gamma", dev, _f32(), (self.H,))
        _check(w_t, "w_t", dev, _bf16_bits(), (self.H, self.V))
        if params is not None:
            _check_params(params, dev, self.gbs)
        _call("tail_forward", _ptr(hidden), _hidden_dtype(hidden), _ptr(gamma), _ptr(w_t),
              self.gbs, self.H, self.H_u, self.V, self.k, self.eps, self.flags, _ptr(params),
              0 if params is None else params.shape[1], _ptr(self.logits), _ptr(self.vals),
              _ptr(self.idx), _ptr(self.tokens if params is not None else None), _ptr(self.ws),
              self.ws.numel(), _stream(self.device))
        return dict(logits=self.logits, vals=self.vals, idx=self.idx,
                    tokens=self.tokens if params is not None else None)

    def noalloc(self, hidden, gamma, w_t, params=None):
        """The same call through tail_forward_noalloc: the library's static
        scratch instead of this object's workspace (raises TailError with
        ERR_SCRATCH_LIMIT when the shapes need more than SCRATCH_BYTES)."""
        dev = self.device
        _check(hidden, "hidden", dev, _hidden_dtypes(), (self.gbs, self.H))
        _check(gamma, "gamma", dev, _f32(), (self.H,))
        _check(w_t, "w_t", dev, _bf16_bits(), (self.H, self.V))
        if params is not None:
            _check_params(params, dev, self.gbs)
        _call("tail_forward_noalloc", _ptr(hidden), _hidden_dtype(hidden), _ptr(gamma), _ptr(w_t),
              self.gbs, self.H, self.H_u, self.V, self.k, self.eps, self.flags, _ptr(params),
              0 if params is None else params.shape[1], _ptr(self.logits), _ptr(self.vals),
              _ptr(self.idx), _ptr(self.tokens if params is not None else None),
              _stream(self.device))
        return dict(logits=self.logits, vals=self.vals, idx=self.idx,
                    tokens=self.tokens if params is not None else None)


def forward(hidden, gamma, w_t, k=256, H_u=None, eps=1e-5, zero_pad=False, deferred=True,
            emit_logits=True, params=None, page=False):
    """tail_forward with freshly allocated outputs; returns a dict of tensors."""
    gbs, H = hidden.shape
    f = Forward(gbs, H, w_t.shape[1], k, H_u, eps, zero_pad, deferred, emit_logits, hidden.device,
                page)
    return f(hidden, gamma, w_t, params)
