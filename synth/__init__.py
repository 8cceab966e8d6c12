"""Seeded synthetic inputs for the decode sampling tail.

This module only draws random numbers and rounds them to the storage type of
each input (float32, float16, bfloat16 bits).  It holds none of the tail's
arithmetic, and both the oracle's callers and the GPU path's callers take
their inputs from it.

The draws come from the counter-based Philox4x32-10 generator in
``philox.c`` (built on first use with the host C compiler).  Each tensor has
its own (seed, stream) pair, so a tensor never depends on the size or the
order of other draws.

The five workloads follow the shapes and distributions of the GPT-OSS tail
(gpt_oss_tail_chunked_megakernel API page, parameters ``hidden_states``,
``gamma``, ``lm_head_weight_t``, ``hidden_actual``, ``zero_interleaved_pad``,
``k``, ``sampling_params``):

* 0 — tiny: gbs 1, H 256, V 4096, k 16, fp32 hidden; params (8, 0.9, 0.7, 0.5).
* 1 — GPT-OSS shaped: gbs 1, H 2880, V 201088, k 256, bf16 hidden with 1 %
  outliers x20; a greedy run and a T = 1 run.
* 2 — gbs 8, fp32 hidden, random per-row sampling parameters.
* 3 — gbs 64, H 3072 with H_u 2880 and 192 interleaved pad lanes (every
  16th lane), fp16 hidden; exact logit ties are planted afterwards with
  :func:`duplicate_columns` (the choice of columns needs logits, so it lives
  with the callers).
* 4 — gbs 256, fp32 hidden N(0, 2) times a per-row scale U[0.1, 10];
  64 rows at temperature 0.

Configs 1-4 share one bf16 lm_head weight N(0, 0.02) [2880, 201088]
(config 3 inserts its zero pad rows into that same weight).
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "philox.c")
_LIB_PATH = os.path.join(_HERE, "_libsynth.so")
_lib = None
_lock = threading.Lock()

# stream tags: one per drawn tensor
S_HIDDEN, S_GAMMA, S_WEIGHT = 1, 2, 3
S_TOPK, S_TOPP, S_TEMP, S_U = 4, 5, 6, 7
S_OUTLIER, S_ROWSCALE, S_GREEDY, S_TIETARGET = 8, 9, 10, 11

WEIGHT_SEED = 1  # the shared GPT-OSS-shaped lm_head weight


def build_lib(force: bool = False) -> str:
    """Compile philox.c into _libsynth.so with gcc (OpenMP)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + f".tmp{os.getpid()}"
        subprocess.run(["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-o", tmp, _SRC, "-lm"],
                       check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build_lib()
            lib = ctypes.CDLL(_LIB_PATH)
            u64, u32, sz, dbl = ctypes.c_uint64, ctypes.c_uint32, ctypes.c_size_t, ctypes.c_double
            vp = ctypes.c_void_p
            lib.synth_normal_f32.argtypes = [u64, u32, u64, sz, dbl, dbl, vp]
            lib.synth_normal_bf16.argtypes = [u64, u32, u64, sz, dbl, dbl, vp]
            lib.synth_uniform_f64.argtypes = [u64, u32, u64, sz, vp]
            lib.synth_uniform_f32.argtypes = [u64, u32, u64, sz, vp]
            lib.synth_philox_block.argtypes = [vp, vp, vp]
            lib.synth_round_bf16.argtypes = [vp, sz, vp]
            for f in (lib.synth_normal_f32, lib.synth_normal_bf16, lib.synth_uniform_f64,
                      lib.synth_uniform_f32, lib.synth_philox_block, lib.synth_round_bf16):
                f.restype = None
            _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


# ---------------------------------------------------------------- primitives
def philox_block(ctr, key) -> np.ndarray:
    c = np.ascontiguousarray(ctr, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.zeros(4, np.uint32)
    _load().synth_philox_block(_ptr(c), _ptr(k), _ptr(out))
    return out


def normal_f32(seed: int, stream: int, n: int, mean: float = 0.0, std: float = 1.0,
               offset: int = 0) -> np.ndarray:
    out = np.empty(n, np.float32)
    _load().synth_normal_f32(seed, stream, offset, n, mean, std, _ptr(out))
    return out


def normal_bf16(seed: int, stream: int, n: int, mean: float = 0.0, std: float = 1.0,
                offset: int = 0) -> np.ndarray:
    """Raw bfloat16 bits (uint16) of bf16_rne(float32(mean + std*z))."""
    out = np.empty(n, np.uint16)
    _load().synth_normal_bf16(seed, stream, offset, n, mean, std, _ptr(out))
    return out


def uniform_f64(seed: int, stream: int, n: int, offset: int = 0) -> np.ndarray:
    out = np.empty(n, np.float64)
    _load().synth_uniform_f64(seed, stream, offset, n, _ptr(out))
    return out


def uniform_f32(seed: int, stream: int, n: int, offset: int = 0) -> np.ndarray:
    """Uniform on [0, 1) on a 2^-24 grid (every value exact in float32, never 1.0)."""
    out = np.empty(n, np.float32)
    _load().synth_uniform_f32(seed, stream, offset, n, _ptr(out))
    return out


def round_bf16(x: np.ndarray) -> np.ndarray:
    """bfloat16 round-to-nearest-even of a float32 array, as raw uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint16)
    _load().synth_round_bf16(_ptr(x), x.size, _ptr(out))
    return out


# ------------------------------------------------------------------- configs
DT_F32, DT_F16, DT_BF16 = 0, 1, 2  # storage dtype codes of the hidden rows


@dataclasses.dataclass
class TailInputs:
    """One workload: every array is host memory in its storage dtype."""
    name: str
    gbs: int
    H: int
    H_u: int
    V: int
    k: int
    eps: float
    zero_pad: bool
    dtype: int              # DT_F32 / DT_F16 / DT_BF16
    hidden: np.ndarray      # [gbs, H]: float32, float16, or uint16 bf16 bits
    gamma: np.ndarray       # [H] float32
    w_t: np.ndarray         # [H, V] uint16 bf16 bits, C-contiguous
    params: list            # list of [gbs, 4] float32 (top_k, top_p, T, u); one per run

    @property
    def pad_stride(self) -> int:
        return self.H // (self.H - self.H_u) if self.H > self.H_u else 0


CONFIG_SHAPES = {
    0: dict(gbs=1, H=256, H_u=256, V=4096, k=16),
    1: dict(gbs=1, H=2880, H_u=2880, V=201088, k=256),
    2: dict(gbs=8, H=2880, H_u=2880, V=201088, k=256),
    3: dict(gbs=64, H=3072, H_u=2880, V=201088, k=256),
    4: dict(gbs=256, H=2880, H_u=2880, V=201088, k=256),
}

_weight_cache: dict = {}


def gptoss_weight(H_u: int = 2880, V: int = 201088) -> np.ndarray:
    """The shared bf16 lm_head weight N(0, 0.02), [H_u, V] (cached)."""
    key = (H_u, V)
    if key not in _weight_cache:
        _weight_cache[key] = normal_bf16(WEIGHT_SEED, S_WEIGHT, H_u * V, 0.0, 0.02).reshape(H_u, V)
    return _weight_cache[key]


def clear_cache():
    _weight_cache.clear()


def pad_lanes(H: int, H_u: int) -> np.ndarray:
    """Indices of the interleaved pad lanes: the last lane of every group of
    s = H/(H-H_u) lanes (h % s == s-1)."""
    if H == H_u:
        return np.zeros(0, np.int64)
    s = H // (H - H_u)
    return np.arange(s - 1, H, s, dtype=np.int64)


def random_params(seed: int, gbs: int, greedy_rows: int = 0) -> np.ndarray:
    """Per-row [top_k, top_p, T, u]: top_k uniform on {1..256}, top_p U[0.5, 1],
    T U[0.3, 1.5], u U[0, 1); `greedy_rows` rows (the smallest of a seeded
    uniform key) get T = 0."""
    p = np.empty((gbs, 4), np.float32)
    p[:, 0] = np.floor(uniform_f32(seed, S_TOPK, gbs) * np.float32(256.0)) + np.float32(1.0)
    p[:, 1] = np.float32(0.5) + np.float32(0.5) * uniform_f32(seed, S_TOPP, gbs)
    p[:, 2] = np.float32(0.3) + np.float32(1.2) * uniform_f32(seed, S_TEMP, gbs)
    p[:, 3] = uniform_f32(seed, S_U, gbs)
    if greedy_rows:
        key = uniform_f64(seed, S_GREEDY, gbs)
        rows = np.argsort(key, kind="stable")[:greedy_rows]
        p[rows, 2] = 0.0
    return p


def make_config(cid: int, seed: int | None = None) -> TailInputs:
    """Workload `cid`; `seed` (default: cid) draws its hidden rows, gamma and
    sampling parameters (the weight has its own fixed seed)."""
    inp = _make_config(cid, cid if seed is None else seed)
    if seed is not None and seed != cid:
        inp.name = f"{inp.name}_seed{seed}"
    return inp


def _make_config(cid: int, seed: int) -> TailInputs:
    s = CONFIG_SHAPES[cid]
    gbs, H, H_u, V, k = s["gbs"], s["H"], s["H_u"], s["V"], s["k"]
    if cid == 0:
        hidden = normal_f32(seed, S_HIDDEN, gbs * H).reshape(gbs, H)
        gamma = normal_f32(seed, S_GAMMA, H, 1.0, 0.1)
        w = normal_bf16(seed, S_WEIGHT, H * V, 0.0, 0.05).reshape(H, V)
        params = [np.array([[8.0, 0.9, 0.7, 0.5]], np.float32)]
        return TailInputs("tiny", gbs, H, H_u, V, k, 1e-5, False, DT_F32, hidden, gamma, w, params)
    gamma = normal_f32(seed, S_GAMMA, H, 1.0, 0.1)
    if cid == 1:
        z = normal_f32(seed, S_HIDDEN, gbs * H)
        out = uniform_f64(seed, S_OUTLIER, gbs * H) < 0.01
        z = np.where(out, z * np.float32(20.0), z).astype(np.float32)
        hidden = round_bf16(z).reshape(gbs, H)
        params = [np.array([[256.0, 1.0, 0.0, 0.5]], np.float32),
                  np.array([[256.0, 1.0, 1.0, 0.5]], np.float32)]
        return TailInputs("gptoss_gbs1", gbs, H, H_u, V, k, 1e-5, False, DT_BF16,
                          hidden, gamma, gptoss_weight(H_u, V), params)
    if cid == 2:
        hidden = normal_f32(seed, S_HIDDEN, gbs * H).reshape(gbs, H)
        return TailInputs("gbs8_sampling", gbs, H, H_u, V, k, 1e-5, False, DT_F32,
                          hidden, gamma, gptoss_weight(H_u, V), [random_params(seed, gbs)])
    if cid == 3:
        pads = pad_lanes(H, H_u)
        hidden = normal_f32(seed, S_HIDDEN, gbs * H).astype(np.float16).reshape(gbs, H)
        hidden[:, pads] = 0
        gamma[pads] = 0
        real = np.setdiff1d(np.arange(H), pads)
        w = np.zeros((H, V), np.uint16)
        w[real] = gptoss_weight(H_u, V)
        return TailInputs("gbs64_pad_ties", gbs, H, H_u, V, k, 1e-5, True, DT_F16,
                          hidden, gamma, w, [random_params(seed, gbs)])
    if cid == 4:
        z = normal_f32(seed, S_HIDDEN, gbs * H, 0.0, 2.0).reshape(gbs, H)
        scale = np.float32(0.1) + np.float32(9.9) * uniform_f32(seed, S_ROWSCALE, gbs)
        hidden = (z * scale[:, None]).astype(np.float32)
        return TailInputs("gbs256_dense", gbs, H, H_u, V, k, 1e-5, False, DT_F32,
                          hidden, gamma, gptoss_weight(H_u, V),
                          [random_params(seed, gbs, greedy_rows=gbs // 4)])
    raise ValueError(cid)


def tie_targets(seed: int, candidates: np.ndarray, n: int) -> np.ndarray:
    """n distinct columns drawn from `candidates` with a seeded uniform key."""
    key = uniform_f64(seed, S_TIETARGET, candidates.size)
    return candidates[np.argsort(key, kind="stable")[:n]]


def duplicate_columns(w_t: np.ndarray, sources: np.ndarray, targets: np.ndarray) -> None:
    """In place: column targets[i] of the weight becomes a copy of sources[i]."""
    w_t[:, targets] = w_t[:, sources]
