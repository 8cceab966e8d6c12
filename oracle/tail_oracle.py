"""Plain fp64 CPU oracle of the GPT-OSS decode sampling tail.

TEST INFRASTRUCTURE.  Only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module; the
product path (the HIP library and its Python binding) never does, and it
shares no code, constant or helper with it.

What it computes, and where it comes from (page: "GPT-OSS Tail Chunked
Megakernel Kernel API Reference", NKI library docs; named by the parameter
whose paragraph states the fact):

1. widen    -- ``hidden_states``: fp32 / fp16 / bf16 rows, a 16-bit input
               widened exactly.
2. pad      -- ``zero_interleaved_pad`` and ``hidden_actual``: interleaved pad
               lanes of a padded hidden are excluded.
3. rmsnorm  -- ``gamma``, ``eps``, ``hidden_actual``, ``deferred_rms``:
               y = x * rsqrt(mean(x^2) + eps) * gamma, mean over H_u lanes.
4. logits   -- ``lm_head_weight_t``: y @ W with the [H, V] bf16 weight.
5. topk     -- ``k`` and the Background section (global top-k over the full
               vocabulary): the k largest logits, descending.
6. sample   -- ``sampling_params``: per-row [top_k, top_p, temperature, (u)],
               u defaulting to the compiled-in deterministic draw 0.5; the
               greedy sampler of the GK decode design doc (argmax) is the
               temperature-0 case.

Every step is the plain definition evaluated in float64 with numpy; there is
no blocking, fusion or reordering beyond chunking the matmul over V so the
fp64 copy of the weight never exists whole.  Readings taken where the page is
silent (each also listed in the design notes):

* mean divisor is H_u (the reason ``hidden_actual`` exists);
* eps is added to the mean square inside the square root;
* a pad lane is the last lane of every group of s = H/(H-H_u) lanes;
* with pad zeroing off, all H lanes are used (the caller guarantees zeros);
* the GEMM input is NOT rounded to bf16 (full-precision activations);
* top-k runs on the logits themselves; ties go to the lower index and
  -0.0 equals +0.0; infinities order as numbers; NaN is an error unless the
  stage-1 fold (``skip_nan_fold`` off) turns it into -inf;
* page precision (optional, ``page=True`` in ``tail``): the page's own
  numerics, from ``deferred_rms`` (one bf16 rounding of the GEMM input per
  element), ``skip_nan_fold`` (bf16 products summed at full width) and
  ``emit_logits`` (the top-k sees the bf16 mirror of the fp32 logits).  The
  rounded activation is computed in float32, as the device computes it, so
  both sides take the same rounding decisions;
* sampler: top-k cut first, then a softmax at T over the kept kk
  candidates, then the nucleus (smallest prefix whose mass is >= top_p of
  the kept mass), then the inverse CDF at u in candidate order (candidate i
  owns [Q_{i-1}, Q_i)); T <= 0 is greedy; top_k outside [1, k] means k;
  u < 0 acts as 0 and u >= 1 picks the last nucleus member.

Every function here is pinned by the CPU tests against brute force, 50-digit
decimal arithmetic, closed forms and invariants; none is parity-unpinned.
"""
from __future__ import annotations

import math

import numpy as np

F32, F16, BF16 = 0, 1, 2  # storage dtype codes of the hidden rows
DETERMINISTIC_DRAW = 0.5  # u when sampling_params has 3 columns


# ------------------------------------------------------------------ 1. widen
def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float64 (exact: a bf16 is the top half of a float32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):  # NaN payloads convert as NaN
        return b.view(np.float32).astype(np.float64)


def widen(hidden: np.ndarray, dtype: int) -> np.ndarray:
    """hidden_states -> float64.  fp16 and bf16 are subsets of fp32 and fp64,
    so this is exact for every dtype."""
    if dtype == F32:
        return np.asarray(hidden, dtype=np.float32).astype(np.float64)
    if dtype == F16:
        return np.asarray(hidden, dtype=np.float16).astype(np.float64)
    if dtype == BF16:
        return bf16_bits_to_f64(hidden)
    raise ValueError(f"unknown dtype {dtype}")


# -------------------------------------------------------------------- 2. pad
def pad_mask(H: int, H_u: int, zero_pad: bool) -> np.ndarray:
    """True on the interleaved pad lanes (zero_interleaved_pad, hidden_actual)."""
    mask = np.zeros(H, dtype=bool)
    if zero_pad and H > H_u:
        if H % (H - H_u) != 0:
            raise ValueError("pad lanes must divide H evenly")
        s = H // (H - H_u)
        mask[s - 1::s] = True
    return mask


# ---------------------------------------------------------------- 3. rmsnorm
def rmsnorm(x: np.ndarray, gamma: np.ndarray, H_u: int, eps: float,
            pad: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Final RMSNorm (gamma, eps, hidden_actual).

    ms_b = sum_{h not pad} x_bh^2 / H_u ; r_b = 1/sqrt(ms_b + eps) ;
    y_bh = x_bh * r_b * gamma_h on real lanes, 0 on pad lanes.
    Returns (y [gbs, H] float64, r [gbs] float64)."""
    x = np.array(x, dtype=np.float64)
    g = np.array(gamma, dtype=np.float64).reshape(-1)
    real = ~pad
    xr = x[:, real]
    ms = np.sum(xr * xr, axis=1) / float(H_u)
    r = 1.0 / np.sqrt(ms + float(eps))
    y = np.zeros_like(x)
    y[:, real] = xr * r[:, None] * g[real][None, :]
    return y, r


# ----------------------------------------------------------------- 4. logits
def logits(y: np.ndarray, w_bits: np.ndarray, pad: np.ndarray, chunk: int = 8192) -> np.ndarray:
    """lm_head: L[b, v] = sum_{h not pad} y[b, h] * W[h, v], in float64.
    W is the [H, V] bf16 weight (raw bits); pad rows are never read."""
    real = np.nonzero(~pad)[0]
    yr = np.ascontiguousarray(y[:, real], dtype=np.float64)
    V = w_bits.shape[1]
    out = np.empty((y.shape[0], V), dtype=np.float64)
    for v0 in range(0, V, chunk):
        v1 = min(V, v0 + chunk)
        wc = bf16_bits_to_f64(w_bits[real, v0:v1])
        out[:, v0:v1] = yr @ wc
    return out


# ------------------------------------------------------------------- 5. topk
def topk(L: np.ndarray, k: int, nan_fold: bool = False) -> tuple[np.ndarray, np.ndarray]:
    """Per row, the k largest values, descending; equal values in ascending
    index order (a full stable sort).  Infinities order as numbers (the page,
    ``skip_nan_fold``: an overflow saturates to +/-inf, which the top-k orders
    fine).  NaN has no place in that order: it is an error, unless nan_fold,
    the stage-1 fold that ``skip_nan_fold`` = False keeps, replaces it by -inf
    (value and rank).  Returns (vals float64 [gbs,k], idx int64 [gbs,k])."""
    L = np.asarray(L, dtype=np.float64)
    if nan_fold:
        L = np.where(np.isnan(L), -np.inf, L)
    if np.any(np.isnan(L)):
        raise ValueError("top-k input must not hold NaN (unless folded)")
    order = np.argsort(-L, axis=1, kind="stable")[:, :k]
    return np.take_along_axis(L, order, axis=1), order.astype(np.int64)


# ---------------------------------------------------------------- 6. sample
def sample_row(vals: np.ndarray, idx: np.ndarray, top_k: float, top_p: float,
               temperature: float, u: float) -> tuple[int, dict]:
    """One row of the sampler over the k candidates (descending order).

    Returns (token, diag).  diag holds kk, m (nucleus size), C (cumulative
    mass over the kk kept candidates, normalized to 1), Q (the CDF over the
    nucleus, normalized to 1) and `greedy`."""
    vals = np.asarray(vals, dtype=np.float64)
    k = vals.shape[0]
    top_k, top_p, T, u = float(top_k), float(top_p), float(temperature), float(u)
    kk = int(top_k) if math.isfinite(top_k) else 0
    if kk < 1 or kk > k:
        kk = k
    if not (T > 0.0):
        return int(idx[0]), dict(kk=kk, m=1, C=None, Q=None, greedy=True)
    e = np.exp((vals[:kk] - vals[0]) / T)
    S = np.cumsum(e)
    total = S[kk - 1]
    hit = np.nonzero(S >= top_p * total)[0]
    m = int(hit[0]) + 1 if hit.size else kk
    mass = S[m - 1]
    above = np.nonzero(S[:m] > u * mass)[0]
    j = int(above[0]) if above.size else m - 1
    return int(idx[j]), dict(kk=kk, m=m, C=S / total, Q=S[:m] / mass, greedy=False)


def sample(vals: np.ndarray, idx: np.ndarray, params: np.ndarray) -> tuple[np.ndarray, list]:
    """sampling_params [gbs, 3|4] -> tokens [gbs] int64 (plus per-row diag)."""
    params = np.asarray(params, dtype=np.float32).astype(np.float64)
    ncols = params.shape[1]
    if ncols not in (3, 4):
        raise ValueError("sampling_params must have 3 or 4 columns")
    toks, diags = [], []
    for b in range(vals.shape[0]):
        u = params[b, 3] if ncols == 4 else DETERMINISTIC_DRAW
        t, d = sample_row(vals[b], idx[b], params[b, 0], params[b, 1], params[b, 2], u)
        toks.append(t)
        diags.append(d)
    return np.array(toks, dtype=np.int64), diags


# ------------------------------------------------------- 7. page precision
def bf16_round(a: np.ndarray) -> np.ndarray:
    """float32 values -> the nearest bfloat16 value, ties to the even one,
    returned as float64.  A bf16 keeps the top 16 bits of a float32, so this
    rounds the low 16 bits away: add 0x7FFF plus the lowest kept bit and
    truncate.  NaN stays NaN."""
    f = np.ascontiguousarray(a, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    out = (r & 0xFFFFFFFF).astype(np.uint32).view(np.float32).astype(np.float64)
    return np.where(np.isnan(f), np.nan, out)


def rmsnorm_page(x: np.ndarray, gamma: np.ndarray, H_u: int, eps: float, pad: np.ndarray,
                 deferred: bool = True) -> tuple[np.ndarray, np.ndarray]:
    """The GEMM input at the page's precision (``deferred_rms``: one bf16
    rounding per element; ``gamma``, ``eps``, ``hidden_actual``).

    r = fp32(1 / sqrt(ms + eps)) with ms the float64 mean square over the
    real lanes.  Deferred: a = bf16(fp32(x * gamma)) and the row is scaled
    by r after the contraction.  In-chain: a = bf16(fp32(fp32(x * r) *
    gamma)) and the scale is 1.  Products are float32 (IEEE, nearest even),
    as the device forms them.  Returns (a [gbs, H] float64, exact bf16
    values, 0 on pad lanes; scale [gbs] float64)."""
    x = np.array(x, dtype=np.float64)
    g = np.asarray(gamma, dtype=np.float32).reshape(-1)
    real = ~pad
    xr = x[:, real]
    ms = np.sum(xr * xr, axis=1) / float(H_u)
    r32 = (1.0 / np.sqrt(ms + float(eps))).astype(np.float32)
    x32 = xr.astype(np.float32)
    if deferred:
        y32 = x32 * g[real][None, :]
        scale = r32.astype(np.float64)
    else:
        y32 = (x32 * r32[:, None]) * g[real][None, :]
        scale = np.ones(x.shape[0])
    a = np.zeros_like(x)
    a[:, real] = bf16_round(y32)
    return a, scale


def mirror(L: np.ndarray) -> np.ndarray:
    """The bf16 mirror of the fp32 logits (``emit_logits``: what the page's
    top-k ranks): bf16(fp32(L)), as float64."""
    return bf16_round(np.asarray(L, dtype=np.float64).astype(np.float32))


# ------------------------------------------------------------------ the tail
def tail(hidden, dtype, gamma, w_bits, H_u, k, eps=1e-5, zero_pad=True, params=None,
         rows=None, page=False, deferred=True):
    """The whole tail for every row (or only `rows`, which the oracle may do
    because rows are independent).  Returns a dict with y, r, logits, vals,
    idx and, when params is given, tokens and diag.  With page=True the
    GEMM input is the page-precision activation (``deferred`` picks its
    realization), y holds it, and the top-k ranks the bf16 mirror (vals are
    mirror values)."""
    H = hidden.shape[1]
    pad = pad_mask(H, H_u, zero_pad)
    x = widen(hidden, dtype)
    if rows is not None:
        x = x[rows]
        params = None if params is None else np.asarray(params)[rows]
    if page:
        y, scale = rmsnorm_page(x, gamma, H_u, eps, pad, deferred)
        r = rmsnorm(x, gamma, H_u, eps, pad)[1]
        L = logits(y, w_bits, pad) * scale[:, None]
        vals, idx = topk(mirror(L), k)
    else:
        y, r = rmsnorm(x, gamma, H_u, eps, pad)
        L = logits(y, w_bits, pad)
        vals, idx = topk(L, k)
    out = dict(y=y, r=r, logits=L, vals=vals, idx=idx)
    if params is not None:
        out["tokens"], out["diag"] = sample(vals, idx, params)
    return out
