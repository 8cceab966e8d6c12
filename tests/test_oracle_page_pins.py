"""Pins of the oracle's page-precision mode (GPT-OSS tail API page,
parameters "deferred_rms", "skip_nan_fold" and "emit_logits": the GEMM input
is rounded to bf16 once per element, the products are summed at full width,
and the top-k ranks the bf16 mirror of the fp32 logits).

The expected values come from the definition of round-to-nearest-even
evaluated by exact distance comparison, from torch's own float -> bfloat16
conversion (a library routine), from values worked out by hand, from Python's
own sort, and from the rounding error bound.  Planted mistakes must fail.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import tail_oracle as T


# ------------------------------------------------------------ bf16 rounding
def _bf16_of(bits16: int) -> float:
    """Value of a bf16 magnitude pattern (sign handled by the caller), with
    0x7F80 meaning 2**128 so that it can serve as the upper neighbour of the
    largest finite value."""
    e, m = (bits16 >> 7) & 0xFF, bits16 & 0x7F
    if e == 0:
        return math.ldexp(m, -133)
    return math.ldexp(128 + m, e - 134)


def _rne_reference(f: float) -> float:
    """Nearest bf16 to the float32 value f by comparing the exact distances
    to its two bf16 neighbours; a tie goes to the neighbour whose last
    mantissa bit is 0.  Past the largest finite bf16 the upper neighbour is
    infinity (IEEE overflow under round-to-nearest)."""
    if math.isnan(f):
        return math.nan
    if math.isinf(f):
        return f
    sign = -1.0 if math.copysign(1.0, f) < 0 else 1.0
    a = abs(f)
    bits = int(np.array(a, np.float32).view(np.uint32)) >> 16  # truncated magnitude
    lo, hi = _bf16_of(bits), _bf16_of(bits + 1)
    dlo, dhi = a - lo, hi - a  # exact: all are doubles with few significant bits
    if dlo < dhi or (dlo == dhi and bits % 2 == 0):
        r, rb = lo, bits
    else:
        r, rb = hi, bits + 1
    if rb >= 0x7F80:
        r = math.inf
    return sign * r


def _rne_direct_f64(v: float) -> float:
    """A double rounded straight to 8 significant bits, ties to even (normal
    range only; no intermediate float32)."""
    if v == 0 or not math.isfinite(v):
        return v
    m, e = math.frexp(abs(v))  # abs(v) = m 2^e, m in [0.5, 1)
    q = math.ldexp(m, 8)
    lo = math.floor(q)
    d = q - lo
    n = lo + 1 if d > 0.5 or (d == 0.5 and lo % 2 == 1) else lo
    return math.copysign(math.ldexp(n, e - 8), v)


def _probe_values() -> np.ndarray:
    """float32 values around every bf16: exact, just above, halfway, just past
    halfway, just below the next (both signs, subnormals and the top of the
    range included), plus random ones."""
    b = np.arange(0x7F80, dtype=np.uint32)  # every finite magnitude
    lows = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF], np.uint32)
    u = ((b[:, None] << 16) | lows[None, :]).reshape(-1)
    u = np.concatenate([u, u | 0x80000000])
    rng = np.random.default_rng(11)
    rnd = rng.integers(0, 0x7F800000, 200_000, dtype=np.uint64).astype(np.uint32)
    rnd |= rng.integers(0, 2, rnd.size, dtype=np.uint64).astype(np.uint32) << 31
    return np.concatenate([u, rnd]).view(np.float32)


def check_bf16_round(fn) -> list:
    fails = []
    f = _probe_values()
    got = np.asarray(fn(f), np.float64)
    # (1) the definition, on a stride of the structured probes and every 50th random one
    sel = np.concatenate([np.arange(0, 0x7F80 * 12, 7), np.arange(0x7F80 * 12, f.size, 50)])
    for i in sel:
        want = _rne_reference(float(f[i]))
        if not (got[i] == want and math.copysign(1, got[i]) == math.copysign(1, want)):
            fails.append(f"{float(f[i])!r}: {got[i]!r} vs {want!r}")
            if len(fails) > 5:
                return fails
    # (2) torch's conversion, on all of them
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).to(torch.float64).numpy()
    bad = ~((got == ref) & (np.signbit(got) == np.signbit(ref)))
    if bad.any():
        i = int(np.flatnonzero(bad)[0])
        fails.append(f"vs torch at {float(f[i])!r}: {got[i]!r} vs {ref[i]!r} ({int(bad.sum())} values)")
    # (3) specials
    sp = fn(np.array([np.nan, np.inf, -np.inf, -0.0, 3.4028234663852886e38], np.float32))
    if not (np.isnan(sp[0]) and sp[1] == np.inf and sp[2] == -np.inf and sp[3] == 0
            and np.signbit(sp[3]) and sp[4] == np.inf):
        fails.append(f"specials {sp!r}")
    return fails


def test_bf16_round():
    assert check_bf16_round(oracle.bf16_round) == []


@pytest.mark.parametrize("mistake", ["truncate", "ties_away", "ties_odd"])
def test_bf16_round_planted_mistakes_fail(mistake):
    def bad(a):
        f = np.ascontiguousarray(a, np.float32)
        u = f.view(np.uint32).astype(np.uint64)
        if mistake == "truncate":
            r = (u >> 16) << 16
        elif mistake == "ties_away":
            r = ((u + 0x8000) >> 16) << 16
        else:
            r = ((u + 0x8000 - ((u >> 16) & 1)) >> 16) << 16
        out = (r & 0xFFFFFFFF).astype(np.uint32).view(np.float32).astype(np.float64)
        return np.where(np.isnan(f), np.nan, out)
    assert check_bf16_round(bad)


# -------------------------------------------------------- page activations
def check_rmsnorm_page(fn) -> list:
    fails = []
    nopad = np.zeros(2, bool)
    x = np.array([[3.0, 4.0]])
    g = np.ones(2, np.float32)
    r32 = float(np.float32(1 / math.sqrt(12.5)))
    # deferred: the GEMM input is x * gamma (here exact), the scale is fp32 r
    a, s = fn(x, g, 2, 0.0, nopad, True)
    if not (np.array_equal(a, [[3.0, 4.0]]) and s[0] == r32):
        fails.append(f"deferred hand example {a!r} {s!r}")
    # in-chain: bf16(3 r) = 217/256 (3 r = 0.848528..., 217.22 steps of 2^-8)
    # and bf16(4 r) = 145/128 (4 r = 1.131370..., 144.82 steps of 2^-7)
    a, s = fn(x, g, 2, 0.0, nopad, False)
    if not (np.array_equal(a, [[217 / 256, 145 / 128]]) and s[0] == 1.0):
        fails.append(f"in-chain hand example {a!r} {s!r}")
    # the product is formed in float32 before the bf16 rounding: here the
    # exact product lies just above the bf16 midpoint 1 + 2^-8, its float32
    # rounding lands on the midpoint, and the tie goes to the even 1.0
    x2 = np.array([[1 + 2.0 ** -8 + 2.0 ** -23, 1.0]])
    g2 = np.array([1 - 2.0 ** -24, 1.0], np.float32)
    a, _ = fn(x2, g2, 2, 0.0, nopad, True)
    if a[0, 0] != 1.0:
        fails.append(f"double rounding: {a[0, 0]!r} (want 1.0)")
    # one rounding per element: within half a bf16 ulp of the fp32 value, and
    # the rounding is really taken on generic data
    rng = np.random.default_rng(5)
    H = 97
    x3 = rng.standard_normal((3, H))
    x3 = x3.astype(np.float32).astype(np.float64)
    g3 = (1 + 0.1 * rng.standard_normal(H)).astype(np.float32)
    for deferred in (True, False):
        a, s = fn(x3, g3, H, 1e-5, np.zeros(H, bool), deferred)
        ms = np.sum(x3 * x3, 1) / H
        r = (1 / np.sqrt(ms + 1e-5)).astype(np.float32)
        ex = (x3 * g3) if deferred else (x3.astype(np.float32) * r[:, None]).astype(np.float64) * g3
        if np.any(np.abs(a - ex) > np.abs(ex) * 2.0 ** -8 + 1e-300):
            fails.append("error above one bf16 rounding")
        if np.array_equal(a, ex):
            fails.append("no rounding taken")
        lo16 = np.asarray(a, np.float32).view(np.uint32) & 0xFFFF
        if np.any(lo16):
            fails.append("values not bf16")
    # pad lanes: zero on output, garbage ignored, equal to the compacted row
    H, H_u = 48, 45
    pad = T.pad_mask(H, H_u, True)
    xp = rng.standard_normal((2, H))
    gp = (1 + 0.1 * rng.standard_normal(H)).astype(np.float32)
    ac, sc = fn(xp[:, ~pad], gp[~pad], H_u, 1e-5, np.zeros(H_u, bool), True)
    xg, gg = xp.copy(), gp.copy()
    xg[:, pad] = np.nan
    gg[pad] = np.nan
    ap, sp = fn(xg, gg, H_u, 1e-5, pad, True)
    if not (np.array_equal(ap[:, ~pad], ac) and np.array_equal(sp, sc) and np.all(ap[:, pad] == 0)):
        fails.append("padded != compacted")
    return fails


def test_rmsnorm_page():
    assert check_rmsnorm_page(oracle.rmsnorm_page) == []


@pytest.mark.parametrize("mistake", ["product_in_f64", "scale_before_rounding_when_deferred",
                                     "truncate", "mean_over_H"])
def test_rmsnorm_page_planted_mistakes_fail(mistake):
    def bad(x, gamma, H_u, eps, pad, deferred=True):
        x = np.array(x, np.float64)
        g = np.asarray(gamma, np.float32)
        real = ~pad
        xr = x[:, real]
        div = x.shape[1] if mistake == "mean_over_H" else H_u
        r32 = (1 / np.sqrt(np.sum(xr * xr, 1) / div + eps)).astype(np.float32)
        if mistake == "product_in_f64":
            y = xr * g[real].astype(np.float64) * (1.0 if deferred else r32[:, None])
        elif mistake == "scale_before_rounding_when_deferred":
            y = (xr.astype(np.float32) * r32[:, None]) * g[real]
        elif deferred:
            y = xr.astype(np.float32) * g[real]
        else:
            y = (xr.astype(np.float32) * r32[:, None]) * g[real]
        if mistake == "truncate":
            u = np.asarray(y, np.float32).view(np.uint32) & 0xFFFF0000
            q = u.view(np.float32).astype(np.float64)
        elif mistake == "product_in_f64":  # round the fp64 product directly, to nearest
            q = np.vectorize(_rne_direct_f64)(y)
        else:
            q = T.bf16_round(np.asarray(y, np.float32))
        a = np.zeros_like(x)
        a[:, real] = q
        scale = r32.astype(np.float64) if deferred else np.ones(x.shape[0])
        return a, scale
    assert check_rmsnorm_page(bad)


# ------------------------------------------------------- mirror and top-k
def check_mirror_topk(mirror, topk) -> list:
    """The top-k of the bf16 mirror equals Python's sort of the mirror values
    computed by the RNE definition, ties to the lower index, -0.0 == +0.0."""
    fails = []
    rng = np.random.default_rng(9)
    for trial in range(40):
        V = int(rng.integers(1, 50))
        k = int(rng.integers(1, V + 1))
        base = np.round(rng.standard_normal(V) * 4) / 4
        # distinct fp32 values that collapse onto one bf16 value, exact
        # midpoints, and signed zeros
        jit = rng.integers(-3, 4, V) * 2.0 ** -12 * np.maximum(np.abs(base), 1)
        L = (base + jit).astype(np.float32).astype(np.float64)
        L[rng.integers(0, V)] = 1 + 2.0 ** -8  # midpoint -> 1.0 (even)
        L[rng.integers(0, V)] = -0.0
        L[rng.integers(0, V)] = 2.0 ** -140    # rounds to +0-ish subnormal region
        m = mirror(L[None, :])[0]
        want_vals = [_rne_reference(float(v)) for v in L.astype(np.float32)]
        if not all(float(m[i]) == want_vals[i] for i in range(V)):
            fails.append(f"trial {trial}: mirror values")
            return fails
        vals, idx = topk(m[None, :], k)
        want = sorted(range(V), key=lambda i: (-want_vals[i], i))[:k]
        if list(idx[0]) != want:
            fails.append(f"trial {trial}: order {list(idx[0])} vs {want}")
            return fails
    return fails


def test_mirror_topk():
    assert check_mirror_topk(oracle.mirror, oracle.topk) == []


def test_mirror_topk_planted_no_mirror_fails():
    assert check_mirror_topk(lambda L: np.asarray(L, np.float64), oracle.topk)


# ------------------------------------------------------- page tail as a whole
def test_page_tail_within_rounding_bound_of_exact():
    """Page logits differ from the exact ones by at most the activation
    rounding (2^-8 relative per product, bounded by sum |y w|) plus the fp32
    scale; the difference is really there; the page top-k ranks the mirror of
    the page logits; padded and deferred/in-chain forms agree with that."""
    rng = np.random.default_rng(21)
    gbs, H, H_u, V, k = 3, 64, 60, 300, 17
    hidden = rng.standard_normal((gbs, H)).astype(np.float32)
    gamma = (1 + 0.1 * rng.standard_normal(H)).astype(np.float32)
    w = (0.05 * rng.standard_normal((H, V))).astype(np.float32)
    w_bits = (w.view(np.uint32) >> 16).astype(np.uint16)
    ex = oracle.tail(hidden, T.F32, gamma, w_bits, H_u, k, zero_pad=True)
    pad = T.pad_mask(H, H_u, True)
    wabs = np.abs(T.bf16_bits_to_f64(w_bits))
    wabs[pad] = 0
    for deferred in (True, False):
        pg = oracle.tail(hidden, T.F32, gamma, w_bits, H_u, k, zero_pad=True, page=True,
                         deferred=deferred)
        bound = (np.abs(ex["y"]) @ wabs) * (2.0 ** -8 + 2.0 ** -23) + 1e-12
        d = np.abs(pg["logits"] - ex["logits"])
        assert np.all(d <= bound)
        rel = np.linalg.norm(d) / np.linalg.norm(ex["logits"])
        assert 1e-5 < rel < 1e-2
        mv, mi = oracle.topk(oracle.mirror(pg["logits"]), k)
        assert np.array_equal(pg["idx"], mi) and np.array_equal(pg["vals"], mv)
        assert np.all((np.asarray(pg["vals"], np.float32).view(np.uint32) & 0xFFFF) == 0)


# ------------------------------------------------------------------ NaN fold
def check_nan_fold(topk) -> list:
    """The fold ranks NaN (either sign) as -inf and returns -inf for it;
    infinities order as numbers; brute force by Python's sort."""
    fails = []
    rng = np.random.default_rng(17)
    for trial in range(40):
        V = int(rng.integers(1, 40))
        k = int(rng.integers(1, V + 1))
        L = np.round(rng.standard_normal(V) * 2) / 2
        L[rng.random(V) < 0.2] = np.nan
        L[rng.random(V) < 0.1] = -np.nan
        L[rng.random(V) < 0.1] = np.inf
        L[rng.random(V) < 0.1] = -np.inf
        vals, idx = topk(L[None, :], k, nan_fold=True)
        folded = [(-math.inf if math.isnan(v) else float(v)) for v in L]
        want = sorted(range(V), key=lambda i: (-folded[i], i))[:k]
        if list(idx[0]) != want:
            fails.append(f"trial {trial}: order {list(idx[0])} vs {want}")
            return fails
        if not np.array_equal(vals[0], np.array([folded[i] for i in want])):
            fails.append(f"trial {trial}: values")
    try:
        topk(np.array([[1.0, np.nan]]), 1)
        fails.append("NaN accepted without the fold")
    except ValueError:
        pass
    v, i = topk(np.array([[np.inf, 1.0, -np.inf, 2.0]]), 4)
    if list(i[0]) != [0, 3, 1, 2]:
        fails.append("infinities out of order")
    return fails


def test_nan_fold():
    assert check_nan_fold(oracle.topk) == []


@pytest.mark.parametrize("mistake", ["nan_as_zero", "nan_dropped_last", "nan_kept"])
def test_nan_fold_planted_mistakes_fail(mistake):
    def bad(L, k, nan_fold=False):
        L = np.asarray(L, np.float64)
        if mistake == "nan_as_zero":
            L = np.where(np.isnan(L), 0.0, L)
        elif mistake == "nan_dropped_last":  # below -inf, by index order among themselves
            key = np.where(np.isnan(L), -np.inf, L)
            order = np.lexsort((np.arange(L.shape[1])[None, :].repeat(L.shape[0], 0),
                                np.isnan(L), -key), axis=1)[:, :k]
            return np.take_along_axis(np.where(np.isnan(L), -np.inf, L), order, 1), order
        else:  # NaN kept as a value that ranks first
            key = np.where(np.isnan(L), np.inf, L)
            order = np.argsort(-key, 1, kind="stable")[:, :k]
            return np.take_along_axis(L, order, 1), order
        order = np.argsort(-L, 1, kind="stable")[:, :k]
        return np.take_along_axis(L, order, 1), order
    assert check_nan_fold(bad)
