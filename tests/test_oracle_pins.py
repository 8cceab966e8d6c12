"""Pins of the fp64 oracle against things other than itself.

Each ``check_*`` function takes the implementation under test and returns a
list of failures.  The oracle must pass every check; planted mistakes (wrong
oracles written below, each a plausible slip) must fail at least one.  The
expected values come from brute force (Python's own sort, pure-Python loops),
50-digit ``decimal`` arithmetic, closed forms derived by hand, invariants the
page states, and the page's own constants (tests/golden/page_constants.json).
"""
import json
import math
import os
from decimal import Decimal, getcontext

import numpy as np
import pytest

import oracle
from oracle import tail_oracle as T

getcontext().prec = 50
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------------ widening
def _bf16_value(bits: int) -> float:
    """Decode a bfloat16 from its fields: 1 sign, 8 exponent (bias 127), 7 mantissa."""
    s, e, m = bits >> 15, (bits >> 7) & 0xFF, bits & 0x7F
    sign = -1.0 if s else 1.0
    if e == 0xFF:
        return sign * math.inf if m == 0 else math.nan
    if e == 0:
        return sign * math.ldexp(m, -126 - 7)
    return sign * math.ldexp(128 + m, e - 127 - 7)


def _f16_value(bits: int) -> float:
    """Decode an IEEE half from its fields: 1 sign, 5 exponent (bias 15), 10 mantissa."""
    s, e, m = bits >> 15, (bits >> 10) & 0x1F, bits & 0x3FF
    sign = -1.0 if s else 1.0
    if e == 0x1F:
        return sign * math.inf if m == 0 else math.nan
    if e == 0:
        return sign * math.ldexp(m, -14 - 10)
    return sign * math.ldexp(1024 + m, e - 15 - 10)


def _same(a: float, b: float) -> bool:
    if math.isnan(a) or math.isnan(b):
        return math.isnan(a) and math.isnan(b)
    return a == b and math.copysign(1, a) == math.copysign(1, b)


def check_widen(widen) -> list:
    fails = []
    allbits = np.arange(65536, dtype=np.uint32)
    wb = widen(allbits.astype(np.uint16), T.BF16)
    for b in range(65536):
        if not _same(float(wb[b]), _bf16_value(b)):
            fails.append(f"bf16 {b:#06x}: {wb[b]!r} vs {_bf16_value(b)!r}")
            break
    wh = widen(allbits.astype(np.uint16).view(np.float16), T.F16)
    for b in range(65536):
        if not _same(float(wh[b]), _f16_value(b)):
            fails.append(f"fp16 {b:#06x}: {wh[b]!r} vs {_f16_value(b)!r}")
            break
    f = np.array([1.0, -0.0, 1e-45, -3.4e38, 0.1, 2.0 ** -149, 123.456], np.float32)
    wf = widen(f, T.F32)
    for a, b in zip(wf, f):
        if not _same(float(a), float(b)):
            fails.append(f"fp32 {b!r}")
    return fails


def test_widen_all_16bit_patterns():
    assert check_widen(oracle.widen) == []


def test_widen_planted_flush_to_zero_fails():
    def bad(h, dt):
        out = T.widen(h, dt)
        out[np.abs(out) < 2.0 ** -126] = 0.0  # subnormals flushed
        return out
    assert check_widen(bad)


# ----------------------------------------------------------------- pad lanes
def check_pad_mask(pad_mask) -> list:
    fails = []
    m = pad_mask(3072, 2880, True)
    if m.sum() != 192:
        fails.append(f"count {m.sum()}")
    want = [h for h in range(3072) if (h + 1) % 16 == 0]  # last lane of each group of 16
    if list(np.nonzero(m)[0]) != want:
        fails.append("positions")
    if pad_mask(3072, 2880, False).any() or pad_mask(256, 256, True).any():
        fails.append("mask without padding")
    m2 = pad_mask(12, 9, True)  # s = 4: lanes 3, 7, 11
    if list(np.nonzero(m2)[0]) != [3, 7, 11]:
        fails.append("small")
    return fails


def test_pad_mask():
    assert check_pad_mask(oracle.pad_mask) == []


def test_pad_mask_planted_first_lane_fails():
    def bad(H, H_u, z):
        m = np.zeros(H, bool)
        if z and H > H_u:
            m[0::H // (H - H_u)] = True
        return m
    assert check_pad_mask(bad)


# -------------------------------------------------- norm + logits vs decimal
def _decimal_norm_logits(x, gamma, w_bits, H_u, eps, pad):
    """50-digit evaluation of rmsnorm followed by the lm_head, loops only."""
    gbs, H = len(x), len(x[0])
    V = len(w_bits[0])
    wv = [[Decimal(_bf16_value(int(w_bits[h][v]))) for v in range(V)] for h in range(H)]
    ys, Ls = [], []
    for b in range(gbs):
        ss = Decimal(0)
        for h in range(H):
            if not pad[h]:
                ss += Decimal(float(x[b][h])) ** 2
        r = 1 / (ss / H_u + Decimal(eps)).sqrt()
        y = [Decimal(0) if pad[h] else Decimal(float(x[b][h])) * r * Decimal(float(gamma[h]))
             for h in range(H)]
        ys.append(y)
        Ls.append([sum((y[h] * wv[h][v] for h in range(H) if not pad[h]), Decimal(0))
                   for v in range(V)])
    return ys, Ls


def _tiny_case(seed, gbs, H, H_u, V, zero_pad):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((gbs, H)).astype(np.float32)
    x[0] *= np.float32(1e-3)  # a low-norm row: eps matters there
    gamma = (1 + 0.1 * rng.standard_normal(H)).astype(np.float32)
    w = rng.standard_normal((H, V)).astype(np.float32) * np.float32(0.05)
    w_bits = (w.view(np.uint32) >> 16).astype(np.uint16)
    return x, gamma, w_bits, oracle.pad_mask(H, H_u, zero_pad)


def check_norm_logits(rmsnorm, logits) -> list:
    fails = []
    for seed, (gbs, H, H_u, V, zp) in enumerate([(3, 16, 16, 11, False), (2, 24, 18, 7, True),
                                                   (1, 40, 40, 5, False)]):
        x, gamma, w_bits, pad = _tiny_case(seed, gbs, H, H_u, V, zp)
        eps = 1e-5
        y, r = rmsnorm(x.astype(np.float64), gamma, H_u, eps, pad)
        L = logits(y, w_bits, pad)
        yd, Ld = _decimal_norm_logits(x, gamma, w_bits, H_u, eps, pad)
        for b in range(gbs):
            for h in range(H):
                ref = float(yd[b][h])
                if abs(y[b, h] - ref) > 1e-13 * max(abs(ref), 1e-300) + 1e-300:
                    fails.append(f"y[{b},{h}] {y[b, h]!r} vs {ref!r}")
                    break
            for v in range(V):
                ref = float(Ld[b][v])
                scale = float(sum(abs(yd[b][h]) for h in range(H))) * 0.2
                if abs(L[b, v] - ref) > 1e-13 * scale:
                    fails.append(f"L[{b},{v}] {L[b, v]!r} vs {ref!r}")
                    break
    return fails


def test_norm_logits_vs_decimal():
    assert check_norm_logits(oracle.rmsnorm, oracle.logits) == []


def test_hand_example_norm():
    # x = [3, 4], gamma = 1, eps = 0: mean square 12.5, y = x / sqrt(12.5); W = I gives L = y
    y, r = oracle.rmsnorm(np.array([[3.0, 4.0]]), np.array([1.0, 1.0]), 2, 0.0, np.zeros(2, bool))
    assert y[0, 0] == pytest.approx(0.8485281374238570, rel=1e-15)
    assert y[0, 1] == pytest.approx(1.1313708498984760, rel=1e-15)
    eye = (np.eye(2, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)
    L = oracle.logits(y, eye, np.zeros(2, bool))
    assert np.array_equal(L, y)


@pytest.mark.parametrize("mistake", ["eps_outside_sqrt", "mean_over_H", "no_gamma", "w_transposed",
                                     "pad_rows_read"])
def test_norm_logits_planted_mistakes_fail(mistake):
    def bad_norm(x, gamma, H_u, eps, pad):
        x = np.array(x, np.float64)
        g = np.asarray(gamma, np.float64)
        real = ~pad
        if mistake == "mean_over_H":
            ms = np.sum(x[:, real] ** 2, 1) / x.shape[1]
        else:
            ms = np.sum(x[:, real] ** 2, 1) / H_u
        r = 1 / np.sqrt(ms) + eps if mistake == "eps_outside_sqrt" else 1 / np.sqrt(ms + eps)
        y = np.zeros_like(x)
        y[:, real] = x[:, real] * r[:, None] * (1.0 if mistake == "no_gamma" else g[real])
        return y, r

    def bad_logits(y, w_bits, pad):
        w = T.bf16_bits_to_f64(w_bits)
        if mistake == "w_transposed":
            w = w.reshape(w.shape[1], w.shape[0]).T  # reinterpreted as [V, H]
        if mistake == "pad_rows_read":
            return y @ w
        return y[:, ~pad] @ w[~pad]

    if mistake in ("w_transposed", "pad_rows_read"):
        fails = check_norm_logits(oracle.rmsnorm, bad_logits)
        if mistake == "pad_rows_read":
            fails += check_pad_invariant(oracle.rmsnorm, bad_logits)
    else:
        fails = check_norm_logits(bad_norm, oracle.logits)
    assert fails


# ---------------------------------------------- pad invariant (and NaN pads)
def check_pad_invariant(rmsnorm, logits) -> list:
    """Padded [H] with H_u real lanes == compacted [H_u], bitwise; garbage in
    the pad lanes (NaN in hidden, gamma and weight rows) changes nothing."""
    fails = []
    gbs, H, H_u, V = 3, 48, 45, 9  # s = 16
    x, gamma, w_bits, pad = _tiny_case(7, gbs, H, H_u, V, True)
    real = ~pad
    yc, rc = rmsnorm(x[:, real].astype(np.float64), gamma[real], H_u, 1e-5, np.zeros(H_u, bool))
    Lc = logits(yc, w_bits[real], np.zeros(H_u, bool))
    xg, gg, wg = x.copy(), gamma.copy(), w_bits.copy()
    xg[:, pad] = np.nan
    gg[pad] = np.nan
    wg[pad] = 0x7FC0  # bf16 NaN
    for xx, g, w in ((np.where(pad, 0, x), np.where(pad, 0, gamma), np.where(pad[:, None], 0, w_bits)),
                     (xg, gg, wg)):
        y, r = rmsnorm(xx.astype(np.float64), g, H_u, 1e-5, pad)
        L = logits(y, w, pad)
        if not (np.array_equal(r, rc) and np.array_equal(y[:, real], yc) and np.array_equal(L, Lc)):
            fails.append("padded != compacted")
    return fails


def test_pad_invariant():
    assert check_pad_invariant(oracle.rmsnorm, oracle.logits) == []


# ---------------------------------------------------------------------- topk
def check_topk(topk) -> list:
    fails = []
    rng = np.random.default_rng(3)
    for trial in range(40):
        V = int(rng.integers(1, 60))
        k = int(rng.integers(1, V + 1))
        L = np.round(rng.standard_normal((2, V)) * 2) / 2  # many exact ties
        L[0, rng.integers(0, V)] = -0.0
        L[1, :: max(1, V // 5)] = 0.0
        L[1, 1::7] = -0.0
        vals, idx = topk(L, k)
        for b in range(2):
            want = sorted(range(V), key=lambda i: (-float(L[b, i]), i))[:k]
            if list(idx[b]) != want:
                fails.append(f"trial {trial} row {b}")
                return fails
            if not np.array_equal(vals[b], L[b, want]):
                fails.append("values")
    try:
        topk(np.array([[1.0, np.nan]]), 1)
        fails.append("NaN accepted")
    except ValueError:
        pass
    return fails


def test_topk_vs_python_sort():
    assert check_topk(oracle.topk) == []


@pytest.mark.parametrize("mistake", ["higher_index", "ascending", "unstable_negzero"])
def test_topk_planted_mistakes_fail(mistake):
    def bad(L, k):
        L = np.asarray(L, np.float64)
        if not np.all(np.isfinite(L)):
            raise ValueError
        if mistake == "higher_index":
            order = (L.shape[1] - 1 - np.argsort(-L[:, ::-1], 1, kind="stable"))[:, :k]
        elif mistake == "ascending":
            order = np.argsort(L, 1, kind="stable")[:, :k]
        else:  # sorts by bit pattern, so -0.0 ranks below +0.0
            key = np.where(L == 0, np.copysign(1e-300, L), L)
            order = np.argsort(-key, 1, kind="stable")[:, :k]
        return np.take_along_axis(L, order, 1), order
    assert check_topk(bad)


# ------------------------------------------------------------------- sampler
def _decimal_sample(vals, idx, top_k, top_p, T_, u):
    """Sampler with 50-digit exp and sums, loops only."""
    k = len(vals)
    kk = int(top_k) if math.isfinite(top_k) else 0
    if kk < 1 or kk > k:
        kk = k
    if not T_ > 0:
        return int(idx[0])
    e = [(Decimal(float(vals[i])) - Decimal(float(vals[0]))) / Decimal(T_) for i in range(kk)]
    e = [x.exp() for x in e]
    S, acc = [], Decimal(0)
    for x in e:
        acc += x
        S.append(acc)
    m = next((i + 1 for i in range(kk) if S[i] >= Decimal(top_p) * S[-1]), kk)
    j = next((i for i in range(m) if S[i] > Decimal(u) * S[m - 1]), m - 1)
    return int(idx[j])


def check_sampler(sample_row) -> list:
    fails = []
    # hand-worked example (derived by hand): logits 2, 1, 0, -1 at T = 1:
    # p = e^{-i} / (1 + e^-1 + e^-2 + e^-3) = 0.643914, 0.236883, 0.087144, 0.032059;
    # cumulative 0.643914, 0.880797, 0.967941, 1 -> top_p 0.9 keeps m = 3;
    # Q = 0.665241, 0.909969, 1 -> u = 0.7 falls in [Q0, Q1): candidate 1.
    vals = np.array([2.0, 1.0, 0.0, -1.0])
    idx = np.array([10, 11, 12, 13])
    tok, d = sample_row(vals, idx, 4, 0.9, 1.0, 0.7)
    if tok != 11 or d["m"] != 3:
        fails.append(f"hand example: token {tok} m {d['m']}")
    if d["Q"] is None or not np.allclose(d["Q"], [0.665241, 0.909969, 1.0], atol=1e-6):
        fails.append(f"hand example Q {d['Q']}")
    for u, want in ((0.0, 10), (0.665, 10), (0.6653, 11), (0.9099, 11), (0.9100, 12), (0.999999, 12)):
        if sample_row(vals, idx, 4, 0.9, 1.0, u)[0] != want:
            fails.append(f"hand example u={u}")
    # T = 0.5: p = 0.864955, 0.117059, 0.015842, 0.002144; top_p 0.95 keeps 2
    t5 = sample_row(vals, idx, 4, 0.95, 0.5, 0.99)
    if t5[0] != 11 or t5[1]["m"] != 2:
        fails.append("T=0.5 example")
    # exact boundaries (all values binary-exact): four equal logits, T = 1 ->
    # cumulative mass 1/4, 1/2, 3/4, 1.  top_p = 1/2 is reached exactly at the
    # second candidate, so the nucleus keeps 2 (">=" at the cut); u = 1/4 is the
    # left end of candidate 1's interval [1/4, 1/2), so it picks candidate 1.
    eq = np.zeros(4)
    if sample_row(eq, idx, 4, 0.5, 1.0, 0.9)[1]["m"] != 2 or sample_row(eq, idx, 4, 0.5, 1.0, 0.9)[0] != 11:
        fails.append("nucleus cut at exact top_p")
    if sample_row(eq, idx, 4, 1.0, 1.0, 0.25)[0] != 11 or sample_row(eq, idx, 4, 1.0, 1.0, 0.5)[0] != 12:
        fails.append("u at the left end of an interval")
    # special cases on random candidate lists
    rng = np.random.default_rng(11)
    for trial in range(300):
        k = int(rng.integers(1, 40))
        vals = np.sort(rng.standard_normal(k) * rng.uniform(0.1, 5))[::-1]
        idx = rng.permutation(1000)[:k]
        tk, tp, tt, u = rng.integers(-3, k + 4), rng.uniform(-0.2, 1.3), rng.uniform(0.05, 2), rng.uniform(-0.1, 1.1)
        if sample_row(vals, idx, tk, tp, 0.0, u)[0] != idx[0]:
            fails.append("T=0 is not argmax")
        if sample_row(vals, idx, 1, tp, tt, u)[0] != idx[0]:
            fails.append("top_k=1 is not argmax")
        d = sample_row(vals, idx, tk, 1.0 + abs(tp), tt, u)[1]
        kk = tk if 1 <= tk <= k else k
        if d["m"] != kk:
            fails.append("top_p >= 1 does not keep kk")
        if sample_row(vals, idx, tk, -abs(tp), tt, u)[1]["m"] != 1:
            fails.append("top_p <= 0 does not keep 1")
        want = _decimal_sample(vals, idx, float(tk), float(tp), float(tt), float(u))
        got, d = sample_row(vals, idx, tk, tp, tt, u)
        near = d["Q"] is not None and (np.min(np.abs(d["Q"] - u)) < 1e-9 or
                                      np.min(np.abs(d["C"] - tp)) < 1e-9)
        if got != want and not near:
            fails.append(f"decimal trial {trial}: {got} vs {want}")
        if len(fails) > 3:
            break
    # u sweep: the tokens reached are exactly the nucleus, each with measure q_i
    vals = np.sort(rng.standard_normal(30))[::-1]
    idx = np.arange(100, 130)
    n = 100000
    grid = (np.arange(n) + 0.5) / n
    toks = np.array([sample_row(vals, idx, 25, 0.8, 0.7, u)[0] for u in grid])
    d = sample_row(vals, idx, 25, 0.8, 0.7, 0.5)[1]
    q = np.diff(np.concatenate([[0.0], d["Q"]]))
    if set(toks.tolist()) != set(idx[:d["m"]].tolist()):
        fails.append("u sweep does not cover exactly the nucleus")
    for i in range(d["m"]):
        if abs(np.mean(toks == idx[i]) - q[i]) > 1e-5 + 1.0 / n:
            fails.append(f"u sweep measure of candidate {i}")
            break
    # the 4th column defaults to the page's deterministic draw
    params3 = np.array([[4, 0.9, 1.0]], np.float32)
    params4 = np.array([[4, 0.9, 1.0, 0.5]], np.float32)
    if oracle.sample(vals[None, :4], idx[None, :4], params3)[0][0] != \
            oracle.sample(vals[None, :4], idx[None, :4], params4)[0][0]:
        fails.append("3-column params do not default u to 0.5")
    return fails


def test_sampler_pins():
    assert check_sampler(oracle.sample_row) == []


@pytest.mark.parametrize("mistake", ["strict_nucleus", "cdf_ascending", "no_temperature",
                                     "u_inclusive", "topk_after_nucleus"])
def test_sampler_planted_mistakes_fail(mistake):
    def bad(vals, idx, top_k, top_p, temperature, u):
        vals = np.asarray(vals, np.float64)
        k = len(vals)
        kk = int(top_k) if math.isfinite(top_k) else 0
        if kk < 1 or kk > k:
            kk = k
        if not temperature > 0:
            return int(idx[0]), dict(kk=kk, m=1, C=None, Q=None, greedy=True)
        Tt = 1.0 if mistake == "no_temperature" else temperature
        n = k if mistake == "topk_after_nucleus" else kk
        e = np.exp((vals[:n] - vals[0]) / Tt)
        S = np.cumsum(e)
        tot = S[-1]
        hit = np.nonzero(S > top_p * tot if mistake == "strict_nucleus" else S >= top_p * tot)[0]
        m = int(hit[0]) + 1 if hit.size else n
        if mistake == "topk_after_nucleus":
            m = min(m, kk)
        mass = S[m - 1]
        if mistake == "cdf_ascending":
            S = np.cumsum(e[:m][::-1])
            above = np.nonzero(S > u * mass)[0]
            j = m - 1 - int(above[0]) if above.size else 0
        else:
            above = np.nonzero(S[:m] >= u * mass if mistake == "u_inclusive" else S[:m] > u * mass)[0]
            j = int(above[0]) if above.size else m - 1
        return int(idx[j]), dict(kk=kk, m=m, C=S / tot, Q=S[:m] / mass, greedy=False)
    assert check_sampler(bad)


# --------------------------------------------------------- page constants
def test_page_constants():
    c = json.load(open(os.path.join(GOLDEN, "page_constants.json")))
    assert oracle.DETERMINISTIC_DRAW == c["deterministic_draw"]["value"]
    import inspect
    assert inspect.signature(oracle.tail).parameters["eps"].default == c["eps"]["value"]
    # the fp32 logit shard the page quotes, gbs * V_s * 4 bytes, is 805 KB (whole
    # KB) at the production shape: within 1 KB of one full 201088-entry row of fp32
    assert abs(201088 * 4 / 1000 - c["emit_logits_kb_at_production_shape"]["value"]) < 1.0


# ------------------------------------------------ end to end, brute force
def test_tiny_config_end_to_end_brute_force():
    """Config 0 (gbs 1, H 256, V 4096, k 16) through pure-Python loops:
    math.fsum norm and dot products, Python's sort, the decimal sampler."""
    import synth
    inp = synth.make_config(0)
    out = oracle.tail(inp.hidden, inp.dtype, inp.gamma, inp.w_t, inp.H_u, inp.k, inp.eps,
                      inp.zero_pad, params=inp.params[0])
    x = [float(v) for v in inp.hidden[0]]
    ms = math.fsum(v * v for v in x) / inp.H_u
    r = 1.0 / math.sqrt(ms + inp.eps)
    y = [x[h] * r * float(inp.gamma[h]) for h in range(inp.H)]
    W = [[_bf16_value(int(b)) for b in row] for row in inp.w_t]
    L = [math.fsum(y[h] * W[h][v] for h in range(inp.H)) for v in range(inp.V)]
    assert np.max(np.abs(np.array(L) - out["logits"][0])) < 1e-12
    order = sorted(range(inp.V), key=lambda i: (-L[i], i))[:inp.k]
    assert list(out["idx"][0]) == order
    p = inp.params[0][0]
    want = _decimal_sample([L[i] for i in order], order, float(p[0]), float(p[1]), float(p[2]), float(p[3]))
    assert int(out["tokens"][0]) == want
