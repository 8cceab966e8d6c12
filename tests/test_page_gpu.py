"""GPU parity of the page-precision mode (TAIL_PAGE_PRECISION: the GEMM input
rounded to bf16 once per element, the top-k over the bf16 mirror of the
logits) against the oracle's page mode, through the C ABI.  Comparison rules:
tests/_cases.py (page-precision section)."""
import numpy as np
import pytest

import oracle
import synth

from _cases import (check_logits, check_mirror_exact, check_mirror_sets,
                    check_sampler_on_gpu_candidates, check_tokens_page, config, oracle_tail_page,
                    to_gpu)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import decode_sampling_tail_amd as dst  # noqa: E402


def np_(t):
    return t.detach().cpu().numpy()


def bf16_bits(w: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(w, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def gpu_bf16(bits: np.ndarray):
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()


def hidden_in(x, dtype):
    if dtype == synth.DT_F16:
        xs = x.astype(np.float16)
        return xs, torch.from_numpy(xs).cuda()
    if dtype == synth.DT_BF16:
        xs = synth.round_bf16(x)
        return xs, gpu_bf16(xs)
    return x, torch.from_numpy(x).cuda()


# ---------------------------------------------------------------- rmsnorm
@pytest.mark.parametrize("dtype", [synth.DT_F32, synth.DT_F16, synth.DT_BF16])
@pytest.mark.parametrize("shape", [(1, 256, 256, False), (5, 2880, 2880, False), (3, 3072, 2880, True),
                                   (4, 48, 45, True)])
@pytest.mark.parametrize("deferred", [False, True])
def test_rmsnorm_page(dtype, shape, deferred):
    """The rounded activations equal the oracle's bit for bit (both round the
    same float32 value); r equals the oracle's fp32 r."""
    gbs, H, H_u, zp = shape
    rng = np.random.default_rng(gbs * 1000 + H + 7)
    x = (rng.standard_normal((gbs, H)) * rng.uniform(0.01, 20, (gbs, 1))).astype(np.float32)
    gamma = (1 + 0.1 * rng.standard_normal(H)).astype(np.float32)
    pad = oracle.pad_mask(H, H_u, zp)
    x[:, pad] = np.nan
    gamma[pad] = np.nan
    xs, xt = hidden_in(x, dtype)
    y, r = dst.rmsnorm(xt, torch.from_numpy(gamma).cuda(), H_u, 1e-5, zp, deferred, page=True)
    torch.cuda.synchronize()
    a, scale = oracle.rmsnorm_page(oracle.widen(xs, dtype), gamma, H_u, 1e-5, pad, deferred)
    r_ref = oracle.rmsnorm(oracle.widen(xs, dtype), gamma, H_u, 1e-5, pad)[1]
    assert np.array_equal(np_(r), r_ref.astype(np.float32))
    assert np.array_equal(np_(y).astype(np.float64), a)


# ---------------------------------------------------------------- lm_head
@pytest.mark.parametrize("gbs,H,V", [(1, 64, 4096), (3, 300, 1160), (5, 130, 264), (17, 96, 776),
                                     (64, 2880, 2056), (130, 2880, 800), (256, 700, 1544),
                                     (300, 64, 264), (3, 8192, 1032), (4, 6144, 1032)])
def test_lm_head_page(gbs, H, V):
    """Given y, both lm_head paths round it to bf16 before the contraction
    (at 3 x 8192 the weight-streaming kernel reads y in its loop, the rows
    being too wide for its LDS activation table, and rounds it there)."""
    rng = np.random.default_rng(V + gbs + 1)
    y = rng.standard_normal((gbs, H)).astype(np.float32)
    w = bf16_bits(rng.standard_normal((H, V)) * 0.02)
    rs = rng.uniform(0.5, 2, gbs).astype(np.float32)
    L = np_(dst.lm_head(torch.from_numpy(y).cuda(), gpu_bf16(w), row_scale=torch.from_numpy(rs).cuda(),
                        page=True))
    ref = oracle.logits(oracle.bf16_round(y), w, np.zeros(H, bool)) * rs[:, None].astype(np.float64)
    fails, rel, mx = check_logits(L, ref)
    assert not fails, fails
    # the rounding is really applied: the unrounded logits are further away
    exact = oracle.logits(y.astype(np.float64), w, np.zeros(H, bool)) * rs[:, None].astype(np.float64)
    assert np.linalg.norm(L - exact) > 10 * np.linalg.norm(L - ref)


@pytest.mark.parametrize("gbs,H,H_u,V,zp,dtype,deferred", [
    (1, 2880, 2880, 4096, False, synth.DT_BF16, True), (1, 2880, 2880, 4096, False, synth.DT_BF16, False),
    (3, 3072, 2880, 2056, True, synth.DT_F16, True), (4, 300, 300, 1160, False, synth.DT_F32, False),
    (3, 8000, 8000, 1032, False, synth.DT_F32, True),   # too wide to fuse: RMSNorm, then the GEMV
    (3, 8000, 8000, 1032, False, synth.DT_F32, False),
    (8, 640, 640, 2048, False, synth.DT_F32, True), (40, 3072, 2880, 1032, True, synth.DT_F16, False),
    (130, 256, 256, 520, False, synth.DT_BF16, True), (256, 2880, 2880, 776, False, synth.DT_F32, True)])
def test_rmsnorm_lm_head_page(gbs, H, H_u, V, zp, dtype, deferred):
    rng = np.random.default_rng(V * 3 + gbs + 1)
    pad = oracle.pad_mask(H, H_u, zp)
    x = (rng.standard_normal((gbs, H)) * rng.uniform(0.1, 10, (gbs, 1))).astype(np.float32)
    x[:, pad] = np.nan if zp else 0.0
    gamma = (1 + 0.1 * rng.standard_normal(H)).astype(np.float32)
    gamma[pad] = np.nan if zp else gamma[pad]
    w = bf16_bits(rng.standard_normal((H, V)) * 0.02)
    w[pad] = 0x7FC0 if zp else 0
    xs, xt = hidden_in(x, dtype)
    L, r = dst.rmsnorm_lm_head(xt, torch.from_numpy(gamma).cuda(), gpu_bf16(w), H_u, 1e-5, zp, deferred,
                               page=True)
    L = np_(L)
    a, scale = oracle.rmsnorm_page(oracle.widen(xs, dtype), gamma, H_u, 1e-5, pad, deferred)
    ref = oracle.logits(a, w, pad) * scale[:, None]
    fails, rel, mx = check_logits(L, ref)
    assert not fails, fails


# ------------------------------------------------------------------- top-k
def _mirror_case(kind, gbs, V, rng):
    if kind == "normal":
        return rng.standard_normal((gbs, V)).astype(np.float32)
    if kind == "collapse":  # distinct fp32 values that share a bf16 value, and exact midpoints
        base = np.round(rng.standard_normal((gbs, V)) * 8) / 8
        L = (base * (1 + rng.integers(-40, 41, (gbs, V)) * 2.0 ** -14)).astype(np.float32)
        mid = rng.random((gbs, V)) < 0.05
        L[mid] = (1 + 2.0 ** -8) * np.sign(base[mid] + 0.5)  # halfway: rounds to even
        return L
    if kind == "zeros":  # signed zeros, and tiny values that round to them
        L = np.where(rng.random((gbs, V)) < 0.5, -0.0, 0.0).astype(np.float32)
        L[rng.random((gbs, V)) < 0.3] = -1e-45
        L[:, rng.integers(0, V, 5)] = 1.0
        return L
    if kind == "spread":
        return (rng.standard_normal((gbs, V)) * 1e4).astype(np.float32)
    raise ValueError(kind)


@pytest.mark.parametrize("kind", ["normal", "collapse", "zeros", "spread"])
@pytest.mark.parametrize("gbs,V,k", [(1, 4096, 16), (3, 201088, 256), (2, 8000, 1024), (4, 1032, 256),
                                     (2, 40, 7)])
def test_topk_mirror(kind, gbs, V, k):
    """Both sides apply the same exact function to the same fp32 input:
    bitwise equal lists."""
    rng = np.random.default_rng(V * 7 + k + 3)
    L = _mirror_case(kind, gbs, V, rng)
    vals, idx = dst.topk(torch.from_numpy(L).cuda(), k, mirror=True)
    vals, idx = np_(vals), np_(idx)
    ov, oi = oracle.topk(oracle.mirror(L.astype(np.float64)), k)
    assert np.array_equal(idx.astype(np.int64), oi)
    assert np.array_equal(vals.view(np.uint32), ov.astype(np.float32).view(np.uint32))
    assert np.all((vals.view(np.uint32) & 0xFFFF) == 0)


# --------------------------------------------------- the five workloads
_gpu = {}


def gpu_config(cid):
    if cid not in _gpu:
        _gpu.clear()
        _gpu[cid] = to_gpu(config(cid))
    return _gpu[cid]


@pytest.mark.parametrize("cid,run,deferred", [(0, 0, True), (1, 1, True), (2, 0, True), (2, 0, False),
                                              (3, 0, True), (4, 0, True)])
def test_workload_page_parity(cid, run, deferred):
    inp = config(cid)
    g = gpu_config(cid)
    f = dst.Forward(inp.gbs, inp.H, inp.V, inp.k, inp.H_u, inp.eps, inp.zero_pad, deferred, True,
                    page=True)
    out = f(g["hidden"], g["gamma"], g["w_t"], g["params"][run])
    torch.cuda.synchronize()
    out = {key: np_(v) for key, v in out.items()}
    ref = oracle_tail_page(inp, run, deferred)
    fails, rel, mx = check_logits(out["logits"], ref["logits"])
    print(f"\npage workload {cid}/{run}: max rel-L2 {rel.max():.3e}, max abs {mx.max():.3e}")
    assert not fails, fails
    assert not check_mirror_exact(out["vals"], out["idx"], out["logits"], inp.k)
    assert not check_mirror_sets(out["idx"], oracle.mirror(ref["logits"]), inp.k)
    params = inp.params[run]
    fails, differ = check_tokens_page(out["tokens"], out["vals"], out["idx"], ref, params)
    print(f"tokens: {len(out['tokens'])} rows, candidate lists differing from the oracle's: {len(differ)}")
    assert not fails, fails
    assert not check_sampler_on_gpu_candidates(out["tokens"], out["vals"], out["idx"], params)
