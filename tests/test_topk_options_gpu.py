"""GPU tests of the top-k options of tail_topk_ex and tail_forward: the NaN
fold (TAIL_NAN_FOLD, the page's "skip_nan_fold" off) against the oracle's
fold, the stage-1 taps against invariants recomputed on the host, and the
page's statement that the fold changes nothing on NaN-free input."""
import numpy as np
import pytest

import oracle

from _cases import config, to_gpu

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import decode_sampling_tail_amd as dst  # noqa: E402


def np_(t):
    return t.detach().cpu().numpy()


def _nan_case(kind, gbs, V, k, rng):
    L = rng.standard_normal((gbs, V)).astype(np.float32)
    if kind == "sparse":      # a few NaN of both signs and infinities
        m = rng.random((gbs, V))
        L[m < 0.01] = np.nan
        L[(m >= 0.01) & (m < 0.02)] = -np.nan
        L[(m >= 0.02) & (m < 0.025)] = np.inf
        L[(m >= 0.025) & (m < 0.03)] = -np.inf
    elif kind == "dense":     # more NaN than V - k: -inf reaches the output
        L[rng.random((gbs, V)) < 1 - 0.5 * k / V] = np.nan
    elif kind == "all":       # every logit NaN: k times -inf, lowest indices
        L[:] = np.nan
    elif kind == "top":       # NaN where the largest logits were
        order = np.argsort(-L, axis=1)[:, :2 * k]
        np.put_along_axis(L, order[:, ::2], np.nan, axis=1)
    return L


@pytest.mark.parametrize("kind", ["sparse", "dense", "all", "top"])
@pytest.mark.parametrize("gbs,V,k", [(2, 4096, 16), (3, 201088, 256), (2, 1032, 256), (2, 40, 7)])
@pytest.mark.parametrize("mirror", [False, True])
def test_topk_nan_fold(kind, gbs, V, k, mirror):
    rng = np.random.default_rng(V + k + len(kind))
    L = _nan_case(kind, gbs, V, k, rng)
    vals, idx = dst.topk(torch.from_numpy(L).cuda(), k, mirror=mirror, nan_fold=True)
    vals, idx = np_(vals), np_(idx)
    ref = L.astype(np.float64)
    if mirror:
        ref = oracle.mirror(ref)  # NaN stays NaN, then folds
    ov, oi = oracle.topk(ref, k, nan_fold=True)
    assert np.array_equal(idx.astype(np.int64), oi)
    assert np.array_equal(vals.view(np.uint32), ov.astype(np.float32).view(np.uint32))


def _keys(f32: np.ndarray) -> np.ndarray:
    """Order-preserving u32 keys of float32 values, -0.0 as +0.0."""
    u = np.ascontiguousarray(f32, np.float32).view(np.uint32).copy()
    u[u == 0x80000000] = 0
    return np.where(u & 0x80000000, ~u, u | 0x80000000).astype(np.uint32)


def _group_size(V, k):
    gs = 64
    while gs > 1 and -(-V // gs) < k:
        gs >>= 1
    while -(-V // gs) > 8192:
        gs <<= 1
    return gs


@pytest.mark.parametrize("kind", ["normal", "ties", "equal", "nan"])
@pytest.mark.parametrize("gbs,V,k", [(2, 4096, 16), (3, 201088, 256), (2, 8000, 1024), (2, 40, 7)])
@pytest.mark.parametrize("mirror", [False, True])
def test_topk_taps(kind, gbs, V, k, mirror):
    rng = np.random.default_rng(V * 3 + k + len(kind))
    if kind == "normal":
        L = rng.standard_normal((gbs, V)).astype(np.float32)
    elif kind == "ties":      # few distinct values: thousands equal to the k-th
        L = (np.round(rng.standard_normal((gbs, V)) * 2) / 2).astype(np.float32)
    elif kind == "equal":
        L = np.full((gbs, V), 0.25, np.float32)
    else:
        L = _nan_case("sparse", gbs, V, k, rng)
    fold = kind == "nan"
    taps = torch.zeros((gbs, 4), dtype=torch.int32, device="cuda")
    vals, idx = dst.topk(torch.from_numpy(L).cuda(), k, mirror=mirror, nan_fold=fold, taps=taps)
    t = np_(taps).view(np.uint32)
    ranked = L.astype(np.float64)
    if mirror:
        ranked = oracle.mirror(ranked)
    if fold:
        ranked = np.where(np.isnan(ranked), -np.inf, ranked)
    keys = _keys(ranked.astype(np.float32))
    gs = _group_size(V, k)
    G = -(-V // gs)
    for b in range(gbs):
        t0, nact, cnt, path = (int(x) for x in t[b])
        kb = keys[b]
        assert cnt == int(np.sum(kb >= t0)), (b, cnt)
        assert cnt >= k
        assert np.sort(kb)[::-1][k - 1] >= t0            # t0 bounds the k-th key from below
        pad = np.zeros(G * gs, np.uint32)
        pad[:V] = kb
        gmax = pad.reshape(G, gs).max(axis=1)
        assert nact == int(np.sum(gmax >= t0)), (b, nact)
        assert path == (1 if cnt > 4096 else 0)
    # the list is still exact
    ov, oi = oracle.topk(ranked, k)
    assert np.array_equal(np_(idx).astype(np.int64), oi)


@pytest.mark.parametrize("cid", [1, 4])
def test_forward_nan_fold_changes_nothing_on_finite_input(cid):
    """With finite inputs the fold must give bitwise the same outputs."""
    inp = config(cid)
    g = to_gpu(inp)
    run = len(inp.params) - 1
    outs = []
    for fold in (False, True):
        f = dst.Forward(inp.gbs, inp.H, inp.V, inp.k, inp.H_u, inp.eps, inp.zero_pad, True, True,
                        nan_fold=fold)
        o = f(g["hidden"], g["gamma"], g["w_t"], g["params"][run])
        torch.cuda.synchronize()
        outs.append({key: np_(v) for key, v in o.items()})
    for key in ("logits", "vals", "idx", "tokens"):
        assert np.array_equal(outs[0][key].view(np.uint8), outs[1][key].view(np.uint8)), key
