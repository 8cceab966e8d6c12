"""The top-k and sampler fused into the large-batch lm_head kernel
(TAIL_FUSED_SELECT=1: one launch after the producer, a grid barrier between
the contraction and the select; GPT-OSS tail API page, Background -- the
tail as one kernel).  Its outputs must be bitwise those of the separate
select launch, which the parity tests check against the oracle, on both
kernel shapes (128-row and 256-row chunks), several launches per batch,
the page-precision mirror ranking, every sampler width (k up to 1024), with
and without emitted logits and sampling; with TAIL_FUSED_SPIN=0 no
workgroup waits at the barrier, so the last one to arrive selects every row
(the path a shared GPU takes when not all workgroups are resident), and with
a limit of 2 polls some workgroups leave while others pass and share the
rows.  A
batch the fused kernel does not take (one-term above 128 rows) falls back
to the separate launch unchanged."""
import numpy as np
import pytest

import oracle
import synth

from _cases import (check_logits, check_sampler_on_gpu_candidates, check_tokens, check_topk_exact,
                    check_topk_sets, config, oracle_tail, to_gpu)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import decode_sampling_tail_amd as dst  # noqa: E402


def np_(t):
    return None if t is None else t.detach().cpu().numpy()


def bf16_bits(w: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(w, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def gpu_bf16(bits: np.ndarray):
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()


def inputs(gbs, H, H_u, V, k, zp, seed):
    rng = np.random.default_rng(seed)
    pad = oracle.pad_mask(H, H_u, zp)
    x = rng.standard_normal((gbs, H)).astype(np.float32)
    x[:, pad] = np.nan if zp else 0.0
    gamma = (1 + 0.1 * rng.standard_normal(H)).astype(np.float32)
    w = bf16_bits(rng.standard_normal((H, V)) * 0.05)
    w[pad] = 0x7FC0 if zp else 0
    p = np.empty((gbs, 4), np.float32)
    p[:, 0] = rng.integers(0, k + 2, gbs)
    p[:, 1] = rng.uniform(0.3, 1.0, gbs)
    p[:, 2] = np.where(rng.random(gbs) < 0.3, 0.0, rng.uniform(0.3, 1.5, gbs))
    p[:, 3] = rng.uniform(0, 1, gbs)
    return x, gamma, w, p


def outputs(f, out):
    torch.cuda.synchronize()
    return {key: np_(v).copy() for key, v in out.items() if v is not None}


def assert_same(a, b, what):
    assert a.keys() == b.keys(), what
    for key in a:
        assert np.array_equal(a[key].view(np.uint8), b[key].view(np.uint8)), (what, key)


def run(monkeypatch, mode, f, args):
    """mode: 'separate', 'fused', 'fused_nowait' (no polling) or
    'fused_short' (2 polls)."""
    monkeypatch.delenv("TAIL_FUSED_SELECT", raising=False)
    monkeypatch.delenv("TAIL_FUSED_SPIN", raising=False)
    if mode != "separate":
        monkeypatch.setenv("TAIL_FUSED_SELECT", "1")
    if mode == "fused_nowait":
        monkeypatch.setenv("TAIL_FUSED_SPIN", "0")
    if mode == "fused_short":
        monkeypatch.setenv("TAIL_FUSED_SPIN", "2")
    f.vals.fill_(float("nan"))
    f.idx.fill_(-1)
    f.tokens.fill_(-1)
    if f.logits is not None:
        f.logits.fill_(float("nan"))
    return outputs(f, f(*args))


# H below 512 padded K lanes: 65-128 rows take the large-batch kernel too
CASES = [
    # gbs, H, H_u, V, k, zp, page, emit, sample
    (100, 256, 256, 16456, 256, False, False, True, True),    # 128-row chunk, ragged last tile
    (128, 192, 180, 12296, 64, True, False, False, True),     # pad lanes, logits not emitted
    (80, 256, 256, 65544, 1000, False, True, True, True),     # page mirror ranking, 16 per lane
    (65, 128, 128, 32776, 512, False, False, True, False),    # one real row in the last tile
    (200, 64, 64, 16456, 256, False, False, False, True),     # 256-row chunk
    (256, 128, 128, 32776, 512, False, False, True, False),   # no sampling
    (300, 96, 96, 16456, 100, False, False, False, True),     # two launches
    (513, 64, 64, 8200, 128, False, False, True, True),       # three launches, one row in the last
    (256, 128, 128, 16456, 256, False, True, True, True),     # one term above 128 rows: not fused
]


@pytest.mark.parametrize("gbs,H,H_u,V,k,zp,page,emit,sample", CASES)
def test_fused_select_bitwise_equal(monkeypatch, gbs, H, H_u, V, k, zp, page, emit, sample):
    x, gamma, w, p = inputs(gbs, H, H_u, V, k, zp, gbs * 131 + V)
    args = (torch.from_numpy(x).cuda(), torch.from_numpy(gamma).cuda(), gpu_bf16(w),
            torch.from_numpy(p).cuda() if sample else None)
    f = dst.Forward(gbs, H, V, k, H_u, 1e-5, zp, True, emit, page=page)
    ref = run(monkeypatch, "separate", f, args)
    for mode in ("fused", "fused_nowait", "fused_short", "fused"):
        assert_same(run(monkeypatch, mode, f, args), ref, (mode, gbs, V, k))


def test_fused_select_oracle_parity(monkeypatch):
    """One shape through the fused kernel against the oracle directly."""
    gbs, H, V, k = 160, 96, 12296, 256
    x, gamma, w, p = inputs(gbs, H, H, V, k, False, 7)
    monkeypatch.setenv("TAIL_FUSED_SELECT", "1")
    out = dst.forward(torch.from_numpy(x).cuda(), torch.from_numpy(gamma).cuda(), gpu_bf16(w), k=k,
                      params=torch.from_numpy(p).cuda())
    torch.cuda.synchronize()
    out = {key: np_(v) for key, v in out.items()}
    ref = oracle.tail(x, synth.DT_F32, gamma, w, H, k, 1e-5, False, params=p)
    ref["vals_k1"] = oracle.topk(ref["logits"], k + 1)[0]
    fails, rel, mx = check_logits(out["logits"], ref["logits"])
    assert not fails, fails
    assert not check_topk_sets(out["idx"], ref["logits"], k)
    assert not check_topk_exact(out["vals"], out["idx"], out["logits"], k)
    fails, exempt, widened = check_tokens(out["tokens"], ref, p, out["logits"], k)
    assert not fails and not widened, (fails, widened)
    assert not check_sampler_on_gpu_candidates(out["tokens"], out["vals"], out["idx"], p)


def test_fused_select_gbs256_workload(monkeypatch):
    """The 256-row GPT-OSS workload: fused and separate bitwise equal, and the
    fused outputs meet the oracle bar."""
    inp = config(4)
    g = to_gpu(inp)
    params = g["params"][0]
    f = dst.Forward(inp.gbs, inp.H, inp.V, inp.k, inp.H_u, inp.eps, inp.zero_pad, True, True)
    args = (g["hidden"], g["gamma"], g["w_t"], params)
    ref = run(monkeypatch, "separate", f, args)
    fused = run(monkeypatch, "fused", f, args)
    assert_same(fused, ref, "gbs256")
    del g
    oref = oracle_tail(inp, 0)
    fails, rel, mx = check_logits(fused["logits"], oref["logits"])
    assert not fails, fails
    assert not check_topk_sets(fused["idx"], oref["logits"], inp.k)
    fails, exempt, widened = check_tokens(fused["tokens"], oref, inp.params[0], fused["logits"],
                                          inp.k)
    assert not fails and not widened, (fails, widened)


def test_fused_select_graph_replay(monkeypatch):
    """A captured fused step replays exactly: the producer kernel clears the
    barrier's counters on every replay (no memset node)."""
    monkeypatch.setenv("TAIL_FUSED_SELECT", "1")
    gbs, H, V, k = 200, 64, 16456, 256
    x, gamma, w, p = inputs(gbs, H, H, V, k, False, 11)
    gamma_t, w_t, p_t = torch.from_numpy(gamma).cuda(), gpu_bf16(w), torch.from_numpy(p).cuda()
    hidden = torch.from_numpy(x).cuda()
    f = dst.Forward(gbs, H, V, k, H, 1e-5, False, True, True)
    eager = dst.Forward(gbs, H, V, k, H, 1e-5, False, True, True)
    f(hidden, gamma_t, w_t, p_t)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        f(hidden, gamma_t, w_t, p_t)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    for rep in range(3):
        new = torch.from_numpy(rng.standard_normal((gbs, H)).astype(np.float32)).cuda()
        hidden.copy_(new)
        graph.replay()
        monkeypatch.setenv("TAIL_FUSED_SELECT", "0")
        want = outputs(eager, eager(new, gamma_t, w_t, p_t))
        monkeypatch.setenv("TAIL_FUSED_SELECT", "1")
        got = {key: np_(getattr(f, key)) for key in ("logits", "vals", "idx", "tokens")}
        assert_same(got, want, ("replay", rep))


def test_fused_select_noalloc(monkeypatch):
    """tail_forward_noalloc takes the fused kernel too (its counters live in
    the static scratch), twice in a row with the second batch smaller."""
    for gbs in (256, 150):
        H, V, k = 64, 16456, 256
        x, gamma, w, p = inputs(gbs, H, H, V, k, False, gbs)
        args = (torch.from_numpy(x).cuda(), torch.from_numpy(gamma).cuda(), gpu_bf16(w),
                torch.from_numpy(p).cuda())
        f = dst.Forward(gbs, H, V, k, H, 1e-5, False, True, True)
        ref = run(monkeypatch, "separate", f, args)
        monkeypatch.setenv("TAIL_FUSED_SELECT", "1")
        f.vals.fill_(float("nan"))
        got = outputs(f, f.noalloc(*args))
        assert_same(got, ref, ("noalloc", gbs))


@pytest.mark.parametrize("V,k,fold", [(16456, 256, True), (8200, 256, False)])
def test_fused_select_falls_back(monkeypatch, V, k, fold):
    """Batches the fused kernel does not take keep the separate launch under
    TAIL_FUSED_SELECT=1: the NaN fold (its group maxima come from a pass of
    their own), and top-k groups other than the lm_head's 64-column groups
    (8200 columns hold 129 groups of 64, fewer than k = 256)."""
    gbs, H = 200, 64
    x, gamma, w, p = inputs(gbs, H, H, V, k, False, V + k)
    args = (torch.from_numpy(x).cuda(), torch.from_numpy(gamma).cuda(), gpu_bf16(w),
            torch.from_numpy(p).cuda())
    f = dst.Forward(gbs, H, V, k, H, 1e-5, False, True, True, nan_fold=fold)
    ref = run(monkeypatch, "separate", f, args)
    assert_same(run(monkeypatch, "fused", f, args), ref, ("fallback", V, k, fold))
