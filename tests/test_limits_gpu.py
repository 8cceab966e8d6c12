"""GPU parity at the limits of the C ABI: the largest batch (TAIL_GBS_MAX),
the widest hidden (TAIL_H_MAX, with and without interleaved pad lanes), a
vocabulary wide enough that the top-k groups grow past 64 columns, and the
smallest vocabulary with every k.  Other dimensions are kept small so the
oracle finishes in seconds; comparison rules as in tests/_cases.py."""
import numpy as np
import pytest

import oracle
import synth

from _cases import (check_logits, check_sampler_on_gpu_candidates, check_tokens, check_topk_exact,
                    check_topk_sets)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import decode_sampling_tail_amd as dst  # noqa: E402


def bf16_bits(w: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(w, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def gpu_bf16(bits: np.ndarray):
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()


def run_case(gbs, H, H_u, V, k, zp, seed, dtype=synth.DT_F32, greedy_frac=0.25):
    rng = np.random.default_rng(seed)
    pad = oracle.pad_mask(H, H_u, zp)
    x = (rng.standard_normal((gbs, H)) * rng.uniform(0.2, 5, (gbs, 1))).astype(np.float32)
    x[:, pad] = np.nan if zp else 0.0
    gamma = (1 + 0.1 * rng.standard_normal(H)).astype(np.float32)
    gamma[pad] = np.nan if zp else gamma[pad]
    w = bf16_bits(rng.standard_normal((H, V)) * (1.0 / np.sqrt(H_u)))
    w[pad] = 0x7FC0 if zp else 0
    p = np.empty((gbs, 4), np.float32)
    p[:, 0] = rng.integers(0, k + 2, gbs)
    p[:, 1] = rng.uniform(0.3, 1.0, gbs)
    p[:, 2] = np.where(rng.random(gbs) < greedy_frac, 0.0, rng.uniform(0.3, 1.5, gbs))
    p[:, 3] = rng.uniform(0, 1, gbs)
    if dtype == synth.DT_F16:
        xs = x.astype(np.float16)
        xt = torch.from_numpy(xs).cuda()
    else:
        xs = x
        xt = torch.from_numpy(x).cuda()
    out = dst.forward(xt, torch.from_numpy(gamma).cuda(), gpu_bf16(w), k=k, H_u=H_u, zero_pad=zp,
                      params=torch.from_numpy(p).cuda())
    torch.cuda.synchronize()
    out = {key: v.cpu().numpy() for key, v in out.items()}
    ref = oracle.tail(xs, dtype, gamma, w, H_u, k, 1e-5, zp, params=p)
    ref["vals_k1"] = oracle.topk(ref["logits"], k + 1)[0] if k < V else None
    fails, rel, mx = check_logits(out["logits"], ref["logits"])
    assert not fails, fails
    assert not check_topk_sets(out["idx"], ref["logits"], k)
    assert not check_topk_exact(out["vals"], out["idx"], out["logits"], k)
    fails, exempt, widened = check_tokens(out["tokens"], ref, p, out["logits"], k)
    assert not fails, fails
    assert not check_sampler_on_gpu_candidates(out["tokens"], out["vals"], out["idx"], p)


def test_max_batch():
    """4096 rows: sixteen 256-row chunks of the matrix-core lm_head, 4096 select rows."""
    run_case(dst.GBS_MAX, 64, 64, 264, 16, False, 1)


@pytest.mark.parametrize("gbs,zp", [(2, False), (6, False), (3, True)])
def test_max_hidden(gbs, zp):
    """65536 lanes: the long-row branches of the RMSNorm (weight-streaming path,
    too wide to fuse) and of the activation producer (matrix-core path)."""
    H = dst.H_MAX
    H_u = H - H // 16 if zp else H
    run_case(gbs, H, H_u, 1032, 32, zp, 2 + gbs, synth.DT_F16)


@pytest.mark.parametrize("V,k", [(524352, 256), (1048576, 1024), (1310720, 256), (2621440, 64)])
def test_wide_vocab_topk(V, k):
    """More than 8192 groups of 64 columns: the groups grow to 128, 256 or 512
    columns, and the group maxima come from a separate pass (tail_topk alone):
    in-place lane combining up to 256 columns, one wave per group above."""
    rng = np.random.default_rng(V)
    L = rng.standard_normal((2, V)).astype(np.float32)
    L[1, rng.integers(0, V, 3000)] = 4.0  # exact ties above the k-th value
    vals, idx = dst.topk(torch.from_numpy(L).cuda(), k)
    ov, oi = oracle.topk(L.astype(np.float64), k)
    assert np.array_equal(idx.cpu().numpy().astype(np.int64), oi)
    assert np.array_equal(vals.cpu().numpy().view(np.uint32), L[np.arange(2)[:, None], oi].view(np.uint32))


@pytest.mark.parametrize("k", [1, 3, 8])
def test_smallest_vocab(k):
    """V = 8 (one 16-byte weight chunk per row), every k up to V."""
    run_case(2, 16, 16, 8, k, False, 10 + k)
