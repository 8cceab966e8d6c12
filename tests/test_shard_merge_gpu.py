"""The vocabulary-sharded design on one GPU: with the vocabulary cut into 8
shards, the per-shard top-k lists merged by one more top-k over their
candidates give, bitwise, the global top-k of the shards' logits (the global
top-k is contained in the union of the shard top-ks), and the sampler on the
merged list gives the token the sampler gives on that global list.  The
shards run through tail_rmsnorm_lm_head and tail_topk at their real shape
(narrow enough that the lm_head splits K); only the candidate exchange
between GPUs is replaced by a concatenation.  The shard logits meet the
parity bar against the single-GPU logits of the whole vocabulary."""
import numpy as np
import pytest

from _cases import check_logits, config, to_gpu

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import decode_sampling_tail_amd as dst  # noqa: E402

SHARDS = 8


@pytest.mark.parametrize("cid", [1, 2, 3])
def test_shard_topk_merge_equals_global(cid):
    inp = config(cid)
    g = to_gpu(inp)
    run = 0
    Vs = inp.V // SHARDS
    full = dst.forward(g["hidden"], g["gamma"], g["w_t"], k=inp.k, H_u=inp.H_u, eps=inp.eps,
                       zero_pad=inp.zero_pad, params=g["params"][run])
    shard_logits, cand_v, cand_i = [], [], []
    for s in range(SHARDS):
        w = g["w_t"][:, s * Vs:(s + 1) * Vs].contiguous()
        L, _ = dst.rmsnorm_lm_head(g["hidden"], g["gamma"], w, inp.H_u, inp.eps, inp.zero_pad, True)
        v, i = dst.topk(L, inp.k)
        shard_logits.append(L)
        cand_v.append(v)
        cand_i.append(i + s * Vs)  # global column index
        del w
    # the exchange: every row's candidates side by side, shard by shard (each
    # shard's list is descending with ties in index order, so position order
    # among equal values is global index order)
    cv = torch.cat(cand_v, dim=1).contiguous()
    ci = torch.cat(cand_i, dim=1).contiguous()
    mv, mpos = dst.topk(cv, inp.k)
    midx = torch.gather(ci, 1, mpos.long()).to(torch.int32).contiguous()
    tok = dst.sample(mv, midx, g["params"][run])
    # the global top-k of the shards' logits, and its token
    Ls = torch.cat(shard_logits, dim=1).contiguous()
    gv, gi = dst.topk(Ls, inp.k)
    gtok = dst.sample(gv, gi, g["params"][run])
    torch.cuda.synchronize()
    assert np.array_equal(gi.cpu().numpy(), midx.cpu().numpy())
    assert np.array_equal(gv.cpu().numpy().view(np.uint32), mv.cpu().numpy().view(np.uint32))
    assert np.array_equal(gtok.cpu().numpy(), tok.cpu().numpy())
    fails, rel, mx = check_logits(Ls.cpu().numpy(), full["logits"].cpu().numpy().astype(np.float64))
    assert not fails, fails
