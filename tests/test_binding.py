"""The Python binding checks every tensor argument before it calls the C ABI:
device, contiguity, dtype and shape.  A tensor on the host, of another dtype
or another shape would otherwise hand a kernel a pointer to memory of the
wrong kind or size; the binding raises ValueError instead and launches
nothing."""
import pytest
import torch

import decode_sampling_tail_amd as dst


def test_host_tensors_are_rejected_without_a_gpu():
    h = torch.zeros(2, 8)
    g = torch.ones(8)
    w = torch.zeros(8, 16, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensor"):
        dst.rmsnorm(h, g)
    with pytest.raises(ValueError, match="GPU tensor"):
        dst.rmsnorm_lm_head(h, g, w)
    with pytest.raises(ValueError, match="GPU tensor"):
        dst.lm_head(h, w)
    with pytest.raises(ValueError, match="GPU tensor"):
        dst.topk(torch.zeros(2, 16), 4)
    with pytest.raises(ValueError, match="GPU tensor"):
        dst.sample(torch.zeros(2, 4), torch.zeros(2, 4, dtype=torch.int32), torch.zeros(2, 3))
    with pytest.raises(ValueError, match="must be a torch tensor"):
        dst.topk([[1.0, 2.0]], 1)


GBS, H, V, K = 4, 64, 1024, 16


@pytest.fixture(scope="module")
def args():
    torch.manual_seed(0)
    dev = torch.device("cuda")
    return dict(hidden=torch.randn(GBS, H, device=dev),
                gamma=torch.ones(H, device=dev),
                w=(torch.randn(H, V, device=dev) * 0.05).to(torch.bfloat16),
                params=torch.tensor([[8, 0.9, 0.7, 0.5]] * GBS, dtype=torch.float32, device=dev))


@pytest.mark.gpu
def test_forward_argument_checks(args):
    f = dst.Forward(GBS, H, V, K, emit_logits=True)
    a = args
    good = f(a["hidden"], a["gamma"], a["w"], a["params"])
    torch.cuda.synchronize()
    assert good["tokens"] is not None
    bad = [
        (dict(params=a["params"].cpu()), "GPU tensor"),                       # host params
        (dict(params=a["params"].double()), "dtype"),                        # float64 params
        (dict(params=a["params"][:2]), "shape"),                             # too few rows
        (dict(w=a["w"][:, : V // 2].contiguous()), "shape"),                 # narrower weight
        (dict(w=a["w"].float()), "dtype"),                                   # fp32 weight
        (dict(w=a["w"].t().contiguous().t()), "contiguous"),                 # a transposed view
        (dict(gamma=a["gamma"].half()), "dtype"),                            # fp16 gamma
        (dict(gamma=a["gamma"][: H // 2]), "shape"),                         # short gamma
        (dict(hidden=a["hidden"].double()), "dtype"),                        # fp64 hidden
        (dict(hidden=a["hidden"][:, : H // 2].contiguous()), "shape"),       # narrower hidden
    ]
    for change, what in bad:
        kw = dict(hidden=a["hidden"], gamma=a["gamma"], w_t=a["w"], params=a["params"])
        kw.update({("w_t" if k == "w" else k): v for k, v in change.items()})
        with pytest.raises(ValueError, match=what):
            f(**kw)


@pytest.mark.gpu
def test_stage_argument_checks(args):
    a = args
    logits, r = dst.rmsnorm_lm_head(a["hidden"], a["gamma"], a["w"])
    vals, idx = dst.topk(logits, K)
    torch.cuda.synchronize()
    with pytest.raises(ValueError, match="dtype"):
        dst.rmsnorm_lm_head(a["hidden"], a["gamma"], a["w"], out=torch.empty(GBS, V, device="cuda",
                                                                              dtype=torch.float16))
    with pytest.raises(ValueError, match="shape"):
        dst.rmsnorm_lm_head(a["hidden"], a["gamma"], a["w"], out_r=torch.empty(GBS + 1, device="cuda"))
    with pytest.raises(ValueError, match="dtype"):
        dst.rmsnorm_lm_head(a["hidden"], a["gamma"], a["w"],
                            ws=torch.empty(1 << 20, dtype=torch.float32, device="cuda"))
    with pytest.raises(ValueError, match="shape"):
        dst.lm_head(a["hidden"], a["w"], row_scale=torch.ones(GBS + 2, device="cuda"))
    with pytest.raises(ValueError, match="GPU tensor"):
        dst.lm_head(a["hidden"], a["w"], row_scale=torch.ones(GBS))
    with pytest.raises(ValueError, match="contiguous"):
        dst.topk(torch.empty(V, GBS, device="cuda").t(), K)
    with pytest.raises(ValueError, match="dtype"):
        dst.topk(logits, K, out_idx=torch.empty(GBS, K, dtype=torch.int64, device="cuda"))
    with pytest.raises(ValueError, match="shape"):
        dst.topk(logits, K, taps=torch.empty(GBS, 3, dtype=torch.int32, device="cuda"))
    with pytest.raises(ValueError, match="dtype"):
        dst.sample(vals, idx.long(), a["params"])
    with pytest.raises(ValueError, match="GPU tensor"):
        dst.sample(vals, idx, a["params"].cpu())
    with pytest.raises(ValueError, match="shape"):
        dst.sample(vals, idx, a["params"], out=torch.empty(GBS - 1, dtype=torch.int32, device="cuda"))
    # the valid calls still work after the rejected ones
    tok = dst.sample(vals, idx, a["params"])
    torch.cuda.synchronize()
    assert tok.shape == (GBS,)
