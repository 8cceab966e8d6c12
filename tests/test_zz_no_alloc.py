"""tail_forward_noalloc, the entry point for callers that cannot allocate, uses
the library's static scratch instead of a workspace argument and must give
the outputs of tail_forward on the same inputs: here bitwise (the same
kernels run in the same order), checked on two calls in a row, the second
with a smaller batch and vocabulary, so the second call reuses scratch that
the first one left filled.  A call that needs more than TAIL_SCRATCH_BYTES is
refused before anything is enqueued."""
import numpy as np
import pytest
import torch

import decode_sampling_tail_amd as dst

pytestmark = pytest.mark.gpu


def inputs(gbs, H, V, seed, dtype=torch.float32):
    g = torch.Generator().manual_seed(seed)
    hidden = torch.randn(gbs, H, generator=g).to(dtype)
    gamma = 1.0 + 0.1 * torch.randn(H, generator=g)
    w = (0.05 * torch.randn(H, V, generator=g)).to(torch.bfloat16)
    params = torch.stack([torch.randint(1, 65, (gbs,), generator=g).float(),
                          0.5 + 0.5 * torch.rand(gbs, generator=g),
                          0.3 + 1.2 * torch.rand(gbs, generator=g),
                          torch.rand(gbs, generator=g)], dim=1)
    params[::4, 2] = 0.0  # some greedy rows
    dev = torch.device("cuda")
    return hidden.to(dev), gamma.to(dev), w.to(dev), params.contiguous().to(dev)


def run_both(gbs, H, V, k, emit, seed, dtype=torch.float32):
    hidden, gamma, w, params = inputs(gbs, H, V, seed, dtype)
    ref = dst.Forward(gbs, H, V, k, emit_logits=emit)
    want = {key: (None if t is None else t.clone()) for key, t in ref(hidden, gamma, w, params).items()}
    got = dst.Forward(gbs, H, V, k, emit_logits=emit).noalloc(hidden, gamma, w, params)
    torch.cuda.synchronize()
    for key in ("vals", "idx", "tokens") + (("logits",) if emit else ()):
        a, b = want[key].cpu().numpy(), got[key].cpu().numpy()
        assert np.array_equal(a.view(np.uint32) if a.dtype == np.float32 else a,
                              b.view(np.uint32) if b.dtype == np.float32 else b), key


def test_noalloc_matches_forward_twice_then_smaller():
    # first: 200 rows (the large-batch matrix-core path), logits emitted
    run_both(200, 512, 32768, 256, True, seed=1)
    # second, smaller: 5 rows (the per-tile path), logits kept in the scratch
    run_both(5, 256, 8192, 64, False, seed=2, dtype=torch.bfloat16)
    # and the weight-streaming path with the scratch holding the logits
    run_both(2, 384, 4096, 16, False, seed=3, dtype=torch.float16)


def test_noalloc_refuses_more_than_the_scratch():
    gbs, H, V, k = 96, 2880, 201088, 256  # the logits alone need 77 MB
    need = dst.workspace_size(gbs, H, H, V, k, 0)
    assert need > dst.SCRATCH_BYTES
    f = dst.Forward(gbs, H, V, k, emit_logits=False)
    dev = torch.device("cuda")
    hidden = torch.zeros(gbs, H, device=dev)
    gamma = torch.ones(H, device=dev)
    w = torch.zeros(H, V, dtype=torch.bfloat16, device=dev)
    f.vals.fill_(7.0)
    with pytest.raises(dst.TailError) as e:
        f.noalloc(hidden, gamma, w)
    assert e.value.status == dst.ERR_SCRATCH_LIMIT
    torch.cuda.synchronize()
    assert bool((f.vals == 7.0).all())  # nothing was enqueued
