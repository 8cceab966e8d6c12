"""No kernel reads workspace memory it has not written in the same call: a
workspace filled with 0xFF bytes before tail_forward gives bitwise the
outputs of a zero-filled one, on the gbs-1 (weight-streaming), gbs-64
(per-tile matrix cores, padded) and gbs-256 (large-batch kernel) workloads,
in both precisions, with the logits emitted and kept internal.  (0xFF bytes
are NaN as fp32 and the largest key as u32, so a stale read would show.)"""
import numpy as np
import pytest

from _cases import config, to_gpu

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import decode_sampling_tail_amd as dst  # noqa: E402


@pytest.mark.parametrize("cid,page", [(1, False), (3, False), (4, False), (4, True), (3, True)])
def test_poisoned_workspace_changes_nothing(cid, page):
    inp = config(cid)
    g = to_gpu(inp)
    run = len(inp.params) - 1
    params = g["params"][run]
    for emit in (True, False):
        outs = []
        for fill in (0x00, 0xFF):
            f = dst.Forward(inp.gbs, inp.H, inp.V, inp.k, inp.H_u, inp.eps, inp.zero_pad, True,
                            emit, page=page)
            f.ws.fill_(fill)
            if f.logits is not None:
                f.logits.fill_(fill)
            f.vals.fill_(0)
            f.idx.fill_(0)
            f.tokens.fill_(0)
            torch.cuda.synchronize()
            out = f(g["hidden"], g["gamma"], g["w_t"], params)
            torch.cuda.synchronize()
            outs.append({k: v.cpu().numpy() for k, v in out.items() if v is not None})
            del f
        for key in outs[0]:
            assert np.array_equal(outs[0][key].view(np.uint8), outs[1][key].view(np.uint8)), \
                (cid, page, emit, key)
    del g
    torch.cuda.empty_cache()
