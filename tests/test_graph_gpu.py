"""tail_forward under HIP graph capture (a decode loop replays one graph per
step): the library launches only kernels on the caller's stream (no
allocation, no memset, no synchronization), so a captured step replays
exactly.  Each replay gets new hidden rows, copied eagerly into the static
input between replays, and must match an eager tail_forward on the same
rows bitwise."""
import numpy as np
import pytest

from _cases import config, to_gpu

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import decode_sampling_tail_amd as dst  # noqa: E402


@pytest.mark.parametrize("cid,page", [(1, False), (3, False), (4, False), (4, True)])
def test_graph_replay_matches_eager(cid, page):
    inp = config(cid)
    g = to_gpu(inp)
    run = len(inp.params) - 1
    params = g["params"][run]
    f = dst.Forward(inp.gbs, inp.H, inp.V, inp.k, inp.H_u, inp.eps, inp.zero_pad, True, True,
                    page=page)
    eager = dst.Forward(inp.gbs, inp.H, inp.V, inp.k, inp.H_u, inp.eps, inp.zero_pad, True, True,
                        page=page)
    hidden = g["hidden"].clone()
    f(hidden, g["gamma"], g["w_t"], params)  # eager warm-up: one-time queries outside capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        f(hidden, g["gamma"], g["w_t"], params)
    torch.cuda.synchronize()
    rng = np.random.default_rng(cid)
    for rep in range(3):
        # new rows: a seeded permutation and scaling of the workload's rows
        perm = torch.from_numpy(rng.permutation(inp.gbs)).cuda()
        scale = float(rng.uniform(0.5, 2.0))
        new = (g["hidden"].float()[perm] * scale).to(g["hidden"].dtype).contiguous()
        hidden.copy_(new)
        graph.replay()
        want = eager(new, g["gamma"], g["w_t"], params)
        torch.cuda.synchronize()
        for key in ("logits", "vals", "idx", "tokens"):
            a = getattr(f, key).cpu().numpy()
            b = want[key].cpu().numpy()
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), (rep, key)
