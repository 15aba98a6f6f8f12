"""The Muon step under HIP graph capture, and run-to-run determinism.

The library only enqueues kernels on the caller's stream (no allocation, no
synchronization, no memset), so a whole optimizer step can be captured once
and replayed.  Each replay is compared with the same step run eagerly on a
twin set of buffers, with unrelated eager work and synchronizations between
replays.  Every kernel reduces in a fixed order, so the comparison is
bit-for-bit.
"""

import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mx():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible MI355X")
    import matrix_aware_optimizer_step_amd as m
    m._lib.load()
    return m


SHAPES = [((2, 300, 700), torch.bfloat16), ((3, 520, 256), torch.bfloat16), ((1, 256, 128), torch.bfloat16)]


def make(mx, seed, compute):
    g = torch.Generator().manual_seed(seed)
    groups, grads = [], []
    for shape, dt in SHAPES:
        w = (0.02 * torch.randn(*shape, generator=g)).to(dt).cuda()
        gr = torch.randn(*shape, generator=g).to(dt).cuda()
        groups.append((w, gr))
        grads.append(gr)
    return mx.MuonStep(groups, compute=compute, lr=0.01, weight_decay=0.1), groups


@pytest.mark.parametrize("compute", [0, 1])
def test_graph_replays_match_eager(mx, compute):
    eager, eg = make(mx, 1, compute)
    graphed, gg = make(mx, 1, compute)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        graphed.step()  # warm-up outside capture, mirrored on the eager twin
    torch.cuda.current_stream().wait_stream(side)
    eager.step()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        graphed.step()
    noise = torch.randn(1 << 20, device="cuda")
    for r in range(4):
        eager.step()
        graph.replay()
        noise.mul_(1.0001).add_(0.5)  # unrelated eager work between replays
        torch.cuda.synchronize()
        for (we, _), (wg, _) in zip(eg, gg):
            assert torch.equal(we, wg), f"replay {r}: weights differ"
        for me, mg in zip(eager.momentum_buffers, graphed.momentum_buffers):
            assert torch.equal(me, mg), f"replay {r}: momentum differs"
        for oe, og in zip(eager.ortho_buffers, graphed.ortho_buffers):
            assert torch.equal(oe, og), f"replay {r}: orthogonalized update differs"


def test_steps_are_deterministic(mx):
    a, ga = make(mx, 7, 1)
    b, gb = make(mx, 7, 1)
    for _ in range(3):
        a.step()
        b.step()
    torch.cuda.synchronize()
    for (wa, _), (wb, _) in zip(ga, gb):
        assert torch.equal(wa, wb)
    for sa, sb in zip(a.sumsq_buffers, b.sumsq_buffers):
        assert torch.equal(sa, sb)
