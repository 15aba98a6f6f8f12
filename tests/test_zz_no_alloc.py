"""GPU check of the allocation-free momentum entry point.

muon_momentum_grouped_noalloc keeps its partial sums in the library's static
device scratch instead of a caller workspace.  Two calls in a row (the
second with fewer and smaller matrices, so stale partials of the first call
sit in the scratch) must give the momentum, the Nesterov blend and the sums
of squares of muon_momentum_grouped bit for bit, and the oracle's values to
the fp32 elementwise bound.
"""

import numpy as np
import pytest
import torch

from oracle import oracle as O
from workloads import synth

pytestmark = pytest.mark.gpu

TOL_EW = 1e-6


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible MI355X")
    from matrix_aware_optimizer_step_amd import _lib as L
    L.load()
    return L


def f64(t):
    return t.detach().to(torch.float64).cpu().numpy()


def desc(t):
    from matrix_aware_optimizer_step_amd import muon as mu
    return mu.batch(t).desc


def run(L, shapes, gdtype, noalloc, seed):
    """One call over groups of the given (count, rows, cols); returns the
    gradients, the momentum before, and the outputs."""
    dev = torch.device("cuda:0")
    grads, moms, nouts, sums = [], [], [], []
    for gi, (c, r, k) in enumerate(shapes):
        g = torch.stack([synth.gaussian(r, k, seed=seed + 100 * gi + i) for i in range(c)]).to(gdtype).to(dev)
        m = torch.stack([0.5 * synth.gaussian(r, k, seed=seed + 100 * gi + 50 + i) for i in range(c)]).to(dev)
        grads.append(g)
        moms.append(m)
        nouts.append(torch.empty(c, r, k, dtype=torch.float32, device=dev))
        sums.append(torch.full((c,), float("nan"), dtype=torch.float32, device=dev))
    m_before = [m.clone() for m in moms]
    stream = torch.cuda.current_stream().cuda_stream
    gd, md, nd = [desc(t) for t in grads], [desc(t) for t in moms], [desc(t) for t in nouts]
    if noalloc:
        L.muon_momentum_grouped_noalloc(gd, md, nd, [s.data_ptr() for s in sums], 0.95, True, stream)
    else:
        need = L.muon_momentum_grouped_workspace([s[0] for s in shapes], [s[1] for s in shapes],
                                                 [s[2] for s in shapes])
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
        L.muon_momentum_grouped(gd, md, nd, [s.data_ptr() for s in sums], 0.95, True, ws.data_ptr(), need, stream)
    torch.cuda.synchronize()
    return grads, m_before, moms, nouts, sums


@pytest.mark.parametrize("shapes,gdtype", [
    ([(3, 300, 700), (2, 1024, 4096), (5, 128, 4096)], torch.bfloat16),   # first call: larger
    ([(1, 64, 96), (2, 33, 17)], torch.float32),                          # second call: smaller, ragged
])
def test_noalloc_momentum_matches_grouped_entry_point(lib, shapes, gdtype):
    print(f"noalloc momentum {shapes} {gdtype}", flush=True)
    a = run(lib, shapes, gdtype, noalloc=False, seed=17)
    b = run(lib, shapes, gdtype, noalloc=True, seed=17)
    for gi in range(len(shapes)):
        for name, x, y in (("momentum", a[2][gi], b[2][gi]), ("nesterov", a[3][gi], b[3][gi]),
                           ("sumsq", a[4][gi], b[4][gi])):
            assert torch.equal(x, y), f"group {gi} {name} differs from muon_momentum_grouped"
        for i in range(shapes[gi][0]):
            M, N = O.momentum(f64(b[1][gi][i]), f64(b[0][gi][i]), 0.95, True)
            assert O.relative_frobenius_error(f64(b[2][gi][i]), M) <= TOL_EW
            assert O.relative_frobenius_error(f64(b[3][gi][i]), N) <= TOL_EW
            ss = O.frobenius_sumsq(N)
            assert abs(float(b[4][gi][i]) - ss) <= TOL_EW * ss


def test_noalloc_momentum_refuses_more_than_its_scratch(lib):
    # 17 matrices of 2^30 elements need more partial sums than the scratch
    # holds; refused before anything is enqueued (the descriptors are never read)
    big = lib.MuonBatch(None, 0x10000, 1 << 30, 17, 32768, 32768, 32768, lib.MUON_F32, 0)
    with pytest.raises(lib.MuonError) as e:
        lib.muon_momentum_grouped_noalloc([big], [big], [big], [0x10000], 0.95, True, 0)
    assert e.value.status == 3
