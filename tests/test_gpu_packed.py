"""GPU parity of the packed pair (muon_momentum_packed_grouped then
muon_orthogonalize_packed_grouped), the path MuonStep takes by default.

The momentum kernel writes the Nesterov blend N into the Newton-Schulz
workspace unnormalized, and the first Newton-Schulz step divides by
sqrt(sumsq) + eps in its epilogues.  Against the fp64 oracle:
* momentum (fp32): bit-identical to the separate muon_momentum_grouped and
  within 1e-6 of the oracle; sum of squares within 1e-6 (it is added per
  64 x 64 tile here, per block there);
* Newton-Schulz, fp32 path: relative Frobenius error <= 1e-5;
* Newton-Schulz, bf16 path: <= 3e-2;
* the updated weight: fp32 within 1e-6 of the oracle's apply step on the
  GPU's own Newton-Schulz output, bf16 within one rounding of it.
Shapes cover both tile classes (128 and 256), tall and wide matrices, ragged
edges, row blocks with ld > cols, pointer arrays and several groups in one
launch.
"""

import numpy as np
import pytest
import torch

from oracle import oracle as O

pytestmark = pytest.mark.gpu

TOL_EW = 1e-6
TOL_F32 = 1e-5
TOL_BF16 = 3e-2


@pytest.fixture(scope="module")
def mx():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible MI355X")
    import matrix_aware_optimizer_step_amd as m
    m._lib.load()
    return m


def f64(t):
    return t.detach().to(torch.float64).cpu().numpy()


def bf16_of(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).to(torch.float64).numpy()


def bf16_ulp(x):
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    return np.where(ax > 0, 2.0 ** (e - 7), 2.0 ** -133)


def randn(shape, seed, dtype, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (scale * torch.randn(*shape, generator=g, dtype=torch.float32)).to(dtype).cuda()


def check_weight(W_got, W0, O_got, lr, wd, dtype):
    W_exact = O.apply_update(W0, O_got, lr, wd)
    if dtype == torch.float32:
        assert O.relative_frobenius_error(W_got, W_exact) <= TOL_EW
    else:
        tol = bf16_ulp(W_exact) + TOL_EW * np.max(np.abs(W_exact))
        assert np.all(np.abs(W_got - bf16_of(W_exact)) <= tol)


CASES = [
    # (count, rows, cols), grad/weight dtype, compute
    ((1, 256, 128), torch.float32, 0),     # tall, fp32 path
    ((1, 256, 128), torch.float32, 1),
    ((3, 100, 72), torch.bfloat16, 1),     # tall, ragged, 128-tile class
    ((2, 130, 300), torch.bfloat16, 1),    # wide, ragged, 256-tile class
    ((2, 520, 256), torch.bfloat16, 1),    # tall, 256-tile class, several row tiles
    ((1, 33, 50), torch.float32, 0),       # scalar (unaligned) momentum path
    ((2, 300, 700), torch.bfloat16, 0),    # fp32 compute from bf16 gradients
]


@pytest.mark.parametrize("shape,dtype,compute", CASES)
@pytest.mark.parametrize("nesterov", [True, False])
def test_packed_step_matches_oracle(mx, shape, dtype, compute, nesterov):
    print(f"packed step {shape} {dtype} compute={compute} nesterov={nesterov}", flush=True)
    c, m, n = shape
    lr, wd = 1.0, 0.5
    W = randn(shape, 11, dtype, 0.02)
    G = torch.empty(shape, dtype=dtype, device="cuda")
    step = mx.MuonStep([(W, G)], compute=compute, nesterov=nesterov, lr=lr, weight_decay=wd)
    assert step.packed
    Mo = [np.zeros((m, n)) for _ in range(c)]
    # the fp32 path writes its output in the weight's dtype: a bf16 output adds
    # one rounding (relative 2^-9 per entry) to the fp32 bound
    tol = (TOL_F32 + (2.0 ** -9 if dtype == torch.bfloat16 else 0.0)) if compute == 0 else TOL_BF16
    for t in range(1, 4):
        G.copy_(randn(shape, 100 + t, dtype, 3.0))
        W0 = [f64(W[i]) for i in range(c)]
        step.step()
        torch.cuda.synchronize()
        for i in range(c):
            Mo[i], N = O.momentum(Mo[i], f64(G[i]), 0.95, nesterov)
            assert O.relative_frobenius_error(f64(step.momentum_buffers[0][i]), Mo[i]) <= TOL_EW
            ss = O.frobenius_sumsq(N)
            assert abs(float(step.sumsq_buffers[0][i]) - ss) <= TOL_EW * ss
            O_got = f64(step.ortho_buffers[0][i])
            err = O.relative_frobenius_error(O_got, O.newton_schulz(N, 5))
            assert err <= tol, (t, i, err)
            check_weight(f64(W[i]), W0[i], O_got, lr, wd, dtype)


def test_packed_momentum_bit_identical_to_separate_calls(mx):
    """Same momentum bits as the unpacked path; Newton-Schulz outputs differ
    only by rounding (both within the bf16 bound of the oracle)."""
    shapes = [(2, 300, 700), (3, 1024, 256), (1, 128, 4096)]
    runs = []
    for packed in (True, False):
        groups = [(randn(s, 20 + k, torch.bfloat16, 0.02), randn(s, 40 + k, torch.bfloat16)) for k, s in
                  enumerate(shapes)]
        st = mx.MuonStep(groups, lr=0.01, weight_decay=0.1, packed=packed)
        assert st.packed == packed
        st.step()
        st.step()
        torch.cuda.synchronize()
        runs.append((st, groups))
    (a, ga), (b, gb) = runs
    for k, s in enumerate(shapes):
        assert torch.equal(a.momentum_buffers[k], b.momentum_buffers[k]), k
        assert torch.allclose(a.sumsq_buffers[k], b.sumsq_buffers[k], rtol=1e-6, atol=0), k
        for i in range(s[0]):
            G = f64(gb[k][1][i])  # the same gradient at both steps
            M1, _ = O.momentum(np.zeros_like(G), G)
            _, N2 = O.momentum(M1, G)
            want = O.newton_schulz(N2, 5)
            assert O.relative_frobenius_error(f64(a.ortho_buffers[k][i]), want) <= TOL_BF16
            assert O.relative_frobenius_error(f64(b.ortho_buffers[k][i]), want) <= TOL_BF16


def test_packed_row_blocks_pointer_arrays_and_many_groups(mx):
    """Column slices of wider weights (ld > cols), per-head row blocks,
    pointer-array groups and ten shape groups (two launches per stage) in one
    MuonStep."""
    wide_w = randn((2, 300, 520), 7, torch.bfloat16, 0.02)
    wide_g = randn((2, 300, 520), 8, torch.bfloat16)
    cols_w = wide_w[:, :, :260]   # (2, 300, 260): the left half of each wider matrix, ld 520
    cols_g = wide_g[:, :, :260]
    heads_w = randn((512, 1024), 9, torch.bfloat16, 0.02).view(4, 128, 1024)
    heads_g = randn((512, 1024), 10, torch.bfloat16).view(4, 128, 1024)
    lists = ([randn((96, 200), 30 + i, torch.bfloat16, 0.02) for i in range(3)],
             [randn((96, 200), 40 + i, torch.bfloat16) for i in range(3)])
    extra = [(randn((1, 64 + 16 * k, 96), 60 + k, torch.float32, 0.02), randn((1, 64 + 16 * k, 96), 80 + k,
                                                                             torch.float32)) for k in range(7)]
    groups = [(cols_w, cols_g), (heads_w, heads_g), lists] + extra
    views = [(cols_w[i], cols_g[i], torch.bfloat16) for i in range(2)] + \
            [(heads_w[i], heads_g[i], torch.bfloat16) for i in range(4)] + \
            [(lists[0][i], lists[1][i], torch.bfloat16) for i in range(3)] + [(w[0], g[0], torch.float32) for w, g in extra]
    W0 = [f64(w) for w, _, _ in views]
    Gs = [f64(g) for _, g, _ in views]
    step = mx.MuonStep(groups, lr=0.5, weight_decay=0.2)
    assert step.packed and len(step.chunks) == 2
    assert step.w[0].desc.ld == 520
    step.step()
    torch.cuda.synchronize()
    got_o = [f64(step.ortho_buffers[0][i]) for i in range(2)] + [f64(step.ortho_buffers[1][i]) for i in range(4)] + \
            [f64(step.ortho_buffers[2][i]) for i in range(3)] + [f64(step.ortho_buffers[3 + k][0]) for k in range(7)]
    for j, (w, _, dt) in enumerate(views):
        _, N = O.momentum(np.zeros_like(Gs[j]), Gs[j])
        assert O.relative_frobenius_error(got_o[j], O.newton_schulz(N, 5)) <= TOL_BF16, j
        check_weight(f64(w), W0[j], got_o[j], 0.5, 0.2, dt)
    # the right halves of the wider weights are not part of any matrix: untouched
    assert torch.equal(wide_w[:, :, 260:], randn((2, 300, 520), 7, torch.bfloat16, 0.02)[:, :, 260:])


@pytest.mark.parametrize("compute", [0, 1])
def test_packed_zero_gradient_gives_pure_decay(mx, compute):
    W = randn((2, 96, 160), 3, torch.float32, 0.02)
    W0 = f64(W)
    G = torch.zeros((2, 96, 160), dtype=torch.float32, device="cuda")
    step = mx.MuonStep([(W, G)], compute=compute, lr=0.1, weight_decay=0.5)
    step.step()
    torch.cuda.synchronize()
    assert torch.count_nonzero(step.ortho_buffers[0]).item() == 0
    assert np.array_equal(f64(W), (W0.astype(np.float32) * np.float32(1.0 - 0.1 * 0.5)).astype(np.float64))


@pytest.mark.parametrize("steps", [1, 2])
def test_packed_short_iterations_through_the_c_abi(mx, steps):
    """The pair called directly, with K = 1 (the first step is also the last:
    its update writes the caller's output) and K = 2."""
    from matrix_aware_optimizer_step_amd import _lib as L
    from matrix_aware_optimizer_step_amd import muon as mu
    shapes = [(2, 260, 130), (3, 64, 200)]
    Gs = [randn(s, 200 + k, torch.bfloat16, 2.0) for k, s in enumerate(shapes)]
    Ms = [torch.zeros(s, dtype=torch.float32, device="cuda") for s in shapes]
    Os = [torch.empty(s, dtype=torch.float32, device="cuda") for s in shapes]
    ss = [torch.empty(s[0], dtype=torch.float32, device="cuda") for s in shapes]
    need = L.muon_packed_grouped_workspace([s[0] for s in shapes], [s[1] for s in shapes], [s[2] for s in shapes],
                                           L.MUON_BF16)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    L.muon_momentum_packed_grouped([mu.batch(g).desc for g in Gs], [mu.batch(m).desc for m in Ms],
                                   [s.data_ptr() for s in ss], 0.9, True, L.MUON_BF16, ws.data_ptr(), need, st)
    L.muon_orthogonalize_packed_grouped([s.data_ptr() for s in ss], [mu.batch(o).desc for o in Os], steps, 3.4445,
                                        -4.7750, 2.0315, 1e-7, L.MUON_BF16, ws.data_ptr(), need, st)
    torch.cuda.synchronize()
    for k, s in enumerate(shapes):
        for i in range(s[0]):
            _, N = O.momentum(np.zeros(s[1:]), f64(Gs[k][i]), 0.9, True)
            err = O.relative_frobenius_error(f64(Os[k][i]), O.newton_schulz(N, steps))
            assert err <= TOL_BF16, (k, i, err)


def test_zero_steps_fall_back_to_the_separate_calls(mx):
    W = randn((1, 64, 96), 5, torch.float32, 0.02)
    G = randn((1, 64, 96), 6, torch.float32)
    step = mx.MuonStep([(W, G)], compute=0, steps=0, lr=0.1, weight_decay=0.0)
    step.step()
    torch.cuda.synchronize()
    _, N = O.momentum(np.zeros((64, 96)), f64(G[0]))
    assert O.relative_frobenius_error(f64(step.ortho_buffers[0][0]), O.newton_schulz(N, 0)) <= TOL_EW
