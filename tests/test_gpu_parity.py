"""GPU parity of libmuon355 against the fp64 oracle, called through the C ABI.

Tolerances (written here, derived in the design notes):
* momentum, sum of squares and apply, fp32: relative error <= 1e-6;
* bf16 outputs of those kernels: within one bf16 rounding of the oracle;
* Newton-Schulz, fp32 path: relative Frobenius error <= 1e-5;
* Newton-Schulz, bf16 MFMA path: relative Frobenius error <= 3e-2.
Sizes span several tiles and ragged tails while the oracle stays fast.
"""

import math

import numpy as np
import pytest
import torch

from oracle import oracle as O
from workloads import synth

pytestmark = pytest.mark.gpu

TOL_EW = 1e-6
TOL_F32 = 1e-5
TOL_BF16 = 3e-2


@pytest.fixture(scope="module")
def mx():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible MI355X")
    import matrix_aware_optimizer_step_amd as m
    m._lib.load()  # raises when the library is missing: there is no fallback
    return m


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to(torch.float64).cpu().numpy()


def bf16_of(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).to(torch.float64).numpy()


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bf16 numbers at |x| (8 significant bits)."""
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    return np.where(ax > 0, 2.0 ** (e - 7), 2.0 ** -133)


def within_one_bf16_rounding(got: np.ndarray, exact: np.ndarray) -> bool:
    """A bf16 result computed in fp32 and rounded once differs from the exact
    value rounded to bf16 by at most one bf16 step, plus the fp32 error of the
    computation before rounding (bounded normwise by 1e-6 of the largest
    entry: entries that nearly cancel carry it in full)."""
    tol = bf16_ulp(exact) + TOL_EW * np.max(np.abs(exact))
    return bool(np.all(np.abs(got - bf16_of(exact)) <= tol))


def rel(got, want):
    return O.relative_frobenius_error(got, want)


def randn(shape, seed, dtype, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (scale * torch.randn(*shape, generator=g, dtype=torch.float32)).to(dtype).cuda()


# ------------------------------------------------------------------ momentum

MOM_CASES = [
    ((1, 256, 128), torch.float32),   # the single fp32 gradient
    ((3, 100, 72), torch.bfloat16),   # ragged rows, vector path
    ((2, 33, 50), torch.float32),     # cols not a multiple of 8: scalar path
    ((1, 8191, 8), torch.bfloat16),   # many rows, one block boundary
]


@pytest.mark.parametrize("shape,gdtype", MOM_CASES)
@pytest.mark.parametrize("nesterov", [True, False])
def test_momentum_three_steps(mx, shape, gdtype, nesterov):
    beta = 0.95
    M = torch.zeros(shape, dtype=torch.float32, device="cuda")
    N = torch.empty(shape, dtype=gdtype, device="cuda")
    ss = torch.empty(shape[0], dtype=torch.float32, device="cuda")
    Mo = [np.zeros(shape[1:]) for _ in range(shape[0])]
    for t in range(1, 4):
        G = randn(shape, 100 + t, gdtype, 3.0)
        mx.momentum(G, M, N, ss, beta, nesterov)
        torch.cuda.synchronize()
        for i in range(shape[0]):
            Mo[i], No = O.momentum(Mo[i], f64(G[i]), beta, nesterov)
            assert rel(f64(M[i]), Mo[i]) <= TOL_EW
            assert np.max(np.abs(f64(M[i]) - Mo[i])) <= TOL_EW * np.max(np.abs(Mo[i]))
            if gdtype == torch.float32:
                assert rel(f64(N[i]), No) <= TOL_EW
            else:
                assert within_one_bf16_rounding(f64(N[i]), No)
            want = O.frobenius_sumsq(No)
            assert abs(float(ss[i]) - want) <= TOL_EW * want


def test_momentum_row_blocks_and_pointer_arrays(mx):
    """ld > cols (row blocks of a wider matrix) and a pointer-array batch."""
    big = randn((3, 64, 160), 7, torch.bfloat16)
    G = big[:, :, 16:144]                       # ld 160, cols 128
    M = torch.zeros(3, 64, 128, device="cuda")
    Nl = [torch.empty(64, 128, dtype=torch.bfloat16, device="cuda") for _ in range(3)]
    ss = torch.empty(3, device="cuda")
    mx.momentum(G, M, Nl, ss, 0.9, True)
    torch.cuda.synchronize()
    for i in range(3):
        Mo, No = O.momentum(np.zeros((64, 128)), f64(G[i]), 0.9, True)
        assert rel(f64(M[i]), Mo) <= TOL_EW
        assert within_one_bf16_rounding(f64(Nl[i]), No)


def test_momentum_nonfinite_propagates(mx):
    G = randn((1, 64, 64), 3, torch.float32)
    G[0, 5, 7] = float("nan")
    M = torch.zeros(1, 64, 64, device="cuda")
    N = torch.empty(1, 64, 64, device="cuda")
    ss = torch.empty(1, device="cuda")
    mx.momentum(G, M, N, ss, 0.95, True)
    torch.cuda.synchronize()
    assert not math.isfinite(float(ss[0]))


GROUPED_EW = [((3, 100, 72), torch.bfloat16), ((2, 33, 50), torch.float32), ((1, 640, 256), torch.bfloat16),
              ((4, 17, 8), torch.bfloat16)]  # 16-byte and element paths, several blocks, tiny matrices


@pytest.mark.parametrize("nesterov", [True, False])
def test_momentum_grouped_equals_separate_calls(mx, nesterov):
    """One grouped launch over shape classes (vector and element paths)
    against separate muon_momentum calls, bit for bit, from a nonzero state;
    and against the oracle."""
    beta = 0.9
    grads = [randn(s, 200 + k, dt, 3.0) for k, (s, dt) in enumerate(GROUPED_EW)]
    m0 = [randn(s, 300 + k, torch.float32) for k, (s, _) in enumerate(GROUPED_EW)]
    M1, M2 = [m.clone() for m in m0], [m.clone() for m in m0]
    N1 = [torch.empty(s, dtype=dt, device="cuda") for s, dt in GROUPED_EW] if nesterov else None
    N2 = [torch.empty(s, dtype=dt, device="cuda") for s, dt in GROUPED_EW] if nesterov else None
    ss1 = [torch.empty(s[0], device="cuda") for s, _ in GROUPED_EW]
    ss2 = [torch.empty(s[0], device="cuda") for s, _ in GROUPED_EW]
    for k in range(len(GROUPED_EW)):
        mx.momentum(grads[k], M1[k], N1[k] if nesterov else None, ss1[k], beta, nesterov)
    mx.momentum_grouped(grads, M2, N2, ss2, beta, nesterov)
    torch.cuda.synchronize()
    for k, (s, dt) in enumerate(GROUPED_EW):
        assert torch.equal(M1[k], M2[k]) and torch.equal(ss1[k], ss2[k]), f"group {k}"
        if nesterov:
            assert torch.equal(N1[k], N2[k]), f"group {k}"
        for i in range(s[0]):
            Mo, No = O.momentum(f64(m0[k][i]), f64(grads[k][i]), beta, nesterov)
            assert rel(f64(M2[k][i]), Mo) <= TOL_EW
            want = O.frobenius_sumsq(No)
            assert abs(float(ss2[k][i]) - want) <= TOL_EW * want


def test_apply_grouped_equals_separate_calls(mx):
    lr, wd = 1.0, 0.5
    w0 = [randn(s, 400 + k, dt, 0.02) for k, (s, dt) in enumerate(GROUPED_EW)]
    Od = [randn(s, 500 + k, dt, 0.05) for k, (s, dt) in enumerate(GROUPED_EW)]
    W1, W2 = [w.clone() for w in w0], [w.clone() for w in w0]
    for k in range(len(GROUPED_EW)):
        mx.apply(W1[k], Od[k], lr, wd, 0, 0.2)
    mx.apply_grouped(W2, Od, lr, wd, 0, 0.2)
    torch.cuda.synchronize()
    for k, (s, dt) in enumerate(GROUPED_EW):
        assert torch.equal(W1[k], W2[k]), f"group {k}"
        for i in range(s[0]):
            want = O.apply_update(f64(w0[k][i]), f64(Od[k][i]), lr, wd, 0, 0.2)
            if dt == torch.float32:
                assert rel(f64(W2[k][i]), want) <= TOL_EW
            else:
                assert within_one_bf16_rounding(f64(W2[k][i]), want)


def test_apply_grouped_pointer_arrays_equal_strided(mx):
    # groups passed as lists of 2-D tensors (device pointer arrays owned by
    # the binding's batches) give the same bits as strided batches
    lr, wd = 1.0, 0.5
    w0 = [randn(s, 600 + k, dt, 0.02) for k, (s, dt) in enumerate(GROUPED_EW)]
    Od = [randn(s, 700 + k, dt, 0.05) for k, (s, dt) in enumerate(GROUPED_EW)]
    W1, W2 = [w.clone() for w in w0], [w.clone() for w in w0]
    mx.apply_grouped(W1, Od, lr, wd, 0, 0.2)
    mx.apply_grouped([list(w.unbind(0)) for w in W2], [list(o.unbind(0)) for o in Od], lr, wd, 0, 0.2)
    torch.cuda.synchronize()
    for k in range(len(GROUPED_EW)):
        assert torch.equal(W1[k], W2[k]), f"group {k}"


# --------------------------------------------------------------------- apply

@pytest.mark.parametrize("mode", [mx_mode for mx_mode in (0, 1, 2)])
@pytest.mark.parametrize("wdtype,shape", [(torch.float32, (2, 96, 200)), (torch.bfloat16, (1, 300, 64)),
                                          (torch.float32, (1, 37, 51))])
def test_apply(mx, mode, wdtype, shape):
    lr, wd = 1.0, 0.5  # the update term dominates, so a mistake in it cannot hide
    W = randn(shape, 11, wdtype, 0.02)
    Od = randn(shape, 12, wdtype, 0.05)
    W0 = f64(W)
    mx.apply(W, Od, lr, wd, mode, 0.2)
    torch.cuda.synchronize()
    for i in range(shape[0]):
        want = O.apply_update(W0[i], f64(Od[i]), lr, wd, mode, 0.2)
        if wdtype == torch.float32:
            assert rel(f64(W[i]), want) <= TOL_EW
        else:
            assert within_one_bf16_rounding(f64(W[i]), want)


# ------------------------------------------------------------ Newton-Schulz

def run_ns(mx, N, compute, steps=5, coeffs=O.QUINTIC, out_dtype=None, eps=O.EPS):
    out = torch.empty(N.shape, dtype=out_dtype or N.dtype, device="cuda")
    mx.orthogonalize(N, out, None, steps, coeffs, eps, compute, device="cuda")
    torch.cuda.synchronize()
    return out


NS_F32_SHAPES = [(256, 128), (128, 256), (200, 333), (333, 200), (300, 300), (1, 64), (64, 1),
                 (700, 520), (129, 900), (40, 2000)]


@pytest.mark.parametrize("shape", NS_F32_SHAPES)
def test_ns_f32(mx, shape):
    N = randn((1,) + shape, sum(shape), torch.float32)
    out = run_ns(mx, N, mx.MUON_F32)
    want = O.newton_schulz(f64(N[0]), 5)
    assert rel(f64(out[0]), want) <= TOL_F32


NS_BF16_SHAPES = [(256, 128), (512, 1024), (1024, 512), (384, 1000), (130, 2000), (1000, 130), (300, 300),
                  (768, 2048)]


@pytest.mark.parametrize("shape", NS_BF16_SHAPES)
def test_ns_bf16(mx, shape):
    G = synth.rank1_sum(*shape, seed=shape[0] * 7 + shape[1], inner=512)
    N = G.to(torch.bfloat16).unsqueeze(0).cuda()
    out = run_ns(mx, N, mx.MUON_BF16)
    want = O.newton_schulz(f64(N[0]), 5)
    assert rel(f64(out[0]), want) <= TOL_BF16


ILL_CASES = [("kappa", 128, 4096), ("kappa", 300, 700), ("kappa", 1100, 260), ("power", 1024, 4096),
             ("power", 520, 1500)]


def ill_conditioned(kind, rows, cols):
    seed = rows * 31 + cols
    if kind == "kappa":
        return synth.condition_number(rows, cols, seed)  # singular values 1 .. 1e-4, geometric
    return synth.power_law(rows, cols, seed)             # singular values 1/k


@pytest.mark.parametrize("compute,tol", [(0, TOL_F32), (1, TOL_BF16)])
@pytest.mark.parametrize("kind,rows,cols", ILL_CASES)
def test_ns_ill_conditioned(mx, compute, tol, kind, rows, cols):
    """Ill-conditioned fp32 inputs: the iteration amplifies rounding in the
    directions of small singular values about a-fold per step, so these
    cases bound how and where each path rounds (the fp32 input is what the
    oracle sees; the bf16 path keeps its fp32 copy of X from it)."""
    N = ill_conditioned(kind, rows, cols).unsqueeze(0).cuda()
    out = run_ns(mx, N, compute, out_dtype=torch.float32)
    want = O.newton_schulz(f64(N[0]), 5)
    assert rel(f64(out[0]), want) <= tol


@pytest.mark.parametrize("compute,tol", [(0, TOL_F32), (1, TOL_BF16)])
@pytest.mark.parametrize("coeffs,steps", [(O.TRACK3, 12), (O.CUBIC, 5), (O.CUBIC, 10)])
@pytest.mark.parametrize("kind,rows,cols", [("gauss", 300, 700), ("gauss", 700, 300), ("kappa", 128, 4096)])
def test_ns_other_coefficient_sets(mx, compute, tol, coeffs, steps, kind, rows, cols):
    """The pages' other iterations on the same kernels: the convergent
    'Track-3' quintic run for 12 steps and the classical cubic.

    The fp32 bound is the Muon iteration's 1e-5 scaled by how much more this
    iteration amplifies rounding: in the directions of small singular values
    each step multiplies a perturbation by the map's slope at zero, a, so by
    a^K over K steps, against 3.4445^5 for Muon's five quintic steps
    (Track-3 x 12: 2^12 / 3.4445^5 = 8.5; the cubic stays at 1e-5)."""
    if compute == 0:
        tol = TOL_F32 * max(1.0, coeffs[0] ** steps / O.QUINTIC[0] ** 5)
    if kind == "gauss":
        N = randn((1, rows, cols), rows + cols, torch.float32)
    else:
        N = ill_conditioned(kind, rows, cols).unsqueeze(0).cuda()
    out = run_ns(mx, N, compute, steps=steps, coeffs=coeffs, out_dtype=torch.float32)
    want = O.newton_schulz(f64(N[0]), steps, coeffs)
    assert rel(f64(out[0]), want) <= tol


@pytest.mark.parametrize("compute,tol", [(0, TOL_F32), (1, TOL_BF16)])
@pytest.mark.parametrize("coeffs", [(1.0, 0.0, 0.0), (0.0, 1.0, 0.0), (0.0, 0.0, 1.0), (0.5, -0.25, 0.125)])
@pytest.mark.parametrize("shape", [(300, 700), (700, 300), (96, 520)])
def test_ns_single_stage(mx, compute, tol, coeffs, shape):
    """One step with coefficients that isolate the identity, the Gram-times-X
    and the polynomial term, so each GEMM stage is checked on its own."""
    dt = torch.float32 if compute == 0 else torch.bfloat16
    N = randn((1,) + shape, 5, dt)
    out = run_ns(mx, N, compute, steps=1, coeffs=coeffs, out_dtype=torch.float32)
    want = O.newton_schulz(f64(N[0]), 1, coeffs)
    assert rel(f64(out[0]), want) <= tol


@pytest.mark.parametrize("compute", [0, 1])
def test_ns_zero_steps_is_normalized_input(mx, compute):
    N = randn((2, 70, 90), 9, torch.float32)
    out = run_ns(mx, N, compute, steps=0)
    for i in range(2):
        assert rel(f64(out[i]), O.newton_schulz(f64(N[i]), 0)) <= 1e-6


@pytest.mark.parametrize("compute", [0, 1])
def test_ns_zero_input_gives_zero(mx, compute):
    N = torch.zeros(1, 64, 96, device="cuda")
    out = run_ns(mx, N, compute)
    assert torch.count_nonzero(out).item() == 0


def test_ns_orthogonal_input(mx):
    q, _ = torch.linalg.qr(torch.randn(512, 128, generator=torch.Generator().manual_seed(4), dtype=torch.float64))
    Q = q.T.contiguous()  # 128 x 512, orthonormal rows
    out = run_ns(mx, Q.float().unsqueeze(0).cuda(), mx.MUON_F32)
    c = 1.0 / (math.sqrt(128) + O.EPS)
    for _ in range(5):
        c = 3.4445 * c - 4.7750 * c ** 3 + 2.0315 * c ** 5
    assert rel(f64(out[0]), c * Q.numpy()) <= TOL_F32


def test_ns_transpose_equivariance(mx):
    N = randn((1, 200, 500), 21, torch.float32)
    a = run_ns(mx, N, mx.MUON_F32)
    b = run_ns(mx, N.transpose(1, 2).contiguous(), mx.MUON_F32)
    # the two orientations sum the squares in different orders
    assert rel(f64(b[0]).T, f64(a[0])) <= TOL_F32


@pytest.mark.parametrize("shape", [(1, 300, 700), (2, 900, 256), (1, 130, 2000), (3, 128, 512)])
def test_bf16_carry_of_x_round_trips(mx, shape):
    """The bf16 path carries X between steps as a bf16 high part plus a
    residual.  With (a, b, c) = (1, 0, 0) one step gives B = 0 exactly and
    X_1 = high part + residual, which an fp32 output returns unrounded: it
    must reproduce X_0 = N/(||N||+eps) to about 16 significant bits.  A
    bf16-only carry would be off by about 2^-9 relative."""
    N = randn(shape, 3 * shape[1] + shape[2], torch.float32)
    out = torch.empty(shape, dtype=torch.float32, device="cuda")
    mx.orthogonalize(N, out, None, 1, (1.0, 0.0, 0.0), O.EPS, mx.MUON_BF16, device="cuda")
    torch.cuda.synchronize()
    for i in range(shape[0]):
        x0 = f64(N[i]) / (np.sqrt(np.sum(f64(N[i]) ** 2)) + O.EPS)
        assert rel(f64(out[i]), x0) <= 3e-5


def _bf16_rne(x32):
    """bf16 rounding (to nearest, ties to even) of finite float32 values, as float32."""
    u = x32.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return r.astype(np.uint32).view(np.float32)


def _carry_model(x32):
    """High part plus decoded residual of the bf16 path's carry of X, from its
    definition: per 32x32 block, lane-group of 16 values (one column, rows
    8q + 4h + e of the block, q, e < 4, h = 0, 1), E = the largest exponent
    field of their bf16 values, codes = residual / 2^(E-142) rounded to
    nearest even and clamped to +-127 (0 when E < 16)."""
    m, n = x32.shape
    mp, np_ = -(-m // 32) * 32, -(-n // 32) * 32
    x = np.zeros((mp, np_), np.float32)
    x[:m, :n] = x32
    hi = _bf16_rne(x)
    out = hi.astype(np.float64)
    for b in range(0, mp, 32):
        for h in range(2):
            rows = [b + 8 * q + 4 * h + e for q in range(4) for e in range(4)]
            hb = hi[rows, :]                                       # 16 x columns
            E = ((hb.view(np.uint32) >> 23) & 0xFF).max(axis=0).astype(np.int64)
            step = np.where(E >= 16, np.ldexp(1.0, E - 142), 0.0)
            inv = np.where(E >= 16, np.ldexp(1.0, 142 - E), 0.0)
            code = np.clip(np.rint((x[rows, :].astype(np.float64) - hb) * inv), -127, 127)
            out[rows, :] = hb + code * step
    return out[:m, :n].astype(np.float32)


@pytest.mark.parametrize("shape", [(2, 96, 200), (1, 256, 700), (1, 300, 520)])
def test_bf16_carry_of_x_is_exact(mx, shape):
    """The carry's format, bit for bit: with (a, b, c) = (1, 0, 0), one step,
    eps = 0 and a given sum of squares of 64 (so X_0 = N / 8 exactly), the
    fp32 output is the high part plus the decoded residual of every X_0
    element, which a host model of the format computes exactly.  Values span
    six decades so that blocks mix exponents."""
    g = np.random.default_rng(7 + shape[1])
    N = (g.standard_normal(shape) * 10.0 ** g.uniform(-3, 3, shape)).astype(np.float32)
    N[:, 0, :5] = 0.0
    Nt = torch.from_numpy(N).cuda()
    ss = torch.full((shape[0],), 64.0, dtype=torch.float32, device="cuda")
    out = torch.empty(shape, dtype=torch.float32, device="cuda")
    mx.orthogonalize(Nt, out, ss, 1, (1.0, 0.0, 0.0), 0.0, mx.MUON_BF16, device="cuda")
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for i in range(shape[0]):
        want = _carry_model(N[i] / np.float32(8.0))
        bad = np.argwhere(got[i].view(np.uint32) != want.view(np.uint32))
        assert bad.size == 0, f"{shape} matrix {i}: {len(bad)} elements differ, first {bad[:3].tolist()}"


@pytest.mark.parametrize("compute", [0, 1])
def test_ns_scale_invariance_and_odd_symmetry(mx, compute):
    """Invariants of the method on the GPU path.  Multiplying N by a power of
    two scales the sum of squares by its square exactly and the norm exactly,
    so X_0 is unchanged (eps = 1e-7 is far below the rounding of a norm near
    40) and so is every later bit, on both paths.  -N gives -O: bit for bit on
    the fp32 path, whose every rounding is to nearest even; on the bf16 path
    to within rounding, because the bf16 MFMA's internal summation does not
    round symmetrically under negation (found by this test: some outputs
    differ in their last bit)."""
    for shape in [(2, 300, 700), (1, 900, 256), (3, 128, 512)]:
        N = randn(shape, sum(shape), torch.float32 if compute == 0 else torch.bfloat16)
        o = run_ns(mx, N, compute)
        assert torch.equal(run_ns(mx, 4 * N, compute), o)
        assert torch.equal(run_ns(mx, N / 8, compute), o)
        neg = run_ns(mx, -N, compute)
        if compute == 0:
            assert torch.equal(neg, -o)
        else:
            for i in range(shape[0]):
                assert rel(-f64(neg[i]), f64(o[i])) <= 1e-2


def test_ns_batched_strided_and_pointer_array(mx):
    """A strided batch (per-head row blocks, ld = 4 x cols) and the same
    matrices as a pointer array give the oracle's answer."""
    big = randn((1, 512, 256), 31, torch.bfloat16)[0]
    heads = big.view(4, 128, 256)                     # contiguous row blocks
    out = torch.empty(4, 128, 256, dtype=torch.bfloat16, device="cuda")
    mx.orthogonalize(heads, out, None, 5, O.QUINTIC, O.EPS, mx.MUON_BF16, device="cuda")
    outl = [torch.empty(128, 256, dtype=torch.bfloat16, device="cuda") for _ in range(4)]
    mx.orthogonalize([heads[i] for i in range(4)], outl, None, 5, O.QUINTIC, O.EPS, mx.MUON_BF16, device="cuda")
    torch.cuda.synchronize()
    for i in range(4):
        want = O.newton_schulz(f64(heads[i]), 5)
        assert rel(f64(out[i]), want) <= TOL_BF16
        assert torch.equal(out[i], outl[i])


def test_grouped_equals_separate_calls(mx):
    shapes = [(2, 300, 700), (3, 128, 640), (1, 900, 256)]
    Ns = [randn(s, 40 + k, torch.bfloat16) for k, s in enumerate(shapes)]
    sep = [run_ns(mx, N, mx.MUON_BF16) for N in Ns]
    outs = [torch.empty_like(N) for N in Ns]
    mx.orthogonalize_grouped(Ns, outs, None, 5, O.QUINTIC, O.EPS, mx.MUON_BF16, device="cuda")
    torch.cuda.synchronize()
    for a, b in zip(sep, outs):
        assert torch.equal(a, b)


def test_grouped_update_reduction_lengths(mx):
    """The bf16 update reads X itself, k-major, at every reduction length: here
    padded short sides of 768, 2304 and 2048 in one grouped call, wide and
    tall, ragged against the 256 tiles.  The grouped call must equal the
    separate calls bit for bit and match the oracle."""
    shapes = [(2, 520, 700), (1, 2100, 2200), (1, 2300, 2050), (1, 1900, 2040)]
    Ns = [randn(s, 70 + k, torch.bfloat16) for k, s in enumerate(shapes)]
    sep = [run_ns(mx, N, mx.MUON_BF16) for N in Ns]
    outs = [torch.empty_like(N) for N in Ns]
    mx.orthogonalize_grouped(Ns, outs, None, 5, O.QUINTIC, O.EPS, mx.MUON_BF16, device="cuda")
    torch.cuda.synchronize()
    for (n, r, c), N, a, b in zip(shapes, Ns, sep, outs):
        assert torch.equal(a, b), f"{r}x{c}"
        for i in range(n):
            assert rel(f64(b[i]), O.newton_schulz(f64(N[i]), 5)) <= TOL_BF16, f"{r}x{c} matrix {i}"


def test_persistent_grid_matches_short_launches(mx):
    """Launches with at least four tiles per resident workgroup run on a
    persistent grid (each workgroup walks tiles blockIdx.x, +grid, ...).
    Three groups sized from the device's CU count so that every stage of both
    tile sizes takes that path, one of them crossing group boundaries; the
    result must equal, bit for bit, chunks of at most 100 matrices (one tile
    per workgroup), and sampled matrices must match the oracle."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    cap256, cap128 = cus & ~7, (2 * cus) & ~7
    nB = 150                                # 640x384: tall, 3 upper tiles of 256
    nA = max(4 * cap256 - 3 * nB, 0) + 64   # 256x512: one Gram tile of 256
    nC = 4 * cap128 + 52                    # 128x256: one Gram tile of 128
    assert nA + 3 * nB >= 4 * cap256 and nC >= 4 * cap128
    shapes = [(nA, 256, 512), (nB, 640, 384), (nC, 128, 256)]
    print(f"[persistent] {cus} CUs, groups {shapes}", flush=True)
    Ns = [randn(s, 60 + k, torch.bfloat16) for k, s in enumerate(shapes)]
    outs = [torch.empty_like(N) for N in Ns]
    mx.orthogonalize_grouped(Ns, outs, None, 5, O.QUINTIC, O.EPS, mx.MUON_BF16, device="cuda")
    short = [torch.empty_like(N) for N in Ns]
    for N, o in zip(Ns, short):
        for s in range(0, N.shape[0], 100):
            mx.orthogonalize(N[s:s + 100], o[s:s + 100], None, 5, O.QUINTIC, O.EPS, mx.MUON_BF16, device="cuda")
    torch.cuda.synchronize()
    for (n, r, c), a, b in zip(shapes, outs, short):
        diff = (a != b).reshape(n, -1).any(dim=1).nonzero().flatten().tolist()
        assert not diff, f"{r}x{c}: matrices {diff[:8]} differ from the short launches"
    for (n, r, c), N, out in zip(shapes, Ns, outs):
        for i in sorted({0, n // 3, n - 1}):
            assert rel(f64(out[i]), O.newton_schulz(f64(N[i]), 5)) <= TOL_BF16, f"{r}x{c} matrix {i}"


def test_muon_step_more_than_eight_groups(mx):
    """MuonStep runs at most 8 groups per grouped launch; 10 shape groups
    (two launches per stage) must equal one MuonStep per group, bit for bit,
    over two steps."""
    shapes = [(1, 64 + 16 * k, 96 + 8 * k) for k in range(10)]
    def make():
        out = []
        for k, s in enumerate(shapes):
            out.append((randn(s, 900 + k, torch.bfloat16, 0.02), randn(s, 950 + k, torch.bfloat16)))
        return out
    together, apart = make(), make()
    big = mx.MuonStep(together, lr=0.01, weight_decay=0.1)
    small = [mx.MuonStep([wg], lr=0.01, weight_decay=0.1) for wg in apart]
    assert len(big.chunks) == 2
    for _ in range(2):
        big.step()
        for st in small:
            st.step()
    torch.cuda.synchronize()
    for k, ((wa, _), (wb, _)) in enumerate(zip(together, apart)):
        assert torch.equal(wa, wb), f"group {k}"


# --------------------------------------------------------------- full steps

@pytest.mark.parametrize("nesterov", [True, False])
def test_single_fp32_gradient_three_steps(mx, nesterov):
    """The 256x128 fp32 configuration, three seeded gradients, whole step."""
    cfg = synth.WORKLOADS["tiny-256x128-f32"]
    lr, wd = 1.0, 0.5
    W = (0.02 * torch.randn(1, 256, 128, generator=torch.Generator().manual_seed(5))).cuda()
    Wo, Mo = f64(W[0]), np.zeros((256, 128))
    grads = [synth.group_gradients(cfg, step=t)[0].cuda() for t in (1, 2, 3)]
    G = torch.empty_like(grads[0])
    step = mx.MuonStep([(W, G)], compute=mx.MUON_F32, nesterov=nesterov, lr=lr, weight_decay=wd)
    for t in range(3):
        G.copy_(grads[t])
        step.step()
        torch.cuda.synchronize()
        Wo, Mo, Oo, sso = O.muon_step(Wo, Mo, f64(grads[t][0]), nesterov=nesterov, lr=lr, weight_decay=wd)
        assert rel(f64(step.momentum_buffers[0][0]), Mo) <= TOL_EW
        assert abs(float(step.sumsq_buffers[0][0]) - sso) <= TOL_EW * sso
        assert rel(f64(step.ortho_buffers[0][0]), Oo) <= TOL_F32
        assert rel(f64(W[0]), Wo) <= TOL_F32


def test_zero_gradient_step_is_pure_decay(mx):
    W = randn((2, 128, 192), 8, torch.float32, 0.02)
    W0 = W.clone()
    G = torch.zeros_like(W)
    step = mx.MuonStep([(W, G)], compute=mx.MUON_BF16, lr=0.01, weight_decay=0.5)
    for _ in range(3):
        step.step()
    torch.cuda.synchronize()
    assert torch.count_nonzero(step.ortho_buffers[0]).item() == 0
    want = f64(W0) * (1 - 0.01 * 0.5) ** 3
    assert rel(f64(W), want) <= TOL_EW


# ------------------------------------------------ hyperparameter groups, debug sync

def f32(x):
    return float(np.float32(x))


def test_groups_with_different_hyperparameters(mx):
    """Two optimizer groups with different momentum, Nesterov, step count,
    coefficients, shape factor, learning rate and decay, stepped in turn on
    one stream for two steps: each matches the oracle run with its own
    hyperparameters (the library holds no state between calls)."""
    hp = [dict(beta=0.9, nesterov=False, steps=4, coeffs=(3.4445, -4.7750, 2.0315), lr=0.5, weight_decay=0.2,
               mode=mx.MUON_SCALE_ORIGINAL, coeff=0.2),
          dict(beta=0.95, nesterov=True, steps=6, coeffs=(2.0, -1.5, 0.5), lr=1.0, weight_decay=0.0,
               mode=mx.MUON_SCALE_MATCH_RMS, coeff=0.16)]
    shapes = [(2, 96, 160), (1, 200, 72)]
    gen = torch.Generator().manual_seed(11)
    W0 = [0.02 * torch.randn(*s, generator=gen) for s in shapes]
    Gs = [[torch.randn(*s, generator=gen) for s in shapes] for _ in range(2)]
    Wd = [w.clone().cuda() for w in W0]
    Gd = [torch.empty(*s, device="cuda") for s in shapes]
    steps = [mx.MuonStep([(Wd[k], Gd[k])], compute=mx.MUON_F32, **hp[k]) for k in range(2)]
    Wo = [[f64(W0[k][i]) for i in range(shapes[k][0])] for k in range(2)]
    Mo = [[np.zeros(shapes[k][1:]) for _ in range(shapes[k][0])] for k in range(2)]
    for t in range(2):
        for k in range(2):
            Gd[k].copy_(Gs[t][k])
            steps[k].step()
        torch.cuda.synchronize()
        for k in range(2):
            h = {key: (f32(v) if isinstance(v, float) else v) for key, v in hp[k].items()}
            for i in range(shapes[k][0]):
                Wo[k][i], Mo[k][i], _, _ = O.muon_step(Wo[k][i], Mo[k][i], f64(Gs[t][k][i]), **h)
                assert rel(f64(Wd[k][i]), Wo[k][i]) <= 1e-5, (t, k, i)


def test_debug_sync_gives_the_same_results(mx, monkeypatch):
    """With MUON355_DEBUG_SYNC=1 every entry point waits for its kernels and
    checks them; the results are bit-identical to the asynchronous run."""
    outs = []
    for flag in (None, "1"):
        if flag is None:
            monkeypatch.delenv("MUON355_DEBUG_SYNC", raising=False)
        else:
            monkeypatch.setenv("MUON355_DEBUG_SYNC", flag)
        gen = torch.Generator().manual_seed(5)
        W = (0.02 * torch.randn(2, 130, 300, generator=gen)).to(torch.bfloat16).cuda()
        G = torch.randn(2, 130, 300, generator=gen).to(torch.bfloat16).cuda()
        st = mx.MuonStep([(W, G)], compute=mx.MUON_BF16, lr=0.01, weight_decay=0.1)
        st.step()
        st.step()
        torch.cuda.synchronize()
        outs.append(W.clone())
    monkeypatch.delenv("MUON355_DEBUG_SYNC", raising=False)
    assert torch.equal(outs[0], outs[1])
