"""GPU parity of the update folded into the last Newton-Schulz step
(muon_momentum_packed_grouped, then muon_orthogonalize_apply_packed_grouped):
W <- (1 - lr*wd) W - lr*s*O is written by the last step's epilogue from the
fp32 accumulator, so O is never stored.

Against the fp64 oracle, on fp32 weights the update term is recovered exactly
enough to read O back: O_rec = ((1 - lr*wd) W_0 - W_1) / (lr*s) must meet the
Newton-Schulz bound of its path (fp32 1e-5, bf16 3e-2).  Against the separate
apply call on the same inputs (the Newton-Schulz kernels are the same until
that epilogue):
* fp32 weights: relative Frobenius difference <= 1e-6 (two roundings of one
  multiply-add);
* bf16 weights: elementwise within one bf16 unit of W plus lr*s*2^-8 |O|, the
  rounding of O to bf16 that the separate path takes and this one does not.
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


def bf16_ulp(x):
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    return np.where(ax > 0, 2.0 ** (e - 7), 2.0 ** -133)


def randn(shape, seed, dtype, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (scale * torch.randn(*shape, generator=g, dtype=torch.float32)).to(dtype).cuda()


def pair(mx, groups, **kw):
    """The same groups stepped by the fused path and by the separate apply
    call, on clones of the weights and the same gradients."""
    twin = []
    for w, g in groups:
        if isinstance(w, (list, tuple)):
            twin.append(([t.clone() for t in w], g))
        else:
            twin.append((w.clone(), g))
    fused = mx.MuonStep(groups, fused_apply=True, **kw)
    plain = mx.MuonStep(twin, **kw)
    assert fused.fused_apply and not plain.fused_apply
    return fused, plain, twin


def close_to_separate(W_f, W_u, O_u, step, dtype, where):
    if dtype == torch.float32:
        err = O.relative_frobenius_error(W_f, W_u)
        assert err <= TOL_EW, f"{where}: fused vs separate apply {err:.3g}"
    else:
        tol = bf16_ulp(np.maximum(np.abs(W_f), np.abs(W_u))) + step * 2.0 ** -8 * np.abs(O_u)
        bad = np.abs(W_f - W_u) > tol
        assert not bad.any(), f"{where}: {int(bad.sum())} elements beyond one rounding of the separate apply"


CASES = [
    # (count, rows, cols), weight/gradient dtype, compute
    ((1, 256, 128), torch.float32, 0),     # tall: fp32 path, output written transposed from LDS
    ((1, 256, 128), torch.float32, 1),
    ((2, 128, 384), torch.float32, 0),     # wide: fp32 path, element stores from the accumulator
    ((3, 100, 72), torch.bfloat16, 1),     # tall, ragged, 128-tile class
    ((2, 130, 300), torch.bfloat16, 1),    # wide, ragged, 256-tile class
    ((2, 520, 256), torch.bfloat16, 1),    # tall, 256-tile class, several row tiles
    ((2, 300, 700), torch.bfloat16, 0),    # fp32 compute on bf16 weights
    ((4, 128, 4096), torch.bfloat16, 1),   # per-head blocks: split Gram
]


@pytest.mark.parametrize("shape,dtype,compute", CASES)
def test_fused_apply_matches_oracle_and_separate_apply(mx, shape, dtype, compute):
    print(f"fused apply {shape} {dtype} compute={compute}", flush=True)
    c, m, n = shape
    lr, wd = 1.0, 0.5
    W = randn(shape, 11, dtype, 0.02)
    G = torch.empty(shape, dtype=dtype, device="cuda")
    fused, plain, twin = pair(mx, [(W, G)], compute=compute, lr=lr, weight_decay=wd)
    with pytest.raises(RuntimeError, match="never stored"):
        fused.ortho_buffers
    Wu = twin[0][0]
    step = lr * O.scale_factor(m, n, O.SCALE_MATCH_RMS, 0.2)
    decay = np.float32(1.0 - lr * wd)
    Mo = [np.zeros((m, n)) for _ in range(c)]
    tol = TOL_F32 if compute == 0 else TOL_BF16
    for t in range(1, 4):
        G.copy_(randn(shape, 100 + t, dtype, 3.0))
        W0 = [f64(W[i]) for i in range(c)]
        fused.step()
        plain.step()
        torch.cuda.synchronize()
        for i in range(c):
            where = f"step {t} matrix {i}"
            Mo[i], N = O.momentum(Mo[i], f64(G[i]))
            assert O.relative_frobenius_error(f64(fused.momentum_buffers[0][i]), Mo[i]) <= TOL_EW, where
            Wf = f64(W[i])
            if dtype == torch.float32:
                O_rec = (W0[i] * float(decay) - Wf) / step
                err = O.relative_frobenius_error(O_rec, O.newton_schulz(N, 5))
                assert err <= tol + 1e-6, f"{where}: recovered update {err:.3g}"
            close_to_separate(Wf, f64(Wu[i]), f64(plain.ortho_buffers[0][i]), step, dtype, where)
        # both paths advance from their own weights: keep them on the same start
        Wu.copy_(W)


@pytest.mark.parametrize("steps", [1, 2])
def test_fused_apply_short_iterations(mx, steps):
    """K = 1: the first Newton-Schulz step (which also normalizes the packed
    input) is the one that applies the update."""
    shape = (2, 260, 130)
    W = randn(shape, 21, torch.float32, 0.02)
    G = randn(shape, 22, torch.float32, 2.0)
    fused, plain, twin = pair(mx, [(W, G)], steps=steps, lr=0.5, weight_decay=0.2)
    W0 = f64(W)
    fused.step()
    plain.step()
    torch.cuda.synchronize()
    step = 0.5 * O.scale_factor(260, 130, O.SCALE_MATCH_RMS, 0.2)
    for i in range(2):
        _, N = O.momentum(np.zeros(shape[1:]), f64(G[i]))
        O_rec = (W0[i] * float(np.float32(1.0 - 0.1)) - f64(W[i])) / step
        assert O.relative_frobenius_error(O_rec, O.newton_schulz(N, steps)) <= TOL_BF16
        close_to_separate(f64(W[i]), f64(twin[0][0][i]), f64(plain.ortho_buffers[0][i]), step, torch.float32, i)


def test_fused_apply_row_blocks_pointer_arrays_and_many_groups(mx):
    """Column slices of wider weights (ld > cols), per-head row blocks,
    pointer-array groups and ten shape groups (two launches per stage)."""
    wide_w = randn((2, 300, 520), 7, torch.bfloat16, 0.02)
    wide_g = randn((2, 300, 520), 8, torch.bfloat16)
    heads_w = randn((512, 1024), 9, torch.bfloat16, 0.02).view(4, 128, 1024)
    heads_g = randn((512, 1024), 10, torch.bfloat16).view(4, 128, 1024)
    lists = ([randn((96, 200), 30 + i, torch.bfloat16, 0.02) for i in range(3)],
             [randn((96, 200), 40 + i, torch.bfloat16) for i in range(3)])
    extra = [(randn((1, 64 + 16 * k, 96), 60 + k, torch.float32, 0.02),
              randn((1, 64 + 16 * k, 96), 80 + k, torch.float32)) for k in range(7)]
    wide_twin = wide_w.clone()
    groups = [(wide_w[:, :, :260], wide_g[:, :, :260]), (heads_w, heads_g), lists] + extra
    twin = [(wide_twin[:, :, :260], wide_g[:, :, :260]), (heads_w.clone(), heads_g),
            ([t.clone() for t in lists[0]], lists[1])] + [(w.clone(), g) for w, g in extra]
    lr, wd = 0.5, 0.2
    fused = mx.MuonStep(groups, lr=lr, weight_decay=wd, fused_apply=True)
    plain = mx.MuonStep(twin, lr=lr, weight_decay=wd)
    assert fused.packed and fused.fused_apply and len(fused.chunks) == 2
    assert fused.w[0].desc.ld == 520
    fused.step()
    plain.step()
    torch.cuda.synchronize()

    def mats(gs):
        w0, w1, w2 = gs[0][0], gs[1][0], gs[2][0]
        return [w0[i] for i in range(2)] + [w1[i] for i in range(4)] + list(w2) + [w[0] for w, _ in gs[3:]]

    ortho = plain.ortho_buffers
    o_mats = [ortho[0][i] for i in range(2)] + [ortho[1][i] for i in range(4)] + [ortho[2][i] for i in range(3)] + \
             [ortho[3 + k][0] for k in range(7)]
    for j, (wf, wu, ou) in enumerate(zip(mats(groups), mats(twin), o_mats)):
        step = lr * O.scale_factor(wf.shape[0], wf.shape[1], O.SCALE_MATCH_RMS, 0.2)
        close_to_separate(f64(wf), f64(wu), f64(ou), step, wf.dtype, j)
    # the right halves of the wider weights are not part of any matrix: untouched
    assert torch.equal(wide_w[:, :, 260:], randn((2, 300, 520), 7, torch.bfloat16, 0.02)[:, :, 260:])


def test_fused_apply_zero_gradient_gives_pure_decay(mx):
    W = randn((2, 96, 160), 3, torch.float32, 0.02)
    W0 = f64(W)
    G = torch.zeros((2, 96, 160), dtype=torch.float32, device="cuda")
    step = mx.MuonStep([(W, G)], lr=0.1, weight_decay=0.5, fused_apply=True)
    step.step()
    torch.cuda.synchronize()
    assert np.array_equal(f64(W), (W0.astype(np.float32) * np.float32(1.0 - 0.1 * 0.5)).astype(np.float64))
