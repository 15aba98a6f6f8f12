"""GPU parity of the SOAP entry points (soap_statistics, soap_qr,
soap_refresh, soap_precondition, and a whole step with muon_apply) against
the fp64 oracle in oracle/soap.py.

The library computes in fp32 (the products on the fp32 matrix cores, the QR
by Householder reflections), the oracle in fp64.  Tolerances, relative
Frobenius error per matrix, from the fp32 arithmetic:

* statistics (sums of up to a few hundred products): 1e-6;
* QR of a well-conditioned matrix (condition number ~10): 1e-5, with
  Q^T Q = I to 1e-5;
* the direction D and the updated weight: 1e-4.  A refresh takes the QR of
  L Q; the forward error of an fp32 Householder QR is at most of order
  n u kappa(L) per basis (n <= 200, u = 6e-8), and the direction carries
  both bases.  On these inputs (Gaussian gradients, statistics from the
  prior I, kappa(L) of a few tens) the measured errors are 1e-6 to 5e-5,
  which the bound holds with a factor of two; a wrong moment carry or a
  transposed basis change shows up at 1e-2 or more.  The errors measured
  are printed;
* one rotated-Adam direction from given bases (no QR): 1e-5.

The multi-step runs start from statistics L_0 = I, R_0 = I (a damping prior,
as Shampoo's eps*I).  From zero statistics one side of a non-square gradient
is rank deficient at the first refresh, and the QR then completes its basis
with directions fixed only by round-off; from step 2 on SOAP's result depends
on that completion (Adam's elementwise steps are not rotation invariant), so
it is not unique.  With the prior every refresh sees a full-rank statistic.

At step 1 Adam's direction in the rotated basis is g / (|g| + eps): a sign
for entries far above eps.  An entry of the rotated gradient within fp32
round-off of zero could take either sign, so the step-by-step comparisons
use eps = 1e-2 (entries ~1), which bounds the direction's sensitivity; the
default eps = 1e-8 is checked after three steps, where the direction is a
ratio of averages over three independent gradients.
"""

import numpy as np
import pytest
import torch

from oracle import adamw as OA
from oracle import oracle as O
from oracle import soap as S
from workloads import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mx():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible MI355X")
    import matrix_aware_optimizer_step_amd as m
    m._lib.load()
    return m


def f64(t):
    return t.detach().to(torch.float64).cpu().numpy()


def rel(a, b):
    return O.relative_frobenius_error(a, b)


def f32(x):
    return float(np.float32(x))


@pytest.mark.parametrize("n", [1, 5, 16, 17, 33, 100, 257, 300, 4200])
def test_qr_matches_oracle(mx, n):
    from matrix_aware_optimizer_step_amd import soap
    print(f"soap_qr n={n}", flush=True)
    count = 2
    A = torch.stack([synth.gaussian(n, n, seed=100 + n + b) for b in range(count)]).float()
    A += 3.0 * float(np.sqrt(n)) * torch.eye(n)
    Ad = A.cuda()
    Q = torch.full_like(Ad, float("nan"))
    soap.qr(Ad, Q)
    torch.cuda.synchronize()
    for b in range(count):
        want, _ = S.qr_nonneg(f64(A[b]))
        got = f64(Q[b])
        assert rel(got, want) <= 1e-5, (n, b, rel(got, want))
        assert np.max(np.abs(got.T @ got - np.eye(n))) <= 1e-5
    assert torch.equal(Ad.cpu(), A), "soap_qr must not modify its input"


def test_qr_rank_deficient_is_orthogonal(mx):
    # zero columns and a repeated column: Q stays orthogonal and Q R = A
    from matrix_aware_optimizer_step_amd import soap
    n = 70
    A = synth.gaussian(n, n, seed=7).float()
    A[:, 10] = 0.0
    A[:, 40] = A[:, 3]
    A[:, 69] = 0.0
    Q = torch.empty(n, n, device="cuda")
    soap.qr(A.cuda(), Q)
    torch.cuda.synchronize()
    q = f64(Q)
    assert np.max(np.abs(q.T @ q - np.eye(n))) <= 1e-5
    R = q.T @ f64(A)
    assert np.max(np.abs(np.tril(R, -1))) <= 1e-4 * np.max(np.abs(R))
    assert np.all(np.diag(R) >= -1e-4 * np.max(np.abs(R)))


@pytest.mark.parametrize("m,n,gdtype", [(64, 96, torch.float32), (130, 70, torch.bfloat16), (1, 33, torch.float32)])
def test_statistics_match_oracle(mx, m, n, gdtype):
    from matrix_aware_optimizer_step_amd import soap
    print(f"soap_statistics {m}x{n} {gdtype}", flush=True)
    count, b = 3, 0.8
    Ld = torch.zeros(count, m, m, device="cuda")
    Rd = torch.zeros(count, n, n, device="cuda")
    Lo = [np.zeros((m, m)) for _ in range(count)]
    Ro = [np.zeros((n, n)) for _ in range(count)]
    for t in range(3):
        G = torch.stack([synth.gaussian(m, n, seed=1000 * t + i) for i in range(count)]).to(gdtype)
        soap.statistics(G.cuda(), Ld, Rd, b)
        for i in range(count):
            Lo[i], Ro[i] = S.statistics(Lo[i], Ro[i], f64(G[i]), f32(b))
    torch.cuda.synchronize()
    for i in range(count):
        assert rel(f64(Ld[i]), Lo[i]) <= 1e-6
        assert rel(f64(Rd[i]), Ro[i]) <= 1e-6
        assert torch.equal(Ld[i], Ld[i].T) and torch.equal(Rd[i], Rd[i].T)


def run_steps(mx, m, n, steps, *, count=2, max_dim=4096, freq=2, eps=1e-2, wdtype=torch.float32,
              gdtype=torch.float32, lr=0.5, wd=0.2, check_each=True, tol=1e-4, seed=0, prior=1.0):
    """Run SoapStep and the oracle side by side from statistics prior*I;
    compare D and W; return the worst D error and the worst basis error."""
    from matrix_aware_optimizer_step_amd import soap
    b1, b2, bs = 0.9, 0.95, 0.8
    W0 = torch.stack([synth.gaussian(m, n, seed=seed + 50 + i) for i in range(count)]).to(wdtype)
    W = W0.cuda()
    G = torch.empty(count, m, n, dtype=gdtype, device="cuda")
    step = soap.SoapStep([(W, G)], lr=lr, weight_decay=wd, betas=(b1, b2), eps=eps, beta_s=bs, freq=freq,
                         max_dim=max_dim)
    states = [S.init_state(m, n, max_dim) for _ in range(count)]
    grp = step.groups[0]
    for st in states:
        if st.L is not None:
            st.L = prior * np.eye(m)
        if st.R is not None:
            st.R = prior * np.eye(n)
    for k in ("L", "R"):
        if grp[k] is not None:
            grp[k].copy_(prior * torch.eye(grp[k].shape[-1], device="cuda"))
    Wo = [f64(W0[i]) for i in range(count)]
    worst = worst_q = 0.0
    for t in range(1, steps + 1):
        Gh = torch.stack([synth.gaussian(m, n, seed=seed + 7919 * t + i) for i in range(count)]).to(gdtype)
        G.copy_(Gh)
        Wprev = [f64(W[i]) for i in range(count)]
        step.step()
        torch.cuda.synchronize()
        for i in range(count):
            # the oracle steps from the weight the GPU held (bf16 rounding of W does not accumulate)
            Wi, D = S.soap_step(Wprev[i], f64(Gh[i]), states[i], lr=f32(lr), weight_decay=f32(wd), beta1=f32(b1),
                                beta2=f32(b2), eps=f32(eps), beta_s=f32(bs), freq=freq)
            Wo[i] = Wi
            for k, q in (("QL", states[i].QL), ("QR", states[i].QR)):
                if grp[k] is not None:
                    worst_q = max(worst_q, rel(f64(grp[k][i]), q))
            if check_each or t == steps:
                e = rel(f64(grp["D"][i]), D)
                worst = max(worst, e)
                assert e <= tol, (t, i, e)
                if wdtype == torch.float32:
                    assert rel(f64(W[i]), Wi) <= tol
                else:
                    ulp = np.abs(Wi) * 2.0 ** -8 + tol * np.max(np.abs(Wi))
                    assert np.all(np.abs(f64(W[i]) - Wi) <= ulp)
    print(f"  {m}x{n}: worst D error {worst:.2e}, worst basis error {worst_q:.2e}")
    return worst, worst_q


@pytest.mark.parametrize("m,n", [(64, 96), (96, 64), (130, 70), (33, 200), (20, 64)])
def test_soap_steps_match_oracle(mx, m, n):
    print(f"soap steps {m}x{n}", flush=True)
    run_steps(mx, m, n, steps=4, freq=2)


def test_soap_one_sided(mx):
    # rows over max_dim: identity basis on the left, the column side only
    print("soap one-sided", flush=True)
    run_steps(mx, 150, 40, steps=3, max_dim=100, freq=1)
    run_steps(mx, 40, 150, steps=3, max_dim=100, freq=1)


def test_soap_identity_bases_is_adamw(mx):
    # both axes over max_dim: the layer is AdamW ([GUIDE] 11.2); the oracle
    # of SOAP then equals the AdamW oracle (pinned on the CPU)
    print("soap identity", flush=True)
    run_steps(mx, 40, 50, steps=3, max_dim=0, tol=1e-6)


def test_soap_default_eps_after_three_steps(mx):
    print("soap default eps", flush=True)
    run_steps(mx, 96, 128, steps=3, freq=2, eps=1e-8, check_each=False, tol=1e-4)


def test_soap_bf16_weight_and_gradient(mx):
    print("soap bf16", flush=True)
    run_steps(mx, 80, 112, steps=3, wdtype=torch.bfloat16, gdtype=torch.bfloat16)


def test_soap_pointer_array_state_matches_strided(mx):
    # the entry points take pointer-array batches as well: one refresh and
    # one precondition with every state tensor passed as a list
    from matrix_aware_optimizer_step_amd import soap
    m, n, c = 48, 80, 3
    G = torch.stack([synth.gaussian(m, n, seed=300 + i) for i in range(c)]).cuda()
    outs = []
    for as_list in (False, True):
        Ls = torch.zeros(c, m, m, device="cuda")
        Rs = torch.zeros(c, n, n, device="cuda")
        QL = torch.eye(m, device="cuda").expand(c, m, m).contiguous()
        QR = torch.eye(n, device="cuda").expand(c, n, n).contiguous()
        Mb = torch.zeros(c, m, n, device="cuda")
        Vb = torch.zeros(c, m, n, device="cuda")
        D = torch.empty(c, m, n, device="cuda")
        lst = (lambda x: list(x.unbind(0))) if as_list else (lambda x: x)
        soap.statistics(lst(G), lst(Ls), lst(Rs), 0.5)
        soap.refresh(lst(Mb), lst(Ls), lst(Rs), lst(QL), lst(QR))
        soap.precondition(lst(G), lst(Mb), lst(Vb), lst(D), 1, lst(QL), lst(QR))
        torch.cuda.synchronize()
        outs.append(D.clone())
    assert torch.equal(outs[0], outs[1])


@pytest.mark.parametrize("m,n,count,max_dim", [(1024, 4096, 2, 8192), (4096, 14336, 1, 8192)])
def test_soap_full_size_layer_matrices(mx, m, n, count, max_dim):
    """The 8B-style layer's Wk/Wv pair (both sides preconditioned, refresh by
    4096-wide QRs) and its down projection (rows only: the 14336 axis keeps
    the identity), at full size through SoapStep as the benchmark runs it.
    The statistics start from a prior comparable to the gradient's largest
    squared singular value, so that each refresh's QR is well conditioned
    (kappa ~2) and the comparison checks the wiring at full size rather
    than fp32 conditioning (covered above)."""
    print(f"soap full size {count}x{m}x{n}", flush=True)
    sig2 = (np.sqrt(m) + np.sqrt(n)) ** 2
    worst, worst_q = run_steps(mx, m, n, steps=2, count=count, max_dim=max_dim, freq=1, eps=1e-2, tol=1e-4,
                               prior=float(sig2), seed=31)
    assert worst_q <= 1e-4


def test_grouped_refresh_matches_per_group(mx):
    """soap_refresh_grouped batches every QR of one order over groups and
    sides (here order 96 is group 0's column side and group 1's row side);
    it matches one refresh per group to fp32 round-off (the batched QR may
    split its reductions differently) and the oracle to the step tolerance."""
    from matrix_aware_optimizer_step_amd import soap
    shapes = [(2, 64, 96), (1, 96, 40)]
    rng = np.random.default_rng(5)

    def spd(c, d):
        G = rng.standard_normal((c, d, 2 * d))
        return np.eye(d) + np.einsum("bij,bkj->bik", G, G) / (2 * d)

    def orth(c, d):
        return np.stack([np.linalg.qr(rng.standard_normal((d, d)))[0] for _ in range(c)])

    host = [dict(L=spd(c, m), R=spd(c, n), QL=orth(c, m), QR=orth(c, n), M=rng.standard_normal((c, m, n)))
            for c, m, n in shapes]
    cu = lambda a: torch.from_numpy(a).float().cuda()
    runs = []
    for grouped in (False, True):
        st = [{k: cu(v) for k, v in h.items()} for h in host]
        if grouped:
            soap.refresh_grouped([x["M"] for x in st], [x["L"] for x in st], [x["R"] for x in st],
                                 [x["QL"] for x in st], [x["QR"] for x in st])
        else:
            for x in st:
                soap.refresh(x["M"], x["L"], x["R"], x["QL"], x["QR"])
        torch.cuda.synchronize()
        runs.append(st)
    for g, (c, m, n) in enumerate(shapes):
        for i in range(c):
            QLn, QRn, Mn = S.refresh(host[g]["L"][i], host[g]["R"][i], host[g]["QL"][i], host[g]["QR"][i],
                                     host[g]["M"][i])
            for k, want in (("QL", QLn), ("QR", QRn), ("M", Mn)):
                a, b = f64(runs[0][g][k][i]), f64(runs[1][g][k][i])
                assert rel(b, a) <= 1e-5, (g, i, k, rel(b, a))
                assert rel(b, want) <= 1e-4, (g, i, k, rel(b, want))


@pytest.mark.gpu
def test_grouped_statistics_bit_identical_to_per_group(mx):
    """soap_statistics_grouped shares launches between groups (one per
    operand layout, longest reduction first); each tile is computed as a
    per-group call computes it, so every statistic is bit-identical.  The
    groups take three layouts: bf16 and fp32 gradients on the vector-load
    path, and a row pitch that is no multiple of 4 (the general path).  The
    oracle checks the result too."""
    from matrix_aware_optimizer_step_amd import soap
    torch.manual_seed(11)
    base = torch.randn(2, 200, 333, device="cuda")
    grads = [torch.randn(2, 96, 300, device="cuda").to(torch.bfloat16),
             torch.randn(1, 260, 130, device="cuda"),
             base[:, :, :330],                       # ld 333: no vector loads
             torch.randn(3, 40, 64, device="cuda").to(torch.bfloat16)]
    sides = [(True, True), (True, False), (True, True), (False, True)]
    prior = lambda c, d: (torch.eye(d, device="cuda") * 0.5).expand(c, d, d).contiguous()
    runs = []
    for grouped in (False, True):
        Ls = [prior(g.shape[0], g.shape[1]) if wl else None for g, (wl, _) in zip(grads, sides)]
        Rs = [prior(g.shape[0], g.shape[2]) if wr else None for g, (_, wr) in zip(grads, sides)]
        print(f"statistics grouped={grouped}", flush=True)
        if grouped:
            soap.statistics_grouped(grads, Ls, Rs, 0.9)
        else:
            for g, l, r in zip(grads, Ls, Rs):
                soap.statistics(g, l, r, 0.9)
        torch.cuda.synchronize()
        runs.append((Ls, Rs))
    for k, g in enumerate(grads):
        for side in (0, 1):
            a, b = runs[0][side][k], runs[1][side][k]
            if a is None:
                continue
            assert torch.equal(a, b), (k, side)
            for i in range(g.shape[0]):
                G = f64(g[i])
                S0 = 0.5 * np.eye(G.shape[side])
                want = S.statistics(S0, None, G, 0.9)[0] if side == 0 else S.statistics(None, S0, G, 0.9)[1]
                assert rel(f64(b[i]), want) <= 1e-6, (k, side, i)


@pytest.mark.gpu
def test_grouped_precondition_bit_identical_to_per_group(mx):
    """soap_precondition_grouped launches each rotation stage for all groups
    together; every direction and moment is bit-identical to one call per
    group.  The groups cover both sides, the left or the right side alone,
    and neither (the identity bases: plain Adam), with bf16 and fp32
    gradients.  The oracle checks one step's direction."""
    from matrix_aware_optimizer_step_amd import soap
    torch.manual_seed(12)
    shapes = [(2, 96, 160), (1, 130, 64), (3, 48, 200), (1, 40, 36)]
    sides = [(True, True), (True, False), (False, True), (False, False)]
    dts = [torch.bfloat16, torch.float32, torch.float32, torch.bfloat16]
    orth = lambda c, d: torch.linalg.qr(torch.randn(c, d, d, dtype=torch.float64))[0].float().contiguous().cuda()
    grads = [torch.randn(c, m, n, device="cuda").to(dt) for (c, m, n), dt in zip(shapes, dts)]
    QLs = [orth(c, m) if wl else None for (c, m, n), (wl, _) in zip(shapes, sides)]
    QRs = [orth(c, n) if wr else None for (c, m, n), (_, wr) in zip(shapes, sides)]
    m0 = [0.1 * torch.randn(c, m, n, device="cuda") for c, m, n in shapes]
    v0 = [0.01 * torch.rand(c, m, n, device="cuda") for c, m, n in shapes]
    runs = []
    for grouped in (False, True):
        mb = [x.clone() for x in m0]
        vb = [x.clone() for x in v0]
        D = [torch.empty(c, m, n, device="cuda") for c, m, n in shapes]
        print(f"precondition grouped={grouped}", flush=True)
        if grouped:
            soap.precondition_grouped(grads, mb, vb, D, 3, QLs, QRs, eps=1e-2)
        else:
            for k in range(len(shapes)):
                soap.precondition(grads[k], mb[k], vb[k], D[k], 3, QLs[k], QRs[k], eps=1e-2)
        torch.cuda.synchronize()
        runs.append((mb, vb, D))
    for k, (c, m, n) in enumerate(shapes):
        for j in range(3):
            assert torch.equal(runs[0][j][k], runs[1][j][k]), (k, j)
        for i in range(c):
            QL = f64(QLs[k][i]) if QLs[k] is not None else np.eye(m)
            QR = f64(QRs[k][i]) if QRs[k] is not None else np.eye(n)
            want, _, _ = S.precondition(f64(grads[k][i]), QL, QR, f64(m0[k][i]), f64(v0[k][i]), 3, S.BETA1, S.BETA2,
                                        1e-2)
            assert rel(f64(runs[1][2][k][i]), want) <= 1e-5, (k, i, rel(f64(runs[1][2][k][i]), want))
