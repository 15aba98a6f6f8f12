"""GPU parity of muon_adamw (and the routing helper) against the fp64 oracles.

The oracle is given the hyperparameters the kernel read: the C ABI takes
them as fp32 (0.999 arrives as 0.999000012), so each is rounded to fp32
first.

Tolerances: fp32 parameters and the fp32 moments, relative Frobenius error
<= 1e-6 per tensor (the elementwise bound); bf16 parameters within one bf16
rounding of the oracle's value computed from the same inputs, plus 1e-6 of
the largest entry for the fp32 error before rounding.  Multi-step runs
check every step from the state the GPU held before it, so bf16 rounding of
the parameters does not accumulate into the comparison.
"""

import numpy as np
import pytest
import torch

import bench
from oracle import adamw as OA
from oracle import oracle as O
from workloads import synth

pytestmark = pytest.mark.gpu

TOL_EW = 1e-6


def f32(x):
    return float(np.float32(x))


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


def check_param(got, want, dtype):
    if dtype == torch.float32:
        assert O.relative_frobenius_error(got, want) <= TOL_EW
    else:
        tol = bf16_ulp(want) + TOL_EW * np.max(np.abs(want))
        assert np.all(np.abs(got - bf16_of(want)) <= tol)


# sizes around the 4096-element chunk and the 8-element vector group, and tiny ones
SIZES = [(1,), (7,), (4096,), (4097,), (8191,), (3, 5), (64, 129), (300, 700), (12345,)]


@pytest.mark.parametrize("pdtype,gdtype", [(torch.float32, torch.float32), (torch.bfloat16, torch.bfloat16),
                                           (torch.float32, torch.bfloat16)])
@pytest.mark.parametrize("wd", [0.0, 0.1])
def test_adamw_tensor_list_three_steps(mx, pdtype, gdtype, wd):
    g0 = torch.Generator().manual_seed(11)
    params = [(0.5 * torch.randn(*s, generator=g0)).to(pdtype).cuda() for s in SIZES]
    grads = [torch.empty(*s, dtype=gdtype, device="cuda") for s in SIZES]
    lr, betas, eps = 1e-2, (0.9, 0.99), 1e-8
    opt = mx.AdamW(params, grads, lr=lr, betas=betas, eps=eps, weight_decay=wd)
    for t in range(1, 4):
        for i, s in enumerate(SIZES):
            gt = torch.Generator().manual_seed(100 * t + i)
            scale = 10.0 ** (i % 5 - 2)  # magnitudes from 1e-2 to 1e2, some near eps after squaring
            grads[i].copy_((scale * torch.randn(*s, generator=gt)).to(gdtype))
        before = [(f64(p), f64(m), f64(v)) for p, m, v in zip(params, opt.exp_avg, opt.exp_avg_sq)]
        opt.step()
        torch.cuda.synchronize()
        for i in range(len(SIZES)):
            th, m, v = OA.adamw_step(before[i][0], f64(grads[i]), before[i][1], before[i][2], t, f32(lr),
                                     f32(betas[0]), f32(betas[1]), f32(eps), f32(wd))
            assert O.relative_frobenius_error(f64(opt.exp_avg[i]), m) <= TOL_EW
            assert O.relative_frobenius_error(f64(opt.exp_avg_sq[i]), v) <= TOL_EW
            check_param(f64(params[i]), th, pdtype)


def test_adamw_late_step_and_zero_gradient(mx):
    """Step 1000 (bias corrections near 1) from a nonzero state, and a zero
    gradient, which still advances the moments and applies the decay."""
    n = 5000
    g0 = torch.Generator().manual_seed(3)
    p = torch.randn(n, generator=g0).cuda()
    g = torch.zeros(n, device="cuda")
    opt = mx.AdamW([p], [g], lr=1e-3, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.5)
    opt.exp_avg[0].copy_(torch.randn(n, generator=g0).cuda())
    opt.exp_avg_sq[0].copy_(torch.rand(n, generator=g0).cuda())
    opt.t = 999
    th0, m0, v0 = f64(p), f64(opt.exp_avg[0]), f64(opt.exp_avg_sq[0])
    opt.step()
    torch.cuda.synchronize()
    th, m, v = OA.adamw_step(th0, np.zeros(n), m0, v0, 1000, f32(1e-3), f32(0.9), f32(0.999), f32(1e-8), 0.5)
    assert O.relative_frobenius_error(f64(p), th) <= TOL_EW
    assert O.relative_frobenius_error(f64(opt.exp_avg[0]), m) <= TOL_EW
    assert O.relative_frobenius_error(f64(opt.exp_avg_sq[0]), v) <= TOL_EW


def test_routing_helper_whole_model_step(mx):
    """A toy model: 2-D hidden matrices go to Muon, embedding and head to
    AdamW with decay, norms and biases to AdamW without; one step() updates
    all of them as the two oracles say."""
    g0 = torch.Generator().manual_seed(21)
    spec = [("embed_tokens.weight", (96, 64)), ("layers.0.attn.wq", (64, 64)), ("layers.0.attn.bias", (64,)),
            ("layers.0.mlp.up", (160, 64)), ("layers.0.mlp.down", (64, 160)), ("layers.0.norm.weight", (64,)),
            ("layers.1.attn.wq", (64, 64)), ("lm_head.weight", (96, 64)), ("unused.weight", (64, 64))]
    named, init = [], {}
    for name, shape in spec:
        p = (0.05 * torch.randn(*shape, generator=g0)).cuda()
        g = None if name.startswith("unused") else torch.randn(*shape, generator=g0).cuda()
        init[name] = f64(p)
        named.append((name, p, g))
    mlr, mwd, alr, awd = 0.02, 0.1, 0.01, 0.2
    opt = mx.OptimizerStep(named, compute=mx.MUON_F32, muon_lr=mlr, muon_weight_decay=mwd, adam_lr=alr,
                           adam_weight_decay=awd)
    assert opt.routing == {"embed_tokens.weight": "adamw", "layers.0.attn.wq": "muon",
                           "layers.0.attn.bias": "adamw_no_decay", "layers.0.mlp.up": "muon",
                           "layers.0.mlp.down": "muon", "layers.0.norm.weight": "adamw_no_decay",
                           "layers.1.attn.wq": "muon", "lm_head.weight": "adamw"}
    opt.step()
    torch.cuda.synchronize()
    for name, p, g in named:
        if g is None:
            assert np.array_equal(f64(p), init[name])  # no gradient: untouched
            continue
        if opt.routing[name] == "muon":
            want = O.muon_step(init[name], np.zeros(p.shape), f64(g), lr=mlr, weight_decay=mwd)[0]
            assert O.relative_frobenius_error(f64(p), want) <= 1e-5
        else:
            wd = awd if opt.routing[name] == "adamw" else 0.0
            want = OA.adamw_step(init[name], f64(g), np.zeros(p.shape), np.zeros(p.shape), 1, f32(alr), f32(0.9),
                                 f32(0.999), f32(1e-8), f32(wd))[0]
            assert O.relative_frobenius_error(f64(p), want) <= TOL_EW


def test_adamw_full_size_benchmark_leg(mx):
    """The benchmark's AdamW leg at its full size (embedding and head of
    128000 x 4096 plus 65 norms, bf16), two steps; sampled elements of the big
    tensors and every norm element against the oracle evaluated element by
    element from the state the GPU held."""
    shapes = synth.adamw_workload()
    names = [n for n, _ in shapes]
    params, grads = synth.adamw_tensors(shapes, step=1, device="cuda")
    opt = bench.make_adamw_step(mx, names, params, grads)
    groups = {id(t): (grp, k) for grp in opt.adamw for k, t in enumerate(grp.params)}
    rng = np.random.default_rng(5)
    picks = {}
    for i, p in enumerate(params):
        flat = p.view(-1)
        picks[i] = torch.from_numpy(rng.choice(flat.numel(), size=min(flat.numel(), 200000), replace=False)).cuda()

    def snap(i):
        grp, k = groups[id(params[i])]
        idx = picks[i]
        return (f64(params[i].view(-1)[idx]), f64(grp.exp_avg[k].view(-1)[idx]), f64(grp.exp_avg_sq[k].view(-1)[idx]),
                grp)

    for t in (1, 2):
        if t == 2:
            new = synth.adamw_tensors(shapes, step=2, device="cuda")[1]
            for g, n in zip(grads, new):
                g.copy_(n)
        before = {i: snap(i) for i in range(len(params))}
        opt.step()
        torch.cuda.synchronize()
        for i in range(len(params)):
            th0, m0, v0, grp = before[i]
            wd = grp.weight_decay
            g = f64(grads[i].view(-1)[picks[i]])
            th, m, v = OA.adamw_step(th0, g, m0, v0, t, f32(bench.ADAM_LR), f32(bench.ADAM_BETAS[0]),
                                     f32(bench.ADAM_BETAS[1]), f32(bench.ADAM_EPS), f32(wd))
            after = snap(i)
            assert O.relative_frobenius_error(after[1], m) <= TOL_EW, names[i]
            assert O.relative_frobenius_error(after[2], v) <= TOL_EW, names[i]
            check_param(after[0], th, torch.bfloat16)
    print(f"[adamw] full-size leg checked on {sum(len(p) for p in picks.values())} sampled elements", flush=True)
