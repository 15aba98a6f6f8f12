"""Checkpoint and resume of a whole-model optimizer step.

A run saved after two steps (optimizer state through torch.save and the safe
loader, plus the weights) and resumed in fresh optimizer objects must give a
third step bit-identical to the uninterrupted run: every kernel reduces in a
fixed order, so the state is all there is.
"""

import io

import pytest
import torch

pytestmark = pytest.mark.gpu

SPEC = [("embed_tokens.weight", (96, 64), torch.bfloat16), ("layers.0.attn.wq", (64, 64), torch.bfloat16),
        ("layers.0.attn.wk", (32, 64), torch.bfloat16), ("layers.0.mlp.up", (160, 64), torch.bfloat16),
        ("layers.0.mlp.down", (64, 160), torch.bfloat16), ("layers.0.norm.weight", (64,), torch.float32),
        ("layers.1.attn.wq", (64, 64), torch.bfloat16), ("lm_head.weight", (96, 64), torch.bfloat16)]


@pytest.fixture(scope="module")
def mx():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible MI355X")
    import matrix_aware_optimizer_step_amd as m
    m._lib.load()
    return m


def model(seed):
    g = torch.Generator().manual_seed(seed)
    return [(name, (0.05 * torch.randn(*shape, generator=g)).to(dt).cuda(),
             torch.zeros(*shape, dtype=dt, device="cuda")) for name, shape, dt in SPEC]


def set_grads(named, step):
    for i, (_, _, g) in enumerate(named):
        gen = torch.Generator().manual_seed(1000 * step + i)
        g.copy_(torch.randn(*g.shape, generator=gen).to(g.dtype))


def make(mx, named):
    return mx.OptimizerStep(named, compute=mx.MUON_BF16, muon_lr=0.02, muon_weight_decay=0.1, adam_lr=0.01,
                            adam_weight_decay=0.2)


def test_resume_after_two_steps_is_bit_identical(mx):
    straight = model(5)
    opt = make(mx, straight)
    for t in (1, 2, 3):
        set_grads(straight, t)
        opt.step()
    torch.cuda.synchronize()

    first = model(5)
    opt1 = make(mx, first)
    for t in (1, 2):
        set_grads(first, t)
        opt1.step()
    torch.cuda.synchronize()
    buf = io.BytesIO()
    torch.save({"optimizer": opt1.state_dict(), "weights": {n: p.cpu() for n, p, _ in first}}, buf)
    del opt1
    buf.seek(0)
    ckpt = torch.load(buf, weights_only=True)

    resumed = model(99)  # different initial values: everything must come from the checkpoint
    for n, p, _ in resumed:
        p.copy_(ckpt["weights"][n])
    opt2 = make(mx, resumed)
    opt2.load_state_dict(ckpt["optimizer"])
    set_grads(resumed, 3)
    opt2.step()
    torch.cuda.synchronize()
    for (n, pa, _), (_, pb, _) in zip(straight, resumed):
        assert torch.equal(pa, pb), n
    for ma, mb in zip(opt.muon.momentum_buffers, opt2.muon.momentum_buffers):
        assert torch.equal(ma, mb)
    for ga, gb in zip(opt.adamw, opt2.adamw):
        assert ga.t == gb.t == 3
        assert all(torch.equal(x, y) for x, y in zip(ga.exp_avg + ga.exp_avg_sq, gb.exp_avg + gb.exp_avg_sq))


def test_state_for_other_parameters_is_rejected(mx):
    a = make(mx, model(1))
    b = make(mx, [t for t in model(1) if t[0] != "lm_head.weight"])
    with pytest.raises(ValueError):
        b.load_state_dict(a.state_dict())


def test_soap_resume_is_bit_identical(mx):
    """SoapStep.state_dict() after two steps (statistics, bases, rotated
    moments and the step count), saved and loaded with the safe loader into a
    fresh SoapStep, gives steps 3 and 4 (a refresh falls on step 3 with
    freq 2) bit-identical to the uninterrupted run."""
    from matrix_aware_optimizer_step_amd import soap
    g = torch.Generator().manual_seed(3)
    shapes = [(2, 48, 80), (1, 96, 40)]
    W0 = [(0.02 * torch.randn(*s, generator=g)).to(torch.bfloat16) for s in shapes]
    grads = [[torch.randn(*s, generator=g).to(torch.bfloat16) for s in shapes] for _ in range(4)]

    def make(ws):
        G = [torch.empty(*s, dtype=torch.bfloat16, device="cuda") for s in shapes]
        st = soap.SoapStep(list(zip(ws, G)), lr=0.01, weight_decay=0.1, freq=2, max_dim=64)
        return st, G

    Wa = [w.cuda() for w in W0]
    a, Ga = make(Wa)
    saved = None
    for t in range(4):
        for gd, gh in zip(Ga, grads[t]):
            gd.copy_(gh)
        a.step()
        if t == 1:
            torch.cuda.synchronize()
            buf = io.BytesIO()
            torch.save({"opt": a.state_dict(), "w": [w.cpu() for w in Wa]}, buf)
            saved = buf.getvalue()
    torch.cuda.synchronize()
    ck = torch.load(io.BytesIO(saved), weights_only=True)
    Wb = [w.cuda() for w in ck["w"]]
    b, Gb = make(Wb)
    b.load_state_dict({"t": ck["opt"]["t"],
                       "groups": [{k: (None if v is None else v.cuda()) for k, v in grp.items()}
                                  for grp in ck["opt"]["groups"]]})
    for t in (2, 3):
        for gd, gh in zip(Gb, grads[t]):
            gd.copy_(gh)
        b.step()
    torch.cuda.synchronize()
    assert b.t == a.t == 4
    for wa, wb in zip(Wa, Wb):
        assert torch.equal(wa, wb)
    for ga, gb in zip(a.groups, b.groups):
        for k in soap.SoapStep.STATE:
            if ga[k] is not None:
                assert torch.equal(ga[k], gb[k]), k
