"""Seeded synthetic gradients shaped like the pages' workloads.

This module only draws random numbers; it holds none of the Muon step's
arithmetic.  The GPU tests, the benchmark and the oracle's callers all take
their inputs from here, so both sides of every parity check see the same
bits.

Seed rule: matrix ``i`` (counted across the whole workload, in group order)
at optimizer step ``t`` (1-based) uses seed ``c*10**6 + i*10 + t`` for the
workload's seed id ``c`` (given in brackets below).

Workloads (the model shapes the pages name: an 8B dense GPT and a
Qwen3-30B-A3B-style MoE, "SOAP, Muon, and Beyond: Pushing LLM Pretraining
Scales"; per-head orthogonalization, "Reading notes on SOAP, Muon and
higher-order optimizers", section 1; MoE effective batch, same notes,
section 3):

tiny-256x128-f32 [1]: one 256x128 fp32 gradient, entries N(0,1), three
   steps.
8b-dense-layer [2]: one dense 8B-style layer in bf16: Wq, Wo 4096x4096; Wk, Wv 1024x4096;
   gate, up 14336x4096; down 4096x14336.  G = D X^T with D (m x 4096) and
   X (n x 4096) N(0,1): a sum of 4096 rank-1 outer products.
8b-dense-32-layers [3]: all 32 layers of those shapes (224 matrices), G = U diag(1/k) V^T with
   random orthogonal U, V (random_orthogonal): a power-law spectrum.
moe-30b-a3b-layer [4]: an MoE layer: 128 experts x (gate 768x2048, up 768x2048, down
   2048x768), G_e = c_e * Z_e with Z_e N(0,1) and c_e the expert's token
   count under top-8-of-128 routing of 65536 tokens with N(0,1) logits.
qkv-heads-kappa1e4 [5]: per-head: the 96 row blocks (128x4096) of Wq, Wk, Wv of a 4096-wide,
   32-head layer, plus gate, up (14336x4096) and down (4096x14336); every
   matrix G = U diag(sigma) V^T with sigma geometric from 1 to 1e-4
   (condition number 1e4) and random orthogonal U, V.
"""

from __future__ import annotations

from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class Group:
    name: str
    count: int
    rows: int
    cols: int


@dataclass(frozen=True)
class Config:
    slug: str
    seed_id: int
    name: str
    groups: tuple
    kind: str
    dtype: torch.dtype

    @property
    def matrices(self) -> int:
        return sum(g.count for g in self.groups)

    @property
    def elements(self) -> int:
        return sum(g.count * g.rows * g.cols for g in self.groups)


def _layer_groups(layers: int):
    return (Group("wq_wo", 2 * layers, 4096, 4096), Group("wk_wv", 2 * layers, 1024, 4096),
            Group("gate_up", 2 * layers, 14336, 4096), Group("down", layers, 4096, 14336))


WORKLOADS = {c.slug: c for c in (
    Config("tiny-256x128-f32", 1, "single 256x128 fp32 gradient", (Group("g", 1, 256, 128),), "gauss",
           torch.float32),
    Config("8b-dense-layer", 2, "one GPT-8B-style dense layer", _layer_groups(1), "rank1_sum", torch.bfloat16),
    Config("8b-dense-32-layers", 3, "32 GPT-8B-style dense layers", _layer_groups(32), "power_law", torch.bfloat16),
    Config("moe-30b-a3b-layer", 4, "30B-A3B-style MoE layer, 128 experts",
           (Group("gate_up", 256, 768, 2048), Group("down", 128, 2048, 768)), "moe", torch.bfloat16),
    Config("qkv-heads-kappa1e4", 5, "per-head QKV blocks + MLP, condition number 1e4",
           (Group("qkv_heads", 96, 128, 4096), Group("gate_up", 2, 14336, 4096), Group("down", 1, 4096, 14336)),
           "kappa", torch.bfloat16),
)}

# the workloads the benchmark times (the tiny one is a parity case only)
BENCH_WORKLOADS = ("8b-dense-layer", "8b-dense-32-layers", "moe-30b-a3b-layer", "qkv-heads-kappa1e4")


def seed_of(seed_id: int, matrix: int, step: int) -> int:
    return seed_id * 10 ** 6 + matrix * 10 + step


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def gaussian(rows: int, cols: int, seed: int, device="cpu") -> torch.Tensor:
    return torch.randn(rows, cols, generator=_gen(seed, device), device=device, dtype=torch.float32)


def rank1_sum(rows: int, cols: int, seed: int, inner: int = 4096, device="cpu") -> torch.Tensor:
    g = _gen(seed, device)
    d = torch.randn(rows, inner, generator=g, device=device, dtype=torch.float32)
    x = torch.randn(cols, inner, generator=g, device=device, dtype=torch.float32)
    return d @ x.T


def haar_host(n: int, gen: torch.Generator) -> torch.Tensor:
    """n x n Haar-distributed orthogonal matrix on the host (fp64): QR of a
    Gaussian with the signs fixed by R's diagonal."""
    z = torch.randn(n, n, generator=gen, dtype=torch.float64)
    q, r = torch.linalg.qr(z)
    return q * torch.sign(torch.diagonal(r)).unsqueeze(0)


def _split(n: int):
    """n = p * q with p the largest divisor of n not above sqrt(n)."""
    p = int(n ** 0.5)
    while n % p:
        p -= 1
    return p, n // p


def _kron_apply(A: torch.Tensor, B: torch.Tensor, Y: torch.Tensor) -> torch.Tensor:
    """(A kron B) @ Y for A (p x p), B (q x q), Y (p*q x k), without forming
    the Kronecker product: row i*q + j of the result is
    sum over a, b of A[i, a] B[j, b] Y[a*q + b]."""
    p, q, k = A.shape[0], B.shape[0], Y.shape[1]
    T = (A @ Y.reshape(p, q * k)).reshape(p, q, k)
    return torch.matmul(B, T).reshape(p * q, k)


def random_orthogonal(n: int, k: int, gen: torch.Generator, device) -> torch.Tensor:
    """n x k fp32 with orthonormal columns (k <= n).

    Up to n = 512, and when n has no divisor other than 1 and itself: the
    first k columns of a Haar matrix drawn on the host.  Above that, the
    first k columns of P1 (A1 kron B1) P2 (A2 kron B2) with A_i (p x p) and
    B_i (q x q) Haar, n = p*q, and P_i random row permutations: a dense,
    well-mixed orthogonal matrix whose only host work is four QRs of order
    about sqrt(n), applied on the device by matrix products.  No LAPACK
    routine runs on the device."""
    p, q = _split(n)
    if n <= 512 or p == 1:
        return haar_host(n, gen)[:, :k].to(device=device, dtype=torch.float32)
    A1, B1, A2, B2 = (haar_host(d, gen).to(device=device, dtype=torch.float32) for d in (p, q, p, q))
    perm1 = torch.randperm(n, generator=gen).to(device)
    perm2 = torch.randperm(n, generator=gen).to(device)
    Y = torch.eye(n, k, device=device, dtype=torch.float32)
    Y = _kron_apply(A2, B2, Y)[perm2]
    return _kron_apply(A1, B1, Y)[perm1]


def with_spectrum(rows: int, cols: int, sigma: torch.Tensor, seed: int, device="cpu") -> torch.Tensor:
    g = _gen(seed, "cpu")
    r = sigma.numel()
    u = random_orthogonal(rows, r, g, device)
    v = random_orthogonal(cols, r, g, device)
    return (u * sigma.to(device=device, dtype=torch.float32).unsqueeze(0)) @ v.T


def power_law(rows: int, cols: int, seed: int, device="cpu") -> torch.Tensor:
    r = min(rows, cols)
    return with_spectrum(rows, cols, 1.0 / torch.arange(1, r + 1, dtype=torch.float64), seed, device)


def condition_number(rows: int, cols: int, seed: int, kappa: float = 1e4, device="cpu") -> torch.Tensor:
    r = min(rows, cols)
    sigma = torch.logspace(0.0, -torch.log10(torch.tensor(kappa)).item(), r, dtype=torch.float64)
    return with_spectrum(rows, cols, sigma, seed, device)


def moe_token_counts(seed: int, tokens: int = 65536, experts: int = 128, topk: int = 8, device="cpu") -> torch.Tensor:
    g = _gen(seed, device)
    logits = torch.randn(tokens, experts, generator=g, device=device, dtype=torch.float32)
    top = torch.topk(logits, topk, dim=1).indices.flatten()
    return torch.bincount(top, minlength=experts)


def gradient(config: Config, matrix: int, rows: int, cols: int, step: int = 1, device="cpu",
             expert_counts: torch.Tensor | None = None) -> torch.Tensor:
    """fp32 gradient of matrix ``matrix`` of ``config`` at ``step``."""
    seed = seed_of(config.seed_id, matrix, step)
    if config.kind == "gauss":
        return gaussian(rows, cols, seed, device)
    if config.kind == "rank1_sum":
        return rank1_sum(rows, cols, seed, device=device)
    if config.kind == "power_law":
        return power_law(rows, cols, seed, device)
    if config.kind == "kappa":
        return condition_number(rows, cols, seed, device=device)
    if config.kind == "moe":
        if expert_counts is None:
            expert_counts = moe_token_counts(seed_of(config.seed_id, 0, 0), device=device)
        expert = matrix % 128
        return float(expert_counts[expert]) * gaussian(rows, cols, seed, device)
    raise ValueError(config.kind)


def group_gradients(config: Config, step: int = 1, device="cpu", dtype=None, groups=None):
    """One tensor (count, rows, cols) per group, in the config's dtype."""
    dtype = dtype or config.dtype
    counts = moe_token_counts(seed_of(config.seed_id, 0, 0), device=device) if config.kind == "moe" else None
    out = []
    i = 0
    for gi, grp in enumerate(config.groups):
        t = torch.empty(grp.count, grp.rows, grp.cols, dtype=dtype, device=device)
        for k in range(grp.count):
            if groups is None or gi in groups:
                t[k] = gradient(config, i, grp.rows, grp.cols, step, device, counts).to(dtype)
            i += 1
        out.append(t)
    return out


def initial_weights(config: Config, device="cpu", dtype=None, std: float = 0.02, seed: int = 7):
    """W_0 ~ N(0, std^2), one tensor (count, rows, cols) per group."""
    dtype = dtype or config.dtype
    g = _gen(config.seed_id * 10 ** 6 + seed * 100003, device)
    return [(std * torch.randn(grp.count, grp.rows, grp.cols, generator=g, device=device,
                               dtype=torch.float32)).to(dtype) for grp in config.groups]


# ---------------------------------------------------------------- AdamW

ADAMW_VOCAB = 128000  # the pages give no vocabulary size for the 8B-style model
ADAMW_HIDDEN = 4096


def adamw_workload(layers: int = 32):
    """(name, shape) of the 8B-style model's parameters that AdamW takes:
    token embedding and output head (vocabulary x hidden) and the RMSNorm
    weights (two per layer and a final one)."""
    out = [("embed_tokens.weight", (ADAMW_VOCAB, ADAMW_HIDDEN)), ("lm_head.weight", (ADAMW_VOCAB, ADAMW_HIDDEN))]
    for i in range(layers):
        out.append((f"layers.{i}.input_norm.weight", (ADAMW_HIDDEN,)))
        out.append((f"layers.{i}.post_norm.weight", (ADAMW_HIDDEN,)))
    out.append(("final_norm.weight", (ADAMW_HIDDEN,)))
    return out


def adamw_tensors(shapes, step: int = 1, device="cpu", dtype=torch.bfloat16, std: float = 0.02, seed: int = 9):
    """Seeded parameters (N(0, std^2); norm weights start at 1) and step-``step``
    gradients (N(0,1)) for the given (name, shape) list."""
    params, grads = [], []
    for i, (name, shape) in enumerate(shapes):
        g = _gen(seed * 10 ** 6 + i * 10 + step, device)
        grads.append(torch.randn(*shape, generator=g, device=device, dtype=torch.float32).to(dtype))
        if len(shape) == 1:
            params.append(torch.ones(*shape, device=device, dtype=dtype))
        else:
            gp = _gen(seed * 10 ** 6 + i * 10, device)
            params.append((std * torch.randn(*shape, generator=gp, device=device, dtype=torch.float32)).to(dtype))
    return params, grads
