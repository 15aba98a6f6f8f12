"""CPU checks of the seeded input generators: the random orthogonal factors
are orthonormal and deterministic, and the spectrum-shaped gradients have
exactly the singular values asked for."""

import numpy as np
import torch

from workloads import synth


def test_random_orthogonal_is_orthonormal_and_seeded():
    for n, k in ((96, 96), (600, 200), (1024, 1024), (4096, 300)):
        U = synth.random_orthogonal(n, k, torch.Generator().manual_seed(3), "cpu").double()
        assert U.shape == (n, k)
        assert torch.allclose(U.T @ U, torch.eye(k, dtype=torch.float64), atol=2e-6)
        V = synth.random_orthogonal(n, k, torch.Generator().manual_seed(3), "cpu").double()
        assert torch.equal(U, V)
        W = synth.random_orthogonal(n, k, torch.Generator().manual_seed(4), "cpu").double()
        assert not torch.equal(U, W)


def test_random_orthogonal_is_dense():
    # entries spread like a Gaussian's of variance 1/n (mean |x| = sqrt(2/pi)/sqrt(n))
    n = 4096
    U = synth.random_orthogonal(n, 256, torch.Generator().manual_seed(5), "cpu").double()
    assert abs(U.abs().mean().item() * n ** 0.5 - (2 / np.pi) ** 0.5) < 0.01
    assert (U == 0).sum().item() == 0


def test_with_spectrum_has_the_requested_singular_values():
    for rows, cols in ((300, 700), (1024, 512)):
        r = min(rows, cols)
        sigma = torch.logspace(0.0, -4.0, r, dtype=torch.float64)
        G = synth.with_spectrum(rows, cols, sigma, seed=11).double()
        s = torch.linalg.svdvals(G)
        assert torch.allclose(s, sigma, rtol=1e-4, atol=1e-6)


def test_power_law_gradient_spectrum():
    G = synth.power_law(512, 1024, seed=2).double()
    s = torch.linalg.svdvals(G)
    assert torch.allclose(s, 1.0 / torch.arange(1, 513, dtype=torch.float64), rtol=1e-4, atol=1e-6)
