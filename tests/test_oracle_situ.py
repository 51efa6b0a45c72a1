"""Pins of the oracle's SiTU: closed forms, limits and symmetries.

SiTU(g, u) = (beta*tanh(g/beta)*sigmoid(g)) * (lam*tanh(u/lam)) ("Cake SiTU backend",
section "Prepared weights and scales"; beta = 4, lam = 25 by default).
"""

import math

import numpy as np
import torch

from oracle import situ


def test_hand_values():
    # At g = beta, u = lam: beta*lam*tanh(1)^2*sigmoid(beta).  tanh(1) = 0.76159415595576
    # and sigmoid(4) = 0.98201379003791 (tables), so 100*0.580025...*0.982013... = 56.9593.
    v = float(situ(np.float32(4.0), np.float32(25.0)))
    assert abs(v - 56.95932) < 1e-4
    # At g = 0 the gate factor is 0 for any u; at u = 0 the linear factor is 0.
    assert float(situ(np.float32(0.0), np.float32(3.0))) == 0.0
    assert float(situ(np.float32(2.0), np.float32(0.0))) == 0.0


def test_limit_is_swiglu():
    # beta, lam -> inf: beta*tanh(g/beta) -> g and lam*tanh(u/lam) -> u, so SiTU -> silu(g)*u.
    g = np.linspace(-6, 6, 49, dtype=np.float32)
    u = np.linspace(-3, 5, 49, dtype=np.float32)
    ours = situ(g, u, beta=np.float32(1e8), lam=np.float32(1e8)).astype(np.float64)
    ref = (torch.nn.functional.silu(torch.from_numpy(g).double()) * torch.from_numpy(u).double()).numpy()
    assert np.allclose(ours, ref, rtol=1e-6, atol=1e-7)


def test_large_gate_limit():
    # g -> +inf: beta*tanh(g/beta)*sigmoid(g) -> beta, so SiTU -> beta*lam*tanh(u/lam).
    u = np.float32(10.0)
    v = float(situ(np.float32(200.0), u))
    assert abs(v - 4 * 25 * math.tanh(10 / 25)) < 1e-4 * abs(v)
    # g -> -inf: the gate factor -> -beta*0 = 0 from below.
    assert abs(float(situ(np.float32(-80.0), u))) < 1e-25


def test_odd_in_u_and_bounded():
    rng = np.random.default_rng(0)
    g = rng.uniform(-20, 20, 1000).astype(np.float32)
    u = rng.uniform(-500, 500, 1000).astype(np.float32)
    a = situ(g, u)
    assert np.array_equal(a, -situ(g, -u))
    assert np.all(np.abs(a) < 4 * 25 + 1e-3)     # |gate factor| < beta, |linear| < lam


def test_gate_and_linear_are_not_interchangeable():
    # The formula is not symmetric: SiTU(1, 3) != SiTU(3, 1).
    assert float(situ(np.float32(1.0), np.float32(3.0))) != float(situ(np.float32(3.0), np.float32(1.0)))


def test_per_expert_parameters_enter_as_beta_and_lambda():
    # With beta = 2, lam = 5 at g = 2, u = 5: 2*tanh(1)*sigmoid(2) * 5*tanh(1).
    v = float(situ(np.float32(2.0), np.float32(5.0), beta=np.float32(2.0), lam=np.float32(5.0)))
    assert abs(v - 10 * 0.7615941559557649 ** 2 * 0.8807970779778823) < 1e-5
