"""Pins for the ALU-only polynomial GELU and for QK-norm (CPU only).

"Training GEM at LLM scale", section "Generalized Dot-Product Attention
(GDPA)", item on the ALU-only activation: the tanh in GELU is replaced by a
6th-order Taylor expansion, accurate on the bounded range that QK-norm
enforces.  What fixes the oracle here:
  * the polynomial against numpy's tanh, with the Taylor remainder bound
    (a wrong coefficient leaves an error of order u^3 or u^5, not u^7);
  * the tanh-form GELU constants against scipy's exact erf GELU;
  * f(x) - f(-x) = x exactly (the tanh replacement is odd);
  * the derivative against central differences;
  * QK-norm against torch.nn.functional.normalize and its autograd;
  * finite differences through QK-norm followed by polynomial-GELU attention.
"""
import math

import numpy as np
import pytest
import torch
from scipy.special import erf

from jagged_variable_length_amd import inputs as gen
from oracle import attention as ora
from oracle import qknorm as qn


def test_tanh_polynomial_matches_tanh_to_seventh_order():
    u = np.linspace(-0.5, 0.5, 2001)
    err = np.abs(np.tanh(u) - ora.tanh_taylor6(u))
    # next term of the series is -17 u^7 / 315; the rest is smaller on |u| <= 0.5
    assert np.all(err <= 0.06 * np.abs(u) ** 7 + 1e-17)
    small = u[np.abs(u) > 0.05]
    ratio = (np.tanh(small) - ora.tanh_taylor6(small)) / small ** 7
    assert np.all(np.abs(ratio + 17.0 / 315.0) < 0.02)


def test_tanh_gelu_constants_against_erf_gelu():
    x = np.linspace(-6, 6, 4001)
    tanh_gelu = 0.5 * x * (1.0 + np.tanh(ora.GELU_TANH_C * (x + ora.GELU_TANH_A * x ** 3)))
    exact = 0.5 * x * (1.0 + erf(x / math.sqrt(2.0)))
    assert np.max(np.abs(tanh_gelu - exact)) < 1e-3


def test_gelu_poly_on_the_bounded_range():
    """|x| <= 0.6 keeps |u| <= 0.5: the polynomial is the tanh-form GELU up
    to the Taylor remainder, and within 2e-4 of the exact erf GELU."""
    x = np.linspace(-0.6, 0.6, 1201)
    u = ora.GELU_TANH_C * (x + ora.GELU_TANH_A * x ** 3)
    assert np.max(np.abs(u)) <= 0.5
    tanh_gelu = 0.5 * x * (1.0 + np.tanh(u))
    assert np.all(np.abs(ora.gelu_poly(x) - tanh_gelu) <= 0.5 * np.abs(x) * 0.06 * np.abs(u) ** 7 + 1e-17)
    assert np.max(np.abs(ora.gelu_poly(x) - ora.gelu(x))) < 2e-4


def test_gelu_poly_odd_part_is_half_identity():
    x = np.linspace(-3, 3, 601)
    np.testing.assert_allclose(ora.gelu_poly(x) - ora.gelu_poly(-x), x, rtol=0, atol=1e-13)


def test_gelu_poly_grad_is_its_derivative():
    x = np.linspace(-2, 2, 401)
    h = 1e-6
    fd = (ora.gelu_poly(x + h) - ora.gelu_poly(x - h)) / (2 * h)
    np.testing.assert_allclose(ora.gelu_poly_grad(x), fd, rtol=0, atol=1e-8)


def test_qknorm_matches_torch_normalize():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((40, 3, 16)) * rng.uniform(0.01, 10, (40, 3, 1))
    x[3, 1] = 0.0  # a zero row stays zero
    y, r = qn.forward(x)
    ref = torch.nn.functional.normalize(torch.from_numpy(x), dim=-1, eps=1e-12).numpy()
    np.testing.assert_allclose(y, ref, rtol=0, atol=1e-15)
    assert np.all(y[3, 1] == 0.0)
    live = np.linalg.norm(x, axis=-1) > 0
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1)[live], 1.0, atol=1e-14)
    np.testing.assert_allclose(r[live], 1.0 / np.linalg.norm(x, axis=-1)[live], rtol=1e-14)


def test_qknorm_backward_matches_autograd():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((30, 2, 32))
    x[5, 0] = 0.0
    dy = rng.standard_normal(x.shape)
    xt = torch.from_numpy(x).requires_grad_()
    (torch.nn.functional.normalize(xt, dim=-1, eps=1e-12) * torch.from_numpy(dy)).sum().backward()
    np.testing.assert_allclose(qn.backward(x, dy), xt.grad.numpy(), rtol=1e-12, atol=1e-12)


def test_qknorm_bounds_scores():
    rng = np.random.default_rng(3)
    q, _ = qn.forward(rng.standard_normal((50, 1, 64)) * 30)
    k, _ = qn.forward(rng.standard_normal((70, 1, 64)) * 30)
    assert np.max(np.abs(q[:, 0] @ k[:, 0].T)) <= 1.0 + 1e-14


def test_single_key_gelu_poly_closed_form():
    rng = np.random.default_rng(4)
    q, k, v = (rng.standard_normal((1, 1, 8)) for _ in range(3))
    off = np.array([0, 1])
    o, lse = ora.forward(q, k, v, off, off, scale=0.7, activation="gelu_poly")
    assert lse is None
    s = 0.7 * float(q[0, 0] @ k[0, 0])
    np.testing.assert_allclose(o[0, 0], ora.gelu_poly(s) * v[0, 0], rtol=0, atol=1e-15)


def test_finite_differences_through_qknorm_and_gelu_poly():
    """loss = sum(attention(qknorm(Q), qknorm(K), V) * dO): the chain of the
    two oracles' backward functions against central differences."""
    lq = [7, 12, 0]
    lk = [9, 3, 4]
    H, D = 2, 8
    rng = np.random.default_rng(5)
    qo, ko = gen.offsets_from_lengths(lq), gen.offsets_from_lengths(lk)
    q = rng.standard_normal((qo[-1], H, D))
    k = rng.standard_normal((ko[-1], H, D))
    v = rng.standard_normal((ko[-1], H, D))
    do = rng.standard_normal((qo[-1], H, D))
    kw = dict(scale=1.0, activation="gelu_poly")

    def loss(q_, k_, v_):
        o, _ = ora.forward(qn.forward(q_)[0], qn.forward(k_)[0], v_, qo, ko, **kw)
        return float(np.sum(o * do))

    dqh, dkh, dv, _ = ora.backward(qn.forward(q)[0], qn.forward(k)[0], v, do, qo, ko, **kw)
    grads = [qn.backward(q, dqh), qn.backward(k, dkh), dv]
    eps = 1e-6
    for which, arr in enumerate([q, k, v]):
        for idx in rng.choice(arr.size, size=10, replace=False):
            args = [q.copy(), k.copy(), v.copy()]
            args[which].reshape(-1)[idx] += eps
            lp = loss(*args)
            args[which].reshape(-1)[idx] -= 2 * eps
            lm = loss(*args)
            fd = (lp - lm) / (2 * eps)
            an = grads[which].reshape(-1)[idx]
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(fd)), (which, idx, fd, an)


def test_planted_wrong_coefficient_is_caught(monkeypatch):
    """A tanh polynomial with 2/15 mistyped as 1/15 fails the remainder pin."""
    monkeypatch.setattr(ora, "tanh_taylor6", lambda u: u - u ** 3 / 3.0 + u ** 5 / 15.0)
    u = np.linspace(-0.5, 0.5, 201)
    err = np.abs(np.tanh(u) - ora.tanh_taylor6(u))
    assert not np.all(err <= 0.06 * np.abs(u) ** 7 + 1e-17)
