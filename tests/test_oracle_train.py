"""Pins of the oracle's MSE training (DeltaKV page, section 3, "Obiettivo di
Training Ibrido", the reconstruction-fidelity term): the backpropagated
gradient against central finite differences of the loss (a separate forward
pass: the C oracle's MLP), the orthogonal pair's zero loss and gradient, the
GELU derivative, and descent."""
import numpy as np
import pytest

import oracle


def _pair(d, h, dc, act, seed, scale=0.4):
    rng = np.random.default_rng(seed)
    comp = oracle.MLP(rng.normal(0, scale, (h, d)), rng.normal(0, 0.1, h),
                      rng.normal(0, scale, (dc, h)), rng.normal(0, 0.1, dc), act)
    dec = oracle.MLP(rng.normal(0, scale, (h, dc)), rng.normal(0, 0.1, h),
                     rng.normal(0, scale, (d, h)), rng.normal(0, 0.1, d), act)
    return comp, dec


@pytest.mark.parametrize("act", [oracle.ACT_GELU, oracle.ACT_IDENTITY])
def test_gradient_equals_central_differences_of_the_loss(act):
    d, h, dc, n = 5, 6, 3, 7
    comp, dec = _pair(d, h, dc, act, seed=11 + act)
    delta = np.random.default_rng(12).normal(0, 1, (n, d))
    loss, g = oracle.reconstruction_grad(delta, comp, dec)
    assert abs(loss - oracle.reconstruction_loss(delta, comp, dec)) <= 1e-13 * max(1.0, loss)
    theta = oracle.pack_params(comp, dec)
    eps = 1e-5
    fd = np.zeros_like(theta)
    for i in range(len(theta)):
        tp, tm = theta.copy(), theta.copy()
        tp[i] += eps
        tm[i] -= eps
        lp = oracle.reconstruction_loss(delta, *oracle.unpack_params(tp, comp, dec))
        lm = oracle.reconstruction_loss(delta, *oracle.unpack_params(tm, comp, dec))
        fd[i] = (lp - lm) / (2 * eps)
    # every parameter (weights and biases of all four layers) is checked
    err = np.abs(fd - g).max() / np.abs(g).max()
    assert err < 1e-7, err
    assert np.abs(g).min() >= 0 and np.count_nonzero(g) == len(g)


def test_orthogonal_pair_reconstructs_exactly_and_has_zero_gradient():
    # identity activations, d_c = d: W2d W1d W2c W1c = Q^T Q = I and zero
    # biases rebuild every residual row, so the loss and its gradient vanish
    d = 8
    q, _ = np.linalg.qr(np.random.default_rng(13).normal(size=(d, d)))
    z = np.zeros(d)
    comp = oracle.MLP(q, z, np.eye(d), z, oracle.ACT_IDENTITY)
    dec = oracle.MLP(q.T, z, np.eye(d), z, oracle.ACT_IDENTITY)
    delta = np.random.default_rng(14).normal(0, 3, (20, d))
    loss, g = oracle.reconstruction_grad(delta, comp, dec)
    assert loss < 1e-28 and np.abs(g).max() < 1e-13
    assert oracle.reconstruction_loss(delta, comp, dec) < 1e-28


def test_gelu_and_its_derivative():
    u = np.linspace(-6, 6, 97)
    assert np.allclose(oracle.gelu_vec(u), [oracle.gelu(x) for x in u], rtol=1e-14, atol=1e-15)
    h = 1e-6
    fd = (oracle.gelu_vec(u + h) - oracle.gelu_vec(u - h)) / (2 * h)
    assert np.abs(fd - oracle.gelu_deriv(u)).max() < 1e-8
    # limits: derivative 0 far left, 1 far right, 1/2 at 0
    assert abs(oracle.gelu_deriv(np.array([0.0]))[0] - 0.5) < 1e-15
    assert abs(oracle.gelu_deriv(np.array([-40.0]))[0]) < 1e-15
    assert abs(oracle.gelu_deriv(np.array([40.0]))[0] - 1.0) < 1e-15


@pytest.mark.parametrize("momentum", [0.0, 0.9])
def test_small_steps_lower_the_loss(momentum):
    d, h, dc, n = 16, 32, 4, 200
    comp, dec = _pair(d, h, dc, oracle.ACT_GELU, seed=15, scale=0.3)
    delta = np.random.default_rng(16).normal(0, 1, (n, d))
    first = oracle.reconstruction_loss(delta, comp, dec)
    vel = None
    losses = []
    for _ in range(30):
        loss, _, comp, dec, vel = oracle.train_step(delta, comp, dec, lr=0.05,
                                                    momentum=momentum, velocity=vel)
        losses.append(loss)
    assert losses[0] == pytest.approx(first, rel=1e-12)
    last = oracle.reconstruction_loss(delta, comp, dec)
    assert last < 0.9 * first
    if momentum == 0.0:   # plain descent with a small step never goes up
        assert all(b <= a for a, b in zip(losses, losses[1:]))
