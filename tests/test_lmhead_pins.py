"""Pins of the lm_head-fused oracle (CPU only): central finite differences of the weighted total
loss with respect to the hidden states and the projection, and the identity-projection case."""

import numpy as np
import pytest

from oracle import lmhead as LM
from oracle import opd_oracle as O


def _problem(seed, R=3, V=7, H=5):
    rng = np.random.default_rng(seed)
    h = rng.normal(0, 1, (R, H))
    W = rng.normal(0, 0.7, (V, H))
    y = rng.normal(0, 1.5, (R, V))
    w = rng.uniform(0.5, 2.0, R)
    return h, W, y, w


def _total(h, W, y, w, alpha, tau):
    z = h @ W.T
    return float(np.dot(w, O.forward_rows(z, y, alpha, tau)["loss"]))


def _clip_margin(h, W, y, tau):
    z = h @ W.T
    m = np.inf
    for r in range(z.shape[0]):
        t = O.row_forward(z[r], y[r], 0.5, tau)["t"]
        m = min(m, float(np.min(np.abs(t - tau))))
    return m


@pytest.mark.parametrize("seed,alpha,tau", [(1, 0.6, 0.05), (2, 1.0, np.inf), (3, 0.0, 0.05), (4, 0.7, 0.02)])
def test_gradients_match_central_differences(seed, alpha, tau):
    h, W, y, w = _problem(seed)
    if np.isfinite(tau):
        assert _clip_margin(h, W, y, tau) > 1e-4  # no term near its clip point: the loss is smooth here
    out = LM.lmhead_fused(h, W, y, alpha, tau, grad_loss=w)
    eps = 1e-6
    for arr, grad in ((h, out["dh"]), (W, out["dW"])):
        fd = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            old = arr[idx]
            arr[idx] = old + eps
            up = _total(h, W, y, w, alpha, tau)
            arr[idx] = old - eps
            dn = _total(h, W, y, w, alpha, tau)
            arr[idx] = old
            fd[idx] = (up - dn) / (2 * eps)
        assert np.allclose(grad, fd, atol=2e-7, rtol=1e-6), np.abs(grad - fd).max()


def test_identity_projection_reduces_to_the_logit_gradient():
    rng = np.random.default_rng(5)
    V = 9
    h = rng.normal(0, 2, (4, V))
    y = rng.normal(0, 2, (4, V))
    out = LM.lmhead_fused(h, np.eye(V), y, 0.5, 0.05)
    dz, _ = O.grad_rows(h, y, 0.5, 0.05)
    assert np.array_equal(out["z"], h)
    assert np.allclose(out["dh"], dz, rtol=0, atol=1e-15)
    assert np.allclose(out["dW"], dz.T @ h, rtol=0, atol=1e-15)
    assert np.array_equal(out["draft_top1"], np.argmax(h, axis=1))


def test_logit_stats_constant_rows():
    # every logit equal: max c, LSE c + log V, and the lowest index of the (tied) maximum is 0
    for V, c in ((1, 0.25), (7, -3.0), (151936, 12.5)):
        mx, arg, lse = LM.logit_stats(np.full((2, V), c))
        assert np.all(mx == c) and np.all(arg == 0)
        assert np.allclose(lse, c + np.log(V), rtol=0, atol=1e-12)


def test_logit_stats_two_level_row_closed_form():
    # k entries at a, the rest at b < a: LSE = a + log(k + (V - k) e^(b - a)); argmax = first a
    V, k, a, b = 1000, 3, 2.0, -1.5
    z = np.full(V, b)
    pos = [17, 400, 999]
    z[pos] = a
    mx, arg, lse = LM.logit_stats(z[None, :])
    assert mx[0] == a and arg[0] == 17
    assert abs(lse[0] - (a + np.log(k + (V - k) * np.exp(b - a)))) < 1e-12


def test_logit_stats_match_an_exact_sum():
    # small rows: e^z summed with math.fsum from the definition, no shift
    import math

    rng = np.random.default_rng(11)
    z = rng.normal(0, 3, (5, 37))
    mx, arg, lse = LM.logit_stats(z)
    for r in range(5):
        assert mx[r] == max(z[r]) and arg[r] == list(z[r]).index(max(z[r]))
        assert abs(lse[r] - math.log(math.fsum(math.exp(v) for v in z[r]))) < 1e-12
