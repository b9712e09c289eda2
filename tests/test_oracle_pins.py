"""Pins for the float64 oracle, independent of its own arithmetic.

Each check compares the oracle with something it does not share code with: scipy / torch library
routines (logsumexp, softmax, rel_entr, kl_div, cross_entropy, autograd), central finite differences
of the loss, closed forms, brute force with mpmath on tiny rows, and invariants that the definition
fixes. Together they are chosen so that a dropped term, a wrong sign, a swapped KL direction, a wrong
clip side or a wrong argmax tie rule fails at least one of them.
"""

import math

import mpmath
import numpy as np
import pytest
import scipy.special as sp
import torch
import torch.nn.functional as F

from oracle import opd_oracle as O


def _rows(seed, n, v, scale=2.0, peak=None):
    rng = np.random.default_rng(seed)
    z = rng.normal(0, scale, size=(n, v))
    y = z + rng.normal(0, 1.0, size=(n, v))
    if peak is not None:
        idx = rng.integers(v, size=n)
        y[np.arange(n), idx] += peak
    return z, y


# ---------------------------------------------------------------- log-normaliser and argmax


@pytest.mark.parametrize("seed", range(5))
def test_logsumexp_matches_scipy(seed):
    rng = np.random.default_rng(seed)
    x = rng.normal(0, 10, size=777)
    assert abs(O.logsumexp(x) - sp.logsumexp(x)) < 1e-12 * max(1.0, abs(sp.logsumexp(x)))


def test_logsumexp_constant_row_closed_form():
    for c, v in [(0.0, 1), (3.5, 7), (-120.0, 1000), (80.0, 151936)]:
        assert abs(O.logsumexp(np.full(v, c)) - (c + math.log(v))) < 1e-12 * max(1.0, abs(c) + math.log(v))


def test_top1_lowest_index_brute_force():
    rng = np.random.default_rng(0)
    for _ in range(200):
        v = int(rng.integers(1, 40))
        x = rng.integers(-3, 3, size=v).astype(np.float64)  # many exact ties
        best, bi = -np.inf, -1
        for i in range(v):
            if x[i] > best:
                best, bi = x[i], i
        assert O.top1(x) == bi


def test_top1_rows_matches_rowwise_brute_force():
    rng = np.random.default_rng(1)
    x = rng.integers(-2, 2, size=(300, 17)).astype(np.float32)
    got = O.top1_rows(x)
    for i in range(x.shape[0]):
        first = min(j for j in range(17) if x[i, j] == x[i].max())
        assert got[i] == first


# ---------------------------------------------------------------- loss: library special cases


@pytest.mark.parametrize("seed", range(4))
def test_unclipped_alpha1_is_reverse_kl_scipy(seed):
    z, y = _rows(seed, 3, 50)
    for i in range(3):
        p, q = sp.softmax(z[i]), sp.softmax(y[i])
        kl_pq = float(np.sum(sp.rel_entr(p, q)))
        f = O.row_forward(z[i], y[i], 1.0, math.inf)
        assert abs(f["loss"] - kl_pq) < 1e-12
        # direction: the forward KL(q || p) is a different number on these rows
        kl_qp = float(np.sum(sp.rel_entr(q, p)))
        assert abs(f["loss"] - kl_qp) > 1e-6


@pytest.mark.parametrize("seed", range(3))
def test_unclipped_alpha1_is_torch_kl_div(seed):
    z, y = _rows(seed + 10, 4, 33)
    zt, yt = torch.tensor(z), torch.tensor(y)
    logp, logq = F.log_softmax(zt, -1), F.log_softmax(yt, -1)
    # kl_div(input=log q, target=log p, log_target) = sum p (log p - log q)
    ref = F.kl_div(logq, logp, log_target=True, reduction="none").sum(-1)
    for i in range(4):
        assert abs(O.row_forward(z[i], y[i], 1.0, math.inf)["loss"] - float(ref[i])) < 1e-12


@pytest.mark.parametrize("seed", range(3))
def test_alpha0_is_torch_cross_entropy_on_target_top1(seed):
    z, y = _rows(seed + 20, 5, 40, peak=3.0)
    zt = torch.tensor(z)
    labels = torch.tensor(np.argmax(y, axis=1))
    ref = F.cross_entropy(zt, labels, reduction="none")
    for i in range(5):
        f = O.row_forward(z[i], y[i], 0.0, 0.05)
        assert abs(f["loss"] - float(ref[i])) < 1e-12
        assert f["target_top1"] == int(labels[i])


def test_loss_is_affine_in_alpha():
    z, y = _rows(7, 3, 60, peak=4.0)
    for i in range(3):
        l0 = O.row_forward(z[i], y[i], 0.0, 0.03)["loss"]
        l1 = O.row_forward(z[i], y[i], 1.0, 0.03)["loss"]
        for a in (0.25, 0.5, 0.7):
            la = O.row_forward(z[i], y[i], a, 0.03)["loss"]
            assert abs(la - (a * l1 + (1 - a) * l0)) < 1e-12


# ---------------------------------------------------------------- clipping: invariants and brute force


def _terms_scipy(z, y):
    """Per-vocabulary reverse-KL terms p_v log(p_v / q_v) from scipy's rel_entr."""
    return sp.rel_entr(sp.softmax(z), sp.softmax(y))


@pytest.mark.parametrize("seed", range(4))
def test_clip_limits_and_slope(seed):
    z, y = _rows(seed + 30, 2, 24, scale=3.0, peak=5.0)
    for i in range(2):
        t = _terms_scipy(z[i], y[i])
        kl = float(t.sum())
        # tau above every term: no clip, plain KL
        assert abs(O.row_forward(z[i], y[i], 1.0, float(t.max()) + 1.0)["rkl_clip"] - kl) < 1e-12
        # tau below every term: every term replaced by tau
        lo = float(t.min()) - 1.0
        assert abs(O.row_forward(z[i], y[i], 1.0, lo)["rkl_clip"] - t.size * lo) < 1e-12
        # piecewise linear in tau with slope = number of terms above tau
        for tau in np.linspace(t.min() + 1e-3, t.max() - 1e-3, 9):
            if np.min(np.abs(t - tau)) < 1e-5:
                continue
            h = 1e-7
            slope = (O.row_forward(z[i], y[i], 1.0, tau + h)["rkl_clip"] -
                     O.row_forward(z[i], y[i], 1.0, tau - h)["rkl_clip"]) / (2 * h)
            assert abs(slope - np.sum(t > tau)) < 1e-5
            r = O.row_forward(z[i], y[i], 1.0, tau)["rkl_clip"]
            assert r <= kl + 1e-12


def test_clip_monotone_in_tau():
    z, y = _rows(41, 1, 30, scale=3.0, peak=6.0)
    vals = [O.row_forward(z[0], y[0], 1.0, tau)["rkl_clip"] for tau in np.linspace(-0.5, 1.5, 101)]
    assert all(b >= a - 1e-14 for a, b in zip(vals, vals[1:]))


def _mp_loss(z, y, alpha, tau, dps=50):
    """Brute-force loss in 50-digit arithmetic straight from probabilities (tiny rows only)."""
    with mpmath.workdps(dps):
        ez = [mpmath.e ** mpmath.mpf(v) for v in z]
        ey = [mpmath.e ** mpmath.mpf(v) for v in y]
        sz, sy = mpmath.fsum(ez), mpmath.fsum(ey)
        p = [e / sz for e in ez]
        q = [e / sy for e in ey]
        terms = [pi * mpmath.log(pi / qi) for pi, qi in zip(p, q)]
        clipped = mpmath.fsum([min(tv, mpmath.mpf(tau)) for tv in terms])
        a = max(range(len(y)), key=lambda k: (y[k], -k))
        ce = -mpmath.log(p[a])
        return float(alpha * clipped + (1 - alpha) * ce)


@pytest.mark.parametrize("case", [
    ([1, 2, 3, 4], [1, 2, 3, 4], 0.5, 0.05),
    ([2, 1, 0, -1], [0, 3, 0, 0], 0.5, 0.05),
    ([0, 1, 2, 0], [1, 3, 3, 0], 0.7, 0.02),
    ([2, 1, 0, -1], [0, 3, 0, 0], 0.0, 0.05),
    ([0.5, -1.0, 2.0, 0.0, 1.5], [3.0, -2.0, 0.1, 0.1, 1.0], 0.3, -0.01),
])
def test_tiny_rows_mpmath_brute_force(case):
    z, y, a, tau = case
    assert abs(O.row_forward(z, y, a, tau)["loss"] - _mp_loss(z, y, a, tau)) < 1e-13


def test_identical_distributions_closed_form():
    # z == y: every reverse-KL term is 0 (never clipped for tau >= 0), so loss = (1-alpha)(LSE - z_a)
    z = np.array([1.0, 2.0, 3.0, 4.0])
    f = O.row_forward(z, z, 0.5, 0.05)
    ce = math.log(1 + math.exp(-1) + math.exp(-2) + math.exp(-3))
    assert abs(f["rkl_clip"]) < 1e-15
    assert abs(f["loss"] - 0.5 * ce) < 1e-14
    assert f["target_top1"] == 3


def test_shift_invariance():
    z, y = _rows(50, 2, 20, peak=2.0)
    for i in range(2):
        f0 = O.row_forward(z[i], y[i], 0.6, 0.04)
        f1 = O.row_forward(z[i] + 7.25, y[i] - 3.5, 0.6, 0.04)
        assert abs(f0["loss"] - f1["loss"]) < 1e-12


# ---------------------------------------------------------------- gradient


def _safe_rows(seed, n, v, tau, scale=2.0, peak=3.0):
    z, y = _rows(seed, n, v, scale=scale, peak=peak)
    keep = []
    for i in range(n):
        t = _terms_scipy(z[i], y[i])
        if np.min(np.abs(t - tau)) > 1e-3:
            keep.append(i)
    return z[keep], y[keep]


@pytest.mark.parametrize("alpha,tau", [(0.5, 0.05), (0.7, 0.02), (1.0, 0.01), (0.3, -0.02)])
def test_gradient_central_finite_differences(alpha, tau):
    z, y = _safe_rows(60, 6, 24, tau, scale=3.0, peak=5.0)
    assert len(z) >= 2
    h = 1e-6
    for i in range(len(z)):
        dz, _ = O.row_grad(z[i], y[i], alpha, tau)
        fd = np.zeros_like(dz)
        for j in range(z.shape[1]):
            zp, zm = z[i].copy(), z[i].copy()
            zp[j] += h
            zm[j] -= h
            fd[j] = (O.row_forward(zp, y[i], alpha, tau)["loss"] - O.row_forward(zm, y[i], alpha, tau)["loss"]) / (2 * h)
        assert np.max(np.abs(fd - dz)) < 1e-7


@pytest.mark.parametrize("alpha,tau", [(0.5, 0.05), (0.7, 0.02), (0.9, 0.1)])
def test_gradient_matches_torch_autograd(alpha, tau):
    z, y = _safe_rows(70, 8, 64, tau, scale=3.0, peak=6.0)
    for i in range(len(z)):
        zt = torch.tensor(z[i], requires_grad=True)
        yt = torch.tensor(y[i])
        logp = F.log_softmax(zt, -1)
        logq = F.log_softmax(yt, -1)
        t = logp.exp() * (logp - logq)
        a = int(torch.argmax(yt))
        loss = alpha * torch.clamp(t, max=tau).sum() + (1 - alpha) * F.cross_entropy(zt[None], torch.tensor([a]))
        loss.backward()
        dz, info = O.row_grad(z[i], y[i], alpha, tau)
        assert abs(info["loss"] - loss.item()) < 1e-12
        assert np.max(np.abs(zt.grad.numpy() - dz)) < 1e-13


def test_gradient_sums_to_zero_and_scales_with_w():
    z, y = _rows(80, 5, 300, scale=3.0, peak=6.0)
    for i in range(5):
        for alpha, tau in [(0.5, 0.05), (0.7, 0.02), (1.0, -1.0), (0.2, math.inf)]:
            dz, _ = O.row_grad(z[i], y[i], alpha, tau)
            assert abs(dz.sum()) < 1e-14
            dz2, _ = O.row_grad(z[i], y[i], alpha, tau, w=-2.5)
            assert np.max(np.abs(dz2 + 2.5 * dz)) < 1e-15


def test_gradient_closed_forms():
    z, y = _rows(90, 3, 40, peak=3.0)
    for i in range(3):
        p = sp.softmax(z[i])
        # z == y: reverse-KL terms vanish and their gradient is 0 -> (1-alpha)(p - e_a)
        dz, _ = O.row_grad(z[i], z[i], 0.5, 0.05)
        e = np.zeros_like(p)
        e[np.argmax(z[i])] = 1
        assert np.max(np.abs(dz - 0.5 * (p - e))) < 1e-15
        # alpha = 1, tau = inf: gradient of KL(p||q) is p (log p - log q - KL)
        q = sp.softmax(y[i])
        kl = float(np.sum(sp.rel_entr(p, q)))
        dz, _ = O.row_grad(z[i], y[i], 1.0, math.inf)
        assert np.max(np.abs(dz - p * (np.log(p) - np.log(q) - kl))) < 1e-14
        # alpha = 0: softmax minus one-hot of the target top-1
        dz, _ = O.row_grad(z[i], y[i], 0.0, 0.05)
        e = np.zeros_like(p)
        e[np.argmax(y[i])] = 1
        assert np.max(np.abs(dz - (p - e))) < 1e-15
        # every term clipped: the reverse-KL part contributes nothing
        dz, _ = O.row_grad(z[i], y[i], 0.6, -10.0)
        assert np.max(np.abs(dz - 0.4 * (p - e))) < 1e-15


def test_tie_on_target_label():
    # y has its maximum at indices 1 and 2: the label is the lowest, 1
    z = np.array([0.0, 1.0, 2.0, 0.0])
    y = np.array([1.0, 3.0, 3.0, 0.0])
    dz, info = O.row_grad(z, y, 0.0, 0.02)
    assert info["target_top1"] == 1
    assert dz[1] < 0 and dz[2] > 0


# ---------------------------------------------------------------- accept length


def _accept_brute(d, a, off, lens):
    out = []
    for b in range(len(lens)):
        s, e = off[b], off[b + 1]
        n = min(max(lens[b], 0), e - s)
        mism = [j for j in range(n) if d[s + j] != a[s + j]]
        out.append(mism[0] if mism else n)
    return out


def test_accept_random_vs_brute_force():
    rng = np.random.default_rng(3)
    for _ in range(200):
        nb = int(rng.integers(0, 9))
        sizes = rng.integers(0, 17, size=nb)
        off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
        n = int(off[-1])
        a = rng.integers(0, 5, size=n)
        d = np.where(rng.random(n) < 0.8, a, rng.integers(0, 5, size=n))
        lens = rng.integers(0, 20, size=nb)
        got, flags = O.accept_lengths(d, a, off, lens)
        assert flags == 0
        assert list(got) == _accept_brute(d, a, off, lens)


def test_accept_malformed_inputs_are_flagged():
    d = np.array([1, 2, 3, 4])
    a = np.array([1, 2, 3, 0])
    got, flags = O.accept_lengths(d, a, [0, 2, 4], [-3, 4])
    assert list(got) == [0, 1] and flags == O.ACCEPT_FLAG_NEG_L
    got, flags = O.accept_lengths(d, a, [0, 3, 2], [4, 4])
    assert list(got) == [3, 0] and flags == O.ACCEPT_FLAG_BAD_OFFSETS
    got, flags = O.accept_lengths(d, a, [0, 5], [4])
    assert list(got) == [0] and flags == O.ACCEPT_FLAG_BAD_OFFSETS
