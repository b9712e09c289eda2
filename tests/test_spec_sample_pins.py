"""Pins of the speculative-sampling verification oracle against things other than itself (CPU only).

* softmax at a temperature: scipy.special.softmax and torch.softmax of the scaled logits;
* the inverse CDF: a worked example by hand and numpy.searchsorted on random weights;
* the output distribution of one verified position equals the target's q (the property that makes
  speculative sampling exact), integrated over the draft token and both uniform draws;
* the small-temperature limit reproduces the pinned greedy verification (accept lengths, and the
  target top-1 as the output token);
* z = y and u = 0 accept every verified proposal; flags for malformed inputs.
"""

import numpy as np
import pytest

from oracle import opd_oracle as O
from oracle import spec_sample as S


@pytest.mark.parametrize("T", [0.25, 0.7, 1.0, 2.0])
def test_softmax_at_temperature_matches_libraries(T):
    scipy_special = pytest.importorskip("scipy.special")
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(1)
    x = rng.normal(0, 4, 257)
    got = S.softmax_t(x, T)
    assert np.allclose(got, scipy_special.softmax(x / T), rtol=1e-13, atol=0)
    ref = torch.softmax(torch.tensor(x, dtype=torch.float64) / T, dim=0).numpy()
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-300)


def test_inverse_cdf_worked_example():
    # weights 1/4, 0, 1/2, 1/4: cumulative 0.25, 0.25, 0.75, 1.0; index 1 has no mass
    w = [0.25, 0.0, 0.5, 0.25]
    for u, want in [(0.0, 0), (0.2, 0), (0.25, 2), (0.5, 2), (0.74, 2), (0.75, 3), (0.999, 3)]:
        assert S.inverse_cdf(w, u) == want, u
    # leading zero weights are skipped even at u = 0
    assert S.inverse_cdf([0.0, 0.0, 3.0, 1.0], 0.0) == 2


def test_inverse_cdf_matches_searchsorted():
    rng = np.random.default_rng(2)
    for _ in range(200):
        n = int(rng.integers(1, 40))
        w = rng.random(n) * (rng.random(n) < 0.7)
        if w.sum() == 0:
            w[int(rng.integers(n))] = 1.0
        u = float(rng.random())
        # smallest i with cumsum[i] > u * total == number of cumsum entries <= u * total
        cs = np.cumsum(w)
        want = int(np.searchsorted(cs, u * cs[-1], side="right"))
        got = S.inverse_cdf(w, u)
        if abs(cs[want] - u * cs[-1]) > 1e-12 * cs[-1] and (want == 0 or abs(cs[want - 1] - u * cs[-1]) > 1e-12 * cs[-1]):
            assert got == want
        assert w[got] > 0


def _one_position_distribution(z, y, T, grid=2000):
    """P(output token = v) for one verified position followed by one more row, integrated over the
    draft token x ~ p, the acceptance draw and the resample draw (midpoint rule on each draw)."""
    V = z.size
    p = S.softmax_t(z, T)
    u = (np.arange(grid) + 0.5) / grid
    out = np.zeros(V)
    for x in range(V):
        # acceptance: `grid` one-row blocks (L = 1) proposing x, one per acceptance draw
        zz = np.tile(z, (grid, 1))
        yy = np.tile(y, (grid, 1))
        off = np.arange(grid + 1)
        r = S.verify_sample(zz, yy, off, np.ones(grid, int), np.full(grid, x), u, np.zeros(grid), T)
        p_acc = r["accept_len"].mean()
        # correction draw after a rejection: two-row blocks whose first proposal is always rejected
        # (u_accept just below 1 rejects whenever q(x) < p(x), the only case where rejection can happen)
        if p_acc < 1.0:
            zz = np.tile(z, (2 * grid, 1))
            yy = np.tile(y, (2 * grid, 1))
            off2 = np.arange(0, 2 * grid + 1, 2)
            ua = np.tile([1.0 - 1e-15, 0.0], grid)
            r2 = S.verify_sample(zz, yy, off2, np.ones(grid, int), np.full(2 * grid, x), ua, u, T)
            assert np.all(r2["accept_len"] == 0)
            corr = np.bincount(r2["token"], minlength=V) / grid
        else:
            corr = np.zeros(V)
        out[x] += p[x] * p_acc
        out += p[x] * (1.0 - p_acc) * corr
    return out


@pytest.mark.parametrize("T", [0.8, 1.5])
def test_one_position_output_distribution_is_the_target(T):
    rng = np.random.default_rng(3)
    z = rng.normal(0, 1.5, 5)
    y = rng.normal(0, 1.5, 5)
    got = _one_position_distribution(z, y, T)
    q = S.softmax_t(y, T)
    # midpoint-rule error: each draw's integrand is a step function, so at most 1/grid per step
    assert np.allclose(got, q, atol=2e-3), (got, q)
    assert got.sum() == pytest.approx(1.0, abs=1e-12)


def _greedy_rows(rng, n, V, gap):
    """Rows whose maximum leads the runner-up by at least `gap` (no near-ties)."""
    x = rng.normal(0, 2, (n, V))
    for r in range(n):
        i = int(rng.integers(V))
        x[r, i] = np.sort(x[r])[-1] + gap
    return x


def test_small_temperature_reduces_to_greedy_verification():
    rng = np.random.default_rng(4)
    V, nb = 64, 6
    n_blocks = 30
    n_rows = n_blocks * nb
    y = _greedy_rows(rng, n_rows, V, 0.5)
    z = y + rng.normal(0, 0.4, (n_rows, V))
    # a third of the rows get a different drafter maximum
    for r in range(n_rows):
        if rng.random() < 0.3:
            z[r, int(rng.integers(V))] = z[r].max() + 0.5
    d = np.argmax(z, axis=1)
    a = np.argmax(y, axis=1)
    off = np.arange(0, n_rows + 1, nb)
    L = rng.integers(0, nb + 1, n_blocks)
    ua = rng.uniform(1e-6, 1.0, n_rows)
    ur = rng.random(n_blocks)
    r = S.verify_sample(z, y, off, L, d, ua, ur, 1e-3)
    acc, fl = O.accept_lengths(d, a, off, L)
    assert fl == 0 and r["flags"] == 0
    assert np.array_equal(r["accept_len"], acc)
    for b in range(n_blocks):
        k = int(acc[b])
        want = a[off[b] + k] if k < nb else -1
        assert r["token"][b] == want, b


def test_identical_logits_and_zero_draws_accept_everything():
    rng = np.random.default_rng(5)
    V, nb, n_blocks = 50, 5, 8
    z = rng.normal(0, 2, (nb * n_blocks, V))
    off = np.arange(0, nb * n_blocks + 1, nb)
    L = np.array([0, 1, 2, 3, 4, 5, 5, 7])
    draft = rng.integers(0, V, nb * n_blocks)
    ur = rng.random(n_blocks)
    want_acc = np.minimum(L, nb)
    # z = y: u p(x) <= p(x) = q(x) for every u in [0, 1)
    r = S.verify_sample(z, z, off, L, draft, rng.uniform(0, 1, nb * n_blocks) * (1 - 1e-12), ur, 0.9)
    assert np.array_equal(r["accept_len"], want_acc)
    # u = 0 accepts whatever the two distributions are
    y = rng.normal(0, 2, z.shape)
    r0 = S.verify_sample(z, y, off, L, draft, np.zeros(nb * n_blocks), ur, 1.3)
    assert np.array_equal(r0["accept_len"], want_acc)
    for b in range(n_blocks):
        if want_acc[b] < nb:  # the bonus draw comes from q of the next row
            row = off[b] + want_acc[b]
            assert r0["token"][b] == S.inverse_cdf(S.softmax_t(y[row], 1.3), ur[b])
            assert r0["trace"][b]["draw"] == (row, "target")
        else:
            assert r0["token"][b] == -1


def test_flags_and_malformed_inputs():
    rng = np.random.default_rng(6)
    V = 10
    z = rng.normal(0, 1, (8, V))
    y = rng.normal(0, 1, (8, V))
    draft = np.array([1, 2, V, 3, 4, -1, 5, 6])
    r = S.verify_sample(z, y, [0, 4, 3, 8], [4, 2, -3], draft, np.zeros(8), np.full(3, 0.5), 1.0)
    assert r["flags"] == S.SAMPLE_FLAG_BAD_TOKEN | S.SAMPLE_FLAG_BAD_OFFSETS | S.SAMPLE_FLAG_NEG_L
    # block 0: rows 0, 1 accepted (u = 0), row 2 proposes V: rejected there, residual draw at row 2
    assert r["accept_len"][0] == 2 and r["trace"][0]["draw"][0] == 2
    # block 1 (4 .. 3) is malformed; block 2 verifies nothing (L < 0) and draws from q at row 3
    assert r["accept_len"][1] == 0 and r["token"][1] == -1
    assert r["accept_len"][2] == 0 and r["trace"][2]["draw"] == (3, "target")
