"""Pins of the length-head epilogue oracle against things other than itself (CPU only).

The loss is checked against torch's binary_cross_entropy_with_logits (library special case), closed
forms (h = 0, the minimum at h = logit(label) with value equal to the binary entropy), the label
symmetry, central finite differences; the block targets against a differently written brute force
(first mismatch from np.nonzero) and against the pinned capped accept length with L = n_b.
"""

import math

import numpy as np
import pytest

from oracle import length_head as LH
from oracle import opd_oracle as O


def _rng(seed):
    return np.random.default_rng(seed)


def test_bce_matches_torch_library():
    torch = pytest.importorskip("torch")
    rng = _rng(1)
    h = np.concatenate([rng.normal(0, 4, 200), [-60.0, -20.0, -1e-9, 0.0, 1e-9, 20.0, 60.0]])
    lab = np.concatenate([rng.uniform(0, 1, 200), [0.0, 1.0, 0.5, 0.25, 1.0, 0.0, 1.0]])
    ref = torch.nn.functional.binary_cross_entropy_with_logits(
        torch.tensor(h, dtype=torch.float64), torch.tensor(lab, dtype=torch.float64), reduction="none").numpy()
    got = np.array([LH.bce_with_logit(a, b)[0] for a, b in zip(h, lab)])
    # absolute floor: torch rounds losses below ~1e-16 (e.g. h = -60, label 0: exact 8.8e-27) to 0
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("label", [0.0, 0.125, 0.5, 0.9375, 1.0])
def test_bce_at_zero_logit_is_log2(label):
    loss, g = LH.bce_with_logit(0.0, label)
    assert loss == pytest.approx(math.log(2.0), rel=1e-15)
    assert g == pytest.approx(0.5 - label, abs=1e-15)


@pytest.mark.parametrize("label", [0.0625, 0.3, 0.5, 0.75, 0.9375])
def test_minimum_at_logit_of_label_equals_binary_entropy(label):
    h = math.log(label / (1.0 - label))
    loss, g = LH.bce_with_logit(h, label)
    assert abs(g) < 1e-15
    entropy = -label * math.log(label) - (1 - label) * math.log(1 - label)
    assert loss == pytest.approx(entropy, rel=1e-13)


def test_label_symmetry():
    rng = _rng(2)
    for h, lab in zip(rng.normal(0, 5, 100), rng.uniform(0, 1, 100)):
        a, ga = LH.bce_with_logit(h, lab)
        b, gb = LH.bce_with_logit(-h, 1 - lab)
        assert a == pytest.approx(b, rel=1e-13)
        assert ga == pytest.approx(-gb, abs=1e-14)


def test_gradient_central_differences():
    rng = _rng(3)
    for h, lab in zip(rng.normal(0, 3, 50), rng.uniform(0, 1, 50)):
        eps = 1e-6
        fd = (LH.bce_with_logit(h + eps, lab)[0] - LH.bce_with_logit(h - eps, lab)[0]) / (2 * eps)
        assert LH.bce_with_logit(h, lab)[1] == pytest.approx(fd, abs=1e-8)


def _brute_targets(d, a, off):
    acc, lab = [], []
    for b in range(len(off) - 1):
        s, e = off[b], off[b + 1]
        mism = np.nonzero(d[s:e] != a[s:e])[0]
        k = int(mism[0]) if mism.size else e - s
        acc.append(k)
        lab.append(k / (e - s) if e > s else 0.0)
    return np.array(acc), np.array(lab)


def test_block_targets_brute_force_and_capped_relation():
    rng = _rng(4)
    for _ in range(50):
        nb = rng.integers(0, 17, size=rng.integers(1, 12))
        off = np.concatenate([[0], np.cumsum(nb)])
        n = int(off[-1])
        a = rng.integers(0, 4, n)
        d = np.where(rng.random(n) < 0.8, a, rng.integers(0, 4, n))
        acc, lab, fl = LH.block_targets(d, a, off)
        bacc, blab = _brute_targets(d, a, off)
        assert fl == 0
        assert np.array_equal(acc, bacc)
        assert np.array_equal(lab, blab)
        capped, _ = O.accept_lengths(d, a, off, np.full(len(nb), 16))
        assert np.array_equal(acc, capped)  # n_b <= 16: the uncapped prefix is the L = k verify
        assert np.all((lab >= 0) & (lab <= 1))
        assert np.array_equal(lab == 1.0, (acc == nb) & (nb > 0))


def test_malformed_offsets_and_empty_blocks():
    d = np.array([1, 2, 3, 4])
    a = np.array([1, 2, 0, 4])
    acc, lab, fl = LH.block_targets(d, a, [0, 0, 3, 2])
    assert fl == LH.LEN_FLAG_BAD_OFFSETS
    assert acc.tolist() == [0, 2, 0]  # empty block, [0..3) stops at row 2, decreasing offsets
    assert lab.tolist() == [0.0, 2 / 3, 0.0]
    out = LH.length_head_epilogue(d, a, [0, 0, 3, 2], [0.5, 0.5, 0.5], grad=[1.0, 2.0, 1.0])
    assert out["loss"][2] == 0.0 and out["dlogit"][2] == 0.0
    assert out["dlogit"][1] == pytest.approx(2.0 * (1 / (1 + math.exp(-0.5)) - 2 / 3), rel=1e-14)
