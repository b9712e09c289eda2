"""The library's host packer and capacity estimate against the oracle (CPU: no GPU is involved).

Packing is integer work and the EMA is the same float64 expression on both sides, so both must
match bit for bit.
"""

import ctypes

import numpy as np
import pytest

import draft_model_distillation_amd as m
from oracle import packer as PK


@pytest.fixture(scope="module")
def lib():
    return m.load_library(require_torch_runtime=False)


def test_first_fit_matches_oracle_bitwise():
    rng = np.random.default_rng(11)
    for _ in range(500):
        n = int(rng.integers(0, 300))
        lengths = rng.integers(1, 17, n)
        budget = int(rng.integers(0, 2500))
        cap = int(rng.choice([0, 0, 1, 7, 64, 128]))
        got = m.pack_first_fit(lengths, budget, cap)
        ref = PK.pack_first_fit(lengths.tolist(), budget, cap)
        assert got["selected"].tolist() == ref["selected"]
        assert got["offsets"].tolist() == ref["offsets"]
        assert got["lengths"].tolist() == ref["lengths"]
        assert got["rows"] == ref["rows"]


def test_capacity_estimate_matches_oracle_bitwise():
    rng = np.random.default_rng(12)
    for beta in [0.0, 0.3, 0.9, 0.99, 1.0]:
        est = m.CapacityEstimate(beta)
        state = None
        for obs in rng.uniform(0, 20000, 200):
            b = est.observe(obs)
            state, rb = PK.ema_update(state, obs, beta)
            assert est.estimate == state  # same float64 expression, same order
            assert b == rb


def test_packer_validation(lib):
    sel = (ctypes.c_int32 * 4)()
    off = (ctypes.c_int32 * 5)()
    pl = (ctypes.c_int32 * 4)()
    n = ctypes.c_int32()
    rows = ctypes.c_int64()
    bad = (ctypes.c_int32 * 4)(3, 0, 2, 1)
    assert lib.opd_pack_first_fit(bad, 4, 10, 0, sel, off, pl, ctypes.byref(n), ctypes.byref(rows)) == 5
    good = (ctypes.c_int32 * 4)(3, 4, 2, 1)
    assert lib.opd_pack_first_fit(good, 4, -1, 0, sel, off, pl, ctypes.byref(n), ctypes.byref(rows)) == 2
    assert lib.opd_pack_first_fit(good, 4, 10, 0, None, off, pl, ctypes.byref(n), ctypes.byref(rows)) == 1
    assert lib.opd_pack_first_fit(None, 0, 10, 0, None, off, None, ctypes.byref(n), ctypes.byref(rows)) == 0
    assert n.value == 0 and off[0] == 0
    c = m._binding.OpdCapacity()
    assert lib.opd_capacity_init(ctypes.byref(c), 1.5) == 5
    assert lib.opd_capacity_init(ctypes.byref(c), 0.5) == 0
    b = ctypes.c_int64()
    assert lib.opd_capacity_observe(ctypes.byref(c), -1.0, ctypes.byref(b)) == 5
    assert lib.opd_capacity_observe(ctypes.byref(c), float("nan"), ctypes.byref(b)) == 5
    assert lib.opd_capacity_observe(ctypes.byref(c), float("inf"), ctypes.byref(b)) == 5
    assert lib.opd_capacity_observe(ctypes.byref(c), 100.5, ctypes.byref(b)) == 0 and b.value == 100
