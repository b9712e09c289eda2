"""Parity checker: HIP results against the float64 oracle, row by row.

Tolerances (fp32 accumulation on the GPU, float64 oracle):
  * target / draft top-1 and accept lengths: bit-exact (argmax is taken on exactly decoded inputs).
  * loss: |gpu - ref| <= 1e-3 |ref| + 1e-5  (the absolute floor covers losses near 0, where fp32
    rounding of the log-normaliser, about half an ulp of LSE, dominates).
  * dz written fp32: |gpu - ref| <= 2e-5.
  * dz written bf16: |gpu - ref| <= 2e-5 + ulp_bf16 / 2 (the oracle value within 2e-5, then rounded
    to nearest even into bf16).
  * clip boundary: a term whose t_v lies within 1e-4 |tau| of tau may fall on either side of the
    clip in fp32; dz is accepted if it matches the oracle under any assignment of those (at most 4)
    terms. The loss is continuous there, so it needs no such allowance.
"""

from __future__ import annotations

import itertools
import math

import numpy as np

from oracle import opd_oracle as O

LOSS_REL = 1e-3
LOSS_ABS = 1e-5
DZ_ABS = 2e-5
AMBIG_REL = 1e-4
MAX_AMBIG = 4


def ulp_bf16(x: np.ndarray) -> np.ndarray:
    ax = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(ax, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def dz_tolerance(ref: np.ndarray, got: np.ndarray, bf16: bool) -> np.ndarray:
    if not bf16:
        return np.full(ref.shape, DZ_ABS)
    return DZ_ABS + 0.5 * ulp_bf16(np.maximum(np.abs(ref), np.abs(got)))


def check_loss(got: float, ref: float) -> bool:
    return abs(got - ref) <= LOSS_REL * abs(ref) + LOSS_ABS


def check_row(z, y, alpha, tau, got_loss, got_dz=None, bf16_dz=False, w=1.0, got_stats=None):
    """Compare one row; returns (ok, message)."""
    dz_ref, info = O.row_grad(z, y, alpha, tau, w)
    if not check_loss(float(got_loss), info["loss"]):
        return False, f"loss {got_loss!r} vs {info['loss']!r}"
    if got_stats is not None:
        lz, ly, s, rk = (float(v) for v in got_stats[:4])
        if abs(lz - info["lse_z"]) > 1e-6 * max(1.0, abs(info["lse_z"])) + 1e-6:
            return False, f"lse_z {lz} vs {info['lse_z']}"
        if abs(ly - info["lse_y"]) > 1e-6 * max(1.0, abs(info["lse_y"])) + 1e-6:
            return False, f"lse_y {ly} vs {info['lse_y']}"
        if not check_loss(rk, info["rkl_clip"]):
            return False, f"rkl_clip {rk} vs {info['rkl_clip']}"
        if len(got_stats) >= 8:
            mz, lnsz, dl, ce = (float(v) for v in got_stats[4:8])
            if mz != float(np.max(z)):
                return False, f"row max {mz} vs {np.max(z)}"
            if abs((mz + lnsz) - info["lse_z"]) > 1e-6 * max(1.0, abs(info["lse_z"])) + 1e-6:
                return False, f"max + log sum {mz + lnsz} vs {info['lse_z']}"
            if abs(dl - (info["lse_z"] - info["lse_y"])) > 2e-6 * max(1.0, abs(info["lse_z"] - info["lse_y"])) + 2e-6:
                return False, f"delta {dl} vs {info['lse_z'] - info['lse_y']}"
            if not check_loss(ce, info["ce"]):
                return False, f"ce {ce} vs {info['ce']}"
    if got_dz is None:
        return True, "ok"
    got_dz = np.asarray(got_dz, dtype=np.float64)
    tol = dz_tolerance(dz_ref, got_dz, bf16_dz)
    if np.all(np.abs(got_dz - dz_ref) <= tol):
        return True, "ok"
    amb = np.nonzero(np.abs(info["t"] - tau) <= AMBIG_REL * abs(tau))[0] if math.isfinite(tau) else np.array([], int)
    if 0 < amb.size <= MAX_AMBIG:
        base = info["clipped"].copy()
        for bits in itertools.product([False, True], repeat=amb.size):
            mask = base.copy()
            mask[amb] = bits
            alt, _ = O.row_grad(z, y, alpha, tau, w, clipped=mask)
            if np.all(np.abs(got_dz - alt) <= dz_tolerance(alt, got_dz, bf16_dz)):
                return True, f"ok (clip-boundary reading, {amb.size} ambiguous terms)"
    err = np.abs(got_dz - dz_ref) - tol
    j = int(np.argmax(err))
    return False, (f"dz[{j}] = {got_dz[j]!r} vs {dz_ref[j]!r} (tol {tol[j]:.3g}); "
                   f"{int(np.sum(err > 0))} elements out; {amb.size} ambiguous clip terms")

