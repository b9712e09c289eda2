"""Seeded synthetic inputs for the OPD loss / verify path.

This module holds no arithmetic of the method itself: it only draws logits, packs requests into
blocks and converts numbers to the storage formats (float32, bfloat16). It is the one piece of code
that both the oracle side (tests, cpu baseline) and the HIP side (tests, bench) use, so that both see
the same bytes.

Workloads (logit rows shaped like serving / training of an 8B model with a 151,936-token vocabulary):

=========  =====================================================================================
name       recipe
=========  =====================================================================================
tiny       V=1000 fp32, 4 blocks x 16 rows; y ~ N(0, 2^2), planted peak +6 at a random token;
           z = y + N(0, 1); L_b ~ U{1..16}; alpha 0.5, tau 0.05; seed 0
tiny_add   as tiny but the peak is added to the token's own value instead of the row maximum
decode1    V=151936 bf16, 1 block x 16 rows; y ~ N(0, 3^2) peak +8; z = y + N(0, 1.5^2); L=16;
           alpha 0.5, tau 0.05; seed 1
conc128    V=151936 bf16, 128 blocks x 16 rows; per-block noise sigma ~ U[0.5, 3]; L_b ~ U{2..16};
           alpha 0.5, tau 0.05; seed 2
train      V=151936 bf16, 8 sequences x 2048 positions = 1024 blocks x 16 rows; base ~ N(0, 3^2)
           peak +8; z = base + N(0, 1.5^2); y = 4 * base (low temperature); L=16; alpha 0.7,
           tau 0.02; dz written bf16; seed 3
packed     V=151936 bf16, 128 requests of n_b = L_b ~ U{1..16} rows packed by int32 offsets;
           each row peaked (sigma 3, +8) or flat (sigma 1, no peak) with probability 1/2;
           noise sigma 1.5; alpha 0.5, tau 0.05; seed 4
=========  =====================================================================================

"Planted peak +P" is read as: the chosen token's logit becomes the row maximum plus P (a literal
+P on a random token of a 151,936-wide row would rarely make it the top-1).

Randomness: row r of a workload draws from ``default_rng(SeedSequence([seed, 0, r]))`` in the order
(flat-or-peaked draw for ``packed``), base normals, peak token, noise normals; block b draws its
length / noise scale from ``SeedSequence([seed, 1, b])``. Every row can therefore be generated on its
own, in any process, with identical bytes.
"""

from __future__ import annotations

import dataclasses
import math
import os
from typing import Optional, Sequence

import numpy as np

VOCAB = 151936


@dataclasses.dataclass(frozen=True)
class Recipe:
    name: str
    vocab: int
    dtype: str            # "f32" or "bf16" storage of z and y
    n_blocks: int
    block_rows: Optional[int]  # fixed rows per block, or None when rows per block = L_b (packed)
    sigma_y: float
    peak: Optional[float]
    sigma_n: float
    peak_mode: str        # "max" (token becomes max + P) or "add" (token += P)
    l_range: Optional[tuple]   # inclusive (lo, hi) for L_b, or None for L = block rows
    sigma_n_range: Optional[tuple] = None   # per-block noise sigma ~ U[lo, hi]
    y_scale: float = 1.0
    flat_prob: float = 0.0     # probability that a row is flat (sigma_flat, no peak)
    sigma_flat: float = 1.0
    alpha: float = 0.5
    tau: float = 0.05
    dz_dtype: str = "f32"
    seed: int = 0


RECIPES = {
    "tiny": Recipe("tiny", 1000, "f32", 4, 16, 2.0, 6.0, 1.0, "max", (1, 16), seed=0),
    "tiny_add": Recipe("tiny_add", 1000, "f32", 4, 16, 2.0, 6.0, 1.0, "add", (1, 16), seed=0),
    "decode1": Recipe("decode1", VOCAB, "bf16", 1, 16, 3.0, 8.0, 1.5, "max", None, dz_dtype="bf16", seed=1),
    "conc128": Recipe("conc128", VOCAB, "bf16", 128, 16, 3.0, 8.0, 1.0, "max", (2, 16),
                      sigma_n_range=(0.5, 3.0), dz_dtype="bf16", seed=2),
    "train": Recipe("train", VOCAB, "bf16", 1024, 16, 3.0, 8.0, 1.5, "max", None, y_scale=4.0,
                    alpha=0.7, tau=0.02, dz_dtype="bf16", seed=3),
    "packed": Recipe("packed", VOCAB, "bf16", 128, None, 3.0, 8.0, 1.5, "max", (1, 16), flat_prob=0.5,
                     sigma_flat=1.0, dz_dtype="bf16", seed=4),
}


# ------------------------------------------------------------------ storage formats


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even); returns uint16 bits.

    Inputs are finite by construction here.
    """
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bfloat16 bit patterns as float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


# ------------------------------------------------------------------ block layout


def block_layout(rec: Recipe):
    """Per-block lengths L, per-block noise sigma, and int32 offsets of the packed rows."""
    lens = np.zeros(rec.n_blocks, dtype=np.int32)
    sig = np.full(rec.n_blocks, rec.sigma_n, dtype=np.float64)
    rows = np.zeros(rec.n_blocks, dtype=np.int64)
    for b in range(rec.n_blocks):
        rng = np.random.default_rng(np.random.SeedSequence([rec.seed, 1, b]))
        if rec.l_range is not None:
            lens[b] = rng.integers(rec.l_range[0], rec.l_range[1] + 1)
        if rec.sigma_n_range is not None:
            sig[b] = rng.uniform(rec.sigma_n_range[0], rec.sigma_n_range[1])
        if rec.block_rows is None:
            rows[b] = lens[b]
        else:
            rows[b] = rec.block_rows
            if rec.l_range is None:
                lens[b] = rec.block_rows
    offsets = np.zeros(rec.n_blocks + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(rows)
    return lens, sig, offsets


def _row_block(offsets: np.ndarray, r: int) -> int:
    return int(np.searchsorted(offsets, r, side="right") - 1)


def gen_row(rec: Recipe, r: int, sigma_n: float):
    """Float64 (z, y) of row r before storage rounding."""
    rng = np.random.default_rng(np.random.SeedSequence([rec.seed, 0, r]))
    flat = False
    if rec.flat_prob > 0:
        flat = bool(rng.random() < rec.flat_prob)
    sigma_y = rec.sigma_flat if flat else rec.sigma_y
    base = rng.normal(0.0, sigma_y, size=rec.vocab)
    tok = int(rng.integers(rec.vocab))
    if rec.peak is not None and not flat:
        if rec.peak_mode == "max":
            base[tok] = base.max() + rec.peak
        else:
            base[tok] += rec.peak
    noise = rng.normal(0.0, sigma_n, size=rec.vocab)
    z = base + noise
    y = base * rec.y_scale
    return z, y


def _store(rec: Recipe, x64: np.ndarray) -> np.ndarray:
    x32 = x64.astype(np.float32)
    return x32 if rec.dtype == "f32" else f32_to_bf16_bits(x32)


@dataclasses.dataclass
class Workload:
    recipe: Recipe
    z: np.ndarray          # [n_rows, ld] float32 or uint16 (bf16 bits)
    y: np.ndarray
    offsets: np.ndarray    # int32 [n_blocks + 1]
    lengths: np.ndarray    # int32 [n_blocks]
    ld: int

    @property
    def n_rows(self) -> int:
        return int(self.offsets[-1])

    @property
    def vocab(self) -> int:
        return self.recipe.vocab

    def rows_f64(self, rows: Sequence[int]):
        """Exact float64 values of the stored (z, y) rows, for the oracle."""
        idx = np.asarray(rows, dtype=np.int64)
        zs = self.z[idx, : self.vocab]
        ys = self.y[idx, : self.vocab]
        if self.recipe.dtype == "f32":
            return zs.astype(np.float64), ys.astype(np.float64)
        return bf16_bits_to_f64(zs), bf16_bits_to_f64(ys)


def _fill_rows(rec, offsets, sig, z, y, r0, r1):
    for r in range(r0, r1):
        z64, y64 = gen_row(rec, r, sig[_row_block(offsets, r)])
        z[r, : rec.vocab] = _store(rec, z64)
        y[r, : rec.vocab] = _store(rec, y64)


def _worker(args):
    from multiprocessing import shared_memory

    name, shm_z, shm_y, shape, dtype, r0, r1 = args
    rec = RECIPES[name]
    lens, sig, offsets = block_layout(rec)
    mz = shared_memory.SharedMemory(name=shm_z)
    my = shared_memory.SharedMemory(name=shm_y)
    try:
        z = np.ndarray(shape, dtype=dtype, buffer=mz.buf)
        y = np.ndarray(shape, dtype=dtype, buffer=my.buf)
        _fill_rows(rec, offsets, sig, z, y, r0, r1)
        del z, y
    finally:
        mz.close()
        my.close()
    return r1 - r0


def default_workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def make(name: str, ld: Optional[int] = None, workers: Optional[int] = None) -> Workload:
    """Generate a whole workload. ``ld`` pads each row (default: V rounded up to 16 bytes).

    Large workloads are generated in parallel in forked worker processes that only run numpy and
    write straight into shared memory; call this before the GPU is first used when possible.
    """
    rec = RECIPES[name]
    lens, sig, offsets = block_layout(rec)
    n_rows = int(offsets[-1])
    esz = 4 if rec.dtype == "f32" else 2
    per_vec = 16 // esz
    if ld is None:
        ld = int(math.ceil(rec.vocab / per_vec) * per_vec)
    if ld < rec.vocab:
        raise ValueError("ld < vocab")
    dtype = np.float32 if rec.dtype == "f32" else np.uint16
    shape = (n_rows, ld)
    if workers is None:
        workers = default_workers() if n_rows * rec.vocab > 8_000_000 else 1
    if workers <= 1 or n_rows < 2:
        z = np.zeros(shape, dtype=dtype)
        y = np.zeros(shape, dtype=dtype)
        _fill_rows(rec, offsets, sig, z, y, 0, n_rows)
        return Workload(rec, z, y, offsets, lens, ld)

    import multiprocessing as mp
    from multiprocessing import shared_memory

    nbytes = max(1, n_rows * ld * esz)
    mz = shared_memory.SharedMemory(create=True, size=nbytes)
    my = shared_memory.SharedMemory(create=True, size=nbytes)
    try:
        zs = np.ndarray(shape, dtype=dtype, buffer=mz.buf)
        ys = np.ndarray(shape, dtype=dtype, buffer=my.buf)
        zs[...] = 0
        ys[...] = 0
        step = max(1, n_rows // (workers * 8))
        tasks = [(name, mz.name, my.name, shape, dtype, r, min(n_rows, r + step), ) for r in range(0, n_rows, step)]
        ctx = mp.get_context("fork")
        with ctx.Pool(workers) as pool:
            done = sum(pool.map_async(_worker, tasks).get(timeout=1800))
        assert done == n_rows
        z = np.array(zs)
        y = np.array(ys)
        del zs, ys
    finally:
        mz.close()
        mz.unlink()
        my.close()
        my.unlink()
    return Workload(rec, z, y, offsets, lens, ld)


def make_rows(name: str, rows: Sequence[int]):
    """Float64 values of selected rows exactly as ``make`` stores them (no full generation)."""
    rec = RECIPES[name]
    lens, sig, offsets = block_layout(rec)
    zs, ys = [], []
    for r in rows:
        z64, y64 = gen_row(rec, int(r), sig[_row_block(offsets, int(r))])
        zq, yq = _store(rec, z64), _store(rec, y64)
        if rec.dtype == "f32":
            zs.append(zq.astype(np.float64))
            ys.append(yq.astype(np.float64))
        else:
            zs.append(bf16_bits_to_f64(zq))
            ys.append(bf16_bits_to_f64(yq))
    return np.array(zs), np.array(ys)
