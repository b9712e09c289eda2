"""GPU parity on every row of the full-size workloads, in both dz output formats.

Each 151,936-wide workload (one 16-row decode, 2048-row serving batch, 1031-row packed batch,
16,384-row training step) runs through the fused call in the launch configuration the benchmark
times. Then every row is compared with the float64 oracle:

- the loss and the row statistics;
- dz, element by element, for dz written as bf16 and as fp32;
- every top-1 and every accept length, bit for bit.

The rows are checked in a pool of forked host processes that read the inputs and the copied-back
results from the parent's memory. Rows whose dz only matches after a term within 1e-4 |tau| of the
clip is moved to the other side of it (the clip-boundary reading) are counted and reported, with the
largest number of such terms seen in one row.
"""

import multiprocessing as mp
import os

import numpy as np
import pytest

import synth
from oracle import opd_oracle as O
from tests import parity

pytestmark = pytest.mark.gpu

_G = {}  # inputs and results shared with the forked checkers
_WL = {}  # the last workload generated (each is checked with both dz formats in turn)


def _say(msg):
    print(f"[gpu-full-rows] {msg}", flush=True)


@pytest.fixture(scope="module")
def lib(gpu_available):
    import draft_model_distillation_amd as m

    m.load_library()
    return m


def _check_range(bounds):
    r0, r1 = bounds
    wl, loss, stats, dz, bf16 = _G["wl"], _G["loss"], _G["stats"], _G["dz"], _G["bf16"]
    rec = wl.recipe
    bad, boundary, max_amb = [], 0, 0
    for r in range(r0, r1):
        zs, ys = wl.rows_f64([r])
        if bf16:
            got = synth.bf16_bits_to_f64(dz[r])
        else:
            got = dz[r].astype(np.float64)
        ok, msg = parity.check_row(zs[0], ys[0], rec.alpha, rec.tau, loss[r], got, bf16_dz=bf16, got_stats=stats[r])
        if not ok:
            bad.append((r, msg))
        elif "clip-boundary" in msg:
            boundary += 1
            max_amb = max(max_amb, int(msg.split("(clip-boundary reading, ")[1].split()[0]))
    return bad, boundary, max_amb


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


CASES = [(name, dz) for name in ("decode1", "packed", "conc128", "train") for dz in ("bf16", "f32")]


@pytest.mark.parametrize("name,dz_dtype", CASES)
def test_every_row_full_size(lib, name, dz_dtype):
    import torch

    if name not in _WL:
        _WL.clear()
        _WL[name] = synth.make(name)
    wl = _WL[name]
    rec = wl.recipe
    n = wl.n_rows
    _say(f"{name}: {n} rows x V={rec.vocab}, dz {dz_dtype}")

    def dev(arr):
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).cuda()

    z = dev(wl.z)[:, : rec.vocab]
    y = dev(wl.y)[:, : rec.vocab]
    off = torch.from_numpy(wl.offsets).cuda()
    lens = torch.from_numpy(wl.lengths).cuda()
    out = lib.opd_fused_fwd_bwd_verify(z, y, off, lens, rec.alpha, rec.tau,
                                       dz_dtype=torch.bfloat16 if dz_dtype == "bf16" else torch.float32)
    torch.cuda.synchronize()
    assert lib.read_flags(clear=True) == 0
    del z, y

    # top-1s and accept lengths: every row and block, exactly
    zf = synth.bf16_bits_to_f32(wl.z[:, : rec.vocab])
    d_ref = O.top1_rows(zf)
    del zf
    yf = synth.bf16_bits_to_f32(wl.y[:, : rec.vocab])
    a_ref = O.top1_rows(yf)
    del yf
    assert np.array_equal(out["draft_top1"].cpu().numpy(), d_ref)
    assert np.array_equal(out["target_top1"].cpu().numpy(), a_ref)
    acc_ref, fl = O.accept_lengths(d_ref, a_ref, wl.offsets, wl.lengths)
    assert fl == 0 and np.array_equal(out["accept_len"].cpu().numpy(), acc_ref)

    # loss, row statistics and dz: every row, every element
    dzt = out["dz"]
    if dz_dtype == "bf16":
        dz_host = dzt.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    else:
        dz_host = dzt.contiguous().cpu().numpy()
    _G.update(wl=wl, loss=out["loss"].cpu().numpy(), stats=out["row_stats"].cpu().numpy(), dz=dz_host,
              bf16=dz_dtype == "bf16")
    del out, dzt
    torch.cuda.empty_cache()
    workers = _workers()
    step = max(1, n // (workers * 8))
    ranges = [(r, min(n, r + step)) for r in range(0, n, step)]
    try:
        with mp.get_context("fork").Pool(workers) as pool:
            res = pool.map(_check_range, ranges)
    finally:
        _G.clear()
    bad = [b for part in res for b in part[0]]
    boundary = sum(part[1] for part in res)
    max_amb = max(part[2] for part in res)
    _say(f"{name} dz {dz_dtype}: {n} rows checked on {workers} processes; {len(bad)} out of tolerance; "
         f"{boundary} rows matched under the clip-boundary reading (at most {max_amb} ambiguous terms in a row)")
    assert not bad, f"{len(bad)} rows out of tolerance, first: {bad[:3]}"
