"""GPU parity of speculative-sampling verification (opd_verify_sample) against the float64 oracle.

Every block's accept length and drawn token are compared with oracle/spec_sample.py under the
rounding rule of tests/sample_check.py; the per-row log2-sums are compared with float64 ones. Sizes:
small ragged vocabularies (several tiles and a partial last vector, padded rows) and the 2048-row
serving workload at V = 151,936, in the launch configuration the benchmark times.
"""

import numpy as np
import pytest

import synth
from oracle import opd_oracle as O
from oracle import spec_sample as S
from tests import sample_check as C

pytestmark = pytest.mark.gpu

LOG2E = 1.4426950408889634


def _say(msg):
    print(f"[gpu-sample] {msg}", flush=True)


@pytest.fixture(scope="module")
def lib(gpu_available):
    import draft_model_distillation_amd as m

    m.load_library()
    return m


def _to_dev(x, ld, dtype_name):
    """[n, v] float64 -> (device view [n, v] with row pitch ld, exact float64 values)."""
    import torch

    n, v = x.shape
    x32 = x.astype(np.float32)
    if dtype_name == "bf16":
        bits = synth.f32_to_bf16_bits(x32)
        buf = np.full((n, ld), 0x7F80, dtype=np.uint16)  # +inf in the pad: never data
        buf[:, :v] = bits
        t = torch.from_numpy(buf.view(np.int16)).view(torch.bfloat16).cuda()
        exact = synth.bf16_bits_to_f64(bits)
    else:
        buf = np.full((n, ld), np.inf, dtype=np.float32)
        buf[:, :v] = x32
        t = torch.from_numpy(buf).cuda()
        exact = x32.astype(np.float64)
    return t[:, :v], exact


def _log2sum(x, T):
    """log2 sum_v 2^(x_v log2(e) / T) per row, float64 (in chunks of rows to bound memory)."""
    out = np.empty(x.shape[0])
    for i in range(0, x.shape[0], 128):
        s = x[i:i + 128] / T
        m = s.max(axis=1, keepdims=True)
        out[i:i + 128] = (m[:, 0] + np.log(np.exp(s - m).sum(axis=1))) * LOG2E
    return out


def _run(lib, zt, yt, off, L, draft, ua, ur, T):
    import torch

    dev = zt.device
    out = lib.verify_sample(zt, yt, torch.from_numpy(np.asarray(off, np.int32)).to(dev),
                            torch.from_numpy(np.asarray(L, np.int32)).to(dev),
                            torch.from_numpy(np.asarray(draft, np.int32)).to(dev),
                            torch.from_numpy(np.asarray(ua, np.float32)).to(dev),
                            torch.from_numpy(np.asarray(ur, np.float32)).to(dev), T)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def _read_rows(off, L, n_rows):
    """Rows the verification can read: the first min(clamp(L, 0, n_b) + 1, n_b) of each block."""
    need = np.zeros(n_rows, dtype=bool)
    for b in range(len(off) - 1):
        s, e = int(off[b]), int(off[b + 1])
        if s < 0 or e < s or e > n_rows:
            continue
        m = min(min(max(int(L[b]), 0), e - s) + 1, e - s)
        need[s:s + m] = True
    return need


def _check_all(zx, yx, off, L, draft, ua, ur, T, got, check_lse=True):
    if check_lse and zx.shape[0]:
        need = _read_rows(off, L, zx.shape[0])
        # rows no verification reads are skipped (left NaN by the binding)
        assert np.all(np.isnan(got["row_lse"][~need]))
        lz = got["row_lse"][need, 0].astype(np.float64) + got["row_lse"][need, 1]
        ly = got["row_lse"][need, 2].astype(np.float64) + got["row_lse"][need, 3]
        for name, g, x in (("z", lz, zx[need]), ("y", ly, yx[need])):
            ref = _log2sum(x, T)
            err = np.abs(g - ref)
            tol = 1e-5 + 2e-6 * np.abs(ref)
            assert np.all(err <= tol), f"log2-sum of {name}: worst {err.max():.3g} at row {int(np.argmax(err - tol))}"
    for b in range(len(off) - 1):
        s, e = int(off[b]), int(off[b + 1])
        if s < 0 or e < s or e > zx.shape[0]:
            assert got["accept_len"][b] == 0 and got["token"][b] == -1
            continue
        msg = C.check_block(zx[s:e], yx[s:e], int(L[b]), draft[s:e], ua[s:e], float(ur[b]), T,
                            int(got["accept_len"][b]), int(got["token"][b]))
        assert msg is None, f"block {b}: {msg}"


def _blocks(rng, sizes):
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    L = np.array([int(rng.integers(-1, n + 3)) if n else int(rng.integers(0, 3)) for n in sizes], dtype=np.int32)
    return off, np.maximum(L, 0)


@pytest.mark.parametrize("dtype_name", ["f32", "bf16"])
@pytest.mark.parametrize("v,T", [(1000, 1.0), (1003, 0.7), (4099, 1.6), (70001, 1.0)])
def test_sample_small_all_blocks(lib, dtype_name, v, T):
    rng = np.random.default_rng(v + int(10 * T))
    sizes = [16, 1, 0, 5, 16, 9, 3, 16, 2, 7, 16, 12]
    off, L = _blocks(rng, sizes)
    n = int(off[-1])
    y = rng.normal(0, 2.5, (n, v))
    peaks = rng.integers(0, v, n)
    y[np.arange(n), peaks] = y.max(axis=1) + rng.uniform(0, 6, n)
    z = y + rng.normal(0, 0.8, (n, v))
    epv = 8 if dtype_name == "bf16" else 4
    ld = ((v + epv - 1) // epv) * epv + 2 * epv
    zt, zx = _to_dev(z, ld, dtype_name)
    yt, yx = _to_dev(y, ld, dtype_name)
    draft = C.sample_drafts(rng, zx, T)
    ua = C.uniforms(rng, n)
    ur = C.uniforms(rng, len(sizes))
    _say(f"small {dtype_name} V={v} T={T} rows={n}")
    got = _run(lib, zt, yt, off, L, draft, ua, ur, T)
    assert lib.read_flags(clear=True) == 0
    _check_all(zx, yx, off, L, draft, ua, ur, T, got)
    # the blocks exercise rejections (residual draws) and full acceptances (draws from q)
    kinds = set()
    for b in range(len(sizes)):
        s, e = off[b], off[b + 1]
        r = S.verify_sample(zx[s:e], yx[s:e], [0, e - s], [L[b]], draft[s:e], ua[s:e], [ur[b]], T)
        kinds.add(r["trace"][0]["draw"][1])
    assert {"residual", "target"} <= kinds


def test_sample_full_size_serving_workload(lib):
    import torch

    wl = synth.make("conc128")
    rec = wl.recipe
    T = 1.0
    z = torch.from_numpy(wl.z.view(np.int16)).view(torch.bfloat16).cuda()[:, : rec.vocab]
    y = torch.from_numpy(wl.y.view(np.int16)).view(torch.bfloat16).cuda()[:, : rec.vocab]
    zx = synth.bf16_bits_to_f64(wl.z[:, : rec.vocab])
    yx = synth.bf16_bits_to_f64(wl.y[:, : rec.vocab])
    rng = np.random.default_rng(11)
    draft = C.sample_drafts(rng, zx, T)
    ua = C.uniforms(rng, wl.n_rows)
    ur = C.uniforms(rng, len(wl.lengths))
    _say(f"full conc128 rows={wl.n_rows} V={rec.vocab} T={T}")
    got = _run(lib, z, y, wl.offsets, wl.lengths, draft, ua, ur, T)
    assert lib.read_flags(clear=True) == 0
    _check_all(zx, yx, wl.offsets, wl.lengths, draft, ua, ur, T, got)
    acc = got["accept_len"]
    assert 0 < acc.sum() < wl.lengths.sum()  # both outcomes occur


def test_sample_edge_cases_and_flags(lib):
    rng = np.random.default_rng(21)
    v, n = 300, 12
    y = rng.normal(0, 2, (n, v))
    z = y + rng.normal(0, 1, (n, v))
    zt, zx = _to_dev(z, v + 4, "f32")
    yt, yx = _to_dev(y, v + 4, "f32")
    draft = C.sample_drafts(rng, zx, 1.0)
    draft[0] = v  # out of range: rejected, flagged
    ua = C.uniforms(rng, n)
    ur = C.uniforms(rng, 5)
    # blocks: [0,4) starting with the bad token, [4,4) empty, [4,8), then (with off_bad) rows 8 .. 7
    # (malformed) and [7,12) with L < 0
    off = np.array([0, 4, 4, 8, 9, 12], dtype=np.int32)
    off_bad = off.copy()
    off_bad[4] = 7  # block 3 = rows 8 .. 7: decreasing
    L = np.array([4, 2, 16, 2, -2], dtype=np.int32)
    got = _run(lib, zt, yt, off_bad, L, draft, ua, ur, 1.0)
    flags = lib.read_flags(clear=True)
    assert flags == lib.OPD_FLAG_BAD_TOKEN | lib.OPD_FLAG_BAD_OFFSETS | lib.OPD_FLAG_NEG_L
    ref = S.verify_sample(zx, yx, off_bad, L, draft, ua, ur, 1.0)
    assert ref["flags"] == flags
    assert got["accept_len"][3] == 0 and got["token"][3] == -1  # malformed
    assert got["accept_len"][1] == 0 and got["token"][1] == -1  # empty block
    assert got["accept_len"][0] == 0  # the bad token at row 0 stops the block
    _check_all(zx, yx, off_bad, L, draft, ua, ur, 1.0, got)

    # z = y accepts every verified proposal; u = 0 as well
    Lfull = np.array([4, 0, 3, 1, 4], dtype=np.int32)
    draft2 = C.sample_drafts(rng, zx, 1.0)
    got = _run(lib, yt, yt, off, Lfull, draft2, ua, ur, 1.0)
    assert lib.read_flags(clear=True) == 0
    assert np.array_equal(got["accept_len"], np.minimum(Lfull, np.diff(off)))
    _check_all(yx, yx, off, Lfull, draft2, ua, ur, 1.0, got)
    got = _run(lib, zt, yt, off, Lfull, draft2, np.zeros(n, np.float32), ur, 1.3)
    assert np.array_equal(got["accept_len"], np.minimum(Lfull, np.diff(off)))
    _check_all(zx, yx, off, Lfull, draft2, np.zeros(n), ur, 1.3, got)

    # z = y with a rejected (out-of-range) proposal: the residual q - p is zero everywhere, so the
    # draw falls back to q at that row
    draft3 = draft2.copy()
    draft3[0] = -5
    got = _run(lib, yt, yt, off, Lfull, draft3, ua, ur, 1.0)
    assert lib.read_flags(clear=True) == lib.OPD_FLAG_BAD_TOKEN
    ref = S.verify_sample(yx, yx, off, Lfull, draft3, ua, ur, 1.0)
    assert ref["trace"][0]["draw"] == (0, "target")
    assert got["accept_len"][0] == 0
    _check_all(yx, yx, off, Lfull, draft3, ua, ur, 1.0, got)


def test_sample_small_temperature_matches_greedy(lib):
    """At T = 0.02 on rows whose maxima lead by >= 0.5 the rule reduces to greedy verification."""
    import torch

    rng = np.random.default_rng(31)
    v, nb, n_blocks = 5000, 16, 24
    n = nb * n_blocks
    y = rng.normal(0, 2, (n, v))
    y[np.arange(n), rng.integers(0, v, n)] = y.max(axis=1) + 1.0
    z = y + rng.normal(0, 0.05, (n, v))
    flip = rng.random(n) < 0.2
    z[np.nonzero(flip)[0], rng.integers(0, v, int(flip.sum()))] = z[flip].max(axis=1) + 1.0
    zt, zx = _to_dev(z, v, "bf16")
    yt, yx = _to_dev(y, v, "bf16")
    d = O.top1_rows(zx)
    a = O.top1_rows(yx)
    off = np.arange(0, n + 1, nb, dtype=np.int32)
    L = rng.integers(0, nb + 1, n_blocks).astype(np.int32)
    ua = np.maximum(C.uniforms(rng, n), np.float32(1e-3))
    ur = C.uniforms(rng, n_blocks)
    got = _run(lib, zt, yt, off, L, d, ua, ur, 0.02)
    assert lib.read_flags(clear=True) == 0
    acc, _ = O.accept_lengths(d, a, off, L)
    assert np.array_equal(got["accept_len"], acc)
    for b in range(n_blocks):
        k = int(acc[b])
        assert got["token"][b] == (a[off[b] + k] if k < nb else -1), b
    # and the GPU's greedy path agrees
    _, _, acc_g = lib.verify_accept_len(zt, yt, torch.from_numpy(off).cuda(), torch.from_numpy(L).cuda())
    assert np.array_equal(acc_g.cpu().numpy(), acc)


def test_sample_deterministic(lib):
    rng = np.random.default_rng(41)
    v, n = 20000, 32
    y = rng.normal(0, 3, (n, v))
    z = y + rng.normal(0, 1.5, (n, v))
    zt, zx = _to_dev(z, v, "bf16")
    yt, yx = _to_dev(y, v, "bf16")
    off = np.arange(0, n + 1, 8, dtype=np.int32)
    L = np.full(4, 8, np.int32)
    draft = C.sample_drafts(rng, zx, 0.9)
    ua, ur = C.uniforms(rng, n), C.uniforms(rng, 4)
    g1 = _run(lib, zt, yt, off, L, draft, ua, ur, 0.9)
    g2 = _run(lib, zt, yt, off, L, draft, ua, ur, 0.9)
    for k in g1:
        assert np.array_equal(g1[k], g2[k]), k
