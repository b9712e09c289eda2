"""GPU parity of the lm_head-fused path (opd_lmhead_fused_fwd_bwd_verify) against the float64 oracle.

The oracle forms z = h W^T in float64 from the exact bf16 inputs; the GPU forms it with fp32
accumulation (the library's MFMA product kernels) and runs the row kernel on it, then dh and dW from
the bf16-rounded dz. The logits product's epilogue statistics (max, lowest argmax, log-sum-exp per
row) are checked against the oracle's definitions (the max and LSE within the fp32-logits bound used
for the row kernel's LSE, the argmax like the draft top-1) and against the row kernel's own draft
top-1 and LSE(z) on the same fp32 logits (the argmax exactly).
Bounds used (per element of dh and dW): the row kernel's dz tolerance (2e-5 absolute) plus the bf16
rounding of dz (a relative 2^-9, allowed as 2^-8) carried through the product with |W| or |h|; the
fp32 accumulation of the products is far below that. The loss within 1e-3 relative + 3e-5 (the
fp32 logits move LSE by ~1e-5 at most here), the target top-1 and accept lengths exactly, the draft
top-1 exactly except where two logits are within 1e-4 (fp32 accumulation may order them either
way). Inputs avoid reverse-KL terms within 1e-3 tau of the clip point, where a term may land on
either side.

Sizes: a few chunks with a ragged last chunk at V = 1000 and 1003, H = 64 / 72 (K steps with a
partial last step in all three products, and dz rows whose bf16 padding the dh product must mask),
one single-row call; the full vocabulary
151,936 with H = 4096 over 64 rows in three chunks (every output compared); and the benchmark's
configuration (2048 rows, one chunk) on sampled rows.
"""

import numpy as np
import pytest

import synth
from oracle import lmhead as LM
from oracle import opd_oracle as O

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu-lmhead] {msg}", flush=True)


@pytest.fixture(scope="module")
def lib(gpu_available):
    import draft_model_distillation_amd as m

    m.load_library()
    return m


def _bf16(x):
    """float array -> (bf16 bit pattern uint16, exact float64 values)."""
    bits = synth.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))
    return bits, synth.bf16_bits_to_f64(bits)


def _problem(seed, R, V, H, wscale, noise=1.0):
    rng = np.random.default_rng(seed)
    hb, h = _bf16(rng.standard_normal((R, H), dtype=np.float32))
    Wb, W = _bf16(rng.standard_normal((V, H), dtype=np.float32) * np.float32(wscale))
    z = h @ W.T
    y = (z + rng.normal(0, noise, (R, V))).astype(np.float32).astype(np.float64)
    return rng, hb, h, Wb, W, y


def _dev(lib, hb, Wb, y, ld):
    import torch

    R, V = y.shape
    ht = torch.from_numpy(hb.view(np.int16)).view(torch.bfloat16).cuda()
    Wt = torch.from_numpy(Wb.view(np.int16)).view(torch.bfloat16).cuda()
    buf = np.full((R, ld), np.inf, dtype=np.float32)
    buf[:, :V] = y
    yt = torch.from_numpy(buf).cuda()[:, :V]
    return ht, Wt, yt


def _clip_margin(z, y, tau, rows=None):
    m = np.inf
    for r in (range(z.shape[0]) if rows is None else rows):
        t = O.row_forward(z[r], y[r], 0.5, tau)["t"]
        m = min(m, float(np.min(np.abs(t - tau))))
    return m


def _check_draft_top1(z, d_gpu, rows):
    for i, r in enumerate(rows):
        d_ref = int(np.argmax(z[i]))
        if int(d_gpu[r]) != d_ref:
            gap = z[i][d_ref] - z[i][int(d_gpu[r])]
            assert gap <= 1e-4 * (1 + abs(z[i][d_ref])), f"row {r}: draft top-1 {d_gpu[r]} vs {d_ref} (gap {gap})"


def _run_and_check_all(lib, seed, R, V, H, ld, chunk, wscale, alpha, tau, blocks):
    import torch

    rng, hb, h, Wb, W, y = _problem(seed, R, V, H, wscale)
    off, L = blocks
    w = rng.uniform(0.5, 1.5, R)
    ref = LM.lmhead_fused(h, W, y, alpha, tau, off, L, grad_loss=w)
    assert _clip_margin(ref["z"], y, tau) > 1e-3 * tau, "inputs put a term at its clip point"
    ht, Wt, yt = _dev(lib, hb, Wb, y, ld)
    _say(f"lmhead R={R} V={V} H={H} chunk={chunk}")
    out = lib.lmhead_fused_fwd_bwd_verify(ht, Wt, yt, torch.from_numpy(off).cuda(), torch.from_numpy(L).cuda(),
                                          alpha, tau, grad_loss=torch.from_numpy(w.astype(np.float32)).cuda(),
                                          chunk_rows=chunk)
    torch.cuda.synchronize()
    assert lib.read_flags(clear=True) == 0
    g = {k: (v.cpu().numpy() if v is not None and k != "scratch" else None) for k, v in out.items()}
    assert np.array_equal(g["target_top1"], ref["target_top1"])
    _check_draft_top1(ref["z"], g["draft_top1"], range(R))
    acc_gpu, _ = O.accept_lengths(g["draft_top1"], g["target_top1"], off, L)
    assert np.array_equal(g["accept_len"], acc_gpu)
    if np.array_equal(g["draft_top1"], ref["draft_top1"]):
        assert np.array_equal(g["accept_len"], ref["accept_len"])
    assert np.all(np.abs(g["loss"] - ref["loss"]) <= 1e-3 * np.abs(ref["loss"]) + 3e-5)
    lse = ref["z"].max(axis=1) + np.log(np.exp(ref["z"] - ref["z"].max(axis=1, keepdims=True)).sum(axis=1))
    assert np.all(np.abs(g["row_stats"][:, 0] - lse) <= 2e-5 * (1 + np.abs(lse)))
    slack = 2e-5 + 2.0 ** -8 * np.abs(ref["dz"])
    tol_dh = slack @ np.abs(W) + 1e-6
    tol_dW = slack.T @ np.abs(h) + 1e-6
    err = np.abs(g["dh"] - ref["dh"])
    assert np.all(err <= tol_dh), f"dh: worst excess {np.max(err - tol_dh):.3g}"
    err = np.abs(g["dW"] - ref["dW"])
    assert np.all(err <= tol_dW), f"dW: worst excess {np.max(err - tol_dW):.3g}"
    # the bound is not vacuous: the typical error sits far below it
    assert np.median(np.abs(g["dh"] - ref["dh"])) < 0.1 * np.median(tol_dh)
    _check_logit_stats(g, ref["logit_max"], ref["logit_lse"], ref["z"], range(R))


def _check_logit_stats(g, mx_ref, lse_ref, z_ref, rows):
    rows = list(rows)
    ml = g["logit_max_lse"][rows]
    assert np.all(np.abs(ml[:, 0] - mx_ref) <= 2e-5 * (1 + np.abs(mx_ref)))
    assert np.all(np.abs(ml[:, 1] - lse_ref) <= 2e-5 * (1 + np.abs(lse_ref)))
    _check_draft_top1(z_ref, g["logit_argmax"], rows)
    # the same fp32 logits as the row kernel's: the same lowest argmax, and LSE(z) to fp32 rounding
    assert np.array_equal(g["logit_argmax"][rows], g["draft_top1"][rows])
    lse_team = g["row_stats"][rows, 0]
    assert np.all(np.abs(ml[:, 1] - lse_team) <= 2e-6 * (1 + np.abs(lse_team)))


@pytest.mark.parametrize("seed,R,V,H,ld,chunk", [(1, 40, 1000, 64, 1000, 16), (2, 37, 1003, 72, 1008, 10),
                                                 (12, 300, 2053, 136, 2056, 300)])
def test_lmhead_small_chunks(lib, seed, R, V, H, ld, chunk):
    off = np.array([0, 16, 20, 20, R], dtype=np.int32)
    L = np.array([16, 3, 0, 9], dtype=np.int32)
    _run_and_check_all(lib, seed, R, V, H, ld, chunk, 0.35, 0.6, 0.05, (off, L))


def test_lmhead_single_row(lib):
    off = np.array([0, 1], dtype=np.int32)
    L = np.array([1], dtype=np.int32)
    _run_and_check_all(lib, 8, 1, 777, 40, 780, 5, 0.35, 0.6, 0.05, (off, L))


def test_lmhead_full_vocab_hidden_4096(lib):
    off = np.array([0, 16, 32, 48, 64], dtype=np.int32)
    L = np.array([16, 16, 8, 16], dtype=np.int32)
    _run_and_check_all(lib, 3, 64, 151936, 4096, 151936, 24, 0.047, 0.5, 0.05, (off, L))


def test_lmhead_benchmark_configuration_sampled_rows(lib):
    """2048 rows, H = 4096, one chunk of 2048 rows (as the benchmark runs it): sampled rows' loss,
    top-1s and dh rows against the oracle, and the determinism of two calls."""
    import torch

    R, V, H = 2048, 151936, 4096
    rng = np.random.default_rng(4)
    hb, h = _bf16(rng.standard_normal((R, H), dtype=np.float32))
    Wb, W = _bf16(rng.standard_normal((V, H), dtype=np.float32) * np.float32(0.047))
    ht = torch.from_numpy(hb.view(np.int16)).view(torch.bfloat16).cuda()
    Wt = torch.from_numpy(Wb.view(np.int16)).view(torch.bfloat16).cuda()
    # target logits: the drafter's own logits (fp32 from torch on the device) plus seeded noise, so
    # that the two distributions are close; the oracle reads the same fp32 values back
    g = torch.Generator(device="cuda").manual_seed(5)
    Wf_t = Wt.float().t().contiguous()
    yt = (torch.matmul(ht.float(), Wf_t) + torch.randn(R, V, generator=g, device="cuda")).contiguous()
    del Wf_t
    off = torch.arange(0, R + 1, 16, dtype=torch.int32, device="cuda")
    L = torch.full((R // 16,), 16, dtype=torch.int32, device="cuda")
    _say("lmhead benchmark configuration R=2048 V=151936 H=4096")
    out = lib.lmhead_fused_fwd_bwd_verify(ht, Wt, yt, off, L, 0.5, 0.05, chunk_rows=2048)
    torch.cuda.synchronize()
    assert lib.read_flags(clear=True) == 0
    rows = np.sort(rng.choice(R, 8, replace=False))
    y_rows = yt[torch.from_numpy(rows).cuda()].cpu().numpy().astype(np.float64)
    z_rows = LM.lmhead_rows(h, W, rows)
    assert _clip_margin(z_rows, y_rows, 0.05) > 5e-5
    loss = out["loss"].cpu().numpy()
    a = out["target_top1"].cpu().numpy()
    d = out["draft_top1"].cpu().numpy()
    dh = out["dh"].cpu().numpy()
    _check_draft_top1(z_rows, d, rows)
    for i, r in enumerate(rows):
        f = O.row_forward(z_rows[i], y_rows[i], 0.5, 0.05)
        assert a[r] == f["target_top1"]
        assert abs(loss[r] - f["loss"]) <= 1e-3 * abs(f["loss"]) + 3e-5
        dz, _ = O.row_grad(z_rows[i], y_rows[i], 0.5, 0.05)
        ref = dz @ W
        tol = (2e-5 + 2.0 ** -8 * np.abs(dz)) @ np.abs(W) + 1e-6
        assert np.all(np.abs(dh[r] - ref) <= tol), f"row {r}"
    g = {k: out[k].cpu().numpy() for k in ("logit_max_lse", "logit_argmax", "draft_top1", "row_stats")}
    mx, _, lse = LM.logit_stats(z_rows)
    _check_logit_stats(g, mx, lse, z_rows, rows)
    # over every row: the epilogue's argmax is the row kernel's draft top-1, its LSE the kernel's LSE(z)
    assert np.array_equal(g["logit_argmax"], g["draft_top1"])
    assert np.all(np.abs(g["logit_max_lse"][:, 1] - g["row_stats"][:, 0]) <= 2e-6 * (1 + np.abs(g["row_stats"][:, 0])))
    out2 = lib.lmhead_fused_fwd_bwd_verify(ht, Wt, yt, off, L, 0.5, 0.05, chunk_rows=2048)
    torch.cuda.synchronize()
    for k in ("loss", "dh", "dW", "accept_len", "logit_max_lse", "logit_argmax"):
        assert torch.equal(out[k], out2[k]), k


def test_lmhead_optional_outputs_and_empty_batch(lib):
    """dh / dW may be skipped (their products are not run) and the rest is unchanged; no rows gives
    a zero dW and no accept lengths to compute."""
    import torch

    rng, hb, h, Wb, W, y = _problem(6, 20, 520, 32, 0.5)
    ht, Wt, yt = _dev(lib, hb, Wb, y, 520)
    off = torch.tensor([0, 8, 20], dtype=torch.int32, device="cuda")
    L = torch.tensor([8, 12], dtype=torch.int32, device="cuda")
    full = lib.lmhead_fused_fwd_bwd_verify(ht, Wt, yt, off, L, 0.5, 0.05, chunk_rows=7)
    part = lib.lmhead_fused_fwd_bwd_verify(ht, Wt, yt, off, L, 0.5, 0.05, chunk_rows=7, want_dh=False, want_dW=False)
    torch.cuda.synchronize()
    assert lib.read_flags(clear=True) == 0
    assert part["dh"] is None and part["dW"] is None
    for k in ("loss", "target_top1", "draft_top1", "row_stats", "accept_len", "logit_max_lse", "logit_argmax"):
        assert torch.equal(full[k], part[k]), k
    nost = lib.lmhead_fused_fwd_bwd_verify(ht, Wt, yt, off, L, 0.5, 0.05, chunk_rows=7, want_logit_stats=False)
    torch.cuda.synchronize()
    assert nost["logit_max_lse"] is None and nost["logit_argmax"] is None
    for k in ("loss", "target_top1", "draft_top1", "row_stats", "accept_len", "dh", "dW"):
        assert torch.equal(full[k], nost[k]), k
    # grad_loss = 0 on every row: zero gradients
    zero = lib.lmhead_fused_fwd_bwd_verify(ht, Wt, yt, off, L, 0.5, 0.05, chunk_rows=7,
                                           grad_loss=torch.zeros(20, dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()
    assert torch.count_nonzero(zero["dh"]) == 0 and torch.count_nonzero(zero["dW"]) == 0
    # no rows
    e = lib.lmhead_fused_fwd_bwd_verify(ht[:0], Wt, yt[:0], None, None, 0.5, 0.05)
    torch.cuda.synchronize()
    assert e["dW"].shape == (520, 32) and torch.count_nonzero(e["dW"]) == 0
