"""CPU tests of the Python binding's argument checks: every size, dtype, layout and device mismatch is
rejected with ValueError before any pointer reaches the library (the kernels trust the sizes they
are given, so these mistakes would otherwise read or write outside an allocation).

The tensors here are CPU tensors: structural checks run before the device check, so each mismatch
is reported as itself; a well-formed call on CPU tensors ends on the device check."""

import os
import subprocess
import sys

import pytest
import torch

import draft_model_distillation_amd as m

R, V = 6, 64


def _zy(dtype=torch.bfloat16, rows=R, vocab=V):
    return torch.zeros(rows, vocab, dtype=dtype), torch.zeros(rows, vocab, dtype=dtype)


def _blocks(n_blocks=2, dtype=torch.int32):
    off = torch.tensor([0, 3, R][: n_blocks + 1], dtype=dtype)
    return off, torch.full((n_blocks,), 3, dtype=dtype)


def _raises(fn, match):
    with pytest.raises(ValueError, match=match):
        fn()


def test_logit_pair_mismatches_are_rejected():
    z, y = _zy()
    _raises(lambda: m.opd_loss_fwd(z, y[:-1], 0.5, 0.05), "same shape")
    _raises(lambda: m.opd_loss_fwd(z, y[:, :-8], 0.5, 0.05), "same shape")
    _raises(lambda: m.opd_loss_fwd(z, y.float(), 0.5, 0.05), "same dtype")
    pad = torch.zeros(R, V + 8, dtype=torch.bfloat16)[:, :V]
    _raises(lambda: m.opd_loss_fwd(z, pad, 0.5, 0.05), "row pitch")
    _raises(lambda: m.opd_loss_fwd(z.half(), y.half(), 0.5, 0.05), "same dtype|unsupported dtype")
    _raises(lambda: m.opd_loss_fwd(z.half(), z.half(), 0.5, 0.05), "unsupported dtype")
    _raises(lambda: m.opd_loss_fwd(z[0], y[0], 0.5, 0.05), "2-D")
    _raises(lambda: m.opd_loss_fwd(z.t(), y.t(), 0.5, 0.05), "unit stride")
    # a view whose last row ends inside its last 16-byte vector, at the end of the storage: the
    # kernels read whole vectors, so the call would read past the allocation
    base = torch.zeros((R - 1) * V + 60, dtype=torch.bfloat16)
    short = base.as_strided((R, 60), (V, 1))
    _raises(lambda: m.opd_loss_fwd(short, short, 0.5, 0.05), "storage ends")
    # well formed, but on the CPU: the device check is the last one
    _raises(lambda: m.opd_loss_fwd(z, y, 0.5, 0.05), "CUDA")


def test_block_arrays_are_checked():
    z, y = _zy()
    off, L = _blocks()
    _raises(lambda: m.verify_accept_len(z, y, off.long(), L), "offsets must be torch.int32")
    _raises(lambda: m.verify_accept_len(z, y, off, L.long()), "L must be torch.int32")
    _raises(lambda: m.verify_accept_len(z, y, off, L[:1]), "L must have 2 elements")
    _raises(lambda: m.verify_accept_len(z, y, off.view(1, -1), L), "1-D")
    _raises(lambda: m.verify_accept_len(z, y, None, None), "required")
    _raises(lambda: m.verify_accept_len(z, y, off[:0], L[:0]), "n_blocks \\+ 1")
    _raises(lambda: m.opd_fused_fwd_bwd_verify(z, y, None, L, 0.5, 0.05), "without offsets")
    _raises(lambda: m.verify_accept_len(z, y, off, L), "CUDA")


def test_backward_inputs_are_checked():
    z, y = _zy()
    stats = torch.zeros(R, 8)
    top = torch.zeros(R, dtype=torch.int32)
    _raises(lambda: m.opd_loss_bwd(z, y, 0.5, 0.05, stats[:, :4].contiguous(), top), "row_stats")
    _raises(lambda: m.opd_loss_bwd(z, y, 0.5, 0.05, stats.double(), top), "row_stats")
    _raises(lambda: m.opd_loss_bwd(z, y, 0.5, 0.05, stats, top[:-1]), "target_top1 must have")
    _raises(lambda: m.opd_loss_bwd(z, y, 0.5, 0.05, stats, top.long()), "target_top1 must be")
    _raises(lambda: m.opd_loss_bwd(z, y, 0.5, 0.05, stats, top, grad_loss=torch.ones(R + 1)), "grad_loss")
    _raises(lambda: m.opd_loss_bwd(z, y, 0.5, 0.05, stats, top, dz=torch.zeros(R - 1, V)), "dz must be")
    _raises(lambda: m.opd_loss_bwd(z, y, 0.5, 0.05, stats, top, dz=torch.zeros(R, V, dtype=torch.int32)),
            "unsupported dtype")
    buf = torch.zeros(2 * R, V, dtype=torch.bfloat16)
    _raises(lambda: m.opd_loss_bwd(buf[:R], y, 0.5, 0.05, stats, top, dz=buf[R // 2: R // 2 + R]), "overlap z")
    _raises(lambda: m.opd_loss_bwd(z, buf[:R], 0.5, 0.05, stats, top, dz=buf[R - 1: 2 * R - 1]), "overlap y")
    # disjoint parts of one buffer are fine: the call gets as far as the device check
    _raises(lambda: m.opd_loss_bwd(buf[:R], y, 0.5, 0.05, stats, top, dz=buf[R:]), "CUDA")


def _fused_out(rows=R, vocab=V, n_blocks=2):
    return {
        "loss": torch.zeros(rows),
        "target_top1": torch.zeros(rows, dtype=torch.int32),
        "draft_top1": torch.zeros(rows, dtype=torch.int32),
        "row_stats": torch.zeros(rows, 8),
        "dz": torch.zeros(rows, vocab, dtype=torch.bfloat16),
        "accept_len": torch.zeros(n_blocks, dtype=torch.int32),
    }


@pytest.mark.parametrize("key,bad,match", [
    ("loss", torch.zeros(R - 1), "loss must have"),
    ("loss", torch.zeros(R, dtype=torch.float64), "loss must be"),
    ("target_top1", torch.zeros(R, dtype=torch.int64), "target_top1 must be"),
    ("draft_top1", torch.zeros(R + 1, dtype=torch.int32), "draft_top1 must have"),
    ("row_stats", torch.zeros(R, 4), "row_stats must be"),
    ("row_stats", torch.zeros(8, R).t(), "row_stats must be"),
    ("dz", torch.zeros(R, V - 8, dtype=torch.bfloat16), "dz must be"),
    ("accept_len", torch.zeros(3, dtype=torch.int32), "accept_len must have"),
    ("accept_len", torch.zeros(2, dtype=torch.float32), "accept_len must be"),
])
def test_fused_outputs_are_checked(key, bad, match):
    z, y = _zy()
    off, L = _blocks()
    o = _fused_out()
    o[key] = bad
    _raises(lambda: m.opd_fused_fwd_bwd_verify(z, y, off, L, 0.5, 0.05, out=o), match)


def test_accept_len_is_ignored_without_blocks():
    z, y = _zy()
    o = _fused_out(n_blocks=5)
    _raises(lambda: m.opd_fused_fwd_bwd_verify(z, y, None, None, 0.5, 0.05, out=o), "CUDA")


def test_fused_missing_output_and_good_call():
    z, y = _zy()
    off, L = _blocks()
    o = _fused_out()
    del o["dz"]
    _raises(lambda: m.opd_fused_fwd_bwd_verify(z, y, off, L, 0.5, 0.05, out=o), "dz")
    o = _fused_out()
    o["draft_top1"] = None
    _raises(lambda: m.opd_fused_fwd_bwd_verify(z, y, off, L, 0.5, 0.05, out=o), "draft_top1 is needed|CUDA")
    _raises(lambda: m.opd_fused_fwd_bwd_verify(z, y, off, L, 0.5, 0.05, out=_fused_out()), "CUDA")
    _raises(lambda: m.opd_fused_fwd_bwd_verify(z, y, off, L, 0.5, 0.05, grad_loss=torch.ones(R, 1, dtype=torch.float64)),
            "grad_loss")


def test_verify_sample_inputs_are_checked():
    z, y = _zy()
    off, L = _blocks()
    tok = torch.zeros(R, dtype=torch.int32)
    ua = torch.zeros(R)
    ur = torch.zeros(2)
    _raises(lambda: m.verify_sample(z, y, off, L, tok[:-1], ua, ur, 1.0), "draft_tokens")
    _raises(lambda: m.verify_sample(z, y, off, L, tok, ua.double(), ur, 1.0), "u_accept")
    _raises(lambda: m.verify_sample(z, y, off, L, tok, ua, ur[:1], 1.0), "u_resample")
    _raises(lambda: m.verify_sample(z, y, off, None, tok, ua, ur, 1.0), "L is required")
    bad = {"accept_len": torch.zeros(2, dtype=torch.int32), "token": torch.zeros(2, dtype=torch.int32),
           "row_lse": torch.zeros(R, 3)}
    _raises(lambda: m.verify_sample(z, y, off, L, tok, ua, ur, 1.0, out=bad), "row_lse")
    _raises(lambda: m.verify_sample(z, y, off, L, tok, ua, ur, 1.0), "CUDA")


def test_length_head_inputs_are_checked():
    a = torch.zeros(R, dtype=torch.int32)
    off, _ = _blocks()
    h = torch.zeros(2)
    _raises(lambda: m.length_head_loss(a, a[:-1], off, h), "draft_top1")
    _raises(lambda: m.length_head_loss(a, a.long(), off, h), "draft_top1")
    _raises(lambda: m.length_head_loss(a, a, off, h[:1]), "head_logit")
    _raises(lambda: m.length_head_loss(a, a, off, h, grad=torch.zeros(3)), "grad")
    _raises(lambda: m.length_head_loss(a, a, off.long(), h), "offsets")
    _raises(lambda: m.length_head_loss(a, a, off, h), "CUDA")


def test_lmhead_inputs_are_checked():
    H = 16
    h = torch.zeros(R, H, dtype=torch.bfloat16)
    W = torch.zeros(V, H, dtype=torch.bfloat16)
    y = torch.zeros(R, V)
    off, L = _blocks()
    _raises(lambda: m.lmhead_fused_fwd_bwd_verify(h, W[:-1], y, off, L, 0.5, 0.05), "shapes")
    _raises(lambda: m.lmhead_fused_fwd_bwd_verify(h.float(), W, y, off, L, 0.5, 0.05), "bfloat16")
    _raises(lambda: m.lmhead_fused_fwd_bwd_verify(h, W, y.bfloat16(), off, L, 0.5, 0.05), "float32")
    o = {"loss": torch.zeros(R), "target_top1": torch.zeros(R, dtype=torch.int32),
         "draft_top1": torch.zeros(R, dtype=torch.int32), "row_stats": torch.zeros(R, 8),
         "accept_len": torch.zeros(2, dtype=torch.int32), "dh": torch.zeros(R, H + 1), "dW": None}
    _raises(lambda: m.lmhead_fused_fwd_bwd_verify(h, W, y, off, L, 0.5, 0.05, out=o), "dh")
    _raises(lambda: m.lmhead_fused_fwd_bwd_verify(h, W, y, off, L, 0.5, 0.05), "CUDA")


def test_exchange_flag_range_restart_marks_workspaces_for_clearing():
    """Host flags of eager calls: when the 2^31 range is used up it restarts, and every workspace
    used before the restart must have its exchange units zeroed before its next launch; a workspace
    seen for the first time is zero by contract and needs nothing."""
    ws_a, ws_b, ws_c = 0x10000, 0x20000, 0x30000
    base, clear = m.debug_reserve_flags(ws_a, 100, next_offset=1000)
    assert base == 0x80000000 + 1000 and not clear
    base, clear = m.debug_reserve_flags(ws_b, 100)
    assert base == 0x80000000 + 1100 and not clear
    # move to the end of the range: the next reservation does not fit and restarts it
    base, clear = m.debug_reserve_flags(ws_a, 50, next_offset=(1 << 31) - 60)
    assert base == 0x80000000 + (1 << 31) - 60 and not clear
    base, clear = m.debug_reserve_flags(ws_a, 50)
    assert base == 0x80000000 and clear  # restarted; ws_a was last used in the old range
    base, clear = m.debug_reserve_flags(ws_a, 50)
    assert base == 0x80000000 + 50 and not clear  # cleared once, not again
    base, clear = m.debug_reserve_flags(ws_b, 10)
    assert clear  # ws_b too, at its first use after the restart
    base, clear = m.debug_reserve_flags(ws_c, 10)
    assert not clear  # never used before
    # every flag stays in the eager half of the 32-bit range, with room for `count` flags
    assert base >= 0x80000000 and base + 10 < (1 << 32)


def test_check_mode_switch_and_environment():
    assert m.check_mode() in (False, True)
    m.set_check(True)
    try:
        assert m.check_mode()
    finally:
        m.set_check(False)
    assert not m.check_mode()
    code = ("import ctypes, sys; sys.path.insert(0, %r); import draft_model_distillation_amd as m; "
            "print(int(m.check_mode()))" % os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    for val, want in (("1", "1"), ("0", "0")):
        env = dict(os.environ, OPD_CHECK=val)
        r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=120)
        assert r.returncode == 0, r.stderr
        assert r.stdout.strip().splitlines()[-1] == want
