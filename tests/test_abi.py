"""CPU tests of the C ABI: the library loads, exports every symbol of include/opd.h, and rejects bad
arguments on the host before making any HIP call (so these run without a GPU)."""

import ctypes
import math
import os
import re

import pytest

import draft_model_distillation_amd as m
from draft_model_distillation_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.lib_path()):
        B.build()
    return m.load_library()


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "opd.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\**\s+\**([A-Za-z_][A-Za-z0-9_]*)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_header_declarations_are_all_exported(lib):
    names = _declared_functions()
    assert len(names) >= 9, names
    for n in names:
        assert hasattr(lib, n), f"{n} declared in opd.h but not exported"
    assert sorted(m.EXPORTED_SYMBOLS) == names


def test_workspace_size_and_status_strings(lib):
    assert lib.opd_workspace_size() > 0
    for s in range(9):
        assert lib.opd_status_string(s).decode().startswith("OPD_")


F32, BF16 = 0, 1
WS = 1 << 20  # any non-null, aligned fake pointers: validation must reject before dereferencing
P = 1 << 24


def _fwd(lib, z=P, y=P, dt=BF16, n=4, v=64, ld=64, a=0.5, t=0.05, loss=P, top=P, stats=P, ws=WS, wsb=None):
    wsb = lib.opd_workspace_size() if wsb is None else wsb
    return lib.opd_loss_fwd(z, y, dt, n, v, ld, a, t, loss, top, None, stats, ws, wsb, None)


def test_forward_validation(lib):
    assert _fwd(lib, z=None) == 1
    assert _fwd(lib, loss=None) == 1
    assert _fwd(lib, n=-1) == 2
    assert _fwd(lib, v=0) == 2
    assert _fwd(lib, v=(1 << 19) + 1, ld=(1 << 19) + 8) == 2
    assert _fwd(lib, ld=32) == 2
    assert _fwd(lib, dt=7) == 3
    assert _fwd(lib, z=P + 4) == 4
    assert _fwd(lib, v=63, ld=63) == 4  # bf16 pitch of 126 bytes
    assert _fwd(lib, a=1.5) == 5
    assert "alpha" in lib.opd_last_error().decode()
    assert _fwd(lib, a=float("nan")) == 5
    assert _fwd(lib, t=float("nan")) == 5
    assert _fwd(lib, ws=None) == 6
    assert _fwd(lib, wsb=16) == 6
    assert "workspace" in lib.opd_last_error().decode()


def test_backward_validation(lib):
    ws = lib.opd_workspace_size()
    assert lib.opd_loss_bwd(P, P, BF16, 4, 64, 64, 0.5, 0.05, None, P, None, P, BF16, 64, WS, ws, None) == 1
    assert lib.opd_loss_bwd(P, P, BF16, 4, 64, 64, 0.5, 0.05, P, P, None, None, BF16, 64, WS, ws, None) == 1
    assert lib.opd_loss_bwd(P, P, BF16, 4, 64, 64, 0.5, 0.05, P, P, None, P, 9, 64, WS, ws, None) == 3
    assert lib.opd_loss_bwd(P, P, BF16, 4, 64, 64, 0.5, 0.05, P, P, None, P, BF16, 60, WS, ws, None) == 2
    assert lib.opd_loss_bwd(P, P, BF16, 4, 64, 64, 0.5, 0.05, P, P, None, P, F32, 66, WS, ws, None) == 4
    assert lib.opd_loss_bwd(P, P, BF16, 4, 64, 64, -0.1, 0.05, P, P, None, P, F32, 64, WS, ws, None) == 5


def test_verify_and_fused_validation(lib):
    ws = lib.opd_workspace_size()
    blocks = m._binding.OpdBlocks(None, None, 2)
    assert lib.verify_accept_len(P, P, BF16, 4, 64, 64, None, P, P, P, WS, ws, None) == 1
    assert lib.verify_accept_len(P, P, BF16, 4, 64, 64, ctypes.byref(blocks), P, P, P, WS, ws, None) == 1
    neg = m._binding.OpdBlocks(P, P, -1)
    assert lib.verify_accept_len(P, P, BF16, 4, 64, 64, ctypes.byref(neg), P, P, P, WS, ws, None) == 2
    ok_blocks = m._binding.OpdBlocks(P, P, 2)
    assert lib.opd_fused_fwd_bwd_verify(P, P, BF16, 4, 64, 64, ctypes.byref(ok_blocks), 0.5, 0.05, None, P, P,
                                        None, P, P, BF16, 64, P, WS, ws, None) == 1
    assert lib.opd_fused_fwd_bwd_verify(P, P, BF16, 4, 64, 64, None, 0.5, float("nan"), None, P, P, P, P, P,
                                        BF16, 64, None, WS, ws, None) == 5
    assert lib.opd_fused_fwd_bwd_verify(P, P, BF16, 4, 64, 64, None, 0.5, 0.05, None, P, P, P, P, P, BF16, 64,
                                        None, WS, 100, None) == 6


def test_verify_sample_validation(lib):
    ws = lib.opd_workspace_size()
    bl = m._binding.OpdBlocks(P, P, 2)

    def call(z=P, dt=BF16, n=4, v=64, ld=64, blocks=bl, draft=P, ua=P, ur=P, t=0.8, acc=P, tok=P, lse=P, wsp=WS,
             wsb=ws):
        b = ctypes.byref(blocks) if blocks is not None else None
        return lib.opd_verify_sample(z, P, dt, n, v, ld, b, draft, ua, ur, t, acc, tok, lse, wsp, wsb, None)

    # (a call that passes validation would launch kernels on the fake pointers: never made here)
    assert call(z=None) == 1
    assert call(blocks=None) == 1
    assert call(draft=None) == 1 and call(ua=None) == 1 and call(lse=None) == 1
    assert call(ur=None) == 1 and call(acc=None) == 1 and call(tok=None) == 1
    assert call(blocks=m._binding.OpdBlocks(P, P, -1)) == 2
    assert call(blocks=m._binding.OpdBlocks(None, P, 2)) == 1
    assert call(dt=5) == 3
    assert call(ld=60) == 2
    assert call(z=P + 8) == 4
    for t in (0.0, -1.0, float("nan"), float("inf"), 1e-7):
        assert call(t=t) == 5, t
    assert "temperature" in lib.opd_last_error().decode()
    assert call(wsb=8) == 6
    # nothing to do: no rows, no blocks
    assert lib.opd_verify_sample(None, None, BF16, 0, 64, 64, ctypes.byref(m._binding.OpdBlocks(None, None, 0)),
                                 None, None, None, 1.0, None, None, None, WS, ws, None) == 0


def test_lmhead_validation(lib):
    ws = lib.opd_workspace_size()
    sc = lib.opd_lmhead_scratch_size(16, 64, 64)
    assert sc >= 16 * 64 * 4 + 16 * 64 * 2
    assert lib.opd_lmhead_scratch_size(0, 64, 64) == 0

    def call(h=P, W=P, H=32, y=P, dt=F32, n=4, v=64, ld=64, a=0.5, t=0.05, loss=P, top=P, dtop=P, st=P, dh=P,
             dW=P, scratch=P, scb=sc, rc=16, wsp=WS, wsb=ws, blocks=None):
        b = ctypes.byref(blocks) if blocks is not None else None
        return lib.opd_lmhead_fused_fwd_bwd_verify(h, W, H, y, dt, n, v, ld, b, a, t, None, loss, top, dtop, st, dh,
                                                   dW, None, None, None, scratch, scb, rc, wsp, wsb, None)

    # (a call that passes validation would launch kernels on the fake pointers: never made here)
    assert call(dt=BF16) == 3
    assert call(y=None) == 1 and call(h=None) == 1 and call(W=None) == 1
    assert call(loss=None) == 1 and call(st=None) == 1
    assert call(H=0) == 2 and call(H=12) == 4
    assert call(h=P + 8) == 4
    assert call(rc=0) == 2
    assert call(a=2.0) == 5
    need = lib.opd_lmhead_scratch_size(4, 64, 64)  # 4 rows: one chunk of min(rc, n) rows
    assert call(scratch=None) == 6 and call(scb=need - 1) == 6
    assert call(wsb=8) == 6
    assert call(blocks=m._binding.OpdBlocks(P, P, 3)) == 1  # accept_len missing
    assert call(n=0, scratch=None, dW=None) == 0  # no rows, nothing to clear: no HIP call


def test_zero_rows_accepts_null_buffers(lib):
    ws = lib.opd_workspace_size()
    # nothing to do: no HIP call is needed and NULL data pointers are fine
    assert lib.opd_loss_fwd(None, None, BF16, 0, 64, 64, 0.5, 0.05, None, None, None, None, WS, ws, None) == 0


def test_infinite_tau_is_a_valid_parameter(lib):
    # +-inf pass validation (they fail later only because there is no device here)
    r = _fwd(lib, t=math.inf, n=0)
    assert r == 0


def test_stream_probe_validation(lib):
    # checked before any HIP call: NULL buffers, a size that is not whole 16-byte vectors, misalignment
    assert lib.opd_stream_probe(None, P, P, 64, None) == 1  # only one of a, b
    assert lib.opd_stream_probe(P, None, None, 64, None) == 1
    assert lib.opd_stream_probe(None, None, None, 64, None) == 1  # nothing to stream
    assert lib.opd_stream_probe(P, P, P, 40, None) == 2
    assert lib.opd_stream_probe(P, P + 8, P, 64, None) == 4
    assert lib.opd_stream_probe(None, None, None, 0, None) == 0


def test_length_head_validation(lib):
    ws = lib.opd_workspace_size()
    # no blocks: nothing to do, NULL everything is fine
    assert lib.opd_length_head_loss(None, None, 0, None, 0, None, None, None, None, None, None, WS, ws, None) == 0
    assert lib.opd_length_head_loss(P, P, 4, P, -1, P, None, P, P, P, P, WS, ws, None) == 2
    assert lib.opd_length_head_loss(P, P, -1, P, 2, P, None, P, P, P, P, WS, ws, None) == 2
    assert lib.opd_length_head_loss(P, P, 4, P, 2, P, None, P, P, None, P, WS, ws, None) == 1
    assert lib.opd_length_head_loss(None, P, 4, P, 2, P, None, P, P, P, P, WS, ws, None) == 1
    assert lib.opd_length_head_loss(P, P, 4, P, 2, P, None, P, P, P, P, WS, 100, None) == 6
