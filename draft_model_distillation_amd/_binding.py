"""ctypes binding of libopd_mi355x.so (the C ABI declared in include/opd.h).

Argument marshalling only: every step of the path runs in the HIP library. PyTorch provides device
memory (tensors) and the stream (``torch.cuda.current_stream().cuda_stream``). If the library is not
built this module raises instead of computing anything another way.
"""

from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional

from . import build as _build

OPD_F32 = 0
OPD_BF16 = 1
OPD_FLAG_NEG_L = 1
OPD_FLAG_BAD_OFFSETS = 2
OPD_FLAG_SPIN_TIMEOUT = 4
OPD_FLAG_BAD_TOKEN = 8

EXPORTED_SYMBOLS = (
    "opd_workspace_size",
    "opd_loss_fwd",
    "opd_loss_bwd",
    "verify_accept_len",
    "opd_fused_fwd_bwd_verify",
    "opd_read_flags",
    "opd_length_head_loss",
    "opd_verify_sample",
    "opd_lmhead_scratch_size",
    "opd_lmhead_fused_fwd_bwd_verify",
    "opd_capacity_init",
    "opd_capacity_observe",
    "opd_pack_first_fit",
    "opd_stream_probe",
    "opd_set_spin_limit",
    "opd_status_string",
    "opd_last_error",
)


class OpdBlocks(ctypes.Structure):
    _fields_ = [("offsets", ctypes.c_void_p), ("L", ctypes.c_void_p), ("n_blocks", ctypes.c_int32)]


_lock = threading.Lock()
_lib = None


def library_path() -> str:
    """The in-tree build, or the file named by OPD_MI355X_LIB (for trying alternative builds)."""
    return os.environ.get("OPD_MI355X_LIB") or _build.lib_path()


def load_library(require_torch_runtime: bool = True) -> ctypes.CDLL:
    """Load the HIP library. torch is imported first so that its HIP runtime is the one in use."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if require_torch_runtime:
            import torch  # noqa: F401  (loads the process's HIP runtime)
        path = library_path()
        if not os.path.exists(path):
            raise ImportError(
                f"HIP library {path} is not built; run `python -m draft_model_distillation_amd.build` "
                "(or __graft_entry__.build()) first"
            )
        lib = ctypes.CDLL(path)
        vp, i64, f32, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int, ctypes.c_size_t
        lib.opd_workspace_size.restype = sz
        lib.opd_workspace_size.argtypes = []
        lib.opd_loss_fwd.restype = i32
        lib.opd_loss_fwd.argtypes = [vp, vp, i32, i64, i64, i64, f32, f32, vp, vp, vp, vp, vp, sz, vp]
        lib.opd_loss_bwd.restype = i32
        lib.opd_loss_bwd.argtypes = [vp, vp, i32, i64, i64, i64, f32, f32, vp, vp, vp, vp, i32, i64, vp, sz, vp]
        lib.verify_accept_len.restype = i32
        lib.verify_accept_len.argtypes = [vp, vp, i32, i64, i64, i64, ctypes.POINTER(OpdBlocks), vp, vp, vp, vp, sz, vp]
        lib.opd_fused_fwd_bwd_verify.restype = i32
        lib.opd_fused_fwd_bwd_verify.argtypes = [vp, vp, i32, i64, i64, i64, ctypes.POINTER(OpdBlocks), f32, f32,
                                                 vp, vp, vp, vp, vp, vp, i32, i64, vp, vp, sz, vp]
        lib.opd_read_flags.restype = i32
        lib.opd_read_flags.argtypes = [vp, sz, i32, ctypes.POINTER(ctypes.c_uint32), vp]
        lib.opd_length_head_loss.restype = i32
        lib.opd_length_head_loss.argtypes = [vp, vp, i64, vp, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.opd_capacity_init.restype = i32
        lib.opd_capacity_init.argtypes = [ctypes.POINTER(OpdCapacity), ctypes.c_double]
        lib.opd_capacity_observe.restype = i32
        lib.opd_capacity_observe.argtypes = [ctypes.POINTER(OpdCapacity), ctypes.c_double,
                                             ctypes.POINTER(ctypes.c_int64)]
        lib.opd_pack_first_fit.restype = i32
        lib.opd_pack_first_fit.argtypes = [vp, i32, i64, i32, vp, vp, vp, ctypes.POINTER(ctypes.c_int32),
                                           ctypes.POINTER(ctypes.c_int64)]
        lib.opd_verify_sample.restype = i32
        lib.opd_verify_sample.argtypes = [vp, vp, i32, i64, i64, i64, ctypes.POINTER(OpdBlocks), vp, vp, vp,
                                          ctypes.c_float, vp, vp, vp, vp, sz, vp]
        lib.opd_lmhead_scratch_size.restype = sz
        lib.opd_lmhead_scratch_size.argtypes = [i64, i64, i64]
        lib.opd_lmhead_fused_fwd_bwd_verify.restype = i32
        lib.opd_lmhead_fused_fwd_bwd_verify.argtypes = [vp, vp, i64, vp, i32, i64, i64, i64, ctypes.POINTER(OpdBlocks),
                                                        ctypes.c_float, ctypes.c_float, vp, vp, vp, vp, vp, vp, vp, vp,
                                                        vp, sz, i64, vp, sz, vp]
        lib.opd_stream_probe.restype = i32
        lib.opd_stream_probe.argtypes = [vp, vp, vp, sz, vp]
        lib.opd_set_spin_limit.restype = None
        lib.opd_set_spin_limit.argtypes = [ctypes.c_uint32]
        lib.opd_status_string.restype = ctypes.c_char_p
        lib.opd_status_string.argtypes = [i32]
        lib.opd_last_error.restype = ctypes.c_char_p
        lib.opd_last_error.argtypes = []
        _lib = lib
        return lib


class OpdError(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str):
        super().__init__(f"{fn} failed with status {status}: {detail}")
        self.status = status


def _check(fn: str, status: int):
    if status != 0:
        lib = load_library()
        s = lib.opd_status_string(status).decode()
        d = lib.opd_last_error().decode()
        raise OpdError(fn, status, f"{s} ({d})")


# ------------------------------------------------------------------ torch-facing helpers


def _torch():
    import torch

    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return OPD_F32
    if t.dtype == torch.bfloat16:
        return OPD_BF16
    raise TypeError(f"unsupported dtype {t.dtype}; expected float32 or bfloat16")


def _matrix(t, name: str):
    """(pointer, rows, cols, ld) of a row-major 2-D device tensor whose rows may be padded."""
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D [rows, vocab]")
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} must have unit stride along the vocabulary")
    ld = t.stride(0) if t.shape[0] > 1 else max(t.stride(0), t.shape[1])
    return t.data_ptr(), t.shape[0], t.shape[1], ld


def _stream(device):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _empty_rows(rows: int, vocab: int, dtype, device):
    """[rows, vocab] tensor whose row pitch is rounded up to 16 bytes (the library's alignment rule)."""
    torch = _torch()
    per = 16 // torch.empty((), dtype=dtype).element_size()
    ld = ((vocab + per - 1) // per) * per
    return torch.empty(rows, ld, dtype=dtype, device=device)[:, :vocab]


_ws_cache = {}


def workspace(device=None):
    """Zero-filled workspace for ``device`` (allocated once per device and reused)."""
    torch = _torch()
    dev = torch.device("cuda") if device is None else torch.device(device)
    if dev.index is None:
        dev = torch.device(dev.type, torch.cuda.current_device())
    key = (dev.type, dev.index)
    ws = _ws_cache.get(key)
    if ws is None:
        n = load_library().opd_workspace_size()
        ws = torch.zeros(n, dtype=torch.uint8, device=dev)
        _ws_cache[key] = ws
    return ws


def set_spin_limit(spins: int):
    load_library().opd_set_spin_limit(int(spins))


def read_flags(ws=None, clear: bool = False, device=None) -> int:
    lib = load_library()
    ws = workspace(device) if ws is None else ws
    out = ctypes.c_uint32(0)
    _check("opd_read_flags", lib.opd_read_flags(ws.data_ptr(), ws.numel(), int(clear), ctypes.byref(out), _stream(ws.device)))
    return int(out.value)


def length_head_loss(target_top1, draft_top1, offsets, head_logit, grad=None, ws=None) -> dict:
    """Length-head epilogue per packed block: accept_full i32, label f32, loss f32, dlogit f32."""
    torch = _torch()
    lib = load_library()
    dev = head_logit.device
    n_blocks = int(offsets.numel()) - 1
    if int(head_logit.numel()) != n_blocks or (grad is not None and int(grad.numel()) != n_blocks):
        raise ValueError("head_logit (and grad) must have one entry per block")
    ws = workspace(dev) if ws is None else ws
    out = {
        "accept_full": torch.empty(n_blocks, dtype=torch.int32, device=dev),
        "label": torch.empty(n_blocks, dtype=torch.float32, device=dev),
        "loss": torch.empty(n_blocks, dtype=torch.float32, device=dev),
        "dlogit": torch.empty(n_blocks, dtype=torch.float32, device=dev),
    }
    _check("opd_length_head_loss", lib.opd_length_head_loss(
        target_top1.data_ptr(), draft_top1.data_ptr(), int(target_top1.numel()), offsets.data_ptr(), n_blocks,
        head_logit.data_ptr(), None if grad is None else grad.data_ptr(), out["accept_full"].data_ptr(),
        out["label"].data_ptr(), out["loss"].data_ptr(), out["dlogit"].data_ptr(), ws.data_ptr(), ws.numel(),
        _stream(dev)))
    return out


class OpdCapacity(ctypes.Structure):
    _fields_ = [("ema", ctypes.c_double), ("beta", ctypes.c_double), ("n_obs", ctypes.c_int32)]


class CapacityEstimate:
    """EMA of the verification capacity (rows) observed per round; observe() returns the next budget."""

    def __init__(self, beta: float):
        self._lib = load_library(require_torch_runtime=False)
        self._c = OpdCapacity()
        _check("opd_capacity_init", self._lib.opd_capacity_init(ctypes.byref(self._c), float(beta)))

    @property
    def estimate(self) -> float:
        return float(self._c.ema)

    def observe(self, observed_rows: float) -> int:
        budget = ctypes.c_int64(0)
        _check("opd_capacity_observe", self._lib.opd_capacity_observe(ctypes.byref(self._c), float(observed_rows),
                                                                      ctypes.byref(budget)))
        return int(budget.value)


def pack_first_fit(lengths, budget_rows: int, max_requests: int = 0) -> dict:
    """First-fit packing in arrival order (host). lengths: sequence of ints >= 1.

    Returns selected (int32 indices), offsets (int32, len(selected) + 1), lengths (int32) and rows.
    """
    import numpy as np

    lib = load_library(require_torch_runtime=False)
    ln = np.ascontiguousarray(np.asarray(lengths, dtype=np.int32))
    n = int(ln.size)
    sel = np.empty(max(n, 1), dtype=np.int32)
    off = np.empty(n + 1, dtype=np.int32)
    pl = np.empty(max(n, 1), dtype=np.int32)
    n_sel = ctypes.c_int32(0)
    rows = ctypes.c_int64(0)
    _check("opd_pack_first_fit", lib.opd_pack_first_fit(
        ln.ctypes.data if n else None, n, int(budget_rows), int(max_requests), sel.ctypes.data, off.ctypes.data,
        pl.ctypes.data, ctypes.byref(n_sel), ctypes.byref(rows)))
    k = int(n_sel.value)
    return {"selected": sel[:k].copy(), "offsets": off[: k + 1].copy(), "lengths": pl[:k].copy(), "rows": int(rows.value)}


def stream_probe(a, b, c) -> None:
    """c = a XOR b over the bytes of equally sized, 16-byte aligned device tensors (bandwidth probe).

    c=None only reads a and b; a=b=None only writes c.
    """
    lib = load_library()
    given = [t for t in (a, b, c) if t is not None]
    if (a is None) != (b is None) or not given:
        raise ValueError("a and b must be both given or both None, and something must be streamed")
    nbytes = given[0].numel() * given[0].element_size()
    if any(t.numel() * t.element_size() != nbytes for t in given):
        raise ValueError("the tensors must hold the same number of bytes")
    if not all(t.is_contiguous() for t in given):
        raise ValueError("the tensors must be contiguous")
    ptr = [0 if t is None else t.data_ptr() for t in (a, b, c)]
    _check("opd_stream_probe", lib.opd_stream_probe(ptr[0], ptr[1], ptr[2], ctypes.c_size_t(nbytes),
                                                    _stream(given[0].device)))


def _blocks(offsets, lengths):
    if offsets is None:
        return None
    n_blocks = int(offsets.numel()) - 1
    if lengths is not None and int(lengths.numel()) != n_blocks:
        raise ValueError("L must have one entry per block (len(offsets) - 1)")
    return OpdBlocks(offsets.data_ptr(), None if lengths is None else lengths.data_ptr(), n_blocks)


def opd_loss_fwd(z, y, alpha: float, tau: float, ws=None, want_draft_top1: bool = True):
    """Returns (loss [R] f32, target_top1 [R] i32, draft_top1 [R] i32 or None, row_stats [R, 8] f32)."""
    torch = _torch()
    lib = load_library()
    zp, rows, vocab, ld = _matrix(z, "z")
    yp, rows_y, vocab_y, ld_y = _matrix(y, "y")
    if (rows, vocab, ld) != (rows_y, vocab_y, ld_y) or z.dtype != y.dtype:
        raise ValueError("z and y must have the same shape, row pitch and dtype")
    dev = z.device
    ws = workspace(dev) if ws is None else ws
    loss = torch.empty(rows, dtype=torch.float32, device=dev)
    a = torch.empty(rows, dtype=torch.int32, device=dev)
    d = torch.empty(rows, dtype=torch.int32, device=dev) if want_draft_top1 else None
    stats = torch.empty(rows, 8, dtype=torch.float32, device=dev)
    st = lib.opd_loss_fwd(zp, yp, _dtype_code(z), rows, vocab, ld, float(alpha), float(tau), loss.data_ptr(),
                          a.data_ptr(), _ptr(d), stats.data_ptr(), ws.data_ptr(), ws.numel(), _stream(dev))
    _check("opd_loss_fwd", st)
    return loss, a, d, stats


def opd_loss_bwd(z, y, alpha: float, tau: float, row_stats, target_top1, grad_loss=None, dz_dtype=None, dz=None,
                 ws=None):
    """Returns dz [R, V] (dz_dtype, default z.dtype) = grad_loss[row] * d loss_row / d z_row."""
    torch = _torch()
    lib = load_library()
    zp, rows, vocab, ld = _matrix(z, "z")
    yp, _, _, _ = _matrix(y, "y")
    dev = z.device
    ws = workspace(dev) if ws is None else ws
    if dz is None:
        dz = _empty_rows(rows, vocab, dz_dtype or z.dtype, dev)
    dzp, _, _, ld_dz = _matrix(dz, "dz")
    st = lib.opd_loss_bwd(zp, yp, _dtype_code(z), rows, vocab, ld, float(alpha), float(tau), row_stats.data_ptr(),
                          target_top1.data_ptr(), _ptr(grad_loss), dzp, _dtype_code(dz), ld_dz, ws.data_ptr(),
                          ws.numel(), _stream(dev))
    _check("opd_loss_bwd", st)
    return dz


def verify_accept_len(z, y, offsets, lengths, ws=None):
    """Returns (target_top1 [R], draft_top1 [R], accept_len [B]) as int32 tensors."""
    torch = _torch()
    lib = load_library()
    zp, rows, vocab, ld = _matrix(z, "z")
    yp, _, _, _ = _matrix(y, "y")
    dev = z.device
    ws = workspace(dev) if ws is None else ws
    blocks = _blocks(offsets, lengths)
    a = torch.empty(rows, dtype=torch.int32, device=dev)
    d = torch.empty(rows, dtype=torch.int32, device=dev)
    acc = torch.empty(max(blocks.n_blocks, 0), dtype=torch.int32, device=dev)
    st = lib.verify_accept_len(zp, yp, _dtype_code(z), rows, vocab, ld, ctypes.byref(blocks), a.data_ptr(),
                               d.data_ptr(), acc.data_ptr() if acc.numel() else None, ws.data_ptr(), ws.numel(),
                               _stream(dev))
    _check("verify_accept_len", st)
    return a, d, acc


def verify_sample(z, y, offsets, lengths, draft_tokens, u_accept, u_resample, temperature: float, ws=None,
                  out=None):
    """Speculative-sampling verification at a temperature (opd_verify_sample).

    Returns a dict: accept_len [B] i32, token [B] i32 (-1 when none), row_lse [R, 4] f32 (reference and
    log2 of the sum of 2^(x log2(e) / T) for z, then for y; written for the rows the verification
    reads, NaN elsewhere when allocated here). ``out`` may hold preallocated tensors under
    the same keys.
    """
    torch = _torch()
    lib = load_library()
    zp, rows, vocab, ld = _matrix(z, "z")
    yp, rows_y, vocab_y, ld_y = _matrix(y, "y")
    if (rows, vocab, ld) != (rows_y, vocab_y, ld_y) or z.dtype != y.dtype:
        raise ValueError("z and y must have the same shape, row pitch and dtype")
    dev = z.device
    ws = workspace(dev) if ws is None else ws
    blocks = _blocks(offsets, lengths)
    if blocks is None or lengths is None:
        raise ValueError("offsets and L are required")
    for name, t, n, dt in (("draft_tokens", draft_tokens, rows, torch.int32), ("u_accept", u_accept, rows, torch.float32),
                           ("u_resample", u_resample, blocks.n_blocks, torch.float32)):
        if t.dtype != dt or t.numel() != n or not t.is_contiguous() or t.device != dev:
            raise ValueError(f"{name} must be a contiguous {dt} tensor of {n} elements on {dev}")
    o = dict(out) if out is not None else {}
    if "accept_len" not in o:
        o["accept_len"] = torch.empty(blocks.n_blocks, dtype=torch.int32, device=dev)
        o["token"] = torch.empty(blocks.n_blocks, dtype=torch.int32, device=dev)
        o["row_lse"] = torch.full((rows, 4), float("nan"), dtype=torch.float32, device=dev)
    st = lib.opd_verify_sample(zp, yp, _dtype_code(z), rows, vocab, ld, ctypes.byref(blocks), draft_tokens.data_ptr(),
                               u_accept.data_ptr(), u_resample.data_ptr(), float(temperature),
                               _ptr(o["accept_len"]) if blocks.n_blocks else None,
                               _ptr(o["token"]) if blocks.n_blocks else None, o["row_lse"].data_ptr(),
                               ws.data_ptr(), ws.numel(), _stream(dev))
    _check("opd_verify_sample", st)
    return o


def lmhead_fused_fwd_bwd_verify(h, W, y, offsets, lengths, alpha: float, tau: float, grad_loss=None,
                                chunk_rows: int = 2048, want_dh: bool = True, want_dW: bool = True, scratch=None,
                                ws=None, out=None):
    """OPD loss fused with the vocabulary projection z = h W^T (opd_lmhead_fused_fwd_bwd_verify).

    h [R, H] bf16, W [V, H] bf16, y [R, V] fp32 (rows may be padded to a 16-byte pitch). Returns a dict
    with loss, target_top1, draft_top1, row_stats, accept_len (if blocks), dh [R, H] f32 and dW [V, H]
    f32. ``out`` may hold preallocated tensors under the same keys and ``scratch`` a uint8 device
    tensor of at least opd_lmhead_scratch_size bytes, so that repeated calls allocate nothing.
    """
    torch = _torch()
    lib = load_library()
    yp, rows, vocab, ld = _matrix(y, "y")
    for name, t in (("h", h), ("W", W)):
        if t.dtype != torch.bfloat16 or t.dim() != 2 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous 2-D bfloat16 tensor")
    hidden = W.shape[1]
    if W.shape[0] != vocab or h.shape != (rows, hidden):
        raise ValueError("shapes must be h [R, H], W [V, H], y [R, V]")
    dev = y.device
    ws = workspace(dev) if ws is None else ws
    blocks = _blocks(offsets, lengths)
    n_blocks = blocks.n_blocks if blocks is not None else 0
    rc = max(1, min(int(chunk_rows), max(rows, 1)))
    need = lib.opd_lmhead_scratch_size(rc, vocab, ld)
    if scratch is None or scratch.numel() < need:
        scratch = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    o = dict(out) if out is not None else {}
    if "loss" not in o:
        o["loss"] = torch.empty(rows, dtype=torch.float32, device=dev)
        o["target_top1"] = torch.empty(rows, dtype=torch.int32, device=dev)
        o["draft_top1"] = torch.empty(rows, dtype=torch.int32, device=dev)
        o["row_stats"] = torch.empty(rows, 8, dtype=torch.float32, device=dev)
        o["accept_len"] = torch.empty(n_blocks, dtype=torch.int32, device=dev)
        o["dh"] = torch.empty(rows, hidden, dtype=torch.float32, device=dev) if want_dh else None
        o["dW"] = torch.empty(vocab, hidden, dtype=torch.float32, device=dev) if want_dW else None
    st = lib.opd_lmhead_fused_fwd_bwd_verify(
        h.data_ptr(), W.data_ptr(), hidden, yp, _dtype_code(y), rows, vocab, ld,
        ctypes.byref(blocks) if blocks is not None else None, float(alpha), float(tau), _ptr(grad_loss),
        o["loss"].data_ptr(), o["target_top1"].data_ptr(), o["draft_top1"].data_ptr(), o["row_stats"].data_ptr(),
        _ptr(o["dh"]), _ptr(o["dW"]), _ptr(o["accept_len"]) if n_blocks else None, scratch.data_ptr(),
        scratch.numel(), rc, ws.data_ptr(), ws.numel(), _stream(dev))
    _check("opd_lmhead_fused_fwd_bwd_verify", st)
    o["scratch"] = scratch
    return o


def opd_fused_fwd_bwd_verify(z, y, offsets, lengths, alpha: float, tau: float, grad_loss=None, dz_dtype=None,
                             out=None, ws=None):
    """One pass: loss, row_stats, both top-1s, dz and accept lengths. Returns a dict of tensors.

    ``out`` may hold preallocated tensors under the same keys (loss, target_top1, draft_top1,
    row_stats, dz, accept_len) so that repeated calls allocate nothing.
    """
    torch = _torch()
    lib = load_library()
    zp, rows, vocab, ld = _matrix(z, "z")
    yp, _, _, _ = _matrix(y, "y")
    dev = z.device
    ws = workspace(dev) if ws is None else ws
    blocks = _blocks(offsets, lengths)
    n_blocks = blocks.n_blocks if blocks is not None else 0
    o = dict(out) if out is not None else {}
    if "loss" not in o:
        o["loss"] = torch.empty(rows, dtype=torch.float32, device=dev)
        o["target_top1"] = torch.empty(rows, dtype=torch.int32, device=dev)
        o["draft_top1"] = torch.empty(rows, dtype=torch.int32, device=dev)
        o["row_stats"] = torch.empty(rows, 8, dtype=torch.float32, device=dev)
        o["dz"] = _empty_rows(rows, vocab, dz_dtype or z.dtype, dev)
        o["accept_len"] = torch.empty(n_blocks, dtype=torch.int32, device=dev)
    dzp, _, _, ld_dz = _matrix(o["dz"], "dz")
    st = lib.opd_fused_fwd_bwd_verify(
        zp, yp, _dtype_code(z), rows, vocab, ld, ctypes.byref(blocks) if blocks is not None else None,
        float(alpha), float(tau), _ptr(grad_loss), o["loss"].data_ptr(), o["target_top1"].data_ptr(),
        o["draft_top1"].data_ptr(), o["row_stats"].data_ptr(), dzp, _dtype_code(o["dz"]), ld_dz,
        o["accept_len"].data_ptr() if o["accept_len"].numel() else None, ws.data_ptr(), ws.numel(), _stream(dev))
    _check("opd_fused_fwd_bwd_verify", st)
    return o
