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
    "opd_fused_fwd_bwd_verify_noalloc",
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
    "opd_set_check",
    "opd_get_check",
    "opd_debug_reserve_flags",
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
        lib.opd_fused_fwd_bwd_verify_noalloc.restype = i32
        lib.opd_fused_fwd_bwd_verify_noalloc.argtypes = [vp, vp, i32, i64, i64, i64, ctypes.POINTER(OpdBlocks), f32,
                                                         f32, vp, vp, vp, vp, vp, vp, i32, i64, vp, vp]
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
                                                        vp, vp, vp, sz, i64, vp, sz, vp]
        lib.opd_stream_probe.restype = i32
        lib.opd_stream_probe.argtypes = [vp, vp, vp, sz, vp]
        lib.opd_set_spin_limit.restype = None
        lib.opd_set_spin_limit.argtypes = [ctypes.c_uint32]
        lib.opd_set_check.restype = None
        lib.opd_set_check.argtypes = [i32]
        lib.opd_get_check.restype = i32
        lib.opd_get_check.argtypes = []
        lib.opd_debug_reserve_flags.restype = i32
        lib.opd_debug_reserve_flags.argtypes = [vp, ctypes.c_uint32, i64, ctypes.POINTER(ctypes.c_uint32),
                                                ctypes.POINTER(ctypes.c_int)]
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
    raise ValueError(f"unsupported dtype {t.dtype}; expected float32 or bfloat16")


def _matrix(t, name: str, whole_vectors: bool = True):
    """(pointer, rows, cols, ld) of a row-major 2-D tensor whose rows may be padded.

    The kernels read inputs in whole 16-byte vectors, so the storage of an input must reach the end
    of the last row's last vector (true of row slices of a padded buffer); outputs are written up to
    the last element only (whole_vectors=False)."""
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D [rows, vocab]")
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} must have unit stride along the vocabulary")
    ld = t.stride(0) if t.shape[0] > 1 else max(t.stride(0), t.shape[1])
    if ld < t.shape[1]:
        raise ValueError(f"{name}: row pitch {ld} is shorter than a row ({t.shape[1]})")
    if t.shape[0] > 0 and t.shape[1] > 0 and t.device.type != "meta":
        per = max(1, 16 // t.element_size()) if whole_vectors else 1
        last = ((t.shape[1] + per - 1) // per) * per
        span = (t.storage_offset() + (t.shape[0] - 1) * ld + last) * t.element_size()
        if span > t.untyped_storage().nbytes():
            raise ValueError(f"{name}: the storage ends before the last row's last 16-byte vector")
    return t.data_ptr(), t.shape[0], t.shape[1], ld


# ------------------------------------------------------------------ argument validation
#
# Every call is checked here before any pointer reaches the library: the library trusts the sizes it
# is given, so a tensor that is too short, of the wrong dtype or on another device would make the
# kernels read or write outside an allocation. Structure and dtypes are checked first, devices last.


def _require(cond: bool, msg: str):
    if not cond:
        raise ValueError(msg)


def _vector(t, name: str, n: int, dtype, optional: bool = False):
    """A 1-D (or any-shape contiguous) tensor of exactly n elements of `dtype`."""
    if t is None:
        _require(optional, f"{name} is required")
        return
    _require(t.dtype == dtype, f"{name} must be {dtype}, got {t.dtype}")
    _require(t.is_contiguous(), f"{name} must be contiguous")
    _require(int(t.numel()) == int(n), f"{name} must have {n} elements, got {int(t.numel())}")


def _rows_matrix(t, name: str, rows: int, cols: int, dtype):
    """A contiguous [rows, cols] tensor of `dtype`."""
    _require(t.dtype == dtype, f"{name} must be {dtype}, got {t.dtype}")
    _require(t.is_contiguous() and tuple(t.shape) == (rows, cols), f"{name} must be a contiguous [{rows}, {cols}] tensor")


def _same_device(dev, named):
    _require(dev.type == "cuda", f"tensors must be on a CUDA (HIP) device, got {dev}")
    for name, t in named:
        if t is not None:
            _require(t.device == dev, f"{name} is on {t.device}, expected {dev}")


def _logit_pair(z, y):
    """Checks z and y against each other; returns (z pointer, y pointer, rows, vocab, ld, dtype code)."""
    zp, rows, vocab, ld = _matrix(z, "z")
    yp, rows_y, vocab_y, ld_y = _matrix(y, "y")
    _require((rows, vocab) == (rows_y, vocab_y), f"z {tuple(z.shape)} and y {tuple(y.shape)} must have the same shape")
    _require(ld == ld_y, f"z and y must have the same row pitch ({ld} vs {ld_y})")
    _require(z.dtype == y.dtype, f"z and y must have the same dtype ({z.dtype} vs {y.dtype})")
    return zp, yp, rows, vocab, ld, _dtype_code(z)


def _blocks_checked(offsets, lengths, required: bool):
    torch = _torch()
    if offsets is None:
        _require(not required and lengths is None, "offsets and L are required" if required else
                 "L given without offsets")
        return None, 0
    _require(offsets.dim() == 1 and offsets.numel() >= 1, "offsets must be a 1-D tensor of n_blocks + 1 entries")
    n_blocks = int(offsets.numel()) - 1
    _vector(offsets, "offsets", n_blocks + 1, torch.int32)
    _vector(lengths, "L", n_blocks, torch.int32, optional=not required)
    return OpdBlocks(offsets.data_ptr(), None if lengths is None else lengths.data_ptr(), n_blocks), n_blocks


def _byte_range(t):
    """[first, last) bytes a 2-D row-major view spans."""
    start = t.data_ptr()
    return start, start + ((t.shape[0] - 1) * t.stride(0) + t.shape[1]) * t.element_size()


def _no_overlap(a, b, an: str, bn: str):
    """The output a must not overlap the input b (the kernels read b while writing a)."""
    if a is None or b is None or a.numel() == 0 or b.numel() == 0 or a.device != b.device:
        return
    a0, a1 = _byte_range(a)
    b0, b1 = _byte_range(b)
    if a0 < b1 and b0 < a1:
        raise ValueError(f"{an} must not overlap {bn}")


def _row_outputs(o: dict, rows: int, n_blocks: int, keys):
    torch = _torch()
    spec = {"loss": (torch.float32, None), "target_top1": (torch.int32, None), "draft_top1": (torch.int32, None),
            "row_stats": (torch.float32, 8), "accept_len": (torch.int32, "blocks")}
    for k in keys:
        t = o.get(k)
        dtype, extra = spec[k]
        if k == "draft_top1" and t is None:
            continue
        _require(t is not None, f"out[{k!r}] is missing")
        if extra == 8:
            _rows_matrix(t, k, rows, 8, dtype)
        elif extra == "blocks":
            if n_blocks > 0:  # ignored by the library when no blocks are given
                _vector(t, k, n_blocks, dtype)
        else:
            _vector(t, k, rows, dtype)


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


def workspace(device=None, stream=None):
    """Zero-filled default workspace for ``device`` and ``stream`` (default: the device's current
    stream), allocated on first use and reused.

    Calls that share a workspace must not run concurrently, so each stream gets its own: calls on
    one stream run in order, calls on different streams may overlap. (A workspace found here for a
    stream handle that was destroyed and reused is simply reused.)"""
    torch = _torch()
    dev = torch.device("cuda") if device is None else torch.device(device)
    if dev.index is None:
        dev = torch.device(dev.type, torch.cuda.current_device())
    st = torch.cuda.current_stream(dev) if stream is None else stream
    key = (dev.type, dev.index, int(st.cuda_stream))
    with _lock:
        ws = _ws_cache.get(key)
    if ws is None:
        n = load_library().opd_workspace_size()
        with torch.cuda.stream(st):
            ws = torch.zeros(n, dtype=torch.uint8, device=dev)
        # the zero fill runs on `st`; the workspace is only ever used on that stream
        with _lock:
            ws = _ws_cache.setdefault(key, ws)
    return ws


def set_check(on: bool) -> None:
    """Check mode of the library (also OPD_CHECK=1 in the environment): every call synchronises its
    stream and raises OpdError (status OPD_ERR_DEVICE = 8) if it set a device flag."""
    load_library().opd_set_check(1 if on else 0)


def check_mode() -> bool:
    return bool(load_library().opd_get_check())


def debug_reserve_flags(ws_address: int, count: int, next_offset: int = -1):
    """Host bookkeeping of the exchange flags (no launch): returns (base, must_clear)."""
    lib = load_library(require_torch_runtime=False)
    base = ctypes.c_uint32(0)
    clear = ctypes.c_int(0)
    _check("opd_debug_reserve_flags", lib.opd_debug_reserve_flags(ws_address, int(count), int(next_offset),
                                                                  ctypes.byref(base), ctypes.byref(clear)))
    return int(base.value), bool(clear.value)


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
    _require(target_top1.dim() == 1, "target_top1 must be 1-D")
    n_rows = int(target_top1.numel())
    _vector(target_top1, "target_top1", n_rows, torch.int32)
    _vector(draft_top1, "draft_top1", n_rows, torch.int32)
    _require(offsets.dim() == 1 and offsets.numel() >= 1, "offsets must be a 1-D tensor of n_blocks + 1 entries")
    n_blocks = int(offsets.numel()) - 1
    _vector(offsets, "offsets", n_blocks + 1, torch.int32)
    _vector(head_logit, "head_logit", n_blocks, torch.float32)
    _vector(grad, "grad", n_blocks, torch.float32, optional=True)
    dev = head_logit.device
    _same_device(dev, [("target_top1", target_top1), ("draft_top1", draft_top1), ("offsets", offsets),
                       ("grad", grad)])
    lib = load_library()
    ws = workspace(dev) if ws is None else ws
    out = {
        "accept_full": torch.empty(n_blocks, dtype=torch.int32, device=dev),
        "label": torch.empty(n_blocks, dtype=torch.float32, device=dev),
        "loss": torch.empty(n_blocks, dtype=torch.float32, device=dev),
        "dlogit": torch.empty(n_blocks, dtype=torch.float32, device=dev),
    }
    _check("opd_length_head_loss", lib.opd_length_head_loss(
        target_top1.data_ptr(), draft_top1.data_ptr(), n_rows, offsets.data_ptr(), n_blocks,
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


def _workspace_arg(ws, dev):
    if ws is None:
        return workspace(dev)
    torch = _torch()
    _require(ws.dtype == torch.uint8 and ws.is_contiguous(), "ws must be a contiguous uint8 tensor")
    _require(ws.device == dev, f"ws is on {ws.device}, expected {dev}")
    return ws


def opd_loss_fwd(z, y, alpha: float, tau: float, ws=None, want_draft_top1: bool = True):
    """Returns (loss [R] f32, target_top1 [R] i32, draft_top1 [R] i32 or None, row_stats [R, 8] f32)."""
    torch = _torch()
    zp, yp, rows, vocab, ld, dt = _logit_pair(z, y)
    dev = z.device
    _same_device(dev, [("y", y)])
    lib = load_library()
    ws = _workspace_arg(ws, dev)
    loss = torch.empty(rows, dtype=torch.float32, device=dev)
    a = torch.empty(rows, dtype=torch.int32, device=dev)
    d = torch.empty(rows, dtype=torch.int32, device=dev) if want_draft_top1 else None
    stats = torch.empty(rows, 8, dtype=torch.float32, device=dev)
    st = lib.opd_loss_fwd(zp, yp, dt, rows, vocab, ld, float(alpha), float(tau), loss.data_ptr(),
                          a.data_ptr(), _ptr(d), stats.data_ptr(), ws.data_ptr(), ws.numel(), _stream(dev))
    _check("opd_loss_fwd", st)
    return loss, a, d, stats


def opd_loss_bwd(z, y, alpha: float, tau: float, row_stats, target_top1, grad_loss=None, dz_dtype=None, dz=None,
                 ws=None):
    """Returns dz [R, V] (dz_dtype, default z.dtype) = grad_loss[row] * d loss_row / d z_row."""
    torch = _torch()
    zp, yp, rows, vocab, ld, dt = _logit_pair(z, y)
    _rows_matrix(row_stats, "row_stats", rows, 8, torch.float32)
    _vector(target_top1, "target_top1", rows, torch.int32)
    _vector(grad_loss, "grad_loss", rows, torch.float32, optional=True)
    if dz is not None:
        _dtype_code(dz)
        _, rows_d, vocab_d, _ = _matrix(dz, "dz", whole_vectors=False)
        _require((rows_d, vocab_d) == (rows, vocab), f"dz must be [{rows}, {vocab}], got {tuple(dz.shape)}")
        _no_overlap(dz, z, "dz", "z")
        _no_overlap(dz, y, "dz", "y")
    dev = z.device
    _same_device(dev, [("y", y), ("row_stats", row_stats), ("target_top1", target_top1), ("grad_loss", grad_loss),
                       ("dz", dz)])
    lib = load_library()
    ws = _workspace_arg(ws, dev)
    if dz is None:
        dz = _empty_rows(rows, vocab, dz_dtype or z.dtype, dev)
    dzp, _, _, ld_dz = _matrix(dz, "dz", whole_vectors=False)
    st = lib.opd_loss_bwd(zp, yp, dt, rows, vocab, ld, float(alpha), float(tau), row_stats.data_ptr(),
                          target_top1.data_ptr(), _ptr(grad_loss), dzp, _dtype_code(dz), ld_dz, ws.data_ptr(),
                          ws.numel(), _stream(dev))
    _check("opd_loss_bwd", st)
    return dz


def verify_accept_len(z, y, offsets, lengths, ws=None):
    """Returns (target_top1 [R], draft_top1 [R], accept_len [B]) as int32 tensors."""
    torch = _torch()
    zp, yp, rows, vocab, ld, dt = _logit_pair(z, y)
    blocks, n_blocks = _blocks_checked(offsets, lengths, required=True)
    dev = z.device
    _same_device(dev, [("y", y), ("offsets", offsets), ("L", lengths)])
    lib = load_library()
    ws = _workspace_arg(ws, dev)
    a = torch.empty(rows, dtype=torch.int32, device=dev)
    d = torch.empty(rows, dtype=torch.int32, device=dev)
    acc = torch.empty(n_blocks, dtype=torch.int32, device=dev)
    st = lib.verify_accept_len(zp, yp, dt, rows, vocab, ld, ctypes.byref(blocks), a.data_ptr(),
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
    zp, yp, rows, vocab, ld, dt = _logit_pair(z, y)
    blocks, n_blocks = _blocks_checked(offsets, lengths, required=True)
    _vector(draft_tokens, "draft_tokens", rows, torch.int32)
    _vector(u_accept, "u_accept", rows, torch.float32)
    _vector(u_resample, "u_resample", n_blocks, torch.float32)
    o = dict(out) if out is not None else {}
    if "accept_len" in o:
        _vector(o.get("accept_len"), "accept_len", n_blocks, torch.int32)
        _vector(o.get("token"), "token", n_blocks, torch.int32)
        _rows_matrix(o.get("row_lse"), "row_lse", rows, 4, torch.float32)
    dev = z.device
    _same_device(dev, [("y", y), ("offsets", offsets), ("L", lengths), ("draft_tokens", draft_tokens),
                       ("u_accept", u_accept), ("u_resample", u_resample)] + [(k, o.get(k)) for k in
                                                                            ("accept_len", "token", "row_lse")])
    lib = load_library()
    ws = _workspace_arg(ws, dev)
    if "accept_len" not in o:
        o["accept_len"] = torch.empty(n_blocks, dtype=torch.int32, device=dev)
        o["token"] = torch.empty(n_blocks, dtype=torch.int32, device=dev)
        o["row_lse"] = torch.full((rows, 4), float("nan"), dtype=torch.float32, device=dev)
    st = lib.opd_verify_sample(zp, yp, dt, rows, vocab, ld, ctypes.byref(blocks), draft_tokens.data_ptr(),
                               u_accept.data_ptr(), u_resample.data_ptr(), float(temperature),
                               _ptr(o["accept_len"]) if n_blocks else None,
                               _ptr(o["token"]) if n_blocks else None, o["row_lse"].data_ptr(),
                               ws.data_ptr(), ws.numel(), _stream(dev))
    _check("opd_verify_sample", st)
    return o


def lmhead_fused_fwd_bwd_verify(h, W, y, offsets, lengths, alpha: float, tau: float, grad_loss=None,
                                chunk_rows: int = 2048, want_dh: bool = True, want_dW: bool = True,
                                want_logit_stats: bool = True, scratch=None, ws=None, out=None):
    """OPD loss fused with the vocabulary projection z = h W^T (opd_lmhead_fused_fwd_bwd_verify).

    h [R, H] bf16, W [V, H] bf16, y [R, V] fp32 (rows may be padded to a 16-byte pitch). Returns a dict
    with loss, target_top1, draft_top1, row_stats, accept_len (if blocks), dh [R, H] f32, dW [V, H]
    f32, and from the logits product's epilogue logit_max_lse [R, 2] f32 (max z, log-sum-exp z) and
    logit_argmax [R] int32. ``out`` may hold preallocated tensors under the same keys and ``scratch``
    a uint8 device tensor of at least opd_lmhead_scratch_size bytes, so that repeated calls allocate
    nothing.
    """
    torch = _torch()
    yp, rows, vocab, ld = _matrix(y, "y")
    _require(y.dtype == torch.float32, "y must be float32")
    for name, t in (("h", h), ("W", W)):
        _require(t.dtype == torch.bfloat16 and t.dim() == 2 and t.is_contiguous(),
                 f"{name} must be a contiguous 2-D bfloat16 tensor")
    hidden = W.shape[1]
    _require(W.shape[0] == vocab and tuple(h.shape) == (rows, hidden), "shapes must be h [R, H], W [V, H], y [R, V]")
    blocks, n_blocks = _blocks_checked(offsets, lengths, required=False)
    _vector(grad_loss, "grad_loss", rows, torch.float32, optional=True)
    o = dict(out) if out is not None else {}
    if "loss" in o:
        _row_outputs(o, rows, n_blocks, ("loss", "target_top1", "draft_top1", "row_stats", "accept_len"))
        if o.get("dh") is not None:
            _rows_matrix(o["dh"], "dh", rows, hidden, torch.float32)
        if o.get("dW") is not None:
            _rows_matrix(o["dW"], "dW", vocab, hidden, torch.float32)
        if o.get("logit_max_lse") is not None:
            _rows_matrix(o["logit_max_lse"], "logit_max_lse", rows, 2, torch.float32)
        if o.get("logit_argmax") is not None:
            _vector(o["logit_argmax"], "logit_argmax", rows, torch.int32)
    dev = y.device
    _same_device(dev, [("h", h), ("W", W), ("offsets", offsets), ("L", lengths), ("grad_loss", grad_loss),
                       ("scratch", scratch)] + [(k, o.get(k)) for k in ("loss", "target_top1", "draft_top1",
                                                                       "row_stats", "accept_len", "dh", "dW",
                                                                       "logit_max_lse", "logit_argmax")])
    lib = load_library()
    ws = _workspace_arg(ws, dev)
    rc = max(1, min(int(chunk_rows), max(rows, 1)))
    need = lib.opd_lmhead_scratch_size(rc, vocab, ld)
    if scratch is None or scratch.numel() * scratch.element_size() < need:
        scratch = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    if "loss" not in o:
        o["loss"] = torch.empty(rows, dtype=torch.float32, device=dev)
        o["target_top1"] = torch.empty(rows, dtype=torch.int32, device=dev)
        o["draft_top1"] = torch.empty(rows, dtype=torch.int32, device=dev)
        o["row_stats"] = torch.empty(rows, 8, dtype=torch.float32, device=dev)
        o["accept_len"] = torch.empty(n_blocks, dtype=torch.int32, device=dev)
        o["dh"] = torch.empty(rows, hidden, dtype=torch.float32, device=dev) if want_dh else None
        o["dW"] = torch.empty(vocab, hidden, dtype=torch.float32, device=dev) if want_dW else None
        o["logit_max_lse"] = torch.empty(rows, 2, dtype=torch.float32, device=dev) if want_logit_stats else None
        o["logit_argmax"] = torch.empty(rows, dtype=torch.int32, device=dev) if want_logit_stats else None
    st = lib.opd_lmhead_fused_fwd_bwd_verify(
        h.data_ptr(), W.data_ptr(), hidden, yp, _dtype_code(y), rows, vocab, ld,
        ctypes.byref(blocks) if blocks is not None else None, float(alpha), float(tau), _ptr(grad_loss),
        o["loss"].data_ptr(), o["target_top1"].data_ptr(), _ptr(o["draft_top1"]), o["row_stats"].data_ptr(),
        _ptr(o["dh"]), _ptr(o["dW"]), _ptr(o.get("logit_max_lse")), _ptr(o.get("logit_argmax")),
        _ptr(o["accept_len"]) if n_blocks else None, scratch.data_ptr(),
        scratch.numel() * scratch.element_size(), rc, ws.data_ptr(), ws.numel(), _stream(dev))
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
    zp, yp, rows, vocab, ld, dt = _logit_pair(z, y)
    blocks, n_blocks = _blocks_checked(offsets, lengths, required=False)
    _vector(grad_loss, "grad_loss", rows, torch.float32, optional=True)
    o = dict(out) if out is not None else {}
    if "loss" in o:
        _row_outputs(o, rows, n_blocks, ("loss", "target_top1", "draft_top1", "row_stats", "accept_len"))
        _require(o.get("dz") is not None, "out['dz'] is missing")
        _dtype_code(o["dz"])
        _, rows_d, vocab_d, _ = _matrix(o["dz"], "dz", whole_vectors=False)
        _require((rows_d, vocab_d) == (rows, vocab), f"dz must be [{rows}, {vocab}], got {tuple(o['dz'].shape)}")
        _no_overlap(o["dz"], z, "dz", "z")
        _no_overlap(o["dz"], y, "dz", "y")
    dev = z.device
    _same_device(dev, [("y", y), ("offsets", offsets), ("L", lengths), ("grad_loss", grad_loss)]
                 + [(k, o.get(k)) for k in ("loss", "target_top1", "draft_top1", "row_stats", "dz", "accept_len")])
    lib = load_library()
    ws = _workspace_arg(ws, dev)
    if "loss" not in o:
        o["loss"] = torch.empty(rows, dtype=torch.float32, device=dev)
        o["target_top1"] = torch.empty(rows, dtype=torch.int32, device=dev)
        o["draft_top1"] = torch.empty(rows, dtype=torch.int32, device=dev)
        o["row_stats"] = torch.empty(rows, 8, dtype=torch.float32, device=dev)
        o["dz"] = _empty_rows(rows, vocab, dz_dtype or z.dtype, dev)
        o["accept_len"] = torch.empty(n_blocks, dtype=torch.int32, device=dev)
    _require(n_blocks == 0 or o.get("draft_top1") is not None, "draft_top1 is needed for verification")
    dzp, _, _, ld_dz = _matrix(o["dz"], "dz", whole_vectors=False)
    st = lib.opd_fused_fwd_bwd_verify(
        zp, yp, dt, rows, vocab, ld, ctypes.byref(blocks) if blocks is not None else None,
        float(alpha), float(tau), _ptr(grad_loss), o["loss"].data_ptr(), o["target_top1"].data_ptr(),
        _ptr(o["draft_top1"]), o["row_stats"].data_ptr(), dzp, _dtype_code(o["dz"]), ld_dz,
        o["accept_len"].data_ptr() if n_blocks else None, ws.data_ptr(), ws.numel(), _stream(dev))
    _check("opd_fused_fwd_bwd_verify", st)
    return o


def opd_fused_fwd_bwd_verify_noalloc(z, y, offsets, lengths, alpha: float, tau: float, out: dict, grad_loss=None):
    """opd_fused_fwd_bwd_verify without a workspace argument and without allocating: the library's
    own per-GPU workspace array is used, and every output comes preallocated in ``out`` (keys loss,
    target_top1, draft_top1, row_stats, dz, accept_len). Calls that overlap on one GPU must not be
    made (they share that array)."""
    torch = _torch()
    zp, yp, rows, vocab, ld, dt = _logit_pair(z, y)
    blocks, n_blocks = _blocks_checked(offsets, lengths, required=False)
    _vector(grad_loss, "grad_loss", rows, torch.float32, optional=True)
    _row_outputs(out, rows, n_blocks, ("loss", "target_top1", "draft_top1", "row_stats", "accept_len"))
    _require(out.get("dz") is not None, "out['dz'] is missing")
    _dtype_code(out["dz"])
    _, rows_d, vocab_d, _ = _matrix(out["dz"], "dz", whole_vectors=False)
    _require((rows_d, vocab_d) == (rows, vocab), f"dz must be [{rows}, {vocab}], got {tuple(out['dz'].shape)}")
    _no_overlap(out["dz"], z, "dz", "z")
    _no_overlap(out["dz"], y, "dz", "y")
    _require(n_blocks == 0 or out.get("draft_top1") is not None, "draft_top1 is needed for verification")
    dev = z.device
    _same_device(dev, [("y", y), ("offsets", offsets), ("L", lengths), ("grad_loss", grad_loss)]
                 + [(k, out.get(k)) for k in ("loss", "target_top1", "draft_top1", "row_stats", "dz", "accept_len")])
    lib = load_library()
    dzp, _, _, ld_dz = _matrix(out["dz"], "dz", whole_vectors=False)
    st = lib.opd_fused_fwd_bwd_verify_noalloc(
        zp, yp, dt, rows, vocab, ld, ctypes.byref(blocks) if blocks is not None else None,
        float(alpha), float(tau), _ptr(grad_loss), out["loss"].data_ptr(), out["target_top1"].data_ptr(),
        _ptr(out["draft_top1"]), out["row_stats"].data_ptr(), dzp, _dtype_code(out["dz"]), ld_dz,
        out["accept_len"].data_ptr() if n_blocks else None, _stream(dev))
    _check("opd_fused_fwd_bwd_verify_noalloc", st)
    return out
