"""MI355X-native on-policy-distillation (OPD) loss / gradient / greedy-verify path.

The computation lives in hand-written gfx950 HIP kernels behind the C ABI of include/opd.h
(libopd_mi355x.so, built by ``draft_model_distillation_amd.build``). This package only binds it:

    opd_loss_fwd, opd_loss_bwd, verify_accept_len, opd_fused_fwd_bwd_verify, verify_sample,
    lmhead_fused_fwd_bwd_verify

take torch device tensors and enqueue on torch's current stream.
"""

from ._binding import (  # noqa: F401
    EXPORTED_SYMBOLS,
    CapacityEstimate,
    OPD_BF16,
    OPD_F32,
    OPD_FLAG_BAD_OFFSETS,
    OPD_FLAG_BAD_TOKEN,
    OPD_FLAG_NEG_L,
    OPD_FLAG_SPIN_TIMEOUT,
    OpdError,
    check_mode,
    debug_reserve_flags,
    length_head_loss,
    lmhead_fused_fwd_bwd_verify,
    library_path,
    load_library,
    opd_fused_fwd_bwd_verify,
    opd_fused_fwd_bwd_verify_noalloc,
    opd_loss_bwd,
    opd_loss_fwd,
    pack_first_fit,
    read_flags,
    set_check,
    set_spin_limit,
    stream_probe,
    verify_accept_len,
    verify_sample,
    workspace,
)
