"""Float64 CPU oracle for the OPD loss fused with the drafter's vocabulary projection.

TEST INFRASTRUCTURE ONLY: the plain definition that the lm_head-fused path of the library is checked
against. Only the test suite, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg
may import it; it shares no code with the product library.

Sources, by page title and section: the loss is the one of ``oracle/opd_oracle.py`` ("AdaFlash:
Adaptive Speculative Decoding with Online Self-Improvement for High-Concurrency LLM Inference",
besthub.dev article, section "1. On-Policy Distillation (OPD) for Domain Adaptation": reverse KL
toward the target with per-vocabulary clipping and top-1 hard labels; "AdaFlash: Adaptive
Speculative Decoding via On-Policy Distilled Diffusion Drafters", project README page, section
"Released Checkpoint": the mixture). The article's section 1 says the drafter is what the online
update trains; its logits are the drafter's final hidden states times its vocabulary projection.

Readings (the pages show neither the drafter's head nor its sizes):

* z = h W^T with h [n_rows, H] the drafter's final hidden states and W [V, H] its vocabulary
  projection (no bias); the loss is the per-row loss of ``opd_oracle.row_forward`` on z;
* the gradient flows to both h and W: dh = dz W, dW = dz^T h, with dz = w_r * d loss_r / d z_r;
  y (the target's logits) takes no gradient.

* the per-row statistics of z that the logits product reports (max, lowest index of the max,
  log-sum-exp) are their plain definitions.

Each step is a library primitive (a matmul) or a function of ``oracle/opd_oracle.py``, whose pins
hold for it. Pinned by ``tests/test_lmhead_pins.py``: central finite differences of
sum_r w_r loss_r with respect to h and W, the special case W = I (then z = h and dh = dz), and for
``logit_stats`` constant rows (LSE = c + log V, argmax 0), a two-level row in closed form and an
exact rational-sum check on small rows. No function here is parity-unpinned.
"""

from __future__ import annotations

import numpy as np

from oracle import opd_oracle as O

__all__ = ["lmhead_rows", "lmhead_fused", "logit_stats"]


def lmhead_rows(h, W, rows) -> np.ndarray:
    """z for the selected rows only: h[rows] @ W^T in float64."""
    h = np.asarray(h, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    return h[np.asarray(rows)] @ W.T


def logit_stats(z):
    """Per row of z: (max, lowest index holding the max, log sum_v exp z_v), in float64."""
    z = np.asarray(z, dtype=np.float64)
    mx = z.max(axis=1)
    arg = np.argmax(z, axis=1)  # the first (lowest) index of the maximum
    lse = mx + np.log(np.exp(z - mx[:, None]).sum(axis=1))
    return mx, arg.astype(np.int64), lse


def lmhead_fused(h, W, y, alpha: float, tau: float, offsets=None, lengths=None, grad_loss=None) -> dict:
    """Loss, top-1s, accept lengths and the gradients w.r.t. h and W of the lm_head-fused path.

    h [R, H], W [V, H], y [R, V] (exact values of the device inputs). Returns z, loss, dz, dh, dW,
    S, target_top1, draft_top1, logit_max, logit_argmax, logit_lse and (with offsets and lengths)
    accept_len and flags.
    """
    h = np.asarray(h, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    z = h @ W.T
    fwd = O.forward_rows(z, y, alpha, tau)
    dz, S = O.grad_rows(z, y, alpha, tau, grad_loss)
    out = {
        "z": z,
        "loss": fwd["loss"],
        "dz": dz,
        "S": S,
        "dh": dz @ W,
        "dW": dz.T @ h,
        "target_top1": fwd["target_top1"],
        "draft_top1": fwd["draft_top1"],
    }
    out["logit_max"], out["logit_argmax"], out["logit_lse"] = logit_stats(z)
    if offsets is not None:
        out["accept_len"], out["flags"] = O.accept_lengths(fwd["draft_top1"], fwd["target_top1"], offsets, lengths)
    return out
