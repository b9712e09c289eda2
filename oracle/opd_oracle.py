"""Float64 CPU oracle for the on-policy-distillation (OPD) loss, its gradient and greedy verification.

TEST INFRASTRUCTURE ONLY. This module is the slow, plain definition that the HIP path is checked
against. Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
may import or run it; the product library and its Python binding never touch it, and it shares no
code, constants or helpers with them.

Sources, by page title and section:

* [OPD] "AdaFlash: Adaptive Speculative Decoding with Online Self-Improvement for High-Concurrency
  LLM Inference" (besthub.dev article), section "1. On-Policy Distillation (OPD) for Domain
  Adaptation": the drafter is trained with reverse KL toward the target plus top-1 hard labels taken
  from the target, and each vocabulary term of the reverse KL is clipped before the sum.
* [LEN] same article, section "2. Adaptive Length Head for Token-Level Variance": drafts are blocks
  of k=16 positions; a head turns k into an expected acceptance length used as the verification
  budget.
* [PACK] same article, section "Infrastructure: Async Training & Variable-Length Batching": requests
  with different verification lengths are packed contiguously into one batch.
* [CKPT] "AdaFlash: Adaptive Speculative Decoding via On-Policy Distilled Diffusion Drafters"
  (project README page), section "Released Checkpoint": the drafter uses an on-policy *mixture*
  reverse-KL loss.

The pages give the loss in words only. The formula used here (and its reading of every open point)
is: with p = softmax(z) (drafter) and q = softmax(y) (target), a = argmax y,

    loss = alpha * sum_v min(p_v (log p_v - log q_v), tau) + (1 - alpha) * (-log p_a)

with alpha and tau explicit parameters, temperature 1, ties of argmax going to the lowest index,
an upper clip only (negative terms pass unchanged), the clip gradient passing at t_v == tau, and no
gradient to y. Greedy verification accepts the longest prefix of a block, within
n = clamp(L, 0, block length), on which argmax z equals argmax y.

Each function below states the passage it follows. Every function here is pinned by the
``-m "not gpu"`` tests in ``tests/test_oracle_pins.py`` (library special cases, closed forms,
finite differences, brute force and invariants); none is parity-unpinned.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "logsumexp",
    "top1",
    "top1_rows",
    "row_forward",
    "row_grad",
    "accept_lengths",
    "forward_rows",
    "grad_rows",
    "ACCEPT_FLAG_NEG_L",
    "ACCEPT_FLAG_BAD_OFFSETS",
]

# Bits of the flag word returned by accept_lengths (same meaning as the library's device flags).
ACCEPT_FLAG_NEG_L = 1        # some block had L < 0 (clamped to 0)
ACCEPT_FLAG_BAD_OFFSETS = 2  # some block had decreasing or out-of-range offsets (accept set to 0)


def _as_f64(x) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    if x.ndim != 1:
        raise ValueError("expected a 1-D row")
    return x


def logsumexp(x) -> float:
    """log sum_v exp(x_v), the log-normaliser of softmax, in float64.

    Definition of softmax used by [OPD] for both p (drafter) and q (target); evaluated with the usual
    max shift so that exp never overflows.
    """
    x = _as_f64(x)
    m = float(np.max(x))
    return m + float(np.log(np.sum(np.exp(x - m))))


def top1(x) -> int:
    """Index of the largest entry; on ties the lowest index.

    The target's top-1 token is the hard label of [OPD]; the drafter's top-1 token is its greedy
    draft. numpy.argmax returns the first occurrence of the maximum, which is the lowest index.
    """
    return int(np.argmax(_as_f64(x)))


def top1_rows(x) -> np.ndarray:
    """``top1`` of every row of a [rows, V] array of exactly represented values (float32 or float64
    hold bf16 and fp32 inputs exactly, so the argmax is the same in either)."""
    x = np.asarray(x)
    if x.ndim != 2:
        raise ValueError("expected a 2-D array")
    return np.argmax(x, axis=1).astype(np.int64)


def row_forward(z, y, alpha: float, tau: float) -> dict:
    """Per-position OPD loss for one drafted position ([OPD] + [CKPT]).

    Steps, in the order the definition gives them:
      1. log p = z - LSE(z), log q = y - LSE(y)  (softmax of drafter / target logits, temperature 1)
      2. r_v = log p_v - log q_v and the reverse-KL term t_v = p_v * r_v  (KL(p || q), mode-seeking)
      3. each term is clipped from above before summation: rkl_clip = sum_v min(t_v, tau)
      4. top-1 hard label a = argmax y, cross entropy ce = -log p_a
      5. mixture: loss = alpha * rkl_clip + (1 - alpha) * ce

    Returns a dict with the scalars and the per-element arrays the gradient needs. ``clipped`` marks
    t_v > tau (the clip is active); at t_v == tau the term counts as unclipped.
    """
    z = _as_f64(z)
    y = _as_f64(y)
    if z.shape != y.shape or z.size == 0:
        raise ValueError("z and y must be non-empty rows of equal length")
    lse_z = logsumexp(z)
    lse_y = logsumexp(y)
    logp = z - lse_z
    logq = y - lse_y
    p = np.exp(logp)
    r = logp - logq
    # 0 * log 0 = 0: a term whose drafter probability underflows contributes nothing.
    t = np.where(p == 0.0, 0.0, p * r)
    clipped = t > tau
    rkl_clip = float(np.sum(np.where(clipped, tau, t)))
    a = top1(y)
    d = top1(z)
    ce = float(-logp[a])
    loss = alpha * rkl_clip + (1.0 - alpha) * ce
    return {
        "loss": loss,
        "rkl_clip": rkl_clip,
        "ce": ce,
        "lse_z": lse_z,
        "lse_y": lse_y,
        "target_top1": a,
        "draft_top1": d,
        "p": p,
        "r": r,
        "t": t,
        "clipped": clipped,
    }


def row_grad(z, y, alpha: float, tau: float, w: float = 1.0, clipped=None) -> tuple[np.ndarray, dict]:
    """Gradient of w * loss with respect to the drafter logits z, for one position.

    The drafter is what the on-policy update trains ([OPD]: the serving draft model is updated from
    the round's target distributions); the target is fixed and its top-1 label is a hard argmax, so
    no gradient flows to y.

    Derivation from the definition in ``row_forward``: d t_v / d z_j = p_v (delta_vj - p_j)(r_v + 1),
    and a clipped term has zero derivative, so with g_v = [t_v <= tau] (r_v + 1) and S = sum_v p_v g_v
    the reverse-KL part gives p_j (g_j - S); the cross entropy gives p_j - [j == a]. Hence

        dz_j = w * (alpha * p_j * (g_j - S) + (1 - alpha) * (p_j - [j == a])).

    ``clipped`` may override the clip mask (used by the parity checker for terms whose t_v lies
    within rounding distance of tau, where either side of the clip is a correct result).
    Returns (dz, info) where info holds the forward dict plus ``S``.
    """
    f = row_forward(z, y, alpha, tau)
    mask = f["clipped"] if clipped is None else np.asarray(clipped, dtype=bool)
    p, r = f["p"], f["r"]
    g = np.where(mask, 0.0, r + 1.0)
    s = float(np.sum(p * g))
    onehot = np.zeros_like(p)
    onehot[f["target_top1"]] = 1.0
    dz = w * (alpha * p * (g - s) + (1.0 - alpha) * (p - onehot))
    info = dict(f)
    info["S"] = s
    info["clip_mask_used"] = mask
    return dz, info


def accept_lengths(draft_top1, target_top1, offsets, lengths) -> tuple[np.ndarray, int]:
    """Greedy accepted-prefix length of each packed verification block ([LEN], [PACK]).

    Block b holds the rows offsets[b] .. offsets[b+1]-1 of the packed batch (requests of different
    lengths packed contiguously). Its verification budget is n = clamp(L_b, 0, n_b) with
    n_b = offsets[b+1] - offsets[b] (the length head's predicted length caps the k-position block).
    The accepted length is the number of leading positions j < n at which the draft top-1 equals the
    target top-1; the target's correction token is not counted.

    Malformed input is defined rather than undefined: L_b < 0 is clamped to 0 and raises
    ACCEPT_FLAG_NEG_L; a block whose offsets decrease or leave [0, n_rows] gets 0 and raises
    ACCEPT_FLAG_BAD_OFFSETS. Returns (accept int32[n_blocks], flags).
    """
    d = np.asarray(draft_top1, dtype=np.int64)
    a = np.asarray(target_top1, dtype=np.int64)
    off = np.asarray(offsets, dtype=np.int64)
    lens = np.asarray(lengths, dtype=np.int64)
    n_rows = d.size
    n_blocks = lens.size
    if off.size != n_blocks + 1:
        raise ValueError("offsets must have n_blocks + 1 entries")
    out = np.zeros(n_blocks, dtype=np.int32)
    flags = 0
    for b in range(n_blocks):
        start, end = int(off[b]), int(off[b + 1])
        if start < 0 or end < start or end > n_rows:
            flags |= ACCEPT_FLAG_BAD_OFFSETS
            continue
        lb = int(lens[b])
        if lb < 0:
            flags |= ACCEPT_FLAG_NEG_L
        n = min(max(lb, 0), end - start)
        k = 0
        while k < n and d[start + k] == a[start + k]:
            k += 1
        out[b] = k
    return out, flags


def forward_rows(z_rows, y_rows, alpha: float, tau: float) -> dict:
    """``row_forward`` applied to every row of [n_rows, V] arrays; returns per-row arrays."""
    z_rows = np.asarray(z_rows)
    y_rows = np.asarray(y_rows)
    n = z_rows.shape[0]
    keys = ("loss", "rkl_clip", "ce", "lse_z", "lse_y")
    out = {k: np.zeros(n, dtype=np.float64) for k in keys}
    out["target_top1"] = np.zeros(n, dtype=np.int64)
    out["draft_top1"] = np.zeros(n, dtype=np.int64)
    for i in range(n):
        f = row_forward(z_rows[i], y_rows[i], alpha, tau)
        for k in keys:
            out[k][i] = f[k]
        out["target_top1"][i] = f["target_top1"]
        out["draft_top1"][i] = f["draft_top1"]
    return out


def grad_rows(z_rows, y_rows, alpha: float, tau: float, w=None) -> tuple[np.ndarray, np.ndarray]:
    """``row_grad`` applied to every row; returns (dz [n_rows, V] float64, S [n_rows])."""
    z_rows = np.asarray(z_rows)
    y_rows = np.asarray(y_rows)
    n = z_rows.shape[0]
    dz = np.zeros(z_rows.shape, dtype=np.float64)
    s = np.zeros(n, dtype=np.float64)
    for i in range(n):
        wi = 1.0 if w is None else float(w[i])
        dz[i], info = row_grad(z_rows[i], y_rows[i], alpha, tau, wi)
        s[i] = info["S"]
    return dz, s
