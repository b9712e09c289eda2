"""Float64 CPU oracle for stochastic verification at a sampling temperature (speculative sampling).

TEST INFRASTRUCTURE ONLY: the plain definition that the HIP sampling-verify kernels are checked
against. Only the test suite, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg
may import it; it shares no code with the product library.

Sources, by page title and section:

* "Adaflash Adaptive Speculative Decoding" (skills-directory card), section "Implementation
  Steps": temperature is one of the parameters to tune
  when the drafter is combined with the target for speculative decoding.
* "AdaFlash: Adaptive Speculative Decoding with Online Self-Improvement for High-Concurrency LLM
  Inference" (besthub.dev article), section "2. Adaptive Length Head for Token-Level Variance": the
  target verifies a block of drafted positions up to a predicted length; section "Infrastructure:
  Async Training & Variable-Length Batching": blocks are packed contiguously (offsets).

The pages give no acceptance rule for sampling at a temperature. The reading used here is the
published speculative-sampling rule (Leviathan, Kalman and Matias, "Fast Inference from
Transformers via Speculative Decoding", 2023; Chen et al., "Accelerating Large Language Model
Decoding with Speculative Sampling", 2023), restated:

* p_r = softmax(z_r / T) is the drafter's distribution at packed row r, q_r = softmax(y_r / T) the
  target's; x_r is the token the drafter proposed there (sampled by the caller);
* block b holds rows s = offsets[b] .. offsets[b+1]-1 (n_b rows); the target verifies the first
  n = clamp(L_b, 0, n_b) of them in order. Row r's proposal is accepted when u_r p_r(x_r) <= q_r(x_r)
  for the caller's uniform draw u_r in [0, 1) (that is, with probability min(1, q/p));
* at the first rejected row r the output token is drawn from the residual max(0, q_r - p_r),
  normalised (from q_r if that residual is zero everywhere); if all n proposals are accepted and
  n < n_b, it is drawn from q at row s + n; if n = n_b there is no row for it and the token is -1;
* a draw from weights w with the block's uniform v in [0, 1) is the inverse CDF in index order: the
  smallest index i with w_0 + ... + w_i > v (w_0 + ... + w_{V-1}). Zero-weight indices are never drawn.

A proposal outside [0, V) counts as rejected and raises SAMPLE_FLAG_BAD_TOKEN; negative L and
malformed offsets raise the same flags as greedy verification (accept 0, token -1 for the latter).
The random numbers are inputs: the oracle and the kernels consume the same draws.

Pinned by ``tests/test_spec_sample_pins.py``: softmax at temperature against scipy and torch, the
inverse CDF against a worked example and numpy.searchsorted, the output distribution of one verified
position against q (the theorem that makes speculative sampling exact), the small-temperature limit
against the pinned greedy verification, and the special cases z = y and u = 0. No function here is
parity-unpinned.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "SAMPLE_FLAG_NEG_L",
    "SAMPLE_FLAG_BAD_OFFSETS",
    "SAMPLE_FLAG_BAD_TOKEN",
    "softmax_t",
    "inverse_cdf",
    "verify_sample",
]

SAMPLE_FLAG_NEG_L = 1        # some block had L < 0 (treated as 0)
SAMPLE_FLAG_BAD_OFFSETS = 2  # some block had decreasing or out-of-range offsets (accept 0, token -1)
SAMPLE_FLAG_BAD_TOKEN = 8    # some verified row proposed a token outside [0, V) (counted as rejected)


def softmax_t(x, temperature: float) -> np.ndarray:
    """softmax(x / T) in float64, shifted by the maximum."""
    x = np.asarray(x, dtype=np.float64) / float(temperature)
    e = np.exp(x - x.max())
    return e / e.sum()


def inverse_cdf(w, u: float) -> int:
    """Smallest index i with w_0 + ... + w_i > u * sum(w), running left to right (w >= 0, u in [0, 1))."""
    w = np.asarray(w, dtype=np.float64)
    total = 0.0
    for wi in w:
        total += wi
    target = float(u) * total
    acc = 0.0
    for i, wi in enumerate(w):
        acc += wi
        if acc > target:
            return i
    # reachable only when u is so close to 1 that u * total rounds to total: the last positive weight
    return int(np.nonzero(w > 0)[0][-1])


def verify_sample(z, y, offsets, L, draft, u_accept, u_resample, temperature: float) -> dict:
    """Speculative-sampling verification of every packed block.

    z, y: [n_rows, V] logits (decoded exactly to float64). offsets [n_blocks + 1], L [n_blocks],
    draft [n_rows] proposed tokens, u_accept [n_rows] and u_resample [n_blocks] uniforms in [0, 1).
    Returns accept_len (int32), token (int32, -1 when there is none), flags, and a per-block trace:
    the decisions as (row, u * p(x), q(x)) and the draw as (row, kind) with kind 'residual',
    'target' or None.
    """
    z = np.asarray(z, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    off = np.asarray(offsets, dtype=np.int64)
    L = np.asarray(L, dtype=np.int64)
    draft = np.asarray(draft, dtype=np.int64)
    n_rows = z.shape[0]
    V = z.shape[1] if z.ndim == 2 else 0
    n_blocks = off.size - 1
    accept = np.zeros(n_blocks, dtype=np.int32)
    token = np.full(n_blocks, -1, dtype=np.int32)
    flags = 0
    trace = []
    for b in range(n_blocks):
        start, end = int(off[b]), int(off[b + 1])
        decisions = []
        if start < 0 or end < start or end > n_rows:
            flags |= SAMPLE_FLAG_BAD_OFFSETS
            trace.append({"decisions": decisions, "draw": (None, None)})
            continue
        nb = end - start
        if L[b] < 0:
            flags |= SAMPLE_FLAG_NEG_L
        n = int(min(max(int(L[b]), 0), nb))
        rejected_row = None
        for j in range(n):
            r = start + j
            x = int(draft[r])
            p = softmax_t(z[r], temperature)
            q = softmax_t(y[r], temperature)
            if x < 0 or x >= V:
                flags |= SAMPLE_FLAG_BAD_TOKEN
                decisions.append((r, None, None))
                rejected_row = r
                break
            lhs = float(u_accept[r]) * p[x]
            decisions.append((r, lhs, q[x]))
            if lhs > q[x]:
                rejected_row = r
                break
        if rejected_row is not None:
            accept[b] = rejected_row - start
            p = softmax_t(z[rejected_row], temperature)
            q = softmax_t(y[rejected_row], temperature)
            resid = np.maximum(q - p, 0.0)
            if resid.sum() > 0.0:
                token[b] = inverse_cdf(resid, u_resample[b])
                draw = (rejected_row, "residual")
            else:
                token[b] = inverse_cdf(q, u_resample[b])
                draw = (rejected_row, "target")
        else:
            accept[b] = n
            if n < nb:
                r = start + n
                token[b] = inverse_cdf(softmax_t(y[r], temperature), u_resample[b])
                draw = (r, "target")
            else:
                draw = (None, None)
        trace.append({"decisions": decisions, "draw": draw})
    return {"accept_len": accept, "token": token, "flags": flags, "trace": trace}
