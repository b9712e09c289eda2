"""Plain CPU oracle for the variable-length request packer and its EMA capacity estimate.

TEST INFRASTRUCTURE ONLY: the definition that the C++ packer of the library is checked against.
Only the test suite may import it; it shares no code with the product library.

Source: "AdaFlash: Adaptive Speculative Decoding with Online Self-Improvement for High-Concurrency
LLM Inference" (besthub.dev article), section "Infrastructure: Async Training & Variable-Length
Batching": requests with different predicted verification lengths are packed into compact batches,
and an exponential moving average estimates the next round's capacity, to keep the GPU busy without
running out of memory. The closing section adds that the scheduler repacks batches as concurrency
and verification lengths change.

Readings (the pages give neither the packing rule nor the EMA's form or constants):

* a pending request r needs L_r >= 1 rows of verification (its predicted length); a batch is a set
  of requests whose rows are laid out contiguously in arrival order (offsets = exclusive prefix sum
  of their L);
* packing is first-fit in arrival order: scan the queue, take each request that still fits in the
  row budget (and under the optional cap on requests per batch), leave the others queued in place;
* the capacity estimate is e_{t+1} = beta e_t + (1 - beta) c_t, with c_t the capacity (rows) the
  caller observed in round t and e_1 = c_0 (the first observation); the next round's row budget is
  floor(e).

Pinned by ``tests/test_packer_pins.py`` (maximality and prefix invariants of first-fit, closed forms
of the EMA); no function here is parity-unpinned.
"""

from __future__ import annotations

import math

__all__ = ["pack_first_fit", "ema_update"]


def pack_first_fit(lengths, budget_rows: int, max_requests: int = 0) -> dict:
    """First-fit packing in arrival order.

    lengths: predicted verification rows of the pending requests, in arrival order (each >= 1).
    budget_rows: row budget of the batch (>= 0). max_requests: cap on requests (0 = none).
    Returns selected (indices, arrival order), offsets (len(selected) + 1), lengths of the packed
    requests and the total rows.
    """
    selected, used = [], 0
    for r, L in enumerate(lengths):
        L = int(L)
        if L < 1:
            raise ValueError("predicted lengths must be >= 1")
        if max_requests and len(selected) == max_requests:
            break
        if used + L <= budget_rows:
            selected.append(r)
            used += L
    offsets = [0]
    for r in selected:
        offsets.append(offsets[-1] + int(lengths[r]))
    return {"selected": selected, "offsets": offsets, "lengths": [int(lengths[r]) for r in selected], "rows": used}


def ema_update(state, observed: float, beta: float):
    """One round of the capacity estimate. state is None before the first observation.

    Returns (new_state, budget_rows) with budget_rows = floor(new_state).
    """
    observed = float(observed)
    if state is None:
        e = observed
    else:
        e = beta * float(state) + (1.0 - beta) * observed
    return e, int(math.floor(e))
