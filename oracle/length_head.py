"""Float64 CPU oracle for the length-head epilogue of verification.

TEST INFRASTRUCTURE ONLY: the plain definition that the HIP epilogue kernel is checked against.
Only the test suite, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may import
it; it shares no code with the product library.

Source: "AdaFlash: Adaptive Speculative Decoding with Online Self-Improvement for High-Concurrency
LLM Inference" (besthub.dev article), section "2. Adaptive Length Head for Token-Level Variance": a
light head predicts the acceptance rate of the current draft block; after verification the true
acceptance rate is a free supervision signal for updating that head online. Packed blocks follow
section "Infrastructure: Async Training & Variable-Length Batching".

Readings (the pages fix neither the head's output form nor its loss):

* the head emits one logit h per block; its predicted rate is sigmoid(h);
* the label is the true acceptance rate of the block: the longest prefix of the block's n_b drafted
  positions on which the draft top-1 equals the target top-1, divided by n_b (0 for an empty
  block). It is not capped by the verification budget L: the training side has the target's top-1
  for every drafted position;
* the loss is the binary cross entropy of sigmoid(h) against that rate,
  -[label log sigmoid(h) + (1 - label) log(1 - sigmoid(h))], and its gradient is taken w.r.t. h.

Pinned by ``tests/test_length_head_pins.py`` (library special case, closed forms, symmetry,
finite differences, brute force); no function here is parity-unpinned.
"""

from __future__ import annotations

import math

import numpy as np

__all__ = ["LEN_FLAG_BAD_OFFSETS", "block_targets", "bce_with_logit", "length_head_epilogue"]

LEN_FLAG_BAD_OFFSETS = 2  # some block had decreasing or out-of-range offsets (its outputs are 0)


def block_targets(draft_top1, target_top1, offsets) -> tuple[np.ndarray, np.ndarray, int]:
    """Uncapped accepted prefix and true acceptance rate of every packed block.

    Block b holds rows offsets[b] .. offsets[b+1]-1. accept_full[b] counts the leading rows of the
    block whose draft top-1 equals the target top-1; label[b] = accept_full[b] / n_b. A block with
    malformed offsets gets 0, 0 and raises LEN_FLAG_BAD_OFFSETS. Returns (accept_full int32,
    label float64, flags).
    """
    d = np.asarray(draft_top1, dtype=np.int64)
    a = np.asarray(target_top1, dtype=np.int64)
    off = np.asarray(offsets, dtype=np.int64)
    n_rows = d.size
    n_blocks = off.size - 1
    acc = np.zeros(n_blocks, dtype=np.int32)
    label = np.zeros(n_blocks, dtype=np.float64)
    flags = 0
    for b in range(n_blocks):
        start, end = int(off[b]), int(off[b + 1])
        if start < 0 or end < start or end > n_rows:
            flags |= LEN_FLAG_BAD_OFFSETS
            continue
        k = 0
        while start + k < end and d[start + k] == a[start + k]:
            k += 1
        acc[b] = k
        label[b] = k / (end - start) if end > start else 0.0
    return acc, label, flags


def bce_with_logit(h: float, label: float) -> tuple[float, float]:
    """Binary cross entropy of sigmoid(h) against label, and its derivative w.r.t. h.

    -[label log s + (1 - label) log(1 - s)] with s = sigmoid(h), written with log s = -log(1 + e^-h)
    and log(1 - s) = -log(1 + e^h) so that float64 keeps full accuracy for large |h|. The
    derivative is s - label.
    """
    h = float(h)
    label = float(label)

    def log1pexp(x: float) -> float:  # log(1 + e^x) without overflow
        return x + math.log1p(math.exp(-x)) if x > 0 else math.log1p(math.exp(x))

    loss = label * log1pexp(-h) + (1.0 - label) * log1pexp(h)
    s = 1.0 / (1.0 + math.exp(-h)) if h >= 0 else math.exp(h) / (1.0 + math.exp(h))
    return loss, s - label


def length_head_epilogue(draft_top1, target_top1, offsets, head_logit, grad=None) -> dict:
    """The whole epilogue per block: accept_full, label, loss and dlogit = grad * dloss/dh.

    Blocks with malformed offsets get accept 0, label 0, loss 0 and dlogit 0.
    """
    acc, label, flags = block_targets(draft_top1, target_top1, offsets)
    h = np.asarray(head_logit, dtype=np.float64)
    w = np.ones_like(h) if grad is None else np.asarray(grad, dtype=np.float64)
    off = np.asarray(offsets, dtype=np.int64)
    n_rows = np.asarray(draft_top1).size
    loss = np.zeros_like(h)
    dlogit = np.zeros_like(h)
    for b in range(h.size):
        start, end = int(off[b]), int(off[b + 1])
        if start < 0 or end < start or end > n_rows:
            continue
        loss[b], g = bce_with_logit(h[b], label[b])
        dlogit[b] = w[b] * g
    return {"accept_full": acc, "label": label, "loss": loss, "dlogit": dlogit, "flags": flags}
