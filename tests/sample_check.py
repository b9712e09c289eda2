"""Comparison of speculative-sampling verification results with the float64 oracle.

Floating point decides integers here: an accept decision compares u p(x) with q(x), and a draw
compares a running sum with u times the total. The kernels take these decisions in fp32, the oracle
in float64, so where the two sides of a comparison lie within rounding of each other either outcome
is correct. The rule applied:

* an accept decision whose sides differ by at most DECISION_RTOL relative may go either way; the
  oracle is then re-run with the kernel's outcome forced at that row, and the rest must match;
* a drawn token must lie in the window of indices whose float64 CDF interval comes within
  DRAW_ATOL of u * total (weights are probabilities, so the CDF is in probability units).

DECISION_RTOL: p(x) and q(x) come from exp2 of an fma against the row's log2-sum, each within a few
fp32 ulps (relative 1e-6) plus the log2-sum's own rounding; 1e-4 leaves two orders of margin.
DRAW_ATOL: each fp32 weight is within ~1e-6 relative of its float64 value, so the CDF at any index
is off by at most ~1e-6 * (sum p + sum q) = 2e-6 absolute, plus the fp32 rounding of the running
sums (at most ~2e-6 over 151,936 terms summed in tiles); 1e-4 again leaves margin.
"""

import numpy as np

from oracle import spec_sample as S

DECISION_RTOL = 1e-4
DRAW_ATOL = 1e-4


def draw_window(w, u):
    """Indices a draw from weights w with uniform u may return within DRAW_ATOL."""
    w = np.asarray(w, dtype=np.float64)
    cdf = np.cumsum(w)
    prev = np.concatenate([[0.0], cdf[:-1]])
    target = float(u) * cdf[-1]
    ok = (cdf >= target - DRAW_ATOL) & (prev <= target + DRAW_ATOL)
    return set(np.nonzero(ok)[0].tolist())


def check_block(z, y, L, draft, ua, ur, T, acc_k, tok_k):
    """z, y, draft, ua: the block's rows. Returns None when the kernel's result is a correct one."""
    ua = np.array(ua, dtype=np.float64)
    n_b = z.shape[0]
    for _ in range(4):
        r = S.verify_sample(z, y, [0, n_b], [L], draft, ua, [ur], T)
        acc_o, tok_o = int(r["accept_len"][0]), int(r["token"][0])
        dec = r["trace"][0]["decisions"]
        if acc_o != acc_k:
            j = min(acc_o, acc_k)
            if j >= len(dec):
                return f"accept {acc_k} vs oracle {acc_o}: no decision at row {j}"
            _, lhs, q = dec[j]
            if lhs is None or abs(lhs - q) > DECISION_RTOL * max(lhs, q):
                return f"accept {acc_k} vs oracle {acc_o}: decision at row {j} not ambiguous (u p = {lhs}, q = {q})"
            if acc_k > j:
                ua[j] = 0.0  # the kernel accepted: force acceptance
            else:
                ua[j] = min(ua[j] * (1.0 + 3.0 * DECISION_RTOL), np.nextafter(1.0, 0.0))
            continue
        if tok_o == tok_k:
            return None
        row, kind = r["trace"][0]["draw"]
        if row is None:
            return f"token {tok_k} vs oracle {tok_o} with no draw"
        p = S.softmax_t(z[row], T)
        q = S.softmax_t(y[row], T)
        w = np.maximum(q - p, 0.0) if kind == "residual" else q
        if tok_k in draw_window(w, ur):
            return None
        return f"token {tok_k} vs oracle {tok_o} (draw at row {row}, {kind}) outside the window"
    return "more than three ambiguous decisions in one block"


def uniforms(rng, n):
    """float32-exact uniforms in [0, 1) (24-bit grid)."""
    return (rng.integers(0, 1 << 24, n) / float(1 << 24)).astype(np.float32)


def sample_drafts(rng, z, T):
    """One proposal per row drawn from softmax(z / T) (host float64, the drafter's own sampling)."""
    out = np.empty(z.shape[0], dtype=np.int32)
    for r in range(z.shape[0]):
        cdf = np.cumsum(S.softmax_t(z[r], T))
        out[r] = min(int(np.searchsorted(cdf, rng.random() * cdf[-1], side="right")), z.shape[1] - 1)
    return out
