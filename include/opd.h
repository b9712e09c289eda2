/*
 * opd.h — C ABI of the MI355X (gfx950) on-policy-distillation loss / verification library.
 *
 * What it computes (one "row" = one drafted position, V = vocabulary size):
 *   p = softmax(z) over the drafter logits z, q = softmax(y) over the target logits y,
 *   a = argmax y (target top-1, lowest index on ties), d = argmax z (draft top-1, same rule),
 *   loss = alpha * sum_v min(p_v (log p_v - log q_v), tau) + (1 - alpha) * (-log p_a)
 *   dz   = w * d loss / d z   (no gradient to y; w = grad_loss[row], default 1)
 *   accept_len[b] = longest prefix of packed block b, within clamp(L_b, 0, n_b) rows, on which
 *                   d == a.
 * Sources, by page title and section:
 *   - "AdaFlash: Adaptive Speculative Decoding with Online Self-Improvement for High-Concurrency
 *     LLM Inference" (besthub.dev article), section "1. On-Policy Distillation (OPD) for Domain
 *     Adaptation": reverse KL (drafter || target) plus top-1 hard labels from the target; each
 *     vocabulary term of the reverse KL is clipped before the sum.
 *   - same article, section "2. Adaptive Length Head for Token-Level Variance": blocks of k = 16
 *     drafted positions, verification budget set by a predicted acceptance length L.
 *   - same article, section "Infrastructure: Async Training & Variable-Length Batching": requests
 *     with different verification lengths packed contiguously into one batch (int32 offsets here).
 *   - "AdaFlash: Adaptive Speculative Decoding via On-Policy Distilled Diffusion Drafters"
 *     (project README page), section "Released Checkpoint": the drafter's loss is a mixture of
 *     reverse KL and the hard-label term.
 * alpha and tau are explicit arguments (the pages do not fix them). Temperature is 1; callers
 * pre-scale logits for other temperatures. The clip is an upper clip only; at t_v == tau the term
 * counts as unclipped (its gradient passes).
 *
 * Conventions shared by every call
 *   - Array arguments are DEVICE pointers, owned by the caller; the library allocates nothing and
 *     keeps no device state apart from what lives in the caller's workspace.
 *   - Logit matrices are row-major [n_rows, ld] with ld >= vocab; the caller's buffer must span
 *     n_rows * ld elements (the pad [vocab, ld) of a row may be read, never written). Base pointer
 *     and row pitch (ld * element size) must be multiples of 16 bytes.
 *   - Calls enqueue work on `stream` (a hipStream_t; NULL = the legacy default stream) and return
 *     without synchronising. Host-checkable errors return before any HIP call is made.
 *   - Results are deterministic: the same inputs give bit-identical outputs (no floating-point
 *     atomics; every reduction has a fixed order).
 *   - Preconditions on values: finite logits with |logit| <= 1e4. Other values give unspecified
 *     numbers but every kernel still terminates.
 *   - A workspace of opd_workspace_size() bytes, zero-filled once when first allocated, must be
 *     passed to every call; calls that share a workspace must not run concurrently. Besides the
 *     sticky flags it holds the state of the cross-workgroup exchanges. A call made while its
 *     stream is being captured into a HIP graph takes that state from an epoch in the workspace,
 *     read and advanced on the device by each launch (about 2 us more per launch), so the graph
 *     may be replayed any number of times; other calls take it from the host.
 *   - Device-side content problems (negative L, malformed offsets, a cross-workgroup wait that
 *     exceeded its bound) set bits in a sticky flag word inside the workspace, read with
 *     opd_read_flags(), or reported by the call itself in check mode (opd_set_check, OPD_CHECK=1).
 *   - The row-team kernels keep all G workgroups of a row resident at once and exchange partial
 *     results between them with bounded waits. The grid is sized for an otherwise idle device; if
 *     other work keeps a member of a team from being scheduled, the waits end on their bound and
 *     the call raises OPD_FLAG_SPIN_TIMEOUT (outputs invalid) instead of hanging.
 */
#ifndef OPD_MI355X_H
#define OPD_MI355X_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { OPD_F32 = 0, OPD_BF16 = 1 } opd_dtype_t;

typedef enum {
  OPD_OK = 0,
  OPD_ERR_NULL = 1,       /* a required pointer is NULL                                       */
  OPD_ERR_SHAPE = 2,      /* n_rows < 0, vocab <= 0 or > 524288, ld < vocab, n_blocks < 0    */
  OPD_ERR_DTYPE = 3,      /* dtype value not in opd_dtype_t                                   */
  OPD_ERR_ALIGN = 4,      /* base pointer or row pitch not a multiple of 16 bytes              */
  OPD_ERR_PARAM = 5,      /* alpha outside [0, 1] or NaN, tau NaN                              */
  OPD_ERR_WORKSPACE = 6,  /* workspace NULL or smaller than opd_workspace_size()              */
  OPD_ERR_HIP = 7,        /* a HIP call failed; opd_last_error() has the HIP error text       */
  OPD_ERR_DEVICE = 8      /* check mode only: the call raised device flags (see opd_set_check) */
} opd_status_t;

/* Bits of the sticky device flag word (see opd_read_flags). */
#define OPD_FLAG_NEG_L 1u        /* some block had L < 0 (treated as 0)                         */
#define OPD_FLAG_BAD_OFFSETS 2u  /* some block had decreasing / out-of-range offsets (accept 0)   */
#define OPD_FLAG_SPIN_TIMEOUT 4u /* a cross-workgroup wait exceeded its bound: outputs invalid    */
#define OPD_FLAG_BAD_TOKEN 8u    /* a verified row proposed a token outside [0, vocab) (rejected)  */

/* Packed verification blocks ("Infrastructure: ... Variable-Length Batching"): block b owns rows
 * offsets[b] .. offsets[b+1]-1; L[b] is the length head's predicted verification length.
 * The struct lives on the host; both arrays are device arrays. */
typedef struct {
  const int32_t* offsets; /* [n_blocks + 1], expected offsets[0] = 0, non-decreasing, <= n_rows */
  const int32_t* L;       /* [n_blocks]                                                          */
  int32_t n_blocks;
} opd_blocks_t;

/* Bytes of workspace every call needs (independent of the problem size). */
size_t opd_workspace_size(void);

/*
 * Forward: per-row loss and the statistics the backward pass reuses.
 *   z, y        [n_rows, ld] drafter / target logits of dtype dt.
 *   loss        [n_rows] float32 out.
 *   target_top1 [n_rows] int32 out (argmax y); draft_top1 [n_rows] int32 out, may be NULL.
 *   row_stats   [n_rows][8] float32 out: (LSE(z), LSE(y), S, clipped reverse KL, max z,
 *               log sum_v e^(z_v - max z), LSE(z) - LSE(y), cross entropy), where
 *               S = sum_v p_v [t_v <= tau] (log p_v - log q_v + 1) is the row constant of the
 *               gradient. Entries 4..6 carry LSE(z) and the LSE difference at full precision for
 *               the backward pass.
 * Errors: OPD_ERR_NULL (z, y, loss, target_top1, row_stats), OPD_ERR_SHAPE, OPD_ERR_DTYPE,
 * OPD_ERR_ALIGN, OPD_ERR_PARAM, OPD_ERR_WORKSPACE, OPD_ERR_HIP.
 */
opd_status_t opd_loss_fwd(const void* z, const void* y, opd_dtype_t dt, int64_t n_rows, int64_t vocab,
                          int64_t ld, float alpha, float tau, float* loss, int32_t* target_top1,
                          int32_t* draft_top1, float* row_stats, void* ws, size_t ws_bytes,
                          hipStream_t stream);

/*
 * Backward: dz = grad_loss[row] * d loss_row / d z_row from the forward's row_stats and
 * target_top1 (one streaming pass: read z and y, write dz).
 *   grad_loss   [n_rows] float32, may be NULL (then 1 for every row).
 *   dz          [n_rows, ld_dz] of dtype dz_dt (bf16 is rounded to nearest even); must not alias
 *               z or y. Pitch ld_dz * size must be a multiple of 16 bytes, ld_dz >= vocab.
 * Errors: as opd_loss_fwd, plus OPD_ERR_NULL for row_stats / target_top1 / dz.
 */
opd_status_t opd_loss_bwd(const void* z, const void* y, opd_dtype_t dt, int64_t n_rows, int64_t vocab,
                          int64_t ld, float alpha, float tau, const float* row_stats,
                          const int32_t* target_top1, const float* grad_loss, void* dz,
                          opd_dtype_t dz_dt, int64_t ld_dz, void* ws, size_t ws_bytes,
                          hipStream_t stream);

/*
 * Greedy verification ("2. Adaptive Length Head ..."): computes both top-1 arrays from the logits
 * and the accepted-prefix length of every packed block.
 *   target_top1, draft_top1 [n_rows] int32 out; accept_len [n_blocks] int32 out.
 * Errors: OPD_ERR_NULL (z, y, blocks and its arrays when n_blocks > 0, the three outputs),
 * OPD_ERR_SHAPE, OPD_ERR_DTYPE, OPD_ERR_ALIGN, OPD_ERR_WORKSPACE, OPD_ERR_HIP.
 */
opd_status_t verify_accept_len(const void* z, const void* y, opd_dtype_t dt, int64_t n_rows,
                               int64_t vocab, int64_t ld, const opd_blocks_t* blocks,
                               int32_t* target_top1, int32_t* draft_top1, int32_t* accept_len,
                               void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Fused forward + backward + verification: everything above in one pass over the logits (each of
 * z and y read once from HBM, dz written once), then the per-block accept lengths.
 *   blocks may be NULL (no verification; accept_len ignored).
 * Outputs and errors: the union of the three calls above.
 */
opd_status_t opd_fused_fwd_bwd_verify(const void* z, const void* y, opd_dtype_t dt, int64_t n_rows,
                                      int64_t vocab, int64_t ld, const opd_blocks_t* blocks,
                                      float alpha, float tau, const float* grad_loss, float* loss,
                                      int32_t* target_top1, int32_t* draft_top1, float* row_stats,
                                      void* dz, opd_dtype_t dz_dt, int64_t ld_dz,
                                      int32_t* accept_len, void* ws, size_t ws_bytes,
                                      hipStream_t stream);

/*
 * opd_fused_fwd_bwd_verify for callers that cannot allocate device memory (code under stream
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same computation, arguments
 * and results, without the workspace arguments. The workspace is a fixed array of
 * opd_workspace_size() bytes inside the library (one per GPU, held until the process ends, zeroed
 * by the first call on each GPU); the call makes no allocation of its own. Every call on a GPU
 * shares that GPU's array, so calls that overlap on one GPU (e.g. on two streams at once) race and
 * must not be made. The array covers every problem size the regular call accepts (a launch uses
 * at most 4096 row-team workgroups); sizes the regular call rejects are rejected the same way.
 * Device flags accumulate in the array and are reported by check mode (opd_set_check / OPD_CHECK=1).
 */
opd_status_t opd_fused_fwd_bwd_verify_noalloc(const void* z, const void* y, opd_dtype_t dt, int64_t n_rows,
                                              int64_t vocab, int64_t ld, const opd_blocks_t* blocks,
                                              float alpha, float tau, const float* grad_loss, float* loss,
                                              int32_t* target_top1, int32_t* draft_top1, float* row_stats,
                                              void* dz, opd_dtype_t dz_dt, int64_t ld_dz,
                                              int32_t* accept_len, hipStream_t stream);

/*
 * Length-head epilogue of verification ("AdaFlash: Adaptive Speculative Decoding with Online
 * Self-Improvement for High-Concurrency LLM Inference", section "2. Adaptive Length Head for
 * Token-Level Variance": the head predicts a draft block's acceptance rate, and the true rate after
 * verification is its free supervision signal). From the top-1s of a packed batch (as produced by
 * opd_fused_fwd_bwd_verify or verify_accept_len), per block b = rows offsets[b] .. offsets[b+1]-1:
 *   accept_full[b] int32 out: longest prefix of the block's n_b rows with draft_top1 == target_top1
 *                  (all rows: not capped by the verification budget L);
 *   label[b]       f32 out: accept_full[b] / n_b, 0 for an empty block;
 *   loss[b]        f32 out: binary cross entropy of sigmoid(head_logit[b]) against label[b];
 *   dlogit[b]      f32 out: grad[b] * (sigmoid(head_logit[b]) - label[b]); grad may be NULL (= 1).
 *   target_top1, draft_top1 [n_rows] int32 device inputs; offsets int32[n_blocks + 1] device;
 *   head_logit [n_blocks] f32 device input. All device pointers, owned by the caller.
 * A block with decreasing or out-of-range offsets gets 0 outputs and raises OPD_FLAG_BAD_OFFSETS.
 * Errors: OPD_ERR_NULL, OPD_ERR_SHAPE (n_rows / n_blocks), OPD_ERR_WORKSPACE, OPD_ERR_HIP.
 */
opd_status_t opd_length_head_loss(const int32_t* target_top1, const int32_t* draft_top1, int64_t n_rows,
                                  const int32_t* offsets, int32_t n_blocks, const float* head_logit,
                                  const float* grad, int32_t* accept_full, float* label, float* loss,
                                  float* dlogit, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Stochastic verification at a sampling temperature (speculative sampling). The pages name the
 * temperature as a parameter to tune when drafter and target are combined ("Adaflash Adaptive
 * Speculative Decoding", skills-directory card, section "Implementation Steps") but give no rule
 * for it; the rule is the published speculative-sampling one (Leviathan et al. 2023; Chen et al.
 * 2023). With p_r = softmax(z_r / T), q_r = softmax(y_r / T) and x_r = draft_tokens[r], per
 * packed block b (rows s = offsets[b] .. offsets[b+1]-1, n_b rows,
 * n = clamp(L[b], 0, n_b)):
 *   - rows s .. s+n-1 are verified in order; row r's proposal is accepted when
 *     u_accept[r] * p_r(x_r) <= q_r(x_r); accept_len[b] = rows accepted before the first rejection;
 *   - out_token[b]: at the first rejected row r, a draw from max(0, q_r - p_r) normalised (from q_r
 *     if that residual is zero everywhere); after n accepted rows with n < n_b, a draw from q at row
 *     s + n; -1 when n = n_b and all were accepted, or the block is malformed. A draw from weights w
 *     with v = u_resample[b] is the smallest index i with w_0 + ... + w_i > v * sum(w).
 *   z, y             [n_rows, ld] logits of dtype dt (as for the other calls).
 *   draft_tokens     [n_rows] int32: proposed tokens; one outside [0, vocab) is rejected and raises
 *                    OPD_FLAG_BAD_TOKEN.
 *   u_accept         [n_rows] f32 uniforms in [0, 1); u_resample [n_blocks] f32 uniforms in [0, 1).
 *                    The random numbers are the caller's: the call draws none.
 *   temperature      T in [1e-6, inf).
 *   accept_len, out_token [n_blocks] int32 out.
 *   row_lse          [n_rows][4] f32 out: (c_z, l_z, c_y, l_y) with log2 sum_v 2^(z_v log2(e) / T) =
 *                    c_z + l_z (c_z a reference near the row maximum, l_z = log2 of the sum relative to
 *                    it), likewise for y; so log of the normaliser of softmax(z / T) is (c_z + l_z) ln 2.
 *                    Written only for the rows the verification can read: the first
 *                    min(n + 1, n_b) rows of every well-formed block; other entries are left as they are.
 * Those rows are read once (z and y) for row_lse; the decisions then read two elements per verified
 * row, and each draw reads its row once more. Decisions and draws are taken in fp32 on sums
 * formed in a fixed order (deterministic); a draw whose target falls on a rounding edge takes the last
 * positive weight before it. Negative L and malformed offsets raise the greedy call's flags.
 * Errors: OPD_ERR_NULL, OPD_ERR_SHAPE, OPD_ERR_DTYPE, OPD_ERR_ALIGN, OPD_ERR_PARAM (temperature),
 * OPD_ERR_WORKSPACE, OPD_ERR_HIP.
 */
opd_status_t opd_verify_sample(const void* z, const void* y, opd_dtype_t dt, int64_t n_rows, int64_t vocab,
                               int64_t ld, const opd_blocks_t* blocks, const int32_t* draft_tokens,
                               const float* u_accept, const float* u_resample, float temperature,
                               int32_t* accept_len, int32_t* out_token, float* row_lse, void* ws,
                               size_t ws_bytes, hipStream_t stream);

/*
 * The OPD loss fused with the drafter's vocabulary projection: the logits z = h W^T are never held
 * for the whole batch. The loss is the one above ("AdaFlash: Adaptive Speculative Decoding with
 * Online Self-Improvement ...", section "1. On-Policy Distillation (OPD) for Domain Adaptation":
 * the drafter is what the online update trains); the pages show neither the drafter's head nor its
 * sizes, so h is read as the drafter's final hidden states and W as its projection (no bias), and
 * the gradient flows to both. Rows are processed in chunks of chunk_rows: per chunk, z (fp32) =
 * h W^T into scratch, the fused loss / gradient / top-1 pass of opd_fused_fwd_bwd_verify over that
 * chunk (dz as bf16 into scratch), dh = dz W and dW (+)= dz^T h; then the accept lengths of all
 * blocks. The three products run on the library's own bf16 MFMA kernels (fp32 accumulation and
 * output); the logits product also forms each row's max, lowest argmax and log-sum-exp in its
 * epilogue.
 *   h          [n_rows, hidden] bf16, row-major, pitch hidden (hidden a multiple of 8).
 *   W          [vocab, hidden] bf16, row-major, pitch hidden.
 *   y          [n_rows, ld_y] target logits, dt_y must be OPD_F32 (the logits chunk is fp32 and the
 *              row kernel reads both with one pitch); ld_y >= vocab, pitch a multiple of 16 bytes.
 *   loss, target_top1, draft_top1, row_stats, accept_len: as opd_fused_fwd_bwd_verify (draft_top1
 *              may be NULL only without blocks); grad_loss [n_rows] or NULL.
 *   dh         [n_rows, hidden] f32 out (overwritten), or NULL to skip.
 *   dW         [vocab, hidden] f32 out (overwritten: the sum over all chunks), or NULL to skip.
 *   logit_max_lse [n_rows][2] f32 out (max z, log sum_v e^z_v) from the product's epilogue, or NULL.
 *   logit_argmax  [n_rows] int32 out (lowest index of max z) from the same epilogue, or NULL. With
 *              both NULL the epilogue statistics are skipped.
 *   scratch    caller device memory of at least opd_lmhead_scratch_size(min(chunk_rows, n_rows),
 *              vocab, ld_y) bytes, 16-byte aligned: one chunk of fp32 logits (which later holds the
 *              dh product's split-K partials) and of bf16 dz (which first holds the logits
 *              statistics partials).
 * dh and dW are formed from the bf16-rounded dz of the row kernel. Size limits of the products:
 * every operand (W: vocab x hidden x 2 bytes; a chunk of h or dz) under 4 GiB, and 256 rows of the
 * logits chunk under 4 GiB (32-bit buffer offsets). Nothing is allocated. This call is not tested
 * under stream capture.
 * Errors: OPD_ERR_NULL, OPD_ERR_SHAPE (including the size limits), OPD_ERR_DTYPE (dt_y not OPD_F32),
 * OPD_ERR_ALIGN, OPD_ERR_PARAM, OPD_ERR_WORKSPACE (ws or scratch too small), OPD_ERR_HIP.
 */
size_t opd_lmhead_scratch_size(int64_t chunk_rows, int64_t vocab, int64_t ld_y);
opd_status_t opd_lmhead_fused_fwd_bwd_verify(const void* h, const void* W, int64_t hidden, const void* y,
                                             opd_dtype_t dt_y, int64_t n_rows, int64_t vocab, int64_t ld_y,
                                             const opd_blocks_t* blocks, float alpha, float tau,
                                             const float* grad_loss, float* loss, int32_t* target_top1,
                                             int32_t* draft_top1, float* row_stats, float* dh, float* dW,
                                             float* logit_max_lse, int32_t* logit_argmax, int32_t* accept_len,
                                             void* scratch, size_t scratch_bytes, int64_t chunk_rows, void* ws,
                                             size_t ws_bytes, hipStream_t stream);

/*
 * Host-side batch scheduling ("AdaFlash: Adaptive Speculative Decoding with Online Self-Improvement
 * for High-Concurrency LLM Inference", section "Infrastructure: Async Training & Variable-Length
 * Batching": requests with different predicted verification lengths are packed into compact batches
 * and an exponential moving average estimates the next round's capacity). These run on the host and
 * take HOST pointers; their output (offsets, lengths) is the packed layout the calls above take.
 *
 * Capacity estimate: e <- beta e + (1 - beta) observed, the first observation initialising e; the
 * next batch's row budget is floor(e). `observed_rows` is the verification capacity (rows) the
 * caller measured in the round just finished (e.g. what fitted in its memory budget).
 * Errors: OPD_ERR_NULL, OPD_ERR_PARAM (beta outside [0, 1], observed negative or not finite).
 */
typedef struct {
  double ema;     /* current estimate (rows) */
  double beta;    /* weight of the previous estimate */
  int32_t n_obs;  /* observations so far */
} opd_capacity_t;
opd_status_t opd_capacity_init(opd_capacity_t* c, double beta);
opd_status_t opd_capacity_observe(opd_capacity_t* c, double observed_rows, int64_t* budget_rows);

/*
 * First-fit packing in arrival order: scans lengths[0 .. n_pending) (predicted verification rows of
 * the pending requests, each >= 1), takes every request that still fits in budget_rows (and, if
 * max_requests > 0, stops after max_requests), and leaves the rest queued.
 *   selected[n_pending] out: indices of the packed requests, in arrival order (first *n_selected);
 *   offsets[n_pending + 1] out: exclusive prefix sum of their lengths (first *n_selected + 1);
 *   packed_lengths[n_pending] out: their lengths; *n_rows out: total rows (<= budget_rows).
 * Errors: OPD_ERR_NULL, OPD_ERR_SHAPE (negative sizes), OPD_ERR_PARAM (a length < 1).
 */
opd_status_t opd_pack_first_fit(const int32_t* lengths, int32_t n_pending, int64_t budget_rows,
                                int32_t max_requests, int32_t* selected, int32_t* offsets,
                                int32_t* packed_lengths, int32_t* n_selected, int64_t* n_rows);

/* Reads the sticky device flag word of a workspace (synchronises `stream`); clears it when
 * `clear` is non-zero. Errors: OPD_ERR_NULL, OPD_ERR_WORKSPACE, OPD_ERR_HIP. */
opd_status_t opd_read_flags(void* ws, size_t ws_bytes, int clear, uint32_t* flags, hipStream_t stream);

/* Measurement aid, not part of the method: streams the HBM traffic pattern of the fused path --
 * two 16-byte reads and one 16-byte write per vector, nontemporal -- with no arithmetic beyond
 * c = a XOR b, so that its rate is the achievable bandwidth for that pattern on this device.
 * With c NULL it only reads a and b; with a and b both NULL it only writes c: the read-only and
 * write-only ceilings of the same device.
 *   a, b   device buffers of `bytes` bytes (read), both given or both NULL.
 *   c      device buffer of `bytes` bytes (written), or NULL; at least one of (a, b) and c is given.
 *          In read-only mode c is NULL and nothing is written.
 *   bytes  multiple of 16; the given pointers 16-byte aligned; 0 is a no-op.
 * Errors: OPD_ERR_NULL (exactly one of a, b given, or nothing to do), OPD_ERR_SHAPE (bytes not a
 * multiple of 16), OPD_ERR_ALIGN, OPD_ERR_HIP. */
opd_status_t opd_stream_probe(const void* a, const void* b, void* c, size_t bytes, hipStream_t stream);

/* Debug knob for tests of the failure path: caps every cross-workgroup wait at `spins` polls
 * (0 restores the default bound). Affects launches made after the call, process-wide. */
void opd_set_spin_limit(uint32_t spins);

/* Check mode, for debugging and for callers that need failures surfaced at once. When on, every
 * call that takes a workspace synchronises its stream after enqueuing its work, reads the sticky
 * flag word, and if a bit is set clears it and returns OPD_ERR_DEVICE (opd_last_error() names the
 * flags); a kernel failure found by the synchronisation returns OPD_ERR_HIP. Calls made while their
 * stream is being captured into a graph are not checked (they cannot synchronise). Off by default;
 * the environment variable OPD_CHECK=1 turns it on at the first call, opd_set_check(0 / 1) at any
 * time (process-wide). opd_get_check() returns the current setting. */
void opd_set_check(int on);
int opd_get_check(void);

/* Exchange-flag bookkeeping of calls made outside stream capture, exposed so that the restart of the
 * flag range can be tested without a GPU. Each launch takes `count` fresh flags from a process-wide
 * range of 2^31; when the range is used up it restarts, and a workspace last used before the
 * restart has its exchange units zeroed (a fill kernel on the call's stream) before its next
 * launch, so that no unit left from the previous range can match a flag handed out again.
 * This function performs the reservation for workspace `ws` (only its address is used) without
 * launching anything: *base = first flag - 1, *must_clear = whether a launch would zero the units
 * first. next_offset >= 0 first moves the range's counter to that offset (tests); -1 leaves it.
 * Errors: OPD_ERR_NULL, OPD_ERR_SHAPE (count 0 or >= 2^30, next_offset >= 2^31). */
opd_status_t opd_debug_reserve_flags(const void* ws, uint32_t count, int64_t next_offset, uint32_t* base,
                                     int* must_clear);

/* Static description of a status code, and the detail text of the last error on this thread. */
const char* opd_status_string(opd_status_t s);
const char* opd_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* OPD_MI355X_H */
