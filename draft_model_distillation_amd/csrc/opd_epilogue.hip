// Length-head epilogue of verification, after "AdaFlash: Adaptive Speculative Decoding with Online
// Self-Improvement for High-Concurrency LLM Inference" (besthub.dev article), section "2. Adaptive
// Length Head for Token-Level Variance": a light head predicts the acceptance rate of a draft block,
// and after verification the true rate is a free label for updating it online.
//
// Per packed block b (rows offsets[b] .. offsets[b+1]-1, section "Infrastructure: ... Variable-Length
// Batching"): the longest prefix on which draft top-1 == target top-1 over all n_b rows (not capped
// by the verification budget), the rate label = prefix / n_b, the binary cross entropy of
// sigmoid(head_logit) against it and its gradient w.r.t. the logit.
//
// This file is compiled with the default IEEE mode (unlike the row kernels), so that expf / log1pf
// come inlined from the device library with their full accuracy.

#include <stdint.h>

#include "opd_internal.h"

namespace opd {
namespace {

// log(1 + e^x) without overflow
__device__ __forceinline__ float softplus(float x) { return fmaxf(x, 0.f) + log1pf(expf(-fabsf(x))); }

// One wave per block: lane j compares row j of each 64-row window, and a ballot gives the first
// mismatch (one round of loads per window instead of one per matching row); lane 0 writes.
constexpr int kBlocksPerGroup = kThreads / 64;

__global__ void __launch_bounds__(kThreads) k_length_head(LengthHeadParams P) {
  const int lane = threadIdx.x & 63;
  const int b = blockIdx.x * kBlocksPerGroup + (threadIdx.x >> 6);
  if (b >= P.n_blocks) return;  // wave-uniform
  const int start = P.offsets[b], end = P.offsets[b + 1];
  int acc = 0;
  float label = 0.f, loss = 0.f, dl = 0.f;
  const bool bad = start < 0 || end < start || end > P.n_rows;
  if (!bad) {
    const int n = end - start;
    acc = n;
    for (int j0 = 0; j0 < n; j0 += 64) {
      const int j = j0 + lane;
      const bool mismatch = j < n && P.draft_top1[start + j] != P.target_top1[start + j];
      const uint64_t m = __builtin_amdgcn_ballot_w64(mismatch);
      if (m) {
        acc = j0 + (int)__builtin_ctzll(m);
        break;
      }
    }
  }
  if (lane != 0) return;
  if (bad) {
    atomicOr(P.flags, kFlagBadOffsets);
  } else {
    label = end > start ? (float)acc / (float)(end - start) : 0.f;
    const float h = P.head_logit[b];
    // -[label log s + (1 - label) log(1 - s)] = label softplus(-h) + (1 - label) softplus(h): both
    // terms are non-negative, so no cancellation
    loss = label * softplus(-h) + (1.f - label) * softplus(h);
    const float s = 1.f / (1.f + expf(-h));
    dl = (P.grad ? P.grad[b] : 1.f) * (s - label);
  }
  P.accept_full[b] = acc;
  P.label[b] = label;
  P.loss[b] = loss;
  P.dlogit[b] = dl;
}

}  // namespace

hipError_t launch_length_head(const LengthHeadParams& p, hipStream_t s) {
  if (p.n_blocks == 0) return hipSuccess;
  dim3 grid((p.n_blocks + kBlocksPerGroup - 1) / kBlocksPerGroup);
  LengthHeadParams copy = p;
  void* args[] = {&copy};
  return hipLaunchKernel((void*)k_length_head, grid, dim3(kThreads), args, 0, s);
}

}  // namespace opd
