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

__global__ void __launch_bounds__(kThreads) k_length_head(LengthHeadParams P) {
  const int b = blockIdx.x * kThreads + threadIdx.x;
  if (b >= P.n_blocks) return;
  const int start = P.offsets[b], end = P.offsets[b + 1];
  int acc = 0;
  float label = 0.f, loss = 0.f, dl = 0.f;
  if (start < 0 || end < start || end > P.n_rows) {
    atomicOr(P.flags, kFlagBadOffsets);
  } else {
    while (start + acc < end && P.draft_top1[start + acc] == P.target_top1[start + acc]) ++acc;
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
  dim3 grid((p.n_blocks + kThreads - 1) / kThreads);
  LengthHeadParams copy = p;
  void* args[] = {&copy};
  return hipLaunchKernel((void*)k_length_head, grid, dim3(kThreads), args, 0, s);
}

}  // namespace opd
