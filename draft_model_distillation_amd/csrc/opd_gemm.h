// Matrix products of the lm_head-fused path (opd_gemm.hip, planned in opd_lmhead.cpp): declarations
// shared by the host code and the kernels' launcher.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "opd.h"

namespace opd {

// bf16 x bf16 -> fp32 products on the matrix cores (opd_gemm.hip): C[m, n] = sum_k A(m, k) B(k, n)
// (+ beta C). A K-major: A(m, k) = A[m * lda + k]; else A(m, k) = A[k * lda + m]. B K-major:
// B(k, n) = B[n * ldb + k]; else B(k, n) = B[k * ldb + n]. Leading dimensions are multiples of 8, the
// bases 16-byte aligned and each operand smaller than 4 GiB (K-major rows may hold anything past K:
// those values are masked). k_split > 1 splits K over that many workgroup slices whose partial
// products go to `partial` ([k_split][M][ldc] fp32) and are summed in slice order. `stats` (K-major
// operands only) receives per row and per wave column of a tile (kGemmStatParts per 256 columns: max,
// lowest index of it as int bits, sum of exp(c - max)): [M][kGemmStatParts * ceil(N / 256)][3].
constexpr int kGemmWaves = 4;                      // waves per workgroup of the product kernel (8 also built: no faster)
constexpr int kGemmStatParts = kGemmWaves / 2;     // statistics partials per 256-column tile
struct GemmParams {
  const uint16_t* A;
  int64_t lda;
  uint32_t a_bytes;  // extent of A (all rows x lda) in bytes, < 2^32
  const uint16_t* B;
  int64_t ldb;
  uint32_t b_bytes;
  float* C;
  int64_t ldc;
  int M, N, K;
  float beta;
  int k_split;
  int kslice;       // set by launch_gemm
  float* partial;   // k_split > 1
  float* stats;     // nullable
  int m_tiles, n_tiles;  // set by launch_gemm
  int m_major;            // set by launch_gemm: tile order keeps the N tiles of one M tile on one XCD
};
hipError_t launch_gemm(GemmParams p, bool a_kmajor, bool b_kmajor, hipStream_t s);
constexpr int kGemmTile = 256;
// Per-row (max, log-sum-exp) pairs and lowest argmax from the product's statistics partials (either
// output may be NULL).
hipError_t launch_zstats_reduce(const float* part, int n_parts, int M, float* maxlse, int32_t* arg, hipStream_t s);

// C[M, N] (pitch ldc) = sum_k A(m, k) B(k, n) (+ beta C) on the MFMA kernels, layouts as GemmParams
// (opd_lmhead.cpp): checks sizes, pitches and the 32-bit offset limits, then launches. k_split > 1
// needs `partial` (k_split x M x ldc floats; beta is applied in the reduction); `stats` (nullable,
// unsplit both-K-major products only) receives the row-statistics partials, M x kGemmStatParts
// ceil(N / 256) x 3 floats, for launch_zstats_reduce.
opd_status_t gemm_bf16_f32(const uint16_t* A, int64_t lda, bool a_kmajor, const uint16_t* B, int64_t ldb,
                           bool b_kmajor, int64_t M, int64_t N, int64_t K, float beta, float* C, int64_t ldc,
                           int k_split, float* partial, float* stats, hipStream_t stream);

}  // namespace opd
