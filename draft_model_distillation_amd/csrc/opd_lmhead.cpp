// Host side of the lm_head-fused path's matrix products: argument checks and launch planning for the
// library's own bf16 MFMA kernels (opd_gemm.hip). The three products of a chunk of rows are
//   logits  z  = h W^T       (M rows, N vocab, K hidden; both operands K-major)
//   dh         = dz W        (M rows, N hidden, K vocab; dz K-major, W N-major; split over K)
//   dW        (+)= dz^T h    (M vocab, N hidden, K rows; both operands M/N-major)
// that the OPD loss of "AdaFlash: Adaptive Speculative Decoding with Online Self-Improvement for
// High-Concurrency LLM Inference", section "1. On-Policy Distillation (OPD) for Domain Adaptation",
// needs when the drafter's vocabulary projection is trained with it.

#include <string>

#include "opd_gemm.h"
#include "opd_internal.h"

namespace opd {
namespace {

constexpr int64_t kTile = kGemmTile;  // rows (or columns) of one workgroup tile
constexpr int64_t kKStep = 64;        // K step of the kernels (and granule of a K slice)

int64_t round_up64(int64_t a, int64_t b) { return (a + b - 1) / b * b; }

// Largest byte offset the kernel can form for an operand (including the rows or k-rows that a last
// tile or step reaches past the matrix, which read as zero); buffer offsets are 32-bit.
bool offsets_fit(bool kmajor, int64_t rows, int64_t K, int64_t ld) {
  const int64_t reach = kmajor ? round_up64(rows, kTile) + kTile : round_up64(K, kKStep) + kKStep;
  return reach * ld * 2 < (int64_t)UINT32_MAX;
}

}  // namespace

opd_status_t gemm_bf16_f32(const uint16_t* A, int64_t lda, bool a_kmajor, const uint16_t* B, int64_t ldb,
                           bool b_kmajor, int64_t M, int64_t N, int64_t K, float beta, float* C, int64_t ldc,
                           int k_split, float* partial, float* stats, hipStream_t stream) {
  if (M <= 0 || N <= 0) return OPD_OK;
  if (M > INT32_MAX || N > INT32_MAX || K > INT32_MAX || K < 0)
    return record_error(OPD_ERR_SHAPE, "matrix product dimensions exceed 32-bit sizes");
  if ((a_kmajor && lda < K) || (!a_kmajor && lda < M) || (b_kmajor && ldb < K) || (!b_kmajor && ldb < N) || ldc < N)
    return record_error(OPD_ERR_SHAPE, "matrix product leading dimension smaller than the matrix");
  if (lda % 8 || ldb % 8) return record_error(OPD_ERR_ALIGN, "bf16 operand pitches must be multiples of 8");
  if (!offsets_fit(a_kmajor, M, K, lda) || !offsets_fit(b_kmajor, N, K, ldb))
    return record_error(OPD_ERR_SHAPE, "an operand of the matrix product spans 4 GiB or more (32-bit buffer offsets)");
  if (kTile * ldc * 4 >= (int64_t)UINT32_MAX)
    return record_error(OPD_ERR_SHAPE, "output pitch too large for 32-bit offsets within a tile");
  if (k_split < 1) k_split = 1;
  if (k_split > 1 && !partial) return record_error(OPD_ERR_WORKSPACE, "split product without partial buffer");
  if (stats && (!a_kmajor || !b_kmajor || k_split > 1 || beta != 0.f))
    return record_error(OPD_ERR_PARAM, "row statistics only for the unsplit logits product");
  GemmParams p{};
  p.A = A;
  p.lda = lda;
  p.a_bytes = (uint32_t)((a_kmajor ? M : K) * lda * 2);
  p.B = B;
  p.ldb = ldb;
  p.b_bytes = (uint32_t)((b_kmajor ? N : K) * ldb * 2);
  p.C = C;
  p.ldc = ldc;
  p.M = (int)M;
  p.N = (int)N;
  p.K = (int)K;
  p.beta = beta;
  p.k_split = k_split;
  p.partial = partial;
  p.stats = stats;
  hipError_t e = launch_gemm(p, a_kmajor, b_kmajor, stream);
  if (e != hipSuccess)
    return record_error(OPD_ERR_HIP, (std::string("matrix product launch: ") + hipGetErrorString(e)).c_str());
  return OPD_OK;
}

}  // namespace opd
