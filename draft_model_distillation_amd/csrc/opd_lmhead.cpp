// Plain dense products of the lm_head-fused path through rocBLAS: bf16 operands, fp32 accumulation
// and output. These three GEMMs (logits = h W^T, dh = dz W, dW = dz^T h) are ordinary library
// matrix products on the MFMA units; the loss, its gradient and the top-1s between them run in the
// library's own row-team kernel.
//
// One rocBLAS handle per device, created on first use and kept for the life of the process (rocBLAS
// allocates its own device workspace inside it). Atomics are disabled on the handle so that every
// product is reproduced bit for bit. Calls serialise on a mutex while they set the handle's stream
// and enqueue.

#include <rocblas/rocblas.h>

#include <mutex>
#include <string>

#include "opd_internal.h"

namespace opd {
namespace {

std::mutex g_blas_mu;
rocblas_handle g_blas[64] = {};

const char* blas_text(rocblas_status s) { return rocblas_status_to_string(s); }

}  // namespace

opd_status_t gemm_bf16_f32(bool trans_a, bool trans_b, int64_t m, int64_t n, int64_t k, const void* A, int64_t lda,
                           const void* B, int64_t ldb, float beta, float* C, int64_t ldc, hipStream_t stream) {
  if (m <= 0 || n <= 0) return OPD_OK;
  if (m > INT32_MAX || n > INT32_MAX || k > INT32_MAX || lda > INT32_MAX || ldb > INT32_MAX || ldc > INT32_MAX)
    return record_error(OPD_ERR_SHAPE, "matrix product dimensions exceed 32-bit sizes");
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
    return record_error(OPD_ERR_HIP, "hipGetDevice failed for the matrix product");
  std::lock_guard<std::mutex> lk(g_blas_mu);
  rocblas_handle& h = g_blas[dev];
  if (!h) {
    rocblas_status s = rocblas_create_handle(&h);
    if (s != rocblas_status_success) {
      h = nullptr;
      return record_error(OPD_ERR_HIP, (std::string("rocblas_create_handle: ") + blas_text(s)).c_str());
    }
    rocblas_set_atomics_mode(h, rocblas_atomics_not_allowed);
  }
  rocblas_status s = rocblas_set_stream(h, stream);
  if (s != rocblas_status_success)
    return record_error(OPD_ERR_HIP, (std::string("rocblas_set_stream: ") + blas_text(s)).c_str());
  const float alpha = 1.f;
  s = rocblas_gemm_ex(h, trans_a ? rocblas_operation_transpose : rocblas_operation_none,
                      trans_b ? rocblas_operation_transpose : rocblas_operation_none, (rocblas_int)m, (rocblas_int)n,
                      (rocblas_int)k, &alpha, A, rocblas_datatype_bf16_r, (rocblas_int)lda, B, rocblas_datatype_bf16_r,
                      (rocblas_int)ldb, &beta, C, rocblas_datatype_f32_r, (rocblas_int)ldc, C, rocblas_datatype_f32_r,
                      (rocblas_int)ldc, rocblas_datatype_f32_r, rocblas_gemm_algo_standard, 0, 0);
  if (s != rocblas_status_success)
    return record_error(OPD_ERR_HIP, (std::string("rocblas_gemm_ex: ") + blas_text(s)).c_str());
  return OPD_OK;
}

}  // namespace opd
