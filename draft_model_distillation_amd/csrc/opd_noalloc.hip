// The fused OPD call for callers that cannot allocate device memory (code under stream capture,
// tight serving loops, harnesses that forbid hipMalloc): opd_fused_fwd_bwd_verify with the
// workspace taken from a fixed device array of this library instead of a caller buffer.
//
// The array lives in the library's code object, one copy per GPU, for as long as the process runs.
// Host code never uses the array's name as an address (in host code it only stands for the device
// symbol): its device address is looked up once per device with hipGetSymbolAddress, with that
// device current, and that pointer is what the kernels receive. Every call on a GPU shares that
// GPU's copy, so calls that overlap on one GPU race (as calls sharing a caller workspace would).

#include <mutex>

#include "opd_internal.h"

// Workspace of the no-allocation entry point: exactly the size of a caller workspace, which covers
// every launch the fused call makes (at most kMaxGrid row-team workgroups).
static __device__ __align__(256) uint8_t scratch[opd::kWorkspaceBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of this GPU's copy of `scratch`, looked up on the first call on the device. The
// first call also zero-fills it on its stream (the workspace contract's initial state) with the
// library's fill kernel; later calls on the device are ordered after it only if they use the same
// stream or the caller orders them (as with any shared workspace).
opd_status_t scratch_for_current_device(hipStream_t stream, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return opd::record_error(OPD_ERR_HIP, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return opd::record_error(OPD_ERR_HIP, "device index out of range");
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      (void)hipGetLastError();
      return opd::record_error(OPD_ERR_HIP, "hipGetSymbolAddress of the no-allocation workspace failed");
    }
    e = opd::launch_fill_u32(static_cast<uint32_t*>(p), 0u, opd::kWorkspaceBytes / sizeof(uint32_t), stream);
    if (e != hipSuccess) return opd::record_error(OPD_ERR_HIP, "zero-filling the no-allocation workspace failed");
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return OPD_OK;
}

}  // namespace

extern "C" opd_status_t opd_fused_fwd_bwd_verify_noalloc(const void* z, const void* y, opd_dtype_t dt, int64_t n_rows,
                                                         int64_t vocab, int64_t ld, const opd_blocks_t* blocks,
                                                         float alpha, float tau, const float* grad_loss, float* loss,
                                                         int32_t* target_top1, int32_t* draft_top1, float* row_stats,
                                                         void* dz, opd_dtype_t dz_dt, int64_t ld_dz,
                                                         int32_t* accept_len, hipStream_t stream) {
  void* ws = nullptr;
  const opd_status_t s = scratch_for_current_device(stream, &ws);
  if (s != OPD_OK) return s;
  return opd_fused_fwd_bwd_verify(z, y, dt, n_rows, vocab, ld, blocks, alpha, tau, grad_loss, loss, target_top1,
                                  draft_top1, row_stats, dz, dz_dt, ld_dz, accept_len, ws, opd::kWorkspaceBytes,
                                  stream);
}
