// C-ABI entry points of the OPD loss / gradient / verify library (declared in include/opd.h).
//
// Host-side responsibilities: validate every argument before any HIP call, choose the launch
// geometry (workgroups per row, rows in flight) from the device's occupancy, hand out the unique
// exchange flags each launch needs, and enqueue the kernels on the caller's stream.

#include "opd.h"

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <unordered_map>

#include "opd_gemm.h"
#include "opd_internal.h"

static_assert(OPD_FLAG_NEG_L == opd::kFlagNegL, "flag mismatch");
static_assert(OPD_FLAG_BAD_OFFSETS == opd::kFlagBadOffsets, "flag mismatch");
static_assert(OPD_FLAG_SPIN_TIMEOUT == opd::kFlagSpinTimeout, "flag mismatch");
static_assert(OPD_FLAG_BAD_TOKEN == opd::kFlagBadToken, "flag mismatch");

namespace {

thread_local std::string g_last_error;
std::atomic<uint32_t> g_spin_limit{0};

// Host-chosen exchange flags: offsets into [2^31, 2^32). When the range is used up it restarts at
// its bottom and the generation count goes up; a workspace last used in an earlier generation may
// hold units whose flags the new range hands out again, so its units are zeroed before its next
// launch. Workspaces are tracked by address.
std::mutex g_flag_mu;
uint32_t g_flag_next = 0;
uint64_t g_flag_gen = 0;
std::unordered_map<const void*, uint64_t> g_ws_gen;

// Check mode (OPD_CHECK=1 in the environment, or opd_set_check): every call synchronises its stream,
// reads the workspace's sticky flag word and returns OPD_ERR_DEVICE if a bit is set.
std::atomic<int> g_check{-1};

constexpr int64_t kMaxVocab = opd::kMaxVocab;

opd_status_t fail(opd_status_t s, const std::string& msg) {
  g_last_error = msg;
  return s;
}

opd_status_t hip_fail(hipError_t e, const char* where) {
  g_last_error = std::string(where) + ": " + hipGetErrorString(e);
  return OPD_ERR_HIP;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t dtype_size(opd_dtype_t dt) { return dt == OPD_F32 ? 4 : 2; }

bool valid_dtype(opd_dtype_t dt) { return dt == OPD_F32 || dt == OPD_BF16; }

opd_status_t check_logits(const void* z, const void* y, opd_dtype_t dt, int64_t n_rows, int64_t vocab,
                          int64_t ld) {
  if (n_rows > 0 && (!z || !y)) return fail(OPD_ERR_NULL, "z and y must be non-NULL");
  if (!valid_dtype(dt)) return fail(OPD_ERR_DTYPE, "logit dtype must be OPD_F32 or OPD_BF16");
  if (n_rows < 0 || n_rows > INT32_MAX) return fail(OPD_ERR_SHAPE, "n_rows out of range");
  if (vocab <= 0 || vocab > kMaxVocab) return fail(OPD_ERR_SHAPE, "vocab must be in [1, 524288]");
  if (ld < vocab) return fail(OPD_ERR_SHAPE, "ld must be >= vocab");
  if (!aligned16(z) || !aligned16(y)) return fail(OPD_ERR_ALIGN, "z and y must be 16-byte aligned");
  if ((ld * (int64_t)dtype_size(dt)) % 16 != 0) return fail(OPD_ERR_ALIGN, "row pitch must be a multiple of 16 bytes");
  return OPD_OK;
}

opd_status_t check_params(float alpha, float tau) {
  if (std::isnan(alpha) || alpha < 0.f || alpha > 1.f) return fail(OPD_ERR_PARAM, "alpha must be in [0, 1]");
  if (std::isnan(tau)) return fail(OPD_ERR_PARAM, "tau must not be NaN");
  return OPD_OK;
}

opd_status_t check_ws(void* ws, size_t ws_bytes) {
  if (!ws || ws_bytes < opd::kWorkspaceBytes) return fail(OPD_ERR_WORKSPACE, "workspace missing or too small");
  if (!aligned16(ws)) return fail(OPD_ERR_ALIGN, "workspace must be 16-byte aligned");
  return OPD_OK;
}

opd_status_t check_dz(const void* dz, opd_dtype_t dz_dt, int64_t n_rows, int64_t vocab, int64_t ld_dz) {
  if (n_rows > 0 && !dz) return fail(OPD_ERR_NULL, "dz must be non-NULL");
  if (!valid_dtype(dz_dt)) return fail(OPD_ERR_DTYPE, "dz dtype must be OPD_F32 or OPD_BF16");
  if (ld_dz < vocab) return fail(OPD_ERR_SHAPE, "ld_dz must be >= vocab");
  if (!aligned16(dz)) return fail(OPD_ERR_ALIGN, "dz must be 16-byte aligned");
  if ((ld_dz * (int64_t)dtype_size(dz_dt)) % 16 != 0) return fail(OPD_ERR_ALIGN, "dz row pitch must be a multiple of 16 bytes");
  return OPD_OK;
}

opd_status_t check_blocks(const opd_blocks_t* blocks, bool required) {
  if (!blocks) return required ? fail(OPD_ERR_NULL, "blocks must be non-NULL") : OPD_OK;
  if (blocks->n_blocks < 0) return fail(OPD_ERR_SHAPE, "n_blocks must be >= 0");
  if (blocks->n_blocks > 0 && (!blocks->offsets || !blocks->L)) return fail(OPD_ERR_NULL, "blocks arrays must be non-NULL");
  return OPD_OK;
}

// Occupancy (workgroups per CU) of each team-kernel variant and the CU count, per device.
struct DeviceInfo {
  int cus = 0;
  int occ[3][2][2][3][2] = {};  // mode, in_bf16, out_bf16, K index (1, 3, 5), device-epoch flags
};
std::mutex g_dev_mu;
DeviceInfo g_dev[64];

opd_status_t device_info(int mode, int in_bf16, int out_bf16, int kidx, int K, int dev_flags, int* cus, int* occ) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= 64) return fail(OPD_ERR_HIP, "device index out of range");
  std::lock_guard<std::mutex> lk(g_dev_mu);
  DeviceInfo& d = g_dev[dev];
  if (d.cus == 0) {
    int n = 0;
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
    d.cus = n;
  }
  int& o = d.occ[mode][in_bf16][out_bf16][kidx][dev_flags];
  if (o == 0) {
    int n = 0;
    e = opd::team_occupancy(mode, in_bf16, out_bf16, K, dev_flags != 0, &n);
    if (e != hipSuccess) return hip_fail(e, "hipOccupancyMaxActiveBlocksPerMultiprocessor");
    if (n <= 0) return fail(OPD_ERR_HIP, "kernel cannot be resident");
    o = n;
  }
  *cus = d.cus;
  *occ = o;
  return OPD_OK;
}

struct Geometry {
  int K, G, chunk_vec, nvec, n_teams, grid;
};

// Workgroups per row (team size) and vectors per chunk for K slots per thread.
int team_geometry(int K, int nvec, int* chunk_vec) {
  const int slots = opd::kThreads * K;
  int G = (nvec + slots - 1) / slots;
  int chunk = (nvec + G - 1) / G;
  chunk = ((chunk + 7) / 8) * 8;  // chunk boundaries on 128-byte lines
  if (chunk > slots) chunk = slots;
  if (chunk_vec) *chunk_vec = chunk;
  return (nvec + chunk - 1) / chunk;
}

// Split a row of nvec 16-byte vectors over G workgroups of 256 threads x K slots each, and choose
// how many rows (teams) are in flight so that the whole grid is co-resident.
opd_status_t plan_k(int mode, int in_bf16, int out_bf16, int dev_flags, int K, int nvec, int64_t n_rows, Geometry* g) {
  const int kidx = K == 1 ? 0 : K == 3 ? 1 : 2;
  int chunk = 0;
  const int G = team_geometry(K, nvec, &chunk);
  if (G > opd::kMaxTeamSize) return fail(OPD_ERR_SHAPE, "vocab too large for one team");
  int cus = 0, occ = 0;
  opd_status_t s = device_info(mode, in_bf16, out_bf16, kidx, K, dev_flags, &cus, &occ);
  if (s != OPD_OK) return s;
  int64_t capacity = (int64_t)cus * occ;
  if (capacity > opd::kMaxGrid) capacity = opd::kMaxGrid;
  int64_t max_teams = capacity / G;
  if (max_teams < 1) return fail(OPD_ERR_SHAPE, "row too wide for the device");
  int64_t teams = n_rows < max_teams ? n_rows : max_teams;
  g->K = K;
  g->G = G;
  g->chunk_vec = chunk;
  g->nvec = nvec;
  g->n_teams = (int)teams;
  g->grid = (int)(teams * G);
  return OPD_OK;
}

// Five slots per thread (the fewest workgroups per row, so the most rows in flight) unless a whole
// batch fits the teams of the three-slot plan at once: then every row starts immediately either
// way, and the shorter chunks finish sooner (a 16-row decode at V = 151,936: 14.3 against 15.1 us
// per call). Rows of at most 256 vectors take one slot per thread.
opd_status_t plan(int mode, int in_bf16, int out_bf16, int dev_flags, int64_t n_rows, int64_t vocab, Geometry* g) {
  const int epv = in_bf16 ? 8 : 4;
  const int nvec = (int)((vocab + epv - 1) / epv);
  if (nvec <= opd::kThreads) return plan_k(mode, in_bf16, out_bf16, dev_flags, 1, nvec, n_rows, g);
  // (the three-slot plan only where its team fits: fp32 rows past 393,216 logits need five slots)
  if (team_geometry(3, nvec, nullptr) <= opd::kMaxTeamSize) {
    opd_status_t s = plan_k(mode, in_bf16, out_bf16, dev_flags, 3, nvec, n_rows, g);
    if (s != OPD_OK) return s;
    if (g->n_teams >= n_rows) return OPD_OK;
  }
  return plan_k(mode, in_bf16, out_bf16, dev_flags, 5, nvec, n_rows, g);
}

// Exchange flags for an eager launch: a fresh range in [2^31 + 1, 2^32), disjoint from the device
// epoch's range [1, 2^31) that captured launches use, so the two kinds never take each other's
// units for their own. Returns the base (first flag minus 1); *must_clear is set when the workspace
// was last used before the range restarted (its units must be zeroed before this launch).
uint32_t reserve_host_flags(const void* ws, uint32_t count, bool* must_clear) {
  std::lock_guard<std::mutex> lk(g_flag_mu);
  if ((uint64_t)g_flag_next + count >= 0x80000000ull) {
    g_flag_next = 0;
    ++g_flag_gen;
  }
  const uint32_t base = 0x80000000u + g_flag_next;
  g_flag_next += count;
  auto it = g_ws_gen.find(ws);
  *must_clear = it != g_ws_gen.end() && it->second != g_flag_gen;
  g_ws_gen[ws] = g_flag_gen;  // a workspace seen for the first time is zero-filled by contract
  return base;
}

bool check_mode() {
  int v = g_check.load();
  if (v < 0) {
    const char* e = std::getenv("OPD_CHECK");
    v = (e && *e && std::strcmp(e, "0") != 0) ? 1 : 0;
    int expected = -1;
    g_check.compare_exchange_strong(expected, v);
    v = g_check.load();
  }
  return v != 0;
}

std::string flag_text(uint32_t f) {
  std::string t;
  if (f & OPD_FLAG_NEG_L) t += " negative L;";
  if (f & OPD_FLAG_BAD_OFFSETS) t += " malformed offsets;";
  if (f & OPD_FLAG_SPIN_TIMEOUT) t += " cross-workgroup wait timed out (outputs invalid);";
  if (f & OPD_FLAG_BAD_TOKEN) t += " proposal outside the vocabulary;";
  return t;
}

// True unless the stream is known not to be capturing: a captured launch takes its flags from the
// device epoch (kernel arguments are frozen for every replay of a graph).
bool stream_may_be_captured(hipStream_t stream) {
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &st) != hipSuccess) {
    (void)hipGetLastError();
    return true;
  }
  return st != hipStreamCaptureStatusNone;
}

uint32_t spin_limit() {
  uint32_t v = g_spin_limit.load();
  return v ? v : opd::kDefaultSpinLimit;
}

opd_status_t run_team(int mode, const void* z, const void* y, opd_dtype_t dt, int64_t n_rows, int64_t vocab,
                      int64_t ld, float alpha, float tau, const float* grad_loss, float* loss, int32_t* target_top1,
                      int32_t* draft_top1, float* row_stats, void* dz, opd_dtype_t dz_dt, int64_t ld_dz, void* ws,
                      hipStream_t stream) {
  if (n_rows == 0) return OPD_OK;
  const int in_bf16 = dt == OPD_BF16;
  const int out_bf16 = (mode == opd::kFused && dz_dt == OPD_BF16) ? 1 : 0;
  // a launch that may be captured into a graph takes its exchange flags from the workspace epoch
  const int dev_flags = stream_may_be_captured(stream) ? 1 : 0;
  Geometry g;
  opd_status_t s = plan(mode, in_bf16, out_bf16, dev_flags, n_rows, vocab, &g);
  if (s != OPD_OK) return s;
  opd::TeamParams p;
  std::memset(&p, 0, sizeof(p));
  p.z = static_cast<const uint8_t*>(z);
  p.y = static_cast<const uint8_t*>(y);
  p.ld_bytes = ld * (int64_t)dtype_size(dt);
  p.vocab = (int32_t)vocab;
  p.nvec = g.nvec;
  p.n_rows = (int32_t)n_rows;
  p.G = g.G;
  p.chunk_vec = g.chunk_vec;
  p.n_teams = g.n_teams;
  p.alpha = alpha;
  p.tau = tau;
  p.grad_loss = grad_loss;
  p.loss = loss;
  p.target_top1 = target_top1;
  p.draft_top1 = draft_top1;
  p.row_stats = row_stats;
  p.dz = static_cast<uint8_t*>(dz);
  p.ld_dz_bytes = ld_dz * (int64_t)dtype_size(dz_dt);
  p.units = reinterpret_cast<uint64_t*>(static_cast<uint8_t*>(ws) + opd::kHeaderBytes);
  p.flags = static_cast<uint32_t*>(ws);
  if ((size_t)g.grid * opd::kUnitBytesPerWg > opd::kWorkspaceBytes - opd::kHeaderBytes)
    return fail(OPD_ERR_WORKSPACE, "launch needs more exchange units than the workspace holds");
  const int64_t iters = (n_rows + g.n_teams - 1) / g.n_teams;
  if (2 * iters + 2 > 0x3fffffff) return fail(OPD_ERR_SHAPE, "too many rows");
  p.flag_count = (uint32_t)(2 * iters + 2);
  bool clear = false;
  p.flag_base = dev_flags ? 0u : reserve_host_flags(ws, p.flag_count, &clear);
  p.spin_limit = spin_limit();
  hipError_t e = hipSuccess;
  if (clear) {  // the host range restarted since this workspace was last used: zero its units
    e = opd::launch_fill_u32(reinterpret_cast<uint32_t*>(p.units), 0u,
                             (opd::kWorkspaceBytes - opd::kHeaderBytes) / sizeof(uint32_t), stream);
    if (e != hipSuccess) return hip_fail(e, "clearing the exchange units");
  }
  e = opd::launch_team(p, mode, in_bf16, out_bf16, g.K, g.grid, stream);
  if (e != hipSuccess) return hip_fail(e, "team kernel launch");
  return OPD_OK;
}

opd_status_t run_accept(const opd_blocks_t* blocks, int64_t n_rows, const int32_t* draft_top1,
                        const int32_t* target_top1, int32_t* accept_len, void* ws, hipStream_t stream) {
  if (!blocks || blocks->n_blocks == 0) return OPD_OK;
  opd::AcceptParams a;
  a.draft_top1 = draft_top1;
  a.target_top1 = target_top1;
  a.offsets = blocks->offsets;
  a.L = blocks->L;
  a.n_blocks = blocks->n_blocks;
  a.n_rows = (int32_t)n_rows;
  a.accept_len = accept_len;
  a.flags = static_cast<uint32_t*>(ws);
  hipError_t e = opd::launch_accept(a, stream);
  if (e != hipSuccess) return hip_fail(e, "accept kernel launch");
  return OPD_OK;
}

// Check mode: once a call's work is enqueued, synchronise the stream, read the sticky flag word and
// report a set bit as OPD_ERR_DEVICE (the word is then cleared). Skipped for a stream that is being
// captured (it cannot be synchronised); launch errors surfaced by the synchronisation are OPD_ERR_HIP.
opd_status_t finish(opd_status_t s, void* ws, hipStream_t stream) {
  if (s != OPD_OK || !ws || !check_mode()) return s;
  if (stream_may_be_captured(stream)) return s;
  uint32_t v = 0;
  hipError_t e = hipMemcpyAsync(&v, ws, sizeof(v), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e, "check mode: reading the device flags");
  if (v == 0) return OPD_OK;
  e = opd::launch_fill_u32(static_cast<uint32_t*>(ws), 0u, 1, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e, "check mode: clearing the device flags");
  char head[40];
  std::snprintf(head, sizeof(head), "device flags 0x%x:", v);
  return fail(OPD_ERR_DEVICE, std::string(head) + flag_text(v));
}

}  // namespace

namespace opd {
opd_status_t record_error(opd_status_t s, const char* msg) { return fail(s, msg); }
}  // namespace opd

extern "C" {

size_t opd_workspace_size(void) { return opd::kWorkspaceBytes; }

static opd_status_t opd_loss_fwd_impl(const void* z, const void* y, opd_dtype_t dt, int64_t n_rows, int64_t vocab, int64_t ld,
                          float alpha, float tau, float* loss, int32_t* target_top1, int32_t* draft_top1,
                          float* row_stats, void* ws, size_t ws_bytes, hipStream_t stream) {
  opd_status_t s = check_logits(z, y, dt, n_rows, vocab, ld);
  if (s != OPD_OK) return s;
  if (n_rows > 0 && (!loss || !target_top1 || !row_stats))
    return fail(OPD_ERR_NULL, "loss, target_top1 and row_stats must be non-NULL");
  if ((s = check_params(alpha, tau)) != OPD_OK) return s;
  if ((s = check_ws(ws, ws_bytes)) != OPD_OK) return s;
  return run_team(opd::kForward, z, y, dt, n_rows, vocab, ld, alpha, tau, nullptr, loss, target_top1, draft_top1,
                  row_stats, nullptr, OPD_F32, vocab, ws, stream);
}

static opd_status_t opd_loss_bwd_impl(const void* z, const void* y, opd_dtype_t dt, int64_t n_rows, int64_t vocab, int64_t ld,
                          float alpha, float tau, const float* row_stats, const int32_t* target_top1,
                          const float* grad_loss, void* dz, opd_dtype_t dz_dt, int64_t ld_dz, void* ws,
                          size_t ws_bytes, hipStream_t stream) {
  opd_status_t s = check_logits(z, y, dt, n_rows, vocab, ld);
  if (s != OPD_OK) return s;
  if (n_rows > 0 && (!row_stats || !target_top1))
    return fail(OPD_ERR_NULL, "row_stats and target_top1 must be non-NULL");
  if ((s = check_dz(dz, dz_dt, n_rows, vocab, ld_dz)) != OPD_OK) return s;
  if ((s = check_params(alpha, tau)) != OPD_OK) return s;
  if ((s = check_ws(ws, ws_bytes)) != OPD_OK) return s;
  if (n_rows == 0) return OPD_OK;
  opd::BwdParams p;
  p.z = static_cast<const uint8_t*>(z);
  p.y = static_cast<const uint8_t*>(y);
  p.ld_bytes = ld * (int64_t)dtype_size(dt);
  p.vocab = (int32_t)vocab;
  p.nvec = (int32_t)((vocab + (dt == OPD_BF16 ? 8 : 4) - 1) / (dt == OPD_BF16 ? 8 : 4));
  p.n_rows = (int32_t)n_rows;
  p.alpha = alpha;
  p.tau = tau;
  p.row_stats = row_stats;
  p.target_top1 = target_top1;
  p.grad_loss = grad_loss;
  p.dz = static_cast<uint8_t*>(dz);
  p.ld_dz_bytes = ld_dz * (int64_t)dtype_size(dz_dt);
  if (n_rows > 65535) {
    // the backward grid uses blockIdx.y for the row: launch in slabs of 65535 rows
    for (int64_t r0 = 0; r0 < n_rows; r0 += 65535) {
      opd::BwdParams q = p;
      const int64_t nr = (n_rows - r0) < 65535 ? (n_rows - r0) : 65535;
      q.z = p.z + r0 * p.ld_bytes;
      q.y = p.y + r0 * p.ld_bytes;
      q.dz = p.dz + r0 * p.ld_dz_bytes;
      q.row_stats = p.row_stats + 8 * r0;
      q.target_top1 = p.target_top1 + r0;
      q.grad_loss = p.grad_loss ? p.grad_loss + r0 : nullptr;
      q.n_rows = (int32_t)nr;
      hipError_t e = opd::launch_bwd(q, dt == OPD_BF16, dz_dt == OPD_BF16, stream);
      if (e != hipSuccess) return hip_fail(e, "backward kernel launch");
    }
    return OPD_OK;
  }
  hipError_t e = opd::launch_bwd(p, dt == OPD_BF16, dz_dt == OPD_BF16, stream);
  if (e != hipSuccess) return hip_fail(e, "backward kernel launch");
  return OPD_OK;
}

static opd_status_t verify_accept_len_impl(const void* z, const void* y, opd_dtype_t dt, int64_t n_rows, int64_t vocab,
                               int64_t ld, const opd_blocks_t* blocks, int32_t* target_top1, int32_t* draft_top1,
                               int32_t* accept_len, void* ws, size_t ws_bytes, hipStream_t stream) {
  opd_status_t s = check_logits(z, y, dt, n_rows, vocab, ld);
  if (s != OPD_OK) return s;
  if ((s = check_blocks(blocks, true)) != OPD_OK) return s;
  if (n_rows > 0 && (!target_top1 || !draft_top1)) return fail(OPD_ERR_NULL, "top-1 outputs must be non-NULL");
  if (blocks->n_blocks > 0 && !accept_len) return fail(OPD_ERR_NULL, "accept_len must be non-NULL");
  if ((s = check_ws(ws, ws_bytes)) != OPD_OK) return s;
  s = run_team(opd::kTop1, z, y, dt, n_rows, vocab, ld, 0.5f, 0.f, nullptr, nullptr, target_top1, draft_top1,
               nullptr, nullptr, OPD_F32, vocab, ws, stream);
  if (s != OPD_OK) return s;
  return run_accept(blocks, n_rows, draft_top1, target_top1, accept_len, ws, stream);
}

static opd_status_t opd_fused_fwd_bwd_verify_impl(const void* z, const void* y, opd_dtype_t dt, int64_t n_rows, int64_t vocab,
                                      int64_t ld, const opd_blocks_t* blocks, float alpha, float tau,
                                      const float* grad_loss, float* loss, int32_t* target_top1, int32_t* draft_top1,
                                      float* row_stats, void* dz, opd_dtype_t dz_dt, int64_t ld_dz,
                                      int32_t* accept_len, void* ws, size_t ws_bytes, hipStream_t stream) {
  opd_status_t s = check_logits(z, y, dt, n_rows, vocab, ld);
  if (s != OPD_OK) return s;
  if ((s = check_blocks(blocks, false)) != OPD_OK) return s;
  if (n_rows > 0 && (!loss || !target_top1 || !row_stats))
    return fail(OPD_ERR_NULL, "loss, target_top1 and row_stats must be non-NULL");
  if (blocks && blocks->n_blocks > 0 && (!accept_len || (n_rows > 0 && !draft_top1)))
    return fail(OPD_ERR_NULL, "draft_top1 and accept_len are required when blocks are given");
  if ((s = check_dz(dz, dz_dt, n_rows, vocab, ld_dz)) != OPD_OK) return s;
  if ((s = check_params(alpha, tau)) != OPD_OK) return s;
  if ((s = check_ws(ws, ws_bytes)) != OPD_OK) return s;
  s = run_team(opd::kFused, z, y, dt, n_rows, vocab, ld, alpha, tau, grad_loss, loss, target_top1, draft_top1,
               row_stats, dz, dz_dt, ld_dz, ws, stream);
  if (s != OPD_OK) return s;
  return run_accept(blocks, n_rows, draft_top1, target_top1, accept_len, ws, stream);
}

static opd_status_t opd_length_head_loss_impl(const int32_t* target_top1, const int32_t* draft_top1, int64_t n_rows,
                                  const int32_t* offsets, int32_t n_blocks, const float* head_logit,
                                  const float* grad, int32_t* accept_full, float* label, float* loss,
                                  float* dlogit, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (n_rows < 0 || n_rows > INT32_MAX) return fail(OPD_ERR_SHAPE, "n_rows out of range");
  if (n_blocks < 0) return fail(OPD_ERR_SHAPE, "n_blocks must be >= 0");
  if (n_blocks == 0) return OPD_OK;
  if (!offsets || !head_logit || !accept_full || !label || !loss || !dlogit)
    return fail(OPD_ERR_NULL, "offsets, head_logit and the four outputs must be non-NULL");
  if (n_rows > 0 && (!target_top1 || !draft_top1)) return fail(OPD_ERR_NULL, "top-1 inputs must be non-NULL");
  opd_status_t s = check_ws(ws, ws_bytes);
  if (s != OPD_OK) return s;
  opd::LengthHeadParams p;
  p.draft_top1 = draft_top1;
  p.target_top1 = target_top1;
  p.offsets = offsets;
  p.n_blocks = n_blocks;
  p.n_rows = (int32_t)n_rows;
  p.head_logit = head_logit;
  p.grad = grad;
  p.accept_full = accept_full;
  p.label = label;
  p.loss = loss;
  p.dlogit = dlogit;
  p.flags = static_cast<uint32_t*>(ws);
  hipError_t e = opd::launch_length_head(p, stream);
  if (e != hipSuccess) return hip_fail(e, "length-head kernel launch");
  return OPD_OK;
}

static opd_status_t opd_verify_sample_impl(const void* z, const void* y, opd_dtype_t dt, int64_t n_rows, int64_t vocab,
                               int64_t ld, const opd_blocks_t* blocks, const int32_t* draft_tokens,
                               const float* u_accept, const float* u_resample, float temperature,
                               int32_t* accept_len, int32_t* out_token, float* row_lse, void* ws,
                               size_t ws_bytes, hipStream_t stream) {
  opd_status_t s = check_logits(z, y, dt, n_rows, vocab, ld);
  if (s != OPD_OK) return s;
  if ((s = check_blocks(blocks, true)) != OPD_OK) return s;
  if (!(temperature > 0.f) || std::isinf(temperature))
    return fail(OPD_ERR_PARAM, "temperature must be positive and finite");
  // fp32 must hold log2(e) / T (and scaled logits of |z| <= 1e4) without overflow
  if (temperature < 1e-6f) return fail(OPD_ERR_PARAM, "temperature must be >= 1e-6");
  if (n_rows > 0 && (!draft_tokens || !u_accept || !row_lse))
    return fail(OPD_ERR_NULL, "draft_tokens, u_accept and row_lse must be non-NULL");
  if (blocks->n_blocks > 0 && (!u_resample || !accept_len || !out_token))
    return fail(OPD_ERR_NULL, "u_resample, accept_len and out_token must be non-NULL");
  if ((s = check_ws(ws, ws_bytes)) != OPD_OK) return s;
  if (n_rows == 0 && blocks->n_blocks == 0) return OPD_OK;
  const int in_bf16 = dt == OPD_BF16;
  const int epv = in_bf16 ? 8 : 4;
  opd::SampleParams p;
  p.z = static_cast<const uint8_t*>(z);
  p.y = static_cast<const uint8_t*>(y);
  p.ld_bytes = ld * (int64_t)dtype_size(dt);
  p.vocab = (int32_t)vocab;
  p.nvec = (int32_t)((vocab + epv - 1) / epv);
  p.n_rows = (int32_t)n_rows;
  p.n_blocks = blocks->n_blocks;
  p.c = (float)(1.4426950408889634 / (double)temperature);
  p.offsets = blocks->offsets;
  p.L = blocks->L;
  p.draft = draft_tokens;
  p.u_accept = u_accept;
  p.u_resample = u_resample;
  p.stats = row_lse;
  p.accept_len = accept_len;
  p.token = out_token;
  p.flags = static_cast<uint32_t*>(ws);
  p.slices = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + opd::kHeaderBytes);
  p.block0 = 0;
  hipError_t e = opd::launch_sample_verify(p, in_bf16, stream);
  if (e != hipSuccess) return hip_fail(e, "sampling-verify kernel launch");
  return OPD_OK;
}

static int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

size_t opd_lmhead_scratch_size(int64_t chunk_rows, int64_t vocab, int64_t ld_y) {
  if (chunk_rows <= 0 || vocab <= 0 || ld_y < vocab) return 0;
  // logits chunk: fp32 with the pitch of y (the row kernel reads both with one pitch); dz chunk: bf16,
  // a region that first holds the logits product's row-statistics partials (3 floats per row and
  // wave column of a 256-column tile)
  const int64_t zb = round_up(chunk_rows * ld_y * 4, 256);
  const int64_t parts = opd::kGemmStatParts * ((vocab + opd::kGemmTile - 1) / opd::kGemmTile);
  const int64_t db = round_up(std::max(chunk_rows * round_up(vocab, 8) * 2, chunk_rows * parts * 12), 256);
  return (size_t)(zb + db);
}

static opd_status_t opd_lmhead_fused_fwd_bwd_verify_impl(const void* h, const void* W, int64_t hidden, const void* y,
                                             opd_dtype_t dt_y, int64_t n_rows, int64_t vocab, int64_t ld_y,
                                             const opd_blocks_t* blocks, float alpha, float tau,
                                             const float* grad_loss, float* loss, int32_t* target_top1,
                                             int32_t* draft_top1, float* row_stats, float* dh, float* dW,
                                             float* logit_max_lse, int32_t* logit_argmax, int32_t* accept_len,
                                             void* scratch, size_t scratch_bytes, int64_t chunk_rows, void* ws,
                                             size_t ws_bytes, hipStream_t stream) {
  opd_status_t s = check_logits(y, y, dt_y, n_rows, vocab, ld_y);
  if (s != OPD_OK) return s;
  if (dt_y != OPD_F32) return fail(OPD_ERR_DTYPE, "y must be fp32 (the logits chunk it is paired with is fp32)");
  if (hidden <= 0 || hidden > INT32_MAX) return fail(OPD_ERR_SHAPE, "hidden must be in [1, 2^31)");
  if (hidden % 8) return fail(OPD_ERR_ALIGN, "hidden must be a multiple of 8 (16-byte bf16 rows)");
  if (vocab > 0 && (!W || (n_rows > 0 && !h))) return fail(OPD_ERR_NULL, "h and W must be non-NULL");
  if (n_rows > 0 && (!loss || !target_top1 || !row_stats))
    return fail(OPD_ERR_NULL, "loss, target_top1 and row_stats must be non-NULL");
  if (!aligned16(h) || !aligned16(W) || !aligned16(dh) || !aligned16(dW))
    return fail(OPD_ERR_ALIGN, "h, W, dh and dW must be 16-byte aligned");
  if ((s = check_blocks(blocks, false)) != OPD_OK) return s;
  if (blocks && blocks->n_blocks > 0 && !accept_len) return fail(OPD_ERR_NULL, "accept_len must be non-NULL");
  if ((s = check_params(alpha, tau)) != OPD_OK) return s;
  if ((s = check_ws(ws, ws_bytes)) != OPD_OK) return s;
  if (chunk_rows <= 0) return fail(OPD_ERR_SHAPE, "chunk_rows must be >= 1");
  if (n_rows > 0 && !draft_top1 && blocks && blocks->n_blocks > 0)
    return fail(OPD_ERR_NULL, "draft_top1 is needed for verification");
  const int64_t rc_max = chunk_rows < n_rows ? chunk_rows : n_rows;
  if (n_rows == 0) {
    if (dW && vocab > 0) {  // no rows: the gradient of the projection is zero
      hipError_t e = opd::launch_fill_u32(reinterpret_cast<uint32_t*>(dW), 0u, (size_t)vocab * hidden, stream);
      if (e != hipSuccess) return hip_fail(e, "clearing dW");
    }
    return run_accept(blocks, 0, draft_top1, target_top1, accept_len, ws, stream);
  }
  if (!scratch || scratch_bytes < opd_lmhead_scratch_size(rc_max, vocab, ld_y))
    return fail(OPD_ERR_WORKSPACE, "scratch missing or smaller than opd_lmhead_scratch_size()");
  if (!aligned16(scratch)) return fail(OPD_ERR_ALIGN, "scratch must be 16-byte aligned");
  const int64_t ld_dz = round_up(vocab, 8);
  float* zc = static_cast<float*>(scratch);
  uint16_t* dzc = reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(scratch) + round_up(rc_max * ld_y * 4, 256));
  // The dz region holds the logits product's row-statistics partials until the row kernel writes dz
  // (rc x kGemmStatParts ceil(V / 256) x 3 floats, well under rc x ld_dz bf16), and the logits region holds the
  // split dh product's partials once the row kernel has read the logits (k_split x rc x hidden floats).
  float* zstats = reinterpret_cast<float*>(dzc);
  const bool want_stats = logit_max_lse || logit_argmax;
  const int n_parts = opd::kGemmStatParts * (int)((vocab + opd::kGemmTile - 1) / opd::kGemmTile);
  const uint16_t* Wb = static_cast<const uint16_t*>(W);
  const uint8_t* hb = static_cast<const uint8_t*>(h);
  const uint8_t* yb = static_cast<const uint8_t*>(y);
  for (int64_t r0 = 0; r0 < n_rows; r0 += chunk_rows) {
    const int64_t rc = (n_rows - r0) < chunk_rows ? (n_rows - r0) : chunk_rows;
    const uint16_t* hc = reinterpret_cast<const uint16_t*>(hb + r0 * hidden * 2);
    // z [rc, V] = h_c W^T, with the per-row max / argmax / log-sum-exp in the product's epilogue
    if ((s = opd::gemm_bf16_f32(hc, hidden, true, Wb, hidden, true, rc, vocab, hidden, 0.f, zc, ld_y, 1, nullptr,
                                want_stats ? zstats : nullptr, stream)) != OPD_OK)
      return s;
    if (want_stats) {
      hipError_t e = opd::launch_zstats_reduce(zstats, n_parts, (int)rc, logit_max_lse ? logit_max_lse + 2 * r0 : nullptr,
                                               logit_argmax ? logit_argmax + r0 : nullptr, stream);
      if (e != hipSuccess) return hip_fail(e, "logits statistics");
    }
    if ((s = run_team(opd::kFused, zc, yb + r0 * ld_y * 4, OPD_F32, rc, vocab, ld_y, alpha, tau,
                      grad_loss ? grad_loss + r0 : nullptr, loss + r0, target_top1 + r0,
                      draft_top1 ? draft_top1 + r0 : nullptr, row_stats + 8 * r0, dzc, OPD_BF16, ld_dz, ws,
                      stream)) != OPD_OK)
      return s;
    // dh [rc, hidden] = dz W: K = V is long and the output small, so K is split over workgroup
    // slices (enough to give every CU a tile, as far as the logits region holds the partials)
    if (dh) {
      const int64_t tiles = ((rc + 255) / 256) * ((hidden + 255) / 256);
      int64_t split = (256 + tiles - 1) / tiles;
      split = std::min<int64_t>(split, std::max<int64_t>(1, ld_y / hidden));
      split = std::min<int64_t>(split, std::max<int64_t>(1, vocab / 1024));
      split = std::min<int64_t>(split, 32);
      if ((s = opd::gemm_bf16_f32(dzc, ld_dz, true, Wb, hidden, false, rc, hidden, vocab, 0.f, dh + r0 * hidden, hidden,
                                  (int)split, zc, nullptr, stream)) != OPD_OK)
        return s;
    }
    // dW [V, hidden] (+)= dz^T h_c, accumulated over the chunks
    if (dW && (s = opd::gemm_bf16_f32(dzc, ld_dz, false, hc, hidden, false, vocab, hidden, rc, r0 == 0 ? 0.f : 1.f,
                                      dW, hidden, 1, nullptr, nullptr, stream)) != OPD_OK)
      return s;
  }
  return run_accept(blocks, n_rows, draft_top1, target_top1, accept_len, ws, stream);
}

opd_status_t opd_read_flags(void* ws, size_t ws_bytes, int clear, uint32_t* flags, hipStream_t stream) {
  if (!flags) return fail(OPD_ERR_NULL, "flags must be non-NULL");
  opd_status_t s = check_ws(ws, ws_bytes);
  if (s != OPD_OK) return s;
  uint32_t v = 0;
  hipError_t e = hipMemcpyAsync(&v, ws, sizeof(v), hipMemcpyDeviceToHost, stream);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync");
  e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  *flags = v;
  if (clear) {
    e = opd::launch_fill_u32(static_cast<uint32_t*>(ws), 0u, 1, stream);
    if (e != hipSuccess) return hip_fail(e, "flag clear");
    e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  }
  return OPD_OK;
}

opd_status_t opd_stream_probe(const void* a, const void* b, void* c, size_t bytes, hipStream_t stream) {
  if (bytes == 0) return OPD_OK;
  if (!a != !b) return fail(OPD_ERR_NULL, "a and b must be both given or both NULL");
  if (!a && !c) return fail(OPD_ERR_NULL, "nothing to stream: a, b and c are NULL");
  if (bytes % 16) return fail(OPD_ERR_SHAPE, "bytes must be a multiple of 16");
  if ((reinterpret_cast<uintptr_t>(a) | reinterpret_cast<uintptr_t>(b) | reinterpret_cast<uintptr_t>(c)) % 16)
    return fail(OPD_ERR_ALIGN, "buffers must be 16-byte aligned");
  hipError_t e = opd::launch_stream_probe(a, b, c, bytes / 16, stream);
  if (e != hipSuccess) return hip_fail(e, "stream probe launch");
  return OPD_OK;
}

// ---- public entry points: the work above, then the check-mode test of the device flags

opd_status_t opd_loss_fwd(const void* z, const void* y, opd_dtype_t dt, int64_t n_rows, int64_t vocab, int64_t ld,
                          float alpha, float tau, float* loss, int32_t* target_top1, int32_t* draft_top1,
                          float* row_stats, void* ws, size_t ws_bytes, hipStream_t stream) {
  return finish(opd_loss_fwd_impl(z, y, dt, n_rows, vocab, ld, alpha, tau, loss, target_top1, draft_top1, row_stats,
                                  ws, ws_bytes, stream),
                ws, stream);
}

opd_status_t opd_loss_bwd(const void* z, const void* y, opd_dtype_t dt, int64_t n_rows, int64_t vocab, int64_t ld,
                          float alpha, float tau, const float* row_stats, const int32_t* target_top1,
                          const float* grad_loss, void* dz, opd_dtype_t dz_dt, int64_t ld_dz, void* ws,
                          size_t ws_bytes, hipStream_t stream) {
  return finish(opd_loss_bwd_impl(z, y, dt, n_rows, vocab, ld, alpha, tau, row_stats, target_top1, grad_loss, dz,
                                  dz_dt, ld_dz, ws, ws_bytes, stream),
                ws, stream);
}

opd_status_t verify_accept_len(const void* z, const void* y, opd_dtype_t dt, int64_t n_rows, int64_t vocab,
                               int64_t ld, const opd_blocks_t* blocks, int32_t* target_top1, int32_t* draft_top1,
                               int32_t* accept_len, void* ws, size_t ws_bytes, hipStream_t stream) {
  return finish(verify_accept_len_impl(z, y, dt, n_rows, vocab, ld, blocks, target_top1, draft_top1, accept_len, ws,
                                       ws_bytes, stream),
                ws, stream);
}

opd_status_t opd_fused_fwd_bwd_verify(const void* z, const void* y, opd_dtype_t dt, int64_t n_rows, int64_t vocab,
                                      int64_t ld, const opd_blocks_t* blocks, float alpha, float tau,
                                      const float* grad_loss, float* loss, int32_t* target_top1, int32_t* draft_top1,
                                      float* row_stats, void* dz, opd_dtype_t dz_dt, int64_t ld_dz,
                                      int32_t* accept_len, void* ws, size_t ws_bytes, hipStream_t stream) {
  return finish(opd_fused_fwd_bwd_verify_impl(z, y, dt, n_rows, vocab, ld, blocks, alpha, tau, grad_loss, loss,
                                              target_top1, draft_top1, row_stats, dz, dz_dt, ld_dz, accept_len, ws,
                                              ws_bytes, stream),
                ws, stream);
}

opd_status_t opd_length_head_loss(const int32_t* target_top1, const int32_t* draft_top1, int64_t n_rows,
                                  const int32_t* offsets, int32_t n_blocks, const float* head_logit,
                                  const float* grad, int32_t* accept_full, float* label, float* loss,
                                  float* dlogit, void* ws, size_t ws_bytes, hipStream_t stream) {
  return finish(opd_length_head_loss_impl(target_top1, draft_top1, n_rows, offsets, n_blocks, head_logit, grad,
                                          accept_full, label, loss, dlogit, ws, ws_bytes, stream),
                ws, stream);
}

opd_status_t opd_verify_sample(const void* z, const void* y, opd_dtype_t dt, int64_t n_rows, int64_t vocab,
                               int64_t ld, const opd_blocks_t* blocks, const int32_t* draft_tokens,
                               const float* u_accept, const float* u_resample, float temperature,
                               int32_t* accept_len, int32_t* out_token, float* row_lse, void* ws,
                               size_t ws_bytes, hipStream_t stream) {
  return finish(opd_verify_sample_impl(z, y, dt, n_rows, vocab, ld, blocks, draft_tokens, u_accept, u_resample,
                                       temperature, accept_len, out_token, row_lse, ws, ws_bytes, stream),
                ws, stream);
}

opd_status_t opd_lmhead_fused_fwd_bwd_verify(const void* h, const void* W, int64_t hidden, const void* y,
                                             opd_dtype_t dt_y, int64_t n_rows, int64_t vocab, int64_t ld_y,
                                             const opd_blocks_t* blocks, float alpha, float tau,
                                             const float* grad_loss, float* loss, int32_t* target_top1,
                                             int32_t* draft_top1, float* row_stats, float* dh, float* dW,
                                             float* logit_max_lse, int32_t* logit_argmax, int32_t* accept_len,
                                             void* scratch, size_t scratch_bytes, int64_t chunk_rows, void* ws,
                                             size_t ws_bytes, hipStream_t stream) {
  return finish(opd_lmhead_fused_fwd_bwd_verify_impl(h, W, hidden, y, dt_y, n_rows, vocab, ld_y, blocks, alpha, tau,
                                                     grad_loss, loss, target_top1, draft_top1, row_stats, dh, dW,
                                                     logit_max_lse, logit_argmax, accept_len, scratch, scratch_bytes,
                                                     chunk_rows, ws, ws_bytes, stream),
                ws, stream);
}

void opd_set_spin_limit(uint32_t spins) { g_spin_limit.store(spins); }

void opd_set_check(int on) { g_check.store(on ? 1 : 0); }

int opd_get_check(void) { return check_mode() ? 1 : 0; }

opd_status_t opd_debug_reserve_flags(const void* ws, uint32_t count, int64_t next_offset, uint32_t* base,
                                     int* must_clear) {
  if (!base || !must_clear) return fail(OPD_ERR_NULL, "base and must_clear must be non-NULL");
  if (count == 0 || count > 0x3fffffffu) return fail(OPD_ERR_SHAPE, "count must be in [1, 2^30)");
  if (next_offset >= 0x80000000ll) return fail(OPD_ERR_SHAPE, "next_offset must be below 2^31");
  if (next_offset >= 0) {
    std::lock_guard<std::mutex> lk(g_flag_mu);
    g_flag_next = (uint32_t)next_offset;
  }
  bool clear = false;
  *base = reserve_host_flags(ws, count, &clear);
  *must_clear = clear ? 1 : 0;
  return OPD_OK;
}

const char* opd_status_string(opd_status_t s) {
  switch (s) {
    case OPD_OK: return "OPD_OK";
    case OPD_ERR_NULL: return "OPD_ERR_NULL: a required pointer is NULL";
    case OPD_ERR_SHAPE: return "OPD_ERR_SHAPE: invalid sizes";
    case OPD_ERR_DTYPE: return "OPD_ERR_DTYPE: unsupported dtype";
    case OPD_ERR_ALIGN: return "OPD_ERR_ALIGN: pointer or row pitch not 16-byte aligned";
    case OPD_ERR_PARAM: return "OPD_ERR_PARAM: alpha or tau invalid";
    case OPD_ERR_WORKSPACE: return "OPD_ERR_WORKSPACE: workspace missing or too small";
    case OPD_ERR_HIP: return "OPD_ERR_HIP: HIP runtime error";
    case OPD_ERR_DEVICE: return "OPD_ERR_DEVICE: the call raised device flags (check mode)";
  }
  return "unknown status";
}

const char* opd_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
