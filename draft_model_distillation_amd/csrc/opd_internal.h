// Internal interface between the C-ABI host layer (opd_api.cpp) and the gfx950 kernels
// (opd_kernels.hip). Not part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "opd.h"

namespace opd {

constexpr int kThreads = 256;  // workgroup size of every row kernel (4 wave64)
constexpr int kStage1Units = 5;  // values per member in exchange 1 (at most): top-1 mode's maxima, indices, z at y's
constexpr int kStage2Units = 5;  // S, clipped sum, lowest indices of the row maxima of z and y, z at the latter
constexpr int kMaxGrid = 4096;  // upper bound on co-resident workgroups the workspace is sized for
// Workspace layout: [0, 256) header, then the exchange units. The header holds the sticky flag word
// (byte 0), the exchange-flag epoch (byte 64) and the count of row-team workgroups that finished the
// current launch (byte 128), each on its own cache line. A zero-filled header is the initial state.
constexpr size_t kHeaderBytes = 256;
constexpr int kEpochWord = 16;   // uint32 index of the epoch in the header
constexpr int kDoneWord = 32;    // uint32 index of the finished-workgroup count
// Three stages per team: exchange 1 alternates between stages 0 and 1 by row-iteration parity (a
// member that moves on to its next row must not overwrite a value a slower member of the team has yet
// to read), exchange 2 uses stage 2.
constexpr int kStages = 3;
constexpr size_t kUnitBytesPerWg = kStages * 8 * 8;  // three stages x up to 8 units x 8 bytes
constexpr size_t kWorkspaceBytes = kHeaderBytes + (size_t)kMaxGrid * kUnitBytesPerWg;

// Sticky device flag bits (same values as the public OPD_FLAG_* macros).
constexpr uint32_t kFlagNegL = 1u;
constexpr uint32_t kFlagBadOffsets = 2u;
constexpr uint32_t kFlagSpinTimeout = 4u;
constexpr uint32_t kFlagBadToken = 8u;
constexpr uint32_t kDefaultSpinLimit = 1u << 22;
// A device epoch past this value is restarted at 0 by the last workgroup of a launch, which first
// zeroes every exchange unit (no flag of the range that ends can then match a stale unit).
constexpr uint32_t kEpochRestart = 0x40000000u;
constexpr int kMaxTeamSize = 128;
constexpr int kMaxVocab = 1 << 19;  // 524,288 logits per row

enum Mode : int { kFused = 0, kForward = 1, kTop1 = 2 };

// One launch of the row-team kernel: G workgroups share a row, each owns a chunk of it.
struct TeamParams {
  const uint8_t* z;
  const uint8_t* y;
  int64_t ld_bytes;  // row pitch of z and y in bytes
  int32_t vocab;
  int32_t nvec;       // 16-byte vectors per row covering vocab
  int32_t n_rows;
  int32_t G;          // workgroups per row
  int32_t chunk_vec;  // vectors per chunk (last chunk may be shorter)
  int32_t n_teams;
  float alpha;
  float tau;
  const float* grad_loss;  // nullable
  float* loss;
  int32_t* target_top1;
  int32_t* draft_top1;  // nullable
  float* row_stats;     // [n_rows][8]; nullable in kTop1 mode
  uint8_t* dz;
  int64_t ld_dz_bytes;
  uint64_t* units;  // exchange units [n_teams][kStages][G][8]
  uint32_t* flags;  // workspace header: sticky flag word, epoch (kEpochWord), done count (kDoneWord)
  uint32_t flag_count;  // exchange flags this launch uses (2 per row iteration + 2)
  uint32_t flag_base;   // first flag minus 1, chosen by the host (>= 2^31); 0: from the workspace epoch
  uint32_t spin_limit;
};

struct BwdParams {
  const uint8_t* z;
  const uint8_t* y;
  int64_t ld_bytes;
  int32_t vocab;
  int32_t nvec;
  int32_t n_rows;
  float alpha;
  float tau;
  const float* row_stats;  // [n_rows][8] from the forward pass
  const int32_t* target_top1;
  const float* grad_loss;
  uint8_t* dz;
  int64_t ld_dz_bytes;
};

struct AcceptParams {
  const int32_t* draft_top1;
  const int32_t* target_top1;
  const int32_t* offsets;
  const int32_t* L;
  int32_t n_blocks;
  int32_t n_rows;
  int32_t* accept_len;
  uint32_t* flags;
};

struct LengthHeadParams {
  const int32_t* draft_top1;
  const int32_t* target_top1;
  const int32_t* offsets;
  int32_t n_blocks;
  int32_t n_rows;
  const float* head_logit;
  const float* grad;  // nullable
  int32_t* accept_full;
  float* label;
  float* loss;
  float* dlogit;
  uint32_t* flags;
};

// Speculative-sampling verification at temperature T (opd_sample.hip).
constexpr int kMaxSampleTiles = 2048;  // 64-vector tiles of the widest row (524288 fp32 logits)
constexpr int kSampleSlices = 16;      // workgroups that sum one draw row
// blocks per launch pair: their slice sums fill the workspace after its header
constexpr int kSampleBatch = (int)((kWorkspaceBytes - kHeaderBytes) / (kSampleSlices * sizeof(float)));
struct SampleParams {
  const uint8_t* z;
  const uint8_t* y;
  int64_t ld_bytes;
  int32_t vocab;
  int32_t nvec;  // 16-byte vectors per row covering vocab
  int32_t n_rows;
  int32_t n_blocks;
  float c;  // log2(e) / T
  const int32_t* offsets;
  const int32_t* L;
  const int32_t* draft;
  const float* u_accept;
  const float* u_resample;
  float* stats;  // [n_rows][4]: reference and log2 of the sum for z / T, then for y / T
  int32_t* accept_len;
  int32_t* token;
  uint32_t* flags;
  float* slices;   // workspace: [kSampleBatch][kSampleSlices] slice sums of the draw rows
  int32_t block0;  // first block of the current batch
};

// in_bf16: 1 if z/y are bf16 (else fp32); out_bf16: 1 if dz is bf16 (else fp32); K: slots per thread
// (1, 3 or 5).
hipError_t launch_team(const TeamParams& p, int mode, int in_bf16, int out_bf16, int K, int grid,
                       hipStream_t s);
// dev_flags: the instantiation that takes its exchange flags from the workspace epoch (flag_base 0).
hipError_t team_occupancy(int mode, int in_bf16, int out_bf16, int K, bool dev_flags, int* blocks_per_cu);
hipError_t launch_bwd(const BwdParams& p, int in_bf16, int out_bf16, hipStream_t s);
hipError_t launch_accept(const AcceptParams& p, hipStream_t s);
hipError_t launch_fill_u32(uint32_t* dst, uint32_t value, size_t count, hipStream_t s);
hipError_t launch_stream_probe(const void* a, const void* b, void* c, size_t n_vec, hipStream_t s);
hipError_t launch_length_head(const LengthHeadParams& p, hipStream_t s);  // opd_epilogue.hip
hipError_t launch_sample_verify(const SampleParams& p, int in_bf16, hipStream_t s);  // opd_sample.hip

// Records the detail text returned by opd_last_error() on this thread (opd_api.cpp).
opd_status_t record_error(opd_status_t s, const char* msg);

}  // namespace opd
