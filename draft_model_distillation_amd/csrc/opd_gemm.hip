// bf16 matrix products on the gfx950 matrix cores for the lm_head-fused OPD loss (opd_api.cpp):
//   logits   z[R, V]  = h[R, H] W[V, H]^T      (both operands K-major)
//   dh       dh[R, H] = dz[R, V] W[V, H]       (dz K-major, W N-major; split over K = V)
//   dW       dW[V, H] = dz[R, V]^T h[R, H]     (both operands M/N-major)
// which the loss of "AdaFlash: Adaptive Speculative Decoding with Online Self-Improvement for
// High-Concurrency LLM Inference", section "1. On-Policy Distillation (OPD) for Domain Adaptation",
// needs when the drafter's vocabulary projection is trained with it.
//
// One kernel template: C[m, n] = sum_k A(m, k) B(k, n) (+ beta C), bf16 operands, fp32 accumulation
// with v_mfma_f32_32x32x16_bf16. Workgroup tile 256 x 256, one workgroup per CU, kGemmWaves waves
// (four: 128 x 128 each, 4 x 4 blocks of 32 x 32 = 256 accumulators per lane, all in the accumulation
// registers; eight, two per SIMD, 128 x 64 each, is also written and measured no faster). Each
// operand tile is staged in LDS as [m or n][k] with rows of 64 bf16 whose 16-byte k vectors are
// XOR-swizzled by the row, so that fragment reads and tile writes spread over the LDS banks.
//   K-major operand (global [m][K]): loaded straight into LDS (buffer loads with the LDS-DMA bit:
//   lane l of an instruction fills 16 bytes at l * 16), the lanes choosing their global vector so that
//   the linear LDS image is the swizzled tile. No registers, no LDS write instructions.
//   M/N-major operand (global [K][m]): 16-byte loads along m into registers, written transposed
//   (byte permutes) between the products.
// K step 64 and two LDS stages with one barrier per step: an LDS-DMA A tile is issued two steps
// ahead (right after the barrier that frees its stage), the B tile and register-held tiles one step
// ahead. A partial K step (K not a multiple of 64) is loaded through registers with the values past
// K zeroed and runs first, so that every step goes through the same pipeline.
// MFMA operand fragments (lane l: row l % 32, k = 8 (l / 32) + 0..7) are single 16-byte LDS reads.
// Optional epilogue (the logits product): per row and per wave column of the tile, the maximum, the
// lowest column index holding it and the sum of exp(c - max), written as partials that
// k_zstats_reduce combines in a fixed order into per-row max, argmax and log-sum-exp.

#include <stdint.h>

#include <type_traits>

#include "opd_gemm.h"
#include "opd_internal.h"

namespace opd {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 256, BN = 256;
// Waves of a workgroup: kGemmWaves / 2 along N, 2 along M. Each wave computes 128 rows x kWaveCols
// columns of the tile: 4 x FJ blocks of 32 x 32 accumulators.
constexpr int kWaves = kGemmWaves;
constexpr int kGemmThreads = 64 * kWaves;
constexpr int kWavesN = kWaves / 2;
constexpr int FI = 4;                    // 32-row A fragments per wave
constexpr int FJ = 8 / kWavesN;          // 32-column B fragments per wave
constexpr int kWaveCols = 32 * FJ;
constexpr int kSliceMfma = FI * FJ;      // products per wave per 16-wide k slice
static_assert(kWaves == 4 || kWaves == 8, "four or eight waves");
static_assert(kGemmStatParts == kWavesN, "one statistics partial per wave column");
constexpr int kLdsBytes = 128 * 1024;  // two stages of 64 KiB

// Pipeline shape of a product and the derived sizes (one shape for all products: K step 64, two LDS
// stages; a ring of four 32-wide stages with loads three steps ahead was measured slower on the
// 2048 x 151936 x 4096 logits product, 3.1 against 2.6 ms, and removed).
template <bool A_KMAJOR, bool B_KMAJOR>
struct Cfg {
  static constexpr int BK = 64;
  static constexpr int kStages = 2;
  static constexpr int kRowBytes = 2 * BK;               // one LDS tile row
  static constexpr int kTileBytes = 256 * kRowBytes;     // one operand tile
  static constexpr int kStageBytes = 2 * kTileBytes;     // A and B
  static constexpr int kVecs = 256 * BK / 8 / kGemmThreads;  // 16-byte vectors per thread per operand tile
  static constexpr int kSlices = BK / 16;                // 16-wide k slices per step
  static constexpr int kRowVecs = BK / 8;                // 16-byte vectors per tile row
  static constexpr int kInstrRows = 1024 / kRowBytes;    // tile rows one LDS-DMA instruction fills
  static_assert(kStages * kStageBytes == kLdsBytes, "LDS ring size");
};

// LDS position of k vector kv of tile row `row`: 16-byte slot kv ^ swz(row). The LDS serves 16 lanes'
// 16-byte accesses per cycle from 64 four-byte banks: 16 bank groups of 16 bytes, group
// (8 row + slot) % 16 for 128-byte rows. ((row >> 1) ^ (row >> 4)) & 7 makes the fragment reads
// (16 consecutive rows, one k vector) conflict-free and keeps the transposed writes of an M/N-major
// operand (rows 8 g + o for 16 consecutive g) at most 2-way.
template <int BK>
__device__ __forceinline__ int swz(int row) {
  static_assert(BK == 64, "128-byte rows");
  return ((row >> 1) ^ (row >> 4)) & 7;
}

// A wave-uniform pointer held in scalar registers (buffer resources must be).
template <typename T>
__device__ __forceinline__ T* uniform_ptr(T* p) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
  return reinterpret_cast<T*>(lo | (hi << 32));
}

// Operand tiles are read through one buffer resource per operand spanning the whole matrix: a load
// at or past its last byte reads as zero, which is what rows past M (or N) and k-rows past K get.
// Offsets are 32-bit (the host checks that they cannot wrap).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t operand_rsrc(const uint16_t* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(const_cast<uint16_t*>(base)), 0, (int)bytes, 0x00020000);
}

// Thread (wave w, lane l)'s kVecs 16-byte vectors of a 256 x BK operand tile:
//   K-major ([row][K], ld bytes per row): vector i is tile row kInstrRows (w kVecs + i) + l / kRowVecs,
//   LDS slot l % kRowVecs, i.e. global k vector (l % kRowVecs) ^ swz(row); the 64 lanes of vector i
//   fill 1 KiB of LDS in lane order. A step moves 2 BK bytes along k.
//   M/N-major ([K][row]): vector i is k-row mn_k(t, i) of the step, rows mn_row(t) .. + 7; a step
//   moves BK k-rows.
template <class C, bool KMAJOR>
__device__ __forceinline__ int kmajor_row(int t, int i) {
  return C::kInstrRows * ((t >> 6) * C::kVecs + i) + (t & 63) / C::kRowVecs;
}
template <class C, bool KMAJOR>
__device__ __forceinline__ int kmajor_kvec(int t, int i) {
  return ((t & 63) % C::kRowVecs) ^ swz<C::BK>(kmajor_row<C, KMAJOR>(t, i));
}
// M/N-major: the k (within the step) of vector i and the first of the thread's 8 tile rows. Four
// waves: k = 8 (t / 32) + i (8 k values: a whole k vector per row), rows 8 (t % 32). Eight waves:
// lane l of wave w covers k vector w, half l & 1 (k = 8 w + 4 (l & 1) + i, 4 k values per row),
// rows 8 (l >> 1).
__device__ __forceinline__ int mn_k(int t, int i) {
  if constexpr (kWaves == 4) return 8 * (t / 32) + i;
  else return 8 * (t >> 6) + 4 * (t & 1) + i;
}
__device__ __forceinline__ int mn_row(int t) {
  if constexpr (kWaves == 4) return 8 * (t % 32);
  else return 8 * ((t & 63) >> 1);
}
template <class C, bool KMAJOR>
__device__ __forceinline__ void tile_offsets(uint32_t ld_bytes, int row0, int k0, int t, uint32_t (&off)[C::kVecs]) {
#pragma unroll
  for (int i = 0; i < C::kVecs; ++i) {
    if constexpr (KMAJOR) {
      off[i] = (uint32_t)(row0 + kmajor_row<C, KMAJOR>(t, i)) * ld_bytes + 2u * (uint32_t)k0 +
               16u * (uint32_t)kmajor_kvec<C, KMAJOR>(t, i);
    } else {
      off[i] = (uint32_t)(k0 + mn_k(t, i)) * ld_bytes + 2u * (uint32_t)(row0 + mn_row(t));
    }
  }
}
template <class C, bool KMAJOR>
__device__ __forceinline__ uint32_t step_bytes(uint32_t ld_bytes) {
  return KMAJOR ? 2u * C::BK : (uint32_t)C::BK * ld_bytes;
}

// K-major tile straight into LDS: vector i of wave w lands at rows kInstrRows (w kVecs + i) ...
template <int NV>
__device__ __forceinline__ void dma_tile(__amdgpu_buffer_rsrc_t r, const uint32_t* off, uint8_t* tile, int wave) {
#pragma unroll
  for (int i = 0; i < NV; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r, (__attribute__((address_space(3))) void*)(tile + 1024 * (wave * NV + i)), 16, off[i], 0, 0, 0);
}

// Loads one operand tile into registers. MASKED (the last, partial K step only): k at or past kend
// reads as zero; a K-major vector can straddle kend (K not a multiple of 8), and its elements past
// kend, which may hold anything (row padding), are zeroed one by one.
template <class C, bool KMAJOR, bool MASKED>
__device__ __forceinline__ void load_tile(__amdgpu_buffer_rsrc_t r, const uint32_t (&off)[C::kVecs], int k0, int kend,
                                          int t, u32x4 (&v)[C::kVecs]) {
#pragma unroll
  for (int i = 0; i < C::kVecs; ++i) {
    u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off[i], 0, 0);
    if constexpr (MASKED) {
      if constexpr (KMAJOR) {
        const int n = kend - (k0 + 8 * kmajor_kvec<C, KMAJOR>(t, i));  // valid elements (<= 0: none)
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = 2 * e + 1 < n ? x[e] : 2 * e < n ? (x[e] & 0xffffu) : 0u;
      } else {
        if (k0 + mn_k(t, i) >= kend) x = u32x4{0, 0, 0, 0};
      }
    }
    v[i] = x;
  }
}

// Writes the registers of load_tile to the (swizzled) LDS tile.
template <class C, bool KMAJOR>
__device__ __forceinline__ void store_tile(uint8_t* tile, int t, const u32x4 (&v)[C::kVecs]) {
  if constexpr (KMAJOR) {  // the image the LDS-DMA loads would have written
#pragma unroll
    for (int i = 0; i < C::kVecs; ++i)
      *reinterpret_cast<u32x4*>(tile + 1024 * ((t >> 6) * C::kVecs + i) + 16 * (t & 63)) = v[i];
  } else if constexpr (kWaves == 4) {
    // v[i] holds rows 8 g .. 8 g + 7 at k = 8 q + i (g = t % 32, q = t / 32); each of the 8 rows gets
    // its 8 k values (k vector q) as one 16-byte write (byte permutes pick the rows' halves)
    const int g = t % 32, q = t / 32;
#pragma unroll
    for (int j = 0; j < 4; ++j) {  // rows 8 g + 2 j (low halves) and 8 g + 2 j + 1 (high halves)
      u32x4 lo, hi;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        lo[e] = __builtin_amdgcn_perm(v[2 * e + 1][j], v[2 * e][j], 0x05040100u);
        hi[e] = __builtin_amdgcn_perm(v[2 * e + 1][j], v[2 * e][j], 0x07060302u);
      }
      const int r0 = 8 * g + 2 * j, r1 = r0 + 1;
      *reinterpret_cast<u32x4*>(tile + r0 * C::kRowBytes + 16 * (q ^ swz<C::BK>(r0))) = lo;
      *reinterpret_cast<u32x4*>(tile + r1 * C::kRowBytes + 16 * (q ^ swz<C::BK>(r1))) = hi;
    }
  } else {
    // v[i] holds rows 8 g .. 8 g + 7 at k = 8 q + 4 h + i (g = l >> 1, h = l & 1, q = the wave); each
    // of the 8 rows gets its 4 k values as one 8-byte write into half h of its k vector q
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const int g = (t & 63) >> 1, h = t & 1, q = t >> 6;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const u32x2 lo = {__builtin_amdgcn_perm(v[1][j], v[0][j], 0x05040100u),
                        __builtin_amdgcn_perm(v[3][j], v[2][j], 0x05040100u)};
      const u32x2 hi = {__builtin_amdgcn_perm(v[1][j], v[0][j], 0x07060302u),
                        __builtin_amdgcn_perm(v[3][j], v[2][j], 0x07060302u)};
      const int r0 = 8 * g + 2 * j, r1 = r0 + 1;
      *reinterpret_cast<u32x2*>(tile + r0 * C::kRowBytes + 16 * (q ^ swz<C::BK>(r0)) + 8 * h) = lo;
      *reinterpret_cast<u32x2*>(tile + r1 * C::kRowBytes + 16 * (q ^ swz<C::BK>(r1)) + 8 * h) = hi;
    }
  }
}

// One wave's MFMA operands for one 16-wide k slice: 4 A fragments (rows of its 128-row half) and 4 B
// fragments (columns of its 128-column half). Lane l holds row (or column) l % 32, k = 8 (l / 32) .. + 7.
// arow / brow: byte offset of the lane's row in the wave's first fragment; slot: the 16-byte slot of the
// slice's k vector in that row. Rows 32 i further on (the halves start at multiples of 128 rows, where
// the swizzles vanish) are swizzled alike for 64-byte rows and by an extra 2 i for 128-byte rows.
struct Frags {
  bf16x8 a[FI], b[FJ];
};
template <class C>
__device__ __forceinline__ void read_frags(const uint8_t* stage, uint32_t arow, uint32_t brow, uint32_t slot,
                                           uint32_t bx, Frags& f) {
  static_assert(C::BK == 64, "128-byte rows");
#pragma unroll
  for (int i = 0; i < FI; ++i)
    f.a[i] = __builtin_bit_cast(
        bf16x8, *reinterpret_cast<const u32x4*>(stage + arow + 32 * i * C::kRowBytes + 16 * (slot ^ (2 * i))));
#pragma unroll
  for (int j = 0; j < FJ; ++j)
    f.b[j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(stage + C::kTileBytes + brow + 32 * j * C::kRowBytes +
                                                                           16 * (slot ^ bx ^ (2 * j))));
}
// Half of one slice's products: A fragments 2 h and 2 h + 1.
__device__ __forceinline__ void mfma_half(const Frags& f, f32x16 (&acc)[FI][FJ], int h) {
#pragma unroll
  for (int i = 2 * h; i < 2 * h + 2; ++i)
#pragma unroll
    for (int j = 0; j < FJ; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
}
__device__ __forceinline__ void mfma_slice(const Frags& f, f32x16 (&acc)[FI][FJ]) {
  mfma_half(f, acc, 0);
  mfma_half(f, acc, 1);
}

// Row statistics of one 32 x 32 output block row-group over a lane's columns: see the epilogue.
__device__ __forceinline__ float half_max(float v) {  // over the 32 lanes of a half wave (same l / 32)
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, true)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, true)));
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_int(v), __float_as_int(v), false, false);
  return fmaxf(__int_as_float((int)p[0]), __int_as_float((int)p[1]));
}
__device__ __forceinline__ float half_sum(float v) {
  v = v + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));
  v = v + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true));
  v = v + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, true));
  v = v + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, true));
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_int(v), __float_as_int(v), false, false);
  return __int_as_float((int)p[0]) + __int_as_float((int)p[1]);
}
__device__ __forceinline__ int half_min(int v) {
  v = min(v, __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, true));
  v = min(v, __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, true));
  v = min(v, __builtin_amdgcn_mov_dpp(v, 0x141, 0xF, 0xF, true));
  v = min(v, __builtin_amdgcn_mov_dpp(v, 0x140, 0xF, 0xF, true));
  const auto p = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return min((int)p[0], (int)p[1]);
}

// Scheduling-group order for one slice's products interleaved with NOTHER other instructions of the
// class MASK (0x010 vector-memory loads, 0x200 LDS writes), spread evenly.
template <int NPROD, int NOTHER, int MASK>
__device__ __forceinline__ void interleave() {
  if constexpr (NOTHER > 0 && NOTHER <= NPROD) {
#pragma unroll
    for (int u = 0; u < NOTHER; ++u) {
      __builtin_amdgcn_sched_group_barrier(0x008, NPROD / NOTHER, 0);
      __builtin_amdgcn_sched_group_barrier(MASK, 1, 0);
    }
  } else if constexpr (NOTHER > NPROD) {
#pragma unroll
    for (int u = 0; u < NPROD; ++u) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(MASK, NOTHER / NPROD, 0);
    }
  }
}

// s_waitcnt immediates (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
constexpr int kWaitLgkm0 = 0xC07F;

template <bool A_KMAJOR, bool B_KMAJOR, bool STATS, bool BETA>
__global__ void __launch_bounds__(kGemmThreads, 1) k_gemm(GemmParams P) {
  using C = Cfg<A_KMAJOR, B_KMAJOR>;
  constexpr int BK = C::BK, NST = C::kStages, NV = C::kVecs;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int t = (int)__builtin_amdgcn_workitem_id_x();
  const int lane = t & 63, wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave / kWavesN, wn = wave % kWavesN;  // this wave's 128 x kWaveCols part of the tile

  // Tile order: the tiles that share a block of the larger operand run on the same XCD (workgroups
  // are dispatched to the XCDs round-robin), so that they read it from that XCD's L2: the M tiles of
  // one N tile when B is the larger operand (more N tiles than M tiles), else the N tiles of one M
  // tile.
  const int b = (int)__builtin_amdgcn_workgroup_id_x();
  const int xcd = b % 8, s = b / 8;
  int m_tile, n_tile;
  if (P.m_major) {
    m_tile = 8 * (s / P.n_tiles) + xcd;
    n_tile = s % P.n_tiles;
    if (m_tile >= P.m_tiles) return;  // padding of the tile order (uniform per workgroup)
  } else {
    n_tile = 8 * (s / P.m_tiles) + xcd;
    m_tile = s % P.m_tiles;
    if (n_tile >= P.n_tiles) return;
  }
  const int m0 = m_tile * BM, n0 = n_tile * BN;
  const int kz = (int)__builtin_amdgcn_workgroup_id_y();
  const int kbeg = kz * P.kslice, kend = min(P.K, kbeg + P.kslice);
  const int nsteps = kend > kbeg ? (kend - kbeg + BK - 1) / BK : 0;
  const int nfull = (kend - kbeg) / BK;  // steps that need no masking

  f32x16 acc[FI][FJ];
#pragma unroll
  for (int i = 0; i < FI; ++i)
#pragma unroll
    for (int j = 0; j < FJ; ++j) acc[i][j] = f32x16{};

  const __amdgpu_buffer_rsrc_t rA = operand_rsrc(P.A, P.a_bytes);
  const __amdgpu_buffer_rsrc_t rB = operand_rsrc(P.B, P.b_bytes);
  const uint32_t ldA = 2u * (uint32_t)P.lda, ldB = 2u * (uint32_t)P.ldb;
  uint32_t oa[NV], ob[NV];  // offsets of the next step to load
  tile_offsets<C, A_KMAJOR>(ldA, m0, kbeg, t, oa);
  tile_offsets<C, B_KMAJOR>(ldB, n0, kbeg, t, ob);
  const uint32_t sa = step_bytes<C, A_KMAJOR>(ldA), sb = step_bytes<C, B_KMAJOR>(ldB);
  u32x4 ra[NV], rb[NV];
  auto stage_ptr = [&](int st) { return smem + (st % NST) * C::kStageBytes; };
  // Issues the loads of one operand of full step `st` (LDS-DMA for a K-major operand, registers
  // otherwise) and moves its offsets on.
  auto issue_a = [&](int st) {
    if constexpr (A_KMAJOR) dma_tile<NV>(rA, oa, stage_ptr(st), wave);
    else load_tile<C, false, false>(rA, oa, 0, 0, t, ra);
#pragma unroll
    for (int i = 0; i < NV; ++i) oa[i] += sa;
  };
  auto issue_b = [&](int st) {
    if constexpr (B_KMAJOR) dma_tile<NV>(rB, ob, stage_ptr(st) + C::kTileBytes, wave);
    else load_tile<C, false, false>(rB, ob, 0, 0, t, rb);
#pragma unroll
    for (int i = 0; i < NV; ++i) ob[i] += sb;
  };

  // Fragment rows: row l % 32 of the wave's halves; slice q reads k vector 2 q + l / 32.
  const int fr = lane & 31, fh = lane >> 5;
  const uint32_t arow = (uint32_t)(wm * 128 + fr) * C::kRowBytes,
                 brow = (uint32_t)(wn * kWaveCols + fr) * C::kRowBytes;
  uint32_t fs[C::kSlices];
#pragma unroll
  for (int q = 0; q < C::kSlices; ++q) fs[q] = (uint32_t)((2 * q + fh) ^ swz<BK>(fr));
  // the swizzle's higher term at the wave's first B row (A halves start at multiples of 128 rows)
  const uint32_t bx = (uint32_t)(((wn * kWaveCols) >> 4) & 7);

  // Step st computes from stage st % 2 (cur) while the next step's tiles arrive in the other (nxt):
  //   - an LDS-DMA A tile (K-major A) is issued two steps ahead, right after the barrier of the step
  //     before, into the stage that barrier has just freed (one load per product of the second half
  //     of the last slice);
  //   - the B tile (LDS-DMA or registers) and a register-held A tile are issued in the first slice,
  //     one load per product or two;
  //   - register-held tiles are written to nxt between the third slice's products;
  //   - the k slices run from LDS with the fragments of slice + 1 read while slice's products run;
  //   - the barrier (after every load of nxt has landed) sits in the middle of the last slice, whose
  //     products around it cover the barrier and the next step's first fragment reads.
  Frags f0, f1;
  auto first_fragments = [&](const uint8_t* stage) {
    __builtin_amdgcn_s_waitcnt(0);  // every load so far (LDS-DMA included) has landed
    __syncthreads();
    read_frags<C>(stage, arow, brow, fs[0], bx, f0);
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  };
  constexpr int kWrites = (A_KMAJOR ? 0 : 8) + (B_KMAJOR ? 0 : 8);  // one per tile row a thread holds
  auto step = [&](auto next_c, auto ahead2_c, int st) {
    constexpr bool NEXT = decltype(next_c)::value;      // a step st + 1 follows: load it
    constexpr bool AHEAD2 = decltype(ahead2_c)::value;  // a step st + 2 follows: issue its LDS-DMA A tile
    const uint8_t* cur = stage_ptr(st);
    uint8_t* nxt = stage_ptr(st + 1);
    // fc: this slice's fragments; fn: the next slice's (or the next step's first)
    auto slice = [&](auto qc, Frags& fc, Frags& fn) {
      constexpr int q = decltype(qc)::value;
      constexpr bool LAST = q == C::kSlices - 1;
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (!LAST) {
        constexpr bool LOAD = q == 0 && NEXT;
        constexpr int kLoadsHere = LOAD ? (A_KMAJOR ? 0 : NV) + NV : 0;
        constexpr bool WRITE = q == C::kSlices - 2 && NEXT && kWrites > 0;  // register-held tiles out
        read_frags<C>(cur, arow, brow, fs[q + 1], bx, fn);
        if constexpr (LOAD) {
          if constexpr (!A_KMAJOR) issue_a(st + 1);
          issue_b(st + 1);
        }
        if constexpr (WRITE) {
          if constexpr (!A_KMAJOR) store_tile<C, false>(nxt, t, ra);
          if constexpr (!B_KMAJOR) store_tile<C, false>(nxt + C::kTileBytes, t, rb);
        }
        mfma_slice(fc, acc);
        if constexpr (kLoadsHere > 0) {
          __builtin_amdgcn_sched_group_barrier(0x100, FI + FJ, 0);  // the fragment reads
          interleave<kSliceMfma, kLoadsHere, 0x010>();
        }
        if constexpr (WRITE) {
          __builtin_amdgcn_sched_group_barrier(0x100, FI + FJ, 0);  // the fragment reads
          interleave<kSliceMfma, kWrites, 0x200>();
        }
      } else {
        mfma_half(fc, acc, 0);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (NEXT) {
          __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // every load of nxt has landed
          __syncthreads();
          read_frags<C>(nxt, arow, brow, fs[0], bx, fn);
          if constexpr (A_KMAJOR && AHEAD2) issue_a(st + 2);  // into cur, which the barrier freed
        }
        mfma_half(fc, acc, 1);
        constexpr int kDma = NEXT && AHEAD2 && A_KMAJOR ? NV : 0;
        if constexpr (kDma > 0) {
          __builtin_amdgcn_sched_group_barrier(0x100, FI + FJ, 0);  // the next step's first fragment reads
          interleave<kSliceMfma / 2, kDma, 0x010>();
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    slice(std::integral_constant<int, 0>{}, f0, f1);
    slice(std::integral_constant<int, 1>{}, f1, f0);
    slice(std::integral_constant<int, 2>{}, f0, f1);
    slice(std::integral_constant<int, 3>{}, f1, f0);
  };
  static_assert(C::kSlices == 4, "four 16-wide slices per step");

  // Steps: a partial one (K not a multiple of BK: the last k range, loaded through registers with
  // masking) goes first, as step 0, so that every step runs through the same pipeline; the full steps
  // follow in k order.
  if (nsteps > 0) {
    if (nfull < nsteps) {
      uint32_t ta[NV], tb[NV];
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        ta[i] = oa[i] + (uint32_t)nfull * sa;
        tb[i] = ob[i] + (uint32_t)nfull * sb;
      }
      const int k1 = kbeg + nfull * BK;
      load_tile<C, A_KMAJOR, true>(rA, ta, k1, kend, t, ra);
      load_tile<C, B_KMAJOR, true>(rB, tb, k1, kend, t, rb);
      store_tile<C, A_KMAJOR>(stage_ptr(0), t, ra);
      store_tile<C, B_KMAJOR>(stage_ptr(0) + C::kTileBytes, t, rb);
    } else {
      issue_a(0);
      issue_b(0);
      if constexpr (!A_KMAJOR) store_tile<C, false>(stage_ptr(0), t, ra);
      if constexpr (!B_KMAJOR) store_tile<C, false>(stage_ptr(0) + C::kTileBytes, t, rb);
    }
    if constexpr (A_KMAJOR)
      if (nsteps > 1) issue_a(1);  // the A tile of step 1, two steps ahead of its use like the rest
    first_fragments(stage_ptr(0));
    int st = 0;
#pragma nounroll
    for (; st + 2 < nsteps; ++st) step(std::true_type{}, std::true_type{}, st);
    if (st + 1 < nsteps) {
      step(std::true_type{}, std::false_type{}, st);
      ++st;
    }
    step(std::false_type{}, std::false_type{}, st);
  }

  // ---- write C (or this K slice's partial) and, for the logits, the row statistics
  float* out = P.k_split > 1 ? P.partial + (int64_t)kz * P.M * (int64_t)P.ldc : P.C;
  const int col = lane & 31, rq = 4 * (lane >> 5);
  // Stores go through a buffer resource based at the tile's corner whose extent ends with the
  // matrix's last row: rows past M are dropped by the range check, columns past N by the lane mask.
  // Lane l holds column 32 j + l % 32 and rows 8 (r / 4) + 4 (l / 32) + r % 4 of block (i, j).
  const int64_t corner = (int64_t)m0 * P.ldc + n0;
  const int64_t remain = ((int64_t)P.M * P.ldc - corner) * 4;
  const __amdgpu_buffer_rsrc_t rC = __builtin_amdgcn_make_buffer_rsrc(
      uniform_ptr(out + corner), 0, __builtin_amdgcn_readfirstlane((int)(remain < 0xFFFFFFFFll ? remain : 0xFFFFFFFFll)),
      0x00020000);
  const uint32_t ldc4 = 4u * (uint32_t)P.ldc;
  const uint32_t lane_off = (uint32_t)(wm * 128 + rq) * ldc4 + 4u * (uint32_t)(wn * kWaveCols + col);
  bool nok[FJ];
#pragma unroll
  for (int j = 0; j < FJ; ++j) nok[j] = n0 + wn * kWaveCols + 32 * j + col < P.N;
#pragma unroll
  for (int j = 0; j < FJ; ++j) {
    if (nok[j]) {
#pragma unroll
      for (int i = 0; i < FI; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const uint32_t off = lane_off + (uint32_t)(32 * i + 8 * (r / 4) + (r % 4)) * ldc4 + 128u * j;
          float v = acc[i][j][r];
          if constexpr (BETA) v += P.beta * __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rC, (int)off, 0, 0));
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), rC, (int)off, 0, 0);
        }
    }
  }
  if constexpr (STATS) {
    // Per row of this wave's part: max over its (valid) kWaveCols columns, the lowest column holding
    // it, and the sum of exp(c - max). Lanes l and l + 32 hold different rows; the 32 lanes of a half
    // hold the 32 columns of a block, FJ blocks per lane.
    float* st_base = P.stats + (kGemmStatParts * n_tile + wn) * 3;
    const int64_t st_ld = kGemmStatParts * P.n_tiles * 3;
#pragma unroll
    for (int i = 0; i < FI; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float v[FJ];
        float lm = -__builtin_inff();
#pragma unroll
        for (int j = 0; j < FJ; ++j) {
          v[j] = nok[j] ? acc[i][j][r] : -__builtin_inff();
          lm = fmaxf(lm, v[j]);
        }
        const float mx = half_max(lm);
        int li = 0x7fffffff;  // lowest column (relative to the wave's part) holding the max
        float ls = 0.f;
#pragma unroll
        for (int j = FJ - 1; j >= 0; --j) {
          if (v[j] == mx) li = 32 * j + col;
          ls += nok[j] ? __expf(v[j] - mx) : 0.f;
        }
        const int ix = half_min(li);
        const float sm = half_sum(ls);
        const int m = m0 + wm * 128 + 32 * i + 8 * (r / 4) + rq + (r % 4);
        if (col == 0 && m < P.M) {
          float* stp = st_base + (int64_t)m * st_ld;
          stp[0] = mx;
          stp[1] = __int_as_float(ix + n0 + wn * kWaveCols);
          stp[2] = sm;
        }
      }
    }
  }
}

// Sums the K slices of a split product in slice order: C = sum_z partial[z] (+ beta C).
__global__ void __launch_bounds__(256) k_splitk_reduce(const float* partial, float* C, int64_t ldc, int M, int N,
                                                       int k_split, float beta) {
  const int64_t total = (int64_t)M * N;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int64_t m = i / N, n = i % N;
    float s = 0.f;
    for (int z = 0; z < k_split; ++z) s += partial[(int64_t)z * M * ldc + m * ldc + n];
    float* c = C + m * ldc + n;
    *c = beta != 0.f ? s + beta * *c : s;
  }
}

// Per-row logits statistics from the product's half-tile partials, combined in column order:
// max, lowest index of the max, log-sum-exp. One wave per row. maxlse [M][2] = (max, LSE) and arg [M]
// may each be NULL.
__global__ void __launch_bounds__(256) k_zstats_reduce(const float* part, int n_parts, int M, float* maxlse,
                                                       int32_t* arg) {
  const int lane = threadIdx.x & 63;
  const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (m >= M) return;
  const float* p = part + (int64_t)m * n_parts * 3;
  float mx = -__builtin_inff();
  for (int q = lane; q < n_parts; q += 64) mx = fmaxf(mx, p[3 * q]);
  for (int o = 32; o; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  int ix = 0x7fffffff;
  float s = 0.f;
  for (int q = lane; q < n_parts; q += 64) {
    const float pm = p[3 * q];
    if (pm == mx) ix = min(ix, __float_as_int(p[3 * q + 1]));
    if (pm > -__builtin_inff()) s += p[3 * q + 2] * __expf(pm - mx);
  }
  for (int o = 32; o; o >>= 1) {
    ix = min(ix, __shfl_xor(ix, o));
    s += __shfl_xor(s, o);
  }
  if (lane == 0) {
    if (maxlse) {
      maxlse[2 * m] = mx;
      maxlse[2 * m + 1] = mx + __logf(s);
    }
    if (arg) arg[m] = ix;
  }
}

typedef void (*GemmKernel)(GemmParams);

template <bool AK, bool BK_, bool S, bool B>
GemmKernel kernel_of() {
  return k_gemm<AK, BK_, S, B>;
}

}  // namespace

hipError_t launch_gemm(GemmParams p, bool a_kmajor, bool b_kmajor, hipStream_t s) {
  p.m_tiles = (p.M + BM - 1) / BM;
  p.n_tiles = (p.N + BN - 1) / BN;
  if (p.k_split < 1) p.k_split = 1;
  p.kslice = ((p.K + p.k_split - 1) / p.k_split + 63) / 64 * 64;  // a multiple of either K step
  const bool beta = p.k_split == 1 && p.beta != 0.f;  // split products apply beta in the reduction
  GemmKernel k = nullptr;
  if (a_kmajor && b_kmajor && !beta) k = p.stats ? kernel_of<true, true, true, false>() : kernel_of<true, true, false, false>();
  else if (a_kmajor && !b_kmajor && !p.stats) k = beta ? kernel_of<true, false, false, true>() : kernel_of<true, false, false, false>();
  else if (!a_kmajor && !b_kmajor && !p.stats) k = beta ? kernel_of<false, false, false, true>() : kernel_of<false, false, false, false>();
  if (!k) return hipErrorInvalidValue;
  // more than 64 KiB of dynamic LDS (set on every launch: the setting is per device)
  hipError_t e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
  if (e != hipSuccess) return e;
  p.m_major = p.m_tiles > p.n_tiles;
  const int grid = p.m_major ? 8 * p.n_tiles * ((p.m_tiles + 7) / 8) : 8 * p.m_tiles * ((p.n_tiles + 7) / 8);
  void* args[] = {&p};
  e = hipLaunchKernel((const void*)k, dim3(grid, p.k_split), dim3(kGemmThreads), args, kLdsBytes, s);
  if (e != hipSuccess) return e;
  if (p.k_split > 1) {
    hipLaunchKernelGGL(k_splitk_reduce, dim3(1024), dim3(256), 0, s, p.partial, p.C, p.ldc, p.M, p.N, p.k_split, p.beta);
    e = hipGetLastError();
  }
  return e;
}

hipError_t launch_zstats_reduce(const float* part, int n_parts, int M, float* maxlse, int32_t* arg, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_zstats_reduce, dim3((M + 3) / 4), dim3(256), 0, s, part, n_parts, M, maxlse, arg);
  return hipGetLastError();
}

}  // namespace opd
