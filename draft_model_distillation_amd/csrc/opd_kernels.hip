// gfx950 kernels of the on-policy-distillation (OPD) loss / gradient / greedy-verify path.
//
// What is computed, per drafted position (one row of V logits), follows the AdaFlash pages:
//  - "AdaFlash: Adaptive Speculative Decoding with Online Self-Improvement for High-Concurrency LLM
//    Inference" (besthub.dev article), section "1. On-Policy Distillation (OPD) for Domain
//    Adaptation": reverse KL of the drafter p = softmax(z) against the target q = softmax(y), each
//    vocabulary term clipped from above before the sum, mixed with cross entropy on the target's
//    top-1 token; the drafter is what gets updated, so the gradient is taken with respect to z.
//  - same article, section "2. Adaptive Length Head for Token-Level Variance": greedy acceptance of
//    a drafted block within the predicted verification length L.
//  - same article, section "Infrastructure: ... Variable-Length Batching": packed ragged blocks.
//
// Design (MI355X): a streaming reduction, no dense contraction (so no MFMA). A 151,936-wide bf16 row
// is 297 KiB per tensor, more than one CU can hold, so a row is split over a *team* of G workgroups;
// each keeps its chunk resident for the whole row (z packed in VGPRs, y in LDS through direct
// buffer-to-LDS loads), so z and y are read from HBM once and dz written once:
//   phase A  per 16-byte vector: max z, max y, max(z - y), and sums of 2^(z log2e - r_z) and of
//            the same terms times (z - y); one running sum of 2^(y log2e - r_y) per lane. r_z, r_y
//            are the lane's first vector's fl(max log2e) (redone from the lane maxima in the rare lane
//            whose values climb more than 96 octaves above them)
//   chunk    maxima, sums rescaled to the chunk maxima
//   -- exchange 1 --  wave 0 publishes 4 values, gathers all members' and combines them in a fixed
//                     order: every member derives identical row constants
//   phase B  S and the clipped reverse KL: vectors whose bound is <= tau provably hold no clipped
//            term and use their phase-A sums; the rest (near the peak) are visited element by element.
//            A per-lane threshold on max z screens the vectors first, so that the bound and its exp2
//            are evaluated only near the peak. Then the chunk's lowest indices of the row maxima
//            (decoded only where a lane holds one)
//   -- exchange 2 --  the two sums, the two indices and z at the target top-1
//   phase C  dz written once (bf16 rounded to nearest even, or fp32)
// The kernel is VALU-heavy for an HBM stream (about 31 VALU instructions per element, 3.4 of them
// exponentials), so the per-element work is kept minimal and the per-row work (reductions,
// exchanges, row constants) runs once per workgroup in wave 0 while the other waves wait at
// barriers and the SIMDs serve the other resident workgroups. The waves of a CU's workgroups are in
// different phases of different rows, and the issue priority of each phase (s_setprio) orders them
// by how much of the team they hold up: the chunk reductions and both exchanges 3 (all G members
// of the team wait on them), phase B 2 (it feeds the second exchange), phase C 1 (it ends the row
// and frees the workgroup for its next loads), the issue of the next row's loads 2 (a short burst
// that must not wait behind the other workgroups), phase A 0. Exchanges use 8-byte
// [value | flag] units written and polled with agent-scope relaxed atomics (sc1: coherent across
// XCDs without L2 writeback / invalidate); the flag is unique per launch, row iteration and stage,
// so nothing has to be reset between launches and a stale unit can never be taken for a fresh one.
// Every wait is bounded and raises a sticky flag instead of hanging.

// Numerics: fp32 throughout with fixed reduction orders (bitwise deterministic). Per row, with
// M = max z, S_z = sum_v e^(z_v - M), delta = LSE(z) - LSE(y), t_v = p_v (z_v - y_v - delta):
//   clipped reverse KL = sum_v min(t_v, tau),  S = sum_v [t_v <= tau] p_v (t_v / p_v + 1),
//   dz_v = w p_v (alpha (z_v - y_v) + alpha (1 - delta - S) + 1 - alpha)  (unclipped)
//   dz_v = w p_v (1 - alpha - alpha S)                                     (clipped)
//   dz_a -= w (1 - alpha).
// p_v is evaluated from M and log S_z held apart (RowConst), so that large logits keep full fp32
// relative accuracy. Vectors proven free of clipped terms contribute to S and the reverse KL
// through their per-vector sums from phase A; vectors near the peak are summed element by element
// and left out of those sums (never subtracted from a total that held them, so there is no
// cancellation between the clipped terms and the rest). The clip decision is the same fp32
// test, from the same per-row floats, in the fused and the separate kernels, so fused and
// forward+backward results are bit-identical.

#include <stdint.h>

#include "opd_internal.h"

namespace opd {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();
constexpr int kBig = 0x7fffffff;

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }  // v_log_f32, normal x

// Work-item and workgroup ids straight from the hardware registers. The kernels are built with the
// IEEE mode bit clear, which the device library is not: its id helpers would not be inlined.
__device__ __forceinline__ int thread_id() { return (int)__builtin_amdgcn_workitem_id_x(); }
__device__ __forceinline__ int block_id_x() { return (int)__builtin_amdgcn_workgroup_id_x(); }
__device__ __forceinline__ int block_id_y() { return (int)__builtin_amdgcn_workgroup_id_y(); }

// ---------------------------------------------------------------- input formats (16-byte vectors)

struct F32In {
  static constexpr int EPV = 4;
  static constexpr int kWavesPerEU = 5;  // 5 workgroups per CU: LDS (27.9 KB each) allows no more
  // -32768 (exact in fp32 and bf16): never a maximum and e^(s - max) underflows to 0, because inputs
  // satisfy |logit| <= 1e4; small enough that s log2(e) keeps a tiny absolute rounding error (a
  // vector made only of sentinels is reduced relative to its own maximum, the sentinel itself).
  static constexpr uint32_t kSentinel = 0xC7000000u;
  __device__ static __forceinline__ void decode(const uint4& v, float (&x)[EPV]) {
    x[0] = __uint_as_float(v.x);
    x[1] = __uint_as_float(v.y);
    x[2] = __uint_as_float(v.z);
    x[3] = __uint_as_float(v.w);
  }
  __device__ static __forceinline__ uint32_t tail_word(uint32_t w, int j, int nvalid) {
    return j < nvalid ? w : kSentinel;
  }
};

struct BF16In {
  static constexpr int EPV = 8;
  static constexpr int kWavesPerEU = 6;  // 80 VGPRs and 26,844 B of LDS (53 allocation granules): 6 workgroups per CU
  static constexpr uint32_t kSentinel = 0xC700C700u;  // two bf16 -32768 (see F32In)
  __device__ static __forceinline__ float lo(uint32_t w) { return __uint_as_float(w << 16); }
  __device__ static __forceinline__ float hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
  __device__ static __forceinline__ void decode(const uint4& v, float (&x)[EPV]) {
    x[0] = lo(v.x);
    x[1] = hi(v.x);
    x[2] = lo(v.y);
    x[3] = hi(v.y);
    x[4] = lo(v.z);
    x[5] = hi(v.z);
    x[6] = lo(v.w);
    x[7] = hi(v.w);
  }
  __device__ static __forceinline__ uint32_t tail_word(uint32_t w, int j, int nvalid) {
    if (2 * j >= nvalid) return kSentinel;
    if (2 * j + 1 >= nvalid) return (w & 0xffffu) | (kSentinel & 0xffff0000u);
    return w;
  }
};

template <class In>
__device__ __forceinline__ void mask_tail(uint4& v, int nvalid) {
  v.x = In::tail_word(v.x, 0, nvalid);
  v.y = In::tail_word(v.y, 1, nvalid);
  v.z = In::tail_word(v.z, 2, nvalid);
  v.w = In::tail_word(v.w, 3, nvalid);
}

__device__ __forceinline__ uint4 splat4(uint32_t s) { return make_uint4(s, s, s, s); }

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Streaming (nontemporal) 16-byte load / store: the logits are read once and dz written once, so
// they are marked not to be kept in the caches.
__device__ __forceinline__ uint4 load_nt(const uint4* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void store_nt(uint8_t* p, uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  const u32x4 v = {a, b, c, d};
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}

// ---------------------------------------------------------------- output formats

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));  // v_cvt_pk_bf16_f32, RNE
}

template <bool OutBF16, int EPV>
__device__ __forceinline__ void store_vec(uint8_t* dst, const float (&o)[EPV]) {
  if constexpr (OutBF16) {
    if constexpr (EPV == 8) {
      store_nt(dst, pack_bf16(o[0], o[1]), pack_bf16(o[2], o[3]), pack_bf16(o[4], o[5]), pack_bf16(o[6], o[7]));
    } else {
      *(uint2*)dst = make_uint2(pack_bf16(o[0], o[1]), pack_bf16(o[2], o[3]));
    }
  } else {
#pragma unroll
    for (int q = 0; q < EPV / 4; ++q) {
      store_nt(dst + 16 * q, __float_as_uint(o[4 * q]), __float_as_uint(o[4 * q + 1]), __float_as_uint(o[4 * q + 2]),
               __float_as_uint(o[4 * q + 3]));
    }
  }
}

template <bool OutBF16, int EPV>
__device__ __forceinline__ void store_partial(uint8_t* dst, const float (&o)[EPV], int nvalid) {
#pragma unroll
  for (int e = 0; e < EPV; ++e) {
    if (e < nvalid) {
      if constexpr (OutBF16) {
        uint32_t pk = pack_bf16(o[e], 0.f);
        *(uint16_t*)(dst + 2 * e) = (uint16_t)(pk & 0xffffu);
      } else {
        *(float*)(dst + 4 * e) = o[e];
      }
    }
  }
}

// ---------------------------------------------------------------- buffer access

// Raw buffer resources (gfx9 descriptor word 3: 32-bit data format, no swizzle). Loads past
// num_records return 0 and stores past it are dropped, so the lanes of a slot that runs past the
// end of a chunk need neither a clamped address nor a branch.
constexpr int kRsrcWord3 = 0x00020000;
constexpr int kNT = 2;  // cache policy: nontemporal (the logits are read once, dz written once)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, kRsrcWord3);
}
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, int off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kNT);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void buf_store16(__amdgpu_buffer_rsrc_t r, int off, uint32_t a, uint32_t b, uint32_t c,
                                            uint32_t d) {
  const u32x4 v = {a, b, c, d};
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, kNT);
}
__device__ __forceinline__ void buf_store8(__amdgpu_buffer_rsrc_t r, int off, uint32_t a, uint32_t b) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  const u32x2 v = {a, b};
  __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, kNT);
}
// 16 bytes per lane straight into LDS: lane i of the wave lands at wave_base + 16 i.
__device__ __forceinline__ void buf_load16_lds(__amdgpu_buffer_rsrc_t r, int off, uint4* wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)wave_base, 16, off, 0, 0, kNT);
}

// dz of one 16-byte input vector (EPV values) through a buffer resource; `off` is the vector's byte
// offset in the output (EPV * OSZ bytes per vector).
template <bool OutBF16, int EPV>
__device__ __forceinline__ void buf_store_vec(__amdgpu_buffer_rsrc_t r, int off, const float (&o)[EPV]) {
  if constexpr (OutBF16) {
    if constexpr (EPV == 8) {
      buf_store16(r, off, pack_bf16(o[0], o[1]), pack_bf16(o[2], o[3]), pack_bf16(o[4], o[5]), pack_bf16(o[6], o[7]));
    } else {
      buf_store8(r, off, pack_bf16(o[0], o[1]), pack_bf16(o[2], o[3]));
    }
  } else {
#pragma unroll
    for (int q = 0; q < EPV / 4; ++q) {
      buf_store16(r, off + 16 * q, __float_as_uint(o[4 * q]), __float_as_uint(o[4 * q + 1]),
                  __float_as_uint(o[4 * q + 2]), __float_as_uint(o[4 * q + 3]));
    }
  }
}

// ---------------------------------------------------------------- cross-workgroup exchange

__device__ __forceinline__ void unit_store(uint64_t* p, uint32_t flag, uint32_t bits) {
  uint64_t u = ((uint64_t)flag << 32) | (uint64_t)bits;
  __hip_atomic_store(p, u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t unit_load(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wave 0 alone gathers the NU values of all G members into rx[c * NU + j]: each lane polls units
// ln, ln + 64, ... two at a time (both loads in flight together). Returns false (wave-uniformly) when
// a wait exceeded its bound.
template <int NU>
__device__ __forceinline__ bool gather_wave(uint32_t* rx, const uint64_t* units, int G, int ln, uint32_t flag,
                                            uint32_t limit) {
  const int n = G * NU;
  bool ok = true;
  for (int base = 0; base < n; base += 128) {
    const int i0 = base + ln, i1 = base + 64 + ln;
    bool d0 = i0 >= n, d1 = i1 >= n;
    const uint64_t* p0 = units + (size_t)(i0 / NU) * 8 + i0 % NU;
    const uint64_t* p1 = units + (size_t)(i1 / NU) * 8 + i1 % NU;
    uint32_t spins = 0;
    while (!(d0 && d1)) {
      const uint64_t u0 = d0 ? 0 : unit_load(p0);
      const uint64_t u1 = d1 ? 0 : unit_load(p1);
      if (!d0 && (uint32_t)(u0 >> 32) == flag) {
        rx[i0] = (uint32_t)u0;
        d0 = true;
      }
      if (!d1 && (uint32_t)(u1 >> 32) == flag) {
        rx[i1] = (uint32_t)u1;
        d1 = true;
      }
      if (d0 && d1) break;
      if (++spins > limit) {
        ok = false;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  return __builtin_amdgcn_ballot_w64(!ok) == 0;
}

// Wave 0 of every member publishes this chunk's NU values from LDS (lanes 0..NU-1, one unit each).
template <int NU>
__device__ __forceinline__ void publish(uint64_t* units, int lane, uint32_t flag, const uint32_t* vals) {
  if (lane < NU) unit_store(units + lane, flag, vals[lane]);
}

// LDS shared by the waves of a workgroup (the chunk of y lives in its own array).
template <int RX>
struct Shared {
  uint32_t rx[RX];  // gathered member values (wave 0)
  uint32_t part[8];  // this chunk's values to publish
  float wred[4][4];  // per-wave partials
  int widx[4][2];    // per-wave first argmax of z and y
  float wza[4];      // z at the wave's argmax of y
  float row[12];     // row constants, written by wave 0
  float pend[5];     // forward mode, chunk 0: row constants of the row whose exchange 2 is pending
  int pend_row;
  uint32_t pend_flag;
  int err;
  int last;          // this workgroup is the last of the launch to finish (device-epoch launches)
  uint32_t fbase;    // first exchange flag of this launch
};

// Row constants in Shared::row.
enum RowSlot : int {
  kRowMz = 0, kRowLnSz, kRowDelta, kRowMy, kRowLnSy, kRowDtop, kRowAtop, kRowZa, kRowS, kRowRkl
};

// ---------------------------------------------------------------- wave reductions (DPP)

// Full-wave reductions: four in-row steps on the DPP crossbar (quad_perm, half-row and row mirrors),
// each folded by the compiler into one VALU op with a DPP source (the move's old value is left
// undefined: every lane of these patterns has a valid source), then the two cross-row steps with the
// gfx950 lane swaps (v_permlane32_swap: halves of the wave; v_permlane16_swap: rows within each half).
// Every lane ends with the result; it is read from the first active lane.
template <int CTRL>
__device__ __forceinline__ int dpp_row(int v) {
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, true);
}
__device__ __forceinline__ void swap32(int v, int& a, int& b) {
  const auto p = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  a = (int)p[0];
  b = (int)p[1];
}
__device__ __forceinline__ void swap16(int v, int& a, int& b) {
  const auto p = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  a = (int)p[0];
  b = (int)p[1];
}
__device__ __forceinline__ float uniform_f(float v) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v)));
}
__device__ __forceinline__ float wmax(float v) {
  v = fmaxf(v, __int_as_float(dpp_row<0xB1>(__float_as_int(v))));
  v = fmaxf(v, __int_as_float(dpp_row<0x4E>(__float_as_int(v))));
  v = fmaxf(v, __int_as_float(dpp_row<0x141>(__float_as_int(v))));
  v = fmaxf(v, __int_as_float(dpp_row<0x140>(__float_as_int(v))));
  int a, b;
  swap32(__float_as_int(v), a, b);
  v = fmaxf(__int_as_float(a), __int_as_float(b));
  swap16(__float_as_int(v), a, b);
  return uniform_f(fmaxf(__int_as_float(a), __int_as_float(b)));
}
// Fixed order: ((row 0 + row 2) + (row 1 + row 3)) of the in-row sums, the same on every call.
__device__ __forceinline__ float wsum(float v) {
  v = v + __int_as_float(dpp_row<0xB1>(__float_as_int(v)));
  v = v + __int_as_float(dpp_row<0x4E>(__float_as_int(v)));
  v = v + __int_as_float(dpp_row<0x141>(__float_as_int(v)));
  v = v + __int_as_float(dpp_row<0x140>(__float_as_int(v)));
  int a, b;
  swap32(__float_as_int(v), a, b);
  v = __int_as_float(a) + __int_as_float(b);
  swap16(__float_as_int(v), a, b);
  return uniform_f(__int_as_float(a) + __int_as_float(b));
}
__device__ __forceinline__ int wmin(int v) {
  v = min(v, dpp_row<0xB1>(v));
  v = min(v, dpp_row<0x4E>(v));
  v = min(v, dpp_row<0x141>(v));
  v = min(v, dpp_row<0x140>(v));
  int a, b;
  swap32(v, a, b);
  v = min(a, b);
  swap16(v, a, b);
  return __builtin_amdgcn_readfirstlane(min(a, b));
}

// Two independent full-wave reductions in one register (all 64 lanes active): v_permlane32_swap
// between the two values leaves a's lanes l and l + 32 in lane l < 32 and b's in lane l + 32, so one
// combine halves both; v_permlane16_swap then brings the two rows of each half together, and four
// in-row DPP steps finish: lane 0 holds a's result, lane 32 b's. Half the instructions of two single
// reductions. Sums in a fixed order: for each lane l of a row, (x_l + x_{l+32}) + (x_{l+16} + x_{l+48}),
// then the in-row steps.
template <class F>
__device__ __forceinline__ int wreduce2(int a, int b, F op, int& rb) {
  const auto p = __builtin_amdgcn_permlane32_swap(a, b, false, false);  // {[a_lo, b_lo], [a_hi, b_hi]}
  int v = op((int)p[0], (int)p[1]);
  const auto q = __builtin_amdgcn_permlane16_swap(v, v, false, false);  // rows 0|1 and 2|3 of each half
  v = op((int)q[0], (int)q[1]);
  v = op(v, dpp_row<0xB1>(v));
  v = op(v, dpp_row<0x4E>(v));
  v = op(v, dpp_row<0x141>(v));
  v = op(v, dpp_row<0x140>(v));
  rb = __builtin_amdgcn_readlane(v, 32);
  return __builtin_amdgcn_readlane(v, 0);
}
__device__ __forceinline__ void wsum2(float& a, float& b) {
  int rb;
  const int ra = wreduce2(__float_as_int(a), __float_as_int(b),
                          [](int x, int y) { return __float_as_int(__int_as_float(x) + __int_as_float(y)); }, rb);
  a = __int_as_float(ra);
  b = __int_as_float(rb);
}
__device__ __forceinline__ void wmax2(float& a, float& b) {
  int rb;
  const int ra = wreduce2(__float_as_int(a), __float_as_int(b),
                          [](int x, int y) { return __float_as_int(fmaxf(__int_as_float(x), __int_as_float(y))); }, rb);
  a = __int_as_float(ra);
  b = __int_as_float(rb);
}
__device__ __forceinline__ void wmin2(int& a, int& b) {
  int rb;
  a = wreduce2(a, b, [](int x, int y) { return min(x, y); }, rb);
  b = rb;
}

// ---------------------------------------------------------------- per-row constants

// Probability of a logit x under the row's softmax, p(x) = exp(x - LSE(z)), evaluated as
// exp2(fma(x, log2 e, -c_hi) - c_lo) with c_hi + c_lo = M_z log2 e + log2 S_z carried in two floats:
// fma forms x log2 e - c_hi with a single rounding, so p keeps full fp32 relative accuracy even for
// logits in the thousands (a single fp32 constant LSE log2 e would be off by up to half an ulp of
// ~1.4e4, i.e. 1e-3 in p). This canonical p is used for every clip decision, in the fused kernel
// and in the separate backward kernel, from the same stored floats, so their decisions agree.
struct RowConst {
  float c_hi, c_lo;  // p(x) = exp2(fma(x, log2e, -c_hi) - c_lo)
  float delta;       // LSE(z) - LSE(y)
  __device__ __forceinline__ void init(float m_z, float ln_sz, float d) {
    c_hi = m_z * kLog2e;
    c_lo = __builtin_fmaf(m_z, kLog2e, -c_hi) + ln_sz * kLog2e;
    delta = d;
  }
  __device__ __forceinline__ float p(float x) const {
    return exp2_fast(__builtin_fmaf(x, kLog2e, -c_hi) - c_lo);
  }
  // p(x) 2^c_lo: dz folds the factor 2^-c_lo into its coefficients (one op less per element)
  __device__ __forceinline__ float e(float x) const { return exp2_fast(__builtin_fmaf(x, kLog2e, -c_hi)); }
};

// dz_v = w p_v (alpha (z_v - y_v) + alpha (1 - delta - S) + 1 - alpha) for an unclipped term,
// w p_v (1 - alpha - alpha S) for a clipped one, minus w (1 - alpha) at the target top-1.
struct DzConst {
  float wa, k0, kc;  // scaled by 2^-c_lo (see RowConst::e)
  float wce;
  __device__ __forceinline__ void init(const RowConst& rc, float S, float alpha, float w) {
    const float f = exp2_fast(-rc.c_lo);
    wa = (w * alpha) * f;
    k0 = (w * (alpha * ((1.f - rc.delta) - S) + (1.f - alpha))) * f;
    kc = (w * ((1.f - alpha) - alpha * S)) * f;
    wce = w * (1.f - alpha);
  }
};

// Vector bound of phase B: every term t_v = p(x_v) ((x_v - y_v) - delta) of a 16-byte vector is at
// most p(max x) max(max(x - y) - delta, 0). p(max x) is replaced by sc = 2^(fl(max x log2 e) - c_hi -
// c_lo), the factor that also scales the vector's phase-A sums; the two differ by a factor below
// 1.003 for |x| <= 1e4, so the test runs against tau / 1.01: a vector that passes holds no term above
// tau (max x is kept rounded up for fp32 inputs, which only raises sc). The same test, from the same
// floats, runs in the fused and the backward kernels.
constexpr float kBoundShrink = 1.f / 1.01f;
__device__ __forceinline__ float vector_scale(const RowConst& rc, float zmax) {
  return exp2_fast((zmax * kLog2e - rc.c_hi) - rc.c_lo);
}
__device__ __forceinline__ bool vector_may_clip(const RowConst& rc, float sc, float dmax, float tau_b) {
  return sc * fmaxf(dmax - rc.delta, 0.f) > tau_b;
}

// dz of one 16-byte vector. `slow` marks a lane whose vector may hold clipped terms (its bound
// exceeds tau); `any_slow` is the wave-uniform OR of it, so the clip tests run only in waves that
// need them. Shared by the fused and the backward kernels (bit-identical results).
template <int EPV>
__device__ __forceinline__ void dz_vector(const float (&x)[EPV], const float (&w)[EPV], bool slow, bool any_slow,
                                          const RowConst& rc, const DzConst& dc, float tau, float (&o)[EPV]) {
#pragma unroll
  for (int e = 0; e < EPV; ++e) o[e] = rc.e(x[e]) * __builtin_fmaf(dc.wa, x[e] - w[e], dc.k0);
  if (any_slow) {
#pragma unroll
    for (int e = 0; e < EPV; ++e) {
      const bool clip = slow && (rc.p(x[e]) * ((x[e] - w[e]) - rc.delta) > tau);
      o[e] = clip ? rc.e(x[e]) * dc.kc : o[e];
    }
  }
}

template <int EPV>
__device__ __forceinline__ void fix_target(float (&o)[EPV], int g0, int atop, float wce) {
  const unsigned rel = (unsigned)(atop - g0);
  if (rel < (unsigned)EPV) {
#pragma unroll
    for (int e = 0; e < EPV; ++e) o[e] = ((unsigned)e == rel) ? o[e] - wce : o[e];
  }
}

// Keeps the packed inputs opaque between phases so that the compiler re-decodes them (1 VALU op per
// element) instead of keeping decoded fp32 copies alive across the exchanges (which doubles the VGPR
// footprint and halves occupancy).
__device__ __forceinline__ void opaque(uint4& v) {
  __asm__ volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w));
}
// Ends a slot: the slot's results must exist here, so the scheduler cannot interleave all K slots
// (which keeps every slot's decoded inputs and exponentials live at once).
__device__ __forceinline__ void fence_vals(float& a) { __asm__ volatile("" : "+v"(a)); }
__device__ __forceinline__ void fence_vals(float& a, float& b) { __asm__ volatile("" : "+v"(a), "+v"(b)); }
__device__ __forceinline__ void fence_vals(float& a, float& b, float& c) {
  __asm__ volatile("" : "+v"(a), "+v"(b), "+v"(c));
}
__device__ __forceinline__ void fence_vals(float& a, float& b, float& c, float& d) {
  __asm__ volatile("" : "+v"(a), "+v"(b), "+v"(c), "+v"(d));
}


// Per-vector maxima kept from phase A to phase B: max z and max(z - y), both in one 32-bit word as
// two bf16. max(z - y) is rounded up, which only loosens the phase-B bound; so is max z for fp32
// inputs (for bf16 inputs it is itself a bf16 value, exact). The backward kernel applies the same
// roundings, so the two kernels decide alike. Where the exact max z is needed (the top-1 search), it
// comes from the resident chunk for fp32 inputs (slot_holds_max).
__device__ __forceinline__ uint32_t bf16_bits_up(float d) {  // bits of the least bf16 >= d (finite d)
  const uint32_t u = __float_as_uint(d);
  return (int32_t)u >= 0 ? (u + 0xffffu) & 0xffff0000u : u & 0xffff0000u;
}
template <int EPV>
struct VecMax {
  uint32_t pk;  // [max(z - y) rounded up : 16][max z rounded up : 16]
  __device__ __forceinline__ void set(float z, float d) { pk = (bf16_bits_up(z) >> 16) | bf16_bits_up(d); }
  __device__ __forceinline__ float z() const { return __uint_as_float(pk << 16); }
  __device__ __forceinline__ float d() const { return __uint_as_float(pk & 0xffff0000u); }
  __device__ __forceinline__ void fence() { __asm__ volatile("" : "+v"(pk)); }
};
template <>
struct VecMax<8> {
  uint32_t pk;  // [max(z - y) rounded up : 16][max z : 16]
  __device__ __forceinline__ void set(float z, float d) { pk = (__float_as_uint(z) >> 16) | bf16_bits_up(d); }
  __device__ __forceinline__ float z() const { return __uint_as_float(pk << 16); }
  __device__ __forceinline__ float d() const { return __uint_as_float(pk & 0xffff0000u); }
  __device__ __forceinline__ void fence() { __asm__ volatile("" : "+v"(pk)); }
};
// The bound's max(z - y) and max z as the fused kernel keeps them (see VecMax).
template <int EPV>
__device__ __forceinline__ float kept_dmax(float d) {
  return __uint_as_float(bf16_bits_up(d));
}
template <int EPV>
__device__ __forceinline__ float kept_zmax(float z) {
  if constexpr (EPV == 8) return z;
  else return __uint_as_float(bf16_bits_up(z));
}

// Sum of the EPV values of a vector in a fixed pairwise order.
template <int EPV>
__device__ __forceinline__ float vsum(const float (&v)[EPV]) {
  if constexpr (EPV == 8) return ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
  else return (v[0] + v[1]) + (v[2] + v[3]);
}
template <int EPV>
__device__ __forceinline__ float vmax(const float (&v)[EPV]) {
  float m = fmaxf(v[0], v[1]);
#pragma unroll
  for (int e = 2; e < EPV; ++e) m = fmaxf(m, v[e]);
  return m;
}
// First e with v[e] == m (EPV if none).
template <int EPV>
__device__ __forceinline__ int first_eq(const float (&v)[EPV], float m) {
  int e0 = EPV;
#pragma unroll
  for (int e = EPV - 1; e >= 0; --e) e0 = (v[e] == m) ? e : e0;
  return e0;
}

// Whether a vector holds the value m as its maximum of z: from the kept maximum where that is exact
// (bf16 inputs), else from the resident vector itself.
template <class In>
__device__ __forceinline__ bool holds_zmax(const VecMax<In::EPV>& v, const uint4& raw, float m) {
  if constexpr (In::EPV == 8) {
    return v.z() == m;
  } else {
    float x[In::EPV];
    In::decode(raw, x);
    return vmax<In::EPV>(x) == m;
  }
}

// Sums of one vector's terms relative to a lane reference: se = sum 2^(x log2e - ref), sb = sum of
// the same terms times d. Phase A and the element-by-element path of phase B call it with the same
// operands and get the same floats.
template <int EPV>
__device__ __forceinline__ void vec_sums(const float (&x)[EPV], const float (&d)[EPV], float ref, float& se,
                                         float& sb) {
  float ez = exp2_fast(__builtin_fmaf(x[0], kLog2e, -ref));
  se = ez;
  sb = ez * d[0];
#pragma unroll
  for (int e = 1; e < EPV; ++e) {
    ez = exp2_fast(__builtin_fmaf(x[e], kLog2e, -ref));
    se += ez;
    sb = __builtin_fmaf(ez, d[e], sb);
  }
}

// Sum of the per-vector values v[k] of a lane in slot order; the second form leaves out the slots
// whose `skip` is set (each a lane mask, so a slot costs one select).
template <int K>
__device__ __forceinline__ float lane_sum(const float (&v)[K]) {
  float a = v[0];
#pragma unroll
  for (int k = 1; k < K; ++k) a += v[k];
  return a;
}
template <int K>
__device__ __forceinline__ float lane_sum(const float (&v)[K], const bool (&skip)[K]) {
  float a = skip[0] ? 0.f : v[0];
#pragma unroll
  for (int k = 1; k < K; ++k) a += skip[k] ? 0.f : v[k];
  return a;
}

// ---------------------------------------------------------------- the row-team kernel
//
// A team of G workgroups owns a row; workgroup `chunk` owns vectors [cv0, cv0 + clen) of it, each
// thread the vectors cv0 + tid + 256 k, k < K. Per row:
//   load     z chunk into VGPRs (packed), y chunk into LDS (direct buffer-to-LDS loads)
//   phase A  per vector: max z, max y, max(z - y), E_k = sum 2^(z log2e - c_k), B_k = sum of the same
//            terms times (z - y), with c_k = fl(max z log2e); per lane: sum of 2^(y log2e - r) with r
//            the first vector's fl(max y log2e) (recomputed from the lane maximum if y climbs more
//            than 96 octaves above it)
//   chunk    maxima, sums rescaled to the chunk maxima (top-1 mode: the lowest indices of the chunk
//            maxima instead of sums)
//   team     wave 0 publishes the chunk's 4 values, gathers the G members' values and forms the row
//            constants (exchange 1)
//   phase B  S and the clipped reverse KL (vector bound; element by element near the peak), then the
//            chunk's lowest indices of the row maxima of z and y and z at the latter (kBig where the
//            chunk does not reach a row maximum: usually only one member of the team decodes);
//            wave 0 exchanges these 5 values (exchange 2) and writes the row outputs (chunk 0)
//   phase C  dz of every vector of the chunk
// Waves other than wave 0 wait at the barriers while wave 0 exchanges: the SIMDs run the other
// resident workgroups meanwhile.

typedef __attribute__((address_space(4))) const TeamParams KParams;

template <class In, bool OutBF16, int K, int MODE, bool DevFlags>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(In::kWavesPerEU))) k_team(TeamParams P) {
  constexpr int EPV = In::EPV;
  constexpr int VB = EPV * (OutBF16 ? 2 : 4);  // dz bytes per input vector
  constexpr bool kSums = MODE != kTop1;
  // Members of a team at most (the widest row, 2^19 logits, in chunks of K * 256 vectors), each with
  // up to kStage1Units values: the gather buffer is sized for this instantiation only, so that a bf16
  // workgroup with K = 5 stays within 53 LDS allocation granules (27,136 B) and six fit on a CU.
  constexpr int kMaxG = (kMaxVocab / EPV + K * kThreads - 1) / (K * kThreads) < kMaxTeamSize
                            ? (kMaxVocab / EPV + K * kThreads - 1) / (K * kThreads) : kMaxTeamSize;
  __shared__ Shared<kMaxG * kStage1Units> sh;
  // The row chunk of y lives in LDS, z in VGPRs: this keeps the register footprint within 5
  // workgroups per CU (more resident teams hide the exchange waits). Each lane only ever reads back
  // its own 16 bytes.
  __shared__ uint4 ylds[K * kThreads];
  __shared__ VecMax<EPV> vmlds[K * kThreads];  // per-vector maxima from phase A to phase B
  const int tid = thread_id();
  // the wave index lives in a scalar register; per-row lane indices are rebuilt from it and the lane
  // number (mbcnt) instead of keeping the work-item id in a vector register for the whole kernel
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Consecutive workgroups form a team, so its members land on different XCDs (round-robin dispatch)
  // and the five workgroups sharing a CU belong to different teams. Forming teams in the order the
  // workgroups start instead (a ticket counter in the workspace) measured 4-10 % slower: the start
  // order clusters members on few XCDs. The grid is sized for an otherwise idle device; a team whose
  // members are not all resident waits on its bound and raises OPD_FLAG_SPIN_TIMEOUT.
  const int b = block_id_x();
  const int team = b / P.G;
  const int chunk = b % P.G;
  const int G = P.G;
  const int cv0 = chunk * P.chunk_vec;
  const int clen0 = min(P.chunk_vec, P.nvec - cv0);  // vectors in this chunk (uniform)
  const bool tail_chunk = (cv0 + clen0 == P.nvec) && (P.nvec * EPV != P.vocab);
  // this team's units: exchange 1 of even / odd row iterations in stages 0 / 1, exchange 2 in stage 2
  uint64_t* const units_team = P.units + (size_t)team * kStages * G * 8;
  uint64_t* const units2 = units_team + (size_t)2 * G * 8;
  // Exchange flags are base + 1 .. base + flag_count. An eager call gets its range from the host
  // (flag_base, flags >= 2^31). A call captured into a graph, whose kernel arguments are frozen for
  // every replay, runs the DevFlags instantiation, which takes the range from the epoch in the
  // workspace header instead (flags < 2^31); the previous device-flag launch on this workspace
  // advanced it when its last workgroup finished. Either way no launch uses a flag an earlier one
  // left in the units; the epoch restarts at 0 rather than let a range pass 2^31 - 1.
  if (tid == 0) {
    uint32_t b = P.flag_base;
    if constexpr (DevFlags) {
      const uint32_t e = __hip_atomic_load(P.flags + kEpochWord, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      b = (uint64_t)e + P.flag_count + 1u > 0x7fffffffull ? 0u : e;
    }
    sh.err = 0;
    sh.fbase = b + 1u;
  }

  // Exchange 2 of one row, wave 0: combines the members' values (gathered into sh.rx, or this chunk's
  // own when the row has one member) in a fixed order and, in chunk 0, writes the row's outputs.
  // Returns S, the clipped sum and the target top-1 through sh.row for phase C.
  auto finish_row = [&](KParams* pp, int r, bool gathered, int ln_, int z0_, float Mz_, float ln_sz_, float My_,
                        float ln_sy_, float delta_, float alpha_) {
    float S = __uint_as_float(sh.part[z0_ + 0]), rkl = __uint_as_float(sh.part[z0_ + 1]);
    int dtop = (int)sh.part[z0_ + 2], atop = (int)sh.part[z0_ + 3];
    float za = __uint_as_float(sh.part[z0_ + 4]);
    if (gathered) {
      float ls = 0.f, lr = 0.f, lza = 0.f;
      int liz = kBig, liy = kBig;
      for (int c = ln_; c < G; c += 64) {
        const uint32_t* u = sh.rx + z0_ + c * kStage2Units;
        ls += __uint_as_float(u[0]);
        lr += __uint_as_float(u[1]);
        liz = min(liz, (int)u[2]);
        if ((int)u[3] < liy) {
          liy = (int)u[3];
          lza = __uint_as_float(u[4]);
        }
      }
      wsum2(ls, lr);
      S = ls;
      rkl = lr;
      dtop = liz;
      atop = liy;
      wmin2(dtop, atop);
      za = wsum(liy == atop ? lza : 0.f);
    }
    if (ln_ == 0) {
      sh.row[z0_ + kRowS] = S;
      sh.row[z0_ + kRowRkl] = rkl;
      sh.row[z0_ + kRowAtop] = __int_as_float(atop);
      if (chunk == 0) {
        const float ce = (Mz_ - za) + ln_sz_;
        float* st = pp->row_stats + 8 * (int64_t)r;
        pp->loss[r] = alpha_ * rkl + (1.f - alpha_) * ce;
        pp->target_top1[r] = atop;
        if (pp->draft_top1) pp->draft_top1[r] = dtop;
        st[0] = Mz_ + ln_sz_;
        st[1] = My_ + ln_sy_;
        st[2] = S;
        st[3] = rkl;
        st[4] = Mz_;
        st[5] = ln_sz_;
        st[6] = delta_;
        st[7] = ce;
      }
    }
  };
  // Forward mode: no member needs the row's sums, so none waits for exchange 2; chunk 0 gathers a
  // row's exchange 2 when its next row is about to publish exchange 1 (every member published its
  // exchange 2 before starting the next row, so that gather does not wait), and after its last row.
  // Exchange 2 keeps one stage: a member overwrites it only after gathering the next exchange 1,
  // which includes chunk 0's, published after chunk 0 has read the pending values.
  auto finish_pending = [&](KParams* pp, int ln_, int z0_) -> bool {
    const bool ok = gather_wave<kStage2Units>(sh.rx + z0_, units2, G, ln_, sh.pend_flag, pp->spin_limit);
    if (ok) finish_row(pp, sh.pend_row, true, ln_, z0_, sh.pend[0], sh.pend[1], sh.pend[2], sh.pend[3], sh.pend[4],
                       pp->alpha);
    return ok;
  };

  int iter = 0;
  for (int row = team; row < P.n_rows; row += P.n_teams, ++iter) {
    __syncthreads();  // the previous row is done with ylds and sh
    // The row's loads go out at a raised issue priority (their address arithmetic must not wait
    // behind the other workgroups' phases); phase A then runs at the lowest.
    __builtin_amdgcn_s_setprio(2);
    // Kernel arguments are re-read (scalar loads) in every row instead of occupying scalar registers
    // for the whole loop.
    KParams* pp = (KParams*)__builtin_amdgcn_kernarg_segment_ptr();
    __asm__ volatile("" : "+s"(pp));
    // LDS fields are addressed from an opaque zero that is re-derived every row: one base register
    // plus instruction offsets, instead of one register per field address held across the loop.
    int z0 = 0;
    __asm__ volatile("" : "+v"(z0));
    // Chunk length made opaque per row: per-slot tests are then evaluated where they are used instead
    // of being hoisted out of the row loop and kept live in scalar registers.
    int clen = clen0;
    __asm__ volatile("" : "+s"(clen));
    // one buffer resource per tensor and row, bounded by the chunk: lanes of a slot past the chunk
    // end read 0 (replaced by the sentinel below)
    const __amdgpu_buffer_rsrc_t rz = rsrc(pp->z + (int64_t)row * pp->ld_bytes + (int64_t)cv0 * 16, clen * 16);
    const __amdgpu_buffer_rsrc_t ry = rsrc(pp->y + (int64_t)row * pp->ld_bytes + (int64_t)cv0 * 16, clen * 16);
    // The ln index is made opaque once per row: otherwise the compiler hoists every per-slot and
    // per-element ln test (sentinels, validity, offsets) out of the row loop and keeps them all
    // live in registers.
    // (mbcnt counts from the opaque zero, so that the lane number is not hoisted out of the loop
    // and held across it either)
    int lt = (wave << 6) + (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, (uint32_t)z0));
    __asm__ volatile("" : "+v"(lt));
    const int voff = lt * 16;
    const int ln = lt & 63, wv = lt >> 6;
    const float alpha = pp->alpha, tau = pp->tau, tau_b = tau * kBoundShrink;
    uint4 zr[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {  // every load of the chunk in flight at once
      zr[k] = buf_load16(rz, voff + k * (16 * kThreads));
      buf_load16_lds(ry, voff + k * (16 * kThreads), ylds + k * kThreads + wave * 64);
    }
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
    for (int k = 0; k < K; ++k) {
      opaque(zr[k]);
      if ((k + 1) * kThreads > clen) {  // uniform: only slots that run past the chunk end
        if (lt + k * kThreads >= clen) {
          zr[k] = splat4(In::kSentinel);
          ylds[k * kThreads + lt] = splat4(In::kSentinel);
        }
      }
    }
    if (tail_chunk) {  // uniform: only the chunk holding a partial last vector
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const int vi = cv0 + lt + k * kThreads;
        if (vi == pp->nvec - 1) {
          uint4 yv = ylds[k * kThreads + lt];
          mask_tail<In>(zr[k], pp->vocab - vi * EPV);
          mask_tail<In>(yv, pp->vocab - vi * EPV);
          ylds[k * kThreads + lt] = yv;
        }
      }
    }

    // ---- phase A
    // Per lane: the maxima of z, y and z - y over its vectors, and three sums relative to the lane's
    // own references (2^fl(max log2 e) of its first vector's z and y): of 2^(z log2e - ref_z), of
    // the same terms times (z - y), and of 2^(y log2e - ref_y). A lane whose maximum climbs more than
    // 96 octaves above its first vector's redoes its sums from its maximum (rare: the terms could
    // otherwise approach the end of the fp32 range).
    float lzmax = kNegInf, ldmax = kNegInf;
    float ek[K], bk[K];  // per-vector sums relative to ref_z
    float ref_z = 0.f;
    float lymax = kNegInf, sy = 0.f, ref_y = 0.f;
    int kym = 0;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      opaque(zr[k]);
      float x[EPV], w[EPV], d[EPV];
      In::decode(zr[k], x);
      In::decode(ylds[k * kThreads + lt], w);
      const float ym = vmax<EPV>(w);
      kym = (k == 0 || ym > lymax) ? k : kym;  // first slot holding the lane's maximum of y
      lymax = fmaxf(lymax, ym);
      if constexpr (kSums) {
        if (k == 0) ref_y = ym * kLog2e;
        float s2 = exp2_fast(__builtin_fmaf(w[0], kLog2e, -ref_y));
#pragma unroll
        for (int e = 1; e < EPV; ++e) s2 += exp2_fast(__builtin_fmaf(w[e], kLog2e, -ref_y));
        sy = k == 0 ? s2 : sy + s2;
      }
#pragma unroll
      for (int e = 0; e < EPV; ++e) d[e] = x[e] - w[e];
      const float zmax = vmax<EPV>(x), dmax = vmax<EPV>(d);
      {
        VecMax<EPV> vk;
        vk.set(zmax, dmax);
        vmlds[k * kThreads + lt] = vk;  // kept in LDS until phase B (registers are the scarce resource)
      }
      lzmax = fmaxf(lzmax, zmax);
      if constexpr (kSums) {
        ldmax = fmaxf(ldmax, dmax);
        if (k == 0) ref_z = zmax * kLog2e;
        vec_sums<EPV>(x, d, ref_z, ek[k], bk[k]);
        fence_vals(ek[k], bk[k], sy);
      }
      fence_vals(lzmax);
      fence_vals(lymax);
    }
    if constexpr (kSums) {
      const bool redo_z = lzmax * kLog2e - ref_z > 96.f;
      const bool redo_y = lymax * kLog2e - ref_y > 96.f;
      if (__builtin_amdgcn_ballot_w64(redo_z || redo_y)) {
        if (redo_z) {
          ref_z = lzmax * kLog2e;
#pragma unroll
          for (int k = 0; k < K; ++k) {
            opaque(zr[k]);
            float x[EPV], w[EPV], d[EPV];
            In::decode(zr[k], x);
            In::decode(ylds[k * kThreads + lt], w);
#pragma unroll
            for (int e = 0; e < EPV; ++e) d[e] = x[e] - w[e];
            vec_sums<EPV>(x, d, ref_z, ek[k], bk[k]);
            fence_vals(ek[k], bk[k]);
          }
        }
        if (redo_y) {
          ref_y = lymax * kLog2e;
          sy = 0.f;
#pragma unroll
          for (int k = 0; k < K; ++k) {
            float w[EPV], ey[EPV];
            In::decode(ylds[k * kThreads + lt], w);
#pragma unroll
            for (int e = 0; e < EPV; ++e) ey[e] = exp2_fast(__builtin_fmaf(w[e], kLog2e, -ref_y));
            sy += vsum<EPV>(ey);
          }
        }
      }
    }

    // ---- chunk maxima
    // From here to the end of the first exchange this team's row is on the critical path of all
    // G workgroups of the team: the waves take the highest issue priority, above every phase of
    // the other workgroups sharing the CU, and drop it once the row constants arrive.
    __builtin_amdgcn_s_setprio(3);
    {
      float a = lzmax, c = lymax;
      wmax2(a, c);
      if (ln == 0) {
        sh.wred[wv][z0 + 0] = a;
        sh.wred[wv][z0 + 1] = c;
      }
    }
    __syncthreads();
    const float Mzc = fmaxf(fmaxf(sh.wred[0][z0 + 0], sh.wred[1][z0 + 0]), fmaxf(sh.wred[2][z0 + 0], sh.wred[3][z0 + 0]));
    const float Myc = fmaxf(fmaxf(sh.wred[0][z0 + 1], sh.wred[1][z0 + 1]), fmaxf(sh.wred[2][z0 + 1], sh.wred[3][z0 + 1]));

    // ---- sums relative to 2^fl(chunk max log2 e), lowest indices of the chunk maxima
    float wsz = 0.f, wsy = 0.f;
    if constexpr (kSums) {
      const float cMz = Mzc * kLog2e, cMy = Myc * kLog2e;
      wsz = lane_sum<K>(ek) * exp2_fast(ref_z - cMz);
      wsy = sy * exp2_fast(ref_y - cMy);
      wsum2(wsz, wsy);
    }
    int wiz = kBig, wiy = kBig;
    float wza = 0.f;
    if constexpr (!kSums) {  // top-1 mode: the chunk's lowest indices of its maxima go into exchange 1
      const bool hz = lzmax == Mzc;
      if (__builtin_amdgcn_ballot_w64(hz)) {  // a wave holding the chunk maximum of z
        int kk = K;
#pragma unroll
        for (int k = K - 1; k >= 0; --k) kk = holds_zmax<In>(vmlds[k * kThreads + lt], zr[k], Mzc) ? k : kk;
        int iz = kBig;
#pragma unroll
        for (int k = 0; k < K; ++k) {
          if (__builtin_amdgcn_ballot_w64(hz && kk == k)) {
            if (hz && kk == k) {
              float x[EPV];
              In::decode(zr[k], x);
              iz = (cv0 + lt + k * kThreads) * EPV + first_eq<EPV>(x, Mzc);
            }
          }
        }
        wiz = wmin(iz);
      }
      const bool hy = lymax == Myc;
      if (__builtin_amdgcn_ballot_w64(hy)) {
        const int kk = kym;
        int iy = kBig;
        float za = 0.f;
#pragma unroll
        for (int k = 0; k < K; ++k) {
          if (__builtin_amdgcn_ballot_w64(hy && kk == k)) {
            if (hy && kk == k) {
              float x[EPV], w[EPV];
              In::decode(zr[k], x);
              In::decode(ylds[k * kThreads + lt], w);
              const int e0 = first_eq<EPV>(w, Myc);
              float zv = x[0];
#pragma unroll
              for (int e = 1; e < EPV; ++e) zv = (e == e0) ? x[e] : zv;
              iy = (cv0 + lt + k * kThreads) * EPV + e0;
              za = zv;
            }
          }
        }
        wiy = wmin(iy);
        wza = wsum(iy == wiy ? za : 0.f);  // the ln holding the index (unique)
      }
    }
    if (ln == 0) {
      sh.wred[wv][z0 + 2] = wsz;
      sh.wred[wv][z0 + 3] = wsy;
      sh.widx[wv][z0 + 0] = wiz;
      sh.widx[wv][z0 + 1] = wiy;
      sh.wza[z0 + wv] = wza;
    }
    __syncthreads();

    // ---- exchange 1: wave 0 publishes the chunk values, gathers the members' values and forms the
    // row constants; the other waves wait at the barrier
    const uint32_t flag1 = sh.fbase + 2u * (uint32_t)iter;
    // Exchange 1 alternates between two stages by row parity. In the forward and top-1 modes a member
    // may finish its row (and publish the next row's exchange 1) before a slower member has gathered
    // this row's values: with one stage it would overwrite them. Two rows later the slot is free
    // again, because this member's gather of the row in between waited for every member to publish
    // it, which each does only after finishing this row.
    uint64_t* const units1 = units_team + (size_t)(iter & 1) * G * 8;
    // values per member in exchange 1: maxima and sums (the top-1 indices follow in exchange 2), or
    // in top-1 mode the maxima and their lowest indices
    constexpr int NU1 = kSums ? 4 : kStage1Units;
    constexpr int kMy = kSums ? 2 : 1;  // where a member's maximum of y sits among its NU1 values
    if (wave == 0) {
      {
        const float sz = (sh.wred[0][z0 + 2] + sh.wred[1][z0 + 2]) + (sh.wred[2][z0 + 2] + sh.wred[3][z0 + 2]);
        const float sy2 = (sh.wred[0][z0 + 3] + sh.wred[1][z0 + 3]) + (sh.wred[2][z0 + 3] + sh.wred[3][z0 + 3]);
        int ciz = kBig, ciy = kBig;
        float cza = 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          ciz = min(ciz, sh.widx[q][z0 + 0]);
          if (sh.widx[q][z0 + 1] < ciy) {
            ciy = sh.widx[q][z0 + 1];
            cza = sh.wza[z0 + q];
          }
        }
        if (ln == 0) {
          if constexpr (kSums) {
            sh.part[z0 + 0] = __float_as_uint(Mzc);
            sh.part[z0 + 1] = __float_as_uint(sz);
            sh.part[z0 + 2] = __float_as_uint(Myc);
            sh.part[z0 + 3] = __float_as_uint(sy2);
          } else {
            sh.part[z0 + 0] = __float_as_uint(Mzc);
            sh.part[z0 + 1] = __float_as_uint(Myc);
            sh.part[z0 + 2] = (uint32_t)ciz;
            sh.part[z0 + 3] = (uint32_t)ciy;
            sh.part[z0 + 4] = __float_as_uint(cza);
          }
        }
      }
      if constexpr (MODE == kForward) {
        if (G > 1 && chunk == 0 && iter > 0 && !finish_pending(pp, ln, z0)) sh.err = 1;
      }
      if (G > 1) {
        publish<NU1>(units1 + (size_t)chunk * 8, ln, flag1, sh.part + z0);
        if (!gather_wave<NU1>(sh.rx + z0, units1, G, ln, flag1, pp->spin_limit)) sh.err = 1;
      }
      float Mz, My, Sz = 0.f, Sy = 0.f, za;
      int dtop, atop;
      if (G > 1) {
        // ln c combines member c (and c + 64); the members are then reduced in a fixed DPP order
        float mz = kNegInf, my = kNegInf, lsz = 0.f, lsy = 0.f, lza = 0.f;
        int liz = kBig, liy = kBig;
        for (int c = ln; c < G; c += 64) {
          mz = fmaxf(mz, __uint_as_float(sh.rx[z0 + c * NU1 + 0]));
          my = fmaxf(my, __uint_as_float(sh.rx[z0 + c * NU1 + kMy]));
        }
        wmax2(mz, my);
        Mz = mz;
        My = my;
        const float cHz = Mz * kLog2e, cHy = My * kLog2e;
        for (int c = ln; c < G; c += 64) {
          const uint32_t* u = sh.rx + z0 + c * NU1;
          const float mzc = __uint_as_float(u[0]), myc = __uint_as_float(u[kMy]);
          if constexpr (kSums) {
            lsz = __builtin_fmaf(__uint_as_float(u[1]), exp2_fast(mzc * kLog2e - cHz), lsz);
            lsy = __builtin_fmaf(__uint_as_float(u[3]), exp2_fast(myc * kLog2e - cHy), lsy);
          } else {
            if (mzc == Mz) liz = min(liz, (int)u[2]);
            if (myc == My && (int)u[3] < liy) {
              liy = (int)u[3];
              lza = __uint_as_float(u[4]);
            }
          }
        }
        if constexpr (kSums) {
          wsum2(lsz, lsy);
          Sz = lsz;
          Sy = lsy;
          dtop = atop = kBig;  // from exchange 2
          za = 0.f;
        } else {
          dtop = liz;
          atop = liy;
          wmin2(dtop, atop);
          za = wsum(liy == atop ? lza : 0.f);
        }
      } else {
        Mz = Mzc;
        My = Myc;
        if constexpr (kSums) {
          Sz = __uint_as_float(sh.part[z0 + 1]);
          Sy = __uint_as_float(sh.part[z0 + 3]);
          dtop = atop = kBig;
          za = 0.f;
        } else {
          dtop = (int)sh.part[z0 + 2];
          atop = (int)sh.part[z0 + 3];
          za = __uint_as_float(sh.part[z0 + 4]);
        }
      }
      if (ln == 0) {
        sh.row[z0 + kRowMz] = Mz;
        sh.row[z0 + kRowMy] = My;
        sh.row[z0 + kRowDtop] = __int_as_float(dtop);
        sh.row[z0 + kRowAtop] = __int_as_float(atop);
        sh.row[z0 + kRowZa] = za;
        if constexpr (kSums) {
          // Sz = sum 2^(z log2e - fl(Mz log2e)); ln of sum e^(z - Mz) takes back the rounding of
          // fl(Mz log2e), which fma recovers exactly
          const float ln_sz = (log2_fast(Sz) - __builtin_fmaf(Mz, kLog2e, -(Mz * kLog2e))) * kLn2;
          const float ln_sy = (log2_fast(Sy) - __builtin_fmaf(My, kLog2e, -(My * kLog2e))) * kLn2;
          sh.row[z0 + kRowLnSz] = ln_sz;
          sh.row[z0 + kRowLnSy] = ln_sy;
          sh.row[z0 + kRowDelta] = (Mz - My) + (ln_sz - ln_sy);
        }
      }
    }
    __syncthreads();
    __builtin_amdgcn_s_setprio(0);
    if (sh.err) break;

    const float Mz = sh.row[z0 + kRowMz];
    if constexpr (MODE == kTop1) {
      if (chunk == 0 && lt == 0) {
        pp->target_top1[row] = __float_as_int(sh.row[z0 + kRowAtop]);
        if (pp->draft_top1) pp->draft_top1[row] = __float_as_int(sh.row[z0 + kRowDtop]);
      }
    } else {
      const float ln_sz = sh.row[z0 + kRowLnSz];
      const float delta = sh.row[z0 + kRowDelta];
      RowConst rc;
      rc.init(Mz, ln_sz, delta);

      // ---- phase B: vectors that pass the bound use their phase-A sums, the rest (near the peak)
      // are summed element by element. Phase B feeds the second exchange: it runs above phases A
      // and C, and the reduction and exchange above that.
      __builtin_amdgcn_s_setprio(2);
      // Screening: a vector whose max z is at most zt passes the exact bound test below (the
      // vector_may_clip test, shared with k_bwd) with room to spare, since its bound
      // sc max(dmax - delta, 0) is at most 2^-1.49 tau_b when every dmax of the lane is counted at
      // the lane's largest; only vectors above zt evaluate the exact test and its exp2, so the set
      // of vectors summed element by element is exactly that of the exact test. tau_b below
      // 2^-100 (including tau <= 0) sends every vector to the exact test.
      const float m_l = fmaxf(kept_dmax<EPV>(ldmax) - delta, 0.f);
      float zt = kNegInf;
      if (tau_b >= 0x1p-100f)
        zt = m_l == 0.f ? -kNegInf
                        : ((rc.c_hi + rc.c_lo) + ((log2_fast(tau_b) - log2_fast(fmaxf(m_l, 0x1p-100f))) - 1.5f)) * kLn2;
      float s_slow = 0.f, r_slow = 0.f;
      bool slow_k[K];  // per slot: the lane's vector is summed element by element (a lane mask each)
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const VecMax<EPV> vk = vmlds[k * kThreads + lt];
        const bool near = vk.z() > zt;
        slow_k[k] = false;
        if (__builtin_amdgcn_ballot_w64(near)) {
          const bool slow = near && vector_may_clip(rc, vector_scale(rc, vk.z()), vk.d(), tau_b);
          if (__builtin_amdgcn_ballot_w64(slow)) {
            slow_k[k] = slow;
            opaque(zr[k]);
            float x[EPV], w[EPV], d[EPV];
            In::decode(zr[k], x);
            In::decode(ylds[k * kThreads + lt], w);
#pragma unroll
            for (int e = 0; e < EPV; ++e) d[e] = x[e] - w[e];
            const int vi = cv0 + lt + k * kThreads;
            const int nvalid = (lt + k * kThreads < clen) ? min(EPV, pp->vocab - vi * EPV) : 0;
#pragma unroll
            for (int e = 0; e < EPV; ++e) {
              const bool valid = slow && e < nvalid;
              const float p = rc.p(x[e]);
              const float t = p * (d[e] - delta);
              const bool clipped = t > tau;
              r_slow += valid ? (clipped ? tau : t) : 0.f;
              s_slow += (valid && !clipped) ? (t + p) : 0.f;
            }
            fence_vals(r_slow, s_slow);
          }
        }
      }
      // Sums of the vectors that pass, scaled from the lane reference to p. The vectors summed
      // element by element are left out rather than subtracted from a total: a subtraction would
      // cancel when such a vector dominates its lane.
      const float scl = exp2_fast((ref_z - rc.c_hi) - rc.c_lo);
      const float pe = lane_sum<K>(ek, slow_k) * scl, pb = lane_sum<K>(bk, slow_k) * scl;
      __builtin_amdgcn_s_setprio(3);
      // lowest indices of the row maxima within this chunk (kBig where the chunk does not reach
      // them), and z at the one of y: only waves holding a row maximum decode, which is usually one
      // wave of one member of the team
      int wiz = kBig, wiy = kBig;
      float wza = 0.f;
      {
        const float Myr = sh.row[z0 + kRowMy];
        int kk = K;  // the lane's first slot holding the row maximum of z
#pragma unroll
        for (int k = K - 1; k >= 0; --k) kk = holds_zmax<In>(vmlds[k * kThreads + lt], zr[k], Mz) ? k : kk;
        const bool hz = kk < K;
        if (__builtin_amdgcn_ballot_w64(hz)) {
          int iz = kBig;
#pragma unroll
          for (int k = 0; k < K; ++k) {
            if (__builtin_amdgcn_ballot_w64(hz && kk == k)) {
              if (hz && kk == k) {
                float x[EPV];
                In::decode(zr[k], x);
                iz = (cv0 + lt + k * kThreads) * EPV + first_eq<EPV>(x, Mz);
              }
            }
          }
          wiz = wmin(iz);
        }
        const bool hy = lymax == Myr;
        if (__builtin_amdgcn_ballot_w64(hy)) {
          int iy = kBig;
          float za = 0.f;
#pragma unroll
          for (int k = 0; k < K; ++k) {
            if (__builtin_amdgcn_ballot_w64(hy && kym == k)) {
              if (hy && kym == k) {
                float x[EPV], w[EPV];
                In::decode(zr[k], x);
                In::decode(ylds[k * kThreads + lt], w);
                const int e0 = first_eq<EPV>(w, Myr);
                float zv = x[0];
#pragma unroll
                for (int e = 1; e < EPV; ++e) zv = (e == e0) ? x[e] : zv;
                iy = (cv0 + lt + k * kThreads) * EPV + e0;
                za = zv;
              }
            }
          }
          wiy = wmin(iy);
          wza = wsum(iy == wiy ? za : 0.f);  // the ln holding the index (unique)
        }
      }
      {
        float a = __builtin_fmaf(1.f - delta, pe, pb) + s_slow;
        float c = __builtin_fmaf(-delta, pe, pb) + r_slow;
        wsum2(a, c);
        if (ln == 0) {
          sh.wred[wv][z0 + 0] = a;
          sh.wred[wv][z0 + 1] = c;
          sh.widx[wv][z0 + 0] = wiz;
          sh.widx[wv][z0 + 1] = wiy;
          sh.wza[z0 + wv] = wza;
        }
      }
      __syncthreads();
      // ---- exchange 2 (wave 0) and the row outputs (chunk 0)
      const uint32_t flag2 = flag1 + 1u;
      if (wave == 0) {
        if (ln == 0) {
          sh.part[z0 + 0] = __float_as_uint((sh.wred[0][z0 + 0] + sh.wred[1][z0 + 0]) + (sh.wred[2][z0 + 0] + sh.wred[3][z0 + 0]));
          sh.part[z0 + 1] = __float_as_uint((sh.wred[0][z0 + 1] + sh.wred[1][z0 + 1]) + (sh.wred[2][z0 + 1] + sh.wred[3][z0 + 1]));
          int ciz = kBig, ciy = kBig;
          float cza = 0.f;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            ciz = min(ciz, sh.widx[q][z0 + 0]);
            if (sh.widx[q][z0 + 1] < ciy) {
              ciy = sh.widx[q][z0 + 1];
              cza = sh.wza[z0 + q];
            }
          }
          sh.part[z0 + 2] = (uint32_t)ciz;
          sh.part[z0 + 3] = (uint32_t)ciy;
          sh.part[z0 + 4] = __float_as_uint(cza);
        }
        if (G > 1) {
          publish<kStage2Units>(units2 + (size_t)chunk * 8, ln, flag2, sh.part + z0);
          if (MODE == kFused && !gather_wave<kStage2Units>(sh.rx + z0, units2, G, ln, flag2, pp->spin_limit)) sh.err = 1;
        }
        if (MODE == kFused || G == 1) {
          finish_row(pp, row, G > 1, ln, z0, Mz, ln_sz, sh.row[z0 + kRowMy], sh.row[z0 + kRowLnSy], delta, alpha);
        } else if (chunk == 0 && ln == 0) {  // forward mode: gathered later (finish_pending)
          sh.pend[0] = Mz;
          sh.pend[1] = ln_sz;
          sh.pend[2] = sh.row[z0 + kRowMy];
          sh.pend[3] = sh.row[z0 + kRowLnSy];
          sh.pend[4] = delta;
          sh.pend_row = row;
          sh.pend_flag = flag2;
        }
      }
      __syncthreads();
      __builtin_amdgcn_s_setprio(1);  // phase C: above the loads and phase A of other workgroups
      if (sh.err) break;

      if constexpr (MODE == kFused) {
        // ---- phase C: dz (formulas shared with k_bwd through dz_vector)
        DzConst dc;
        dc.init(rc, sh.row[z0 + kRowS], alpha, pp->grad_loss ? pp->grad_loss[row] : 1.f);
        const __amdgpu_buffer_rsrc_t rd = rsrc(pp->dz + (int64_t)row * pp->ld_dz_bytes + (int64_t)cv0 * VB, clen * VB);
        __asm__ volatile("" : "+v"(lt));  // fresh offsets: not kept live from the loads
        // the one vector holding the target top-1 (if it lies in this chunk), from exchange 2; the
        // index is the same in every lane, so it is moved to a scalar register and the slot test
        // below is scalar code
        const int atop = __builtin_amdgcn_readfirstlane(__float_as_int(sh.row[z0 + kRowAtop]));
        const int va = atop / EPV - cv0;
        const int ka = (va >= 0 && va < clen) ? va / kThreads : -1;
#pragma unroll
        for (int k = 0; k < K; ++k) {
          opaque(zr[k]);
          float x[EPV], w[EPV], o[EPV];
          In::decode(zr[k], x);
          In::decode(ylds[k * kThreads + lt], w);
          const bool slow = slow_k[k];
          dz_vector<EPV>(x, w, slow, __builtin_amdgcn_ballot_w64(slow) != 0, rc, dc, tau, o);
          const int vi = cv0 + lt + k * kThreads;
          if (k == ka) fix_target<EPV>(o, vi * EPV, atop, dc.wce);
#pragma unroll
          for (int e = 0; e < EPV; e += 4) fence_vals(o[e], o[e + 1], o[e + 2], o[e + 3]);
          int off = (lt + k * kThreads) * VB;  // past num_records for lanes beyond the chunk: dropped
          if (tail_chunk && vi == pp->nvec - 1) {  // partial last vector: element stores
            store_partial<OutBF16, EPV>(pp->dz + (int64_t)row * pp->ld_dz_bytes + (int64_t)vi * VB, o,
                                        pp->vocab - vi * EPV);
            off = 0x7fffffff & ~(VB - 1);
          }
          buf_store_vec<OutBF16, EPV>(rd, off, o);
        }
      }
    }
  }
  if constexpr (MODE == kForward) {  // the last row's exchange 2
    if (P.G > 1 && chunk == 0 && iter > 0 && wave == 0 && !sh.err) {
      KParams* pp = (KParams*)__builtin_amdgcn_kernarg_segment_ptr();
      const int ln = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
      if (!finish_pending(pp, ln, 0)) sh.err = 1;
    }
  }
  const int tid_end = (wave << 6) + (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  if (tid_end == 0) {
    if (sh.err) atomicOr(P.flags, (uint32_t)kFlagSpinTimeout);
    // Device-mode flags: the last workgroup to finish advances the epoch for the next launch; by
    // then every workgroup of this launch has read it. Relaxed agent-scope atomics; the kernel
    // boundary orders them before the next launch's read.
    if constexpr (DevFlags) {
      // this wave published every exchange value of the workgroup: wait until those stores are
      // done before counting the workgroup as finished (the last one may zero the units below)
      __builtin_amdgcn_s_waitcnt(0);
      const uint32_t grid = (uint32_t)(P.n_teams * P.G);
      const uint32_t done = __hip_atomic_fetch_add(P.flags + kDoneWord, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      sh.last = done + 1u == grid;
    }
  }
  if constexpr (DevFlags) {
    __syncthreads();
    if (sh.last) {
      uint32_t next = (sh.fbase - 1u) + P.flag_count;
      if (next > kEpochRestart) {
        // The range restarts: zero every exchange unit first, so that no unit written in the range
        // that ends can carry a flag of the next one. No other workgroup of this launch is left.
        constexpr size_t n_units = (kWorkspaceBytes - kHeaderBytes) / 8;
        for (size_t i = tid_end; i < n_units; i += kThreads)
          __hip_atomic_store(P.units + i, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        next = 0;
      }
      if (tid_end == 0) {
        __hip_atomic_store(P.flags + kDoneWord, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(P.flags + kEpochWord, next, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

// ---------------------------------------------------------------- streaming backward

constexpr int kBwdVecPerThread = 4;

template <class In, bool OutBF16>
__global__ void __launch_bounds__(kThreads) k_bwd(BwdParams P) {
  constexpr int EPV = In::EPV;
  constexpr int OSZ = OutBF16 ? 2 : 4;
  const int row = block_id_y();
  const float* st = P.row_stats + 8 * (int64_t)row;
  RowConst rc;
  rc.init(st[4], st[5], st[6]);
  DzConst dc;
  dc.init(rc, st[2], P.alpha, P.grad_loss ? P.grad_loss[row] : 1.f);
  const int atop = P.target_top1[row];
  const float tau = P.tau;
  const uint4* zrow = (const uint4*)(P.z + (int64_t)row * P.ld_bytes);
  const uint4* yrow = (const uint4*)(P.y + (int64_t)row * P.ld_bytes);
  uint8_t* drow = P.dz + (int64_t)row * P.ld_dz_bytes;
  const int v0 = block_id_x() * (kThreads * kBwdVecPerThread) + thread_id();
  uint4 zr[kBwdVecPerThread], yr[kBwdVecPerThread];
#pragma unroll
  for (int k = 0; k < kBwdVecPerThread; ++k) {
    const int vc = min(v0 + k * kThreads, P.nvec - 1);
    zr[k] = load_nt(zrow + vc);
    yr[k] = load_nt(yrow + vc);
  }
#pragma unroll
  for (int k = 0; k < kBwdVecPerThread; ++k) {
    opaque(zr[k]);
    opaque(yr[k]);
  }
  if (P.nvec * EPV != P.vocab) {  // uniform: rows whose last vector is partial
#pragma unroll
    for (int k = 0; k < kBwdVecPerThread; ++k) {
      const int vi = v0 + k * kThreads;
      if (vi == P.nvec - 1) {
        mask_tail<In>(zr[k], P.vocab - vi * EPV);
        mask_tail<In>(yr[k], P.vocab - vi * EPV);
      }
    }
  }
#pragma unroll
  for (int k = 0; k < kBwdVecPerThread; ++k) {
    const int vi = v0 + k * kThreads;
    float x[EPV], w[EPV], o[EPV];
    In::decode(zr[k], x);
    In::decode(yr[k], w);
    // the fused kernel's vector bound, recomputed: same decisions, bit-identical dz
    float d[EPV];
#pragma unroll
    for (int e = 0; e < EPV; ++e) d[e] = x[e] - w[e];
    const float sc = vector_scale(rc, kept_zmax<EPV>(vmax<EPV>(x)));
    const bool slow = vector_may_clip(rc, sc, kept_dmax<EPV>(vmax<EPV>(d)), tau * kBoundShrink);
    dz_vector<EPV>(x, w, slow, __builtin_amdgcn_ballot_w64(slow) != 0, rc, dc, tau, o);
    const int g0 = vi * EPV;
    fix_target<EPV>(o, g0, atop, dc.wce);
    if (vi < P.nvec) {
      uint8_t* dst = drow + (int64_t)g0 * OSZ;
      if (g0 + EPV <= P.vocab) {
        store_vec<OutBF16, EPV>(dst, o);
      } else {
        store_partial<OutBF16, EPV>(dst, o, P.vocab - g0);
      }
    }
  }
}

// ---------------------------------------------------------------- accept length per packed block

// One wave per block: lane j compares row j of each 64-row window of the block, and a ballot gives
// the first mismatch, so a block costs one round of loads instead of one per accepted row.
constexpr int kAcceptBlocksPerGroup = kThreads / 64;

__global__ void __launch_bounds__(kThreads) k_accept(AcceptParams P) {
  const int lane = thread_id() & 63;
  const int b = block_id_x() * kAcceptBlocksPerGroup + (thread_id() >> 6);
  if (b >= P.n_blocks) return;  // wave-uniform
  const int start = P.offsets[b], end = P.offsets[b + 1];
  uint32_t fl = 0;
  int acc = 0;
  if (start < 0 || end < start || end > P.n_rows) {
    fl |= kFlagBadOffsets;
  } else {
    int lb = P.L[b];
    if (lb < 0) {
      fl |= kFlagNegL;
      lb = 0;
    }
    const int n = min(lb, end - start);
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
  if (lane == 0) {
    P.accept_len[b] = acc;
    if (fl) atomicOr(P.flags, fl);
  }
}

__global__ void __launch_bounds__(kThreads) k_fill_u32(uint32_t* dst, uint32_t value, size_t count, size_t stride) {
  for (size_t i = block_id_x() * (size_t)kThreads + thread_id(); i < count; i += stride) dst[i] = value;
}

// Bandwidth probe with no arithmetic, for the achievable-bandwidth figures reported beside the
// kernels: KIND 0 reads a and b and writes c = a ^ b (the fused path's two reads and one write per
// 16-byte vector), KIND 1 only reads a and b (the xor of everything read is stored only if it equals
// a value the caller passes and never produces, which keeps the loads alive), KIND 2 only writes c.
// One-shot workgroups, each streaming U * 256 consecutive vectors per tensor with U vectors per
// tensor in flight per thread: in a sweep on MI355X this shape streamed faster for all three
// patterns than persistent grid-stride loops over 256 to 8192 workgroups.
template <int KIND, int U>
__global__ void __launch_bounds__(kThreads) k_stream_probe(const uint4* a, const uint4* b, uint8_t* c, size_t n,
                                                           uint32_t never) {
  uint32_t acc = 0;
  const size_t v0 = (size_t)block_id_x() * (kThreads * U) + thread_id();
  uint4 x[U], y[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const size_t i = v0 + (size_t)u * kThreads;
    if (KIND != 2 && i < n) {
      x[u] = load_nt(a + i);
      y[u] = load_nt(b + i);
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const size_t i = v0 + (size_t)u * kThreads;
    if (i >= n) continue;
    if constexpr (KIND == 0) {
      store_nt(c + 16 * i, x[u].x ^ y[u].x, x[u].y ^ y[u].y, x[u].z ^ y[u].z, x[u].w ^ y[u].w);
    } else if constexpr (KIND == 1) {
      acc ^= (x[u].x ^ y[u].x) ^ (x[u].y ^ y[u].y) ^ (x[u].z ^ y[u].z) ^ (x[u].w ^ y[u].w);
    } else {
      store_nt(c + 16 * i, (uint32_t)i, (uint32_t)(i >> 32), 0u, 0u);
    }
  }
  if (KIND == 1 && acc == never && c) store_nt(c, acc, 0u, 0u, 0u);
}

// ---------------------------------------------------------------- instantiation tables

template <class In, bool OutBF16, int MODE, bool D>
void* team_kernel_k(int K) {
  return K == 1 ? (void*)k_team<In, OutBF16, 1, MODE, D>
       : K == 3 ? (void*)k_team<In, OutBF16, 3, MODE, D>
                : (void*)k_team<In, OutBF16, 5, MODE, D>;
}

template <int MODE, bool D>
void* team_kernel(int in_bf16, int out_bf16, int K) {
  if (MODE != kFused) out_bf16 = 0;
  if (in_bf16) return out_bf16 ? team_kernel_k<BF16In, true, MODE, D>(K) : team_kernel_k<BF16In, false, MODE, D>(K);
  return out_bf16 ? team_kernel_k<F32In, true, MODE, D>(K) : team_kernel_k<F32In, false, MODE, D>(K);
}

template <bool D>
void* team_kernel_mode(int mode, int in_bf16, int out_bf16, int K) {
  switch (mode) {
    case kFused: return team_kernel<kFused, D>(in_bf16, out_bf16, K);
    case kForward: return team_kernel<kForward, D>(in_bf16, out_bf16, K);
    default: return team_kernel<kTop1, D>(in_bf16, out_bf16, K);
  }
}

void* team_kernel_any(int mode, int in_bf16, int out_bf16, int K, bool dev_flags) {
  return dev_flags ? team_kernel_mode<true>(mode, in_bf16, out_bf16, K)
                   : team_kernel_mode<false>(mode, in_bf16, out_bf16, K);
}

}  // namespace

hipError_t launch_team(const TeamParams& p, int mode, int in_bf16, int out_bf16, int K, int grid, hipStream_t s) {
  void* fn = team_kernel_any(mode, in_bf16, out_bf16, K, p.flag_base == 0);
  TeamParams copy = p;
  void* args[] = {&copy};
  return hipLaunchKernel(fn, dim3(grid), dim3(kThreads), args, 0, s);
}

constexpr int kTeamMaxPerCu = 6;

hipError_t team_occupancy(int mode, int in_bf16, int out_bf16, int K, bool dev_flags, int* blocks_per_cu) {
  const void* fn = team_kernel_any(mode, in_bf16, out_bf16, K, dev_flags);
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, fn, kThreads, 0);
  if (e != hipSuccess) return e;
  // The team kernels need every workgroup of the grid resident at once, so the count must not be
  // optimistic. LDS is allocated in 512-byte granules; the runtime's count was seen to assume a
  // finer allocation (a workgroup of 27,260 B was reported to fit six times in 160 KiB, where
  // 6 x 27,648 B do not). Bound the count by the granule-rounded LDS per CU.
  hipFuncAttributes attr;
  e = hipFuncGetAttributes(&attr, fn);
  if (e != hipSuccess) return e;
  int dev = 0, lds_cu = 0;
  if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
  if ((e = hipDeviceGetAttribute(&lds_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev)) != hipSuccess)
    return e;
  const size_t lds = ((attr.sharedSizeBytes + 511) / 512) * 512;
  if (lds > 0 && lds_cu > 0) {
    const int by_lds = (int)((size_t)lds_cu / lds);
    if (by_lds < *blocks_per_cu) *blocks_per_cu = by_lds;
  }
  // Nor does the count include the trap handler's 16 scalar registers that every wave holds on this
  // part beside its own (allocated in granules of 16, at most 112): with 800 per SIMD, a wave using
  // 97-112 leaves room for 6 per SIMD, not the 7 the runtime reports (a team kernel with 104
  // measured one workgroup per CU short: its teams waited for members that were not resident).
  // One wave per SIMD per workgroup, so 6 workgroups per CU hold for any scalar register use.
  if (*blocks_per_cu > kTeamMaxPerCu) *blocks_per_cu = kTeamMaxPerCu;
  return hipSuccess;
}

hipError_t launch_bwd(const BwdParams& p, int in_bf16, int out_bf16, hipStream_t s) {
  const int per_block = kThreads * kBwdVecPerThread;
  dim3 grid((p.nvec + per_block - 1) / per_block, p.n_rows);
  BwdParams copy = p;
  void* args[] = {&copy};
  void* fn;
  if (in_bf16) fn = out_bf16 ? (void*)k_bwd<BF16In, true> : (void*)k_bwd<BF16In, false>;
  else fn = out_bf16 ? (void*)k_bwd<F32In, true> : (void*)k_bwd<F32In, false>;
  return hipLaunchKernel(fn, grid, dim3(kThreads), args, 0, s);
}

hipError_t launch_accept(const AcceptParams& p, hipStream_t s) {
  dim3 grid((p.n_blocks + kAcceptBlocksPerGroup - 1) / kAcceptBlocksPerGroup);
  AcceptParams copy = p;
  void* args[] = {&copy};
  return hipLaunchKernel((void*)k_accept, grid, dim3(kThreads), args, 0, s);
}

hipError_t launch_stream_probe(const void* a, const void* b, void* c, size_t n_vec, hipStream_t s) {
  if (n_vec == 0) return hipSuccess;
  // two vectors per tensor in flight per thread: the fastest of 1, 2, 4 and 8 for the read-read-write
  // pattern in the sweep (4 was within 1 %, 8 slower); read-only and write-only streams use the same
  constexpr int U = 2;
  const int kind = (a && b && c) ? 0 : (a && b) ? 1 : 2;
  const size_t blocks = (n_vec + (size_t)kThreads * U - 1) / ((size_t)kThreads * U);
  if (blocks > 0x7fffffffull) return hipErrorInvalidValue;
  const uint4* pa = (const uint4*)a;
  const uint4* pb = (const uint4*)b;
  uint8_t* pc = (uint8_t*)c;
  if (kind == 0)
    hipLaunchKernelGGL((k_stream_probe<0, U>), dim3((unsigned)blocks), dim3(kThreads), 0, s, pa, pb, pc, n_vec, 0u);
  else if (kind == 1)
    hipLaunchKernelGGL((k_stream_probe<1, U>), dim3((unsigned)blocks), dim3(kThreads), 0, s, pa, pb, pc, n_vec,
                       0x9e3779b9u);
  else
    hipLaunchKernelGGL((k_stream_probe<2, U>), dim3((unsigned)blocks), dim3(kThreads), 0, s, pa, pb, pc, n_vec, 0u);
  return hipGetLastError();
}

hipError_t launch_fill_u32(uint32_t* dst, uint32_t value, size_t count, hipStream_t s) {
  size_t blocks = (count + kThreads - 1) / kThreads;
  if (blocks > 1024) blocks = 1024;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(k_fill_u32, dim3((unsigned)blocks), dim3(kThreads), 0, s, dst, value, count,
                     blocks * (size_t)kThreads);
  return hipGetLastError();
}

}  // namespace opd
