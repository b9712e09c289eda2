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
// Design (MI355X): the path is HBM-bound streaming (no dense contraction, so no MFMA). A 151,936-wide
// bf16 row is 297 KiB per tensor, more than one CU can hold, so a row is split over a *team* of G
// workgroups. Each workgroup keeps its chunk of z and y in VGPRs (packed bf16) for the whole row:
//   phase A  chunk max, sum-exp of z and y, per-vector sums of e^(z_v - m) and e^(z_v - m)(z_v - y_v),
//            first argmax of z and y
//   -- exchange 1 --  every member combines the G partials in the same fixed order
//   phase B  S and the clipped reverse KL: vectors whose bound max(p) * max(z - y - delta, 0) is
//            <= tau provably hold no clipped term and use their phase-A sums; the rest are visited
//            element by element
//   -- exchange 2 --
//   phase C  dz written once (bf16 rounded to nearest even, or fp32)
// so z and y are read from HBM once and dz written once. Exchanges use 8-byte [value | flag] units
// written and polled with agent-scope relaxed atomics (sc1: coherent across XCDs without L2
// writeback / invalidate); the flag is unique per launch, row iteration and stage, so nothing has to
// be reset between launches and a stale unit can never be taken for a fresh one. Every wait is
// bounded and raises a sticky flag instead of hanging. Team members are mapped to one XCD when the
// team count allows (workgroups are dispatched round-robin over the 8 XCDs).
//
// Numerics: fp32 throughout with fixed reduction orders (bitwise deterministic). Per row, with
// M = max z, S_z = sum_v e^(z_v - M), delta = LSE(z) - LSE(y), t_v = p_v (z_v - y_v - delta):
//   clipped reverse KL = sum_v min(t_v, tau),  S = sum_v [t_v <= tau] p_v (t_v / p_v + 1),
//   dz_v = w p_v (alpha (z_v - y_v) + alpha (1 - delta - S) + 1 - alpha)  (unclipped)
//   dz_v = w p_v (1 - alpha - alpha S)                                     (clipped)
//   dz_a -= w (1 - alpha).
// p_v is evaluated from M and log S_z held apart (RowConst), so that large logits keep full fp32
// relative accuracy. Vectors proven free of clipped terms contribute to S and the reverse KL
// through their per-vector sums from phase A; vectors near the peak are summed element by element
// (no cancellation between the clipped terms and the rest). The clip decision is the same fp32
// test, from the same per-row floats, in the fused and the separate kernels, so fused and
// forward+backward results are bit-identical.

#include <stdint.h>

#include "opd_internal.h"

namespace opd {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_inff();
constexpr int kBig = 0x7fffffff;

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------- input formats (16-byte vectors)

struct F32In {
  static constexpr int EPV = 4;
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

// ---------------------------------------------------------------- cross-workgroup exchange

__device__ __forceinline__ void unit_store(uint64_t* p, uint32_t flag, uint32_t bits) {
  uint64_t u = ((uint64_t)flag << 32) | (uint64_t)bits;
  __hip_atomic_store(p, u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Poll one unit until its flag matches; returns false when the bound was exceeded.
__device__ __forceinline__ bool unit_wait(const uint64_t* p, uint32_t flag, uint32_t limit, uint32_t& bits) {
  uint32_t spins = 0;
  while (true) {
    uint64_t u = __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if ((uint32_t)(u >> 32) == flag) {
      bits = (uint32_t)u;
      return true;
    }
    if (++spins > limit) return false;
    __builtin_amdgcn_s_sleep(1);
  }
}

struct Shared {
  float red[4][8];
  int ired[4][4];
  float out[8];
  uint32_t rx[128 * kStage1Units];
  int err;
};

// Publish NU values of this chunk and gather every chunk's values into sh.rx[c * NU + j].
// Returns false (uniformly over the workgroup) if a wait exceeded its bound.
template <int NU>
__device__ __forceinline__ bool exchange(Shared& sh, const TeamParams& P, int team, int chunk, int stage,
                                         uint32_t flag, bool receive) {
  uint64_t* base = P.units + ((size_t)team * 2 + stage) * (size_t)P.G * 8;
  const int tid = threadIdx.x;
  if (tid < NU) {
    unit_store(base + (size_t)chunk * 8 + tid, flag, __float_as_uint(sh.out[tid]));
  }
  if (receive) {
    bool ok = true;
    for (int i = tid; i < P.G * NU; i += kThreads) {
      uint32_t bits = 0;
      const int c = i / NU, j = i - c * NU;
      if (!unit_wait(base + (size_t)c * 8 + j, flag, P.spin_limit, bits)) ok = false;
      sh.rx[i] = bits;
    }
    if (!ok) sh.err = 1;
  }
  __syncthreads();
  return sh.err == 0;
}

// ---------------------------------------------------------------- wave reductions (DPP)

// Full-wave reductions on the DPP crossbar (quad_perm, row mirrors, row broadcasts): six ALU ops
// instead of six LDS-permute round trips. The result is read from lane 63 and is wave-uniform.
template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp_mov(int v, int identity) {
  return __builtin_amdgcn_update_dpp(identity, v, CTRL, ROWS, 0xF, false);
}
__device__ __forceinline__ float dppf(float v, float id, int which) {
  switch (which) {
    case 0: return __int_as_float(dpp_mov<0xB1, 0xF>(__float_as_int(v), __float_as_int(id)));
    case 1: return __int_as_float(dpp_mov<0x4E, 0xF>(__float_as_int(v), __float_as_int(id)));
    case 2: return __int_as_float(dpp_mov<0x141, 0xF>(__float_as_int(v), __float_as_int(id)));
    case 3: return __int_as_float(dpp_mov<0x140, 0xF>(__float_as_int(v), __float_as_int(id)));
    case 4: return __int_as_float(dpp_mov<0x142, 0xA>(__float_as_int(v), __float_as_int(id)));
    default: return __int_as_float(dpp_mov<0x143, 0xC>(__float_as_int(v), __float_as_int(id)));
  }
}
__device__ __forceinline__ int dppi(int v, int id, int which) {
  switch (which) {
    case 0: return dpp_mov<0xB1, 0xF>(v, id);
    case 1: return dpp_mov<0x4E, 0xF>(v, id);
    case 2: return dpp_mov<0x141, 0xF>(v, id);
    case 3: return dpp_mov<0x140, 0xF>(v, id);
    case 4: return dpp_mov<0x142, 0xA>(v, id);
    default: return dpp_mov<0x143, 0xC>(v, id);
  }
}
__device__ __forceinline__ float uniform_f(float v) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
__device__ __forceinline__ float wmax(float v) {
#pragma unroll
  for (int s = 0; s < 6; ++s) v = fmaxf(v, dppf(v, kNegInf, s));
  return uniform_f(v);
}
__device__ __forceinline__ float wsum(float v) {
#pragma unroll
  for (int s = 0; s < 6; ++s) v = v + dppf(v, 0.f, s);
  return uniform_f(v);
}
__device__ __forceinline__ int wmin(int v) {
#pragma unroll
  for (int s = 0; s < 6; ++s) v = min(v, dppi(v, kBig, s));
  return __builtin_amdgcn_readlane(v, 63);
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
__device__ __forceinline__ void fence_vals(float& a, float& b, float& c, float& d) {
  __asm__ volatile("" : "+v"(a), "+v"(b), "+v"(c), "+v"(d));
}

// Workgroup-wide combine of wave-uniform values through LDS (4 waves).
__device__ __forceinline__ void put4(Shared& sh, int slot, float v) {
  if ((threadIdx.x & 63) == 0) sh.red[threadIdx.x >> 6][slot] = v;
}

// ---------------------------------------------------------------- the row-team kernel

template <class In, bool OutBF16, int K, int MODE>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(5))) k_team(TeamParams P) {
  constexpr int EPV = In::EPV;
  constexpr int OSZ = OutBF16 ? 2 : 4;
  __shared__ Shared sh;
  // The row chunk of y lives in LDS (written by direct global->LDS loads), z in VGPRs: this keeps
  // the register footprint within 5 workgroups per CU (the occupancy the kernel is built for, as
  // more resident teams hide the exchange waits). Each lane only ever reads back its own 16 bytes.
  __shared__ uint4 ylds[K * kThreads];
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  int team, chunk;
  if (P.xcd_map) {
    const int x = b & 7, local = b >> 3;
    team = (local / P.G) * 8 + x;
    chunk = local % P.G;
  } else {
    team = b / P.G;
    chunk = b % P.G;
  }
  const int cv0 = chunk * P.chunk_vec;
  const int cv1 = min(cv0 + P.chunk_vec, P.nvec);
  const int clen = cv1 - cv0;  // vectors in this chunk (uniform)
  const float alpha = P.alpha, tau = P.tau;
  const bool tail_chunk = (cv1 == P.nvec) && (P.nvec * EPV != P.vocab);
  if (tid == 0) sh.err = 0;

  uint4 zr[K];
  int iter = 0;
  for (int row = team; row < P.n_rows; row += P.n_teams, ++iter) {
    __syncthreads();
    // Per-thread vector index, made opaque each row: otherwise the compiler hoists every element's
    // index and bounds test out of the row loop and keeps them all in registers.
    int tv = cv0 + tid;
    __asm__ volatile("" : "+v"(tv));
    {
      // All loads of the chunk are issued back to back (indices clamped into the chunk: no branch,
      // no wait between them): z into VGPRs, y straight into this lane's LDS slots.
      const uint4* zrow = (const uint4*)(P.z + (int64_t)row * P.ld_bytes);
      const uint4* yrow = (const uint4*)(P.y + (int64_t)row * P.ld_bytes);
      const int wbase = (tid >> 6) << 6;
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const int vc = min(tv + k * kThreads, cv1 - 1);
        zr[k] = load_nt(zrow + vc);
        __builtin_amdgcn_global_load_lds(yrow + vc, (__attribute__((address_space(3))) void*)(ylds + k * kThreads + wbase),
                                         16, 0, 0);
      }
      __builtin_amdgcn_s_waitcnt(0);
    }
#pragma unroll
    for (int k = 0; k < K; ++k) {  // the current row must be in registers from here on
      opaque(zr[k]);
    }
#pragma unroll
    for (int k = 0; k < K; ++k) {
      if ((k + 1) * kThreads > clen) {  // uniform: only slots that can run past the chunk end
        if (tv + k * kThreads >= cv1) {
          zr[k] = splat4(In::kSentinel);
          ylds[k * kThreads + tid] = splat4(In::kSentinel);
        }
      }
    }
    if (tail_chunk) {  // uniform: only the chunk holding a partial last vector
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const int vi = tv + k * kThreads;
        if (vi == P.nvec - 1) {
          uint4 yv = ylds[k * kThreads + tid];
          mask_tail<In>(zr[k], P.vocab - vi * EPV);
          mask_tail<In>(yv, P.vocab - vi * EPV);
          ylds[k * kThreads + tid] = yv;
        }
      }
    }

    // ---- phase A (one pass): per 8-element vector, its z max, y max and max(z - y), and the sums
    // E_k = sum e^(z - zmax_k), B_k = sum e^(z - zmax_k)(z - y), sum e^(y - ymax_k) relative to that
    // vector's own maxima (so no workgroup maximum is needed first). Exponents use
    // c = fl(max log2 e); the rounding of c is undone once per vector when folding into the lane's
    // running (max, sum) pairs, and phase B rescales E_k, B_k by 2^(c_k - c_row).
    float zmv[K], dmv[K], ek[K], bk[K];
    float lzmax = kNegInf, lymax = kNegInf, lsz = 0.f, lsy = 0.f;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      opaque(zr[k]);
      float x[EPV], w[EPV];
      In::decode(zr[k], x);
      In::decode(ylds[k * kThreads + tid], w);
      float zm = x[0], ym = w[0], dm = x[0] - w[0];
#pragma unroll
      for (int e = 1; e < EPV; ++e) {
        zm = fmaxf(zm, x[e]);
        ym = fmaxf(ym, w[e]);
        dm = fmaxf(dm, x[e] - w[e]);
      }
      zmv[k] = zm;
      dmv[k] = dm;
      if constexpr (MODE != kTop1) {
        const float cz = zm * kLog2e, cy = ym * kLog2e;
        float se = 0.f, sb = 0.f, sey = 0.f;
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
          const float ez = exp2_fast(__builtin_fmaf(x[e], kLog2e, -cz));
          se += ez;
          sb = __builtin_fmaf(ez, x[e] - w[e], sb);
          sey += exp2_fast(__builtin_fmaf(w[e], kLog2e, -cy));
        }
        ek[k] = se;
        bk[k] = sb;
        // fold into the lane's (max, sum) pairs; exponent offsets: (max_k - M) log2e - (rounding of c)
        const float nz = fmaxf(lzmax, zm), ny = fmaxf(lymax, ym);
        lsz = __builtin_fmaf(lsz, exp2_fast((lzmax - nz) * kLog2e),
                             se * exp2_fast((zm - nz) * kLog2e - __builtin_fmaf(zm, kLog2e, -cz)));
        lsy = __builtin_fmaf(lsy, exp2_fast((lymax - ny) * kLog2e),
                             sey * exp2_fast((ym - ny) * kLog2e - __builtin_fmaf(ym, kLog2e, -cy)));
        lzmax = nz;
        lymax = ny;
        fence_vals(lzmax, lymax, lsz, lsy);
        fence_vals(zmv[k], dmv[k], ek[k], bk[k]);
      } else {
        lzmax = fmaxf(lzmax, zm);
        lymax = fmaxf(lymax, ym);
        fence_vals(lzmax, lymax);
      }
    }
    put4(sh, 0, wmax(lzmax));
    put4(sh, 1, wmax(lymax));
    __syncthreads();
    const float m_z = fmaxf(fmaxf(sh.red[0][0], sh.red[1][0]), fmaxf(sh.red[2][0], sh.red[3][0]));
    const float m_y = fmaxf(fmaxf(sh.red[0][1], sh.red[1][1]), fmaxf(sh.red[2][1], sh.red[3][1]));

    // ---- lowest index of each chunk maximum: only lanes holding it scan, from the top down with
    // selects, so the last hit is the lowest index
    int iz = kBig, iy = kBig;
    float zat = 0.f;
    if (lzmax == m_z) {
      int code = 0;
#pragma unroll
      for (int k = K - 1; k >= 0; --k) {
        opaque(zr[k]);
        float x[EPV];
        In::decode(zr[k], x);
#pragma unroll
        for (int e = EPV - 1; e >= 0; --e) code = (x[e] == m_z) ? k * EPV + e : code;
      }
      iz = (tv + (code / EPV) * kThreads) * EPV + code % EPV;
    }
    if (lymax == m_y) {
      int code = 0;
#pragma unroll
      for (int k = K - 1; k >= 0; --k) {
        opaque(zr[k]);
        float x[EPV], w[EPV];
        In::decode(zr[k], x);
        In::decode(ylds[k * kThreads + tid], w);
#pragma unroll
        for (int e = EPV - 1; e >= 0; --e) {
          const bool hit = (w[e] == m_y);
          code = hit ? k * EPV + e : code;
          zat = hit ? x[e] : zat;
        }
      }
      iy = (tv + (code / EPV) * kThreads) * EPV + code % EPV;
    }
    {
      const int wiz = wmin(iz);
      const int wiy = wmin(iy);
      const float wza = wsum(iy == wiy ? zat : 0.f);  // the lane that owns the index (unique)
      if constexpr (MODE != kTop1) {
        // chunk sums relative to the chunk maxima (lane pairs rescaled exactly: bf16/fp32 maxima)
        put4(sh, 2, wsum(lsz * exp2_fast((lzmax - m_z) * kLog2e)));
        put4(sh, 3, wsum(lsy * exp2_fast((lymax - m_y) * kLog2e)));
      }
      put4(sh, 4, __int_as_float(wiz));
      put4(sh, 5, __int_as_float(wiy));
      put4(sh, 6, wza);
    }
    __syncthreads();
    if (tid == 0) {
      const float tsz = (sh.red[0][2] + sh.red[1][2]) + (sh.red[2][2] + sh.red[3][2]);
      const float tsy = (sh.red[0][3] + sh.red[1][3]) + (sh.red[2][3] + sh.red[3][3]);
      int tiz = kBig, tiy = kBig;
      float tz = 0.f;
      for (int q = 0; q < 4; ++q) {
        tiz = min(tiz, __float_as_int(sh.red[q][4]));
        const int qi = __float_as_int(sh.red[q][5]);
        if (qi < tiy) {
          tiy = qi;
          tz = sh.red[q][6];
        }
      }
      sh.out[0] = m_z;
      sh.out[1] = tsz;
      sh.out[2] = m_y;
      sh.out[3] = tsy;
      sh.out[4] = __int_as_float(tiz);
      sh.out[5] = __int_as_float(tiy);
      sh.out[6] = tz;
    }
    __syncthreads();

    const uint32_t flag1 = P.flag_base + 2u * (uint32_t)iter;
    if (P.G > 1) {
      if (!exchange<kStage1Units>(sh, P, team, chunk, 0, flag1, true)) break;
    }

    // ---- combine the G chunk partials (each lane takes chunks lane, lane+64, ... in order, then a
    // fixed DPP tree: identical in every member, deterministic)
    float Mz, My, Sz, Sy, za;
    int dtop, atop;
    if (P.G > 1) {
      const int lane = tid & 63;
      float mz = kNegInf, my = kNegInf;
      for (int c = lane; c < P.G; c += 64) {
        mz = fmaxf(mz, __uint_as_float(sh.rx[c * kStage1Units + 0]));
        my = fmaxf(my, __uint_as_float(sh.rx[c * kStage1Units + 2]));
      }
      Mz = wmax(mz);
      My = wmax(my);
      float lsz = 0.f, lsy = 0.f, lza = 0.f;
      int liz = kBig, liy = kBig;
      for (int c = lane; c < P.G; c += 64) {
        const uint32_t* u = sh.rx + c * kStage1Units;
        const float mzc = __uint_as_float(u[0]), myc = __uint_as_float(u[2]);
        if constexpr (MODE != kTop1) {
          lsz = __builtin_fmaf(__uint_as_float(u[1]), exp2_fast((mzc - Mz) * kLog2e), lsz);
          lsy = __builtin_fmaf(__uint_as_float(u[3]), exp2_fast((myc - My) * kLog2e), lsy);
        }
        if (liz == kBig && mzc == Mz) liz = (int)u[4];
        if (liy == kBig && myc == My) {
          liy = (int)u[5];
          lza = __uint_as_float(u[6]);
        }
      }
      Sz = (MODE != kTop1) ? wsum(lsz) : 0.f;
      Sy = (MODE != kTop1) ? wsum(lsy) : 0.f;
      dtop = wmin(liz);
      atop = wmin(liy);
      za = wsum(liy == atop ? lza : 0.f);
    } else {
      Mz = sh.out[0];
      Sz = sh.out[1];
      My = sh.out[2];
      Sy = sh.out[3];
      dtop = __float_as_int(sh.out[4]);
      atop = __float_as_int(sh.out[5]);
      za = sh.out[6];
    }

    if constexpr (MODE == kTop1) {
      if (chunk == 0 && tid == 0) {
        P.target_top1[row] = atop;
        P.draft_top1[row] = dtop;
      }
    } else {
      const float ln_sz = logf(Sz);
      const float ln_sy = logf(Sy);
      RowConst rc;
      rc.init(Mz, ln_sz, (Mz - My) + (ln_sz - ln_sy));
      const float delta = rc.delta;

      // ---- phase B. Vector bound: every t_v of a vector is <= p(max z) * max(max(z - y) - delta, 0)
      // (same monotone p() and subtraction as the element test), so a vector whose bound is <= tau
      // holds no clipped term and its S / reverse-KL contributions come from E_k, B_k. Vectors near
      // the peak are summed element by element.
      const float one_m_delta = 1.f - delta;
      float s_fast = 0.f, r_fast = 0.f, s_slow = 0.f, r_slow = 0.f;
      bool slowv[K];
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const float ub = rc.p(zmv[k]) * fmaxf(dmv[k] - delta, 0.f);
        slowv[k] = ub > tau;
        // e-units of vector k (relative to 2^(fl(zmax_k log2e))) -> probabilities
        const float scale = exp2_fast((zmv[k] * kLog2e - rc.c_hi) - rc.c_lo);
        s_fast += slowv[k] ? 0.f : scale * __builtin_fmaf(one_m_delta, ek[k], bk[k]);
        r_fast += slowv[k] ? 0.f : scale * __builtin_fmaf(-delta, ek[k], bk[k]);
        if (__builtin_amdgcn_ballot_w64(slowv[k])) {
          opaque(zr[k]);
          float x[EPV], w[EPV];
          In::decode(zr[k], x);
          In::decode(ylds[k * kThreads + tid], w);
          const int vi = tv + k * kThreads;
#pragma unroll
          for (int e = 0; e < EPV; ++e) {
            const bool valid = slowv[k] && (vi < cv1) && (vi * EPV + e < P.vocab);
            const float p = rc.p(x[e]);
            const float t = p * ((x[e] - w[e]) - delta);
            const bool clipped = t > tau;
            r_slow += valid ? (clipped ? tau : t) : 0.f;
            s_slow += (valid && !clipped) ? (t + p) : 0.f;
          }
          fence_vals(r_slow, s_slow);
        }
      }
      put4(sh, 6, wsum(s_fast + s_slow));
      put4(sh, 7, wsum(r_fast + r_slow));
      __syncthreads();
      if (tid == 0) {
        sh.out[0] = (sh.red[0][6] + sh.red[1][6]) + (sh.red[2][6] + sh.red[3][6]);
        sh.out[1] = (sh.red[0][7] + sh.red[1][7]) + (sh.red[2][7] + sh.red[3][7]);
      }
      __syncthreads();
      float S = 0.f, rkl = 0.f;
      const bool need_rx2 = (MODE == kFused) || chunk == 0;
      if (P.G > 1) {
        if (!exchange<kStage2Units>(sh, P, team, chunk, 1, flag1 + 1u, need_rx2)) break;
        if (need_rx2) {
          const int lane = tid & 63;
          float ls = 0.f, lr = 0.f;
          for (int c = lane; c < P.G; c += 64) {
            ls += __uint_as_float(sh.rx[c * kStage2Units + 0]);
            lr += __uint_as_float(sh.rx[c * kStage2Units + 1]);
          }
          S = wsum(ls);
          rkl = wsum(lr);
        }
      } else {
        S = sh.out[0];
        rkl = sh.out[1];
      }
      if (chunk == 0 && tid == 0) {
        const float ce = (Mz - za) + ln_sz;
        float* st = P.row_stats + 8 * (int64_t)row;
        P.loss[row] = alpha * rkl + (1.f - alpha) * ce;
        P.target_top1[row] = atop;
        if (P.draft_top1) P.draft_top1[row] = dtop;
        st[0] = Mz + ln_sz;
        st[1] = My + ln_sy;
        st[2] = S;
        st[3] = rkl;
        st[4] = Mz;
        st[5] = ln_sz;
        st[6] = delta;
        st[7] = ce;
      }

      if constexpr (MODE == kFused) {
        // ---- phase C: dz (formulas shared with k_bwd through dz_vector)
        DzConst dc;
        dc.init(rc, S, alpha, P.grad_loss ? P.grad_loss[row] : 1.f);
        uint8_t* drow = P.dz + (int64_t)row * P.ld_dz_bytes;
#pragma unroll
        for (int k = 0; k < K; ++k) {
          opaque(zr[k]);
          float x[EPV], w[EPV], o[EPV];
          In::decode(zr[k], x);
          In::decode(ylds[k * kThreads + tid], w);
          dz_vector<EPV>(x, w, slowv[k], __builtin_amdgcn_ballot_w64(slowv[k]) != 0, rc, dc, tau, o);
          const int vi = tv + k * kThreads;
          const int g0 = vi * EPV;
          fix_target<EPV>(o, g0, atop, dc.wce);
#pragma unroll
          for (int e = 0; e < EPV; e += 4) fence_vals(o[e], o[e + 1], o[e + 2], o[e + 3]);
          uint8_t* dst = drow + (int64_t)g0 * OSZ;
          if ((k + 1) * kThreads <= clen && !tail_chunk) {  // uniform: every lane holds a full vector
            store_vec<OutBF16, EPV>(dst, o);
          } else if (vi < cv1) {
            if (g0 + EPV <= P.vocab) {
              store_vec<OutBF16, EPV>(dst, o);
            } else {
              store_partial<OutBF16, EPV>(dst, o, P.vocab - g0);
            }
          }
        }
      }
    }
  }
  if (sh.err && tid == 0) atomicOr(P.flags, (uint32_t)kFlagSpinTimeout);
}

// ---------------------------------------------------------------- streaming backward

constexpr int kBwdVecPerThread = 4;

template <class In, bool OutBF16>
__global__ void __launch_bounds__(kThreads) k_bwd(BwdParams P) {
  constexpr int EPV = In::EPV;
  constexpr int OSZ = OutBF16 ? 2 : 4;
  const int row = blockIdx.y;
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
  const int v0 = blockIdx.x * (kThreads * kBwdVecPerThread) + threadIdx.x;
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
    float zm = x[0], dm = x[0] - w[0];
#pragma unroll
    for (int e = 1; e < EPV; ++e) {
      zm = fmaxf(zm, x[e]);
      dm = fmaxf(dm, x[e] - w[e]);
    }
    const bool slow = rc.p(zm) * fmaxf(dm - rc.delta, 0.f) > tau;
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

__global__ void __launch_bounds__(kThreads) k_accept(AcceptParams P) {
  const int b = blockIdx.x * kThreads + threadIdx.x;
  if (b >= P.n_blocks) return;
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
    while (acc < n && P.draft_top1[start + acc] == P.target_top1[start + acc]) ++acc;
  }
  P.accept_len[b] = acc;
  if (fl) atomicOr(P.flags, fl);
}

__global__ void k_fill_u32(uint32_t* dst, uint32_t value, size_t count) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < count; i += (size_t)gridDim.x * blockDim.x) {
    dst[i] = value;
  }
}

// ---------------------------------------------------------------- instantiation tables

template <int MODE>
void* team_kernel(int in_bf16, int out_bf16, int K) {
  if (MODE != kFused) out_bf16 = 0;
  if (in_bf16) {
    if (out_bf16) return K == 1 ? (void*)k_team<BF16In, true, 1, MODE> : (void*)k_team<BF16In, true, 5, MODE>;
    return K == 1 ? (void*)k_team<BF16In, false, 1, MODE> : (void*)k_team<BF16In, false, 5, MODE>;
  }
  if (out_bf16) return K == 1 ? (void*)k_team<F32In, true, 1, MODE> : (void*)k_team<F32In, true, 5, MODE>;
  return K == 1 ? (void*)k_team<F32In, false, 1, MODE> : (void*)k_team<F32In, false, 5, MODE>;
}

void* team_kernel_any(int mode, int in_bf16, int out_bf16, int K) {
  switch (mode) {
    case kFused: return team_kernel<kFused>(in_bf16, out_bf16, K);
    case kForward: return team_kernel<kForward>(in_bf16, out_bf16, K);
    default: return team_kernel<kTop1>(in_bf16, out_bf16, K);
  }
}

}  // namespace

hipError_t launch_team(const TeamParams& p, int mode, int in_bf16, int out_bf16, int K, int grid, hipStream_t s) {
  void* fn = team_kernel_any(mode, in_bf16, out_bf16, K);
  TeamParams copy = p;
  void* args[] = {&copy};
  return hipLaunchKernel(fn, dim3(grid), dim3(kThreads), args, 0, s);
}

hipError_t team_occupancy(int mode, int in_bf16, int out_bf16, int K, int* blocks_per_cu) {
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, team_kernel_any(mode, in_bf16, out_bf16, K),
                                                      kThreads, 0);
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
  dim3 grid((p.n_blocks + kThreads - 1) / kThreads);
  AcceptParams copy = p;
  void* args[] = {&copy};
  return hipLaunchKernel((void*)k_accept, grid, dim3(kThreads), args, 0, s);
}

hipError_t launch_fill_u32(uint32_t* dst, uint32_t value, size_t count, hipStream_t s) {
  size_t blocks = (count + kThreads - 1) / kThreads;
  if (blocks > 1024) blocks = 1024;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(k_fill_u32, dim3((unsigned)blocks), dim3(kThreads), 0, s, dst, value, count);
  return hipGetLastError();
}

}  // namespace opd
