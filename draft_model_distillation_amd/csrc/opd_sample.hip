// Stochastic verification at a sampling temperature (speculative sampling) of packed draft blocks.
//
// The pages name temperature as a parameter to tune when the drafter is combined with the target
// ("AdaFlash: Adaptive Speculative Decoding via On-Policy Distilled Diffusion Drafters", skills
// directory page, section "Implementation Steps") but give no acceptance rule for it; the rule here
// is the published speculative-sampling one (Leviathan et al. 2023; Chen et al. 2023): a proposal x
// at row r is kept when u_r p_r(x) <= q_r(x), with p = softmax(z / T), q = softmax(y / T); at the
// first rejection the output token is drawn from max(0, q - p) (normalised), after a fully accepted
// budget n < n_b from q of the next row. Blocks are the packed layout of "AdaFlash: Adaptive
// Speculative Decoding with Online Self-Improvement ..." (besthub.dev article), sections "2. Adaptive
// Length Head for Token-Level Variance" and "Infrastructure: Async Training & Variable-Length
// Batching".
//
// Two kernels:
//   k_row_lse_t     one workgroup per row: one streaming read of z and y (4V bytes for bf16) giving
//                   log2 sum 2^(x log2e / T) of both rows as (reference, log2 of the sum relative to
//                   it), with per-vector references so that no row maximum is needed first.
//   k_sample_verify one workgroup per block: the accept decisions of its verified rows (one lane
//                   each, two element gathers per row), then, if a token is to be drawn, the inverse
//                   CDF of the draw row's weights in index order: wave-sized tiles of 64 vectors,
//                   tile sums from an inclusive wave scan, a scan over lane groups of tiles to find
//                   the tile, and the same wave scan inside that tile to find the element.
// Draws are taken on sums formed in a fixed order, so results are deterministic; where rounding of
// those sums leaves the target at a tile or vector edge, the last positive weight before the edge
// is taken.
//
// Compiled with the default IEEE mode, like the epilogue kernels.

#include <stdint.h>

#include "opd_internal.h"

namespace opd {
namespace {

constexpr float kNegInf = -__builtin_inff();
constexpr int kWaves = kThreads / 64;

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ uint4 ld16(const uint8_t* p) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// 16 bytes of logits -> EPV floats (bf16 -> fp32 is exact)
template <bool BF16>
struct Dec;
template <>
struct Dec<true> {
  static constexpr int EPV = 8;
  __device__ static void run(const uint4& v, float (&x)[8]) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  __device__ static float elem(const uint8_t* row, int i) {
    return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(row)[i] << 16);
  }
};
template <>
struct Dec<false> {
  static constexpr int EPV = 4;
  __device__ static void run(const uint4& v, float (&x)[4]) {
    x[0] = __uint_as_float(v.x);
    x[1] = __uint_as_float(v.y);
    x[2] = __uint_as_float(v.z);
    x[3] = __uint_as_float(v.w);
  }
  __device__ static float elem(const uint8_t* row, int i) { return reinterpret_cast<const float*>(row)[i]; }
};

// Adds one vector to a running (reference, sum) pair: sum 2^(x c - ref). The vector's own
// reference cm = fl(max x * c) makes every exponent fma(x, c, -cm) <= 0 and exact near the maximum;
// one more exp2 moves whichever sum has the smaller reference.
template <int EPV>
__device__ __forceinline__ void add_vector(const float (&x)[EPV], float c, float& ref, float& sum) {
  float m = x[0];
#pragma unroll
  for (int e = 1; e < EPV; ++e) m = fmaxf(m, x[e]);
  const float cm = m * c;
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < EPV; ++e) s += ex2(__builtin_fmaf(x[e], c, -cm));
  if (m == kNegInf) return;  // a vector wholly past the vocabulary
  const bool up = cm > ref;
  const float f = (ref == kNegInf) ? 0.f : ex2(up ? ref - cm : cm - ref);
  sum = up ? __builtin_fmaf(sum, f, s) : __builtin_fmaf(s, f, sum);
  ref = up ? cm : ref;
}

__device__ __forceinline__ void combine(float& ref, float& sum, float ref2, float sum2) {
  const float r = fmaxf(ref, ref2);
  if (r == kNegInf) return;
  const float a = (ref == kNegInf) ? 0.f : sum * ex2(ref - r);
  const float b = (ref2 == kNegInf) ? 0.f : sum2 * ex2(ref2 - r);
  ref = r;
  sum = a + b;
}

template <bool BF16>
__global__ void __launch_bounds__(kThreads) k_row_lse_t(SampleParams P) {
  using D = Dec<BF16>;
  constexpr int EPV = D::EPV;
  constexpr int U = 4;  // vectors per tensor in flight per thread
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const uint8_t* zr = P.z + (int64_t)row * P.ld_bytes;
  const uint8_t* yr = P.y + (int64_t)row * P.ld_bytes;
  const float c = P.c;
  const int nvec = P.nvec;
  float rz = kNegInf, sz = 0.f, ry = kNegInf, sy = 0.f;
  for (int v0 = tid; v0 < nvec; v0 += kThreads * U) {
    uint4 a[U], b[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int v = v0 + u * kThreads;
      if (v < nvec) {
        a[u] = ld16(zr + (int64_t)v * 16);
        b[u] = ld16(yr + (int64_t)v * 16);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int v = v0 + u * kThreads;
      if (v < nvec) {
        float x[EPV], w[EPV];
        D::run(a[u], x);
        D::run(b[u], w);
        if (v == nvec - 1) {  // the pad past the vocabulary takes no part
          const int valid = P.vocab - v * EPV;
#pragma unroll
          for (int e = 0; e < EPV; ++e) {
            x[e] = e < valid ? x[e] : kNegInf;
            w[e] = e < valid ? w[e] : kNegInf;
          }
        }
        add_vector<EPV>(x, c, rz, sz);
        add_vector<EPV>(w, c, ry, sy);
      }
    }
  }
  // wave butterfly, then the four waves in a fixed order
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const float r2 = __shfl_xor(rz, m), s2 = __shfl_xor(sz, m);
    const float r3 = __shfl_xor(ry, m), s3 = __shfl_xor(sy, m);
    combine(rz, sz, r2, s2);
    combine(ry, sy, r3, s3);
  }
  __shared__ float part[kWaves][4];
  const int lane = tid & 63, wave = tid >> 6;
  if (lane == 0) {
    part[wave][0] = rz;
    part[wave][1] = sz;
    part[wave][2] = ry;
    part[wave][3] = sy;
  }
  __syncthreads();
  if (tid == 0) {
    float a = part[0][0], sa = part[0][1], b = part[0][2], sb = part[0][3];
    for (int q = 1; q < kWaves; ++q) {
      combine(a, sa, part[q][0], part[q][1]);
      combine(b, sb, part[q][2], part[q][3]);
    }
    float* st = P.stats + 4 * (int64_t)row;
    st[0] = a;
    st[1] = __builtin_amdgcn_logf(sa);  // log2
    st[2] = b;
    st[3] = __builtin_amdgcn_logf(sb);
  }
}

// Weights of the draw row: kind 1 = max(0, q - p), kind 2 = q.
struct DrawRow {
  const uint8_t* z;
  const uint8_t* y;
  float c, cz, lz, cy, ly;
  int kind;
};

template <bool BF16>
__device__ __forceinline__ void vector_weights(const DrawRow& d, int v, int nvec, int vocab,
                                               float (&w)[Dec<BF16>::EPV]) {
  using D = Dec<BF16>;
  constexpr int EPV = D::EPV;
  if (v >= nvec) {
#pragma unroll
    for (int e = 0; e < EPV; ++e) w[e] = 0.f;
    return;
  }
  float yv[EPV];
  D::run(ld16(d.y + (int64_t)v * 16), yv);
  if (d.kind == 1) {
    float zv[EPV];
    D::run(ld16(d.z + (int64_t)v * 16), zv);
#pragma unroll
    for (int e = 0; e < EPV; ++e) {
      const float q = ex2(__builtin_fmaf(yv[e], d.c, -d.cy) - d.ly);
      const float p = ex2(__builtin_fmaf(zv[e], d.c, -d.cz) - d.lz);
      w[e] = fmaxf(q - p, 0.f);
    }
  } else {
#pragma unroll
    for (int e = 0; e < EPV; ++e) w[e] = ex2(__builtin_fmaf(yv[e], d.c, -d.cy) - d.ly);
  }
  const int valid = vocab - v * EPV;
#pragma unroll
  for (int e = 0; e < EPV; ++e) w[e] = e < valid ? w[e] : 0.f;
}

// inclusive scan over the 64 lanes of a wave (fixed order of additions)
__device__ __forceinline__ float wave_scan(float x, int lane) {
#pragma unroll
  for (int k = 1; k < 64; k <<= 1) {
    const float t = __shfl_up(x, k);
    x += lane >= k ? t : 0.f;
  }
  return x;
}

template <bool BF16>
__global__ void __launch_bounds__(kThreads) k_sample_verify(SampleParams P) {
  using D = Dec<BF16>;
  constexpr int EPV = D::EPV;
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ float tile_sum[kMaxSampleTiles];
  __shared__ int s_first;
  __shared__ int s_tile;
  __shared__ float s_rem;
  __shared__ int s_idx;

  const int start = P.offsets[b], end = P.offsets[b + 1];
  if (start < 0 || end < start || end > P.n_rows) {
    if (tid == 0) {
      atomicOr(P.flags, kFlagBadOffsets);
      P.accept_len[b] = 0;
      P.token[b] = -1;
    }
    return;
  }
  const int nb = end - start;
  const int Lb = P.L[b];
  if (Lb < 0 && tid == 0) atomicOr(P.flags, kFlagNegL);
  const int n = min(max(Lb, 0), nb);

  // ---- decisions: one lane per verified row, the first rejected row wins
  int first = n;
  for (int j0 = 0; j0 < n; j0 += kThreads) {
    if (tid == 0) s_first = 0x7fffffff;
    __syncthreads();
    const int j = j0 + tid;
    if (j < n) {
      const int r = start + j;
      const int x = P.draft[r];
      bool rej;
      if (x < 0 || x >= P.vocab) {
        rej = true;
        atomicOr(P.flags, kFlagBadToken);
      } else {
        const float* st = P.stats + 4 * (int64_t)r;
        const float zx = D::elem(P.z + (int64_t)r * P.ld_bytes, x);
        const float yx = D::elem(P.y + (int64_t)r * P.ld_bytes, x);
        const float p = ex2(__builtin_fmaf(zx, P.c, -st[0]) - st[1]);
        const float q = ex2(__builtin_fmaf(yx, P.c, -st[2]) - st[3]);
        rej = P.u_accept[r] * p > q;
      }
      if (rej) atomicMin(&s_first, j);
    }
    __syncthreads();
    const int f = s_first;
    __syncthreads();
    if (f != 0x7fffffff) {
      first = f;
      break;
    }
  }
  if (tid == 0) P.accept_len[b] = first;

  DrawRow d;
  int draw_row;
  if (first < n) {
    draw_row = start + first;
    d.kind = 1;
  } else if (n < nb) {
    draw_row = start + n;
    d.kind = 2;
  } else {
    if (tid == 0) P.token[b] = -1;
    return;
  }
  d.z = P.z + (int64_t)draw_row * P.ld_bytes;
  d.y = P.y + (int64_t)draw_row * P.ld_bytes;
  d.c = P.c;
  {
    const float* st = P.stats + 4 * (int64_t)draw_row;
    d.cz = st[0];
    d.lz = st[1];
    d.cy = st[2];
    d.ly = st[3];
  }
  const int nvec = P.nvec;
  const int n_tiles = (nvec + 63) / 64;

  // ---- pass 1: per tile (64 vectors, one wave) the sum of its weights, from the same wave scan
  // that pass 2 repeats inside the chosen tile; a residual that vanishes everywhere falls back to q
  for (int attempt = 0; attempt < 2; ++attempt) {
    for (int t = wave; t < n_tiles; t += kWaves) {
      float w[EPV];
      vector_weights<BF16>(d, t * 64 + lane, nvec, P.vocab, w);
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < EPV; ++e) s += w[e];
      s = wave_scan(s, lane);
      if (lane == 63) tile_sum[t] = s;
    }
    __syncthreads();
    if (d.kind == 2) break;
    // any positive tile?
    int any = 0;
    for (int t = tid; t < n_tiles; t += kThreads) any |= tile_sum[t] > 0.f;
    if (__syncthreads_or(any)) break;
    d.kind = 2;
  }

  // ---- find the tile: lane l of wave 0 owns a contiguous group of tiles
  if (wave == 0) {
    const int g = (n_tiles + 63) / 64;
    const int t0 = min(lane * g, n_tiles), t1 = min(t0 + g, n_tiles);
    float own = 0.f;
    for (int t = t0; t < t1; ++t) own += tile_sum[t];
    const float incl = wave_scan(own, lane);
    const float total = __shfl(incl, 63);
    const float target = P.u_resample[b] * total;
    const float before = __shfl_up(incl, 1);
    const float lo = lane == 0 ? 0.f : before;
    const bool here = lo <= target && target < incl;
    const uint64_t m = __ballot(here);
    if (m) {
      const int l = __ffsll((unsigned long long)m) - 1;
      if (lane == l) {
        float acc = lo;
        int tile = -1;
        float rem = 0.f;
        int last_pos = -1;
        for (int t = t0; t < t1; ++t) {
          if (tile_sum[t] > 0.f) last_pos = t;
          if (acc + tile_sum[t] > target) {
            tile = t;
            rem = target - acc;
            break;
          }
          acc += tile_sum[t];
        }
        if (tile < 0) {  // rounding left the target at the group's end
          tile = last_pos;
          rem = tile_sum[last_pos];
        }
        s_tile = tile;
        s_rem = rem;
      }
    } else if (lane == 0) {  // u * total rounded up to total: the last tile with weight
      int tile = -1;
      for (int t = n_tiles - 1; t >= 0; --t)
        if (tile_sum[t] > 0.f) {
          tile = t;
          break;
        }
      s_tile = tile;
      s_rem = tile >= 0 ? tile_sum[tile] : 0.f;
    }
  }
  __syncthreads();

  // ---- pass 2: inside the tile, the same wave scan over its 64 vectors, then one lane's elements
  if (wave == 0) {
    const int tile = s_tile;
    int idx = -1;
    if (tile >= 0) {
      const float rem = s_rem;
      const int v = tile * 64 + lane;
      float w[EPV];
      vector_weights<BF16>(d, v, nvec, P.vocab, w);
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < EPV; ++e) s += w[e];
      const float incl = wave_scan(s, lane);
      const float before = __shfl_up(incl, 1);
      const float lo = lane == 0 ? 0.f : before;
      // last positive weight of this lane's vector (for the edge cases)
      int lastp = -1;
#pragma unroll
      for (int e = 0; e < EPV; ++e) lastp = w[e] > 0.f ? v * EPV + e : lastp;
      const bool here = lo <= rem && rem < incl;
      const uint64_t m = __ballot(here);
      int pick = -1;
      if (m) {
        const int l = __ffsll((unsigned long long)m) - 1;
        if (lane == l) {
          float acc = lo;
#pragma unroll
          for (int e = 0; e < EPV; ++e) {
            acc += w[e];
            if (pick < 0 && acc > rem) pick = v * EPV + e;
          }
          if (pick < 0) pick = lastp;
        }
        pick = __shfl(pick, l);
      } else {  // rem at or past the tile's end: the tile's last positive weight
        int best = lastp;
#pragma unroll
        for (int k = 32; k >= 1; k >>= 1) best = max(best, __shfl_xor(best, k));
        pick = best;
      }
      idx = pick;
    }
    if (lane == 0) P.token[b] = idx;
  }
}

}  // namespace

hipError_t launch_sample_verify(const SampleParams& p, int in_bf16, hipStream_t s) {
  SampleParams copy = p;
  void* args[] = {&copy};
  if (p.n_rows > 0) {
    void* fn = in_bf16 ? (void*)k_row_lse_t<true> : (void*)k_row_lse_t<false>;
    hipError_t e = hipLaunchKernel(fn, dim3((unsigned)p.n_rows), dim3(kThreads), args, 0, s);
    if (e != hipSuccess) return e;
  }
  if (p.n_blocks > 0) {
    void* fn = in_bf16 ? (void*)k_sample_verify<true> : (void*)k_sample_verify<false>;
    hipError_t e = hipLaunchKernel(fn, dim3((unsigned)p.n_blocks), dim3(kThreads), args, 0, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace opd
