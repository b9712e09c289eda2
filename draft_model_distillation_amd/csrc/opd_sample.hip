// Stochastic verification at a sampling temperature (speculative sampling) of packed draft blocks.
//
// The pages name temperature as a parameter to tune when the drafter is combined with the target
// ("Adaflash Adaptive Speculative Decoding", skills-directory card, section "Implementation
// Steps") but give no acceptance rule for it; the rule here is the published speculative-sampling
// one (Leviathan et al. 2023; Chen et al. 2023): a proposal x at row r is kept when
// u_r p_r(x) <= q_r(x), with p = softmax(z / T), q = softmax(y / T); at the first rejection the
// output token is drawn from max(0, q - p) (normalised), after a fully accepted budget n < n_b from
// q of the next row. Blocks are the packed layout of "AdaFlash: Adaptive
// Speculative Decoding with Online Self-Improvement ..." (besthub.dev article), sections "2. Adaptive
// Length Head for Token-Level Variance" and "Infrastructure: Async Training & Variable-Length
// Batching".
//
// Three kernels:
//   k_row_lse_t     one workgroup per row the verification can read (a block's n verified rows and
//                   the row after them): one streaming read of z and y (4V bytes for bf16) giving
//                   log2 sum 2^(x log2e / T) of both rows as (reference, log2 of the sum relative to
//                   it), with per-vector references so that no row maximum is needed first.
//   k_sample_slices (block, slice) workgroups: each takes the block's accept decisions (one lane per
//                   verified row, two element gathers each) and, if a token is to be drawn, the
//                   weight sum of one of kSampleSlices contiguous slices of the draw row, so that the
//                   draw row is read by many workgroups at once.
//   k_sample_pick   one workgroup per block: the decisions again (writing accept_len), the slice
//                   whose running sum passes u * total, the tile (64 vectors) inside it, and the
//                   element inside the tile, each level from the same sums as the level above.
// A tile's sum is the last value of an inclusive wave scan, a slice's the sequential sum of its tile
// sums, the total the sequential sum of the slice sums: fixed orders, so results are deterministic;
// where rounding leaves the target at a slice, tile or vector edge, the last positive weight before
// the edge is taken.
//
// Compiled with the default IEEE mode, like the epilogue kernels.

#include <stdint.h>

#include "opd_internal.h"

namespace opd {
namespace {

constexpr float kNegInf = -__builtin_inff();
constexpr int kWaves = kThreads / 64;
constexpr unsigned kRowSlots = 17;  // a k = 16 block's verified rows and its bonus row

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
__device__ void row_lse_one(const SampleParams& P, int row) {
  using D = Dec<BF16>;
  constexpr int EPV = D::EPV;
  constexpr int U = 8;  // vectors per tensor in flight per thread
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

template <bool BF16>
__global__ void __launch_bounds__(kThreads) k_row_lse_t(SampleParams P) {
  // Only rows the verification can read: the first min(n + 1, n_b) rows of block blockIdx.x (the n
  // verified ones and the row a bonus token would be drawn from), rows blockIdx.y, + gridDim.y, ...
  const int b = blockIdx.x;
  const int start = P.offsets[b], end = P.offsets[b + 1];
  if (start < 0 || end < start || end > P.n_rows) return;
  const int nb = end - start;
  const int m = min(min(max(P.L[b], 0), nb) + 1, nb);
  for (int j = blockIdx.y; j < m; j += gridDim.y) {
    if (j != (int)blockIdx.y) __syncthreads();  // the previous row is done with `part`
    row_lse_one<BF16>(P, start + j);
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

// Sum of the weights of tile t (64 vectors, one per lane of the calling wave): the last value of
// the inclusive wave scan, so that the search inside a tile sees exactly this total.
template <bool BF16>
__device__ __forceinline__ float tile_total(const DrawRow& d, int t, int nvec, int vocab, int lane) {
  constexpr int EPV = Dec<BF16>::EPV;
  float w[EPV];
  vector_weights<BF16>(d, t * 64 + lane, nvec, vocab, w);
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < EPV; ++e) s += w[e];
  return __shfl(wave_scan(s, lane), 63);
}

// Outcome of a block's decisions: accept length, and the row and kind of the draw (kind 0: none).
// bad = malformed offsets. Every thread of the workgroup calls it (it synchronises).
struct Outcome {
  int first;
  int row;
  int kind;
  bool bad;
};

template <bool BF16>
__device__ Outcome decide(const SampleParams& P, int b, bool raise_flags, int* s_first) {
  using D = Dec<BF16>;
  const int tid = threadIdx.x;
  Outcome o{0, -1, 0, false};
  const int start = P.offsets[b], end = P.offsets[b + 1];
  if (start < 0 || end < start || end > P.n_rows) {
    if (raise_flags && tid == 0) atomicOr(P.flags, kFlagBadOffsets);
    o.bad = true;
    return o;
  }
  const int nb = end - start;
  const int Lb = P.L[b];
  if (raise_flags && Lb < 0 && tid == 0) atomicOr(P.flags, kFlagNegL);
  const int n = min(max(Lb, 0), nb);
  int first = n;
  for (int j0 = 0; j0 < n; j0 += kThreads) {
    if (tid == 0) *s_first = 0x7fffffff;
    __syncthreads();
    const int j = j0 + tid;
    if (j < n) {
      const int r = start + j;
      const int x = P.draft[r];
      bool rej;
      if (x < 0 || x >= P.vocab) {
        rej = true;
        if (raise_flags) atomicOr(P.flags, kFlagBadToken);
      } else {
        const float* st = P.stats + 4 * (int64_t)r;
        const float zx = D::elem(P.z + (int64_t)r * P.ld_bytes, x);
        const float yx = D::elem(P.y + (int64_t)r * P.ld_bytes, x);
        const float p = ex2(__builtin_fmaf(zx, P.c, -st[0]) - st[1]);
        const float q = ex2(__builtin_fmaf(yx, P.c, -st[2]) - st[3]);
        rej = P.u_accept[r] * p > q;
      }
      if (rej) atomicMin(s_first, j);
    }
    __syncthreads();
    const int f = *s_first;
    __syncthreads();
    if (f != 0x7fffffff) {
      first = f;
      break;
    }
  }
  o.first = first;
  if (first < n) {
    o.row = start + first;
    o.kind = 1;
  } else if (n < nb) {
    o.row = start + n;
    o.kind = 2;
  }
  return o;
}

template <bool BF16>
__device__ __forceinline__ DrawRow draw_row(const SampleParams& P, int row, int kind) {
  DrawRow d;
  d.z = P.z + (int64_t)row * P.ld_bytes;
  d.y = P.y + (int64_t)row * P.ld_bytes;
  d.c = P.c;
  const float* st = P.stats + 4 * (int64_t)row;
  d.cz = st[0];
  d.lz = st[1];
  d.cy = st[2];
  d.ly = st[3];
  d.kind = kind;
  return d;
}

// Tiles [t0, t1) of slice s of a row with n_tiles tiles.
__device__ __forceinline__ void slice_tiles(int s, int n_tiles, int& t0, int& t1) {
  const int per = (n_tiles + kSampleSlices - 1) / kSampleSlices;
  t0 = min(s * per, n_tiles);
  t1 = min(t0 + per, n_tiles);
}

// Sums of the tiles of one slice into tsum[0 .. t1-t0) (all four waves), then their sequential sum.
template <bool BF16>
__device__ float slice_total(const DrawRow& d, int t0, int t1, int nvec, int vocab, float* tsum) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int t = t0 + wave; t < t1; t += kWaves) {
    const float v = tile_total<BF16>(d, t, nvec, vocab, lane);
    if (lane == 0) tsum[t - t0] = v;
  }
  __syncthreads();
  float acc = 0.f;
  for (int t = t0; t < t1; ++t) acc += tsum[t - t0];  // every thread: the same sequence
  return acc;
}

// Grid (blocks of this batch, kSampleSlices): the weight sum of one slice of each block's draw row.
template <bool BF16>
__global__ void __launch_bounds__(kThreads) k_sample_slices(SampleParams P) {
  __shared__ int s_first;
  __shared__ float tsum[kMaxSampleTiles / kSampleSlices];
  const int b = P.block0 + blockIdx.x;
  const int s = blockIdx.y;
  const Outcome o = decide<BF16>(P, b, false, &s_first);
  if (o.kind == 0) return;
  const DrawRow d = draw_row<BF16>(P, o.row, o.kind);
  const int n_tiles = (P.nvec + 63) / 64;
  int t0, t1;
  slice_tiles(s, n_tiles, t0, t1);
  const float total = slice_total<BF16>(d, t0, t1, P.nvec, P.vocab, tsum);
  if (threadIdx.x == 0) P.slices[(int64_t)blockIdx.x * kSampleSlices + s] = total;
}

// Grid (blocks of this batch): accept length, then the draw: slice, tile, element.
template <bool BF16>
__global__ void __launch_bounds__(kThreads) k_sample_pick(SampleParams P) {
  using D = Dec<BF16>;
  constexpr int EPV = D::EPV;
  __shared__ int s_first;
  __shared__ float tsum[kMaxSampleTiles / kSampleSlices];
  __shared__ float ssum[kSampleSlices];
  __shared__ int s_tile;
  __shared__ float s_rem;
  const int b = P.block0 + blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const Outcome o = decide<BF16>(P, b, true, &s_first);
  if (tid == 0) P.accept_len[b] = o.bad ? 0 : o.first;
  if (o.kind == 0) {
    if (tid == 0) P.token[b] = -1;
    return;
  }
  const int n_tiles = (P.nvec + 63) / 64;
  DrawRow d = draw_row<BF16>(P, o.row, o.kind);
  if (tid < kSampleSlices) {
    float* const slot = P.slices + (int64_t)blockIdx.x * kSampleSlices + tid;
    ssum[tid] = *slot;
    // The slice sums share the workspace with the row-team kernel's exchange units; zeros there read
    // as units holding flag 0, which no exchange ever waits for.
    *slot = 0.f;
  }
  __syncthreads();
  float total = 0.f;
  for (int s = 0; s < kSampleSlices; ++s) total += ssum[s];
  if (d.kind == 1 && !(total > 0.f)) {
    // the residual vanished everywhere: draw from q, whose slice sums this workgroup forms itself
    // (rare: q <= p at every index in fp32)
    d.kind = 2;
    for (int s = 0; s < kSampleSlices; ++s) {
      int t0, t1;
      slice_tiles(s, n_tiles, t0, t1);
      const float v = slice_total<BF16>(d, t0, t1, P.nvec, P.vocab, tsum);
      __syncthreads();  // tsum is reused by the next slice
      if (tid == 0) ssum[s] = v;
    }
    __syncthreads();
    total = 0.f;
    for (int s = 0; s < kSampleSlices; ++s) total += ssum[s];
  }
  const float target = P.u_resample[b] * total;
  // the slice: first whose running sum passes the target; at a rounding edge the last with weight
  int sl = -1;
  float rem = 0.f;
  {
    float acc = 0.f;
    int last = -1;
    for (int s = 0; s < kSampleSlices; ++s) {
      if (ssum[s] > 0.f) last = s;
      if (sl < 0 && acc + ssum[s] > target) {
        sl = s;
        rem = target - acc;
      }
      if (sl < 0) acc += ssum[s];
    }
    if (sl < 0) {
      sl = last;
      rem = last >= 0 ? ssum[last] : 0.f;
    }
  }
  if (sl < 0) {  // no weight at all
    if (tid == 0) P.token[b] = -1;
    return;
  }
  // the tile inside the slice, from the same tile sums the slice total was made of
  int t0, t1;
  slice_tiles(sl, n_tiles, t0, t1);
  slice_total<BF16>(d, t0, t1, P.nvec, P.vocab, tsum);
  if (tid == 0) {
    float acc = 0.f;
    int tile = -1, last = -1;
    float r2 = 0.f;
    for (int t = t0; t < t1; ++t) {
      const float v = tsum[t - t0];
      if (v > 0.f) last = t;
      if (acc + v > rem) {
        tile = t;
        r2 = rem - acc;
        break;
      }
      acc += v;
    }
    if (tile < 0) {
      tile = last;
      r2 = last >= 0 ? tsum[last - t0] : 0.f;
    }
    s_tile = tile;
    s_rem = r2;
  }
  __syncthreads();
  // the element inside the tile: the same wave scan over its 64 vectors, then one lane's elements
  if (wave == 0) {
    const int tile = s_tile;
    int idx = -1;
    if (tile >= 0) {
      const float r = s_rem;
      const int v = tile * 64 + lane;
      float w[EPV];
      vector_weights<BF16>(d, v, P.nvec, P.vocab, w);
      float sv = 0.f;
#pragma unroll
      for (int e = 0; e < EPV; ++e) sv += w[e];
      const float incl = wave_scan(sv, lane);
      const float before = __shfl_up(incl, 1);
      const float lo = lane == 0 ? 0.f : before;
      int lastp = -1;  // last positive weight of this lane's vector (for the edge cases)
#pragma unroll
      for (int e = 0; e < EPV; ++e) lastp = w[e] > 0.f ? v * EPV + e : lastp;
      const uint64_t m = __ballot(lo <= r && r < incl);
      if (m) {
        const int l = __ffsll((unsigned long long)m) - 1;
        int pick = -1;
        if (lane == l) {
          float acc = lo;
#pragma unroll
          for (int e = 0; e < EPV; ++e) {
            acc += w[e];
            if (pick < 0 && acc > r) pick = v * EPV + e;
          }
          if (pick < 0) pick = lastp;
        }
        idx = __shfl(pick, l);
      } else {  // r at or past the tile's end: the tile's last positive weight
        int best = lastp;
#pragma unroll
        for (int k = 32; k >= 1; k >>= 1) best = max(best, __shfl_xor(best, k));
        idx = best;
      }
    }
    if (lane == 0) P.token[b] = idx;
  }
}

}  // namespace

hipError_t launch_sample_verify(const SampleParams& p, int in_bf16, hipStream_t s) {
  SampleParams q = p;
  void* args[] = {&q};
  if (p.n_rows > 0 && p.n_blocks > 0) {
    // one workgroup per (block, row slot): a block of up to kRowSlots rows needs one pass
    void* fn = in_bf16 ? (void*)k_row_lse_t<true> : (void*)k_row_lse_t<false>;
    hipError_t e = hipLaunchKernel(fn, dim3((unsigned)p.n_blocks, kRowSlots), dim3(kThreads), args, 0, s);
    if (e != hipSuccess) return e;
  }
  // blocks in batches whose slice sums fit the workspace
  for (int32_t b0 = 0; b0 < p.n_blocks; b0 += kSampleBatch) {
    q.block0 = b0;
    const unsigned nb = (unsigned)min(p.n_blocks - b0, kSampleBatch);
    void* f1 = in_bf16 ? (void*)k_sample_slices<true> : (void*)k_sample_slices<false>;
    hipError_t e = hipLaunchKernel(f1, dim3(nb, kSampleSlices), dim3(kThreads), args, 0, s);
    if (e != hipSuccess) return e;
    void* f2 = in_bf16 ? (void*)k_sample_pick<true> : (void*)k_sample_pick<false>;
    e = hipLaunchKernel(f2, dim3(nb), dim3(kThreads), args, 0, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace opd
