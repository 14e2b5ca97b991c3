// Batched lossless draft verification: HIP kernels for gfx950 (MI355X) and the C-ABI in sv.h.
//
// The acceptance rule ("From draft-then-verify to DSpark", section "How speculative decoding
// works") needs, per request, the full-vocabulary normalisers of 2k+1 softmax rows (k+1 target,
// k draft), the probabilities p(x), q(x) of the k proposals, the first rejected slot, and one
// inverse-CDF draw from max(0, p - q) at that slot (or from p at the slot after the last draft).
// Everything but the normalisers and the final draw is O(k) work; the normalisers and the draw
// stream whole vocabulary rows from HBM, so the kernels are organised around reading each used
// row once with 128-bit loads:
//
//   sv_row_stats    (pass 1) one work-group per (request, row, vocabulary chunk). Each thread
//                   keeps an online (offset, sum) pair: the sum of 2^(c*z - o) over its elements,
//                   with c = log2(e) / temperature and o an integer upper bound of c * max(z).
//                   Because o is an integer, rescaling a partial sum to a new offset is an exact
//                   power-of-two scaling (ldexp), so the cross-lane, cross-wave and cross-chunk
//                   combines add no rounding beyond the additions themselves.
//   sv_resolve      (pass 2) one work-group per (request, vocabulary chunk). Every group combines
//                   the request's pass-1 partials in fp64, recomputes p(x), q(x), the accept
//                   decisions and the first rejection n (a few dozen values, identical in every
//                   group), then sums its chunk of the draw weights w into fp64. The last group
//                   of the request to finish (atomic counter) scans the fp64 chunk sums, picks
//                   the chunk holding r * Z, and finds the token with a block-wide fp64 scan.
//   sv_greedy_stats / sv_greedy_finish: per-chunk argmax (lowest index on ties), then a
//                   per-request combine and match scan.
//
// No MFMA: nothing here is a dense contraction. All floating-point contraction is explicit
// (the file is compiled with -ffp-contract=off) so that the same weight is computed bit for bit
// in the chunk-sum pass and in the final scan.

#include <hip/hip_runtime.h>

#include <float.h>
#include <math.h>
#include <stdint.h>

#include <climits>
#include <cstdio>
#include <string>

#include "sv.h"

namespace {

constexpr int kBlock = 256;  // threads per work-group: 4 wave64s
constexpr int kWaves = kBlock / 64;
constexpr int kMaxK = 64;
constexpr int kMaxB = 1 << 20;
constexpr int kMaxV = 1 << 26;
constexpr int kUnroll = 4;  // 128-bit loads in flight per thread in the streaming loops

// ---------------------------------------------------------------------------------------------
// Work decomposition (host side, shared by the workspace query and the launches).

struct Plan {
  int C;   // vocabulary chunks per row, sampling pass 1
  int C2;  // vocabulary chunks per request, sampling pass 2
  int Cg;  // vocabulary chunks per row, greedy pass
};

int chunks_for(long rows, int V, long target_groups, int min_elems, int max_chunks) {
  long c = (target_groups + rows - 1) / rows;
  long cap = V / min_elems;
  if (c > cap) c = cap;
  if (c > max_chunks) c = max_chunks;
  if (c < 1) c = 1;
  return (int)c;
}

Plan make_plan(int B, int K, int V) {
  Plan p;
  p.C = chunks_for((long)B * (2 * K + 1), V, 8192, 4096, 256);
  p.C2 = chunks_for(B, V, 2048, 2048, 64);
  p.Cg = chunks_for((long)B * (K + 1), V, 8192, 4096, 256);
  return p;
}

struct Layout {
  size_t stats;     // float2 [B][2K+1][C]   sampling pass-1 partials (offset, sum)
  size_t zpart;     // double [B][C2]        sampling pass-2 chunk sums
  size_t counters;  // uint32 [B]            sampling pass-2 arrival counters
  size_t gstats;    // float2 [B][K+1][Cg]   greedy partials (value, index bits)
  size_t total;
};

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

Layout make_layout(int B, int K, int V, const Plan& p) {
  Layout L;
  size_t off = 0;
  L.stats = off;
  off = align_up(off + sizeof(float2) * (size_t)B * (2 * K + 1) * p.C, 256);
  L.zpart = off;
  off = align_up(off + sizeof(double) * (size_t)B * p.C2, 256);
  L.counters = off;
  off = align_up(off + sizeof(uint32_t) * (size_t)B, 256);
  L.gstats = 0;  // greedy calls reuse the front of the workspace
  size_t g = align_up(sizeof(float2) * (size_t)B * (K + 1) * p.Cg, 256);
  L.total = off > g ? off : g;
  return L;
}

// ---------------------------------------------------------------------------------------------
// Row access: groups of E consecutive elements, one 128-bit load per group when the rows are
// 16-byte aligned (VEC), one element per group otherwise. Raw loads are kept separate from the
// unpacking so that the streaming loops can hold the next groups in flight while the current
// ones are reduced.

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

template <typename T, bool VEC>
struct Rows;

template <>
struct Rows<float, true> {
  static constexpr int E = 4;
  using Raw = float4;
  __device__ static Raw load(const float* row, int g) {
    return reinterpret_cast<const float4*>(row)[g];
  }
  __device__ static void unpack(const Raw& v, float* f) {
    f[0] = v.x; f[1] = v.y; f[2] = v.z; f[3] = v.w;
  }
  __device__ static float at(const float* row, int i) { return row[i]; }
};

template <>
struct Rows<uint16_t, true> {
  static constexpr int E = 8;
  using Raw = uint4;
  __device__ static Raw load(const uint16_t* row, int g) {
    return reinterpret_cast<const uint4*>(row)[g];
  }
  __device__ static void unpack(const Raw& v, float* f) {
    f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x); f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
    f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z); f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
  }
  __device__ static float at(const uint16_t* row, int i) {
    return __uint_as_float((uint32_t)row[i] << 16);
  }
};

template <>
struct Rows<float, false> {
  static constexpr int E = 1;
  using Raw = float;
  __device__ static Raw load(const float* row, int g) { return row[g]; }
  __device__ static void unpack(const Raw& v, float* f) { f[0] = v; }
  __device__ static float at(const float* row, int i) { return row[i]; }
};

template <>
struct Rows<uint16_t, false> {
  static constexpr int E = 1;
  using Raw = uint16_t;
  __device__ static Raw load(const uint16_t* row, int g) { return row[g]; }
  __device__ static void unpack(const Raw& v, float* f) {
    f[0] = __uint_as_float((uint32_t)v << 16);
  }
  __device__ static float at(const uint16_t* row, int i) {
    return __uint_as_float((uint32_t)row[i] << 16);
  }
};

__device__ __forceinline__ int clamp_k(const int32_t* num_draft, int b, int K) {
  if (num_draft == nullptr) return K;
  const int k = num_draft[b];
  return k < 0 ? 0 : (k > K ? K : k);
}

// Streams groups [g0, g1) of one row (or of two rows in lock-step when TWO) through `acc`.
// Thread t takes groups g0 + t, g0 + t + kBlock, ...; a round is U groups per thread, issued as
// U unconditional 128-bit loads. Two register sets alternate (ping-pong, no copies), so the
// loads of the next round are in flight while the current round is reduced. The rounds in which
// some threads have fewer than U groups go through a one-group tail loop.
// acc.consume<N>(a, b, g) receives N groups unpacked to floats (a from the first row, b from the
// second or unused) starting at group g, with stride kBlock.
template <typename T, bool VEC, int U, bool TWO>
struct RoundBuf {
  typename Rows<T, VEC>::Raw a[U], b[TWO ? U : 1];
  __device__ __forceinline__ void load(const T* __restrict__ ra, const T* __restrict__ rb,
                                       int g) {
#pragma unroll
    for (int j = 0; j < U; ++j) {
      a[j] = Rows<T, VEC>::load(ra, g + j * kBlock);
      if (TWO) b[j] = Rows<T, VEC>::load(rb, g + j * kBlock);
    }
    // keep the loads where they are issued: the scheduler would otherwise sink them below the
    // reduction of the previous round and serialise memory and arithmetic
    __builtin_amdgcn_sched_barrier(0);
  }
  template <class Acc>
  __device__ __forceinline__ void consume(Acc& acc, int g) const {
    constexpr int E = Rows<T, VEC>::E;
    float fa[U][E], fb[TWO ? U : 1][E];
#pragma unroll
    for (int j = 0; j < U; ++j) {
      Rows<T, VEC>::unpack(a[j], fa[j]);
      if (TWO) Rows<T, VEC>::unpack(b[j], fb[j]);
    }
    acc.template consume<U>(fa, fb, g);
  }
};

template <typename T, bool VEC, int U, bool TWO, class Acc>
__device__ __forceinline__ void stream_groups(const T* __restrict__ ra, const T* __restrict__ rb,
                                              int g0, int g1, Acc& acc) {
  using R = Rows<T, VEC>;
  constexpr int E = R::E;
  constexpr int step = U * kBlock;
  const int full = (g1 - g0) / step;  // rounds in which every thread has U groups (uniform)
  int g = g0 + (int)threadIdx.x;
  if (full > 0) {
    RoundBuf<T, VEC, U, TWO> x, y;
    x.load(ra, rb, g);
    int it = 0;
    for (; it + 2 < full; it += 2) {  // at least three rounds left: y and the next x exist
      y.load(ra, rb, g + step);
      x.consume(acc, g);
      x.load(ra, rb, g + 2 * step);
      y.consume(acc, g + step);
      g += 2 * step;
    }
    if (full - it == 2) {
      y.load(ra, rb, g + step);
      x.consume(acc, g);
      y.consume(acc, g + step);
      g += 2 * step;
    } else {
      x.consume(acc, g);
      g += step;
    }
  }
  for (; g < g1; g += kBlock) {
    float fa[1][E], fb[1][E];
    R::unpack(R::load(ra, g), fa[0]);
    if (TWO) R::unpack(R::load(rb, g), fb[0]);
    acc.template consume<1>(fa, fb, g);
  }
}

// Exact power-of-two rescale of a partial sum from integer offset `from` to `to` (to >= from).
__device__ __forceinline__ float rescale(float s, float from, float to) {
  float d = from - to;  // <= 0, integer-valued (or hugely negative)
  d = d < -512.0f ? -512.0f : d;
  return ldexpf(s, (int)d);
}

// Merge two (offset, sum) partials.
__device__ __forceinline__ void merge_stats(float& o, float& s, float o2, float s2) {
  const float on = fmaxf(o, o2);
  s = rescale(s, o, on) + rescale(s2, o2, on);
  o = on;
}

// Online softmax statistics: o is an integer >= c * max(z) seen so far, s0 + s1 is the sum of
// 2^(fma(z, c, -o)). The offset moves once per round of N groups, not per element.
template <int E>
struct SoftmaxAcc {
  float c, o, s0, s1;
  template <int N, class A, class Bv>
  __device__ __forceinline__ void consume(const A& f, const Bv&, int) {
    float bm = -INFINITY;
#pragma unroll
    for (int j = 0; j < N; ++j)
#pragma unroll
      for (int e = 0; e < E; ++e) bm = fmaxf(bm, f[j][e]);
    const float on = fmaxf(o, ceilf(bm * c));
    s0 = rescale(s0, o, on);
    s1 = rescale(s1, o, on);
    o = on;
#pragma unroll
    for (int j = 0; j < N; ++j)
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float t = __builtin_amdgcn_exp2f(fmaf(f[j][e], c, -o));
        if ((j * E + e) & 1) s1 += t;
        else s0 += t;
      }
  }
};

// Running argmax over elements in ascending index order; the first maximum is kept.
template <int E>
struct ArgmaxAcc {
  float best;
  int idx;
  template <int N, class A, class Bv>
  __device__ __forceinline__ void consume(const A& f, const Bv&, int g) {
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const int base = (g + j * kBlock) * E;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        if (f[j][e] > best) {
          best = f[j][e];
          idx = base + e;
        }
      }
    }
  }
};

// ---------------------------------------------------------------------------------------------
// Pass 1: per-chunk softmax statistics of every used row.
//
// grid.x = B * (2K+1) * C, ordered (request, row slot, chunk). Row slot s <= K is target row s,
// slot K+1+d is draft row d. Unused rows (s > k_b, d >= k_b) exit at once without a read.
// Writes stats[(b*(2K+1) + s)*C + c] = (o, sum) with sum = sum_v 2^(fma(z_v, c32, -o)).
// Group 0 also clears the pass-2 arrival counters of every request.

template <typename T, bool VEC>
__global__ __launch_bounds__(kBlock) void sv_row_stats(
    const T* __restrict__ target, const T* __restrict__ draft, int B, int K, int V,
    const int32_t* __restrict__ num_draft, float c32, int C, float2* __restrict__ stats,
    uint32_t* __restrict__ counters) {
  constexpr int E = Rows<T, VEC>::E;
  const long wg = blockIdx.x;
  if (wg == 0) {
    for (int i = threadIdx.x; i < B; i += kBlock) counters[i] = 0u;
  }
  const int NR = 2 * K + 1;
  const int c = (int)(wg % C);
  const long rs = wg / C;
  const int slot = (int)(rs % NR);
  const int b = (int)(rs / NR);
  const int k = clamp_k(num_draft, b, K);
  const T* row;
  if (slot <= K) {
    if (slot > k) return;
    row = target + ((size_t)b * (K + 1) + slot) * (size_t)V;
  } else {
    const int d = slot - K - 1;
    if (d >= k) return;
    row = draft + ((size_t)b * K + d) * (size_t)V;
  }
  const int G = VEC ? V / E : V;
  const int g0 = (int)((long)G * c / C), g1 = (int)((long)G * (c + 1) / C);

  SoftmaxAcc<E> acc{c32, -FLT_MAX, 0.0f, 0.0f};
  stream_groups<T, VEC, kUnroll, false>(row, row, g0, g1, acc);
  float o = acc.o, s = acc.s0 + acc.s1;

  // wave reduce, then across the 4 waves through LDS
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const float o2 = __shfl_xor(o, m);
    const float s2 = __shfl_xor(s, m);
    merge_stats(o, s, o2, s2);
  }
  __shared__ float so[kWaves], ss[kWaves];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    so[wave] = o;
    ss[wave] = s;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kWaves; ++w) merge_stats(o, s, so[w], ss[w]);
    stats[((size_t)b * NR + slot) * C + c] = make_float2(o, s);
  }
}

// ---------------------------------------------------------------------------------------------
// Pass 2 helpers.

struct DrawRow {
  float oT, iT;  // offset and fp32 reciprocal normaliser of the target row
  float oD, iD;  // same for the draft row (residual draws only)
  float c32;
};

// Draw weight of one element: max(0, p - q) at a rejected slot (RESID), p otherwise. The same
// code runs in the chunk-sum loop and in the final scan, so both see identical fp32 values.
template <bool RESID>
__device__ __forceinline__ float draw_weight(float zt, float zd, const DrawRow& w) {
  const float pt = __builtin_amdgcn_exp2f(fmaf(zt, w.c32, -w.oT)) * w.iT;
  if (!RESID) return pt;
  const float pd = __builtin_amdgcn_exp2f(fmaf(zd, w.c32, -w.oD)) * w.iD;
  const float diff = pt - pd;
  return diff > 0.0f ? diff : 0.0f;
}

template <int E, bool RESID>
struct WeightSumAcc {
  DrawRow w;
  double acc;
  template <int N, class A, class Bv>
  __device__ __forceinline__ void consume(const A& ft, const Bv& fd, int) {
#pragma unroll
    for (int j = 0; j < N; ++j)
#pragma unroll
      for (int e = 0; e < E; ++e)
        acc += (double)draw_weight<RESID>(ft[j][e], RESID ? fd[j][e] : 0.0f, w);
  }
};

__device__ __forceinline__ double block_sum_f64(double v, double* red) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  double t = 0.0;
  for (int i = 0; i < kWaves; ++i) t += red[i];
  return t;  // every thread gets the same total (same order of additions)
}

// Inclusive block scan of one fp64 value per thread; returns the inclusive prefix and writes the
// block total to *total.
__device__ __forceinline__ double block_scan_f64(double v, double* red, double* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const double u = __shfl_up(v, d);
    if (lane >= d) v += u;
  }
  __syncthreads();
  if (lane == 63) red[wave] = v;
  __syncthreads();
  double before = 0.0, all = 0.0;
  for (int i = 0; i < kWaves; ++i) {
    if (i < wave) before += red[i];
    all += red[i];
  }
  *total = all;
  return before + v;
}

__device__ __forceinline__ int block_min_i32(int v, int* red) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = min(v, __shfl_xor(v, m));
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  int t = red[0];
  for (int i = 1; i < kWaves; ++i) t = min(t, red[i]);
  return t;
}

__device__ __forceinline__ int block_max_i32(int v, int* red) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = max(v, __shfl_xor(v, m));
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  int t = red[0];
  for (int i = 1; i < kWaves; ++i) t = max(t, red[i]);
  return t;
}

// Sum of the draw weights over groups [g0, g1) (fp64 accumulation per element), block-wide.
template <typename T, bool VEC, bool RESID>
__device__ double weight_sum(const T* rt, const T* rd, const DrawRow& w, int g0, int g1,
                             double* red) {
  WeightSumAcc<Rows<T, VEC>::E, RESID> acc{w, 0.0};
  stream_groups<T, VEC, 2, RESID>(rt, RESID ? rd : rt, g0, g1, acc);
  return block_sum_f64(acc.acc, red);
}

// Inverse CDF inside groups [g0, g1): the first element index v with
// (sum of weights from element g0*E up to and including v) > target, in ascending order with
// fp64 running sums. If no element qualifies (rounding), the last element with positive weight;
// -1 if the range has none.
template <typename T, bool VEC, bool RESID>
__device__ int scan_find(const T* rt, const T* rd, const DrawRow& w, int g0, int g1,
                         double target, double* red, int* ired) {
  using R = Rows<T, VEC>;
  constexpr int E = R::E;
  double base = 0.0;
  int last_pos = -1;
  for (int tile = g0; tile < g1; tile += kBlock) {
    const int g = tile + (int)threadIdx.x;
    float wv[E];
    double mine = 0.0;
    if (g < g1) {
      float ft[E], fd[E];
      R::unpack(R::load(rt, g), ft);
      if (RESID) R::unpack(R::load(rd, g), fd);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        wv[e] = draw_weight<RESID>(ft[e], RESID ? fd[e] : 0.0f, w);
        mine += (double)wv[e];
        if (wv[e] > 0.0f) last_pos = g * E + e;
      }
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) wv[e] = 0.0f;
    }
    double total;
    const double incl = block_scan_f64(mine, red, &total);
    int cand = INT_MAX;
    if (g < g1 && base + incl > target) {
      double run = base + (incl - mine);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        run += (double)wv[e];
        if (cand == INT_MAX && run > target) cand = g * E + e;
      }
    }
    const int found = block_min_i32(cand, ired);
    if (found != INT_MAX) return found;
    base += total;
  }
  return block_max_i32(last_pos, ired);
}

// ---------------------------------------------------------------------------------------------
// Pass 2: accept scan, draw-weight chunk sums, and (last group per request) the inverse CDF.
//
// grid.x = B * C2, ordered (request, chunk).

template <typename T, bool VEC>
__global__ __launch_bounds__(kBlock) void sv_resolve(
    const T* __restrict__ target, const T* __restrict__ draft, int B, int K, int V,
    const int32_t* __restrict__ num_draft, float c32, const int32_t* __restrict__ tokens,
    const float* __restrict__ uniforms, const float* __restrict__ residual, int C,
    const float2* __restrict__ stats, int C2, double* zpart, uint32_t* counters,
    int32_t* __restrict__ accepted_len, int32_t* __restrict__ committed,
    float* __restrict__ target_prob, float* __restrict__ draft_prob) {
  constexpr int E = Rows<T, VEC>::E;
  const int b = blockIdx.x / C2, c2 = blockIdx.x % C2;
  const int NR = 2 * K + 1;
  const int k = clamp_k(num_draft, b, K);

  __shared__ float s_o[2 * kMaxK + 1];
  __shared__ double s_S[2 * kMaxK + 1];
  __shared__ double red[kWaves];
  __shared__ int ired[kWaves];
  __shared__ int s_n, s_last, s_chunk, s_mode;
  __shared__ double s_target;

  // 1. Row normalisers of the request: combine the C pass-1 partials of each used row in fp64.
  for (int j = threadIdx.x; j < 2 * k + 1; j += kBlock) {
    const int slot = j <= k ? j : K + 1 + (j - k - 1);
    const float2* st = stats + ((size_t)b * NR + slot) * C;
    float O = -FLT_MAX;
    for (int c = 0; c < C; ++c) O = fmaxf(O, st[c].x);
    double S = 0.0;
    for (int c = 0; c < C; ++c) {
      float d = st[c].x - O;
      d = d < -2000.0f ? -2000.0f : d;
      S += ldexp((double)st[c].y, (int)d);
    }
    s_o[slot] = O;
    s_S[slot] = S;
  }
  __syncthreads();

  // 2. p(x), q(x), accept decisions and the first rejection (slots 0..k-1 live in wave 0).
  if (threadIdx.x < 64) {
    const int i = threadIdx.x;
    double a = 0.0, q = 0.0;
    bool rej = false;
    if (i < k) {
      const int x = tokens[(size_t)b * K + i];
      if (x >= 0 && x < V) {
        const T* trow = target + ((size_t)b * (K + 1) + i) * (size_t)V;
        const T* drow = draft + ((size_t)b * K + i) * (size_t)V;
        const double zt = (double)Rows<T, VEC>::at(trow, x);
        const double zd = (double)Rows<T, VEC>::at(drow, x);
        a = exp2(zt * (double)c32 - (double)s_o[i]) / s_S[i];
        q = exp2(zd * (double)c32 - (double)s_o[K + 1 + i]) / s_S[K + 1 + i];
      }
      const double t = q > 0.0 ? fmin(1.0, a / q) : (a > 0.0 ? 1.0 : 0.0);
      rej = !((double)uniforms[(size_t)b * K + i] < t);
    }
    const unsigned long long m = __ballot(rej);
    const int n = m ? (__ffsll((long long)m) - 1) : k;
    if (i == 0) s_n = n;
    if (c2 == 0 && i < K) {
      target_prob[(size_t)b * K + i] = (float)a;
      if (draft_prob != nullptr) draft_prob[(size_t)b * K + i] = (float)q;
    }
  }
  __syncthreads();
  const int n = s_n;
  if (c2 == 0) {
    for (int i = threadIdx.x; i <= K; i += kBlock) {
      if (i < n) committed[(size_t)b * (K + 1) + i] = tokens[(size_t)b * K + i];
      else if (i > n) committed[(size_t)b * (K + 1) + i] = -1;
    }
    if (threadIdx.x == 0) accepted_len[b] = n;
  }

  // 3. The draw row: target row n, minus draft row n when slot n was rejected.
  const bool resid = n < k;
  const T* rt = target + ((size_t)b * (K + 1) + n) * (size_t)V;
  const T* rd = resid ? draft + ((size_t)b * K + n) * (size_t)V : rt;
  DrawRow w;
  w.oT = s_o[n];
  w.iT = (float)(1.0 / s_S[n]);
  w.oD = resid ? s_o[K + 1 + n] : 0.0f;
  w.iD = resid ? (float)(1.0 / s_S[K + 1 + n]) : 0.0f;
  w.c32 = c32;
  const int G = VEC ? V / E : V;

  // 4. This group's chunk sum, published for the last group of the request.
  {
    const int g0 = (int)((long)G * c2 / C2), g1 = (int)((long)G * (c2 + 1) / C2);
    const double z = resid ? weight_sum<T, VEC, true>(rt, rd, w, g0, g1, red)
                           : weight_sum<T, VEC, false>(rt, rd, w, g0, g1, red);
    if (threadIdx.x == 0) {
      __hip_atomic_store(&zpart[(size_t)b * C2 + c2], z, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
      __threadfence();
      const uint32_t prev = atomicAdd(&counters[b], 1u);
      s_last = (prev == (uint32_t)(C2 - 1));
    }
    __syncthreads();
    if (!s_last) return;
  }
  __threadfence();

  // 5. Last group: pick the chunk holding r * Z from the fp64 chunk sums, then scan it.
  if (threadIdx.x == 0) {
    counters[b] = 0u;  // every group of this request has arrived; leave it clean
    const double r = (double)residual[b];
    double Z = 0.0;
    for (int c = 0; c < C2; ++c)
      Z += __hip_atomic_load(&zpart[(size_t)b * C2 + c], __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
    int chunk = -1, mode = 0;
    double tgt = 0.0;
    if (Z > 0.0) {
      const double rz = r * Z;
      double cum = 0.0;
      int last_pos = -1;
      for (int c = 0; c < C2; ++c) {
        const double zc = __hip_atomic_load(&zpart[(size_t)b * C2 + c], __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT);
        if (zc > 0.0) last_pos = c;
        if (chunk < 0 && cum + zc > rz) {
          chunk = c;
          tgt = rz - cum;
        }
        cum += zc;
      }
      if (chunk < 0) {  // rounding: fall back to the last chunk with mass, past its end
        chunk = last_pos;
        tgt = INFINITY;
      }
    } else {
      mode = 1;  // zero residual mass (rounding only): draw from p at slot n
    }
    s_chunk = chunk;
    s_target = tgt;
    s_mode = mode;
  }
  __syncthreads();
  int y;
  if (s_mode == 0) {
    const int chunk = s_chunk;
    const int g0 = (int)((long)G * chunk / C2), g1 = (int)((long)G * (chunk + 1) / C2);
    y = resid ? scan_find<T, VEC, true>(rt, rd, w, g0, g1, s_target, red, ired)
              : scan_find<T, VEC, false>(rt, rd, w, g0, g1, s_target, red, ired);
  } else {
    const double Zp = weight_sum<T, VEC, false>(rt, rd, w, 0, G, red);
    y = scan_find<T, VEC, false>(rt, rd, w, 0, G, (double)residual[b] * Zp, red, ired);
  }
  if (threadIdx.x == 0) committed[(size_t)b * (K + 1) + n] = y < 0 ? 0 : y;
}

// ---------------------------------------------------------------------------------------------
// Greedy: per-chunk argmax (lowest index among equal maxima), then per-request combine.

__device__ __forceinline__ void merge_argmax(float& v, int& i, float v2, int i2) {
  if (v2 > v || (v2 == v && i2 < i)) {
    v = v2;
    i = i2;
  }
}

template <typename T, bool VEC>
__global__ __launch_bounds__(kBlock) void sv_greedy_stats(const T* __restrict__ target, int B,
                                                          int K, int V,
                                                          const int32_t* __restrict__ num_draft,
                                                          int C, float2* __restrict__ gstats) {
  constexpr int E = Rows<T, VEC>::E;
  const long wg = blockIdx.x;
  const int NR = K + 1;
  const int c = (int)(wg % C);
  const long rs = wg / C;
  const int slot = (int)(rs % NR);
  const int b = (int)(rs / NR);
  const int k = clamp_k(num_draft, b, K);
  if (slot > k) return;
  const T* row = target + ((size_t)b * (K + 1) + slot) * (size_t)V;
  const int G = VEC ? V / E : V;
  const int g0 = (int)((long)G * c / C), g1 = (int)((long)G * (c + 1) / C);

  // Each thread visits its elements in ascending index order and keeps the first maximum.
  ArgmaxAcc<E> acc{-INFINITY, INT_MAX};
  stream_groups<T, VEC, kUnroll, false>(row, row, g0, g1, acc);
  float best = acc.best;
  int bi = acc.idx;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const float v2 = __shfl_xor(best, m);
    const int i2 = __shfl_xor(bi, m);
    merge_argmax(best, bi, v2, i2);
  }
  __shared__ float sv[kWaves];
  __shared__ int si[kWaves];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    sv[wave] = best;
    si[wave] = bi;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kWaves; ++w) merge_argmax(best, bi, sv[w], si[w]);
    gstats[((size_t)b * NR + slot) * C + c] = make_float2(best, __int_as_float(bi));
  }
}

// grid.x = B; 128 threads (row slots 0..K <= 64 fit, draft slots 0..K-1 live in wave 0).
__global__ __launch_bounds__(128) void sv_greedy_finish(int B, int K,
                                                        const int32_t* __restrict__ num_draft,
                                                        const int32_t* __restrict__ tokens, int C,
                                                        const float2* __restrict__ gstats,
                                                        int32_t* __restrict__ accepted_len,
                                                        int32_t* __restrict__ committed) {
  const int b = blockIdx.x;
  const int NR = K + 1;
  const int k = clamp_k(num_draft, b, K);
  __shared__ int s_g[kMaxK + 1];
  __shared__ int s_n;
  for (int i = threadIdx.x; i <= k; i += blockDim.x) {
    const float2* st = gstats + ((size_t)b * NR + i) * C;
    float v = -INFINITY;
    int idx = INT_MAX;
    for (int c = 0; c < C; ++c) merge_argmax(v, idx, st[c].x, __float_as_int(st[c].y));
    s_g[i] = idx == INT_MAX ? 0 : idx;  // a row of -inf only: index 0
  }
  __syncthreads();
  if (threadIdx.x < 64) {
    const int i = threadIdx.x;
    const bool miss = i < k && tokens[(size_t)b * K + i] != s_g[i];
    const unsigned long long m = __ballot(miss);
    if (i == 0) s_n = m ? (__ffsll((long long)m) - 1) : k;
  }
  __syncthreads();
  const int n = s_n;
  for (int i = threadIdx.x; i <= K; i += blockDim.x) {
    int v;
    if (i < n) v = tokens[(size_t)b * K + i];
    else if (i == n) v = s_g[n];
    else v = -1;
    committed[(size_t)b * (K + 1) + i] = v;
  }
  if (threadIdx.x == 0) accepted_len[b] = n;
}

// ---------------------------------------------------------------------------------------------
// Host side: validation and launches.

thread_local std::string g_last_error;

int fail(int status, const std::string& msg) {
  g_last_error = msg;
  return status;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int check_shape(int B, int K, int V) {
  if (B < 1 || B > kMaxB) return fail(SV_ERR_INVALID_ARG, "B must be in [1, 1048576]");
  if (K < 1 || K > kMaxK) return fail(SV_ERR_INVALID_ARG, "K must be in [1, 64]");
  if (V < 1 || V > kMaxV) return fail(SV_ERR_INVALID_ARG, "V must be in [1, 67108864]");
  return SV_OK;
}

int check_workspace(void* ws, size_t have, size_t need) {
  if (ws == nullptr) return fail(SV_ERR_WORKSPACE, "workspace is NULL");
  if (!aligned(ws, 8)) return fail(SV_ERR_WORKSPACE, "workspace must be 8-byte aligned");
  if (have < need)
    return fail(SV_ERR_WORKSPACE, "workspace too small: need " + std::to_string(need) +
                                      " bytes, got " + std::to_string(have));
  return SV_OK;
}

int launch_status(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(SV_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
  return SV_OK;
}

template <typename T, bool VEC>
int launch_sample(const void* target, const void* draft, int B, int K, int V, float c32,
                  const int32_t* tokens, const int32_t* num_draft, const float* uniforms,
                  const float* residual, int32_t* accepted_len, int32_t* committed,
                  float* target_prob, float* draft_prob, char* ws, const Plan& p,
                  const Layout& L, hipStream_t stream) {
  float2* stats = reinterpret_cast<float2*>(ws + L.stats);
  double* zpart = reinterpret_cast<double*>(ws + L.zpart);
  uint32_t* counters = reinterpret_cast<uint32_t*>(ws + L.counters);
  const long g1 = (long)B * (2 * K + 1) * p.C;
  hipLaunchKernelGGL((sv_row_stats<T, VEC>), dim3((unsigned)g1), dim3(kBlock), 0, stream,
                     static_cast<const T*>(target), static_cast<const T*>(draft), B, K, V,
                     num_draft, c32, p.C, stats, counters);
  int st = launch_status("sv_row_stats");
  if (st != SV_OK) return st;
  const long g2 = (long)B * p.C2;
  hipLaunchKernelGGL((sv_resolve<T, VEC>), dim3((unsigned)g2), dim3(kBlock), 0, stream,
                     static_cast<const T*>(target), static_cast<const T*>(draft), B, K, V,
                     num_draft, c32, tokens, uniforms, residual, p.C, stats, p.C2, zpart,
                     counters, accepted_len, committed, target_prob, draft_prob);
  return launch_status("sv_resolve");
}

template <typename T, bool VEC>
int launch_greedy(const void* target, int B, int K, int V, const int32_t* tokens,
                  const int32_t* num_draft, int32_t* accepted_len, int32_t* committed, char* ws,
                  const Plan& p, const Layout& L, hipStream_t stream) {
  float2* gstats = reinterpret_cast<float2*>(ws + L.gstats);
  const long g1 = (long)B * (K + 1) * p.Cg;
  hipLaunchKernelGGL((sv_greedy_stats<T, VEC>), dim3((unsigned)g1), dim3(kBlock), 0, stream,
                     static_cast<const T*>(target), B, K, V, num_draft, p.Cg, gstats);
  int st = launch_status("sv_greedy_stats");
  if (st != SV_OK) return st;
  hipLaunchKernelGGL(sv_greedy_finish, dim3((unsigned)B), dim3(128), 0, stream, B, K, num_draft,
                     tokens, p.Cg, gstats, accepted_len, committed);
  return launch_status("sv_greedy_finish");
}

// A launch's total work-items must stay below 2^32 in grid.x.
int check_grid(long groups) {
  if (groups * (long)kBlock >= (1L << 32))
    return fail(SV_ERR_UNSUPPORTED, "batch too large for one launch: " +
                                        std::to_string(groups) + " work-groups");
  return SV_OK;
}

size_t elem_size(int dtype) { return dtype == SV_DTYPE_F32 ? 4 : 2; }

bool rows_vectorisable(const void* a, const void* b, int dtype, int V) {
  return aligned(a, 16) && (b == nullptr || aligned(b, 16)) &&
         ((size_t)V * elem_size(dtype)) % 16 == 0;
}

}  // namespace

extern "C" {

size_t sv_workspace_bytes(int B, int K, int V) {
  if (B < 1 || B > kMaxB || K < 1 || K > kMaxK || V < 1 || V > kMaxV) return 0;
  const Plan p = make_plan(B, K, V);
  return make_layout(B, K, V, p).total;
}

const char* sv_status_string(int status) {
  switch (status) {
    case SV_OK: return "ok";
    case SV_ERR_INVALID_ARG: return "invalid argument";
    case SV_ERR_UNSUPPORTED: return "unsupported";
    case SV_ERR_WORKSPACE: return "workspace missing or too small";
    case SV_ERR_HIP: return "HIP launch failure";
    default: return "unknown status";
  }
}

const char* sv_last_error(void) { return g_last_error.c_str(); }

int sv_verify_batch(const void* target_logits, const void* draft_logits, int dtype, int B, int K,
                    int V, float temperature, const int32_t* draft_tokens,
                    const int32_t* num_draft, const float* uniforms,
                    const float* residual_uniform, int32_t* accepted_len, int32_t* committed,
                    float* target_prob, float* draft_prob, void* workspace,
                    size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  int st = check_shape(B, K, V);
  if (st != SV_OK) return st;
  if (dtype != SV_DTYPE_F32 && dtype != SV_DTYPE_BF16)
    return fail(SV_ERR_INVALID_ARG, "dtype must be SV_DTYPE_F32 or SV_DTYPE_BF16");
  if (!target_logits || !draft_logits || !draft_tokens || !uniforms || !residual_uniform ||
      !accepted_len || !committed || !target_prob)
    return fail(SV_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!(temperature > 0.0f) || !isfinite(temperature))
    return fail(SV_ERR_INVALID_ARG, "temperature must be finite and > 0");
  const double c64 = 1.4426950408889634074 / (double)temperature;  // log2(e) / temperature
  if (!(c64 >= (double)FLT_MIN && c64 <= 2097152.0))
    return fail(SV_ERR_INVALID_ARG, "temperature out of range");
  const float c32 = (float)c64;
  const Plan p = make_plan(B, K, V);
  const Layout L = make_layout(B, K, V, p);
  st = check_workspace(workspace, workspace_bytes, L.total);
  if (st != SV_OK) return st;
  st = check_grid((long)B * (2 * K + 1) * p.C);
  if (st != SV_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  const bool vec = rows_vectorisable(target_logits, draft_logits, dtype, V);
  if (dtype == SV_DTYPE_F32) {
    return vec ? launch_sample<float, true>(target_logits, draft_logits, B, K, V, c32,
                                            draft_tokens, num_draft, uniforms, residual_uniform,
                                            accepted_len, committed, target_prob, draft_prob, ws,
                                            p, L, s)
               : launch_sample<float, false>(target_logits, draft_logits, B, K, V, c32,
                                             draft_tokens, num_draft, uniforms, residual_uniform,
                                             accepted_len, committed, target_prob, draft_prob,
                                             ws, p, L, s);
  }
  return vec ? launch_sample<uint16_t, true>(target_logits, draft_logits, B, K, V, c32,
                                             draft_tokens, num_draft, uniforms, residual_uniform,
                                             accepted_len, committed, target_prob, draft_prob,
                                             ws, p, L, s)
             : launch_sample<uint16_t, false>(target_logits, draft_logits, B, K, V, c32,
                                              draft_tokens, num_draft, uniforms,
                                              residual_uniform, accepted_len, committed,
                                              target_prob, draft_prob, ws, p, L, s);
}

int sv_verify_greedy(const void* target_logits, int dtype, int B, int K, int V,
                     const int32_t* draft_tokens, const int32_t* num_draft,
                     int32_t* accepted_len, int32_t* committed, void* workspace,
                     size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  int st = check_shape(B, K, V);
  if (st != SV_OK) return st;
  if (dtype != SV_DTYPE_F32 && dtype != SV_DTYPE_BF16)
    return fail(SV_ERR_INVALID_ARG, "dtype must be SV_DTYPE_F32 or SV_DTYPE_BF16");
  if (!target_logits || !draft_tokens || !accepted_len || !committed)
    return fail(SV_ERR_INVALID_ARG, "a required pointer is NULL");
  const Plan p = make_plan(B, K, V);
  const Layout L = make_layout(B, K, V, p);
  st = check_workspace(workspace, workspace_bytes, L.total);
  if (st != SV_OK) return st;
  st = check_grid((long)B * (K + 1) * p.Cg);
  if (st != SV_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  const bool vec = rows_vectorisable(target_logits, nullptr, dtype, V);
  if (dtype == SV_DTYPE_F32) {
    return vec ? launch_greedy<float, true>(target_logits, B, K, V, draft_tokens, num_draft,
                                            accepted_len, committed, ws, p, L, s)
               : launch_greedy<float, false>(target_logits, B, K, V, draft_tokens, num_draft,
                                             accepted_len, committed, ws, p, L, s);
  }
  return vec ? launch_greedy<uint16_t, true>(target_logits, B, K, V, draft_tokens, num_draft,
                                             accepted_len, committed, ws, p, L, s)
             : launch_greedy<uint16_t, false>(target_logits, B, K, V, draft_tokens, num_draft,
                                              accepted_len, committed, ws, p, L, s);
}

}  // extern "C"
