// Batched lossless draft verification: HIP kernels for gfx950 (MI355X) and the C-ABI in sv.h.
//
// The acceptance rule ("From draft-then-verify to DSpark", section "How speculative decoding
// works") needs, per request, the full-vocabulary normalisers of 2k+1 softmax rows (k+1 target,
// k draft), the probabilities p(x), q(x) of the k proposals, the first rejected slot n, and one
// inverse-CDF draw from max(0, p - q) at that slot (or from p at the slot after the last draft).
// Only the normalisers and the final draw touch whole vocabulary rows, so the work is built
// around streaming each used row once from HBM with 128-bit loads.
//
// Sampling mode is one launch of sv_verify_sample with two kinds of work-groups:
//   row-stat groups  (request, row, vocabulary chunk), first in the grid. Each thread keeps an
//                    online (offset, sum) pair: the sum of 2^(c*z - o) over its elements, with
//                    c = log2(e) / temperature and o an integer upper bound of c * max(z). As o
//                    is an integer, moving a partial sum to a new offset is an exact power-of-two
//                    scaling (ldexp), so every combine adds no rounding beyond the additions.
//                    The group whose chunk holds a draft token also records that token's logit.
//   draw groups      (request, vocabulary chunk), after all row-stat groups. Each waits until
//                    every row-stat group of its request has published, combines the partials in
//                    fp64, forms p(x), q(x), the accept decisions and n (identical in every group
//                    of the request), and sums the draw weights w of its chunk per 512-element
//                    tile in fp64. The last draw group of the request to finish scans the tile
//                    sums to the tile holding r * Z and finds the token with a one-wave fp64 scan.
//
// Greedy mode is one launch of sv_verify_greedy: per-chunk argmax groups (lowest index on ties);
// the last group of each request to finish combines them and runs the match scan.
//
// Cross-work-group data inside a launch is published with agent-scope atomic stores (sc1,
// coherent across the XCDs' L2 caches) and read with agent-scope atomic loads; a publisher
// waits for its stores to complete (s_waitcnt vmcnt(0)) before bumping the request's counter.
// No device-wide cache writeback or invalidate is issued. A draw group only waits on
// row-stat groups, which precede it in the grid and so are all dispatched before it; the wait is
// bounded regardless. Counters live at the front of the workspace and every call leaves them at
// zero.
//
// No MFMA: nothing here is a dense contraction. All floating-point contraction is explicit
// (the file is compiled with -ffp-contract=off) so that the same weight is computed bit for bit
// in the tile-sum pass and in the final scan.

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
constexpr int kMaxB = 1 << 16;
constexpr int kMaxV = 1 << 26;
constexpr int kUnroll = 4;      // 128-bit loads in flight per thread in the streaming loops
constexpr int kTile = 512;      // elements per draw tile: 64 lanes x 8 elements
constexpr int kTileUnroll = 4;  // draw tiles in flight per wave
// Each request's two arrival counters sit in their own 256-byte block: counters of different
// requests packed together put every arrival of the launch on one memory channel, where the
// device-scope atomics serialise.
constexpr int kCtrStride = 64;  // uint32 slots between two requests' counters
constexpr int kPollSleep = 2;   // s_sleep units (64 clocks each) between two polls
constexpr int kStageMax = 2048;  // row-stat partials of one request staged in LDS: (2K+1)*C
constexpr int kPickRegs = 4;     // tile sums per thread held in registers by the pick
constexpr int kSpinLimit = 1 << 21;  // polls (about 1 us each) before a draw group gives up
constexpr int32_t kTimedOut = -2;    // accepted_len value reported by a group that gave up

// ---------------------------------------------------------------------------------------------
// Work decomposition (host side, shared by the workspace query and the launches).

struct Plan {
  int C;   // vocabulary chunks per row, row-stat groups
  int C2;  // vocabulary chunks per request, draw groups
  int NT;  // draw tiles per request: ceil(V / 512)
  int Cg;  // vocabulary chunks per row, greedy
};

int chunks_for(long rows, long units, long target_groups, long min_units, int max_chunks) {
  long c = (target_groups + rows - 1) / rows;
  long cap = units / min_units;
  if (c > cap) c = cap;
  if (c > max_chunks) c = max_chunks;
  if (c < 1) c = 1;
  return (int)c;
}

Plan make_plan(int B, int K, int V) {
  Plan p;
  p.C = chunks_for((long)B * (2 * K + 1), V, 8192, 4096, kStageMax / (2 * K + 1));
  p.NT = (V + kTile - 1) / kTile;
  p.C2 = chunks_for(B, p.NT, 2048, 4, 1024);  // at least 4 tiles (one per wave) per group
  p.Cg = chunks_for((long)B * (K + 1), V, 8192, 4096, 256);
  return p;
}

// Per-request values of the draw: which row, and its normalisers.
struct DrawParams {
  int n;      // accepted drafts
  int resid;  // 1: draw from max(0, p_n - q_n); 0: draw from p_n
  float oT, iT, oD, iD;  // offsets and fp32 reciprocal normalisers of target / draft row n
};

struct Layout {
  size_t counters;  // uint32 [kMaxB][64]    per-request arrival counters (zero between calls)
  size_t stats;     // uint64 [B][2K+1][C]   row-stat partials: float2 (offset, sum) bits
  size_t gath;      // uint32 [B][2K]        logit at the draft token: target slot i, draft K+i
  size_t tsum;      // double [B][NT]        draw weight sum per tile
  size_t gstats;    // uint64 [B][K+1][Cg]   greedy partials: float value, int index
  size_t total;
};

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

Layout make_layout(int B, int K, int V, const Plan& p) {
  Layout L;
  size_t off = 0;
  L.counters = off;
  off = align_up(off + sizeof(uint32_t) * kCtrStride * (size_t)kMaxB, 256);
  const size_t data = off;
  L.stats = off;
  off = align_up(off + sizeof(uint64_t) * (size_t)B * (2 * K + 1) * p.C, 256);
  L.gath = off;
  off = align_up(off + sizeof(uint32_t) * (size_t)B * 2 * K, 256);
  L.tsum = off;
  off = align_up(off + sizeof(double) * (size_t)B * p.NT, 256);
  L.gstats = data;  // greedy calls reuse the data area
  const size_t g = align_up(data + sizeof(uint64_t) * (size_t)B * (K + 1) * p.Cg, 256);
  L.total = off > g ? off : g;
  return L;
}

// ---------------------------------------------------------------------------------------------
// Coherent accesses for data that crosses work-groups within one launch.

template <typename U>
__device__ __forceinline__ void st_coh(U* p, U v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename U>
__device__ __forceinline__ U ld_coh(const U* p) {
  return __hip_atomic_load(const_cast<U*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until this wave's stores have completed (s_waitcnt vmcnt(0); lgkm/exp counts untouched).
__device__ __forceinline__ void wait_own_stores() { __builtin_amdgcn_s_waitcnt(0x0F70); }

__device__ __forceinline__ uint64_t pack2(float a, float b) {
  return (uint64_t)__float_as_uint(a) | ((uint64_t)__float_as_uint(b) << 32);
}
__device__ __forceinline__ float lo_f(uint64_t v) { return __uint_as_float((uint32_t)v); }
__device__ __forceinline__ float hi_f(uint64_t v) { return __uint_as_float((uint32_t)(v >> 32)); }

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
// Sampling mode.

struct SampleArgs {
  const void* target;  // [B][K+1][V]
  const void* draft;   // [B][K][V]
  int B, K, V;
  const int32_t* num_draft;
  const int32_t* tokens;
  const float* uniforms;
  const float* residual;
  float c32;  // log2(e) / temperature, rounded to fp32
  int C, C2, NT;
  long n_stat_groups;  // B * (2K+1) * C: groups before this index are row-stat groups
  uint32_t* counters;  // [kMaxB][kCtrStride]: [b][0] row-stat arrivals, [b][1] draw arrivals
  uint64_t* stats;
  uint32_t* gath;
  double* tsum;
  int32_t* accepted_len;
  int32_t* committed;
  float* target_prob;
  float* draft_prob;
};

// Row-stat group wg = (b * (2K+1) + slot) * C + c. Row slot s <= K is target row s, slot K+1+d
// is draft row d. Unused rows (s > k_b, d >= k_b) return at once without a read or an arrival.
// Publishes stats[(b*(2K+1) + s)*C + c] = (o, sum) with sum = sum_v 2^(fma(z_v, c32, -o)), and,
// for target slots i < k_b and draft slots d < k_b, the group whose chunk holds the draft token
// publishes its logit in gath[b][i] (target) or gath[b][K+d] (draft).
template <typename T, bool VEC>
__device__ void row_stat_group(const SampleArgs& a, long wg) {
  constexpr int E = Rows<T, VEC>::E;
  const int K = a.K, V = a.V, C = a.C;
  const int NR = 2 * K + 1;
  const int c = (int)(wg % C);
  const long rs = wg / C;
  const int slot = (int)(rs % NR);
  const int b = (int)(rs / NR);
  const int k = clamp_k(a.num_draft, b, K);
  const T* row;
  int tslot;  // draft slot whose logit this row provides, or -1 (the extra-draw row)
  int gidx;   // where that logit goes in gath
  if (slot <= K) {
    if (slot > k) return;
    row = static_cast<const T*>(a.target) + ((size_t)b * (K + 1) + slot) * (size_t)V;
    tslot = slot < k ? slot : -1;
    gidx = slot;
  } else {
    const int d = slot - K - 1;
    if (d >= k) return;
    row = static_cast<const T*>(a.draft) + ((size_t)b * K + d) * (size_t)V;
    tslot = d;
    gidx = K + d;
  }
  const int G = VEC ? V / E : V;
  const int g0 = (int)((long)G * c / C), g1 = (int)((long)G * (c + 1) / C);

  if (threadIdx.x == 0 && tslot >= 0) {
    const int x = a.tokens[(size_t)b * K + tslot];
    if (x >= 0 && x < V && x >= g0 * E && x < g1 * E)
      st_coh(&a.gath[(size_t)b * 2 * K + gidx], __float_as_uint(Rows<T, VEC>::at(row, x)));
  }

  SoftmaxAcc<E> acc{a.c32, -FLT_MAX, 0.0f, 0.0f};
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
    st_coh(&a.stats[((size_t)b * NR + slot) * C + c], pack2(o, s));
    wait_own_stores();  // the stats (and gath) stores of this thread are complete
    __hip_atomic_fetch_add(&a.counters[(size_t)kCtrStride * b], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// ---------------------------------------------------------------------------------------------
// Draw weights.
//
// A draw tile is 512 consecutive vocabulary entries handled by one wave, 8 per lane: with E
// elements per group, lane l holds groups t*64*TG + 64*j + l for j < TG = 8/E, so sub-tile j
// covers 64*E consecutive elements in lane order.

template <bool RESID>
__device__ __forceinline__ float draw_weight(float zt, float zd, const DrawParams& w, float c32) {
  const float pt = __builtin_amdgcn_exp2f(fmaf(zt, c32, -w.oT)) * w.iT;
  if (!RESID) return pt;
  const float pd = __builtin_amdgcn_exp2f(fmaf(zd, c32, -w.oD)) * w.iD;
  const float diff = pt - pd;
  return diff > 0.0f ? diff : 0.0f;
}

template <typename T, bool VEC, bool RESID>
struct TileRows {
  using R = Rows<T, VEC>;
  static constexpr int E = R::E;
  static constexpr int TG = 8 / E;
  typename R::Raw a[TG], b[RESID ? TG : 1];
  bool ok[TG];
  // Issues the loads of tile t for this lane. Groups past G load the last group instead (always
  // in bounds, no branch around the loads) and are masked to weight 0.
  __device__ __forceinline__ void load(const T* rt, const T* rd, int t, int G, int lane) {
#pragma unroll
    for (int j = 0; j < TG; ++j) {
      const int g = t * 64 * TG + 64 * j + lane;
      ok[j] = g < G;
      const int gc = ok[j] ? g : G - 1;
      a[j] = R::load(rt, gc);
      if (RESID) b[j] = R::load(rd, gc);
    }
  }
  // Weights of sub-tile j for this lane (0 for masked groups).
  __device__ __forceinline__ void weights(int j, const DrawParams& w, float c32,
                                          float (&out)[E]) const {
    float ft[E], fd[E];
    if (ok[j]) {
      R::unpack(a[j], ft);
      if (RESID) R::unpack(b[j], fd);
#pragma unroll
      for (int e = 0; e < E; ++e)
        out[e] = draw_weight<RESID>(ft[e], RESID ? fd[e] : 0.0f, w, c32);
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) out[e] = 0.0f;
    }
  }
  // fp64 sum of this lane's 8 weights, in element order.
  __device__ __forceinline__ double lane_sum(const DrawParams& w, float c32) const {
    double s = 0.0;
#pragma unroll
    for (int j = 0; j < TG; ++j) {
      float v[E];
      weights(j, w, c32, v);
#pragma unroll
      for (int e = 0; e < E; ++e) s += (double)v[e];
    }
    return s;
  }
};

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}

__device__ __forceinline__ double wave_incl_scan_f64(double v, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const double u = __shfl_up(v, d);
    if (lane >= d) v += u;
  }
  return v;
}

__device__ __forceinline__ int wave_min_i32(int v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = min(v, __shfl_xor(v, m));
  return v;
}

__device__ __forceinline__ int wave_max_i32(int v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = max(v, __shfl_xor(v, m));
  return v;
}

__device__ __forceinline__ double block_sum_f64(double v, double* red) {
  v = wave_sum_f64(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  double t = 0.0;
  for (int i = 0; i < kWaves; ++i) t += red[i];
  return t;  // every thread gets the same total (same order of additions)
}

// Inclusive block scan of one fp64 value per thread; *total receives the block total.
__device__ __forceinline__ double block_scan_f64(double v, double* red, double* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_incl_scan_f64(v, lane);
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
  v = wave_min_i32(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  int t = red[0];
  for (int i = 1; i < kWaves; ++i) t = min(t, red[i]);
  return t;
}

// Per-tile weight sums of tiles [t0, t1) by the 4 waves of the group, kTileUnroll tiles per wave
// in flight. Tile sums are published to tsum[t] (one store per tile by lane 0 of its wave).
template <typename T, bool VEC, bool RESID>
__device__ __forceinline__ void tile_sums(const T* rt, const T* rd, const DrawParams& w,
                                          float c32, int G, int t0, int t1, double* tsum) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  for (int t = t0 + wave; t < t1; t += kWaves * kTileUnroll) {
    TileRows<T, VEC, RESID> tr[kTileUnroll];
#pragma unroll
    for (int u = 0; u < kTileUnroll; ++u) {
      const int tu = t + u * kWaves;
      if (tu < t1) tr[u].load(rt, rd, tu, G, lane);
    }
#pragma unroll
    for (int u = 0; u < kTileUnroll; ++u) {
      const int tu = t + u * kWaves;
      if (tu < t1) {
        const double s = wave_sum_f64(tr[u].lane_sum(w, c32));
        if (lane == 0) st_coh(&tsum[tu], s);
      }
    }
  }
}

// One wave: inverse CDF inside tile t. Returns the first element v of the tile whose running sum
// (from the start of the tile, element order) exceeds `target`; if none does (rounding), the last
// element of the tile with positive weight; -1 if the tile has none.
template <typename T, bool VEC, bool RESID>
__device__ int tile_find(const T* rt, const T* rd, const DrawParams& w, float c32, int G, int t,
                         double target) {
  using TR = TileRows<T, VEC, RESID>;
  constexpr int E = TR::E;
  const int lane = threadIdx.x & 63;
  TR tr;
  tr.load(rt, rd, t, G, lane);
  double base = 0.0;
  int last_pos = -1;
#pragma unroll
  for (int j = 0; j < TR::TG; ++j) {
    float v[E];
    tr.weights(j, w, c32, v);
    const int first = (t * 64 * TR::TG + 64 * j + lane) * E;
    double mine = 0.0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      mine += (double)v[e];
      if (v[e] > 0.0f) last_pos = first + e;
    }
    const double incl = wave_incl_scan_f64(mine, lane);
    int cand = INT_MAX;
    if (base + incl > target) {
      double run = base + (incl - mine);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        run += (double)v[e];
        if (cand == INT_MAX && run > target) cand = first + e;
      }
    }
    const int found = wave_min_i32(cand);
    if (found != INT_MAX) return found;
    base += __shfl(incl, 63);
  }
  return wave_max_i32(last_pos);
}

// Finds the tile holding r * Z from the published tile sums (fp64). Returns the tile and the
// target relative to the tile start; tile = -1 when Z == 0. Up to kBlock * kPickRegs tiles,
// thread t holds the P consecutive tile sums starting at t * P in registers (one pass, one
// round of coherent loads); longer rows go through a loop over blocks of kBlock tiles.
__device__ void pick_tile(const double* ts, int NT, double r, double* red, int* ired,
                          int* tile_out, double* rel_out) {
  __shared__ double s_rel;
  if (NT <= kBlock * kPickRegs) {
    const int P = (NT + kBlock - 1) / kBlock;
    const int t0 = (int)threadIdx.x * P;
    double v[kPickRegs];
#pragma unroll
    for (int i = 0; i < kPickRegs; ++i) {
      const int t = t0 + i;
      const double x = ld_coh(&ts[t < NT ? t : NT - 1]);  // clamped, no branch around the load
      v[i] = (i < P && t < NT) ? x : 0.0;
    }
    double mine = 0.0;
#pragma unroll
    for (int i = 0; i < kPickRegs; ++i) mine += v[i];
    double Z;
    const double incl = block_scan_f64(mine, red, &Z);
    if (!(Z > 0.0)) {
      *tile_out = -1;
      *rel_out = 0.0;
      return;
    }
    const double target = r * Z;
    double run = incl - mine;
    int cand = INT_MAX, last_pos = -1;
    double rel = 0.0;
#pragma unroll
    for (int i = 0; i < kPickRegs; ++i) {
      if (v[i] > 0.0) last_pos = t0 + i;
      if (cand == INT_MAX && v[i] > 0.0 && run + v[i] > target) {
        cand = t0 + i;
        rel = target - run;
      }
      run += v[i];
    }
    const int found = block_min_i32(cand, ired);
    if (found != INT_MAX) {
      if (cand == found) s_rel = rel;
      __syncthreads();
      *tile_out = found;
      *rel_out = s_rel;
      return;
    }
    *tile_out = -block_min_i32(-last_pos, ired);  // rounding only: past the last tile with mass
    *rel_out = INFINITY;
    return;
  }
  double z = 0.0;
  for (int t = threadIdx.x; t < NT; t += kBlock) z += ld_coh(&ts[t]);
  const double Z = block_sum_f64(z, red);
  if (!(Z > 0.0)) {
    *tile_out = -1;
    *rel_out = 0.0;
    return;
  }
  const double target = r * Z;
  double base = 0.0;
  int last_pos = -1;
  for (int t0 = 0; t0 < NT; t0 += kBlock) {
    const int t = t0 + threadIdx.x;
    const double v = t < NT ? ld_coh(&ts[t]) : 0.0;
    if (v > 0.0) last_pos = t;
    double total;
    const double incl = block_scan_f64(v, red, &total);
    const int cand = (t < NT && base + incl > target) ? t : INT_MAX;
    const int found = block_min_i32(cand, ired);
    if (found != INT_MAX) {
      if (t == found) s_rel = target - (base + (incl - v));
      __syncthreads();
      *tile_out = found;
      *rel_out = s_rel;
      return;
    }
    base += total;
  }
  *tile_out = -block_min_i32(-last_pos, ired);  // rounding only: past the last tile with mass
  *rel_out = INFINITY;
}

// Draw group j = b * C2 + c2; chunk c2 covers tiles [NT*c2/C2, NT*(c2+1)/C2).
template <typename T, bool VEC>
__device__ void draw_group(const SampleArgs& a, long j) {
  constexpr int E = Rows<T, VEC>::E;
  const int K = a.K, V = a.V, C = a.C, C2 = a.C2, NT = a.NT;
  const int b = (int)(j / C2), c2 = (int)(j % C2);
  const int NR = 2 * K + 1;
  const int k = clamp_k(a.num_draft, b, K);
  const float c32 = a.c32;

  __shared__ uint64_t s_stage[kStageMax];
  __shared__ float s_o[2 * kMaxK + 1];
  __shared__ double s_S[2 * kMaxK + 1];
  __shared__ float s_zt[64], s_zd[64];
  __shared__ double red[kWaves];
  __shared__ int ired[kWaves];
  __shared__ int s_n, s_flag, s_y;

  // 0. Wait until every used row of the request has published its statistics.
  if (threadIdx.x == 0) {
    const uint32_t need = (uint32_t)((2 * k + 1) * C);
    int spins = 0;
    while (ld_coh(&a.counters[(size_t)kCtrStride * b]) < need && spins < kSpinLimit) {
      __builtin_amdgcn_s_sleep(kPollSleep);
      ++spins;
    }
    s_flag = spins < kSpinLimit;
  }
  __syncthreads();
  if (!s_flag) {
    if (threadIdx.x == 0) a.accepted_len[b] = kTimedOut;
    return;
  }

  // 1. Row normalisers of the request: stage the C partials of every used row in LDS (one
  //    coherent load per entry, all issued back to back), then combine each row in fp64.
  const int nrow = 2 * k + 1, nent = nrow * C;  // nent <= kStageMax by the plan
  for (int e0 = 0; e0 < nent; e0 += kBlock * 4) {
    uint64_t v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      int e = e0 + u * kBlock + (int)threadIdx.x;
      e = e < nent ? e : nent - 1;  // clamped: always a valid entry, no branch around the load
      const int r = e / C, c = e % C;
      const int slot = r <= k ? r : K + 1 + (r - k - 1);
      v[u] = ld_coh(&a.stats[((size_t)b * NR + slot) * C + c]);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = e0 + u * kBlock + (int)threadIdx.x;
      if (e < nent) s_stage[e] = v[u];
    }
  }
  if (threadIdx.x < 64) {  // the draft-token logits: target slot i in lane i, draft in s_zd
    const int i = threadIdx.x;
    const int ii = i < k ? i : 0;
    const uint32_t zt = ld_coh(&a.gath[(size_t)b * 2 * K + ii]);
    const uint32_t zd = ld_coh(&a.gath[(size_t)b * 2 * K + K + ii]);
    s_zt[i] = __uint_as_float(zt);
    s_zd[i] = __uint_as_float(zd);
  }
  __syncthreads();
  for (int r = threadIdx.x; r < nrow; r += kBlock) {
    const int slot = r <= k ? r : K + 1 + (r - k - 1);
    const uint64_t* st = s_stage + r * C;
    float O = -FLT_MAX;
    for (int c = 0; c < C; ++c) O = fmaxf(O, lo_f(st[c]));
    double S = 0.0;
    for (int c = 0; c < C; ++c) {
      float d = lo_f(st[c]) - O;
      d = d < -2000.0f ? -2000.0f : d;
      S += ldexp((double)hi_f(st[c]), (int)d);
    }
    s_o[slot] = O;
    s_S[slot] = S;
  }
  __syncthreads();

  // 2. p(x), q(x), accept decisions and the first rejection (slots 0..k-1 live in wave 0).
  if (threadIdx.x < 64) {
    const int i = threadIdx.x;
    double p = 0.0, q = 0.0;
    bool rej = false;
    if (i < k) {
      const int x = a.tokens[(size_t)b * K + i];
      if (x >= 0 && x < V) {
        const double zt = (double)s_zt[i];
        const double zd = (double)s_zd[i];
        p = exp2(zt * (double)c32 - (double)s_o[i]) / s_S[i];
        q = exp2(zd * (double)c32 - (double)s_o[K + 1 + i]) / s_S[K + 1 + i];
      }
      const double t = q > 0.0 ? fmin(1.0, p / q) : (p > 0.0 ? 1.0 : 0.0);
      rej = !((double)a.uniforms[(size_t)b * K + i] < t);
    }
    const unsigned long long m = __ballot(rej);
    const int n = m ? (__ffsll((long long)m) - 1) : k;
    if (i == 0) s_n = n;
    if (c2 == 0 && i < K) {
      a.target_prob[(size_t)b * K + i] = (float)p;
      if (a.draft_prob != nullptr) a.draft_prob[(size_t)b * K + i] = (float)q;
    }
  }
  __syncthreads();
  const int n = s_n;

  // 3. The draw row: target row n, minus draft row n when slot n was rejected.
  const bool resid = n < k;
  DrawParams w;
  w.n = n;
  w.resid = resid ? 1 : 0;
  w.oT = s_o[n];
  w.iT = (float)(1.0 / s_S[n]);
  w.oD = resid ? s_o[K + 1 + n] : 0.0f;
  w.iD = resid ? (float)(1.0 / s_S[K + 1 + n]) : 0.0f;
  if (c2 == 0) {
    for (int i = threadIdx.x; i <= K; i += kBlock) {
      if (i < n) a.committed[(size_t)b * (K + 1) + i] = a.tokens[(size_t)b * K + i];
      else if (i > n) a.committed[(size_t)b * (K + 1) + i] = -1;
    }
    if (threadIdx.x == 0) a.accepted_len[b] = n;
  }
  const T* rt = static_cast<const T*>(a.target) + ((size_t)b * (K + 1) + n) * (size_t)V;
  const T* rd = resid ? static_cast<const T*>(a.draft) + ((size_t)b * K + n) * (size_t)V : rt;
  const int G = VEC ? V / E : V;
  double* ts = a.tsum + (size_t)b * NT;

  // 4. Tile sums of this chunk, then arrival; the last group of the request goes on to draw.
  const int t0 = (int)((long)NT * c2 / C2), t1 = (int)((long)NT * (c2 + 1) / C2);
  if (resid) tile_sums<T, VEC, true>(rt, rd, w, c32, G, t0, t1, ts);
  else tile_sums<T, VEC, false>(rt, rd, w, c32, G, t0, t1, ts);
  wait_own_stores();
  __syncthreads();  // every wave's tile-sum stores are complete
  if (threadIdx.x == 0) {
    const uint32_t prev =
        __hip_atomic_fetch_add(&a.counters[(size_t)kCtrStride * b + 1], 1u, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    s_flag = prev == (uint32_t)(C2 - 1);
  }
  __syncthreads();
  if (!s_flag) return;

  // 5. Last group: the tile holding r * Z, then the token inside it.
  const double r = (double)a.residual[b];
  bool rs = resid;
  int tile;
  double rel;
  pick_tile(ts, NT, r, red, ired, &tile, &rel);
  if (tile < 0) {
    // Zero residual mass (rounding only): draw from p at slot n instead. Recompute the tile
    // sums of p over the whole row in place, then pick again.
    rs = false;
    tile_sums<T, VEC, false>(rt, rd, w, c32, G, 0, NT, ts);
    wait_own_stores();
    __syncthreads();
    pick_tile(ts, NT, r, red, ired, &tile, &rel);
  }
  if (threadIdx.x < 64) {
    int y = -1;
    if (tile >= 0)
      y = rs ? tile_find<T, VEC, true>(rt, rd, w, c32, G, tile, rel)
             : tile_find<T, VEC, false>(rt, rd, w, c32, G, tile, rel);
    if (threadIdx.x == 0) s_y = y;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    a.committed[(size_t)b * (K + 1) + n] = s_y < 0 ? 0 : s_y;
    // every row-stat and draw group of this request has arrived: leave the counters at zero
    st_coh(&a.counters[(size_t)kCtrStride * b], 0u);
    st_coh(&a.counters[(size_t)kCtrStride * b + 1], 0u);
  }
}

// Grid order: every row-stat group, then every draw group. Draw groups therefore wait only on
// groups dispatched before them. (Interleaving each request's draw groups a few requests behind
// its row-stat groups measured slower: draw groups spend most of their life waiting on memory
// latency, and inside the stream they take work-group slots from it.)
template <typename T, bool VEC>
__global__ __launch_bounds__(kBlock) void sv_verify_sample(SampleArgs a) {
  const long wg = blockIdx.x;
  if (wg < a.n_stat_groups) row_stat_group<T, VEC>(a, wg);
  else draw_group<T, VEC>(a, wg - a.n_stat_groups);
}

// ---------------------------------------------------------------------------------------------
// Greedy mode: per-chunk argmax (lowest index among equal maxima); the last group of a request
// to arrive combines the chunks and runs the match scan.

__device__ __forceinline__ void merge_argmax(float& v, int& i, float v2, int i2) {
  if (v2 > v || (v2 == v && i2 < i)) {
    v = v2;
    i = i2;
  }
}

struct GreedyArgs {
  const void* target;  // [B][K+1][V]
  int B, K, V;
  const int32_t* num_draft;
  const int32_t* tokens;
  int C;
  uint32_t* counters;
  uint64_t* gstats;
  int32_t* accepted_len;
  int32_t* committed;
};

template <typename T, bool VEC>
__global__ __launch_bounds__(kBlock) void sv_verify_greedy_kernel(GreedyArgs a) {
  constexpr int E = Rows<T, VEC>::E;
  const long wg = blockIdx.x;
  const int K = a.K, V = a.V, C = a.C;
  const int NR = K + 1;
  const int c = (int)(wg % C);
  const long rs = wg / C;
  const int slot = (int)(rs % NR);
  const int b = (int)(rs / NR);
  const int k = clamp_k(a.num_draft, b, K);
  if (slot > k) return;
  const T* row = static_cast<const T*>(a.target) + ((size_t)b * (K + 1) + slot) * (size_t)V;
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
  __shared__ int s_last;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    sv[wave] = best;
    si[wave] = bi;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kWaves; ++w) merge_argmax(best, bi, sv[w], si[w]);
    st_coh(&a.gstats[((size_t)b * NR + slot) * C + c],
           (uint64_t)__float_as_uint(best) | ((uint64_t)(uint32_t)bi << 32));
    wait_own_stores();
    const uint32_t prev = __hip_atomic_fetch_add(&a.counters[(size_t)kCtrStride * b], 1u, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    s_last = prev == (uint32_t)((k + 1) * C - 1);
  }
  __syncthreads();
  if (!s_last) return;

  // Last group of the request: row argmaxes, match scan, outputs.
  __shared__ int s_g[kMaxK + 1];
  __shared__ int s_n;
  for (int i = threadIdx.x; i <= k; i += kBlock) {
    const uint64_t* st = a.gstats + ((size_t)b * NR + i) * C;
    float v = -INFINITY;
    int idx = INT_MAX;
    for (int cc = 0; cc < C; ++cc) {
      const uint64_t u = ld_coh(&st[cc]);
      merge_argmax(v, idx, lo_f(u), (int)(uint32_t)(u >> 32));
    }
    s_g[i] = idx == INT_MAX ? 0 : idx;  // a row of -inf only: index 0
  }
  __syncthreads();
  if (threadIdx.x < 64) {
    const int i = threadIdx.x;
    const bool miss = i < k && a.tokens[(size_t)b * K + i] != s_g[i];
    const unsigned long long m = __ballot(miss);
    if (i == 0) s_n = m ? (__ffsll((long long)m) - 1) : k;
  }
  __syncthreads();
  const int n = s_n;
  for (int i = threadIdx.x; i <= K; i += kBlock) {
    int v;
    if (i < n) v = a.tokens[(size_t)b * K + i];
    else if (i == n) v = s_g[n];
    else v = -1;
    a.committed[(size_t)b * (K + 1) + i] = v;
  }
  if (threadIdx.x == 0) {
    a.accepted_len[b] = n;
    st_coh(&a.counters[(size_t)kCtrStride * b], 0u);
  }
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
  if (B < 1 || B > kMaxB) return fail(SV_ERR_INVALID_ARG, "B must be in [1, 65536]");
  if (K < 1 || K > kMaxK) return fail(SV_ERR_INVALID_ARG, "K must be in [1, 64]");
  if (V < 1 || V > kMaxV) return fail(SV_ERR_INVALID_ARG, "V must be in [1, 67108864]");
  return SV_OK;
}

int check_workspace(void* ws, size_t have, size_t need) {
  if (ws == nullptr) return fail(SV_ERR_WORKSPACE, "workspace is NULL");
  if (!aligned(ws, 256)) return fail(SV_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (have < need)
    return fail(SV_ERR_WORKSPACE, "workspace too small: need " + std::to_string(need) +
                                      " bytes, got " + std::to_string(have));
  return SV_OK;
}

// A launch's total work-items must stay below 2^32 in grid.x.
int check_grid(long groups) {
  if (groups * (long)kBlock >= (1L << 32))
    return fail(SV_ERR_UNSUPPORTED, "batch too large for one launch: " +
                                        std::to_string(groups) + " work-groups");
  return SV_OK;
}

int launch_status(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(SV_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
  return SV_OK;
}

size_t elem_size(int dtype) { return dtype == SV_DTYPE_F32 ? 4 : 2; }

bool rows_vectorisable(const void* a, const void* b, int dtype, int V) {
  return aligned(a, 16) && (b == nullptr || aligned(b, 16)) &&
         ((size_t)V * elem_size(dtype)) % 16 == 0;
}

template <typename T, bool VEC>
int launch_sample(const SampleArgs& a, long groups, hipStream_t stream) {
  hipLaunchKernelGGL((sv_verify_sample<T, VEC>), dim3((unsigned)groups), dim3(kBlock), 0, stream,
                     a);
  return launch_status("sv_verify_sample");
}

template <typename T, bool VEC>
int launch_greedy(const GreedyArgs& a, long groups, hipStream_t stream) {
  hipLaunchKernelGGL((sv_verify_greedy_kernel<T, VEC>), dim3((unsigned)groups), dim3(kBlock), 0,
                     stream, a);
  return launch_status("sv_verify_greedy");
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
  const Plan p = make_plan(B, K, V);
  const Layout L = make_layout(B, K, V, p);
  st = check_workspace(workspace, workspace_bytes, L.total);
  if (st != SV_OK) return st;
  const long n_stat = (long)B * (2 * K + 1) * p.C;
  const long groups = n_stat + (long)B * p.C2;
  st = check_grid(groups);
  if (st != SV_OK) return st;
  char* ws = static_cast<char*>(workspace);
  SampleArgs a;
  a.target = target_logits;
  a.draft = draft_logits;
  a.B = B;
  a.K = K;
  a.V = V;
  a.num_draft = num_draft;
  a.tokens = draft_tokens;
  a.uniforms = uniforms;
  a.residual = residual_uniform;
  a.c32 = (float)c64;
  a.C = p.C;
  a.C2 = p.C2;
  a.NT = p.NT;
  a.n_stat_groups = n_stat;
  a.counters = reinterpret_cast<uint32_t*>(ws + L.counters);
  a.stats = reinterpret_cast<uint64_t*>(ws + L.stats);
  a.gath = reinterpret_cast<uint32_t*>(ws + L.gath);
  a.tsum = reinterpret_cast<double*>(ws + L.tsum);
  a.accepted_len = accepted_len;
  a.committed = committed;
  a.target_prob = target_prob;
  a.draft_prob = draft_prob;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool vec = rows_vectorisable(target_logits, draft_logits, dtype, V);
  if (dtype == SV_DTYPE_F32)
    return vec ? launch_sample<float, true>(a, groups, s) : launch_sample<float, false>(a, groups, s);
  return vec ? launch_sample<uint16_t, true>(a, groups, s)
             : launch_sample<uint16_t, false>(a, groups, s);
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
  const long groups = (long)B * (K + 1) * p.Cg;
  st = check_grid(groups);
  if (st != SV_OK) return st;
  char* ws = static_cast<char*>(workspace);
  GreedyArgs a;
  a.target = target_logits;
  a.B = B;
  a.K = K;
  a.V = V;
  a.num_draft = num_draft;
  a.tokens = draft_tokens;
  a.C = p.Cg;
  a.counters = reinterpret_cast<uint32_t*>(ws + L.counters);
  a.gstats = reinterpret_cast<uint64_t*>(ws + L.gstats);
  a.accepted_len = accepted_len;
  a.committed = committed;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool vec = rows_vectorisable(target_logits, nullptr, dtype, V);
  if (dtype == SV_DTYPE_F32)
    return vec ? launch_greedy<float, true>(a, groups, s) : launch_greedy<float, false>(a, groups, s);
  return vec ? launch_greedy<uint16_t, true>(a, groups, s)
             : launch_greedy<uint16_t, false>(a, groups, s);
}

}  // extern "C"
