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
//                    The group whose chunk holds a draft token also publishes that token's logit.
//   draw groups      (request, vocabulary chunk), after all row-stat groups. Each waits for the
//                    partials of its request, combines them in fp64, forms p(x), q(x), the accept
//                    decisions and n (identical in every group of the request), sums the draw
//                    weights w of its chunk per 512-element tile (fp64), and publishes its chunk
//                    total. Once it has every chunk total of its request, the one group whose
//                    chunk holds r * Z picks the tile and finds the token with a one-wave scan.
//
// Greedy mode is one launch of sv_verify_greedy: per-chunk argmax groups (lowest index on ties),
// then one finishing group per request that combines them and runs the match scan.
//
// Hand-off between work-groups inside a launch (no atomics, no device-wide cache maintenance):
// every published value is a 64-bit word whose high half is the call's tag, a number the host
// draws fresh for every call (never 0), and whose low half is the payload. Words are written
// with agent-scope atomic stores (coherent across the XCDs' L2 caches) and read with agent-scope
// atomic loads, so a reader knows a word is from this call exactly when its tag matches. A
// waiting group only waits on groups that precede it in the grid, which are dispatched before
// it; the wait is bounded regardless.
//
// No MFMA: nothing here is a dense contraction. All floating-point contraction is explicit
// (the file is compiled with -ffp-contract=off) so that the same weight is computed bit for bit
// in the tile-sum pass and in the final scan.

#include <hip/hip_runtime.h>

#include <float.h>
#include <math.h>
#include <stdint.h>

#include <atomic>
#include <climits>
#include <cstdio>
#include <mutex>
#include <string>

#include "sv.h"
#include "sv_internal.h"

namespace {

constexpr int kBlock = 256;  // threads per work-group: 4 wave64s
constexpr int kWaves = kBlock / 64;
constexpr int kMaxK = 64;
constexpr int kMaxB = 1 << 20;
constexpr int kMaxV = 1 << 26;
constexpr int kUnroll = 4;        // 128-bit loads in flight per thread in the streaming loops
constexpr int kTile = 512;        // elements per draw tile: 64 lanes x 8 elements
constexpr int kTileUnroll = 4;    // draw tiles in flight per wave
constexpr int kStageMax = 2048;   // partials of one request staged in LDS: (2K+1)*C, (K+1)*Cg
constexpr int kChunkTiles = 512;  // draw tiles per draw group, at most
constexpr int kMaxC2 = 512;       // draw groups per request, at most
constexpr int kDrawGroups = 1024;  // draw groups per launch the plan aims at
constexpr int kSegGroups = 64 * kUnroll;  // groups per segment of a bonus row: one wave's round
constexpr int kSegMax = 1024;     // segments per bonus row, at most (else the tile draw is used)
constexpr int kLaneRowChunks = 32;  // up to this many chunks per row, one lane combines a row
constexpr int kSpinLimit = 1 << 21;  // polls (about 1 us each) before a waiting group gives up
constexpr int32_t kTimedOut = -2;    // accepted_len value reported by a group that gave up
constexpr int kPollSleep = 2;        // s_sleep units (64 clocks each) between two polls
constexpr int kMaxDevices = 64;      // devices the host-side caches keep an entry for
constexpr int kBf16Chunks = 6;       // chunks per 16-byte bf16 row, at most
constexpr int kF32Chunks = 12;       // chunks per 16-byte float32 row, at most (larger batches)

// ---------------------------------------------------------------------------------------------
// Work decomposition (host side, shared by the workspace query and the launches).

struct Plan {
  int C;   // vocabulary chunks per row, row-stat groups
  int NT;  // draw tiles per request: ceil(V / 512)
  int C2;  // vocabulary chunks per request, draw groups
  int Cg;  // vocabulary chunks per row, greedy
  int NSmax;  // segment slots per request in the workspace: min(ceil(V / 64), kSegMax)
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
  // about 6144 row-stat groups: fewer, longer groups stream with less per-group overhead (each
  // ends with a block reduction and a publish), more, shorter ones shorten the drain of the
  // stream, and a chunk close to a whole number of rounds leaves a short tail loop
  p.C = chunks_for((long)B * (2 * K + 1), V, 6144, 4096, kStageMax / (2 * K + 1));
  p.NT = (V + kTile - 1) / kTile;
  // About kDrawGroups draw groups in all, so that every one of them is resident once the
  // row-stat groups drain (more queue behind each other and delay the last requests' draws);
  // at least 8 tiles (two per wave) per group: with one tile per wave, small batches (B <= 16)
  // measured 0.8-1.6 us slower per call (more chunk totals to exchange, more groups deciding).
  p.C2 = chunks_for(B, p.NT, kDrawGroups, 8, kMaxC2);
  // At most kWaves * kTileUnroll tiles per group, so that each wave loads its tiles in one
  // round, unless that would more than double the draw groups.
  const long one_round = (p.NT + kWaves * kTileUnroll - 1) / (kWaves * kTileUnroll);
  if (p.C2 < one_round && (long)B * one_round <= 2L * kDrawGroups) p.C2 = (int)one_round;
  const int need = (p.NT + kChunkTiles - 1) / kChunkTiles;
  if (p.C2 < need) p.C2 = need;
  p.Cg = chunks_for((long)B * (K + 1), V, 8192, 4096, kStageMax / (K + 1));
  const long ns = ((long)V + kSegGroups - 1) / kSegGroups;
  p.NSmax = (int)(ns < kSegMax ? ns : kSegMax);
  return p;
}

bool plan_supported(const Plan& p) { return p.C2 <= kMaxC2; }  // V <= kMaxC2 * kChunkTiles * 512

// Per-request values of the draw: which row, and its normalisers.
struct DrawParams {
  int n;      // accepted drafts
  int resid;  // 1: draw from max(0, p_n - q_n); 0: draw from p_n
  float oT, iT, oD, iD;  // offsets and fp32 reciprocal normalisers of target / draft row n
};

struct Layout {
  size_t stats;   // uint64 [B][2K+1][C][2]  row-stat partials: tagged offset, tagged sum
  size_t gath;    // uint64 [B][K][2]        tagged logits at draft token i: target row, draft row
  size_t ctot;    // uint64 [B][C2][2]       tagged draw chunk totals (fp64 high, low halves)
  size_t seg;     // uint64 [B][NSmax][2]    tagged segment partials of each request's bonus row
  size_t gstats;  // uint64 [B][K+1][Cg][2]  greedy partials: tagged value, tagged index
  size_t total;
};

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

Layout make_layout(int B, int K, int V, const Plan& p) {
  Layout L;
  size_t off = 0;
  L.stats = off;
  off = align_up(off + 16 * (size_t)B * (2 * K + 1) * (p.C + 1), 256);  // a launch may add a chunk
  L.gath = off;
  off = align_up(off + 8 * (size_t)B * 2 * K, 256);
  L.ctot = off;
  off = align_up(off + 16 * (size_t)B * p.C2, 256);
  L.seg = off;
  off = align_up(off + 16 * (size_t)B * p.NSmax, 256);
  L.gstats = 0;  // greedy calls reuse the front of the workspace
  const size_t g = align_up(16 * (size_t)B * (K + 1) * p.Cg, 256);
  L.total = off > g ? off : g;
  return L;
}

// ---------------------------------------------------------------------------------------------
// Tagged words for the hand-off between work-groups within one launch.

__device__ __forceinline__ void publish(uint64_t* p, uint32_t tag, uint32_t payload) {
  __hip_atomic_store(p, ((uint64_t)tag << 32) | payload, __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t fetch(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool tagged(uint64_t w, uint32_t tag) { return (uint32_t)(w >> 32) == tag; }

__device__ __forceinline__ uint32_t payload(uint64_t w) { return (uint32_t)w; }

// ---------------------------------------------------------------------------------------------
// Wave primitives on DPP: cross-lane moves done inside the vector ALU, without the LDS round trip
// of a lane permute. A scan combines each lane with the lanes 1, 2, 4 and 8 below it inside its
// row of 16 lanes, then adds lane 15 of each row into the next row and lane 31 into rows 2 and 3,
// so lane l ends up holding the combination of lanes 0..l (lane 63: the whole wave). A source
// lane outside the row, or a row that the mask leaves out, reads the identity. Every scan runs
// with the whole wave active.

constexpr int kDppRowShr1 = 0x111, kDppRowShr2 = 0x112, kDppRowShr4 = 0x114, kDppRowShr8 = 0x118;
constexpr int kDppWaveShr1 = 0x138, kDppRowBcast15 = 0x142, kDppRowBcast31 = 0x143;

template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x, uint32_t identity) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)identity, (int)x, CTRL, ROWS, 0xf, false);
}
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_f32(float x, float identity) {
  return __uint_as_float(dpp_u32<CTRL, ROWS>(__float_as_uint(x), __float_as_uint(identity)));
}
template <int CTRL, int ROWS>
__device__ __forceinline__ double dpp_f64(double x) {  // identity 0.0
  const uint64_t v = (uint64_t)__double_as_longlong(x);
  const uint32_t lo = dpp_u32<CTRL, ROWS>((uint32_t)v, 0u);
  const uint32_t hi = dpp_u32<CTRL, ROWS>((uint32_t)(v >> 32), 0u);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Value of lane l (l wave-uniform), as a wave-uniform value.
__device__ __forceinline__ uint32_t lane_u32(uint32_t x, int l) {
  return (uint32_t)__builtin_amdgcn_readlane((int)x, l);
}
__device__ __forceinline__ float lane_f32(float x, int l) {
  return __uint_as_float(lane_u32(__float_as_uint(x), l));
}
__device__ __forceinline__ double lane_f64(double x, int l) {
  const uint64_t v = (uint64_t)__double_as_longlong(x);
  const uint32_t lo = lane_u32((uint32_t)v, l), hi = lane_u32((uint32_t)(v >> 32), l);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Applies one scan step to the state of every lane: f(state, state of the source lane).
#define SV_SCAN_STEPS(STEP)   \
  STEP(kDppRowShr1, 0xf);     \
  STEP(kDppRowShr2, 0xf);     \
  STEP(kDppRowShr4, 0xf);     \
  STEP(kDppRowShr8, 0xf);     \
  STEP(kDppRowBcast15, 0xa);  \
  STEP(kDppRowBcast31, 0xc)

// Inclusive prefix sum of one fp64 value per lane.
__device__ __forceinline__ double wave_scan_f64(double x) {
#define SV_ADD_STEP(CTRL, ROWS) x += dpp_f64<CTRL, ROWS>(x)
  SV_SCAN_STEPS(SV_ADD_STEP);
#undef SV_ADD_STEP
  return x;
}

// Sum over the wave, wave-uniform.
__device__ __forceinline__ double wave_sum_f64(double x) { return lane_f64(wave_scan_f64(x), 63); }

// Maximum over the wave, wave-uniform.
__device__ __forceinline__ int wave_max_i32(int x) {
#define SV_MAX_STEP(CTRL, ROWS) x = max(x, (int)dpp_u32<CTRL, ROWS>((uint32_t)x, (uint32_t)INT_MIN))
  SV_SCAN_STEPS(SV_MAX_STEP);
#undef SV_MAX_STEP
  return (int)lane_u32((uint32_t)x, 63);
}

// Sum over the wave in fp32, wave-uniform: a tree of depth 6 (relative error <= 6 ulp).
__device__ __forceinline__ float wave_sum_f32(float x) {
#define SV_FADD_STEP(CTRL, ROWS) x += dpp_f32<CTRL, ROWS>(x, 0.0f)
  SV_SCAN_STEPS(SV_FADD_STEP);
#undef SV_FADD_STEP
  return lane_f32(x, 63);
}

// Maximum over the wave, wave-uniform (NaN-free inputs give the largest; -inf the identity).
__device__ __forceinline__ float wave_max_f32(float x) {
#define SV_FMAX_STEP(CTRL, ROWS) x = fmaxf(x, dpp_f32<CTRL, ROWS>(x, -INFINITY))
  SV_SCAN_STEPS(SV_FMAX_STEP);
#undef SV_FMAX_STEP
  return lane_f32(x, 63);
}

// Awaits up to four tagged word pairs (p[u], p[u] + 1), those with live[u]: loads them all, then
// re-reads only the words that do not carry the tag yet, all in flight together, until every
// word carries it or the thread's poll budget is spent. Between two polls the wave sleeps
// kPollSleep units, which keeps waiting groups from flooding the memory system with requests
// while other groups stream. Returns false when the budget ran out.
__device__ __forceinline__ bool await4(const uint64_t* const (&p)[4], const bool (&live)[4],
                                       uint32_t tag, uint64_t (&w0)[4], uint64_t (&w1)[4]) {
  const uint64_t done = (uint64_t)tag << 32;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    w0[u] = live[u] ? fetch(p[u]) : done;
    w1[u] = live[u] ? fetch(p[u] + 1) : done;
  }
  for (int left = kSpinLimit; left > 0; --left) {
    bool all = true;
#pragma unroll
    for (int u = 0; u < 4; ++u) all = all && tagged(w0[u], tag) && tagged(w1[u], tag);
    if (all) return true;
    if (kPollSleep > 0) __builtin_amdgcn_s_sleep(kPollSleep);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (!tagged(w0[u], tag)) w0[u] = fetch(p[u]);
      if (!tagged(w1[u], tag)) w1[u] = fetch(p[u] + 1);
    }
  }
  return false;
}

// ---------------------------------------------------------------------------------------------
// Row access: groups of E consecutive elements, one 128-bit load per group when the rows are
// 16-byte aligned (VEC), one element per group otherwise. Raw loads are kept separate from the
// unpacking so that the streaming loops can hold the next groups in flight while the current
// ones are reduced. Streamed rows are read with non-temporal loads: each byte is used once, and
// the streaming hint measured 6-12% faster than cached loads for these row streams.

typedef unsigned int v4u32 __attribute__((ext_vector_type(4)));
typedef float v4f32 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

template <typename T, bool VEC>
struct Rows;

template <>
struct Rows<float, true> {
  static constexpr int E = 4;
  using Raw = float4;
  __device__ static Raw load(const float* row, int g) {
    const v4f32 v = __builtin_nontemporal_load(reinterpret_cast<const v4f32*>(row) + g);
    return make_float4(v.x, v.y, v.z, v.w);
  }
  __device__ static Raw load_cached(const float* row, int g) {
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
    const v4u32 v = __builtin_nontemporal_load(reinterpret_cast<const v4u32*>(row) + g);
    return make_uint4(v.x, v.y, v.z, v.w);
  }
  __device__ static Raw load_cached(const uint16_t* row, int g) {
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
  __device__ static Raw load(const float* row, int g) { return __builtin_nontemporal_load(row + g); }
  __device__ static Raw load_cached(const float* row, int g) { return row[g]; }
  __device__ static void unpack(const Raw& v, float* f) { f[0] = v; }
  __device__ static float at(const float* row, int i) { return row[i]; }
};

template <>
struct Rows<uint16_t, false> {
  static constexpr int E = 1;
  using Raw = uint16_t;
  __device__ static Raw load(const uint16_t* row, int g) {
    return __builtin_nontemporal_load(row + g);
  }
  __device__ static Raw load_cached(const uint16_t* row, int g) { return row[g]; }
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

// (offset, sum) partials of the whole wave merged, wave-uniform.
__device__ __forceinline__ void wave_merge_stats(float& o, float& s) {
#define SV_STATS_STEP(CTRL, ROWS) \
  merge_stats(o, s, dpp_f32<CTRL, ROWS>(o, -FLT_MAX), dpp_f32<CTRL, ROWS>(s, 0.0f))
  SV_SCAN_STEPS(SV_STATS_STEP);
#undef SV_STATS_STEP
  o = lane_f32(o, 63);
  s = lane_f32(s, 63);
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

// Running argmax over elements in ascending index order; the first maximum is kept. A round's
// maximum m is taken first; only when it beats the running best is the round searched for the
// first element equal to m (the same answer as a strict-greater scan: the elements before it are
// smaller; NaN never compares greater or equal, as in the scan).
template <int E>
struct ArgmaxAcc {
  float best;
  int idx;
  template <int N, class A, class Bv>
  __device__ __forceinline__ void consume(const A& f, const Bv&, int g) {
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < N; ++j)
#pragma unroll
      for (int e = 0; e < E; ++e) m = fmaxf(m, f[j][e]);
    if (m > best) {
      int found = INT_MAX;
#pragma unroll
      for (int j = N - 1; j >= 0; --j)
#pragma unroll
        for (int e = E - 1; e >= 0; --e)
          if (f[j][e] == m) found = (g + j * kBlock) * E + e;
      best = m;
      idx = found;
    }
  }
};

__device__ __forceinline__ void merge_argmax(float& v, int& i, float v2, int i2) {
  if (v2 > v || (v2 == v && i2 < i)) {
    v = v2;
    i = i2;
  }
}

// (value, index) of the whole wave merged, wave-uniform.
__device__ __forceinline__ void wave_merge_argmax(float& v, int& i) {
#define SV_ARGMAX_STEP(CTRL, ROWS)                          \
  merge_argmax(v, i, dpp_f32<CTRL, ROWS>(v, -INFINITY), \
               (int)dpp_u32<CTRL, ROWS>((uint32_t)i, (uint32_t)INT_MAX))
  SV_SCAN_STEPS(SV_ARGMAX_STEP);
#undef SV_ARGMAX_STEP
  v = lane_f32(v, 63);
  i = (int)lane_u32((uint32_t)i, 63);
}

// Argmax partial of groups [g0, g1) of one row by the whole group: (value bits, index) of the
// first maximum, published as two tagged words at st. Each thread visits its elements in
// ascending index order and keeps the first maximum; the merges prefer the lower index.
template <typename T, bool VEC>
__device__ void argmax_chunk(const T* row, int g0, int g1, uint64_t* st, uint32_t tag) {
  constexpr int E = Rows<T, VEC>::E;
  ArgmaxAcc<E> acc{-INFINITY, INT_MAX};
  // eight-element groups (bf16) hold twice the values per load: half the loads per round keep
  // the unpacked round within the register budget of the other paths
  stream_groups<T, VEC, (E == 8 ? kUnroll / 2 : kUnroll), false>(row, row, g0, g1, acc);
  float best = acc.best;
  int bi = acc.idx;
  wave_merge_argmax(best, bi);
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
    publish(st, tag, __float_as_uint(best));
    publish(st + 1, tag, (uint32_t)bi);
  }
}


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
  int L;               // draw groups of request b follow the rows of request b + L (grid order)
  int CS;              // chunk stride in groups (whole rounds), or 0: an even split
  uint32_t tag;        // this call's tag
  uint64_t* stats;
  uint64_t* gath;  // [B][K][2]
  uint64_t* ctot;
  uint64_t* seg;  // [B][NSmax][2]
  int NS;         // segments of a bonus row, or 0: bonus tokens are drawn like residual ones
  int NSmax;
  int32_t* accepted_len;
  int32_t* committed;
  float* target_prob;
  float* draft_prob;
  // Flattened, mixed calls only:
  const int32_t* t_start;  // [B] first row of request b in the flat target array
  const int32_t* d_start;  // [B] first row of request b in the flat draft array
  long n_trows, n_drows;   // rows of the flat arrays
  const float* temps;      // [B] temperature of request b; 0 makes it a greedy request
};

constexpr double kLog2e = 1.4426950408889634074;
constexpr double kTauMin = kLog2e / 2097152.0;  // smallest sampling temperature: c <= 2^21
constexpr int32_t kBadRequest = -3;             // accepted_len of an invalid request

// What every group of request b needs: k_b, its first target and draft rows, the logit scale
// c = log2(e) / temperature (fp32), and, in flattened mixed calls (GEN), whether it is a greedy
// request or an invalid one (rows outside the flat arrays, k_b outside [0, K], temperature
// negative, not finite or below kTauMin): an invalid request reads nothing.
template <typename T>
struct Req {
  int k;
  bool greedy, bad;
  float c;
  const T* t0;
  const T* d0;
};

template <typename T, bool GEN>
__device__ __forceinline__ Req<T> request_of(const SampleArgs& a, int b) {
  Req<T> q;
  const size_t V = a.V;
  if (!GEN) {
    q.k = clamp_k(a.num_draft, b, a.K);
    q.greedy = q.bad = false;
    q.c = a.c32;
    q.t0 = static_cast<const T*>(a.target) + (size_t)b * (a.K + 1) * V;
    q.d0 = static_cast<const T*>(a.draft) + (size_t)b * a.K * V;
    return q;
  }
  const int k = a.num_draft[b];
  const float tau = a.temps[b];
  const long ts = a.t_start[b], ds = a.d_start[b];
  q.greedy = tau == 0.0f;
  bool ok = k >= 0 && k <= a.K && (q.greedy || ((double)tau >= kTauMin && tau < INFINITY));
  ok = ok && ts >= 0 && ts + k + 1 <= a.n_trows;
  if (!q.greedy && k > 0) ok = ok && ds >= 0 && ds + k <= a.n_drows;
  q.bad = !ok;
  q.k = ok ? k : 0;
  q.c = (ok && !q.greedy) ? (float)(kLog2e / (double)tau) : 0.0f;
  q.t0 = static_cast<const T*>(a.target) + (ok ? (size_t)ts * V : 0);
  q.d0 = static_cast<const T*>(a.draft) + ((ok && !q.greedy && k > 0) ? (size_t)ds * V : 0);
  return q;
}

// Bonus row of a request (target row k_b, the row the token after an all-accepted block is drawn
// from). Streamed like the other rows, except that a wave's round of kUnroll loads covers one run
// of kSegGroups consecutive groups (load j: 64 groups at 64 j), a segment, and that each round's
// offset is one for the whole wave. So every round also gives its segment's sum of
// 2^(fma(z, c, -o)), which is published with its offset: segment s covers groups
// [s kSegGroups, (s + 1) kSegGroups), and the chunk bounds of a bonus row are multiples of
// kSegGroups. The draw then locates p_k's inverse CDF down to one segment without a second pass
// over the row. Sums are fp32 trees: over a load's E elements, over the kUnroll loads, then over
// the wave (depth 3 + 2 + 6), so a segment sum is within 11 ulp (relative) of the exact sum of its
// fp32 weights, and the inverse CDF built from them is off by less than 7e-7 of the row's mass.
// Loads of groups past g1 are clamped to g1 - 1 and masked to -inf, so every round issues the
// same loads and every lane takes part in the wave reductions.
template <typename T, bool VEC>
struct SegBuf {
  typename Rows<T, VEC>::Raw a[kUnroll];
  // Round starting at group `seg`, the first group of this wave's segment.
  __device__ __forceinline__ void load(const T* __restrict__ row, int seg, int g1) {
    const int g = seg + (int)(threadIdx.x & 63);
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) {
      const int gj = g + 64 * j;
      a[j] = Rows<T, VEC>::load(row, gj < g1 ? gj : g1 - 1);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
};

template <typename T, bool VEC>
__device__ __forceinline__ void seg_round(const SegBuf<T, VEC>& x, int seg, int g1, float c,
                                          float& o, float& s, uint64_t* segs, uint32_t tag) {
  constexpr int E = Rows<T, VEC>::E;
  const int g = seg + (int)(threadIdx.x & 63);
  float f[kUnroll][E];
  float bm = -INFINITY;
#pragma unroll
  for (int j = 0; j < kUnroll; ++j) {
    Rows<T, VEC>::unpack(x.a[j], f[j]);
    const bool ok = g + 64 * j < g1;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      f[j][e] = ok ? f[j][e] : -INFINITY;
      bm = fmaxf(bm, f[j][e]);
    }
  }
  const float on = fmaxf(o, ceilf(wave_max_f32(bm) * c));
  s = rescale(s, o, on);
  o = on;
  float x4[kUnroll];
#pragma unroll
  for (int j = 0; j < kUnroll; ++j) {
    float x[E];
#pragma unroll
    for (int e = 0; e < E; ++e) x[e] = __builtin_amdgcn_exp2f(fmaf(f[j][e], c, -o));
#pragma unroll
    for (int h = 1; h < E; h *= 2)
#pragma unroll
      for (int e = 0; e + h < E; e += 2 * h) x[e] += x[e + h];
    x4[j] = x[0];
  }
#pragma unroll
  for (int h = 1; h < kUnroll; h *= 2)
#pragma unroll
    for (int j = 0; j + h < kUnroll; j += 2 * h) x4[j] += x4[j + h];
  s += x4[0];
  const float st = wave_sum_f32(x4[0]);
  if ((threadIdx.x & 63) == 0 && seg < g1) {
    uint64_t* w = segs + (seg / kSegGroups) * 2;
    publish(w, tag, __float_as_uint(o));
    publish(w + 1, tag, __float_as_uint(st));
  }
}

// Streams groups [g0, g1) of a bonus row (g0 a multiple of kSegGroups) into the thread's (o, s),
// publishing the segment partials on the way. Rounds of kBlock * kUnroll groups (wave w takes
// the w-th segment of the round), two register sets in turn, as in stream_groups.
template <typename T, bool VEC>
__device__ __forceinline__ void stream_segments(const T* __restrict__ row, int g0, int g1, float c,
                                                uint64_t* segs, uint32_t tag, float& o, float& s) {
  constexpr int step = kUnroll * kBlock;
  const int rounds = (g1 - g0 + step - 1) / step;
  const int seg = g0 + kSegGroups * (int)(threadIdx.x >> 6);
  o = -FLT_MAX;
  s = 0.0f;
  if (rounds <= 0) return;
  SegBuf<T, VEC> x, y;
  x.load(row, seg, g1);
  int r = 0;
  for (; r + 2 < rounds; r += 2) {
    y.load(row, seg + (r + 1) * step, g1);
    seg_round<T, VEC>(x, seg + r * step, g1, c, o, s, segs, tag);
    x.load(row, seg + (r + 2) * step, g1);
    seg_round<T, VEC>(y, seg + (r + 1) * step, g1, c, o, s, segs, tag);
  }
  if (rounds - r == 2) {
    y.load(row, seg + (r + 1) * step, g1);
    seg_round<T, VEC>(x, seg + r * step, g1, c, o, s, segs, tag);
    seg_round<T, VEC>(y, seg + (r + 1) * step, g1, c, o, s, segs, tag);
  } else {
    seg_round<T, VEC>(x, seg + r * step, g1, c, o, s, segs, tag);
  }
}

// Chunk c of C of a row of G groups: [G c / C, G (c + 1) / C), with both ends rounded down to a
// multiple of `align` (a power of two; the last chunk ends at G).
__device__ __forceinline__ void chunk_bounds(int G, int c, int C, int CS, int align, int& g0,
                                             int& g1) {
  if (CS > 0) {  // chunks of CS groups (a multiple of every alignment), the last one shorter
    g0 = c * CS < G ? c * CS : G;
    g1 = c + 1 == C ? G : ((c + 1) * CS < G ? (c + 1) * CS : G);
    return;
  }
  g0 = (int)((long)G * c / C) & ~(align - 1);
  g1 = c + 1 == C ? G : (int)((long)G * (c + 1) / C) & ~(align - 1);
}

// Row-stat group (b, slot, c): chunk c of row slot `slot` of request b. Slot s <= K is target row
// s, slot K+1+d is draft row d. Unused rows (s > k_b, d >= k_b) return at once without a read.
// Publishes stats[b][s][c] = (o, sum) with sum = sum_v 2^(fma(z_v, c32, -o)), and, for target
// slots i < k_b and draft slots i < k_b, the group whose chunk holds the draft token x_i
// publishes its logit in gath[b][i][0] (target row i) or gath[b][i][1] (draft row i).
template <typename T, bool VEC, bool GEN>
__device__ void row_stat_group(const SampleArgs& a, int b, int slot, int c) {
  constexpr int E = Rows<T, VEC>::E;
  const int K = a.K, V = a.V, C = a.C;
  const int NR = 2 * K + 1;
  const Req<T> q = request_of<T, GEN>(a, b);
  if (GEN && q.bad) return;
  const int k = q.k;
  const int G = VEC ? V / E : V;
  const bool bonus = slot == k && a.NS > 0;  // the row of p_k, streamed in segments
  int g0, g1;
  chunk_bounds(G, c, C, a.CS, bonus ? kSegGroups : 1, g0, g1);
  if (GEN && q.greedy) {  // greedy request: argmax partials of target rows 0..k, no draft rows
    if (slot > k) return;
    argmax_chunk<T, VEC>(q.t0 + (size_t)slot * V, g0, g1,
                         a.stats + (((size_t)b * NR + slot) * C + c) * 2, a.tag);
    return;
  }
  const T* row;
  int tslot;  // draft slot whose logit this row provides, or -1 (the extra-draw row)
  int gidx;   // 0: the logit is a target logit, 1: a draft logit
  if (slot <= K) {
    if (slot > k) return;
    row = q.t0 + (size_t)slot * V;
    tslot = slot < k ? slot : -1;
    gidx = 0;
  } else {
    const int d = slot - K - 1;
    if (d >= k) return;
    row = q.d0 + (size_t)d * V;
    tslot = d;
    gidx = 1;
  }

  if (threadIdx.x == 0 && tslot >= 0) {
    // a token outside the vocabulary has no logit: chunk 0 publishes a placeholder instead, so
    // that the word of every slot below k_b is published
    const int x = a.tokens[(size_t)b * K + tslot];
    const bool valid = x >= 0 && x < V;
    if (valid ? (x >= g0 * E && x < g1 * E) : c == 0)
      publish(&a.gath[((size_t)b * K + tslot) * 2 + gidx], a.tag,
              valid ? __float_as_uint(Rows<T, VEC>::at(row, x)) : 0u);
  }

  float o, s;
  if (bonus) {
    stream_segments<T, VEC>(row, g0, g1, q.c, a.seg + (size_t)b * a.NSmax * 2, a.tag, o, s);
  } else {
    SoftmaxAcc<E> acc{q.c, -FLT_MAX, 0.0f, 0.0f};
    stream_groups<T, VEC, kUnroll, false>(row, row, g0, g1, acc);
    o = acc.o;
    s = acc.s0 + acc.s1;
  }

  // wave reduce, then across the 4 waves through LDS
  wave_merge_stats(o, s);
  __shared__ float so[kWaves], ss[kWaves];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    so[wave] = o;
    ss[wave] = s;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kWaves; ++w) merge_stats(o, s, so[w], ss[w]);
    uint64_t* st = a.stats + (((size_t)b * NR + slot) * C + c) * 2;
    publish(st, a.tag, __float_as_uint(o));
    publish(st + 1, a.tag, __float_as_uint(s));
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
  // in bounds, no branch around the loads) and are masked to weight 0. Cached loads: the group
  // that finds the token reads its tile a second time, from L2.
  __device__ __forceinline__ void load(const T* rt, const T* rd, int t, int G, int lane) {
#pragma unroll
    for (int j = 0; j < TG; ++j) {
      const int g = t * 64 * TG + 64 * j + lane;
      ok[j] = g < G;
      const int gc = ok[j] ? g : G - 1;
      a[j] = R::load_cached(rt, gc);
      if (RESID) b[j] = R::load_cached(rd, gc);
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

// Staged row-stat entry that merges as nothing: offset -FLT_MAX, sum 0.
constexpr uint64_t kEmptyStat = (uint64_t)0xff7fffffu << 32;

// Merges eight staged partials v[0..7] into (O, S): the new offset is the largest of them all,
// then every term is rescaled to it (exact) and added in order. Branch-free; equal, up to the
// order of the additions, to merging them one at a time.
__device__ __forceinline__ void merge_stats8(float& O, double& S, const uint64_t (&v)[8]) {
  float on = O;
#pragma unroll
  for (int u = 0; u < 8; ++u) on = fmaxf(on, __uint_as_float((uint32_t)(v[u] >> 32)));
  float d = fmaxf(O - on, -2000.0f);
  double acc = ldexp(S, (int)d);
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    d = fmaxf(__uint_as_float((uint32_t)(v[u] >> 32)) - on, -2000.0f);
    acc += ldexp((double)__uint_as_float((uint32_t)v[u]), (int)d);
  }
  O = on;
  S = acc;
}

// Merges the (O, S) pairs of aligned groups of RL lanes (RL a power of two, at most 64); every
// lane of a group ends with the group's pair. Pairs of lanes exchange through DPP (quad
// permutations, then the half-row and row mirrors, which pair the already merged quads and
// half-rows), and through lane permutes across rows.
__device__ __forceinline__ void merge_pair_f64(float& O, double& S, float o2, double s2) {
  const float on = fmaxf(O, o2);
  float d1 = O - on, d2 = o2 - on;
  d1 = d1 < -2000.0f ? -2000.0f : d1;
  d2 = d2 < -2000.0f ? -2000.0f : d2;
  S = ldexp(S, (int)d1) + ldexp(s2, (int)d2);  // the same sum in both lanes of a pair
  O = on;
}
__device__ __forceinline__ void merge_row_lanes(float& O, double& S, int RL) {
  if (RL >= 2) merge_pair_f64(O, S, dpp_f32<0xB1, 0xf>(O, 0.0f), dpp_f64<0xB1, 0xf>(S));  // l^1
  if (RL >= 4) merge_pair_f64(O, S, dpp_f32<0x4E, 0xf>(O, 0.0f), dpp_f64<0x4E, 0xf>(S));  // l^2
  if (RL >= 8) merge_pair_f64(O, S, dpp_f32<0x141, 0xf>(O, 0.0f), dpp_f64<0x141, 0xf>(S));
  if (RL >= 16) merge_pair_f64(O, S, dpp_f32<0x140, 0xf>(O, 0.0f), dpp_f64<0x140, 0xf>(S));
  if (RL >= 32) merge_pair_f64(O, S, __shfl_xor(O, 16), __shfl_xor(S, 16));
  if (RL >= 64) merge_pair_f64(O, S, __shfl_xor(O, 32), __shfl_xor(S, 32));
}

// One wave: inverse CDF inside tile t. Returns the first element v of the tile whose running sum
// (from the start of the tile, element order) exceeds `target`; if none does (rounding), the last
// element of the tile with positive weight; -1 if the tile has none. Sub-tile j is scanned over
// the lanes (fp64 lane sums in element order, then a wave prefix sum); the first lane whose
// prefix passes the target walks its own elements.
template <typename T, bool VEC, bool RESID>
__device__ int tile_find_loaded(const TileRows<T, VEC, RESID>& tr, const DrawParams& w, float c32,
                                int t, double target) {
  using TR = TileRows<T, VEC, RESID>;
  constexpr int E = TR::E;
  const int lane = threadIdx.x & 63;
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
    const double incl = wave_scan_f64(mine);
    const double excl = dpp_f64<kDppWaveShr1, 0xf>(incl);  // exactly the previous lane's prefix
    const uint64_t hit = __ballot(base + incl > target);
    if (hit) {
      const int L = __ffsll((long long)hit) - 1;
      int cand = INT_MAX;
      if (lane == L) {
        double run = base + excl;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          run += (double)v[e];
          if (cand == INT_MAX && v[e] > 0.0f && run > target) cand = first + e;
        }
      }
      cand = (int)lane_u32((uint32_t)cand, L);
      if (cand != INT_MAX) return cand;
    }
    base += lane_f64(incl, 63);
  }
  return wave_max_i32(last_pos);
}

template <typename T, bool VEC, bool RESID>
__device__ int tile_find(const T* rt, const T* rd, const DrawParams& w, float c32, int G, int t,
                         double target) {
  TileRows<T, VEC, RESID> tr;
  tr.load(rt, rd, t, G, threadIdx.x & 63);
  return tile_find_loaded<T, VEC, RESID>(tr, w, c32, t, target);
}

// Per-tile weight sums of tiles [t0, t1) by the 4 waves of the group, kTileUnroll tiles per wave
// in flight. The sum of tile t goes to out[t - t0] (LDS).
template <typename T, bool VEC, bool RESID>
__device__ __forceinline__ void tile_sums(const T* rt, const T* rd, const DrawParams& w,
                                          float c32, int G, int t0, int t1, double* out) {
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
        if (lane == 0) out[tu - t0] = s;
      }
    }
  }
}

struct Pick {
  int idx;       // chosen index; -1 when the total is 0
  bool found;    // false: no prefix exceeded the target (rounding); idx = last positive entry
  double rel;    // target minus the sum of the entries before idx (infinite when not found)
  double total;  // sum of all n entries
};

// Inverse CDF over n fp64 weights in LDS, by one wave, in index order: the first index with a
// positive weight whose inclusive prefix exceeds the target, which is frac * total when
// frac >= 0, else `fixed`. Lane l sums the block [l*m, (l+1)*m) (m = ceil(n/64)) in index order,
// a wave prefix sum over the block sums gives each block's starting prefix, and the first lane
// whose prefix passes the target walks its block. The result is wave-uniform, and every wave
// that runs it on the same values gets the same answer.
__device__ Pick wave_pick(const double* vals, int n, double frac, double fixed) {
  const int lane = threadIdx.x & 63;
  const int m = (n + 63) >> 6;
  const int i0 = min(n, lane * m), i1 = min(n, i0 + m);
  double blk = 0.0;
  int last_pos = -1;
  for (int i = i0; i < i1; ++i) {
    const double v = vals[i];
    blk += v;
    if (v > 0.0) last_pos = i;
  }
  const double incl = wave_scan_f64(blk);
  const double excl = dpp_f64<kDppWaveShr1, 0xf>(incl);
  Pick p;
  p.total = lane_f64(incl, 63);
  p.idx = -1;
  p.found = false;
  p.rel = INFINITY;
  if (!(p.total > 0.0)) return p;
  const double target = frac >= 0.0 ? frac * p.total : fixed;
  const uint64_t hit = __ballot(incl > target);
  if (hit) {
    const int L = __ffsll((long long)hit) - 1;
    int idx = -1;
    double rel = 0.0;
    if (lane == L) {
      double run = excl;
      for (int i = i0; i < i1; ++i) {
        const double v = vals[i];
        const double nx = run + v;
        if (v > 0.0 && nx > target) {
          idx = i;
          rel = target - run;
          break;
        }
        run = nx;
      }
    }
    idx = (int)lane_u32((uint32_t)idx, L);
    if (idx >= 0) {
      p.idx = idx;
      p.found = true;
      p.rel = lane_f64(rel, L);
      return p;
    }
  }
  p.idx = wave_max_i32(last_pos);
  return p;
}

// Zero residual mass at a rejected slot (possible only through fp32 rounding): draw from p_n
// over the whole row instead, with one group, in blocks of kChunkTiles tiles (two passes). Every
// wave runs the picks on the same tile sums, so all waves take the same branches. Returns the
// token (wave 0 only; -1 if the row has no positive weight).
template <typename T, bool VEC>
__device__ int full_row_draw(const T* rt, const DrawParams& w, float c32, int G, int NT,
                             double r, double* tsum) {
  double total = 0.0;
  for (int t0 = 0; t0 < NT; t0 += kChunkTiles) {
    const int t1 = min(NT, t0 + kChunkTiles);
    tile_sums<T, VEC, false>(rt, rt, w, c32, G, t0, t1, tsum);
    __syncthreads();
    total += wave_pick(tsum, t1 - t0, -1.0, INFINITY).total;
    __syncthreads();
  }
  const double target = r * total;
  double acc = 0.0;
  int tile = -1;
  double rel = INFINITY;
  for (int t0 = 0; t0 < NT; t0 += kChunkTiles) {
    const int t1 = min(NT, t0 + kChunkTiles);
    tile_sums<T, VEC, false>(rt, rt, w, c32, G, t0, t1, tsum);
    __syncthreads();
    const Pick p = wave_pick(tsum, t1 - t0, -1.0, target - acc);
    __syncthreads();
    if (p.found) {
      tile = t0 + p.idx;
      rel = p.rel;
      break;
    }
    if (p.idx >= 0) tile = t0 + p.idx;  // last tile with mass so far, drawn past its end
    acc += p.total;
  }
  int y = -1;
  if (threadIdx.x < 64 && tile >= 0) y = tile_find<T, VEC, false>(rt, rt, w, c32, G, tile, rel);
  return y;
}

// One wave: inverse CDF inside segment t of a bonus row, with the weights its row-stat group
// summed, 2^(fma(z, c, -o_t)). `target` is on that scale, measured from the segment's start.
// Returns the first element whose running sum (fp64, element order) exceeds it; if none does
// (rounding), the last element of the segment with positive weight; -1 if it has none. The
// segment's kUnroll blocks of 64 groups are scanned in order (fp64 lane sums, a wave prefix sum),
// and the first lane whose prefix passes the target walks its own elements.
template <typename T, bool VEC>
__device__ int segment_find(const T* rt, float c, float ot, int G, int t, double target) {
  using R = Rows<T, VEC>;
  constexpr int E = R::E;
  const int lane = threadIdx.x & 63;
  typename R::Raw raw[kUnroll];
#pragma unroll
  for (int j = 0; j < kUnroll; ++j) {
    const int g = t * kSegGroups + 64 * j + lane;
    raw[j] = R::load_cached(rt, g < G ? g : G - 1);
  }
  double base = 0.0;
  int last_pos = -1;
#pragma unroll
  for (int j = 0; j < kUnroll; ++j) {
    const int g = t * kSegGroups + 64 * j + lane;
    const bool ok = g < G;
    float f[E], v[E];
    R::unpack(raw[j], f);
    double mine = 0.0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      v[e] = ok ? __builtin_amdgcn_exp2f(fmaf(f[e], c, -ot)) : 0.0f;
      mine += (double)v[e];
      if (v[e] > 0.0f) last_pos = g * E + e;
    }
    const double incl = wave_scan_f64(mine);
    const double excl = dpp_f64<kDppWaveShr1, 0xf>(incl);
    const uint64_t hit = __ballot(base + incl > target);
    if (hit) {
      const int L = __ffsll((long long)hit) - 1;
      int cand = INT_MAX;
      if (lane == L) {
        double run = base + excl;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          run += (double)v[e];
          if (cand == INT_MAX && v[e] > 0.0f && run > target) cand = g * E + e;
        }
      }
      cand = (int)lane_u32((uint32_t)cand, L);
      if (cand != INT_MAX) return cand;
    }
    base += lane_f64(incl, 63);
  }
  return wave_max_i32(last_pos);
}

// True in every thread of the group when v is true in any thread: one barrier. `flags` is a
// kWaves-entry LDS array that no other code touches between the barrier before and after.
__device__ __forceinline__ bool block_any(bool v, int* flags) {
  const uint64_t m = __ballot(v);
  if ((threadIdx.x & 63) == 0) flags[threadIdx.x >> 6] = m != 0;
  __syncthreads();
  bool any = false;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) any = any || flags[w] != 0;
  return any;
}

// Normaliser (O, S) of one row from its C staged partials st[c * stride], by one lane, eight LDS
// reads in flight at a time. Partials are staged chunk-major (stride = rows staged), so the lanes
// of a wave, one row each, read consecutive words: no bank conflicts.
__device__ __forceinline__ void row_norm(const uint64_t* st, int C, int stride, float& O,
                                         double& S) {
  O = -FLT_MAX;
  S = 0.0;
  for (int c0 = 0; c0 < C; c0 += 8) {
    uint64_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = c0 + u < C ? st[(c0 + u) * stride] : kEmptyStat;
    merge_stats8(O, S, v);
  }
}

// 2^a for a <= 0 in fp64, to about fp32's relative accuracy: an exact split into the integer
// part and the fraction, which goes through v_exp_f32 (relative error ~1e-7).
// Exponents below -1100 (a logit of -inf among them: probability 0) give 0, as 2^a rounds to 0
// in fp64 there; taking the split of -inf itself would give NaN.
__device__ __forceinline__ double exp2_split(double a) {
  a = fmax(a, -1100.0);
  const double fl = floor(a);
  const float fr = (float)(a - fl);  // [0, 1]
  return ldexp((double)__builtin_amdgcn_exp2f(fr), (int)fl);
}

// Greedy request inside a mixed call, by its chunk-0 draw group: waits for the argmax partials of
// target rows 0..k, merges them per row (lane i: row i; lane 0 also row 64 when k = 64; the
// lowest index among equal maxima), n = first i < k with x_i != g_i, else k; writes
// x_0..x_{n-1}, g_n, -1... and probabilities 0.
__device__ void greedy_request_finish(const SampleArgs& a, int b, int k, uint64_t* g_stage,
                                      int* g_late) {
  const int K = a.K, C = a.C, NR = 2 * K + 1;
  const uint32_t tag = a.tag;
  const int lane = threadIdx.x & 63;
  const int nent = (k + 1) * C;  // <= kStageMax by the plan
  const int xi = lane < k ? a.tokens[(size_t)b * K + lane] : -1;
  bool late = false;
  for (int e0 = 0; e0 < nent; e0 += kBlock * 4) {
    const uint64_t* p[4];
    bool live[4];
    uint64_t wv[4], wi[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      int e = e0 + u * kBlock + (int)threadIdx.x;
      live[u] = e < nent;
      e = live[u] ? e : nent - 1;
      p[u] = a.stats + (((size_t)b * NR + e / C) * C + e % C) * 2;  // target slot e / C
    }
    late = late || !await4(p, live, tag, wv, wi);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = e0 + u * kBlock + (int)threadIdx.x;
      if (e < nent) g_stage[e] = ((uint64_t)payload(wv[u]) << 32) | payload(wi[u]);
    }
  }
  if (block_any(late, g_late)) {
    if (threadIdx.x == 0) a.accepted_len[b] = kTimedOut;
    return;
  }
  if (threadIdx.x >= 64) return;
  auto row_argmax = [&](int r) {
    float v = -INFINITY;
    int idx = INT_MAX;
    for (int c = 0; c < C; ++c) {
      const uint64_t w = g_stage[r * C + c];
      merge_argmax(v, idx, __uint_as_float((uint32_t)(w >> 32)), (int)(uint32_t)w);
    }
    return idx == INT_MAX ? 0 : idx;  // a row of -inf only: index 0
  };
  const int g = lane <= k ? row_argmax(lane) : 0;
  const int gx = (k == kMaxK && lane == 0) ? row_argmax(kMaxK) : 0;
  const uint64_t m = __ballot(lane < k && xi != g);
  const int n = m ? (__ffsll((long long)m) - 1) : k;
  const int gn = n < 64 ? (int)lane_u32((uint32_t)g, n) : (int)lane_u32((uint32_t)gx, 0);
  for (int i = lane; i <= K; i += 64) {
    int v = -1;
    if (i < n) v = a.tokens[(size_t)b * K + i];
    else if (i == n) v = gn;
    a.committed[(size_t)b * (K + 1) + i] = v;
    if (i < K) {
      a.target_prob[(size_t)b * K + i] = 0.0f;
      if (a.draft_prob != nullptr) a.draft_prob[(size_t)b * K + i] = 0.0f;
    }
  }
  if (lane == 0) a.accepted_len[b] = n;
}

// Draw group (b, c2) of request b; chunk c2 covers tiles [NT*c2/C2, NT*(c2+1)/C2).
template <typename T, bool VEC, bool GEN>
__device__ void draw_group(const SampleArgs& a, int b, int c2) {
  constexpr int E = Rows<T, VEC>::E;
  const int K = a.K, V = a.V, C = a.C, C2 = a.C2, NT = a.NT;
  const int NR = 2 * K + 1;
  const Req<T> q = request_of<T, GEN>(a, b);
  const int k = q.k;
  const float c32 = q.c;
  const uint32_t tag = a.tag;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // s_buf stages the row-stat partials from its start, and holds tile sums and chunk totals at
  // its end.
  __shared__ double s_buf[kStageMax];
  __shared__ float s_o[2 * kMaxK + 1];
  __shared__ double s_S[2 * kMaxK + 1];
  __shared__ float s_zt[kMaxK], s_zd[kMaxK];
  __shared__ int s_late1[kWaves], s_late2[kWaves];
  uint64_t* stage = reinterpret_cast<uint64_t*>(s_buf);

  if constexpr (GEN) {
   if (q.bad || q.greedy) {
    if (c2 != 0) return;
    if (q.bad) {
      for (int i = threadIdx.x; i <= K; i += kBlock) {
        a.committed[(size_t)b * (K + 1) + i] = -1;
        if (i < K) {
          a.target_prob[(size_t)b * K + i] = 0.0f;
          if (a.draft_prob != nullptr) a.draft_prob[(size_t)b * K + i] = 0.0f;
        }
      }
      if (threadIdx.x == 0) a.accepted_len[b] = kBadRequest;
      return;
    }
    greedy_request_finish(a, b, k, stage, s_late1);
    return;
   }
  }


  // Per-request inputs, read before the wait. Lane i < k of every wave holds slot i.
  const double r = (double)a.residual[b];
  const int xi = lane < k ? a.tokens[(size_t)b * K + lane] : -1;
  const float uni = lane < k ? a.uniforms[(size_t)b * K + lane] : 0.0f;
  const bool want_x = xi >= 0 && xi < V;

  // 1. Wait for the partials the decision needs and the logits at the draft tokens to carry
  //    this call's tag; the words read in the last round are the data. Entries e < nent are
  //    row-stat partials, e = row * C + chunk (staged chunk-major as offset bits, sum bits),
  //    entries nent + i the two logits of draft token i. The partials of target row k (row k
  //    of the staging) are awaited only when an all-accepted block's token is drawn by tiles
  //    (NS == 0): the segment draw needs only the row's segment partials, so the decision
  //    does not wait for that row; its staged entries stay empty.
  const int nrow = 2 * k + 1, nent = nrow * C;  // nent <= kStageMax by the plan
  const int ntot = nent + k;
  const bool want_row_k = a.NS == 0;
  bool late = false;
  for (int e0 = 0; e0 < ntot; e0 += kBlock * 4) {
    const uint64_t* p[4];
    bool live[4];
    uint64_t w0[4], w1[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = e0 + u * kBlock + (int)threadIdx.x;
      live[u] = e < ntot && (want_row_k || e / C != k || e >= nent);
      if (e < nent) {
        const int r_ = e / C, c = e % C;
        const int slot = r_ <= k ? r_ : K + 1 + (r_ - k - 1);
        p[u] = a.stats + (((size_t)b * NR + slot) * C + c) * 2;
      } else {
        const int i = live[u] ? e - nent : 0;
        p[u] = a.gath + ((size_t)b * K + i) * 2;
      }
    }
    late = late || !await4(p, live, tag, w0, w1);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = e0 + u * kBlock + (int)threadIdx.x;
      if (e < nent) {
        stage[(e % C) * nrow + e / C] =
            live[u] ? ((uint64_t)payload(w0[u]) << 32) | payload(w1[u]) : kEmptyStat;
      } else if (e < ntot) {
        s_zt[e - nent] = __uint_as_float(payload(w0[u]));
        s_zd[e - nent] = __uint_as_float(payload(w1[u]));
      }
    }
  }
  if (block_any(late, s_late1)) {
    if (threadIdx.x == 0) a.accepted_len[b] = kTimedOut;
    return;
  }

  // 2. Normalisers of the rows that slot `lane` uses, in every wave: target row lane
  //    (lane <= k) and draft row lane (lane < k); with k = 64 lane 0 also takes target row 64.
  //    Up to kLaneRowChunks chunks per row one lane combines a row; beyond that RL lanes share
  //    a row and the results go through LDS.
  float Ot = -FLT_MAX, Od = -FLT_MAX, Ox = -FLT_MAX;
  double St = 0.0, Sd = 0.0, Sx = 0.0;
  if (C <= kLaneRowChunks) {
    if (lane <= k) row_norm(stage + lane, C, nrow, Ot, St);
    if (lane < k) row_norm(stage + k + 1 + lane, C, nrow, Od, Sd);
    if (k == kMaxK && lane == 0) row_norm(stage + kMaxK, C, nrow, Ox, Sx);
  } else {
    int RL = 1;
    while (RL * 16 < C) RL <<= 1;  // C <= kStageMax, so RL <= 128: capped below
    RL = RL > 64 ? 64 : RL;
    for (int t0 = 0; t0 < nrow * RL; t0 += kBlock) {
      const int t = t0 + (int)threadIdx.x;
      const int row = t / RL, li = t % RL;
      const bool live = row < nrow;
      const uint64_t* st = stage + (live ? row : 0);
      float O = -FLT_MAX;
      double S = 0.0;
      for (int c0 = li; c0 < C; c0 += 8 * RL) {
        uint64_t v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int c = c0 + u * RL;
          v[u] = c < C ? st[c * nrow] : kEmptyStat;
        }
        merge_stats8(O, S, v);
      }
      merge_row_lanes(O, S, RL);
      if (live && li == 0) {
        const int slot = row <= k ? row : K + 1 + (row - k - 1);
        s_o[slot] = O;
        s_S[slot] = S;
      }
    }
    __syncthreads();
    if (lane <= k) {
      Ot = s_o[lane];
      St = s_S[lane];
    }
    if (lane < k) {
      Od = s_o[K + 1 + lane];
      Sd = s_S[K + 1 + lane];
    }
    if (k == kMaxK && lane == 0) {
      Ox = s_o[kMaxK];
      Sx = s_S[kMaxK];
    }
  }

  // 3. p(x) = et / St, q(x) = ed / Sd, the accept decisions and the first rejection n, in every
  //    wave. Slot i is kept when u_i < min(1, p/q), i.e. (u_i < 1) when u_i ed St < et Sd: no
  //    division on the way to n (the same comparison up to rounding; q = 0 keeps the slot exactly
  //    when p > 0, a token outside the vocabulary is rejected).
  int n;
  {
    double et = 0.0, ed = 0.0;
    bool rej = false;
    if (lane < k) {
      if (want_x) {
        et = exp2_split((double)s_zt[lane] * (double)c32 - (double)Ot);
        ed = exp2_split((double)s_zd[lane] * (double)c32 - (double)Od);
      }
      rej = !(want_x && (double)uni * ed * St < et * Sd);
    }
    const uint64_t m = __ballot(rej);
    n = m ? (__ffsll((long long)m) - 1) : k;
    if (c2 == 0 && wave == 0 && lane < K) {  // slots k..K-1 get 0
      a.target_prob[(size_t)b * K + lane] = lane < k ? (float)(et / St) : 0.0f;
      if (a.draft_prob != nullptr)
        a.draft_prob[(size_t)b * K + lane] = lane < k ? (float)(ed / Sd) : 0.0f;
    }
  }

  // 4. The draw row: target row n, minus draft row n when slot n was rejected.
  const bool resid = n < k;
  DrawParams w;
  w.n = n;
  w.resid = resid ? 1 : 0;
  w.oT = n < 64 ? lane_f32(Ot, n) : lane_f32(Ox, 0);
  w.iT = (float)(1.0 / (n < 64 ? lane_f64(St, n) : lane_f64(Sx, 0)));
  w.oD = resid ? lane_f32(Od, n) : 0.0f;
  w.iD = resid ? (float)(1.0 / lane_f64(Sd, n)) : 0.0f;
  if (c2 == 0) {
    for (int i = threadIdx.x; i <= K; i += kBlock) {
      if (i < n) a.committed[(size_t)b * (K + 1) + i] = a.tokens[(size_t)b * K + i];
      else if (i > n) a.committed[(size_t)b * (K + 1) + i] = -1;
    }
    if (threadIdx.x == 0) a.accepted_len[b] = n;
  }
  const T* rt = q.t0 + (size_t)n * V;
  const T* rd = resid ? q.d0 + (size_t)n * V : rt;
  const int G = VEC ? V / E : V;

  // 4'. Every draft kept: the token is drawn from p_n (n = k) by the request's first draw group
  //     alone, from the segment partials of its row-stat groups: await them, scale them to the
  //     largest segment offset (exact), pick the segment holding r * Z (every wave, the same
  //     answer), and wave 0 finds the token inside it. The draw needs no normaliser of the row:
  //     r * Z and the running sums are on one scale. The staged partials are dead by now (every
  //     wave has its normalisers), so the segment values reuse s_buf: fp64 values, then their
  //     fp32 offsets.
  if (!resid && a.NS > 0) {
    if (c2 != 0) return;
    const int NS = a.NS;  // <= kSegMax
    double* vals = s_buf;
    float* offs = reinterpret_cast<float*>(s_buf + kSegMax);
    __shared__ float s_omax[kWaves];
    const uint64_t* sg = a.seg + (size_t)b * a.NSmax * 2;
    __syncthreads();
    bool late3 = false;
    float om = -FLT_MAX;
    for (int e0 = 0; e0 < NS; e0 += kBlock * 4) {
      const uint64_t* p[4];
      bool live[4];
      uint64_t wo[4], ws[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int e = e0 + u * kBlock + (int)threadIdx.x;
        live[u] = e < NS;
        p[u] = sg + 2 * (live[u] ? e : 0);
      }
      late3 = late3 || !await4(p, live, tag, wo, ws);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int e = e0 + u * kBlock + (int)threadIdx.x;
        if (e < NS) {
          const float os = __uint_as_float(payload(wo[u]));
          vals[e] = (double)__uint_as_float(payload(ws[u]));
          offs[e] = os;
          om = fmaxf(om, os);
        }
      }
    }
    om = wave_max_f32(om);
    if (lane == 0) s_omax[wave] = om;
    if (block_any(late3, s_late2)) {
      if (threadIdx.x == 0) a.accepted_len[b] = kTimedOut;
      return;
    }
#pragma unroll
    for (int w2 = 0; w2 < kWaves; ++w2) om = fmaxf(om, s_omax[w2]);
    for (int e = threadIdx.x; e < NS; e += kBlock)
      vals[e] = ldexp(vals[e], (int)fmaxf(offs[e] - om, -2000.0f));  // exponent <= 0
    __syncthreads();
    const Pick pk = wave_pick(vals, NS, r, 0.0);
    if (pk.idx < 0) {  // no mass at all (non-finite logits): the tile draw over the whole row
      DrawParams wk = w;
      wk.oT = om;
      wk.iT = 1.0f;
      const int y = full_row_draw<T, VEC>(rt, wk, c32, G, NT, r, s_buf + kStageMax - kChunkTiles);
      if (threadIdx.x == 0) a.committed[(size_t)b * (K + 1) + n] = y < 0 ? 0 : y;
      return;
    }
    if (wave != 0) return;
    const float os = offs[pk.idx];
    const double rel = pk.found ? ldexp(pk.rel, (int)fmaxf(om - os, 0.0f)) : INFINITY;
    const int y = segment_find<T, VEC>(rt, c32, os, G, pk.idx, rel);
    if (lane == 0) a.committed[(size_t)b * (K + 1) + n] = y < 0 ? 0 : y;
    return;
  }

  // 5. Tile sums of this chunk (LDS); wave 0 publishes the chunk total for the other groups of
  //    the request (the same sum that its own pick over the tile sums computes). Tile sums and
  //    chunk totals sit at the end of s_buf; when the staged partials reach that far, every
  //    wave must be done reading them first.
  double* tsum = s_buf + kStageMax - kChunkTiles - kMaxC2;  // [kChunkTiles]
  double* ctot = tsum + kChunkTiles;                         // [kMaxC2]
  if (nent > kStageMax - kChunkTiles - kMaxC2) __syncthreads();
  const int t0 = (int)((long)NT * c2 / C2), t1 = (int)((long)NT * (c2 + 1) / C2);
  // A residual chunk of one round keeps its tiles in registers (tile t0 + wave + u * kWaves in
  // held[u]): the wave that loaded the chosen tile finds the token in it without reading it again.
  // Only 16-byte bf16 rows of the padded call: there a tile takes 8 registers per lane, and the
  // other kernels' register budgets have no room for it.
  constexpr bool kMayHold = !GEN && VEC && sizeof(T) == 2;
  TileRows<T, VEC, true> held[kMayHold ? kTileUnroll : 1];
  const bool hold = kMayHold && resid && t1 - t0 <= kWaves * kTileUnroll;
  if constexpr (kMayHold) {
    if (hold) {
#pragma unroll
      for (int u = 0; u < kTileUnroll; ++u) {
        const int tu = t0 + wave + u * kWaves;
        if (tu < t1) held[u].load(rt, rd, tu, G, lane);
      }
#pragma unroll
      for (int u = 0; u < kTileUnroll; ++u) {
        const int tu = t0 + wave + u * kWaves;
        if (tu < t1) {
          const double sum = wave_sum_f64(held[u].lane_sum(w, c32));
          if (lane == 0) tsum[tu - t0] = sum;
        }
      }
    }
  }
  if (hold) {
  } else if (resid) {
    tile_sums<T, VEC, true>(rt, rd, w, c32, G, t0, t1, tsum);
  } else {
    tile_sums<T, VEC, false>(rt, rd, w, c32, G, t0, t1, tsum);
  }
  __syncthreads();
  uint64_t* ct = a.ctot + (size_t)b * C2 * 2;
  if (wave == 0) {
    const double mine = wave_pick(tsum, t1 - t0, -1.0, INFINITY).total;
    if (lane == 0) {
      const uint64_t bits = (uint64_t)__double_as_longlong(mine);
      publish(&ct[2 * c2], tag, (uint32_t)(bits >> 32));
      publish(&ct[2 * c2 + 1], tag, (uint32_t)bits);
    }
  }

  // 6. Every chunk total of the request (awaited as above), then the chunk holding r * Z, in
  //    every wave (the same answer in every wave and every group of the request).
  {
    bool late2 = false;
    for (int c0 = 0; c0 < C2; c0 += kBlock * 4) {
      const uint64_t* p[4];
      bool live[4];
      uint64_t hi[4], lo[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        int c = c0 + u * kBlock + (int)threadIdx.x;
        live[u] = c < C2;
        c = live[u] ? c : C2 - 1;
        p[u] = &ct[2 * c];
      }
      late2 = late2 || !await4(p, live, tag, hi, lo);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int c = c0 + u * kBlock + (int)threadIdx.x;
        if (c < C2)
          ctot[c] = __longlong_as_double(
              (long long)(((uint64_t)payload(hi[u]) << 32) | payload(lo[u])));
      }
    }
    if (block_any(late2, s_late2)) {
      if (threadIdx.x == 0) a.accepted_len[b] = kTimedOut;
      return;
    }
  }
  const Pick pc = wave_pick(ctot, C2, r, 0.0);
  if (pc.idx < 0) {  // zero residual mass (rounding only): chunk 0's group draws from p_n
    if (c2 != 0) return;
    const int y = full_row_draw<T, VEC>(rt, w, c32, G, NT, r, tsum);
    if (threadIdx.x == 0) a.committed[(size_t)b * (K + 1) + n] = y < 0 ? 0 : y;
    return;
  }
  if (pc.idx != c2) return;

  // 7. This group holds r * Z: every wave picks the tile inside the chunk (the same answer); the
  //    wave that holds it (wave 0 when the tiles were not held) finds the token inside it.
  const Pick pt = wave_pick(tsum, t1 - t0, -1.0, pc.rel);
  const int finder = hold && pt.idx >= 0 ? pt.idx % kWaves : 0;
  if (wave != finder) return;
  int y = -1;
  if (pt.idx >= 0) {
    const double rel = pc.found ? pt.rel : INFINITY;
    if constexpr (kMayHold) {
      if (hold) {
        const int sel = pt.idx / kWaves;  // wave-uniform; copied out without indexing registers
        TileRows<T, VEC, true> tr = held[0];
#pragma unroll
        for (int u = 1; u < kTileUnroll; ++u)
          if (sel == u) tr = held[u];
        y = tile_find_loaded<T, VEC, true>(tr, w, c32, t0 + pt.idx, rel);
      }
    }
    if (!hold) {
      y = resid ? tile_find<T, VEC, true>(rt, rd, w, c32, G, t0 + pt.idx, rel)
                : tile_find<T, VEC, false>(rt, rd, w, c32, G, t0 + pt.idx, rel);
    }
  }
  if (lane == 0) a.committed[(size_t)b * (K + 1) + n] = y < 0 ? 0 : y;
}

// Grid order. Request by request, the (2K+1)*C row-stat groups of request j (slot by slot,
// chunk by chunk), followed, once j >= L, by the C2 draw groups of request j - L; after the last
// request, the draw groups of the last L requests. With a lag L of about the number of requests
// whose row-stat groups are resident at once (the host sets it from the kernel's occupancy), a
// request's draw groups are dispatched when its rows have mostly been streamed: they draw while
// later requests stream, instead of all together after the last row. Every wait is on groups
// earlier in the grid, which are dispatched first.
struct SampleRole {
  bool draw;
  int b, slot, c;  // row-stat group: request, row slot, chunk; draw group: request, -, chunk
};

// (32-bit arithmetic: the host keeps a grid below 2^24 groups, and 64-bit divisions at every
// group's start measured 0.2-0.3 us slower on the batched call.)
__device__ __forceinline__ SampleRole sample_role(const SampleArgs& a, long idx_l) {
  const uint32_t K = a.K, C = a.C, L = a.L;
  const uint32_t F = (2u * K + 1u) * C;
  const uint32_t Q = a.C2;
  const uint32_t n1 = L * F, n2 = ((uint32_t)a.B - L) * (F + Q);
  const uint32_t idx = (uint32_t)idx_l;
  SampleRole r;
  uint32_t q;
  if (idx < n1) {
    r.b = (int)(idx / F);
    q = idx % F;
    r.draw = false;
  } else if (idx < n1 + n2) {
    const uint32_t i = idx - n1;
    q = i % (F + Q);
    r.draw = q >= F;
    r.b = (int)(L + i / (F + Q) - (r.draw ? L : 0));
    if (r.draw) q -= F;
  } else {
    const uint32_t i = idx - n1 - n2;
    r.b = (int)((uint32_t)a.B - L + i / Q);
    q = i % Q;
    r.draw = true;
  }
  if (r.draw) {
    r.slot = 0;
    r.c = (int)q;
  } else {
    r.slot = (int)(q / C);
    r.c = (int)(q % C);
  }
  return r;
}

template <typename T, bool VEC>
__global__ __launch_bounds__(kBlock) void sv_verify_sample(SampleArgs a) {
  const SampleRole r = sample_role(a, (long)blockIdx.x);
  if (!r.draw) row_stat_group<T, VEC, false>(a, r.b, r.slot, r.c);
  else draw_group<T, VEC, false>(a, r.b, r.c);
}

// Flattened, mixed calls: the same grid and groups, each request read through its own rows and
// temperature.
template <typename T, bool VEC>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(VEC ? 6 : 1))) void sv_verify_ragged_kernel(SampleArgs a) {
  const SampleRole r = sample_role(a, (long)blockIdx.x);
  if (!r.draw) row_stat_group<T, VEC, true>(a, r.b, r.slot, r.c);
  else draw_group<T, VEC, true>(a, r.b, r.c);
}

// ---------------------------------------------------------------------------------------------
// Greedy mode: per-chunk argmax (lowest index among equal maxima), then one finishing group per
// request.

struct GreedyArgs {
  const void* target;  // [B][K+1][V]
  int B, K, V;
  const int32_t* num_draft;
  const int32_t* tokens;
  int C;
  long n_argmax_groups;  // B * (K+1) * C: groups before this index are argmax groups
  uint32_t tag;
  uint64_t* gstats;
  int32_t* accepted_len;
  int32_t* committed;
};

template <typename T, bool VEC>
__device__ void argmax_group(const GreedyArgs& a, long wg) {
  constexpr int E = Rows<T, VEC>::E;
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
  argmax_chunk<T, VEC>(row, g0, g1, a.gstats + (((size_t)b * NR + slot) * C + c) * 2, a.tag);
}

template <typename T, bool VEC>
__device__ void finish_group(const GreedyArgs& a, int b) {
  const int K = a.K, C = a.C;
  const int NR = K + 1;
  const int k = clamp_k(a.num_draft, b, K);
  const uint32_t tag = a.tag;
  __shared__ uint64_t stage[kStageMax];
  __shared__ int s_g[kMaxK + 1];
  __shared__ int s_n;
  const int nent = (k + 1) * C;  // <= kStageMax by the plan
  bool late = false;
  for (int e0 = 0; e0 < nent; e0 += kBlock * 4) {
    const uint64_t* p[4];
    bool live[4];
    uint64_t wv[4], wi[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      int e = e0 + u * kBlock + (int)threadIdx.x;
      live[u] = e < nent;
      e = live[u] ? e : nent - 1;
      p[u] = a.gstats + ((size_t)b * NR * C + e) * 2;  // rows 0..k come first
    }
    late = late || !await4(p, live, tag, wv, wi);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = e0 + u * kBlock + (int)threadIdx.x;
      if (e < nent) stage[e] = ((uint64_t)payload(wv[u]) << 32) | payload(wi[u]);
    }
  }
  __shared__ int s_late[kWaves];
  if (block_any(late, s_late)) {
    if (threadIdx.x == 0) a.accepted_len[b] = kTimedOut;
    return;
  }
  for (int i = threadIdx.x; i <= k; i += kBlock) {
    float v = -INFINITY;
    int idx = INT_MAX;
    for (int c = 0; c < C; ++c) {
      const uint64_t u = stage[i * C + c];
      merge_argmax(v, idx, __uint_as_float((uint32_t)(u >> 32)), (int)(uint32_t)u);
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
  if (threadIdx.x == 0) a.accepted_len[b] = n;
}

template <typename T, bool VEC>
__global__ __launch_bounds__(kBlock) void sv_verify_greedy_kernel(GreedyArgs a) {
  const long wg = blockIdx.x;
  if (wg < a.n_argmax_groups) argmax_group<T, VEC>(a, wg);
  else finish_group<T, VEC>(a, (int)(wg - a.n_argmax_groups));
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

// Segments of a bonus row (kSegGroups groups of 16-byte vectors or of single elements), or 0 when
// they do not fit the workspace's slots: then bonus tokens take the tile draw.
int segments_per_row(int V, int dtype, bool vec, const Plan& p) {
  const long G = vec ? (long)V * (long)elem_size(dtype) / 16 : (long)V;
  const long ns = (G + kSegGroups - 1) / kSegGroups;
  return ns <= p.NSmax ? (int)ns : 0;
}

// Work-groups of `kernel` resident at once on the current device (cached per device; host
// threads that fill an entry at the same time store the same value).
long resident_groups(const void* kernel, std::atomic<long>* cache) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 1536;
  long n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kBlock, 0) != hipSuccess ||
        per_cu < 1)
      per_cu = 6;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus < 1)
      cus = 256;
    n = (long)per_cu * cus;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

template <typename T, bool VEC, bool GEN>
int launch_sample(const SampleArgs& args, hipStream_t stream) {
  const void* kernel = GEN ? reinterpret_cast<const void*>(&sv_verify_ragged_kernel<T, VEC>)
                           : reinterpret_cast<const void*>(&sv_verify_sample<T, VEC>);
  static std::atomic<long> cache[kMaxDevices] = {};
  SampleArgs a = args;
  // Fewer, longer chunks than the plan's for 16-byte rows (the plan sizes the workspace for its
  // C; fewer chunks use less of it): at most kBf16Chunks per bf16 row, and kF32Chunks per float32
  // row once that still leaves 1024 row-stat groups (about three rounds of 16-byte loads per
  // chunk at V = 151936; fewer partials for the decision to gather). Measured at V = 151936,
  // K = 8 against the plan's 12-37 chunks: bf16 B = 1-48 3-30% faster, float32 B = 8-16 10-17%
  // faster, B = 1-4 the same or slower with 12 (there 37 chunks of one round each fill the GPU).
  if (VEC && sizeof(T) == 2 && a.C > kBf16Chunks) a.C = kBf16Chunks;
  if (VEC && sizeof(T) == 4 && a.C > kF32Chunks && (long)a.B * (2 * a.K + 1) * kF32Chunks >= 1024)
    a.C = kF32Chunks;
  // Chunks of whole rounds: when an even split leaves each chunk a few groups past a whole number
  // of rounds (kUnroll loads per thread), those few go through the one-group tail, one more memory
  // round trip in every chunk; one more chunk (the workspace has room for it), all the others of
  // whole rounds and the last one shorter, avoids it. (B = 1, float32, V = 151936: 37 chunks of
  // 1027 groups became 38 of 1024.)
  a.CS = 0;
  {
    const long E = VEC ? 16 / (long)sizeof(T) : 1;
    const long G = VEC ? a.V / E : a.V;
    const long R = (long)kUnroll * kBlock;
    const long S = (G + a.C - 1) / a.C;
    const long m = S / R;
    if (m >= 1 && S - m * R <= R / 16) {
      const long C1 = (G + m * R - 1) / (m * R);
      if (C1 <= args.C + 1 && (2L * a.K + 1) * C1 <= kStageMax) {
        a.C = (int)C1;
        a.CS = (int)(m * R);
      }
    }
  }
  // The lag: about the number of requests whose row-stat groups are resident at once, plus two.
  // In ragged batches (verify lengths per request) the rows past k_b are skipped, so the host
  // cannot tell how many requests stream at once; a lag too short makes draw groups wait for
  // their rows while holding slots the stream needs, which measured slower than no lag at all,
  // so there every draw group follows the last row-stat group (L = B).
  const long per_request = (2L * a.K + 1) * a.C;
  long L = (resident_groups(kernel, cache) + per_request - 1) / per_request + 2;
  if (GEN || a.num_draft != nullptr || L > a.B) L = a.B;
  a.L = (int)L;
  // the grid of this C: the row-stat groups, then the draw groups
  const long groups = (long)a.B * (2L * a.K + 1) * a.C + (long)a.B * a.C2;
  if (GEN)
    hipLaunchKernelGGL((sv_verify_ragged_kernel<T, VEC>), dim3((unsigned)groups), dim3(kBlock),
                       0, stream, a);
  else
    hipLaunchKernelGGL((sv_verify_sample<T, VEC>), dim3((unsigned)groups), dim3(kBlock), 0,
                       stream, a);
  return launch_status(GEN ? "sv_verify_ragged" : "sv_verify_sample");
}

template <typename T, bool VEC>
int launch_greedy(const GreedyArgs& a, long groups, hipStream_t stream) {
  hipLaunchKernelGGL((sv_verify_greedy_kernel<T, VEC>), dim3((unsigned)groups), dim3(kBlock), 0,
                     stream, a);
  return launch_status("sv_verify_greedy");
}

// Scratch memory of sv_verify_batch_noalloc: a file-scope device array, one per GPU the library
// runs on, held until the process ends. Host code never passes the array's name to a kernel (on
// the host it is only a stand-in for the symbol): the device address comes from
// hipGetSymbolAddress, once per device with that device current, and is kept here.
constexpr size_t kScratchBytes = (size_t)16 << 20;
constexpr uint32_t kScratchTag = 1;  // the one tag of calls on the scratch (cleared before each)
}  // namespace

static __device__ __align__(256) uint64_t scratch[kScratchBytes / 8];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SV_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(SV_ERR_UNSUPPORTED, "device index above 63");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(SV_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") +
                                  (e != hipSuccess ? hipGetErrorString(e) : "null address"));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SV_OK;
}

}  // namespace

// Error reporting shared with the library's other source files (sv_internal.h).
int sv_internal_fail(int status, const char* msg) { return fail(status, msg); }
void sv_internal_clear_error() { g_last_error.clear(); }

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

}  // extern "C"

namespace {

// sv_verify_batch; with fixed_tag != 0 the call's tag is that value instead of one drawn from the
// call counter (the caller has zero-filled the workspace words the call uses on `stream`).
int verify_batch(const void* target_logits, const void* draft_logits, int dtype, int B, int K,
                 int V, float temperature, const int32_t* draft_tokens, const int32_t* num_draft,
                 const float* uniforms, const float* residual_uniform, int32_t* accepted_len,
                 int32_t* committed, float* target_prob, float* draft_prob, void* workspace,
                 size_t workspace_bytes, void* stream, uint32_t fixed_tag) {
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
  const bool vec = rows_vectorisable(target_logits, draft_logits, dtype, V);
  const Plan p = make_plan(B, K, V);
  if (!plan_supported(p)) return fail(SV_ERR_UNSUPPORTED, "vocabulary too large");
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
  hipStream_t s = static_cast<hipStream_t>(stream);
  // a fresh call tag: words published by earlier calls (or the zeros of a fresh workspace)
  // never pass for this call's
  if (fixed_tag != 0) {
    a.tag = fixed_tag;
  } else {
    st = sv_internal_call_tags(1, workspace, workspace_bytes, s, &a.tag);
    if (st != SV_OK) return st;
  }
  a.stats = reinterpret_cast<uint64_t*>(ws + L.stats);
  a.gath = reinterpret_cast<uint64_t*>(ws + L.gath);
  a.ctot = reinterpret_cast<uint64_t*>(ws + L.ctot);
  a.seg = reinterpret_cast<uint64_t*>(ws + L.seg);
  a.NSmax = p.NSmax;
  a.accepted_len = accepted_len;
  a.committed = committed;
  a.target_prob = target_prob;
  a.draft_prob = draft_prob;
  a.t_start = a.d_start = nullptr;
  a.n_trows = a.n_drows = 0;
  a.temps = nullptr;
  a.NS = segments_per_row(V, dtype, vec, p);
  if (dtype == SV_DTYPE_F32)
    return vec ? launch_sample<float, true, false>(a, s)
               : launch_sample<float, false, false>(a, s);
  return vec ? launch_sample<uint16_t, true, false>(a, s)
             : launch_sample<uint16_t, false, false>(a, s);
}

}  // namespace

extern "C" {

int sv_verify_batch(const void* target_logits, const void* draft_logits, int dtype, int B, int K,
                    int V, float temperature, const int32_t* draft_tokens,
                    const int32_t* num_draft, const float* uniforms,
                    const float* residual_uniform, int32_t* accepted_len, int32_t* committed,
                    float* target_prob, float* draft_prob, void* workspace,
                    size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  return verify_batch(target_logits, draft_logits, dtype, B, K, V, temperature, draft_tokens,
                      num_draft, uniforms, residual_uniform, accepted_len, committed,
                      target_prob, draft_prob, workspace, workspace_bytes, stream, 0u);
}

int sv_verify_batch_noalloc(const void* target_logits, const void* draft_logits, int dtype, int B,
                            int K, int V, float temperature, const int32_t* draft_tokens,
                            const int32_t* num_draft, const float* uniforms,
                            const float* residual_uniform, int32_t* accepted_len,
                            int32_t* committed, float* target_prob, float* draft_prob,
                            void* stream) {
  g_last_error.clear();
  const size_t need = sv_workspace_bytes(B, K, V);  // 0: a shape outside the limits
  if (need == 0)  // sv_verify_batch reports which argument is invalid, before any GPU call
    return sv_verify_batch(target_logits, draft_logits, dtype, B, K, V, temperature,
                           draft_tokens, num_draft, uniforms, residual_uniform, accepted_len,
                           committed, target_prob, draft_prob, nullptr, 0, stream);
  if (need > kScratchBytes)
    return fail(SV_ERR_UNSUPPORTED, "sv_verify_batch_noalloc: this batch needs " +
                                        std::to_string(need) + " bytes of scratch, more than the " +
                                        std::to_string(kScratchBytes) +
                                        " the library holds per GPU; call sv_verify_batch with a "
                                        "workspace instead");
  void* ws = nullptr;
  int st = scratch_of_current_device(&ws);
  if (st != SV_OK) return st;
  // Every call clears the scratch words it uses and hands off under one fixed tag, so that the
  // same launches are correct when a captured call is replayed: nothing depends on the host's
  // call counter. Validation first, so that a rejected call enqueues nothing.
  st = verify_batch(target_logits, draft_logits, dtype, B, K, V, temperature, draft_tokens,
                    num_draft, uniforms, residual_uniform, accepted_len, committed, target_prob,
                    draft_prob, nullptr, 0, stream, kScratchTag);
  if (st != SV_ERR_WORKSPACE) return st == SV_OK ? fail(SV_ERR_HIP, "unreachable") : st;
  g_last_error.clear();
  st = sv_internal_zero_fill(ws, need, static_cast<hipStream_t>(stream));
  if (st != SV_OK) return st;
  return verify_batch(target_logits, draft_logits, dtype, B, K, V, temperature, draft_tokens,
                      num_draft, uniforms, residual_uniform, accepted_len, committed, target_prob,
                      draft_prob, ws, need, stream, kScratchTag);
}

int sv_verify_ragged(const void* target_logits, const void* draft_logits, int dtype, int B,
                     int K, int V, int64_t n_target_rows, int64_t n_draft_rows,
                     const int32_t* target_row_start, const int32_t* draft_row_start,
                     const int32_t* num_draft, const float* temperature,
                     const int32_t* draft_tokens, const float* uniforms,
                     const float* residual_uniform, int32_t* accepted_len, int32_t* committed,
                     float* target_prob, float* draft_prob, void* workspace,
                     size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  int st = check_shape(B, K, V);
  if (st != SV_OK) return st;
  if (dtype != SV_DTYPE_F32 && dtype != SV_DTYPE_BF16)
    return fail(SV_ERR_INVALID_ARG, "dtype must be SV_DTYPE_F32 or SV_DTYPE_BF16");
  if (!target_logits || !target_row_start || !draft_row_start || !num_draft || !temperature ||
      !draft_tokens || !uniforms || !residual_uniform || !accepted_len || !committed ||
      !target_prob)
    return fail(SV_ERR_INVALID_ARG, "a required pointer is NULL");
  if (n_target_rows < 1 || n_draft_rows < 0)
    return fail(SV_ERR_INVALID_ARG, "n_target_rows must be >= 1 and n_draft_rows >= 0");
  if (n_draft_rows > 0 && !draft_logits)
    return fail(SV_ERR_INVALID_ARG, "draft_logits is NULL but n_draft_rows > 0");
  if ((unsigned long long)n_target_rows * (unsigned long long)V > (1ull << 46) ||
      (unsigned long long)n_draft_rows * (unsigned long long)V > (1ull << 46))
    return fail(SV_ERR_UNSUPPORTED, "flat logit arrays too large");
  const Plan p = make_plan(B, K, V);
  if (!plan_supported(p)) return fail(SV_ERR_UNSUPPORTED, "vocabulary too large");
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
  a.draft = n_draft_rows > 0 ? draft_logits : target_logits;  // never read when empty
  a.B = B;
  a.K = K;
  a.V = V;
  a.num_draft = num_draft;
  a.tokens = draft_tokens;
  a.uniforms = uniforms;
  a.residual = residual_uniform;
  a.c32 = 0.0f;  // per request
  a.C = p.C;
  a.C2 = p.C2;
  a.NT = p.NT;
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = sv_internal_call_tags(1, workspace, workspace_bytes, s, &a.tag);
  if (st != SV_OK) return st;
  a.stats = reinterpret_cast<uint64_t*>(ws + L.stats);
  a.gath = reinterpret_cast<uint64_t*>(ws + L.gath);
  a.ctot = reinterpret_cast<uint64_t*>(ws + L.ctot);
  a.seg = reinterpret_cast<uint64_t*>(ws + L.seg);
  a.NSmax = p.NSmax;
  a.accepted_len = accepted_len;
  a.committed = committed;
  a.target_prob = target_prob;
  a.draft_prob = draft_prob;
  a.t_start = target_row_start;
  a.d_start = draft_row_start;
  a.n_trows = (long)n_target_rows;
  a.n_drows = (long)n_draft_rows;
  a.temps = temperature;
  const bool vec = rows_vectorisable(target_logits, a.draft, dtype, V);
  a.NS = segments_per_row(V, dtype, vec, p);
  if (dtype == SV_DTYPE_F32)
    return vec ? launch_sample<float, true, true>(a, s)
               : launch_sample<float, false, true>(a, s);
  return vec ? launch_sample<uint16_t, true, true>(a, s)
             : launch_sample<uint16_t, false, true>(a, s);
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
  const long n_argmax = (long)B * (K + 1) * p.Cg;
  const long groups = n_argmax + B;
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
  a.n_argmax_groups = n_argmax;
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = sv_internal_call_tags(1, workspace, workspace_bytes, s, &a.tag);
  if (st != SV_OK) return st;
  a.gstats = reinterpret_cast<uint64_t*>(ws + L.gstats);
  a.accepted_len = accepted_len;
  a.committed = committed;
  const bool vec = rows_vectorisable(target_logits, nullptr, dtype, V);
  if (dtype == SV_DTYPE_F32)
    return vec ? launch_greedy<float, true>(a, groups, s) : launch_greedy<float, false>(a, groups, s);
  return vec ? launch_greedy<uint16_t, true>(a, groups, s)
             : launch_greedy<uint16_t, false>(a, groups, s);
}

}  // extern "C"
