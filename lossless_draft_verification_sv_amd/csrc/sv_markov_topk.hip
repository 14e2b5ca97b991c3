// Top-K Markov drafting (declared in sv.h): the candidates of every draft position are picked
// from its base logits first, and the Markov correction of a draft block is applied to those
// rows only ("Bringing DSpark to vLLM Metal", Making the draft cheaper; the head itself:
// "Accelerating Large-Model Inference ...", section 3, Markov Head, and the DSpark paper
// review, 4.1).
//
// Four launches per call:
//   topk_chunk   one work-group per (row, chunk of kChunk logits): the row's kc largest logits
//                within the chunk (NaN below every number, ties to the lower index), in index
//                order. All B*K rows at once: the candidates do not depend on the tokens.
//   topk_chunk_exact  the chunks the first pass flagged (many ties at its bound, or fewer than
//                kc numbers): an exact pass over every entry; the others return at once.
//   topk_bias    one work-group per row (b, k): merges the chunk candidates of rows k-1 and k
//                (the kc largest of each, ascending index), then the candidate-to-candidate bias
//                table M_k[i][j] = L[cand_{k-1}[i]] . Rf[cand_k[j]] on MFMA (for k = 0 the one
//                row of the anchor). The token chosen at k-1 is one of cand_{k-1}, so this table
//                holds every bias position k can need, and no position waits for the one before.
//                For every row i of the table it also takes the pick after a previous token in
//                slot i: the best z_j = logit_j + M_k[i][j] (the lowest index on ties).
//   topk_walk    one wave per request: left to right, the slot after prev is row prev's pick,
//                the token is that slot's candidate.
//
// Selection keys are the logits' bits mapped to an unsigned order (NaN lowest); a selection
// keeps the kc largest keys, ties to the earlier entry. A thread owns a contiguous run of
// entries, so thread order is index order. A chunk first bounds its kc-th largest value from
// below by thread maxima, keeps the few entries at or above the bound in LDS and lets one wave
// finish the selection with ballots.

#include <hip/hip_runtime.h>

#include <limits.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "sv.h"
#include "sv_internal.h"

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kMaxCand = 64;                 // kc limit: one MFMA-tiled 64 x 64 bias table
constexpr int kPerThread = 128;               // entries a thread selects over
constexpr int kChunk = kThreads * kPerThread;  // logits per chunk work-group
constexpr int kCompact = 1024;               // chunk entries above the first bound kept in LDS
constexpr int kExactPer = 16;                // chunks one exact-pass work-group looks at
constexpr int kMergeList = 2048;             // chunk candidates a merge selects over in LDS
constexpr int kMaxRank = 256;
constexpr int kRow = kMaxRank + 8;           // LDS row stride of staged factor rows, in bf16

typedef unsigned int v4u32 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float float16_t __attribute__((ext_vector_type(16)));

// Unsigned order of a float: larger keys for larger values, NaN the lowest (key 0).
__device__ __forceinline__ uint32_t order_key(float x) {
  if (x != x) return 0u;
  const uint32_t b = __float_as_uint(x);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Wave primitives on DPP row shifts and row broadcasts (no LDS round trips).
template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp_i32(int x, int identity) {
  return __builtin_amdgcn_update_dpp(identity, x, CTRL, ROWS, 0xf, false);
}
#define TOPK_SCAN_STEPS(STEP) \
  STEP(0x111, 0xf);           \
  STEP(0x112, 0xf);           \
  STEP(0x114, 0xf);           \
  STEP(0x118, 0xf);           \
  STEP(0x142, 0xa);           \
  STEP(0x143, 0xc)

// Inclusive prefix sum over the wave's lanes.
__device__ __forceinline__ int wave_scan(int x) {
#define TOPK_ADD(C, R) x += dpp_i32<C, R>(x, 0)
  TOPK_SCAN_STEPS(TOPK_ADD);
#undef TOPK_ADD
  return x;
}

// Largest value over the wave's lanes (every lane gets it).
__device__ __forceinline__ float wave_max(float x) {
  int v = __float_as_int(x);
#define TOPK_MAX(C, R) \
  v = __float_as_int(fmaxf(__int_as_float(v), __int_as_float(dpp_i32<C, R>(v, __float_as_int(-INFINITY)))))
  TOPK_SCAN_STEPS(TOPK_MAX);
#undef TOPK_MAX
  return __int_as_float(__builtin_amdgcn_readlane(v, 63));
}

// (value, slot) order of a candidate pick: the larger value, then the lower slot.
__device__ __forceinline__ bool pick_better(float z, int i, float best, int bi) {
  return z > best || (z == best && i < bi);
}
// One exchange step of a pick over lanes, inside the vector ALU (DPP, every lane active): CTRL
// 0xB1 and 0x4E swap lanes l ^ 1 and l ^ 2 inside each quad, 0x141 and 0x140 mirror each group
// of 8 and of 16 lanes (after the steps before it each half of the group is uniform).
template <int CTRL>
__device__ __forceinline__ void pick_step(float& best, int& bi) {
  const float b2 =
      __uint_as_float((uint32_t)__builtin_amdgcn_mov_dpp((int)__float_as_uint(best), CTRL, 0xf,
                                                          0xf, false));
  const int i2 = __builtin_amdgcn_mov_dpp(bi, CTRL, 0xf, 0xf, false);
  if (pick_better(b2, i2, best, bi)) {
    best = b2;
    bi = i2;
  }
}

// Smallest and largest value over the wave's lanes (every lane gets them).
__device__ __forceinline__ uint32_t wave_umax(uint32_t v) {
#define TOPK_UMAX1(C, R) v = max(v, (uint32_t)dpp_i32<C, R>((int)v, 0))
  TOPK_SCAN_STEPS(TOPK_UMAX1);
#undef TOPK_UMAX1
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
__device__ __forceinline__ uint32_t wave_umin(uint32_t v) { return ~wave_umax(~v); }

// The q-th largest of a wave's keys, given lo <= it <= hi and count(c) = the number of keys
// >= c (the same in every lane): the largest c with count(c) >= q. Bits above the highest bit
// where lo and hi differ are fixed; below `low` every key has all bits 0 or all bits 1 (keys of
// bf16 logits: low = 16), so one more step settles them. Keys equal to 0 never count (c >= 1).
template <class Count>
__device__ __forceinline__ uint32_t kth_key(uint32_t lo, uint32_t hi, int q, int low,
                                            Count count) {
  if (lo >= hi) return lo;
  const int hb = 31 - __builtin_clz(lo ^ hi);
  uint32_t T = hb == 31 ? 0u : (lo & ~((2u << hb) - 1u));
  for (int bit = hb; bit >= low; --bit) {
    const uint32_t c = T | (1u << bit);
    if (count(c) >= q) T = c;
  }
  if (low > 0) {
    const uint32_t c = T | ((1u << low) - 1u);
    if (count(c) >= q) T = c;
  }
  return T;
}

// Inclusive sum over the work-group (thread order); red holds one int per wave.
__device__ int block_scan(int v, int* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_scan(v);
  __syncthreads();  // earlier readers of red are done
  if (lane == 63) red[wave] = v;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += red[w];
  return before + v;
}

// Largest value over the work-group (every thread gets it).
__device__ uint32_t block_max(uint32_t v, int* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#define TOPK_UMAX(C, R) v = max(v, (uint32_t)dpp_i32<C, R>((int)v, 0))
  TOPK_SCAN_STEPS(TOPK_UMAX);
#undef TOPK_UMAX
  __syncthreads();
  if (lane == 63) red[wave] = (int)v;
  __syncthreads();
  uint32_t m = 0;
  for (int w = 0; w < kWaves; ++w) m = max(m, (uint32_t)red[w]);
  return m;
}

__device__ int block_sum(int v, int* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_scan(v);
  __syncthreads();
  if (lane == 63) red[wave] = v;
  __syncthreads();
  int s = 0;
  for (int w = 0; w < kWaves; ++w) s += red[w];
  return s;
}

template <int CAP>
struct SelShared {
  uint64_t list[CAP];  // (key << 32 | index) of the entries kept, in entry order
  uint32_t bound[kWaves];
  int lanes[kWaves];
  int red[kWaves];
  int n_all;
};

__device__ __forceinline__ uint32_t key_of(uint64_t e) { return (uint32_t)(e >> 32); }

// Wave 0 only: the q-th largest key of list[0 .. n) (q <= n). Up to REG rows of 64 entries are
// held in registers; longer lists are read from LDS at every step.
template <int REG, int CAP>
__device__ uint32_t list_kth(const SelShared<CAP>& sh, int n, int q, int low) {
  const int lane = threadIdx.x & 63, rows = (n + 63) / 64;
  auto at = [&](int i) -> uint32_t {
    return i * 64 + lane < n ? key_of(sh.list[i * 64 + lane]) : 0u;
  };
  uint32_t lo = 0xFFFFFFFFu, hi = 0u;
  for (int i = 0; i < rows; ++i) {
    if (i * 64 + lane < n) {
      const uint32_t k = at(i);
      lo = k < lo ? k : lo;
      hi = k > hi ? k : hi;
    }
  }
  lo = wave_umin(lo);
  hi = wave_umax(hi);
  if (rows <= REG) {  // uniform
    uint32_t x[REG];
#pragma unroll
    for (int i = 0; i < REG; ++i) x[i] = i < rows ? at(i) : 0u;
    return kth_key(lo, hi, q, low, [&](uint32_t c) {
      int cnt = 0;
#pragma unroll
      for (int i = 0; i < REG; ++i) cnt += __popcll(__ballot(x[i] >= c));
      return cnt;
    });
  }
  return kth_key(lo, hi, q, low, [&](uint32_t c) {
    int cnt = 0;
    for (int i = 0; i < rows; ++i) cnt += __popcll(__ballot(at(i) >= c));
    return cnt;
  });
}

// Wave 0 only: the kc largest keys of list[0 .. n) (ties to the earlier entry, n <= CAP;
// kc <= n). emit(slot, entry) for each, slots 0 .. kc-1 in entry order. Returns the kc-th
// largest key.
template <int REG, int CAP, class Emit>
__device__ uint32_t list_select(const SelShared<CAP>& sh, int n, int kc, int low, Emit emit) {
  const int lane = threadIdx.x & 63;
  const int rows = (n + 63) / 64;
  const uint64_t below = (1ull << lane) - 1ull;
  const uint32_t T = list_kth<REG>(sh, n, kc, low);
  int gt_all = 0;
  for (int i = 0; i < rows; ++i)
    gt_all += __popcll(__ballot(i * 64 + lane < n && key_of(sh.list[i * 64 + lane]) > T));
  const int need = kc - gt_all;  // keys equal to T to take, earliest first
  int eq_seen = 0, taken = 0;
  for (int i = 0; i < rows; ++i) {
    const bool valid = i * 64 + lane < n;
    const uint64_t e = valid ? sh.list[i * 64 + lane] : 0ull;
    const bool gt = valid && key_of(e) > T, eq = valid && key_of(e) == T;
    const uint64_t beq = __ballot(eq);
    const bool take = gt || (eq && eq_seen + __popcll(beq & below) < need);
    const uint64_t bt = __ballot(take);
    if (take) emit(taken + __popcll(bt & below), e);
    eq_seen += __popcll(beq);
    taken += __popcll(bt);
  }
  return T;
}

// Every thread: the kc largest of the work-group's keys, thread t owning entries t*N .. t*N+N-1
// (key(e) its e-th; ties to the earlier entry). emit(slot, e) for each of this thread's chosen
// entries. The slow path: every entry is visited once per bit.
template <int N, int CAP, class Key, class Emit>
__device__ __forceinline__ uint32_t register_select(Key key, int kc, SelShared<CAP>& sh,
                                                    Emit emit) {
  uint32_t T = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t c = T | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int e = 0; e < N; ++e) cnt += key(e) >= c;
    if (block_sum(cnt, sh.red) >= kc) T = c;
  }
  int n_gt = 0, n_eq = 0;
#pragma unroll
  for (int e = 0; e < N; ++e) {
    const uint32_t x = key(e);
    n_gt += x > T;
    n_eq += x == T;
  }
  const int gt_all = block_sum(n_gt, sh.red);
  const int need0 = kc - gt_all - (block_scan(n_eq, sh.red) - n_eq);
  int need = need0, n_take = 0;
#pragma unroll
  for (int e = 0; e < N; ++e) {
    const uint32_t x = key(e);
    n_take += x > T || (x == T && need > 0);
    need -= x == T;
  }
  int slot = block_scan(n_take, sh.red) - n_take;
  need = need0;
#pragma unroll
  for (int e = 0; e < N; ++e) {
    const uint32_t x = key(e);
    if (x > T || (x == T && need > 0)) emit(slot++, e);
    need -= x == T;
  }
  return T;
}

// Loads thread tid's kPerThread logits of chunk c of a row as raw 32-bit words (entries past V
// read the row's first logit; the caller masks them). VEC: 16-byte rows, V a multiple of the
// vector, so a vector is all inside the row or all outside.
template <typename T, bool VEC>
__device__ __forceinline__ void load_chunk(uint32_t (&raw)[kPerThread * sizeof(T) / 4],
                                           const T* __restrict__ row, int V, int v0) {
  constexpr int kWords = kPerThread * (int)sizeof(T) / 4;
  if constexpr (VEC) {
    constexpr int kVec = 16 / (int)sizeof(T);
#pragma unroll
    for (int w = 0; w < kWords / 4; ++w) {
      const int v = v0 + w * kVec;
      const v4u32 x = *reinterpret_cast<const v4u32*>(row + (v < V ? v : 0));
      raw[4 * w] = x.x;
      raw[4 * w + 1] = x.y;
      raw[4 * w + 2] = x.z;
      raw[4 * w + 3] = x.w;
    }
  } else {
#pragma unroll
    for (int w = 0; w < kWords; ++w) {
      if constexpr (sizeof(T) == 4) {
        const int v = v0 + w;
        raw[w] = __float_as_uint(row[v < V ? v : 0]);
      } else {
        const int v1 = v0 + 2 * w, v2 = v1 + 1;
        raw[w] = (uint32_t)row[v1 < V ? v1 : 0] | ((uint32_t)row[v2 < V ? v2 : 0] << 16);
      }
    }
  }
}

template <typename T>
__device__ __forceinline__ float raw_value(const uint32_t (&raw)[kPerThread * sizeof(T) / 4],
                                           int e) {
  if constexpr (sizeof(T) == 4) return __uint_as_float(raw[e]);
  else return __uint_as_float((e & 1) ? (raw[e / 2] & 0xffff0000u) : (raw[e / 2] << 16));
}

// Chunk c of row r: its kc largest logits as (key << 32 | index) words, in index order, when a
// first bound leaves few entries; otherwise flags the chunk for topk_chunk_exact.
template <typename T, bool VEC>
__global__ __launch_bounds__(kThreads) void topk_chunk(const T* __restrict__ base, int V,
                                                       int nchunk, int kc, int q_thr,
                                                       uint64_t* __restrict__ out,
                                                       uint32_t* __restrict__ thr,
                                                       int32_t* __restrict__ flag) {
  __shared__ SelShared<kCompact> sh;
  const int r = blockIdx.x, c = blockIdx.y, tid = threadIdx.x, lane = tid & 63;
  const int wave = tid >> 6;
  const T* row = base + (size_t)r * V;
  const int v0 = c * kChunk + tid * kPerThread;
  uint32_t raw[kPerThread * sizeof(T) / 4];
  load_chunk<T, VEC>(raw, row, V, v0);
  if (v0 + kPerThread > V) {  // entries past the row become NaN, which no step below keeps
#pragma unroll
    for (int w = 0; w < kPerThread * (int)sizeof(T) / 4; ++w) {
      if constexpr (sizeof(T) == 4) {
        raw[w] = v0 + w < V ? raw[w] : 0x7FC00000u;
      } else {
        const uint32_t lo = v0 + 2 * w < V ? (raw[w] & 0xffffu) : 0x7FC0u;
        const uint32_t hi = v0 + 2 * w + 1 < V ? (raw[w] >> 16) : 0x7FC0u;
        raw[w] = lo | (hi << 16);
      }
    }
  }
  // 1. a first bound from the thread maxima (over numbers inside the row). Wave w has n_w
  //    threads with a number; it takes q_w = ceil(kc n_w / N) of them (N = the sum, so the
  //    q_w add up to at least kc and none exceeds n_w) and finds its q_w-th largest maximum;
  //    each such thread holds an entry at or above it, so the smallest of these bounds leaves
  //    at least kc entries at or above it. With N < kc there is no bound.
  float mx = __uint_as_float(0x7FC00000u);  // fmaxf skips NaN: mx stays NaN only without numbers
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) mx = fmaxf(mx, raw_value<T>(raw, e));
  const bool has = mx == mx;
  const uint32_t mkey = has ? order_key(mx) : 0u;
  const int wave_lanes = (int)__popcll(__ballot(has));  // the whole wave votes
  if (lane == 0) sh.lanes[wave] = wave_lanes;
  __syncthreads();
  int n_lanes = 0;
  for (int w = 0; w < kWaves; ++w) n_lanes += sh.lanes[w];
  const int q = n_lanes >= kc ? (kc * sh.lanes[wave] + n_lanes - 1) / n_lanes : 0;
  constexpr int kLow = sizeof(T) == 2 ? 16 : 0;  // bf16 keys: low 16 bits all 0 or all 1
  uint32_t pre = 0xFFFFFFFFu;  // a wave that takes no thread sets no bound
  if (q > 0) {
    const uint32_t lo = wave_umin(has ? mkey : 0xFFFFFFFFu), hi = wave_umax(mkey);
    pre = kth_key(lo, hi, q, kLow, [&](uint32_t cc) { return (int)__popcll(__ballot(mkey >= cc)); });
  }
  if (lane == 0) sh.bound[wave] = pre;
  __syncthreads();
  uint32_t t0 = sh.bound[0];
  for (int w = 1; w < kWaves; ++w) t0 = sh.bound[w] < t0 ? sh.bound[w] : t0;
  if (n_lanes < kc) t0 = 0u;
  // 2. the entries at or above the bound (a value compare: it may add a -0 beside +0, which
  //    changes nothing), kept in LDS when few
  int n_ge = 0;
  const float f0 = key_value(t0);
  if (t0 != 0u) {
#pragma unroll
    for (int w = 0; w < kPerThread * (int)sizeof(T) / 4; ++w) {
      uint32_t word[1] = {raw[w]};
      asm volatile("" : "+v"(word[0]));  // unpack afresh here: no unpacked copies stay live
      constexpr int kPer = 4 / (int)sizeof(T);
#pragma unroll
      for (int x = 0; x < kPer; ++x) {
        const float f = sizeof(T) == 4 ? __uint_as_float(word[0])
                                       : __uint_as_float(x ? (word[0] & 0xffff0000u) : (word[0] << 16));
        n_ge += f >= f0;  // NaN: false
      }
    }
  }
  const int incl = block_scan(n_ge, sh.red);
  if (tid == kThreads - 1) sh.n_all = incl;
  __syncthreads();
  const int n_all = sh.n_all;
  const bool fast = t0 != 0u && n_all <= kCompact;
  if (tid == 0) flag[(size_t)r * nchunk + c] = fast ? 0 : 1;
  if (!fast) return;  // uniform: ties at the bound, or too few numbers
  int at = incl - n_ge;
#pragma unroll
  for (int w = 0; w < kPerThread * (int)sizeof(T) / 4; ++w) {
    uint32_t word = raw[w];
    asm volatile("" : "+v"(word));
    constexpr int kPer = 4 / (int)sizeof(T);
#pragma unroll
    for (int x = 0; x < kPer; ++x) {
      const float f = sizeof(T) == 4 ? __uint_as_float(word)
                                     : __uint_as_float(x ? (word & 0xffff0000u) : (word << 16));
      if (f >= f0) sh.list[at++] = ((uint64_t)order_key(f) << 32) | (uint32_t)(v0 + kPer * w + x);
    }
  }
  __syncthreads();
  uint64_t* dst = out + ((size_t)r * nchunk + c) * kMaxCand;
  if (wave == 0) {  // the two selections read the list only: one wave each, side by side
    list_select<4>(sh, n_all, kc, kLow, [&](int slot, uint64_t e) { dst[slot] = e; });
  } else if (wave == 1) {
    const uint32_t t = list_kth<4>(sh, n_all, q_thr, kLow);
    if (lane == 0) thr[(size_t)r * nchunk + c] = t;
  }
}

// The chunks topk_chunk flagged: an exact pass over every entry (every key visited once per
// bit of the threshold). Work-group g looks at chunks g * kExactPer .. + kExactPer - 1
// (row-major over rows and chunks) and returns at once when none is flagged.
template <typename T, bool VEC>
__global__ __launch_bounds__(kThreads) void topk_chunk_exact(const T* __restrict__ base, int V,
                                                             int nchunk, int kc, int q_thr,
                                                             int total,
                                                             uint64_t* __restrict__ out,
                                                             uint32_t* __restrict__ thr,
                                                             const int32_t* __restrict__ flag) {
  __shared__ SelShared<64> sh;
  __shared__ int todo[kThreads];
  __shared__ int n_todo;
  const int tid = threadIdx.x, id = (int)blockIdx.x * kExactPer + tid;
  const bool mine = tid < kExactPer && id < total && flag[id] != 0;
  const int before = block_scan(mine ? 1 : 0, sh.red);
  if (mine) todo[before - 1] = id;
  if (tid == kThreads - 1) n_todo = before;
  __syncthreads();
  for (int j = 0; j < n_todo; ++j) {  // uniform
    const int ch = todo[j], r = ch / nchunk, c = ch % nchunk;
    const int v0 = c * kChunk + tid * kPerThread;
    uint32_t raw[kPerThread * sizeof(T) / 4];
    load_chunk<T, VEC>(raw, base + (size_t)r * V, V, v0);
    uint32_t key[kPerThread];
#pragma unroll
    for (int e = 0; e < kPerThread; ++e)
      key[e] = v0 + e < V ? order_key(raw_value<T>(raw, e)) : 0u;
    uint64_t* dst = out + (size_t)ch * kMaxCand;
    const uint32_t t = register_select<kPerThread>([&](int e) { return key[e]; }, q_thr, sh,
                                                   [&](int, int) {});
    register_select<kPerThread>([&](int e) { return key[e]; }, kc, sh, [&](int slot, int e) {
      dst[slot] = ((uint64_t)key[e] << 32) | (uint32_t)(v0 + e);
    });
    if (tid == 0) thr[ch] = t;
    __syncthreads();
  }
}

// Rows r - 1 (when prev) and r: the kc largest of each row's chunk candidates (entries in index
// order; n <= kMergeList), emitted by emit0 / emit1 (slot, entry), wave 0 selecting row r - 1
// and wave 1 row r. Every thread calls it. thr[c] is chunk c's q-th largest key, q =
// ceil(kc / nchunk): a row's chunks together hold at least kc keys at or above the smallest of
// these, which so bounds the row's kc-th largest key from below; only the entries at or above
// it are kept for the selection.
template <class Emit0, class Emit1>
__device__ void merge_rows(const uint64_t* __restrict__ chunks, const uint32_t* __restrict__ thr,
                           int r, bool prev, int nchunk, int kc, int low,
                           SelShared<kMergeList> (&m)[2], Emit0 emit0, Emit1 emit1) {
  const int n = nchunk * kc, tid = threadIdx.x;
  constexpr int kPer = kMergeList / kThreads;
  uint32_t t0[2] = {0xFFFFFFFFu, 0xFFFFFFFFu};
  for (int c = tid; c < nchunk; c += kThreads) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if (j == 1 || prev) {
        const uint32_t t = thr[(size_t)(r - 1 + j) * nchunk + c];
        t0[j] = t < t0[j] ? t : t0[j];
      }
    }
  }
  t0[0] = ~block_max(~t0[0], m[0].red);  // the smallest
  t0[1] = ~block_max(~t0[1], m[1].red);
  const int per = (n + kThreads - 1) / kThreads;  // contiguous entries per thread, <= kPer
  uint64_t w[2][kPer];
  int n_ge[2] = {0, 0};
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const int i = tid * per + e;
      const bool ok = (j == 1 || prev) && e < per && i < n;
      w[j][e] = ok ? chunks[((size_t)(r - 1 + j) * nchunk + i / kc) * kMaxCand + i % kc] : 0ull;
      n_ge[j] += ok && key_of(w[j][e]) >= t0[j];
    }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int incl = block_scan(n_ge[j], m[j].red);
    if (tid == kThreads - 1) m[j].n_all = incl;
    int at = incl - n_ge[j];
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const int i = tid * per + e;
      if ((j == 1 || prev) && e < per && i < n && key_of(w[j][e]) >= t0[j]) m[j].list[at++] = w[j][e];
    }
  }
  __syncthreads();
  const int wave = tid >> 6;
  if (wave == 0 && prev) list_select<4>(m[0], m[0].n_all, kc, low, emit0);
  if (wave == 1) list_select<4>(m[1], m[1].n_all, kc, low, emit1);
  __syncthreads();
}

// Row (b, k): merges the candidates of rows k-1 and k, writes row k's (cand, val, and the
// caller's candidates output), then table[i][j] = L[p_i] . Rf[cand_k[j]], p = cand_{k-1}
// (k > 0) or the anchor alone (k = 0, row 0 only); rows and columns past kc, and an anchor
// outside [0, V), are zero.
__global__ __launch_bounds__(kThreads) void topk_bias(
    const uint64_t* __restrict__ chunks, const uint32_t* __restrict__ thr, int nchunk, int K,
    int V, int kc, int low,
    const uint16_t* __restrict__ left, const uint16_t* __restrict__ right, int R,
    const int32_t* __restrict__ anchor, int32_t* __restrict__ cand, float* __restrict__ cand_val,
    int32_t* __restrict__ cand_out, float* __restrict__ table, int32_t* __restrict__ next) {
  // the merge lists and the staged factor rows are used one after the other
  __shared__ union __attribute__((aligned(16))) {
    SelShared<kMergeList> m[2];
    struct {
      uint16_t a[kMaxCand][kRow];
      uint16_t b[kMaxCand][kRow];
    } f;
  } lds;
  __shared__ int32_t cidx[2][kMaxCand];  // candidates of rows k-1 and k, -1 past kc
  __shared__ float cval[kMaxCand];        // logits of row k's candidates
  __shared__ float s_pv[kMaxCand][4];      // per table row, the pick over each 16 columns
  __shared__ int s_pj[kMaxCand][4];
  uint16_t (*sa)[kRow] = lds.f.a;
  uint16_t (*sb)[kRow] = lds.f.b;
  const int r = blockIdx.x, b = r / K, k = r % K;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid < 2 * kMaxCand) cidx[tid / kMaxCand][tid % kMaxCand] = -1;
  __syncthreads();
  merge_rows(
      chunks, thr, r, k > 0, nchunk, kc, low, lds.m,
      [&](int slot, uint64_t e) { cidx[0][slot] = (int32_t)(uint32_t)e; },
      [&](int slot, uint64_t e) {
        const int32_t v = (int32_t)(uint32_t)e;
        cidx[1][slot] = v;
        cand[(size_t)r * kMaxCand + slot] = v;
        cand_val[(size_t)r * kMaxCand + slot] = key_value(key_of(e));
        cval[slot] = key_value(key_of(e));
        if (cand_out != nullptr) cand_out[(size_t)r * kc + slot] = v;
      });
  // stage: thread covers rows tid / 32 + 8 u, word tid % 32; every load in flight first
  const int nw = R / 8, sw = tid & 31;
  const int wd = sw < nw ? sw : nw - 1;
  const int pa0 = (k == 0 && anchor != nullptr) ? anchor[b] : -1;
  v4u32 xa[kMaxCand / 8], xb[kMaxCand / 8];
  bool oka[kMaxCand / 8], okb[kMaxCand / 8];
#pragma unroll
  for (int u = 0; u < kMaxCand / 8; ++u) {
    const int i = (tid >> 5) + 8 * u;
    const int pa = k > 0 ? cidx[0][i] : (i == 0 ? pa0 : -1);
    const int pb = cidx[1][i];
    oka[u] = pa >= 0 && pa < V && sw < nw;
    okb[u] = pb >= 0 && pb < V && sw < nw;
    xa[u] = reinterpret_cast<const v4u32*>(left + (size_t)(oka[u] ? pa : 0) * R)[wd];
    xb[u] = reinterpret_cast<const v4u32*>(right + (size_t)(okb[u] ? pb : 0) * R)[wd];
  }
#pragma unroll
  for (int u = 0; u < kMaxCand / 8; ++u) {
    const int i = (tid >> 5) + 8 * u;
    *reinterpret_cast<v4u32*>(&sa[i][8 * sw]) = oka[u] ? xa[u] : v4u32{0u, 0u, 0u, 0u};
    *reinterpret_cast<v4u32*>(&sb[i][8 * sw]) = okb[u] ? xb[u] : v4u32{0u, 0u, 0u, 0u};
  }
  __syncthreads();
  // wave w: the 32x32 block (rows 32 (w / 2), columns 32 (w % 2)) over R / 16 steps
  const int i0 = 32 * (wave >> 1), j0 = 32 * (wave & 1), h = lane >> 5, c = lane & 31;
  float16_t acc = {};
  for (int t = 0; t < R / 16; ++t) {
    const v4u32 a = *reinterpret_cast<const v4u32*>(&sa[i0 + c][16 * t + 8 * h]);
    const v4u32 bq = *reinterpret_cast<const v4u32*>(&sb[j0 + c][16 * t + 8 * h]);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, bq), acc, 0, 0, 0);
  }
  // register i of lane (h, c) holds row 8 (i / 4) + 4 h + i % 4, column c of the block
  float* dst = table + (size_t)r * kMaxCand * kMaxCand;
#pragma unroll
  for (int i = 0; i < 16; ++i)
    dst[(size_t)(i0 + 8 * (i / 4) + 4 * h + (i % 4)) * kMaxCand + j0 + c] = acc[i];
  // The walk's choice after every previous slot: for table row i, the slot j < kc with the
  // largest logit_j + M[i][j] (NaN never wins; among equals the lowest slot, the lowest
  // vocabulary index), as the walk takes it after a previous token in slot i. Each row of 16
  // lanes picks over its 16 columns on DPP; the four picks of a table row meet in LDS.
  {
    const int j = j0 + c;
    const float cv = j < kc ? cval[j] : 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float z = cv + acc[i];
      float pv = (j < kc && z == z) ? z : -INFINITY;
      int pj = j;
      pick_step<0xB1>(pv, pj);
      pick_step<0x4E>(pv, pj);
      pick_step<0x141>(pv, pj);
      pick_step<0x140>(pv, pj);
      if ((c & 15) == 15) {
        const int row = i0 + 8 * (i / 4) + 4 * h + (i % 4);
        s_pv[row][2 * (wave & 1) + (c >> 4)] = pv;
        s_pj[row][2 * (wave & 1) + (c >> 4)] = pj;
      }
    }
  }
  __syncthreads();
  if (tid < kMaxCand) {
    float pv = s_pv[tid][0];
    int pj = s_pj[tid][0];
#pragma unroll
    for (int q = 1; q < 4; ++q)
      if (pick_better(s_pv[tid][q], s_pj[tid][q], pv, pj)) {
        pv = s_pv[tid][q];
        pj = s_pj[tid][q];
      }
    next[(size_t)r * kMaxCand + tid] = pj;
  }
}

// Request b, left to right: the token after previous slot prev is the candidate in slot
// next_k[prev] (prev = row 0 at k = 0), the pick topk_bias made over z_j = logit_j +
// table_k[prev][j]. One wave: the next-slot lists of kWalkBlock positions at a time are loaded
// together (lane i holds entry i), and the walk chases them with readlane. The candidates' logits
// on the path (z of the chosen row) are read from the tables only when asked for.
constexpr int kWalkBlock = 8;

__global__ __launch_bounds__(64) void topk_walk(const int32_t* __restrict__ cand,
                                                const float* __restrict__ cand_val,
                                                const float* __restrict__ table,
                                                const int32_t* __restrict__ next, int K, int kc,
                                                int32_t* __restrict__ tokens,
                                                float* __restrict__ cand_logits) {
  const int b = blockIdx.x, lane = threadIdx.x & 63;
  int prev = 0;  // slot of the previous token among the previous position's candidates
  for (int k0 = 0; k0 < K; k0 += kWalkBlock) {
    const int nk = K - k0 < kWalkBlock ? K - k0 : kWalkBlock;
    int nx[kWalkBlock];
    int32_t idx[kWalkBlock];
#pragma unroll
    for (int kk = 0; kk < kWalkBlock; ++kk) {
      const size_t rk = ((size_t)b * K + k0 + (kk < nk ? kk : 0)) * kMaxCand + lane;
      nx[kk] = next[rk];
      idx[kk] = cand[rk];
    }
    int rows[kWalkBlock];
#pragma unroll
    for (int kk = 0; kk < kWalkBlock; ++kk) {
      if (kk < nk) {  // uniform
        const int k = k0 + kk;
        const int row = k == 0 ? 0 : prev;
        rows[kk] = row;
        prev = __builtin_amdgcn_readlane(nx[kk], row);
        const int tok = __builtin_amdgcn_readlane(idx[kk], prev);
        if (lane == 0) tokens[(size_t)b * K + k] = tok;
      }
    }
    if (cand_logits != nullptr && lane < kc) {
      float z[kWalkBlock];
#pragma unroll
      for (int kk = 0; kk < kWalkBlock; ++kk) {
        const size_t rk = (size_t)b * K + k0 + (kk < nk ? kk : 0);
        z[kk] = cand_val[rk * kMaxCand + lane] +
                table[(rk * kMaxCand + (kk < nk ? rows[kk] : 0)) * kMaxCand + lane];
      }
#pragma unroll
      for (int kk = 0; kk < kWalkBlock; ++kk)
        if (kk < nk) cand_logits[((size_t)b * K + k0 + kk) * kc + lane] = z[kk];
    }
  }
}

bool aligned16(const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; }

int chunks_of(int V) { return (V + kChunk - 1) / kChunk; }

struct TopkWorkspace {
  size_t chunks, thr, flag, cand, val, table, next, total;
};

TopkWorkspace topk_layout(int B, int K, int V) {
  TopkWorkspace w;
  const size_t rows = (size_t)B * K;
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  w.chunks = 0;
  w.thr = up(w.chunks + rows * chunks_of(V) * kMaxCand * sizeof(uint64_t));
  w.flag = up(w.thr + rows * chunks_of(V) * sizeof(uint32_t));
  w.cand = up(w.flag + rows * chunks_of(V) * sizeof(int32_t));
  w.val = up(w.cand + rows * kMaxCand * sizeof(int32_t));
  w.table = up(w.val + rows * kMaxCand * sizeof(float));
  w.next = up(w.table + rows * kMaxCand * kMaxCand * sizeof(float));
  w.total = up(w.next + rows * kMaxCand * sizeof(int32_t));
  return w;
}

}  // namespace

extern "C" size_t sv_markov_topk_workspace_bytes(int B, int K, int V) {
  if (B < 1 || K < 1 || V < 1) return 0;
  return topk_layout(B, K, V).total;
}

extern "C" int sv_markov_topk(const void* base_logits, int dtype, int B, int K, int V,
                              const uint16_t* left_factor, const uint16_t* right_factor, int R,
                              int kc, const int32_t* anchor, int32_t* draft_tokens,
                              int32_t* candidates, float* cand_logits, void* workspace,
                              size_t workspace_bytes, void* stream) {
  sv_internal_clear_error();
  if (B < 1 || B > (1 << 16) || K < 1 || K > 64 || V < 1 || V > (1 << 26))
    return sv_internal_fail(SV_ERR_INVALID_ARG, "need 1 <= B <= 65536, 1 <= K <= 64, 1 <= V <= 2^26");
  if (dtype != SV_DTYPE_F32 && dtype != SV_DTYPE_BF16)
    return sv_internal_fail(SV_ERR_INVALID_ARG, "dtype must be SV_DTYPE_F32 or SV_DTYPE_BF16");
  if (R < 16 || R > kMaxRank || R % 16 != 0)
    return sv_internal_fail(SV_ERR_INVALID_ARG, "rank R must be a multiple of 16 in [16, 256]");
  if (kc < 1 || kc > kMaxCand || kc > V)
    return sv_internal_fail(SV_ERR_INVALID_ARG, "need 1 <= kc <= min(64, V)");
  if ((long)chunks_of(V) * kc > kMergeList)
    return sv_internal_fail(SV_ERR_UNSUPPORTED, "vocabulary too large for this candidate count");
  if (!base_logits || !left_factor || !right_factor || !draft_tokens)
    return sv_internal_fail(SV_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!aligned16(left_factor) || !aligned16(right_factor))
    return sv_internal_fail(SV_ERR_INVALID_ARG, "factors must be 16-byte aligned");
  const TopkWorkspace w = topk_layout(B, K, V);
  if (!workspace || workspace_bytes < w.total || reinterpret_cast<uintptr_t>(workspace) % 256)
    return sv_internal_fail(SV_ERR_WORKSPACE, "workspace missing, too small or not 256-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  sv_internal_untagged_use(workspace);  // the tables below are untagged words
  uint64_t* chunks = reinterpret_cast<uint64_t*>(ws + w.chunks);
  int32_t* flag = reinterpret_cast<int32_t*>(ws + w.flag);
  uint32_t* thr = reinterpret_cast<uint32_t*>(ws + w.thr);
  int32_t* cand = reinterpret_cast<int32_t*>(ws + w.cand);
  float* val = reinterpret_cast<float*>(ws + w.val);
  float* table = reinterpret_cast<float*>(ws + w.table);
  int32_t* next = reinterpret_cast<int32_t*>(ws + w.next);
  const int nchunk = chunks_of(V), rows = B * K;
  const size_t es = dtype == SV_DTYPE_F32 ? 4 : 2;
  const bool vec = aligned16(base_logits) && ((size_t)V * es) % 16 == 0;
  const dim3 g1(rows, nchunk);
  auto chunk_pass = [&](auto tag, auto vec_tag) {
    using T = decltype(tag);
    constexpr bool kVecRows = decltype(vec_tag)::value;
    const T* bp = static_cast<const T*>(base_logits);
    const int q_thr = (kc + nchunk - 1) / nchunk;
    hipLaunchKernelGGL((topk_chunk<T, kVecRows>), g1, dim3(kThreads), 0, s, bp, V, nchunk, kc,
                       q_thr, chunks, thr, flag);
    const int total = rows * nchunk;
    hipLaunchKernelGGL((topk_chunk_exact<T, kVecRows>), dim3((total + kExactPer - 1) / kExactPer),
                       dim3(kThreads), 0, s, bp, V, nchunk, kc, q_thr, total, chunks, thr, flag);
  };
  if (dtype == SV_DTYPE_F32) {
    if (vec) chunk_pass(float{}, std::true_type{});
    else chunk_pass(float{}, std::false_type{});
  } else {
    if (vec) chunk_pass(uint16_t{}, std::true_type{});
    else chunk_pass(uint16_t{}, std::false_type{});
  }
  hipLaunchKernelGGL(topk_bias, dim3(rows), dim3(kThreads), 0, s, chunks, thr, nchunk, K, V, kc,
                     dtype == SV_DTYPE_BF16 ? 16 : 0,
                     left_factor, right_factor, R, anchor, cand, val, candidates, table, next);
  hipLaunchKernelGGL(topk_walk, dim3(B), dim3(64), 0, s, cand, val, table, next, K, kc,
                     draft_tokens, cand_logits);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return sv_internal_fail(SV_ERR_HIP, hipGetErrorString(e));
  return SV_OK;
}
