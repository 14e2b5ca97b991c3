// Markov-head correction of a parallel draft block (declared in sv.h): left to right over the K
// positions, position k's base logits get the low-rank bias of the token chosen at k-1 (the
// anchor at k = 0), bias[v] = sum_j L[prev][j] * Rf[v][j], and the position's token is the
// argmax of the corrected logits ("Accelerating Large-Model Inference ...", section 3, Markov
// Head; the DSpark paper review, 4.1).
//
// Per position, two launches:
//   markov_bias_tile: work-group (vocabulary tile of 128, request block of 64); the bias block
//     [64 requests x 128 tokens] = L[prev rows] x Rf[tile rows]^T is a dense contraction over
//     the rank R, done on MFMA (v_mfma_f32_32x32x8_bf16: each wave two 32x32 blocks, bf16 in,
//     fp32 accumulate). Its epilogue adds the base logits, writes the corrected logits (the
//     block's draft logits) and the tile's argmax per request (value, index) to the workspace.
//   markov_finish: one work-group per request reduces the tile argmaxes (lowest index on ties)
//     to the position's token, which the next position's launch reads as its previous token.
// The rank index is permuted identically in both operands (each lane reads 16 contiguous bytes
// of its factor row per pair of MFMA steps); the contraction sums over all of it.

#include <hip/hip_runtime.h>

#include <float.h>
#include <limits.h>
#include <math.h>
#include <stdint.h>

#include <atomic>

#include "sv.h"
#include "sv_internal.h"

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kReqBlock = 64;            // requests per work-group: two 32-row MFMA blocks
constexpr int kTileV = 32 * kWaves;      // vocabulary entries per work-group: 32 per wave
constexpr int kRankChunk = 256;          // rank indices per pass (one pass at the usual rank)
constexpr int kPairs = kRankChunk / 16;  // pairs of MFMA steps per pass
constexpr int kARow = kRankChunk + 8;    // LDS row stride of the staged left rows, in bf16
constexpr int kMaxRank = 1024;
constexpr int kFinishLoads = 8;          // partials each finishing thread has in flight

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float float16_t __attribute__((ext_vector_type(16)));
typedef unsigned int v4u32 __attribute__((ext_vector_type(4)));

template <typename T>
struct Logit;
template <>
struct Logit<float> {
  __device__ static float get(float x) { return x; }
  __device__ static void put(float* p, float x) { *p = x; }
  __device__ static float stored(float x) { return x; }  // the value put() leaves
};
template <>
struct Logit<uint16_t> {
  __device__ static float get(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }
  __device__ static void put(uint16_t* p, float x) {  // round to nearest, ties to even
    const uint32_t b = __float_as_uint(x);
    *p = (x != x) ? (uint16_t)0x7FC0 : (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
  }
  // the value put() (and the vector stores' conversion) leaves, as a float
  __device__ static float stored(float x) { return (float)(__bf16)x; }
};

__device__ __forceinline__ short4_t lo4(v4u32 v) {
  short4_t s;
  s[0] = (short)(v.x & 0xffff); s[1] = (short)(v.x >> 16);
  s[2] = (short)(v.y & 0xffff); s[3] = (short)(v.y >> 16);
  return s;
}
__device__ __forceinline__ short4_t hi4(v4u32 v) {
  short4_t s;
  s[0] = (short)(v.z & 0xffff); s[1] = (short)(v.z >> 16);
  s[2] = (short)(v.w & 0xffff); s[3] = (short)(v.w >> 16);
  return s;
}

// (value, index) order of the argmax: larger value first, then the lower index.
__device__ __forceinline__ bool better(float z, int i, float best, int bi) {
  return z > best || (z == best && i < bi);
}

// Exchanges inside the vector ALU (DPP, every lane of the wave active): the value of lane l ^ 1
// and of lane l ^ 2 (quad permutes), and of the mirror lane inside each group of 8 and of 16.
// After the quad steps every quad holds one value, so the mirror in 8 brings the other quad's;
// after that the mirror in 16 brings the other group of 8's.
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;
template <int CTRL>
__device__ __forceinline__ float dpp_xchg_f32(float x) {
  return __uint_as_float(
      (uint32_t)__builtin_amdgcn_mov_dpp((int)__float_as_uint(x), CTRL, 0xf, 0xf, false));
}
template <int CTRL>
__device__ __forceinline__ void argmax_step(float& best, int& bi) {
  const float b2 = dpp_xchg_f32<CTRL>(best);
  const int i2 = __builtin_amdgcn_mov_dpp(bi, CTRL, 0xf, 0xf, false);
  if (better(b2, i2, best, bi)) {
    best = b2;
    bi = i2;
  }
}
// The wave's argmax, (largest value, lowest index among equals), in every lane: within rows of
// 16 on DPP, then the four rows' results (lanes 0, 16, 32, 48) read out and combined.
__device__ __forceinline__ void wave_argmax(float& best, int& bi) {
  argmax_step<kDppXor1>(best, bi);
  argmax_step<kDppXor2>(best, bi);
  argmax_step<kDppHalfMirror>(best, bi);
  argmax_step<kDppMirror>(best, bi);
  float rb = __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(best), 0));
  int ri = __builtin_amdgcn_readlane(bi, 0);
#pragma unroll
  for (int r = 1; r < 4; ++r) {
    const float b2 =
        __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(best), 16 * r));
    const int i2 = __builtin_amdgcn_readlane(bi, 16 * r);
    if (better(b2, i2, rb, ri)) {
      rb = b2;
      ri = i2;
    }
  }
  best = rb;
  bi = ri;
}

// Work-group g of a position covers vocabulary tile g / nrb and request block g % nrb; the
// launch index is spread so that the work-groups of one XCD (launch index mod 8) take a
// contiguous range of g, and so the request blocks of a tile share that XCD's L2.
template <typename T>
__global__ __launch_bounds__(kThreads) void markov_bias_tile(
    const T* __restrict__ base, T* __restrict__ out, int B, int K, int V, int k,
    const uint16_t* __restrict__ left, const uint16_t* __restrict__ right, int R,
    const int32_t* __restrict__ prev_tok, int prev_stride, uint64_t* __restrict__ part, int ntile,
    int nrb) {
  __shared__ union __attribute__((aligned(16))) {
    uint16_t a[kReqBlock][kARow];        // left-factor rows of the block's previous tokens
    float z[kReqBlock][kTileV + 1];      // corrected logits, for the tile argmax
  } sm;
  const int n = ntile * nrb, per = (n + 7) / 8;
  const int g = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
  if (g >= n) return;  // uniform over the work-group
  const int tile = g / nrb, b0 = (g % nrb) * kReqBlock;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, c = lane & 31;
  const int v = tile * kTileV + wave * 32 + c;  // this lane's column of the B operand
  const int vr = v < V ? v : V - 1;

  // staging rows of this thread: m = tid / 32 + 8 u, 16-byte word tid % 32 of the rank chunk
  const int sw = tid & 31;
  int srow[kReqBlock / 8];
#pragma unroll
  for (int u = 0; u < kReqBlock / 8; ++u) {
    const int b = b0 + (tid >> 5) + 8 * u;
    const int p = (b < B && prev_tok != nullptr) ? prev_tok[(size_t)b * prev_stride] : -1;
    srow[u] = (p >= 0 && p < V) ? p : -1;
  }
  // base logits of this lane's 32 outputs, loaded ahead of the contraction
  T bv[2][16];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      int b = b0 + rb * 32 + 8 * (i / 4) + 4 * h + (i % 4);
      b = b < B ? b : B - 1;
      bv[rb][i] = base[((size_t)b * K + k) * (size_t)V + vr];
    }

  float16_t acc[2] = {{}, {}};
  const v4u32 zero4 = {0u, 0u, 0u, 0u};
  for (int c0 = 0; c0 < R; c0 += kRankChunk) {
    const int np = (R - c0) / 16 < kPairs ? (R - c0) / 16 : kPairs;  // pairs in this pass
    // B operand: rank indices c0 + 16 t + 8 h .. + 7 of factor row vr, all passes in flight
    const v4u32* rrow = reinterpret_cast<const v4u32*>(right + (size_t)vr * R + c0);
    v4u32 bq[kPairs];
#pragma unroll
    for (int t = 0; t < kPairs; ++t) bq[t] = rrow[2 * (t < np ? t : np - 1) + h];
    // A operand: stage the block's left rows (zero for no previous token or past the rank)
    v4u32 aw[kReqBlock / 8];
#pragma unroll
    for (int u = 0; u < kReqBlock / 8; ++u) {
      const int row = srow[u] < 0 ? 0 : srow[u];
      const int w = 2 * np > sw ? sw : 2 * np - 1;
      aw[u] = reinterpret_cast<const v4u32*>(left + (size_t)row * R + c0)[w];
    }
    if (c0 > 0) __syncthreads();  // the previous pass has read the staged rows
#pragma unroll
    for (int u = 0; u < kReqBlock / 8; ++u) {
      const bool ok = srow[u] >= 0 && sw < 2 * np;
      *reinterpret_cast<v4u32*>(&sm.a[(tid >> 5) + 8 * u][8 * sw]) = ok ? aw[u] : zero4;
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < kPairs; ++t) {
      const v4u32 b = t < np ? bq[t] : zero4;
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const v4u32 a = *reinterpret_cast<const v4u32*>(&sm.a[rb * 32 + c][16 * t + 8 * h]);
        acc[rb] = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(lo4(a), lo4(b), acc[rb], 0, 0, 0);
        acc[rb] = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(hi4(a), hi4(b), acc[rb], 0, 0, 0);
      }
    }
  }
  __syncthreads();  // every wave is done with the staged rows before they become sm.z
  // epilogue: register i of lane (h, c) holds row 8*(i/4) + 4*h + i%4 of the 32x32 block
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int m = rb * 32 + 8 * (i / 4) + 4 * h + (i % 4);
      const int b = b0 + m;
      const bool ok = b < B && v < V;
      const float z = ok ? Logit<T>::get(bv[rb][i]) + acc[rb][i] : -INFINITY;
      if (ok && out != nullptr) Logit<T>::put(out + ((size_t)b * K + k) * (size_t)V + v, z);
      sm.z[m][wave * 32 + c] = z;
    }
  }
  __syncthreads();
  // tile argmax per request: 4 threads per row, 32 columns each, ascending index
  const int m = tid >> 2, q = tid & 3;
  float best = -INFINITY;
  int bi = INT_MAX;
  for (int j = 0; j < 32; ++j) {
    const int col = q * 32 + j;
    const float z = sm.z[m][col];
    if (z > best) {
      best = z;
      bi = tile * kTileV + col;
    }
  }
  argmax_step<kDppXor1>(best, bi);
  argmax_step<kDppXor2>(best, bi);
  const int b = b0 + m;
  if (q == 0 && b < B)
    part[(size_t)b * ntile + tile] = ((uint64_t)__float_as_uint(best) << 32) | (uint32_t)bi;
}

// Ranks up to kRankChunk: a persistent form of the same step. Work-group w walks a contiguous
// range of items (request block, vocabulary tile of kStreamTile), request block slowest. The
// left rows of the request block stay in LDS while the tiles stream through; the factor rows of
// the next item are loaded while the current one is contracted and finished. Each wave owns 16
// columns (v_mfma_f32_16x16x32_bf16: one step per 32 rank indices and 16x16 block, four blocks
// for the 64 requests), so a lane holds its share of a factor row in R/8 registers and two
// items' worth fit beside the accumulators. The epilogue goes through LDS so that base and
// corrected logits move as 16-byte vectors along each request's row.
constexpr int kStreamTile = 16 * kWaves;     // vocabulary entries per item
constexpr int kSteps = kRankChunk / 32;      // MFMA steps per item at the largest rank
constexpr int kZRow = kStreamTile + 4;       // LDS row stride of the corrected tile, in floats
constexpr int kAhead = 2;                    // items whose operands are in flight

template <typename T>
struct Base {
  static constexpr int kVec = 16 / (int)sizeof(T);  // logits per 16-byte vector
  static constexpr int kWords = 16 / kVec;          // vectors of the 16 logits a thread finishes
  v4u32 w[kWords];
};

// Logit e (0..15) of a thread's finishing set, from its raw 16-byte vectors.
template <typename T>
__device__ __forceinline__ float logit_at(const Base<T>& bv, int e) {
  constexpr int kVec = Base<T>::kVec, kPer32 = 4 / (int)sizeof(T);  // logits per 32-bit word
  const uint32_t word = bv.w[e / kVec][(e % kVec) / kPer32];
  if constexpr (sizeof(T) == 4) return __uint_as_float(word);
  else return __uint_as_float((e & 1) ? (word & 0xffff0000u) : (word << 16));
}

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float float4_t __attribute__((ext_vector_type(4)));

// Factor row words of this lane's column of the tile (lane % 16): rank indices
// 32 s + 8 (lane / 16) .. + 7 for step s, 16-byte word 4 s + lane / 16 of the row. Words past
// the row (R not a multiple of 32, or steps past ns) re-read its last word; the contraction
// zeroes them.
__device__ __forceinline__ void load_factor(v4u32 (&bq)[kSteps], const uint16_t* __restrict__ right,
                                            int V, int R, int tile) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = R / 8;
  const int v = tile * kStreamTile + wave * 16 + (lane & 15);
  const v4u32* rrow = reinterpret_cast<const v4u32*>(right + (size_t)(v < V ? v : V - 1) * R);
#pragma unroll
  for (int t = 0; t < kSteps; ++t) {
    const int wi = 4 * t + (lane >> 4);
    bq[t] = rrow[wi < nw ? wi : nw - 1];
  }
}

// Base logits that thread (m, q) finishes: row m of the block, columns 16 q .. 16 q + 15 of the
// tile, clamped into the batch and the vocabulary (the epilogue masks them). VEC: rows are
// 16-byte aligned and V is a multiple of the vector, so a vector starting inside the row lies
// inside it; otherwise element by element.
template <typename T, bool VEC>
__device__ __forceinline__ void load_base(Base<T>& bv, const T* __restrict__ base, int B, int K,
                                          int V, int k, int tile, int b0) {
  constexpr int kVec = Base<T>::kVec;
  const int tid = threadIdx.x;
  int b = b0 + (tid >> 2);
  b = b < B ? b : B - 1;
  const T* row = base + ((size_t)b * K + k) * (size_t)V;
#pragma unroll
  for (int w = 0; w < Base<T>::kWords; ++w) {
    const int v0 = tile * kStreamTile + 16 * (tid & 3) + w * kVec;
    if constexpr (VEC) {
      bv.w[w] = *reinterpret_cast<const v4u32*>(row + (v0 < V ? v0 : V - kVec));
    } else {
      uint32_t e[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        if constexpr (sizeof(T) == 4) {
          e[x] = __float_as_uint(row[v0 + x < V ? v0 + x : V - 1]);
        } else {
          const int v1 = v0 + 2 * x < V ? v0 + 2 * x : V - 1;
          const int v2 = v0 + 2 * x + 1 < V ? v0 + 2 * x + 1 : V - 1;
          e[x] = (uint32_t)row[v1] | ((uint32_t)row[v2] << 16);
        }
      }
      bv.w[w] = v4u32{e[0], e[1], e[2], e[3]};
    }
  }
}

// Previous tokens of the rows this thread stages (rows tid / 32 + 8 u of the request block at
// b0); -1 where there is none (past B, no previous tokens, or outside [0, V)).
__device__ __forceinline__ void stage_tokens(int (&p)[kReqBlock / 8],
                                             const int32_t* __restrict__ prev_tok,
                                             int prev_stride, int B, int V, int b0) {
#pragma unroll
  for (int u = 0; u < kReqBlock / 8; ++u) {
    const int b = b0 + ((int)threadIdx.x >> 5) + 8 * u;
    const int x = (b < B && prev_tok != nullptr) ? prev_tok[(size_t)b * prev_stride] : -1;
    p[u] = (x >= 0 && x < V) ? x : -1;
  }
}

// Stages the left-factor rows of the block's previous tokens into sa (rank words past R and
// rows without a token are zero), then waits for the whole work-group. NB rows per batch of
// loads in flight (fewer: fewer registers).
template <int NB = kReqBlock / 8>
__device__ __forceinline__ void stage_rows(uint16_t (*sa)[kARow], const int (&p)[kReqBlock / 8],
                                           const uint16_t* __restrict__ left, int R) {
  const int sw = threadIdx.x & 31, nw = R / 8;  // 16-byte words per row
  const int wd = sw < nw ? sw : nw - 1;
#pragma unroll
  for (int u0 = 0; u0 < kReqBlock / 8; u0 += NB) {
    v4u32 aw[NB];
#pragma unroll
    for (int u = 0; u < NB; ++u)
      aw[u] = reinterpret_cast<const v4u32*>(left + (size_t)(p[u0 + u] >= 0 ? p[u0 + u] : 0) * R)[wd];
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const bool ok = p[u0 + u] >= 0 && sw < nw;
      *reinterpret_cast<v4u32*>(&sa[(threadIdx.x >> 5) + 8 * (u0 + u)][8 * sw]) =
          ok ? aw[u] : v4u32{0u, 0u, 0u, 0u};
    }
  }
  __syncthreads();
}

struct StreamArgs {
  int B, K, V, k, R, ns, ntile, prev_stride;
  const uint16_t* left;
  const uint16_t* right;
  const int32_t* prev_tok;
  uint64_t* part;
};

// One item of the staged request block: contract with the factor words in cur (those of the
// item kAhead on are requested into nxt first), add the base logits, write the corrected logits
// and the tile argmax of every request of the block.
template <typename T>
struct Stage {
  v4u32 f[kSteps];  // factor row words of this lane's column
  Base<T> bv;       // base logits this thread finishes
};

// Requests item j's operands into st (j clamped to the run's last item, so that every trip
// issues the same loads and the waits stay exact).
template <typename T, bool VEC>
__device__ __forceinline__ void load_stage(Stage<T>& st, const StreamArgs& a,
                                           const T* __restrict__ base, int j, int jend) {
  j = j < jend ? j : jend - 1;
  const int tile = j % a.ntile;
  load_base<T, VEC>(st.bv, base, a.B, a.K, a.V, a.k, tile, (j / a.ntile) * kReqBlock);
  load_factor(st.f, a.right, a.V, a.R, tile);
}

template <typename T, bool VEC, bool FULL>
__device__ __forceinline__ void stream_item(const StreamArgs& a, const T* __restrict__ base,
                                            T* __restrict__ out, uint16_t (*sa)[kARow],
                                            float (*sz)[kZRow], int j, int jend,
                                            const Stage<T>& cur, Stage<T>& nxt) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tile = j % a.ntile, b0 = (j / a.ntile) * kReqBlock;
  load_stage<T, VEC>(nxt, a, base, j + kAhead, jend);
  const Base<T>& bv = cur.bv;
  float4_t acc[4] = {{}, {}, {}, {}};
#pragma unroll
  for (int t = 0; t < kSteps; ++t) {
    if (FULL || t < a.ns) {  // uniform
      const bool inside = FULL || 4 * t + (lane >> 4) < a.R / 8;
      const bf16x8_t bfr =
          __builtin_bit_cast(bf16x8_t, inside ? cur.f[t] : v4u32{0u, 0u, 0u, 0u});
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        const v4u32 x =
            *reinterpret_cast<const v4u32*>(&sa[rb * 16 + (lane & 15)][32 * t + 8 * (lane >> 4)]);
        acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, x), bfr,
                                                          acc[rb], 0, 0, 0);
      }
    }
  }
  // register i of lane l holds row 4 (l / 16) + i, column l % 16 of the 16x16 block
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      sz[rb * 16 + 4 * (lane >> 4) + i][wave * 16 + (lane & 15)] = acc[rb][i];
  __syncthreads();
  // thread (m, q): row m of the block, columns 16 q .. 16 q + 15, ascending; a wave's 16 rows
  // are rows 16 w .. 16 w + 15, and a wave with no request among them skips the epilogue
  const int m = tid >> 2, q = tid & 3, b = b0 + m;
  const int v0 = tile * kStreamTile + 16 * q;
  float best = -INFINITY;
  int bi = INT_MAX;
  if (b0 + 16 * wave < a.B) {  // uniform over the wave
    float z[16];
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const float4 acc4 = *reinterpret_cast<const float4*>(&sz[m][16 * q + 4 * x]);
      z[4 * x] = logit_at<T>(bv, 4 * x) + acc4.x;
      z[4 * x + 1] = logit_at<T>(bv, 4 * x + 1) + acc4.y;
      z[4 * x + 2] = logit_at<T>(bv, 4 * x + 2) + acc4.z;
      z[4 * x + 3] = logit_at<T>(bv, 4 * x + 3) + acc4.w;
    }
    const bool row_ok = b < a.B;
    const int ncol = a.V - v0;  // columns of this thread inside the vocabulary (may be <= 0)
    int e_best = -1;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const bool take = row_ok && e < ncol && z[e] > best;
      best = take ? z[e] : best;
      e_best = take ? e : e_best;
    }
    bi = e_best < 0 ? INT_MAX : v0 + e_best;
    if (out != nullptr && row_ok) {
      T* orow = out + ((size_t)b * a.K + a.k) * (size_t)a.V + v0;
      if constexpr (VEC) {  // whole vectors: the row ends on a vector boundary
        constexpr int kVec = Base<T>::kVec;
#pragma unroll
        for (int w = 0; w < Base<T>::kWords; ++w) {
          if (w * kVec < ncol) {
            if constexpr (sizeof(T) == 4) {
              *reinterpret_cast<float4*>(orow + 4 * w) =
                  make_float4(z[4 * w], z[4 * w + 1], z[4 * w + 2], z[4 * w + 3]);
            } else {  // round to nearest even
              uint32_t r[4];
#pragma unroll
              for (int x = 0; x < 4; ++x)
                r[x] = __builtin_bit_cast(uint32_t, bf16x2_t{(__bf16)z[8 * w + 2 * x],
                                                             (__bf16)z[8 * w + 2 * x + 1]});
              *reinterpret_cast<v4u32*>(orow + 8 * w) = v4u32{r[0], r[1], r[2], r[3]};
            }
          }
        }
      } else {
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (e < ncol) Logit<T>::put(orow + e, z[e]);
      }
    }
    argmax_step<kDppXor1>(best, bi);
    argmax_step<kDppXor2>(best, bi);
  }
  if (q == 0 && b < a.B)
    a.part[(size_t)b * a.ntile + tile] = ((uint64_t)__float_as_uint(best) << 32) | (uint32_t)bi;
  __syncthreads();  // sz is rewritten by the next item
}

template <typename T, bool VEC, bool FULL>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void markov_stream(const T* __restrict__ base,
                                                          T* __restrict__ out, StreamArgs a,
                                                          int nrb, int per_group) {
  __shared__ __attribute__((aligned(16))) uint16_t sa[kReqBlock][kARow];
  __shared__ __attribute__((aligned(16))) float sz[kReqBlock][kZRow];
  const int n = a.ntile * nrb, lanes8 = (int)gridDim.x / 8;
  const int w = (int)(blockIdx.x & 7) * lanes8 + (int)(blockIdx.x >> 3);
  const int j0 = w * per_group, j1 = j0 + per_group < n ? j0 + per_group : n;
  if (j0 >= j1) return;  // uniform over the work-group
  Stage<T> s0, s1, s2;
  for (int j = j0; j < j1;) {  // runs of items that share a request block
    const int rbk = j / a.ntile;
    const int jend = (rbk + 1) * a.ntile < j1 ? (rbk + 1) * a.ntile : j1;
    {  // previous tokens first, then the first items' operands, then the left rows
      int p[kReqBlock / 8];
      stage_tokens(p, a.prev_tok, a.prev_stride, a.B, a.V, rbk * kReqBlock);
      load_stage<T, VEC>(s0, a, base, j, jend);
      load_stage<T, VEC>(s1, a, base, j + 1, jend);
      if (j > j0) __syncthreads();  // the previous block's rows are no longer read
      stage_rows(sa, p, a.left, a.R);
    }
    // three items per trip, the operand stages rotating; whole trips only, so that the loads
    // still in flight at the loop's back edge are always the same two stages
    for (; j + 3 <= jend; j += 3) {
      stream_item<T, VEC, FULL>(a, base, out, sa, sz, j, jend, s0, s2);
      stream_item<T, VEC, FULL>(a, base, out, sa, sz, j + 1, jend, s1, s0);
      stream_item<T, VEC, FULL>(a, base, out, sa, sz, j + 2, jend, s2, s1);
    }
    if (j < jend) stream_item<T, VEC, FULL>(a, base, out, sa, sz, j, jend, s0, s2);
    if (j + 1 < jend) stream_item<T, VEC, FULL>(a, base, out, sa, sz, j + 1, jend, s1, s0);
    j = jend;
  }
}

// One work-group per request: the argmax over the tile partials (lowest index on ties) is the
// position's token. A request whose logits are all -inf or NaN gets token 0.
__global__ __launch_bounds__(kThreads) void markov_finish(const uint64_t* __restrict__ part,
                                                          int ntile, int K, int k,
                                                          int32_t* __restrict__ tokens) {
  const int b = blockIdx.x;
  const uint64_t* row = part + (size_t)b * ntile;
  float best = -INFINITY;
  int bi = INT_MAX;
  for (int t0 = 0; t0 < ntile; t0 += kThreads * kFinishLoads) {
    uint64_t w[kFinishLoads];
#pragma unroll
    for (int u = 0; u < kFinishLoads; ++u) {
      const int t = t0 + u * kThreads + (int)threadIdx.x;
      w[u] = row[t < ntile ? t : ntile - 1];
    }
#pragma unroll
    for (int u = 0; u < kFinishLoads; ++u) {
      const float z = __uint_as_float((uint32_t)(w[u] >> 32));
      const int i = (int)(uint32_t)w[u];
      if (better(z, i, best, bi)) {  // a repeated last partial changes nothing
        best = z;
        bi = i;
      }
    }
  }
  wave_argmax(best, bi);
  __shared__ float sb[kWaves];
  __shared__ int si[kWaves];
  if ((threadIdx.x & 63) == 0) {
    sb[threadIdx.x >> 6] = best;
    si[threadIdx.x >> 6] = bi;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kWaves; ++w)
      if (better(sb[w], si[w], best, bi)) {
        best = sb[w];
        bi = si[w];
      }
    tokens[(size_t)b * K + k] = bi == INT_MAX ? 0 : bi;
  }
}


// ---------------------------------------------------------------------------------------------
// All K positions in one launch, for up to 64 requests at ranks up to 256. Work-group w owns
// vocabulary tiles [w per, (w + 1) per) (per <= kResItems) for every position and holds their
// right-factor rows in registers from the first position to the last, so that a position moves
// only its base and corrected logits (and the left rows of the previous tokens). Between two
// positions the work-groups hand off through tagged words (the call's tag plus the position in
// the upper half, the payload in the lower; agent-scope atomic stores and loads):
//   * each work-group publishes, per request, the argmax (value, index) over its tiles;
//   * work-group b (b < B) waits for those of request b, reduces them (lowest index on ties) to
//     the position's token, writes it and publishes it;
//   * every work-group waits for the B tokens, gathers their left rows, and goes on.
// Every wait depends only on work-groups that are resident at the same time (the grid is at
// most one work-group per slot) and is bounded: after kResSpin polls it gives up, and the
// request's token at that position and after is reported as -2.
constexpr int kResItems = 5;       // vocabulary tiles per work-group, factor rows in registers
constexpr int kResSpin = 1 << 21;  // polls before a wait gives up
constexpr int32_t kResFailed = -2;

struct ResArgs {
  int B, K, V, R, ns, ntile, per, nwg;
  int nfull;  // work-groups w < nfull own per tiles, the others per - 1
  const uint16_t* left;
  const uint16_t* right;
  const int32_t* anchor;
  int32_t* tokens;  // [B][K]
  uint64_t* part;   // [B][nwg][2] tagged (value bits, index) of each work-group's tiles
  uint64_t* tok;    // [B] tagged token of the latest position
  uint32_t tag;     // position k (stage s of markov_pipe) publishes with tag + k (tag + s): the
                    // call owns tags [tag, tag + 2K + 2), at least one past its last stage 2K
  // sampled form only
  const float* tau;  // [B] temperatures: 0 argmax, >= kTauMin and finite a draw, else invalid
  const float* uni;  // [B][K] one uniform per position
  uint64_t* dec;     // [B][2] tagged draw decision: owning work-group, target in its scale
};

constexpr double kLog2e = 1.4426950408889634074;
constexpr double kTauMin = kLog2e / 2097152.0;  // smallest sampling temperature: c <= 2^21
constexpr int32_t kInvalid = -3;                 // tokens of a request whose temperature is invalid
constexpr uint32_t kNoOwner = 0xFFFFFFFFu;       // decision payload: no work-group draws
constexpr int kDecideLoads = 4;                  // partials per thread of a draw decision

// Weight of a stored logit y in a draw at inverse temperature c (log2 e / tau), relative to the
// offset m (a value >= every y it is applied to): 2^((y - m) c); NaN and -inf weigh 0, and y == m
// weighs 1 (also when both are +inf).
__device__ __forceinline__ float draw_weight(float y, float m, float c) {
  return y > -INFINITY ? __builtin_amdgcn_exp2f(y == m ? 0.0f : (y - m) * c) : 0.0f;
}

__device__ __forceinline__ void res_publish(uint64_t* p, uint32_t tag, uint32_t payload) {
  __hip_atomic_store(p, ((uint64_t)tag << 32) | payload, __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t res_fetch(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Polls *p until its tag is `tag` (at most kResSpin polls). Returns the payload, or fails.
__device__ __forceinline__ bool res_await(const uint64_t* p, uint32_t tag, uint32_t& payload) {
  uint64_t v = res_fetch(p);
  for (int left = kResSpin; (uint32_t)(v >> 32) != tag; --left) {
    if (left == 0) return false;
    __builtin_amdgcn_s_sleep(2);
    v = res_fetch(p);
  }
  payload = (uint32_t)v;
  return true;
}

// A barrier for LDS traffic only: this wave's LDS accesses complete, then the work-group meets.
// (__syncthreads would also wait for every global load and store in flight, among them the
// ring's loads.) The empty asm statements keep the compiler from moving memory accesses across.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// One tile of the work-group at position k: contract the staged left rows with the tile's factor
// words f (registers), add the base logits bv, write the corrected logits and fold the tile's
// per-request argmax into (run, run_i) (every thread of a row holds the row's).
template <typename T, bool VEC, bool FULL, bool SAMPLED>
__device__ __forceinline__ void res_tile(const ResArgs& a, T* __restrict__ out,
                                         uint16_t (*sa)[kARow], float (*sz)[kZRow], int k,
                                         int tile, const v4u32 (&f)[kSteps], const Base<T>& bv,
                                         float& run, int& run_i, float c, float& sm, float& ss) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float4_t acc[4] = {{}, {}, {}, {}};
#pragma unroll
  for (int t = 0; t < kSteps; ++t) {
    if (FULL || t < a.ns) {  // uniform
      const bool inside = FULL || 4 * t + (lane >> 4) < a.R / 8;
      const bf16x8_t bfr = __builtin_bit_cast(bf16x8_t, inside ? f[t] : v4u32{0u, 0u, 0u, 0u});
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        const v4u32 x =
            *reinterpret_cast<const v4u32*>(&sa[rb * 16 + (lane & 15)][32 * t + 8 * (lane >> 4)]);
        acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, x), bfr,
                                                          acc[rb], 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      sz[rb * 16 + 4 * (lane >> 4) + i][wave * 16 + (lane & 15)] = acc[rb][i];
  lds_barrier();
  const int m = tid >> 2, q = tid & 3;
  const int v0 = tile * kStreamTile + 16 * q;
  if (16 * wave < a.B) {  // uniform over the wave
    float z[16];
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const float4 acc4 = *reinterpret_cast<const float4*>(&sz[m][16 * q + 4 * x]);
      z[4 * x] = logit_at<T>(bv, 4 * x) + acc4.x;
      z[4 * x + 1] = logit_at<T>(bv, 4 * x + 1) + acc4.y;
      z[4 * x + 2] = logit_at<T>(bv, 4 * x + 2) + acc4.z;
      z[4 * x + 3] = logit_at<T>(bv, 4 * x + 3) + acc4.w;
    }
    const bool row_ok = m < a.B;
    const int ncol = a.V - v0;
    float best = -INFINITY;
    int e_best = -1;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const bool take = row_ok && e < ncol && z[e] > best;
      best = take ? z[e] : best;
      e_best = take ? e : e_best;
    }
    int bi = e_best < 0 ? INT_MAX : v0 + e_best;
    if (out != nullptr && row_ok) {
      T* orow = out + ((size_t)m * a.K + k) * (size_t)a.V + v0;
      if constexpr (VEC) {
        constexpr int kVec = Base<T>::kVec;
#pragma unroll
        for (int w = 0; w < Base<T>::kWords; ++w) {
          if (w * kVec < ncol) {
            if constexpr (sizeof(T) == 4) {
              *reinterpret_cast<float4*>(orow + 4 * w) =
                  make_float4(z[4 * w], z[4 * w + 1], z[4 * w + 2], z[4 * w + 3]);
            } else {
              uint32_t r[4];
#pragma unroll
              for (int x = 0; x < 4; ++x)
                r[x] = __builtin_bit_cast(uint32_t, bf16x2_t{(__bf16)z[8 * w + 2 * x],
                                                             (__bf16)z[8 * w + 2 * x + 1]});
              *reinterpret_cast<v4u32*>(orow + 8 * w) = v4u32{r[0], r[1], r[2], r[3]};
            }
          }
        }
      } else {
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (e < ncol) Logit<T>::put(orow + e, z[e]);
      }
    }
    argmax_step<kDppXor1>(best, bi);
    argmax_step<kDppXor2>(best, bi);
    if (better(best, bi, run, run_i)) {
      run = best;
      run_i = bi;
    }
    if constexpr (SAMPLED) {
      // the row's mass over the work-group's tiles, online: sm the largest stored value so far,
      // ss the sum of draw_weight(y, sm, c) (each thread of a row holds the row's)
      float y[16];
      float tm = -INFINITY;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        y[e] = Logit<T>::stored(z[e]);
        y[e] = (row_ok && e < ncol) ? y[e] : -INFINITY;
        tm = y[e] > tm ? y[e] : tm;
      }
      tm = fmaxf(tm, dpp_xchg_f32<kDppXor1>(tm));
      tm = fmaxf(tm, dpp_xchg_f32<kDppXor2>(tm));
      const float nm = fmaxf(sm, tm);
      float ts = 0.0f;
#pragma unroll
      for (int e = 0; e < 16; ++e) ts += draw_weight(y[e], nm, c);
      ts += dpp_xchg_f32<kDppXor1>(ts);
      ts += dpp_xchg_f32<kDppXor2>(ts);
      ss = ss * (sm == nm ? 1.0f : __builtin_amdgcn_exp2f((sm - nm) * c)) + ts;
      sm = nm;
    }
  }
  lds_barrier();  // sz is rewritten by the next tile
}

// Cross-lane moves inside the vector ALU (DPP), for the reductions and scans of the draws: each
// lane combines the lanes 1, 2, 4 and 8 below it inside its row of 16, then lane 15 of rows 0
// and 2 is folded into rows 1 and 3 and lane 31 into rows 2 and 3, so lane l ends up with the
// combination of lanes 0..l (lane 63: the whole wave). A source lane outside the row, or a row
// that the mask leaves out, reads the identity. Every call runs with the whole wave active.
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_move(uint32_t x, uint32_t identity) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)identity, (int)x, CTRL, ROWS, 0xf, false);
}
#define SV_MK_SCAN(STEP) \
  STEP(0x111, 0xf);      \
  STEP(0x112, 0xf);      \
  STEP(0x114, 0xf);      \
  STEP(0x118, 0xf);      \
  STEP(0x142, 0xa);      \
  STEP(0x143, 0xc)

// Inclusive prefix sum over the wave (fp32), and the exclusive one (the inclusive sum of the lane
// below, by a whole-wave shift; lane 0: 0).
__device__ __forceinline__ float wave_incl_sum(float x) {
#define SV_STEP(C, R) x += __uint_as_float(dpp_move<C, R>(__float_as_uint(x), 0u))
  SV_MK_SCAN(SV_STEP);
#undef SV_STEP
  return x;
}
__device__ __forceinline__ float wave_excl_of(float incl) {
  return __uint_as_float(dpp_move<0x138, 0xf>(__float_as_uint(incl), 0u));  // wave_shr:1
}
__device__ __forceinline__ float wave_max_all(float x) {  // NaN-free inputs
#define SV_STEP(C, R) x = fmaxf(x, __uint_as_float(dpp_move<C, R>(__float_as_uint(x), 0xff800000u)))
  SV_MK_SCAN(SV_STEP);
#undef SV_STEP
  return __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(x), 63));
}
__device__ __forceinline__ int wave_min_all(int x) {
#define SV_STEP(C, R) x = min(x, (int)dpp_move<C, R>((uint32_t)x, (uint32_t)INT_MAX))
  SV_MK_SCAN(SV_STEP);
#undef SV_STEP
  return __builtin_amdgcn_readlane(x, 63);
}

// Sum over the work-group of one value per thread: returns this thread's exclusive prefix (in
// thread order) and the total through `total`. s_w: kWaves floats of LDS. Every thread calls it.
__device__ __forceinline__ float block_scan_excl(float x, float* s_w, float& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float incl = wave_incl_sum(x);
  const float excl = wave_excl_of(incl);
  if (lane == 63) s_w[wave] = incl;
  lds_barrier();
  float before = 0.0f, all = 0.0f;
#pragma unroll
  for (int v = 0; v < kWaves; ++v) {
    before = v < wave ? before + s_w[v] : before;
    all += s_w[v];
  }
  lds_barrier();  // s_w is reused by the caller
  total = all;
  return before + excl;
}

__device__ __forceinline__ float block_max(float x, float* s_w) {
  x = wave_max_all(x);
  if ((threadIdx.x & 63) == 0) s_w[threadIdx.x >> 6] = x;
  lds_barrier();
  float r = s_w[0];
#pragma unroll
  for (int v = 1; v < kWaves; ++v) r = fmaxf(r, s_w[v]);
  lds_barrier();
  return r;
}

__device__ __forceinline__ int block_min_i(int x, int* s_w) {
  x = wave_min_all(x);
  if ((threadIdx.x & 63) == 0) s_w[threadIdx.x >> 6] = x;
  lds_barrier();
  int r = s_w[0];
#pragma unroll
  for (int v = 1; v < kWaves; ++v) r = min(r, s_w[v]);
  lds_barrier();
  return r;
}

// Work-group b, whose request draws at position k: waits for every work-group's (sm, ss) of the
// request (its largest stored value and its mass relative to it), scales them to the row's
// largest value M, and finds the first work-group j (ascending, so ascending vocabulary) whose
// share of the CDF passes u S, S the row's mass and u the position's uniform clamped to [0, 1]
// (NaN as 0). Publishes j and the target measured from the start of j's share in j's own scale
// (j scans its entries for it); past every share (rounding) the last work-group with mass and an
// infinite target. Without mass the token is 0, after a wait that gave up kResFailed: then the
// token itself is published, with kNoOwner as the decision.
__device__ __forceinline__ void res_decide(const ResArgs& a, int b, int k, uint32_t tg, float c,
                                           bool failed, float* s_f, int* s_i, int* s_i2,
                                           float* s_tgt1, float* s_pm, float* s_ps) {
  const int tid = threadIdx.x;
  const uint64_t* row = a.part + (size_t)b * a.nwg * 2;
  // the partials into LDS, one per thread at a time
  bool late = false;
  for (int j0 = 0; j0 < a.nwg; j0 += kThreads) {  // nwg <= kDecideLoads * kThreads
    const int j = j0 + tid;
    if (j < a.nwg) {
      uint64_t v0 = res_fetch(row + 2 * j), v1 = res_fetch(row + 2 * j + 1);
      for (int left = kResSpin; !late;) {
        if ((uint32_t)(v0 >> 32) == tg && (uint32_t)(v1 >> 32) == tg) break;
        if (--left == 0) late = true;
        __builtin_amdgcn_s_sleep(2);
        if ((uint32_t)(v0 >> 32) != tg) v0 = res_fetch(row + 2 * j);
        if ((uint32_t)(v1 >> 32) != tg) v1 = res_fetch(row + 2 * j + 1);
      }
      s_pm[j] = __uint_as_float((uint32_t)v0);
      s_ps[j] = __uint_as_float((uint32_t)v1);
    }
  }
  const bool any_late = __syncthreads_or(late) != 0;
  // thread t: partials kDecideLoads t .. + kDecideLoads - 1 (ascending)
  const int j0 = kDecideLoads * tid;
  float tmax = -INFINITY;
#pragma unroll
  for (int i = 0; i < kDecideLoads; ++i) {
    if (j0 + i < a.nwg && s_ps[j0 + i] > 0.0f) tmax = fmaxf(tmax, s_pm[j0 + i]);
  }
  const float M = block_max(tmax, s_f);
  // the share of partial j in the row's scale: s_j 2^((m_j - M) c)
  auto share = [&](int j) {
    const float m = s_pm[j], sj = s_ps[j];
    return sj > 0.0f ? sj * (m == M ? 1.0f : __builtin_amdgcn_exp2f((m - M) * c)) : 0.0f;
  };
  float tsum = 0.0f;
#pragma unroll
  for (int i = 0; i < kDecideLoads; ++i)
    if (j0 + i < a.nwg) tsum += share(j0 + i);
  float S;
  float P = block_scan_excl(tsum, s_f, S);
  const float u = a.uni[(size_t)b * a.K + k];
  const float T = (u > 0.0f ? fminf(u, 1.0f) : 0.0f) * S;
  int found = INT_MAX, last = -1;
  float tgt = 0.0f;
#pragma unroll
  for (int i = 0; i < kDecideLoads; ++i) {
    const float x = j0 + i < a.nwg ? share(j0 + i) : 0.0f;
    if (x > 0.0f) {
      if (found == INT_MAX && P + x > T) {
        found = j0 + i;
        tgt = fmaxf(T - P, 0.0f) / x * s_ps[j0 + i];  // a fraction of j's share, in j's scale
      }
      last = j0 + i;
    }
    P += x;
  }
  // one exchange for the first work-group past the target (with its target, from the lane that
  // found it: partial indices are distinct) and the last one with mass
  {
    const int lane = tid & 63, wave = tid >> 6;
    const int wf = wave_min_all(found);
    const uint64_t who = __ballot(found == wf && wf != INT_MAX);
    const float wt =
        who != 0 ? __uint_as_float((uint32_t)__builtin_amdgcn_readlane(
                       (int)__float_as_uint(tgt), (int)__ffsll((long long)who) - 1))
                 : 0.0f;
    const int wl = -wave_min_all(-last);
    if (lane == 0) {
      s_i[wave] = wf;
      s_f[wave] = wt;
      s_i2[wave] = wl;
    }
  }
  lds_barrier();
  if (tid == 0) {
    int jf = INT_MAX, jl = -1;
    for (int v = 0; v < kWaves; ++v) {
      if (s_i[v] < jf) {
        jf = s_i[v];
        *s_tgt1 = s_f[v];
      }
      jl = max(jl, s_i2[v]);
    }
    int token = -1;
    if (failed || any_late) token = kResFailed;
    else if (!(S > 0.0f) || jl < 0) token = 0;
    if (token != -1) {
      a.tokens[(size_t)b * a.K + k] = token;
      res_publish(a.tok + b, tg, (uint32_t)token);
      res_publish(a.dec + 2 * b, tg, kNoOwner);
    } else {
      const bool hit = jf != INT_MAX;
      res_publish(a.dec + 2 * b + 1, tg, __float_as_uint(hit ? *s_tgt1 : INFINITY));
      res_publish(a.dec + 2 * b, tg, (uint32_t)(hit ? jf : jl));
    }
  }
}

// One wave of the work-group that owns request b's draw at position k: the entries of its tiles
// (vocabulary t0 * kStreamTile up to the tiles' end), read back from the draft row it wrote, are
// weighed exactly as the tile epilogue weighed them (offset m, the work-group's largest value);
// the token is the first entry at which the running sum passes `target` (ascending; lane l holds
// entries l E .. l E + E - 1), else (rounding) the last entry with mass.
template <typename T>
__device__ __forceinline__ void res_owner_draw(const ResArgs& a, const T* __restrict__ out, int b,
                                               int k, uint32_t tg, int t0, int nit, float m,
                                               float c, float target) {
  const int lane = threadIdx.x & 63;
  const int v0 = t0 * kStreamTile;
  const int vend = (t0 + nit) * kStreamTile < a.V ? (t0 + nit) * kStreamTile : a.V;
  const int n = vend - v0;  // >= 1: the work-group reported mass
  const int E = (n + 63) >> 6;  // <= kResItems
  const T* row = out + ((size_t)b * a.K + k) * (size_t)a.V + v0 + lane * E;
  const int mine = n - lane * E < E ? n - lane * E : E;  // this lane's entries (may be <= 0)
  // the lane's entries, all loads in flight together, weighed once and kept for the walk
  float wv[kResItems];
#pragma unroll
  for (int i = 0; i < kResItems; ++i)
    wv[i] = i < mine ? draw_weight(Logit<T>::get(row[i]), m, c) : 0.0f;
  float lsum = 0.0f;
#pragma unroll
  for (int i = 0; i < kResItems; ++i)
    if (i < mine) lsum += wv[i];
  const float incl = wave_incl_sum(lsum);
  float cum = wave_excl_of(incl);
  int pick = -1, lastw = -1;
#pragma unroll
  for (int i = 0; i < kResItems; ++i) {  // the same weights in the same order
    const float w = i < mine ? wv[i] : 0.0f;
    if (w > 0.0f) {
      cum += w;
      pick = (pick < 0 && cum > target) ? i : pick;
      lastw = i;
    }
  }
  pick = pick < 0 ? lastw : pick;
  const uint64_t hit = __ballot(lsum > 0.0f && incl > target);
  const uint64_t mass = __ballot(lsum > 0.0f);
  int L, e;
  if (hit != 0) {
    L = __builtin_ctzll(hit);
    e = __builtin_amdgcn_readlane(pick, L);
  } else if (mass != 0) {
    L = 63 - __builtin_clzll(mass);
    e = __builtin_amdgcn_readlane(lastw, L);
  } else {
    L = 0;
    e = 0;
  }
  const int token = v0 + L * E + e;
  if (lane == 0) {
    a.tokens[(size_t)b * a.K + k] = token;
    res_publish(a.tok + b, tg, (uint32_t)token);
  }
}

template <typename T, bool VEC, bool FULL, bool SAMPLED>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void
markov_resident(const T* __restrict__ base, T* __restrict__ out, ResArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t sa[kReqBlock][kARow];
  __shared__ __attribute__((aligned(16))) float sz[kReqBlock][kZRow];
  __shared__ int s_tok[kReqBlock];
  __shared__ float s_best[kWaves];
  __shared__ int s_bi[kWaves], s_late[kWaves];
  // sampled form: per request its mode (0 argmax, 1 draw, 2 invalid), inverse temperature, this
  // work-group's largest stored value, and the draws this work-group owns
  __shared__ int s_mode[SAMPLED ? kReqBlock : 1], s_own[SAMPLED ? kReqBlock : 1];
  __shared__ float s_c[SAMPLED ? kReqBlock : 1], s_m[SAMPLED ? kReqBlock : 1];
  __shared__ float s_tgt[SAMPLED ? kReqBlock : 1], s_tgt1[1];
  __shared__ float s_pm[SAMPLED ? kDecideLoads * kThreads : 1];  // a decision's partials
  __shared__ float s_ps[SAMPLED ? kDecideLoads * kThreads : 1];
  const int w = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // work-groups w < nfull own per tiles, the others per - 1 (contiguous, ascending)
  const int t0 = w < a.nfull ? w * a.per : a.nfull * a.per + (w - a.nfull) * (a.per - 1);
  const int nit = w < a.nfull ? a.per : a.per - 1;
  if constexpr (SAMPLED) {
    if (tid < kReqBlock) {
      const float tau = tid < a.B ? a.tau[tid] : 0.0f;
      const bool draw = (double)tau >= kTauMin && tau < INFINITY;
      s_mode[tid] = tau == 0.0f ? 0 : (draw ? 1 : 2);
      s_c[tid] = draw ? (float)(kLog2e / (double)tau) : 1.0f;
    }
  }
  v4u32 f[kResItems][kSteps];
#pragma unroll
  for (int i = 0; i < kResItems; ++i) {
    const int tile = t0 + i < a.ntile ? t0 + i : a.ntile - 1;
    load_factor(f[i], a.right, a.V, a.R, tile);
  }
  for (int k = 0; k < a.K; ++k) {
    const uint32_t tg = a.tag + (uint32_t)k;
    Base<T> bb[2];
    load_base<T, VEC>(bb[0], base, a.B, a.K, a.V, k, t0 < a.ntile ? t0 : a.ntile - 1, 0);
    // 1. the previous tokens (the anchor at k = 0)
    if (tid < kReqBlock) {
      int x = -1;
      if (tid < a.B) {
        if (k == 0) {
          x = a.anchor != nullptr ? a.anchor[tid] : -1;
        } else {
          uint32_t pl;
          x = res_await(a.tok + tid, tg - 1u, pl) ? (int)pl : kResFailed;
        }
      }
      s_tok[tid] = x;
    }
    lds_barrier();
    int p[kReqBlock / 8];
#pragma unroll
    for (int u = 0; u < kReqBlock / 8; ++u) {
      const int x = s_tok[(tid >> 5) + 8 * u];
      p[u] = (x >= 0 && x < a.V) ? x : -1;
    }
    stage_rows(sa, p, a.left, a.R);
    // 2. the work-group's tiles, the base logits of the next one in flight
    float run = -INFINITY;
    int run_i = INT_MAX;
    const float c = SAMPLED ? s_c[tid >> 2] : 1.0f;
    float sm = -INFINITY, ss = 0.0f;
#pragma unroll
    for (int i = 0; i < kResItems; ++i) {
      if (i < nit) {  // uniform
        if (i + 1 < nit)
          load_base<T, VEC>(bb[(i + 1) & 1], base, a.B, a.K, a.V, k, t0 + i + 1, 0);
        res_tile<T, VEC, FULL, SAMPLED>(a, out, sa, sz, k, t0 + i, f[i], bb[i & 1], run, run_i,
                                        c, sm, ss);
      }
    }
    // 3. this work-group's argmax of each request, or (sampled) its largest value and mass
    if ((tid & 3) == 0 && (tid >> 2) < a.B) {
      const bool draw = SAMPLED && s_mode[tid >> 2] == 1;
      uint64_t* pp = a.part + ((size_t)(tid >> 2) * a.nwg + w) * 2;
      res_publish(pp, tg, __float_as_uint(draw ? sm : run));
      res_publish(pp + 1, tg, draw ? __float_as_uint(ss) : (uint32_t)run_i);
      if constexpr (SAMPLED) s_m[tid >> 2] = sm;
    }
    // 4. work-group b < B: the token of request b (or, drawing, who draws it)
    const int mode = (SAMPLED && w < a.B) ? s_mode[w] : 0;
    if (w < a.B && mode == 1) {
      res_decide(a, w, k, tg, s_c[w], s_tok[w] == kResFailed, s_best, s_bi, s_late, s_tgt1, s_pm,
                 s_ps);
    } else if (w < a.B && mode == 2) {
      if (tid == 0) {
        a.tokens[(size_t)w * a.K + k] = kInvalid;
        res_publish(a.tok + w, tg, (uint32_t)kInvalid);
      }
    } else if (w < a.B) {
      const int b = w;
      float best = -INFINITY;
      int bi = INT_MAX;
      bool late = false;
      for (int j0 = 0; j0 < a.nwg; j0 += 2 * kThreads) {  // two partials per thread in flight
        const uint64_t* pp[2];
        uint64_t v[4];
        bool live[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int j = j0 + u * kThreads + tid;
          live[u] = j < a.nwg;
          pp[u] = a.part + ((size_t)b * a.nwg + (live[u] ? j : 0)) * 2;
          v[2 * u] = live[u] ? res_fetch(pp[u]) : (uint64_t)tg << 32;
          v[2 * u + 1] = live[u] ? res_fetch(pp[u] + 1) : (uint64_t)tg << 32;
        }
        for (int left = kResSpin;; --left) {
          bool all = true;
#pragma unroll
          for (int x = 0; x < 4; ++x) all = all && (uint32_t)(v[x] >> 32) == tg;
          if (all) break;
          if (left == 0) {
            late = true;
            break;
          }
          __builtin_amdgcn_s_sleep(2);
#pragma unroll
          for (int x = 0; x < 4; ++x)
            if ((uint32_t)(v[x] >> 32) != tg) v[x] = res_fetch(pp[x >> 1] + (x & 1));
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          if (live[u]) {
            const float z = __uint_as_float((uint32_t)v[2 * u]);
            const int i = (int)(uint32_t)v[2 * u + 1];
            if (better(z, i, best, bi)) {
              best = z;
              bi = i;
            }
          }
        }
      }
      wave_argmax(best, bi);
      const bool wave_late = __ballot(late) != 0;
      if (lane == 0) {
        s_best[wave] = best;
        s_bi[wave] = bi;
        s_late[wave] = wave_late;
      }
      lds_barrier();
      if (tid == 0) {
        bool any_late = false;
        for (int v = 0; v < kWaves; ++v) {
          any_late = any_late || s_late[v] != 0;
          if (better(s_best[v], s_bi[v], best, bi)) {
            best = s_best[v];
            bi = s_bi[v];
          }
        }
        const bool failed = any_late || s_tok[b] == kResFailed;
        const int token = failed ? kResFailed : (bi == INT_MAX ? 0 : bi);
        a.tokens[(size_t)b * a.K + k] = token;
        res_publish(a.tok + b, tg, (uint32_t)token);
      }
    }
    // 5. (sampled) the draws whose CDF target falls in this work-group's tiles
    if constexpr (SAMPLED) {
      if (tid < kReqBlock) {
        int own = 0;
        float t = 0.0f;
        if (tid < a.B && s_mode[tid] == 1) {
          uint32_t pl;
          if (res_await(a.dec + 2 * tid, tg, pl) && pl == (uint32_t)w) {
            uint32_t pf;
            if (res_await(a.dec + 2 * tid + 1, tg, pf)) {
              own = 1;
              t = __uint_as_float(pf);
            }
          }
        }
        s_own[tid] = own;
        s_tgt[tid] = t;
      }
      __syncthreads();  // also: this work-group's stores of the corrected rows are complete
      // the i-th draw this work-group owns goes to wave i mod 4: a work-group that owns several
      // spreads them over its waves
      const uint64_t owned = __ballot(lane < a.B && s_own[lane] != 0);  // the same in every wave
      int i = 0;
      for (uint64_t m = owned; m != 0; m &= m - 1, ++i) {
        if (i % kWaves != wave) continue;
        const int b = __ffsll((long long)m) - 1;
        res_owner_draw<T>(a, out, b, k, tg, t0, nit, s_m[b], s_c[b], s_tgt[b]);
      }
    }
    lds_barrier();  // s_tok, s_best are rewritten at the next position
  }
}

// ---------------------------------------------------------------------------------------------
// The argmax head's one-launch form, pipelined over two halves of the request block. A position
// runs as two stages, requests 0..31 then 32..63; stage s = 2k + h needs only the tokens of half
// h at position k - 1, so the hand-off of one half (its partials, the finishing reduction, the
// token) runs while the work-groups contract the other half's tiles. Work-group b < B finishes
// request b during the next stage (the other half's), between that stage's second and third
// tile; one stage past the last position finishes the last half. Everything else is the
// one-launch form above: the factor words of the work-group's tiles stay in registers, tagged
// words (the call's tag plus the stage) carry the partials and tokens, every wait is bounded.

// Stages the left-factor rows of half h's previous tokens p (rows 32 h + tid / 32 + 8 u) into sa,
// then waits for the whole work-group.
__device__ __forceinline__ void stage_half(uint16_t (*sa)[kARow], const int (&p)[4],
                                           const uint16_t* __restrict__ left, int R, int r0) {
  const int sw = threadIdx.x & 31, nw = R / 8;  // 16-byte words per row
  const int wd = sw < nw ? sw : nw - 1;
  v4u32 aw[4];
#pragma unroll
  for (int u = 0; u < 4; ++u)
    aw[u] = reinterpret_cast<const v4u32*>(left + (size_t)(p[u] >= 0 ? p[u] : 0) * R)[wd];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const bool ok = p[u] >= 0 && sw < nw;
    *reinterpret_cast<v4u32*>(&sa[r0 + (threadIdx.x >> 5) + 8 * u][8 * sw]) =
        ok ? aw[u] : v4u32{0u, 0u, 0u, 0u};
  }
  __syncthreads();
}

// Base logits that thread t finishes in a half's tile: row 32 h + t / 8 of the block, columns
// 8 (t % 8) .. + 7 of the tile (clamped into the batch and the vocabulary; the epilogue masks).
template <typename T>
struct HBase {
  static constexpr int kVec = 16 / (int)sizeof(T);  // logits per 16-byte vector
  static constexpr int kWords = 8 / kVec;           // vectors of the 8 logits
  v4u32 w[kWords];
};

template <typename T>
__device__ __forceinline__ float hlogit_at(const HBase<T>& bv, int e) {
  constexpr int kVec = HBase<T>::kVec, kPer32 = 4 / (int)sizeof(T);
  const uint32_t word = bv.w[e / kVec][(e % kVec) / kPer32];
  if constexpr (sizeof(T) == 4) return __uint_as_float(word);
  else return __uint_as_float((e & 1) ? (word & 0xffff0000u) : (word << 16));
}

template <typename T, bool VEC>
__device__ __forceinline__ void load_half(HBase<T>& bv, const T* __restrict__ base, int B, int K,
                                          int V, int k, int tile, int r0) {
  constexpr int kVec = HBase<T>::kVec;
  const int tid = threadIdx.x;
  int b = r0 + (tid >> 3);
  b = b < B ? b : B - 1;
  const T* row = base + ((size_t)b * K + k) * (size_t)V;
#pragma unroll
  for (int w = 0; w < HBase<T>::kWords; ++w) {
    const int v0 = tile * kStreamTile + 8 * (tid & 7) + w * kVec;
    if constexpr (VEC) {
      bv.w[w] = *reinterpret_cast<const v4u32*>(row + (v0 < V ? v0 : V - kVec));
    } else {
      uint32_t e[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        if constexpr (sizeof(T) == 4) {
          e[x] = __float_as_uint(row[v0 + x < V ? v0 + x : V - 1]);
        } else {
          const int v1 = v0 + 2 * x < V ? v0 + 2 * x : V - 1;
          const int v2 = v0 + 2 * x + 1 < V ? v0 + 2 * x + 1 : V - 1;
          e[x] = (uint32_t)row[v1] | ((uint32_t)row[v2] << 16);
        }
      }
      bv.w[w] = v4u32{e[0], e[1], e[2], e[3]};
    }
  }
}

// One tile for half h (rows 32 h .. 32 h + 31): every wave contracts its 16 columns for the
// half's two 16-row blocks; then thread t adds the base logits bv to row 32 h + t / 8, columns
// 8 (t % 8) .. + 7, writes the corrected logits and folds the argmax into (run, run_i) (every
// thread of a row holds the row's).
template <typename T, bool VEC, bool FULL>
__device__ __forceinline__ void pipe_tile(const ResArgs& a, T* __restrict__ out,
                                          uint16_t (*sa)[kARow], float (*sz)[kZRow], int k,
                                          int tile, const v4u32 (&f)[kSteps], const HBase<T>& bv,
                                          float& run, int& run_i, int h) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r0 = 32 * h;
  float4_t acc[2] = {{}, {}};
#pragma unroll
  for (int t = 0; t < kSteps; ++t) {
    if (FULL || t < a.ns) {  // uniform
      const bool inside = FULL || 4 * t + (lane >> 4) < a.R / 8;
      const bf16x8_t bfr = __builtin_bit_cast(bf16x8_t, inside ? f[t] : v4u32{0u, 0u, 0u, 0u});
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const v4u32 x = *reinterpret_cast<const v4u32*>(
            &sa[r0 + rb * 16 + (lane & 15)][32 * t + 8 * (lane >> 4)]);
        acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, x), bfr,
                                                          acc[rb], 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      sz[r0 + rb * 16 + 4 * (lane >> 4) + i][wave * 16 + (lane & 15)] = acc[rb][i];
  lds_barrier();
  const int m = r0 + (tid >> 3), q = tid & 7;
  const int v0 = tile * kStreamTile + 8 * q;
  if (r0 + 8 * wave < a.B) {  // uniform over the wave
    float z[8];
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const float4 acc4 = *reinterpret_cast<const float4*>(&sz[m][8 * q + 4 * x]);
      z[4 * x] = hlogit_at<T>(bv, 4 * x) + acc4.x;
      z[4 * x + 1] = hlogit_at<T>(bv, 4 * x + 1) + acc4.y;
      z[4 * x + 2] = hlogit_at<T>(bv, 4 * x + 2) + acc4.z;
      z[4 * x + 3] = hlogit_at<T>(bv, 4 * x + 3) + acc4.w;
    }
    const bool row_ok = m < a.B;
    const int ncol = a.V - v0;
    float best = -INFINITY;
    int e_best = -1;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const bool take = row_ok && e < ncol && z[e] > best;
      best = take ? z[e] : best;
      e_best = take ? e : e_best;
    }
    int bi = e_best < 0 ? INT_MAX : v0 + e_best;
    if (out != nullptr && row_ok) {
      T* orow = out + ((size_t)m * a.K + k) * (size_t)a.V + v0;
      if constexpr (VEC) {
        constexpr int kVec = HBase<T>::kVec;
#pragma unroll
        for (int w = 0; w < HBase<T>::kWords; ++w) {
          if (w * kVec < ncol) {
            if constexpr (sizeof(T) == 4) {
              *reinterpret_cast<float4*>(orow + 4 * w) =
                  make_float4(z[4 * w], z[4 * w + 1], z[4 * w + 2], z[4 * w + 3]);
            } else {
              uint32_t r[4];
#pragma unroll
              for (int x = 0; x < 4; ++x)
                r[x] = __builtin_bit_cast(uint32_t,
                                          bf16x2_t{(__bf16)z[2 * x], (__bf16)z[2 * x + 1]});
              *reinterpret_cast<v4u32*>(orow) = v4u32{r[0], r[1], r[2], r[3]};
            }
          }
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (e < ncol) Logit<T>::put(orow + e, z[e]);
      }
    }
    argmax_step<kDppXor1>(best, bi);
    argmax_step<kDppXor2>(best, bi);
    argmax_step<kDppHalfMirror>(best, bi);
    if (better(best, bi, run, run_i)) {
      run = best;
      run_i = bi;
    }
  }
  lds_barrier();  // sz is rewritten by the next tile
}

template <typename T, bool VEC, bool FULL>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void
markov_pipe(const T* __restrict__ base, T* __restrict__ out, ResArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t sa[kReqBlock][kARow];
  __shared__ __attribute__((aligned(16))) float sz[kReqBlock][kZRow];
  __shared__ int s_tok[kReqBlock];
  __shared__ float s_best[kWaves];
  __shared__ int s_bi[kWaves], s_late[kWaves];
  const int w = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // work-groups w < nfull own per tiles, the others per - 1 (the last B of them finish requests)
  const int t0 = w < a.nfull ? w * a.per : a.nfull * a.per + (w - a.nfull) * (a.per - 1);
  const int nit = w < a.nfull ? a.per : a.per - 1;
  const int fb = w - (a.nwg - a.B);  // the request this work-group finishes, if fb >= 0
  v4u32 f[kResItems][kSteps];
#pragma unroll
  for (int i = 0; i < kResItems; ++i) {
    const int tile = t0 + i < a.ntile ? t0 + i : a.ntile - 1;
    load_factor(f[i], a.right, a.V, a.R, tile);
  }
  const int nstage = 2 * a.K;
  for (int s = 0; s <= nstage; ++s) {
    const int k = s >> 1, h = s & 1, r0 = 32 * h;
    // the last stage only finishes; with at most 32 requests the second half has none
    const bool work = s < nstage && (h == 0 || a.B > 32);
    const uint32_t tg = a.tag + (uint32_t)s;
    HBase<T> bb[3];  // the base logits of the next two tiles in flight
    if (work) {
      load_half<T, VEC>(bb[0], base, a.B, a.K, a.V, k, t0 < a.ntile ? t0 : a.ntile - 1, r0);
      if (nit > 1) load_half<T, VEC>(bb[1], base, a.B, a.K, a.V, k, t0 + 1, r0);
      // 1. the half's previous tokens (the anchors at k = 0)
      if (tid >= r0 && tid < r0 + 32) {
        int x = -1;
        if (tid < a.B) {
          if (k == 0) {
            x = a.anchor != nullptr ? a.anchor[tid] : -1;
          } else {
            uint32_t pl;
            x = res_await(a.tok + tid, tg - 2u, pl) ? (int)pl : kResFailed;
          }
        }
        s_tok[tid] = x;
      }
      lds_barrier();
      int p[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int x = s_tok[r0 + (tid >> 5) + 8 * u];
        p[u] = (x >= 0 && x < a.V) ? x : -1;
      }
      stage_half(sa, p, a.left, a.R, r0);
    }
    float run = -INFINITY;
    int run_i = INT_MAX;
    // 2. the first two tiles
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      if (work && i < nit) {  // uniform
        if (i + 2 < nit) load_half<T, VEC>(bb[(i + 2) % 3], base, a.B, a.K, a.V, k, t0 + i + 2, r0);
        pipe_tile<T, VEC, FULL>(a, out, sa, sz, k, t0 + i, f[i], bb[i % 3], run, run_i, h);
      }
    }
    // 3. the work-group finishing request b, when b is in the other half: the previous stage
    if (s >= 1 && fb >= 0 && (fb >> 5) == ((s - 1) & 1)) {
      const int b = fb, kp = (s - 1) >> 1;
      const uint32_t tp = tg - 1u;
      float best = -INFINITY;
      int bi = INT_MAX;
      bool late = false;
      for (int j0 = 0; j0 < a.nwg; j0 += 2 * kThreads) {  // two partials per thread in flight
        const uint64_t* pp[2];
        uint64_t v[4];
        bool live[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int j = j0 + u * kThreads + tid;
          live[u] = j < a.nwg;
          pp[u] = a.part + ((size_t)b * a.nwg + (live[u] ? j : 0)) * 2;
          v[2 * u] = live[u] ? res_fetch(pp[u]) : (uint64_t)tp << 32;
          v[2 * u + 1] = live[u] ? res_fetch(pp[u] + 1) : (uint64_t)tp << 32;
        }
        for (int left = kResSpin;; --left) {
          bool all = true;
#pragma unroll
          for (int x = 0; x < 4; ++x) all = all && (uint32_t)(v[x] >> 32) == tp;
          if (all) break;
          if (left == 0) {
            late = true;
            break;
          }
          __builtin_amdgcn_s_sleep(2);
#pragma unroll
          for (int x = 0; x < 4; ++x)
            if ((uint32_t)(v[x] >> 32) != tp) v[x] = res_fetch(pp[x >> 1] + (x & 1));
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          if (live[u]) {
            const float z = __uint_as_float((uint32_t)v[2 * u]);
            const int i = (int)(uint32_t)v[2 * u + 1];
            if (better(z, i, best, bi)) {
              best = z;
              bi = i;
            }
          }
        }
      }
      wave_argmax(best, bi);
      const bool wave_late = __ballot(late) != 0;
      if (lane == 0) {
        s_best[wave] = best;
        s_bi[wave] = bi;
        s_late[wave] = wave_late;
      }
      lds_barrier();
      if (tid == 0) {
        bool any_late = false;
        for (int v = 0; v < kWaves; ++v) {
          any_late = any_late || s_late[v] != 0;
          if (better(s_best[v], s_bi[v], best, bi)) {
            best = s_best[v];
            bi = s_bi[v];
          }
        }
        // s_tok[b] still holds request b's previous token: only its own half's stages write it
        const bool failed = any_late || s_tok[b] == kResFailed;
        const int token = failed ? kResFailed : (bi == INT_MAX ? 0 : bi);
        a.tokens[(size_t)b * a.K + kp] = token;
        res_publish(a.tok + b, tp, (uint32_t)token);
      }
      lds_barrier();  // s_best is rewritten by the next finishing step
    }
    // 4. the remaining tiles
#pragma unroll
    for (int i = 2; i < kResItems; ++i) {
      if (work && i < nit) {  // uniform
        if (i + 2 < nit) load_half<T, VEC>(bb[(i + 2) % 3], base, a.B, a.K, a.V, k, t0 + i + 2, r0);
        pipe_tile<T, VEC, FULL>(a, out, sa, sz, k, t0 + i, f[i], bb[i % 3], run, run_i, h);
      }
    }
    // 5. this work-group's argmax of each of the half's requests
    if (work && (tid & 7) == 0 && r0 + (tid >> 3) < a.B) {
      uint64_t* pp = a.part + ((size_t)(r0 + (tid >> 3)) * a.nwg + w) * 2;
      res_publish(pp, tg, __float_as_uint(run));
      res_publish(pp + 1, tg, (uint32_t)run_i);
    }
    lds_barrier();  // s_tok is rewritten by the next stage
  }
}

// The per-position form's finishing launch for the sampled head: one work-group per request,
// after position k's tile launch (its draft row is complete in memory). Temperature 0: the
// argmax over the tile partials, as markov_finish. A drawing temperature: softmax(stored row /
// tau) by inverse CDF with the position's uniform (clamped to [0, 1], NaN as 0) in ascending
// vocabulary order; the row's largest stored value is the stored value of the largest tile
// partial (rounding keeps order); thread t sums the weights of a contiguous chunk of the row, the
// chunks are scanned in order, and the thread whose chunk holds the target walks it again (the
// same weights in the same order), else (rounding) the last entry with mass is taken. An invalid
// temperature: kInvalid.
template <typename T>
__global__ __launch_bounds__(kThreads) void markov_finish_sampled(
    const uint64_t* __restrict__ part, int ntile, int K, int V, int k, const T* __restrict__ out,
    const float* __restrict__ tau, const float* __restrict__ uni, int32_t* __restrict__ tokens) {
  __shared__ float s_best[kWaves], s_w[kWaves];
  __shared__ int s_bi[kWaves], s_i[kWaves];
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int32_t* tok = tokens + (size_t)b * K + k;
  const float t = tau[b];
  const bool draw = (double)t >= kTauMin && t < INFINITY;
  if (t != 0.0f && !draw) {  // uniform over the work-group
    if (tid == 0) *tok = kInvalid;
    return;
  }
  // the argmax over the tile partials (lowest index on ties)
  const uint64_t* prow = part + (size_t)b * ntile;
  float best = -INFINITY;
  int bi = INT_MAX;
  for (int t0 = 0; t0 < ntile; t0 += kThreads) {
    if (t0 + tid < ntile) {
      const uint64_t w = prow[t0 + tid];
      const float z = __uint_as_float((uint32_t)(w >> 32));
      const int i = (int)(uint32_t)w;
      if (better(z, i, best, bi)) {
        best = z;
        bi = i;
      }
    }
  }
  wave_argmax(best, bi);
  if (lane == 0) {
    s_best[wave] = best;
    s_bi[wave] = bi;
  }
  __syncthreads();
  for (int v = 0; v < kWaves; ++v)
    if (better(s_best[v], s_bi[v], best, bi)) {
      best = s_best[v];
      bi = s_bi[v];
    }
  if (!draw || bi == INT_MAX) {  // argmax, or no entry above -inf (token 0); uniform
    if (tid == 0) *tok = bi == INT_MAX ? 0 : bi;
    return;
  }
  const float m = Logit<T>::stored(best), c = (float)(kLog2e / (double)t);
  const T* row = out + ((size_t)b * K + k) * (size_t)V;
  const int chunk = (V + kThreads - 1) / kThreads;
  const int lo = tid * chunk < V ? tid * chunk : V;
  const int hi = lo + chunk < V ? lo + chunk : V;
  float sum = 0.0f;
  int lastw = -1;
#pragma unroll 8
  for (int v = lo; v < hi; ++v) {
    const float w = draw_weight(Logit<T>::get(row[v]), m, c);
    sum += w;
    lastw = w > 0.0f ? v : lastw;
  }
  float S;
  const float P = block_scan_excl(sum, s_w, S);
  const float u = uni[(size_t)b * K + k];
  const float target = (u > 0.0f ? fminf(u, 1.0f) : 0.0f) * S;
  const int owner = block_min_i(sum > 0.0f && P + sum > target ? tid : INT_MAX, s_i);
  const int last = -block_min_i(-lastw, s_i);
  if (owner == INT_MAX) {
    if (tid == 0) *tok = last >= 0 ? last : 0;
  } else if (tid == owner) {
    float cum = P;
    int pick = -1;
    for (int v = lo; v < hi && pick < 0; ++v) {
      const float w = draw_weight(Logit<T>::get(row[v]), m, c);
      if (w > 0.0f) {
        cum += w;
        pick = cum > target ? v : pick;
      }
    }
    *tok = pick >= 0 ? pick : lastw;
  }
}

bool aligned16(const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; }

// Compute units of the current device (cached per device; host threads that fill an entry at
// the same time store the same value).
int cu_count() {
  static std::atomic<int> cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// The argmax head takes the pipelined kernel (markov_pipe), the sampled head markov_resident.
template <typename T, bool SAMPLED>
const void* resident_kernel(bool full, bool vec_rows) {
  if constexpr (!SAMPLED)
    return full ? (vec_rows ? reinterpret_cast<const void*>(&markov_pipe<T, true, true>)
                            : reinterpret_cast<const void*>(&markov_pipe<T, false, true>))
                : (vec_rows ? reinterpret_cast<const void*>(&markov_pipe<T, true, false>)
                            : reinterpret_cast<const void*>(&markov_pipe<T, false, false>));
  else
    return full ? (vec_rows ? reinterpret_cast<const void*>(&markov_resident<T, true, true, true>)
                            : reinterpret_cast<const void*>(&markov_resident<T, false, true, true>))
                : (vec_rows ? reinterpret_cast<const void*>(&markov_resident<T, true, false, true>)
                            : reinterpret_cast<const void*>(&markov_resident<T, false, false, true>));
}

// The one-launch form (markov_resident) when it applies: up to 64 requests, ranks up to 256,
// every tile of the vocabulary in a resident work-group's registers (at most kResItems each),
// and at least one work-group per request (the sampled form: at most kDecideLoads * kThreads
// work-groups, the partials one decision reads). Sets the kernel, tiles per work-group and
// work-groups; returns false when it does not apply.
template <typename T, bool SAMPLED>
bool resident_plan(int B, int V, int R, bool vec_rows, const void** fn, int* per, int* nwg) {
  if (B > kReqBlock || R > kRankChunk) return false;
  const int ntile = (V + kStreamTile - 1) / kStreamTile;
  *fn = resident_kernel<T, SAMPLED>(R == kRankChunk, vec_rows);
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, *fn, kThreads, 0) != hipSuccess ||
      per_cu < 1)
    return false;
  // the tiles over up to ntile + B work-groups, balanced (the sampled head: at most the
  // kDecideLoads * kThreads partials a draw decision reads)
  int cap = per_cu * cu_count();
  if (SAMPLED && cap > kDecideLoads * kThreads) cap = kDecideLoads * kThreads;
  const long want = (long)ntile + B;
  const int n = want < cap ? (int)want : cap;
  *per = (ntile + n - 1) / n;
  if (*per > kResItems || n < B) return false;
  *nwg = n;
  return true;
}

// Workspace of one launch of the one-launch form: [B][nwg][2] tagged partials, [B] tagged
// tokens, [B][2] tagged draw decisions. The launch is cooperative: the runtime either makes every
// work-group of the grid resident at once, which the waits between work-groups rely on, or
// refuses the launch. Returns SV_OK, SV_ERR_UNSUPPORTED when the cooperative launch was refused
// (nothing was enqueued but, possibly, the workspace's zero fill), or SV_ERR_HIP.
template <typename T, bool SAMPLED>
int launch_resident_plan(const void* fn, int per, int nwg, const void* base, void* out, int B,
                         int K, int V, const uint16_t* left, const uint16_t* right, int R,
                         const int32_t* anchor, const float* tau, const float* uni,
                         int32_t* tokens, uint64_t* ws, size_t ws_bytes, hipStream_t s) {
  ResArgs a;
  a.B = B;
  a.K = K;
  a.V = V;
  a.R = R;
  a.ns = (R + 31) / 32;
  a.ntile = (V + kStreamTile - 1) / kStreamTile;
  a.per = per;
  a.nwg = nwg;
  a.nfull = a.ntile - (per - 1) * nwg;  // work-groups with per tiles (1 .. nwg)
  a.left = left;
  a.right = right;
  a.anchor = anchor;
  a.tokens = tokens;
  a.part = ws;
  a.tok = ws + (size_t)2 * B * nwg;
  a.dec = a.tok + B;
  a.tau = tau;
  a.uni = uni;
  const int st = sv_internal_call_tags((uint32_t)(2 * K + 2), ws, ws_bytes, s, &a.tag);
  if (st != SV_OK) return st;
  const T* base_t = static_cast<const T*>(base);
  T* out_t = static_cast<T*>(out);
  void* args[] = {&base_t, &out_t, &a};
  const hipError_t e = hipLaunchCooperativeKernel(fn, dim3(nwg), dim3(kThreads), args, 0, s);
  if (e == hipSuccess) return SV_OK;
  (void)hipGetLastError();  // clear the refusal; the caller takes another form
  return sv_internal_fail(SV_ERR_UNSUPPORTED, hipGetErrorString(e));
}

// SV_ERR_UNSUPPORTED when the one-launch form does not apply or its launch was refused.
template <typename T>
int launch_resident(const void* base, void* out, int B, int K, int V, const uint16_t* left,
                    const uint16_t* right, int R, const int32_t* anchor, int32_t* tokens,
                    uint64_t* ws, size_t ws_bytes, bool vec_rows, hipStream_t s) {
  const void* fn = nullptr;
  int per = 0, nwg = 0;
  if (!resident_plan<T, false>(B, V, R, vec_rows, &fn, &per, &nwg)) return SV_ERR_UNSUPPORTED;
  return launch_resident_plan<T, false>(fn, per, nwg, base, out, B, K, V, left, right, R, anchor,
                                        nullptr, nullptr, tokens, ws, ws_bytes, s);
}

// tau, uni non-NULL: the sampled head in the per-position form (the finishing launch draws).
template <typename T>
int launch_all(const void* base, void* out, int B, int K, int V, const uint16_t* left,
               const uint16_t* right, int R, const int32_t* anchor, int32_t* tokens,
               uint64_t* part, size_t ws_bytes, hipStream_t s, const float* tau = nullptr,
               const float* uni = nullptr) {
  const int nrb = (B + kReqBlock - 1) / kReqBlock;
  const bool stream = R <= kRankChunk;
  const int ntile = stream ? (V + kStreamTile - 1) / kStreamTile : (V + kTileV - 1) / kTileV;
  const int n = ntile * nrb;
  const int groups = 8 * ((n + 7) / 8);
  const bool vec_rows = aligned16(base) && aligned16(out) && ((size_t)V * sizeof(T)) % 16 == 0;
  if (tau == nullptr && B <= 2 * kReqBlock) {
    // up to 64 requests: one launch; up to 128: one-launch calls of up to 64 requests in turn
    // (measured faster there than the per-position form, which reads the factor for every
    // 64-request block at every position; at 256 requests the two are equal). A refused
    // cooperative launch falls through to the per-position form below.
    const void* fn0 = nullptr;
    int per0 = 0, nwg0 = 0;
    if (resident_plan<T, false>(B < kReqBlock ? B : kReqBlock, V, R, vec_rows, &fn0, &per0,
                                &nwg0)) {
      int st = SV_OK;
      for (int b0 = 0; b0 < B && st == SV_OK; b0 += kReqBlock) {
        const int nb = B - b0 < kReqBlock ? B - b0 : kReqBlock;
        const size_t off = (size_t)b0 * K * V * sizeof(T);
        st = launch_resident<T>(static_cast<const char*>(base) + off,
                                out != nullptr ? static_cast<char*>(out) + off : nullptr, nb, K,
                                V, left, right, R, anchor != nullptr ? anchor + b0 : nullptr,
                                tokens + (size_t)b0 * K, part, ws_bytes, vec_rows, s);
      }
      if (st == SV_OK) {
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return sv_internal_fail(SV_ERR_HIP, hipGetErrorString(e));
        return SV_OK;
      }
      if (st != SV_ERR_UNSUPPORTED) return st;
      // a launch was refused: the per-position form below recomputes every request (in stream
      // order after any block that did run)
      sv_internal_clear_error();
    }
  }
  // per-position form: its per-tile argmaxes are untagged words
  sv_internal_untagged_use(part);
  // persistent form: as many work-groups as are resident at once, each a contiguous run of
  // equally many items
  const bool full = R == kRankChunk;
  const void* fn = full ? (vec_rows ? reinterpret_cast<const void*>(&markov_stream<T, true, true>)
                                    : reinterpret_cast<const void*>(&markov_stream<T, false, true>))
                        : (vec_rows ? reinterpret_cast<const void*>(&markov_stream<T, true, false>)
                                    : reinterpret_cast<const void*>(&markov_stream<T, false, false>));
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kThreads, 0) != hipSuccess ||
      per_cu < 1)
    per_cu = 1;
  const int slots = per_cu * cu_count();
  const int per = (n + slots - 1) / slots;
  const int pgroups = 8 * (((n + per - 1) / per + 7) / 8);
  for (int k = 0; k < K; ++k) {
    const int32_t* prev = k == 0 ? anchor : tokens + (k - 1);
    const int stride = k == 0 ? 1 : K;
    if (stream) {
      const StreamArgs a{B, K, V, k, R, (R + 31) / 32, ntile, stride, left, right, prev, part};
      hipLaunchKernelGGL(reinterpret_cast<void (*)(const T*, T*, StreamArgs, int, int)>(
                             const_cast<void*>(fn)),
                         dim3(pgroups), dim3(kThreads), 0, s, static_cast<const T*>(base),
                         static_cast<T*>(out), a, nrb, per);
    } else {
      hipLaunchKernelGGL(markov_bias_tile<T>, dim3(groups), dim3(kThreads), 0, s,
                         static_cast<const T*>(base), static_cast<T*>(out), B, K, V, k, left,
                         right, R, prev, stride, part, ntile, nrb);
    }
    if (tau != nullptr)
      hipLaunchKernelGGL(markov_finish_sampled<T>, dim3(B), dim3(kThreads), 0, s, part, ntile, K,
                         V, k, static_cast<const T*>(out), tau, uni, tokens);
    else
      hipLaunchKernelGGL(markov_finish, dim3(B), dim3(kThreads), 0, s, part, ntile, K, k, tokens);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return sv_internal_fail(SV_ERR_HIP, hipGetErrorString(e));
  return SV_OK;
}

// The sampled head: the one-launch form in blocks of up to 64 requests, one launch per block,
// in order on the stream (each block's launch reuses the workspace under its own tag).
template <typename T>
int launch_sampled(const void* base, void* out, int B, int K, int V, const uint16_t* left,
                   const uint16_t* right, int R, const int32_t* anchor, const float* tau,
                   const float* uni, int32_t* tokens, uint64_t* ws, size_t ws_bytes,
                   hipStream_t s) {
  const bool vec_rows = aligned16(base) && aligned16(out) && ((size_t)V * sizeof(T)) % 16 == 0;
  {
    const void* fn = nullptr;
    int per = 0, nwg = 0;
    if (!resident_plan<T, true>(B < kReqBlock ? B : kReqBlock, V, R, vec_rows, &fn, &per, &nwg))
      return launch_all<T>(base, out, B, K, V, left, right, R, anchor, tokens, ws, ws_bytes, s,
                           tau, uni);
  }
  for (int b0 = 0; b0 < B; b0 += kReqBlock) {
    const int nb = B - b0 < kReqBlock ? B - b0 : kReqBlock;
    const void* fn = nullptr;
    int per = 0, nwg = 0;
    if (!resident_plan<T, true>(nb, V, R, vec_rows, &fn, &per, &nwg))
      return sv_internal_fail(SV_ERR_UNSUPPORTED, "a request block did not fit one launch");
    const size_t off = (size_t)b0 * K * V * sizeof(T);
    const int st = launch_resident_plan<T, true>(
        fn, per, nwg, static_cast<const char*>(base) + off, static_cast<char*>(out) + off, nb, K,
        V, left, right, R, anchor != nullptr ? anchor + b0 : nullptr, tau + b0,
        uni + (size_t)b0 * K, tokens + (size_t)b0 * K, ws, ws_bytes, s);
    if (st == SV_ERR_UNSUPPORTED && b0 == 0) {  // cooperative launch refused: per-position form
      sv_internal_clear_error();
      return launch_all<T>(base, out, B, K, V, left, right, R, anchor, tokens, ws, ws_bytes, s,
                           tau, uni);
    }
    if (st != SV_OK) return st;
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return sv_internal_fail(SV_ERR_HIP, hipGetErrorString(e));
  return SV_OK;
}

}  // namespace

extern "C" size_t sv_markov_workspace_bytes(int B, int V) {
  if (B < 1 || V < 1) return 0;
  const size_t ntile = (V + kStreamTile - 1) / kStreamTile;
  const size_t per_position = (size_t)B * ntile * 8;  // tile partials of the per-position form
  // one launch of the one-launch forms (at most 64 requests): [Bl][nwg][2] tagged partials
  // (nwg <= ntile + Bl), [Bl] tagged tokens, [Bl][2] tagged draw decisions
  const size_t Bl = B < kReqBlock ? (size_t)B : (size_t)kReqBlock;
  const size_t one_launch = Bl * (ntile + Bl) * 16 + Bl * 8 + Bl * 16;
  return per_position > one_launch ? per_position : one_launch;
}

extern "C" int sv_markov_draft_sampled(const void* base_logits, int dtype, int B, int K, int V,
                                       const uint16_t* left_factor, const uint16_t* right_factor,
                                       int R, const int32_t* anchor, const float* temperature,
                                       const float* uniforms, int32_t* draft_tokens,
                                       void* draft_logits, void* workspace, size_t workspace_bytes,
                                       void* stream) {
  sv_internal_clear_error();
  if (B < 1 || B > (1 << 20) || K < 1 || K > 64 || V < 1 || V > (1 << 26))
    return sv_internal_fail(SV_ERR_INVALID_ARG, "need 1 <= B <= 2^20, 1 <= K <= 64, 1 <= V <= 2^26");
  if (dtype != SV_DTYPE_F32 && dtype != SV_DTYPE_BF16)
    return sv_internal_fail(SV_ERR_INVALID_ARG, "dtype must be SV_DTYPE_F32 or SV_DTYPE_BF16");
  if (R < 16 || R > kMaxRank || R % 16 != 0)
    return sv_internal_fail(SV_ERR_INVALID_ARG, "rank R must be a multiple of 16 in [16, 1024]");
  if (!base_logits || !left_factor || !right_factor || !temperature || !uniforms ||
      !draft_tokens || !draft_logits)
    return sv_internal_fail(SV_ERR_INVALID_ARG, "a required pointer is NULL");
  if (reinterpret_cast<uintptr_t>(left_factor) % 16 || reinterpret_cast<uintptr_t>(right_factor) % 16)
    return sv_internal_fail(SV_ERR_INVALID_ARG, "factors must be 16-byte aligned");
  const size_t need = sv_markov_workspace_bytes(B, V);
  if (!workspace || workspace_bytes < need || reinterpret_cast<uintptr_t>(workspace) % 256)
    return sv_internal_fail(SV_ERR_WORKSPACE, "workspace missing, too small or not 256-byte aligned");
  if ((long)((V + kStreamTile - 1) / kStreamTile) * ((B + kReqBlock - 1) / kReqBlock) >= (1L << 30))
    return sv_internal_fail(SV_ERR_UNSUPPORTED, "grid too large");
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint64_t* ws = static_cast<uint64_t*>(workspace);
  if (dtype == SV_DTYPE_F32)
    return launch_sampled<float>(base_logits, draft_logits, B, K, V, left_factor, right_factor, R,
                                 anchor, temperature, uniforms, draft_tokens, ws, workspace_bytes,
                                 s);
  return launch_sampled<uint16_t>(base_logits, draft_logits, B, K, V, left_factor, right_factor,
                                  R, anchor, temperature, uniforms, draft_tokens, ws,
                                  workspace_bytes, s);
}

extern "C" int sv_markov_draft(const void* base_logits, int dtype, int B, int K, int V,
                               const uint16_t* left_factor, const uint16_t* right_factor, int R,
                               const int32_t* anchor, int32_t* draft_tokens, void* draft_logits,
                               void* workspace, size_t workspace_bytes, void* stream) {
  sv_internal_clear_error();
  if (B < 1 || B > (1 << 20) || K < 1 || K > 64 || V < 1 || V > (1 << 26))
    return sv_internal_fail(SV_ERR_INVALID_ARG, "need 1 <= B <= 2^20, 1 <= K <= 64, 1 <= V <= 2^26");
  if (dtype != SV_DTYPE_F32 && dtype != SV_DTYPE_BF16)
    return sv_internal_fail(SV_ERR_INVALID_ARG, "dtype must be SV_DTYPE_F32 or SV_DTYPE_BF16");
  if (R < 16 || R > kMaxRank || R % 16 != 0)
    return sv_internal_fail(SV_ERR_INVALID_ARG, "rank R must be a multiple of 16 in [16, 1024]");
  if (!base_logits || !left_factor || !right_factor || !draft_tokens)
    return sv_internal_fail(SV_ERR_INVALID_ARG, "a required pointer is NULL");
  if (reinterpret_cast<uintptr_t>(left_factor) % 16 || reinterpret_cast<uintptr_t>(right_factor) % 16)
    return sv_internal_fail(SV_ERR_INVALID_ARG, "factors must be 16-byte aligned");
  const size_t need = sv_markov_workspace_bytes(B, V);
  if (!workspace || workspace_bytes < need || reinterpret_cast<uintptr_t>(workspace) % 256)
    return sv_internal_fail(SV_ERR_WORKSPACE, "workspace missing, too small or not 256-byte aligned");
  if ((long)((V + kStreamTile - 1) / kStreamTile) * ((B + kReqBlock - 1) / kReqBlock) >= (1L << 30))
    return sv_internal_fail(SV_ERR_UNSUPPORTED, "grid too large");
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint64_t* part = static_cast<uint64_t*>(workspace);
  if (dtype == SV_DTYPE_F32)
    return launch_all<float>(base_logits, draft_logits, B, K, V, left_factor, right_factor, R,
                             anchor, draft_tokens, part, workspace_bytes, s);
  return launch_all<uint16_t>(base_logits, draft_logits, B, K, V, left_factor, right_factor, R,
                              anchor, draft_tokens, part, workspace_bytes, s);
}
