// Confidence-scheduled prefix selection for libsv (declared in sv.h): how many draft tokens of
// each request go to verification ("DSpark" paper review, 4.2.1 Confidence Head and 4.2.2
// Hardware-Aware Prefix Scheduler). It runs on the device so that confidences from the drafter,
// the chosen lengths and the flattened row starts of the verify call never cross to the host.
//
// Hardware-aware mode, one launch of ceil(B*K / 8) ranking groups and one finishing group:
//   * every group loads the B*K confidences and forms, in LDS, the survivals
//     s[b][k] = c[b][0] * ... * c[b][k] (clamped to [0, 1], NaN = 0, float32 products left to
//     right) and each request's exclusive fp64 prefix sums of them, position-major with a row
//     stride SB of B rounded up to a multiple of 32 (request r of any row sits in bank r mod 32:
//     lanes that work on consecutive requests never collide, whatever positions they read).
//     A request's survivals never increase along its block, so its tokens are already in rank
//     order.
//   * ranking group g takes tokens 8g .. 8g+7, half a wave per token. The tokens ranked before
//     token e = (b, k) (higher survival, then earlier position, then lower request) form a
//     prefix of every request's block; lane l binary-searches the blocks of requests l, l+32, ...
//     for that prefix (eight searches in lockstep, a fixed ladder of steps) and adds its length
//     and its survival sum. Summed over the half-wave: the rank of e and the sum of every
//     survival ranked before it. So token e is the N-th ranked, N = rank + 1, and
//     E(N) = B + that sum + s[b][k]: the rate of cutting after e is E(N) / step_time[B + N].
//     No sort: each token's place comes from B binary searches.
//     The group's best (largest rate, then smallest N) is published as tagged words.
//   * the finishing group, last in the grid, adds N = 0 (no drafts, rate B / step_time[B]),
//     awaits every ranking group's best, keeps the best of all, and gives request b the tokens
//     of its block ranked at or before the chosen token (one binary search per request).
// Threshold mode, the finishing group alone: request b keeps its drafts up to the first
// confidence below the threshold.
// Both modes end with num_draft and the flattened row starts (exclusive sums of k_b + 1 and of
// k_b).

#include <hip/hip_runtime.h>

#include <float.h>
#include <limits.h>
#include <math.h>
#include <stdint.h>

#include "sv.h"
#include "sv_internal.h"

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kTokensPerGroup = 8;    // tokens ranked by one ranking group
constexpr int kThreadsPerToken = 32;  // kThreads / kTokensPerGroup: half a wave per token
constexpr int kBatch = 8;             // binary searches in flight per thread
constexpr int kMaxTokens = 4096;      // B * K, at most
constexpr int kMaxK = 64;
constexpr int kWordsPerGroup = 3;     // a ranking group's best: rate (2 words), N and token
constexpr int kSpinLimit = 1 << 21;   // polls (about 1 us each) before the finisher gives up
constexpr int kPollSleep = 2;         // s_sleep units between two polls

__device__ __forceinline__ float clamp01(float c) {
  if (!(c > 0.0f)) return 0.0f;  // NaN and non-positive values
  return c < 1.0f ? c : 1.0f;
}

__device__ __forceinline__ void publish(uint64_t* p, uint32_t tag, uint32_t payload) {
  __hip_atomic_store(p, ((uint64_t)tag << 32) | payload, __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t fetch(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Row stride of the LDS tables: B rounded up to a multiple of 32 when K such rows fit in
// kMaxTokens + kMaxK entries, else B + 1 (a few shapes with B just above a multiple of 32 and K
// near 64).
__device__ __forceinline__ int row_stride(int B, int K) {
  const int padded = (B + 31) & ~31;
  return K * padded <= kMaxTokens + kMaxK ? padded : B + 1;
}

// Survivals s[k*SB + b] and exclusive prefix sums P[k*SB + b] = s[b][0] + ... + s[b][k-1] (fp64,
// left to right) of every request, in LDS.
__device__ void survivals(const float* __restrict__ conf, int B, int K, float* s, double* P) {
  const int SB = row_stride(B, K);
  for (int b = threadIdx.x; b < B; b += kThreads) {
    const float* c = conf + (size_t)b * K;
    float acc = 1.0f;
    double run = 0.0;
#pragma unroll 8
    for (int k = 0; k < K; ++k) {
      acc = acc * clamp01(c[k]);
      s[k * SB + b] = acc;
      P[k * SB + b] = run;
      run += (double)acc;
    }
  }
  __syncthreads();
}

// Whether token (j, r) with survival s1 is ranked before token (k, b) with survival sv: higher
// survival, then earlier position, then lower request. Formed without branches: a short-circuit
// form of it, inlined into the unrolled searches, compiled to code that dropped the tied case.
__device__ __forceinline__ bool ranked_before(float s1, int j, int r, float sv, int k, int b) {
  return (s1 > sv) | ((s1 == sv) & ((j < k) | ((j == k) & (r < b))));
}

// The ladder of a search over K tokens: the largest power of two <= K, then halves. Each step
// tests the last of the next `step` tokens; they are all ranked before the searched token
// exactly when that one is, since those that are form a prefix of every block.
__device__ __forceinline__ int ladder_top(int K) {
  int top = 1;
  while (top * 2 <= K) top *= 2;
  return top;
}

// Number of tokens of request r's block ranked before token (b, k) with survival sv.
__device__ __forceinline__ int prefix_before(const float* s, int SB, int K, int r, float sv, int k,
                                             int b) {
  int lo = 0;
  for (int step = ladder_top(K); step >= 1; step >>= 1) {
    const int j = lo + step - 1;
    const float s1 = s[(j < K ? j : K - 1) * SB + r];
    lo += ((j < K) & ranked_before(s1, j, r, sv, k, b)) ? step : 0;
  }
  return lo;
}

// The better of two candidate cuts: the larger rate, then the smaller N; n < 0 marks none.
__device__ __forceinline__ bool better(double r1, int n1, double r2, int n2) {
  if (n1 < 0) return false;
  if (n2 < 0) return true;
  return r1 > r2 || (r1 == r2 && n1 < n2);
}

struct Cut {
  double rate;
  int n;    // tokens verified; -1: none usable
  int tok;  // b * K + k of the N-th ranked token (n > 0)
};

// Cross-lane moves inside the vector ALU (DPP). A lane whose source lies outside its row of 16,
// or whose row the mask leaves out, gets `identity`.
constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118;
constexpr int kRowBcast15 = 0x142, kRowBcast31 = 0x143;

template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x, uint32_t identity) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)identity, (int)x, CTRL, ROWS, 0xf, false);
}
template <int CTRL, int ROWS>
__device__ __forceinline__ double dpp_f64(double x, double identity) {
  const uint64_t v = (uint64_t)__double_as_longlong(x);
  const uint64_t d = (uint64_t)__double_as_longlong(identity);
  const uint32_t lo = dpp_u32<CTRL, ROWS>((uint32_t)v, (uint32_t)d);
  const uint32_t hi = dpp_u32<CTRL, ROWS>((uint32_t)(v >> 32), (uint32_t)(d >> 32));
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Inclusive scans with DPP: every lane combines the lanes 1, 2, 4 and 8 below it in its row,
// then lane 15 of rows 0 and 2 is folded into rows 1 and 3 (lane 31 then holds lanes 0..31, lane
// 63 lanes 32..63) and, for a whole-wave scan, lane 31 into rows 2 and 3 (lane 63: the wave).
#define SV_HALF_SCAN(STEP) \
  STEP(kRowShr1, 0xf);     \
  STEP(kRowShr2, 0xf);     \
  STEP(kRowShr4, 0xf);     \
  STEP(kRowShr8, 0xf);     \
  STEP(kRowBcast15, 0xa)

__device__ __forceinline__ int half_sum_i32(int x) {  // inclusive scans of the two halves
#define SV_STEP(C, R) x += (int)dpp_u32<C, R>((uint32_t)x, 0u)
  SV_HALF_SCAN(SV_STEP);
#undef SV_STEP
  return x;
}
__device__ __forceinline__ double half_sum_f64(double x) {
#define SV_STEP(C, R) x += dpp_f64<C, R>(x, 0.0)
  SV_HALF_SCAN(SV_STEP);
#undef SV_STEP
  return x;
}
__device__ __forceinline__ double wave_max_f64(double x) {
#define SV_STEP(C, R) x = fmax(x, dpp_f64<C, R>(x, -INFINITY))
  SV_HALF_SCAN(SV_STEP);
  SV_STEP(kRowBcast31, 0xc);
#undef SV_STEP
  const uint64_t v = (uint64_t)__double_as_longlong(x);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 63);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 63);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
__device__ __forceinline__ int wave_scan_i32(int x) {  // inclusive; lane 63 holds the total
  x = half_sum_i32(x);
  return x + (int)dpp_u32<kRowBcast31, 0xc>((uint32_t)x, 0u);
}
__device__ __forceinline__ int wave_min_i32(int x) {
#define SV_STEP(C, R) x = min(x, (int)dpp_u32<C, R>((uint32_t)x, (uint32_t)INT_MAX))
  SV_HALF_SCAN(SV_STEP);
  SV_STEP(kRowBcast31, 0xc);
#undef SV_STEP
  return __builtin_amdgcn_readlane(x, 63);
}

// Best cut over the wave, in every lane: the largest rate, then the smallest N among the lanes
// that hold it (every N belongs to one token, so that lane's token comes with it).
__device__ __forceinline__ Cut wave_best(const Cut& c) {
  const double r = wave_max_f64(c.n < 0 ? -INFINITY : c.rate);
  const int n = wave_min_i32(c.n >= 0 && c.rate == r ? c.n : INT_MAX);
  const uint64_t who = __ballot(c.n >= 0 && c.n == n);
  if (who == 0) return Cut{-INFINITY, -1, 0};
  const int src = __ffsll((long long)who) - 1;
  return Cut{r, n, __builtin_amdgcn_readlane(c.tok, src)};
}

// Best cut over the block; every thread gets it. red holds kWaves entries.
__device__ Cut block_best(Cut c, Cut* red) {
  c = wave_best(c);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[wave] = c;
  __syncthreads();
  c = red[0];
  for (int w = 1; w < kWaves; ++w)
    if (better(red[w].rate, red[w].n, c.rate, c.n)) c = red[w];
  return c;
}

// Exclusive block scan of one int per thread; red holds kWaves ints; *total gets the sum.
__device__ int block_exclusive_scan(int v, int* red, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int x = wave_scan_i32(v);
  __syncthreads();
  if (lane == 63) red[wave] = x;
  __syncthreads();
  int before = 0, all = 0;
  for (int w = 0; w < kWaves; ++w) {
    if (w < wave) before += red[w];
    all += red[w];
  }
  *total = all;
  return before + x - v;
}

__global__ __launch_bounds__(kThreads) void sv_schedule_kernel(
    const float* __restrict__ conf, int B, int K, const float* __restrict__ step_time,
    float threshold, uint64_t* words, uint32_t tag, int32_t* num_draft, int32_t* t_start,
    int32_t* d_start, float* summary) {
  __shared__ float s[kMaxTokens + kMaxK];
  __shared__ double P[kMaxTokens + kMaxK];  // later: per-request counts (int)
  __shared__ Cut red_cut[kWaves];
  __shared__ int red_i[kWaves];
  __shared__ int s_late;
  const int M = B * K, SB = row_stride(B, K);
  const int n_rank = (M + kTokensPerGroup - 1) / kTokensPerGroup;
  const bool hardware = step_time != nullptr;
  const int tid = threadIdx.x;

  if (hardware) survivals(conf, B, K, s, P);

  if (hardware && (int)blockIdx.x < n_rank) {
    // ranking group
    const int e = (int)blockIdx.x * kTokensPerGroup + tid / kThreadsPerToken;
    const int l = tid % kThreadsPerToken;
    Cut c{-INFINITY, -1, 0};
    if (e < M) {
      const int b = e / K, k = e % K;
      const float sv = s[k * SB + b];
      const int top = ladder_top(K);
      const int last_row = (K - 1) * SB;
      int cnt = 0;
      double sum = 0.0;
      // Token (j, r) is ranked before e exactly when the 64-bit key (survival bits, 65 - j)
      // exceeds (sv bits, 65 - k - [r < b]): survivals are non-negative, so their bits order
      // like their values, and among equal survivals the earlier position (then, at the same
      // position, the lower request) comes first.
      const uint64_t sv_hi = (uint64_t)__float_as_uint(sv) << 32;
      for (int r0 = l; r0 < B; r0 += kThreadsPerToken * kBatch) {
        int lo[kBatch];
        uint64_t key_e[kBatch];
#pragma unroll
        for (int i = 0; i < kBatch; ++i) {
          const int r = r0 + i * kThreadsPerToken;
          lo[i] = 0;
          // no token passes this key when r >= B
          key_e[i] = r < B ? sv_hi | (uint32_t)(kMaxK + 1 - k - (r < b ? 1 : 0)) : ~0ull;
        }
        // lo[i] = tokens of request r0 + i*32 ranked before e (prefix_before, eight in lockstep)
        for (int step = top; step >= 1; step >>= 1) {
#pragma unroll
          for (int i = 0; i < kBatch; ++i) {
            const int j = lo[i] + step - 1;
            const int col = min(r0 + i * kThreadsPerToken, B - 1);
            const float s1 = s[__umul24(min(j, K - 1), SB) + col];
            const uint64_t key = ((uint64_t)__float_as_uint(s1) << 32) | (uint32_t)(kMaxK + 1 - j);
            lo[i] += ((j < K) & (key > key_e[i])) ? step : 0;
          }
        }
#pragma unroll
        for (int i = 0; i < kBatch; ++i) {
          const int r = r0 + i * kThreadsPerToken, p = lo[i];
          if (r < B) {
            cnt += p;
            sum += p < K ? P[p * SB + r] : P[last_row + r] + (double)s[last_row + r];
          }
        }
      }
      // token totals: lane 31 of each half-wave
      cnt = half_sum_i32(cnt);
      sum = half_sum_f64(sum);
      if (l == kThreadsPerToken - 1) {
        const int n = cnt + 1;
        const float t = step_time[B + n];
        if (isfinite(t) && t > 0.0f) c = Cut{((double)B + sum + (double)sv) / (double)t, n, e};
      }
    }
    c = block_best(c, red_cut);
    if (tid == 0) {
      const uint64_t bits = (uint64_t)__double_as_longlong(c.rate);
      uint64_t* w = words + (size_t)blockIdx.x * kWordsPerGroup;
      publish(w, tag, (uint32_t)(bits >> 32));
      publish(w + 1, tag, (uint32_t)bits);
      publish(w + 2, tag, ((uint32_t)(c.n + 1) << 12) | (uint32_t)c.tok);
    }
    return;
  }

  // finishing group: counts[b] in the LDS of P
  int* count = reinterpret_cast<int*>(P);
  float chosen_rate = 0.0f;
  int chosen_n = 0;
  bool late = false;
  if (!hardware) {
    for (int b = tid; b < B; b += kThreads) {
      int k = K;
      for (int i = 0; i < K; ++i) {
        if (clamp01(conf[(size_t)b * K + i]) < threshold) {
          k = i;
          break;
        }
      }
      count[b] = k;
    }
  } else {
    Cut c{-INFINITY, -1, 0};
    if (tid == 0) {  // N = 0: no drafts
      const float t0 = step_time[B];
      if (isfinite(t0) && t0 > 0.0f) c = Cut{(double)B / (double)t0, 0, 0};
    }
    for (int g = tid; g < n_rank; g += kThreads) {
      const uint64_t* w = words + (size_t)g * kWordsPerGroup;
      uint64_t w0 = fetch(w), w1 = fetch(w + 1), w2 = fetch(w + 2);
      int left = kSpinLimit;
      while (left > 0 && ((uint32_t)(w0 >> 32) != tag || (uint32_t)(w1 >> 32) != tag ||
                          (uint32_t)(w2 >> 32) != tag)) {
        __builtin_amdgcn_s_sleep(kPollSleep);
        if ((uint32_t)(w0 >> 32) != tag) w0 = fetch(w);
        if ((uint32_t)(w1 >> 32) != tag) w1 = fetch(w + 1);
        if ((uint32_t)(w2 >> 32) != tag) w2 = fetch(w + 2);
        --left;
      }
      if (left == 0) {
        late = true;
        continue;
      }
      const Cut o{__longlong_as_double((long long)(((w0 & 0xffffffffull) << 32) |
                                                  (w1 & 0xffffffffull))),
                  (int)((uint32_t)w2 >> 12) - 1, (int)((uint32_t)w2 & 0xfff)};
      if (better(o.rate, o.n, c.rate, c.n)) c = o;
    }
    if (tid == 0) s_late = 0;
    __syncthreads();
    if (late) s_late = 1;
    c = block_best(c, red_cut);  // its barriers also order s_late
    late = s_late != 0;
    chosen_n = late || c.n < 0 ? 0 : c.n;
    chosen_rate = late || c.n < 0 ? 0.0f : (float)c.rate;
    const int bs = c.tok / K, ks = c.tok % K;
    const float ss = s[ks * SB + bs];
    __syncthreads();  // every thread is done with P before it holds counts
    for (int b = tid; b < B; b += kThreads)
      count[b] = chosen_n == 0 ? 0 : prefix_before(s, SB, K, b, ss, ks, bs) + (b == bs ? 1 : 0);
  }
  __syncthreads();

  // num_draft and row starts: thread t takes requests [t*per, (t+1)*per)
  const int per = (B + kThreads - 1) / kThreads;
  const int b0 = tid * per < B ? tid * per : B, b1 = b0 + per < B ? b0 + per : B;
  int my_t = 0, my_d = 0;
  for (int b = b0; b < b1; ++b) {
    my_t += count[b] + 1;
    my_d += count[b];
  }
  // one scan for both sums: target rows in the high 16 bits, draft rows in the low 16 (the
  // totals, at most B + B*K <= 8192 and B*K <= 4096, never carry across)
  int tot;
  const int run = block_exclusive_scan((my_t << 16) | my_d, red_i, &tot);
  int run_t = run >> 16, run_d = run & 0xffff;
  for (int b = b0; b < b1; ++b) {
    const int k = count[b];
    num_draft[b] = k;
    if (t_start != nullptr) t_start[b] = run_t;
    if (d_start != nullptr) d_start[b] = run_d;
    run_t += k + 1;
    run_d += k;
  }
  if (tid == 0 && summary != nullptr) {
    summary[0] = late ? -1.0f : (float)chosen_n;
    summary[1] = chosen_rate;
  }
}

size_t words_bytes(int B, int K) {
  const size_t groups = ((size_t)B * K + kTokensPerGroup - 1) / kTokensPerGroup;
  const size_t bytes = groups * kWordsPerGroup * sizeof(uint64_t);
  return (bytes + 255) / 256 * 256;
}

}  // namespace

extern "C" size_t sv_schedule_workspace_bytes(int B, int K) {
  if (B < 1 || K < 1 || K > 64 || (long)B * K > kMaxTokens) return 0;
  return words_bytes(B, K);
}

extern "C" int sv_schedule_prefix(const float* confidence, int B, int K, const float* step_time,
                                  int T, float threshold, int32_t* num_draft,
                                  int32_t* target_row_start, int32_t* draft_row_start,
                                  float* summary, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  sv_internal_clear_error();
  if (B < 1 || K < 1 || K > 64 || (long)B * K > kMaxTokens)
    return sv_internal_fail(SV_ERR_INVALID_ARG, "need B >= 1, 1 <= K <= 64 and B*K <= 4096");
  if (!confidence || !num_draft)
    return sv_internal_fail(SV_ERR_INVALID_ARG, "a required pointer is NULL");
  if (step_time != nullptr && (long)T < (long)B + (long)B * K + 1)
    return sv_internal_fail(SV_ERR_INVALID_ARG, "the step-time table must cover B + B*K tokens");
  if (step_time == nullptr && !isfinite(threshold))
    return sv_internal_fail(SV_ERR_INVALID_ARG, "threshold must be finite");
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint32_t tag = 0;
  unsigned groups = 1;
  if (step_time != nullptr) {
    if (workspace == nullptr || ((uintptr_t)workspace & 7) != 0)
      return sv_internal_fail(SV_ERR_WORKSPACE, "workspace must be non-NULL and 8-byte aligned");
    if (workspace_bytes < words_bytes(B, K))
      return sv_internal_fail(SV_ERR_WORKSPACE, "workspace too small");
    const int st = sv_internal_call_tags(1, workspace, workspace_bytes, s, &tag);
    if (st != SV_OK) return st;
    groups = (unsigned)(((long)B * K + kTokensPerGroup - 1) / kTokensPerGroup) + 1;
  }
  hipLaunchKernelGGL(sv_schedule_kernel, dim3(groups), dim3(kThreads), 0, s, confidence, B, K,
                     step_time, threshold, static_cast<uint64_t*>(workspace), tag, num_draft,
                     target_row_start, draft_row_start, summary);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return sv_internal_fail(SV_ERR_HIP, hipGetErrorString(e));
  return SV_OK;
}
