// Confidence-scheduled prefix selection for libsv (declared in sv.h): how many draft tokens of
// each request go to verification ("DSpark" paper review, 4.2.1 Confidence Head and 4.2.2
// Hardware-Aware Prefix Scheduler). It runs on the device so that confidences from the drafter,
// the chosen lengths and the flattened row starts of the verify call never cross to the host.
//
// One work-group of 1024 threads:
//   1. survival s[b][k] = c[b][0] * ... * c[b][k] (confidences clamped to [0, 1], NaN = 0),
//      float32 products left to right, one thread per request;
//   2. every token becomes a 64-bit key (descending survival, then ascending position, then
//      ascending request) and the keys are sorted in LDS (bitonic);
//   3. hardware-aware mode: E(N) = B + the fp64 sum of the first N ranked survivals (every
//      request also commits the target's own token); the N in 0 .. B*K with the largest
//      E(N) / step_time[B + N] wins (the whole table is searched; the smallest N among equal
//      rates; non-finite or non-positive step times are unusable); request b keeps its tokens
//      among the first N, always a prefix because survival never increases along a block.
//      Threshold mode: request b keeps its drafts up to the first confidence below the
//      threshold;
//   4. num_draft and the flattened row starts (exclusive sums of k_b + 1 and of k_b).

#include <hip/hip_runtime.h>

#include <float.h>
#include <math.h>
#include <stdint.h>

#include "sv.h"
#include "sv_internal.h"

namespace {

constexpr int kThreads = 1024;
constexpr int kMaxTokens = 4096;  // B * K, at most
constexpr int kMaxRequests = 4096;

__device__ __forceinline__ float clamp01(float c) {
  if (!(c > 0.0f)) return 0.0f;  // NaN and non-positive values
  return c < 1.0f ? c : 1.0f;
}

// Inclusive prefix sum over kThreads doubles (one per thread), in a fixed order; red holds one
// double per wave.
__device__ double block_scan(double v, double* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int d = 1; d < 64; d <<= 1) {
    const double u = __shfl_up(v, d);
    if (lane >= d) v += u;
  }
  __syncthreads();
  if (lane == 63) red[wave] = v;
  __syncthreads();
  double before = 0.0;
  for (int w = 0; w < wave; ++w) before += red[w];
  return before + v;
}

__device__ int block_scan_int(int v, int* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int d = 1; d < 64; d <<= 1) {
    const int u = __shfl_up(v, d);
    if (lane >= d) v += u;
  }
  __syncthreads();
  if (lane == 63) red[wave] = v;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += red[w];
  return before + v;
}

__global__ __launch_bounds__(kThreads) void sv_schedule_kernel(
    const float* __restrict__ conf, int B, int K, const float* __restrict__ step_time, int T,
    float threshold, int32_t* num_draft, int32_t* t_start, int32_t* d_start, float* summary) {
  __shared__ uint64_t keys[kMaxTokens];
  __shared__ int count[kMaxRequests];
  __shared__ double red_d[kThreads / 64];
  __shared__ int red_i[kThreads / 64];
  __shared__ double best_rate[kThreads / 64];
  __shared__ int best_n[kThreads / 64];
  const int tid = threadIdx.x;
  const int M = B * K;

  for (int b = tid; b < B; b += kThreads) count[b] = 0;
  float chosen_rate = 0.0f;
  int chosen_n = 0;

  if (step_time == nullptr) {  // threshold mode
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
    __syncthreads();
  } else {
    int M2 = 1;
    while (M2 < M) M2 <<= 1;
    // 1-2. survivals and keys
    for (int b = tid; b < B; b += kThreads) {
      float s = 1.0f;
      for (int k = 0; k < K; ++k) {
        s = s * clamp01(conf[(size_t)b * K + k]);
        const uint32_t bits = __float_as_uint(s);
        keys[b * K + k] = ((uint64_t)(~bits) << 32) | ((uint64_t)k << 16) | (uint64_t)b;
      }
    }
    for (int i = M + tid; i < M2; i += kThreads) keys[i] = ~0ull;
    __syncthreads();
    for (int size = 2; size <= M2; size <<= 1) {
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        for (int i = tid; i < M2 / 2; i += kThreads) {
          const int lo = 2 * i - (i & (stride - 1));
          const int hi = lo + stride;
          const bool up = (lo & size) == 0;
          const uint64_t a = keys[lo], c = keys[hi];
          if ((a > c) == up) {
            keys[lo] = c;
            keys[hi] = a;
          }
        }
        __syncthreads();
      }
    }
    // 3. E(N) for N = 1 .. M: thread t owns ranked tokens [t*per, (t+1)*per); the running sum
    //    walks them in order after a block scan of the per-thread sums
    const int per = (M + kThreads - 1) / kThreads;
    const int i0 = tid * per, i1 = min(M, i0 + per);
    double mine = 0.0;
    for (int i = i0; i < i1; ++i) mine += (double)__uint_as_float(~(uint32_t)(keys[i] >> 32));
    const double incl = block_scan(mine, red_d);
    double run = (double)B + (incl - mine);
    double rate = -INFINITY;
    int n_best = -1;
    if (tid == 0) {  // N = 0: no drafts
      const float t0 = B < T ? step_time[B] : NAN;
      if (isfinite(t0) && t0 > 0.0f) {
        rate = (double)B / (double)t0;
        n_best = 0;
      }
    }
    for (int i = i0; i < i1; ++i) {
      run += (double)__uint_as_float(~(uint32_t)(keys[i] >> 32));
      const int n = i + 1;
      const float tn = step_time[B + n];
      if (isfinite(tn) && tn > 0.0f) {
        const double r = run / (double)tn;
        if (r > rate) {
          rate = r;
          n_best = n;
        }
      }
    }
    // first maximum over the block: larger rate, then smaller N
    for (int m = 32; m >= 1; m >>= 1) {
      const double r2 = __shfl_xor(rate, m);
      const int n2 = __shfl_xor(n_best, m);
      if (r2 > rate || (r2 == rate && n2 >= 0 && (n_best < 0 || n2 < n_best))) {
        rate = r2;
        n_best = n2;
      }
    }
    const int lane = tid & 63, wave = tid >> 6;
    if (lane == 0) {
      best_rate[wave] = rate;
      best_n[wave] = n_best;
    }
    __syncthreads();
    rate = best_rate[0];
    n_best = best_n[0];
    for (int w = 1; w < kThreads / 64; ++w) {
      if (best_rate[w] > rate || (best_rate[w] == rate && best_n[w] >= 0 &&
                                  (n_best < 0 || best_n[w] < n_best))) {
        rate = best_rate[w];
        n_best = best_n[w];
      }
    }
    chosen_n = n_best < 0 ? 0 : n_best;
    chosen_rate = n_best < 0 ? 0.0f : (float)rate;
    for (int i = tid; i < chosen_n; i += kThreads)
      atomicAdd(&count[(int)(keys[i] & 0xffff)], 1);
    __syncthreads();
  }

  // 4. outputs: lengths and flattened row starts, requests in order
  __shared__ int tot_t, tot_d;
  int carry_t = 0, carry_d = 0;
  for (int b0 = 0; b0 < B; b0 += kThreads) {
    const int b = b0 + tid;
    const int k = b < B ? count[b] : 0;
    const int vt = b < B ? k + 1 : 0;
    const int it = block_scan_int(vt, red_i);
    const int id = block_scan_int(k, red_i);
    if (b < B) {
      num_draft[b] = k;
      if (t_start != nullptr) t_start[b] = carry_t + it - vt;
      if (d_start != nullptr) d_start[b] = carry_d + id - k;
    }
    if (tid == kThreads - 1) {
      tot_t = it;
      tot_d = id;
    }
    __syncthreads();
    carry_t += tot_t;
    carry_d += tot_d;
    __syncthreads();
  }
  if (tid == 0 && summary != nullptr) {
    summary[0] = (float)chosen_n;
    summary[1] = chosen_rate;
  }
}

}  // namespace

extern "C" int sv_schedule_prefix(const float* confidence, int B, int K, const float* step_time,
                                  int T, float threshold, int32_t* num_draft,
                                  int32_t* target_row_start, int32_t* draft_row_start,
                                  float* summary, void* stream) {
  sv_internal_clear_error();
  if (B < 1 || K < 1 || K > 64 || (long)B * K > kMaxTokens)
    return sv_internal_fail(SV_ERR_INVALID_ARG, "need B >= 1, 1 <= K <= 64 and B*K <= 4096");
  if (!confidence || !num_draft)
    return sv_internal_fail(SV_ERR_INVALID_ARG, "a required pointer is NULL");
  if (step_time != nullptr && (long)T < (long)B + (long)B * K + 1)
    return sv_internal_fail(SV_ERR_INVALID_ARG, "the step-time table must cover B + B*K tokens");
  if (step_time == nullptr && !isfinite(threshold))
    return sv_internal_fail(SV_ERR_INVALID_ARG, "threshold must be finite");
  hipLaunchKernelGGL(sv_schedule_kernel, dim3(1), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), confidence, B, K, step_time, T, threshold,
                     num_draft, target_row_start, draft_row_start, summary);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return sv_internal_fail(SV_ERR_HIP, hipGetErrorString(e));
  return SV_OK;
}
