// Read probe of libsv (declared in sv.h): the plainest stream over a buffer, for the read
// bandwidth the row stream of the verify kernels is compared with. Not a step of the method.

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "sv.h"
#include "sv_internal.h"

namespace {

constexpr int kBlock = 256;  // threads per work-group: 4 wave64s
constexpr int kInFlight = 8;  // 16-byte non-temporal loads in flight per thread

typedef unsigned int v4u32 __attribute__((ext_vector_type(4)));

// Work-group g sums (wrapping 32-bit adds) the 16-byte words of its contiguous range
// [n*g/G, n*(g+1)/G): rounds of kInFlight loads per thread, thread t taking words t, t + 256, ...
// of the round, and writes its sum to partial[g].
__global__ __launch_bounds__(kBlock) void sv_read_probe_kernel(const v4u32* __restrict__ data,
                                                               size_t n, uint32_t* partial) {
  const size_t G = gridDim.x;
  const size_t w0 = n * blockIdx.x / G, w1 = n * (blockIdx.x + 1) / G;
  constexpr size_t kRound = (size_t)kInFlight * kBlock;
  size_t i = w0 + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kInFlight - 1) * kBlock < w1; i += kRound) {
    v4u32 v[kInFlight];
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) v[u] = __builtin_nontemporal_load(data + i + u * kBlock);
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) acc += (v[u].x + v[u].y) + (v[u].z + v[u].w);
  }
  for (; i < w1; i += kBlock) {
    const v4u32 a = __builtin_nontemporal_load(data + i);
    acc += (a.x + a.y) + (a.z + a.w);
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
  __shared__ uint32_t red[kBlock / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) partial[blockIdx.x] = red[0] + red[1] + red[2] + red[3];
}

}  // namespace

extern "C" int sv_read_probe(const void* data, size_t bytes, uint32_t* partial, int groups,
                             void* stream) {
  sv_internal_clear_error();
  if (!data || !partial) return sv_internal_fail(SV_ERR_INVALID_ARG, "a required pointer is NULL");
  if (reinterpret_cast<uintptr_t>(data) % 16 != 0 || bytes % 16 != 0)
    return sv_internal_fail(SV_ERR_INVALID_ARG,
                            "data must be 16-byte aligned and bytes a multiple of 16");
  if (groups < 1 || groups > (1 << 20))
    return sv_internal_fail(SV_ERR_INVALID_ARG, "groups must be in [1, 2^20]");
  hipLaunchKernelGGL(sv_read_probe_kernel, dim3((unsigned)groups), dim3(kBlock), 0,
                     static_cast<hipStream_t>(stream), static_cast<const v4u32*>(data),
                     bytes / 16, partial);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return sv_internal_fail(SV_ERR_HIP, hipGetErrorString(e));
  return SV_OK;
}
