// Call tags of libsv (see sv_internal.h) and the zero fill that keeps them unambiguous across a
// wrap of the tag counter; the test hook sv_set_call_counter (sv.h).

#include <hip/hip_runtime.h>

#include <stdint.h>

#include <atomic>
#include <mutex>
#include <unordered_map>

#include "sv.h"
#include "sv_internal.h"

namespace {

constexpr int kFillBlock = 256;

// Zeroes n 64-bit words with vector stores, grid-stride.
__global__ __launch_bounds__(kFillBlock) void sv_zero_fill(uint64_t* p, size_t n) {
  const size_t stride = (size_t)gridDim.x * kFillBlock;
  for (size_t i = (size_t)blockIdx.x * kFillBlock + threadIdx.x; i < n; i += stride) p[i] = 0;
}

std::atomic<uint64_t> g_counter{0};

struct Seen {
  uint64_t epoch;  // the counter's wrap period (upper 32 bits) when the workspace was filled
  size_t bytes;    // bytes filled in that period
};
std::mutex g_mu;
std::unordered_map<uintptr_t, Seen> g_seen;
constexpr size_t kMaxSeen = 1 << 16;  // forgotten workspaces are simply filled again

int fill(void* ws, size_t from, size_t to, hipStream_t s) {
  const size_t n = (to - from) / 8;
  if (n == 0) return SV_OK;
  size_t groups = (n + kFillBlock - 1) / kFillBlock;
  if (groups > 4096) groups = 4096;
  hipLaunchKernelGGL(sv_zero_fill, dim3((unsigned)groups), dim3(kFillBlock), 0, s,
                     reinterpret_cast<uint64_t*>(static_cast<char*>(ws) + from), n);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? SV_OK : sv_internal_fail(SV_ERR_HIP, hipGetErrorString(e));
}

}  // namespace

int sv_internal_call_tags(uint32_t step, void* ws, size_t bytes, hipStream_t s, uint32_t* tag) {
  if (step == 0) step = 1;
  uint64_t c;
  for (;;) {
    c = g_counter.fetch_add(step, std::memory_order_relaxed);
    const uint64_t lo = c & 0xffffffffull;
    if (lo != 0 && lo + step - 1 <= 0xffffffffull) break;  // else take the next range
  }
  *tag = (uint32_t)c;
  const uint64_t epoch = c >> 32;
  size_t from = 0;
  bool need = false;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_seen.size() >= kMaxSeen) g_seen.clear();
    auto it = g_seen.find(reinterpret_cast<uintptr_t>(ws));
    if (it == g_seen.end() || it->second.epoch != epoch) {
      need = true;
      g_seen[reinterpret_cast<uintptr_t>(ws)] = Seen{epoch, bytes};
    } else if (it->second.bytes < bytes) {
      need = true;
      from = it->second.bytes & ~(size_t)7;
      it->second.bytes = bytes;
    }
  }
  return need ? fill(ws, from, bytes, s) : SV_OK;
}

int sv_internal_zero_fill(void* ws, size_t bytes, hipStream_t s) {
  return fill(ws, 0, bytes & ~(size_t)7, s);
}

void sv_internal_untagged_use(void* ws) {
  std::lock_guard<std::mutex> lock(g_mu);
  g_seen.erase(reinterpret_cast<uintptr_t>(ws));
}

extern "C" void sv_set_call_counter(uint64_t value) {
  g_counter.store(value, std::memory_order_relaxed);
}
