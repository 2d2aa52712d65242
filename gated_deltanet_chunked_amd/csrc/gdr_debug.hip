// gdr_debug.hip -- optional checks of the values the entry points cannot see
// on the host: cu_seqlens starts at 0, never decreases and ends at T, and
// every gate g is finite and <= 0 (the decay exp(g) of the rule, Qwen3-Next
// blog post section 5(2), with g = -A softplus(.) from section 4, lies in
// (0, 1]).  Off by default; switched on by GDR_DEBUG=1 in the environment or
// by gdr_set_debug(1).  A checked call runs one extra kernel and waits for it,
// then returns GDR_ERR_CONTRACT before any other launch if a value is wrong.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdlib>
#include <mutex>

#include "../../include/gdr.h"
#include "gdr_internal.h"

namespace gdr {
namespace {

constexpr int kMaxDevices = 64;

// Which contract a call broke (bit 0: cu[0] != 0, bit 1: cu decreases,
// bit 2: cu[N] != T, bit 3: a gate is positive or not finite).  One word per
// GPU, found with hipGetSymbolAddress (the name in host code is only a
// stand-in); checked calls on one GPU that overlap in time share it.
__device__ unsigned debug_word;

__global__ void debug_clear_kernel(unsigned* w) { *w = 0u; }

__global__ __launch_bounds__(256) void debug_check_kernel(const int32_t* cu, int32_t N, int32_t T,
                                                          const float* g, int64_t ng, unsigned* w) {
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t nth = (int64_t)gridDim.x * blockDim.x;
  unsigned bits = 0u;
  if (cu) {
    for (int64_t i = tid; i <= N; i += nth) {
      const int32_t c = cu[i];
      if (i == 0 && c != 0) bits |= 1u;
      if (i > 0 && c < cu[i - 1]) bits |= 2u;
      if (i == N && c != T) bits |= 4u;
    }
  }
  for (int64_t i = tid; i < ng; i += nth) {
    const float x = g[i];
    if (!(x <= 0.0f) || !__builtin_isfinite(x)) bits |= 8u;
  }
  if (bits) atomicOr(w, bits);
}

std::atomic<int> debug_mode{-1};   // -1: not yet read from the environment
thread_local uint32_t last_broken = 0u;
std::mutex word_mu;
unsigned* word_dev[kMaxDevices] = {};

gdr_status word_ptr(unsigned** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return GDR_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return GDR_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(word_mu);
  if (!word_dev[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(debug_word)) != hipSuccess || !p) return GDR_ERR_HIP;
    word_dev[dev] = static_cast<unsigned*>(p);
  }
  *out = word_dev[dev];
  return GDR_OK;
}

}  // namespace

bool debug_enabled() {
  int m = debug_mode.load(std::memory_order_relaxed);
  if (m < 0) {
    const char* e = std::getenv("GDR_DEBUG");
    const int env = (e && e[0] && !(e[0] == '0' && e[1] == 0)) ? 1 : 0;
    int expected = -1;
    debug_mode.compare_exchange_strong(expected, env);
    m = debug_mode.load(std::memory_order_relaxed);
  }
  return m == 1;
}

gdr_status debug_check(const int32_t* cu, int32_t N, int32_t T, const float* g, int64_t ng,
                       hipStream_t st, uint32_t* broken) {
  *broken = 0u;
  last_broken = 0u;
  unsigned* w = nullptr;
  gdr_status s = word_ptr(&w);
  if (s != GDR_OK) return s;
  const int64_t work = (ng > (int64_t)N + 1 ? ng : (int64_t)N + 1);
  const int64_t want = (work + 255) / 256;
  const unsigned blocks = (unsigned)(want < 1 ? 1 : (want > 4096 ? 4096 : want));
  hipLaunchKernelGGL(debug_clear_kernel, dim3(1), dim3(1), 0, st, w);
  hipLaunchKernelGGL(debug_check_kernel, dim3(blocks), dim3(256), 0, st, cu, N, T, g, ng, w);
  if (hipGetLastError() != hipSuccess) return GDR_ERR_HIP;
  unsigned host = 0u;
  if (hipMemcpyAsync(&host, w, sizeof(host), hipMemcpyDeviceToHost, st) != hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess)
    return GDR_ERR_HIP;
  *broken = host;
  last_broken = host;
  return host ? GDR_ERR_CONTRACT : GDR_OK;
}

}  // namespace gdr

extern "C" int gdr_set_debug(int mode) {
  const int before = gdr::debug_enabled() ? 1 : 0;
  if (mode == 0 || mode == 1) gdr::debug_mode.store(mode, std::memory_order_relaxed);
  return before;
}

extern "C" uint32_t gdr_debug_broken(void) { return gdr::last_broken; }
