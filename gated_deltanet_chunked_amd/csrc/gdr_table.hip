// gdr_table.hip -- first stage of the chunkwise forward: the chunk table.
//
// Chunks of L tokens (128, or 64) restart at every sequence start (Qwen3-Next
// blog post, section 5(1)c: the gate cumsum restarts at each chunk), so
// sequence b owns ceil(len_b / L) chunk slots starting at choff[b].
#include "gdr_device.h"
#include "gdr_kernels.h"

namespace gdr {

// One workgroup of 1024 threads.  Token ranges are clamped into [0, T] so a
// malformed cu_seqlens can only produce wrong numbers, never an access
// outside the caller's buffers; slots beyond nslots are dropped.
__global__ __launch_bounds__(1024) void table_kernel(const int32_t* __restrict__ cu, int32_t N,
                                                     int32_t T, int32_t L, int32_t nslots,
                                                     int4* __restrict__ table,
                                                     int32_t* __restrict__ choff) {
  __shared__ int32_t part[1024];
  const int tid = threadIdx.x;
  const int per = (N + 1023) / 1024;
  const int b0 = min(N, tid * per), b1 = min(N, b0 + per);
  auto range = [&](int b, int& lo, int& hi) {
    lo = min(max(cu[b], 0), T);
    hi = min(max(cu[b + 1], lo), T);
  };
  int32_t local = 0;
  for (int b = b0; b < b1; ++b) {
    int lo, hi;
    range(b, lo, hi);
    local += (hi - lo + L - 1) / L;
  }
  part[tid] = local;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int32_t x = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += x;
    __syncthreads();
  }
  int32_t run = part[tid] - local;
  for (int b = b0; b < b1; ++b) {
    int lo, hi;
    range(b, lo, hi);
    choff[b] = min(run, nslots);
    const int nch = (hi - lo + L - 1) / L;
    for (int m = 0; m < nch; ++m) {
      const int s = run + m;
      if (s < nslots) table[s] = make_int4(b, lo + L * m, min(L, hi - lo - L * m), 0);
    }
    run += nch;
  }
  const int32_t total = min(part[1023], nslots);
  if (tid == 0) choff[N] = total;
  for (int s = total + tid; s < nslots; s += 1024) table[s] = make_int4(-1, 0, 0, 0);
}

void launch_table(const int32_t* cu, int32_t N, int32_t T, int32_t L, int32_t nslots, int4* table,
                  int32_t* choff, hipStream_t stream, LaunchEvents ev) {
  hipExtLaunchKernelGGL(table_kernel, dim3(1), dim3(1024), 0, stream, ev.start, ev.stop, 0, cu, N, T,
                        L, nslots, table, choff);
}

}  // namespace gdr
