// gdr_prep.hip -- first stage of the chunkwise forward: the chunk table, the
// query/key L2 norms and the chunk-local cumulative sum of the gates.
//
// Chunks of 128 tokens restart at every sequence start (Qwen3-Next blog post,
// section 5(1)c: the gate cumsum restarts at each chunk), so sequence b owns
// ceil(len_b / 128) chunk slots starting at choff[b].  The L2 norm is the
// Ascend operator page's x / sqrt(sum x^2 + eps) with eps = 1e-6 (blog post
// section 5(1)a uses the same eps); only the reciprocal norms are stored, the
// kernels that follow apply them as row scalings.
#include "gdr_device.h"
#include "gdr_kernels.h"

namespace gdr {

// One workgroup of 1024 threads.  Token ranges are clamped into [0, T] so a
// malformed cu_seqlens can only produce wrong numbers, never an access
// outside the caller's buffers; slots beyond nslots are dropped.
__global__ __launch_bounds__(1024) void table_kernel(const int32_t* __restrict__ cu, int32_t N,
                                                     int32_t T, int32_t nslots,
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
    local += (hi - lo + 127) / 128;
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
    const int nch = (hi - lo + 127) / 128;
    for (int m = 0; m < nch; ++m) {
      const int s = run + m;
      if (s < nslots) table[s] = make_int4(b, lo + 128 * m, min(128, hi - lo - 128 * m), 0);
    }
    run += nch;
  }
  const int32_t total = min(part[1023], nslots);
  if (tid == 0) choff[N] = total;
  for (int s = total + tid; s < nslots; s += 1024) table[s] = make_int4(-1, 0, 0, 0);
}

// One workgroup per chunk slot: 1/|q|, 1/|k| of its tokens for every
// query/key head and the chunk-local cumulative sum of g (in fp64: the
// differences gcum_r - gcum_i of this sum feed exp(), and fp32 would lose
// their low bits once the sum is large).
template <typename Tin>
__global__ __launch_bounds__(256) void prep_kernel(const Tin* __restrict__ q, const Tin* __restrict__ k,
                                                   const float* __restrict__ g,
                                                   const int4* __restrict__ table, int32_t T,
                                                   int32_t Nqk, int32_t Nv, float scale, int norm,
                                                   float* __restrict__ rq, float* __restrict__ rk,
                                                   double* __restrict__ gcum) {
  const int4 e = table[blockIdx.x];
  if (e.x < 0) return;
  const int start = e.y, len = e.z;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int rows = len * Nqk * 2;
  for (int row = w; row < rows; row += 4) {
    const int which = row & 1;
    const int tj = row >> 1;
    const int t = start + tj / Nqk, j = tj % Nqk;
    const Tin* p = (which ? k : q) + ((size_t)t * Nqk + j) * kD;
    const float x0 = to_f32(p[2 * l]), x1 = to_f32(p[2 * l + 1]);
    const float ss = wave_sum(x0 * x0 + x1 * x1);
    if (l == 0) {
      const float r = norm ? 1.0f / sqrtf(ss + 1e-6f) : 1.0f;
      if (which) rk[(size_t)j * T + t] = r;
      else rq[(size_t)j * T + t] = r * scale;
    }
  }
  for (int h = tid; h < Nv; h += 256) {
    double acc = 0.0;
    for (int m = 0; m < len; ++m) {
      acc += (double)g[(size_t)(start + m) * Nv + h];
      gcum[(size_t)h * T + start + m] = acc;
    }
  }
}

void launch_table(const int32_t* cu, int32_t N, int32_t T, int32_t nslots, int4* table,
                  int32_t* choff, hipStream_t stream) {
  hipLaunchKernelGGL(table_kernel, dim3(1), dim3(1024), 0, stream, cu, N, T, nslots, table, choff);
}

template <typename Tin>
void launch_prep(const Tin* q, const Tin* k, const float* g, const int4* table, int32_t nslots,
                 int32_t T, int32_t Nqk, int32_t Nv, float scale, int norm, float* rq, float* rk,
                 double* gcum, hipStream_t stream) {
  hipLaunchKernelGGL(prep_kernel<Tin>, dim3(nslots), dim3(256), 0, stream, q, k, g, table, T, Nqk,
                     Nv, scale, norm, rq, rk, gcum);
}

template void launch_prep<float>(const float*, const float*, const float*, const int4*, int32_t,
                                 int32_t, int32_t, int32_t, float, int, float*, float*, double*,
                                 hipStream_t);
template void launch_prep<__bf16>(const __bf16*, const __bf16*, const float*, const int4*, int32_t,
                                  int32_t, int32_t, int32_t, float, int, float*, float*, double*,
                                  hipStream_t);

}  // namespace gdr
