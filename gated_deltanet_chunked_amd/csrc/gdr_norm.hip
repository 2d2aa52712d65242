// gdr_norm.hip -- the gated RMSNorm in front of the output projection
// (Qwen3-Next blog post: RMSNormGated, sections 1 and 6; the RMS form is the
// _norm of its Zero-Centered RMSNorm section), with the SiLU output gate:
//   y[r][i] = x[r][i] / sqrt(mean_j x[r][j]^2 + eps) * w[i] * SiLU(z[r][i]).
//
// HBM bound (three rows of 128 values move per row).  A row belongs to 16
// consecutive lanes, 8 values each, so a row's loads are one contiguous
// 256-byte (bf16) or 512-byte (fp32) run and its sum of squares reduces across
// the 16 lanes on DPP.  Each thread takes two rows per pass of a grid-stride
// loop (rows r and r + 16, so a workgroup's 32 rows are one contiguous run of
// x and of z; rows a grid apart measured 7% slower) so that four loads are in
// flight before the first reduction.
#include "gdr_device.h"
#include "gdr_kernels.h"

namespace gdr {
namespace {

// 8 consecutive values as float, one 16-byte load (bf16) or two (fp32).
__device__ __forceinline__ void load8(const __bf16* p, float* x) {
  const bf16x8 a = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = (float)a[e];
}
__device__ __forceinline__ void load8(const float* p, float* x) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
  for (int e = 0; e < 4; ++e) { x[e] = a[e]; x[e + 4] = b[e]; }
}
__device__ __forceinline__ void store8(__bf16* p, const float* y) {
  bf16x8 a;
#pragma unroll
  for (int e = 0; e < 8; ++e) a[e] = (__bf16)y[e];   // round to nearest even
  *reinterpret_cast<bf16x8*>(p) = a;
}
__device__ __forceinline__ void store8(float* p, const float* y) {
  *reinterpret_cast<f32x4*>(p) = f32x4{y[0], y[1], y[2], y[3]};
  *reinterpret_cast<f32x4*>(p + 4) = f32x4{y[4], y[5], y[6], y[7]};
}

// y = x * inv_rms * w * SiLU(z) for the 8 values of one lane; all 16 lanes of
// the row take part in the reduction.
__device__ __forceinline__ void gate_row(const float* x, const float* z, const float* w, float eps,
                                         float* y) {
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) ss += x[e] * x[e];
  ss = group16_sum(ss);
  const float inv = 1.0f / sqrtf(ss * (1.0f / kD) + eps);
#pragma unroll
  for (int e = 0; e < 8; ++e) y[e] = x[e] * inv * w[e] * silu(z[e]);
}

// x and y may be the same buffer (in place), so neither is restrict.
template <typename T>
__global__ __launch_bounds__(256) void gated_rmsnorm_kernel(const T* x, const T* __restrict__ z,
                                                            const T* __restrict__ w, int64_t rows,
                                                            float eps, T* y) {
  const int cg = threadIdx.x & 15;
  const int64_t stride = 16;
  float wv[8];
  if (w) load8(w + 8 * cg, wv);
  else
#pragma unroll
    for (int e = 0; e < 8; ++e) wv[e] = 1.0f;
  // rows r and r + 16 per pass; the second may lie past the end, for a
  // whole 16-lane row at once, so the reductions stay within active rows
  for (int64_t r = (int64_t)blockIdx.x * 32 + (threadIdx.x >> 4); r < rows;
       r += (int64_t)gridDim.x * 32) {
    const int64_t r2 = r + stride;
    const bool two = r2 < rows;
    float xa[8], za[8], xb[8], zb[8], ya[8], yb[8];
    load8(x + r * kD + 8 * cg, xa);
    load8(z + r * kD + 8 * cg, za);
    if (two) {
      load8(x + r2 * kD + 8 * cg, xb);
      load8(z + r2 * kD + 8 * cg, zb);
    }
    gate_row(xa, za, wv, eps, ya);
    store8(y + r * kD + 8 * cg, ya);
    if (two) {
      gate_row(xb, zb, wv, eps, yb);
      store8(y + r2 * kD + 8 * cg, yb);
    }
  }
}

}  // namespace

template <typename T>
void launch_gated_rmsnorm(const T* x, const T* z, const T* w, int64_t rows, float eps, T* y,
                          hipStream_t stream, LaunchEvents ev) {
  // enough workgroups for every CU's full occupancy; each thread then takes
  // two rows per pass
  const int64_t want = (rows + 31) / 32;
  const unsigned blocks = (unsigned)(want < 8192 ? (want > 0 ? want : 1) : 8192);
  hipExtLaunchKernelGGL(gated_rmsnorm_kernel<T>, dim3(blocks), dim3(256), 0, stream, ev.start,
                        ev.stop, 0, x, z, w, rows, eps, y);
}

template void launch_gated_rmsnorm<float>(const float*, const float*, const float*, int64_t, float,
                                          float*, hipStream_t, LaunchEvents);
template void launch_gated_rmsnorm<__bf16>(const __bf16*, const __bf16*, const __bf16*, int64_t,
                                           float, __bf16*, hipStream_t, LaunchEvents);

}  // namespace gdr
