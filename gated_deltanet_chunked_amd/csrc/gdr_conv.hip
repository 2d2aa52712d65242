// gdr_conv.hip -- the steps in front of the chunkwise path for packed
// sequences (Qwen3-Next blog post, sections 3 and 4): the causal depthwise
// conv (kernel size 4) over each sequence's tokens, with the cached window of
// the sequence (or zeros) in front of its first token, SiLU, cast to the
// activation dtype, split into q | k | v; the gates
//   beta = sigmoid(b),  g = -exp(A_log) softplus(a + dt_bias);
// and each sequence's new window (the last 4 values of window + tokens).
// Bandwidth bound: the projected channels are read once (the 3 earlier
// values of a window come from the same lines, through the cache) and the
// activations written once.
#include "gdr_device.h"
#include "gdr_kernels.h"

namespace gdr {

namespace {

template <typename T>
__device__ __forceinline__ void get4(const T* p, float* x);
template <>
__device__ __forceinline__ void get4<float>(const float* p, float* x) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
}
template <>
__device__ __forceinline__ void get4<__bf16>(const __bf16* p, float* x) {
  typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
  const bf16x4 a = *reinterpret_cast<const bf16x4*>(p);
#pragma unroll
  for (int e = 0; e < 4; ++e) x[e] = (float)a[e];
}

// Sequence owning token t: the last b with cu[b] <= t (cu clamped into [0, T]).
__device__ __forceinline__ int owner(const int32_t* cu, int32_t N, int32_t T, int t) {
  int lo = 0, hi = N - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (min(max(cu[mid], 0), T) <= t) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

}  // namespace

// One workgroup per (16 tokens, 2048 channels): a thread owns 8 consecutive
// channels (one 16-byte piece of a bf16 row; the q | k | v boundaries are
// multiples of 128 channels, so a piece never straddles two parts) and walks
// them through the 16 tokens with the window's three older values in
// registers, so each projected value is read once, 16 bytes per access; at a
// sequence start the window restarts from that sequence's cached values.
// Workgroup ids run over the channel blocks first, so the workgroups in
// flight read and write whole token rows (231 -> 210 us at T = 32768 against
// token blocks first); the grid is one-dimensional, so any T fits.
constexpr int kTokPerBlock = 16;
constexpr int kChPerThread = 8;
constexpr int kChPerBlock = 256 * kChPerThread;

// 8 consecutive values of type T as float (one 16-byte load for bf16, two for
// fp32), and the other way.
template <typename T>
__device__ __forceinline__ void get8(const T* p, float* x) {
  get4<T>(p, x);
  get4<T>(p + 4, x + 4);
}
template <>
__device__ __forceinline__ void get8<__bf16>(const __bf16* p, float* x) {
  const bf16x8 a = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = (float)a[e];
}
template <typename T>
__device__ __forceinline__ void put8(T* p, const float* y) {
#pragma unroll
  for (int e = 0; e < 8; ++e) p[e] = from_f32<T>(y[e]);
}
template <>
__device__ __forceinline__ void put8<__bf16>(__bf16* p, const float* y) {
  bf16x8 a;
#pragma unroll
  for (int e = 0; e < 8; ++e) a[e] = (__bf16)y[e];
  *reinterpret_cast<bf16x8*>(p) = a;
}
template <>
__device__ __forceinline__ void put8<float>(float* p, const float* y) {
  *reinterpret_cast<f32x4*>(p) = f32x4{y[0], y[1], y[2], y[3]};
  *reinterpret_cast<f32x4*>(p + 4) = f32x4{y[4], y[5], y[6], y[7]};
}

// Raw 8 values of type T (kept unconverted while in flight).
template <typename T>
struct Raw8 {
  typedef __attribute__((ext_vector_type(8))) T type;
};

template <typename T>
__global__ __launch_bounds__(256) void conv_prefill_kernel(ConvPrefillArgs<T> p) {
  const int ncb = (p.C + kChPerBlock - 1) / kChPerBlock;
  const int cbk = (int)(blockIdx.x % (unsigned)ncb), tbk = (int)(blockIdx.x / (unsigned)ncb);
  const int t0 = tbk * kTokPerBlock;
  const int t1 = min(t0 + kTokPerBlock, p.Ttok);
  const int c = (cbk * 256 + threadIdx.x) * kChPerThread;
  if (c < p.C) {
    // kernels of the 8 channels: 32 consecutive values of [C, 4]
    float w[kChPerThread][4];
#pragma unroll
    for (int e = 0; e < kChPerThread; ++e) get4<T>(p.w + (size_t)(c + e) * 4, w[e]);
    float bias[kChPerThread];
    if (p.bias) get8<T>(p.bias + c, bias);
    else
#pragma unroll
      for (int e = 0; e < kChPerThread; ++e) bias[e] = 0.0f;
    int b = owner(p.cu, p.N, p.Ttok, t0);
    int start = min(max(p.cu[b], 0), p.Ttok);
    int end = min(max(p.cu[b + 1], start), p.Ttok);
    // window values 1..3 places before sequence bb's first token, from its
    // cached window [bb][c + e][4] (zeros without a cache)
    auto cached = [&](int bb, int back, float* x) {
      if (p.cs_in) {
#pragma unroll
        for (int e = 0; e < kChPerThread; ++e)
          x[e] = to_f32(p.cs_in[((size_t)bb * p.C + c + e) * 4 + 4 - back]);
      } else {
#pragma unroll
        for (int e = 0; e < kChPerThread; ++e) x[e] = 0.0f;
      }
    };
    // the values at position pos < t0, in the sequence of t0
    auto before = [&](int pos, float* x) {
      if (pos >= start) get8<T>(p.x + (size_t)pos * p.C + c, x);
      else cached(b, min(start - pos, 3), x);
    };
    // all of the block's token values at once (the tail repeats the block's
    // last token, which exists), so the loads are in flight together
    typename Raw8<T>::type xs[kTokPerBlock];
#pragma unroll
    for (int i = 0; i < kTokPerBlock; ++i)
      xs[i] = *reinterpret_cast<const typename Raw8<T>::type*>(
          p.x + (size_t)min(t0 + i, t1 - 1) * p.C + c);
    float w1[kChPerThread], w2[kChPerThread], w3[kChPerThread];
    before(t0 - 3, w1);
    before(t0 - 2, w2);
    before(t0 - 1, w3);
    const int qk = p.Nqk * kD;
    T* dst;
    int stride;
    if (c < qk) { dst = p.q + c; stride = qk; }
    else if (c < 2 * qk) { dst = p.k + (c - qk); stride = qk; }
    else { dst = p.v + (c - 2 * qk); stride = p.C - 2 * qk; }
#pragma unroll
    for (int i = 0; i < kTokPerBlock; ++i) {
      const int t = t0 + i;
      if (t >= t1) break;
      if (t >= end) {   // a new sequence (after any empty ones) starts here
        b = owner(p.cu, p.N, p.Ttok, t);
        start = min(max(p.cu[b], 0), p.Ttok);
        end = min(max(p.cu[b + 1], start), p.Ttok);
        cached(b, 3, w1);
        cached(b, 2, w2);
        cached(b, 1, w3);
      }
      float y[kChPerThread];
#pragma unroll
      for (int e = 0; e < kChPerThread; ++e) {
        const float xt = to_f32(xs[i][e]);
        float a = bias[e] + w[e][0] * w1[e] + w[e][1] * w2[e] + w[e][2] * w3[e] + w[e][3] * xt;
        y[e] = silu(a);
        w1[e] = w2[e];
        w2[e] = w3[e];
        w3[e] = xt;
      }
      put8<T>(dst + (size_t)t * stride, y);
    }
  }
  // the gates of the block's tokens, dealt over the channel blocks
  {
    const int per = (t1 - t0) * p.Nv, nb = ncb;
    for (int idx = threadIdx.x + 256 * cbk; idx < per; idx += 256 * nb) {
      const int t = t0 + idx / p.Nv, h = idx % p.Nv;
      const size_t gi = (size_t)t * p.Nv + h;
      const float z = p.a[gi] + p.dt_bias[h];
      const float softplus = fmaxf(z, 0.0f) + log1pf(expf(-fabsf(z)));
      p.g[gi] = -expf(p.A_log[h]) * softplus;
      p.beta[gi] = 1.0f / (1.0f + expf(-p.b[gi]));
    }
  }
}

// One thread per (sequence, channel): the new window, the last 4 values of
// (cached window, tokens).  A thread reads only the window it writes, so the
// update may be in place.
template <typename T>
__global__ __launch_bounds__(256) void conv_window_kernel(ConvPrefillArgs<T> p) {
  const int b = blockIdx.x;
  const int c = blockIdx.y * 256 + threadIdx.x;
  if (c >= p.C) return;
  const int start = min(max(p.cu[b], 0), p.Ttok);
  const int end = min(max(p.cu[b + 1], start), p.Ttok);
  float old[4] = {0.f, 0.f, 0.f, 0.f};
  if (p.cs_in) get4<T>(p.cs_in + ((size_t)b * p.C + c) * 4, old);
  float nw[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int pos = end - 4 + i;
    const int back = 4 - (start - pos);   // 0..3 when pos < start (end >= start)
    const float cached = back <= 0 ? old[0] : back == 1 ? old[1] : back == 2 ? old[2] : old[3];
    nw[i] = pos >= start ? to_f32(p.x[(size_t)pos * p.C + c]) : cached;
  }
  T* o = p.cs_out + ((size_t)b * p.C + c) * 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = from_f32<T>(nw[i]);   // exact: values of type T
}

template <typename T>
void launch_conv_prefill(const ConvPrefillArgs<T>& p, hipStream_t stream, LaunchEvents ev_conv,
                         LaunchEvents ev_window) {
  const unsigned cb = (unsigned)((p.C + 255) / 256);
  if (p.Ttok > 0)
    hipExtLaunchKernelGGL(conv_prefill_kernel<T>,
                          dim3((unsigned)((p.Ttok + kTokPerBlock - 1) / kTokPerBlock) *
                               (unsigned)((p.C + kChPerBlock - 1) / kChPerBlock)),
                          dim3(256), 0, stream, ev_conv.start, ev_conv.stop, 0, p);
  if (p.cs_out)
    hipExtLaunchKernelGGL(conv_window_kernel<T>, dim3((unsigned)p.N, cb), dim3(256), 0, stream,
                          ev_window.start, ev_window.stop, 0, p);
}

template void launch_conv_prefill<float>(const ConvPrefillArgs<float>&, hipStream_t, LaunchEvents,
                                         LaunchEvents);
template void launch_conv_prefill<__bf16>(const ConvPrefillArgs<__bf16>&, hipStream_t,
                                          LaunchEvents, LaunchEvents);

}  // namespace gdr
