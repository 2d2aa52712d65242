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

// One workgroup per (16 tokens, 256 channels).  A thread walks its channel
// through the 16 tokens with the window's three older values in registers,
// so each projected value is read once; at a sequence start the window
// restarts from that sequence's cached values.
constexpr int kTokPerBlock = 16;

template <typename T>
__global__ __launch_bounds__(256) void conv_prefill_kernel(ConvPrefillArgs<T> p) {
  const int t0 = blockIdx.x * kTokPerBlock;
  const int t1 = min(t0 + kTokPerBlock, p.Ttok);
  const int c = blockIdx.y * 256 + threadIdx.x;
  if (c < p.C) {
    float w[4];
    get4<T>(p.w + (size_t)c * 4, w);
    const float bias = p.bias ? to_f32(p.bias[c]) : 0.0f;
    int b = owner(p.cu, p.N, p.Ttok, t0);
    int start = min(max(p.cu[b], 0), p.Ttok);
    int end = min(max(p.cu[b + 1], start), p.Ttok);
    // value `back` (1..3) places before sequence b's first token: its cached window
    auto cached = [&](int bb, int back) -> float {
      return p.cs_in ? to_f32(p.cs_in[((size_t)bb * p.C + c) * 4 + 4 - back]) : 0.0f;
    };
    // value at position pos < t0, in the sequence of t0
    auto before = [&](int pos) -> float {
      return pos >= start ? to_f32(p.x[(size_t)pos * p.C + c]) : cached(b, min(start - pos, 3));
    };
    // all of the block's token values at once (the tail repeats the block's
    // last token, which exists), so the loads are in flight together
    T xs[kTokPerBlock];
#pragma unroll
    for (int i = 0; i < kTokPerBlock; ++i) xs[i] = p.x[(size_t)min(t0 + i, t1 - 1) * p.C + c];
    float w1 = before(t0 - 3), w2 = before(t0 - 2), w3 = before(t0 - 1);
    const int qk = p.Nqk * kD;
#pragma unroll
    for (int i = 0; i < kTokPerBlock; ++i) {
      const int t = t0 + i;
      if (t >= t1) break;
      if (t >= end) {   // a new sequence (after any empty ones) starts here
        b = owner(p.cu, p.N, p.Ttok, t);
        start = min(max(p.cu[b], 0), p.Ttok);
        end = min(max(p.cu[b + 1], start), p.Ttok);
        w1 = cached(b, 3);
        w2 = cached(b, 2);
        w3 = cached(b, 1);
      }
      const float xt = to_f32(xs[i]);
      float y = bias + w[0] * w1 + w[1] * w2 + w[2] * w3 + w[3] * xt;
      y = y / (1.0f + expf(-y));
      if (c < qk) p.q[(size_t)t * qk + c] = from_f32<T>(y);
      else if (c < 2 * qk) p.k[(size_t)t * qk + (c - qk)] = from_f32<T>(y);
      else p.v[(size_t)t * (p.C - 2 * qk) + (c - 2 * qk)] = from_f32<T>(y);
      w1 = w2;
      w2 = w3;
      w3 = xt;
    }
  }
  if (blockIdx.y == 0) {
    for (int idx = threadIdx.x; idx < (t1 - t0) * p.Nv; idx += 256) {
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
                          dim3((unsigned)((p.Ttok + kTokPerBlock - 1) / kTokPerBlock), cb), dim3(256),
                          0, stream,
                          ev_conv.start, ev_conv.stop, 0, p);
  if (p.cs_out)
    hipExtLaunchKernelGGL(conv_window_kernel<T>, dim3((unsigned)p.N, cb), dim3(256), 0, stream,
                          ev_window.start, ev_window.stop, 0, p);
}

template void launch_conv_prefill<float>(const ConvPrefillArgs<float>&, hipStream_t, LaunchEvents,
                                         LaunchEvents);
template void launch_conv_prefill<__bf16>(const ConvPrefillArgs<__bf16>&, hipStream_t,
                                          LaunchEvents, LaunchEvents);

}  // namespace gdr
