// gdr_decode.hip -- one decode step of the gated delta rule (Qwen3-Next blog
// post, section 5(2), a single iteration of the token loop):
//   S  <- exp(g) S;  u = S kh;  S <- S + beta (v - u) kh^T;  o = S qh
// computed in one pass over S as
//   a = S_old kh,  b = S_old qh,  delta = beta (v - exp(g) a),
//   o = exp(g) b + delta (kh . qh),  S_new = exp(g) S_old + delta kh^T.
// Bandwidth bound: each (sequence, head) state is read once and written once,
// 64 KiB in fp32 or 32 KiB when it is stored in bf16 (a bf16 state cache, as
// the generic "Gated DeltaNet" article's section 6.3 advises; the arithmetic
// stays fp32 and only the stored state is rounded, to nearest even).  One
// workgroup of 256 threads per (sequence, head); thread t holds 8 columns of
// rows (t >> 4) + 16 i, i < 8, so each row belongs to 16 consecutive threads
// and the two row dot products reduce across those 16 lanes.  Which columns
// (piece_col) is chosen so that every 16-byte access of the 16 lanes covers
// contiguous whole lines: with bf16 states a lane's 8 columns are one 16-byte
// piece; with fp32 states they are two 4-column pieces, one in each half of
// the row (two separate 16-byte pieces side by side would leave every store
// instruction covering alternate halves of 32-byte sectors).
#include "gdr_device.h"
#include "gdr_kernels.h"

namespace gdr {

// First column of half `half` (0 or 1) of the 8 columns lane cg (0..15) of a
// row group holds: element e of the lane is column piece_col(cg, e / 4) + e % 4.
template <typename ST>
__device__ __forceinline__ int piece_col(int cg, int half) {
  return sizeof(ST) == 4 ? 4 * cg + 64 * half : 8 * cg + 4 * half;
}

template <typename T>
__device__ __forceinline__ void load4(const T* p, float* x);
template <>
__device__ __forceinline__ void load4<float>(const float* p, float* x) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
}
template <>
__device__ __forceinline__ void load4<__bf16>(const __bf16* p, float* x) {
  typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
  const bf16x4 a = *reinterpret_cast<const bf16x4*>(p);
#pragma unroll
  for (int e = 0; e < 4; ++e) x[e] = (float)a[e];
}

// Four values stored as type T (8 or 16 bytes, one access).
template <typename T>
__device__ __forceinline__ void put4(T* p, float a, float b, float c, float d);
template <>
__device__ __forceinline__ void put4<float>(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
}
template <>
__device__ __forceinline__ void put4<__bf16>(__bf16* p, float a, float b, float c, float d) {
  typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
  const bf16x4 y = {(__bf16)a, (__bf16)b, (__bf16)c, (__bf16)d};
  *reinterpret_cast<bf16x4*>(p) = y;
}

// The 8 values of a row of q, k (D entries, type T) at the columns lane cg
// holds for state storage ST.
template <typename T, typename ST>
__device__ __forceinline__ void load_cols(const T* row, int cg, float* x) {
  load4<T>(row + piece_col<ST>(cg, 0), x);
  load4<T>(row + piece_col<ST>(cg, 1), x + 4);
}

// The 8 state values of one row that lane cg holds (columns as piece_col):
// two 16-byte pieces of fp32 or one of bf16, moved with non-temporal accesses
// (the state is touched once).
template <typename ST>
struct StatePiece;
template <>
struct StatePiece<float> {
  f32x4 a, b;
  __device__ __forceinline__ void load(const float* row, int cg) {
    a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(row + piece_col<float>(cg, 0)));
    b = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(row + piece_col<float>(cg, 1)));
  }
  __device__ __forceinline__ float get(int e) const { return e < 4 ? a[e] : b[e - 4]; }
  __device__ __forceinline__ static void store(float* row, int cg, const float* x) {
    const f32x4 y0 = {x[0], x[1], x[2], x[3]}, y1 = {x[4], x[5], x[6], x[7]};
    __builtin_nontemporal_store(y0, reinterpret_cast<f32x4*>(row + piece_col<float>(cg, 0)));
    __builtin_nontemporal_store(y1, reinterpret_cast<f32x4*>(row + piece_col<float>(cg, 1)));
  }
};
template <>
struct StatePiece<__bf16> {
  u32x4 raw;
  __device__ __forceinline__ void load(const __bf16* row, int cg) {
    raw = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(row + piece_col<__bf16>(cg, 0)));
  }
  __device__ __forceinline__ float get(int e) const {
    return (float)__builtin_bit_cast(bf16x8, raw)[e];
  }
  __device__ __forceinline__ static void store(__bf16* row, int cg, const float* x) {
    bf16x8 y;
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = (__bf16)x[e];   // round to nearest even
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4, y),
                                reinterpret_cast<u32x4*>(row + piece_col<__bf16>(cg, 0)));
  }
};

template <typename T, typename ST>
__global__ __launch_bounds__(256) void decode_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                     const T* __restrict__ v, const float* __restrict__ g,
                                                     const float* __restrict__ beta,
                                                     const ST* state_in, ST* state_out,
                                                     int32_t Nqk, int32_t Nv, float scale, int norm,
                                                     T* __restrict__ out, const T* __restrict__ gz,
                                                     const T* __restrict__ gw, float geps) {
  const int bh = blockIdx.x;
  const int n = bh / Nv, h = bh % Nv;
  const int j = h / (Nv / Nqk);
  const int tid = threadIdx.x, l = tid & 63;
  const int cg = tid & 15, rg = tid >> 4;
  const size_t sb = (size_t)bh * kD * kD;

  // the token's operands first (a few small loads, kept raw so that issuing
  // them does not wait), then all of the thread's state pieces; the small
  // loads then arrive while the state is still in flight
  typedef __attribute__((ext_vector_type(4))) T vec4;
  const T* kp = k + ((size_t)n * Nqk + j) * kD;
  const T* qp = q + ((size_t)n * Nqk + j) * kD;
  const vec4 k0 = *reinterpret_cast<const vec4*>(kp + piece_col<ST>(cg, 0));
  const vec4 k1 = *reinterpret_cast<const vec4*>(kp + piece_col<ST>(cg, 1));
  const vec4 q0 = *reinterpret_cast<const vec4*>(qp + piece_col<ST>(cg, 0));
  const vec4 q1 = *reinterpret_cast<const vec4*>(qp + piece_col<ST>(cg, 1));
  const T* vp = v + ((size_t)n * Nv + h) * kD;
  T vr[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) vr[i] = vp[rg + 16 * i];
  const float gv = g[(size_t)n * Nv + h];
  const float bt = beta[(size_t)n * Nv + h];
  // gated norm (gz not NULL): lane cg < 8 of row group rg finishes row
  // rg + 16 cg, so it loads that row's gate and weight
  float zr = 0.f, wr = 1.f;
  if (gz && cg < 8) {
    zr = to_f32(gz[((size_t)n * Nv + h) * kD + rg + 16 * cg]);
    if (gw) wr = to_f32(gw[rg + 16 * cg]);
  }

  StatePiece<ST> s[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) s[i].load(state_in + sb + (size_t)(rg + 16 * i) * kD, cg);

  float kh[8], qh[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    kh[e] = to_f32(k0[e]); kh[e + 4] = to_f32(k1[e]);
    qh[e] = to_f32(q0[e]); qh[e + 4] = to_f32(q1[e]);
  }
  float ssk = 0.f, ssq = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) { ssk += kh[e] * kh[e]; ssq += qh[e] * qh[e]; }
  ssk = group16_sum(ssk);
  ssq = group16_sum(ssq);
  const float rk = norm ? 1.0f / sqrtf(ssk + 1e-6f) : 1.0f;
  const float rq = (norm ? 1.0f / sqrtf(ssq + 1e-6f) : 1.0f) * scale;
  float kq = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) { kh[e] *= rk; qh[e] *= rq; kq += kh[e] * qh[e]; }
  kq = group16_sum(kq);
  const float alpha = expf(gv);
  T* op = out + ((size_t)n * Nv + h) * kD;
  float ov[8];   // the group's output rows rg + 16 i, as stored (dtype T)

#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = rg + 16 * i;
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = s[i].get(e);
    float a = 0.f, b = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) { a += x[e] * kh[e]; b += x[e] * qh[e]; }
    a = group16_sum(a);
    b = group16_sum(b);
    const float delta = bt * (to_f32(vr[i]) - alpha * a);
    ov[i] = to_f32(from_f32<T>(alpha * b + delta * kq));
    if (cg == 0 && !gz) op[row] = from_f32<T>(ov[i]);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = alpha * x[e] + delta * kh[e];
    StatePiece<ST>::store(state_out + sb + (size_t)row * kD, cg, x);
  }
  if (gz) {
    // out = o / sqrt(mean(o^2) + eps) * w * SiLU(z) over the head's 128 rows
    // (blog post section 6): the 16 row groups' sums of squares meet in LDS
    // and every thread adds them in the same order
    __shared__ float part[16];
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) ss += ov[i] * ov[i];
    if (cg == 0) part[rg] = ss;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) tot += part[r];
    const float inv = 1.0f / sqrtf(tot * (1.0f / kD) + geps);
    float o = ov[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) o = cg == i ? ov[i] : o;
    if (cg < 8) op[rg + 16 * cg] = from_f32<T>(o * inv * wr * silu(zr));
  }
  (void)l;
}

// A few tokens per sequence (blog post section 5(2), the token loop run over
// each sequence of a packed batch): the decode step above applied to the
// tokens of sequence n in order, with the state kept in registers in between,
// so S is read once and written once per call whatever the number of tokens.
// Sequence n owns tokens [cu[n], cu[n+1]), clamped into [0, T] so a malformed
// cu_seqlens can only give wrong numbers, never an access outside the caller's
// buffers.  NULL state_in means zeros; NULL state_out skips the final store.
// The next token's operands are loaded while the current one is applied.
template <typename T>
__global__ __launch_bounds__(256) void multi_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                    const T* __restrict__ v, const float* __restrict__ g,
                                                    const float* __restrict__ beta,
                                                    const float* state_in, const int32_t* __restrict__ cu,
                                                    int32_t T_total, float* state_out, int32_t Nqk,
                                                    int32_t Nv, float scale, int norm, T* __restrict__ out) {
  const int bh = blockIdx.x;
  const int n = bh / Nv, h = bh % Nv;
  const int j = h / (Nv / Nqk);
  const int tid = threadIdx.x;
  const int cg = tid & 15, rg = tid >> 4;
  const size_t sb = (size_t)bh * kD * kD;
  const int lo = min(max(cu[n], 0), T_total);
  const int hi = min(max(cu[n + 1], lo), T_total);

  // operands of one token, kept raw until used: this lane's two k and q
  // pieces, the value entries of its 8 rows, the gate and beta
  typedef __attribute__((ext_vector_type(4))) T vec4;
  struct Raw {
    vec4 k0, k1, q0, q1;
    T vr[8];
    float gg, bb;
  };
  auto fetch = [&](int t, Raw& o) {
    const T* kp = k + ((size_t)t * Nqk + j) * kD;
    const T* qp = q + ((size_t)t * Nqk + j) * kD;
    o.k0 = *reinterpret_cast<const vec4*>(kp + piece_col<float>(cg, 0));
    o.k1 = *reinterpret_cast<const vec4*>(kp + piece_col<float>(cg, 1));
    o.q0 = *reinterpret_cast<const vec4*>(qp + piece_col<float>(cg, 0));
    o.q1 = *reinterpret_cast<const vec4*>(qp + piece_col<float>(cg, 1));
    const T* vp = v + ((size_t)t * Nv + h) * kD;
#pragma unroll
    for (int i = 0; i < 8; ++i) o.vr[i] = vp[rg + 16 * i];
    o.gg = g[(size_t)t * Nv + h];
    o.bb = beta[(size_t)t * Nv + h];
  };

  // the first token's operands, then the state: the small loads arrive while
  // the state is in flight
  // (token lo when the sequence has tokens, else token 0, which exists when
  // T > 0; with T = 0 the inputs may be NULL and nothing is fetched)
  Raw cur;
  if (T_total > 0) fetch(lo < hi ? lo : 0, cur);
  float x[8][8];
  if (state_in) {
    StatePiece<float> s[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) s[i].load(state_in + sb + (size_t)(rg + 16 * i) * kD, cg);
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) x[i][e] = s[i].get(e);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) x[i][e] = 0.f;
  }

#pragma unroll 1
  for (int t = lo; t < hi; ++t) {
    Raw nxt;
    fetch(min(t + 1, hi - 1), nxt);   // the last token fetches itself again: in bounds
    float kk[8], qq[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      kk[e] = to_f32(cur.k0[e]); kk[e + 4] = to_f32(cur.k1[e]);
      qq[e] = to_f32(cur.q0[e]); qq[e + 4] = to_f32(cur.q1[e]);
    }
    float ssk = 0.f, ssq = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) { ssk += kk[e] * kk[e]; ssq += qq[e] * qq[e]; }
    ssk = group16_sum(ssk);
    ssq = group16_sum(ssq);
    const float rk = norm ? 1.0f / sqrtf(ssk + 1e-6f) : 1.0f;
    const float rq = (norm ? 1.0f / sqrtf(ssq + 1e-6f) : 1.0f) * scale;
    float kh[8], qh[8], kq = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) { kh[e] = kk[e] * rk; qh[e] = qq[e] * rq; kq += kh[e] * qh[e]; }
    kq = group16_sum(kq);
    const float alpha = expf(cur.gg);
    T* op = out + ((size_t)t * Nv + h) * kD;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float a = 0.f, b = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) { a += x[i][e] * kh[e]; b += x[i][e] * qh[e]; }
      a = group16_sum(a);
      b = group16_sum(b);
      const float delta = cur.bb * (to_f32(cur.vr[i]) - alpha * a);
      if (cg == 0) op[rg + 16 * i] = from_f32<T>(alpha * b + delta * kq);
#pragma unroll
      for (int e = 0; e < 8; ++e) x[i][e] = alpha * x[i][e] + delta * kh[e];
    }
    cur = nxt;
  }

  if (state_out) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      StatePiece<float>::store(state_out + sb + (size_t)(rg + 16 * i) * kD, cg, x[i]);
  }
}

template <typename T>
void launch_multi(const T* q, const T* k, const T* v, const float* g, const float* beta,
                  const float* state_in, const int32_t* cu, int32_t N, int32_t T_total,
                  float* state_out, int32_t Nqk, int32_t Nv, float scale, int norm, T* out,
                  hipStream_t stream, LaunchEvents ev) {
  hipExtLaunchKernelGGL(multi_kernel<T>, dim3((unsigned)N * (unsigned)Nv), dim3(256), 0, stream,
                        ev.start, ev.stop, 0, q, k, v, g, beta, state_in, cu, T_total, state_out,
                        Nqk, Nv, scale, norm, out);
}

template void launch_multi<float>(const float*, const float*, const float*, const float*,
                                  const float*, const float*, const int32_t*, int32_t, int32_t,
                                  float*, int32_t, int32_t, float, int, float*, hipStream_t,
                                  LaunchEvents);
template void launch_multi<__bf16>(const __bf16*, const __bf16*, const __bf16*, const float*,
                                   const float*, const float*, const int32_t*, int32_t, int32_t,
                                   float*, int32_t, int32_t, float, int, __bf16*, hipStream_t,
                                   LaunchEvents);

// ---- decode step with its prologue (blog post sections 3 and 4) fused in
// front: the token's projected q|k|v passes through the causal depthwise conv
// update (each channel's window of 4 cached values gains the new value and
// drops its oldest; output = SiLU(kernel . window + bias), cast to the
// activation dtype T), and the gates are formed from a and b:
//   beta = sigmoid(b),  g = -exp(A_log) softplus(a + dt_bias).
template <typename T>
struct ConvArgs {
  const T* x;          // [N, C] projected q|k|v of the token, C = (2 Nqk + Nv) 128
  const T* cs_in;      // [N, C, 4] cached windows, oldest first
  T* cs_out;           // [N, C, 4] updated windows; never overlaps cs_in
  const T* w;          // [C, 4] kernels (cross-correlation order)
  const T* bias;       // [C] or nullptr
  const float* a;      // [N, Nv]
  const float* b;      // [N, Nv]
  const float* A_log;  // [Nv]
  const float* dt_bias;   // [Nv]
  int32_t C;
};

// The loads of one channel's conv inputs, kept raw so that issuing them does
// not wait for them: the window, the kernel, the new value and the bias.
template <typename T>
struct ConvLoad {
  typedef __attribute__((ext_vector_type(4))) T vec4;
  vec4 win, w;
  T x, bias;
  __device__ __forceinline__ void issue(const ConvArgs<T>& p, int n, int c) {
    const size_t wi = ((size_t)n * p.C + c) * 4;
    win = *reinterpret_cast<const vec4*>(p.cs_in + wi);
    w = *reinterpret_cast<const vec4*>(p.w + (size_t)c * 4);
    x = p.x[(size_t)n * p.C + c];
    bias = p.bias ? p.bias[c] : from_f32<T>(0.0f);
  }
  // Channel c after the conv update, as the activation dtype holds it;
  // `write` also stores the channel's new window.
  __device__ __forceinline__ float finish(const ConvArgs<T>& p, int n, int c, bool write) const {
    const float s1 = to_f32(win[1]), s2 = to_f32(win[2]), s3 = to_f32(win[3]), xf = to_f32(x);
    float y = to_f32(w[0]) * s1 + to_f32(w[1]) * s2 + to_f32(w[2]) * s3 + to_f32(w[3]) * xf;
    y += to_f32(bias);
    y = silu(y);
    if (write) put4<T>(p.cs_out + ((size_t)n * p.C + c) * 4, s1, s2, s3, xf);   // exact
    return to_f32(from_f32<T>(y));
  }
};

// One workgroup per (sequence, value head), the decode kernel's layout.  The
// conv outputs are computed once per workgroup into LDS: thread t takes q/k
// channel t of the group's q/k head (q for t < 128, k after) and, for t < 128,
// v channel t of its value head.  Their loads are issued before the state's,
// so the conv work overlaps the state's arrival.  The first value head of each
// group writes the q/k windows; every head writes its v windows.
template <typename T>
__global__ __launch_bounds__(256) void decode_conv_kernel(ConvArgs<T> p, const float* state_in,
                                                          float* state_out, int32_t Nqk, int32_t Nv,
                                                          float scale, int norm,
                                                          T* __restrict__ out) {
  __shared__ float qk_act[2 * kD], v_act[kD];
  const int bh = blockIdx.x;
  const int n = bh / Nv, h = bh % Nv;
  const int G = Nv / Nqk, j = h / G;
  const int tid = threadIdx.x;
  const int cg = tid & 15, rg = tid >> 4;
  const size_t sb = (size_t)bh * kD * kD;

  const int c_qk = (tid < kD ? j : Nqk + j - 1) * kD + tid;        // q: j*128 + t; k: (Nqk+j)*128 + t-128
  const int c_v = (2 * Nqk + h) * kD + (tid & (kD - 1));            // lanes >= 128 repeat a channel
  ConvLoad<T> lqk, lv;
  lqk.issue(p, n, c_qk);
  lv.issue(p, n, c_v);

  StatePiece<float> s[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) s[i].load(state_in + sb + (size_t)(rg + 16 * i) * kD, cg);

  qk_act[tid] = lqk.finish(p, n, c_qk, h % G == 0);
  const float vt = lv.finish(p, n, c_v, tid < kD);
  if (tid < kD) v_act[tid] = vt;
  const size_t gi = (size_t)n * Nv + h;
  const float z = p.a[gi] + p.dt_bias[h];
  const float softplus = fmaxf(z, 0.0f) + log1pf(expf(-fabsf(z)));
  const float alpha = expf(-expf(p.A_log[h]) * softplus);
  const float bt = 1.0f / (1.0f + expf(-p.b[gi]));
  __syncthreads();

  float kh[8], qh[8], vv[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int col = piece_col<float>(cg, e >> 2) + (e & 3);
    qh[e] = qk_act[col];
    kh[e] = qk_act[kD + col];
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) vv[i] = v_act[rg + 16 * i];

  float ssk = 0.f, ssq = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) { ssk += kh[e] * kh[e]; ssq += qh[e] * qh[e]; }
  ssk = group16_sum(ssk);
  ssq = group16_sum(ssq);
  const float rk = norm ? 1.0f / sqrtf(ssk + 1e-6f) : 1.0f;
  const float rq = (norm ? 1.0f / sqrtf(ssq + 1e-6f) : 1.0f) * scale;
  float kq = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) { kh[e] *= rk; qh[e] *= rq; kq += kh[e] * qh[e]; }
  kq = group16_sum(kq);
  T* op = out + gi * kD;

#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = rg + 16 * i;
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = s[i].get(e);
    float a = 0.f, b = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) { a += x[e] * kh[e]; b += x[e] * qh[e]; }
    a = group16_sum(a);
    b = group16_sum(b);
    const float delta = bt * (vv[i] - alpha * a);
    if (cg == 0) op[row] = from_f32<T>(alpha * b + delta * kq);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = alpha * x[e] + delta * kh[e];
    StatePiece<float>::store(state_out + sb + (size_t)row * kD, cg, x);
  }
}

template <typename T>
void launch_decode_conv(const T* x, const T* cs_in, T* cs_out, const T* w, const T* bias,
                        const float* a, const float* b, const float* A_log, const float* dt_bias,
                        const float* state_in, float* state_out, int32_t N, int32_t Nqk, int32_t Nv,
                        float scale, int norm, T* out, hipStream_t stream, LaunchEvents ev) {
  ConvArgs<T> p{x, cs_in, cs_out, w, bias, a, b, A_log, dt_bias, (2 * Nqk + Nv) * kD};
  hipExtLaunchKernelGGL(decode_conv_kernel<T>, dim3((unsigned)N * (unsigned)Nv), dim3(256), 0,
                        stream, ev.start, ev.stop, 0, p, state_in, state_out, Nqk, Nv, scale, norm,
                        out);
}

#define GDR_CONV_INST(T)                                                                        \
  template void launch_decode_conv<T>(const T*, const T*, T*, const T*, const T*, const float*, \
                                      const float*, const float*, const float*, const float*,   \
                                      float*, int32_t, int32_t, int32_t, float, int, T*,        \
                                      hipStream_t, LaunchEvents);
GDR_CONV_INST(float)
GDR_CONV_INST(__bf16)
#undef GDR_CONV_INST

template <typename T, typename ST>
void launch_decode(const T* q, const T* k, const T* v, const float* g, const float* beta,
                   const ST* state_in, ST* state_out, int32_t N, int32_t Nqk, int32_t Nv,
                   float scale, int norm, T* out, hipStream_t stream, LaunchEvents ev,
                   const T* gate_z, const T* gate_w, float gate_eps) {
  hipExtLaunchKernelGGL(decode_kernel<T, ST>, dim3((unsigned)N * (unsigned)Nv), dim3(256), 0,
                        stream, ev.start, ev.stop, 0, q, k, v, g, beta, state_in, state_out, Nqk,
                        Nv, scale, norm, out, gate_z, gate_w, gate_eps);
}

#define GDR_DECODE_INST(T, ST)                                                                   \
  template void launch_decode<T, ST>(const T*, const T*, const T*, const float*, const float*,  \
                                     const ST*, ST*, int32_t, int32_t, int32_t, float, int, T*, \
                                     hipStream_t, LaunchEvents, const T*, const T*, float);
GDR_DECODE_INST(float, float)
GDR_DECODE_INST(__bf16, float)
GDR_DECODE_INST(float, __bf16)
GDR_DECODE_INST(__bf16, __bf16)
#undef GDR_DECODE_INST

}  // namespace gdr
