// gdr_intra.hip -- the intra-chunk half of the chunkwise gated delta rule.
//
// One workgroup (4 waves) per (chunk, value head), all chunks independent.
// Notation of the Qwen3-Next blog post, section 5(1): in a chunk of l <= 128
// rows with normalised keys K, queries Q (scale folded in), values V,
// write strengths beta and chunk-local gate cumsum gc,
//   Gamma[r][i] = exp(gc_r - gc_i) for i <= r, else 0        (subsection c)
//   A+ = strictLower(diag(beta) (K K^T) * Gamma)               (subsection d)
//   T  = (I + A+)^-1                                           (subsection d)
//   U  = T diag(beta) V,  W = T diag(beta exp(gc)) K           (subsection e)
//   P  = (Q K^T) * Gamma, diagonal kept                        (subsection f)
// and the chunk's output and state update (subsection f) are
//   O      = Q_dec S^T + P (U - W S^T),   Q_dec = diag(exp(gc)) Q
//   S_next = exp(gc_last) S + (U - W S^T)^T K_dec,  K_dec = diag(exp(gc_last - gc)) K.
// Both are affine in the chunk's incoming state S, so this kernel folds every
// product that does not involve S into four matrices (R = P T, Z = T^T K_dec):
//   Mt   = M'^T,  M' = -W^T K_dec = -K^T diag(beta exp(gc)) Z   [Dk x Dk]
//   Qp   = Q_dec - P W = Q_dec - R diag(beta exp(gc)) K         [l x Dk]
//   Bm   = U^T K_dec = V^T diag(beta) Z                         [Dv x Dk]
//   OuT  = (P U)^T = (R diag(beta) V)^T                         [Dv x l]
// leaving the chunk-serial pass (gdr_inter.hip) with
//   O = Qp S^T + Ou,   S_next = exp(gc_last) S + S M' + Bm.
// The triangular inverse follows the blog's subsection d in blocked form:
// 16x16 diagonal blocks by substitution, then three doubling merges
// [X Y; 0 Z]^-1 = [X^-1, -X^-1 Y Z^-1; 0, Z^-1] on the matrix cores (the
// Ascend operator page's inverse sub-kernels use the same doubling idea).
// The kernel inverts I + A+^T (upper triangular), whose inverse is T^T, the
// operand every later product needs.
//
// The kernel also does the per-row preparation: the L2 norms of the staged
// key and query rows, kept as reciprocal row scalings (K = diag(rk) k,
// Q = diag(rq) q with rq including scale), so raw bf16/fp32 inputs feed the
// matrix cores exactly and the scalings are applied in fp32; and the
// chunk-local gate cumsum, in fp64 because exp() is taken of differences of
// it.  exp(gc_last) of every (chunk, head) goes to gam_out for the state pass.
#include "gdr_device.h"
#include "gdr_kernels.h"

namespace gdr {

template <typename T>
struct IntraLds {
  static constexpr int LD = kD + 16 / (int)sizeof(T);   // padded row stride (elements)
  static constexpr int LDW = 64 + 16 / (int)sizeof(T);
  T a[128 * LD];
  T b[128 * LD];
  T w[64 * LDW];
  double gc[128];
  float beta[128], rk[128], rq[128];
  float ck[128];   // exp(gc_last - gc_i) * rk_i
  float xk[128];   // beta_i exp(gc_i) rk_i
  float qs[128];   // exp(gc_i) rq_i
};

// 4-element vector store of fp32 values converted to T.
template <typename T>
__device__ __forceinline__ void store4(T* p, float x0, float x1, float x2, float x3);
template <>
__device__ __forceinline__ void store4<float>(float* p, float x0, float x1, float x2, float x3) {
  *reinterpret_cast<float4*>(p) = make_float4(x0, x1, x2, x3);
}
template <>
__device__ __forceinline__ void store4<__bf16>(__bf16* p, float x0, float x1, float x2, float x3) {
  bf16x4 v;
  v[0] = (__bf16)x0; v[1] = (__bf16)x1; v[2] = (__bf16)x2; v[3] = (__bf16)x3;
  *reinterpret_cast<bf16x4*>(p) = v;
}

template <typename T>
__device__ __forceinline__ void load4(const T* p, float& x0, float& x1, float& x2, float& x3);
template <>
__device__ __forceinline__ void load4<float>(const float* p, float& x0, float& x1, float& x2, float& x3) {
  const float4 v = *reinterpret_cast<const float4*>(p);
  x0 = v.x; x1 = v.y; x2 = v.z; x3 = v.w;
}
template <>
__device__ __forceinline__ void load4<__bf16>(const __bf16* p, float& x0, float& x1, float& x2, float& x3) {
  const bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
  x0 = (float)v[0]; x1 = (float)v[1]; x2 = (float)v[2]; x3 = (float)v[3];
}

// Copy rows [0, len) of a 128-wide global matrix (row stride gstride
// elements) into LDS rows of stride LD; rows [len, 128) are zeroed.
template <typename T, int LD>
__device__ __forceinline__ void stage_rows(T* dst, const T* src, size_t gstride, int len) {
  constexpr int VE = 16 / sizeof(T);            // elements per 16-byte vector
  constexpr int VPR = kD / VE;                  // vectors per row
  typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
  for (int idx = threadIdx.x; idx < 128 * VPR; idx += 256) {
    const int r = idx / VPR, c = (idx % VPR) * VE;
    u32x4 val = {0u, 0u, 0u, 0u};
    if (r < len) val = *reinterpret_cast<const u32x4*>(src + (size_t)r * gstride + c);
    *reinterpret_cast<u32x4*>(dst + r * LD + c) = val;
  }
}

// dst[c][r] = src[r][c] for rows r < len of a 128-wide global matrix; the
// columns r >= len of dst are zeroed.
template <typename T, int LD>
__device__ __forceinline__ void stage_transposed(T* dst, const T* src, size_t gstride, int len) {
  constexpr int VE = 16 / sizeof(T);
  constexpr int VPR = kD / VE;
  for (int idx = threadIdx.x; idx < 128 * VPR; idx += 256) {
    const int r = idx / VPR, c = (idx % VPR) * VE;
    T val[VE];
    if (r < len) {
      typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
      const u32x4 raw = *reinterpret_cast<const u32x4*>(src + (size_t)r * gstride + c);
      const T* pv = reinterpret_cast<const T*>(&raw);
#pragma unroll
      for (int e = 0; e < VE; ++e) val[e] = pv[e];
    } else {
#pragma unroll
      for (int e = 0; e < VE; ++e) val[e] = from_f32<T>(0.0f);
    }
#pragma unroll
    for (int e = 0; e < VE; ++e) dst[(c + e) * LD + r] = val[e];
  }
}

// Writes a wave's 64x64 accumulator block transposed into LDS:
// dst[col][row..row+3] = f(row + x, col) * acc, i.e. dst = (acc-matrix)^T,
// each element multiplied by scale[row + x] (or 1 when scale == nullptr).
template <typename T, int LD>
__device__ __forceinline__ void put_transposed(T* dst, const f32x4 (&acc)[4][4], int m0, int n0,
                                               const float* scale) {
  const int l = lane_id();
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = m0 + 16 * i + 4 * (l >> 4);
      const int col = n0 + 16 * j + (l & 15);
      float s0 = 1.f, s1 = 1.f, s2 = 1.f, s3 = 1.f;
      if (scale) { s0 = scale[row]; s1 = scale[row + 1]; s2 = scale[row + 2]; s3 = scale[row + 3]; }
      store4<T>(dst + col * LD + row, acc[i][j][0] * s0, acc[i][j][1] * s1, acc[i][j][2] * s2,
                acc[i][j][3] * s3);
    }
}

// Same, to a global 128x128 row-major matrix, values negated when neg.
template <typename T>
__device__ __forceinline__ void store_transposed_global(T* dst, const f32x4 (&acc)[4][4], int m0,
                                                        int n0, float sign) {
  const int l = lane_id();
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = m0 + 16 * i + 4 * (l >> 4);
      const int col = n0 + 16 * j + (l & 15);
      store4<T>(dst + col * kD + row, sign * acc[i][j][0], sign * acc[i][j][1],
                sign * acc[i][j][2], sign * acc[i][j][3]);
    }
}

// (I + N)^-1 in place for N strictly upper triangular, 128x128 in s.a.
template <typename T>
__device__ __forceinline__ void invert_unit_upper(IntraLds<T>& s) {
  constexpr int LD = IntraLds<T>::LD, LDW = IntraLds<T>::LDW;
  const int tid = threadIdx.x, w = tid >> 6;
  // 1) 16x16 diagonal blocks by back substitution, one column per thread:
  //    V[i][c] = delta_ic - sum_{i < m <= c} N[i][m] V[m][c].
  if (tid < 128) {
    const int b0 = 16 * (tid >> 4), c = tid & 15;
    float col[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) col[i] = (i == c) ? 1.0f : 0.0f;
#pragma unroll
    for (int i = 14; i >= 0; --i) {
      const T* nrow = s.a + (b0 + i) * LD + b0;
      float acc = 0.0f;
#pragma unroll
      for (int m = i + 1; m < 16; ++m) acc += to_f32(nrow[m]) * col[m];
      if (i < c) col[i] = -acc;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) s.a[(b0 + i) * LD + b0 + c] = from_f32<T>(col[i]);
  }
  __syncthreads();
  // 2) doubling merges: the top-right block of each 2s x 2s diagonal block
  //    becomes -X Y Z with X, Z its (already inverted) diagonal blocks and Y
  //    the original top-right block.
  const int l = lane_id();
#pragma unroll 1
  for (int sz = 16; sz < 128; sz *= 2) {
    const int tiles_side = sz / 16;
    const int tiles_pair = tiles_side * tiles_side;
    const int ntiles = (128 / (2 * sz)) * tiles_pair;   // sz / 4
    // W1 = Y Z into s.w (pair p at rows p * sz)
    for (int tt = w; tt < ntiles; tt += 4) {
      const int p = tt / tiles_pair, ti = (tt % tiles_pair) / tiles_side, tj = tt % tiles_side;
      const int b0 = 2 * sz * p;
      const Operand<T, true> Y{s.a + b0 * LD + (b0 + sz), LD};
      const Operand<T, false> Z{s.a + (b0 + sz) * LD + (b0 + sz), LD};
      f32x4 acc = zero4();
      const int r = l & 15, kq = (l >> 4) * Mma<T>::E;
      for (int k = 0; k < sz; k += Mma<T>::K) {
        const bool live = k + kq < sz;
        auto a = live ? Y.frag(16 * ti + r, k + kq) : Mma<T>::zero();
        auto bf = live ? Z.frag(16 * tj + r, k + kq) : Mma<T>::zero();
        acc = Mma<T>::mma(a, bf, acc);
      }
      const int row = 16 * ti + 4 * (l >> 4), col = 16 * tj + (l & 15);
#pragma unroll
      for (int x = 0; x < 4; ++x) s.w[(p * sz + row + x) * LDW + col] = from_f32<T>(acc[x]);
    }
    __syncthreads();
    // top-right = -X W1
    for (int tt = w; tt < ntiles; tt += 4) {
      const int p = tt / tiles_pair, ti = (tt % tiles_pair) / tiles_side, tj = tt % tiles_side;
      const int b0 = 2 * sz * p;
      const Operand<T, true> X{s.a + b0 * LD + b0, LD};
      const Operand<T, false> W1{s.w + (p * sz) * LDW, LDW};
      f32x4 acc = zero4();
      const int r = l & 15, kq = (l >> 4) * Mma<T>::E;
      for (int k = 0; k < sz; k += Mma<T>::K) {
        const bool live = k + kq < sz;
        auto a = live ? X.frag(16 * ti + r, k + kq) : Mma<T>::zero();
        auto bf = live ? W1.frag(16 * tj + r, k + kq) : Mma<T>::zero();
        acc = Mma<T>::mma(a, bf, acc);
      }
      const int row = 16 * ti + 4 * (l >> 4), col = 16 * tj + (l & 15);
#pragma unroll
      for (int x = 0; x < 4; ++x) s.a[(b0 + row + x) * LD + (b0 + sz + col)] = from_f32<T>(-acc[x]);
    }
    __syncthreads();
  }
}

template <typename T>
__global__ __launch_bounds__(256) void intra_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, const int4* __restrict__ table,
    int32_t Nqk, int32_t Nv, int32_t slot0, float scale, int norm, T* __restrict__ inter,
    float* __restrict__ gam_out) {
  constexpr int LD = IntraLds<T>::LD;
  __shared__ IntraLds<T> s;
  const int local_slot = blockIdx.x, h = blockIdx.y;
  const int4 e = table[slot0 + local_slot];
  if (e.x < 0) return;
  const int start = e.y, len = e.z;
  const int j = h / (Nv / Nqk);
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int m0 = 64 * (w >> 1), n0 = 64 * (w & 1);
  const size_t qk_stride = (size_t)Nqk * kD, v_stride = (size_t)Nv * kD;
  const T* kc = k + ((size_t)start * Nqk + j) * kD;
  const T* qc = q + ((size_t)start * Nqk + j) * kD;
  const T* vc = v + ((size_t)start * Nv + h) * kD;
  T* dst = inter + ((size_t)local_slot * Nv + h) * 4 * (size_t)(kD * kD);

  stage_rows<T, LD>(s.b, kc, qk_stride, len);
  stage_rows<T, LD>(s.a, qc, qk_stride, len);

  // Chunk-local inclusive cumsum of g in fp64 (blog post section 5(1)c),
  // rows r < 128 on waves 0 and 1.  Padded rows (r >= len) carry g = 0, so
  // their cumsum equals the chunk total and they act as empty rows.
  double gsum = 0.0;
  float bt = 0.0f;
  if (tid < 128) {
    const bool ok = tid < len;
    gsum = ok ? (double)g[(size_t)(start + tid) * Nv + h] : 0.0;
    bt = ok ? beta[(size_t)(start + tid) * Nv + h] : 0.0f;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const double y = __shfl_up(gsum, off, 64);
      if (l >= off) gsum += y;
    }
    if (tid == 63) s.gc[0] = gsum;   // wave 0's total, read by wave 1 below
  }
  __syncthreads();

  // L2 norms of the staged key and query rows (Ascend operator page,
  // x / sqrt(sum x^2 + eps), eps = 1e-6), two threads per row.
  {
    const int r = tid >> 1, half = tid & 1;
    float sk = 0.0f, sq = 0.0f;
#pragma unroll 8
    for (int c = 64 * half; c < 64 * half + 64; ++c) {
      const float xk = to_f32(s.b[r * LD + c]), xq = to_f32(s.a[r * LD + c]);
      sk += xk * xk;
      sq += xq * xq;
    }
    sk += __shfl_xor(sk, 1, 64);
    sq += __shfl_xor(sq, 1, 64);
    if (half == 0) {
      const bool ok = r < len;
      s.rk[r] = ok ? (norm ? 1.0f / sqrtf(sk + 1e-6f) : 1.0f) : 0.0f;
      s.rq[r] = ok ? (norm ? scale / sqrtf(sq + 1e-6f) : scale) : 0.0f;
    }
  }
  const double wave0_total = s.gc[0];
  __syncthreads();
  if (tid < 128) {
    if (w == 1) gsum += wave0_total;
    s.gc[tid] = gsum;
    s.beta[tid] = bt;
  }
  __syncthreads();
  if (tid < 128) {
    const int r = tid;
    const double glast = s.gc[127];
    const double gc = s.gc[r];
    const float gm = __expf((float)gc);
    s.ck[r] = __expf((float)(glast - gc)) * s.rk[r];
    s.xk[r] = s.beta[r] * gm * s.rk[r];
    s.qs[r] = gm * s.rq[r];
    if (r == 0) gam_out[(size_t)(slot0 + local_slot) * Nv + h] = __expf((float)glast);
  }

  // Grams on raw inputs: KK[a][c] = k_a.k_c and C2[i][r] = k_i.q_r
  f32x4 acc1[4][4], acc2[4][4];
  zero_acc(acc1);
  zero_acc(acc2);
  {
    const Operand<T, true> Kop{s.b, LD}, Qop{s.a, LD};
    mma_block64(acc1, Kop, Kop, m0, n0, kD);
    mma_block64(acc2, Kop, Qop, m0, n0, kD);
  }
  __syncthreads();

  // N = A+^T into s.a:  N[c][a] = beta_a rk_a rk_c Gamma[a][c] KK[a][c] for c < a
  // P into s.b:         P[r][i] = rq_r rk_i Gamma[r][i] (q_r.k_i)   for i <= r
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int row = m0 + 16 * i + 4 * (l >> 4);
      const int col = n0 + 16 * jj + (l & 15);
      float nv[4], pv[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int a = row + x;   // acc1: (a, c = col);  acc2: (i = a, r = col)
        nv[x] = 0.0f;
        if (col < a)
          nv[x] = s.beta[a] * s.rk[a] * s.rk[col] * __expf((float)(s.gc[a] - s.gc[col])) * acc1[i][jj][x];
        pv[x] = 0.0f;
        if (a <= col)
          pv[x] = s.rq[col] * s.rk[a] * __expf((float)(s.gc[col] - s.gc[a])) * acc2[i][jj][x];
      }
      store4<T>(s.a + col * LD + row, nv[0], nv[1], nv[2], nv[3]);
      store4<T>(s.b + col * LD + row, pv[0], pv[1], pv[2], pv[3]);
    }
  __syncthreads();

  invert_unit_upper<T>(s);   // s.a = T^T

  // R^T = T^T P^T:  accR[j][r] = sum_i T^T[j][i] P[r][i]  (so lane holds R[r][j..j+3])
  f32x4 accR[4][4];
  zero_acc(accR);
  mma_block64(accR, Operand<T, true>{s.a, LD}, Operand<T, true>{s.b, LD}, m0, n0, kD);
  __syncthreads();

  // T^T diag(ck) in place; raw K^T into s.b
  for (int idx = tid; idx < 128 * 128; idx += 256) {
    const int r = idx >> 7, c = idx & 127;
    s.a[r * LD + c] = from_f32<T>(to_f32(s.a[r * LD + c]) * s.ck[c]);
  }
  stage_transposed<T, LD>(s.b, kc, qk_stride, len);
  __syncthreads();

  // Z = T^T K_dec:  accZ[j][d] = sum_i (T^T diag(ck))[j][i] K^T[d][i]
  f32x4 accZ[4][4];
  zero_acc(accZ);
  mma_block64(accZ, Operand<T, true>{s.a, LD}, Operand<T, true>{s.b, LD}, m0, n0, kD);
  __syncthreads();

  // M' = -K^T diag(xk) Z:  C[e][d] = sum_j K^T[e][j] (Z[j][d] xk_j);  store Mt[d][e] = M'[e][d]
  put_transposed<T, LD>(s.a, accZ, m0, n0, s.xk);   // s.a[d][j] = Z[j][d] xk_j
  __syncthreads();
  {
    f32x4 acc[4][4];
    zero_acc(acc);
    mma_block64(acc, Operand<T, true>{s.b, LD}, Operand<T, true>{s.a, LD}, m0, n0, kD);
    store_transposed_global<T>(dst + 0 * kD * kD, acc, m0, n0, -1.0f);
  }
  __syncthreads();

  // Qp = Q_dec - R diag(xk) K:  C[d][r] = sum_j K^T[d][j] (R[r][j] xk_j)
  put_transposed<T, LD>(s.a, accR, m0, n0, s.xk);   // s.a[r][j] = R[r][j] xk_j
  __syncthreads();
  {
    f32x4 acc[4][4];
    zero_acc(acc);
    mma_block64(acc, Operand<T, true>{s.b, LD}, Operand<T, true>{s.a, LD}, m0, n0, kD);
    T* qp = dst + 1 * kD * kD;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int d = m0 + 16 * i + 4 * (l >> 4);
        const int r = n0 + 16 * jj + (l & 15);
        float x0 = 0.f, x1 = 0.f, x2 = 0.f, x3 = 0.f;
        if (r < len) load4<T>(qc + (size_t)r * qk_stride + d, x0, x1, x2, x3);
        const float qsr = s.qs[r];
        store4<T>(qp + r * kD + d, qsr * x0 - acc[i][jj][0], qsr * x1 - acc[i][jj][1],
                  qsr * x2 - acc[i][jj][2], qsr * x3 - acc[i][jj][3]);
      }
  }
  __syncthreads();

  // Ou = R diag(beta) V:  C[r][e] = sum_j (R[r][j] beta_j) V^T[e][j];  store OuT[e][r]
  stage_transposed<T, LD>(s.b, vc, v_stride, len);
  put_transposed<T, LD>(s.a, accR, m0, n0, s.beta);   // s.a[r][j] = R[r][j] beta_j
  __syncthreads();
  {
    f32x4 acc[4][4];
    zero_acc(acc);
    mma_block64(acc, Operand<T, true>{s.a, LD}, Operand<T, true>{s.b, LD}, m0, n0, kD);
    store_transposed_global<T>(dst + 3 * kD * kD, acc, m0, n0, 1.0f);
  }
  __syncthreads();

  // Bm = V^T diag(beta) Z:  C[d][e] = sum_j (Z[j][d] beta_j) V^T[e][j];  store Bm[e][d]
  put_transposed<T, LD>(s.a, accZ, m0, n0, s.beta);   // s.a[d][j] = Z[j][d] beta_j
  __syncthreads();
  {
    f32x4 acc[4][4];
    zero_acc(acc);
    mma_block64(acc, Operand<T, true>{s.a, LD}, Operand<T, true>{s.b, LD}, m0, n0, kD);
    store_transposed_global<T>(dst + 2 * kD * kD, acc, m0, n0, 1.0f);
  }
}

template <typename T>
hipError_t launch_intra(const T* q, const T* k, const T* v, const float* g, const float* beta,
                        const int4* table, int32_t Nqk, int32_t Nv, int32_t slot0, int32_t nseg,
                        float scale, int norm, T* inter, float* gam, hipStream_t stream) {
  hipLaunchKernelGGL(intra_kernel<T>, dim3(nseg, Nv), dim3(256), 0, stream, q, k, v, g, beta, table,
                     Nqk, Nv, slot0, scale, norm, inter, gam);
  return hipGetLastError();
}

template hipError_t launch_intra<float>(const float*, const float*, const float*, const float*,
                                        const float*, const int4*, int32_t, int32_t, int32_t,
                                        int32_t, float, int, float*, float*, hipStream_t);
template hipError_t launch_intra<__bf16>(const __bf16*, const __bf16*, const __bf16*, const float*,
                                         const float*, const int4*, int32_t, int32_t, int32_t,
                                         int32_t, float, int, __bf16*, float*, hipStream_t);

}  // namespace gdr
