// gdr_inter.hip -- the chunk-serial half of the chunkwise gated delta rule.
//
// The state pass of the Qwen3-Next blog post, section 5(1)f, in the affine
// form prepared by gdr_intra.hip: for each chunk of a sequence, in order,
//   O      = Qp S^T + Ou                        (the chunk's output rows)
//   S_next = exp(gc_last) S + S M' + Bm         (the state after the chunk)
// with S in R^{Dv x Dk} (row = value index, as in the Ascend operator page's
// state_new [Dv, Dk]).  Rows of S never mix (every term acts on each row of
// S alone), so a workgroup owns 16 rows of S of one (sequence, value head)
// and keeps them in registers, fp32, for the whole sequence: 8 workgroups per
// (sequence, head).  Each of the 4 waves owns 32 key columns of those rows
// (two 16x16 tiles of S^T) and 32 output rows of the chunk; per chunk the
// waves exchange S once through LDS, as the shared B operand of one
// [Mt; Qp] (256 x 128) x S^T (128 x 16) product on the matrix cores.
// Chunk boundaries restart at sequence starts, so a varlen boundary inside a
// 128-token grid needs no special case: a short last chunk only writes its
// first len output rows.
#include "gdr_device.h"
#include "gdr_kernels.h"

namespace gdr {

template <typename T>
__device__ __forceinline__ void put4(T* p, const float* x);
template <>
__device__ __forceinline__ void put4<float>(float* p, const float* x) {
  *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
}
template <>
__device__ __forceinline__ void put4<__bf16>(__bf16* p, const float* x) {
  bf16x4 v;
  v[0] = (__bf16)x[0]; v[1] = (__bf16)x[1]; v[2] = (__bf16)x[2]; v[3] = (__bf16)x[3];
  *reinterpret_cast<bf16x4*>(p) = v;
}

template <typename T>
__device__ __forceinline__ void get4(const T* p, float* x);
template <>
__device__ __forceinline__ void get4<float>(const float* p, float* x) {
  const float4 v = *reinterpret_cast<const float4*>(p);
  x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
}
template <>
__device__ __forceinline__ void get4<__bf16>(const __bf16* p, float* x) {
  const bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
  x[0] = (float)v[0]; x[1] = (float)v[1]; x[2] = (float)v[2]; x[3] = (float)v[3];
}

// Operands of one chunk held by one lane: its A fragments of [Mt; Qp], its
// entries of Bm and Ou, and the chunk's decay exp(gc_last).
template <typename T>
struct ChunkOps {
  static constexpr int KSTEPS = kD / Mma<T>::K;
  typename Mma<T>::frag a[4][KSTEPS];
  float bm[2][4], ou[2][4];
  float gC;
};

template <typename T>
__device__ __forceinline__ void load_ops(ChunkOps<T>& o, const T* __restrict__ mats,
                                         const float* __restrict__ gam, int w, int l, int vcol) {
  constexpr int KSTEPS = ChunkOps<T>::KSTEPS;
  const int r16 = l & 15, kq = (l >> 4) * Mma<T>::E;
  const T* Mt = mats;
  const T* Qp = mats + kD * kD;
  const T* Bm = mats + 2 * kD * kD;
  const T* OuT = mats + 3 * kD * kD;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const T* base = (i < 2 ? Mt : Qp) + (size_t)(32 * w + 16 * (i & 1) + r16) * kD;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) o.a[i][ks] = Mma<T>::load_contig(base + ks * Mma<T>::K + kq);
  }
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int kr = 32 * w + 16 * t + 4 * (l >> 4);
    get4<T>(Bm + (size_t)vcol * kD + kr, o.bm[t]);
    get4<T>(OuT + (size_t)vcol * kD + kr, o.ou[t]);
  }
  o.gC = *gam;
}

template <typename T>
__global__ __launch_bounds__(256) void inter_kernel(
    const T* __restrict__ inter, const int4* __restrict__ table, const int32_t* __restrict__ choff,
    const float* __restrict__ gam, const float* state_in, float* carry, float* state_out,
    int32_t N, int32_t Nv, int32_t slot0, int32_t nseg, int first_segment, T* __restrict__ out) {
  constexpr int LDS_S = kD + 16 / (int)sizeof(T);
  constexpr int KSTEPS = ChunkOps<T>::KSTEPS;
  __shared__ T sS[2][16 * LDS_S];

  // Block -> (sequence b, head h, 16-row block vb).  The 8 row blocks of one
  // (b, h) read the same Mt / Qp matrices, so when possible they are placed
  // on the same XCD (blocks are dealt to the 8 XCDs round-robin) to share
  // that XCD's L2.
  const int id = blockIdx.x;
  const int pairs = N * Nv;
  int bh, vb;
  if ((pairs & 7) == 0) {
    bh = (id & 7) + 8 * (id >> 6);
    vb = (id >> 3) & 7;
  } else {
    bh = id >> 3;
    vb = id & 7;
  }
  const int b = bh / Nv, h = bh % Nv;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int vcol = 16 * vb + (l & 15);          // value row of S held by this lane
  const size_t sbase = (size_t)bh * kD * kD + (size_t)vcol * kD;
  const int c0 = choff[b], c1 = choff[b + 1];

  if (c0 == c1) {
    // empty sequence: its final state is its initial state
    if (first_segment && state_out && state_out != state_in) {
      for (int idx = tid; idx < 16 * kD / 4; idx += 256) {
        const int r = idx / (kD / 4), c = (idx % (kD / 4)) * 4;
        const size_t off = (size_t)bh * kD * kD + (size_t)(16 * vb + r) * kD + c;
        float4 val = make_float4(0.f, 0.f, 0.f, 0.f);
        if (state_in) val = *reinterpret_cast<const float4*>(state_in + off);
        *reinterpret_cast<float4*>(state_out + off) = val;
      }
    }
    return;
  }
  const int cb = max(c0, slot0), ce = min(c1, slot0 + nseg);
  if (cb >= ce) return;
  const float* src = (cb == c0) ? state_in : carry;
  float* dstS = (ce == c1) ? state_out : carry;
  const size_t mstride = (size_t)Nv * 4 * (size_t)(kD * kD);
  const T* mats0 = inter + (size_t)h * 4 * (size_t)(kD * kD) - (size_t)slot0 * mstride;

  // S^T tiles: rows (key index) kr(t, x) = 32 w + 16 t + 4 (l >> 4) + x, column vcol
  float S[2][4];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int kr = 32 * w + 16 * t + 4 * (l >> 4);
    if (src) get4<float>(src + sbase + kr, S[t]);
    else S[t][0] = S[t][1] = S[t][2] = S[t][3] = 0.f;
  }

  const int r16 = l & 15, kq = (l >> 4) * Mma<T>::E;
  int buf = 0;
  // One chunk of the state pass with its operands already in registers.
  auto step = [&](const ChunkOps<T>& o, int c) {
    // S (this block's 16 rows) as the B operand, [v][k] in LDS
#pragma unroll
    for (int t = 0; t < 2; ++t) put4<T>(&sS[buf][r16 * LDS_S + 32 * w + 16 * t + 4 * (l >> 4)], S[t]);
    __syncthreads();
    f32x4 acc[4] = {zero4(), zero4(), zero4(), zero4()};
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      const auto bfr = Mma<T>::load_contig(&sS[buf][r16 * LDS_S + ks * Mma<T>::K + kq]);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = Mma<T>::mma(o.a[i][ks], bfr, acc[i]);
    }
    const int4 e = table[c];
    const int start = e.y, len = e.z;
    // outputs of this chunk (from the state at its start)
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int r = 32 * w + 16 * t + 4 * (l >> 4);
#pragma unroll
      for (int x = 0; x < 4; ++x)
        if (r + x < len)
          out[((size_t)(start + r + x) * Nv + h) * kD + vcol] = from_f32<T>(acc[2 + t][x] + o.ou[t][x]);
    }
    // state update
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int x = 0; x < 4; ++x) S[t][x] = o.gC * S[t][x] + acc[t][x] + o.bm[t][x];
    buf ^= 1;
  };

  // Two register sets: the operands of the next chunk are in flight while
  // the current one is computed (they do not depend on the state).
  ChunkOps<T> A, B;
  load_ops<T>(A, mats0 + (size_t)cb * mstride, gam + (size_t)cb * Nv + h, w, l, vcol);
#pragma unroll 1
  for (int c = cb; c < ce; c += 2) {
    if (c + 1 < ce) load_ops<T>(B, mats0 + (size_t)(c + 1) * mstride, gam + (size_t)(c + 1) * Nv + h, w, l, vcol);
    step(A, c);
    if (c + 1 >= ce) break;
    if (c + 2 < ce) load_ops<T>(A, mats0 + (size_t)(c + 2) * mstride, gam + (size_t)(c + 2) * Nv + h, w, l, vcol);
    step(B, c + 1);
  }

  if (dstS) {
#pragma unroll
    for (int t = 0; t < 2; ++t) put4<float>(dstS + sbase + 32 * w + 16 * t + 4 * (l >> 4), S[t]);
  }
}

template <typename T>
void launch_inter(const T* inter, const int4* table, const int32_t* choff, const float* gam,
                  const float* state_in, float* carry, float* state_out, int32_t N, int32_t Nv,
                  int32_t slot0, int32_t nseg, bool first_segment, T* out, hipStream_t stream) {
  const unsigned blocks = (unsigned)N * (unsigned)Nv * 8u;
  hipLaunchKernelGGL(inter_kernel<T>, dim3(blocks), dim3(256), 0, stream, inter, table, choff, gam,
                     state_in, carry, state_out, N, Nv, slot0, nseg, first_segment ? 1 : 0, out);
}

template void launch_inter<float>(const float*, const int4*, const int32_t*, const float*,
                                  const float*, float*, float*, int32_t, int32_t, int32_t, int32_t,
                                  bool, float*, hipStream_t);
template void launch_inter<__bf16>(const __bf16*, const int4*, const int32_t*, const float*,
                                   const float*, float*, float*, int32_t, int32_t, int32_t, int32_t,
                                   bool, __bf16*, hipStream_t);

}  // namespace gdr
