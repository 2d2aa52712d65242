// gdr_device.h -- device-side building blocks shared by the libgdr kernels:
// element types, 16x16 matrix-core (MFMA) fragments for gfx950, and wave
// reductions.  gfx950 only; wave64.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdr {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr int kD = 128;      // head dimension (Dk = Dv)
constexpr int kL = 128;      // chunk length
constexpr int kWave = 64;

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(__bf16 x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ __bf16 from_f32<__bf16>(float x) { return (__bf16)x; }

// ---------------------------------------------------------------------------
// 16x16 output-tile MFMA.  For every operand type the lane layout is:
//   A fragment: row  (lane & 15), k = (lane >> 4) * E + e, e < E
//   B fragment: col  (lane & 15), k = (lane >> 4) * E + e, e < E
//   C (f32x4):  col  (lane & 15), row = (lane >> 4) * 4 + i, i < 4
// with E = K / 4 values per lane (bf16: K = 32, E = 8; f32: K = 4, E = 1).
// ---------------------------------------------------------------------------
template <typename T> struct Mma;

template <> struct Mma<__bf16> {
  static constexpr int K = 32;
  static constexpr int E = 8;
  typedef bf16x8 frag;
  static __device__ __forceinline__ f32x4 mma(const frag& a, const frag& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  // E consecutive elements at p (16-byte aligned)
  static __device__ __forceinline__ frag load_contig(const __bf16* p) {
    return *reinterpret_cast<const bf16x8*>(p);
  }
  static __device__ __forceinline__ frag load_strided(const __bf16* p, int stride) {
    frag f;
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = p[e * stride];
    return f;
  }
  static __device__ __forceinline__ frag zero() {
    frag f;
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = (__bf16)0.0f;
    return f;
  }
};

template <> struct Mma<float> {
  static constexpr int K = 4;
  static constexpr int E = 1;
  typedef float frag;
  static __device__ __forceinline__ f32x4 mma(const frag& a, const frag& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ frag load_contig(const float* p) { return *p; }
  static __device__ __forceinline__ frag load_strided(const float* p, int) { return *p; }
  static __device__ __forceinline__ frag zero() { return 0.0f; }
};

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Lane index, opaque to the optimiser: every use recomputes the addresses
// derived from it instead of keeping them live across phases (and out of
// loops), which keeps the register pressure of the long kernels down.
__device__ __forceinline__ int lane_id() {
  int l = threadIdx.x & 63;
  asm volatile("" : "+v"(l));
  return l;
}

// Operand view of a row-major matrix in memory (LDS or global):
// element (r, c) = base[r * ld + c].  A GEMM reads operand A as (m, k) and
// operand B as (n, k).  With KCONTIG the k index is the column c (k runs along
// a row, one vector load per fragment); otherwise k is the row r.
template <typename T, bool KCONTIG>
struct Operand {
  const T* base;
  int ld;
  __device__ __forceinline__ typename Mma<T>::frag frag(int mn, int k) const {
    if (KCONTIG) return Mma<T>::load_contig(base + (size_t)mn * ld + k);
    return Mma<T>::load_strided(base + (size_t)k * ld + mn, ld);
  }
};

// One 16x16 output tile: acc += sum_k A(m0 + ., k) B(n0 + ., k) over k in [k0, k1).
template <typename T, bool AK, bool BK>
__device__ __forceinline__ void mma_tile(f32x4& acc, const Operand<T, AK>& A, const Operand<T, BK>& B,
                                         int m0, int n0, int k0, int k1) {
  const int l = lane_id();
  const int r = l & 15;
  const int kq = (l >> 4) * Mma<T>::E;
  for (int k = k0; k < k1; k += Mma<T>::K) {
    auto a = A.frag(m0 + r, k + kq);
    auto b = B.frag(n0 + r, k + kq);
    acc = Mma<T>::mma(a, b, acc);
  }
}

// A wave's 64x64 block of a 128x128 product: tiles (m0 + 16i, n0 + 16j),
// i, j < 4, reduction over k in [0, K).  A and B fragments are each loaded
// once per k step and reused four times.
template <typename T, bool AK, bool BK>
__device__ __forceinline__ void mma_block64(f32x4 (&acc)[4][4], const Operand<T, AK>& A,
                                            const Operand<T, BK>& B, int m0, int n0, int K) {
  const int l = lane_id();
  const int r = l & 15;
  const int kq = (l >> 4) * Mma<T>::E;
#pragma unroll 2
  for (int k = 0; k < K; k += Mma<T>::K) {
    typename Mma<T>::frag a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = A.frag(m0 + 16 * i + r, k + kq);
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = B.frag(n0 + 16 * j + r, k + kq);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = Mma<T>::mma(a[i], b[j], acc[i][j]);
  }
}

// ---------------------------------------------------------------------------
// Swizzled LDS tiles.  A tile holds rows of W elements of T (W = 128 or 64)
// with no padding; the 16-byte chunks of row r are permuted by XOR with the
// low bits of r.  A matrix-core fragment read (16 lanes reading 16
// consecutive rows at the same 16-byte column chunk) and a row-wise 16-byte
// store then both touch every LDS bank once.
// ---------------------------------------------------------------------------
template <typename T, int W = 128>
struct Sw {
  static constexpr int EPC = 16 / (int)sizeof(T);     // elements per 16-byte chunk
  static constexpr int CPR = W / EPC;                 // chunks per row
  static constexpr int MASK = CPR < 16 ? CPR - 1 : 15;
  static __device__ __forceinline__ int at(int r, int c) {
    const unsigned ur = (unsigned)r, uc = (unsigned)c;
    return (int)(ur * W + (((uc / EPC) ^ (ur & MASK)) * EPC) + (uc % EPC));
  }
};

// Fragment of a swizzled tile at (row, k); k is a multiple of the fragment's
// element count, so the E elements are contiguous.
template <typename T, int W = 128>
__device__ __forceinline__ typename Mma<T>::frag sw_frag(const T* tile, int row, int k) {
  return Mma<T>::load_contig(tile + Sw<T, W>::at(row, k));
}

// acc[i][j] += sum_k A(m0 + 16 i + ., k) B(n0 + 16 j + ., k), k in [0, 128),
// both operands swizzled 128-wide LDS tiles holding rows with k along the row.
template <typename T>
__device__ __forceinline__ void sw_gemm64(f32x4 (&acc)[4][4], const T* A, const T* B, int m0, int n0) {
  const int l = lane_id();
  const int r = l & 15;
  const int kq = (l >> 4) * Mma<T>::E;
  if constexpr (sizeof(T) == 2) {
    // bf16: four k-steps, unrolled with two fragment sets (the reads of step
    // k+1 go out before the products of step k)
    constexpr int KS = kD / Mma<T>::K;
    typename Mma<T>::frag a[2][4], b[2][4];
    auto load = [&](int set, int k) {
#pragma unroll
      for (int i = 0; i < 4; ++i) a[set][i] = sw_frag<T>(A, m0 + 16 * i + r, k + kq);
#pragma unroll
      for (int j = 0; j < 4; ++j) b[set][j] = sw_frag<T>(B, n0 + 16 * j + r, k + kq);
    };
    load(0, 0);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks + 1 < KS) load((ks + 1) & 1, (ks + 1) * Mma<T>::K);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = Mma<T>::mma(a[ks & 1][i], b[ks & 1][j], acc[i][j]);
    }
    return;
  }
#pragma unroll 2
  for (int k = 0; k < kD; k += Mma<T>::K) {
    typename Mma<T>::frag a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = sw_frag<T>(A, m0 + 16 * i + r, k + kq);
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = sw_frag<T>(B, n0 + 16 * j + r, k + kq);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = Mma<T>::mma(a[i], b[j], acc[i][j]);
  }
}

// Two products sharing the A operand: acc1 += A B1^T, acc2 += A B2^T.
template <typename T>
__device__ __forceinline__ void sw_gemm64x2(f32x4 (&acc1)[4][4], f32x4 (&acc2)[4][4], const T* A,
                                            const T* B1, const T* B2, int m0, int n0) {
  const int l = lane_id();
  const int r = l & 15;
  const int kq = (l >> 4) * Mma<T>::E;
#pragma unroll 1
  for (int k = 0; k < kD; k += Mma<T>::K) {
    typename Mma<T>::frag a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = sw_frag<T>(A, m0 + 16 * i + r, k + kq);
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = sw_frag<T>(B1, n0 + 16 * j + r, k + kq);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc1[i][j] = Mma<T>::mma(a[i], b[j], acc1[i][j]);
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = sw_frag<T>(B2, n0 + 16 * j + r, k + kq);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc2[i][j] = Mma<T>::mma(a[i], b[j], acc2[i][j]);
  }
}

// ---------------------------------------------------------------------------
// Workspace order of the four per-(chunk, head) matrices, chosen so that the
// chunk-serial pass reads every operand as whole contiguous blocks (one
// 16-byte, or 8-byte, piece per lane, lanes in order):
//   frag_off(row, k): matrix-core operand order.  Block (row / 16, k / K)
//     holds the 16 x K tile; lane (row % 16) + 16 ((k % K) / E) holds its E
//     consecutive k values.  Used for Mt (rows d) and Qp (rows r).
//   bm_off(v, d): accumulator order of the state waves of the pass
//     (value row v, key column d).
//   ou_off(r, v): accumulator order of its output waves (chunk row r, value v).
// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ int frag_off(int row, int k) {
  constexpr int K = Mma<T>::K, E = Mma<T>::E;
  const int blk = (row >> 4) * (kD / K) + k / K;
  const int lane = (row & 15) + 16 * ((k % K) / E);
  return blk * 64 * E + lane * E + (k % E);
}
// block (vb, wave half, 16-row tile i, 16-column tile t) of 64 lanes x 4 values;
// t is outside wh and i, so the blocks of the 16 state rows 32 vb + 16 t .. are
// one contiguous 4 KiB run (and those of 32 vb .. one 8 KiB run)
__device__ __forceinline__ int pass_blk(int vb, int wh, int i, int t) {
  return (((vb * 2 + t) * 2 + wh) * 4 + i) * 256;
}
__device__ __forceinline__ int bm_off(int v, int d) {
  return pass_blk(v >> 5, d >> 6, (d & 63) >> 4, (v & 31) >> 4) + ((v & 15) + 16 * ((d & 15) >> 2)) * 4 +
         (d & 3);
}
__device__ __forceinline__ int ou_off(int r, int v) {
  return pass_blk(v >> 5, r >> 6, (r & 63) >> 4, (v & 31) >> 4) + ((r & 15) + 16 * ((v & 15) >> 2)) * 4 +
         (v & 3);
}

// Fragment of a k-major swizzled 128-wide bf16 tile X (row index = k):
// lane (i = lane & 15, q = lane >> 4) gets X[k0 + 8 q + e][o0 + i], e < 8,
// from two LDS transpose reads (gfx950 ds_read_b64_tr_b16).  Within each
// group of 16 lanes that instruction hands output lane 4a + b element b of
// the 4 values read by lanes a, a + 4, a + 8 and a + 12, so lane s of the
// group points at X[k0 + 8 q + s / 4][o0 + 4 (s % 4)] (4 values in one
// 16-byte chunk of the tile).
__device__ __forceinline__ bf16x8 sw_frag_tr(const __bf16* tile, int o0, int k0) {
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  const int l = lane_id(), sl = l & 15, q = l >> 4;
  const int row = k0 + 8 * q + (sl >> 2), col = o0 + 4 * (sl & 3);
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16*)(tile + Sw<__bf16>::at(row, col)));
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16*)(tile + Sw<__bf16>::at(row + 4, col)));
  typedef short v8i16 __attribute__((ext_vector_type(8)));
  const v8i16 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, both);
}

// sw_gemm64 with either operand read from a k-major tile (ATR / BTR) through
// transpose reads; bf16 only.  The four k-steps are unrolled with two
// fragment sets: the reads of step k+1 are issued before the products of
// step k, so each step's LDS latency hides behind the previous step's
// matrix instructions.
template <bool ATR, bool BTR>
__device__ __forceinline__ void sw_gemm64_tr(f32x4 (&acc)[4][4], const __bf16* A, const __bf16* B,
                                             int m0, int n0) {
  typedef __bf16 T;
  constexpr int KS = kD / Mma<T>::K;
  const int l = lane_id();
  const int r = l & 15;
  const int kq = (l >> 4) * Mma<T>::E;
  typename Mma<T>::frag a[2][4], b[2][4];
  auto load = [&](int set, int k) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      a[set][i] = ATR ? sw_frag_tr(A, m0 + 16 * i, k) : sw_frag<T>(A, m0 + 16 * i + r, k + kq);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      b[set][j] = BTR ? sw_frag_tr(B, n0 + 16 * j, k) : sw_frag<T>(B, n0 + 16 * j + r, k + kq);
  };
  load(0, 0);
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    if (ks + 1 < KS) load((ks + 1) & 1, (ks + 1) * Mma<T>::K);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = Mma<T>::mma(a[ks & 1][i], b[ks & 1][j], acc[i][j]);
  }
}

template <int M, int N>
__device__ __forceinline__ void zero_acc(f32x4 (&acc)[M][N]) {
#pragma unroll
  for (int i = 0; i < M; ++i)
#pragma unroll
    for (int j = 0; j < N; ++j) acc[i][j] = zero4();
}

// Sum over the 64 lanes of a wave; every lane gets the total.
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

// Lane permutation within rows of 16 lanes by a DPP control (no LDS trip).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL,
                                                               0xF, 0xF, false));
}

// Sum over aligned groups of 16 lanes; every lane of the group gets the total.
// SiLU(x) = x sigmoid(x) = x / (1 + e^-x) with the hardware exponential and
// reciprocal (v_exp_f32, v_rcp_f32, about 1 ulp each): it runs once per
// element of the HBM-bound activation kernels, where the exact division and
// exponential cost more issue slots than the bytes take; its results are
// rounded to the activation dtype or enter fp32 sums far above that error.
// Saturates like the exact form: e^-x = inf gives -0, e^-x = 0 gives x.
__device__ __forceinline__ float silu(float x) {
  return x * __builtin_amdgcn_rcpf(1.0f + __expf(-x));
}

// Butterfly on DPP: swap neighbours, swap pairs (quad sums), mirror within 8
// (half-row sums), mirror within 16 (row sums).
__device__ __forceinline__ float group16_sum(float x) {
  x += dpp_f32<0xB1>(x);    // quad_perm [1,0,3,2]
  x += dpp_f32<0x4E>(x);    // quad_perm [2,3,0,1]
  x += dpp_f32<0x141>(x);   // row_half_mirror
  x += dpp_f32<0x140>(x);   // row_mirror
  return x;
}

}  // namespace gdr
