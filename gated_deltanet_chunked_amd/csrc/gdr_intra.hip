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
//   Ou   = P U = R diag(beta) V                                 [l x Dv]
// leaving the chunk-serial pass (gdr_inter.hip) with
//   O = Qp S^T + Ou,   S_next = exp(gc_last) S + S M' + Bm.
//
// Data flow.  Every product is C = A B^T with both operands read as rows of
// a swizzled LDS tile (k along the row), and every result leaves the
// accumulators transposed (C^T rows are contiguous in a lane), so no operand
// is ever read with a stride.  Two 128x128 LDS slots carry the whole chain:
//   K, Q      -> Grams KK^T (symmetric) and KQ^T, sharing the K fragments
//   N = A+^T  -> slot 0; P stays in registers; slot 1 holds the lower
//                triangular inverse as it is built
//   T^T       -> slot 0 (blocked inverse, below);  P -> slot 1
//   R^T = T^T P^T;  Z = (T^T diag ck) K^T with K staged into slot 1
//   K's rows scaled by xk = beta exp(gc) rk in place; R, then Z^T, into
//   slot 0:  Qp from (R, xk K), Mt from (xk K, Z^T)
//   V's rows scaled by beta into slot 1:  Bm from (Z^T, beta V), then R
//   into slot 0 again:  Ou from (R, beta V)
// so R and Z leave registers for LDS unscaled, and Z's registers are free
// from the Mt product on.
// The four matrices go to the workspace in the order Mt, Qp, Bm, Ou, each in
// the element order the state pass reads (frag_off, bm_off, ou_off in
// gdr_device.h), so that pass loads them as contiguous blocks.
// The triangular inverse follows the blog's subsection d in blocked form:
// 16x16 diagonal blocks by substitution, then three doubling merges
// [X Y; 0 Z]^-1 = [X^-1, -X^-1 Y Z^-1; 0, Z^-1] on the matrix cores (the
// Ascend operator page's inverse sub-kernels use the same doubling idea).
// It inverts I + A+^T (upper triangular), whose inverse T^T is the operand
// every later product needs, and keeps the transpose (lower form) of each
// finished block beside it so that Z^-1 can also be read by rows.
//
// The kernel also does the per-row preparation: the L2 norms of the key and
// query rows, kept as reciprocal row scalings (K = diag(rk) k, Q = diag(rq) q
// with rq including scale), so raw bf16/fp32 inputs feed the matrix cores
// exactly and the scalings are applied in fp32; and the chunk-local gate
// cumsum, in fp64 because exp() is taken of differences of it.  exp(gc_last)
// of every (chunk, head) goes to gam_out for the state pass.
#include "gdr_device.h"
#include "gdr_kernels.h"

namespace gdr {

template <typename T>
struct IntraLds {
  T t0[kD * kD];      // slot 0
  T t1[kD * kD];      // slot 1
  T w[64 * 64];       // inverse scratch (a 64-wide swizzled tile)
  double gc[128];     // chunk-local inclusive cumsum of g
  float beta[128], rk[128], rq[128];
  float ck[128];      // exp(gc_last - gc_i) rk_i
  float xk[128];      // beta_i exp(gc_i) rk_i
  float qs[128];      // exp(gc_i) rq_i
  double part;        // wave 0's cumsum total
};
// 16-byte vector reads of four consecutive rows of gc, beta, rk
static_assert(offsetof(IntraLds<__bf16>, gc) % 16 == 0 && offsetof(IntraLds<float>, gc) % 16 == 0);
static_assert(offsetof(IntraLds<__bf16>, beta) % 16 == 0 && offsetof(IntraLds<float>, beta) % 16 == 0);
static_assert(offsetof(IntraLds<__bf16>, rk) % 16 == 0 && offsetof(IntraLds<float>, rk) % 16 == 0);

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

// Accumulator values kept between products in the storage type (4 per tile).
template <typename T> struct Pack4;
template <> struct Pack4<__bf16> {
  bf16x4 v;
  __device__ __forceinline__ void set(const f32x4& a) {
    v[0] = (__bf16)a[0]; v[1] = (__bf16)a[1]; v[2] = (__bf16)a[2]; v[3] = (__bf16)a[3];
  }
  __device__ __forceinline__ float get(int x) const { return (float)v[x]; }
};
template <> struct Pack4<float> {
  f32x4 v;
  __device__ __forceinline__ void set(const f32x4& a) { v = a; }
  __device__ __forceinline__ float get(int x) const { return v[x]; }
};

// Element (r, c) of a row-major chunk with row stride gs elements, addressed
// with a 32-bit byte offset from the chunk's (workgroup-uniform) base, so a
// load needs one address register.  The host limits head counts so that
// 128 rows of any input span less than 2 GiB.
template <typename T>
__device__ __forceinline__ const T* at_row(const T* base, int r, size_t gs, int c) {
  const uint32_t off = ((uint32_t)r * (uint32_t)gs + (uint32_t)c) * (uint32_t)sizeof(T);
  return reinterpret_cast<const T*>(reinterpret_cast<const char*>(base) + off);
}

// Global loads of padded rows.  A chunk's rows past its length are read
// from a clamped, valid row and then replaced by zeros with a select: a load
// under a branch would be waited for inside the branch, serialising every
// load of a staging loop behind the previous one.

// Four consecutive elements of T loaded raw from global memory; zeros when
// !ok (p must still be a valid address).
template <typename T> struct Quad4;
template <> struct Quad4<__bf16> {
  bf16x4 v;
  __device__ __forceinline__ void load(const __bf16* p, bool ok) {
    const bf16x4 x = *reinterpret_cast<const bf16x4*>(p);
    v = ok ? x : bf16x4{(__bf16)0.f, (__bf16)0.f, (__bf16)0.f, (__bf16)0.f};
  }
  __device__ __forceinline__ float get(int x) const { return (float)v[x]; }
};
template <> struct Quad4<float> {
  f32x4 v;
  __device__ __forceinline__ void load(const float* p, bool ok) {
    const f32x4 x = *reinterpret_cast<const f32x4*>(p);
    v = ok ? x : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  __device__ __forceinline__ float get(int x) const { return v[x]; }
};

// Natural staging: rows [0, len) of a 128-wide global matrix (row stride gs
// elements) into registers, 16 bytes per piece; rows >= len read as zero
// (len >= 1).
template <typename T>
struct RowPieces {
  static constexpr int EPC = 16 / (int)sizeof(T);
  static constexpr int CPR = kD / EPC;              // pieces per row
  static constexpr int N = kD * CPR / 256;          // pieces per thread
  u32x4 p[N];
  // The thread index is made opaque in load and store so the compiler does
  // not hold these addresses live from one staging to the next.
  __device__ __forceinline__ void load(const T* src, size_t gs, int len) {
    int t = threadIdx.x;
    asm volatile("" : "+v"(t));
#pragma unroll
    for (int it = 0; it < N; ++it) {
      const int idx = t + 256 * it;
      const int r = idx / CPR, c = (idx % CPR) * EPC;
      const u32x4 x = *reinterpret_cast<const u32x4*>(at_row(src, min(r, len - 1), gs, c));
      p[it] = r < len ? x : u32x4{0u, 0u, 0u, 0u};
    }
  }
  __device__ __forceinline__ void store(T* tile) const {
    int t = threadIdx.x;
    asm volatile("" : "+v"(t));
#pragma unroll
    for (int it = 0; it < N; ++it) {
      const int idx = t + 256 * it;
      const int r = idx / CPR, c = (idx % CPR) * EPC;
      *reinterpret_cast<u32x4*>(tile + Sw<T>::at(r, c)) = p[it];
    }
  }
  // store with row r of the tile scaled by f[r]
  __device__ __forceinline__ void store_scaled(T* tile, const float* f) const {
    int t = threadIdx.x;
    asm volatile("" : "+v"(t));
#pragma unroll
    for (int it = 0; it < N; ++it) {
      const int idx = t + 256 * it;
      const int r = idx / CPR, c = (idx % CPR) * EPC;
      const float fr = f[r];
      u32x4 raw = p[it];
      T* e = reinterpret_cast<T*>(&raw);
#pragma unroll
      for (int x = 0; x < EPC; ++x) e[x] = from_f32<T>(to_f32(e[x]) * fr);
      *reinterpret_cast<u32x4*>(tile + Sw<T>::at(r, c)) = raw;
    }
  }
  // sum of squares of the piece's elements
  __device__ __forceinline__ float sumsq(int it) const {
    const T* e = reinterpret_cast<const T*>(&p[it]);
    float s = 0.0f;
#pragma unroll
    for (int x = 0; x < EPC; ++x) { const float f = to_f32(e[x]); s += f * f; }
    return s;
  }
};

// Sum over aligned groups of CPR lanes (CPR = 16 or 32), on DPP within
// each 16-lane row (no LDS round trip), one lane swap across row pairs.
template <int CPR>
__device__ __forceinline__ float row_sum(float x) {
  x = group16_sum(x);
  if constexpr (CPR == 32) x += __shfl_xor(x, 16, 64);
  return x;
}

// Transposed staging: tile[d][i] = src[i][d] for tokens i < len (zero
// beyond).  Loaded into registers first (load), written later (store).
template <typename T> struct ColPieces;

// bf16: a wave owns 8-dimension groups cg = w, w + 4, w + 8, w + 12; lane p
// holds tokens 2p and 2p + 1, so each LDS write is one 32-bit word holding a
// token pair, and the 64 lanes of a write cover one full row of the tile.
template <> struct ColPieces<__bf16> {
  u32x4 a[4], b[4];
  __device__ __forceinline__ void load(const __bf16* src, size_t gs, int len) {
    const int w = threadIdx.x >> 6, p = threadIdx.x & 63;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = 8 * (w + 4 * u);
      const u32x4 x = *reinterpret_cast<const u32x4*>(src + (size_t)min(2 * p, len - 1) * gs + c);
      const u32x4 y = *reinterpret_cast<const u32x4*>(src + (size_t)min(2 * p + 1, len - 1) * gs + c);
      a[u] = 2 * p < len ? x : u32x4{0u, 0u, 0u, 0u};
      b[u] = 2 * p + 1 < len ? y : u32x4{0u, 0u, 0u, 0u};
    }
  }
  __device__ __forceinline__ void store(__bf16* tile) const {
    // opaque lane index: keeps the compiler from holding these addresses
    // live from one staging to the next
    int t = threadIdx.x;
    asm volatile("" : "+v"(t));
    const int w = t >> 6, p = t & 63;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = 8 * (w + 4 * u);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t lo = (a[u][e >> 1] >> (16 * (e & 1))) & 0xffffu;
        const uint32_t hi = (b[u][e >> 1] >> (16 * (e & 1))) & 0xffffu;
        *reinterpret_cast<uint32_t*>(tile + Sw<__bf16>::at(c + e, 2 * p)) = lo | (hi << 16);
      }
    }
  }
};

// fp32: a wave owns 4-dimension groups cg = w + 4 u (u < 8) for both token
// halves; lane l holds token l (+ 64).
template <> struct ColPieces<float> {
  f32x4 a[16];
  __device__ __forceinline__ void load(const float* src, size_t gs, int len) {
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int c = 4 * (w + 4 * (u >> 1)), i = l + 64 * (u & 1);
      const f32x4 x = *reinterpret_cast<const f32x4*>(src + (size_t)min(i, len - 1) * gs + c);
      a[u] = i < len ? x : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  // tile[d][i] = src[i][d] * f[i] (f == nullptr: 1)
  __device__ __forceinline__ void store(float* tile, const float* f = nullptr) const {
    int t = threadIdx.x;
    asm volatile("" : "+v"(t));
    const int w = t >> 6, l = t & 63;
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int c = 4 * (w + 4 * (u >> 1)), i = l + 64 * (u & 1);
      const float fi = f ? f[i] : 1.0f;
#pragma unroll
      for (int e = 0; e < 4; ++e) tile[Sw<float>::at(c + e, i)] = a[u][e] * fi;
    }
  }
};

// One 16x16 tile of C = A B^T over k in [0, K): A rows ar + (lane & 15) from
// columns ac + k of a WA-wide swizzled tile, B likewise.  k positions past K
// read as zero (the bf16 fragment spans 32 values of k).
template <typename T, int WA, int WB>
__device__ __forceinline__ f32x4 tile_mma(const T* A, int ar, int ac, const T* B, int br, int bc,
                                          int K) {
  const int l = lane_id();
  const int r = l & 15, kq = (l >> 4) * Mma<T>::E;
  f32x4 acc = zero4();
  for (int k = 0; k < K; k += Mma<T>::K) {
    const bool live = k + kq < K;
    const auto a = live ? sw_frag<T, WA>(A, ar + r, ac + k + kq) : Mma<T>::zero();
    const auto b = live ? sw_frag<T, WB>(B, br + r, bc + k + kq) : Mma<T>::zero();
    acc = Mma<T>::mma(a, b, acc);
  }
  return acc;
}

// One doubling merge of the blocked inverse for finished SZ-blocks: for the
// pair at b0, X = U block (b0, b0), Z = U block (b0+SZ, b0+SZ) whose rows-as-
// columns are the L block, Y = the original N block (b0, b0+SZ).  The new
// top-right block is -X (Y Z); its transpose goes to L's bottom-left block
// (not needed after the last level).
template <typename T, int SZ>
__device__ __forceinline__ void merge_level(IntraLds<T>& s, int w, int l) {
  constexpr int side = SZ / 16, per = side * side;
  constexpr int TPW = (128 / (2 * SZ)) * per / 4;   // 16x16 tiles per wave
  // W^T = (Y Z)^T into the scratch: pair p at scratch rows p * SZ
  {
    f32x4 acc[TPW];
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const int tt = w + 4 * u;
      const int p = tt / per, ti = (tt % per) / side, tj = tt % side;
      const int b0 = 2 * SZ * p;
      acc[u] = tile_mma<T, 128, 128>(s.t0, b0 + 16 * ti, b0 + SZ, s.t1, b0 + SZ + 16 * tj, b0 + SZ, SZ);
    }
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const int tt = w + 4 * u;
      const int p = tt / per, ti = (tt % per) / side, tj = tt % side;
      const int row = p * SZ + 16 * tj + (l & 15), col = 16 * ti + 4 * (l >> 4);
      store4<T>(s.w + Sw<T, 64>::at(row, col), acc[u][0], acc[u][1], acc[u][2], acc[u][3]);
    }
  }
  __syncthreads();
  {
    f32x4 acc[TPW];
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const int tt = w + 4 * u;
      const int p = tt / per, ti = (tt % per) / side, tj = tt % side;
      const int b0 = 2 * SZ * p;
      // C = X W  (rows i of X, rows j of W^T)
      acc[u] = tile_mma<T, 128, 64>(s.t0, b0 + 16 * ti, b0, s.w, p * SZ + 16 * tj, 0, SZ);
    }
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const int tt = w + 4 * u;
      const int p = tt / per, ti = (tt % per) / side, tj = tt % side;
      const int b0 = 2 * SZ * p;
      const int i0 = b0 + 16 * ti + 4 * (l >> 4), j0 = b0 + SZ + 16 * tj + (l & 15);
#pragma unroll
      for (int x = 0; x < 4; ++x) s.t0[Sw<T>::at(i0 + x, j0)] = from_f32<T>(-acc[u][x]);
      if (SZ < 64) store4<T>(s.t1 + Sw<T>::at(j0, i0), -acc[u][0], -acc[u][1], -acc[u][2], -acc[u][3]);
    }
  }
  __syncthreads();
}

// (I + N)^-1 for N strictly upper triangular, 128x128, in place in s.t0
// (upper form U); s.t1 receives the lower form L = U^T block by block (it
// must hold zeros above the diagonal on entry).
template <typename T>
__device__ __forceinline__ void invert_unit_upper(IntraLds<T>& s) {
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  // 1) 16x16 diagonal blocks by back substitution, one column per thread:
  //    x_i = delta_ic - sum_{m > i} N[i][m] x_m, then the block is
  //    overwritten in place.  The 16 threads of a block are lanes of one wave.
  //    The block's rows are read as 16-byte pieces (row i needs the pieces
  //    holding columns > i), four rows at a time and one group ahead of the
  //    rows being solved, so each group costs one LDS round trip.
  if (tid < 128) {
    constexpr int EPC = 16 / (int)sizeof(T);   // elements per piece
    constexpr int PPR = 16 / EPC;               // pieces per block row
    const int b0 = 16 * (tid >> 4), c = tid & 15;
    u32x4 piece[16][PPR];
    auto read_rows = [&](int lo, int hi) {     // rows lo..hi-1
#pragma unroll
      for (int i = lo; i < hi; ++i)
#pragma unroll
        for (int pc = 0; pc < PPR; ++pc)
          if (i < 15 && EPC * pc + EPC - 1 > i)
            piece[i][pc] = *reinterpret_cast<const u32x4*>(s.t0 + Sw<T>::at(b0 + i, b0 + EPC * pc));
    };
    float col[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) col[i] = (i == c) ? 1.0f : 0.0f;
    auto solve_rows = [&](int lo, int hi) {    // rows hi-1 down to lo
#pragma unroll
      for (int i = hi - 1; i >= lo; --i) {
        if (i == 15) continue;
        float acc = 0.0f;
#pragma unroll
        for (int m = i + 1; m < 16; ++m)
          acc += to_f32(reinterpret_cast<const T*>(&piece[i][m / EPC])[m % EPC]) * col[m];
        if (i < c) col[i] = -acc;
      }
    };
    read_rows(12, 16);
    read_rows(8, 12);
    __builtin_amdgcn_sched_barrier(0);
    solve_rows(12, 16);
    read_rows(4, 8);
    __builtin_amdgcn_sched_barrier(0);
    solve_rows(8, 12);
    read_rows(0, 4);
    __builtin_amdgcn_sched_barrier(0);
    solve_rows(4, 8);
    solve_rows(0, 4);
    // every lane's reads of the block come before any lane's writes: the
    // wave issues its LDS accesses in order, and this barrier keeps the
    // compiler from moving the writes above the reads
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int i = 0; i < 16; ++i) s.t0[Sw<T>::at(b0 + i, b0 + c)] = from_f32<T>(col[i]);
    // row c of the lower form is column c of the upper form
#pragma unroll
    for (int i = 0; i < 16; i += 4)
      store4<T>(s.t1 + Sw<T>::at(b0 + c, b0 + i), col[i], col[i + 1], col[i + 2], col[i + 3]);
  }
  __syncthreads();
  // 2) doubling merges 16 -> 32 -> 64 -> 128
  merge_level<T, 16>(s, w, l);
  merge_level<T, 32>(s, w, l);
  merge_level<T, 64>(s, w, l);
}

// In-place scaling of a 128x128 swizzled tile: element (r, c) times f[r]
// (ROWS) or f[c].
template <typename T, bool ROWS>
__device__ __forceinline__ void scale_tile(T* tile, const float* f) {
  constexpr int EPC = 16 / (int)sizeof(T);
  constexpr int NP = kD * kD / EPC / 256;
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
#pragma unroll
  for (int it = 0; it < NP; ++it) {
    const int idx = t + 256 * it;
    const int r = idx / (kD / EPC), c = (idx % (kD / EPC)) * EPC;
    T* p = tile + Sw<T>::at(r, c);
    u32x4 raw = *reinterpret_cast<const u32x4*>(p);
    T* ev = reinterpret_cast<T*>(&raw);
#pragma unroll
    for (int x = 0; x < EPC; ++x) ev[x] = from_f32<T>(to_f32(ev[x]) * (ROWS ? f[r] : f[c + x]));
    *reinterpret_cast<u32x4*>(p) = raw;
  }
}

// Scale-and-store of a wave's 64x64 accumulator block, transposed, into a
// swizzled tile: tile[n][m..m+3] = acc(m.., n) * f[m..m+3] (f == nullptr: 1).
template <typename T, typename Acc>
__device__ __forceinline__ void put_t(T* tile, const Acc (&acc)[4][4], int m0, int n0, const float* f) {
  int l = lane_id();
  asm volatile("" : "+v"(l));   // recompute the addresses at every call
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = m0 + 16 * i + 4 * (l >> 4), n = n0 + 16 * j + (l & 15);
      float s0 = 1.f, s1 = 1.f, s2 = 1.f, s3 = 1.f;
      if (f) { s0 = f[m]; s1 = f[m + 1]; s2 = f[m + 2]; s3 = f[m + 3]; }
      store4<T>(tile + Sw<T>::at(n, m), acc[i][j].get(0) * s0, acc[i][j].get(1) * s1,
                acc[i][j].get(2) * s2, acc[i][j].get(3) * s3);
    }
}

// Four values of row n, columns m..m+3 (m a multiple of 4), stored at
// dst + off(n, m + x).  The pass layouts keep the four contiguous; the
// operand layout does for bf16 (8 consecutive k per lane) but not for fp32.
enum class Lay { Frag, Bm, Ou };
template <typename T, Lay L>
__device__ __forceinline__ int lay_off(int n, int m) {
  if (L == Lay::Frag) return frag_off<T>(n, m);
  if (L == Lay::Bm) return bm_off(n, m);
  return ou_off(n, m);
}
template <typename T, Lay L>
__device__ __forceinline__ void store4_lay(T* dst, int n, int m, float x0, float x1, float x2, float x3) {
  if (L == Lay::Frag && sizeof(T) == 4) {
    dst[lay_off<T, L>(n, m)] = from_f32<T>(x0);
    dst[lay_off<T, L>(n, m + 1)] = from_f32<T>(x1);
    dst[lay_off<T, L>(n, m + 2)] = from_f32<T>(x2);
    dst[lay_off<T, L>(n, m + 3)] = from_f32<T>(x3);
  } else {
    store4<T>(dst + lay_off<T, L>(n, m), x0, x1, x2, x3);
  }
}

// Transposed store of a wave's 64x64 accumulator block into a workspace
// matrix: element (row n, column m) = sign * acc(m, n).
template <typename T, Lay L>
__device__ __forceinline__ void store_t_global(T* dst, const f32x4 (&acc)[4][4], int m0, int n0,
                                               float sign) {
  const int l = lane_id();
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = m0 + 16 * i + 4 * (l >> 4), n = n0 + 16 * j + (l & 15);
      store4_lay<T, L>(dst, n, m, sign * acc[i][j][0], sign * acc[i][j][1], sign * acc[i][j][2],
                       sign * acc[i][j][3]);
    }
}

struct F4 {   // adapter so raw accumulators fit put_t
  f32x4 v;
  __device__ __forceinline__ float get(int x) const { return v[x]; }
};

template <typename T>
__global__ __launch_bounds__(256, 2) void intra_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, Chunks chunks, int32_t Nqk,
    int32_t Nv, int32_t slot0, float scale, int norm, T* __restrict__ inter,
    float* __restrict__ gam_out) {
  __shared__ IntraLds<T> s;
  // bf16 reads K^T and V^T straight from the row-major K and V tiles with
  // LDS transpose reads; fp32 (no 32-bit transpose read) stages K^T and V^T
  constexpr bool kTr = sizeof(T) == 2;
  const int local_slot = blockIdx.x, h = blockIdx.y;
  int start, len;
  if (!chunks.slot(slot0 + local_slot, start, len)) return;
  const int j = h / (Nv / Nqk);
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int m0 = 64 * (w >> 1), n0 = 64 * (w & 1);
  const size_t qk_stride = (size_t)Nqk * kD, v_stride = (size_t)Nv * kD;
  const T* kc = k + ((size_t)start * Nqk + j) * kD;
  const T* qc = q + ((size_t)start * Nqk + j) * kD;
  const T* vc = v + ((size_t)start * Nv + h) * kD;
  T* dst = inter + ((size_t)local_slot * Nv + h) * 4 * (size_t)(kD * kD);

  // ---- 1. k and q rows into registers; gate cumsum; row norms
  RowPieces<T> kr, qr;
  kr.load(kc, qk_stride, len);
  qr.load(qc, qk_stride, len);

  // chunk-local inclusive cumsum of g in fp64 (blog post section 5(1)c) on
  // waves 0 and 1; padded rows (r >= len) carry g = 0 and beta = 0, so they
  // act as empty rows
  double gsum = 0.0;
  float bt = 0.0f;
  if (tid < 128) {
    const bool ok = tid < len;
    const size_t gi = (size_t)(start + min(tid, len - 1)) * Nv + h;
    const float gv = g[gi], bv = beta[gi];
    gsum = ok ? (double)gv : 0.0;
    bt = ok ? bv : 0.0f;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const double y = __shfl_up(gsum, off, 64);
      if (l >= off) gsum += y;
    }
    if (tid == 63) s.part = gsum;
  }

  // L2 norms (Ascend operator page, x / sqrt(sum x^2 + eps), eps = 1e-6)
  constexpr int CPR = RowPieces<T>::CPR;
#pragma unroll
  for (int it = 0; it < RowPieces<T>::N; ++it) {
    const float sk = row_sum<CPR>(kr.sumsq(it));
    const float sq = row_sum<CPR>(qr.sumsq(it));
    const int idx = tid + 256 * it;
    if (idx % CPR == 0) {
      const int r = idx / CPR;
      const bool ok = r < len;
      s.rk[r] = ok ? (norm ? 1.0f / sqrtf(sk + 1e-6f) : 1.0f) : 0.0f;
      s.rq[r] = ok ? (norm ? scale / sqrtf(sq + 1e-6f) : scale) : 0.0f;
    }
  }
  kr.store(s.t0);
  qr.store(s.t1);
  __syncthreads();
  if (tid < 128) {
    if (w == 1) gsum += s.part;
    s.gc[tid] = gsum;
    s.beta[tid] = bt;
  }

  // ---- 2. Grams on raw inputs: G1[a][c] = k_a.k_c, G2[i][r] = k_i.q_r
  f32x4 a1[4][4], a2[4][4];
  zero_acc(a1);
  zero_acc(a2);
  sw_gemm64x2<T>(a1, a2, s.t0, s.t0, s.t1, m0, n0);
  __syncthreads();

  // ---- 3. decay mask and scalings.  Per element (a, c) one exponential
  // serves all three matrices: exp(-|gc_a - gc_c|) is Gamma[a][c] below the
  // diagonal and Gamma[c][a] above it (gc is non-increasing for g <= 0).
  //   N[c][a]  = beta_a rk_a rk_c Gamma[a][c] G1[a][c]   (c < a)  -> slot 0
  //   P[r][i]  = rq_r rk_i Gamma[r][i] G2[i][r]          (i <= r) -> registers
  // The row and column scalars of a lane are read once, rows as vectors
  // (4 consecutive rows a..a+3), before the element loop.  P is kept packed
  // in the storage type (it is stored as such after the inverse).
  Pack4<T> Pp[4][4];
  {
    double gcc[4];
    float rkc[4], rqc[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int c = n0 + 16 * jj + (l & 15);
      gcc[jj] = s.gc[c];
      rkc[jj] = s.rk[c];
      rqc[jj] = s.rq[c];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int a = m0 + 16 * i + 4 * (l >> 4);
      const double2 g01 = *reinterpret_cast<const double2*>(&s.gc[a]);
      const double2 g23 = *reinterpret_cast<const double2*>(&s.gc[a + 2]);
      const f32x4 rka = *reinterpret_cast<const f32x4*>(&s.rk[a]);
      const f32x4 bta = *reinterpret_cast<const f32x4*>(&s.beta[a]);
      const double ga[4] = {g01.x, g01.y, g23.x, g23.y};
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int c = n0 + 16 * jj + (l & 15);
        float nv[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const float ex = __expf(-(float)fabs(ga[x] - gcc[jj]));
          nv[x] = (c < a + x) ? bta[x] * rka[x] * rkc[jj] * ex * a1[i][jj][x] : 0.0f;
          a2[i][jj][x] = (a + x <= c) ? rqc[jj] * rka[x] * ex * a2[i][jj][x] : 0.0f;
        }
        Pp[i][jj].set(a2[i][jj]);
        store4<T>(s.t0 + Sw<T>::at(c, a), nv[0], nv[1], nv[2], nv[3]);
      }
    }
  }
  // zero slot 1: the lower form of the inverse is built into it
  {
    constexpr int NZ = kD * kD * (int)sizeof(T) / 16 / 256;
#pragma unroll
    for (int it = 0; it < NZ; ++it)
      reinterpret_cast<u32x4*>(s.t1)[tid + 256 * it] = u32x4{0u, 0u, 0u, 0u};
  }
  if (tid < 128) {
    const int r = tid;
    const double glast = s.gc[127];
    const double gcr = s.gc[r];
    const float gm = __expf((float)gcr);
    s.ck[r] = __expf((float)(glast - gcr)) * s.rk[r];
    s.xk[r] = s.beta[r] * gm * s.rk[r];
    s.qs[r] = gm * s.rq[r];
    if (r == 0) gam_out[(size_t)(slot0 + local_slot) * Nv + h] = __expf((float)glast);
  }
  __syncthreads();

  // bf16: the K rows that phase 7 stages again are loaded here, so the
  // inverse hides their latency (no stores are outstanding yet)
  RowPieces<T> kn;
  if constexpr (kTr) kn.load(kc, qk_stride, len);

  // ---- 4. T^T = (I + A+^T)^-1 in slot 0
  invert_unit_upper<T>(s);

  // ---- 5. P into slot 1 (the lower form is no longer needed)
  put_t<T>(s.t1, Pp, m0, n0, nullptr);
  __syncthreads();

  // ---- 6. R^T = T^T P^T: acc[j][r] = sum_i T^T[j][i] P[r][i] = R[r][j]
  Pack4<T> Rp[4][4];
  {
    f32x4 acc[4][4];
    zero_acc(acc);
    sw_gemm64<T>(acc, s.t0, s.t1, m0, n0);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) Rp[i][jj].set(acc[i][jj]);
  }
  __syncthreads();

  // ---- 7. T^T diag(ck) in place; K^T into slot 1
  scale_tile<T, false>(s.t0, s.ck);
  // bf16: K rows as they are (coalesced loads), read transposed by the
  // products below; fp32: K^T staged through registers
  if constexpr (kTr) {
    kn.store(s.t1);
  } else {
    ColPieces<T> kt;
    kt.load(kc, qk_stride, len);
    kt.store(s.t1);
  }
  __syncthreads();

  // ---- 8. Z = T^T diag(ck) K:  acc[j][d] = sum_i (T^T ck)[j][i] K^T[d][i]
  Pack4<T> Zp[4][4];
  {
    f32x4 acc[4][4];
    zero_acc(acc);
    if constexpr (kTr) sw_gemm64_tr<false, true>(acc, s.t0, s.t1, m0, n0);
    else sw_gemm64<T>(acc, s.t0, s.t1, m0, n0);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) Zp[i][jj].set(acc[i][jj]);
  }
  __syncthreads();

  // q[r][d..d+3] in the layout of the Qp product (phase 10), loaded here so
  // phase 9 and the product hide their latency
  Quad4<T> qx[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int d = m0 + 16 * i + 4 * (l >> 4);
      const int r = n0 + 16 * jj + (l & 15);
      qx[i][jj].load(at_row(qc, min(r, len - 1), qk_stride, d), r < len);
    }

  // ---- 9. K rows scaled by xk in slot 1, in place (both products with K
  // take diag(xk) on the same side); R into slot 0
  scale_tile<T, kTr>(s.t1, s.xk);   // bf16: rows of K; fp32: columns of K^T
  put_t<T>(s.t0, Rp, m0, n0, nullptr);
  __syncthreads();

  // ---- 10. Qp = Q_dec - R (xk K):  acc[d][r] = sum_j (xk K)^T[d][j] R[r][j]
  RowPieces<T> vn;
  {
    f32x4 acc[4][4];
    zero_acc(acc);
    if constexpr (kTr) sw_gemm64_tr<true, false>(acc, s.t1, s.t0, m0, n0);
    else sw_gemm64<T>(acc, s.t1, s.t0, m0, n0);
    Pack4<T> res[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const float qsr = s.qs[n0 + 16 * jj + (l & 15)];
        res[i][jj].set(f32x4{qsr * qx[i][jj].get(0) - acc[i][jj][0],
                             qsr * qx[i][jj].get(1) - acc[i][jj][1],
                             qsr * qx[i][jj].get(2) - acc[i][jj][2],
                             qsr * qx[i][jj].get(3) - acc[i][jj][3]});
      }
    // bf16: the V rows staged in phase 13 are loaded between the product and
    // its stores: a wave's memory counter retires in order, so loads issued
    // after the stores would wait for them
    if constexpr (kTr) vn.load(vc, v_stride, len);
    T* qp = dst + 1 * kD * kD;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int d = m0 + 16 * i + 4 * (l >> 4);
        const int r = n0 + 16 * jj + (l & 15);
        store4_lay<T, Lay::Frag>(qp, r, d, res[i][jj].get(0), res[i][jj].get(1), res[i][jj].get(2),
                                 res[i][jj].get(3));
      }
  }
  __syncthreads();

  // ---- 11. Z^T into slot 0:  t0[d][j] = Z[j][d]
  put_t<T>(s.t0, Zp, m0, n0, nullptr);
  __syncthreads();

  // ---- 12. M' = -(xk K)^T Z:  acc[e][d] = sum_j (xk K)^T[e][j] Z^T[d][j];  Mt[d][e] = -acc
  {
    f32x4 acc[4][4];
    zero_acc(acc);
    if constexpr (kTr) sw_gemm64_tr<true, false>(acc, s.t1, s.t0, m0, n0);
    else sw_gemm64<T>(acc, s.t1, s.t0, m0, n0);
    store_t_global<T, Lay::Frag>(dst + 0 * kD * kD, acc, m0, n0, -1.0f);
  }
  __syncthreads();

  // ---- 13. V rows scaled by beta into slot 1 (Z^T stays in slot 0)
  if constexpr (kTr) {
    vn.store_scaled(s.t1, s.beta);
  } else {
    ColPieces<T> vt;
    vt.load(vc, v_stride, len);
    vt.store(s.t1, s.beta);
  }
  __syncthreads();

  // ---- 14. Bm = (beta V)^T Z:  acc[d][e] = sum_j Z^T[d][j] (beta V)^T[e][j];  Bm[e][d]
  {
    f32x4 acc[4][4];
    zero_acc(acc);
    if constexpr (kTr) sw_gemm64_tr<false, true>(acc, s.t0, s.t1, m0, n0);
    else sw_gemm64<T>(acc, s.t0, s.t1, m0, n0);
    store_t_global<T, Lay::Bm>(dst + 2 * kD * kD, acc, m0, n0, 1.0f);
  }
  __syncthreads();

  // ---- 15. R into slot 0
  put_t<T>(s.t0, Rp, m0, n0, nullptr);
  __syncthreads();

  // ---- 16. Ou = R (beta V):  acc[e][r] = sum_j (beta V)^T[e][j] R[r][j];  Ou[r][e]
  {
    f32x4 acc[4][4];
    zero_acc(acc);
    if constexpr (kTr) sw_gemm64_tr<true, false>(acc, s.t1, s.t0, m0, n0);
    else sw_gemm64<T>(acc, s.t1, s.t0, m0, n0);
    store_t_global<T, Lay::Ou>(dst + 3 * kD * kD, acc, m0, n0, 1.0f);
  }
}

template <typename T>
hipError_t launch_intra(const T* q, const T* k, const T* v, const float* g, const float* beta,
                        Chunks chunks, int32_t Nqk, int32_t Nv, int32_t slot0, int32_t nseg,
                        float scale, int norm, T* inter, float* gam, hipStream_t stream,
                        LaunchEvents ev) {
  if constexpr (sizeof(T) == 2) {
    // bf16 inputs have their own kernel (gdr_intra_bf16.hip)
    return launch_intra_bf16(q, k, v, g, beta, chunks, Nqk, Nv, slot0, nseg, scale, norm, inter,
                             gam, stream, ev);
  } else {
    hipExtLaunchKernelGGL(intra_kernel<T>, dim3(nseg, Nv), dim3(256), 0, stream, ev.start, ev.stop,
                          0, q, k, v, g, beta, chunks, Nqk, Nv, slot0, scale, norm, inter, gam);
    return hipGetLastError();
  }
}

template hipError_t launch_intra<float>(const float*, const float*, const float*, const float*,
                                        const float*, Chunks, int32_t, int32_t, int32_t,
                                        int32_t, float, int, float*, float*, hipStream_t,
                                        LaunchEvents);
template hipError_t launch_intra<__bf16>(const __bf16*, const __bf16*, const __bf16*, const float*,
                                         const float*, Chunks, int32_t, int32_t, int32_t,
                                         int32_t, float, int, __bf16*, float*, hipStream_t,
                                         LaunchEvents);

}  // namespace gdr
