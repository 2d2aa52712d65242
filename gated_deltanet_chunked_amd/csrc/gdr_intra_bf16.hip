// gdr_intra_bf16.hip -- the intra-chunk half of the chunkwise gated delta
// rule for bf16 inputs.
//
// It computes, per (chunk, value head), the same four matrices as the fp32
// kernel in gdr_intra.hip (notation of the Qwen3-Next blog post, section 5(1);
// R = P T, Z = T^T diag(ck) K):
//   Mt = M'^T,  M' = -K^T diag(beta exp(gc)) Z                 [Dk x Dk]
//   Qp = diag(exp(gc)) Q - R diag(beta exp(gc)) K              [l x Dk]
//   Bm = V^T diag(beta) Z                                      [Dv x Dk]
//   Ou = R diag(beta) V                                        [l x Dv]
// in the workspace orders the chunk-serial pass reads (store_block below),
// and exp(gc_last) of the chunk.
//
// What differs from the fp32 kernel is how the work maps onto gfx950:
//  * K, Q and V enter the matrix cores as the raw bf16 inputs (exact); the
//    L2 norms (the Ascend operator page's x / sqrt(sum x^2 + 1e-6)), q's
//    scale, beta and the decays are fp32 row and column factors applied to
//    accumulators or folded into one scaled copy.
//  * The two Grams share one pass: the strictly lower tiles of the 128x128
//    product are K K^T (for A+), the upper ones K Q^T (for P), and only the
//    8 diagonal tiles need both, so a wave whose 64x64 block lies off the
//    diagonal computes one product.
//  * Every LDS address is a per-lane offset computed once at kernel start
//    plus a compile-time constant (the 16-byte swizzle of a row depends only
//    on the row's low bits and the lane), so fragment reads and tile stores
//    cost no vector ALU work, and the reads of the next k-step go out
//    between the current step's matrix instructions.
//  * 64-token chunks go two to a workgroup, as a block-diagonal 128-row unit
//    (the PAIR instantiation of the kernel).
#include "gdr_device.h"
#include "gdr_kernels.h"

namespace gdr {
namespace {

typedef __bf16 bf;
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));

constexpr uint32_t kT0 = 0;          // byte offset of LDS slot 0
constexpr uint32_t kT1 = 32768;      // slot 1
constexpr uint32_t kW = 65536;       // inverse scratch (64 rows of 64)

struct Lds {
  bf t0[128 * 128];
  bf t1[128 * 128];
  bf w[64 * 64];
  float gc[128];        // chunk-local cumsum of g times log2(e) (fp32, from an fp64 scan)
  float beta[128];
  float rk[128];        // 1 / |k_r| (0 past the chunk's end)
  float rq[128];        // scale / |q_r|
  float brk[128];       // beta_r rk_r
  float ck[128];        // exp(gc_last - gc_r) rk_r
  float xk[128];        // beta_r exp(gc_r) rk_r
  float qs[128];        // exp(gc_r) rq_r
  double part[2];       // each scanning wave's total of g
};
static_assert(offsetof(Lds, t1) == kT1 && offsetof(Lds, w) == kW, "LDS layout");
static_assert(offsetof(Lds, gc) % 16 == 0 && offsetof(Lds, rk) % 16 == 0 &&
              offsetof(Lds, brk) % 16 == 0, "float4 rows");

__device__ __forceinline__ const char* lds_c(const Lds& s) { return reinterpret_cast<const char*>(&s); }
__device__ __forceinline__ char* lds_m(Lds& s) { return reinterpret_cast<char*>(&s); }

__device__ __forceinline__ bf16x8 rd16(const Lds& s, uint32_t off) {
  return *reinterpret_cast<const bf16x8*>(lds_c(s) + off);
}
__device__ __forceinline__ v4i16 rd_tr(const Lds& s, uint32_t off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16*)(lds_c(s) + off));
}
__device__ __forceinline__ void wr8(Lds& s, uint32_t off, float x0, float x1, float x2, float x3) {
  bf16x4 v;
  v[0] = (bf)x0; v[1] = (bf)x1; v[2] = (bf)x2; v[3] = (bf)x3;
  *reinterpret_cast<bf16x4*>(lds_m(s) + off) = v;
}

// Workgroup barrier for LDS hand-offs only.  __syncthreads() also waits for
// the wave's outstanding global loads and stores, which would expose the
// latency of every prefetch and every store of a finished matrix at the next
// barrier; here only LDS operations are waited for, and global accesses stay
// in flight across the barrier (no other wave reads what they write).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// XOR key of row r's 16-byte chunk indices: r mod 16, with bit 0 also folded
// into bits 2 and 3.  Measured on gfx950, ds_read_b128 serves 16 lanes and
// ds_read_b64_tr_b16 32 lanes per cycle from 64 banks (a 256-byte line).  Any
// 16 consecutive rows from a multiple of 16 get 16 distinct keys, so a row
// fragment read (16 rows, one chunk each) is conflict-free; the 8 rows
// {8 q + x + 4 h} (q < 2, x < 4) of half a transposed read (two adjacent
// chunks each) get 8 distinct keys / 2, so it is conflict-free too (with
// r mod 16 alone: two-way).  Rows 16 apart share the key.
__device__ __forceinline__ uint32_t swkey(uint32_t r) { return (r & 15u) ^ ((r & 1u) * 12u); }

// Byte offset of element (r, c) of a swizzled 128-wide bf16 tile.
__device__ __forceinline__ uint32_t sw(uint32_t r, uint32_t c) {
  return r * 256u + ((((c >> 3) ^ swkey(r))) << 4) + ((c & 7u) << 1);
}
// The same for the 64-wide scratch (8 chunks per row, two rows per 256-byte
// line): the key (r / 2) mod 8 gives 16 consecutive rows 16 distinct chunk
// positions (with r mod 8, rows r and r + 8 met on the same banks).
__device__ __forceinline__ uint32_t sw64(uint32_t r, uint32_t c) {
  return kW + r * 128u + ((((c >> 3) ^ ((r >> 1) & 7u))) << 4) + ((c & 7u) << 1);
}

// Per-lane LDS offsets, fixed for the whole kernel.  A wave owns the 64x64
// output block (m0, n0) of every 128x128 product; r16 = lane % 16, q = lane / 16.
struct Lane {
  uint32_t fa[4], fb[4];     // fragment rows m0 + r16 / n0 + r16 at k-step ks (+ 4096 i)
  uint32_t ta[4][2];         // transposed fragment of operand rows m0 + 16 i (lo, hi reads; + 8192 ks)
  uint32_t tflip;            // ta ^ tflip: the same for rows n0 + 16 j (m0 and n0 differ by 0 or 64)
  uint32_t pt[4];            // accumulator tile (i, j) stored transposed: + 4096 j
  uint32_t stg;              // staging piece of thread t (row t / 16, chunk t % 16; + 4096 it)
};

__device__ __forceinline__ Lane make_lane(int m0, int n0) {
  Lane L;
  const uint32_t t = threadIdx.x, l = t & 63u, r16 = l & 15u, q = l >> 4;
#pragma unroll
  for (uint32_t ks = 0; ks < 4; ++ks) {
    L.fa[ks] = (m0 + r16) * 256u + ((((4u * ks + q) ^ swkey(r16))) << 4);
    L.fb[ks] = (n0 + r16) * 256u + ((((4u * ks + q) ^ swkey(r16))) << 4);
  }
#pragma unroll
  for (uint32_t i = 0; i < 4; ++i) {
#pragma unroll
    for (uint32_t h = 0; h < 2; ++h) {
      // lane (r16, q) of a transposed read points at row 8 q + r16 / 4 (+ 4 for
      // the high half) and column o0 + 4 (r16 % 4): ds_read_b64_tr_b16 then
      // hands every lane 4 consecutive rows of its column (gdr_device.h)
      const uint32_t row = 8u * q + (r16 >> 2) + 4u * h;
      L.ta[i][h] = sw(row, m0 + 16u * i + 4u * (r16 & 3u));
    }
    L.pt[i] = sw(n0 + r16, m0 + 16u * i + 4u * q);
  }
  // columns c and c ^ 64 differ in bit 3 of the chunk index only, which the
  // swizzle leaves in place: their offsets differ in bit 7
  L.tflip = (uint32_t)(m0 ^ n0) << 1;
  L.stg = sw(t >> 4, (t & 15u) * 8u);
  return L;
}

// Transposed fragment (8 consecutive k of one output index) from two reads.
__device__ __forceinline__ bf16x8 frag_tr(const Lds& s, uint32_t lo, uint32_t hi) {
  const v8i16 both = __builtin_shufflevector(rd_tr(s, lo), rd_tr(s, hi), 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, both);
}

__device__ __forceinline__ f32x4 mma(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// A wave's 64x64 block of C = A B^T over k in [32 KB, 32 KE): A rows m0 + 16 i from
// the tile at ABASE (ATR: read transposed, i.e. A(m, k) = X[k][m]), B rows
// n0 + 16 j from BBASE likewise.  DB: the reads of k-step ks + 1 are issued
// before the matrix instructions of step ks (two fragment sets); without it
// one set, for phases where registers are short.  A k range narrower than
// [0, 4) serves products over token rows where the other rows contribute
// exact zeros (a pair of 64-token chunks).
template <uint32_t ABASE, bool ATR, uint32_t BBASE, bool BTR, bool DB = true, int KB = 0,
          int KE = 4>
__device__ __forceinline__ void gemm64(f32x4 (&acc)[4][4], const Lds& s, const Lane& L) {
  constexpr int NS = DB ? 2 : 1;
  bf16x8 a[NS][4], b[NS][4];
  auto load = [&](int set, int ks) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      a[set][i] = ATR ? frag_tr(s, ABASE + L.ta[i][0] + 8192u * ks, ABASE + L.ta[i][1] + 8192u * ks)
                      : rd16(s, ABASE + L.fa[ks] + 4096u * i);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      b[set][j] = BTR ? frag_tr(s, BBASE + (L.ta[j][0] ^ L.tflip) + 8192u * ks,
                                BBASE + (L.ta[j][1] ^ L.tflip) + 8192u * ks)
                      : rd16(s, BBASE + L.fb[ks] + 4096u * j);
  };
  constexpr int NR = (ATR ? 8 : 4) + (BTR ? 8 : 4);   // LDS reads per k-step
  if (DB) load(0, KB);
#pragma unroll
  for (int ks = KB; ks < KE; ++ks) {
    if (DB) __builtin_amdgcn_sched_barrier(0);
    if (!DB) load(0, ks);
    else if (ks + 1 < KE) load((ks - KB + 1) % NS, ks + 1);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = mma(a[(ks - KB) % NS][i], b[(ks - KB) % NS][j], acc[i][j]);
    if (DB && ks + 1 < KE) {
      // the next step's reads go out between this step's matrix instructions
#pragma unroll
      for (int x = 0; x < NR; ++x) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      if (NR < 16) __builtin_amdgcn_sched_group_barrier(0x008, 16 - NR, 0);
    }
    if (DB) __builtin_amdgcn_sched_barrier(0);
  }
}

// gemm64 over the k-steps of one 64-row half: [0, 2) for hi == 0, else [2, 4)
// (hi is uniform over the wave).
template <uint32_t ABASE, bool ATR, uint32_t BBASE, bool BTR, bool DB = true>
__device__ __forceinline__ void gemm64_half(f32x4 (&acc)[4][4], const Lds& s, const Lane& L, int hi) {
  if (hi) gemm64<ABASE, ATR, BBASE, BTR, DB, 2, 4>(acc, s, L);
  else gemm64<ABASE, ATR, BBASE, BTR, DB, 0, 2>(acc, s, L);
}

template <int M, int N>
__device__ __forceinline__ void zero(f32x4 (&acc)[M][N]) {
#pragma unroll
  for (int i = 0; i < M; ++i)
#pragma unroll
    for (int j = 0; j < N; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// Accumulator values kept packed in bf16 between phases (4 per tile).
struct P4 {
  bf16x4 v[4][4];
  __device__ __forceinline__ void set(int i, int j, float x0, float x1, float x2, float x3) {
    v[i][j][0] = (bf)x0; v[i][j][1] = (bf)x1; v[i][j][2] = (bf)x2; v[i][j][3] = (bf)x3;
  }
  __device__ __forceinline__ void set(int i, int j, const f32x4& a) { set(i, j, a[0], a[1], a[2], a[3]); }
};

// Store the wave's 64x64 block transposed into slot BASE:
// tile[n0 + 16 j + r16][m0 + 16 i + 4 q ..] = X(m0 + 16 i + 4 q .., n0 + 16 j + r16).
template <uint32_t BASE>
__device__ __forceinline__ void put_t(Lds& s, const P4& p, const Lane& L) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<bf16x4*>(lds_m(s) + BASE + L.pt[i] + 4096u * j) = p.v[i][j];
}

// Rows [0, 128) of a 128-wide global matrix (row stride gs elements) in
// registers, one 16-byte piece of row t / 16 + 16 it per thread and it < 8.
// Rows >= len repeat row len - 1 (len >= 1): every factor that multiplies
// such a row in the products is zero (rk, rq, beta, ck and xk of rows past
// the chunk's end), so no select is needed, and none may keep a load waiting.
struct Pieces {
  u32x4 p[8];
  __device__ __forceinline__ void load(const bf* src, uint32_t gs, int len) {
    // an opaque thread index: the addresses are formed here, not hoisted to
    // the kernel's start and kept live (or spilled) until the load
    uint32_t t = threadIdx.x;
    asm volatile("" : "+v"(t));
    const uint32_t c = (t & 15u) * 8u;
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int r = (int)(t >> 4) + 16 * it;
      const uint32_t rr = (uint32_t)min(r, len - 1);
      p[it] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(src) + (rr * gs + c) * 2u);
    }
  }
  // Rows 0..63 from chunk A (la rows at srcA), rows 64..127 from chunk B (lb
  // at srcB), each half clamped to its own last row like `load` (la, lb >= 1).
  __device__ __forceinline__ void load_pair(const bf* srcA, int la, const bf* srcB, int lb,
                                            uint32_t gs) {
    uint32_t t = threadIdx.x;
    asm volatile("" : "+v"(t));
    const uint32_t c = (t & 15u) * 8u;
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int r = (int)(t >> 4) + 16 * (it & 3);   // row within the half
      const uint32_t rr = (uint32_t)min(r, (it < 4 ? la : lb) - 1);
      p[it] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(it < 4 ? srcA : srcB) +
                                              (rr * gs + c) * 2u);
    }
  }
  // sum of squares of piece it, bf16 pairs on the dot-product unit (the
  // pairs are shuffled out of the whole piece: this compiler lowers a bit
  // cast of one 32-bit element to a bf16 pair as element 0)
  __device__ __forceinline__ float sumsq(int it) const {
    const bf16x8 e = __builtin_bit_cast(bf16x8, p[it]);
    float acc = 0.0f;
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(e, e, 0, 1),
                                          __builtin_shufflevector(e, e, 0, 1), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(e, e, 2, 3),
                                          __builtin_shufflevector(e, e, 2, 3), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(e, e, 4, 5),
                                          __builtin_shufflevector(e, e, 4, 5), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(e, e, 6, 7),
                                          __builtin_shufflevector(e, e, 6, 7), acc, false);
    return acc;
  }
  // the pieces as they are, into slot BASE
  template <uint32_t BASE>
  __device__ __forceinline__ void store(Lds& s, const Lane& L) const {
#pragma unroll
    for (int it = 0; it < 8; ++it)
      *reinterpret_cast<u32x4*>(lds_m(s) + BASE + L.stg + 4096u * it) = p[it];
  }
  // piece it times f, stored into slot BASE
  template <uint32_t BASE>
  __device__ __forceinline__ void store_scaled(Lds& s, const Lane& L, int it, float f) const {
    u32x4 raw = p[it];
    bf* e = reinterpret_cast<bf*>(&raw);
#pragma unroll
    for (int x = 0; x < 8; ++x) e[x] = (bf)((float)e[x] * f);
    *reinterpret_cast<u32x4*>(lds_m(s) + BASE + L.stg + 4096u * it) = raw;
  }
  // every piece times the factor of its row, f[row]
  template <uint32_t BASE>
  __device__ __forceinline__ void store_rows(Lds& s, const Lane& L, const float* f) const {
    const uint32_t r0 = threadIdx.x >> 4;
#pragma unroll
    for (int it = 0; it < 8; ++it) store_scaled<BASE>(s, L, it, f[r0 + 16 * it]);
  }
};

// Slot BASE scaled in place: element (r, c) times f[c].  All eight pieces
// are read before the first is written back, so the reads are in flight
// together (one LDS round trip instead of eight).
template <uint32_t BASE>
__device__ __forceinline__ void scale_cols(Lds& s, const Lane& L, const float* f) {
  const uint32_t c0 = (threadIdx.x & 15u) * 8u;
  const f32x4 f0 = *reinterpret_cast<const f32x4*>(f + c0);
  const f32x4 f1 = *reinterpret_cast<const f32x4*>(f + c0 + 4);
  u32x4 raw[8];
#pragma unroll
  for (int it = 0; it < 8; ++it)
    raw[it] = *reinterpret_cast<const u32x4*>(lds_m(s) + BASE + L.stg + 4096u * it);
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    bf* e = reinterpret_cast<bf*>(&raw[it]);
#pragma unroll
    for (int x = 0; x < 4; ++x) e[x] = (bf)((float)e[x] * f0[x]);
#pragma unroll
    for (int x = 0; x < 4; ++x) e[4 + x] = (bf)((float)e[4 + x] * f1[x]);
    *reinterpret_cast<u32x4*>(lds_m(s) + BASE + L.stg + 4096u * it) = raw[it];
  }
}

// Slot BASE scaled in place: element (r, c) times f[r]; reads first, as above.
template <uint32_t BASE>
__device__ __forceinline__ void scale_rows(Lds& s, const Lane& L, const float* f) {
  const uint32_t r0 = threadIdx.x >> 4;
  u32x4 raw[8];
  float fr[8];
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    raw[it] = *reinterpret_cast<const u32x4*>(lds_m(s) + BASE + L.stg + 4096u * it);
    fr[it] = f[r0 + 16 * it];
  }
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    bf* e = reinterpret_cast<bf*>(&raw[it]);
#pragma unroll
    for (int x = 0; x < 8; ++x) e[x] = (bf)((float)e[x] * fr[it]);
    *reinterpret_cast<u32x4*>(lds_m(s) + BASE + L.stg + 4096u * it) = raw[it];
  }
}

// ---------------------------------------------------------------------------
// Triangular inverse (blog post section 5(1)d), blocked: T^T = (I + N)^-1 for
// N = A+^T strictly upper triangular, in place in slot 0 (upper form U); slot
// 1 (zero on entry) receives the lower form U^T block by block, so that a
// finished block can also be read by rows of its transpose.
// ---------------------------------------------------------------------------

// One doubling merge for finished SZ-blocks: for the pair at b0, with
// X = U(b0, b0), Z = U(b0 + SZ, b0 + SZ) and Y the original N block
// (b0, b0 + SZ), the new block U(b0, b0 + SZ) is -X (Y Z):
//   [X^-1 Y'; 0 Z^-1]^-1 = [X, -X Y' Z; 0, Z]  (Y' = N block).
// Step 1 leaves W = Y Z in the scratch as W^T rows; step 2 computes C = X W and
// C^T = W^T X^T from the same fragments and stores -C by rows into slot 0
// and -C^T by rows into slot 1 (the latter not needed after the last level).
template <int SZ>
__device__ __forceinline__ void merge_level(Lds& s, int w, int l) {
  constexpr int side = SZ / 16, per = side * side;
  constexpr int TPW = (128 / (2 * SZ)) * per / 4;   // tiles per wave
  const uint32_t r16 = l & 15, q = l >> 4;
  // k fragment of a 16x16 operand tile at (row R, col K0) of a 128-wide slot,
  // k = K0 + 8 q ..: for SZ = 16 only the first 16 k exist (lanes q >= 2 zero)
  auto frag128 = [&](uint32_t base, uint32_t R, uint32_t K0) -> bf16x8 {
    const uint32_t qq = SZ == 16 ? (q & 1u) : q;
    const bf16x8 f = rd16(s, base + sw(R + r16, K0 + 8u * qq));
    if (SZ == 16 && q >= 2) return bf16x8{};
    return f;
  };
  auto frag64 = [&](uint32_t R, uint32_t K0) -> bf16x8 {
    const uint32_t qq = SZ == 16 ? (q & 1u) : q;
    const bf16x8 f = *reinterpret_cast<const bf16x8*>(lds_c(s) + sw64(R + r16, K0 + 8u * qq));
    if (SZ == 16 && q >= 2) return bf16x8{};
    return f;
  };
  {
    f32x4 acc[TPW];
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const int tt = w + 4 * u;
      const int p = tt / per, ti = (tt % per) / side, tj = tt % side;
      const uint32_t b0 = 2 * SZ * p;
      acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < SZ; k += 32)
        acc[u] = mma(frag128(kT0, b0 + 16 * ti, b0 + SZ + k), frag128(kT1, b0 + SZ + 16 * tj, b0 + SZ + k),
                     acc[u]);
    }
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const int tt = w + 4 * u;
      const int p = tt / per, ti = (tt % per) / side, tj = tt % side;
      // scratch row p SZ + 16 tj + r16 holds column (16 tj + r16) of W
      const uint32_t row = p * SZ + 16 * tj + r16, col = 16 * ti + 4 * q;
      *reinterpret_cast<bf16x4*>(lds_m(s) + sw64(row, col)) =
          bf16x4{(bf)acc[u][0], (bf)acc[u][1], (bf)acc[u][2], (bf)acc[u][3]};
    }
  }
  lds_barrier();
  {
    f32x4 c[TPW], ct[TPW];
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const int tt = w + 4 * u;
      const int p = tt / per, ti = (tt % per) / side, tj = tt % side;
      const uint32_t b0 = 2 * SZ * p;
      c[u] = ct[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < SZ; k += 32) {
        const bf16x8 x = frag128(kT0, b0 + 16 * ti, b0 + k);          // rows of X
        const bf16x8 wt = frag64(p * SZ + 16 * tj, k);                  // rows of W^T
        c[u] = mma(x, wt, c[u]);      // C(16 ti + ., 16 tj + .)
        ct[u] = mma(wt, x, ct[u]);    // C^T(16 tj + ., 16 ti + .)
      }
    }
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const int tt = w + 4 * u;
      const int p = tt / per, ti = (tt % per) / side, tj = tt % side;
      const uint32_t b0 = 2 * SZ * p;
      // U form: row b0 + 16 ti + r16, columns b0 + SZ + 16 tj + 4 q .. of -C
      wr8(s, kT0 + sw(b0 + 16 * ti + r16, b0 + SZ + 16 * tj + 4 * q), -ct[u][0], -ct[u][1],
          -ct[u][2], -ct[u][3]);
      // lower form: row b0 + SZ + 16 tj + r16, columns b0 + 16 ti + 4 q .. of -C^T
      if (SZ < 64)
        wr8(s, kT1 + sw(b0 + SZ + 16 * tj + r16, b0 + 16 * ti + 4 * q), -c[u][0], -c[u][1], -c[u][2],
            -c[u][3]);
    }
  }
  lds_barrier();
}

// BLOCKDIAG: the 64-row halves are independent (a pair of 64-token chunks):
// the last merge would only form the zero block between them, and is left out.
template <bool BLOCKDIAG = false>
__device__ __forceinline__ void invert_unit_upper(Lds& s) {
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  // 16x16 diagonal blocks by back substitution, one column per thread (the
  // 16 threads of a block are lanes of one wave):
  //   x_i = delta_ic - sum_{m > i} N[i][m] x_m,  i = 15 .. 0.
  if (tid < 128) {
    const uint32_t b = tid >> 4, c = tid & 15, b0 = 16 * b;
    // rows are read in groups of four, the next group before the current
    // one is solved, so each group costs one LDS round trip
    u32x4 piece[15][2];
    auto read_rows = [&](int lo, int hi) {
#pragma unroll
      for (int i = lo; i < hi; ++i)
#pragma unroll
        for (int pc = 0; pc < 2; ++pc)
          if (i < 15 && 8 * pc + 7 > i)
            piece[i][pc] = *reinterpret_cast<const u32x4*>(lds_c(s) + kT0 + sw(b0 + i, b0 + 8 * pc));
    };
    float col[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) col[i] = (i == (int)c) ? 1.0f : 0.0f;
    auto solve_rows = [&](int lo, int hi) {   // rows hi - 1 down to lo
#pragma unroll
      for (int i = hi - 1; i >= lo; --i) {
        if (i == 15) continue;
        float acc = 0.0f;
#pragma unroll
        for (int m = i + 1; m < 16; ++m)
          acc += (float)reinterpret_cast<const bf*>(&piece[i][m >> 3])[m & 7] * col[m];
        if (i < (int)c) col[i] = -acc;
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
    // the wave's reads of the block come before its writes
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int i = 0; i < 16; ++i)
      *reinterpret_cast<bf*>(lds_m(s) + kT0 + sw(b0 + i, b0 + c)) = (bf)col[i];
#pragma unroll
    for (int i = 0; i < 16; i += 4)
      wr8(s, kT1 + sw(b0 + c, b0 + i), col[i], col[i + 1], col[i + 2], col[i + 3]);
  }
  lds_barrier();
  merge_level<16>(s, w, l);
  merge_level<32>(s, w, l);
  if (!BLOCKDIAG) merge_level<64>(s, w, l);
}

// Global store of a 64x64 accumulator block, transposed, in one of the bf16
// state pass's workspace orders: element (row n, column m) = sign * acc(m, n),
// n = n0 + 16 j + r16, m = m0 + 16 i + 4 q ..  In every order a lane's values
// of two neighbouring 16-wide tiles form one 16-byte piece, so a lane stores
// 8 pieces per matrix:
//   Frag (Mt, Qp; rows n, k = m): 1 KiB block (n / 16, m / 32); lane
//     (n % 16) + 16 ((m % 16) / 4) holds value m % 4 + 4 ((m % 32) / 16), i.e.
//     lane group q holds k = {4q .. 4q + 3, 16 + 4q .. 16 + 4q + 3} of the
//     32 k of a matrix-core step.  The state pass keeps its copy of S in the
//     same k order (gdr_inter_bf16.hip), so both operands of its products
//     pair the same k.
//   Bm (rows v = n, columns d = m): 4 KiB per 16 rows v, then block
//     (d / 64, (d % 64) / 32); lane (v % 16) + 16 ((d % 16) / 4) holds value
//     d % 4 + 4 ((d % 32) / 16).
//   Ou (rows r = n, columns v = m): 4 KiB per 16 columns v, then block r / 32;
//     lane (r % 16) + 16 ((v % 16) / 4) holds value v % 4 + 4 ((r % 32) / 16).
enum class Lay { Frag, Bm, Ou };
template <Lay LY>
__device__ __forceinline__ void store_block(bf* dst, const f32x4 (&acc)[4][4], int m0, int n0,
                                            float sign) {
  const uint32_t l = threadIdx.x & 63u;
  uint32_t base;
  if (LY == Lay::Frag) base = ((uint32_t)(n0 >> 4) * 4u + (uint32_t)(m0 >> 5)) * 512u + l * 8u;
  else if (LY == Lay::Bm) base = (uint32_t)(n0 >> 4) * 2048u + (uint32_t)(m0 >> 6) * 1024u + l * 8u;
  else base = (uint32_t)(m0 >> 4) * 2048u + (uint32_t)(n0 >> 5) * 512u + l * 8u;
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      // Frag, Bm: column tiles i = 2p, 2p + 1 of row tile j = a;
      // Ou: row tiles j = 2p, 2p + 1 of column tile i = a
      const f32x4& x0 = LY == Lay::Ou ? acc[a][2 * p] : acc[2 * p][a];
      const f32x4& x1 = LY == Lay::Ou ? acc[a][2 * p + 1] : acc[2 * p + 1][a];
      *reinterpret_cast<bf16x8*>(dst + base + (uint32_t)a * 2048u + (uint32_t)p * 512u) =
          bf16x8{(bf)(sign * x0[0]), (bf)(sign * x0[1]), (bf)(sign * x0[2]), (bf)(sign * x0[3]),
                 (bf)(sign * x1[0]), (bf)(sign * x1[1]), (bf)(sign * x1[2]), (bf)(sign * x1[3])};
    }
}

// The Grams of the raw rows and the decay mask on a wave's 64x64 block.
// Tiles strictly below the diagonal need K K^T (g1: k_a . k_c, for A+), tiles
// above it K Q^T (g2: k_a . q_c, for P), diagonal tiles both; rows
// a = m0 + 16 i + 4 q + x, columns c = n0 + 16 j + r16.  WT: 0 = block on the
// diagonal, 1 = block above it (P only), 2 = block below it (N only), 3 = a
// block between the two chunks of a pair (no terms: zeros).
// The barrier between the products and the mask is inside.
template <int WT>
__device__ __forceinline__ void gram_mask(Lds& s, const Lane& L, P4& Pp, int m0, int n0) {
  const uint32_t l = threadIdx.x & 63u, r16 = l & 15u, qd = l >> 4;
  if (WT == 3) {
    lds_barrier();   // the other waves' Grams still read the slots
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        Pp.set(i, jj, 0.f, 0.f, 0.f, 0.f);
        wr8(s, kT0 + L.pt[i] + 4096u * jj, 0.f, 0.f, 0.f, 0.f);
      }
    return;
  }
  f32x4 g1[4][4], g2[4][4];
  zero(g1);
  zero(g2);
  if (WT == 2) {
    gemm64<kT0, false, kT0, false>(g1, s, L);
  } else if (WT == 1) {
    gemm64<kT0, false, kT1, false>(g2, s, L);
  } else {
    bf16x8 a[2][4], bk[2][4], bq[2][4];
    auto load = [&](int set, int ks) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[set][i] = rd16(s, kT0 + L.fa[ks] + 4096u * i);
        bk[set][i] = rd16(s, kT0 + L.fb[ks] + 4096u * i);
        bq[set][i] = rd16(s, kT1 + L.fb[ks] + 4096u * i);
      }
    };
    load(0, 0);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if (ks + 1 < 4) load((ks + 1) & 1, ks + 1);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          if (i >= jj) g1[i][jj] = mma(a[ks & 1][i], bk[ks & 1][jj], g1[i][jj]);
          if (i <= jj) g2[i][jj] = mma(a[ks & 1][i], bq[ks & 1][jj], g2[i][jj]);
        }
    }
  }
  lds_barrier();

  float gcc[4], fc[4];
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const int c = n0 + 16 * jj + (int)r16;
    gcc[jj] = s.gc[c];
    fc[jj] = WT == 2 ? s.rk[c] : (WT == 1 ? s.rq[c] : 0.0f);
  }
  float rkc[4], rqc[4];
  if (WT == 0) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      rkc[jj] = s.rk[n0 + 16 * jj + (int)r16];
      rqc[jj] = s.rq[n0 + 16 * jj + (int)r16];
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int a = m0 + 16 * i + 4 * (int)qd;
    const f32x4 ga = *reinterpret_cast<const f32x4*>(&s.gc[a]);
    const f32x4 fn = *reinterpret_cast<const f32x4*>(&s.brk[a]);   // row factor of N
    const f32x4 fp = *reinterpret_cast<const f32x4*>(&s.rk[a]);    // row factor of P
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      float nv[4], pv[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const float ex = __builtin_amdgcn_exp2f(-fabsf(ga[x] - gcc[jj]));
        if (WT == 2) {
          nv[x] = fn[x] * fc[jj] * ex * g1[i][jj][x];
          pv[x] = 0.0f;
        } else if (WT == 1) {
          nv[x] = 0.0f;
          pv[x] = fp[x] * fc[jj] * ex * g2[i][jj][x];
        } else if (i > jj) {
          nv[x] = fn[x] * rkc[jj] * ex * g1[i][jj][x];
          pv[x] = 0.0f;
        } else if (i < jj) {
          nv[x] = 0.0f;
          pv[x] = fp[x] * rqc[jj] * ex * g2[i][jj][x];
        } else {
          const bool lower = (int)r16 < 4 * (int)qd + x;
          nv[x] = lower ? fn[x] * rkc[jj] * ex * g1[i][jj][x] : 0.0f;
          pv[x] = lower ? 0.0f : fp[x] * rqc[jj] * ex * g2[i][jj][x];
        }
      }
      Pp.set(i, jj, pv[0], pv[1], pv[2], pv[3]);
      wr8(s, kT0 + L.pt[i] + 4096u * jj, nv[0], nv[1], nv[2], nv[3]);
    }
  }
}

// PAIR: 64-token chunks, two per workgroup.  Chunk slots 2u (rows 0..63)
// and 2u + 1 (rows 64..127) of the segment share the unit's 128 rows; their
// gate cumsums restart at row 64, every term between the two chunks is zero
// (the Grams' cross blocks are not formed), so T, R and Z come out block
// diagonal, and the products over token rows take only the k-steps of the
// half they need.  M' and Bm, which sum over a chunk's rows, are formed per
// chunk from its half of the k range.  Each chunk's matrices go to its own
// slot in the workspace (Qp and Ou in rows 0..63, the rows the state pass
// reads for 64-token chunks).
template <bool PAIR>
__global__ __launch_bounds__(256, 2) void intra_bf16_kernel(
    const bf* __restrict__ q, const bf* __restrict__ k, const bf* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, Chunks chunks, int32_t Nqk,
    int32_t Nv, int32_t slot0, int32_t nseg, float scale, int norm, bf* __restrict__ inter,
    float* __restrict__ gam_out) {
  __shared__ Lds s;
  // Workgroup id -> (unit, value head); a unit is one chunk slot, or two
  // (PAIR).  Workgroups go to the 8 XCDs round-robin by id; the G = Nv / Nqk
  // value heads of one (unit, q/k head) read the same k and q rows, so they
  // are given ids with the same id % 8 and share that XCD's L2.  Groups
  // p = unit * Nqk + j are dealt in order; ids past the last group (the grid
  // is padded to whole rounds of 8 G) exit.
  const int units = PAIR ? (nseg + 1) / 2 : nseg;
  const int G = Nv / Nqk;
  const int id = blockIdx.x, xcd = id & 7, r = id >> 3;
  const int p = (r / G) * 8 + xcd;
  if (p >= units * Nqk) return;
  const int unit = p / Nqk, j = p % Nqk, h = j * G + r % G;
  // the unit's chunks: A (rows 0..63, or all 128) and B (rows 64..127, PAIR)
  const int slA = PAIR ? 2 * unit : unit, slB = slA + 1;
  int sa = 0, la = 0, sb = 0, lb = 0;
  const bool hasA = chunks.slot(slot0 + slA, sa, la);
  const bool hasB = PAIR && slB < nseg && chunks.slot(slot0 + slB, sb, lb);
  if (!hasA && !hasB) return;
  if (!hasA) { sa = sb; la = 0; }
  if (!hasB) { sb = sa; lb = 0; }
  // uniform over the workgroup: kept in scalar registers
  sa = __builtin_amdgcn_readfirstlane(sa);
  la = __builtin_amdgcn_readfirstlane(la);
  sb = __builtin_amdgcn_readfirstlane(sb);
  lb = __builtin_amdgcn_readfirstlane(lb);
  // rows past a chunk's end repeat its last row (an absent chunk: the other
  // one's first row); every factor of such a row is zero
  const int lac = max(la, 1), lbc = max(lb, 1);
  const int len = PAIR ? 0 : la;   // the single chunk's length
  const int tid = threadIdx.x, l = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m0 = 64 * (w >> 1), n0 = 64 * (w & 1);
  const uint32_t r16 = l & 15, qd = l >> 4;
  const uint32_t qk_gs = (uint32_t)Nqk * 128u, v_gs = (uint32_t)Nv * 128u;
  const bf* kc = k + ((size_t)sa * Nqk + j) * 128;
  const bf* qc = q + ((size_t)sa * Nqk + j) * 128;
  const bf* vc = v + ((size_t)sa * Nv + h) * 128;
  // chunk B's rows and matrices, formed where they are used
  auto rowsB = [&](const bf* base, uint32_t gs, int hh) { return base + ((size_t)sb * gs / 128 + hh) * 128; };
  bf* dst = inter + ((size_t)slA * Nv + h) * 4 * (size_t)(128 * 128);
  auto dstB = [&]() { return dst + (size_t)Nv * 4 * (128 * 128); };   // slot slA + 1
  // row r of the unit is a real token row
  auto valid = [&](int row) { return PAIR ? (row < 64 ? row < la : row - 64 < lb) : row < len; };
  const Lane L = make_lane(m0, n0);

  // ---- 1. k, q rows; norms; gate cumsum (fp64, waves 0 and 1)
  Pieces kr, qr;
  if (PAIR) {
    kr.load_pair(kc, lac, rowsB(k, qk_gs, j), lbc, qk_gs);
    qr.load_pair(qc, lac, rowsB(q, qk_gs, j), lbc, qk_gs);
  } else {
    kr.load(kc, qk_gs, len);
    qr.load(qc, qk_gs, len);
  }
  double gsum = 0.0;
  float bt = 0.0f;
  if (tid < 128) {
    // row tid; in PAIR mode wave 0 holds chunk A's rows and wave 1 chunk B's
    const int row = PAIR ? l : tid;
    const int st = PAIR && w == 1 ? sb : sa, ln = PAIR ? (w == 1 ? lb : la) : len;
    const bool ok = row < ln;
    const size_t gi = (size_t)(st + min(row, max(ln, 1) - 1)) * Nv + h;
    const float gv = g[gi], bv = beta[gi];
    gsum = ok ? (double)gv : 0.0;
    bt = ok ? bv : 0.0f;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const double y = __shfl_up(gsum, off, 64);
      if (l >= off) gsum += y;
    }
    if (l == 63) s.part[w] = gsum;
  }
  // L2 norms over the 16 lanes holding a row; every lane has all 16 sums
  // of its row group (rows tid / 16 + 16 it of k and of q) and finishes one:
  // lane c takes piece c mod 8 of k (c < 8) or of q
  {
    float ssk[8], ssq[8];
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      ssk[it] = group16_sum(kr.sumsq(it));
      ssq[it] = group16_sum(qr.sumsq(it));
    }
    const int c = tid & 15, it = c & 7;
    const bool isq = c >= 8;
    float ss = isq ? ssq[0] : ssk[0];
#pragma unroll
    for (int x = 1; x < 8; ++x)
      if (it == x) ss = isq ? ssq[x] : ssk[x];
    const int row = (tid >> 4) + 16 * it;
    const float f = (norm ? __builtin_amdgcn_rsqf(ss + 1e-6f) : 1.0f) * (isq ? scale : 1.0f);
    (isq ? s.rq : s.rk)[row] = valid(row) ? f : 0.0f;
  }
  kr.store<kT0>(s, L);
  qr.store<kT1>(s, L);
  lds_barrier();

  // ---- 2. per-row factors (waves 0, 1) and the Grams of the raw rows
  if (tid < 128) {
    // a pair's second chunk starts its own cumsum at row 64
    const double gcd = PAIR ? gsum : gsum + (w == 1 ? s.part[0] : 0.0);
    const double glast = PAIR ? s.part[w] : s.part[0] + s.part[1];
    const float e = __expf((float)gcd), rk = s.rk[tid];
    s.gc[tid] = (float)(gcd * 1.4426950408889634);   // in log2 units, for the mask
    s.beta[tid] = bt;
    s.brk[tid] = bt * rk;
    s.ck[tid] = __expf((float)(glast - gcd)) * rk;
    s.xk[tid] = bt * e * rk;
    s.qs[tid] = e * s.rq[tid];
    if (PAIR) {
      if (l == 0 && (w == 0 ? hasA : hasB))
        gam_out[(size_t)(slot0 + (w == 0 ? slA : slB)) * Nv + h] = __expf((float)glast);
    } else if (tid == 0) {
      gam_out[(size_t)(slot0 + slA) * Nv + h] = __expf((float)glast);
    }
  }
  // ---- 3. Grams and decay mask, one code path per kind of wave block
  P4 Pp;
  if (PAIR && m0 != n0) gram_mask<3>(s, L, Pp, m0, n0);
  else if (m0 > n0) gram_mask<2>(s, L, Pp, m0, n0);
  else if (m0 < n0) gram_mask<1>(s, L, Pp, m0, n0);
  else gram_mask<0>(s, L, Pp, m0, n0);
  // zero slot 1: the lower form of the inverse is built into it
#pragma unroll
  for (int it = 0; it < 8; ++it)
    *reinterpret_cast<u32x4*>(lds_m(s) + kT1 + 16u * (tid + 256 * it)) = u32x4{0u, 0u, 0u, 0u};
  lds_barrier();

  // k rows for phase 7, loaded now so the inverse hides their latency
  Pieces kn;
  if (PAIR) kn.load_pair(kc, lac, rowsB(k, qk_gs, j), lbc, qk_gs);
  else kn.load(kc, qk_gs, len);

  // ---- 4. T^T = (I + N)^-1 in slot 0
  invert_unit_upper<PAIR>(s);

  // ---- 5. P into slot 1 (rows r: P[r][i])
  put_t<kT1>(s, Pp, L);
  lds_barrier();

  // ---- 6. R^T = T^T P^T: acc[j][r] = sum_i T^T[j][i] P[r][i] = R[r][j]
  // (PAIR: zero between the chunks; within one, i runs over its half)
  P4 Rp;
  {
    f32x4 acc[4][4];
    zero(acc);
    if (!PAIR) gemm64<kT0, false, kT1, false>(acc, s, L);
    else if (m0 == n0) gemm64_half<kT0, false, kT1, false>(acc, s, L, m0);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) Rp.set(i, jj, acc[i][jj]);
  }
  lds_barrier();

  // ---- 7. T^T diag(ck) in place; k rows into slot 1
  scale_cols<kT0>(s, L, s.ck);
  kn.store<kT1>(s, L);
  lds_barrier();

  // ---- 8. Z = T^T diag(ck) K:  acc[j][d] = sum_i (T^T ck)[j][i] K[i][d]
  // (PAIR: i over the half of row j)
  P4 Zp;
  {
    f32x4 acc[4][4];
    zero(acc);
    if (!PAIR) gemm64<kT0, false, kT1, true, false>(acc, s, L);
    else gemm64_half<kT0, false, kT1, true, false>(acc, s, L, m0);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) Zp.set(i, jj, acc[i][jj]);
  }
  lds_barrier();

  // raw q[r][d..d+3] in the layout of the Qp product (r = n0 + 16 jj + r16,
  // d = m0 + 16 i + 4 qd), loaded here so phase 9 and the product hide them
  // (rows past the chunk's end repeat its last row; their qs is zero)
  bf16x4 qx[4][4];
  {
    // PAIR: a wave's rows r all lie in one chunk (n0 = 0: A, 64: B)
    const bf* qsrc = PAIR && n0 ? rowsB(q, qk_gs, j) : qc;
    const int rbase = PAIR ? 0 : n0, rlen = PAIR ? (n0 ? lbc : lac) : len;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const uint32_t rr = (uint32_t)min(rbase + 16 * jj + (int)r16, rlen - 1);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        qx[i][jj] = *reinterpret_cast<const bf16x4*>(
            reinterpret_cast<const char*>(qsrc) + (rr * qk_gs + (uint32_t)(m0 + 16 * i) + 4u * qd) * 2u);
    }
  }

  // ---- 9. k rows times xk in slot 1 (both products with K take diag(xk) on
  // that side); R into slot 0
  scale_rows<kT1>(s, L, s.xk);
  put_t<kT0>(s, Rp, L);
  lds_barrier();

  // ---- 10. Qp = diag(qs) q - R (xk K):  acc[d][r] = sum_j (xk K)^T[d][j] R[r][j]
  // (PAIR: j over the half of row r)
  Pieces vn;
  {
    f32x4 acc[4][4];
    zero(acc);
    if (!PAIR) gemm64<kT1, true, kT0, false, false>(acc, s, L);
    else gemm64_half<kT1, true, kT0, false, false>(acc, s, L, n0);
    // q is converted only here: without this the compiler hoists the
    // conversions of the first pieces into phase 9, whose scalings then
    // wait for the loads
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) asm volatile("" : "+v"(qx[i][jj]));
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const float qsr = s.qs[n0 + 16 * jj + r16];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int x = 0; x < 4; ++x) acc[i][jj][x] = qsr * (float)qx[i][jj][x] - acc[i][jj][x];
    }
    // v rows for phase 13 go out between the product and its stores (a
    // wave's memory counter retires in order)
    if (PAIR) vn.load_pair(vc, lac, rowsB(v, v_gs, h), lbc, v_gs);
    else vn.load(vc, v_gs, len);
    // PAIR: rows 64..127 are chunk B's rows 0..63
    if (!PAIR) store_block<Lay::Frag>(dst + 1 * 128 * 128, acc, m0, n0, 1.0f);
    else if (n0 ? hasB : hasA)
      store_block<Lay::Frag>((n0 ? dstB() : dst) + 1 * 128 * 128, acc, m0, 0, 1.0f);
  }
  lds_barrier();

  // ---- 11. Z^T into slot 0: t0[d][j] = Z[j][d]
  put_t<kT0>(s, Zp, L);
  lds_barrier();

  // ---- 12. M' = -(xk K)^T Z:  acc[e][d] = sum_j (xk K)^T[e][j] Z^T[d][j];  Mt[d][e] = -acc
  // (PAIR: one M' per chunk, j over its half)
  if (!PAIR) {
    f32x4 acc[4][4];
    zero(acc);
    gemm64<kT1, true, kT0, false>(acc, s, L);
    store_block<Lay::Frag>(dst + 0 * 128 * 128, acc, m0, n0, -1.0f);
  } else {
    {
      f32x4 acc[4][4];
      zero(acc);
      gemm64<kT1, true, kT0, false, true, 0, 2>(acc, s, L);
      if (hasA) store_block<Lay::Frag>(dst + 0 * 128 * 128, acc, m0, n0, -1.0f);
    }
    {
      f32x4 acc[4][4];
      zero(acc);
      gemm64<kT1, true, kT0, false, true, 2, 4>(acc, s, L);
      if (hasB) store_block<Lay::Frag>(dstB() + 0 * 128 * 128, acc, m0, n0, -1.0f);
    }
  }
  lds_barrier();

  // ---- 13. v rows times beta into slot 1 (Z^T stays in slot 0)
  vn.store_rows<kT1>(s, L, s.beta);
  lds_barrier();

  // ---- 14. Bm = (beta V)^T Z:  acc[d][e] = sum_j Z^T[d][j] (beta V)^T[e][j];  Bm[e][d]
  // (PAIR: one Bm per chunk, j over its half)
  if (!PAIR) {
    f32x4 acc[4][4];
    zero(acc);
    gemm64<kT0, false, kT1, true>(acc, s, L);
    store_block<Lay::Bm>(dst + 2 * 128 * 128, acc, m0, n0, 1.0f);
  } else {
    {
      f32x4 acc[4][4];
      zero(acc);
      gemm64<kT0, false, kT1, true, true, 0, 2>(acc, s, L);
      if (hasA) store_block<Lay::Bm>(dst + 2 * 128 * 128, acc, m0, n0, 1.0f);
    }
    {
      f32x4 acc[4][4];
      zero(acc);
      gemm64<kT0, false, kT1, true, true, 2, 4>(acc, s, L);
      if (hasB) store_block<Lay::Bm>(dstB() + 2 * 128 * 128, acc, m0, n0, 1.0f);
    }
  }
  lds_barrier();

  // ---- 15. R into slot 0
  put_t<kT0>(s, Rp, L);
  lds_barrier();

  // ---- 16. Ou = R (beta V):  acc[e][r] = sum_j (beta V)^T[e][j] R[r][j];  Ou[r][e]
  // (PAIR: j over the half of row r; rows 64..127 are chunk B's rows 0..63)
  {
    f32x4 acc[4][4];
    zero(acc);
    if (!PAIR) gemm64<kT1, true, kT0, false>(acc, s, L);
    else gemm64_half<kT1, true, kT0, false>(acc, s, L, n0);
    if (!PAIR) store_block<Lay::Ou>(dst + 3 * 128 * 128, acc, m0, n0, 1.0f);
    else if (n0 ? hasB : hasA)
      store_block<Lay::Ou>((n0 ? dstB() : dst) + 3 * 128 * 128, acc, m0, 0, 1.0f);
  }
}

}  // namespace

hipError_t launch_intra_bf16(const __bf16* q, const __bf16* k, const __bf16* v, const float* g,
                             const float* beta, Chunks chunks, int32_t Nqk, int32_t Nv,
                             int32_t slot0, int32_t nseg, float scale, int norm, __bf16* inter,
                             float* gam, hipStream_t stream, LaunchEvents ev) {
  // 64-token chunks go two per workgroup
  const bool pair = chunks.L <= 64;
  const unsigned units = pair ? ((unsigned)nseg + 1u) / 2u : (unsigned)nseg;
  const unsigned groups = units * (unsigned)Nqk;
  const unsigned blocks = (groups + 7u) / 8u * 8u * (unsigned)(Nv / Nqk);
  if (pair)
    hipExtLaunchKernelGGL(intra_bf16_kernel<true>, dim3(blocks), dim3(256), 0, stream, ev.start,
                          ev.stop, 0, q, k, v, g, beta, chunks, Nqk, Nv, slot0, nseg, scale, norm,
                          inter, gam);
  else
    hipExtLaunchKernelGGL(intra_bf16_kernel<false>, dim3(blocks), dim3(256), 0, stream, ev.start,
                          ev.stop, 0, q, k, v, g, beta, chunks, Nqk, Nv, slot0, nseg, scale, norm,
                          inter, gam);
  return hipGetLastError();
}

}  // namespace gdr
