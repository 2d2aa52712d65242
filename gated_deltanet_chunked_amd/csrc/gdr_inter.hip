// gdr_inter.hip -- the chunk-serial half of the chunkwise gated delta rule.
//
// The state pass of the Qwen3-Next blog post, section 5(1)f, in the affine
// form prepared by gdr_intra.hip: for each chunk of a sequence, in order,
//   O      = Qp S^T + Ou                        (the chunk's output rows)
//   S_next = exp(gc_last) S + S M' + Bm         (the state after the chunk)
// with S in R^{Dv x Dk} (row = value index, as in the Ascend operator page's
// state_new [Dv, Dk]).  Rows of S never mix (every term acts on each row of
// S alone), so a workgroup owns BV = 32 rows of S of one (sequence, value
// head): 4 workgroups per (sequence, head), placed on one XCD so they share
// its L2.
//
// Per chunk the workgroup computes two products on the matrix cores, both
// reading S (bf16 copy of the fp32 state, exchanged once through LDS) by rows:
//   waves 0, 1 (state):  C[d][v] = sum_e Mt[d][e] S[v][e] = (S M')[v][d],
//                        64 key rows d each; they keep S^T in fp32 registers
//                        and apply S = exp(gc_last) S + S M' + Bm;
//   waves 2, 3 (output): C[v][r] = sum_d S[v][d] Qp[r][d] = (Qp S^T)[r][v],
//                        64 chunk rows r each; out[r][v..v+3] = C + Ou.
// The per-chunk operands (rows of Mt or Qp, entries of Bm or Ou, the chunk's
// decay and table entry) do not depend on S, so each lane loads them DEPTH
// chunks ahead into a ring of register sets.  Chunk boundaries restart at
// sequence starts, so a varlen boundary inside a 128-token grid needs no
// special case: a short last chunk only writes its first len output rows.
#include <type_traits>

#include "gdr_device.h"
#include "gdr_internal.h"
#include "gdr_kernels.h"

namespace gdr {

constexpr int kBV = 32;   // state rows (value indices) per workgroup

// Four consecutive elements of T as fp32.
template <typename T> struct Quad;
template <> struct Quad<__bf16> {
  bf16x4 v;
  __device__ __forceinline__ void load(const __bf16* p) { v = *reinterpret_cast<const bf16x4*>(p); }
  __device__ __forceinline__ float operator[](int x) const { return (float)v[x]; }
};
template <> struct Quad<float> {
  f32x4 v;
  __device__ __forceinline__ void load(const float* p) { v = *reinterpret_cast<const f32x4*>(p); }
  __device__ __forceinline__ float operator[](int x) const { return v[x]; }
};

template <typename T>
__device__ __forceinline__ void put4(T* p, float x0, float x1, float x2, float x3);
template <>
__device__ __forceinline__ void put4<float>(float* p, float x0, float x1, float x2, float x3) {
  *reinterpret_cast<float4*>(p) = make_float4(x0, x1, x2, x3);
}
template <>
__device__ __forceinline__ void put4<__bf16>(__bf16* p, float x0, float x1, float x2, float x3) {
  bf16x4 v;
  v[0] = (__bf16)x0; v[1] = (__bf16)x1; v[2] = (__bf16)x2; v[3] = (__bf16)x3;
  *reinterpret_cast<bf16x4*>(p) = v;
}

// Prefetch depth per operand type: how many chunks ahead a lane's operands
// are loaded (fp32 fragments take twice the registers).
template <typename T> struct Depth { static constexpr int value = 2; };
template <> struct Depth<float> { static constexpr int value = 1; };

// One chunk's operands held by one lane.
template <typename T>
struct ChunkOps {
  static constexpr int KSTEPS = kD / Mma<T>::K;
  typename Mma<T>::frag a[4][KSTEPS];   // rows of Mt (state waves) or Qp (output waves)
  Quad<T> x[4][2];                      // Bm (state waves) or Ou (output waves) entries
  float gC;                             // exp(gc_last) of the chunk
  int start, len;                       // the chunk's tokens
  uint32_t warm[2];                     // L2 warming loads in flight (values unused)
};

// Chunks ahead whose operands are pulled into L2 by touch loads: one 4-byte
// load per 128-byte line, so a warming instruction covers 8 KiB where an
// operand load covers 1 KiB, and the operand loads later hit in L2.
constexpr int kWarmAhead = 5;

template <typename T>
__global__ __launch_bounds__(256, 1) void inter_kernel(
    const T* __restrict__ inter, Chunks chunks, const float* __restrict__ gam, const float* state_in, float* carry, float* state_out,
    int32_t Nv, int32_t slot0, int32_t nseg, T* __restrict__ out, T* __restrict__ discard) {
  constexpr int KSTEPS = ChunkOps<T>::KSTEPS;
  constexpr int DEPTH = Depth<T>::value;
  constexpr int NSET = DEPTH + 1;
  constexpr int VB = kD / kBV;   // workgroups per (sequence, head)
  __shared__ T sS[2][kBV * kD];  // bf16/fp32 copy of S rows [v][k], swizzled
  // the segment's chunk table and decays, staged once: a scalar load in the
  // chunk loop would make every LDS wait also wait for global memory
  __shared__ int2 sTab[kMaxSegSlots];
  __shared__ float sGam[kMaxSegSlots];

  // blockIdx.x -> (head h, row block vb), blockIdx.y -> the sequence b of the
  // y-th run of slots in the segment.  Blocks are dealt to the 8 XCDs
  // round-robin in id order; the VB row blocks of one (b, h) read the same
  // Mt and Qp, so when possible they land on the same XCD.
  const int x = blockIdx.x;
  int h, vb;
  if ((Nv & 7) == 0) {
    h = (x & 7) + 8 * (x / (8 * VB));
    vb = (x >> 3) % VB;
  } else {
    h = x / VB;
    vb = x % VB;
  }
  int b;
  if (!chunks.run_sequence(slot0, nseg, blockIdx.y, b)) return;
  const int bh = b * Nv + h;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const bool state_wave = w < 2;
  const int rb = 64 * (w & 1);               // first row (d or r) of this wave's block
  const int v0 = kBV * vb;                   // first state row of the workgroup
  const size_t sb = (size_t)bh * kD * kD;    // this (b, h)'s state
  int c0, c1;
  chunks.seq_slots(b, c0, c1);
  const int cb = max(c0, slot0), ce = min(c1, slot0 + nseg);
  if (cb >= ce) return;
  const float* src = (cb == c0) ? state_in : carry;
  float* dstS = (ce == c1) ? state_out : carry;
  const size_t mstride = (size_t)Nv * 4 * (size_t)(kD * kD);
  // matrices of (slot c, head h): Mt, Qp, Bm, Ou
  const T* mats0 = inter + (size_t)h * 4 * (size_t)(kD * kD) - (size_t)slot0 * mstride;

  const int r16 = l & 15, q4 = l >> 4, kq = q4 * Mma<T>::E;
  for (int idx = tid; idx < ce - cb; idx += 256) {
    int st, ln;
    chunks.slot(cb + idx, st, ln);
    sTab[idx] = make_int2(st, ln);
    sGam[idx] = gam[(size_t)(cb + idx) * Nv + h];
  }
  __syncthreads();

  // Every operand load below is one contiguous block per wave: the workspace
  // holds Mt and Qp in matrix-core operand order (frag_off) and Bm and Ou in
  // this pass's accumulator order (bm_off, ou_off).
  auto load_ops = [&](ChunkOps<T>& o, int c) {
    const T* m = mats0 + (size_t)c * mstride;
    // rows rb + 16 i + r16 of Mt (state waves) or Qp (output waves)
    const T* A = m + (state_wave ? 0 : kD * kD) + (size_t)(rb >> 4) * KSTEPS * 64 * Mma<T>::E +
                 l * Mma<T>::E;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks)
        o.a[i][ks] = Mma<T>::load_contig(A + (size_t)(i * KSTEPS + ks) * 64 * Mma<T>::E);
    // state waves: Bm[v][d..d+3], v = v0 + 16 t + r16, d = rb + 16 i + 4 q4;
    // output waves: Ou[r][v..v+3], r = rb + 16 i + r16, v = v0 + 16 t + 4 q4
    const T* X = m + (state_wave ? 2 : 3) * kD * kD + l * 4;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int t = 0; t < 2; ++t) o.x[i][t].load(X + pass_blk(vb, rb >> 6, i, t));
    o.gC = sGam[c - cb];
    const int2 e = sTab[c - cb];
    o.start = e.x;
    o.len = e.y;
  };

  // State waves: S^T tiles st[i][t] hold S[v][d..d+3] for d = rb + 16 i + 4 q4 + x,
  // v = v0 + 16 t + r16 (the layout of the state product's accumulators).
  f32x4 st[4][2];
  if (state_wave) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        st[i][t] = zero4();
        if (src)
          st[i][t] = *reinterpret_cast<const f32x4*>(
              src + sb + (size_t)(v0 + 16 * t + r16) * kD + rb + 16 * i + 4 * q4);
      }
  }

  // Lines this workgroup warms per chunk: its quarter of Mt and of Qp (the
  // other row blocks of the (b, h) warm the rest, through the shared L2) and
  // its own quarters of Bm and Ou.  Each quarter is a contiguous range.
  constexpr int QB = kD * kD * (int)sizeof(T) / 4;   // bytes per quarter matrix
  constexpr int NWARM = 4 * QB / 128;                // lines per chunk
  auto warm = [&](ChunkOps<T>& o, int c) {
    const char* m = reinterpret_cast<const char*>(mats0 + (size_t)c * mstride);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      int L = tid + 256 * u;
      if (L >= NWARM) L -= NWARM;                // duplicates are harmless
      const int mat = L / (QB / 128), k = L % (QB / 128);
      o.warm[u] = *reinterpret_cast<const uint32_t*>(m + (size_t)mat * 4 * QB + (size_t)vb * QB + k * 128);
    }
  };
  uint32_t sink = 0;

  ChunkOps<T> ops[NSET];
#pragma unroll
  for (int k = 0; k < NSET; ++k) ops[k].warm[0] = ops[k].warm[1] = 0u;
#pragma unroll
  for (int k = 0; k < DEPTH; ++k) load_ops(ops[k], min(cb + k, ce - 1));

  // One chunk of the pass for one wave role (STATE: state product and update;
  // else output product and stores).  The two roles run as separate loops so
  // each is straight-line code and the memory waits are counted exactly.
  int buf = 0;
  auto step = [&](auto role, ChunkOps<T>& o, ChunkOps<T>& next, int c) {
    constexpr bool STATE = decltype(role)::value;
    T* sbuf = sS[buf];
    if (STATE) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int t = 0; t < 2; ++t)
          put4<T>(sbuf + Sw<T>::at(16 * t + r16, rb + 16 * i + 4 * q4), st[i][t][0], st[i][t][1],
                  st[i][t][2], st[i][t][3]);
    }
    __syncthreads();
    // Output waves queue the next operands' loads before their products: the
    // workgroup's loads go through one vector-memory path, and starting them
    // here keeps it busy while the state waves' products (the serial chain)
    // run.  State waves issue theirs after their products.
    if (!STATE) {
      load_ops(next, min(c + DEPTH, ce - 1));
      sink ^= o.warm[0] ^ o.warm[1];
      warm(o, min(c + kWarmAhead, ce - 1));
    }
    f32x4 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i][0] = acc[i][1] = zero4();
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      const auto s0 = sw_frag<T>(sbuf, r16, ks * Mma<T>::K + kq);
      const auto s1 = sw_frag<T>(sbuf, 16 + r16, ks * Mma<T>::K + kq);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (STATE) {
          acc[i][0] = Mma<T>::mma(o.a[i][ks], s0, acc[i][0]);
          acc[i][1] = Mma<T>::mma(o.a[i][ks], s1, acc[i][1]);
        } else {
          acc[i][0] = Mma<T>::mma(s0, o.a[i][ks], acc[i][0]);
          acc[i][1] = Mma<T>::mma(s1, o.a[i][ks], acc[i][1]);
        }
      }
    }
    // next operands: chunk c + DEPTH (clamped: past the end it reloads the
    // last chunk, which keeps the loop free of branches)
    if (STATE) {
      load_ops(next, min(c + DEPTH, ce - 1));
      // the warming loads held in this set were issued NSET chunks ago
      sink ^= o.warm[0] ^ o.warm[1];
      warm(o, min(c + kWarmAhead, ce - 1));
    }
    if (STATE) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int x = 0; x < 4; ++x)
            st[i][t][x] = o.gC * st[i][t][x] + acc[i][t][x] + o.x[i][t][x];
    } else {
      // acc[i][t] holds O[r][v..v+3] - Ou for r = rb + 16 i + r16, v = 16 t + 4 q4
#pragma unroll
      // rows past the chunk's end are written to the discard line instead, so
      // every step issues the same stores and the memory waits of later
      // steps never cover them
      for (int i = 0; i < 4; ++i) {
        const int r = rb + 16 * i + r16;
        T* orow = r < o.len ? out + ((size_t)(o.start + r) * Nv + h) * kD + v0 : discard;
#pragma unroll
        for (int t = 0; t < 2; ++t)
          put4<T>(orow + 16 * t + 4 * q4, acc[i][t][0] + o.x[i][t][0], acc[i][t][1] + o.x[i][t][1],
                  acc[i][t][2] + o.x[i][t][2], acc[i][t][3] + o.x[i][t][3]);
      }
    }
    buf ^= 1;
  };

  // The ring of NSET register sets, unrolled so every set index is static;
  // whole groups of NSET chunks first, then the remainder.
  auto chunk_loop = [&](auto role) {
    int c = cb;
#pragma unroll 1
    for (; c + NSET <= ce; c += NSET) {
#pragma unroll
      for (int k = 0; k < NSET; ++k) step(role, ops[k], ops[(k + DEPTH) % NSET], c + k);
    }
#pragma unroll
    for (int k = 0; k < NSET - 1; ++k)
      if (c + k < ce) step(role, ops[k], ops[(k + DEPTH) % NSET], c + k);
  };
  if (state_wave) chunk_loop(std::true_type{});
  else chunk_loop(std::false_type{});

  asm volatile("" ::"v"(sink));   // keeps the warming loads alive
  if (state_wave && dstS) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int t = 0; t < 2; ++t)
        *reinterpret_cast<f32x4*>(dstS + sb + (size_t)(v0 + 16 * t + r16) * kD + rb + 16 * i +
                                  4 * q4) = st[i][t];
  }
}

template <typename T>
void launch_inter(const T* inter, Chunks chunks, const float* gam, const float* state_in,
                  float* carry, float* state_out, int32_t N, int32_t Nv, int32_t slot0,
                  int32_t nseg, T* out, T* discard, hipStream_t stream, LaunchEvents ev) {
  if constexpr (sizeof(T) == 2) {
    // bf16 has its own kernel (gdr_inter_bf16.hip)
    launch_inter_bf16(inter, chunks, gam, state_in, carry, state_out, N, Nv, slot0, nseg, out,
                      discard, stream, ev);
  } else {
    const unsigned runs = chunks.table ? (unsigned)(N < nseg ? N : nseg) : 1u;
    hipExtLaunchKernelGGL(inter_kernel<T>, dim3((unsigned)Nv * (unsigned)(kD / kBV), runs),
                          dim3(256), 0, stream, ev.start, ev.stop, 0, inter, chunks, gam, state_in,
                          carry, state_out, Nv, slot0, nseg, out, discard);
  }
}

template void launch_inter<float>(const float*, Chunks, const float*, const float*, float*, float*,
                                  int32_t, int32_t, int32_t, int32_t, float*, float*, hipStream_t,
                                  LaunchEvents);
template void launch_inter<__bf16>(const __bf16*, Chunks, const float*, const float*, float*,
                                   float*, int32_t, int32_t, int32_t, int32_t, __bf16*, __bf16*,
                                   hipStream_t, LaunchEvents);

}  // namespace gdr
