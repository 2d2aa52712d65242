// gdr_inter_bf16.hip -- the chunk-serial half of the chunkwise gated delta
// rule for bf16 inputs.
//
// The same pass as the fp32 kernel in gdr_inter.hip (Qwen3-Next blog post,
// section 5(1)f, in the affine form prepared by the intra-chunk kernel): for
// each chunk of a sequence, in order,
//   O      = Qp S^T + Ou                        (the chunk's output rows)
//   S_next = exp(gc_last) S + S M' + Bm         (the state after the chunk)
// with S in R^{Dv x Dk}; a workgroup owns BV = 16 rows of S of one (sequence,
// value head), eight workgroups per (sequence, head) on one XCD, so a single
// sequence of 32 heads fills all 256 compute units.
//
// What bounds a chunk step is the compute unit's vector memory path: per
// chunk a workgroup reads its full Mt and Qp (32 KiB each) and its slices of
// Bm and Ou (4 KiB each), and writes 32 bytes of each of the chunk's 128
// output rows (a partial line each).  Leaving each out in turn (timing only)
// shortens a launch of 32 chunks by: Qp 8 us, the output stores 7 us, half
// of Mt 4.5 us, the Bm slice 2.5 us (of 34).  The operands come in the
// workspace orders the intra-chunk kernel
// writes (store_block in gdr_intra_bf16.hip): Mt and Qp in matrix-core operand
// order with the 32 k of a step permuted per lane group (k = 4q .. 4q + 3,
// 16 + 4q .. 16 + 4q + 3), which the copy of S in LDS repeats, and Bm and Ou
// as 16-byte pieces per lane.  A wave issues its instructions in order, so a wave
// that issues loads stalls while the path is busy.  Here the waves on the
// serial chain never issue one:
//   waves 0, 1 (state):   (S M')^T for 64 key rows each, and the update of S
//                         they keep in fp32 registers; operands from LDS only;
//   waves 2-5 (output):   (Qp S^T) for 32 chunk rows each, + Ou, the output
//                         stores; Qp and Ou prefetched two chunks ahead into a
//                         ring of register sets;
//   waves 6, 7 (loaders): copy each chunk's Mt and the workgroup's slice of
//                         Bm into a four-deep LDS ring, three chunks ahead,
//                         with direct global-to-LDS loads, then wait for the
//                         chunk the next step needs.
// One barrier per chunk step hands over the ring slot and the bf16 copy of S
// (double-buffered).  The ring takes 144 KiB of the 160 KiB of LDS.
#include "gdr_device.h"
#include "gdr_internal.h"
#include "gdr_kernels.h"

namespace gdr {
namespace {

typedef __bf16 bf;
constexpr int kBV = 16;                       // state rows per workgroup
constexpr int kMtBytes = 128 * 128 * 2;       // one chunk's Mt (32 KiB)
constexpr int kBmBytes = kBV * 128 * 2;       // the workgroup's Bm slice (4 KiB)
constexpr int kRing = 4;
constexpr int kDmaPerChunk = 16 + 2;          // 1 KiB pieces per loader wave per chunk
// the loaders' waits count the pieces of the two chunks issued after the one
// they wait for
static_assert(2 * kDmaPerChunk == 36, "s_waitcnt vmcnt(36) below");

struct InterLds {
  char mt[kRing][kMtBytes];   // Mt of chunks c .. c + 3 (workspace fragment order)
  char bm[kRing][kBmBytes];   // the workgroup's Bm blocks (workspace order)
  bf s[2][kBV * 128];         // bf16 copy of the workgroup's rows of S, swizzled
  int2 tab[kMaxSegSlots];     // {first token, length} of the segment's chunks
  float gam[kMaxSegSlots];    // exp(gc_last) of the segment's chunks
};

__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// One 16-byte piece per lane, global to LDS: the 64 lanes of the wave fill
// the 1 KiB at dst (lane l at dst + 16 l).
__device__ __forceinline__ void dma16(const char* src_wave, char* dst_wave, int lane) {
  __builtin_amdgcn_global_load_lds(src_wave + 16 * lane,
                                   (__attribute__((address_space(3))) void*)dst_wave, 16, 0, 0);
}

__global__ __launch_bounds__(512, 1) void inter_bf16_kernel(
    const bf* __restrict__ inter, Chunks chunks, const float* __restrict__ gam,
    const float* state_in, float* carry, float* state_out, int32_t Nv, int32_t slot0,
    int32_t nseg, bf* __restrict__ out, bf* __restrict__ discard) {
  constexpr int VB = 128 / kBV;
  __shared__ InterLds s;

  // blockIdx.x -> (value head h, row block vb), blockIdx.y -> the sequence b
  // of the y-th run of slots in the segment
  const int x = blockIdx.x;
  int h, vb;
  if ((Nv & 7) == 0) {
    // the VB row blocks of one (b, h) read the same Mt and Qp: deal them to
    // the same XCD (workgroups go to the 8 XCDs round-robin in id order, and
    // a row of the grid is Nv VB workgroups, a multiple of 8)
    h = (x & 7) + 8 * (x / (8 * VB));
    vb = (x >> 3) % VB;
  } else {
    h = x / VB;
    vb = x % VB;
  }
  int b;
  if (!chunks.run_sequence(slot0, nseg, blockIdx.y, b)) return;
  const int bh = b * Nv + h;
  const int tid = threadIdx.x, l = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int v0 = kBV * vb;
  const size_t sb = (size_t)bh * 128 * 128;
  int c0, c1;
  chunks.seq_slots(b, c0, c1);
  const int cb = max(c0, slot0), ce = min(c1, slot0 + nseg);
  if (cb >= ce) return;
  const float* src = (cb == c0) ? state_in : carry;
  float* dstS = (ce == c1) ? state_out : carry;
  const size_t mstride = (size_t)Nv * 4 * 128 * 128;
  // matrices of (slot c, head h): Mt, Qp, Bm, Ou
  const bf* mats0 = inter + (size_t)h * 4 * 128 * 128 - (size_t)slot0 * mstride;
  auto mats = [&](int c) { return mats0 + (size_t)c * mstride; };

  for (int idx = tid; idx < ce - cb; idx += 512) {
    int st, ln;
    chunks.slot(cb + idx, st, ln);
    s.tab[idx] = make_int2(st, ln);
    s.gam[idx] = gam[(size_t)(cb + idx) * Nv + h];
  }

  const int r16 = l & 15, q4 = l >> 4;

  if (w >= 6) {
    // ---------------- loaders: Mt blocks 16 lw .. 16 lw + 15 and Bm blocks
    // 2 lw, 2 lw + 1 of each chunk, three chunks ahead
    const int lw = w - 6;
    auto issue = [&](int c, int slot) {
      const char* m = reinterpret_cast<const char*>(mats(c));
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const int bi = 16 * lw + k;
        dma16(m + bi * 1024, s.mt[slot] + bi * 1024, l);
      }
      // the workgroup's 16 rows of Bm: one 4 KiB run
      const char* bmv = reinterpret_cast<const char*>(mats(c) + 2 * 128 * 128) + vb * kBmBytes;
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int bj = 2 * lw + k;
        dma16(bmv + bj * 1024, s.bm[slot] + bj * 1024, l);
      }
    };
    issue(cb, 0);
    issue(min(cb + 1, ce - 1), 1);
    issue(min(cb + 2, ce - 1), 2);
    asm volatile("s_waitcnt vmcnt(36)" ::: "memory");   // chunk cb in LDS
    lds_barrier();                                         // tables, ring slot 0, S(cb)
    int slot = 3;
    for (int c = cb; c < ce; ++c) {
      // ring slot (c + 3) % 4 was read in step c - 1, which ended at the
      // last barrier; past the end the last chunk is loaded again, so every
      // step issues the same loads and the wait below stays exact
      issue(min(c + 3, ce - 1), slot);
      slot = slot == kRing - 1 ? 0 : slot + 1;
      asm volatile("s_waitcnt vmcnt(36)" ::: "memory");   // chunk c + 1 in LDS
      lds_barrier();
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    return;
  }

  if (w < 2) {
    // ---------------- state waves: rows v0 .. v0 + 15 of S, key rows
    // rb .. rb + 63 of the product (S M')^T
    const int rb = 64 * w;
    f32x4 st[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      st[i] = zero4();
      if (src)
        st[i] = *reinterpret_cast<const f32x4*>(src + sb + (size_t)(v0 + r16) * 128 + rb + 16 * i +
                                                4 * q4);
    }
    // S's columns in the k order of the workspace's Mt and Qp (see the
    // header): column rb + 16 i + 4 q4 + x goes to 16-byte chunk
    // 4 ((rb + 16 i) / 32) + q4 of the row, half i % 2
    auto put_s = [&](int buf) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        bf16x4 v;
        v[0] = (bf)st[i][0]; v[1] = (bf)st[i][1]; v[2] = (bf)st[i][2]; v[3] = (bf)st[i][3];
        const int col = (4 * ((rb >> 5) + (i >> 1)) + q4) * 8 + 4 * (i & 1);
        *reinterpret_cast<bf16x4*>(s.s[buf] + Sw<bf>::at(r16, col)) = v;
      }
    };
    put_s(0);
    lds_barrier();
    int slot = 0, buf = 0;
    for (int c = cb; c < ce; ++c) {
      const float gC = s.gam[c - cb];
      f32x4 acc[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = zero4();
      const char* mt = s.mt[slot];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 s0 = sw_frag<bf>(s.s[buf], r16, ks * 32 + 8 * q4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          // block (key row block rb / 16 + i, k-step ks) of Mt: lane l's 8 values
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(
              mt + (((rb >> 4) + i) * 4 + ks) * 1024 + l * 16);
          acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, s0, acc[i], 0, 0, 0);
        }
      }
      // S = exp(gc_last) S + S M' + Bm; this wave's Bm blocks are (d / 64 = w,
      // pair p): lane l's 8 values are tiles i = 2p and 2p + 1
      const char* bmw = s.bm[slot] + w * 2048;
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const bf16x8 x = *reinterpret_cast<const bf16x8*>(bmw + p * 1024 + l * 16);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          st[2 * p][e] = gC * st[2 * p][e] + acc[2 * p][e] + (float)x[e];
          st[2 * p + 1][e] = gC * st[2 * p + 1][e] + acc[2 * p + 1][e] + (float)x[4 + e];
        }
      }
      buf ^= 1;
      put_s(buf);
      slot = slot == kRing - 1 ? 0 : slot + 1;
      lds_barrier();
    }
    if (dstS) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<f32x4*>(dstS + sb + (size_t)(v0 + r16) * 128 + rb + 16 * i + 4 * q4) = st[i];
    }
    return;
  }

  // ---------------- output waves: chunk rows rr0 .. rr0 + 31, the 16 state rows
  const int ow = w - 2, rr0 = 32 * ow;
  // with 64-token chunks no chunk has rows past 63: the waves of rows 64 ..
  // 127 have nothing to load or store (a wave that has ended no longer
  // counts at the barriers)
  if (rr0 >= chunks.L) return;
  struct Ops {
    bf16x8 a[2][4];     // rows rr0 + 16 i of Qp, k-step ks
    bf16x8 x;           // Ou[rr0 + 16 i + r16][v0 + 4 q ..], i = 0 (first 4), 1
  };
  auto load_ops = [&](Ops& o, int c) {
    const bf* m = mats(c);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        o.a[i][ks] = *reinterpret_cast<const bf16x8*>(
            m + 128 * 128 + ((((rr0 >> 4) + i) * 4 + ks) * 512) + l * 8);
    // Ou: the workgroup's 16 columns, block rr0 / 32, 8 values per lane
    o.x = *reinterpret_cast<const bf16x8*>(m + 3 * 128 * 128 + vb * 2048 + ow * 512 + l * 8);
  };
  Ops ops[3];
  load_ops(ops[0], cb);
  load_ops(ops[1], min(cb + 1, ce - 1));
  lds_barrier();
  int buf = 0;
  auto step = [&](Ops& o, Ops& next, int c) {
    // the chunk two ahead (past the end, the last chunk again)
    load_ops(next, min(c + 2, ce - 1));
    const int2 e = s.tab[c - cb];
    f32x4 acc[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) acc[i] = zero4();
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8 s0 = sw_frag<bf>(s.s[buf], r16, ks * 32 + 8 * q4);
#pragma unroll
      for (int i = 0; i < 2; ++i)
        acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(s0, o.a[i][ks], acc[i], 0, 0, 0);
    }
    // acc[i] = (Qp S^T)[r][v .. v + 3], r = rr0 + 16 i + r16, v = v0 + 4 q4.
    // One 16-byte store per lane: a swap between neighbouring 16-lane rows
    // (q4 = 2p, 2p + 1) gives the even row the 8 values of r = rr0 + r16 and
    // the odd row those of r = rr0 + 16 + r16, columns v0 + 8 p ..  Rows past
    // the chunk's end go to the discard line (the store count stays fixed, so
    // the memory waits of later steps stay exact).
    {
      bf16x4 va, vb;
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        va[x] = (bf)(acc[0][x] + (float)o.x[x]);
        vb[x] = (bf)(acc[1][x] + (float)o.x[4 + x]);
      }
      const u32x2 a2 = __builtin_bit_cast(u32x2, va), b2 = __builtin_bit_cast(u32x2, vb);
      const auto s0 = __builtin_amdgcn_permlane16_swap(a2[0], b2[0], false, false);
      const auto s1 = __builtin_amdgcn_permlane16_swap(a2[1], b2[1], false, false);
      const int odd = q4 & 1;
      const int r = rr0 + 16 * odd + r16;
      bf* orow = r < e.y ? out + ((size_t)(e.x + r) * Nv + h) * 128 + v0 : discard;
      *reinterpret_cast<u32x4*>(orow + 4 * (q4 - odd)) = u32x4{s0[0], s1[0], s0[1], s1[1]};
    }
    buf ^= 1;
    lds_barrier();
  };
  int c = cb;
#pragma unroll 1
  for (; c + 3 <= ce; c += 3) {
    step(ops[0], ops[2], c);
    step(ops[1], ops[0], c + 1);
    step(ops[2], ops[1], c + 2);
  }
  if (c < ce) step(ops[0], ops[2], c);
  if (c + 1 < ce) step(ops[1], ops[0], c + 1);
}

}  // namespace

void launch_inter_bf16(const __bf16* inter, Chunks chunks, const float* gam, const float* state_in,
                       float* carry, float* state_out, int32_t N, int32_t Nv, int32_t slot0,
                       int32_t nseg, __bf16* out, __bf16* discard,
                       hipStream_t stream, LaunchEvents ev) {
  const unsigned runs = chunks.table ? (unsigned)(N < nseg ? N : nseg) : 1u;
  hipExtLaunchKernelGGL(inter_bf16_kernel, dim3((unsigned)Nv * (unsigned)(128 / kBV), runs),
                        dim3(512), 0, stream, ev.start, ev.stop, 0, inter, chunks, gam, state_in,
                        carry, state_out, Nv, slot0, nseg, out, discard);
}

}  // namespace gdr
