// gdr_validate.cpp -- argument checks and workspace layout of libgdr.
// Plain C++: no HIP calls, so every error path runs without a GPU.
#include <stdint.h>

#include <cmath>

#include "gdr_internal.h"

namespace gdr {
namespace {

constexpr uint32_t kKnownFlags = GDR_FLAG_QK_L2NORM | GDR_FLAG_CHUNK64;

int64_t align256(int64_t x) { return (x + 255) & ~int64_t(255); }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// [p, p + n) and [q, q + m) overlap (both non-empty).
bool overlap(const void* p, int64_t n, const void* q, int64_t m) {
  if (!p || !q || n <= 0 || m <= 0) return false;
  const uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(q);
  return a < b + static_cast<uintptr_t>(m) && b < a + static_cast<uintptr_t>(n);
}

gdr_status common_sizes(int32_t Nqk, int32_t Nv, int32_t D, gdr_dtype dtype, uint32_t flags) {
  if (D != 128 || Nv > kMaxNv) return GDR_ERR_UNSUPPORTED;
  if (dtype != GDR_F32 && dtype != GDR_BF16) return GDR_ERR_UNSUPPORTED;
  if (flags & ~kKnownFlags) return GDR_ERR_UNSUPPORTED;
  if (Nqk <= 0 || Nv <= 0 || Nv % Nqk != 0) return GDR_ERR_INVALID_ARGUMENT;
  return GDR_OK;
}

}  // namespace

Workspace plan_workspace(int64_t T, int64_t N, int64_t Nqk, int64_t Nv, gdr_dtype dtype,
                         int64_t budget, int64_t L) {
  Workspace w{};
  const int64_t es = static_cast<int64_t>(dtype_size(dtype));
  const int64_t per_slot = Nv * kInterMats * kMatElems * es;
  w.nslots = max_slots(T, N, L);
  // everything but the segment's matrices
  const int64_t fixed = align256(w.nslots * 4 * 4) + align256((N + 1) * 4) + align256(N * 4) +
                        align256(w.nslots * Nv * 4) + align256(N * Nv * kMatElems * 4) + 256;
  if (budget > 0) {
    // the largest segment that fits the budget, then the slots split evenly
    int64_t cap = (budget - fixed) / per_slot;
    if (cap > kMaxSegSlots) cap = kMaxSegSlots;
    if (cap < 1) {
      w.total = -1;   // does not fit
      return w;
    }
    // at least one segment, also for no slot at all (then of no slot)
    const int64_t nsegs = w.nslots > cap ? (w.nslots + cap - 1) / cap : 1;
    w.seg_slots = (w.nslots + nsegs - 1) / nsegs;
  } else {
    w.seg_slots = segment_slots(w.nslots, Nv, es);
  }
  int64_t off = 0;
  w.table = off; off = align256(off + w.nslots * 4 * 4);
  w.choff = off; off = align256(off + (N + 1) * 4);
  w.nonempty = off; off = align256(off + N * 4);
  w.gam = off; off = align256(off + w.nslots * Nv * 4);
  w.inter = off;
  off = align256(off + w.seg_slots * per_slot);
  w.carry = off; off = align256(off + N * Nv * kMatElems * 4);
  w.discard = off; off = align256(off + 256);
  w.total = off;
  return w;
}

gdr_status validate_chunk(const ChunkArgs& a) {
  gdr_status s = common_sizes(a.Nqk, a.Nv, a.D, a.dtype, a.flags);
  if (s != GDR_OK) return s;
  if (a.N < 1 || a.T < 0) return GDR_ERR_INVALID_ARGUMENT;
  // every element offset must fit comfortably in 63 bits; the kernels also
  // index tokens with 32-bit integers
  if (static_cast<int64_t>(a.T) * a.Nv > (int64_t(1) << 40)) return GDR_ERR_INVALID_ARGUMENT;
  if (a.no_workspace && static_cast<int64_t>(a.N) * a.Nv >= (int64_t(1) << 24))
    return GDR_ERR_INVALID_ARGUMENT;   // one workgroup of 256 threads per (sequence, head)
  if (!a.cu_seqlens || (!a.workspace && !a.no_workspace)) return GDR_ERR_INVALID_ARGUMENT;
  if (a.T > 0 && (!a.q || !a.k || !a.v || !a.g || !a.beta || !a.out)) return GDR_ERR_INVALID_ARGUMENT;
  const void* ptrs[] = {a.q, a.k, a.v, a.g, a.beta, a.state_in, a.cu_seqlens, a.out, a.state_out};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return GDR_ERR_INVALID_ARGUMENT;
  if (!a.no_workspace) {
    if ((reinterpret_cast<uintptr_t>(a.workspace) & 255u) != 0) return GDR_ERR_INVALID_ARGUMENT;
    const Workspace w = plan_workspace(a.T, a.N, a.Nqk, a.Nv, a.dtype, a.budget, chunk_len(a.flags));
    if (w.total < 0 || a.workspace_bytes < static_cast<size_t>(w.total))
      return GDR_ERR_WORKSPACE_TOO_SMALL;
  }

  const int64_t es = static_cast<int64_t>(dtype_size(a.dtype));
  const int64_t qk_bytes = static_cast<int64_t>(a.T) * a.Nqk * 128 * es;
  const int64_t v_bytes = static_cast<int64_t>(a.T) * a.Nv * 128 * es;
  const int64_t gb_bytes = static_cast<int64_t>(a.T) * a.Nv * 4;
  const int64_t st_bytes = static_cast<int64_t>(a.N) * a.Nv * 128 * 128 * 4;
  const int64_t cu_bytes = (static_cast<int64_t>(a.N) + 1) * 4;
  // out overlaps nothing else
  struct R { const void* p; int64_t n; } in[] = {
      {a.q, qk_bytes}, {a.k, qk_bytes}, {a.v, v_bytes}, {a.g, gb_bytes}, {a.beta, gb_bytes},
      {a.state_in, st_bytes}, {a.cu_seqlens, cu_bytes}, {a.state_out, st_bytes},
      {a.workspace, static_cast<int64_t>(a.workspace_bytes)}};
  for (const R& r : in)
    if (overlap(a.out, v_bytes, r.p, r.n)) return GDR_ERR_INVALID_ARGUMENT;
  // state_out may equal state_in exactly, but not overlap it partially, and
  // overlaps no other input
  if (a.state_out) {
    if (a.state_out != a.state_in && overlap(a.state_out, st_bytes, a.state_in, st_bytes))
      return GDR_ERR_INVALID_ARGUMENT;
    R others[] = {{a.q, qk_bytes}, {a.k, qk_bytes}, {a.v, v_bytes}, {a.g, gb_bytes},
                  {a.beta, gb_bytes}, {a.cu_seqlens, cu_bytes},
                  {a.workspace, static_cast<int64_t>(a.workspace_bytes)}};
    for (const R& r : others)
      if (overlap(a.state_out, st_bytes, r.p, r.n)) return GDR_ERR_INVALID_ARGUMENT;
  }
  return GDR_OK;
}

gdr_status validate_step(const StepArgs& a) {
  gdr_status s = common_sizes(a.Nqk, a.Nv, a.D, a.dtype, a.flags);
  if (s != GDR_OK) return s;
  if (a.N < 0) return GDR_ERR_INVALID_ARGUMENT;
  // one workgroup of 256 threads per (sequence, head): the grid stays below 2^32 work-items
  if (static_cast<int64_t>(a.N) * a.Nv >= (int64_t(1) << 24)) return GDR_ERR_INVALID_ARGUMENT;
  if (a.N == 0) return GDR_OK;
  if (!a.q || !a.k || !a.v || !a.g || !a.beta || !a.state_in || !a.state_out || !a.out)
    return GDR_ERR_INVALID_ARGUMENT;
  const void* ptrs[] = {a.q, a.k, a.v, a.g, a.beta, a.state_in, a.state_out, a.out};
  for (const void* p : ptrs)
    if (!aligned16(p)) return GDR_ERR_INVALID_ARGUMENT;
  const int64_t es = static_cast<int64_t>(dtype_size(a.dtype));
  const int64_t qk_bytes = static_cast<int64_t>(a.N) * a.Nqk * 128 * es;
  const int64_t v_bytes = static_cast<int64_t>(a.N) * a.Nv * 128 * es;
  const int64_t gb_bytes = static_cast<int64_t>(a.N) * a.Nv * 4;
  const int64_t st_bytes = static_cast<int64_t>(a.N) * a.Nv * 128 * 128 * (a.state_bf16 ? 2 : 4);
  struct R { const void* p; int64_t n; } in[] = {
      {a.q, qk_bytes}, {a.k, qk_bytes}, {a.v, v_bytes}, {a.g, gb_bytes}, {a.beta, gb_bytes},
      {a.state_in, st_bytes}, {a.state_out, st_bytes}};
  for (const R& r : in)
    if (overlap(a.out, v_bytes, r.p, r.n)) return GDR_ERR_INVALID_ARGUMENT;
  if (a.state_out != a.state_in && overlap(a.state_out, st_bytes, a.state_in, st_bytes))
    return GDR_ERR_INVALID_ARGUMENT;
  R others[] = {{a.q, qk_bytes}, {a.k, qk_bytes}, {a.v, v_bytes}, {a.g, gb_bytes}, {a.beta, gb_bytes}};
  for (const R& r : others)
    if (overlap(a.state_out, st_bytes, r.p, r.n)) return GDR_ERR_INVALID_ARGUMENT;
  if (a.z) {
    if (!aligned16(a.z) || (a.nw && !aligned16(a.nw))) return GDR_ERR_INVALID_ARGUMENT;
    if (!std::isfinite(a.norm_eps) || a.norm_eps < 0.0f) return GDR_ERR_INVALID_ARGUMENT;
    if (overlap(a.out, v_bytes, a.z, v_bytes) || overlap(a.out, v_bytes, a.nw, 128 * es) ||
        overlap(a.state_out, st_bytes, a.z, v_bytes) || overlap(a.state_out, st_bytes, a.nw, 128 * es))
      return GDR_ERR_INVALID_ARGUMENT;
  }
  return GDR_OK;
}

gdr_status validate_norm(const NormArgs& a) {
  if (a.D != 128) return GDR_ERR_UNSUPPORTED;
  if (a.dtype != GDR_F32 && a.dtype != GDR_BF16) return GDR_ERR_UNSUPPORTED;
  if (a.rows < 0 || a.rows >= (int64_t(1) << 31)) return GDR_ERR_INVALID_ARGUMENT;
  if (!std::isfinite(a.eps) || a.eps < 0.0f) return GDR_ERR_INVALID_ARGUMENT;
  if (a.rows == 0) return GDR_OK;
  if (!a.x || !a.z || !a.y) return GDR_ERR_INVALID_ARGUMENT;
  if (!aligned16(a.x) || !aligned16(a.z) || !aligned16(a.y) || (a.w && !aligned16(a.w)))
    return GDR_ERR_INVALID_ARGUMENT;
  const int64_t es = static_cast<int64_t>(dtype_size(a.dtype));
  const int64_t bytes = a.rows * 128 * es;
  if (a.y != a.x && overlap(a.y, bytes, a.x, bytes)) return GDR_ERR_INVALID_ARGUMENT;
  if (overlap(a.y, bytes, a.z, bytes) || overlap(a.y, bytes, a.w, 128 * es))
    return GDR_ERR_INVALID_ARGUMENT;
  return GDR_OK;
}

gdr_status validate_conv_step(const ConvStepArgs& a) {
  gdr_status s = common_sizes(a.Nqk, a.Nv, a.D, a.dtype, a.flags);
  if (s != GDR_OK) return s;
  if (a.conv_k != 4) return GDR_ERR_UNSUPPORTED;
  if (a.N < 0) return GDR_ERR_INVALID_ARGUMENT;
  // one workgroup of 256 threads per (sequence, head): the grid stays below 2^32 work-items
  if (static_cast<int64_t>(a.N) * a.Nv >= (int64_t(1) << 24)) return GDR_ERR_INVALID_ARGUMENT;
  if (a.N == 0) return GDR_OK;
  const void* req[] = {a.x, a.cs_in, a.cs_out, a.w, a.a, a.b, a.A_log, a.dt_bias, a.state_in,
                       a.state_out, a.out};
  for (const void* p : req)
    if (!p || !aligned16(p)) return GDR_ERR_INVALID_ARGUMENT;
  if (a.bias && !aligned16(a.bias)) return GDR_ERR_INVALID_ARGUMENT;
  const int64_t es = static_cast<int64_t>(dtype_size(a.dtype));
  const int64_t C = (2 * static_cast<int64_t>(a.Nqk) + a.Nv) * 128;
  const int64_t x_bytes = a.N * C * es, cs_bytes = a.N * C * 4 * es, w_bytes = C * 4 * es;
  const int64_t b_bytes = C * es, nv_bytes = static_cast<int64_t>(a.N) * a.Nv * 4;
  const int64_t h_bytes = static_cast<int64_t>(a.Nv) * 4;
  const int64_t st_bytes = static_cast<int64_t>(a.N) * a.Nv * 128 * 128 * 4;
  const int64_t o_bytes = static_cast<int64_t>(a.N) * a.Nv * 128 * es;
  struct R { const void* p; int64_t n; };
  const R in[] = {{a.x, x_bytes}, {a.cs_in, cs_bytes}, {a.w, w_bytes}, {a.bias, b_bytes},
                  {a.a, nv_bytes}, {a.b, nv_bytes}, {a.A_log, h_bytes}, {a.dt_bias, h_bytes},
                  {a.state_in, st_bytes}};
  // each output overlaps no input and no other output; state_out may equal
  // state_in exactly (in-place update of the recurrent state)
  const R outs[] = {{a.cs_out, cs_bytes}, {a.state_out, st_bytes}, {a.out, o_bytes}};
  constexpr int kOuts = 3, kStateOut = 1, kIns = 9, kStateIn = 8;
  static_assert(sizeof(in) / sizeof(in[0]) == kIns && sizeof(outs) / sizeof(outs[0]) == kOuts,
                "index constants out of date");
  for (int i = 0; i < kOuts; ++i) {
    for (int r = 0; r < kIns; ++r) {
      if (i == kStateOut && r == kStateIn && a.state_out == a.state_in) continue;
      if (overlap(outs[i].p, outs[i].n, in[r].p, in[r].n)) return GDR_ERR_INVALID_ARGUMENT;
    }
    for (int r = 0; r < kOuts; ++r)   // distinct outputs, even at the same address
      if (r != i && overlap(outs[i].p, outs[i].n, outs[r].p, outs[r].n))
        return GDR_ERR_INVALID_ARGUMENT;
  }
  return GDR_OK;
}

gdr_status validate_conv_prefill(const ConvPrefillCheck& a) {
  gdr_status s = common_sizes(a.Nqk, a.Nv, a.D, a.dtype, 0u);
  if (s != GDR_OK) return s;
  if (a.conv_k != 4) return GDR_ERR_UNSUPPORTED;
  if (a.N < 1 || a.T < 0) return GDR_ERR_INVALID_ARGUMENT;
  // the window update runs one row of 256-thread workgroups per sequence
  if (a.N >= (int32_t(1) << 24)) return GDR_ERR_INVALID_ARGUMENT;
  const int64_t C = (2 * static_cast<int64_t>(a.Nqk) + a.Nv) * 128;
  if (static_cast<int64_t>(a.T) * C > (int64_t(1) << 40)) return GDR_ERR_INVALID_ARGUMENT;
  if (!a.w || !a.A_log || !a.dt_bias || !a.cu) return GDR_ERR_INVALID_ARGUMENT;
  if (a.T > 0 && (!a.x || !a.a || !a.b || !a.q || !a.k || !a.v || !a.g || !a.beta))
    return GDR_ERR_INVALID_ARGUMENT;
  const void* ptrs[] = {a.x, a.cs_in, a.cs_out, a.w, a.bias, a.a, a.b, a.A_log, a.dt_bias,
                        a.cu, a.q, a.k, a.v, a.g, a.beta};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return GDR_ERR_INVALID_ARGUMENT;
  const int64_t es = static_cast<int64_t>(dtype_size(a.dtype));
  const int64_t T = a.T, N = a.N;
  const int64_t qk_bytes = T * a.Nqk * 128 * es, v_bytes = T * a.Nv * 128 * es;
  const int64_t tv_bytes = T * a.Nv * 4, h_bytes = static_cast<int64_t>(a.Nv) * 4;
  const int64_t cs_bytes = N * C * 4 * es;
  struct R { const void* p; int64_t n; };
  const R in[] = {{a.x, T * C * es}, {a.cs_in, cs_bytes}, {a.w, C * 4 * es}, {a.bias, C * es},
                  {a.a, tv_bytes}, {a.b, tv_bytes}, {a.A_log, h_bytes}, {a.dt_bias, h_bytes},
                  {a.cu, (N + 1) * 4}};
  const R outs[] = {{a.cs_out, cs_bytes}, {a.q, qk_bytes}, {a.k, qk_bytes}, {a.v, v_bytes},
                    {a.g, tv_bytes}, {a.beta, tv_bytes}};
  constexpr int kIns = 9, kOuts = 6, kCsIn = 1, kCsOut = 0;
  static_assert(sizeof(in) / sizeof(in[0]) == kIns && sizeof(outs) / sizeof(outs[0]) == kOuts,
                "index constants out of date");
  // each output overlaps no input and no other output; the new windows may
  // replace the cached ones exactly (in place)
  for (int i = 0; i < kOuts; ++i) {
    for (int r = 0; r < kIns; ++r) {
      if (i == kCsOut && r == kCsIn && a.cs_out == a.cs_in) continue;
      if (overlap(outs[i].p, outs[i].n, in[r].p, in[r].n)) return GDR_ERR_INVALID_ARGUMENT;
    }
    for (int r = 0; r < kOuts; ++r)
      if (r != i && overlap(outs[i].p, outs[i].n, outs[r].p, outs[r].n))
        return GDR_ERR_INVALID_ARGUMENT;
  }
  return GDR_OK;
}

}  // namespace gdr
