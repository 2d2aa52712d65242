// gdr_internal.h -- host-side plumbing of libgdr: workspace layout and the
// HIP-free argument validation shared by the C entry points.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/gdr.h"

namespace gdr {

// Number of chunk slots (chunks of L = 128 or 64 tokens) reserved for T packed
// tokens in N sequences.  Chunks restart at every sequence start, so sequence
// b needs ceil(len_b / L) <= (len_b + L - 1) / L slots, and the sum over b is
// at most floor((T + (L - 1) N) / L).  For one sequence that is exactly its chunk
// count, so no segment carries an empty slot (at T = 32768 and 32 heads a
// segment of 32 slots is 1024 units of the intra kernel: two full rounds of
// two workgroups per CU, where a 33rd slot would start a third).
inline int64_t max_slots(int64_t T, int64_t N, int64_t L = 128) { return (T + (L - 1) * N) / L; }

// Chunk length of a chunkwise call: 128, or 64 with GDR_FLAG_CHUNK64.
inline int32_t chunk_len(uint32_t flags) { return (flags & GDR_FLAG_CHUNK64) ? 64 : 128; }

// Upper bound on the chunk slots of one segment (the state pass stages a
// segment's chunk table in LDS).
constexpr int kMaxSegSlots = 512;

// Largest number of value heads.  It keeps the 128 rows of a chunk of v (row
// stride Nv * 128 elements of at most 4 bytes) within 2 GiB, so the kernels
// address a chunk's rows with 32-bit byte offsets from a per-chunk base, and
// every launch's grid within 2^32 work-items (the intra-chunk kernel runs up
// to 512 slots x Nv workgroups of 256 threads per segment).
constexpr int32_t kMaxNv = 16384;

// Chunk slots processed per segment: the intra-chunk products of one segment
// are written to the workspace and consumed by the state pass of the same
// segment before the next segment reuses the buffer.  A segment's matrices
// are kept to about 128 MiB (at most 1.5x that) so they stay in the 256 MB Infinity Cache between
// the two kernels, and the slots are split evenly over the segments.
inline int64_t segment_slots(int64_t nslots, int64_t Nv, int64_t elem_bytes) {
  const int64_t per_slot = Nv * 4 * 128 * 128 * elem_bytes;
  int64_t cap = (int64_t(128) << 20) / per_slot;
  if (cap < 8) cap = 8;
  int64_t nsegs = (nslots + cap / 2) / cap;   // nearest whole number of segments
  if (nsegs < 1) nsegs = 1;
  const int64_t most = (nslots + kMaxSegSlots - 1) / kMaxSegSlots;
  if (nsegs < most) nsegs = most;
  return (nslots + nsegs - 1) / nsegs;
}

// Per (chunk slot, value head): four 128x128 matrices of the chunk's affine
// state transition and output terms (see gdr_intra.hip).
constexpr int64_t kInterMats = 4;
constexpr int64_t kMatElems = 128 * 128;

struct Workspace {
  int64_t table;      // int32 [nslots][4]: {sequence, first token, length, 0}; sequence -1 = unused
  int64_t choff;      // int32 [N + 1]: first slot of each sequence
  int64_t nonempty;   // int32 [N]: the non-empty sequences in order (-1 past the last)
  int64_t gam;        // float [nslots][Nv]: exp(sum of g over the chunk)
  int64_t inter;      // [seg_slots][Nv][4][128][128] of the matrix-core operand type
  int64_t carry;      // float [N][Nv][128][128]: state between segments
  int64_t discard;    // 256 bytes: target of the state pass's stores for rows past a chunk's end
  int64_t total;
  int64_t nslots;
  int64_t seg_slots;
};

// Layout of the workspace.  budget = 0: segments of about 128 MiB of matrices
// (segment_slots).  budget > 0: the largest even split whose whole layout
// fits in `budget` bytes; total = -1 when not even one chunk slot fits.
Workspace plan_workspace(int64_t T, int64_t N, int64_t Nqk, int64_t Nv, gdr_dtype dtype,
                         int64_t budget = 0, int64_t L = 128);

struct ChunkArgs {
  const void* q; const void* k; const void* v;
  const float* g; const float* beta;
  const float* state_in; const int32_t* cu_seqlens;
  int32_t N, T, Nqk, Nv, D;
  gdr_dtype dtype;
  float scale;
  uint32_t flags;
  void* out; float* state_out;
  void* workspace; size_t workspace_bytes;
  bool no_workspace;   // gdr_recurrent_multi: the same arguments, no workspace
  int64_t budget;      // > 0: the workspace is a fixed buffer of this many bytes (plan_workspace)
};

struct StepArgs {
  const void* q; const void* k; const void* v;
  const float* g; const float* beta;
  const void* state_in; void* state_out;   // float, or bf16 when state_bf16
  int32_t N, Nqk, Nv, D;
  gdr_dtype dtype;
  float scale;
  uint32_t flags;
  void* out;
  bool state_bf16;
  // gated RMSNorm behind the step (z NULL: none); weight NULL means ones
  const void* z = nullptr;
  const void* nw = nullptr;
  float norm_eps = 0.f;
};

struct NormArgs {
  const void* x; const void* z; const void* w;
  int64_t rows;
  int32_t D;
  gdr_dtype dtype;
  float eps;
  void* y;
};

struct ConvStepArgs {
  const void* x; const void* cs_in; void* cs_out; const void* w; const void* bias;
  int32_t conv_k;
  const float* a; const float* b; const float* A_log; const float* dt_bias;
  const float* state_in; float* state_out;
  int32_t N, Nqk, Nv, D;
  gdr_dtype dtype;
  float scale;
  uint32_t flags;
  void* out;
};

struct ConvPrefillCheck {
  const void* x; const void* cs_in; void* cs_out; const void* w; const void* bias;
  int32_t conv_k;
  const float* a; const float* b; const float* A_log; const float* dt_bias;
  const int32_t* cu;
  int32_t N, T, Nqk, Nv, D;
  gdr_dtype dtype;
  void* q; void* k; void* v; float* g; float* beta;
};

gdr_status validate_conv_prefill(const ConvPrefillCheck& a);
gdr_status validate_chunk(const ChunkArgs& a);
gdr_status validate_conv_step(const ConvStepArgs& a);
gdr_status validate_step(const StepArgs& a);
gdr_status validate_norm(const NormArgs& a);

inline size_t dtype_size(gdr_dtype d) { return d == GDR_BF16 ? 2 : 4; }

}  // namespace gdr
