// gdr_table.hip -- first stage of the chunkwise forward: the chunk table, and
// the final states of empty sequences.
//
// Chunks of L tokens (128, or 64) restart at every sequence start (Qwen3-Next
// blog post, section 5(1)c: the gate cumsum restarts at each chunk), so
// sequence b owns ceil(len_b / L) chunk slots starting at choff[b].
#include "gdr_device.h"
#include "gdr_kernels.h"

namespace gdr {

// Workgroup 0 (with build) builds the table with 1024 threads.  Token ranges
// are clamped into [0, T] so a malformed cu_seqlens can only produce wrong
// numbers, never an access outside the caller's buffers; slots beyond
// nslots are dropped.  Alongside the chunk offsets it ranks the non-empty
// sequences (a second scan), so that the state pass can launch over a
// segment's runs of slots rather than over all N sequences.
__device__ void build_table(const int32_t* __restrict__ cu, int32_t N, int32_t T, int32_t L,
                            int32_t nslots, int4* __restrict__ table, int32_t* __restrict__ choff,
                            int32_t* __restrict__ nonempty) {
  __shared__ int32_t part[1024], npart[1024];
  const int tid = threadIdx.x;
  const int per = (N + 1023) / 1024;
  const int b0 = min(N, tid * per), b1 = min(N, b0 + per);
  auto range = [&](int b, int& lo, int& hi) {
    lo = min(max(cu[b], 0), T);
    hi = min(max(cu[b + 1], lo), T);
  };
  int32_t local = 0, nlocal = 0;
  for (int b = b0; b < b1; ++b) {
    int lo, hi;
    range(b, lo, hi);
    local += (hi - lo + L - 1) / L;
    nlocal += hi > lo ? 1 : 0;
  }
  part[tid] = local;
  npart[tid] = nlocal;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int32_t x = tid >= off ? part[tid - off] : 0;
    const int32_t y = tid >= off ? npart[tid - off] : 0;
    __syncthreads();
    part[tid] += x;
    npart[tid] += y;
    __syncthreads();
  }
  int32_t run = part[tid] - local, rank = npart[tid] - nlocal;
  for (int b = b0; b < b1; ++b) {
    int lo, hi;
    range(b, lo, hi);
    choff[b] = min(run, nslots);
    const int nch = (hi - lo + L - 1) / L;
    if (nch > 0) nonempty[rank] = b;
    for (int m = 0; m < nch; ++m) {
      const int s = run + m;
      if (s < nslots) table[s] = make_int4(b, lo + L * m, min(L, hi - lo - L * m), rank);
    }
    run += nch;
    rank += nch > 0 ? 1 : 0;
  }
  const int32_t total = min(part[1023], nslots);
  if (tid == 0) choff[N] = total;
  for (int s = total + tid; s < nslots; s += 1024) table[s] = make_int4(-1, 0, 0, 0);
  for (int r = npart[1023] + tid; r < N; r += 1024) nonempty[r] = -1;
}

// The other workgroups (all of them without build): the final state of every
// empty sequence, its initial state (zeros without one), over (sequence,
// head) pairs with a grid stride; a sequence is empty exactly when the table
// gives it no slot.
__global__ __launch_bounds__(1024) void table_kernel(const int32_t* __restrict__ cu, int32_t N,
                                                     int32_t T, int32_t L, int32_t nslots,
                                                     int4* __restrict__ table,
                                                     int32_t* __restrict__ choff,
                                                     int32_t* __restrict__ nonempty, int build,
                                                     int32_t Nv, const float* state_in,
                                                     float* state_out) {
  if (build && blockIdx.x == 0) {
    build_table(cu, N, T, L, nslots, table, choff, nonempty);
    return;
  }
  const int first = build ? 1 : 0;
  const int64_t pairs = (int64_t)N * Nv;
  for (int64_t p = blockIdx.x - first; p < pairs; p += gridDim.x - first) {
    const int b = (int)(p / Nv);
    const int lo = min(max(cu[b], 0), T);
    const int hi = min(max(cu[b + 1], lo), T);
    if (hi > lo) continue;
    const size_t base = (size_t)p * 128 * 128;
    for (int i = threadIdx.x; i < 128 * 128 / 4; i += 1024) {
      float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
      if (state_in) x = reinterpret_cast<const float4*>(state_in + base)[i];
      reinterpret_cast<float4*>(state_out + base)[i] = x;
    }
  }
}

void launch_table(const int32_t* cu, int32_t N, int32_t T, int32_t L, int32_t nslots, int4* table,
                  int32_t* choff, int32_t* nonempty, bool build, bool copy, int32_t Nv,
                  const float* state_in, float* state_out, hipStream_t stream, LaunchEvents ev) {
  const int64_t pairs = copy ? (int64_t)N * Nv : 0;
  const unsigned blocks = (build ? 1u : 0u) + (unsigned)(pairs < 1024 ? pairs : 1024);
  if (blocks == 0) return;
  hipExtLaunchKernelGGL(table_kernel, dim3(blocks), dim3(1024), 0, stream, ev.start, ev.stop, 0, cu,
                        N, T, L, nslots, table, choff, nonempty, build ? 1 : 0, Nv, state_in,
                        state_out);
}

}  // namespace gdr
