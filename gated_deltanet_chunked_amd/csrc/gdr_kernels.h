// gdr_kernels.h -- host-callable launchers of the libgdr kernels.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/gdr.h"

namespace gdr {

// Optional timing of one launch: events recorded by the runtime at the
// kernel's start and end (hipExtLaunchKernelGGL).  Null events: no timing.
struct LaunchEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};

// Chunk slots of the packed sequences.  Chunks restart at every sequence
// start (Qwen3-Next blog post, section 5(1)c).  With a chunk table (built
// from cu_seqlens by table_kernel) slot s is {sequence, first token, length,
// rank of the sequence among the non-empty ones}, and nonempty[r] is the
// sequence of rank r; for a single sequence (table == nullptr) slot s covers
// tokens [lo + L s, min(lo + L (s + 1), hi)), lo and hi being cu_seqlens[0..1]
// clamped into [0, T]: the entries the table kernel would write.
struct Chunks {
  const int4* table;
  const int32_t* choff;
  const int32_t* nonempty;
  const int32_t* cu;
  int32_t T;
  int32_t L;   // chunk length: 128, or 64
  int32_t N;   // sequences
  __device__ __forceinline__ void one_range(int& lo, int& hi) const {
    lo = min(max(cu[0], 0), T);
    hi = min(max(cu[1], lo), T);
  }
  // tokens of slot s; false for an unused slot
  __device__ __forceinline__ bool slot(int s, int& start, int& len) const {
    if (table) {
      const int4 e = table[s];
      start = e.y;
      len = e.z;
      return e.x >= 0;
    }
    int lo, hi;
    one_range(lo, hi);
    start = lo + L * s;
    len = min(L, hi - start);
    return start < hi;
  }
  // The sequence b of the r-th run of one sequence's slots among slots
  // [s0, s0 + n) (a segment); false when the segment holds fewer runs.  The
  // runs of a segment are sequences of consecutive ranks, at most n of them,
  // so a launch over a segment needs min(N, n) of them whatever N is.
  __device__ __forceinline__ bool run_sequence(int s0, int n, int r, int& b) const {
    if (!table) {
      b = 0;
      return r == 0;
    }
    const int4 e = table[s0];
    if (e.x < 0) return false;   // the segment lies past the used slots
    const int rank = e.w + r;
    if (rank >= N) return false;
    b = nonempty[rank];
    return b >= 0 && choff[b] < s0 + n;
  }
  // slots [c0, c1) of sequence b
  __device__ __forceinline__ void seq_slots(int b, int& c0, int& c1) const {
    if (table) {
      c0 = choff[b];
      c1 = choff[b + 1];
      return;
    }
    int lo, hi;
    one_range(lo, hi);
    c0 = 0;
    c1 = (hi - lo + L - 1) / L;
  }
};

// One launch in front of the chunkwise passes, with up to two parts: the
// chunk table (build: table, choff, nonempty; for N > 1), and the final
// states of the empty sequences (copy: state_out[b] = state_in[b], or zeros
// without state_in), which the state pass, running over chunk slots only,
// never visits.
void launch_table(const int32_t* cu, int32_t N, int32_t T, int32_t L, int32_t nslots, int4* table,
                  int32_t* choff, int32_t* nonempty, bool build, bool copy, int32_t Nv,
                  const float* state_in, float* state_out, hipStream_t stream,
                  LaunchEvents ev = {});

// Intra-chunk products for chunk slots [slot0, slot0 + nseg) of every value head;
// also writes exp(total gate of the chunk) to gam[slot][head].
template <typename Tin>
hipError_t launch_intra(const Tin* q, const Tin* k, const Tin* v, const float* g, const float* beta,
                        Chunks chunks, int32_t Nqk, int32_t Nv, int32_t slot0, int32_t nseg,
                        float scale, int norm, Tin* inter, float* gam, hipStream_t stream,
                        LaunchEvents ev = {});

// The bf16 kernel behind launch_intra<__bf16> (gdr_intra_bf16.hip).
hipError_t launch_intra_bf16(const __bf16* q, const __bf16* k, const __bf16* v, const float* g,
                             const float* beta, Chunks chunks, int32_t Nqk, int32_t Nv,
                             int32_t slot0, int32_t nseg, float scale, int norm, __bf16* inter,
                             float* gam, hipStream_t stream, LaunchEvents ev = {});

// Chunk-serial state pass over chunk slots [slot0, slot0 + nseg), for the
// sequences with slots there (grid: value heads x row blocks, then the
// segment's runs of slots, at most min(N, nseg)).  `discard` is 256 bytes of
// scratch that absorbs the stores of rows past a chunk's end.
template <typename Tin>
void launch_inter(const Tin* inter, Chunks chunks, const float* gam,
                  const float* state_in, float* carry, float* state_out, int32_t N, int32_t Nv,
                  int32_t slot0, int32_t nseg, Tin* out, Tin* discard,
                  hipStream_t stream, LaunchEvents ev = {});

// The bf16 kernel behind launch_inter<__bf16> (gdr_inter_bf16.hip).
void launch_inter_bf16(const __bf16* inter, Chunks chunks, const float* gam, const float* state_in,
                       float* carry, float* state_out, int32_t N, int32_t Nv, int32_t slot0,
                       int32_t nseg, __bf16* out, __bf16* discard,
                       hipStream_t stream, LaunchEvents ev = {});

// One decode step; the state is stored as St (float, or __bf16 for a bf16
// state cache), the arithmetic is fp32 either way.
template <typename Tin, typename St>
void launch_decode(const Tin* q, const Tin* k, const Tin* v, const float* g, const float* beta,
                   const St* state_in, St* state_out, int32_t N, int32_t Nqk, int32_t Nv,
                   float scale, int norm, Tin* out, hipStream_t stream, LaunchEvents ev = {},
                   const Tin* gate_z = nullptr, const Tin* gate_w = nullptr, float gate_eps = 0.f);

// Debug checks of device-side values (gdr_debug.hip): on when GDR_DEBUG is
// set in the environment or after gdr_set_debug(1).  debug_check runs one
// kernel over cu_seqlens (may be NULL) and ng gates and waits for it; it
// returns GDR_ERR_CONTRACT with the broken contracts' bits in *broken.
bool debug_enabled();
gdr_status debug_check(const int32_t* cu, int32_t N, int32_t T, const float* g, int64_t ng,
                       hipStream_t st, uint32_t* broken);

// The gated RMSNorm y = x / rms(x) * w * SiLU(z) over rows of kD values; x may
// equal y.  w NULL: ones.
template <typename T>
void launch_gated_rmsnorm(const T* x, const T* z, const T* w, int64_t rows, float eps, T* y,
                          hipStream_t stream, LaunchEvents ev = {});

// Several tokens per sequence, token by token with the state in registers;
// sequence n owns tokens [cu[n], cu[n+1]) of the packed batch.
template <typename Tin>
void launch_multi(const Tin* q, const Tin* k, const Tin* v, const float* g, const float* beta,
                  const float* state_in, const int32_t* cu, int32_t N, int32_t T_total,
                  float* state_out, int32_t Nqk, int32_t Nv, float scale, int norm, Tin* out,
                  hipStream_t stream, LaunchEvents ev = {});

// One decode step with the conv update and gate functions fused in front
// (conv kernel size 4).
template <typename Tin>
void launch_decode_conv(const Tin* x, const Tin* cs_in, Tin* cs_out, const Tin* w,
                        const Tin* bias, const float* a, const float* b, const float* A_log,
                        const float* dt_bias, const float* state_in, float* state_out, int32_t N,
                        int32_t Nqk, int32_t Nv, float scale, int norm, Tin* out,
                        hipStream_t stream, LaunchEvents ev = {});

// The conv/gate prologue of the chunkwise path over packed sequences.
template <typename T>
struct ConvPrefillArgs {
  const T* x;           // [T, C] projected q|k|v, C = (2 Nqk + Nv) 128
  const T* cs_in;       // [N, C, 4] cached windows (oldest first), or nullptr for zeros
  T* cs_out;            // [N, C, 4] new windows, or nullptr; may equal cs_in
  const T* w;           // [C, 4]
  const T* bias;        // [C] or nullptr
  const float* a;       // [T, Nv]
  const float* b;       // [T, Nv]
  const float* A_log;   // [Nv]
  const float* dt_bias; // [Nv]
  const int32_t* cu;    // [N + 1]
  int32_t N, Ttok, Nqk, Nv, C;   // Ttok: tokens in the batch
  T* q;                 // [T, Nqk, 128]
  T* k;                 // [T, Nqk, 128]
  T* v;                 // [T, Nv, 128]
  float* g;             // [T, Nv]
  float* beta;          // [T, Nv]
};

// Conv + gates over the tokens (skipped for T = 0), then the new windows
// (when cs_out is set): up to two launches.
template <typename T>
void launch_conv_prefill(const ConvPrefillArgs<T>& p, hipStream_t stream, LaunchEvents ev_conv = {},
                         LaunchEvents ev_window = {});

}  // namespace gdr
