// gdr_api.hip -- the extern "C" entry points of libgdr (declared in
// include/gdr.h): argument validation, workspace carving and kernel launches
// on the caller's stream.  No allocation, no synchronisation.
#include <hip/hip_runtime.h>

#include <mutex>
#include <vector>

#include "../../include/gdr.h"
#include "gdr_internal.h"
#include "gdr_kernels.h"

using namespace gdr;

namespace {

// Optional per-launch timing: launch i gets the event pair ev[2i], ev[2i+1],
// which the runtime records at that kernel's start and end.  With span_only,
// only the first launch's start (ev[0]) and the last launch's end (ev[1]) are
// recorded, `total` being the number of launches.  With no event array every
// launch is untimed.
struct Recorder {
  hipEvent_t* ev = nullptr;
  int32_t* kind = nullptr;
  int32_t cap = 0;
  int32_t n = 0;
  bool span_only = false;
  int32_t total = 0;
  LaunchEvents next(int32_t k) {
    LaunchEvents e;
    if (ev && span_only) {
      if (n == 0) e.start = ev[0];
      if (n == total - 1) e.stop = ev[1];
    } else if (ev && n < cap) {
      kind[n] = k;
      e.start = ev[2 * n];
      e.stop = ev[2 * n + 1];
    }
    ++n;
    return e;
  }
};

// Event pairs for timed launches, destroyed with the object.
struct EventPairs {
  std::vector<hipEvent_t> ev;
  bool create(int32_t launches) {
    if (launches < 0) return false;
    ev.reserve(2 * static_cast<size_t>(launches));
    while (ev.size() < 2 * static_cast<size_t>(launches)) {
      hipEvent_t e;
      if (hipEventCreate(&e) != hipSuccess) return false;
      ev.push_back(e);
    }
    return true;
  }
  ~EventPairs() {
    for (hipEvent_t e : ev) (void)hipEventDestroy(e);
  }
};

// The launch in front of the segments: the chunk table for packed batches
// (a single sequence needs none: Chunks derives its slots from cu_seqlens
// directly), and the final states of empty sequences, which the state pass
// never visits (only a packed batch, or a single sequence with T = 0, can
// have one; in place there is nothing to copy).
bool table_build(const ChunkArgs& a) { return a.N > 1; }
bool table_copy(const ChunkArgs& a) {
  return a.state_out && a.state_out != a.state_in && (a.N > 1 || a.T == 0);
}

// Launches of one call: the table launch (when it has work), then two per
// segment.
int32_t launches_needed(const ChunkArgs& a, const Workspace& w) {
  // no slot at all (a single empty sequence): no segment
  const int64_t segs = w.seg_slots > 0 ? (w.nslots + w.seg_slots - 1) / w.seg_slots : 0;
  return static_cast<int32_t>((table_build(a) || table_copy(a) ? 1 : 0) + 2 * segs);
}

template <typename T>
gdr_status run_chunk(const ChunkArgs& a, hipStream_t st, Recorder& rec) {
  const int32_t L = chunk_len(a.flags);
  const Workspace w = plan_workspace(a.T, a.N, a.Nqk, a.Nv, a.dtype, a.budget, L);
  char* ws = static_cast<char*>(a.workspace);
  int4* table = reinterpret_cast<int4*>(ws + w.table);
  int32_t* choff = reinterpret_cast<int32_t*>(ws + w.choff);
  int32_t* nonempty = reinterpret_cast<int32_t*>(ws + w.nonempty);
  float* gam = reinterpret_cast<float*>(ws + w.gam);
  T* inter = reinterpret_cast<T*>(ws + w.inter);
  float* carry = a.state_out ? a.state_out : reinterpret_cast<float*>(ws + w.carry);
  T* discard = reinterpret_cast<T*>(ws + w.discard);
  const T* q = static_cast<const T*>(a.q);
  const T* k = static_cast<const T*>(a.k);
  const T* v = static_cast<const T*>(a.v);
  T* out = static_cast<T*>(a.out);
  const int norm = (a.flags & GDR_FLAG_QK_L2NORM) ? 1 : 0;
  const int32_t nslots = static_cast<int32_t>(w.nslots);

  // Every launch is checked at once: hipGetLastError also clears the error,
  // so a failed launch followed by a good one would otherwise go unseen.
  Chunks chunks{nullptr, nullptr, nullptr, a.cu_seqlens, a.T, L, a.N};
  const bool build = table_build(a), copy = table_copy(a);
  if (build || copy) {
    launch_table(a.cu_seqlens, a.N, a.T, L, nslots, table, choff, nonempty, build, copy, a.Nv,
                 a.state_in, a.state_out, st, rec.next(GDR_STAGE_TABLE));
    if (hipGetLastError() != hipSuccess) return GDR_ERR_HIP;
  }
  if (build) {
    chunks.table = table;
    chunks.choff = choff;
    chunks.nonempty = nonempty;
  }
  for (int64_t s0 = 0; s0 < w.nslots; s0 += w.seg_slots) {
    const int32_t nseg = static_cast<int32_t>(w.nslots - s0 < w.seg_slots ? w.nslots - s0 : w.seg_slots);
    if (launch_intra<T>(q, k, v, a.g, a.beta, chunks, a.Nqk, a.Nv, static_cast<int32_t>(s0), nseg,
                        a.scale, norm, inter, gam, st, rec.next(GDR_STAGE_INTRA)) != hipSuccess)
      return GDR_ERR_HIP;
    launch_inter<T>(inter, chunks, gam, a.state_in, carry, a.state_out, a.N, a.Nv,
                    static_cast<int32_t>(s0), nseg, out, discard, st, rec.next(GDR_STAGE_INTER));
    if (hipGetLastError() != hipSuccess) return GDR_ERR_HIP;
  }
  return GDR_OK;
}

// With debug checks on: cu_seqlens and the gates, checked on the device
// before any other launch (the call then waits for the check).
gdr_status chunk_contract(const ChunkArgs& a, hipStream_t st) {
  if (!debug_enabled()) return GDR_OK;
  uint32_t broken = 0u;
  return debug_check(a.cu_seqlens, a.N, a.T, a.g, static_cast<int64_t>(a.T) * a.Nv, st, &broken);
}

gdr_status dispatch_chunk(const ChunkArgs& a, hipStream_t st, Recorder& rec) {
  if (a.dtype == GDR_BF16) return run_chunk<__bf16>(a, st, rec);
  return run_chunk<float>(a, st, rec);
}

}  // namespace

extern "C" size_t gdr_chunk_fwd_workspace_size(int32_t T, int32_t N, int32_t Nqk, int32_t Nv,
                                               int32_t D, gdr_dtype dtype) {
  if (T < 0 || N < 1 || Nqk < 1 || Nv < 1 || Nv > kMaxNv || Nv % Nqk != 0 || D != 128) return 0;
  if (dtype != GDR_F32 && dtype != GDR_BF16) return 0;
  if (static_cast<int64_t>(T) * Nv > (int64_t(1) << 40)) return 0;
  // enough for either chunk length (64-token chunks need more table slots)
  const int64_t a = plan_workspace(T, N, Nqk, Nv, dtype, 0, 128).total;
  const int64_t b = plan_workspace(T, N, Nqk, Nv, dtype, 0, 64).total;
  return static_cast<size_t>(a > b ? a : b);
}

extern "C" gdr_status gdr_chunk_fwd(const void* q, const void* k, const void* v, const float* g,
                                    const float* beta, const float* state_in,
                                    const int32_t* cu_seqlens, int32_t N, int32_t T, int32_t Nqk,
                                    int32_t Nv, int32_t D, gdr_dtype dtype, float scale,
                                    uint32_t flags, void* out, float* state_out, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  ChunkArgs a{q, k, v, g, beta, state_in, cu_seqlens, N, T, Nqk, Nv, D, dtype, scale, flags,
              out, state_out, workspace, workspace_bytes};
  gdr_status s = validate_chunk(a);
  if (s != GDR_OK) return s;
  s = chunk_contract(a, static_cast<hipStream_t>(stream));
  if (s != GDR_OK) return s;
  Recorder none;
  return dispatch_chunk(a, static_cast<hipStream_t>(stream), none);
}

extern "C" gdr_status gdr_chunk_fwd_timed(const void* q, const void* k, const void* v,
                                          const float* g, const float* beta,
                                          const float* state_in, const int32_t* cu_seqlens,
                                          int32_t N, int32_t T, int32_t Nqk, int32_t Nv, int32_t D,
                                          gdr_dtype dtype, float scale, uint32_t flags, void* out,
                                          float* state_out, void* workspace,
                                          size_t workspace_bytes, void* stream, float* kernel_ms,
                                          int32_t* kernel_kind, int32_t max_kernels, int32_t* n,
                                          float* span_ms) {
  ChunkArgs a{q, k, v, g, beta, state_in, cu_seqlens, N, T, Nqk, Nv, D, dtype, scale, flags,
              out, state_out, workspace, workspace_bytes};
  gdr_status s = validate_chunk(a);
  if (s != GDR_OK) return s;
  if (!kernel_ms || !kernel_kind || !n || max_kernels < 0) return GDR_ERR_INVALID_ARGUMENT;
  s = chunk_contract(a, static_cast<hipStream_t>(stream));
  if (s != GDR_OK) return s;
  const int32_t need = launches_needed(a, plan_workspace(T, N, Nqk, Nv, dtype, 0, chunk_len(flags)));
  // more launches than the caller's arrays hold: the span alone is timed
  const bool span_only = need > max_kernels;
  hipStream_t st = static_cast<hipStream_t>(stream);
  EventPairs pairs;
  if (!pairs.create(span_only ? 1 : need)) return GDR_ERR_HIP;
  Recorder rec;
  rec.ev = pairs.ev.data();
  rec.kind = kernel_kind;
  rec.cap = need;
  rec.span_only = span_only;
  rec.total = need;
  s = dispatch_chunk(a, st, rec);
  if (s != GDR_OK) return s;
  if (rec.n == 0) {
    // nothing was launched (T = 0 and no state to copy)
    *n = 0;
    if (span_ms) *span_ms = 0.0f;
    return GDR_OK;
  }
  const hipEvent_t first = pairs.ev[0];
  const hipEvent_t last = span_only ? pairs.ev[1] : pairs.ev[2 * rec.n - 1];
  if (hipEventSynchronize(last) != hipSuccess) s = GDR_ERR_HIP;
  if (s == GDR_OK) {
    const int32_t timed = span_only ? 0 : rec.n;
    for (int32_t i = 0; i < timed; ++i)
      if (hipEventElapsedTime(&kernel_ms[i], pairs.ev[2 * i], pairs.ev[2 * i + 1]) != hipSuccess)
        s = GDR_ERR_HIP;
    if (span_ms && hipEventElapsedTime(span_ms, first, last) != hipSuccess) s = GDR_ERR_HIP;
    *n = timed;
  }
  return s;
}

// ---------------------------------------------------------------------------
// gdr_chunk_fwd_no_alloc: gdr_chunk_fwd with its workspace in a fixed
// device-resident array instead of a caller buffer, for callers that cannot
// allocate.  Each GPU the library runs on holds its own copy of the array
// until the process ends.  Its address on a device is looked up once, with
// that device current (hipGetSymbolAddress; the array's name in host code is
// only a stand-in, never a device address), and kept per device.
// ---------------------------------------------------------------------------
namespace {

constexpr int64_t kScratchBytes = int64_t(64) << 20;
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex scratch_mu;
void* scratch_dev[kMaxDevices] = {};

gdr_status scratch_ptr(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return GDR_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return GDR_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_dev[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return GDR_ERR_HIP;
    scratch_dev[dev] = p;
  }
  *out = scratch_dev[dev];
  return GDR_OK;
}

}  // namespace

extern "C" size_t gdr_chunk_fwd_no_alloc_scratch_bytes(void) {
  return static_cast<size_t>(kScratchBytes);
}

extern "C" gdr_status gdr_chunk_fwd_no_alloc(const void* q, const void* k, const void* v,
                                             const float* g, const float* beta,
                                             const float* state_in, const int32_t* cu_seqlens,
                                             int32_t N, int32_t T, int32_t Nqk, int32_t Nv,
                                             int32_t D, gdr_dtype dtype, float scale,
                                             uint32_t flags, void* out, float* state_out,
                                             void* stream) {
  // every check that needs no workspace first, then the sizes against the
  // fixed scratch: a call that cannot fit is refused before any HIP call
  const ChunkArgs pre{q, k, v, g, beta, state_in, cu_seqlens, N, T, Nqk, Nv, D, dtype, scale,
                      flags, out, state_out, nullptr, 0, true, 0};
  gdr_status s = validate_chunk(pre);
  if (s != GDR_OK) return s;
  if (plan_workspace(T, N, Nqk, Nv, dtype, kScratchBytes, chunk_len(flags)).total < 0)
    return GDR_ERR_WORKSPACE_TOO_SMALL;
  void* ws = nullptr;
  const gdr_status p = scratch_ptr(&ws);
  if (p != GDR_OK) return p;
  ChunkArgs a{q, k, v, g, beta, state_in, cu_seqlens, N, T, Nqk, Nv, D, dtype, scale, flags,
              out, state_out, ws, static_cast<size_t>(kScratchBytes), false, kScratchBytes};
  s = validate_chunk(a);
  if (s != GDR_OK) return s;
  s = chunk_contract(a, static_cast<hipStream_t>(stream));
  if (s != GDR_OK) return s;
  Recorder none;
  return dispatch_chunk(a, static_cast<hipStream_t>(stream), none);
}

namespace {

template <typename St>
void step_as(const StepArgs& a, int norm, hipStream_t st, LaunchEvents ev) {
  const St* sin = static_cast<const St*>(a.state_in);
  St* sout = static_cast<St*>(a.state_out);
  if (a.dtype == GDR_BF16)
    launch_decode<__bf16, St>(static_cast<const __bf16*>(a.q), static_cast<const __bf16*>(a.k),
                              static_cast<const __bf16*>(a.v), a.g, a.beta, sin, sout, a.N, a.Nqk,
                              a.Nv, a.scale, norm, static_cast<__bf16*>(a.out), st, ev,
                              static_cast<const __bf16*>(a.z), static_cast<const __bf16*>(a.nw),
                              a.norm_eps);
  else
    launch_decode<float, St>(static_cast<const float*>(a.q), static_cast<const float*>(a.k),
                             static_cast<const float*>(a.v), a.g, a.beta, sin, sout, a.N, a.Nqk,
                             a.Nv, a.scale, norm, static_cast<float*>(a.out), st, ev,
                             static_cast<const float*>(a.z), static_cast<const float*>(a.nw),
                             a.norm_eps);
}

gdr_status run_step(const StepArgs& a, hipStream_t st, LaunchEvents ev) {
  const int norm = (a.flags & GDR_FLAG_QK_L2NORM) ? 1 : 0;
  if (a.state_bf16) step_as<__bf16>(a, norm, st, ev);
  else step_as<float>(a, norm, st, ev);
  return hipGetLastError() == hipSuccess ? GDR_OK : GDR_ERR_HIP;
}

// Validation, then the launch, timed when kernel_ms is not NULL (the call
// then waits for the kernel's end event).
gdr_status step_entry(const StepArgs& a, hipStream_t st, float* kernel_ms) {
  gdr_status s = validate_step(a);
  if (s != GDR_OK) return s;
  if (kernel_ms) *kernel_ms = 0.0f;
  if (a.N == 0) return GDR_OK;
  if (debug_enabled()) {
    uint32_t broken = 0u;
    s = debug_check(nullptr, a.N, 0, a.g, static_cast<int64_t>(a.N) * a.Nv, st, &broken);
    if (s != GDR_OK) return s;
  }
  if (!kernel_ms) return run_step(a, st, LaunchEvents{});
  EventPairs pairs;
  if (!pairs.create(1)) return GDR_ERR_HIP;
  s = run_step(a, st, LaunchEvents{pairs.ev[0], pairs.ev[1]});
  if (s == GDR_OK && (hipEventSynchronize(pairs.ev[1]) != hipSuccess ||
                      hipEventElapsedTime(kernel_ms, pairs.ev[0], pairs.ev[1]) != hipSuccess))
    s = GDR_ERR_HIP;
  return s;
}

}  // namespace

extern "C" gdr_status gdr_recurrent_step(const void* q, const void* k, const void* v,
                                         const float* g, const float* beta, const float* state_in,
                                         float* state_out, int32_t N, int32_t Nqk, int32_t Nv,
                                         int32_t D, gdr_dtype dtype, float scale, uint32_t flags,
                                         void* out, void* stream) {
  StepArgs a{q, k, v, g, beta, state_in, state_out, N, Nqk, Nv, D, dtype, scale, flags, out, false};
  return step_entry(a, static_cast<hipStream_t>(stream), nullptr);
}

extern "C" gdr_status gdr_recurrent_step_timed(const void* q, const void* k, const void* v,
                                               const float* g, const float* beta,
                                               const float* state_in, float* state_out, int32_t N,
                                               int32_t Nqk, int32_t Nv, int32_t D,
                                               gdr_dtype dtype, float scale, uint32_t flags,
                                               void* out, void* stream, float* kernel_ms) {
  if (!kernel_ms) return GDR_ERR_INVALID_ARGUMENT;
  StepArgs a{q, k, v, g, beta, state_in, state_out, N, Nqk, Nv, D, dtype, scale, flags, out, false};
  return step_entry(a, static_cast<hipStream_t>(stream), kernel_ms);
}

extern "C" gdr_status gdr_recurrent_step_bf16_state(const void* q, const void* k, const void* v,
                                                    const float* g, const float* beta,
                                                    const uint16_t* state_in, uint16_t* state_out,
                                                    int32_t N, int32_t Nqk, int32_t Nv, int32_t D,
                                                    gdr_dtype dtype, float scale, uint32_t flags,
                                                    void* out, void* stream, float* kernel_ms) {
  StepArgs a{q, k, v, g, beta, state_in, state_out, N, Nqk, Nv, D, dtype, scale, flags, out, true};
  return step_entry(a, static_cast<hipStream_t>(stream), kernel_ms);
}

extern "C" gdr_status gdr_recurrent_step_gated(const void* q, const void* k, const void* v,
                                               const float* g, const float* beta,
                                               const float* state_in, float* state_out, int32_t N,
                                               int32_t Nqk, int32_t Nv, int32_t D,
                                               gdr_dtype dtype, float scale, uint32_t flags,
                                               const void* z, const void* weight, float norm_eps,
                                               void* out, void* stream, float* kernel_ms) {
  if (N > 0 && !z) return GDR_ERR_INVALID_ARGUMENT;
  StepArgs a{q, k, v, g, beta, state_in, state_out, N, Nqk, Nv, D, dtype, scale, flags, out, false,
             z, weight, norm_eps};
  return step_entry(a, static_cast<hipStream_t>(stream), kernel_ms);
}

extern "C" gdr_status gdr_gated_rmsnorm(const void* x, const void* z, const void* weight,
                                        int64_t rows, int32_t D, gdr_dtype dtype, float eps,
                                        void* y, void* stream, float* kernel_ms) {
  const NormArgs a{x, z, weight, rows, D, dtype, eps, y};
  gdr_status s = validate_norm(a);
  if (s != GDR_OK) return s;
  if (kernel_ms) *kernel_ms = 0.0f;
  if (rows == 0) return GDR_OK;
  EventPairs pairs;
  LaunchEvents ev{};
  if (kernel_ms) {
    if (!pairs.create(1)) return GDR_ERR_HIP;
    ev = LaunchEvents{pairs.ev[0], pairs.ev[1]};
  }
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (dtype == GDR_BF16)
    launch_gated_rmsnorm<__bf16>(static_cast<const __bf16*>(x), static_cast<const __bf16*>(z),
                                 static_cast<const __bf16*>(weight), rows, eps,
                                 static_cast<__bf16*>(y), st, ev);
  else
    launch_gated_rmsnorm<float>(static_cast<const float*>(x), static_cast<const float*>(z),
                                static_cast<const float*>(weight), rows, eps,
                                static_cast<float*>(y), st, ev);
  if (hipGetLastError() != hipSuccess) return GDR_ERR_HIP;
  if (kernel_ms && (hipEventSynchronize(pairs.ev[1]) != hipSuccess ||
                    hipEventElapsedTime(kernel_ms, pairs.ev[0], pairs.ev[1]) != hipSuccess))
    return GDR_ERR_HIP;
  return GDR_OK;
}

extern "C" gdr_status gdr_recurrent_multi(const void* q, const void* k, const void* v,
                                          const float* g, const float* beta, const float* state_in,
                                          const int32_t* cu_seqlens, int32_t N, int32_t T,
                                          int32_t Nqk, int32_t Nv, int32_t D, gdr_dtype dtype,
                                          float scale, uint32_t flags, void* out,
                                          float* state_out, void* stream, float* kernel_ms) {
  ChunkArgs a{q, k, v, g, beta, state_in, cu_seqlens, N, T, Nqk, Nv, D, dtype, scale, flags,
              out, state_out, nullptr, 0, true};
  gdr_status s = validate_chunk(a);
  if (s != GDR_OK) return s;
  if (kernel_ms) *kernel_ms = 0.0f;
  s = chunk_contract(a, static_cast<hipStream_t>(stream));
  if (s != GDR_OK) return s;
  if (T == 0 && !state_out) return GDR_OK;   // nothing to write
  EventPairs pairs;
  LaunchEvents ev{};
  if (kernel_ms) {
    if (!pairs.create(1)) return GDR_ERR_HIP;
    ev = LaunchEvents{pairs.ev[0], pairs.ev[1]};
  }
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const int norm = (flags & GDR_FLAG_QK_L2NORM) ? 1 : 0;
  if (dtype == GDR_BF16)
    launch_multi<__bf16>(static_cast<const __bf16*>(q), static_cast<const __bf16*>(k),
                         static_cast<const __bf16*>(v), g, beta, state_in, cu_seqlens, N, T,
                         state_out, Nqk, Nv, scale, norm, static_cast<__bf16*>(out), st, ev);
  else
    launch_multi<float>(static_cast<const float*>(q), static_cast<const float*>(k),
                        static_cast<const float*>(v), g, beta, state_in, cu_seqlens, N, T,
                        state_out, Nqk, Nv, scale, norm, static_cast<float*>(out), st, ev);
  if (hipGetLastError() != hipSuccess) return GDR_ERR_HIP;
  if (kernel_ms && (hipEventSynchronize(pairs.ev[1]) != hipSuccess ||
                    hipEventElapsedTime(kernel_ms, pairs.ev[0], pairs.ev[1]) != hipSuccess))
    return GDR_ERR_HIP;
  return GDR_OK;
}

extern "C" gdr_status gdr_recurrent_step_conv(
    const void* mixed_qkv, const void* conv_state_in, void* conv_state_out,
    const void* conv_weight, const void* conv_bias, int32_t conv_k, const float* a,
    const float* b, const float* A_log, const float* dt_bias, const float* state_in,
    float* state_out, int32_t N, int32_t Nqk, int32_t Nv, int32_t D, gdr_dtype dtype, float scale,
    uint32_t flags, void* out, void* stream, float* kernel_ms) {
  ConvStepArgs c{mixed_qkv, conv_state_in, conv_state_out, conv_weight, conv_bias, conv_k, a, b,
                 A_log, dt_bias, state_in, state_out, N, Nqk, Nv, D, dtype, scale, flags, out};
  const gdr_status s = validate_conv_step(c);
  if (s != GDR_OK) return s;
  if (kernel_ms) *kernel_ms = 0.0f;
  if (N == 0) return GDR_OK;
  EventPairs pairs;
  LaunchEvents ev{};
  if (kernel_ms) {
    if (!pairs.create(1)) return GDR_ERR_HIP;
    ev = LaunchEvents{pairs.ev[0], pairs.ev[1]};
  }
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const int norm = (flags & GDR_FLAG_QK_L2NORM) ? 1 : 0;
  if (dtype == GDR_BF16)
    launch_decode_conv<__bf16>(static_cast<const __bf16*>(mixed_qkv),
                               static_cast<const __bf16*>(conv_state_in),
                               static_cast<__bf16*>(conv_state_out),
                               static_cast<const __bf16*>(conv_weight),
                               static_cast<const __bf16*>(conv_bias), a, b, A_log, dt_bias,
                               state_in, state_out, N, Nqk, Nv, scale, norm,
                               static_cast<__bf16*>(out), st, ev);
  else
    launch_decode_conv<float>(static_cast<const float*>(mixed_qkv),
                              static_cast<const float*>(conv_state_in),
                              static_cast<float*>(conv_state_out),
                              static_cast<const float*>(conv_weight),
                              static_cast<const float*>(conv_bias), a, b, A_log, dt_bias, state_in,
                              state_out, N, Nqk, Nv, scale, norm, static_cast<float*>(out), st, ev);
  if (hipGetLastError() != hipSuccess) return GDR_ERR_HIP;
  if (kernel_ms && (hipEventSynchronize(pairs.ev[1]) != hipSuccess ||
                    hipEventElapsedTime(kernel_ms, pairs.ev[0], pairs.ev[1]) != hipSuccess))
    return GDR_ERR_HIP;
  return GDR_OK;
}

extern "C" gdr_status gdr_conv_prefill(const void* mixed_qkv, const void* conv_state_in,
                                       void* conv_state_out, const void* conv_weight,
                                       const void* conv_bias, int32_t conv_k, const float* a,
                                       const float* b, const float* A_log, const float* dt_bias,
                                       const int32_t* cu_seqlens, int32_t N, int32_t T,
                                       int32_t Nqk, int32_t Nv, int32_t D, gdr_dtype dtype,
                                       void* q, void* k, void* v, float* g, float* beta,
                                       void* stream, float* kernel_ms) {
  ConvPrefillCheck c{mixed_qkv, conv_state_in, conv_state_out, conv_weight, conv_bias, conv_k,
                     a, b, A_log, dt_bias, cu_seqlens, N, T, Nqk, Nv, D, dtype, q, k, v, g, beta};
  gdr_status s = validate_conv_prefill(c);
  if (s != GDR_OK) return s;
  if (kernel_ms) *kernel_ms = 0.0f;
  if (T == 0 && !conv_state_out) return GDR_OK;
  if (debug_enabled()) {
    uint32_t broken = 0u;
    s = debug_check(cu_seqlens, N, T, nullptr, 0, static_cast<hipStream_t>(stream), &broken);
    if (s != GDR_OK) return s;
  }
  EventPairs pairs;
  LaunchEvents e0{}, e1{};
  if (kernel_ms) {
    // one pair spans both launches: start of the first, end of the last
    if (!pairs.create(1)) return GDR_ERR_HIP;
    if (T > 0) e0.start = pairs.ev[0];
    else e1.start = pairs.ev[0];
    if (conv_state_out) e1.stop = pairs.ev[1];
    else e0.stop = pairs.ev[1];
  }
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const int32_t C = (2 * Nqk + Nv) * 128;
  if (dtype == GDR_BF16) {
    ConvPrefillArgs<__bf16> p{static_cast<const __bf16*>(mixed_qkv),
                              static_cast<const __bf16*>(conv_state_in),
                              static_cast<__bf16*>(conv_state_out),
                              static_cast<const __bf16*>(conv_weight),
                              static_cast<const __bf16*>(conv_bias), a, b, A_log, dt_bias,
                              cu_seqlens, N, T, Nqk, Nv, C, static_cast<__bf16*>(q),
                              static_cast<__bf16*>(k), static_cast<__bf16*>(v), g, beta};
    launch_conv_prefill<__bf16>(p, st, e0, e1);
  } else {
    ConvPrefillArgs<float> p{static_cast<const float*>(mixed_qkv),
                             static_cast<const float*>(conv_state_in),
                             static_cast<float*>(conv_state_out),
                             static_cast<const float*>(conv_weight),
                             static_cast<const float*>(conv_bias), a, b, A_log, dt_bias,
                             cu_seqlens, N, T, Nqk, Nv, C, static_cast<float*>(q),
                             static_cast<float*>(k), static_cast<float*>(v), g, beta};
    launch_conv_prefill<float>(p, st, e0, e1);
  }
  if (hipGetLastError() != hipSuccess) return GDR_ERR_HIP;
  if (kernel_ms && (hipEventSynchronize(pairs.ev[1]) != hipSuccess ||
                    hipEventElapsedTime(kernel_ms, pairs.ev[0], pairs.ev[1]) != hipSuccess))
    return GDR_ERR_HIP;
  return GDR_OK;
}

extern "C" const char* gdr_status_string(gdr_status s) {
  switch (s) {
    case GDR_OK: return "ok";
    case GDR_ERR_INVALID_ARGUMENT: return "invalid argument";
    case GDR_ERR_UNSUPPORTED: return "unsupported size, dtype or flag";
    case GDR_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case GDR_ERR_HIP: return "HIP runtime error";
    case GDR_ERR_CONTRACT: return "device values break the contract (debug checks)";
  }
  return "unknown status";
}

extern "C" const char* gdr_version(void) { return "libgdr 0.2"; }
