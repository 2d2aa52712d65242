// gdr_api.hip -- the extern "C" entry points of libgdr (declared in
// include/gdr.h): argument validation, workspace carving and kernel launches
// on the caller's stream.  No allocation, no synchronisation.
#include <hip/hip_runtime.h>

#include "../../include/gdr.h"
#include "gdr_internal.h"
#include "gdr_kernels.h"

using namespace gdr;

namespace {

// Optional per-launch timing: launch i gets the event pair ev[2i], ev[2i+1],
// which the runtime records at that kernel's start and end.  With no event
// array every launch is untimed.
struct Recorder {
  hipEvent_t* ev = nullptr;
  int32_t* kind = nullptr;
  int32_t cap = 0;
  int32_t n = 0;
  LaunchEvents next(int32_t k) {
    LaunchEvents e;
    if (ev && n < cap) {
      kind[n] = k;
      e.start = ev[2 * n];
      e.stop = ev[2 * n + 1];
    }
    ++n;
    return e;
  }
};

// Event pairs for up to kMaxTimed timed launches, destroyed with the object.
constexpr int32_t kMaxTimed = 64;
struct EventPairs {
  hipEvent_t ev[2 * kMaxTimed];
  int32_t made = 0;
  bool create(int32_t launches) {
    if (launches < 0 || launches > kMaxTimed) return false;
    for (; made < 2 * launches; ++made)
      if (hipEventCreate(&ev[made]) != hipSuccess) return false;
    return true;
  }
  ~EventPairs() {
    for (int32_t i = 0; i < made; ++i) (void)hipEventDestroy(ev[i]);
  }
};

// A single sequence needs no chunk table (Chunks derives its slots from
// cu_seqlens directly), so its call is two launches per segment.
int32_t launches_needed(const Workspace& w, int64_t N) {
  const int64_t segs = (w.nslots + w.seg_slots - 1) / w.seg_slots;
  return static_cast<int32_t>((N > 1 ? 1 : 0) + 2 * segs);
}

template <typename T>
gdr_status run_chunk(const ChunkArgs& a, hipStream_t st, Recorder& rec) {
  const Workspace w = plan_workspace(a.T, a.N, a.Nqk, a.Nv, a.dtype);
  char* ws = static_cast<char*>(a.workspace);
  int4* table = reinterpret_cast<int4*>(ws + w.table);
  int32_t* choff = reinterpret_cast<int32_t*>(ws + w.choff);
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

  Chunks chunks{nullptr, nullptr, a.cu_seqlens, a.T};
  if (a.N > 1) {
    launch_table(a.cu_seqlens, a.N, a.T, nslots, table, choff, st, rec.next(GDR_STAGE_TABLE));
    chunks.table = table;
    chunks.choff = choff;
  }
  for (int64_t s0 = 0; s0 < w.nslots; s0 += w.seg_slots) {
    const int32_t nseg = static_cast<int32_t>(w.nslots - s0 < w.seg_slots ? w.nslots - s0 : w.seg_slots);
    launch_intra<T>(q, k, v, a.g, a.beta, chunks, a.Nqk, a.Nv, static_cast<int32_t>(s0), nseg,
                    a.scale, norm, inter, gam, st, rec.next(GDR_STAGE_INTRA));
    launch_inter<T>(inter, chunks, gam, a.state_in, carry, a.state_out, a.N, a.Nv,
                    static_cast<int32_t>(s0), nseg, s0 == 0, out, discard, st,
                    rec.next(GDR_STAGE_INTER));
  }
  return hipGetLastError() == hipSuccess ? GDR_OK : GDR_ERR_HIP;
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
  return static_cast<size_t>(plan_workspace(T, N, Nqk, Nv, dtype).total);
}

extern "C" gdr_status gdr_chunk_fwd(const void* q, const void* k, const void* v, const float* g,
                                    const float* beta, const float* state_in,
                                    const int32_t* cu_seqlens, int32_t N, int32_t T, int32_t Nqk,
                                    int32_t Nv, int32_t D, gdr_dtype dtype, float scale,
                                    uint32_t flags, void* out, float* state_out, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  ChunkArgs a{q, k, v, g, beta, state_in, cu_seqlens, N, T, Nqk, Nv, D, dtype, scale, flags,
              out, state_out, workspace, workspace_bytes};
  const gdr_status s = validate_chunk(a);
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
  const int32_t need = launches_needed(plan_workspace(T, N, Nqk, Nv, dtype), N);
  if (need > max_kernels) return GDR_ERR_INVALID_ARGUMENT;
  hipStream_t st = static_cast<hipStream_t>(stream);
  EventPairs pairs;
  if (!pairs.create(need)) return need > kMaxTimed ? GDR_ERR_INVALID_ARGUMENT : GDR_ERR_HIP;
  Recorder rec;
  rec.ev = pairs.ev;
  rec.kind = kernel_kind;
  rec.cap = need;
  s = dispatch_chunk(a, st, rec);
  if (s == GDR_OK && hipEventSynchronize(pairs.ev[2 * rec.n - 1]) != hipSuccess) s = GDR_ERR_HIP;
  if (s == GDR_OK) {
    for (int32_t i = 0; i < rec.n; ++i)
      if (hipEventElapsedTime(&kernel_ms[i], pairs.ev[2 * i], pairs.ev[2 * i + 1]) != hipSuccess)
        s = GDR_ERR_HIP;
    if (span_ms && hipEventElapsedTime(span_ms, pairs.ev[0], pairs.ev[2 * rec.n - 1]) != hipSuccess)
      s = GDR_ERR_HIP;
    *n = rec.n;
  }
  return s;
}

namespace {

template <typename St>
void step_as(const StepArgs& a, int norm, hipStream_t st, LaunchEvents ev) {
  const St* sin = static_cast<const St*>(a.state_in);
  St* sout = static_cast<St*>(a.state_out);
  if (a.dtype == GDR_BF16)
    launch_decode<__bf16, St>(static_cast<const __bf16*>(a.q), static_cast<const __bf16*>(a.k),
                              static_cast<const __bf16*>(a.v), a.g, a.beta, sin, sout, a.N, a.Nqk,
                              a.Nv, a.scale, norm, static_cast<__bf16*>(a.out), st, ev);
  else
    launch_decode<float, St>(static_cast<const float*>(a.q), static_cast<const float*>(a.k),
                             static_cast<const float*>(a.v), a.g, a.beta, sin, sout, a.N, a.Nqk,
                             a.Nv, a.scale, norm, static_cast<float*>(a.out), st, ev);
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
  const gdr_status s = validate_conv_prefill(c);
  if (s != GDR_OK) return s;
  if (kernel_ms) *kernel_ms = 0.0f;
  if (T == 0 && !conv_state_out) return GDR_OK;
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
  }
  return "unknown status";
}

extern "C" const char* gdr_version(void) { return "libgdr 0.2"; }
