/*
 * gdr.h -- libgdr: the gated delta rule of Gated DeltaNet on MI355X (gfx950).
 *
 * The rule (Qwen3-Next blog post "Code-Qwen3-Next", section 5; Ascend PyPTO
 * "Qwen3Next" operator page, math formulas).  Per sequence and value head h,
 * with query/key head j = h / (Nv / Nqk) (grouped heads, blog section 4), a
 * state S in R^{Dv x Dk} (S[i][c]: i = value index, c = key index) evolves
 * token by token:
 *
 *   kh = k_t / sqrt(|k_t|^2 + 1e-6),   qh = scale * q_t / sqrt(|q_t|^2 + 1e-6)
 *   S  = exp(g_t) S + beta_t (v_t - exp(g_t) S kh) kh^T
 *   o_t = S qh
 *
 * Two entry points compute it:
 *   gdr_chunk_fwd      -- prefill: packed variable-length sequences, in the
 *                         chunkwise form with chunk length 128 (blog post
 *                         section 5(1); operator page "chunk_gated_delta_rule");
 *   gdr_recurrent_step -- decode: one token per sequence (blog post 5(2)).
 * and two variants of the token loop:
 *   gdr_recurrent_step_bf16_state -- decode with the state stored in bf16;
 *   gdr_recurrent_multi           -- a few tokens per sequence, token by token;
 *   gdr_recurrent_step_conv       -- decode with the conv update and gates fused
 *                                    in front;
 * and the conv/gate prologue of the chunkwise path:
 *   gdr_conv_prefill              -- q, k, v, g, beta from projected channels;
 * and the gated RMSNorm after the rule (blog post section 6):
 *   gdr_gated_rmsnorm             -- on any output rows (e.g. gdr_chunk_fwd's);
 *   gdr_recurrent_step_gated      -- decode with the norm fused behind it.
 *
 * Conventions shared by all calls:
 *   - All tensor pointers are DEVICE pointers, caller-owned, contiguous,
 *     row-major, 16-byte aligned.  The library allocates no memory and keeps
 *     no pointer after a call returns.
 *   - Calls only enqueue kernels on `stream` and return; results are valid
 *     once the caller synchronises that stream.  The library keeps no mutable
 *     global state, so calls on different streams may run concurrently as long
 *     as their buffers do not overlap.
 *   - D (= Dk = Dv) must be 128; Nv must be a multiple of Nqk (operator page,
 *     parameter constraints) and at most 16384 (GDR_ERR_UNSUPPORTED beyond,
 *     so that a chunk's rows span less than 2 GiB of any input and every
 *     launch stays within 2^32 work-items).
 *   - `dtype` is the storage type of q, k, v and out.  g, beta and the states
 *     are always float32.  Arithmetic accumulates in float32; bf16 inputs are
 *     multiplied on bf16 matrix cores, f32 inputs on f32 matrix cores.
 *   - Errors are reported by the returned status; nothing aborts or prints.
 *     Argument validation happens before any launch, and on a validation
 *     error no output is touched.  Values that live only on the device
 *     (cu_seqlens starting at 0, non-decreasing, with cu[N] = T; every g
 *     finite and <= 0) are the caller's contract and are not checked by
 *     default.  With debug checks on (GDR_DEBUG set to anything but "" or
 *     "0" in the environment when the library first looks, or
 *     gdr_set_debug(1)), every call that reads them first runs one checking
 *     kernel and waits for it, and returns GDR_ERR_CONTRACT, with no output
 *     touched, if a value breaks the contract (gdr_debug_broken says which).
 *     Checked calls block the host, so they cannot be captured in a graph.
 */
#ifndef GDR_H
#define GDR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { GDR_F32 = 0, GDR_BF16 = 1 } gdr_dtype;

typedef enum {
    GDR_OK = 0,
    GDR_ERR_INVALID_ARGUMENT = -1,   /* bad size, null pointer, misalignment, ... */
    GDR_ERR_UNSUPPORTED = -2,        /* D != 128, Nv > 16384, unknown dtype or flag */
    GDR_ERR_WORKSPACE_TOO_SMALL = -3,
    GDR_ERR_HIP = -4,                /* a HIP runtime call or launch failed */
    GDR_ERR_CONTRACT = -5            /* debug checks on: a device value breaks the contract */
} gdr_status;

/* Normalise q and k by their L2 norm inside the call (the blog's
 * use_qk_l2norm_in_kernel).  Without the flag, q and k are used as given
 * (then scale still multiplies q). */
#define GDR_FLAG_QK_L2NORM 1u

/* Chunkwise calls only: chunks of 64 tokens instead of 128 (the Blog's
 * torch_chunk_gated_delta_rule default chunk_size=64).  The chunkwise form is
 * exact for any chunk length, so the results equal those with 128 up to
 * rounding; the kernels are the same (a 64-token chunk is a 128-row tile with
 * its last 64 rows absent), so it costs about twice the time.  The other
 * calls ignore it. */
#define GDR_FLAG_CHUNK64 2u

/* The default chunk length of the chunkwise form (operator page: 128). */
#define GDR_CHUNK 128

/*
 * Bytes of device workspace gdr_chunk_fwd needs for these sizes.
 * Returns 0 for invalid sizes.  The workspace is scratch: its contents on
 * entry do not matter and are undefined on return.
 */
size_t gdr_chunk_fwd_workspace_size(int32_t T, int32_t N, int32_t Nqk, int32_t Nv,
                                    int32_t D, gdr_dtype dtype);

/*
 * Chunkwise forward over N packed sequences (prefill).
 *
 * q, k       [T, Nqk, D]  dtype
 * v          [T, Nv, D]   dtype
 * g, beta    [T, Nv]      float32; g is the natural-log decay (finite, <= 0),
 *                         beta the write strength
 * state_in   [N, Nv, D, D] float32 initial states (row = value index), or NULL
 *                         for zeros
 * cu_seqlens [N + 1]      int32, device: cu[0] = 0 <= cu[1] <= ... <= cu[N] = T;
 *                         sequence b owns tokens [cu[b], cu[b+1]).  Chunks of
 *                         128 (or 64) tokens restart at every sequence start,
 *                         so a sequence boundary may fall anywhere.
 * scale      multiplies the normalised query (the blog uses 1/sqrt(D))
 * flags      any of GDR_FLAG_QK_L2NORM, GDR_FLAG_CHUNK64
 * out        [T, Nv, D]   dtype, written for every token; must not alias inputs
 * state_out  [N, Nv, D, D] float32 final states, or NULL.  May equal state_in
 *                         (in-place update); must not partially overlap it.
 * workspace  device scratch of at least gdr_chunk_fwd_workspace_size() bytes,
 *            256-byte aligned.
 * stream     hipStream_t (passed as void*; NULL = the default stream)
 *
 * A zero-length sequence leaves its state unchanged (state_out = state_in).
 * T = 0 is allowed.  Requires N >= 1.
 */
gdr_status gdr_chunk_fwd(const void* q, const void* k, const void* v,
                         const float* g, const float* beta,
                         const float* state_in, const int32_t* cu_seqlens,
                         int32_t N, int32_t T, int32_t Nqk, int32_t Nv, int32_t D,
                         gdr_dtype dtype, float scale, uint32_t flags,
                         void* out, float* state_out,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * One decode step: one token for each of N independent sequences.
 *
 * q, k       [N, Nqk, D]  dtype
 * v          [N, Nv, D]   dtype
 * g, beta    [N, Nv]      float32
 * state_in   [N, Nv, D, D] float32 (required)
 * state_out  [N, Nv, D, D] float32 (required); may equal state_in for an
 *            in-place update
 * out        [N, Nv, D]   dtype
 * Requires N >= 0 (N = 0 does nothing) and N * Nv < 2^24 (one workgroup per
 * (sequence, head); GDR_ERR_INVALID_ARGUMENT beyond), which holds for every
 * batch whose states fit in memory.  The same bound applies to the decode
 * variants below.
 */
gdr_status gdr_recurrent_step(const void* q, const void* k, const void* v,
                              const float* g, const float* beta,
                              const float* state_in, float* state_out,
                              int32_t N, int32_t Nqk, int32_t Nv, int32_t D,
                              gdr_dtype dtype, float scale, uint32_t flags,
                              void* out, void* stream);

/*
 * gdr_chunk_fwd without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The same computation, arguments and
 * results as gdr_chunk_fwd, except that the scratch lives in a fixed array of
 * gdr_chunk_fwd_no_alloc_scratch_bytes() bytes (64 MiB) inside the library:
 * every GPU the library runs on holds one copy of it until the process ends,
 * located on the first call made with that device current.  The call
 * allocates nothing; it only enqueues kernels on `stream`.
 *
 * Sizes whose scratch does not fit return GDR_ERR_WORKSPACE_TOO_SMALL before
 * any HIP call.  The fit depends on N * Nv (a 64 KiB carried state per
 * sequence and head when state_out is NULL) and on Nv (one chunk of
 * intra-chunk matrices per head); long sequences are split into more
 * segments, never refused.  All calls on one GPU share its array, so calls
 * that may overlap on one GPU (different streams, threads) race: serialise
 * them.  No part of the array needs to start at zero.
 */
gdr_status gdr_chunk_fwd_no_alloc(const void* q, const void* k, const void* v,
                                  const float* g, const float* beta,
                                  const float* state_in, const int32_t* cu_seqlens,
                                  int32_t N, int32_t T, int32_t Nqk, int32_t Nv, int32_t D,
                                  gdr_dtype dtype, float scale, uint32_t flags,
                                  void* out, float* state_out, void* stream);

/* Size in bytes of the fixed scratch array gdr_chunk_fwd_no_alloc uses. */
size_t gdr_chunk_fwd_no_alloc_scratch_bytes(void);

/*
 * Profiling variant of gdr_chunk_fwd: the same computation, plus the GPU time
 * of every kernel it launches.  Each launch gets a pair of HIP events that the
 * runtime records at that kernel's start and end (hipExtLaunchKernelGGL), so
 * a duration excludes the gaps between launches.  The call waits for the last
 * event (so, unlike gdr_chunk_fwd, it blocks the host until the work is done)
 * and writes, for launch i < *n:
 *   kernel_ms[i]   GPU time of launch i, from the kernel's start to its end;
 *   kernel_kind[i] which stage it was (GDR_STAGE_*);
 * and, if span_ms is not NULL, the time from the first kernel's start to the
 * last kernel's end (the call's GPU time, gaps between its kernels included).
 * max_kernels bounds both arrays.  A call needing more launches than that
 * still runs, but times only its span: *n is then 0 and the arrays are not
 * written.  The number of launches is 2 * ceil(slots / segment), plus 1 (the
 * chunk table) when N > 1: a handful for the configurations of the pages.
 */
#define GDR_STAGE_TABLE 0   /* chunk table from cu_seqlens, final states of empty sequences */
#define GDR_STAGE_INTRA 1   /* norms, gate cumsum, intra-chunk products; parallel over chunks */
#define GDR_STAGE_INTER 2   /* chunk-serial state pass and outputs */
gdr_status gdr_chunk_fwd_timed(const void* q, const void* k, const void* v,
                               const float* g, const float* beta,
                               const float* state_in, const int32_t* cu_seqlens,
                               int32_t N, int32_t T, int32_t Nqk, int32_t Nv, int32_t D,
                               gdr_dtype dtype, float scale, uint32_t flags,
                               void* out, float* state_out,
                               void* workspace, size_t workspace_bytes, void* stream,
                               float* kernel_ms, int32_t* kernel_kind, int32_t max_kernels,
                               int32_t* n, float* span_ms);

/*
 * Profiling variant of gdr_recurrent_step: the same computation, plus the GPU
 * time of its one kernel, from the kernel's start to its end, in *kernel_ms
 * (0 for N = 0).  Blocks the host until the step is done.  kernel_ms must not
 * be NULL (GDR_ERR_INVALID_ARGUMENT).
 */
gdr_status gdr_recurrent_step_timed(const void* q, const void* k, const void* v,
                                    const float* g, const float* beta,
                                    const float* state_in, float* state_out,
                                    int32_t N, int32_t Nqk, int32_t Nv, int32_t D,
                                    gdr_dtype dtype, float scale, uint32_t flags,
                                    void* out, void* stream, float* kernel_ms);

/*
 * One decode step with the state stored in bfloat16: a bf16 state cache, as
 * the generic "Gated DeltaNet" article's deployment advice (section 6.3)
 * names it.  The same rule as gdr_recurrent_step (blog post 5(2)) and the
 * same arguments, except:
 *
 * state_in   [N, Nv, D, D] bfloat16 bit patterns (required)
 * state_out  [N, Nv, D, D] bfloat16 bit patterns (required); may equal
 *            state_in for an in-place update, must not overlap it otherwise
 * kernel_ms  NULL, or where to write the kernel's GPU time (start to end);
 *            with a pointer the call blocks until the step is done
 *
 * The arithmetic is fp32, on the stored bf16 values.  The output comes from
 * the new state before it is rounded; the new state is rounded to the nearest
 * bf16 value (ties to even) when it is stored.  Half the state bytes of
 * gdr_recurrent_step, for the cost of that rounding at every step.  Errors
 * as for gdr_recurrent_step.
 */
gdr_status gdr_recurrent_step_bf16_state(const void* q, const void* k, const void* v,
                                         const float* g, const float* beta,
                                         const uint16_t* state_in, uint16_t* state_out,
                                         int32_t N, int32_t Nqk, int32_t Nv, int32_t D,
                                         gdr_dtype dtype, float scale, uint32_t flags,
                                         void* out, void* stream, float* kernel_ms);

/*
 * Several tokens per sequence, token by token (blog post 5(2), the token loop
 * run over each sequence): for batches of short sequences, e.g. a few tokens
 * per sequence when verifying speculative tokens, where chunks of 128 would
 * be mostly padding.  Same arguments, layouts and results as gdr_chunk_fwd
 * (packed tokens, cu_seqlens in device memory, NULL state_in = zeros, NULL
 * state_out = final state not written, state_out may equal state_in), but no
 * workspace.  One workgroup per (sequence, value head) keeps its state in
 * registers across the sequence's tokens, so the state is read and written
 * once per call.  Any sequence length works; its time grows linearly with the
 * longest sequence, so long sequences belong to gdr_chunk_fwd.
 * kernel_ms: NULL, or where to write the kernel's GPU time (the call then
 * blocks until the kernel ends).  Errors as for gdr_chunk_fwd, plus
 * GDR_ERR_INVALID_ARGUMENT when N * Nv >= 2^24.
 */
gdr_status gdr_recurrent_multi(const void* q, const void* k, const void* v,
                               const float* g, const float* beta,
                               const float* state_in, const int32_t* cu_seqlens,
                               int32_t N, int32_t T, int32_t Nqk, int32_t Nv, int32_t D,
                               gdr_dtype dtype, float scale, uint32_t flags,
                               void* out, float* state_out, void* stream, float* kernel_ms);

/*
 * One decode step with the steps in front of it fused (Qwen3-Next blog post,
 * sections 3 and 4): the token's projected q|k|v goes through the causal
 * depthwise conv update with SiLU, the gates come from a and b, then the rule
 * runs as in gdr_recurrent_step.  Per channel c (C = (2 Nqk + Nv) D channels,
 * q then k then v, each head's D consecutive):
 *   window  = conv_state_in[n][c][1..K-1], then mixed_qkv[n][c]   (oldest first)
 *   y       = SiLU(sum_i conv_weight[c][i] window[i] + conv_bias[c]), cast to dtype
 *   conv_state_out[n][c] = window
 * and per (sequence, value head):
 *   beta = sigmoid(b),  g = -exp(A_log[h]) softplus(a + dt_bias[h]).
 *
 * mixed_qkv      [N, C]     dtype
 * conv_state_in  [N, C, K]  dtype
 * conv_state_out [N, C, K]  dtype; must not overlap conv_state_in or any
 *                other buffer: the value heads of a group read the same q/k
 *                windows, so the update cannot be made in place
 * conv_weight    [C, K]     dtype;  conv_bias [C] dtype, or NULL for none
 * conv_k         K; must be 4 (Qwen3-Next's kernel size; GDR_ERR_UNSUPPORTED)
 * a, b           [N, Nv]    float32;  A_log, dt_bias [Nv] float32
 * state_in, state_out, out, scale, flags: as for gdr_recurrent_step
 *                (states float32; state_out may equal state_in)
 * kernel_ms      NULL, or where to write the kernel's GPU time (the call then
 *                blocks until the kernel ends)
 */
gdr_status gdr_recurrent_step_conv(const void* mixed_qkv, const void* conv_state_in,
                                   void* conv_state_out, const void* conv_weight,
                                   const void* conv_bias, int32_t conv_k,
                                   const float* a, const float* b, const float* A_log,
                                   const float* dt_bias, const float* state_in, float* state_out,
                                   int32_t N, int32_t Nqk, int32_t Nv, int32_t D,
                                   gdr_dtype dtype, float scale, uint32_t flags, void* out,
                                   void* stream, float* kernel_ms);

/*
 * The steps in front of gdr_chunk_fwd for packed sequences (Qwen3-Next blog
 * post, sections 3 and 4, the prefill branch): per sequence b and channel c
 * (C = (2 Nqk + Nv) D channels, q then k then v, each head's D consecutive),
 * the causal depthwise conv over the sequence's tokens with the cached window
 * conv_state_in[b][c][0..K-1] (oldest first; NULL = zeros, the blog's
 * prefill padding) in front of its first token:
 *   y[t][c] = SiLU(sum_i conv_weight[c][i] x[t - K + 1 + i][c] + conv_bias[c])
 * cast to dtype and split into q, k, v in the layouts gdr_chunk_fwd takes;
 * the gates beta = sigmoid(b), g = -exp(A_log[h]) softplus(a + dt_bias[h]);
 * and, if conv_state_out is not NULL, each sequence's new window, the last K
 * values of (cached window, tokens).
 *
 * mixed_qkv      [T, C] dtype (the projected channels of every token)
 * conv_state_in  [N, C, K] dtype, or NULL
 * conv_state_out [N, C, K] dtype, or NULL; may equal conv_state_in
 * conv_weight    [C, K] dtype;  conv_bias [C] dtype, or NULL
 * conv_k         K; must be 4 (GDR_ERR_UNSUPPORTED otherwise)
 * a, b           [T, Nv] float32;  A_log, dt_bias [Nv] float32
 * cu_seqlens     [N + 1] int32, device, as for gdr_chunk_fwd
 * q, k           [T, Nqk, D] dtype;  v [T, Nv, D] dtype;  g, beta [T, Nv] float32
 * kernel_ms      NULL, or where to write the GPU time from the first kernel's
 *                start to the last one's end (the call then blocks)
 * Outputs overlap no input and no other output (except conv_state_out ==
 * conv_state_in).  Two launches at most.
 */
gdr_status gdr_conv_prefill(const void* mixed_qkv, const void* conv_state_in,
                            void* conv_state_out, const void* conv_weight, const void* conv_bias,
                            int32_t conv_k, const float* a, const float* b, const float* A_log,
                            const float* dt_bias, const int32_t* cu_seqlens, int32_t N,
                            int32_t T, int32_t Nqk, int32_t Nv, int32_t D, gdr_dtype dtype,
                            void* q, void* k, void* v, float* g, float* beta, void* stream,
                            float* kernel_ms);

/*
 * The gated RMSNorm in front of the output projection (Qwen3-Next blog post:
 * RMSNormGated in section 1, applied to the rule's output and the output gate
 * z in section 6; the RMS form is the _norm of its Zero-Centered RMSNorm
 * section).  Per row r of D values (one token and value head):
 *   y[r][i] = x[r][i] / sqrt(mean_j x[r][j]^2 + eps) * weight[i] * SiLU(z[r][i])
 * with SiLU(t) = t * sigmoid(t).  The pages name the module but not its gate
 * function; SiLU is the library's reading (the activation the pages use for
 * the block's conv and for gating in its MLP).  The arithmetic is float32 on
 * the stored values; y is rounded to dtype (nearest even) when stored.
 *
 * x, z      [rows, D] dtype (row-major; the rule's out [T, Nv, D] is
 *           rows = T * Nv)
 * weight    [D] dtype, or NULL for ones (RMSNormGated's initial weight)
 * rows      >= 0 and < 2^31;  D must be 128 (GDR_ERR_UNSUPPORTED)
 * eps       >= 0 and finite (Qwen3-Next uses 1e-6)
 * y         [rows, D] dtype; may equal x (in place), must not overlap x
 *           otherwise, nor z or weight
 * kernel_ms NULL, or where to write the kernel's GPU time (the call then
 *           blocks until the kernel ends)
 * One launch, HBM bound: 3 D dtype values move per row.
 */
gdr_status gdr_gated_rmsnorm(const void* x, const void* z, const void* weight, int64_t rows,
                             int32_t D, gdr_dtype dtype, float eps, void* y, void* stream,
                             float* kernel_ms);

/*
 * One decode step with the gated RMSNorm fused behind it (blog post sections
 * 5(2) and 6): the step of gdr_recurrent_step, its output o cast to dtype,
 * then out = gated RMSNorm of o as gdr_gated_rmsnorm defines it, per
 * (sequence, value head).  Same arguments, layouts and errors as
 * gdr_recurrent_step, plus:
 *
 * z          [N, Nv, D] dtype, the output gate (required); must not overlap out
 * weight     [D] dtype, or NULL for ones
 * norm_eps   >= 0 and finite
 * kernel_ms  NULL, or where to write the kernel's GPU time (the call then
 *            blocks until the kernel ends)
 *
 * out receives the normalised, gated rows only; o itself is not stored.
 */
gdr_status gdr_recurrent_step_gated(const void* q, const void* k, const void* v,
                                    const float* g, const float* beta,
                                    const float* state_in, float* state_out,
                                    int32_t N, int32_t Nqk, int32_t Nv, int32_t D,
                                    gdr_dtype dtype, float scale, uint32_t flags,
                                    const void* z, const void* weight, float norm_eps,
                                    void* out, void* stream, float* kernel_ms);

/*
 * Debug checks of the device-side contract (see the conventions above).
 * mode 1 switches them on, 0 off, any other value only queries; returns the
 * state before the call (1 on, 0 off).  The setting is process-wide.
 */
int gdr_set_debug(int mode);

/*
 * Which contracts the calling thread's last checked call found broken
 * (0: none, or no checked call yet): bit 0 cu_seqlens[0] != 0, bit 1
 * cu_seqlens decreases somewhere, bit 2 cu_seqlens[N] != T, bit 3 a gate g
 * is positive, infinite or NaN.
 */
uint32_t gdr_debug_broken(void);

/* A static, human-readable name for a status code. */
const char* gdr_status_string(gdr_status s);

/* Library version, for logging: "libgdr <major>.<minor>". */
const char* gdr_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDR_H */
