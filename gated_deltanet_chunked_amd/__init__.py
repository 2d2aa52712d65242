"""Python binding of libgdr, the gated delta rule on MI355X (gfx950).

Thin ctypes marshalling over the C ABI in ``include/gdr.h``: every step of the
computation runs in the HIP kernels of ``libgdr.so``.  PyTorch provides device
memory and the current stream only.  There is no fallback: if the library is
missing, every call raises.

    out, state = chunk_fwd(q, k, v, g, beta, cu_seqlens, state_in=s0)
    out = recurrent_step(q, k, v, g, beta, state, state_out=state)   # in place
    y = gated_rmsnorm(out, z, weight)                                 # before out_proj
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgdr.so")

GDR_F32 = 0
GDR_BF16 = 1
GDR_FLAG_QK_L2NORM = 1
GDR_FLAG_CHUNK64 = 2
CHUNK = 128
D = 128

STATUS = {0: "GDR_OK", -1: "GDR_ERR_INVALID_ARGUMENT", -2: "GDR_ERR_UNSUPPORTED",
          -3: "GDR_ERR_WORKSPACE_TOO_SMALL", -4: "GDR_ERR_HIP", -5: "GDR_ERR_CONTRACT"}

_lib = None


class GdrError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {STATUS.get(status, status)}")
        self.status = status


def load(path: str = LIB_PATH):
    """Load libgdr.so and declare the C signatures (no GPU needed)."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    try:
        # torch ships its own HIP runtime; loading torch first makes libgdr bind
        # to that same runtime (one HIP runtime per process)
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(path):
        raise RuntimeError(f"libgdr.so not built at {path}: run `python -m gated_deltanet_chunked_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, u32, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint32, ctypes.c_float, ctypes.c_size_t
    lib.gdr_chunk_fwd_workspace_size.argtypes = [i32, i32, i32, i32, i32, ctypes.c_int]
    lib.gdr_chunk_fwd_workspace_size.restype = sz
    lib.gdr_chunk_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, ctypes.c_int,
                                  f32, u32, vp, vp, vp, sz, vp]
    lib.gdr_chunk_fwd.restype = ctypes.c_int
    lib.gdr_recurrent_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, ctypes.c_int,
                                       f32, u32, vp, vp]
    lib.gdr_recurrent_step.restype = ctypes.c_int
    lib.gdr_chunk_fwd_timed.argtypes = lib.gdr_chunk_fwd.argtypes + [
        ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_int32), i32,
        ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_float)]
    lib.gdr_chunk_fwd_timed.restype = ctypes.c_int
    lib.gdr_recurrent_step_timed.argtypes = lib.gdr_recurrent_step.argtypes + [
        ctypes.POINTER(ctypes.c_float)]
    lib.gdr_recurrent_step_timed.restype = ctypes.c_int
    lib.gdr_recurrent_step_bf16_state.argtypes = lib.gdr_recurrent_step_timed.argtypes
    lib.gdr_recurrent_step_bf16_state.restype = ctypes.c_int
    lib.gdr_recurrent_multi.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                        ctypes.c_int, f32, u32, vp, vp, vp,
                                        ctypes.POINTER(ctypes.c_float)]
    lib.gdr_recurrent_multi.restype = ctypes.c_int
    lib.gdr_recurrent_step_conv.argtypes = [vp, vp, vp, vp, vp, i32, vp, vp, vp, vp, vp, vp,
                                            i32, i32, i32, i32, ctypes.c_int, f32, u32, vp, vp,
                                            ctypes.POINTER(ctypes.c_float)]
    lib.gdr_recurrent_step_conv.restype = ctypes.c_int
    lib.gdr_conv_prefill.argtypes = [vp, vp, vp, vp, vp, i32, vp, vp, vp, vp, vp, i32, i32, i32,
                                     i32, i32, ctypes.c_int, vp, vp, vp, vp, vp, vp,
                                     ctypes.POINTER(ctypes.c_float)]
    lib.gdr_conv_prefill.restype = ctypes.c_int
    lib.gdr_chunk_fwd_no_alloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                           ctypes.c_int, f32, u32, vp, vp, vp]
    lib.gdr_chunk_fwd_no_alloc.restype = ctypes.c_int
    lib.gdr_chunk_fwd_no_alloc_scratch_bytes.argtypes = []
    lib.gdr_chunk_fwd_no_alloc_scratch_bytes.restype = sz
    lib.gdr_gated_rmsnorm.argtypes = [vp, vp, vp, ctypes.c_int64, i32, ctypes.c_int, f32, vp, vp,
                                      ctypes.POINTER(ctypes.c_float)]
    lib.gdr_gated_rmsnorm.restype = ctypes.c_int
    lib.gdr_recurrent_step_gated.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32,
                                             ctypes.c_int, f32, u32, vp, vp, f32, vp, vp,
                                             ctypes.POINTER(ctypes.c_float)]
    lib.gdr_recurrent_step_gated.restype = ctypes.c_int
    lib.gdr_set_debug.argtypes = [ctypes.c_int]
    lib.gdr_set_debug.restype = ctypes.c_int
    lib.gdr_debug_broken.argtypes = []
    lib.gdr_debug_broken.restype = u32
    lib.gdr_status_string.argtypes = [ctypes.c_int]
    lib.gdr_status_string.restype = ctypes.c_char_p
    lib.gdr_version.argtypes = []
    lib.gdr_version.restype = ctypes.c_char_p
    if path == LIB_PATH:
        _lib = lib
    return lib


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return GDR_BF16
    if t.dtype == torch.float32:
        return GDR_F32
    raise TypeError(f"q/k/v must be bfloat16 or float32, got {t.dtype}")


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _check(t, name, shape, dtype, device):
    if t is None:
        return
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must be on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")


def _stream() -> int:
    import torch
    return torch.cuda.current_stream().cuda_stream


def workspace_size(T: int, N: int, Nqk: int, Nv: int, dtype_code: int) -> int:
    return int(load().gdr_chunk_fwd_workspace_size(T, N, Nqk, Nv, D, dtype_code))


STAGE_NAMES = {0: "table", 1: "intra", 2: "inter"}


def _chunk_flags(l2norm: bool, chunk: int) -> int:
    if chunk not in (64, 128):
        raise ValueError(f"chunk must be 64 or 128, got {chunk}")
    return (GDR_FLAG_QK_L2NORM if l2norm else 0) | (GDR_FLAG_CHUNK64 if chunk == 64 else 0)


def chunk_fwd(q, k, v, g, beta, cu_seqlens, state_in=None, *, scale: Optional[float] = None,
              out=None, state_out=None, want_state: bool = True, workspace=None,
              l2norm: bool = True, chunk: int = CHUNK, timings: Optional[list] = None
              ) -> Tuple["torch.Tensor", Optional["torch.Tensor"]]:
    """Chunkwise gated delta rule over packed sequences (``gdr_chunk_fwd``).

    q, k [T, Nqk, 128], v [T, Nv, 128] (bf16 or f32); g, beta [T, Nv] f32;
    cu_seqlens [N + 1] int32 (device); state_in [N, Nv, 128, 128] f32 or None.
    Returns (out [T, Nv, 128] in q's dtype, state_out or None).
    ``state_out`` may be ``state_in`` for an in-place update.  ``chunk``: the
    chunk length, 128 or 64 (``GDR_FLAG_CHUNK64``; same results up to rounding).
    With a list as ``timings`` the call goes through ``gdr_chunk_fwd_timed``
    (blocking) and appends one (stage name, GPU milliseconds) per kernel, then
    ("span", milliseconds from the first kernel's start to the last one's end).
    """
    import torch
    lib = load()
    T, Nqk, _ = q.shape
    Nv = v.shape[1]
    N = cu_seqlens.shape[0] - 1
    dev = q.device
    dt = q.dtype
    code = _dtype_code(q)
    _check(q, "q", (T, Nqk, D), dt, dev)
    _check(k, "k", (T, Nqk, D), dt, dev)
    _check(v, "v", (T, Nv, D), dt, dev)
    _check(g, "g", (T, Nv), torch.float32, dev)
    _check(beta, "beta", (T, Nv), torch.float32, dev)
    _check(cu_seqlens, "cu_seqlens", (N + 1,), torch.int32, dev)
    _check(state_in, "state_in", (N, Nv, D, D), torch.float32, dev)
    if out is None:
        out = torch.empty((T, Nv, D), dtype=dt, device=dev)
    _check(out, "out", (T, Nv, D), dt, dev)
    if state_out is None and want_state:
        state_out = torch.empty((N, Nv, D, D), dtype=torch.float32, device=dev)
    _check(state_out, "state_out", (N, Nv, D, D), torch.float32, dev)
    need = workspace_size(T, N, Nqk, Nv, code)
    if need == 0:
        raise GdrError(-1, "gdr_chunk_fwd_workspace_size")
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if scale is None:
        scale = D ** -0.5
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state_in),
            _ptr(cu_seqlens), N, T, Nqk, Nv, D, code, float(scale),
            _chunk_flags(l2norm, chunk), _ptr(out), _ptr(state_out),
            _ptr(workspace), workspace.numel(), _stream())
    if timings is None:
        st = lib.gdr_chunk_fwd(*args)
        if st != 0:
            raise GdrError(st, "gdr_chunk_fwd")
        return out, state_out
    cap = 1024
    ms = (ctypes.c_float * cap)()
    kind = (ctypes.c_int32 * cap)()
    n = ctypes.c_int32(0)
    span = ctypes.c_float(0.0)
    st = lib.gdr_chunk_fwd_timed(*args, ms, kind, cap, ctypes.byref(n), ctypes.byref(span))
    if st != 0:
        raise GdrError(st, "gdr_chunk_fwd_timed")
    timings.extend((STAGE_NAMES.get(kind[i], str(kind[i])), float(ms[i])) for i in range(n.value))
    timings.append(("span", float(span.value)))
    return out, state_out


def chunk_fwd_no_alloc(q, k, v, g, beta, cu_seqlens, state_in, out, state_out, *,
                       scale: Optional[float] = None, l2norm: bool = True, chunk: int = CHUNK):
    """``gdr_chunk_fwd_no_alloc``: the chunkwise forward with the library's
    fixed scratch as workspace.  The caller passes every buffer (``state_in``
    and ``state_out`` may be None), so this function allocates nothing either.
    Returns (out, state_out)."""
    import torch
    lib = load()
    T, Nqk, _ = q.shape
    Nv = v.shape[1]
    N = cu_seqlens.shape[0] - 1
    dev = q.device
    dt = q.dtype
    code = _dtype_code(q)
    _check(q, "q", (T, Nqk, D), dt, dev)
    _check(k, "k", (T, Nqk, D), dt, dev)
    _check(v, "v", (T, Nv, D), dt, dev)
    _check(g, "g", (T, Nv), torch.float32, dev)
    _check(beta, "beta", (T, Nv), torch.float32, dev)
    _check(cu_seqlens, "cu_seqlens", (N + 1,), torch.int32, dev)
    _check(state_in, "state_in", (N, Nv, D, D), torch.float32, dev)
    _check(out, "out", (T, Nv, D), dt, dev)
    _check(state_out, "state_out", (N, Nv, D, D), torch.float32, dev)
    if scale is None:
        scale = D ** -0.5
    st = lib.gdr_chunk_fwd_no_alloc(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                    _ptr(state_in), _ptr(cu_seqlens), N, T, Nqk, Nv, D, code,
                                    float(scale), _chunk_flags(l2norm, chunk), _ptr(out),
                                    _ptr(state_out), _stream())
    if st != 0:
        raise GdrError(st, "gdr_chunk_fwd_no_alloc")
    return out, state_out


def recurrent_multi(q, k, v, g, beta, cu_seqlens, state_in=None, *, scale: Optional[float] = None,
                    out=None, state_out=None, want_state: bool = True, l2norm: bool = True,
                    timings: Optional[list] = None):
    """A few tokens per sequence, token by token (``gdr_recurrent_multi``).

    Same arguments and results as ``chunk_fwd`` (packed q, k [T, Nqk, 128],
    v [T, Nv, 128]; g, beta [T, Nv]; cu_seqlens [N + 1] int32 on the device;
    state_in [N, Nv, 128, 128] f32 or None), without a workspace.  With a list
    as ``timings`` the call waits for the kernel and appends ("multi", ms).
    """
    import torch
    lib = load()
    T, Nqk, _ = q.shape
    Nv = v.shape[1]
    N = cu_seqlens.shape[0] - 1
    dev = q.device
    dt = q.dtype
    code = _dtype_code(q)
    _check(q, "q", (T, Nqk, D), dt, dev)
    _check(k, "k", (T, Nqk, D), dt, dev)
    _check(v, "v", (T, Nv, D), dt, dev)
    _check(g, "g", (T, Nv), torch.float32, dev)
    _check(beta, "beta", (T, Nv), torch.float32, dev)
    _check(cu_seqlens, "cu_seqlens", (N + 1,), torch.int32, dev)
    _check(state_in, "state_in", (N, Nv, D, D), torch.float32, dev)
    if out is None:
        out = torch.empty((T, Nv, D), dtype=dt, device=dev)
    _check(out, "out", (T, Nv, D), dt, dev)
    if state_out is None and want_state:
        state_out = torch.empty((N, Nv, D, D), dtype=torch.float32, device=dev)
    _check(state_out, "state_out", (N, Nv, D, D), torch.float32, dev)
    if scale is None:
        scale = D ** -0.5
    ms = ctypes.c_float(0.0)
    st = lib.gdr_recurrent_multi(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state_in),
                                 _ptr(cu_seqlens), N, T, Nqk, Nv, D, code, float(scale),
                                 GDR_FLAG_QK_L2NORM if l2norm else 0, _ptr(out), _ptr(state_out),
                                 _stream(), ctypes.byref(ms) if timings is not None else None)
    if st != 0:
        raise GdrError(st, "gdr_recurrent_multi")
    if timings is not None:
        timings.append(("multi", float(ms.value)))
    return out, state_out


def recurrent_step_conv(mixed_qkv, conv_state_in, conv_weight, conv_bias, a, b, A_log, dt_bias,
                        state_in, *, conv_state_out=None, state_out=None, out=None,
                        scale: Optional[float] = None, l2norm: bool = True,
                        timings: Optional[list] = None):
    """One decode step with the conv update and gates fused in front
    (``gdr_recurrent_step_conv``).

    mixed_qkv [N, C] (q | k | v channels, C = (2 Nqk + Nv) 128) in the
    activation dtype; conv_state_in [N, C, 4] and conv_weight [C, 4] in the same
    dtype; conv_bias [C] or None; a, b [N, Nv] f32; A_log, dt_bias [Nv] f32;
    state_in [N, Nv, 128, 128] f32.  ``state_out`` defaults to ``state_in`` (in
    place); ``conv_state_out`` is a new tensor unless given (never the input).
    Returns (out [N, Nv, 128], conv_state_out).  With a list as ``timings`` the
    call waits for the kernel and appends ("decode_conv", ms).
    """
    import torch
    lib = load()
    N, C = mixed_qkv.shape
    Nv = a.shape[1]
    Nqk = (C // D - Nv) // 2
    K = conv_state_in.shape[2]
    dev = mixed_qkv.device
    dt = mixed_qkv.dtype
    code = _dtype_code(mixed_qkv)
    if (2 * Nqk + Nv) * D != C:
        raise ValueError(f"mixed_qkv has {C} channels, not (2 Nqk + Nv) * {D}")
    _check(conv_state_in, "conv_state_in", (N, C, K), dt, dev)
    _check(conv_weight, "conv_weight", (C, K), dt, dev)
    _check(conv_bias, "conv_bias", (C,), dt, dev)
    _check(a, "a", (N, Nv), torch.float32, dev)
    _check(b, "b", (N, Nv), torch.float32, dev)
    _check(A_log, "A_log", (Nv,), torch.float32, dev)
    _check(dt_bias, "dt_bias", (Nv,), torch.float32, dev)
    _check(state_in, "state_in", (N, Nv, D, D), torch.float32, dev)
    if state_out is None:
        state_out = state_in
    _check(state_out, "state_out", (N, Nv, D, D), torch.float32, dev)
    if conv_state_out is None:
        conv_state_out = torch.empty_like(conv_state_in)
    _check(conv_state_out, "conv_state_out", (N, C, K), dt, dev)
    if out is None:
        out = torch.empty((N, Nv, D), dtype=dt, device=dev)
    _check(out, "out", (N, Nv, D), dt, dev)
    if scale is None:
        scale = D ** -0.5
    ms = ctypes.c_float(0.0)
    st = lib.gdr_recurrent_step_conv(
        _ptr(mixed_qkv), _ptr(conv_state_in), _ptr(conv_state_out), _ptr(conv_weight),
        _ptr(conv_bias), K, _ptr(a), _ptr(b), _ptr(A_log), _ptr(dt_bias), _ptr(state_in),
        _ptr(state_out), N, Nqk, Nv, D, code, float(scale), GDR_FLAG_QK_L2NORM if l2norm else 0,
        _ptr(out), _stream(), ctypes.byref(ms) if timings is not None else None)
    if st != 0:
        raise GdrError(st, "gdr_recurrent_step_conv")
    if timings is not None:
        timings.append(("decode_conv", float(ms.value)))
    return out, conv_state_out


def conv_prefill(mixed_qkv, conv_state_in, conv_weight, conv_bias, a, b, A_log, dt_bias,
                 cu_seqlens, *, conv_state_out=None, want_conv_state: bool = True,
                 timings: Optional[list] = None):
    """The conv/gate prologue of the chunkwise path (``gdr_conv_prefill``).

    mixed_qkv [T, C] (q | k | v channels, C = (2 Nqk + Nv) 128); conv_state_in
    [N, C, 4] or None (zeros); conv_weight [C, 4]; conv_bias [C] or None, all
    in the activation dtype; a, b [T, Nv] f32; A_log, dt_bias [Nv] f32;
    cu_seqlens [N + 1] int32 on the device.  Returns (q [T, Nqk, 128],
    k, v [T, Nv, 128], g [T, Nv], beta [T, Nv], conv_state_out or None), ready
    for ``chunk_fwd``.  With a list as ``timings`` the call waits for its
    kernels and appends ("conv_prefill", ms).
    """
    import torch
    lib = load()
    T, C = mixed_qkv.shape
    Nv = a.shape[1]
    Nqk = (C // D - Nv) // 2
    N = cu_seqlens.shape[0] - 1
    K = conv_weight.shape[1]
    dev = mixed_qkv.device
    dt = mixed_qkv.dtype
    code = _dtype_code(mixed_qkv)
    if (2 * Nqk + Nv) * D != C:
        raise ValueError(f"mixed_qkv has {C} channels, not (2 Nqk + Nv) * {D}")
    _check(conv_state_in, "conv_state_in", (N, C, K), dt, dev)
    _check(conv_weight, "conv_weight", (C, K), dt, dev)
    _check(conv_bias, "conv_bias", (C,), dt, dev)
    _check(a, "a", (T, Nv), torch.float32, dev)
    _check(b, "b", (T, Nv), torch.float32, dev)
    _check(A_log, "A_log", (Nv,), torch.float32, dev)
    _check(dt_bias, "dt_bias", (Nv,), torch.float32, dev)
    _check(cu_seqlens, "cu_seqlens", (N + 1,), torch.int32, dev)
    if conv_state_out is None and want_conv_state:
        conv_state_out = torch.empty((N, C, K), dtype=dt, device=dev)
    _check(conv_state_out, "conv_state_out", (N, C, K), dt, dev)
    q = torch.empty((T, Nqk, D), dtype=dt, device=dev)
    k = torch.empty((T, Nqk, D), dtype=dt, device=dev)
    v = torch.empty((T, Nv, D), dtype=dt, device=dev)
    g = torch.empty((T, Nv), dtype=torch.float32, device=dev)
    beta = torch.empty((T, Nv), dtype=torch.float32, device=dev)
    ms = ctypes.c_float(0.0)
    st = lib.gdr_conv_prefill(_ptr(mixed_qkv), _ptr(conv_state_in), _ptr(conv_state_out),
                              _ptr(conv_weight), _ptr(conv_bias), K, _ptr(a), _ptr(b), _ptr(A_log),
                              _ptr(dt_bias), _ptr(cu_seqlens), N, T, Nqk, Nv, D, code, _ptr(q),
                              _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _stream(),
                              ctypes.byref(ms) if timings is not None else None)
    if st != 0:
        raise GdrError(st, "gdr_conv_prefill")
    if timings is not None:
        timings.append(("conv_prefill", float(ms.value)))
    return q, k, v, g, beta, conv_state_out


def recurrent_step(q, k, v, g, beta, state_in, *, state_out=None, out=None,
                   scale: Optional[float] = None, l2norm: bool = True,
                   timings: Optional[list] = None):
    """One decode step for N sequences (``gdr_recurrent_step``).

    q, k [N, Nqk, 128], v [N, Nv, 128]; g, beta [N, Nv]; state_in [N, Nv, 128, 128].
    ``state_out`` defaults to ``state_in`` (in-place update).  Returns out [N, Nv, 128].
    States in float32 go to ``gdr_recurrent_step``; states in bfloat16 (a bf16
    state cache) go to ``gdr_recurrent_step_bf16_state``.
    With a list as ``timings`` the call is timed (``gdr_recurrent_step_timed``,
    or the bf16-state call with a time pointer; it then waits for the step)
    and appends ("decode", kernel milliseconds).
    """
    import torch
    lib = load()
    N, Nqk, _ = q.shape
    Nv = v.shape[1]
    dev = q.device
    dt = q.dtype
    code = _dtype_code(q)
    _check(q, "q", (N, Nqk, D), dt, dev)
    _check(k, "k", (N, Nqk, D), dt, dev)
    _check(v, "v", (N, Nv, D), dt, dev)
    _check(g, "g", (N, Nv), torch.float32, dev)
    _check(beta, "beta", (N, Nv), torch.float32, dev)
    st_dt = state_in.dtype
    if st_dt not in (torch.float32, torch.bfloat16):
        raise TypeError(f"state_in: dtype {st_dt}, expected float32 or bfloat16")
    _check(state_in, "state_in", (N, Nv, D, D), st_dt, dev)
    if state_out is None:
        state_out = state_in
    _check(state_out, "state_out", (N, Nv, D, D), st_dt, dev)
    if out is None:
        out = torch.empty((N, Nv, D), dtype=dt, device=dev)
    _check(out, "out", (N, Nv, D), dt, dev)
    if scale is None:
        scale = D ** -0.5
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state_in), _ptr(state_out), N,
            Nqk, Nv, D, code, float(scale), GDR_FLAG_QK_L2NORM if l2norm else 0, _ptr(out),
            _stream())
    if st_dt == torch.bfloat16:
        ms = ctypes.c_float(0.0)
        st = lib.gdr_recurrent_step_bf16_state(*args, ctypes.byref(ms) if timings is not None else None)
        if st != 0:
            raise GdrError(st, "gdr_recurrent_step_bf16_state")
        if timings is not None:
            timings.append(("decode", float(ms.value)))
        return out
    if timings is None:
        st = lib.gdr_recurrent_step(*args)
        if st != 0:
            raise GdrError(st, "gdr_recurrent_step")
        return out
    ms = ctypes.c_float(0.0)
    st = lib.gdr_recurrent_step_timed(*args, ctypes.byref(ms))
    if st != 0:
        raise GdrError(st, "gdr_recurrent_step_timed")
    timings.append(("decode", float(ms.value)))
    return out


NORM_EPS = 1e-6


def gated_rmsnorm(x, z, weight=None, *, eps: float = NORM_EPS, out=None,
                  timings: Optional[list] = None):
    """Gated RMSNorm over the last dimension (``gdr_gated_rmsnorm``):
    y = x / sqrt(mean(x^2) + eps) * weight * SiLU(z).

    x, z [..., 128] of one dtype (bf16 or f32), e.g. the rule's out [T, Nv, 128];
    weight [128] of that dtype or None (ones).  ``out`` may be ``x`` (in place).
    With a list as ``timings`` the call is timed (blocking) and appends
    ("gated_rmsnorm", kernel milliseconds).
    """
    lib = load()
    dev = x.device
    dt = x.dtype
    code = _dtype_code(x)
    if x.shape[-1] != D:
        raise ValueError(f"x: last dimension {x.shape[-1]}, expected {D}")
    _check(x, "x", tuple(x.shape), dt, dev)
    _check(z, "z", tuple(x.shape), dt, dev)
    _check(weight, "weight", (D,), dt, dev)
    if out is None:
        import torch
        out = torch.empty_like(x)
    _check(out, "out", tuple(x.shape), dt, dev)
    rows = x.numel() // D
    ms = ctypes.c_float(0.0)
    st = lib.gdr_gated_rmsnorm(_ptr(x), _ptr(z), _ptr(weight), rows, D, code, float(eps), _ptr(out),
                               _stream(), ctypes.byref(ms) if timings is not None else None)
    if st != 0:
        raise GdrError(st, "gdr_gated_rmsnorm")
    if timings is not None:
        timings.append(("gated_rmsnorm", float(ms.value)))
    return out


def recurrent_step_gated(q, k, v, g, beta, state_in, z, weight=None, *, state_out=None, out=None,
                         scale: Optional[float] = None, l2norm: bool = True,
                         norm_eps: float = NORM_EPS, timings: Optional[list] = None):
    """One decode step with the gated RMSNorm fused behind it
    (``gdr_recurrent_step_gated``).  Arguments as ``recurrent_step`` (float32
    states), plus z [N, Nv, 128] and weight [128] (or None) in q's dtype.
    Returns the gated, normalised output [N, Nv, 128]."""
    import torch
    lib = load()
    N, Nqk, _ = q.shape
    Nv = v.shape[1]
    dev = q.device
    dt = q.dtype
    code = _dtype_code(q)
    _check(q, "q", (N, Nqk, D), dt, dev)
    _check(k, "k", (N, Nqk, D), dt, dev)
    _check(v, "v", (N, Nv, D), dt, dev)
    _check(g, "g", (N, Nv), torch.float32, dev)
    _check(beta, "beta", (N, Nv), torch.float32, dev)
    _check(state_in, "state_in", (N, Nv, D, D), torch.float32, dev)
    if state_out is None:
        state_out = state_in
    _check(state_out, "state_out", (N, Nv, D, D), torch.float32, dev)
    _check(z, "z", (N, Nv, D), dt, dev)
    _check(weight, "weight", (D,), dt, dev)
    if out is None:
        out = torch.empty((N, Nv, D), dtype=dt, device=dev)
    _check(out, "out", (N, Nv, D), dt, dev)
    if scale is None:
        scale = D ** -0.5
    ms = ctypes.c_float(0.0)
    st = lib.gdr_recurrent_step_gated(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                      _ptr(state_in), _ptr(state_out), N, Nqk, Nv, D, code,
                                      float(scale), GDR_FLAG_QK_L2NORM if l2norm else 0, _ptr(z),
                                      _ptr(weight), float(norm_eps), _ptr(out), _stream(),
                                      ctypes.byref(ms) if timings is not None else None)
    if st != 0:
        raise GdrError(st, "gdr_recurrent_step_gated")
    if timings is not None:
        timings.append(("decode_gated", float(ms.value)))
    return out


def set_debug(on: bool) -> bool:
    """Switch the library's device-side contract checks on or off
    (``gdr_set_debug``); returns the previous setting."""
    return bool(load().gdr_set_debug(1 if on else 0))


def debug_broken() -> int:
    """Bits of the contracts the calling thread's last checked call found
    broken (``gdr_debug_broken``): 1 cu[0] != 0, 2 cu decreases, 4 cu[N] != T,
    8 a gate is positive or not finite."""
    return int(load().gdr_debug_broken())
