"""CPU fp64 oracle of the gated delta rule -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg import
this package.  The HIP library and its Python binding never do.

``recurrent`` runs the per-token recurrence in C (``gdr_oracle.c``), the
plain definition the chunkwise form must reproduce (Qwen3-Next blog post,
section 5(2)).  ``oracle.alt`` holds two independently written codings of the
same rule (the DeltaNet matrix form and the chunkwise form of section 5(1)),
used only to pin ``recurrent`` in the oracle's own tests.
``recurrent_step_bf16_state`` is one decode step whose stored state is
rounded to bfloat16 (``round_bf16``), pinned in
``tests/test_oracle_bf16_state.py``; ``decode_prologue`` and
``recurrent_step_conv`` add the conv update and gates in front of a decode
step, pinned in ``tests/test_oracle_prologue.py``; ``gated_rmsnorm`` and
``recurrent_step_gated`` are the gated RMSNorm after the rule, pinned in
``tests/test_oracle_gated_norm.py``.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(HERE, "liboracle.so")
_lib = None

EPS = 1e-6


def load_library(path: str):
    """Open an oracle shared library and declare its C signatures."""
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    lib.gdr_oracle_run.argtypes = [dp, dp, dp, dp, dp, dp, ctypes.POINTER(ctypes.c_int32),
                                   ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                   ctypes.c_int32, ctypes.c_int32,
                                   ctypes.c_double, ctypes.c_double, ctypes.c_int32,
                                   dp, dp, ctypes.c_int32]
    lib.gdr_oracle_run.restype = ctypes.c_int
    lib.gdr_oracle_threads.argtypes = [ctypes.c_int32]
    lib.gdr_oracle_threads.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b
        _b.build()
    _lib = load_library(_LIB_PATH)
    return _lib


def _f64(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def threads(n: int = 0) -> int:
    return int(_load().gdr_oracle_threads(int(n)))


def recurrent(q, k, v, g, beta, state_in: Optional[np.ndarray], cu_seqlens,
              scale: float, eps: float = EPS, nthreads: int = 0,
              want_state: bool = True, lib=None, l2norm: bool = True) -> Tuple[np.ndarray, Optional[np.ndarray]]:
    """Per-token gated delta rule in fp64.

    Shapes: q, k [T, Nqk, Dk]; v [T, Nv, Dv]; g, beta [T, Nv];
    state_in [N, Nv, Dv, Dk] or None (zeros); cu_seqlens [N + 1].
    Returns (out [T, Nv, Dv], state_out [N, Nv, Dv, Dk] or None), float64.
    ``l2norm=False`` skips the query/key normalisation.
    ``lib`` selects another build of the oracle (used by the mutation tests).
    """
    lib = _load() if lib is None else lib
    q, k, v, g, beta = (_f64(x) for x in (q, k, v, g, beta))
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
    T, Nqk, Dk = q.shape
    Nv, Dv = v.shape[1], v.shape[2]
    N = cu.shape[0] - 1
    if k.shape != q.shape or v.shape[0] != T or g.shape != (T, Nv) or beta.shape != (T, Nv):
        raise ValueError("shape mismatch")
    if int(cu[-1]) != T:
        raise ValueError("cu_seqlens[-1] must equal T")
    sin = None if state_in is None else _f64(state_in)
    if sin is not None and sin.shape != (N, Nv, Dv, Dk):
        raise ValueError("state_in shape mismatch")
    out = np.zeros((T, Nv, Dv), dtype=np.float64)
    sout = np.zeros((N, Nv, Dv, Dk), dtype=np.float64) if want_state else None
    rc = lib.gdr_oracle_run(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                            _ptr(sin) if sin is not None else None,
                            cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                            N, Nqk, Nv, Dk, Dv, float(scale), float(eps), int(bool(l2norm)),
                            _ptr(out), _ptr(sout) if sout is not None else None, int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle rejected its arguments (code {rc})")
    return out, sout


def round_bf16(x) -> np.ndarray:
    """Each fp64 value rounded to the nearest bfloat16 value, ties to even.

    bfloat16 keeps 8 significant bits (7 stored) and fp32's exponent range;
    below 2**-126 its spacing stays 2**-133 (subnormals).  Written from that
    definition: x = m * 2**e with 0.5 <= |m| < 1, so the spacing of bf16
    values near x is 2**(e - 8); x / spacing is rounded to the nearest
    integer, halves to even (np.rint).  Values beyond the largest finite
    bf16 value after rounding become +-inf.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    quantum = np.ldexp(1.0, np.maximum(e, -125) - 8)
    r = np.rint(x / quantum) * quantum
    big = np.abs(r) > 3.3895313892515355e38   # (2 - 2**-7) * 2**127
    return np.where(big, np.copysign(np.inf, x), r)


def recurrent_step_bf16_state(q, k, v, g, beta, state_in, scale: float, eps: float = EPS,
                              nthreads: int = 0, l2norm: bool = True, lib=None):
    """One decode step whose state is stored in bfloat16 between steps.

    The generic "Gated DeltaNet" article (section 6.3, deployment advice)
    names a bfloat16 state cache.  Reading taken: the stored state holds
    bf16 values; the step itself is the exact rule of the blog post's
    section 5(2) on those values (so the output comes from the unrounded new
    state), and only the new state is rounded to bf16 when it is stored.

    Shapes: q, k [N, Nqk, Dk]; v [N, Nv, Dv]; g, beta [N, Nv];
    state_in [N, Nv, Dv, Dk] (bf16 values, given as floats).
    Returns (out [N, Nv, Dv], state_out [N, Nv, Dv, Dk] rounded to bf16).
    """
    N = np.asarray(q).shape[0]
    cu = np.arange(N + 1, dtype=np.int32)
    out, sout = recurrent(q, k, v, g, beta, _f64(state_in), cu, scale, eps=eps, nthreads=nthreads,
                          want_state=True, lib=lib, l2norm=l2norm)
    return out, round_bf16(sout)


def _activate(y, conv_b, activation_bf16: bool):
    """Conv outputs [.., C] plus the bias, through SiLU (x / (1 + e^-x)), cast
    to the activation dtype (bf16 via ``round_bf16`` when asked)."""
    if conv_b is not None:
        y = y + _f64(conv_b)[None, :]
    y = y / (1.0 + np.exp(-y))
    if activation_bf16:
        y = round_bf16(y)
    return y


def _gates(a, b, A_log, dt_bias):
    """Blog post section 4: g = -exp(A_log) softplus(a + dt_bias), beta =
    sigmoid(b); softplus in its overflow-free form max(z, 0) + log1p(e^-|z|)."""
    z = _f64(a) + _f64(dt_bias)[None, :]
    softplus = np.maximum(z, 0.0) + np.log1p(np.exp(-np.abs(z)))
    g = -np.exp(_f64(A_log))[None, :] * softplus
    beta = 1.0 / (1.0 + np.exp(-_f64(b)))
    return g, beta


def decode_prologue(mixed_qkv, conv_state, conv_w, conv_b, a, b, A_log, dt_bias, Nqk: int,
                    Nv: int, D: int = 128, activation_bf16: bool = True):
    """The steps in front of a decode step (blog post, sections 3 and 4), in fp64.

    Causal depthwise conv update (section 3, the decode branch): the cached
    window of each channel gains the new value and drops its oldest one; the
    channel's output is the cross-correlation of the new window with that
    channel's kernel plus its bias, through SiLU (x / (1 + e^-x)), cast to the
    activation dtype (bf16 when ``activation_bf16``, via ``round_bf16``).  The
    output splits into q | k | v (Nqk*D, Nqk*D and Nv*D channels).  The gates
    (section 4): beta = sigmoid(b), g = -exp(A_log) * softplus(a + dt_bias).

    Shapes: mixed_qkv [N, C]; conv_state [N, C, K]; conv_w [C, K]; conv_b [C]
    or None; a, b [N, Nv]; A_log, dt_bias [Nv].  Returns
    (q [N, Nqk, D], k [N, Nqk, D], v [N, Nv, D], g [N, Nv], beta [N, Nv],
    new conv_state [N, C, K]).
    """
    x = _f64(mixed_qkv)
    cs = _f64(conv_state)
    w = _f64(conv_w)
    N, C = x.shape
    if C != (2 * Nqk + Nv) * D or cs.shape[:2] != (N, C) or w.shape != (C, cs.shape[2]):
        raise ValueError("shape mismatch")
    new_state = np.concatenate([cs[:, :, 1:], x[:, :, None]], axis=2)
    y = np.sum(new_state * w[None, :, :], axis=2)
    y = _activate(y, conv_b, activation_bf16)
    q = y[:, :Nqk * D].reshape(N, Nqk, D)
    k = y[:, Nqk * D:2 * Nqk * D].reshape(N, Nqk, D)
    v = y[:, 2 * Nqk * D:].reshape(N, Nv, D)
    g, beta = _gates(a, b, A_log, dt_bias)
    return q, k, v, g, beta, new_state


def prefill_prologue(mixed_qkv, conv_state, conv_w, conv_b, a, b, A_log, dt_bias, cu_seqlens,
                     Nqk: int, Nv: int, D: int = 128, activation_bf16: bool = True):
    """The steps in front of the chunkwise path for packed sequences (blog post
    sections 3 and 4), in fp64: per sequence and channel, the causal depthwise
    conv over the sequence's tokens, with the cached window (conv_state, or
    zeros when None) in front of its first token; SiLU; cast to the activation
    dtype; split into q | k | v.  The gates per token as in ``decode_prologue``.
    The new window of a sequence is the last K values of (window, tokens).

    Shapes: mixed_qkv [T, C]; conv_state [N, C, K] or None; conv_w [C, K];
    conv_b [C] or None; a, b [T, Nv]; A_log, dt_bias [Nv]; cu_seqlens [N + 1].
    Returns (q [T, Nqk, D], k [T, Nqk, D], v [T, Nv, D], g [T, Nv],
    beta [T, Nv], new conv_state [N, C, K]).
    """
    x = _f64(mixed_qkv)
    w = _f64(conv_w)
    T, C = x.shape
    K = w.shape[1]
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    N = cu.shape[0] - 1
    if C != (2 * Nqk + Nv) * D or w.shape[0] != C:
        raise ValueError("shape mismatch")
    cs = np.zeros((N, C, K)) if conv_state is None else _f64(conv_state)
    y = np.zeros((T, C))
    new_state = np.zeros((N, C, K))
    for n in range(N):
        seq = x[cu[n]:cu[n + 1]].T                            # [C, len]
        full = np.concatenate([cs[n], seq], axis=1)           # [C, K + len]
        for t in range(seq.shape[1]):
            # token t's window: the K values ending at it (positions t+1 .. t+K)
            y[cu[n] + t] = np.sum(full[:, t + 1:t + 1 + K] * w, axis=1)
        new_state[n] = full[:, -K:]
    y = _activate(y, conv_b, activation_bf16)
    q = y[:, :Nqk * D].reshape(T, Nqk, D)
    k = y[:, Nqk * D:2 * Nqk * D].reshape(T, Nqk, D)
    v = y[:, 2 * Nqk * D:].reshape(T, Nv, D)
    g, beta = _gates(a, b, A_log, dt_bias)
    return q, k, v, g, beta, new_state


def recurrent_step_conv(mixed_qkv, conv_state, conv_w, conv_b, a, b, A_log, dt_bias, state_in,
                        Nqk: int, Nv: int, scale: float, activation_bf16: bool = True,
                        l2norm: bool = True, nthreads: int = 0):
    """``decode_prologue`` followed by one decode step of the rule.

    Returns (out [N, Nv, D], state_out [N, Nv, D, D], new conv_state).
    """
    D = np.asarray(state_in).shape[-1]
    q, k, v, g, beta, cs = decode_prologue(mixed_qkv, conv_state, conv_w, conv_b, a, b, A_log,
                                           dt_bias, Nqk, Nv, D, activation_bf16=activation_bf16)
    N = q.shape[0]
    out, sout = recurrent(q, k, v, g, beta, state_in, np.arange(N + 1, dtype=np.int32), scale,
                          nthreads=nthreads, l2norm=l2norm)
    return out, sout, cs


NORM_EPS = 1e-6


def gated_rmsnorm(x, z, weight=None, eps: float = NORM_EPS, out_bf16: bool = False) -> np.ndarray:
    """The gated RMSNorm in front of the output projection (Qwen3-Next blog
    post: RMSNormGated in section 1, ``self.norm(core_attn_out, z)`` in section
    6; the norm is the ``_norm`` of the Zero-Centered RMSNorm section,
    x * rsqrt(mean(x^2) + eps), over each head's last dimension).

    Reading taken where the pages are silent: the output gate z enters through
    SiLU, z * sigmoid(z) (the activation the pages use for this block's conv and
    for gating in the MLP), multiplied element-wise with the normalised output
    and the per-channel weight w (None: ones, the initial value of the plain
    RMSNorm the blog says RMSNormGated uses; the zero-centred form passes 1 + g):

        y = x / sqrt(mean(x^2) + eps) * w * z * sigmoid(z)

    Shapes: x, z [..., D]; weight [D].  fp64; ``out_bf16`` rounds y to bf16
    (the result is cast back to the activation dtype).
    """
    x = _f64(x)
    z = _f64(z)
    w = np.ones(x.shape[-1]) if weight is None else _f64(weight)
    inv = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    y = x * inv * w * (z / (1.0 + np.exp(-z)))
    return round_bf16(y) if out_bf16 else y


def recurrent_step_gated(q, k, v, g, beta, state_in, z, weight, scale: float, eps: float = EPS,
                         norm_eps: float = NORM_EPS, out_bf16: bool = False, nthreads: int = 0,
                         l2norm: bool = True):
    """One decode step followed by the gated RMSNorm of its output (blog post
    sections 5(2) and 6).  The step's output is cast to the activation dtype
    before the norm, as the blog's recurrence returns it (``out_bf16``: bf16).

    Returns (y [N, Nv, Dv], state_out [N, Nv, Dv, Dk]).
    """
    N = np.asarray(q).shape[0]
    cu = np.arange(N + 1, dtype=np.int32)
    out, sout = recurrent(q, k, v, g, beta, state_in, cu, scale, eps=eps, nthreads=nthreads,
                          l2norm=l2norm)
    o = round_bf16(out) if out_bf16 else out
    return gated_rmsnorm(o, z, weight, norm_eps, out_bf16=False), sout


def rel_l2(x, ref) -> float:
    """||x - ref||_2 / ||ref||_2 over the whole array, in fp64."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = float(np.linalg.norm(ref.ravel()))
    num = float(np.linalg.norm((x - ref).ravel()))
    if den == 0.0:
        return num
    return num / den
