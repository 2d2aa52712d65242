"""Independent codings of the gated delta rule -- TEST INFRASTRUCTURE ONLY.

These exist to pin ``oracle.recurrent`` (the C per-token recurrence) against
other statements of the same rule on the Qwen3-Next blog post
("Code-Qwen3-Next"):

* ``matrix_form``: the gated DeltaNet transition written as a matrix product,
  S_t = S_{t-1} (alpha_t (I - beta_t k_t k_t^T)) + beta_t v_t k_t^T, from the
  derivation that closes section 5(2) (stated there for the key-by-value
  storage; here transposed to value-by-key).
* ``chunked``: the chunkwise form of section 5(1) (equations (1)-(9) of
  subsection a and the steps b-g), for any chunk size, with the strictly lower
  triangular system solved by the row recurrence of subsection d.

Both are slow numpy fp64 code.  They share nothing with the C oracle.
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np


def _normalise(x: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(sum x^2 + eps) along the last axis (Ascend operator page, L2Norm)."""
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def matrix_form(q, k, v, g, beta, state_in, cu_seqlens, scale, eps=1e-6):
    """Token-by-token rule as S <- S (alpha (I - beta kh kh^T)) + beta v kh^T."""
    q, k, v, g, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, beta))
    T, Nqk, Dk = q.shape
    Nv, Dv = v.shape[1], v.shape[2]
    N = len(cu_seqlens) - 1
    grp = Nv // Nqk
    out = np.zeros((T, Nv, Dv))
    sout = np.zeros((N, Nv, Dv, Dk))
    eye = np.eye(Dk)
    for b in range(N):
        for h in range(Nv):
            j = h // grp
            S = np.zeros((Dv, Dk)) if state_in is None else np.array(state_in[b, h], dtype=np.float64)
            for t in range(int(cu_seqlens[b]), int(cu_seqlens[b + 1])):
                kh = _normalise(k[t, j], eps)
                qh = scale * _normalise(q[t, j], eps)
                alpha = np.exp(g[t, h])
                S = S @ (alpha * (eye - beta[t, h] * np.outer(kh, kh))) + beta[t, h] * np.outer(v[t, h], kh)
                out[t, h] = S @ qh
            sout[b, h] = S
    return out, sout


def unit_lower_inverse_rows(A: np.ndarray) -> np.ndarray:
    """(I - A)^-1 for strictly lower triangular A via the row recurrence.

    With T~ = (I - A)^-1 - I (strictly lower), row i obeys
    T~[i, :i] = A[i, :i] + A[i, :i] @ T~[:i, :i]   (section 5(1)d).
    """
    n = A.shape[0]
    Tt = np.zeros_like(A, dtype=np.float64)
    for i in range(1, n):
        row = A[i, :i]
        Tt[i, :i] = row + row @ Tt[:i, :i]
    return Tt + np.eye(n)


def chunked(q, k, v, g, beta, state_in, cu_seqlens, scale, chunk: int, eps=1e-6):
    """Chunkwise gated delta rule, sequence by sequence, chunks restart at each sequence."""
    q, k, v, g, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, beta))
    T, Nqk, Dk = q.shape
    Nv, Dv = v.shape[1], v.shape[2]
    N = len(cu_seqlens) - 1
    grp = Nv // Nqk
    out = np.zeros((T, Nv, Dv))
    sout = np.zeros((N, Nv, Dv, Dk))
    for b in range(N):
        t0, t1 = int(cu_seqlens[b]), int(cu_seqlens[b + 1])
        for h in range(Nv):
            j = h // grp
            # state kept value-by-key: S[i, c]
            S = np.zeros((Dv, Dk)) if state_in is None else np.array(state_in[b, h], dtype=np.float64)
            for c0 in range(t0, t1, chunk):
                c1 = min(c0 + chunk, t1)
                Kc = _normalise(k[c0:c1, j], eps)
                Qc = scale * _normalise(q[c0:c1, j], eps)
                Vc = v[c0:c1, h]
                bc = beta[c0:c1, h]
                gc = np.cumsum(g[c0:c1, h])             # restarts at the chunk start
                n = c1 - c0
                diff = gc[:, None] - gc[None, :]
                low = np.tril(np.ones((n, n), dtype=bool))
                Gam = np.where(low, np.exp(np.where(low, diff, 0.0)), 0.0)   # decay mask
                strict = np.tril(np.ones((n, n), dtype=bool), -1)
                A = -np.where(strict, (bc[:, None] * Kc) @ Kc.T * Gam, 0.0)
                Tm = unit_lower_inverse_rows(A)          # [I + strictLower(...)]^-1
                U = Tm @ (bc[:, None] * Vc)
                Wl = Tm @ (bc[:, None] * Kc * np.exp(gc)[:, None])
                P = np.where(low, Qc @ Kc.T * Gam, 0.0)
                Vnew = U - Wl @ S.T
                Ql = Qc * np.exp(gc)[:, None]
                out[c0:c1, h] = Ql @ S.T + P @ Vnew
                Kr = Kc * np.exp(gc[-1] - gc)[:, None]
                S = np.exp(gc[-1]) * S + Vnew.T @ Kr
            sout[b, h] = S
    return out, sout
