"""Pins of the CPU oracle: facts fixed by the pages and by mathematics.

Each check takes ``rec``, a callable with the signature of
``oracle.recurrent``, so the same checks run against the real oracle
(``test_oracle.py``) and against deliberately broken copies of it
(``test_oracle_mutants.py``).  Each returns a list of failure messages.

Sources of the facts (Qwen3-Next blog post "Code-Qwen3-Next", section 5;
Ascend PyPTO "Qwen3Next" operator page, math formulas):
* hand-worked two-token example (tests/golden/hand_d2.json);
* beta = 0: the write vanishes, so the state only decays: S_T = exp(sum g) S_0
  and o_t = exp(sum_{s<=t} g_s) S_0 qh_t;
* g = 0, beta = 1, orthonormal keys: each write sets S k_i = v_i and leaves
  the other keys' values alone (the DeltaNet form at the end of section 5(2));
* one token from a zero state: S = beta v kh^T, o = beta (kh . qh) v;
* the matrix form and the chunkwise form (oracle.alt) give the same numbers;
* exact rational brute force (Fractions) on tiny inputs with unit-norm keys.
"""
from __future__ import annotations

import json
import os
from fractions import Fraction

import numpy as np

from oracle import alt

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rand_case(seed, lengths, Nqk, Nv, dk, dv, state=True, A_hi=2.0):
    rng = np.random.default_rng(seed)
    T = sum(lengths)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    q = rng.standard_normal((T, Nqk, dk))
    k = rng.standard_normal((T, Nqk, dk))
    v = rng.standard_normal((T, Nv, dv))
    g = -rng.uniform(0.0, A_hi, size=(T, Nv))
    beta = rng.uniform(0.05, 0.95, size=(T, Nv))
    s0 = rng.standard_normal((len(lengths), Nv, dv, dk)) if state else None
    return q, k, v, g, beta, s0, cu


def _rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    d = np.linalg.norm(b.ravel())
    return np.linalg.norm((a - b).ravel()) / (d if d > 0 else 1.0)


def check_golden(rec):
    with open(os.path.join(GOLDEN, "hand_d2.json")) as f:
        gd = json.load(f)
    toks = gd["tokens"]
    T = len(toks)
    q = np.array([t["q"] for t in toks], dtype=np.float64)[:, None, :]
    k = np.array([t["k"] for t in toks], dtype=np.float64)[:, None, :]
    v = np.array([t["v"] for t in toks], dtype=np.float64)[:, None, :]
    g = np.log(np.array([t["alpha"] for t in toks]))[:, None]
    beta = np.array([t["beta"] for t in toks])[:, None]
    s0 = np.array(gd["state_in"], dtype=np.float64)[None, None]
    out, st = rec(q, k, v, g, beta, s0, np.array([0, T], dtype=np.int32), gd["scale"], eps=gd["eps"])
    errs = []
    if not np.allclose(out[:, 0, :], np.array(gd["expected_out"]), rtol=0, atol=1e-12):
        errs.append(f"golden out {out[:, 0, :].tolist()} != {gd['expected_out']}")
    if not np.allclose(st[0, 0], np.array(gd["expected_state"]), rtol=0, atol=1e-12):
        errs.append(f"golden state {st[0, 0].tolist()} != {gd['expected_state']}")
    return errs


def check_pure_decay(rec):
    q, k, v, g, beta, s0, cu = _rand_case(11, [7, 5], 1, 2, 6, 5)
    beta = np.zeros_like(beta)
    scale = 0.37
    out, st = rec(q, k, v, g, beta, s0, cu, scale)
    errs = []
    for b in range(2):
        t0, t1 = cu[b], cu[b + 1]
        for h in range(2):
            csum = np.cumsum(g[t0:t1, h])
            exp_state = np.exp(csum[-1]) * s0[b, h]
            if _rel(st[b, h], exp_state) > 1e-13:
                errs.append(f"pure decay state b={b} h={h}")
            qh = scale * q[t0:t1, 0] / np.sqrt(np.sum(q[t0:t1, 0] ** 2, axis=1, keepdims=True) + 1e-6)
            exp_out = np.exp(csum)[:, None] * (qh @ s0[b, h].T)
            if _rel(out[t0:t1, h], exp_out) > 1e-13:
                errs.append(f"pure decay output b={b} h={h}")
    return errs


def check_retrieval(rec):
    """n orthonormal writes with beta = 1, g = 0, then reads q = k_i, beta = 0."""
    from gated_deltanet_chunked_amd.inputs import orthonormal_keys
    dk, dv, n = 16, 8, 12
    keys = orthonormal_keys(n, dk, seed=5)
    rng = np.random.default_rng(6)
    vals = rng.standard_normal((n, dv))
    s0 = rng.standard_normal((1, 1, dv, dk))
    T = 2 * n
    q = np.zeros((T, 1, dk)); k = np.zeros((T, 1, dk)); v = np.zeros((T, 1, dv))
    beta = np.zeros((T, 1)); g = np.zeros((T, 1))
    k[:n, 0] = keys; v[:n, 0] = vals; beta[:n, 0] = 1.0
    q[:n, 0] = rng.standard_normal((n, dk))
    q[n:, 0] = keys; k[n:, 0] = rng.standard_normal((n, dk)); v[n:, 0] = rng.standard_normal((n, dv))
    scale = 0.5
    out, st = rec(q, k, v, g, beta, s0, np.array([0, T], dtype=np.int32), scale, eps=0.0)
    errs = []
    if _rel(st[0, 0] @ keys.T, vals.T) > 1e-13:
        errs.append("retrieval: S k_i != v_i")
    if _rel(out[n:, 0], scale * vals) > 1e-13:
        errs.append("retrieval: read outputs != scale * v_i")
    return errs


def check_single_token(rec):
    q, k, v, g, beta, _, cu = _rand_case(3, [1, 1, 1], 2, 4, 8, 8, state=False)
    scale = 0.8
    out, st = rec(q, k, v, g, beta, None, cu, scale)
    errs = []
    for b in range(3):
        for h in range(4):
            j = h // 2
            kh = k[b, j] / np.sqrt(np.sum(k[b, j] ** 2) + 1e-6)
            qh = scale * q[b, j] / np.sqrt(np.sum(q[b, j] ** 2) + 1e-6)
            if _rel(st[b, h], beta[b, h] * np.outer(v[b, h], kh)) > 1e-14:
                errs.append(f"single token state b={b} h={h}")
            if _rel(out[b, h], beta[b, h] * np.dot(kh, qh) * v[b, h]) > 1e-14:
                errs.append(f"single token output b={b} h={h}")
    return errs


def check_matrix_form(rec):
    q, k, v, g, beta, s0, cu = _rand_case(21, [9, 1, 0, 14], 2, 6, 8, 7)
    o1, s1 = rec(q, k, v, g, beta, s0, cu, 0.3)
    o2, s2 = alt.matrix_form(q, k, v, g, beta, s0, cu, 0.3)
    errs = []
    if _rel(o1, o2) > 1e-12:
        errs.append(f"matrix form output rel {_rel(o1, o2):.3e}")
    if _rel(s1, s2) > 1e-12:
        errs.append(f"matrix form state rel {_rel(s1, s2):.3e}")
    return errs


def check_chunked(rec, Ts=(1, 5, 8, 13, 300), chunks=(1, 2, 4, 8, 128)):
    errs = []
    for T in Ts:
        q, k, v, g, beta, s0, cu = _rand_case(100 + T, [T], 1, 2, 8, 8, A_hi=0.3)
        o1, s1 = rec(q, k, v, g, beta, s0, cu, 0.35)
        for c in chunks:
            o2, s2 = alt.chunked(q, k, v, g, beta, s0, cu, 0.35, chunk=c)
            if _rel(o1, o2) > 1e-11 or _rel(s1, s2) > 1e-11:
                errs.append(f"chunked T={T} chunk={c}: out {_rel(o1, o2):.2e} state {_rel(s1, s2):.2e}")
    return errs


def _unit(num, den):
    return [Fraction(n, den) for n in num]


def _exact_rule(qs, ks, vs, betas, S0):
    """Exact arithmetic on unit keys/queries (eps = 0, scale = 1, g = 0)."""
    S = [row[:] for row in S0]
    outs = []
    for qv, kv, vv, bt in zip(qs, ks, vs, betas):
        u = [sum(S[i][c] * kv[c] for c in range(len(kv))) for i in range(len(S))]
        for i in range(len(S)):
            d = bt * (vv[i] - u[i])
            for c in range(len(kv)):
                S[i][c] += d * kv[c]
        outs.append([sum(S[i][c] * qv[c] for c in range(len(qv))) for i in range(len(S))])
    return outs, S


def check_fraction_bruteforce(rec):
    # unit vectors with rational coordinates: (3,4,0,12)/13, (0,0,3,4)/5, ...
    ks = [_unit([3, 4, 0, 12], 13), _unit([0, 0, 3, 4], 5), _unit([2, -1, 2, 0], 3),
          _unit([1, 2, 2, 4], 5)]
    qs = [_unit([0, 3, 4, 0], 5), _unit([1, 0, 0, 0], 1), _unit([4, 0, 0, 3], 5),
          _unit([-2, 2, 1, 0], 3)]
    vs = [[Fraction(x) for x in row] for row in ([1, -2, 3], [0, 5, -1], [2, 2, 2], [-3, 1, 4])]
    betas = [Fraction(1, 2), Fraction(1, 3), Fraction(3, 4), Fraction(1)]
    S0 = [[Fraction(i - 2 * c, 7) for c in range(4)] for i in range(3)]
    exp_out, exp_S = _exact_rule(qs, ks, vs, betas, S0)
    T = len(ks)
    f = lambda rows: np.array([[float(x) for x in r] for r in rows])
    q = f(qs)[:, None, :]; k = f(ks)[:, None, :]; v = f(vs)[:, None, :]
    beta = np.array([float(b) for b in betas])[:, None]
    out, st = rec(q, k, v, np.zeros((T, 1)), beta, f(S0)[None, None],
                  np.array([0, T], dtype=np.int32), 1.0, eps=0.0)
    errs = []
    if np.max(np.abs(out[:, 0, :] - f(exp_out))) > 1e-14:
        errs.append("fraction brute force output")
    if np.max(np.abs(st[0, 0] - f(exp_S))) > 1e-14:
        errs.append("fraction brute force state")
    return errs


ALL_PINS = [check_golden, check_pure_decay, check_retrieval, check_single_token,
            check_matrix_form, check_chunked, check_fraction_bruteforce]
