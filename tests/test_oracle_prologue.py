"""Pins of the oracle's decode prologue (CPU only): the causal conv update with
SiLU and the gate functions of the Qwen3-Next blog post (sections 3 and 4),
checked against hand-worked values and torch's own conv1d, silu, sigmoid and
softplus in fp64."""
import math

import numpy as np
import torch
import torch.nn.functional as F

import oracle


def test_conv_window_hand_example():
    """One channel of each part, kernel size 4: the window [1, 2, 3, 4] gains 5
    and drops 1; a kernel picking the oldest entry gives silu(2)."""
    Nqk, Nv, D = 1, 1, 1
    C = 3
    cs = np.array([[[1.0, 2.0, 3.0, 4.0], [0.0, 0.0, 0.0, 1.0], [2.0, 2.0, 2.0, 2.0]]])
    x = np.array([[5.0, -1.0, 0.5]])
    w = np.array([[1.0, 0.0, 0.0, 0.0], [0.0, 0.0, 0.0, 1.0], [0.25, 0.25, 0.25, 0.25]])
    q, k, v, _, _, new = oracle.decode_prologue(x, cs, w, None, np.zeros((1, 1)), np.zeros((1, 1)),
                                                np.zeros(1), np.zeros(1), Nqk, Nv, D,
                                                activation_bf16=False)
    assert np.array_equal(new[0], [[2, 3, 4, 5], [0, 0, 1, -1], [2, 2, 2, 0.5]])
    silu = lambda t: t / (1 + math.exp(-t))
    assert math.isclose(q[0, 0, 0], silu(2.0), rel_tol=1e-15)          # 1.7615941559557646
    assert math.isclose(q[0, 0, 0], 1.7615941559557646, rel_tol=1e-15)
    assert math.isclose(k[0, 0, 0], silu(-1.0), rel_tol=1e-15)
    assert math.isclose(v[0, 0, 0], silu(0.25 * (2 + 2 + 2 + 0.5)), rel_tol=1e-15)
    assert C == 3


def test_conv_matches_torch_conv1d_and_silu():
    """The decode branch equals torch's grouped conv1d over the concatenated
    window (last output position), bias included, then silu."""
    rng = np.random.default_rng(3)
    Nqk, Nv, D, K, N = 2, 4, 8, 4, 3
    C = (2 * Nqk + Nv) * D
    x = rng.standard_normal((N, C))
    cs = rng.standard_normal((N, C, K))
    w = rng.standard_normal((C, K))
    bias = rng.standard_normal(C)
    q, k, v, _, _, new = oracle.decode_prologue(x, cs, w, bias, np.zeros((N, Nv)), np.zeros((N, Nv)),
                                                np.zeros(Nv), np.zeros(Nv), Nqk, Nv, D,
                                                activation_bf16=False)
    win = torch.from_numpy(np.concatenate([cs, x[:, :, None]], axis=2))
    ref = F.conv1d(win, torch.from_numpy(w).unsqueeze(1), torch.from_numpy(bias), groups=C)
    ref = F.silu(ref[:, :, -1]).numpy()
    got = np.concatenate([q.reshape(N, -1), k.reshape(N, -1), v.reshape(N, -1)], axis=1)
    assert np.allclose(got, ref, rtol=1e-13, atol=1e-14)
    assert np.array_equal(new, win.numpy()[:, :, -K:])


def test_activation_rounding_is_bf16():
    rng = np.random.default_rng(4)
    Nqk, Nv, D, K, N = 1, 2, 4, 4, 2
    C = (2 * Nqk + Nv) * D
    args = (rng.standard_normal((N, C)), rng.standard_normal((N, C, K)), rng.standard_normal((C, K)),
            None, np.zeros((N, Nv)), np.zeros((N, Nv)), np.zeros(Nv), np.zeros(Nv), Nqk, Nv, D)
    q0, k0, v0, *_ = oracle.decode_prologue(*args, activation_bf16=False)
    q1, k1, v1, *_ = oracle.decode_prologue(*args, activation_bf16=True)
    for exact, rounded in ((q0, q1), (k0, k1), (v0, v1)):
        want = torch.from_numpy(exact).to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
        # fp64 -> bf16 directly can differ from fp64 -> fp32 -> bf16 only at a
        # double-rounding tie, which random values do not hit
        assert np.array_equal(rounded, want)


def test_gates_hand_values_and_torch():
    Nv = 5
    A_log = np.array([0.0, math.log(2.0), 0.0, 1.0, -3.0])
    dt_bias = np.array([0.0, 0.0, 0.0, 1.0, 0.5])
    a = np.array([[0.0, 0.0, 60.0, -60.0, 0.3]])
    b = np.array([[0.0, 2.0, -40.0, 40.0, -0.7]])
    C = (2 + Nv) * 1
    _, _, _, g, beta, _ = oracle.decode_prologue(np.zeros((1, C)), np.zeros((1, C, 4)),
                                                 np.zeros((C, 4)), None, a, b, A_log, dt_bias,
                                                 1, Nv, 1, activation_bf16=False)
    # softplus(0) = ln 2, with A = exp(0) = 1: g = -ln 2, exp(g) = 1/2
    assert math.isclose(g[0, 0], -math.log(2.0), rel_tol=1e-15)
    assert math.isclose(g[0, 1], -2 * math.log(2.0), rel_tol=1e-15)   # A = 2
    assert math.isclose(g[0, 2], -60.0, rel_tol=1e-15)               # softplus(60) = 60 + e^-60
    assert g[0, 3] < 0 and math.isclose(g[0, 3], -math.e * math.log1p(math.exp(-59.0)), rel_tol=1e-12)
    assert beta[0, 0] == 0.5
    assert math.isclose(beta[0, 1], 1 / (1 + math.exp(-2.0)), rel_tol=1e-15)
    ref_g = -torch.exp(torch.from_numpy(A_log)) * F.softplus(torch.from_numpy(a + dt_bias))
    assert np.allclose(g, ref_g.numpy(), rtol=1e-13, atol=0)
    assert np.allclose(beta, torch.sigmoid(torch.from_numpy(b)).numpy(), rtol=1e-13, atol=1e-300)


def test_fused_step_from_zero_state_closed_form():
    """Zero conv kernels leave silu(bias) in every channel; from S = 0 one step
    gives o = beta (kh . qh) v."""
    rng = np.random.default_rng(5)
    Nqk, Nv, D, K, N = 1, 2, 4, 4, 2
    C = (2 * Nqk + Nv) * D
    bias = rng.standard_normal(C)
    a = rng.standard_normal((N, Nv))
    b = rng.standard_normal((N, Nv))
    A_log = rng.standard_normal(Nv)
    dt_bias = rng.standard_normal(Nv)
    out, st, _ = oracle.recurrent_step_conv(rng.standard_normal((N, C)),
                                            rng.standard_normal((N, C, K)), np.zeros((C, K)), bias,
                                            a, b, A_log, dt_bias, np.zeros((N, Nv, D, D)), Nqk, Nv,
                                            0.5, activation_bf16=False)
    y = bias / (1 + np.exp(-bias))
    qv, kv = y[:D], y[D:2 * D]
    kh = kv / math.sqrt(kv @ kv + oracle.EPS)
    qh = 0.5 * qv / math.sqrt(qv @ qv + oracle.EPS)
    for n in range(N):
        for h in range(Nv):
            vv = y[2 * D + h * D:2 * D + (h + 1) * D]
            bt = 1 / (1 + math.exp(-b[n, h]))
            assert np.allclose(out[n, h], bt * (kh @ qh) * vv, rtol=1e-12, atol=1e-15)
            assert np.allclose(st[n, h], bt * np.outer(vv, kh), rtol=1e-12, atol=1e-15)


def test_prefill_conv_matches_torch_conv1d_with_cached_window():
    """Per sequence: torch's grouped conv1d over (cached window, tokens), the
    outputs at the token positions, bias, silu; the new window is the last K
    values.  Ragged lengths, including an empty sequence and ones shorter than
    the window."""
    rng = np.random.default_rng(8)
    Nqk, Nv, D, K = 1, 2, 4, 4
    C = (2 * Nqk + Nv) * D
    lengths = [5, 0, 2, 1, 9]
    cu = np.concatenate([[0], np.cumsum(lengths)])
    T = int(cu[-1])
    x = rng.standard_normal((T, C))
    cs = rng.standard_normal((len(lengths), C, K))
    w = rng.standard_normal((C, K))
    bias = rng.standard_normal(C)
    q, k, v, _, _, new = oracle.prefill_prologue(x, cs, w, bias, np.zeros((T, Nv)),
                                                 np.zeros((T, Nv)), np.zeros(Nv), np.zeros(Nv), cu,
                                                 Nqk, Nv, D, activation_bf16=False)
    got = np.concatenate([q.reshape(T, -1), k.reshape(T, -1), v.reshape(T, -1)], axis=1)
    for n, L in enumerate(lengths):
        seq = torch.from_numpy(np.concatenate([cs[n], x[cu[n]:cu[n + 1]].T], axis=1))[None]
        ref = F.conv1d(seq, torch.from_numpy(w).unsqueeze(1), torch.from_numpy(bias), groups=C)
        ref = F.silu(ref[0, :, 1:]).numpy().T                 # outputs at the L token positions
        assert ref.shape == (L, C)
        assert np.allclose(got[cu[n]:cu[n + 1]], ref, rtol=1e-13, atol=1e-14)
        assert np.array_equal(new[n], seq[0, :, -K:].numpy())


def test_prefill_equals_repeated_decode_prologue():
    """Token by token, the decode branch gives the same outputs and windows."""
    rng = np.random.default_rng(9)
    Nqk, Nv, D, K, L = 1, 1, 2, 4, 6
    C = (2 * Nqk + Nv) * D
    x = rng.standard_normal((L, C))
    cs = rng.standard_normal((1, C, K))
    w = rng.standard_normal((C, K))
    a = rng.standard_normal((L, Nv))
    b = rng.standard_normal((L, Nv))
    A_log, dt_bias = rng.standard_normal(Nv), rng.standard_normal(Nv)
    pq, pk, pv, pg, pb, pnew = oracle.prefill_prologue(x, cs, w, None, a, b, A_log, dt_bias,
                                                       [0, L], Nqk, Nv, D)
    st = cs
    for t in range(L):
        dq, dk, dv, dg, db, st = oracle.decode_prologue(x[t:t + 1], st, w, None, a[t:t + 1],
                                                        b[t:t + 1], A_log, dt_bias, Nqk, Nv, D)
        assert np.array_equal(dq[0], pq[t]) and np.array_equal(dk[0], pk[t])
        assert np.array_equal(dv[0], pv[t])
        assert np.allclose(dg[0], pg[t], rtol=1e-15) and np.allclose(db[0], pb[t], rtol=1e-15)
    assert np.array_equal(st, pnew)
