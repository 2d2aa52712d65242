"""Pins of the oracle's bf16-state decode step (CPU only).

The step is the fp64 rule followed by one rounding of the stored state to
bfloat16 (generic "Gated DeltaNet" article, section 6.3: a bf16 state
cache).  The rounding is pinned against hand-worked ties and against torch's
own fp32 -> bf16 conversion; the composition against closed forms that fix
where the rounding happens.
"""
import math

import numpy as np
import pytest
import torch

import oracle


def test_round_bf16_hand_values():
    r = oracle.round_bf16
    one = 1.0
    # the spacing of bf16 values in [1, 2) is 2**-7
    assert r(one + 2.0 ** -9) == one                       # below half: down
    assert r(one + 2.0 ** -8) == one                       # tie, 1.0 is even
    assert r(one + 3 * 2.0 ** -8) == one + 2.0 ** -6       # tie, up to the even neighbour
    assert r(one + 2.0 ** -8 + 2.0 ** -30) == one + 2.0 ** -7   # just above half: up
    assert r(-(one + 2.0 ** -8)) == -one                   # sign symmetric
    assert r(0.0) == 0.0 and r(3.0) == 3.0 and r(-0.15625) == -0.15625   # exact values stay
    # subnormal range: the spacing stays 2**-133
    assert r(2.0 ** -130 + 2.0 ** -133) == 2.0 ** -130 + 2.0 ** -133
    assert r(0.5 * 2.0 ** -133) == 0.0                     # tie to even (0)
    assert r(1.5 * 2.0 ** -133) == 2.0 ** -132             # tie to even (2 quanta)
    # the largest finite value, and the tie above it, which overflows
    big = (2 - 2.0 ** -7) * 2.0 ** 127
    assert r(big) == big
    assert np.isinf(r((2 - 2.0 ** -8) * 2.0 ** 127))


def test_round_bf16_matches_torch_conversion():
    rng = np.random.default_rng(11)
    mag = np.exp2(rng.uniform(-140, 120, size=20000))
    x = (mag * rng.choice([-1.0, 1.0], size=mag.shape)).astype(np.float32)
    # exact ties: a bf16 value plus half its spacing (representable in fp32)
    base = torch.from_numpy(x[:5000]).to(torch.bfloat16).to(torch.float64).numpy()
    _, e = np.frexp(base)
    ties = (base + np.ldexp(1.0, np.maximum(e, -125) - 9)).astype(np.float32)
    allx = np.concatenate([x, ties]).astype(np.float64)
    want = torch.from_numpy(allx.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.round_bf16(allx)
    assert np.array_equal(got, want)


def _case(seed, N=3, Nqk=2, Nv=4, D=8):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((N, Nqk, D))
    k = rng.standard_normal((N, Nqk, D))
    v = rng.standard_normal((N, Nv, D))
    g = -rng.uniform(0.0, 1.0, (N, Nv))
    beta = rng.uniform(0.0, 1.0, (N, Nv))
    s0 = oracle.round_bf16(rng.standard_normal((N, Nv, D, D)))
    return q, k, v, g, beta, s0


def test_no_decay_no_write_keeps_the_state():
    q, k, v, g, beta, s0 = _case(1)
    _, s1 = oracle.recurrent_step_bf16_state(q, k, v, np.zeros_like(g), np.zeros_like(beta), s0, 0.3)
    assert np.array_equal(s1, s0)


def test_halving_decay_is_exact():
    q, k, v, g, beta, s0 = _case(2)
    _, s1 = oracle.recurrent_step_bf16_state(q, k, v, np.full_like(g, -math.log(2.0)),
                                             np.zeros_like(beta), s0, 0.3)
    assert np.array_equal(s1, s0 / 2)


def test_single_token_from_zero_closed_form():
    """From S = 0: S' = beta v kh^T, o = beta (kh . qh) v.  The output comes from
    the unrounded state; only the stored state is rounded."""
    q, k, v, g, beta, _ = _case(3)
    N, Nqk, D = q.shape
    Nv = v.shape[1]
    scale = 0.37
    out, s1 = oracle.recurrent_step_bf16_state(q, k, v, g, beta, np.zeros((N, Nv, D, D)), scale)
    for n in range(N):
        for h in range(Nv):
            j = h // (Nv // Nqk)
            kh = k[n, j] / math.sqrt(k[n, j] @ k[n, j] + oracle.EPS)
            qh = scale * q[n, j] / math.sqrt(q[n, j] @ q[n, j] + oracle.EPS)
            exact = beta[n, h] * np.outer(v[n, h], kh)
            assert np.allclose(out[n, h], beta[n, h] * (kh @ qh) * v[n, h], rtol=1e-12, atol=1e-14)
            assert np.array_equal(s1[n, h], oracle.round_bf16(exact))


def test_state_within_half_a_bf16_spacing_of_the_exact_state():
    q, k, v, g, beta, s0 = _case(4)
    exact_out, exact = oracle.recurrent(q, k, v, g, beta, s0, np.arange(q.shape[0] + 1), 0.3)
    out, s1 = oracle.recurrent_step_bf16_state(q, k, v, g, beta, s0, 0.3)
    assert np.allclose(out, exact_out, rtol=1e-12, atol=1e-14)
    # bf16 keeps 8 significant bits: a rounding moves x = m 2**e (1/2 <= |m| < 1)
    # by at most half the spacing 2**(e - 8), i.e. by at most 2**-8 |x|
    assert np.all(np.abs(s1 - exact) <= 2.0 ** -8 * np.abs(exact))
    assert np.max(np.abs(s1 - exact) / np.abs(exact)) > 2.0 ** -9   # the bound is nearly reached
    assert np.array_equal(oracle.round_bf16(s1), s1)


@pytest.mark.parametrize("l2norm", [True, False])
def test_bf16_state_steps_track_the_fp64_recurrence(l2norm):
    """Several bf16-state steps stay close to the fp64 recurrence of the same
    tokens (the rounding errors do not grow under decay)."""
    rng = np.random.default_rng(5)
    N, Nqk, Nv, D, steps = 2, 1, 2, 8, 20
    s = oracle.round_bf16(0.1 * rng.standard_normal((N, Nv, D, D)))
    qs = rng.standard_normal((steps, N, Nqk, D))
    ks = rng.standard_normal((steps, N, Nqk, D))
    vs = rng.standard_normal((steps, N, Nv, D))
    gs = -rng.uniform(0.05, 0.5, (steps, N, Nv))
    bs = rng.uniform(0.0, 1.0, (steps, N, Nv))
    ref = s.copy()
    for t in range(steps):
        _, s = oracle.recurrent_step_bf16_state(qs[t], ks[t], vs[t], gs[t], bs[t], s, 0.3,
                                                l2norm=l2norm)
        _, ref = oracle.recurrent(qs[t], ks[t], vs[t], gs[t], bs[t], ref, np.arange(N + 1), 0.3,
                                  l2norm=l2norm)
    assert oracle.rel_l2(s, ref) < 1e-2
