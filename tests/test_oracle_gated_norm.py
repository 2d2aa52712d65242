"""Pins of the oracle's gated RMSNorm (CPU only): the norm in front of the
output projection of the Qwen3-Next blog post (RMSNormGated in sections 1 and
6, the ``_norm`` of its Zero-Centered RMSNorm section) with a SiLU output gate.

The pins are hand-worked values, torch's own ``rms_norm`` and ``silu`` in fp64,
and invariants of the definition (scale and sign of x, the role of eps, the
per-head reduction), chosen so that a dropped term, a sum in place of a mean,
eps outside the root, a sigmoid in place of SiLU or a reduction over the wrong
axis fails at least one.  ``recurrent_step_gated`` is pinned through the
direction and length of its output against the separately pinned recurrence.
"""
import math

import numpy as np
import torch
import torch.nn.functional as F

import oracle


def _silu(t):
    return t / (1.0 + math.exp(-t))


def test_hand_example():
    """x = (3, 4): mean(x^2) = 12.5; with eps = 0 the normalised row is
    (3, 4) / sqrt(12.5) = (0.8485.., 1.1313..).  Gate z = (0, 1) zeroes the
    first entry and multiplies the second by silu(1) = 0.7310585786300049."""
    y = oracle.gated_rmsnorm([[3.0, 4.0]], [[0.0, 1.0]], eps=0.0)
    assert y.shape == (1, 2)
    assert y[0, 0] == 0.0
    assert math.isclose(y[0, 1], 4.0 / math.sqrt(12.5) * 0.7310585786300049, rel_tol=1e-15)
    assert math.isclose(y[0, 1], 0.8270983654302005, rel_tol=1e-14)


def test_constant_row_normalises_to_its_sign():
    """A row of equal entries c has rms |c|: with eps = 0 the norm gives
    sign(c) in every entry, so y = sign(c) * w * silu(z).  z = ln 3 gives
    sigmoid = 3/4 and silu = 0.75 ln 3."""
    D = 16
    w = np.linspace(0.5, 2.0, D)
    z = np.full((2, D), math.log(3.0))
    x = np.stack([np.full(D, 2.5), np.full(D, -0.125)])
    y = oracle.gated_rmsnorm(x, z, w, eps=0.0)
    s = 0.75 * math.log(3.0)
    assert np.allclose(y[0], w * s, rtol=1e-14, atol=0)
    assert np.allclose(y[1], -w * s, rtol=1e-14, atol=0)


def test_eps_inside_the_root():
    """x = (a, a) with a^2 = eps: mean(x^2) + eps = 2 eps, so the norm gives
    1/sqrt(2) (eps added under the root, not to the root).  A large gate z makes
    silu(z) = z to 1e-15."""
    eps = 1e-6
    a = math.sqrt(eps)
    y = oracle.gated_rmsnorm([[a, a]], [[40.0, 40.0]], eps=eps)
    assert np.allclose(y, 40.0 / math.sqrt(2.0), rtol=1e-14, atol=0)
    assert oracle.NORM_EPS == 1e-6


def test_matches_torch_rms_norm_and_silu():
    """Random rows, several heads: equal to torch's rms_norm over the last
    dimension (eps inside the root) times silu(z), in fp64."""
    rng = np.random.default_rng(11)
    T, H, D = 5, 3, 128
    x = rng.standard_normal((T, H, D)) * rng.uniform(0.01, 10.0, (T, H, 1))
    z = rng.standard_normal((T, H, D)) * 3
    w = rng.uniform(-2.0, 2.0, D)
    got = oracle.gated_rmsnorm(x, z, w)
    tx, tz, tw = (torch.from_numpy(a) for a in (x, z, w))
    ref = F.rms_norm(tx, (D,), tw, eps=1e-6) * F.silu(tz)
    assert np.allclose(got, ref.numpy(), rtol=1e-13, atol=1e-15)
    # weight None is a weight of ones
    ref1 = F.rms_norm(tx, (D,), None, eps=1e-6) * F.silu(tz)
    assert np.allclose(oracle.gated_rmsnorm(x, z), ref1.numpy(), rtol=1e-13, atol=1e-15)


def test_scale_and_sign_invariance_at_eps_zero():
    """With eps = 0 the norm is unchanged by x -> alpha x for alpha > 0 and
    flips sign with x; rows are independent (a change in one head leaves the
    others)."""
    rng = np.random.default_rng(12)
    x = rng.standard_normal((4, 2, 32))
    z = rng.standard_normal((4, 2, 32))
    y = oracle.gated_rmsnorm(x, z, eps=0.0)
    assert np.allclose(oracle.gated_rmsnorm(7.5 * x, z, eps=0.0), y, rtol=1e-13, atol=1e-15)
    assert np.allclose(oracle.gated_rmsnorm(-x, z, eps=0.0), -y, rtol=1e-13, atol=1e-15)
    x2 = x.copy()
    x2[1, 0] *= 1e3
    x2[2, 1, 5] += 4.0
    y2 = oracle.gated_rmsnorm(x2, z, eps=0.0)
    same = np.ones((4, 2), dtype=bool)
    same[2, 1] = False
    assert np.allclose(y2[same], y[same], rtol=1e-13, atol=1e-15)
    assert not np.allclose(y2[2, 1], y[2, 1])


def test_unit_gate_gives_unit_rms():
    """With w = 1 and silu(z) = 1 in every entry, each row of y has rms
    sqrt(m / (m + eps)), m = mean(x^2): 1 up to eps."""
    zs = 1.278464542761074   # silu(zs) = 1 (root of t * sigmoid(t) = 1)
    assert math.isclose(_silu(zs), 1.0, rel_tol=1e-15)
    rng = np.random.default_rng(13)
    x = rng.standard_normal((6, 64)) * 1e-3
    y = oracle.gated_rmsnorm(x, np.full_like(x, zs))
    m = np.mean(x * x, axis=-1)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=-1)), np.sqrt(m / (m + 1e-6)), rtol=1e-14)


def test_bf16_output_rounding():
    rng = np.random.default_rng(14)
    x = rng.standard_normal((3, 128))
    z = rng.standard_normal((3, 128))
    y = oracle.gated_rmsnorm(x, z)
    yb = oracle.gated_rmsnorm(x, z, out_bf16=True)
    ref = torch.from_numpy(y).to(torch.bfloat16).double().numpy()
    assert np.array_equal(yb, ref)


def _decode_inputs(rng, N=3, Nqk=2, Nv=4, D=128):
    q = rng.standard_normal((N, Nqk, D))
    k = rng.standard_normal((N, Nqk, D))
    v = rng.standard_normal((N, Nv, D))
    g = -rng.uniform(0.0, 1.0, (N, Nv))
    beta = rng.uniform(0.0, 1.0, (N, Nv))
    s0 = rng.standard_normal((N, Nv, D, D)) * 0.1
    z = rng.standard_normal((N, Nv, D)) * 2
    w = rng.uniform(0.5, 1.5, D)
    return q, k, v, g, beta, s0, z, w


def test_gated_step_direction_and_length():
    """The gated decode step's y, divided by w * silu(z), is parallel to the
    recurrence's output o (bf16-cast when out_bf16) and has rms
    sqrt(m / (m + eps)); its state equals the recurrence's."""
    rng = np.random.default_rng(15)
    q, k, v, g, beta, s0, z, w = _decode_inputs(rng)
    N = q.shape[0]
    scale = 1 / math.sqrt(128)
    o, s_ref = oracle.recurrent(q, k, v, g, beta, s0, np.arange(N + 1, dtype=np.int32), scale)
    for out_bf16 in (False, True):
        y, s = oracle.recurrent_step_gated(q, k, v, g, beta, s0, z, w, scale, out_bf16=out_bf16)
        assert np.array_equal(s, s_ref)
        u = y / (w * (z / (1 + np.exp(-z))))
        ob = torch.from_numpy(o).to(torch.bfloat16).double().numpy() if out_bf16 else o
        cos = np.sum(u * ob, -1) / np.linalg.norm(u, axis=-1) / np.linalg.norm(ob, axis=-1)
        assert np.all(np.abs(cos - 1) < 1e-13)
        m = np.mean(ob * ob, -1)
        assert np.allclose(np.sqrt(np.mean(u * u, -1)), np.sqrt(m / (m + 1e-6)), rtol=1e-12)
        if out_bf16:
            # the cast is taken before the norm: u is not parallel to the fp64 o
            cos64 = np.sum(u * o, -1) / np.linalg.norm(u, axis=-1) / np.linalg.norm(o, axis=-1)
            assert np.max(np.abs(cos64 - 1)) > 1e-9
