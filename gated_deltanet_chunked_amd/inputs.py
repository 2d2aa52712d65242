"""Seeded synthetic inputs for the gated delta rule.

This module only draws random numbers and rounds them to the storage dtype.
It holds none of the rule's arithmetic, so both the CPU oracle and the HIP
path can be fed from it.

Recipe (shared by every test and the benchmark):

* draws come from ``numpy.random.default_rng(seed)`` (PCG64) in a fixed order:
  sequence lengths (varlen only), q, k, v (standard normal), a, b (standard
  normal, one per token and value head), A (uniform, one per value head),
  then the initial state (``state_std`` * standard normal) when requested;
* the gates follow the module initialisation of the Qwen3-Next blog post
  ("Code-Qwen3-Next", section 1 and the gate lines of section 4):
  dt_bias = 1, A ~ U(A_lo, A_hi), g = -A * softplus(a + dt_bias),
  beta = sigmoid(b); both are computed in float64 and stored as float32;
* for bf16 inputs, q, k and v are rounded to bfloat16 (round to nearest even)
  and those rounded values are what both sides receive.
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Sequence

import numpy as np

D = 128


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    out = r.astype(np.uint32).view(np.float32)
    nan = np.isnan(x)
    if nan.any():
        out = out.copy()
        out[nan] = np.nan
    return out


def _softplus(x: np.ndarray) -> np.ndarray:
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


@dataclasses.dataclass
class GdrInputs:
    """One workload: packed tokens delimited by ``cu_seqlens``."""

    q: np.ndarray            # [T, Nqk, D] float32 (bf16-representable when dtype == "bf16")
    k: np.ndarray            # [T, Nqk, D]
    v: np.ndarray            # [T, Nv, D]
    g: np.ndarray            # [T, Nv] float32, natural-log decay (<= 0)
    beta: np.ndarray         # [T, Nv] float32 in (0, 1)
    state_in: Optional[np.ndarray]  # [N, Nv, D, D] float32 (row = value index) or None
    cu_seqlens: np.ndarray   # [N + 1] int32
    dtype: str               # "f32" or "bf16": storage type of q, k, v and out
    seed: int
    name: str = ""

    @property
    def T(self) -> int:
        return int(self.q.shape[0])

    @property
    def N(self) -> int:
        return int(self.cu_seqlens.shape[0] - 1)

    @property
    def Nqk(self) -> int:
        return int(self.q.shape[1])

    @property
    def Nv(self) -> int:
        return int(self.v.shape[1])


def make_inputs(lengths: Sequence[int], Nqk: int, Nv: int, *, dtype: str = "bf16",
                seed: int = 0, state_std: Optional[float] = 0.01,
                A_range=(0.0, 16.0), dk: int = D, dv: int = D,
                name: str = "") -> GdrInputs:
    """Draw one workload with the given per-sequence lengths."""
    lengths = [int(x) for x in lengths]
    rng = np.random.default_rng(seed)
    return _draw(rng, lengths, Nqk, Nv, dtype, seed, state_std, A_range, dk, dv, name)


def _draw(rng, lengths, Nqk, Nv, dtype, seed, state_std, A_range, dk, dv, name):
    if dtype not in ("f32", "bf16"):
        raise ValueError(f"unknown dtype {dtype!r}")
    T = int(sum(lengths))
    N = len(lengths)
    cu = np.zeros(N + 1, dtype=np.int32)
    cu[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64)).astype(np.int32)
    q = rng.standard_normal((T, Nqk, dk)).astype(np.float32)
    k = rng.standard_normal((T, Nqk, dk)).astype(np.float32)
    v = rng.standard_normal((T, Nv, dv)).astype(np.float32)
    a = rng.standard_normal((T, Nv))
    b = rng.standard_normal((T, Nv))
    A = rng.uniform(A_range[0], A_range[1], size=Nv)
    state = None
    if state_std is not None:
        state = (state_std * rng.standard_normal((N, Nv, dv, dk))).astype(np.float32)
    dt_bias = 1.0
    g = (-A[None, :] * _softplus(a + dt_bias)).astype(np.float32)
    beta = (1.0 / (1.0 + np.exp(-b))).astype(np.float32)
    if dtype == "bf16":
        q, k, v = round_to_bf16(q), round_to_bf16(k), round_to_bf16(v)
    return GdrInputs(q=q, k=k, v=v, g=g, beta=beta, state_in=state, cu_seqlens=cu,
                     dtype=dtype, seed=seed, name=name)


def make_gate(shape, *, dtype: str = "bf16", seed: int = 0, weight: bool = True):
    """Inputs of the gated RMSNorm after the rule: the output gate z
    (2 * standard normal, so that SiLU(z) spans its curved part and its linear
    tail) of ``shape`` [..., D] and, with ``weight``, a per-channel weight
    U(0.5, 1.5) of [D] (None otherwise: the norm's initial ones).  Rounded to
    bf16 when dtype is "bf16".  Returns (z, w) as float32 arrays."""
    rng = np.random.default_rng(seed)
    z = (2.0 * rng.standard_normal(shape)).astype(np.float32)
    w = rng.uniform(0.5, 1.5, size=shape[-1]).astype(np.float32) if weight else None
    if dtype == "bf16":
        z = round_to_bf16(z)
        w = None if w is None else round_to_bf16(w)
    return z, w


# The named full-size workloads the benchmark times and the parity tests run,
# each with its own seed.
WORKLOADS = {
    "tiny": "tiny chunk fwd: B=1 T=512 Nqk=2 Nv=4 D=128 fp32, zero initial state",
    "prefill": "prefill: B=1 T=4096 Nqk=16 Nv=32 D=128 bf16",
    "varlen": "varlen packed prefill: 8 sequences, lengths U[1,8192], Nqk=16 Nv=32 bf16",
    "long": "long-context prefill: B=1 T=32768 Nqk=16 Nv=32 bf16",
    "decode": "decode step: N=256 sequences x 1 token, Nqk=16 Nv=32 bf16, fp32 states",
}
WORKLOAD_SEEDS = {"tiny": 0, "prefill": 1, "varlen": 2, "long": 3, "decode": 4}


def workload_inputs(name: str) -> GdrInputs:
    """The seeded inputs of the named workload (see WORKLOADS)."""
    if name not in WORKLOADS:
        raise ValueError(f"no workload {name!r}")
    c = WORKLOAD_SEEDS[name]
    rng = np.random.default_rng(c)
    what = WORKLOADS[name]
    if name == "tiny":
        return _draw(rng, [512], 2, 4, "f32", c, None, (0.0, 16.0), D, D, what)
    if name == "prefill":
        return _draw(rng, [4096], 16, 32, "bf16", c, 0.01, (0.0, 16.0), D, D, what)
    if name == "varlen":
        lengths = rng.integers(1, 8192, size=8, endpoint=True).tolist()
        return _draw(rng, lengths, 16, 32, "bf16", c, 0.01, (0.0, 16.0), D, D, what)
    if name == "long":
        return _draw(rng, [32768], 16, 32, "bf16", c, 0.01, (0.0, 16.0), D, D, what)
    return _draw(rng, [1] * 256, 16, 32, "bf16", c, 0.01, (0.0, 16.0), D, D, what)


def orthonormal_keys(n: int, dk: int, seed: int) -> np.ndarray:
    """n <= dk orthonormal rows (QR of a Gaussian), float64."""
    rng = np.random.default_rng(seed)
    m = rng.standard_normal((dk, dk))
    qm, r = np.linalg.qr(m)
    qm = qm * np.sign(np.diag(r))[None, :]
    return np.ascontiguousarray(qm.T[:n])


@dataclasses.dataclass
class PrologueInputs:
    """Raw inputs of a decode step with its conv/gate prologue (no arithmetic
    of the prologue or the rule is done here)."""

    mixed_qkv: np.ndarray     # [N, C] float32 (bf16-representable for "bf16"), C = (2 Nqk + Nv) D
    conv_state: np.ndarray    # [N, C, K] same
    conv_w: np.ndarray        # [C, K] same
    conv_b: Optional[np.ndarray]   # [C] same, or None
    a: np.ndarray             # [N, Nv] float32
    b: np.ndarray             # [N, Nv] float32
    A_log: np.ndarray         # [Nv] float32
    dt_bias: np.ndarray       # [Nv] float32
    state_in: np.ndarray      # [N, Nv, D, D] float32
    Nqk: int
    Nv: int
    dtype: str


def prologue_inputs(N: int, Nqk: int, Nv: int, *, dtype: str = "bf16", seed: int = 0,
                    K: int = 4, bias: bool = False, state_std: float = 0.01) -> PrologueInputs:
    """Seeded draw: activations and cached windows N(0, 1); conv kernels
    U(-1/sqrt(K), 1/sqrt(K)) (PyTorch's default conv init; Qwen3-Next's conv
    has no bias, so none unless asked); a, b N(0, 1); A ~ U(0, 16) per value
    head stored as A_log = log(A); dt_bias = 1; states state_std * N(0, 1)."""
    rng = np.random.default_rng(seed)
    C = (2 * Nqk + Nv) * D
    x = rng.standard_normal((N, C)).astype(np.float32)
    cs = rng.standard_normal((N, C, K)).astype(np.float32)
    lim = 1.0 / np.sqrt(K)
    w = rng.uniform(-lim, lim, (C, K)).astype(np.float32)
    cb = rng.uniform(-lim, lim, C).astype(np.float32) if bias else None
    a = rng.standard_normal((N, Nv)).astype(np.float32)
    b = rng.standard_normal((N, Nv)).astype(np.float32)
    A_log = np.log(rng.uniform(0.0, 16.0, Nv)).astype(np.float32)
    dt_bias = np.ones(Nv, dtype=np.float32)
    state = (state_std * rng.standard_normal((N, Nv, D, D))).astype(np.float32)
    if dtype == "bf16":
        x, cs, w = round_to_bf16(x), round_to_bf16(cs), round_to_bf16(w)
        cb = None if cb is None else round_to_bf16(cb)
    return PrologueInputs(mixed_qkv=x, conv_state=cs, conv_w=w, conv_b=cb, a=a, b=b, A_log=A_log,
                          dt_bias=dt_bias, state_in=state, Nqk=Nqk, Nv=Nv, dtype=dtype)


@dataclasses.dataclass
class PrefillPrologueInputs:
    """Raw inputs of the conv/gate prologue over packed sequences."""

    mixed_qkv: np.ndarray     # [T, C] float32 (bf16-representable for "bf16")
    conv_state: Optional[np.ndarray]   # [N, C, K] same, or None
    conv_w: np.ndarray        # [C, K]
    conv_b: Optional[np.ndarray]       # [C] or None
    a: np.ndarray             # [T, Nv] float32
    b: np.ndarray             # [T, Nv] float32
    A_log: np.ndarray         # [Nv] float32
    dt_bias: np.ndarray       # [Nv] float32
    cu_seqlens: np.ndarray    # [N + 1] int32
    Nqk: int
    Nv: int
    dtype: str


def prefill_prologue_inputs(lengths: Sequence[int], Nqk: int, Nv: int, *, dtype: str = "bf16",
                            seed: int = 0, K: int = 4, bias: bool = False,
                            cached: bool = True) -> PrefillPrologueInputs:
    """Seeded draw with the distributions of ``prologue_inputs``, for packed
    sequences of the given lengths; ``cached=False`` gives no cached windows."""
    rng = np.random.default_rng(seed)
    lengths = [int(x) for x in lengths]
    T, N = int(sum(lengths)), len(lengths)
    cu = np.zeros(N + 1, dtype=np.int32)
    cu[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64)).astype(np.int32)
    C = (2 * Nqk + Nv) * D
    x = rng.standard_normal((T, C)).astype(np.float32)
    cs = rng.standard_normal((N, C, K)).astype(np.float32) if cached else None
    lim = 1.0 / np.sqrt(K)
    w = rng.uniform(-lim, lim, (C, K)).astype(np.float32)
    cb = rng.uniform(-lim, lim, C).astype(np.float32) if bias else None
    a = rng.standard_normal((T, Nv)).astype(np.float32)
    b = rng.standard_normal((T, Nv)).astype(np.float32)
    A_log = np.log(rng.uniform(0.0, 16.0, Nv)).astype(np.float32)
    dt_bias = np.ones(Nv, dtype=np.float32)
    if dtype == "bf16":
        x, w = round_to_bf16(x), round_to_bf16(w)
        cs = None if cs is None else round_to_bf16(cs)
        cb = None if cb is None else round_to_bf16(cb)
    return PrefillPrologueInputs(mixed_qkv=x, conv_state=cs, conv_w=w, conv_b=cb, a=a, b=b,
                                 A_log=A_log, dt_bias=dt_bias, cu_seqlens=cu, Nqk=Nqk, Nv=Nv,
                                 dtype=dtype)
