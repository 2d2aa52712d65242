"""Helpers shared by the GPU tests: move seeded inputs to the device, call the
library through its binding, and run the fp64 oracle on the same inputs (whole,
or on a subset of value heads, which the rule treats independently)."""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np

import oracle
from gated_deltanet_chunked_amd.inputs import GdrInputs

SCALE = 128 ** -0.5
TOL = {"f32": 1e-4, "bf16": 1e-2}


def device_tensors(inp: GdrInputs, device="cuda:0", with_state: bool = True) -> Dict[str, object]:
    import torch
    dt = torch.bfloat16 if inp.dtype == "bf16" else torch.float32
    t = {
        "q": torch.from_numpy(inp.q).to(device=device, dtype=dt).contiguous(),
        "k": torch.from_numpy(inp.k).to(device=device, dtype=dt).contiguous(),
        "v": torch.from_numpy(inp.v).to(device=device, dtype=dt).contiguous(),
        "g": torch.from_numpy(inp.g).to(device),
        "beta": torch.from_numpy(inp.beta).to(device),
        "cu": torch.from_numpy(inp.cu_seqlens).to(device),
        "state_in": None,
    }
    if with_state and inp.state_in is not None:
        t["state_in"] = torch.from_numpy(inp.state_in).to(device)
    return t


def to_f64(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float64).cpu().numpy()


def oracle_full(inp: GdrInputs, state_in: Optional[np.ndarray] = "default", l2norm: bool = True):
    s0 = inp.state_in if isinstance(state_in, str) else state_in
    return oracle.recurrent(inp.q, inp.k, inp.v, inp.g, inp.beta, s0, inp.cu_seqlens, SCALE,
                            l2norm=l2norm)


def oracle_heads(inp: GdrInputs, heads: Sequence[int], seqs: Optional[Sequence[int]] = None):
    """Oracle outputs for value heads ``heads`` (and sequences ``seqs``) only.

    Returns {(b, h): (out [len_b, Dv], state [Dv, Dk])}.
    """
    G = inp.Nv // inp.Nqk
    cu = inp.cu_seqlens
    seqs = range(inp.N) if seqs is None else seqs
    res = {}
    for b in seqs:
        t0, t1 = int(cu[b]), int(cu[b + 1])
        for h in heads:
            j = h // G
            s0 = None if inp.state_in is None else inp.state_in[b:b + 1, h:h + 1]
            o, s = oracle.recurrent(inp.q[t0:t1, j:j + 1], inp.k[t0:t1, j:j + 1],
                                    inp.v[t0:t1, h:h + 1], inp.g[t0:t1, h:h + 1],
                                    inp.beta[t0:t1, h:h + 1], s0,
                                    np.array([0, t1 - t0], np.int32), SCALE)
            res[(b, h)] = (o[:, 0], s[0, 0])
    return res


rel_l2 = oracle.rel_l2


def per_seq_head_rel(got_out, ref_out, got_st, ref_st, cu) -> Dict[str, np.ndarray]:
    """Relative L2 error of every (sequence, value head) separately.

    Returns {"out": [N, Nv], "state": [N, Nv]} (state only when both states are
    given).  Empty sequences have no output and get NaN there.  Where the
    reference is all zeros the absolute L2 error stands in (as in rel_l2).
    """
    cu = np.asarray(cu, dtype=np.int64)
    N = cu.shape[0] - 1
    res = {}
    d2 = ((np.asarray(got_out, np.float64) - ref_out) ** 2).sum(axis=-1)   # [T, Nv]
    r2 = (np.asarray(ref_out, np.float64) ** 2).sum(axis=-1)
    Nv = d2.shape[1] if d2.ndim == 2 else ref_out.shape[1]
    eo = np.full((N, Nv), np.nan)
    for b in range(N):
        t0, t1 = cu[b], cu[b + 1]
        if t1 > t0:
            num = np.sqrt(d2[t0:t1].sum(axis=0))
            den = np.sqrt(r2[t0:t1].sum(axis=0))
            eo[b] = np.where(den > 0, num / np.where(den > 0, den, 1.0), num)
    res["out"] = eo
    if got_st is not None and ref_st is not None:
        num = np.sqrt(((np.asarray(got_st, np.float64) - ref_st) ** 2).sum(axis=(-2, -1)))
        den = np.sqrt((np.asarray(ref_st, np.float64) ** 2).sum(axis=(-2, -1)))
        res["state"] = np.where(den > 0, num / np.where(den > 0, den, 1.0), num)
    return res


def assert_close_per_seq_head(got_out, ref_out, got_st, ref_st, cu, tol, name=""):
    """Relative L2 within ``tol`` over each whole tensor AND for every
    (sequence, value head) on its own, so an error confined to one short
    sequence or one head is not diluted by the rest.  Prints the worst."""
    for what, g, r in (("out", got_out, ref_out), ("state", got_st, ref_st)):
        if g is None or r is None:
            continue
        assert np.isfinite(g).all(), f"{name} {what}: non-finite values"
        err = rel_l2(g, r)
        print(f"{name} {what}: rel L2 {err:.3e} (tolerance {tol:.0e})")
        assert err <= tol, f"{name} {what}: rel L2 {err:.3e} > {tol:.0e}"
    per = per_seq_head_rel(got_out, ref_out, got_st, ref_st, cu)
    for what, e in per.items():
        if np.all(np.isnan(e)):
            continue
        b, h = np.unravel_index(np.nanargmax(e), e.shape)
        worst = float(e[b, h])
        print(f"{name} {what}: worst (sequence, head) ({b}, {h}) rel L2 {worst:.3e}")
        assert worst <= tol, f"{name} {what}: (sequence {b}, head {h}) rel L2 {worst:.3e} > {tol:.0e}"
    return per
