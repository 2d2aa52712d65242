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
