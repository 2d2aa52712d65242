"""GPU tests of the optional device-side contract checks (gdr_set_debug /
GDR_DEBUG): with them on, a call whose cu_seqlens or gates break the
contract returns GDR_ERR_CONTRACT before any other launch, leaves its outputs
untouched and names the broken contract; a call within the contract gives the
same results as with the checks off.  Inputs that break the contract are only
ever passed with the checks on: the checking kernel reads exactly N + 1
offsets and T * Nv gates, and nothing else runs."""
import numpy as np
import pytest

import gated_deltanet_chunked_amd as gdr
from gated_deltanet_chunked_amd.inputs import make_inputs
from tests.gpu_util import SCALE, device_tensors

pytestmark = pytest.mark.gpu

CONTRACT = -5


@pytest.fixture(autouse=True)
def _debug_on():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    before = gdr.set_debug(True)
    yield
    gdr.set_debug(before)
    torch.cuda.synchronize()


def _chunk(t, cu, g, out, sout):
    return gdr.chunk_fwd(t["q"], t["k"], t["v"], g, t["beta"], cu, t["state_in"], scale=SCALE,
                         out=out, state_out=sout)


@pytest.mark.parametrize("case,bit", [("first_not_zero", 1), ("decreasing", 2), ("last_not_T", 4),
                                      ("positive_gate", 8), ("nan_gate", 8), ("neg_inf_gate", 8)])
def test_chunk_fwd_rejects_broken_contract(case, bit):
    import torch
    inp = make_inputs([100, 200, 60], 2, 4, dtype="bf16", seed=61)
    t = device_tensors(inp)
    cu = t["cu"].clone()
    g = t["g"].clone()
    if case == "first_not_zero":
        cu[0] = 3
    elif case == "decreasing":
        cu[1], cu[2] = 250, 120
    elif case == "last_not_T":
        cu[-1] = inp.T - 1
    elif case == "positive_gate":
        g[37, 2] = 0.25
    elif case == "nan_gate":
        g[359, 3] = float("nan")
    else:
        g[0, 0] = float("-inf")
    out = torch.full((inp.T, inp.Nv, 128), 7.0, dtype=torch.bfloat16, device="cuda:0")
    sout = torch.full_like(t["state_in"], 7.0)
    with pytest.raises(gdr.GdrError) as e:
        _chunk(t, cu, g, out, sout)
    assert e.value.status == CONTRACT
    assert gdr.debug_broken() == bit
    torch.cuda.synchronize()
    assert bool((out == 7.0).all()) and bool((sout == 7.0).all()), "outputs touched"


def test_checked_calls_match_unchecked():
    """Within the contract the checks change nothing: chunk_fwd,
    recurrent_multi and recurrent_step give the same bits with and without
    them, and report no broken contract."""
    import torch
    inp = make_inputs([100, 0, 300, 1], 2, 4, dtype="bf16", seed=62)
    t = device_tensors(inp)
    o1, s1 = gdr.chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu"], t["state_in"],
                           scale=SCALE)
    m1, ms1 = gdr.recurrent_multi(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu"],
                                  t["state_in"], scale=SCALE)
    assert gdr.debug_broken() == 0
    gdr.set_debug(False)
    o2, s2 = gdr.chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu"], t["state_in"],
                           scale=SCALE)
    m2, ms2 = gdr.recurrent_multi(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu"],
                                  t["state_in"], scale=SCALE)
    gdr.set_debug(True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    assert torch.equal(m1, m2) and torch.equal(ms1, ms2)
    dec = make_inputs([1] * 8, 2, 4, dtype="bf16", seed=63)
    d = device_tensors(dec)
    sa, sb = d["state_in"].clone(), d["state_in"].clone()
    ya = gdr.recurrent_step(d["q"], d["k"], d["v"], d["g"], d["beta"], sa, scale=SCALE)
    gdr.set_debug(False)
    yb = gdr.recurrent_step(d["q"], d["k"], d["v"], d["g"], d["beta"], sb, scale=SCALE)
    gdr.set_debug(True)
    torch.cuda.synchronize()
    assert torch.equal(ya, yb) and torch.equal(sa, sb)


def test_other_entry_points_check_their_inputs():
    """recurrent_multi (cu_seqlens and gates), the decode step (gates) and
    the prefill prologue (cu_seqlens) reject broken values the same way."""
    import torch
    inp = make_inputs([5, 7], 2, 4, dtype="bf16", seed=64)
    t = device_tensors(inp)
    cu = t["cu"].clone()
    cu[1] = 13
    with pytest.raises(gdr.GdrError) as e:
        gdr.recurrent_multi(t["q"], t["k"], t["v"], t["g"], t["beta"], cu, t["state_in"],
                            scale=SCALE)
    assert e.value.status == CONTRACT and gdr.debug_broken() == 2
    dec = make_inputs([1] * 4, 2, 4, dtype="bf16", seed=65)
    d = device_tensors(dec)
    g = d["g"].clone()
    g[3, 1] = 1e-3
    s = d["state_in"].clone()
    with pytest.raises(gdr.GdrError) as e:
        gdr.recurrent_step(d["q"], d["k"], d["v"], g, d["beta"], s, scale=SCALE)
    assert e.value.status == CONTRACT and gdr.debug_broken() == 8
    torch.cuda.synchronize()
    assert torch.equal(s, d["state_in"])
    from gated_deltanet_chunked_amd.inputs import prefill_prologue_inputs
    pp = prefill_prologue_inputs([5, 7], 2, 4, seed=66)
    x = torch.from_numpy(pp.mixed_qkv).to("cuda:0", torch.bfloat16)
    w = torch.from_numpy(pp.conv_w).to("cuda:0", torch.bfloat16)
    f = {k: torch.from_numpy(getattr(pp, k)).to("cuda:0") for k in ("a", "b", "A_log", "dt_bias")}
    pcu = torch.from_numpy(pp.cu_seqlens).to("cuda:0")
    pcu[0] = 1
    with pytest.raises(gdr.GdrError) as e:
        gdr.conv_prefill(x, None, w, None, f["a"], f["b"], f["A_log"], f["dt_bias"], pcu)
    assert e.value.status == CONTRACT and gdr.debug_broken() == 1
