"""GPU parity of libgdr against the fp64 oracle, through the C ABI.

Tolerances (relative L2): 1e-4 for float32 inputs, 1e-2 for bfloat16
inputs; outputs and final states are compared separately, over each whole
tensor and for every (sequence, value head) on its own, so an error confined
to one short sequence or one head is not diluted by the rest.  Every case,
the full-size prefill workloads included, is compared on all heads.
"""
import numpy as np
import pytest

import gated_deltanet_chunked_amd as gdr
from gated_deltanet_chunked_amd.inputs import make_inputs, workload_inputs
from tests.gpu_util import (SCALE, TOL, assert_close_per_seq_head, device_tensors, oracle_full,
                            rel_l2, to_f64)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gdr.load()
    yield
    torch.cuda.synchronize()


def _chunk(inp, want_state=True, state="in", l2norm=True):
    import torch
    t = device_tensors(inp)
    s_in = t["state_in"] if state == "in" else None
    out, st = gdr.chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu"], s_in,
                            scale=SCALE, want_state=want_state, l2norm=l2norm)
    torch.cuda.synchronize()
    return to_f64(out), (to_f64(st) if st is not None else None)


def _assert_close(name, got, ref, tol):
    err = rel_l2(got, ref)
    print(f"{name}: rel L2 {err:.3e} (tolerance {tol:.0e})")
    assert np.isfinite(got).all(), f"{name}: non-finite values"
    assert err <= tol, f"{name}: rel L2 {err:.3e} > {tol:.0e}"
    return err


# ----------------------------------------------------------------- prefill


def test_tiny_fp32_workload():
    """B=1, T=512 (4 chunks), Nqk=2, Nv=4, fp32, zero initial state."""
    inp = workload_inputs("tiny")
    out, st = _chunk(inp)
    ro, rs = oracle_full(inp)
    assert_close_per_seq_head(out, ro, st, rs, inp.cu_seqlens, TOL["f32"])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("lengths,Nqk,Nv", [
    ([300, 1, 128, 129, 0, 77, 255], 2, 4),   # ragged tails, empty and one-token sequences
    ([640], 1, 4),                            # G = 4
    ([200, 57], 4, 4),                        # G = 1
    ([128, 256, 384], 2, 2),                  # whole chunks only
    ([1000, 37], 1, 1),                       # a single head
    ([513, 64, 3], 2, 8),                     # Nv = 8 (operator page), G = 4
])
def test_ragged(dtype, lengths, Nqk, Nv):
    inp = make_inputs(lengths, Nqk, Nv, dtype=dtype, seed=11 + len(lengths), state_std=0.01)
    out, st = _chunk(inp)
    ro, rs = oracle_full(inp)
    assert_close_per_seq_head(out, ro, st, rs, inp.cu_seqlens, TOL[dtype])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_large_initial_state(dtype):
    """A state of unit scale (not 0.01) makes the inter-chunk terms dominate."""
    inp = make_inputs([333, 70], 2, 4, dtype=dtype, seed=21, state_std=1.0)
    out, st = _chunk(inp)
    ro, rs = oracle_full(inp)
    assert_close_per_seq_head(out, ro, st, rs, inp.cu_seqlens, TOL[dtype])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_slow_decay(dtype):
    """A ~ U(0, 0.05): gates near 1, the state carries across many chunks."""
    inp = make_inputs([1000], 1, 2, dtype=dtype, seed=22, state_std=0.5, A_range=(0.0, 0.05))
    out, st = _chunk(inp)
    ro, rs = oracle_full(inp)
    assert_close_per_seq_head(out, ro, st, rs, inp.cu_seqlens, TOL[dtype])


def test_no_initial_state_and_no_final_state():
    inp = make_inputs([257, 3], 2, 4, dtype="bf16", seed=23, state_std=0.01)
    out, st = _chunk(inp, want_state=False, state=None)
    assert st is None
    ro, _ = oracle_full(inp, state_in=None)
    assert_close_per_seq_head(out, ro, None, None, inp.cu_seqlens, TOL["bf16"])


def test_without_l2norm():
    """Flag off: q, k are used as given (here pre-normalised rows)."""
    inp = make_inputs([300], 2, 4, dtype="f32", seed=24, state_std=0.01)
    inp.q = (inp.q / np.linalg.norm(inp.q, axis=-1, keepdims=True)).astype(np.float32)
    inp.k = (inp.k / np.linalg.norm(inp.k, axis=-1, keepdims=True)).astype(np.float32)
    out, st = _chunk(inp, l2norm=False)
    ro, rs = oracle_full(inp, l2norm=False)
    assert_close_per_seq_head(out, ro, st, rs, inp.cu_seqlens, TOL["f32"])


def test_in_place_state():
    import torch
    inp = make_inputs([390, 5], 2, 4, dtype="bf16", seed=25, state_std=0.01)
    t = device_tensors(inp)
    s = t["state_in"].clone()
    out, st = gdr.chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu"], s, state_out=s,
                            scale=SCALE)
    torch.cuda.synchronize()
    assert st.data_ptr() == s.data_ptr()
    ro, rs = oracle_full(inp)
    assert_close_per_seq_head(to_f64(out), ro, to_f64(s), rs, inp.cu_seqlens, TOL["bf16"])


def test_empty_input():
    """T = 0: every sequence is empty and its final state is its initial state."""
    import torch
    dev = "cuda:0"
    N, Nqk, Nv = 3, 2, 4
    q = torch.empty((0, Nqk, 128), dtype=torch.bfloat16, device=dev)
    v = torch.empty((0, Nv, 128), dtype=torch.bfloat16, device=dev)
    g = torch.empty((0, Nv), dtype=torch.float32, device=dev)
    cu = torch.zeros(N + 1, dtype=torch.int32, device=dev)
    s0 = torch.randn((N, Nv, 128, 128), device=dev)
    out, st = gdr.chunk_fwd(q, q, v, g, g, cu, s0, scale=SCALE)
    torch.cuda.synchronize()
    assert out.shape == (0, Nv, 128)
    assert torch.equal(st, s0)
    out, st = gdr.chunk_fwd(q, q, v, g, g, cu, None, scale=SCALE)
    torch.cuda.synchronize()
    assert torch.count_nonzero(st).item() == 0


def test_prefill_workload_full():
    """T=4096, Nqk=16, Nv=32, bf16, initial state N(0, 0.01): every head compared."""
    inp = workload_inputs("prefill")
    out, st = _chunk(inp)
    ro, rs = oracle_full(inp)
    assert_close_per_seq_head(out, ro, st, rs, inp.cu_seqlens, TOL["bf16"])


@pytest.mark.parametrize("name", ["varlen", "long"])
def test_full_size_all_heads(name):
    """Varlen (8 sequences, lengths U[1, 8192]) and long-context (T=32768)
    workloads at full size, in the launch configuration the benchmark times,
    compared on every sequence and every value head."""
    inp = workload_inputs(name)
    out, st = _chunk(inp)
    ro, rs = oracle_full(inp)
    assert_close_per_seq_head(out, ro, st, rs, inp.cu_seqlens, TOL["bf16"], name=name)


# ------------------------------------------------------------------ decode


def _step(inp, in_place=True):
    import torch
    t = device_tensors(inp)
    s = t["state_in"].clone()
    s_out = s if in_place else torch.empty_like(s)
    out = gdr.recurrent_step(t["q"], t["k"], t["v"], t["g"], t["beta"], s, state_out=s_out,
                             scale=SCALE)
    torch.cuda.synchronize()
    if not in_place:
        assert torch.equal(s, t["state_in"]), "state_in modified by an out-of-place step"
    return to_f64(out), to_f64(s_out)


@pytest.mark.parametrize("in_place", [True, False])
def test_decode_workload(in_place):
    """256 sequences x 1 token, Nqk=16, Nv=32, bf16, fp32 states N(0, 0.01)."""
    inp = workload_inputs("decode")
    out, st = _step(inp, in_place)
    ro, rs = oracle_full(inp)
    assert_close_per_seq_head(out, ro, st, rs, inp.cu_seqlens, TOL["bf16"])


def test_decode_fp32_small():
    inp = make_inputs([1] * 5, 1, 3, dtype="f32", seed=31, state_std=1.0)
    out, st = _step(inp)
    ro, rs = oracle_full(inp)
    assert_close_per_seq_head(out, ro, st, rs, inp.cu_seqlens, TOL["f32"])


def test_chunk_equals_repeated_steps():
    """The prefill of a sequence equals its tokens fed one by one to the decode step."""
    import torch
    inp = make_inputs([150], 2, 4, dtype="f32", seed=32, state_std=0.1)
    out, st = _chunk(inp)
    t = device_tensors(inp)
    s = t["state_in"].clone()
    outs = []
    for i in range(inp.T):
        outs.append(gdr.recurrent_step(t["q"][i:i + 1].contiguous(), t["k"][i:i + 1].contiguous(),
                                       t["v"][i:i + 1].contiguous(), t["g"][i:i + 1].contiguous(),
                                       t["beta"][i:i + 1].contiguous(), s, scale=SCALE))
    torch.cuda.synchronize()
    steps = to_f64(torch.cat(outs))
    _assert_close("out", out, steps, 1e-4)
    _assert_close("state", st, to_f64(s), 1e-4)


# ------------------------------------------------------- timed entry points


@pytest.mark.parametrize("lengths", [[640], [300, 1, 129]], ids=["one-sequence", "packed"])
def test_timed_entry_points_match_untimed(lengths):
    """gdr_chunk_fwd_timed and gdr_recurrent_step_timed (the benchmark's
    calls) compute exactly what the plain calls compute, and report one
    positive duration per kernel and a span that covers them."""
    import torch
    inp = make_inputs(lengths, 2, 4, dtype="bf16", seed=41, state_std=0.01)
    t = device_tensors(inp)
    args = (t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu"], t["state_in"])
    out0, st0 = gdr.chunk_fwd(*args, scale=SCALE)
    tim = []
    out1, st1 = gdr.chunk_fwd(*args, scale=SCALE, timings=tim)
    torch.cuda.synchronize()
    assert torch.equal(out0, out1) and torch.equal(st0, st1)
    kernels = [(n, ms) for n, ms in tim if n != "span"]
    span = [ms for n, ms in tim if n == "span"]
    expect = {"intra", "inter"} | ({"table"} if len(lengths) > 1 else set())
    assert {n for n, _ in kernels} == expect
    assert len(span) == 1 and all(ms > 0 for _, ms in kernels)
    assert span[0] >= max(ms for _, ms in kernels)

    dec = make_inputs([1] * 6, 2, 4, dtype="bf16", seed=43, state_std=0.01)
    d = device_tensors(dec)
    s_a, s_b = d["state_in"].clone(), d["state_in"].clone()
    o_a = gdr.recurrent_step(d["q"], d["k"], d["v"], d["g"], d["beta"], s_a, scale=SCALE)
    tim = []
    o_b = gdr.recurrent_step(d["q"], d["k"], d["v"], d["g"], d["beta"], s_b, scale=SCALE,
                             timings=tim)
    torch.cuda.synchronize()
    assert torch.equal(o_a, o_b) and torch.equal(s_a, s_b)
    assert len(tim) == 1 and tim[0][0] == "decode" and tim[0][1] > 0


# ------------------------------------------------- decode, bf16 state cache


def _bf16_state_step(inp, s_bf16, in_place=True):
    """One step through gdr_recurrent_step_bf16_state; returns (out, new state)
    as fp64 arrays (the state's bf16 values exactly)."""
    import torch
    t = device_tensors(inp, with_state=False)
    s_in = s_bf16.clone()
    s_out = s_in if in_place else torch.empty_like(s_in)
    out = gdr.recurrent_step(t["q"], t["k"], t["v"], t["g"], t["beta"], s_in, state_out=s_out,
                             scale=SCALE)
    torch.cuda.synchronize()
    if not in_place:
        assert torch.equal(s_in, s_bf16), "state_in modified by an out-of-place step"
    return to_f64(out), to_f64(s_out)


def _check_rounded_state(got, exact):
    """The stored state is the new state rounded to bf16.  The kernel rounds
    its fp32 value, the oracle the exact one, so the two may differ where fp32
    error moves a value across a rounding boundary: near a tie, or near zero
    where the update alpha S + delta kh^T cancels.  Rounding is monotone, so
    every bf16 value the kernel may store lies in [round(x - e), round(x + e)],
    e bounding the fp32 error (here 1e-5 of the head's largest |S'|, about 100
    times fp32's error on terms of that size); and such differences must be
    rare."""
    import oracle
    ref = oracle.round_bf16(exact)
    assert np.array_equal(oracle.round_bf16(got), got), "stored state is not bf16"
    diff = got != ref
    frac = float(diff.mean())
    print(f"state: {diff.sum()} of {diff.size} values round differently ({frac:.2e})")
    assert frac <= 1e-3
    e = 1e-5 * np.abs(exact).max(axis=(-2, -1), keepdims=True)
    lo, hi = oracle.round_bf16(exact - e), oracle.round_bf16(exact + e)
    bad = (got < lo) | (got > hi)
    assert not bad.any(), f"{int(bad.sum())} values outside the fp32 error band"


@pytest.mark.parametrize("in_place", [True, False])
def test_decode_bf16_state_workload(in_place):
    """The decode workload (256 sequences, Nqk=16, Nv=32, bf16) with the state
    stored in bf16 (the workload's states rounded once)."""
    import oracle
    import torch
    inp = workload_inputs("decode")
    s0 = torch.from_numpy(inp.state_in).to("cuda:0").to(torch.bfloat16)
    s0_64 = to_f64(s0)
    out, st = _bf16_state_step(inp, s0, in_place)
    ro, exact = oracle.recurrent(inp.q, inp.k, inp.v, inp.g, inp.beta, s0_64, inp.cu_seqlens, SCALE)
    _assert_close("out", out, ro, TOL["bf16"])
    _assert_close("state", st, exact, TOL["bf16"])
    _check_rounded_state(st, exact)


def test_decode_bf16_state_fp32_inputs():
    import oracle
    import torch
    inp = make_inputs([1] * 6, 2, 4, dtype="f32", seed=41, state_std=1.0)
    s0 = torch.from_numpy(inp.state_in).to("cuda:0").to(torch.bfloat16)
    out, st = _bf16_state_step(inp, s0)
    ro, exact = oracle.recurrent(inp.q, inp.k, inp.v, inp.g, inp.beta, to_f64(s0), inp.cu_seqlens,
                                 SCALE)
    _assert_close("out", out, ro, TOL["f32"])
    _check_rounded_state(st, exact)


def test_decode_bf16_state_chained_steps():
    """Ten steps in a row, each rounding the stored state, against the
    oracle's bf16-state step chained the same way."""
    import oracle
    import torch
    steps, N, Nqk, Nv = 10, 8, 2, 4
    s = torch.from_numpy(make_inputs([1] * N, Nqk, Nv, seed=50, state_std=0.1).state_in)
    s = s.to("cuda:0").to(torch.bfloat16)
    ref = to_f64(s)
    for i in range(steps):
        inp = make_inputs([1] * N, Nqk, Nv, seed=51 + i, state_std=0.1)
        out, st = _bf16_state_step(inp, s)
        ro, ref = oracle.recurrent_step_bf16_state(inp.q, inp.k, inp.v, inp.g, inp.beta, ref, SCALE)
        _assert_close(f"out step {i}", out, ro, TOL["bf16"])
        s = torch.from_numpy(st).to("cuda:0").to(torch.bfloat16)
    _assert_close("state after 10 steps", st, ref, TOL["bf16"])


# ------------------------------------------- several tokens per sequence


def _multi(inp, state="in", want_state=True, l2norm=True, in_place=False):
    import torch
    t = device_tensors(inp)
    s_in = t["state_in"] if state == "in" else None
    s_out = s_in if (in_place and s_in is not None) else None
    out, st = gdr.recurrent_multi(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu"], s_in,
                                  scale=SCALE, state_out=s_out, want_state=want_state,
                                  l2norm=l2norm)
    torch.cuda.synchronize()
    return to_f64(out), (to_f64(st) if st is not None else None)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_multi_token_ragged(dtype):
    """Short packed sequences (0 to 16 tokens), the verification shape of
    speculative decoding, with initial states."""
    inp = make_inputs([3, 1, 0, 16, 7, 2, 5, 4], 2, 4, dtype=dtype, seed=61, state_std=0.5)
    out, st = _multi(inp)
    ro, rs = oracle_full(inp)
    assert_close_per_seq_head(out, ro, st, rs, inp.cu_seqlens, TOL[dtype])


def test_multi_token_no_states_and_no_norm():
    inp = make_inputs([5, 9, 1], 1, 2, dtype="f32", seed=62, state_std=0.5)
    out, st = _multi(inp, state=None, want_state=False, l2norm=False)
    assert st is None
    ro, _ = oracle_full(inp, state_in=None, l2norm=False)
    _assert_close("out", out, ro, TOL["f32"])


def test_multi_token_in_place_and_long_sequence():
    """The state updated in place; one sequence far longer than the loop is
    meant for (still exact, only slower)."""
    inp = make_inputs([300, 2], 2, 4, dtype="bf16", seed=63, state_std=0.5)
    out, st = _multi(inp, in_place=True)
    ro, rs = oracle_full(inp)
    assert_close_per_seq_head(out, ro, st, rs, inp.cu_seqlens, TOL["bf16"])


def test_multi_token_verification_workload():
    """256 sequences x 4 tokens, Nqk=16, Nv=32, bf16, fp32 states: the decode
    workload with four tokens per sequence, compared in full."""
    inp = make_inputs([4] * 256, 16, 32, dtype="bf16", seed=64, state_std=0.01)
    out, st = _multi(inp)
    ro, rs = oracle_full(inp)
    assert_close_per_seq_head(out, ro, st, rs, inp.cu_seqlens, TOL["bf16"])


def test_multi_token_matches_chunk_fwd():
    """The token loop and the chunkwise form agree on the same packed batch."""
    inp = make_inputs([16, 3, 11, 8], 2, 4, dtype="f32", seed=65, state_std=0.5)
    o_m, s_m = _multi(inp)
    o_c, s_c = _chunk(inp)
    _assert_close("out", o_m, o_c, TOL["f32"])
    _assert_close("state", s_m, s_c, TOL["f32"])


# -------------------------------------- decode with the conv/gate prologue


def _conv_step(p, in_place=True):
    import torch
    dt = torch.bfloat16 if p.dtype == "bf16" else torch.float32
    dv = lambda x, t=None: None if x is None else torch.from_numpy(x).to("cuda:0", t or torch.float32)
    x, cs, w = dv(p.mixed_qkv, dt), dv(p.conv_state, dt), dv(p.conv_w, dt)
    cb = dv(p.conv_b, dt)
    s = dv(p.state_in)
    s_out = s if in_place else torch.empty_like(s)
    cs_keep = cs.clone()
    out, cs_out = gdr.recurrent_step_conv(x, cs, w, cb, dv(p.a), dv(p.b), dv(p.A_log),
                                          dv(p.dt_bias), s, state_out=s_out, scale=SCALE)
    torch.cuda.synchronize()
    assert torch.equal(cs, cs_keep), "conv_state_in modified"
    return to_f64(out), to_f64(s_out), to_f64(cs_out)


def _conv_oracle(p):
    import oracle
    return oracle.recurrent_step_conv(p.mixed_qkv, p.conv_state, p.conv_w, p.conv_b, p.a, p.b,
                                      p.A_log, p.dt_bias, p.state_in, p.Nqk, p.Nv, SCALE,
                                      activation_bf16=(p.dtype == "bf16"))


@pytest.mark.parametrize("in_place", [True, False])
def test_decode_conv_workload(in_place):
    """The decode workload (256 sequences, Nqk=16, Nv=32, bf16) with the conv
    update and gates fused in front; the new conv windows are bit-exact."""
    from gated_deltanet_chunked_amd.inputs import prologue_inputs
    p = prologue_inputs(256, 16, 32, seed=71)
    out, st, cs = _conv_step(p, in_place)
    ro, rs, rcs = _conv_oracle(p)
    assert_close_per_seq_head(out, ro, st, rs, np.arange(257), TOL["bf16"])
    assert np.array_equal(cs, rcs), "conv windows differ"


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_conv_with_bias(dtype):
    from gated_deltanet_chunked_amd.inputs import prologue_inputs
    p = prologue_inputs(5, 2, 4, dtype=dtype, seed=72, bias=True, state_std=0.5)
    out, st, cs = _conv_step(p)
    ro, rs, rcs = _conv_oracle(p)
    assert_close_per_seq_head(out, ro, st, rs, np.arange(6), TOL[dtype])
    assert np.array_equal(cs, rcs), "conv windows differ"


def test_multi_token_empty_input():
    """T = 0 (the token buffers may be empty): every state passes through."""
    import torch
    dev = "cuda:0"
    N, Nqk, Nv = 3, 2, 4
    q = torch.empty((0, Nqk, 128), dtype=torch.bfloat16, device=dev)
    v = torch.empty((0, Nv, 128), dtype=torch.bfloat16, device=dev)
    g = torch.empty((0, Nv), dtype=torch.float32, device=dev)
    cu = torch.zeros(N + 1, dtype=torch.int32, device=dev)
    s0 = torch.randn((N, Nv, 128, 128), dtype=torch.float32, device=dev)
    out, st = gdr.recurrent_multi(q, q, v, g, g, cu, s0, scale=SCALE)
    torch.cuda.synchronize()
    assert out.shape == (0, Nv, 128)
    assert torch.equal(st, s0)


# ------------------------------------- conv/gate prologue of the chunked path


def _conv_prefill(p, in_place=False, want_state=True):
    import torch
    dt = torch.bfloat16 if p.dtype == "bf16" else torch.float32
    dv = lambda x, t=None: None if x is None else torch.from_numpy(x).to("cuda:0", t or torch.float32)
    x, w, cb = dv(p.mixed_qkv, dt), dv(p.conv_w, dt), dv(p.conv_b, dt)
    cs = dv(p.conv_state, dt)
    cs_keep = None if cs is None else cs.clone()
    res = gdr.conv_prefill(x, cs, w, cb, dv(p.a), dv(p.b), dv(p.A_log), dv(p.dt_bias),
                           torch.from_numpy(p.cu_seqlens).to("cuda:0"),
                           conv_state_out=cs if in_place else None, want_conv_state=want_state)
    torch.cuda.synchronize()
    if cs is not None and not in_place:
        assert torch.equal(cs, cs_keep), "conv_state_in modified"
    return res


def _conv_prefill_oracle(p):
    import oracle
    return oracle.prefill_prologue(p.mixed_qkv, p.conv_state, p.conv_w, p.conv_b, p.a, p.b, p.A_log,
                                   p.dt_bias, p.cu_seqlens, p.Nqk, p.Nv,
                                   activation_bf16=(p.dtype == "bf16"))


def _check_conv_prefill(res, ref, dtype, want_state=True):
    q, k, v, g, beta, cs = res
    rq, rk, rv, rg, rb, rcs = ref
    for name, got, want in (("q", q, rq), ("k", k, rk), ("v", v, rv)):
        _assert_close(name, to_f64(got), want, TOL[dtype])
    # gates: fp32 exp/log1p against fp64
    _assert_close("g", to_f64(g), rg, 1e-5)
    _assert_close("beta", to_f64(beta), rb, 1e-5)
    if want_state:
        assert np.array_equal(to_f64(cs), rcs), "conv windows differ"
    else:
        assert cs is None


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_conv_prefill_ragged(dtype):
    """Packed sequences shorter and longer than the window, one empty, cached
    windows and a conv bias."""
    from gated_deltanet_chunked_amd.inputs import prefill_prologue_inputs
    p = prefill_prologue_inputs([5, 0, 2, 1, 9, 300], 2, 4, dtype=dtype, seed=81, bias=True)
    _check_conv_prefill(_conv_prefill(p), _conv_prefill_oracle(p), dtype)


def test_conv_prefill_no_cache_and_in_place():
    from gated_deltanet_chunked_amd.inputs import prefill_prologue_inputs
    p = prefill_prologue_inputs([7, 3], 1, 2, seed=82, cached=False)
    _check_conv_prefill(_conv_prefill(p, want_state=False), _conv_prefill_oracle(p), "bf16",
                        want_state=False)
    p = prefill_prologue_inputs([7, 0, 3, 2], 1, 2, seed=83)
    _check_conv_prefill(_conv_prefill(p, in_place=True), _conv_prefill_oracle(p), "bf16")


def test_conv_prefill_then_chunk_fwd():
    """The prologue feeding the chunkwise path at the prefill shape (T = 4096,
    Nqk = 16, Nv = 32, bf16), end to end against the oracle's prologue and
    recurrence."""
    import oracle
    import torch
    from gated_deltanet_chunked_amd.inputs import prefill_prologue_inputs
    p = prefill_prologue_inputs([4096], 16, 32, seed=84)
    q, k, v, g, beta, _ = _conv_prefill(p, want_state=False)
    cu = torch.from_numpy(p.cu_seqlens).to("cuda:0")
    out, st = gdr.chunk_fwd(q, k, v, g, beta, cu, None, scale=SCALE)
    torch.cuda.synchronize()
    rq, rk, rv, rg, rb, _ = _conv_prefill_oracle(p)
    ro, rs = oracle.recurrent(rq, rk, rv, rg, rb, None, p.cu_seqlens, SCALE)
    assert_close_per_seq_head(to_f64(out), ro, to_f64(st), rs, p.cu_seqlens, TOL["bf16"])
