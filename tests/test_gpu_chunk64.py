"""GPU parity of the chunkwise forward with 64-token chunks (GDR_FLAG_CHUNK64,
the Blog's torch_chunk_gated_delta_rule default chunk_size=64) against the
fp64 oracle, through the C ABI.  The chunkwise form is exact for any chunk
length, so the oracle is the same per-token recurrence and the tolerances
are those of the 128-token path (relative L2 1e-4 for float32, 1e-2 for
bf16, per (sequence, value head)); the two chunk lengths also agree with
each other."""
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


def _chunk(inp, chunk, timings=None):
    import torch
    t = device_tensors(inp)
    out, st = gdr.chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu"], t["state_in"],
                            scale=SCALE, chunk=chunk, timings=timings)
    torch.cuda.synchronize()
    return to_f64(out), to_f64(st)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("lengths,Nqk,Nv", [
    ([1, 63, 64, 65, 300, 0, 129], 2, 4),    # around the 64-token boundary, empty and 1-token
    ([640], 1, 4),                          # one sequence: no chunk table
    ([200, 57], 4, 4),
])
def test_chunk64_ragged(dtype, lengths, Nqk, Nv):
    inp = make_inputs(lengths, Nqk, Nv, dtype=dtype, seed=71 + len(lengths), state_std=0.01)
    out, st = _chunk(inp, 64)
    ro, rs = oracle_full(inp)
    assert_close_per_seq_head(out, ro, st, rs, inp.cu_seqlens, TOL[dtype], name=f"L=64 {dtype}")


def test_chunk64_slow_decay_long():
    """A ~ U(0, 0.05) over 2000 tokens: 32 chunks of 64 carry the state."""
    inp = make_inputs([2000], 1, 2, dtype="bf16", seed=75, state_std=0.5, A_range=(0.0, 0.05))
    out, st = _chunk(inp, 64)
    ro, rs = oracle_full(inp)
    assert_close_per_seq_head(out, ro, st, rs, inp.cu_seqlens, TOL["bf16"], name="L=64 slow decay")


def test_chunk64_prefill_workload_all_heads():
    """T=4096, Nqk=16, Nv=32, bf16 (64 chunks of 64 tokens per head): every
    head against the oracle, and against the 128-token call."""
    inp = workload_inputs("prefill")
    o64, s64 = _chunk(inp, 64)
    ro, rs = oracle_full(inp)
    assert_close_per_seq_head(o64, ro, s64, rs, inp.cu_seqlens, TOL["bf16"], name="L=64 T=4096")
    o128, s128 = _chunk(inp, 128)
    e_o, e_s = rel_l2(o64, o128), rel_l2(s64, s128)
    print(f"L=64 vs L=128: out {e_o:.2e}, state {e_s:.2e}")
    assert e_o <= TOL["bf16"] and e_s <= TOL["bf16"]


def test_chunk64_timed_and_no_alloc_match():
    """The timed entry point and the no-allocation entry point give the same
    bits as gdr_chunk_fwd with 64-token chunks."""
    import torch
    inp = make_inputs([300, 1, 700], 2, 4, dtype="bf16", seed=76, state_std=0.01)
    o, s = _chunk(inp, 64)
    tim = []
    o2, s2 = _chunk(inp, 64, timings=tim)
    assert np.array_equal(o, o2) and np.array_equal(s, s2)
    assert any(n == "intra" for n, _ in tim) and tim[-1][0] == "span"
    t = device_tensors(inp)
    out = torch.empty((inp.T, inp.Nv, 128), dtype=torch.bfloat16, device="cuda:0")
    sout = torch.empty_like(t["state_in"])
    gdr.chunk_fwd_no_alloc(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu"], t["state_in"], out,
                           sout, scale=SCALE, chunk=64)
    torch.cuda.synchronize()
    assert np.array_equal(to_f64(out), o) and np.array_equal(to_f64(sout), s)


def test_chunk64_odd_segments_all_heads():
    """T = 4160 (65 chunks of 64 tokens) at Nqk = 16, Nv = 32: the segments
    hold 33 and 32 chunk slots, so the first segment ends with a pair whose
    second chunk is absent, and the state crosses a segment boundary in the
    middle of the sequence.  Every head against the oracle."""
    inp = make_inputs([65 * 64], 16, 32, dtype="bf16", seed=77, state_std=0.01)
    out, st = _chunk(inp, 64)
    ro, rs = oracle_full(inp)
    assert_close_per_seq_head(out, ro, st, rs, inp.cu_seqlens, TOL["bf16"], name="L=64 odd segments")
