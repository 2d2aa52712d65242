"""gdr_chunk_fwd_no_alloc, the chunkwise forward whose workspace is the
library's fixed device array: through the C ABI it gives what gdr_chunk_fwd
gives on the same inputs, call after call (the array keeps the previous
call's contents, and a smaller call follows a larger one), and it refuses
sizes that do not fit the array before touching the GPU."""
import ctypes

import numpy as np
import pytest

import gated_deltanet_chunked_amd as gdr
from gated_deltanet_chunked_amd.inputs import make_inputs
from tests.gpu_util import SCALE, TOL, assert_close_per_seq_head, device_tensors, oracle_full, to_f64

WS_SMALL = -3


def _both(inp, with_states=True):
    """(gdr_chunk_fwd result, gdr_chunk_fwd_no_alloc result) on the same inputs."""
    import torch
    t = device_tensors(inp)
    s_in = t["state_in"] if with_states else None
    ref_o, ref_s = gdr.chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu"], s_in,
                                 scale=SCALE, want_state=with_states)
    out = torch.full_like(ref_o, float("nan"))
    st = torch.full_like(ref_s, float("nan")) if with_states else None
    gdr.chunk_fwd_no_alloc(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu"], s_in, out, st,
                           scale=SCALE)
    torch.cuda.synchronize()
    return (to_f64(ref_o), None if ref_s is None else to_f64(ref_s),
            to_f64(out), None if st is None else to_f64(st))


@pytest.mark.gpu
def test_no_alloc_matches_chunk_fwd_on_consecutive_calls():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cases = [
        # the prefill workload: several segments of the 64 MiB array
        (make_inputs([4096], 16, 32, dtype="bf16", seed=121, state_std=0.01), True),
        # smaller, packed, ragged, final state carried through the array
        (make_inputs([300, 1, 0, 129, 77], 2, 4, dtype="bf16", seed=122, state_std=0.1), False),
        # fp32, several sequences spanning segments
        (make_inputs([1500, 900, 3], 8, 32, dtype="f32", seed=123, state_std=0.1), True),
    ]
    for i, (inp, with_states) in enumerate(cases):
        ro, rs, no, ns = _both(inp, with_states)
        tol = TOL[inp.dtype]
        same = np.array_equal(ro, no) and (rs is None or np.array_equal(rs, ns))
        print(f"call {i}: T={inp.T} N={inp.N} Nv={inp.Nv} {inp.dtype}: "
              f"{'bit-identical' if same else 'differs'} to gdr_chunk_fwd")
        assert_close_per_seq_head(no, ro, ns, rs, inp.cu_seqlens, tol, name=f"call {i} vs chunk_fwd")
        oo, os_ = oracle_full(inp, state_in=(inp.state_in if with_states else None))
        assert_close_per_seq_head(no, oo, ns, os_ if with_states else None, inp.cu_seqlens, tol,
                                  name=f"call {i} vs oracle")


def test_no_alloc_refuses_sizes_beyond_its_array():
    """64 sequences x 32 heads with no state_out would carry 128 MiB of state
    through the 64 MiB array: refused during validation (no HIP call, so fake
    aligned addresses are safe)."""
    lib = gdr.load()
    assert lib.gdr_chunk_fwd_no_alloc_scratch_bytes() == 64 << 20
    fake = ctypes.c_void_p(1 << 20)
    N, T, Nqk, Nv = 64, 64 * 100, 16, 32
    st = lib.gdr_chunk_fwd_no_alloc(fake, fake, fake, fake, fake, None, fake, N, T, Nqk, Nv, 128,
                                    gdr.GDR_BF16, 0.1, 1, ctypes.c_void_p(1 << 40), None, None)
    assert st == WS_SMALL
    # invalid sizes are refused as by gdr_chunk_fwd
    st = lib.gdr_chunk_fwd_no_alloc(fake, fake, fake, fake, fake, None, fake, 1, 100, 3, 4, 128,
                                    gdr.GDR_BF16, 0.1, 1, ctypes.c_void_p(1 << 40), None, None)
    assert st == -1
