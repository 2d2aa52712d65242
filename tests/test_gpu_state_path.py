"""GPU tests of the state path of the chunkwise form and the decode step,
through the C ABI: closed forms, long slow-decay runs, wide query/key groups,
split invariance, every way a multi-segment call carries the state, and
guard bands around every output.

Closed forms (Qwen3-Next blog post, section 5(2): the state decays, then the
delta write; o_t = S_t qh_t):
* beta = 0: no write, so S_T = exp(sum g) S_0 and o_t = exp(sum_{s<=t} g_s) S_0 qh_t;
* g = 0, beta = 1 with orthonormal keys k_i: from S_0 = 0 each write adds
  c v_i k_i^T (c = 1/sqrt(1 + eps), the normalised key's length), so reading
  with q = k_i (beta = 0) returns scale c^2 v_i, and S = c sum_i v_i k_i^T.
Every case is also compared with the fp64 oracle per (sequence, value head).
"""
import numpy as np
import pytest

import gated_deltanet_chunked_amd as gdr
from gated_deltanet_chunked_amd.inputs import GdrInputs, make_inputs, orthonormal_keys, round_to_bf16
from tests.gpu_util import (SCALE, TOL, assert_close_per_seq_head, device_tensors, oracle_full,
                            rel_l2, to_f64)

pytestmark = pytest.mark.gpu

EPS = 1e-6


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gdr.load()
    yield
    torch.cuda.synchronize()


def _chunk(inp, state="in", want_state=True, in_place=False):
    import torch
    t = device_tensors(inp)
    s_in = t["state_in"] if state == "in" else None
    s_out = s_in if (in_place and s_in is not None) else None
    out, st = gdr.chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu"], s_in,
                            scale=SCALE, state_out=s_out, want_state=want_state)
    torch.cuda.synchronize()
    if in_place and s_in is not None:
        assert st.data_ptr() == s_in.data_ptr()
    return to_f64(out), (to_f64(st) if st is not None else None)


def _normalised(x):
    x = np.asarray(x, np.float64)
    return x / np.sqrt((x * x).sum(axis=-1, keepdims=True) + EPS)


# -------------------------------------------------------------- beta = 0


def _pure_decay_closed_form(inp):
    """o and S_out of beta = 0 written out from the closed form (fp64)."""
    G = inp.Nv // inp.Nqk
    cu = inp.cu_seqlens
    qh = SCALE * _normalised(inp.q)                       # [T, Nqk, D]
    out = np.zeros((inp.T, inp.Nv, 128))
    st = np.zeros((inp.N, inp.Nv, 128, 128))
    s0 = inp.state_in.astype(np.float64)
    for b in range(inp.N):
        t0, t1 = cu[b], cu[b + 1]
        decay = np.exp(np.cumsum(inp.g[t0:t1].astype(np.float64), axis=0))   # [len, Nv]
        for h in range(inp.Nv):
            Sq = qh[t0:t1, h // G] @ s0[b, h].T                              # rows S_0 qh_t
            out[t0:t1, h] = decay[:, h:h + 1] * Sq
            st[b, h] = (decay[-1, h] if t1 > t0 else 1.0) * s0[b, h]
    return out, st


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_beta_zero_chunk_is_pure_decay(dtype):
    inp = make_inputs([300, 77, 129], 2, 4, dtype=dtype, seed=101, state_std=1.0,
                      A_range=(0.0, 0.02))
    inp.beta[:] = 0.0
    out, st = _chunk(inp)
    co, cs = _pure_decay_closed_form(inp)
    assert_close_per_seq_head(out, co, st, cs, inp.cu_seqlens, TOL[dtype], name="closed form")
    ro, rs = oracle_full(inp)
    assert_close_per_seq_head(out, ro, st, rs, inp.cu_seqlens, TOL[dtype], name="oracle")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_beta_zero_decode_is_pure_decay(dtype):
    import torch
    inp = make_inputs([1] * 6, 2, 4, dtype=dtype, seed=102, state_std=1.0)
    inp.beta[:] = 0.0
    t = device_tensors(inp)
    s = t["state_in"].clone()
    out = gdr.recurrent_step(t["q"], t["k"], t["v"], t["g"], t["beta"], s, scale=SCALE)
    torch.cuda.synchronize()
    co, cs = _pure_decay_closed_form(inp)
    assert_close_per_seq_head(to_f64(out), co, to_f64(s), cs, inp.cu_seqlens, TOL[dtype],
                              name="closed form")


# ------------------------------------------------------ exact retrieval


def _retrieval_inputs(dtype, seqs, Nqk=2, Nv=4, seed=103):
    """Per sequence of n: n writes (g = 0, beta = 1, orthonormal keys k_i,
    random values), then n reads (beta = 0, g = 0, q = k_perm(i)).  Returns the
    inputs and, per sequence, (first read token, permutation)."""
    rng = np.random.default_rng(seed)
    T = 2 * sum(seqs)
    q = rng.standard_normal((T, Nqk, 128))
    k = np.zeros((T, Nqk, 128))
    v = rng.standard_normal((T, Nv, 128))
    g = np.zeros((T, Nv))
    beta = np.zeros((T, Nv))
    reads = []
    t = 0
    for si, n in enumerate(seqs):
        perm = rng.permutation(n)
        for j in range(Nqk):
            keys = orthonormal_keys(n, 128, seed=seed + 17 * si + j)
            k[t:t + n, j] = keys
            q[t + n:t + 2 * n, j] = keys[perm]
            k[t + n:t + 2 * n, j] = keys[perm]
        beta[t:t + n] = 1.0
        reads.append((t + n, perm))
        t += 2 * n
    cu = np.concatenate([[0], np.cumsum([2 * n for n in seqs])]).astype(np.int32)
    f = np.float32
    if dtype == "bf16":
        from gated_deltanet_chunked_amd.inputs import round_to_bf16
        rd = lambda x: round_to_bf16(x.astype(f))
    else:
        rd = lambda x: x.astype(f)
    inp = GdrInputs(q=rd(q), k=rd(k), v=rd(v), g=g.astype(f), beta=beta.astype(f), state_in=None,
                    cu_seqlens=cu, dtype=dtype, seed=seed)
    return inp, reads


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_exact_retrieval_chunk(dtype):
    """Writes and reads inside one chunk (64 + 64), across a chunk boundary
    (100 + 100) and a full basis (128 + 128)."""
    seqs = [64, 100, 128]
    inp, reads = _retrieval_inputs(dtype, seqs)
    out, st = _chunk(inp, state=None)
    ro, rs = oracle_full(inp, state_in=None)
    assert_close_per_seq_head(out, ro, st, rs, inp.cu_seqlens, TOL[dtype], name="oracle")
    c2 = 1.0 / (1.0 + EPS)
    G = inp.Nv // inp.Nqk
    for (r0, perm), n, b in zip(reads, seqs, range(len(seqs))):
        w0 = r0 - n
        want = SCALE * c2 * inp.v[w0:r0][perm].astype(np.float64)          # [n, Nv, D]
        got = out[r0:r0 + n]
        # fp32 keys are orthonormal to ~1e-7; bf16-rounded keys only to ~4e-3
        tol = 1e-4 if dtype == "f32" else 2e-2
        err = rel_l2(got, want)
        print(f"sequence {b}: retrieved values rel L2 {err:.3e}")
        assert err <= tol
        if dtype == "f32":
            for h in range(inp.Nv):
                keys = inp.k[w0:r0, h // G].astype(np.float64)
                S = np.sqrt(c2) * inp.v[w0:r0, h].astype(np.float64).T @ keys
                assert rel_l2(st[b, h], S) <= 1e-4


# ------------------------------------------------ long slow-decay runs


def test_long_slow_decay_bf16():
    """T = 32768 (256 serial chunks), Nqk = 16, Nv = 32, bf16, gates near 1
    (A ~ U(0, 0.05)) and a unit-scale initial state: the state carries across
    the whole sequence, so rounding in the state pass would accumulate."""
    inp = make_inputs([32768], 16, 32, dtype="bf16", seed=104, state_std=1.0,
                      A_range=(0.0, 0.05))
    out, st = _chunk(inp)
    ro, rs = oracle_full(inp)
    assert_close_per_seq_head(out, ro, st, rs, inp.cu_seqlens, TOL["bf16"], name="T=32768")


# ------------------------------------------------- wide query/key groups


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("Nqk", [4, 2], ids=["G8", "G16"])
def test_wide_groups(dtype, Nqk):
    """Nv = 32 value heads on 4 (G = 8) or 2 (G = 16) query/key heads."""
    inp = make_inputs([700, 1, 333], Nqk, 32, dtype=dtype, seed=105 + Nqk, state_std=0.1,
                      A_range=(0.0, 1.0))
    out, st = _chunk(inp)
    ro, rs = oracle_full(inp)
    assert_close_per_seq_head(out, ro, st, rs, inp.cu_seqlens, TOL[dtype])


# ----------------------------------------------------- split invariance


def _slice(inp, t0, t1, state):
    return GdrInputs(q=inp.q[t0:t1], k=inp.k[t0:t1], v=inp.v[t0:t1], g=inp.g[t0:t1],
                     beta=inp.beta[t0:t1], state_in=state,
                     cu_seqlens=np.array([0, t1 - t0], np.int32), dtype=inp.dtype, seed=inp.seed)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_split_sequence_equals_whole(dtype):
    """chunk_fwd on tokens [0, 1000), then on [1000, 2100) from its final
    state, equals chunk_fwd on [0, 2100): the state carries a sequence across
    calls (the operator page's state reuse)."""
    inp = make_inputs([2100], 2, 4, dtype=dtype, seed=107, state_std=0.5, A_range=(0.0, 0.5))
    whole_o, whole_s = _chunk(inp)
    o1, s1 = _chunk(_slice(inp, 0, 1000, inp.state_in))
    o2, s2 = _chunk(_slice(inp, 1000, 2100, s1.astype(np.float32)))
    split_o = np.concatenate([o1, o2])
    ro, rs = oracle_full(inp)
    assert_close_per_seq_head(split_o, ro, s2, rs, inp.cu_seqlens, TOL[dtype], name="split")
    assert_close_per_seq_head(whole_o, ro, whole_s, rs, inp.cu_seqlens, TOL[dtype], name="whole")
    assert_close_per_seq_head(split_o, whole_o, s2, whole_s, inp.cu_seqlens, TOL[dtype],
                              name="split vs whole")


# ------------------------------------------- multi-segment state carry


@pytest.mark.parametrize("mode", ["in_place", "no_state_out", "no_state_in", "fp32"])
def test_multi_segment_carry(mode):
    """Calls long enough to take several segments (the intra-chunk products
    of one segment are consumed before the next segment's are made), with
    sequences spanning segment boundaries, and every way the state is
    carried between segments: in place, through the workspace (no state_out),
    from zeros (no state_in), and in fp32 (smaller segments)."""
    if mode == "fp32":
        inp = make_inputs([2500, 1700, 900], 8, 32, dtype="f32", seed=108, state_std=0.5,
                          A_range=(0.0, 0.5))
    else:
        inp = make_inputs([3000, 5000, 2100], 16, 32, dtype="bf16", seed=109, state_std=0.5,
                          A_range=(0.0, 0.5))
    state = None if mode == "no_state_in" else "in"
    out, st = _chunk(inp, state=state, want_state=(mode != "no_state_out"),
                     in_place=(mode == "in_place"))
    ro, rs = oracle_full(inp, state_in=None) if state is None else oracle_full(inp)
    if mode == "no_state_out":
        assert st is None
        rs = None
    assert_close_per_seq_head(out, ro, st, rs, inp.cu_seqlens, TOL[inp.dtype], name=mode)


def test_single_sequence_multi_segment_in_place():
    inp = make_inputs([9000], 16, 32, dtype="bf16", seed=110, state_std=0.5, A_range=(0.0, 0.5))
    out, st = _chunk(inp, in_place=True)
    ro, rs = oracle_full(inp)
    assert_close_per_seq_head(out, ro, st, rs, inp.cu_seqlens, TOL["bf16"])


# ------------------------------------------------------- guard bands


PAD = 4096   # elements of guard band on each side (16-byte multiples for both dtypes)


def _guarded(shape, dtype, fill):
    """A tensor of `shape` inside a larger buffer whose guard bands hold `fill`."""
    import torch
    n = int(np.prod(shape))
    buf = torch.full((PAD + n + PAD,), fill, dtype=dtype, device="cuda:0")
    return buf, buf[PAD:PAD + n].view(*shape)


def _check_guards(buf, fill, name):
    import torch
    lo, hi = buf[:PAD], buf[-PAD:]
    assert torch.all(lo == fill).item() and torch.all(hi == fill).item(), \
        f"{name}: a kernel wrote outside its buffer"


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_guard_bands_chunk(dtype):
    """out, state_out and the workspace sit between guard bands; no kernel
    writes outside them (ragged tails, one-token and empty sequences, several
    segments)."""
    import torch
    lengths = [300, 1, 0, 129, 77, 5000]
    inp = make_inputs(lengths, 16, 32, dtype=dtype, seed=111, state_std=0.1)
    t = device_tensors(inp)
    tdt = t["q"].dtype
    ob, out = _guarded((inp.T, inp.Nv, 128), tdt, -7.0)
    sb, st = _guarded((inp.N, inp.Nv, 128, 128), torch.float32, -9.0)
    need = gdr.workspace_size(inp.T, inp.N, inp.Nqk, inp.Nv,
                              gdr.GDR_BF16 if dtype == "bf16" else gdr.GDR_F32)
    wb = torch.full((need + 2 * PAD,), 0xA5, dtype=torch.uint8, device="cuda:0")
    ws = wb[PAD:PAD + need]
    gdr.chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu"], t["state_in"],
                  scale=SCALE, out=out, state_out=st, workspace=ws)
    torch.cuda.synchronize()
    _check_guards(ob, -7.0, "out")
    _check_guards(sb, -9.0, "state_out")
    assert torch.all(wb[:PAD] == 0xA5).item() and torch.all(wb[-PAD:] == 0xA5).item(), \
        "workspace: a kernel wrote outside it"
    ro, rs = oracle_full(inp)
    assert_close_per_seq_head(to_f64(out), ro, to_f64(st), rs, inp.cu_seqlens, TOL[dtype])


def test_guard_bands_decode_and_multi():
    import torch
    inp = make_inputs([1] * 7, 2, 4, dtype="bf16", seed=112, state_std=0.1)
    t = device_tensors(inp)
    ob, out = _guarded((inp.N, inp.Nv, 128), torch.bfloat16, -7.0)
    sb, st = _guarded((inp.N, inp.Nv, 128, 128), torch.float32, -9.0)
    gdr.recurrent_step(t["q"], t["k"], t["v"], t["g"], t["beta"], t["state_in"], state_out=st,
                       out=out, scale=SCALE)
    torch.cuda.synchronize()
    _check_guards(ob, -7.0, "decode out")
    _check_guards(sb, -9.0, "decode state_out")
    ro, rs = oracle_full(inp)
    assert_close_per_seq_head(to_f64(out), ro, to_f64(st), rs, inp.cu_seqlens, TOL["bf16"])

    inp = make_inputs([3, 0, 16, 5], 2, 4, dtype="bf16", seed=113, state_std=0.1)
    t = device_tensors(inp)
    ob, out = _guarded((inp.T, inp.Nv, 128), torch.bfloat16, -7.0)
    sb, st = _guarded((inp.N, inp.Nv, 128, 128), torch.float32, -9.0)
    gdr.recurrent_multi(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu"], t["state_in"],
                        out=out, state_out=st, scale=SCALE)
    torch.cuda.synchronize()
    _check_guards(ob, -7.0, "multi out")
    _check_guards(sb, -9.0, "multi state_out")
    ro, rs = oracle_full(inp)
    assert_close_per_seq_head(to_f64(out), ro, to_f64(st), rs, inp.cu_seqlens, TOL["bf16"])


def test_timed_call_with_fewer_slots_than_launches_times_the_span():
    """gdr_chunk_fwd_timed with room for fewer kernel times than launches still
    computes the same result and reports only the span (n = 0)."""
    import ctypes
    import torch
    inp = make_inputs([300, 1, 129], 2, 4, dtype="bf16", seed=114, state_std=0.1)
    t = device_tensors(inp)
    ref_o, ref_s = gdr.chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu"], t["state_in"],
                                 scale=SCALE)
    out, st = torch.empty_like(ref_o), torch.empty_like(ref_s)
    need = gdr.workspace_size(inp.T, inp.N, inp.Nqk, inp.Nv, gdr.GDR_BF16)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda:0")
    lib = gdr.load()
    kms = (ctypes.c_float * 1)()
    kind = (ctypes.c_int32 * 1)()
    n = ctypes.c_int32(-1)
    span = ctypes.c_float(0.0)
    p = lambda x: x.data_ptr()
    rc = lib.gdr_chunk_fwd_timed(p(t["q"]), p(t["k"]), p(t["v"]), p(t["g"]), p(t["beta"]),
                                 p(t["state_in"]), p(t["cu"]), inp.N, inp.T, inp.Nqk, inp.Nv, 128,
                                 gdr.GDR_BF16, SCALE, gdr.GDR_FLAG_QK_L2NORM, p(out), p(st), p(ws),
                                 need, torch.cuda.current_stream().cuda_stream, kms, kind, 1,
                                 ctypes.byref(n), ctypes.byref(span))
    torch.cuda.synchronize()
    assert rc == 0 and n.value == 0 and span.value > 0
    assert torch.equal(out, ref_o) and torch.equal(st, ref_s)


# ------------------------------------------------------- many sequences


@pytest.mark.parametrize("dtype,chunk", [("f32", 128), ("bf16", 128), ("bf16", 64)])
def test_many_short_sequences(dtype, chunk):
    """1,500 packed sequences, most of 0-39 tokens (empty and one-token ones
    among them) and every 200th of 600 tokens: more sequences than the chunk
    table's 1,024 threads (several per thread), more chunk slots than one
    segment holds (the long sequences span segment boundaries and carry their
    state), and, with 64-token chunks, pairs of slots from different
    sequences in one workgroup of the intra-chunk kernel."""
    rng = np.random.default_rng(120)
    lengths = rng.integers(0, 40, size=1500)
    lengths[::200] = 600
    inp = make_inputs(lengths, 1, 2, dtype=dtype, seed=121, state_std=0.1)
    import torch
    t = device_tensors(inp)
    out, st = gdr.chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu"], t["state_in"],
                            scale=SCALE, chunk=chunk)
    torch.cuda.synchronize()
    ro, rs = oracle_full(inp)
    assert_close_per_seq_head(to_f64(out), ro, to_f64(st), rs, inp.cu_seqlens, TOL[dtype],
                              name=f"N=1500 {dtype} L={chunk}")
    empty = np.flatnonzero(lengths == 0)
    assert empty.size > 0
    assert np.array_equal(to_f64(st)[empty], inp.state_in[empty].astype(np.float64))


# ------------------------------------------------------- the q scale


@pytest.mark.parametrize("path,dtype", [("chunk", "f32"), ("chunk", "bf16"), ("chunk64", "bf16"),
                                        ("multi", "bf16"), ("step", "f32"), ("step", "bf16")])
def test_scale_other_than_the_default(path, dtype):
    """Every entry point takes q's scale as an argument (the Blog's D^-1/2 is
    only the default): a scale of 0.37 against the oracle at the same scale,
    with and without the L2 norms, so that a constant built into a kernel, or
    the scale applied to k, fails."""
    import oracle
    import torch
    sc = 0.37
    lengths = [1] * 6 if path == "step" else ([200, 57, 1] if path != "multi" else [5, 1, 16])
    for l2 in (True, False):
        inp = make_inputs(lengths, 2, 4, dtype=dtype, seed=130, state_std=0.1)
        if not l2:
            # used as given: rows of norm U(0.5, 1) (so a norm applied anyway
            # would show), rounded again for bf16 so both sides see the same
            rng = np.random.default_rng(131)
            for name in ("q", "k"):
                x = getattr(inp, name)
                x = x / np.linalg.norm(x, axis=-1, keepdims=True) * rng.uniform(0.5, 1.0, x.shape[:-1] + (1,))
                x = x.astype(np.float32)
                setattr(inp, name, round_to_bf16(x) if dtype == "bf16" else x)
        t = device_tensors(inp)
        if path == "step":
            s = t["state_in"].clone()
            out = gdr.recurrent_step(t["q"], t["k"], t["v"], t["g"], t["beta"], s, scale=sc, l2norm=l2)
            st = s
        elif path == "multi":
            out, st = gdr.recurrent_multi(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu"],
                                          t["state_in"], scale=sc, l2norm=l2)
        else:
            out, st = gdr.chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu"], t["state_in"],
                                    scale=sc, l2norm=l2, chunk=64 if path == "chunk64" else 128)
        torch.cuda.synchronize()
        ro, rs = oracle.recurrent(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.state_in, inp.cu_seqlens,
                                  sc, l2norm=l2)
        assert_close_per_seq_head(to_f64(out), ro, to_f64(st), rs, inp.cu_seqlens, TOL[dtype],
                                  name=f"{path} {dtype} scale {sc} l2norm={l2}")


# ------------------------------------------------------- extreme decays


@pytest.mark.parametrize("path,dtype", [("chunk", "f32"), ("chunk", "bf16"), ("chunk64", "bf16"),
                                        ("multi", "bf16")])
def test_hard_resets_and_underflowing_decays(path, dtype):
    """Gates far outside the trained range, still finite and <= 0: every 37th
    token has g = -1e4 (the state before it is forgotten exactly; within a
    chunk the decay mask and the chunk factors underflow to zero), one
    sequence has g = -200 throughout (e^-200 underflows in fp32, not in the
    fp64 oracle: a difference far below the tolerance), and g = 0 elsewhere on
    some heads (no decay at all)."""
    import oracle
    import torch
    lengths = [300, 200, 129] if path != "multi" else [9, 16, 3]
    inp = make_inputs(lengths, 2, 4, dtype=dtype, seed=140, state_std=0.5)
    g = inp.g.copy()
    g[::37, :] = -1e4
    t0, t1 = int(inp.cu_seqlens[1]), int(inp.cu_seqlens[2])
    g[t0:t1, :] = -200.0
    g[:t0, 3] = 0.0
    inp.g = g.astype(np.float32)
    t = device_tensors(inp)
    if path == "multi":
        out, st = gdr.recurrent_multi(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu"],
                                      t["state_in"], scale=SCALE)
    else:
        out, st = gdr.chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu"], t["state_in"],
                                scale=SCALE, chunk=64 if path == "chunk64" else 128)
    torch.cuda.synchronize()
    ro, rs = oracle_full(inp)
    assert_close_per_seq_head(to_f64(out), ro, to_f64(st), rs, inp.cu_seqlens, TOL[dtype],
                              name=f"{path} {dtype} extreme gates")


# ------------------------------------------- empty calls, huge packed batches


def test_single_empty_sequence_keeps_its_state():
    """N = 1, T = 0: no chunk slot at all, so no intra-chunk or state-pass
    launch; the final state is still the initial state (zeros without one),
    in place nothing is touched, and the timed call reports no kernel."""
    import ctypes
    import torch
    dev = "cuda:0"
    q = torch.empty((0, 1, 128), dtype=torch.bfloat16, device=dev)
    v = torch.empty((0, 2, 128), dtype=torch.bfloat16, device=dev)
    g = torch.empty((0, 2), dtype=torch.float32, device=dev)
    cu = torch.zeros(2, dtype=torch.int32, device=dev)
    s0 = torch.randn((1, 2, 128, 128), device=dev)
    for chunk in (128, 64):
        st = torch.full_like(s0, 7.0)
        out, st = gdr.chunk_fwd(q, q, v, g, g, cu, s0, state_out=st, scale=SCALE, chunk=chunk)
        torch.cuda.synchronize()
        assert out.shape == (0, 2, 128) and torch.equal(st, s0)
        st = torch.full_like(s0, 7.0)
        _, st = gdr.chunk_fwd(q, q, v, g, g, cu, None, state_out=st, scale=SCALE, chunk=chunk)
        torch.cuda.synchronize()
        assert torch.count_nonzero(st).item() == 0
    s = s0.clone()
    tim = []
    _, st = gdr.chunk_fwd(q, q, v, g, g, cu, s, state_out=s, scale=SCALE, timings=tim)
    torch.cuda.synchronize()
    assert torch.equal(s, s0) and tim == [("span", 0.0)]
    tim = []
    out, st = gdr.chunk_fwd(q, q, v, g, g, cu, s0, scale=SCALE, timings=tim)
    torch.cuda.synchronize()
    assert torch.equal(st, s0) and [n for n, _ in tim] == ["table", "span"]


@pytest.mark.parametrize("dtype,chunk", [("bf16", 128), ("bf16", 64), ("f32", 128)])
def test_many_sequences_mostly_empty(dtype, chunk):
    """6,000 packed sequences, 70% of them empty and the rest 1-40 tokens
    (every 500th 700 tokens): the state pass launches over each segment's runs
    of slots (at most one per slot), not over all 6,000 sequences, so a
    segment's sequence ids span far more than its slots; the empty sequences
    get their initial states from the table launch."""
    import time
    import torch
    rng = np.random.default_rng(160)
    N = 6000
    lengths = np.where(rng.random(N) < 0.7, 0, rng.integers(1, 41, size=N))
    lengths[::500] = 700
    inp = make_inputs(lengths, 1, 2, dtype=dtype, seed=161, state_std=0.1)
    t = device_tensors(inp)
    args = (t["q"], t["k"], t["v"], t["g"], t["beta"], t["cu"], t["state_in"])
    gdr.chunk_fwd(*args, scale=SCALE, chunk=chunk)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    out, st = gdr.chunk_fwd(*args, scale=SCALE, chunk=chunk)
    torch.cuda.synchronize()
    print(f"N={N} T={inp.T} {dtype} L={chunk}: {1e3 * (time.perf_counter() - t0):.2f} ms", flush=True)
    ro, rs = oracle_full(inp)
    assert_close_per_seq_head(to_f64(out), ro, to_f64(st), rs, inp.cu_seqlens, TOL[dtype],
                              name=f"N={N} mostly empty {dtype} L={chunk}")
    empty = np.flatnonzero(lengths == 0)
    assert np.array_equal(to_f64(st)[empty], inp.state_in[empty].astype(np.float64))
