"""CPU tests of the C ABI: the library loads, exports every declared symbol,
sizes its workspace, and rejects bad arguments before touching the GPU.

Only validation paths run here: every call below fails validation, which
happens before any HIP call, so fake (aligned, non-null) addresses are safe.
"""
import ctypes
import os
import re

import pytest

import gated_deltanet_chunked_amd as gdr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdr.h")

OK, INVALID, UNSUPPORTED, WS_SMALL = 0, -1, -2, -3


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdr_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("gdr_chunk_fwd", "gdr_recurrent_step", "gdr_chunk_fwd_workspace_size",
              "gdr_status_string", "gdr_version", "gdr_chunk_fwd_timed",
              "gdr_recurrent_step_timed", "gdr_recurrent_step_bf16_state", "gdr_recurrent_multi",
              "gdr_recurrent_step_conv", "gdr_gated_rmsnorm", "gdr_recurrent_step_gated"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = gdr.load()
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_version_and_status_strings():
    lib = gdr.load()
    assert lib.gdr_version().startswith(b"libgdr")
    for code in (0, -1, -2, -3, -4, -5):
        assert lib.gdr_status_string(code)
    assert lib.gdr_status_string(7) == b"unknown status"


def test_workspace_size():
    ws = lambda *a: gdr.workspace_size(*a)
    small = ws(512, 1, 2, 4, gdr.GDR_F32)
    assert small > 0
    assert ws(4096, 1, 16, 32, gdr.GDR_BF16) > 0
    # invalid sizes give 0
    lib = gdr.load()
    assert lib.gdr_chunk_fwd_workspace_size(512, 1, 2, 4, 64, 0) == 0   # D != 128
    assert lib.gdr_chunk_fwd_workspace_size(512, 1, 3, 4, 128, 0) == 0  # Nv % Nqk
    assert lib.gdr_chunk_fwd_workspace_size(512, 0, 2, 4, 128, 0) == 0  # N < 1
    assert lib.gdr_chunk_fwd_workspace_size(-1, 1, 2, 4, 128, 0) == 0
    assert lib.gdr_chunk_fwd_workspace_size(512, 1, 2, 4, 128, 5) == 0  # dtype
    assert lib.gdr_chunk_fwd_workspace_size(512, 1, 1, 16385, 128, 0) == 0  # Nv > 16384
    assert lib.gdr_chunk_fwd_workspace_size(512, 1, 1, 16384, 128, 0) > 0
    # bounded by the segment buffer: grows slowly with T
    assert ws(1 << 20, 1, 16, 32, gdr.GDR_BF16) < 2 * ws(1 << 16, 1, 16, 32, gdr.GDR_BF16) + (1 << 30)


class FakeBuffers:
    """Distinct, 256-byte aligned, non-overlapping fake device addresses."""

    def __init__(self, T=256, N=2, Nqk=2, Nv=4, es=2):
        base = 1 << 40
        sizes = dict(q=T * Nqk * 128 * es, k=T * Nqk * 128 * es, v=T * Nv * 128 * es,
                     g=T * Nv * 4, beta=T * Nv * 4, state_in=N * Nv * 128 * 128 * 4,
                     cu=(N + 1) * 4, out=T * Nv * 128 * es, state_out=N * Nv * 128 * 128 * 4,
                     ws=gdr.workspace_size(T, N, Nqk, Nv, gdr.GDR_BF16 if es == 2 else gdr.GDR_F32))
        self.addr = {}
        for name, n in sizes.items():
            self.addr[name] = base
            base += (n + (1 << 20)) & ~255
        self.sizes = sizes
        self.T, self.N, self.Nqk, self.Nv = T, N, Nqk, Nv


def call_chunk(fb, **over):
    lib = gdr.load()
    a = dict(q=fb.addr["q"], k=fb.addr["k"], v=fb.addr["v"], g=fb.addr["g"], beta=fb.addr["beta"],
             state_in=fb.addr["state_in"], cu=fb.addr["cu"], N=fb.N, T=fb.T, Nqk=fb.Nqk, Nv=fb.Nv,
             D=128, dtype=gdr.GDR_BF16, scale=0.1, flags=gdr.GDR_FLAG_QK_L2NORM,
             out=fb.addr["out"], state_out=fb.addr["state_out"], ws=fb.addr["ws"],
             ws_bytes=fb.sizes["ws"], stream=None)
    a.update(over)
    return lib.gdr_chunk_fwd(a["q"], a["k"], a["v"], a["g"], a["beta"], a["state_in"], a["cu"],
                             a["N"], a["T"], a["Nqk"], a["Nv"], a["D"], a["dtype"], a["scale"],
                             a["flags"], a["out"], a["state_out"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("over,expect", [
    (dict(D=64), UNSUPPORTED),
    (dict(dtype=7), UNSUPPORTED),
    (dict(flags=4), UNSUPPORTED),
    (dict(Nqk=1, Nv=16385), UNSUPPORTED),   # more than 16384 value heads
    (dict(Nqk=3), INVALID),            # Nv % Nqk != 0
    (dict(N=0), INVALID),
    (dict(T=-1), INVALID),
    (dict(q=None), INVALID),
    (dict(out=None), INVALID),
    (dict(cu=None), INVALID),
    (dict(ws=None), INVALID),
    (dict(ws_bytes=1024), WS_SMALL),
], ids=lambda x: str(x))
def test_chunk_fwd_rejects(over, expect):
    fb = FakeBuffers()
    assert call_chunk(fb, **over) == expect


def test_chunk_fwd_rejects_misalignment():
    fb = FakeBuffers()
    assert call_chunk(fb, q=fb.addr["q"] + 8) == INVALID
    assert call_chunk(fb, ws=fb.addr["ws"] + 16) == INVALID   # workspace needs 256 bytes


def test_chunk_fwd_rejects_aliasing():
    fb = FakeBuffers()
    assert call_chunk(fb, out=fb.addr["v"]) == INVALID
    assert call_chunk(fb, out=fb.addr["q"] + 256) == INVALID
    # partial overlap of the two states
    assert call_chunk(fb, state_out=fb.addr["state_in"] + 4096) == INVALID
    assert call_chunk(fb, state_out=fb.addr["ws"]) == INVALID


def call_step(fb, **over):
    lib = gdr.load()
    a = dict(q=fb.addr["q"], k=fb.addr["k"], v=fb.addr["v"], g=fb.addr["g"], beta=fb.addr["beta"],
             state_in=fb.addr["state_in"], state_out=fb.addr["state_out"], N=fb.N, Nqk=fb.Nqk,
             Nv=fb.Nv, D=128, dtype=gdr.GDR_BF16, scale=0.1, flags=gdr.GDR_FLAG_QK_L2NORM,
             out=fb.addr["out"], stream=None)
    a.update(over)
    return lib.gdr_recurrent_step(a["q"], a["k"], a["v"], a["g"], a["beta"], a["state_in"],
                                  a["state_out"], a["N"], a["Nqk"], a["Nv"], a["D"], a["dtype"],
                                  a["scale"], a["flags"], a["out"], a["stream"])


@pytest.mark.parametrize("over,expect", [
    (dict(D=256), UNSUPPORTED),
    (dict(dtype=3), UNSUPPORTED),
    (dict(Nqk=3), INVALID),
    (dict(N=-1), INVALID),
    (dict(state_in=None), INVALID),
    (dict(state_out=None), INVALID),
    (dict(out=None), INVALID),
    (dict(k=1 << 40 | 4), INVALID),
    (dict(N=1 << 21, Nqk=8, Nv=8), INVALID),   # 2^24 workgroups: beyond a grid's 2^32 work-items
], ids=lambda x: str(x))
def test_recurrent_step_rejects(over, expect):
    fb = FakeBuffers(T=2, N=2)
    assert call_step(fb, **over) == expect


def test_recurrent_step_zero_sequences_is_a_no_op():
    fb = FakeBuffers(T=2, N=2)
    assert call_step(fb, N=0, q=None, k=None, v=None, state_in=None, state_out=None, out=None) == OK


def test_timed_entry_points_validate_before_launching():
    """The profiling variants check their extra arguments on the host."""
    import ctypes
    lib = gdr.load()
    fb = FakeBuffers(T=2, N=2)
    a = [fb.addr["q"], fb.addr["k"], fb.addr["v"], fb.addr["g"], fb.addr["beta"],
         fb.addr["state_in"], fb.addr["state_out"], fb.N, fb.Nqk, fb.Nv, 128, gdr.GDR_BF16, 0.1,
         gdr.GDR_FLAG_QK_L2NORM, fb.addr["out"], None]
    assert lib.gdr_recurrent_step_timed(*a, None) == INVALID     # no kernel_ms
    ms = ctypes.c_float(1.0)
    a0 = list(a)
    a0[7] = 0                                                     # N = 0: nothing to time
    assert lib.gdr_recurrent_step_timed(*a0, ctypes.byref(ms)) == OK and ms.value == 0.0
    fc = FakeBuffers()
    c = [fc.addr["q"], fc.addr["k"], fc.addr["v"], fc.addr["g"], fc.addr["beta"], fc.addr["state_in"],
         fc.addr["cu"], fc.N, fc.T, fc.Nqk, fc.Nv, 128, gdr.GDR_BF16, 0.1, gdr.GDR_FLAG_QK_L2NORM,
         fc.addr["out"], fc.addr["state_out"], fc.addr["ws"], fc.sizes["ws"], None]
    kms = (ctypes.c_float * 4)()
    kind = (ctypes.c_int32 * 4)()
    n = ctypes.c_int32(0)
    # missing result arrays or a negative capacity: rejected (fewer slots than
    # launches is allowed: only the span is then timed, a GPU test checks it)
    assert lib.gdr_chunk_fwd_timed(*c, None, kind, 4, ctypes.byref(n), None) == INVALID
    assert lib.gdr_chunk_fwd_timed(*c, kms, None, 4, ctypes.byref(n), None) == INVALID
    assert lib.gdr_chunk_fwd_timed(*c, kms, kind, -1, ctypes.byref(n), None) == INVALID
    assert lib.gdr_chunk_fwd_timed(*c, kms, kind, 4, None, None) == INVALID


def test_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(RuntimeError):
        gdr.load(str(tmp_path / "missing.so"))


def test_bf16_state_step_validates_before_launching():
    """gdr_recurrent_step_bf16_state: the same checks, with 2-byte states."""
    import ctypes
    lib = gdr.load()
    fb = FakeBuffers(T=2, N=2)

    def call(**over):
        a = dict(q=fb.addr["q"], k=fb.addr["k"], v=fb.addr["v"], g=fb.addr["g"],
                 beta=fb.addr["beta"], state_in=fb.addr["state_in"],
                 state_out=fb.addr["state_out"], N=fb.N, Nqk=fb.Nqk, Nv=fb.Nv, D=128,
                 dtype=gdr.GDR_BF16, flags=gdr.GDR_FLAG_QK_L2NORM, out=fb.addr["out"], ms=None)
        a.update(over)
        return lib.gdr_recurrent_step_bf16_state(
            a["q"], a["k"], a["v"], a["g"], a["beta"], a["state_in"], a["state_out"], a["N"],
            a["Nqk"], a["Nv"], a["D"], a["dtype"], 0.1, a["flags"], a["out"], None, a["ms"])

    st_bytes = fb.N * fb.Nv * 128 * 128 * 2
    assert call(D=64) == UNSUPPORTED
    assert call(flags=4) == UNSUPPORTED
    assert call(Nqk=3) == INVALID
    assert call(state_in=None) == INVALID
    assert call(state_out=None) == INVALID
    assert call(state_out=fb.addr["state_in"] + 8) == INVALID                 # misaligned
    assert call(state_out=fb.addr["state_in"] + st_bytes - 256) == INVALID    # partial overlap
    assert call(out=fb.addr["state_in"] + st_bytes - 256) == INVALID          # out inside state_in
    ms = ctypes.c_float(1.0)
    assert call(N=0, ms=ctypes.byref(ms)) == OK and ms.value == 0.0


def test_multi_token_validates_before_launching():
    """gdr_recurrent_multi: the checks of gdr_chunk_fwd, without a workspace."""
    import ctypes
    lib = gdr.load()
    fb = FakeBuffers()

    def call(**over):
        a = dict(q=fb.addr["q"], k=fb.addr["k"], v=fb.addr["v"], g=fb.addr["g"],
                 beta=fb.addr["beta"], state_in=fb.addr["state_in"], cu=fb.addr["cu"], N=fb.N,
                 T=fb.T, Nqk=fb.Nqk, Nv=fb.Nv, D=128, dtype=gdr.GDR_BF16,
                 flags=gdr.GDR_FLAG_QK_L2NORM, out=fb.addr["out"],
                 state_out=fb.addr["state_out"], ms=None)
        a.update(over)
        return lib.gdr_recurrent_multi(a["q"], a["k"], a["v"], a["g"], a["beta"], a["state_in"],
                                       a["cu"], a["N"], a["T"], a["Nqk"], a["Nv"], a["D"],
                                       a["dtype"], 0.1, a["flags"], a["out"], a["state_out"], None,
                                       a["ms"])

    assert call(D=64) == UNSUPPORTED
    assert call(dtype=9) == UNSUPPORTED
    assert call(flags=4) == UNSUPPORTED
    assert call(Nqk=3) == INVALID
    assert call(N=0) == INVALID
    assert call(T=-1) == INVALID
    assert call(cu=None) == INVALID
    assert call(q=None) == INVALID
    assert call(out=None) == INVALID
    assert call(q=fb.addr["q"] + 8) == INVALID                       # misaligned
    assert call(out=fb.addr["v"]) == INVALID                         # out aliases v
    assert call(state_out=fb.addr["state_in"] + 4096) == INVALID     # partial overlap
    assert call(N=1 << 20, Nqk=1, Nv=1024) == INVALID                # too many workgroups
    ms = ctypes.c_float(1.0)
    assert call(T=0, state_out=None, ms=ctypes.byref(ms)) == OK and ms.value == 0.0


def test_conv_step_validates_before_launching():
    """gdr_recurrent_step_conv: sizes, kernel size, pointers and overlaps."""
    import ctypes
    lib = gdr.load()
    N, Nqk, Nv = 2, 2, 4
    C = (2 * Nqk + Nv) * 128
    sizes = dict(x=N * C * 2, cs_in=N * C * 8, cs_out=N * C * 8, w=C * 8, bias=C * 2, a=N * Nv * 4,
                 b=N * Nv * 4, A_log=Nv * 4, dt_bias=Nv * 4, s_in=N * Nv * 65536,
                 s_out=N * Nv * 65536, out=N * Nv * 256)
    base, addr = 1 << 40, {}
    for k_, n in sizes.items():
        addr[k_] = base
        base += (n + (1 << 20)) & ~255

    def call(**over):
        a = dict(addr, K=4, N=N, Nqk=Nqk, Nv=Nv, D=128, dtype=gdr.GDR_BF16,
                 flags=gdr.GDR_FLAG_QK_L2NORM, ms=None)
        a.update(over)
        return lib.gdr_recurrent_step_conv(a["x"], a["cs_in"], a["cs_out"], a["w"], a["bias"],
                                           a["K"], a["a"], a["b"], a["A_log"], a["dt_bias"],
                                           a["s_in"], a["s_out"], a["N"], a["Nqk"], a["Nv"], a["D"],
                                           a["dtype"], 0.1, a["flags"], a["out"], None, a["ms"])

    assert call(K=3) == UNSUPPORTED
    assert call(D=64) == UNSUPPORTED
    assert call(flags=8) == UNSUPPORTED
    assert call(Nqk=3) == INVALID
    assert call(N=-1) == INVALID
    for name in ("x", "cs_in", "cs_out", "w", "a", "b", "A_log", "dt_bias", "s_in", "s_out", "out"):
        assert call(**{name: None}) == INVALID, name
    assert call(bias=addr["bias"] + 2) == INVALID                        # misaligned bias
    assert call(cs_out=addr["cs_in"]) == INVALID                         # conv update not in place
    assert call(cs_out=addr["cs_in"] + sizes["cs_in"] - 256) == INVALID
    assert call(out=addr["x"]) == INVALID
    assert call(s_out=addr["cs_out"]) == INVALID                         # outputs overlap
    assert call(s_out=addr["s_in"] + 4096) == INVALID                    # partial state overlap
    ms = ctypes.c_float(1.0)
    assert call(N=0, ms=ctypes.byref(ms)) == OK and ms.value == 0.0


def test_conv_prefill_validates_before_launching():
    """gdr_conv_prefill: sizes, kernel size, pointers and overlaps."""
    import ctypes
    lib = gdr.load()
    T, N, Nqk, Nv = 16, 2, 2, 4
    C = (2 * Nqk + Nv) * 128
    sizes = dict(x=T * C * 2, cs_in=N * C * 8, cs_out=N * C * 8, w=C * 8, bias=C * 2, a=T * Nv * 4,
                 b=T * Nv * 4, A_log=Nv * 4, dt_bias=Nv * 4, cu=(N + 1) * 4, q=T * Nqk * 256,
                 k=T * Nqk * 256, v=T * Nv * 256, g=T * Nv * 4, beta=T * Nv * 4)
    base, addr = 1 << 40, {}
    for k_, n in sizes.items():
        addr[k_] = base
        base += (n + (1 << 20)) & ~255

    def call(**over):
        a = dict(addr, K=4, N=N, T=T, Nqk=Nqk, Nv=Nv, D=128, dtype=gdr.GDR_BF16, ms=None)
        a.update(over)
        return lib.gdr_conv_prefill(a["x"], a["cs_in"], a["cs_out"], a["w"], a["bias"], a["K"],
                                    a["a"], a["b"], a["A_log"], a["dt_bias"], a["cu"], a["N"],
                                    a["T"], a["Nqk"], a["Nv"], a["D"], a["dtype"], a["q"], a["k"],
                                    a["v"], a["g"], a["beta"], None, a["ms"])

    assert call(K=2) == UNSUPPORTED
    assert call(D=64) == UNSUPPORTED
    assert call(Nqk=3) == INVALID
    assert call(N=0) == INVALID
    assert call(N=1 << 24) == INVALID                              # beyond a grid's 2^32 work-items
    assert call(T=-1) == INVALID
    for name in ("x", "w", "a", "b", "A_log", "dt_bias", "cu", "q", "k", "v", "g", "beta"):
        assert call(**{name: None}) == INVALID, name
    assert call(q=addr["q"] + 4) == INVALID                        # misaligned
    assert call(q=addr["x"]) == INVALID                            # output over an input
    assert call(k=addr["q"]) == INVALID                            # two outputs at one address
    assert call(cs_out=addr["cs_in"] + 256) == INVALID             # partial window overlap
    assert call(g=addr["beta"]) == INVALID
    ms = ctypes.c_float(1.0)
    assert call(T=0, cs_out=None, ms=ctypes.byref(ms)) == OK and ms.value == 0.0


def test_gated_rmsnorm_validates_before_launching():
    """gdr_gated_rmsnorm: D, dtype, rows, eps, pointers and overlaps."""
    lib = gdr.load()
    rows = 64
    nb = rows * 128 * 2
    addr = dict(x=1 << 40, z=(1 << 40) + (1 << 24), w=(1 << 40) + (2 << 24), y=(1 << 40) + (3 << 24))

    def call(**over):
        a = dict(addr, rows=rows, D=128, dtype=gdr.GDR_BF16, eps=1e-6, ms=None)
        a.update(over)
        return lib.gdr_gated_rmsnorm(a["x"], a["z"], a["w"], a["rows"], a["D"], a["dtype"], a["eps"],
                                     a["y"], None, a["ms"])

    assert call(D=64) == UNSUPPORTED
    assert call(dtype=3) == UNSUPPORTED
    assert call(rows=-1) == INVALID
    assert call(rows=1 << 31) == INVALID
    assert call(eps=-1e-6) == INVALID
    assert call(eps=float("inf")) == INVALID
    assert call(eps=float("nan")) == INVALID
    for name in ("x", "z", "y"):
        assert call(**{name: None}) == INVALID, name
    assert call(x=addr["x"] + 8) == INVALID                  # misaligned
    assert call(w=addr["w"] + 4) == INVALID
    assert call(y=addr["x"] + 256) == INVALID                # partial overlap with x
    assert call(y=addr["z"]) == INVALID                      # over the gate
    assert call(y=addr["w"] - nb + 128) == INVALID           # over the weight
    ms = ctypes.c_float(1.0)
    assert call(rows=0, x=None, z=None, y=None, ms=ctypes.byref(ms)) == OK and ms.value == 0.0


def test_recurrent_step_gated_validates_before_launching():
    """gdr_recurrent_step_gated: the step's checks plus the gate's."""
    lib = gdr.load()
    N, Nqk, Nv = 2, 2, 4
    sizes = dict(q=N * Nqk * 256, k=N * Nqk * 256, v=N * Nv * 256, g=N * Nv * 4, beta=N * Nv * 4,
                 s_in=N * Nv * 65536, s_out=N * Nv * 65536, z=N * Nv * 256, w=256, out=N * Nv * 256)
    base, addr = 1 << 40, {}
    for k_, n in sizes.items():
        addr[k_] = base
        base += (n + (1 << 20)) & ~255

    def call(**over):
        a = dict(addr, N=N, Nqk=Nqk, Nv=Nv, D=128, dtype=gdr.GDR_BF16, eps=1e-6, ms=None)
        a.update(over)
        return lib.gdr_recurrent_step_gated(a["q"], a["k"], a["v"], a["g"], a["beta"], a["s_in"],
                                            a["s_out"], a["N"], a["Nqk"], a["Nv"], a["D"],
                                            a["dtype"], 0.088, 1, a["z"], a["w"], a["eps"],
                                            a["out"], None, a["ms"])

    assert call(D=64) == UNSUPPORTED
    assert call(Nqk=3) == INVALID
    assert call(z=None) == INVALID                           # the gate is required
    assert call(z=addr["z"] + 4) == INVALID
    assert call(w=addr["w"] + 4) == INVALID
    assert call(eps=-1.0) == INVALID
    assert call(eps=float("nan")) == INVALID
    assert call(out=addr["z"]) == INVALID                    # output over the gate
    assert call(s_out=addr["z"]) == INVALID                  # state over the gate
    assert call(q=None) == INVALID
    ms = ctypes.c_float(1.0)
    assert call(N=0, z=None, ms=ctypes.byref(ms)) == OK and ms.value == 0.0


def test_debug_switch_and_contract_status():
    """gdr_set_debug toggles the device-side contract checks and reports the
    previous setting; the contract status has its own name.  No GPU call."""
    lib = gdr.load()
    before = lib.gdr_set_debug(-1)
    try:
        assert lib.gdr_set_debug(1) == before
        assert lib.gdr_set_debug(-1) == 1
        assert lib.gdr_set_debug(0) == 1
        assert lib.gdr_set_debug(7) == 0          # any other value only queries
        assert lib.gdr_set_debug(-1) == 0
    finally:
        lib.gdr_set_debug(before)
    assert lib.gdr_status_string(-5) == b"device values break the contract (debug checks)"
    assert gdr.STATUS[-5] == "GDR_ERR_CONTRACT"
    assert lib.gdr_debug_broken() == 0            # no checked call in this thread


def test_chunk64_flag_and_workspace():
    """GDR_FLAG_CHUNK64 is a known flag of the chunkwise call; the workspace
    size covers both chunk lengths (64-token chunks need more table slots)."""
    lib = gdr.load()
    assert gdr.GDR_FLAG_CHUNK64 == 2
    b = FakeBuffers()
    a = b.addr
    T, N, Nqk, Nv = 256, 2, 2, 4

    def call(flags, ws_bytes):
        return lib.gdr_chunk_fwd(a["q"], a["k"], a["v"], a["g"], a["beta"], a["state_in"], a["cu"],
                                 N, T, Nqk, Nv, 128, gdr.GDR_BF16, 0.088, flags, a["out"],
                                 a["state_out"], a["ws"], ws_bytes, None)

    # a missing workspace is rejected for both lengths, before any launch
    need = gdr.workspace_size(T, N, Nqk, Nv, gdr.GDR_BF16)
    assert call(gdr.GDR_FLAG_CHUNK64 | 1, 0) == WS_SMALL
    assert call(1, 0) == WS_SMALL
    assert call(4, need) == UNSUPPORTED                      # unknown flag
    # the size covers a 64-token-chunk call of many short sequences
    assert gdr.workspace_size(4096, 64, 16, 32, gdr.GDR_BF16) >= \
        gdr.workspace_size(4096, 1, 16, 32, gdr.GDR_BF16)
    with pytest.raises(ValueError):
        gdr._chunk_flags(True, 32)
    assert gdr._chunk_flags(True, 64) == 3 and gdr._chunk_flags(False, 128) == 0


def test_single_empty_sequence_plans_without_dividing_by_zero():
    """N = 1, T = 0 has no chunk slot: planning the workspace (the
    no-allocation entry point plans against its fixed array) and counting the
    timed call's launches must not divide by a segment of zero slots.  Here,
    without a GPU, each call gets past validation and planning and then
    fails at its first HIP call, or does nothing."""
    import ctypes
    lib = gdr.load()
    fb = FakeBuffers(T=0, N=1, Nqk=1, Nv=2)
    HIP_ERR = -4
    rc = lib.gdr_chunk_fwd_no_alloc(None, None, None, None, None, fb.addr["state_in"], fb.addr["cu"],
                                    1, 0, 1, 2, 128, gdr.GDR_BF16, 0.1, gdr.GDR_FLAG_QK_L2NORM,
                                    None, fb.addr["state_out"], None)
    assert rc in (OK, HIP_ERR)
    kms = (ctypes.c_float * 4)()
    kind = (ctypes.c_int32 * 4)()
    n = ctypes.c_int32(-1)
    span = ctypes.c_float(-1.0)
    for state_out in (fb.addr["state_out"], fb.addr["state_in"], None):
        rc = lib.gdr_chunk_fwd_timed(None, None, None, None, None, fb.addr["state_in"], fb.addr["cu"],
                                     1, 0, 1, 2, 128, gdr.GDR_BF16, 0.1, gdr.GDR_FLAG_QK_L2NORM,
                                     None, state_out, fb.addr["ws"], fb.sizes["ws"], None, kms, kind,
                                     4, ctypes.byref(n), ctypes.byref(span))
        assert rc in (OK, HIP_ERR)
        if state_out != fb.addr["state_out"]:
            # nothing to launch: no HIP call at all
            assert rc == OK and n.value == 0 and span.value == 0.0
