"""GPU parity at the longest context the operator page lists (T up to 1M+,
its supported-configurations table): one sequence of 2^20 tokens with
Nqk = 16, Nv = 32, bf16, through gdr_chunk_fwd in the launch configuration
the benchmark times (segments of 32 chunk slots: 256 segments here).

The oracle cannot replay a million tokens per head in a test, so the check
samples what it can compute exactly:
- the first 4096 tokens of four value heads, from the given initial state;
- the last 2048 tokens and the final state of the same heads: every head
  decays by at least exp(-0.5 softplus(a + 1)) per token here, so the
  oracle starts 128 tokens earlier from a zero state and the state it
  leaves out has been scaled by about e^-90 (or less) before the compared
  tokens begin, far below the tolerance (without those 128 tokens the
  first rows differ: head 0 decays by only e^-1 per token).
Output offsets past 2^31 elements (token 2^20 - 1 of head 31 sits at element
4.29e9) exercise the 64-bit indexing of every kernel on the path.

Inputs are drawn on the GPU with a seeded torch generator (a 24 GiB input set
is too large to draw with NumPy in a test); only the sampled slices are
copied to the host for the oracle, so both sides see the same values."""
import numpy as np
import pytest

import gated_deltanet_chunked_amd as gdr
from tests.gpu_util import SCALE, TOL, oracle, rel_l2

pytestmark = pytest.mark.gpu

T = 1 << 20
NQK, NV, D = 16, 32, 128
HEADS = (0, 9, 22, 31)
HEAD_LEN, TAIL_LEN, WARM = 4096, 2048, 128


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gdr.load()
    yield
    torch.cuda.synchronize()


def _draw(dev):
    import torch
    gen = torch.Generator(device=dev)
    gen.manual_seed(20)

    def normal(*shape):
        return torch.randn(*shape, device=dev, generator=gen)

    q = normal(T, NQK, D).to(torch.bfloat16)
    k = normal(T, NQK, D).to(torch.bfloat16)
    v = normal(T, NV, D).to(torch.bfloat16)
    a = normal(T, NV)
    b = normal(T, NV)
    A = 0.5 + 15.5 * torch.rand(NV, device=dev, generator=gen)   # every head decays
    g = (-A * torch.nn.functional.softplus(a + 1.0)).float().contiguous()
    beta = torch.sigmoid(b).float().contiguous()
    state = (0.01 * normal(1, NV, D, D)).float().contiguous()
    return q, k, v, g, beta, state


def _host(t):
    import torch
    return t.detach().to(torch.float32).cpu().numpy()


def _oracle(q, k, v, g, beta, s0, h):
    """Oracle over a token slice for value head h (its q/k head h // G)."""
    j = h // (NV // NQK)
    n = q.shape[0]
    o, s = oracle.recurrent(_host(q[:, j:j + 1]), _host(k[:, j:j + 1]), _host(v[:, h:h + 1]),
                            _host(g[:, h:h + 1]), _host(beta[:, h:h + 1]),
                            None if s0 is None else _host(s0[:, h:h + 1]),
                            np.array([0, n], np.int32), SCALE)
    return o[:, 0], s[0, 0]


def test_million_token_sequence_sampled():
    import torch
    dev = "cuda:0"
    q, k, v, g, beta, state = _draw(dev)
    cu = torch.tensor([0, T], dtype=torch.int32, device=dev)
    print(f"T={T} Nqk={NQK} Nv={NV} bf16: chunk_fwd", flush=True)
    out, st = gdr.chunk_fwd(q, k, v, g, beta, cu, state, scale=SCALE)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all().item() and torch.isfinite(st).all().item()
    tol = TOL["bf16"]
    lo, hi, warm = slice(0, HEAD_LEN), slice(T - TAIL_LEN, T), slice(T - TAIL_LEN - WARM, T)
    for h in HEADS:
        ro, _ = _oracle(q[lo], k[lo], v[lo], g[lo], beta[lo], state, h)
        e_head = rel_l2(_host(out[lo, h]), ro)
        ro, rs = _oracle(q[warm], k[warm], v[warm], g[warm], beta[warm], None, h)
        e_tail = rel_l2(_host(out[hi, h]), ro[WARM:])
        e_state = rel_l2(_host(st[0, h]), rs)
        print(f"head {h}: first {HEAD_LEN} tokens {e_head:.2e}, last {TAIL_LEN} tokens {e_tail:.2e}, "
              f"final state {e_state:.2e}", flush=True)
        assert e_head <= tol and e_tail <= tol and e_state <= tol
