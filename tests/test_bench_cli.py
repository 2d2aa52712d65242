"""bench.py's command line on the CPU: more than one GPU is refused with a
message before anything touches a GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def _bench():
    sys.path.insert(0, ROOT)
    import bench
    return bench


def test_algorithmic_flops_match_the_stated_figures():
    """The FLOP count behind the roofline: per full 128-token chunk at Nqk =
    16, Nv = 32 it is Nqk 2 D L^2 + Nv (3 D L (L + 1) + 6 L D^2 + L^3 / 3)
    = 695.0 MFLOP (5.43 MFLOP per token), so T = 32768 is 177.9 GFLOP and
    T = 4096 is 22.24 GFLOP; a short tail chunk counts its own length."""
    b = _bench()
    intra, inter = b.alg_flops_chunk([128], 16, 32)
    D, L = 128, 128
    assert intra == 16 * 2 * D * L * L + 32 * (L ** 3 / 3 + 3 * D * L * (L + 1))
    assert inter == 32 * 6 * L * D * D
    assert abs((intra + inter) / 1e6 - 695.0) < 0.05
    assert abs(sum(b.alg_flops_chunk([32768], 16, 32)) / 1e9 - 177.9) < 0.05
    assert abs(sum(b.alg_flops_chunk([4096], 16, 32)) / 1e9 - 22.24) < 0.005
    # a 130-token sequence: one full chunk and a 2-token tail
    t_intra, t_inter = b.alg_flops_chunk([2], 16, 32)
    f = b.alg_flops_chunk([130], 16, 32)
    assert f == (intra + t_intra, inter + t_inter)
    # 64-token chunks: the same formula at L = 64
    i64, e64 = b.alg_flops_chunk([128], 16, 32, chunk=64)
    assert i64 == 2 * (16 * 2 * D * 64 * 64 + 32 * (64 ** 3 / 3 + 3 * D * 64 * 65))
    assert e64 == inter


def test_decode_bytes_match_the_stated_figure():
    """256 sequences x 32 heads of fp32 128x128 states read and written, plus
    q/k/v, g/beta and out: 1,080,098,816 bytes; a bf16 state halves the state
    part."""
    b = _bench()
    assert b.alg_bytes_decode(256, 16, 32) == 1_080_098_816
    state = 256 * 32 * 128 * 128 * 4 * 2
    assert b.alg_bytes_decode(256, 16, 32, state_es=2) == 1_080_098_816 - state // 2
