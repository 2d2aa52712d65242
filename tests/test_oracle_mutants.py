"""Plant one mistake at a time in a copy of the oracle and check a pin fails.

Each mutant is a textual edit of ``oracle/gdr_oracle.c`` compiled into a
temporary library on the CPU.  A mutant that passes every pin would mean the
pins cannot tell that mistake from the rule, so each must fail at least one.
"""
import functools
import os
import subprocess

import pytest

import oracle
from tests import oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "gdr_oracle.c")

MUTANTS = {
    "read_before_decay": ("for (int32_t c = 0; c < Dk; ++c) { Sr[c] *= alpha; u += Sr[c] * kh[c]; }",
                          "for (int32_t c = 0; c < Dk; ++c) { u += Sr[c] * kh[c]; Sr[c] *= alpha; }"),
    "output_before_write": ("{ Sr[c] += delta * kh[c]; o += Sr[c] * qh[c]; }",
                            "{ o += Sr[c] * qh[c]; Sr[c] += delta * kh[c]; }"),
    "beta_dropped": ("const double delta = bt * (vt[r0 + r] - u);",
                     "const double delta = (vt[r0 + r] - u);"),
    "delta_sign": ("const double delta = bt * (vt[r0 + r] - u);",
                   "const double delta = bt * (vt[r0 + r] + u);"),
    "state_transposed": ("state_in[state_off + (size_t)(r0 + r) * Dk + c]",
                         "state_in[state_off + (size_t)c * Dv + (r0 + r)]"),
    "gqa_interleaved": ("const int32_t j = h / group;", "const int32_t j = h % Nqk;"),
    "eps_outside_sqrt": ("const double rk = l2norm ? 1.0 / sqrt(ssk + eps) : 1.0;",
                         "const double rk = l2norm ? 1.0 / (sqrt(ssk) + eps) : 1.0;"),
    "scale_dropped": ("const double rq = l2norm ? scale / sqrt(ssq + eps) : scale;",
                      "const double rq = l2norm ? 1.0 / sqrt(ssq + eps) : scale;"),
    "gate_wrong_head": ("const double alpha = exp(g[(size_t)t * Nv + h]);",
                        "const double alpha = exp(g[(size_t)t * Nv + j]);"),
    "query_unnormalised": ("ssq += qt[c] * qt[c];", "ssq += 1.0;"),
    "decay_squared": ("Sr[c] *= alpha;", "Sr[c] *= alpha * alpha;"),
    "write_unnormalised_key": ("{ Sr[c] += delta * kh[c]; o += Sr[c] * qh[c]; }",
                               "{ Sr[c] += delta * kt[c]; o += Sr[c] * qh[c]; }"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    path = tmp_path / f"{name}.c"
    path.write_text(src.replace(old, new))
    lib_path = tmp_path / f"lib{name}.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", str(path),
                    "-o", str(lib_path), "-lm"], check=True)
    lib = oracle.load_library(str(lib_path))
    rec = functools.partial(oracle.recurrent, lib=lib)
    failures = []
    for pin in pins.ALL_PINS:
        try:
            failures += pin(rec)
        except Exception as e:  # a crash on a mutant also counts as caught
            failures.append(f"{pin.__name__} raised {e!r}")
    assert failures, f"mutant {name} passed every pin"
