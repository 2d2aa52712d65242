"""Plant one mistake at a time in a copy of the oracle's Python functions (the
bf16 rounding, the bf16-state step, the decode prologue and the gated RMSNorm)
and check that a pin fails.

Each mutant is a textual edit of ``oracle/__init__.py`` loaded as a separate
module.  Its functions replace the oracle's while the pins of
``test_oracle_bf16_state.py``, ``test_oracle_prologue.py`` and
``test_oracle_gated_norm.py`` run; a mutant that passes every pin would mean
those pins cannot tell that mistake from the definition, so each must fail at
least one.
"""
import importlib.util
import inspect
import os

import pytest

import oracle
from tests import test_oracle_bf16_state as pins_bf16
from tests import test_oracle_gated_norm as pins_norm
from tests import test_oracle_prologue as pins_prologue

SRC = os.path.join(os.path.dirname(oracle.__file__), "__init__.py")

MUTANTS = {
    "round_ties_away": ("r = np.rint(x / quantum) * quantum", "r = np.floor(x / quantum + 0.5) * quantum"),
    "round_truncates": ("r = np.rint(x / quantum) * quantum", "r = np.trunc(x / quantum) * quantum"),
    "round_spacing_doubled": ("np.maximum(e, -125) - 8", "np.maximum(e, -125) - 7"),
    "state_not_rounded": ("return out, round_bf16(sout)", "return out, sout"),
    "conv_kernel_flipped": ("y = np.sum(new_state * w[None, :, :], axis=2)",
                            "y = np.sum(new_state * w[None, :, ::-1], axis=2)"),
    "conv_on_old_window": ("y = np.sum(new_state * w[None, :, :], axis=2)",
                           "y = np.sum(cs * w[None, :, :], axis=2)"),
    "window_shifted_wrong_way": ("new_state = np.concatenate([cs[:, :, 1:], x[:, :, None]], axis=2)",
                                 "new_state = np.concatenate([x[:, :, None], cs[:, :, :-1]], axis=2)"),
    "silu_dropped": ("y = y / (1.0 + np.exp(-y))", "y = y"),
    "bias_dropped": ("        y = y + _f64(conv_b)[None, :]", "        y = y"),
    "q_and_k_swapped": ("q = y[:, :Nqk * D].reshape(N, Nqk, D)",
                        "q = y[:, Nqk * D:2 * Nqk * D].reshape(N, Nqk, D)"),
    "softplus_dropped": ("g = -np.exp(_f64(A_log))[None, :] * softplus",
                         "g = -np.exp(_f64(A_log))[None, :] * z"),
    "dt_bias_dropped": ("z = _f64(a) + _f64(dt_bias)[None, :]", "z = _f64(a)"),
    "beta_sign": ("beta = 1.0 / (1.0 + np.exp(-_f64(b)))", "beta = 1.0 / (1.0 + np.exp(_f64(b)))"),
    "activation_not_rounded": ("    if activation_bf16:\n        y = round_bf16(y)",
                               "    if False:\n        y = round_bf16(y)"),
    "prefill_window_off_by_one": ("full[:, t + 1:t + 1 + K] * w", "full[:, t:t + K] * w"),
    "prefill_new_window_from_start": ("new_state[n] = full[:, -K:]", "new_state[n] = full[:, :K]"),
    "A_log_not_exponentiated": ("g = -np.exp(_f64(A_log))[None, :] * softplus",
                                "g = -_f64(A_log)[None, :] * softplus"),
    "norm_sum_not_mean": ("inv = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)",
                          "inv = 1.0 / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)"),
    "norm_eps_outside_root": ("inv = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)",
                              "inv = 1.0 / (np.sqrt(np.mean(x * x, axis=-1, keepdims=True)) + eps)"),
    "norm_over_wrong_axis": ("inv = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)",
                             "inv = 1.0 / np.sqrt(np.mean(x * x, axis=0, keepdims=True) + eps)"),
    "gate_sigmoid_not_silu": ("y = x * inv * w * (z / (1.0 + np.exp(-z)))",
                              "y = x * inv * w * (1.0 / (1.0 + np.exp(-z)))"),
    "gate_dropped": ("y = x * inv * w * (z / (1.0 + np.exp(-z)))", "y = x * inv * w"),
    "norm_weight_dropped": ("y = x * inv * w * (z / (1.0 + np.exp(-z)))",
                            "y = x * inv * (z / (1.0 + np.exp(-z)))"),
    "norm_weight_one_plus": ("w = np.ones(x.shape[-1]) if weight is None else _f64(weight)",
                             "w = np.ones(x.shape[-1]) if weight is None else 1.0 + _f64(weight)"),
    "gated_step_not_cast": ("o = round_bf16(out) if out_bf16 else out", "o = out"),
}

REPLACED = ("round_bf16", "recurrent_step_bf16_state", "decode_prologue", "prefill_prologue",
            "recurrent_step_conv", "gated_rmsnorm", "recurrent_step_gated")


def _mutant_module(name, old, new):
    text = open(SRC).read()
    assert text.count(old) == 1, f"{name}: anchor not found once"
    spec = importlib.util.spec_from_loader(f"oracle_mutant_{name}", loader=None)
    mod = importlib.util.module_from_spec(spec)
    mod.__dict__["__file__"] = SRC
    exec(compile(text.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    mod._lib = oracle._load()   # the C recurrence is not mutated here
    return mod


def _pins():
    for mod in (pins_bf16, pins_prologue, pins_norm):
        for n, fn in sorted(vars(mod).items()):
            if n.startswith("test_") and callable(fn):
                yield n, fn


def _run(fn):
    params = inspect.signature(fn).parameters
    if "l2norm" in params:
        fn(l2norm=True)
    else:
        fn()


def test_pins_pass_on_the_oracle():
    for _, fn in _pins():
        _run(fn)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    mod = _mutant_module(name, *MUTANTS[name])
    for attr in REPLACED:
        monkeypatch.setattr(oracle, attr, getattr(mod, attr))
    failed = []
    for pin, fn in _pins():
        try:
            _run(fn)
        except (AssertionError, ValueError, FloatingPointError):
            failed.append(pin)
    assert failed, f"mutant {name} passes every pin"
