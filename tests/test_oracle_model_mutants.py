"""Mutation check of the layer oracle's pins (CPU only).

Each case loads a copy of oracle/model.py with one plausible wiring mistake planted in it
(x instead of u into an x_proj product, the gate from u or from the un-normed stream, the
conv fed with u, keys kept as values, a layer reading the raw stream, a dropped residual,
the SwiGLU factors swapped, the sequence form diverging from the step form ...) and checks
that at least one pin in test_oracle_model_wiring / test_oracle_model_pins fails against
that copy.  The modules' own `model` is restored after every case.
"""
import inspect
import os
import types

import pytest

from oracle import model as real_model
from tests import test_oracle_model_pins as pins
from tests import test_oracle_model_wiring as wiring

SRC = os.path.join(os.path.dirname(real_model.__file__), "model.py")

MUTANTS = {
    "B_from_x": ("Bm, Cm = act(linear(u, w_b)), act(linear(u, w_c))", "Bm, Cm = act(linear(x, w_b)), act(linear(u, w_c))"),
    "C_from_x": ("Bm, Cm = act(linear(u, w_b)), act(linear(u, w_c))", "Bm, Cm = act(linear(u, w_b)), act(linear(x, w_c))"),
    "dt_from_x": ("dt = act(linear(act(linear(u, w_r)), ly[\"w_dt_up\"]))",
                  "dt = act(linear(act(linear(x, w_r)), ly[\"w_dt_up\"]))"),
    "gate_from_u": ("y = act(oracle.decode_step(x, dt, Bm, Cm, z,", "y = act(oracle.decode_step(x, dt, Bm, Cm, u,"),
    "gate_unnormed": ("x, z = act(linear(hn, w_in)), act(linear(hn, w_g))",
                      "x, z = act(linear(hn, w_in)), act(linear(hidden, w_g))"),
    "gate_and_input_swapped": ("x, z = act(linear(hn, w_in)), act(linear(hn, w_g))",
                               "z, x = act(linear(hn, w_in)), act(linear(hn, w_g))"),
    "conv_fed_with_u_history": ("y = act(oracle.decode_step(x, dt, Bm, Cm, z,", "y = act(oracle.decode_step(u, dt, Bm, Cm, z,"),
    "mamba_input_unnormed": ("x, z = act(linear(hn, w_in))", "x, z = act(linear(hidden, w_in))"),
    "mamba_residual_dropped": ("hidden += linear(y, ly[\"w_out\"])", "hidden = linear(y, ly[\"w_out\"])"),
    "swa_values_are_keys": ("state.v[i][s] = np.concatenate([state.v[i][s], v[s][None]])",
                            "state.v[i][s] = np.concatenate([state.v[i][s], k[s][None]])"),
    "swa_output_unprojected": ("hidden += linear(act(o.reshape(S, H * dh)), ly[\"w_o\"])",
                               "hidden += act(o.reshape(S, H * dh))[:, :hidden.shape[1]]"),
    "swa_inactive_attends": ("                if p < 0:\n                    continue\n",
                             "                if p < 0:\n                    p = 0\n"),
    "mlp_unnormed": ("m = act(swiglu(hn, ly[\"w12\"][:dff], ly[\"w12\"][dff:]))",
                     "m = act(swiglu(hidden, ly[\"w12\"][:dff], ly[\"w12\"][dff:]))"),
    "swiglu_factors_swapped": ("return linear(x, w1_t) * silu(linear(x, w2_t))",
                               "return silu(linear(x, w1_t)) * linear(x, w2_t)"),
    "rmsnorm_without_sqrt": ("x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)",
                             "x / (np.mean(x * x, axis=-1, keepdims=True) + eps)"),
    "final_norm_missing": ("    return hidden, rmsnorm(hidden, final_norm_w, eps)\n\n\ndef prefill",
                           "    return hidden, hidden.copy()\n\n\ndef prefill"),
    "prefill_B_from_x": ("Bm = linear(u2, w_b).reshape(S, L, -1)", "Bm = linear(x.reshape(S * L, de), w_b).reshape(S, L, -1)"),
    "prefill_gate_from_u": ("y, _, _ = oracle.prefill(x, dt, Bm, Cm, z,", "y, _, _ = oracle.prefill(x, dt, Bm, Cm, u,"),
}
# The same reading mistaken in both the step form and the sequence form (a conceptual error
# their agreement cannot show): only the wiring pins can catch these.
MUTANTS_BOTH = {
    "both_B_from_x": [MUTANTS["B_from_x"], MUTANTS["prefill_B_from_x"]],
    "both_gate_from_u": [MUTANTS["gate_from_u"], MUTANTS["prefill_gate_from_u"]],
    "both_dt_from_x": [MUTANTS["dt_from_x"],
                       ("dt = linear(linear(u2, w_r), ly[\"w_dt_up\"]).reshape(S, L, de)",
                        "dt = linear(linear(x.reshape(S * L, de), w_r), ly[\"w_dt_up\"]).reshape(S, L, de)")],
    "both_C_from_x": [MUTANTS["C_from_x"],
                      ("Cm = linear(u2, w_c).reshape(S, L, -1)", "Cm = linear(x.reshape(S * L, de), w_c).reshape(S, L, -1)")],
}

PIN_MODULES = (wiring, pins)


def _load_mutant(edits):
    src = open(SRC).read()
    for old, new in edits:
        assert src.count(old) == 1, "mutation site not found exactly once: %r" % old
        src = src.replace(old, new)
    mod = types.ModuleType("oracle_model_mutant")
    mod.__file__ = SRC
    exec(compile(src, SRC + " (mutant)", "exec"), mod.__dict__)
    return mod


def _run_pins():
    failed = []
    for pm in PIN_MODULES:
        for name, fn in inspect.getmembers(pm, inspect.isfunction):
            if not name.startswith("test_") or fn.__module__ != pm.__name__:
                continue
            try:
                fn()
            except Exception:  # an assertion or an exception caused by the mistake
                failed.append(name)
    return failed


def test_unmutated_layer_oracle_passes_every_pin():
    assert _run_pins() == []


ALL = {**{k: [v] for k, v in MUTANTS.items()}, **MUTANTS_BOTH}


@pytest.mark.parametrize("name", sorted(ALL))
def test_planted_mistake_is_caught(name):
    mut = _load_mutant(ALL[name])
    saved = [pm.model for pm in PIN_MODULES]
    try:
        for pm in PIN_MODULES:
            pm.model = mut
        failed = _run_pins()
    finally:
        for pm, m in zip(PIN_MODULES, saved):
            pm.model = m
    assert failed, "mutant %s passes every pin" % name
