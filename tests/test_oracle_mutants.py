"""Mutation check of the oracle's pins (CPU only).

Each case compiles a copy of the oracle with one plausible mistake planted in it (a
dropped term, a wrong sign or index, a reversed tap order ...) and checks that at least
one pin in test_oracle_pins fails against that copy.  The real oracle is restored after
every case.
"""
import inspect
import os
import subprocess
import tempfile

import pytest

import oracle
from tests import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "samba_oracle.c")

MUTANTS = {
    "drop_D_skip": ("acc += dsk * u;", "acc += 0.0 * u;"),
    "skip_uses_preconv_x": ("acc += dsk * u;", "acc += dsk * x[ix];"),
    "A_sign_flipped": ("exp(delta * A[(size_t)d * N + n])", "exp(-delta * A[(size_t)d * N + n])"),
    "Bbar_without_delta": ("du = delta * u;", "du = u;"),
    "input_term_preconv": ("du = delta * u;", "du = delta * x[ix];"),
    "conv_taps_reversed": ("pre += w[k] * win[k];", "pre += w[ORACLE_K - 1 - k] * win[k];"),
    "conv_history_not_shifted": ("for (k = 0; k < ORACLE_K - 1; ++k) win[k] = win[k + 1];", ";"),
    "conv_bias_dropped": ("double pre = cb, u", "double pre = 0.0 * cb, u"),
    "readout_uses_old_state": (
        "hs[n] = abar * hs[n] + du * B[(size_t)t * N + n];\n                acc += C[(size_t)t * N + n] * hs[n];",
        "acc += C[(size_t)t * N + n] * hs[n];\n                hs[n] = abar * hs[n] + du * B[(size_t)t * N + n];"),
    "B_index_t_minus_1": ("du * B[(size_t)t * N + n]", "du * B[(size_t)(t > 0 ? t - 1 : 0) * N + n]"),
    "C_transposed_with_B": ("acc += C[(size_t)t * N + n]", "acc += B[(size_t)t * N + n]"),
    "softplus_missing_max": ("return (a > 0.0 ? a : 0.0) + log1p(exp(-fabs(a)));", "return log1p(exp(-fabs(a)));"),
    "gate_is_sigmoid": ("y[ix] = z ? acc * oracle_silu(z[ix]) : acc;", "y[ix] = z ? acc / (1.0 + exp(-z[ix])) : acc;"),
    "gate_missing": ("y[ix] = z ? acc * oracle_silu(z[ix]) : acc;", "y[ix] = acc;"),
    "dt_bias_dropped": ("delta = oracle_softplus(dt[ix] + bias);", "delta = oracle_softplus(dt[ix]);"),
    "silu_is_sigmoid": ("return v / (1.0 + exp(-v));", "return 1.0 / (1.0 + exp(-v));"),
    "state_not_carried_in": ("for (n = 0; n < N; ++n) hs[n] = h[(size_t)d * N + n];", "for (n = 0; n < N; ++n) hs[n] = 0.0;"),
    "conv_alone_bias_dropped": ("double pre = cb;\n", "double pre = 0.0 * cb;\n"),
    "conv_alone_current_token_late": (
        "double pre = cb;\n            win[ORACLE_K - 1] = x[ix];\n            for (k = 0; k < ORACLE_K; ++k) pre += w[k] * win[k];",
        "double pre = cb;\n            for (k = 0; k < ORACLE_K; ++k) pre += w[k] * win[k];\n            win[ORACLE_K - 1] = x[ix];"),
    "bwd_adjoint_not_decayed": ("R[n] = G * abar;", "R[n] = G;"),
    "bwd_dA_without_delta": ("dA[(size_t)d * N + n] += G * abar * hp * delta[t];",
                             "dA[(size_t)d * N + n] += G * abar * hp;"),
    "bwd_gate_derivative_sigmoid_only": ("dz[ix] = dout[ix] * y[t] * sz * (1.0 + z[ix] * (1.0 - sz));",
                                         "dz[ix] = dout[ix] * y[t] * sz;"),
    "bwd_silu_derivative_dropped": ("dpre = du * sp * (1.0 + pre[t] * (1.0 - sp));", "dpre = du * sp;"),
    "bwd_conv_transpose_taps_reversed": ("dx[ix] = P1 + w[3] * dpre;", "dx[ix] = P1 + w[0] * dpre;"),
    "bwd_dB_missing_u": ("dB[(size_t)t * N + n] += G * delta[t] * u[t];", "dB[(size_t)t * N + n] += G * delta[t];"),
    "bwd_du_missing_skip": ("du = gy * dsk;", "du = 0.0;"),
    "bwd_previous_state_is_current": (
        "const double hp = t > 0 ? hs[(size_t)(t - 1) * N + n] : h0[(size_t)d * N + n];",
        "const double hp = hs[(size_t)t * N + n];"),
    "bwd_softplus_derivative_dropped": ("da = ddel * sigm(av[t]);", "da = ddel;"),
    "swa_window_off_by_one": ("const int lo = t - window > t0 ? t - window : t0;",
                              "const int lo = t - window + 1 > t0 ? t - window + 1 : t0;"),
    "swa_rope_rotation_reversed": ("v[2 * i] = a * c - b * sn;\n        v[2 * i + 1] = a * sn + b * c;",
                                   "v[2 * i] = a * c + b * sn;\n        v[2 * i + 1] = -a * sn + b * c;"),
    "swa_rope_frequency_exponent": ("pow(base, -2.0 * i / dh)", "pow(base, -1.0 * i / dh)"),
    "swa_scale_missing": ("sc[j - lo] = dot / sqrt((double)dh);", "sc[j - lo] = dot;"),
    "swa_kv_head_interleaved": ("const int hk = h / group;", "const int hk = h % Hkv;"),
    "swa_absolute_positions": ("oracle_rope(kv, dh, (double)(j - t0), base);", "oracle_rope(kv, dh, (double)j, base);"),
    "u_scan_drop_skip": ("acc += dsk * uu;", "acc += 0.0 * uu;"),
    "u_scan_input_without_u": ("const double du = delta * uu;", "const double du = delta;"),
    "u_scan_bias_dropped": ("const double delta = oracle_softplus(dt[ix] + bias);\n                const double du = delta * uu;",
                            "const double delta = oracle_softplus(dt[ix]);\n                const double du = delta * uu;"),
    "u_scan_gate_missing": ("y[ix] = z ? acc * oracle_silu(z[ix]) : acc;\n            }\n            for (n = 0; n < N; ++n) hseq",
                            "y[ix] = acc;\n            }\n            for (n = 0; n < N; ++n) hseq"),
    "history_not_carried_in": ("for (k = 0; k < ORACLE_K - 1; ++k) win[k] = hist[(size_t)k * ldh + d];",
                               "for (k = 0; k < ORACLE_K - 1; ++k) win[k] = 0.0;"),
}

PIN_TESTS = [(n, f) for n, f in inspect.getmembers(pins, inspect.isfunction) if n.startswith("test_")]


def _run_pins():
    failed = []
    for name, fn in PIN_TESTS:
        params = inspect.signature(fn).parameters
        variants = [{}]
        if "with_hist" in params:
            variants = [{"with_hist": False}, {"with_hist": True}]
        if "with_h0" in params:
            variants = [{"with_h0": False}, {"with_h0": True}]
        if "gate" in params:
            variants = [{"gate": True}, {"gate": False}]
        if "Hq" in params:
            variants = [{"Hq": 4, "Hkv": 4}, {"Hq": 6, "Hkv": 2}]
        for kw in variants:
            try:
                fn(**kw)
            except AssertionError:
                failed.append(name)
    return failed


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_pins_catch_planted_mistake(mutant):
    old, new = MUTANTS[mutant]
    src = open(SRC).read()
    assert src.count(old) >= 1, "mutation anchor not found: " + mutant
    with tempfile.TemporaryDirectory() as td:
        c = os.path.join(td, "mut.c")
        so = os.path.join(td, "libmut.so")
        open(c, "w").write(src.replace(old, new))
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", so, c, "-lm"])
        oracle._use_library(so)
        try:
            failed = _run_pins()
        finally:
            oracle._reset()
    assert failed, "no pin caught mutant " + mutant


def test_unmutated_oracle_passes_all_pins():
    oracle._reset()
    assert _run_pins() == []
