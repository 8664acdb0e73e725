"""The fp64 oracle against its pins (CPU only), and proof that the pins bite:
mutated copies of the oracle source, each carrying one plausible mistake, must
fail at least one pin."""
import os
import shutil
import tempfile

import pytest

import oracle
from tests import oracle_pins as pins


@pytest.fixture(scope="module")
def o():
    return oracle.default()


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(o, pin):
    pin(o)


_UPDATE = """    for (int p = 0; p < P; ++p)
        for (int n = 0; n < N; ++n)
            S[(size_t)p * N + n] = a * S[(size_t)p * N + n] + dt * x[p] * Bv[n];
"""
_READ = """    for (int p = 0; p < P; ++p) {
        double acc = 0.0;
        for (int n = 0; n < N; ++n) acc += Cv[n] * S[(size_t)p * N + n];
        y[p] = acc + Dh * x[p];
    }
"""

# One plausible mistake per entry: (name, text in ssd_oracle.c, replacement).
MUTATIONS = [
    ("dropped_decay", "S[(size_t)p * N + n] = a * S[(size_t)p * N + n]", "S[(size_t)p * N + n] = S[(size_t)p * N + n]"),
    ("dropped_dt_on_input", "+ dt * x[p] * Bv[n]", "+ x[p] * Bv[n]"),
    ("decay_sign", "double a = exp(dt * A);", "double a = exp(-dt * A);"),
    ("read_with_B", "acc += Cv[n] * S", "acc += Bv[n] * S"),
    ("output_before_update", _UPDATE + _READ, _READ + _UPDATE),
    ("dropped_skip", "y[p] = acc + Dh * x[p];", "y[p] = acc;"),
    ("taps_reversed", "v += w[k] * win[k];", "v += w[K - 1 - k] * win[k];"),
    ("conv_offset", "t - (K - 1) + k, c);", "t - K + k, c);"),
    ("no_doc_reset_scan", "if (doc && t > 0 && doc[row] != doc[row - 1])", "if (0)"),
    ("no_doc_reset_conv", "return tau >= seg ? raw_b[(size_t)tau * C + c] : 0.0;", "return raw_b[(size_t)tau * C + c];"),
    ("wrong_group", "const int g = h / hpg;\n            double *S", "const int g = h % G;\n            double *S"),
    ("softplus_no_bias", "d = softplus(d + (dt_bias ? dt_bias[h] : 0.0));", "d = softplus(d);"),
    ("gate_sigmoid_only", "if (z) v *= silu(z[row * HP", "if (z) v *= 1.0 / (1.0 + exp(-z[row * HP"),
    ("state_transposed", "S[(size_t)p * N + n] = a * S[(size_t)p * N + n] + dt * x[p] * Bv[n];",
     "S[(size_t)n * P + p] = a * S[(size_t)n * P + p] + dt * x[p] * Bv[n];"),
    ("conv_state_shift", "memcpy(cs + (size_t)k * C, cs + (size_t)(k + 1) * C", "memcpy(cs + (size_t)(k + 1) * C, cs + (size_t)k * C"),
    ("step_no_round", "xbc[c] = round_bf16 ? oracle_round_bf16(v) : v;", "xbc[c] = v;"),
    ("round_truncates", "double r = rint(v / q) * q;", "double r = trunc(v / q) * q;"),
    # the Mamba-1 S6 scan
    ("s6_decay_one_rate", "h[n] = exp(dtv * Ad[n]) * h[n]", "h[n] = exp(dtv * Ad[0]) * h[n]"),
    ("s6_A_transposed", "h[n] = exp(dtv * Ad[n]) * h[n]", "h[n] = exp(dtv * A[(size_t)n * D + d]) * h[n]"),
    ("s6_dropped_dt_on_input", "+ dtv * Bt[n] * xv;", "+ Bt[n] * xv;"),
    ("s6_read_with_B", "acc += Ct[n] * h[n];", "acc += Bt[n] * h[n];"),
    ("s6_dropped_skip", "double v = acc + (D_skip ? D_skip[d] : 0.0) * xv;", "double v = acc;"),
    ("s6_no_doc_reset", "if (doc && t > 0 && doc[row] != doc[row - 1]) memset(h", "if (0) memset(h"),
    ("s6_bias_outside", "dtv = softplus(dtv + (dt_bias ? dt_bias[d] : 0.0));",
     "dtv = softplus(dtv) + (dt_bias ? dt_bias[d] : 0.0);"),
    # the backward (VJP)
    ("bwd_adjoint_not_decayed", "dS[i] = reset ? 0.0 : a * dS[i];", "dS[i] = reset ? 0.0 : dS[i];"),
    ("bwd_adjoint_not_reset", "dS[i] = reset ? 0.0 : a * dS[i];", "dS[i] = a * dS[i];"),
    ("bwd_decay_uses_new_state", "if (!reset) da += g_pn * Sp[", "if (!reset) da += g_pn * Sc["),
    ("bwd_dB_without_dt", "dBv[n] += d * g_pn * xv[p];", "dBv[n] += g_pn * xv[p];"),
    ("bwd_dx_without_skip", "dxv[p] = Dh * dyr;", "dxv[p] = 0.0;"),
    ("bwd_dC_from_old_state", "dCv[n] += dyr * Sc[", "dCv[n] += dyr * Sp["),
    ("bwd_dt_no_decay_term", "dd += da * a * Ah;", "dd += 0.0 * da;"),
    ("bwd_dA_without_dt", "sA += da * a * d;", "sA += da * a;"),
    ("bwd_softplus_chain_dropped", "ddt[row * H + h] = dd * s;", "ddt[row * H + h] = dd;"),
    ("bwd_gate_derivative_as_silu", "gyv * yr * dsilu(zv)", "gyv * yr * silu(zv)"),
    ("bwd_adjoint_misses_output", "dS[(size_t)p * N + n] += Cv[n] * dyr;", "dS[(size_t)p * N + n] += Bv[n] * dyr;"),
    ("conv_bwd_taps_reversed", "draw[((size_t)b * L + tau) * C + c] += w[(size_t)c * K + k] * gp;",
     "draw[((size_t)b * L + tau) * C + c] += w[(size_t)c * K + (K - 1 - k)] * gp;"),
    ("conv_bwd_no_act_derivative", "go * dsilu(pre)", "go"),
    ("conv_bwd_ignores_documents", "if (tau >= seg && tau >= 0) {", "if (tau >= 0) {"),
    ("conv_bwd_dt_no_sigmoid", "ddt_raw[i] = ddt[i] * s;", "ddt_raw[i] = ddt[i];"),
]


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_planted_mistakes(name, old, new):
    with open(oracle.SOURCE) as f:
        src = f.read()
    assert src.count(old) >= 1, f"mutation {name}: pattern not found in the oracle source"
    if name == "gate_sigmoid_only":
        new_src = src.replace(old, new).replace("+ (size_t)h * P + p]);\n                    y[row",
                                                "+ (size_t)h * P + p]));\n                    y[row", 1)
    else:
        new_src = src.replace(old, new, 1)
    d = tempfile.mkdtemp(prefix="oracle_mut_")
    try:
        path = os.path.join(d, "m.c")
        with open(path, "w") as f:
            f.write(new_src)
        mutant = oracle.Oracle(oracle.compile_source(path, os.path.join(d, "libm.so")))
        failed = []
        for pin in pins.ALL_PINS:
            try:
                pin(mutant)
            except (AssertionError, ValueError, FloatingPointError):
                failed.append(pin.__name__)
        assert failed, f"no pin caught the planted mistake '{name}'"
    finally:
        shutil.rmtree(d, ignore_errors=True)
