"""Plant plausible mistakes in copies of oracle.c (on the CPU) and check that
the pins catch every one of them.  This is what makes the pins trustworthy:
a dropped term, a wrong sign or index, a transposed operand each fail at
least one pin."""
import os

import pytest

import oracle
from oracle_pins import ALL_PINS

with open(oracle.SOURCE) as _f:
    _SRC = _f.read()

# (name, text to find, replacement); each must occur in oracle.c
MUTANTS = [
    ("euler_bbar", "*bcoef = expm1(delta * a) / a;", "*bcoef = delta;"),
    ("bbar_missing_delta", "*bcoef = expm1(delta * a) / a;",
     "*bcoef = expm1(delta * a) / (delta * a);"),
    ("abar_sign", "*abar = exp(delta * a);", "*abar = exp(-delta * a);"),
    ("no_softplus", "double delta = oracle_softplus(dtv + bias);",
     "double delta = exp(dtv + bias);"),
    ("bias_dropped", "oracle_softplus(dtv + bias)", "oracle_softplus(dtv)"),
    ("b_c_swapped", "bcoef * Bt[n] * xv;", "bcoef * Ct[n] * xv;"),
    ("readout_before_update",
     "        h[n] = abar * h[n] + bcoef * Bt[n] * xv;\n    }\n    for (int64_t n = 0; n < N; ++n)\n        y += Ct[n] * h[n];",
     "        y += Ct[n] * h[n];\n        h[n] = abar * h[n] + bcoef * Bt[n] * xv;\n    }"),
    ("gate_excludes_skip", "    y += Dv * xv;\n    if (zv)\n        y *= oracle_silu(*zv);",
     "    if (zv)\n        y *= oracle_silu(*zv);\n    y += Dv * xv;"),
    ("silu_is_sigmoid", "return z / (1.0 + exp(-z));", "return 1.0 / (1.0 + exp(-z));"),
    ("h0_ignored", "h[n] = h0 ? h0[n] : 0.0;", "h[n] = 0.0;"),
    ("conv_taps_reversed", "acc += w[d * K + k] * xr[s];",
     "acc += w[d * K + (K - 1 - k)] * xr[s];"),
    ("conv_off_by_one", "int64_t s = t - (K - 1) + k;", "int64_t s = t - K + k;"),
    ("conv_bias_dropped", "double acc = bias ? bias[d] : 0.0;", "double acc = 0.0;"),
    ("dskip_channel_index", "j->Dskip ? j->Dskip[d] : 0.0", "j->Dskip ? j->Dskip[0] : 0.0"),
    ("a_row_index", "j->A + d * j->N,", "j->A,"),
    ("bwd_ddelta_drops_state", "dDelta += lam * ab * (Ad[n] * hp + Bt[n] * xr[t]);",
     "dDelta += lam * ab * (Bt[n] * xr[t]);"),
    ("bwd_adjoint_not_decayed", "nu[n] = ab * lam;", "nu[n] = lam;"),
    ("bwd_dbcoef_wrong_power", "return (u * exp(u) - expm1(u)) / (a * a);",
     "return (u * exp(u) - expm1(u)) / a;"),
    ("bwd_no_softplus_slope", "ddt[c * L + t] = dDelta / (1.0 + exp(-v));",
     "ddt[c * L + t] = dDelta;"),
    ("bwd_dC_uses_previous_state", "dCt[n] += dy * hist[(t + 1) * N + n];",
     "dCt[n] += dy * hist[t * N + n];"),
    ("conv_window_not_moved", "                st[k] = st[k + 1];", "                st[k] = st[k];"),
    ("conv_update_new_input_tap", "acc += w[d * K + K - 1] * x[c];", "acc += w[d * K] * x[c];"),
    ("ssd_group_index", "const int64_t g = h / heads_per_group;",
     "const int64_t g = h % G;"),
    ("ssd_readout_before_update",
     "                        S[p * N + n] = abar * S[p * N + n] + bcoef * Bt[n] * xv;\n"
     "                        acc += Ct[n] * S[p * N + n];",
     "                        acc += Ct[n] * S[p * N + n];\n"
     "                        S[p * N + n] = abar * S[p * N + n] + bcoef * Bt[n] * xv;"),
    ("ssd_dt_per_channel", "oracle_softplus(dt[(b * L + t) * H + h] + bias)",
     "oracle_softplus(dt[(b * L + t) * H] + bias)"),
    ("ssd_h0_transposed", "S[i] = h0 ? h0[(b * H + h) * P * N + i] : 0.0;",
     "S[i] = h0 ? h0[(b * H + h) * P * N + (i % N) * P + i / N] : 0.0;"),
    ("ssd_skip_head_index", "const double Dv = Dskip ? Dskip[h] : 0.0;",
     "const double Dv = Dskip ? Dskip[0] : 0.0;"),
]


@pytest.mark.parametrize("name,find,repl", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(tmp_path, name, find, repl):
    assert _SRC.count(find) >= 1, f"mutation site for {name} not found in oracle.c"
    src = tmp_path / f"oracle_{name}.c"
    src.write_text(_SRC.replace(find, repl))
    lib = oracle.compile_oracle(str(src), str(tmp_path / f"lib_{name}.so"))
    mutant = oracle.Oracle(lib)
    caught = []
    for pin in ALL_PINS:
        try:
            pin(mutant)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin detects the planted mistake {name}"
    os.remove(lib)
