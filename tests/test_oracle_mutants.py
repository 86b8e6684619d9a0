"""Sensitivity of the pins: plant one plausible mistake at a time in a copy of
oracle.c (CPU only, in a temporary directory), rebuild it, and require that
at least one pin fails.  Every mutation keeps all memory accesses in bounds."""
import os

import pytest

import oracle
from oracle_pins import ALL_PINS

# (name, text in oracle.c, replacement)
MUTANTS = [
    ("conv_taps_reversed", "(double)w[d * K + k] * (double)x[(b * L + t - k) * D + d]",
     "(double)w[d * K + (K - 1 - k)] * (double)x[(b * L + t - k) * D + d]"),
    ("conv_bias_dropped", "double acc = bias ? (double)bias[d] : 0.0;", "double acc = 0.0;"),
    ("conv_not_causal_at_k", "if (t >= k) acc +=", "if (t > k) acc +="),
    ("silu_sign", "return v / (1.0 + exp(-v));", "return v / (1.0 + exp(v));"),
    ("softplus_no_abs", "log1p(exp(-fabs(v)))", "log1p(exp(-v))"),
    ("clamp_lo_moved", "A_LOG_LO = -10.0;", "A_LOG_LO = -9.0;"),
    ("clamp_hi_moved", "A_LOG_HI = 5.0;", "A_LOG_HI = 6.0;"),
    ("a_sign", "    return -exp(c);", "    return exp(-c);"),
    ("zoh_missing_div_a", "return expm1(dv * A) / A * Bv;", "return expm1(dv * A) * Bv;"),
    ("zoh_wrong_sign", "return expm1(dv * A) / A * Bv;", "return expm1(-dv * A) / A * Bv;"),
    ("euler_missing_dv", "    return dv * Bv;", "    return Bv;"),
    ("no_decay", "h[n] = ab * h[n] + bb * uv;", "h[n] = h[n] + bb * uv;"),
    ("output_uses_B", "acc += (double)a->Cm[r * N + n] * h[n];",
     "acc += (double)a->Bm[r * N + n] * h[n];"),
    ("skip_dropped", "double acc = Dd * uv;", "double acc = 0.0;"),
    ("gate_dropped", "y[t * y_stride] = a->z ? acc * silu((double)a->z[r * D + d]) : acc;",
     "y[t * y_stride] = acc;"),
    ("hcache_before_update",
     "h[n] = ab * h[n] + bb * uv;\n            if (hc) hc[t * hc_stride + n] = h[n];",
     "if (hc) hc[t * hc_stride + n] = h[n];\n            h[n] = ab * h[n] + bb * uv;"),
    ("row_ignores_batch", "const int64_t r = b * L + t;", "const int64_t r = t;"),
    ("h0_transposed", "a->h0[(b * D + d) * N + n]", "a->h0[(d * a->B + b) * N + n]"),
    ("step_window_reversed", "acc += (double)w_conv[d * K + k] * win[S - k];",
     "acc += (double)w_conv[d * K + k] * win[k - 1];"),
    ("step_state_not_shifted", "(j + 1 < S) ? win[j + 1] : xv", "(j + 1 < S) ? win[j] : xv"),
    ("step_dt_ignored_in_input", "const double bb = b_bar(disc, dv, A, (double)Bm[b * N + n]);",
     "const double bb = b_bar(disc, 1.0, A, (double)Bm[b * N + n]);"),
    # backward of the scan and the gate
    ("bwd_dab_uses_current_state", "const double dab = dh * hprev;", "const double dab = dh * hcur;"),
    ("bwd_carry_not_decayed", "g[n] = dh * ab;", "g[n] = dh;"),
    ("bwd_dC_uses_previous_state", "dC_col[t * N + n] = dY * hcur;",
     "dC_col[t * N + n] = dY * hprev;"),
    ("bwd_zoh_ddv_input_term_dropped", "ddv += dab * A[n] * ab + dbb * ab * Bv;",
     "ddv += dab * A[n] * ab;"),
    ("bwd_euler_ddv_input_term_decayed", "ddv += dab * A[n] * ab + dbb * Bv;",
     "ddv += dab * A[n] * ab + dbb * ab * Bv;"),
    ("bwd_zoh_dA_input_term_dropped",
     "dA[n] += dab * dv * ab + dbb * Bv * dv * dv * phi_zoh(x);", "dA[n] += dab * dv * ab;"),
    ("bwd_phi_series_coefficient", "term += (double)(k - 1) / fact * xp;",
     "term += (double)k / fact * xp;"),
    ("bwd_zoh_dB_missing_div_a", "dB_col[t * N + n] = dbb * expm1(x) / A[n];",
     "dB_col[t * N + n] = dbb * expm1(x);"),
    ("bwd_euler_dB_missing_dv", "dB_col[t * N + n] = dbb * dv;", "dB_col[t * N + n] = dbb;"),
    ("bwd_gate_grad_is_sigmoid", "dz[r * D + d] = go * ys[t] * silu_grad(zv);",
     "dz[r * D + d] = go * ys[t] * sigmoid(zv);"),
    ("bwd_dY_ungated", "dY = go * silu(zv);", "dY = go;"),
    ("bwd_skip_missing_in_du", "double duv = dY * Dd;", "double duv = 0.0;"),
    ("bwd_dD_uses_dout", "dDsum += dY * uv;", "dDsum += go * uv;"),
    ("bwd_softplus_grad_dropped", "ddelta[r * D + d] = ddv * sigmoid(dl);",
     "ddelta[r * D + d] = ddv;"),
    ("bwd_clamp_grad_not_zeroed", "(al <= A_LOG_LO || al >= A_LOG_HI) ? 0.0 : dA[n] * A[n]",
     "dA[n] * A[n]"),
    ("bwd_dAlog_missing_chain", ": dA[n] * A[n];", ": dA[n];"),
    ("bwd_h0_not_used", "hs[n] = a->h0 ? (double)a->h0[(b * D + d) * N + n] : 0.0;",
     "hs[n] = 0.0;"),
    # backward of conv1d + SiLU
    ("cbwd_silu_grad_is_sigmoid", "silu_grad(conv_at(x, w, bias, L, D, K, b, t, d))",
     "sigmoid(conv_at(x, w, bias, L, D, K, b, t, d))"),
    ("cbwd_dx_taps_reversed", "dx[(r - k) * D + d] += dc * (double)w[d * K + k];",
     "dx[(r - k) * D + d] += dc * (double)w[d * K + (K - 1 - k)];"),
    ("cbwd_dw_not_shifted", "sw[k] += dc * (double)x[(r - k) * D + d];",
     "sw[k] += dc * (double)x[r * D + d];"),
    ("cbwd_bias_grad_dropped", "db[d] = sb;", "db[d] = 0.0;"),
    # Mamba-2 SSD scan
    ("ssd_group_of_head", "g = h / hpg;", "g = h % G;"),
    ("ssd_dt_bias_dropped", "const double bias = dt_bias ? (double)dt_bias[h] : 0.0;",
     "const double bias = 0.0;"),
    ("ssd_input_without_factor", "*s = a * *s + f * xv * (double)Bm[r * GN + g * N + n];",
     "*s = a * *s + xv * (double)Bm[r * GN + g * N + n];"),
    ("ssd_factor_ignores_disc", "const double f = b_bar(disc, dv, A, 1.0);",
     "const double f = dv;"),
    ("ssd_decay_without_dv", "const double a = exp(dv * A);", "const double a = exp(A);"),
    ("ssd_output_uses_B", "acc += (double)Cm[r * GN + g * N + n] * *s;",
     "acc += (double)Bm[r * GN + g * N + n] * *s;"),
    ("ssd_skip_dropped", "double acc = Dh * xv;", "double acc = 0.0;"),
    ("ssd_h0_ignored", "S[i] = h0 ? (double)h0[bh * P * N + i] : 0.0;", "S[i] = 0.0;"),
    ("ssd_output_before_update",
     "*s = a * *s + f * xv * (double)Bm[r * GN + g * N + n];\n                        acc += (double)Cm[r * GN + g * N + n] * *s;",
     "acc += (double)Cm[r * GN + g * N + n] * *s;\n                        *s = a * *s + f * xv * (double)Bm[r * GN + g * N + n];"),
]


@pytest.fixture(scope="module")
def src():
    with open(os.path.join(os.path.dirname(oracle.__file__), "oracle.c")) as f:
        return f.read()


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(tmp_path, src, name, old, new):
    # A text that occurs more than once (e.g. the row index in the forward and
    # the backward column loops) is mutated everywhere: the same slip made
    # consistently.
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    path = tmp_path / "oracle_mut.c"
    path.write_text(src.replace(old, new))
    lib = oracle.load(oracle.build(str(path), str(tmp_path / "liboracle_mut.so")))
    orc = oracle.Bound(lib)
    caught = []
    for pin in ALL_PINS:
        try:
            pin(orc)
        except (AssertionError, ValueError, FloatingPointError) as e:  # noqa: PERF203
            caught.append(pin.__name__)
    assert caught, f"no pin caught mutant {name}"
