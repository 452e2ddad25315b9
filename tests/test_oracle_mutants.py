"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check that
the pins catch every one of them: a dropped term, a wrong sign, a wrong index,
a transposed operand, a wrong readout order, a broken storage-type widening.

Each mutant is a textual edit of oracle/ssm_oracle.c compiled into a temporary
directory; the real oracle is never touched.
"""
import os

import pytest

import oracle
import pins

MUTANTS = {
    "decay_sign": ("const double abar = exp(dt * a_dn);\n            const double bu",
                   "const double abar = exp(-dt * a_dn);\n            const double bu"),
    "drop_delta_in_input": ("return delta * b_tn * u;", "return b_tn * u;"),
    "zoh_missing_delta": ("expm1(delta * a_dn) / a_dn", "expm1(delta * a_dn) / (delta * a_dn)"),
    "zoh_limit_wrong": (": delta;\n        return coef", ": 1.0;\n        return coef"),
    "a_transposed": ("const double a_dn = A[d * N + n];\n            const double abar",
                     "const double a_dn = A[n * dim + d];\n            const double abar"),
    "b_ignores_time": ("const double bu = input_term(disc, dt, a_dn, load(B, type, row * N + n), ut);",
                       "const double bu = input_term(disc, dt, a_dn, load(B, type, b * L * N + n), ut);"),
    "c_from_b": ("yt += load(C, type, row * N + n) * h[n];", "yt += load(B, type, row * N + n) * h[n];"),
    "readout_before_update": (
        "            h[n] = abar * h[n] + bu;\n            yt += load(C, type, row * N + n) * h[n];",
        "            yt += load(C, type, row * N + n) * h[n];\n            h[n] = abar * h[n] + bu;"),
    "drop_skip": ("yt += dskip * ut;", "yt += 0.0 * ut;"),
    "skip_wrong_channel": ("h[n] = h0 ? h0[(b * dim + d) * N + n] : 0.0;\n    const double dskip = D ? D[d] : 0.0;",
                           "h[n] = h0 ? h0[(b * dim + d) * N + n] : 0.0;\n    const double dskip = D ? D[0] : 0.0;"),
    "gate_sign": ("return z / (1.0 + exp(-z));", "return z / (1.0 + exp(z));"),
    "gate_is_sigmoid": ("return z / (1.0 + exp(-z));", "return 1.0 / (1.0 + exp(-z));"),
    "h0_transposed": ("h[n] = h0 ? h0[(b * dim + d) * N + n] : 0.0;",
                      "h[n] = h0 ? h0[(b * N + n) * dim + d] : 0.0;"),
    "state_not_decayed": ("h[n] = abar * h[n] + bu;", "h[n] = h[n] + bu;"),
    "bf16_shift": ("<< 16;", "<< 15;"),
    "f32_truncated": ("return (double)((const float *)p)[i];", "return (double)(float)(int)((const float *)p)[i];"),
    "decode_b_row": ("load(B, type, b * N + n), xt);", "load(B, type, n), xt);"),
    "decode_c_row": ("yt += load(C, type, b * N + n) * hc[n];", "yt += load(C, type, n) * hc[n];"),
    "decode_no_skip": ("yt += (D ? D[d] : 0.0) * xt;", "yt += 0.0 * xt;"),
    "decode_no_gate": ("            yt *= silu(load(z, type, c));", "            yt *= 1.0;"),
    "last_state_not_written": ("hl[n] = h[n];", "hl[n] = 0.0 * h[n];"),
    # backward
    "bwd_no_decay_path": ("ddt += da * abar * a_dn;", "ddt += 0.0 * da * abar * a_dn;"),
    "bwd_dA_missing_delta": ("dA_c[n] += da * abar * dt;", "dA_c[n] += da * abar;"),
    "bwd_adjoint_not_decayed": ("lam[n] = abar * l;", "lam[n] = l;"),
    "bwd_dC_uses_prev_state": ("dC[row * N + n] += ds * hs[(t + 1) * N + n];", "dC[row * N + n] += ds * hs[t * N + n];"),
    "bwd_dB_missing_delta": ("dB[row * N + n] += l * dt * ut;", "dB[row * N + n] += l * ut;"),
    "bwd_du_missing_delta": ("dut += l * dt * Bt;", "dut += l * Bt;"),
    "bwd_silu_grad": ("return sg * (1.0 + z * (1.0 - sg));", "return sg;"),
    "bwd_gate_not_applied": ("ds = dyt * silu(zt);", "ds = dyt;"),
    "bwd_zoh_dfdA_sign": ("(dt * abar - f) / a_dn", "(f - dt * abar) / a_dn"),
    "bwd_zoh_dfdA_limit": (": 0.5 * dt * dt;", ": dt * dt;"),
    "bwd_zoh_ddelta": ("ddt += l * abar * Bt * ut;", "ddt += l * Bt * ut;"),
    "bwd_zoh_dB": ("dB[row * N + n] += l * f * ut;", "dB[row * N + n] += l * dt * ut;"),
    "bwd_skip_grad": ("double dut = dskip * ds;", "double dut = dskip * dyt;"),
    "bwd_dD_ungated": ("dDacc += ds * ut;", "dDacc += dyt * ut;"),
    "bwd_dh_last_ignored": ("lam[n] = dh_last ? dh_last[(b * dim + d) * N + n] : 0.0;", "lam[n] = 0.0;"),
    "bwd_hprev_is_current": ("const double hprev = hs[t * N + n];", "const double hprev = hs[(t + 1) * N + n];"),
    "bwd_readout_adjoint_missing": ("const double l = lam[n] + Ct * ds;", "const double l = lam[n];"),
    # step size: bias and softplus
    "softplus_positive_branch": ("return x > 0.0 ? x + log1p(exp(-x)) : log1p(exp(x));",
                                 "return x > 0.0 ? x : log1p(exp(x));"),
    "delta_bias_ignored": ("double x = load(delta, type, i) + (bias ? bias[d] : 0.0);",
                           "double x = load(delta, type, i);"),
    "softplus_grad_missing": ("        ddt *= dstep;", "        ddt *= 1.0;"),
    "softplus_grad_sign": ("*dgrad = 1.0 / (1.0 + exp(-x));", "*dgrad = 1.0 / (1.0 + exp(x));"),
    # convolution prologue
    "conv_tap_shift": ("const int64_t s = t - (W - 1) + k;\n        if (s >= 0)",
                       "const int64_t s = t - W + k;\n        if (s >= 0)"),
    "conv_no_silu": ("    return acc / (1.0 + exp(-acc));", "    return acc;"),
    "conv_taps_reversed": ("acc += cw[d * W + k] * load(x, type, (b * L + s) * dim + d);",
                           "acc += cw[d * W + (W - 1 - k)] * load(x, type, (b * L + s) * dim + d);"),
    "conv_grad_no_silu_grad": ("const double dp = gu[t] * sg * (1.0 + p * (1.0 - sg));", "const double dp = gu[t];"),
    "conv_dx_wrong_tap": ("du[s] += cw[d * W + k] * dp;", "du[s] += cw[d * W] * dp;"),
    "conv_dw_uses_output_time": ("dcw_c[k] += dp * load(u, type, (b * L + s) * dim + d);",
                                 "dcw_c[k] += dp * load(u, type, (b * L + t) * dim + d);"),
    # Mamba-2 SSD layer
    "ssd_group_index": ("const int64_t g = hh / (H / G);", "const int64_t g = hh % G;"),
    "ssd_decay_sign": ("const double abar = exp(step * a);", "const double abar = exp(-step * a);"),
    "ssd_hold_coefficient": ("? expm1(step * a) / a : step;", "? expm1(step * a) : step;"),
    "ssd_input_missing_step": ("*s = abar * *s + wbar * xv * load(B, type, bc + n);",
                               "*s = abar * *s + xv * load(B, type, bc + n);"),
    "ssd_b_c_swapped": ("yt += load(C, type, bc + n) * *s;", "yt += load(B, type, bc + n) * *s;"),
    "ssd_skip_wrong_head": ("yt += (D ? D[hh] : 0.0) * xv;", "yt += (D ? D[0] : 0.0) * xv;"),
    "ssd_gate_wrong_index": ("yt *= silu(load(z, type, (row * H + hh) * P + p));",
                             "yt *= silu(load(z, type, (row * H + hh) * P));"),
    "ssd_h0_transposed": ("st[i] = h0 ? h0[(b * H + hh) * P * N + i] : 0.0;",
                          "st[i] = h0 ? h0[(b * H + hh) * P * N + (i % N) * P + i / N] : 0.0;"),
    "ssd_dt_wrong_head": ("step_size(dt, type, row * H + hh, hh, dt_bias, sp, NULL);",
                          "step_size(dt, type, row * H, hh, dt_bias, sp, NULL);"),
    "ssd_x_wrong_stride": ("const double xv = load(x, type, (row * H + hh) * P + p);",
                           "const double xv = load(x, type, (row * P + p) * H + hh);"),
}


def _source():
    with open(oracle.SOURCE) as f:
        return f.read()


def test_mutations_apply_once():
    src = _source()
    for name, (old, new) in MUTANTS.items():
        assert src.count(old) == 1, name


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = _source().replace(old, new)
    c_path = os.path.join(tmp_path, "mutant.c")
    with open(c_path, "w") as f:
        f.write(src)
    lib = oracle.build(source=c_path, output=os.path.join(tmp_path, "libmutant.so"), strict=False)
    o = oracle.Oracle(lib, threads=1)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(o)
        except (AssertionError, ValueError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, "mutant %s survived every pin" % name
