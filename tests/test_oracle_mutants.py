"""The pins must catch plausible mistakes in the oracle.

Each case below plants one mistake in a copy of oracle/kda_oracle.c (a
dropped term, a wrong sign, a wrong operand, a wrong order), builds it with
gcc into a temporary directory, and checks that at least one pin from
tests/oracle_pins.py rejects it. The real oracle is never modified.
"""
import os

import pytest

from oracle.build import build
from oracle.kda_oracle import Oracle
from tests.oracle_pins import ALL_PINS

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "kda_oracle.c")

MUTANTS = {
    "no_decay": [("Sbh[(long)i * dv + j] *= a;", "Sbh[(long)i * dv + j] *= 1.0 + 0.0 * a;")],
    "decay_sign": [("const double a = exp(gt[i]);", "const double a = exp(-gt[i]);")],
    "decay_after_read": [
        ("Sbh[(long)i * dv + j] *= a;", "(void)a;"),
        ("Sbh[(long)i * dv + j] += bt * kh[i] * (vh[j] - r[j]);",
         "Sbh[(long)i * dv + j] = exp(gt[i]) * Sbh[(long)i * dv + j]"
         " + bt * kh[i] * (vh[j] - r[j]);"),
    ],
    "delta_sign": [("(vh[j] - r[j]);", "(vh[j] + r[j]);")],
    "no_beta": [("+= bt * kh[i] * (vh[j] - r[j]);", "+= kh[i] * (vh[j] - r[j]);")],
    "read_with_q": [("r[j] += Sbh[(long)i * dv + j] * kh[i];",
                     "r[j] += Sbh[(long)i * dv + j] * qh[i];")],
    "write_along_q": [("+= bt * kh[i] * (vh[j] - r[j]);", "+= bt * qh[i] * (vh[j] - r[j]);")],
    "readout_before_write": [
        ("acc += Sbh[(long)i * dv + j] * qh[i];",
         "acc += (Sbh[(long)i * dv + j] - bt * kh[i] * (vh[j] - r[j])) * qh[i];")],
    "readout_with_k": [("acc += Sbh[(long)i * dv + j] * qh[i];",
                        "acc += Sbh[(long)i * dv + j] * kh[i];")],
    "no_q_norm": [("l2_normalise(qh, dk, eps);", "(void)0;")],
    "no_k_norm": [("l2_normalise(kh, dk, eps);", "(void)0;")],
    "no_silu": [("return y / (1.0 + exp(-y));", "return y;")],
    "conv_taps_reversed": [
        ("double y = w[0] * raw_at(x, x_stride_t, t, 3,", "double y = w[3] * raw_at(x, x_stride_t, t, 3,"),
        ("w[3] * raw_at(x, x_stride_t, t, 0,", "w[0] * raw_at(x, x_stride_t, t, 0,"),
    ],
    "ring_history_reversed": [("return ring_b[(long)(3 + s) * Ctot + c];",
                               "return ring_b[(long)(-1 - s) * Ctot + c];")],
    "ring_not_saved": [("ring_update(T, H, dk, dv, b, h, q, k, v, ring);\n    free", "free")],
    # the output gate
    "rms_sum_not_mean": [("sqrt(ss / n + eps)", "sqrt(ss + eps)")],
    "rms_no_sqrt": [("sqrt(ss / n + eps)", "(ss / n + eps)")],
    "rms_eps_outside_sqrt": [("sqrt(ss / n + eps)", "(sqrt(ss / n) + eps)")],
    "gate_swish": [("yr[j] = xr[j] / rms * w[j] * gate;", "yr[j] = xr[j] / rms * w[j] * gate * zr[j];")],
    "gate_missing": [("yr[j] = xr[j] / rms * w[j] * gate;", "yr[j] = xr[j] / rms * w[j];")],
    "gate_sign": [("1.0 / (1.0 + exp(-zr[j]))", "1.0 / (1.0 + exp(zr[j]))")],
    "norm_weight_missing": [("yr[j] = xr[j] / rms * w[j] * gate;", "yr[j] = xr[j] / rms * gate;")],
    # gates from raw projections
    "decay_is_sigmoid": [("-log1p(exp(-a[i])) : a[i] - log1p(exp(a[i]))",
                          "1.0 / (1.0 + exp(-a[i])) : 1.0 / (1.0 + exp(-a[i]))")],
    "decay_branch_swapped": [("a[i] >= 0.0 ? -log1p", "a[i] < 0.0 ? -log1p")],
    "decay_sign_of_a": [("-log1p(exp(-a[i])) : a[i] - log1p(exp(a[i]))",
                         "-log1p(exp(a[i])) : -a[i] - log1p(exp(-a[i]))")],
    "beta_not_squashed": [("beta[i] = 1.0 / (1.0 + exp(-b[i]));", "beta[i] = b[i];")],
    # the gradient of the recurrence
    "bwd_no_decay_carry": [("G[(long)i * dv + j] = exp(gt[i]) * dsp;", "G[(long)i * dv + j] = dsp;")],
    "bwd_dk_misses_read": [("ak += G[(long)i * dv + j] * del[j] + Sp[(long)i * dv + j] * drj;",
                            "ak += G[(long)i * dv + j] * del[j];")],
    "bwd_dq_from_old_state": [("aq += St[(long)i * dv + j] * dot[j];",
                               "aq += Sp[(long)i * dv + j] * dot[j];")],
    "bwd_dbeta_without_read": [("db += dd[j] * (vt[j] - r[j]);", "db += dd[j] * vt[j];")],
    "bwd_readout_added_late": [("          G[(long)i * dv + j] += qt[i] * dot[j];\n", ""),
                               ("        dgt[i] = ag;\n", "        dgt[i] = ag;\n        (void)qt;\n")],
    # the gradient of the prologue
    "pbwd_no_norm_projection": [("dzt[i] = (dxh[(long)t * st + i] - silu(yt[i]) / nrm * dot) / nrm;",
                                 "dzt[i] = dxh[(long)t * st + i] / nrm;")],
    "pbwd_silu_slope_only_sigmoid": [("const double dy = dzt[i] * (sg + yt[i] * sg * (1.0 - sg));",
                                      "const double dy = dzt[i] * sg;")],
    "pbwd_conv_taps_reversed": [("dxe[(long)i * (T + 3) + t + j] += w[j] * dy;",
                                 "dxe[(long)i * (T + 3) + t + j] += w[3 - j] * dy;")],
    "pbwd_weight_grad_wrong_token": [("dw[j] += dy * xe[(long)i * (T + 3) + t + j];",
                                      "dw[j] += dy * xe[(long)i * (T + 3) + t + 3];")],
    "pbwd_ring_grad_dropped": [("dring[((long)b * 3 + s) * Ctot + c0 + i] = dxe[(long)i * (T + 3) + s];",
                                "dring[((long)b * 3 + s) * Ctot + c0 + i] = 0.0;")],
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    src = open(SRC).read()
    for old, new in MUTANTS[name]:
        assert src.count(old) == 1, f"mutation site not unique/absent: {old!r}"
        src = src.replace(old, new)
    path = tmp_path / f"{name}.c"
    path.write_text(src)
    lib = build(src=str(path), out=str(tmp_path / f"lib{name}.so"))
    orc = Oracle(lib)
    caught = []
    for pin in ALL_PINS:
        try:
            pin(orc)
        except Exception as e:  # any failure of a pin counts
            caught.append((pin.__name__, type(e).__name__))
            break
    assert caught, f"mutant {name} passed every pin"
