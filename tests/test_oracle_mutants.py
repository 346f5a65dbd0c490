"""Plant plausible mistakes in copies of the oracle (on the CPU) and check that the pins catch each.

Every mutant is a text edit of ``oracle/attn_oracle.c`` compiled into a
temporary library; the real oracle is never touched.  A mutant that passes every
pin would mean the pins cannot see that kind of slip.
"""
import os
import subprocess

import pytest

from oracle import attn_oracle
from tests import oracle_pins

MUTANTS = {
    "mask_strict": ("return !causal || j <= i;", "return !causal || j < i;"),
    "mask_reversed": ("return !causal || j <= i;", "return !causal || j >= i;"),
    "scale_dropped": ("p[j] = J->scale * acc;", "p[j] = acc;"),
    "lse_no_max": ("if (lse_out) lse_out[r] = m + log(l);", "if (lse_out) lse_out[r] = log(l);"),
    "lse_log2": ("if (lse_out) lse_out[r] = m + log(l);", "if (lse_out) lse_out[r] = m + log2(l);"),
    "norm_wrong": ("if (visible(J->causal, i, j)) p[j] /= l;", "if (visible(J->causal, i, j)) p[j] /= (l + 1.0);"),
    "v_rows_reversed": ("out[t] += p[j] * V[(int64_t)j * d + t];", "out[t] += p[j] * V[(int64_t)(Sk - 1 - j) * d + t];"),
    "k_feature_reversed": ("acc += Q[(int64_t)i * d + t] * K[(int64_t)j * d + t];",
                           "acc += Q[(int64_t)i * d + t] * K[(int64_t)j * d + (d - 1 - t)];"),
    "q_index_dropped": ("acc += Q[(int64_t)i * d + t] * K[(int64_t)j * d + t];",
                        "acc += Q[(int64_t)i * d] * K[(int64_t)j * d + t];"),
    "max_wrong_sign": ("if (visible(J->causal, i, j) && p[j] > m) m = p[j];",
                       "if (visible(J->causal, i, j) && -p[j] > m) m = -p[j];"),
    "online_alpha_inverted": ("exp(m - mnew);", "exp(mnew - m);"),
    "online_l_not_rescaled": ("        l *= alpha;\n", "\n"),
    "online_acc_not_rescaled": ("for (int t = 0; t < d; ++t) acc[t] *= alpha;", ""),
    "online_causal_count": ("return (i + 1 < J->Sk) ? i + 1 : J->Sk;", "return (i < J->Sk) ? i : J->Sk;"),
    "e4m3_bias": ("else mag = ldexp(1.0 + (double)m / 8.0, e - 7);", "else mag = ldexp(1.0 + (double)m / 8.0, e - 8);"),
    "e4m3_subnormal": ("if (e == 0) mag = ldexp((double)m / 8.0, -6);", "if (e == 0) mag = ldexp((double)m / 8.0, -7);"),
    "e4m3_sign": ("return s ? -mag : mag;", "return mag;"),
    "descale_block_index": ("descale[bh * nblk + r / blk]", "descale[bh * nblk + (r + 1) / blk]"),
    "e4m3_ties_to_odd": ("(err == best_err && (c & 1) == 0)", "(err == best_err && (c & 1) == 1)"),
    "e4m3_scan_short": ("const int top = fmt ? 0x7b : 0x7e;", "const int top = fmt ? 0x7b : 0x77;"),
    "e4m3_sign_dropped": ("return (uint8_t)(best | (signbit(x) ? 0x80 : 0));", "return (uint8_t)best;"),
    "quant_descale_240": ("const float fmax = fmt ? 57344.0f : 448.0f;", "const float fmax = fmt ? 57344.0f : 240.0f;"),
    "quant_block_short": ("const int r0 = j * blk, r1 = (r0 + blk < S) ? r0 + blk : S;",
                          "const int r0 = j * blk, r1 = (r0 + blk < S) ? r0 + blk - 1 : S;"),
    "e5m2_bias": ("else mag = ldexp(1.0 + (double)m / 4.0, e - 15);", "else mag = ldexp(1.0 + (double)m / 4.0, e - 16);"),
    "e5m2_subnormal": ("if (e == 0) mag = ldexp((double)m / 4.0, -14);", "if (e == 0) mag = ldexp((double)m / 4.0, -15);"),
    "e5m2_top_code": ("const int top = fmt ? 0x7b : 0x7e;", "const int top = fmt ? 0x7a : 0x7e;"),
    "e5m2_fmax": ("const float fmax = fmt ? 57344.0f : 448.0f;", "const float fmax = fmt ? 49152.0f : 448.0f;"),
    "rms_eps_outside": ("const double r = 1.0 / sqrt(eps + ms);", "const double r = 1.0 / sqrt(ms) + eps;"),
    "rms_sum_not_mean": ("const double ms = ss / ((double)H * d);", "const double ms = ss / (double)d;"),
    "rms_weight_index": ("* r * w[h * d + t];", "* r * w[t];"),
    "rms_per_head": ("            double ss = 0.0;\n            for (int h = 0; h < H; ++h)",
                     "            double ss = 0.0;\n            for (int h = 0; h < 1; ++h)"),
    "rms_no_inverse": ("const double r = 1.0 / sqrt(eps + ms);", "const double r = sqrt(eps + ms);"),
    "quant_amax_signed": ("const float v = fabsf(x[(bh * S + r) * (int64_t)d + t]);",
                          "const float v = x[(bh * S + r) * (int64_t)d + t];"),
}


def _caught(lib_path):
    o = attn_oracle.Oracle(lib_path)
    failed = []
    for check in oracle_pins.ALL_CHECKS:
        try:
            check(o)
        except (AssertionError, ValueError, IndexError):
            failed.append(check.__name__)
    return failed


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(attn_oracle.SRC).read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    mut = src.replace(old, new)
    path = os.path.join(tmp_path, f"attn_oracle_{name}.c")
    with open(path, "w") as f:
        f.write(mut)
    lib = os.path.join(tmp_path, f"liboracle_{name}.so")
    attn_oracle.build(path, lib)
    failed = _caught(lib)
    assert failed, f"mutant {name} passed every pin"
