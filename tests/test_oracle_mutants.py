"""Each plausible slip, planted in a copy of the oracle's C source, must fail
at least one pin.  The copy is compiled and exercised in a subprocess, so a
mutant that crashes cannot take the test run down with it."""
import json
import os
import subprocess
import sys

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))

# name -> list of (exact text in attn_oracle.c, replacement)
MUTANTS = {
    "scale_dropped": [("srow[j] = scale * dot;", "srow[j] = dot;")],
    "causal_mask_dropped": [("if (!causal) return Tk - 1;", "if (causal >= 0) return Tk - 1;")],
    "mask_off_by_one": [("long lim = q_offset + i;", "long lim = q_offset + i + 1;")],
    "mask_top_left_aligned": [("long lim = q_offset + i;", "long lim = i;")],
    "masked_scores_zero_filled": [(
        "        srow[j] = scale * dot;\n    }\n",
        "        srow[j] = scale * dot;\n    }\n"
        "    for (long j = lim + 1; j < Tk; ++j) srow[j] = 0.0;\n    lim = Tk - 1;\n")],
    "gqa_heads_tiled": [("return hq / (Hq / Hkv);", "return hq % Hkv;")],
    "softmax_not_normalised": [("for (long c = 0; c < dv; ++c) oi[c] /= l;",
                                "for (long c = 0; c < dv; ++c) oi[c] /= 1.0;")],
    "value_row_index_wrong": [("oi[c] += srow[j] * vj[c];", "oi[c] += srow[j] * vh[c];")],
    "value_rows_strided_by_key_width": [("const double* vj = vh + j * dv;", "const double* vj = vh + j * dk;")],
    "key_channels_reversed": [("dot += qi[c] * kj[c];", "dot += qi[c] * kj[dk - 1 - c];")],
    "lse_without_max": [("*lse_i = m + log(l);", "*lse_i = log(l);")],
    "bwd_dv_uses_unnormalised_weights": [("for (long j = 0; j <= lim; ++j) alpha[j] /= l;", "")],
    "bwd_softmax_jacobian_term_dropped": [("const double ds = alpha[j] * (g[j] - ag);",
                                           "const double ds = alpha[j] * g[j];")],
    "bwd_dk_missing_scale": [("dkh[j * d + c] += scale * ds * qi[c];", "dkh[j * d + c] += ds * qi[c];")],
    "bwd_dq_uses_query_not_key": [("dqi[c] += scale * ds * kj[c];", "dqi[c] += scale * ds * qi[c];")],
    "bwd_dv_uses_values": [("dvh[j * d + c] += alpha[j] * gi[c];", "dvh[j * d + c] += alpha[j] * vj[c];")],
    "rope_sign_flipped": [("xr[a] = x1 * cs - x2 * sn;", "xr[a] = x1 * cs + x2 * sn;")],
    "rope_frequency_halved_exponent": [("pow(base, -2.0 * (double)p / (double)d)",
                                        "pow(base, -1.0 * (double)p / (double)d)")],
    "rope_frequency_index_shifted": [("pow(base, -2.0 * (double)p / (double)d)",
                                      "pow(base, -2.0 * (double)(p + 1) / (double)d)")],
    "rope_ignores_pos0": [("double pos = (double)(pos0 + t);", "double pos = (double)t;")],
    "rope_sin_cos_swapped": [("double cs = cos(theta), sn = sin(theta);",
                              "double cs = sin(theta), sn = cos(theta);")],
    "rope_table_cos_sin_swapped": [("out[(t * half + p) * 2 + 0] = (float)cos(theta);",
                                    "out[(t * half + p) * 2 + 0] = (float)sin(theta);"),
                                   ("out[(t * half + p) * 2 + 1] = (float)sin(theta);",
                                    "out[(t * half + p) * 2 + 1] = (float)cos(theta);")],
    "rope_table_frequency_index_shifted": [("pow(base, -(2.0 * (double)p) / (double)d)",
                                            "pow(base, -(2.0 * (double)(p + 1)) / (double)d)")],
    "rope_table_ignores_pos0": [("const double position = (double)(pos0 + t);",
                                 "const double position = (double)t;")],
    "rope_split_half_uses_adjacent_pairs": [
        ("long a = pairing == 0 ? p : 2 * p;", "long a = 2 * p;"),
        ("long b2 = pairing == 0 ? p + half : 2 * p + 1;", "long b2 = 2 * p + 1;")],
}


@pytest.fixture(scope="module")
def source():
    with open(oracle.SOURCE) as f:
        return f.read()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, source, tmp_path):
    text = source
    for old, new in MUTANTS[name]:
        assert text.count(old) == 1, f"mutation site not found once: {old!r}"
        text = text.replace(old, new)
    src = tmp_path / "mutant.c"
    src.write_text(text)
    lib = oracle.compile_library(str(src), str(tmp_path / "libmutant.so"))
    res = subprocess.run([sys.executable, os.path.join(HERE, "oracle_pins.py"), lib],
                         capture_output=True, text=True, timeout=300)
    if res.returncode != 0:
        return  # the mutant crashed the pin run: caught
    results = json.loads(res.stdout.strip().splitlines()[-1])
    failed = [k for k, v in results.items() if v != "ok"]
    assert failed, f"mutant {name} passed every pin"
