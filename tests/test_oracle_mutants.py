"""The pins are strong enough: every planted mistake in the oracle fails one.

Each mutant is a copy of ``oracle/moe_oracle.c`` with one plausible mistake
(a dropped term, a wrong sign, index or operand), compiled with gcc into a
temporary directory.  The test passes when at least one pin rejects it.
CPU only; the real oracle source is never modified.
"""
import json
import os
import subprocess
import sys

import pytest

import oracle
from oracle import build as obuild

SRC = obuild.SRC

MUTANTS = {
    "f_over_T_not_Tk": ("double fe = (double)cnt[e] / total;",
                        "double fe = (double)cnt[e] / (double)Tm;"),
    "P_missing_normaliser": ("psum[e] += exp(row[e] - m) / s;",
                             "psum[e] += exp(row[e] - m);"),
    "P_masked_to_picks": ("psum[e] += exp(row[e] - m) / s;",
                          "psum[e] += 0.0;"),
    "tie_to_higher_index": ("if (best < 0 || row[e] > row[best])",
                            "if (best < 0 || row[e] >= row[best])"),
    "aux_missing_alpha": ("aux[mb] = alpha * (double)E * dot;",
                          "aux[mb] = (double)E * dot;"),
    "aux_missing_N": ("aux[mb] = alpha * (double)E * dot;",
                      "aux[mb] = alpha * dot;"),
    "capacity_ignores_k": ("long long per_expert = (Tm * k + E - 1) / E;",
                           "long long per_expert = (Tm + E - 1) / E;"),
    "capacity_floor": ("long long per_expert = (Tm * k + E - 1) / E;",
                       "long long per_expert = (Tm * k) / E + (Tm * k) % 2;"),
    "capacity_double_product": ("cap = (num + den - 1) / den;",
                                "cap = (unsigned __int128)ceil(strtod(cf_text, NULL) * (double)per_expert);"),
    "capacity_fp32_factor": ("cap = (num + den - 1) / den;",
                             "cap = (unsigned __int128)ceil((double)strtof(cf_text, NULL) * (double)per_expert);"),
    "capacity_product_truncated": ("cap = (num + den - 1) / den;", "cap = num / den;"),
    "drop_off_by_one": ("dropped[a] = (uint8_t)(capacity >= 0 && r >= capacity);",
                        "dropped[a] = (uint8_t)(capacity >= 0 && r > capacity);"),
    "perm_reversed_in_expert": ("long long pos = off[e] + r;",
                                "long long pos = off[e + 1] - 1 - r;"),
    "offsets_inclusive": ("off[e + 1] = off[e] + cnt[e];",
                          "off[e + 1] = off[e] + cnt[e] + (e == 0);"),
    "cv_sample_std": ("var /= (double)E;", "var /= (double)(E - 1);"),
    "renorm_ignored": ("topk_w[t * k + j] = renorm ? p / picked : p;",
                       "topk_w[t * k + j] = p;"),
    "grad_sign": ("dlogits[t * E + j] = p[j] * (G[j] - gp);",
                  "dlogits[t * E + j] = p[j] * (gp - G[j]);"),
    "grad_missing_p": ("dlogits[t * E + j] = p[j] * (G[j] - gp);",
                       "dlogits[t * E + j] = (G[j] - gp);"),
    "grad_missing_E": ("G[i] = p_masked ? 0.0 : g * alpha * (double)E * ((double)cnt[i] / total) / (double)Tm;",
                       "G[i] = p_masked ? 0.0 : g * alpha * ((double)cnt[i] / total) / (double)Tm;"),
    "grad_masked_over_Tm": ("G[i] += g * alpha * (double)E * ((double)cnt[i] / total) / total;",
                            "G[i] += g * alpha * (double)E * ((double)cnt[i] / total) / (double)Tm;"),
    "grad_renorm_no_cross_term": ("G[i] -= d_topk_w[t * k + j2] * p[topk_idx[t * k + j2]] / (z * z);",
                                  "G[i] -= 0.0 * z;"),
    "grad_weight_term_ignored": ("G[i] += d_topk_w[t * k + j]; /* w_j = p_i */",
                                 "G[i] += 0.0; /* w_j = p_i */"),
    "masked_P_over_Tm": ("double pe = psum[e] / (p_masked ? total : (double)Tm);",
                         "double pe = psum[e] / (double)Tm;"),
    "masked_P_all_tokens": ("            if (!p_masked)\n                for (long long e = 0; e < E; ++e)",
                            "            if (1)\n                for (long long e = 0; e < E; ++e)"),
    "gate_transposed_Wg": ("acc += bf16_to_double(X[t * d + i]) * bf16_to_double(Wg[i * E + e]);",
                           "acc += bf16_to_double(X[t * d + i]) * bf16_to_double(Wg[(e * d + i) % (d * E)]);"),
    "entropy_log2": ("ent -= fe * log(fe);", "ent -= fe * log2(fe);"),
    "balance_degree_sign": ("x[1] = 1.0 - (cmax - mean) / mean;",
                            "x[1] = 1.0 + (cmax - mean) / mean;"),
    "gate_dX_transposed_Wg": ("acc += dlogits[t * E + e] * bf16_to_double(Wg[i * E + e]);",
                              "acc += dlogits[t * E + e] * bf16_to_double(Wg[(e * d + i) % (d * E)]);"),
    "gate_dWg_wrong_row": ("acc += bf16_to_double(X[t * d + i]) * dlogits[t * E + e];",
                           "acc += bf16_to_double(X[t * d + (i + 1) % d]) * dlogits[t * E + e];"),
    "eplb_replicate_by_weight": ("if ((long long)weight[e] * logcnt[best] > (long long)weight[best] * logcnt[e])",
                                 "if ((long long)weight[e] > (long long)weight[best])"),
    "eplb_sort_ascending": ("if (l != r) return l > r ? -1 : 1;", "if (l != r) return l > r ? 1 : -1;"),
    "eplb_heaviest_pack": ("if (cnt[b] < cap && (best < 0 || pack_load[b] < pack_load[best]))",
                           "if (cnt[b] < cap && (best < 0 || pack_load[b] > pack_load[best]))"),
    "eplb_ignores_full": ("if (cnt[b] < cap && (best < 0 || pack_load[b] < pack_load[best]))",
                          "if ((best < 0 || pack_load[b] < pack_load[best]))"),
    "eplb_pack_tie_higher": ("if (cnt[b] < cap && (best < 0 || pack_load[b] < pack_load[best]))",
                             "if (cnt[b] < cap && (best < 0 || pack_load[b] <= pack_load[best]))"),
    "eplb_item_weight_not_per_replica": ("it[i].den = logcnt[phy2log[i]];", "it[i].den = 1;"),
    "sinkhorn_kernel_sign": ("K[i] = exp(-C[i] / eps);", "K[i] = exp(C[i] / eps);"),
    "sinkhorn_u_uses_column": ("s += K[i * R + j] * v[j];", "s += K[j * R + i] * v[j];"),
    "sinkhorn_v_from_old_u": ("u[i] = a[i] / (s > tiny ? s : tiny);", "u[i] = (it == 0) ? a[i] / (s > tiny ? s : tiny) : u[i];"),
    "bias_ignored": ("topk_row(selrow, E, k, idx, taken);",
                     "topk_row(row, E, k, idx, taken);"),
    "bias_added_in_double": ("selrow[e] = (double)biased;",
                             "selrow[e] = row[e] + (double)select_bias[e]; (void)biased;"),
    "bias_update_sign": ("bias[e] = bias[e] - gamma;", "bias[e] = bias[e] + gamma;"),
    "bias_update_first_mb_only": ("for (long long mb = 0; mb < n_micro; ++mb)\n            load += counts[mb * E + e];",
                                  "load += counts[e] * n_micro;"),
}


_RUNNER = r"""
import json, sys
sys.path[:0] = [sys.argv[1], sys.argv[2]]
import oracle
lib = oracle.load_library(sys.argv[3])
failed = []
for pin in ALL_PINS:
    try:
        pin(lib)
    except AssertionError:
        failed.append(pin.__name__)
print(json.dumps(failed))
"""


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    with open(SRC) as fh:
        src = fh.read()
    assert src.count(old) == 1, f"mutation site for {name} not unique/found"
    csrc = os.path.join(tmp_path, "mutant.c")
    with open(csrc, "w") as fh:
        fh.write(src.replace(old, new))
    so = obuild.build(src=csrc, out=os.path.join(tmp_path, "libmutant.so"))
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    tests = os.path.join(root, "tests")
    # A subprocess, so that a mutant that writes out of bounds and crashes
    # counts as caught instead of taking the test runner down.
    r = subprocess.run([sys.executable, "-c", _RUNNER, root, tests, so],
                       capture_output=True, text=True, timeout=600)
    if r.returncode != 0:
        return  # crashed or raised: the mutant is caught
    failed = json.loads(r.stdout.strip().splitlines()[-1])
    assert failed, f"no pin rejects mutant {name}"
