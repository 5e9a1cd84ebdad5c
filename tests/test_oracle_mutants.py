"""Plant plausible mistakes in copies of the oracle; some pin must catch each.

The mistakes are textual edits of ref_attn.c compiled to a temporary library
(the oracle's own source is untouched).  This shows the pins are strong
enough: a dropped term, a wrong sign or index, or a transposed operand makes
at least one pin fail.
"""
import os

import pytest

import oracle
from tests import oracle_pins as P

MUTANTS = {
    "drop_scale": ("S[i * N + j] = scale * acc + ref_bias(i, j, var);", "S[i * N + j] = acc + ref_bias(i, j, var);"),
    "alibi_sign": ("-var->slope * (double)(i > j ? i - j : j - i)", "var->slope * (double)(i > j ? i - j : j - i)"),
    "alibi_signed_distance": ("(double)(i > j ? i - j : j - i)", "(double)(i - j)"),
    "alibi_head_index": ("slopes[bh % H]", "slopes[0]"),
    "window_left_off_by_one": ("j < i - var->wl", "j <= i - var->wl"),
    "window_right_off_by_one": ("j > i + var->wr", "j >= i + var->wr"),
    "window_sides_swapped": ("v.wl = wl;\n    v.wr = wr;", "v.wl = wr;\n    v.wr = wl;"),
    "causal_strict": ("if (causal && j > i) return 0;", "if (causal && j >= i) return 0;"),
    "mask_transposed": ("mask[(i / REF_MASK_BLOCK) * nb + (j / REF_MASK_BLOCK)]",
                        "mask[(j / REF_MASK_BLOCK) * nb + (i / REF_MASK_BLOCK)]"),
    "no_normalize": ("exp(S[i * N + j] - m) / z : 0.0;", "exp(S[i * N + j] - m) : 0.0;"),
    "lse_no_log": ("lse[i] = m + log(z);", "lse[i] = m + z;"),
    "lse_no_max": ("lse[i] = m + log(z);", "lse[i] = log(z);"),
    "qk_transposed": ("for (long c = 0; c < d; c++) acc += q[i * d + c] * k[j * d + c];\n            S[i * N + j]",
                      "for (long c = 0; c < d; c++) acc += q[j * d + c] * k[i * d + c];\n            S[i * N + j]"),
    "bwd_drop_D": ("dS[i * N + j] = P[i * N + j] * (dP[i * N + j] - acc);",
                   "dS[i * N + j] = P[i * N + j] * dP[i * N + j];"),
    "bwd_dk_no_scale": ("dkh[j * d + c] *= scale;", "dkh[j * d + c] *= 1.0;"),
    "bwd_dq_no_scale": ("dqh[i * d + c] *= scale;", "dqh[i * d + c] *= 1.0;"),
    "bwd_dv_uses_dS": ("dvh[j * d + c] += p * doh[i * d + c];", "dvh[j * d + c] += s * doh[i * d + c];"),
    "bwd_dP_transposed": ("acc += doh[i * d + c] * vh[j * d + c];", "acc += doh[j * d + c] * vh[i * d + c];"),
    "online_no_rescale": ("oi[c] *= corr;", "oi[c] *= 1.0;"),
    "paged_group_map": ("hk = h / group;", "hk = h % Hkv;"),
    "paged_causal_offset": ("long n = causal ? L - Nq + i + 1 : L;", "long n = causal ? L - Nq + i : L;"),
    "paged_no_scale": ("s[t] = scale * acc;", "s[t] = acc;"),
    "paged_v_from_k": ("const double* vt = v_cache +", "const double* vt = k_cache +"),
    "e4m3_bias": ("ldexp(8.0 + m, e - 10)", "ldexp(8.0 + m, e - 9)"),
    "e4m3_ties_odd": ("c = (lo & 1) ? hi : lo;", "c = (lo & 1) ? lo : hi;"),
    "hadamard_sign": ("acc += (__builtin_popcountl((unsigned long)(i & j)) & 1) ? -t : t;",
                      "acc += (__builtin_popcountl((unsigned long)(i | j)) & 1) ? -t : t;"),
    "hadamard_k_side": ("y[i] = inverse_side ? acc / (double)d : acc;", "y[i] = acc;"),
    "block_scale_floor": ("while (ldexp(amax, -(e - 1)) <= 448.0) e--;", "e--;"),
}


@pytest.fixture(scope="module")
def src():
    return oracle.source_text()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, src, tmp_path):
    old, new = MUTANTS[name]
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    text = src.replace(old, new, 1)
    path = oracle.build_variant(text, os.path.join(str(tmp_path), f"mut_{name}.so"))
    orc = oracle.Oracle(path)
    failed = []
    for pin in P.ALL_PINS:
        try:
            pin(orc)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"no pin catches mutant {name}"
