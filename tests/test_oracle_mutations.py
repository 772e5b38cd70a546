"""Plant plausible mistakes in copies of the CPU oracle and check that the pins catch each one.

Every mutant is compiled from a modified copy of oracle/mep_oracle.c into a temporary directory
and loaded in place of the real oracle for the duration of one check.  CPU only; the product
library is not involved."""
import os
import subprocess
import tempfile

import numpy as np
import pytest

import oracle
import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "mep_oracle.c")

# (name, exact text in the oracle, replacement)
MUTANTS = [
    ("tie_to_higher_index", "return ia < ib;", "return ia > ib;"),
    ("sigmoid_sign", "double s = 1.0 / (1.0 + exp(-xd));", "double s = 1.0 / (1.0 + exp(xd));"),
    ("bias_dropped", "key[e] = s[e] + b; /* one binary32 addition */", "key[e] = s[e];"),
    ("group_sum_keeps_last_only", "sum = (j == 0) ? key[best] : sum + key[best];",
     "sum = key[best];"),
    ("group_order_ascending", "if (best < 0 || beats(gscore[g], g, gscore[best], best)) best = g;",
     "if (best < 0 || !beats(gscore[g], g, gscore[best], best)) best = g;"),
    ("softmax_den_drops_last", "for (int k = 0; k < K; ++k) den += exp((double)x[sel[k]] - m);",
     "for (int k = 0; k < K - 1; ++k) den += exp((double)x[sel[k]] - m);"),
    ("sigmoid_scale_not_applied", "w = (double)s[sel[k]];\n                    topk_weights[t * K + k] = (float)(w * (double)scale);",
     "w = (double)s[sel[k]];\n                    topk_weights[t * K + k] = (float)(w);"),
    ("full_softmax_uses_topk", "for (int e = 0; e < E; ++e) den += exp((double)x[e] - m);",
     "for (int k = 0; k < K; ++k) den += exp((double)x[sel[k]] - m);"),
    ("pad_exact_multiples", "int64_t padded = count[e] > 0 ? ((count[e] + A - 1) / A) * A : 0;",
     "int64_t padded = count[e] > 0 ? (count[e] / A + 1) * A : 0;"),
    ("scatter_not_stable", "int64_t p = cu[e] + fill[e];",
     "int64_t p = cu[e] + count[e] - 1 - fill[e];"),
    ("sentinel_zero", "for (int64_t p = 0; p < T; ++p) permuted_to_expanded[p] = -1;",
     "for (int64_t p = 0; p < T; ++p) permuted_to_expanded[p] = 0;"),
    ("zero_fill_start", "zero_fill[2 * e] = (int32_t)(cu[e] + count[e]);",
     "zero_fill[2 * e] = (int32_t)(cu[e]);"),
    ("owner_modulo", "itr[t * R + ids[t * K + k] / epn] = 1;", "itr[t * R + ids[t * K + k] % R] = 1;"),
    ("rank_prefix_exclusive", "for (int64_t s2 = 0; s2 <= s; ++s2)", "for (int64_t s2 = 0; s2 < s; ++s2)"),
    ("channel_end_off_by_one", "int64_t e_ = (c + 1) * q < n ? (c + 1) * q : n;",
     "int64_t e_ = (c + 1) * q - 1 < n ? (c + 1) * q - 1 : n;"),
    ("dup_encoding_without_minus_one", "dst[i] = (int32_t)(earlier ? -raw - 1 : raw);",
     "dst[i] = (int32_t)(earlier ? -raw : raw);"),
    ("dst_offset_from_expert", "int64_t raw = (int64_t)r * NvS + (expanded_to_permuted[i] - cu_seqlens[r * epn]);",
     "int64_t raw = (int64_t)r * NvS + (expanded_to_permuted[i] - cu_seqlens[ids[i]]);"),
    ("dup_begin_global", "int64_t begin = dpos - dseg;", "int64_t begin = dpos;"),
    ("recv_zero_fill_not_rebased",
     "recv_zero_fill[2 * e] = (int32_t)(cu_seqlens[e] + cnt - cu_seqlens[r * epn]);",
     "recv_zero_fill[2 * e] = (int32_t)(cu_seqlens[e] + cnt);"),
    ("recv_cu_wrong_base",
     "recv_cu_seqlens[r * (epn + 1) + j] = cu_seqlens[r * epn + j] - cu_seqlens[r * epn];",
     "recv_cu_seqlens[r * (epn + 1) + j] = cu_seqlens[r * epn + j] - cu_seqlens[r];"),
    ("dup_offsets_inclusive", "gtot += ng[r];\n        dtot += nd[r];\n    }",
     "gtot += ng[r];\n        dtot += nd[r];\n        if (dup_offsets) { dup_offsets[2 * r] = (int32_t)gtot; }\n    }"),
    ("tile_count_floor", "num_cta[e] = ((int64_t)counts[e] + A - 1) / A;",
     "num_cta[e] = ((int64_t)counts[e]) / A;"),
    ("tile_limit_exclusive_end", "int64_t lim1 = (cta_offset[e] + cta + 1) * (int64_t)A;",
     "int64_t lim1 = (cta_offset[e] + cta) * (int64_t)A;"),
    ("tile_limit_ignores_count", "int64_t lim2 = cta_offset[e] * (int64_t)A + counts[e];",
     "int64_t lim2 = (cta_offset[e] + num_cta[e]) * (int64_t)A;"),
    ("permute_wrong_token", "(const char*)x + (size_t)t * row, row);",
     "(const char*)x + (size_t)((t * K + k) % N) * row, row);"),
    ("permute_no_zero_fill", "if (len == 0) continue;", "continue;"),
    ("combine_drops_weight", "float prod = topk_weights[t * K + k] * v;", "float prod = v;"),
    ("combine_weight_reversed", "float prod = topk_weights[t * K + k] * v;",
     "float prod = topk_weights[t * K + (K - 1 - k)] * v;"),
    ("combine_reverse_order", "for (int k = 0; k < K; ++k) {\n                int64_t p = expanded_to_permuted[t * K + k];\n                float v",
     "for (int k = K - 1; k >= 0; --k) {\n                int64_t p = expanded_to_permuted[t * K + k];\n                float v"),
    ("bf16_truncates_ties", "if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u))) upper += 1;",
     "if (lower > 0x8000u) upper += 1;"),
    ("balance_surplus_tie_high", "if (beats_max_low(bal[r], r, bal[sr], sr)) sr = r;",
     "if (beats_max_high(bal[r], r, bal[sr], sr)) sr = r;"),
    ("balance_move_capped_by_surplus", "int64_t move = -bal[dr];",
     "int64_t move = -bal[dr] < bal[sr] ? -bal[dr] : bal[sr];"),
    ("quota_remaining_tie_high", "if (beats_max_low(rem[j], j, rem[sj], sj)) sj = j;",
     "if (beats_max_high(rem[j], j, rem[sj], sj)) sj = j;"),
    ("copy_tie_low", "if (beats_max_high(remote[e], e, remote[best], best)) best = e;",
     "if (beats_max_low(remote[e], e, remote[best], best)) best = e;"),
    ("group_end_is_start", "cu_out[(int64_t)d * G + g] = (int32_t)(base + padded);",
     "cu_out[(int64_t)d * G + g] = (int32_t)(base);"),
    ("search_takes_equal", "if (ac > q) hi = mid;", "if (ac >= q) hi = mid;"),
    ("balanced_no_dup_encoding", "if (seen) dst[t * K + k] = -dst[t * K + k] - 1;", "(void)seen;"),
    ("unpicked_remote_dropped", "if (!picked[g]) { cnt = counts[g]; ex = g; }",
     "if (!picked[g] && g / epn == d) { cnt = counts[g]; ex = g; }"),
]


def _battery():
    """The pins, run in order; the first failure ends the battery."""
    pins.test_hand_example()
    pins.test_sigmoid_random_fp32_and_specials()
    for seed in range(3):
        for E, K in [(6, 2), (8, 3)]:
            pins.test_softmax_topk_matches_brute_force(seed, E, K)
        for args in [(8, 4, 2, 2, 2), (16, 4, 2, 4, 2), (16, 8, 3, 3, 2)]:
            pins.test_sigmoid_group_topk_matches_brute_force(seed, *args)
    pins.test_weights_k1_equal_scale()
    pins.test_weights_k2_softmax_is_logistic()
    pins.test_weights_full_softmax_and_sums()
    pins.test_weights_sigmoid_renorm_closed_form()
    for args in [(37, 8, 2, 128), (500, 16, 4, 3), (333, 128, 8, 1)]:
        pins.test_layout_equals_stable_sort(*args)
    for args in [(128, 8, 2, 2, 2, 24, 1), (96, 8, 2, 8, 8, 5, 128), (256, 64, 8, 8, 4, 24, 16),
                 (240, 32, 6, 4, 3, 7, 3)]:
        pins.test_plan_invariants(*args)
    pins.test_tile_map_hand_example()
    for seed in range(2):
        for E, A in [(5, 4), (16, 3)]:
            pins.test_tile_map_matches_row_enumeration(seed, E, A)
    for dtype in ("f32", "bf16"):
        pins.test_permute_then_combine_round_trip(dtype, 37, 8, 2, 4, 16)
        pins.test_combine_small_integers_exact(dtype)
    pins.test_combine_sums_in_slot_order()
    pins.test_combine_bf16_rounding_matches_torch()
    pins.test_balanced_hand_examples()
    pins.test_balanced_without_moves_is_the_plain_plan(64, 8, 2, 2, 1)
    pins.test_balanced_invariants(0, 16, 4, 4, 2, 3)


def test_real_oracle_passes_battery():
    _battery()


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new, monkeypatch):
    text = open(SRC).read()
    assert text.count(old) == 1, "mutation anchor must match exactly once: " + name
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "m.c")
        so = os.path.join(d, "m.so")
        open(c, "w").write(text.replace(old, new))
        subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-shared", "-fPIC", c,
                        "-o", so, "-lquadmath", "-lm"], check=True, capture_output=True)
        monkeypatch.setattr(oracle, "_lib", oracle.load(so))
        with pytest.raises((AssertionError, ValueError, IndexError)):
            with np.errstate(all="ignore"):
                _battery()
