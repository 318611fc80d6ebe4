"""The pins must be strong enough to catch plausible mistakes in the oracle.

Each case copies oracle.c, plants one mistake (a dropped ReLU, a wrong index, an
off-by-one causal limit, a reversed tie rule, a missing division, truncation
instead of rounding, ...), compiles the copy with gcc into a temporary
directory and runs the pin battery against it: at least one pin must fail.
All of this runs on the CPU; the real oracle is never modified.
"""
import os
import shutil
import subprocess
import tempfile

import pytest

import oracle
from pins import ALL_PINS

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = {
    "relu_dropped": ("double relu = dot > 0.0 ? dot : 0.0;", "double relu = dot;"),
    "relu_is_abs": ("double relu = dot > 0.0 ? dot : 0.0;", "double relu = fabs(dot);"),
    "weight_of_head0": ("total += (double)w[j] * relu;", "total += (double)w[0] * relu;"),
    "weight_dropped": ("total += (double)w[j] * relu;", "total += relu;"),
    "mass_abs_of_dot": ("bound += fabs((double)w[j]) * adot;", "bound += fabs((double)w[j]) * fabs(dot);"),
    "mass_inflated": ("bound += fabs((double)w[j]) * adot;", "bound += 10.0 * fabs((double)w[j]) * adot;"),
    "mass_signed_weight": ("bound += fabs((double)w[j]) * adot;", "bound += (double)w[j] * adot;"),
    "mass_unweighted": ("bound += fabs((double)w[j]) * adot;", "bound += adot;"),
    "mass_signed_products": ("adot += fabs(p);", "adot += p;"),
    "candidate_after_last": ("if (s < 0 || s > t_last || seen[s])",
                             "if (s < 0 || s > t_last + 1 || (s <= t_last && seen[s]))"),
    "candidate_tail_unchecked": ("} else if (s != -1) {", "} else if (s < -1) {"),
    "candidate_tail_negative_ok": ("} else if (s != -1) {", "} else if (s >= 0) {"),
    "candidate_list_short": ("int64_t want = c < t_last + 1 ? c : t_last + 1;",
                             "int64_t want = c < t_last + 1 ? c - 1 : t_last;"),
    "candidate_duplicates_ok": ("if (s < 0 || s > t_last || seen[s])", "if (s < 0 || s > t_last)"),
    "query_of_head0": ("double p = qd[(int64_t)j * d + e] * kd[e];", "double p = qd[e] * kd[e];"),
    "key_element0": ("kd[e] = bf16_to_double(K[s * d + e]);", "kd[e] = bf16_to_double(K[s * d]);"),
    "causal_strict": ("int64_t n = L - q_len + r + 1;", "int64_t n = L - q_len + r;"),
    "position_ignores_qlen": ("int64_t n = L - q_len + r + 1;", "int64_t n = r + 1;"),
    "ties_to_higher_index": ("if (a->idx < b->idx)\n        return -1;\n    if (a->idx > b->idx)\n        return 1;",
                             "if (a->idx > b->idx)\n        return -1;\n    if (a->idx < b->idx)\n        return 1;"),
    "ascending_scores": ("if (a->score > b->score)\n        return -1;\n    if (a->score < b->score)\n        return 1;",
                         "if (a->score < b->score)\n        return -1;\n    if (a->score > b->score)\n        return 1;"),
    "proxy_not_divided": ("qbar[x] = float_to_bf16_rne(acc / cnt);", "qbar[x] = float_to_bf16_rne(acc);"),
    "proxy_truncates": ("u += 0x7FFFu + lsb;", "u += 0u * lsb;"),
    "proxy_rounds_half_up": ("u += 0x7FFFu + lsb;", "u += 0x8000u + 0u * lsb;"),
    "proxy_count_is_g": ("int64_t wn = (window == 0 || window >= n) ? n : window;",
                         "int64_t wn = (window == 0 || window >= n) ? g : window;"),
    "proxy_weight_first_member": ("wbar[j] = acc / cnt;", "wbar[j] = W[a * H + j];"),
    "proxy_window_from_first_member": ("        a = r1 - wn;\n", "        a = r0;\n"),
    "proxy_last_is_first": ("        a = r1 - 1;\n", "        a = r0;\n        b = r0 + 1;\n        (void)0;\n"),
    "refine_not_causal": ("if (cand[x] >= 0 && cand[x] <= pos)", "if (cand[x] >= 0 && cand[x] <= t_last)"),
    "scan_stops_early": ("int64_t t_last = L - q_len + r1 - 1;", "int64_t t_last = L - q_len + r1 - 2;"),
    "scan_starts_group": ("int64_t t_last = L - q_len + r1 - 1;", "int64_t t_last = L - q_len + r0;"),
    "chunk_mean_not_divided": ("float_to_bf16_rne(sum / nkeys);", "float_to_bf16_rne(sum);"),
    "chunk_mean_first_chunk_size": ("float nkeys = (float)(end - first);", "float nkeys = (float)cend[0];"),
    "chunk_mean_skips_first_key": ("for (int64_t s = first; s < end; ++s)", "for (int64_t s = first + 1; s < end; ++s)"),
    "chunk_in_progress_scored": ("cend[ncomp] <= t_last + 1)", "(ncomp == 0 ? 0 : cend[ncomp - 1]) <= t_last)"),
    "chunk_complete_strict": ("cend[ncomp] <= t_last + 1)", "cend[ncomp] < t_last + 1)"),
    "tail_dropped": ("s <= t_last && rc == ORC_OK; ++s) {", "s < 0 && rc == ORC_OK; ++s) {"),
    "tail_starts_late": ("for (int64_t s = (ncomp == 0 ? 0 : cend[ncomp - 1]); s <=",
                         "for (int64_t s = (ncomp == 0 ? 0 : cend[ncomp - 1]) + 1; s <="),
    "chunk_refine_not_causal": ("if (trow[x] > pos)", "if (trow[x] > t_last)"),
    "chunks_in_rank_order": ("for (int64_t x = 1; x < nsc; ++x)", "for (int64_t x = 1; x < 0; ++x)"),
    "chunk_expansion_past_end": ("s < cend[b]; ++s) {", "s <= cend[b] && s < L; ++s) {"),
    "dispersion_no_mean_term": ("total += s2 - s1 * s1 / n;", "total += s2;"),
    "split_lowest_gain_first": ("qsort(gain, (size_t)nfull, sizeof(orc_rank), rank_desc);",
                                "qsort(gain, (size_t)nfull, sizeof(orc_rank), rank_asc);"),
    "merge_highest_loss_first": ("qsort(loss, (size_t)npair, sizeof(orc_rank), rank_asc);",
                                 "qsort(loss, (size_t)npair, sizeof(orc_rank), rank_desc);"),
    "gain_ties_to_higher_block": ("a->key < b->key)\n        return 1;\n    return a->idx < b->idx ? -1 : (a->idx > b->idx ? 1 : 0);",
                                  "a->key < b->key)\n        return 1;\n    return a->idx > b->idx ? -1 : (a->idx < b->idx ? 1 : 0);"),
    "chunk_group_ends_early": ("int64_t t_last = (L - q_len) + r1 - 1;", "int64_t t_last = (L - q_len) + r1 - 2;"),
    "chunk_group_at_first_member": ("int64_t t_last = (L - q_len) + r1 - 1;", "int64_t t_last = (L - q_len) + r0;"),
    "greedy_accepts_equal": ("!(gain[ia].key > loss[ib].key)", "!(gain[ia].key >= loss[ib].key)"),
    "greedy_one_step": ("        ++ia;\n        ++ib;\n", "        ++ia;\n        ++ib;\n        break;\n"),
    "merge_ignores_split_blocks": ("int conflict = split[2 * j] || split[2 * j + 1] ||", "int conflict = 0 ||"),
    "split_ignores_merged_pair": ("while (ia < nfull && gain[ia].idx / 2 < npair && merged[gain[ia].idx / 2])",
                                  "while (ia < nfull && 0)"),
    "split_point_off": ("cend[out++] = (int32_t)(a + h);", "cend[out++] = (int32_t)(a + h + 1);"),
}


@pytest.fixture(scope="module")
def workdir():
    d = tempfile.mkdtemp(prefix="oracle_mutants_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


def test_unmutated_copy_passes(workdir):
    src = open(SRC).read()
    path = os.path.join(workdir, "orig.c")
    with open(path, "w") as f:
        f.write(src)
    lib = oracle.load(oracle.build(path, os.path.join(workdir, "orig.so")))
    for pin in ALL_PINS:
        pin(lib)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, workdir):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    path = os.path.join(workdir, f"{name}.c")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    so = os.path.join(workdir, f"{name}.so")
    try:
        lib = oracle.load(oracle.build(path, so))
    except subprocess.CalledProcessError:
        pytest.fail(f"mutant {name} does not compile")
    caught = []
    for pin in ALL_PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches the mutant {name}"
