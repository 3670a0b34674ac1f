"""The pins have teeth: plant a plausible mistake in a copy of the oracle, on
the CPU, and check that at least one pin of test_oracle_pins rejects it.

Each mutant is one textual change of oracle/gsa_oracle.c, compiled with the
same flags into a temporary library that the pins then run against.
"""
import os

import pytest

import oracle
from tests import _util as U
from tests import test_oracle_pins as P
from tests import test_oracle_levels as PL
from tests import test_oracle_prefill as PP
from long_context_sparse_gist_amd import inputs as gi

MUTANTS = {
    "scale_dropped": ("z[j] = tau * dot_q(", "z[j] = dot_q("),
    "ties_to_higher_index": ("return (a->id < b->id) ? -1 : (a->id > b->id);",
                             "return (a->id > b->id) ? -1 : (a->id < b->id);"),
    "keys_ascending": ("if (a->s > b->s) return -1;\n        if (a->s < b->s) return 1;",
                       "if (a->s < b->s) return -1;\n        if (a->s > b->s) return 1;"),
    "gist_slot_off_by_one": (" rows[m] = slot_base(&sv, (long)m * (C + 1) + C);\n        ids[m] = m;",
                             " rows[m] = slot_base(&sv, (long)m * (C + 1) + C - 1);\n        ids[m] = m;"),
    "head_to_group_transposed": ("dot_q(c, q, b, g * G + j, kv, kb)",
                                 "dot_q(c, q, b, j * c->num_kv_heads + g, kv, kb)"),
    "raw_tail_dropped": ("for (int r = 0; r < tail; r++) { T[nT].arr_k = kc; T[nT].arr_v = vc; "
                         "T[nT].row = slot_base(&sv, (long)n * (C + 1) + r); nT++; }\n    /* O4 */",
                         "for (int r = 0; r < 0; r++) { T[nT].arr_k = kc; T[nT].arr_v = vc; "
                         "T[nT].row = slot_base(&sv, (long)n * (C + 1) + r); nT++; }\n    /* O4 */"),
    "first_raw_token_dropped": (
        "long s0 = (long)m * (C + 1);\n        if (is_sel[m])\n            for (int r = 0; r < C; r++)"
        " { T[nT].arr_k = kc; T[nT].arr_v = vc; T[nT].row = slot_base(&sv, s0 + r); nT++; }\n"
        "        if (is_sel[m] || all_gists)",
        "long s0 = (long)m * (C + 1);\n        if (is_sel[m])\n            for (int r = 1; r < C; r++)"
        " { T[nT].arr_k = kc; T[nT].arr_v = vc; T[nT].row = slot_base(&sv, s0 + r); nT++; }\n"
        "        if (is_sel[m] || all_gists)"),
    "v_read_from_k": ("o[i] += p * ld(T[t].arr_v, T[t].row + i, c->dtype);",
                      "o[i] += p * ld(T[t].arr_k, T[t].row + i, c->dtype);"),
    "softmax_not_normalised": ("for (int i = 0; i < d; i++) o[i] /= lam;",
                               "for (int i = 0; i < d; i++) o[i] /= 1.0;"),
    "page_layout_heads_outer": (
        "return (((size_t)phys * c->num_kv_heads + sv->g) * spp + off) * c->head_dim;",
        "return (((size_t)sv->g * c->num_pages + phys) * spp + off) * c->head_dim;"),
    "bf16_widened_wrong": ("(uint32_t)((const uint16_t *)p)[i] << 16;",
                           "(uint32_t)((const uint16_t *)p)[i] << 15;"),
    "candidates_wrong_group": ("cids[nc++] = sel1[i] * R + j;", "cids[nc++] = sel1[i] + j * nm;"),
    "tail_gists_not_candidates": ("for (int m = nm * R; m < n; m++) cids[nc++] = m;",
                                  "for (int m = nm * R; m < nm * R; m++) cids[nc++] = m;"),
    "ext_sel_ignored": ("    if (ext_sel) {\n        ns = 0;", "    if (0) {\n        ns = 0;"),
    "ext_sel_range_unchecked": ("if (ext_sel[i] >= 0 && ext_sel[i] < n) sel[ns++]",
                                "if (ext_sel[i] >= 0 && ext_sel[i] < c->num_chunks) sel[ns++]"),
    "ext1_ignored": ("    if (ext1) {", "    if (0) {"),
    "ext2_ignored": ("    if (ext2) {", "    if (0) {"),
    "level_children_wrong": ("cand[nc++] = sel[l][i] * R + j;", "cand[nc++] = sel[l][i] + j * cnt[l];"),
    "level_tail_not_candidates": ("for (int r = cnt[l] * R; r < cnt[l - 1]; r++) cand[nc++] = r;",
                                  "for (int r = cnt[l] * R; r < cnt[l] * R; r++) cand[nc++] = r;"),
    "level_keys_from_v": ("routing_keys(c, q, b, g, ARR_K(l), rows, nc, S);",
                          "routing_keys(c, q, b, g, ARR_V(l), rows, nc, S);"),
    "level_kept_not_attended": ("if (l == L || in[r] || r >= past)", "if (l == L || r >= past)"),
    "level_tail_not_attended": ("if (l == L || in[r] || r >= past)", "if (l == L || in[r])"),
    "top_level_only_kept_attended": ("if (l == L || in[r] || r >= past)",
                                     "if (in[r] || (l < L && r >= past))"),
    "level_gist_tail_dropped": ("if (L == 0 || is_sel[m] || m >= past0)", "if (L == 0 || is_sel[m])"),
    "prefill_gist_slot_off_by_one": ("for (long mp = 0; mp < m; mp++) krow[j++] = slot_base(&sv, mp * (C + 1) + C);",
                                     "for (long mp = 0; mp < m; mp++) krow[j++] = slot_base(&sv, mp * (C + 1) + C - 1);"),
    "prefill_scale_dropped": ("z[j] = tau * acc;", "z[j] = acc;"),
    "prefill_wrong_kv_head": ("seqview sv = {c, k_cache, v_cache, block_table, b, h / G};",
                              "seqview sv = {c, k_cache, v_cache, block_table, b, h % c->num_kv_heads};"),
    "prefill_v_from_k": ("o[e] += p * ld(v_cache, krow[j] + e, c->dtype);",
                         "o[e] += p * ld(k_cache, krow[j] + e, c->dtype);"),
    "prefill_query_slot_shifted": ("long s = (long)q_start[b] + t;",
                                   "long s = (long)q_start[b] + t - (t > 0);"),
    "meta_gists_not_attended": ("for (int r = 0; r < nm; r++) { T[nT].arr_k = km;",
                                "for (int r = 0; r < 0; r++) { T[nT].arr_k = km;"),
}


def pin_battery():
    """Every pin, as (name, thunk)."""
    out = []
    for wl in (P.SMALL_BF16, P.SMALL_F32, P.SMALL_D128):
        for lens in ("full", "ragged"):
            out.append((f"keys_topk/{wl.name}/{lens}",
                        lambda wl=wl, lens=lens: P.test_keys_and_topk_match_brute_force(wl, lens)))
        out.append((f"pa/{wl.name}", lambda wl=wl: P.test_pa_all_chunks_is_dense_attention(wl)))
        for fl in (0, oracle.SET_SELECTED_GISTS):
            out.append((f"pc/{wl.name}/{fl}",
                        lambda wl=wl, fl=fl: P.test_pc_masked_dense_invariant(wl, fl)))
    out += [("pb", P.test_pb_planted_selection_tiny_f32), ("pd", P.test_pd_k0_gists_only),
            ("pe", P.test_pe_ties_go_to_lower_index), ("pf", P.test_pf_page_permutation_and_sharing),
            ("pg", P.test_pg_group_collapse), ("ph", P.test_ph_hierarchy_reduces_to_flat_topk),
            ("pa_h", P.test_pa_hierarchy_all_kept_is_dense_over_meta_and_sequence),
            ("h_full", lambda: P.test_hgsa_matches_brute_force("full")),
            ("h_ragged", lambda: P.test_hgsa_matches_brute_force("ragged")),
            ("sum_probs", P.test_sum_of_probs_keys)]
    for fl in (0, oracle.SET_SELECTED_GISTS):
        out.append((f"o6_flat/{fl}", lambda fl=fl: P.test_o6_external_selection_flat(fl)))
    for which in ("meta", "gist", "both"):
        out.append((f"o6_h/{which}", lambda which=which: P.test_o6_external_selection_hgsa(which)))
    for wl in (P.SMALL_BF16, P.SMALL_F32):
        out.append((f"pi/{wl.name}", lambda wl=wl: P.test_pi_convex_hull(wl)))
    out += [("lv_flat", PL.test_no_meta_level_is_flat_gsa),
            ("lv_hgsa", PL.test_one_meta_level_is_two_level_hgsa),
            ("lv_f32", PL.test_levels_f32_and_planted_ancestors),
            ("lv_dense", PL.test_everything_kept_is_dense_over_all_levels)]
    for fo, tp in [((4, 3), (5, 2)), ((3, 2, 2), (4, 3, 2)), ((2, 2, 2), (3, 2, 1))]:
        for lens in ("full", "ragged"):
            out.append((f"lv_bf/{fo}/{lens}",
                        lambda fo=fo, tp=tp, lens=lens: PL.test_levels_match_brute_force(fo, tp, lens)))
    for which in (0, 1, 2):
        out.append((f"lv_ext/{which}", lambda which=which: PL.test_caller_selection_at_a_level(which)))
    for name in sorted(PL.CASES):
        out.append((f"lv_golden/{name}", lambda name=name: PL.test_levels_hand_worked(name)))
    for wl in (PP.SMALL, PP.SMALL_F32):
        for start in ("chunk", "mid", "tail"):
            out.append((f"pf_dense/{wl.name}/{start}",
                        lambda wl=wl, start=start: PP.test_prefill_matches_masked_dense(wl, start)))
    out += [("pf_decode", PP.test_prefill_tail_query_is_decode_with_no_chunk_unfolded),
            ("pf_first", PP.test_prefill_first_slot_and_first_gist),
            ("pf_pages", PP.test_prefill_page_order_invariant)]
    for name in sorted(PP.CASES):
        out.append((f"pf_golden/{name}", lambda name=name: PP.test_prefill_hand_worked(name)))
    return out


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    find, repl = MUTANTS[name]
    src = open(oracle._SRC).read()
    assert src.count(find) == 1, f"mutation site of {name} not unique"
    path = os.path.join(tmp_path, "mutant.c")
    with open(path, "w") as f:
        f.write(src.replace(find, repl))
    lib = oracle.load(oracle.compile_source(path, os.path.join(tmp_path, "libmutant.so")))
    caught = []
    saved = U.ORACLE_LIB
    U.ORACLE_LIB = lib
    try:
        for pin, fn in pin_battery():
            try:
                fn()
            except (AssertionError, ValueError):
                caught.append(pin)
                break
    finally:
        U.ORACLE_LIB = saved
    assert caught, f"no pin catches the mutant {name}"


def test_unmutated_copy_passes_every_pin(tmp_path):
    lib = oracle.load(oracle.compile_source(oracle._SRC, os.path.join(tmp_path, "libcopy.so")))
    saved = U.ORACLE_LIB
    U.ORACLE_LIB = lib
    try:
        for _, fn in pin_battery():
            fn()
    finally:
        U.ORACLE_LIB = saved
