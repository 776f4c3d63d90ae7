"""The pins must catch plausible mistakes in the oracle.

Each case copies ``oracle/hisparse_oracle.c``, plants one mistake by text
substitution, builds it with gcc into a temporary library, points the oracle
module at it and runs a quick subset of the pins. Every mutant must fail at
least one pin. Nothing here touches the real oracle build."""

import os
import subprocess
import tempfile

import numpy as np
import pytest

import oracle

SRC = os.path.join(os.path.dirname(oracle.__file__), "hisparse_oracle.c")

MUTANTS = {
    "victim_from_newest_end": ("const int16_t v = evict[M];", "const int16_t v = evict[ne - 1 - M];"),
    "hits_before_fills": ("for (int32_t e = 0; e < M; ++e) new_lru[q++] = evict[e];\n"
                          "    for (int32_t h = 0; h < nh; ++h) new_lru[q++] = hits[h];",
                          "for (int32_t h = 0; h < nh; ++h) new_lru[q++] = hits[h];\n"
                          "    for (int32_t e = 0; e < M; ++e) new_lru[q++] = evict[e];"),
    "fills_before_stale": ("for (int32_t e = M; e < ne; ++e) new_lru[q++] = evict[e];\n"
                           "    for (int32_t e = 0; e < M; ++e) new_lru[q++] = evict[e];",
                           "for (int32_t e = 0; e < M; ++e) new_lru[q++] = evict[e];\n"
                           "    for (int32_t e = M; e < ne; ++e) new_lru[q++] = evict[e];"),
    "newest_not_bound": ("if (t == newest) {", "if (t == L) {"),
    "pool_row_off_by_one": ("pending[j].token : pool_row(a, r, pending[j].token);",
                            "pending[j].token : pool_row(a, r, pending[j].token) + 1;"),
    "misses_in_token_order": ("qsort(pending, (size_t)np, sizeof(pending_t), cmp_by_index);", ""),
    "table_not_updated": ("tokens[v] = pending[j].token;", ""),
    "seq_len_bound_inclusive": ("if (t < 0 || t >= L || t >= a->ctx_stride)",
                                "if (t < 0 || t > L || t >= a->ctx_stride)"),
    "newest_slot_off_by_one": ("out[i] = (int32_t)hot_row(a, r, H);", "out[i] = (int32_t)hot_row(a, r, H - 1);"),
    "hit_output_wrong_slot": ("out[f->index] = (int32_t)hot_row(a, r, s);",
                              "out[f->index] = (int32_t)hot_row(a, r, p);"),
    "lru_transposed_index": ("const int16_t s = lru[p];", "const int16_t s = (int16_t)p;"),
    "no_padding": ("if (b >= nreal || r < 0 || r >= a->R) {", "if (r < 0 || r >= a->R) {"),
    "plan_list_at_entry_index": ("a->list_src[(int64_t)b * K + M] = src;\n"
                                 "        a->list_dst[(int64_t)b * K + M] = (int32_t)dst;",
                                 "a->list_src[(int64_t)b * K + pending[j].index] = src;\n"
                                 "        a->list_dst[(int64_t)b * K + pending[j].index] = (int32_t)dst;"),
    "plan_mask_not_set": ("if (mask) mask[pending[j].index] = 1;", ""),
    "replay_count_clamp_off_by_one": ("if (n > K) n = K;", "if (n > K) n = K - 1;"),
    "replay_no_zero_fill": ("memset(to, 0, (size_t)row_bytes);", ""),
    "replay_row_zero_has_no_source": ("if (s < pool_nrows) {", "if (s > 0 && s < pool_nrows) {"),
    "kv_swap_v_from_k_pool": ("memcpy(a->hot_v + dst * a->row_bytes, a->pool_v + src * a->row_bytes",
                              "memcpy(a->hot_v + dst * a->row_bytes, a->pool + src * a->row_bytes"),
    "kv_swap_v_not_copied": ("      if (a->pool_v)\n        memcpy(a->hot_v", "      if (0)\n        memcpy(a->hot_v"),
    "kv_transfer_v_from_k": ("v_src_layers[l] + s * row_bytes", "k_src_layers[l] + s * row_bytes"),
    "kv_scatter_v_k_stride": ("v_src + j * v_src_stride", "v_src + j * k_src_stride"),
    "paged_null_block_accepted": ("      if (pb > 0) *g = pb * p->src_block_size", "      if (pb >= 0) *g = pb * p->src_block_size"),
    "paged_resident_ignored": ("if (res >= 0) { out[i] = (int32_t)res; continue; }", ""),
    "paged_hot_offset_divides": ("return blk * p->hot_block_size + s % p->hot_block_size;",
                                 "return blk * p->hot_block_size + s / p->hot_block_size;"),
    "paged_key_is_position": ("pending[np].token = (int32_t)g;", "pending[np].token = (int32_t)t;"),
    "invalidate_row_zero": ("if (slot_keys[r * S_r + s] == g) { slot_keys[r * S_r + s] = -1;",
                            "if (slot_keys[s] == g) { slot_keys[s] = -1;"),
    "attention_offset_wrong": ("                               o % p->hot_block_size);",
                               "                               o % p->attention_block_stride);"),
    "stats_hits_are_evictables": ("a->stats[0] += (uint64_t)nh;", "a->stats[0] += (uint64_t)ne;"),
    "stats_misses_not_added": ("a->stats[1] += (uint64_t)M;", ""),
    "paged_resident_null_block_ignored": ("if (pb != p->resident_null_block && pb >= 0)",
                                          "if (pb >= 0)"),
    "negative_pool_row_accepted": ("if (pr < 0 || pr >= a->pool_nrows) { out[i] = -1; continue; }",
                                   "if (pr >= a->pool_nrows) { out[i] = -1; continue; }"),
    "state_row_past_R_processed": ("if (b >= nreal || r < 0 || r >= a->R) {", "if (b >= nreal || r < 0) {"),
    "resident_row_past_int32_served": ("    if (*res > INT32_MAX) *res = -1;\n", ""),
    "replay_negative_source_zeroed": ("if (s < 0 || d < 0 || d >= hot_nrows) continue;",
                                      "if (d < 0 || d >= hot_nrows) continue;\n        if (s < 0) { memset(hot_layers[l] + d * row_bytes, 0, (size_t)row_bytes); continue; }"),
}


def _pins():
    """A quick subset of the pins; returns the names of those that failed."""
    import test_oracle_closed_forms as cf
    import test_oracle_golden as g
    import test_oracle_model as m
    import test_oracle_plan as pl
    import test_oracle_kv as kvt
    import test_oracle_paged as pgt
    import test_oracle_copies_and_errors as ce
    failed = []
    checks = [
        ("golden1", lambda: g.test_swap_in_worked_examples("swap_in_worked_example_1.json")),
        ("golden2", lambda: g.test_swap_in_worked_examples("swap_in_worked_example_2.json")),
        ("model_random", lambda: m.test_random_multirow_with_tables(0)),
        ("textbook_lru", lambda: m.test_topk1_is_textbook_lru(4, 9, 1)),
        ("cold", lambda: cf.test_cold_start(64, 16)),
        ("disjoint", lambda: cf.test_disjoint_step_evicts_oldest(0)),
        ("replay_golden", pl.test_replay_worked_example),
        ("replay_numpy", lambda: pl.test_replay_layers_matches_numpy(1)),
        ("kv_golden", kvt.test_kv_copies_worked_example),
        ("kv_swap_golden", lambda: kvt.test_swap_in_v_rows_follow_k_rows("swap_in_worked_example_1.json")),
        ("kv_model", lambda: m.test_random_multirow_kv(0)),
        ("paged_golden", pgt.test_paged_worked_example),
        ("paged_model", lambda: pgt.test_paged_matches_model(0)),
        ("state_row_past_R", ce.test_state_row_past_R_is_padding_with_otherwise_valid_ids),
        ("resident_past_int32", pgt.test_resident_row_past_int32_is_not_resident),
    ]
    for name, fn in checks:
        try:
            fn()
        except (AssertionError, oracle.OracleError):
            failed.append(name)
    return failed


def test_unmutated_passes_pins():
    oracle.use_library(None)
    assert _pins() == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "mutant.c")
        open(c, "w").write(src.replace(old, new))
        lib = os.path.join(d, "libmutant.so")
        subprocess.check_call(["gcc", "-std=c11", "-O1", "-w", "-fPIC", "-shared",
                               "-I", os.path.dirname(SRC), "-o", lib, c])
        oracle.use_library(lib)
        try:
            failed = _pins()
        finally:
            oracle.use_library(None)
    assert failed, f"mutant {name} passed every pin"
