"""Planted mistakes in copies of the oracle must each fail at least one pin.

Every mutant is the oracle source with one plausible slip applied textually (a dropped term, a
wrong sign or index, a swapped operand, a wrong tie-break, an unsafe in-place order), built with
gcc into a temporary directory.  The real oracle is never modified.
"""
import os

import pytest

import oracle

from . import pins

MUTANTS = {
    "self_not_in_ancestors": ("for (int32_t j = i; j >= 0; j = parent[j]) {",
                              "if (i == 0) rev[n++] = 0;\n    for (int32_t j = parent[i]; j >= 0; j = parent[j]) {"),
    "gqa_modulo_mapping": ("const int32_t g = h / G;", "const int32_t g = h % hkv;"),
    "prefix_off_by_one": ("for (int32_t t = t0; t < L; ++t) slots[nvis++] = token_slot(",
                          "for (int32_t t = t0 + 1; t < L; ++t) slots[nvis++] = token_slot("),
    "window_keeps_one_more": ("return (window > 0 && L > window) ? L - window : 0;",
                              "return (window > 0 && L > window) ? L - window - 1 : 0;"),
    "page_row_from_page_index": ("* page_size + t % page_size;", "* page_size + t / page_size;"),
    "paged_compact_descending_in_place": (
        "            for (int32_t t = 0; t < len; ++t) {\n"
        "                const size_t dst = lo + (size_t)token_slot(NULL, block_table, bt_stride, page_size, b, L + t) * row;\n"
        "                const size_t src = lo + (size_t)token_slot(NULL, block_table, bt_stride, page_size, b, L + path[t]) * row;\n"
        "                memcpy((char *)k_out + dst, (const char *)k_in + src, row);\n"
        "                memcpy((char *)v_out + dst, (const char *)v_in + src, row);",
        "            for (int32_t t = len - 1; t >= 0; --t) {\n"
        "                const size_t dst = lo + (size_t)token_slot(NULL, block_table, bt_stride, page_size, b, L + t) * row;\n"
        "                const size_t src = lo + (size_t)token_slot(NULL, block_table, bt_stride, page_size, b, L + path[t]) * row;\n"
        "                memcpy((char *)k_out + dst, (const char *)k_out + src, row);\n"
        "                memcpy((char *)v_out + dst, (const char *)v_out + src, row);"),
    "philox_weyl_constant": ("k[0] += 0x9E3779B9u;", "k[0] += 0x9E3779BBu;"),
    "philox_nine_rounds": ("for (int r = 0; r < 10; ++r) {\n        if (r) {", "for (int r = 0; r < 9; ++r) {\n        if (r) {"),
    "philox_multiplier": ("(uint64_t)0xCD9E8D57u * x[2]", "(uint64_t)0xCD9E8D55u * x[2]"),
    "sample_word_order_reversed": ("const uint32_t word = out[v % 4];", "const uint32_t word = out[3 - v % 4];"),
    "sample_offset_words_swapped": ("(uint32_t)row, (uint32_t)offset, (uint32_t)(offset >> 32)}",
                                    "(uint32_t)row, (uint32_t)(offset >> 32), (uint32_t)offset}"),
    "sample_noise_sign": ("fmaf(z, c, -log2f(-log2f(u)))", "fmaf(z, c, log2f(-log2f(u)))"),
    "sample_temperature_ignored": ("return (float)(1.4426950408889634 / (double)temperature);",
                                   "return 1.4426950408889634f;"),
    "sample_exponential_noise": ("fmaf(z, c, -log2f(-log2f(u)))", "fmaf(z, c, -log2f(u))"),
    "softmax_sign": ("scratch[t] = exp(scratch[t] - m);", "scratch[t] = exp(m - scratch[t]);"),
    "scale_dropped": ("scratch[t] = sm_scale * dot;", "scratch[t] = dot;"),
    "k_v_swapped": ("dot += elem(q, dtype, qrow + c) * elem(k, dtype, krow + c);",
                    "dot += elem(q, dtype, qrow + c) * elem(v, dtype, krow + c);"),
    "lse_base2": ("*lse = m + log(sum);", "*lse = m + log2(sum);"),
    "argmax_last_tie": ("if (x > bv) { best = t; bv = x; }", "if (x >= bv) { best = t; bv = x; }"),
    "argmax_ignores_nan": ("if (isnan(x)) { best = t; bv = x; break; }", "if (0) { best = t; bv = x; break; }"),
    "accept_highest_index_tie": ("if (acc[i] && depth[i] > depth[best]) best = i;",
                                 "if (acc[i] && depth[i] >= depth[best]) best = i;"),
    "accept_ignores_ancestors": ("acc[i] = acc[p] && draft[s + i] == target[s + p];",
                                 "acc[i] = draft[s + i] == target[s + p];"),
    "accept_own_target": ("acc[i] = acc[p] && draft[s + i] == target[s + p];",
                          "acc[i] = acc[p] && draft[s + i] == target[s + i];"),
    "bonus_from_root": ("*bonus = target[s + best];", "*bonus = target[s];"),
    # sampled acceptance: the deepest-path rule of the greedy case applied to the draws, and the
    # last (not the first) child holding the draw
    "sampled_accept_deepest_rule": (
        "                           int32_t *out_tokens, int32_t *seq_err) {\n",
        "                           int32_t *out_tokens, int32_t *seq_err) {\n"
        "    oracle_greedy_accept(node_start, parent, draft, target, batch, max_nodes, vocab, accept_len,\n"
        "                         accept_path, bonus_token, out_tokens, seq_err);\n"
        "    if (batch >= 0) return;\n"),
    "sampled_accept_last_child": ("next = c;\n                    break;", "next = c;"),
    "compact_descending_in_place": (
        "            for (int32_t t = 0; t < len; ++t) {\n"
        "                const size_t dst = lo + (size_t)(base + t) * row;\n"
        "                const size_t src = lo + (size_t)(base + path[t]) * row;\n"
        "                memcpy((char *)k_out + dst, (const char *)k_in + src, row);\n"
        "                memcpy((char *)v_out + dst, (const char *)v_in + src, row);",
        "            for (int32_t t = len - 1; t >= 0; --t) {\n"
        "                const size_t dst = lo + (size_t)(base + t) * row;\n"
        "                const size_t src = lo + (size_t)(base + path[t]) * row;\n"
        "                memcpy((char *)k_out + dst, (const char *)k_out + src, row);\n"
        "                memcpy((char *)v_out + dst, (const char *)v_out + src, row);"),
    "new_len_excludes_bonus": ("new_len[b] = prefix_len[b] + len;", "new_len[b] = prefix_len[b] + len - 1;"),
    "tree_rule_allows_self_parent": ("if (parent[i] < 0 || parent[i] >= i) err |= 1;",
                                     "if (parent[i] < 0 || parent[i] > i) err |= 1;"),
}


@pytest.fixture(scope="module")
def source():
    with open(os.path.join(os.path.dirname(oracle.__file__), "ev_oracle.c")) as f:
        return f.read()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, source, tmp_path):
    old, new = MUTANTS[name]
    assert source.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    src = tmp_path / "mutant.c"
    src.write_text(source.replace(old, new))
    lib = oracle.load(oracle.build(str(src), str(tmp_path / "libmutant.so")))
    failed = []
    for pin in pins.ALL_PINS:
        try:
            pin(lib)
        except (AssertionError, IndexError, ValueError):
            failed.append(pin.__name__)
    assert failed, f"no pin catches mutant {name}"
