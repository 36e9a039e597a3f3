"""The pins are strong enough: each plausible mistake planted into a copy of
the oracle's source (a dropped term, a wrong index, a reversed tie-break, a
missing scale, a transposed head map ...) makes at least one pin fail.
The planted copies are built with gcc into a temporary directory; the real
oracle is untouched."""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
import test_oracle_accept as tac
import test_oracle_commit as tcm
import test_oracle_layer as tly
import test_oracle_mask_attn as tma
import test_oracle_selective as tse
import test_oracle_topk as tto
import test_oracle_tree as ttr

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "oracle.c")

# (name, text in oracle.c, replacement, pin that must fail)
MUTATIONS = [
    ("lse drops first term", "        for (int v = 0; v < vocab; ++v)\n                s += exp(",
     "        for (int v = 1; v < vocab; ++v)\n                s += exp(",
     lambda: tto.test_lse_constant_row_closed_form()),
    ("top-K tie goes to larger id", "return (a->id > b->id) - (a->id < b->id);",
     "return (a->id < b->id) - (a->id > b->id);",
     lambda: tto.test_topk_matches_bruteforce_with_ties("bf16", 8)),
    ("children use q_d instead of q_{d+1}",
     "front[nf].logrho = nd.logrho + lq[(int64_t)nd.depth * K + j];",
     "front[nf].logrho = nd.logrho + lq[(int64_t)(nd.depth - 1) * K + j];",
     lambda: ttr.test_best_first_order_is_global_sort(3, 3, 4, False)),
    ("depth tie-break reversed", "if (a->depth != b->depth) return a->depth < b->depth;",
     "if (a->depth != b->depth) return a->depth > b->depth;",
     lambda: ttr.test_best_first_order_is_global_sort(4, 4, 3, "degenerate")),
    ("token tie-break reversed", "if (a->token != b->token) return a->token < b->token;",
     "if (a->token != b->token) return a->token > b->token;",
     lambda: ttr.test_best_first_order_is_global_sort(4, 4, 3, True)),
    ("parent tie-break reversed", "return a->parent < b->parent;", "return a->parent > b->parent;",
     lambda: ttr.test_best_first_order_is_global_sort(4, 4, 3, "degenerate")),
    ("cost model drops the knee term", "return ca + cb * (double)n + cc * over;",
     "return ca + cb * (double)n;",
     lambda: ttr.test_stop_is_smallest_argmax_of_S("qwen3_8b_stress")),
    ("stop one node late", "if (use_stop && !(s_next > s_now))",
     "if (use_stop && !(s_next > s_now) && n > 0 && tok[n] < -5)",
     lambda: ttr.test_worked_example_cat_dog()),
    ("root not counted in A_hat", "double ahat = ahat0;", "double ahat = 0.0;",
     lambda: ttr.test_root_token_and_empty_budget()),
    ("mask misses self", "set[(size_t)i * nq_max + i] = 1;", "(void)0;",
     lambda: tma.test_mask_is_ancestor_or_self(17)),
    ("attention without scale", "sc[j] = s * scale;", "sc[j] = s;",
     lambda: tma.test_attention_matches_torch_sdpa("f32", 4, 2)),
    ("GQA head map transposed", "int g = h / group;", "int g = h % hkv;",
     lambda: tma.test_attention_matches_torch_sdpa("f32", 4, 2)),
    ("attention drops last context key", "for (int64_t j = 0; j < L; ++j) {\n                    double p",
     "for (int64_t j = 0; j + 1 < L; ++j) {\n                    double p",
     lambda: tma.test_attention_special_trees("root")),
    ("accept compares child's own target", "if (par[c] == u && tok[c] == tgt[u])",
     "if (par[c] == u && tok[c] == tgt[c])",
     lambda: tac.test_hand_built([5, 9, 0, 2, 0, 4, -1], 3, [0, 1, 3, 5], 4)),
    ("bonus from the parent of the last accepted", "bonus_token[b] = tgt[u];",
     "bonus_token[b] = tgt[u > 0 ? par[u] : 0];",
     lambda: tac.test_hand_built([5, 9, 0, 2, 0, 4, -1], 3, [0, 1, 3, 5], 4)),
    ("commit skips the root", "for (int j = 0; j <= A; ++j) {\n            int node",
     "for (int j = 1; j <= A; ++j) {\n            int node",
     lambda: tcm.test_commit_follows_greedy_chain()),
    ("commit takes the path's parent rows",
     "int node = accept_path[(int64_t)b * (block + 1) + j];",
     "int node = accept_path[(int64_t)b * (block + 1) + (j > 0 ? j - 1 : 0)];",
     lambda: tcm.test_committed_prefix_reproduces_tree_attention()),
    ("commit ignores the region end", "if (L >= region) break;", "(void)region;",
     lambda: tcm.test_commit_stops_at_the_region_end()),
    ("threshold drops a node exactly at it", "if (min_logrho < 0.0 && nd.logrho < min_logrho)",
     "if (min_logrho < 0.0 && nd.logrho <= min_logrho)",
     lambda: tse.test_threshold_is_a_prefix_of_the_global_order(0, 40)),
    ("branch cap ignored at the root", "for (int j = 0; j < nb; ++j) { /* children of the root",
     "for (int j = 0; j < K; ++j) { /* children of the root",
     lambda: tse.test_branch_cap_is_the_order_over_low_ranks(1)),
    ("rotation sign flipped", "x[j + d / 2] = x2 * c + x1 * s;", "x[j + d / 2] = x2 * c - x1 * s;",
     lambda: tly.test_rotation_is_complex_multiplication()),
    ("rotary frequencies halved", "double ang = pos * pow(rope_base, -2.0 * j / d);",
     "double ang = pos * pow(rope_base, -1.0 * j / d);",
     lambda: tly.test_rotation_is_complex_multiplication()),
    ("position ignores depth", "double pos = (double)(len + depth);", "double pos = (double)len;",
     lambda: tly.test_rotation_is_complex_multiplication()),
    ("argmax tie to the larger id", "if (acc > m1) { /* strictly larger",
     "if (acc >= m1) { /* strictly larger",
     lambda: tly.test_argmax_matches_library_product_with_ties()),
    ("attention ignores context lengths", "if (!ctx_lengths) return region;", "return region;",
     lambda: tcm.test_attention_over_context_lengths_equals_compacted()),
]


@pytest.mark.parametrize("name,old,new,pin", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(tmp_path, name, old, new, pin):
    src = open(SRC).read()
    assert src.count(old) == 1, name
    bad = tmp_path / "oracle_mut.c"
    bad.write_text(src.replace(old, new))
    lib = tmp_path / "liboracle_mut.so"
    subprocess.run(["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fPIC", "-shared", "-o",
                    str(lib), str(bad), "-lm"], check=True)
    oracle.use_library(str(lib))
    try:
        with pytest.raises((AssertionError, oracle.OracleError)):
            pin()
    finally:
        oracle.use_library(None)
