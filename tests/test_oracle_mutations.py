"""The pins bite: plant a plausible mistake in the oracle (CPU only) and check
that at least one pin test fails on it.

Each mutation edits one line of an oracle function's source, re-executes it
in a copy of its module namespace and patches it in for the duration of the
pin; the real oracle is untouched afterwards.
"""
import inspect
import textwrap

import pytest

import test_oracle_attention as A
import test_oracle_kvcache as K
import test_oracle_numerics as N
import test_oracle_prep as P
from oracle import attention, kvcache, numerics, prep


def _mutant(module, fn_name, old, new):
    src = textwrap.dedent(inspect.getsource(getattr(module, fn_name)))
    assert old in src, (fn_name, old)
    ns = dict(vars(module))
    exec(compile(src.replace(old, new, 1), module.__file__, "exec"), ns)
    return ns[fn_name]


MUTATIONS = [
    # (module, function, original text, planted mistake, pin that must fail)
    (attention, "route_a", "t <= int(q_pos[i])", "t < int(q_pos[i])",
     lambda: A.test_route_a_equals_brute_force("bf16", 0)),
    (attention, "route_a", "sm_scale * (qh @ kk.T)", "(qh @ kk.T)",
     lambda: A.test_route_a_equals_brute_force("bf16", 0)),
    (attention, "route_a", "q_bits[i, g * G:(g + 1) * G]", "q_bits[i, g:g + G]",
     lambda: A.test_dense_support_equals_library_attention("bf16")),
    (attention, "route_a", "(t < kv_len)", "(t <= kv_len)",
     lambda: A.test_dense_support_positions_past_cache_end()),
    (attention, "route_a", "Kg[pages].reshape(-1, d)[keep]", "Kg[pages].reshape(-1, d)[::-1][keep]",
     lambda: A.test_route_a_equals_brute_force("fp8", 1)),
    (attention, "_softmax_pv", "(e @ v) / l", "(e @ v)",
     lambda: A.test_closed_form_zero_query_is_mean()),
    (attention, "route_b", "sel & (t <= int(q_pos[m]))", "(t <= int(q_pos[m]))",
     lambda: A.test_grouping_invariance_route_b("bf16")),
    (numerics, "e4m3fn_value", "e - 7", "e - 8",
     lambda: N.test_e4m3fn_special_values()),
    (prep, "group_affinity", "score > best_score", "score >= best_score",
     lambda: P.test_fig2_printed_counts()),
    (prep, "group_affinity", "(bits_g[c] & union)", "(bits_g[c] & bits_g[seed])",
     lambda: P.test_group_hand_trace_union_not_seed()),
    (prep, "group_affinity", "seed = remaining.pop(0)", "seed = remaining.pop()",
     lambda: P.test_group_special_cases()),
    (prep, "union_stats", "slots += n * len(members)", "slots += n",
     lambda: P.test_fig2_printed_counts()),
    (prep, "union_tables", "qm |= 1 << j", "qm |= 1 << (len(members) - 1 - j)",
     lambda: P.test_union_tables_set_algebra()),
    (attention, "route_c", "(w[:, :, None] * outs).sum(axis=0)", "outs.sum(axis=0)",
     lambda: A.test_direct_page_union_route_c_equals_definition("bf16")),
    (attention, "route_c", "keep = (t <= int(q_pos[i])) & (t < kv_len)", "keep = (t < kv_len)",
     lambda: A.test_direct_page_union_route_c_equals_definition("fp8")),
    (attention, "_route_a_batch", "(t <= pos[:, None, None])", "(t < pos[:, None, None])",
     lambda: A.test_route_a_batched_equals_route_a("bf16", 5, 2)),
    (attention, "_route_a_batch", "(pages[:, :, None] >= 0) & ", "",
     lambda: A.test_route_a_batched_equals_route_a("fp8", 64, 3)),
    (attention, "_route_a_batch", "q_bits[ids, g * G:(g + 1) * G]", "q_bits[ids, g:g + G]",
     lambda: A.test_route_a_batched_equals_route_a("bf16", 1, 1)),
    (attention, "_route_a_batch", "& (t < kv_len)", "& (t <= kv_len)",
     lambda: A.test_route_a_batched_equals_route_a("bf16", 64, 3)),
    (attention, "_route_a_batch", "pages = np.asarray(sorted(sets[0]), dtype=np.int64)[None, :]",
     "pages = np.asarray(sorted(sets[0]), dtype=np.int64)[None, 1:]",
     lambda: A.test_route_a_batched_shared_table_equals_route_a()),
    (prep, "page_items", "support_rank(bits_g[q], p)", "support_rank(bits_g[q], p + 1)",
     lambda: P.test_page_items_hand_trace()),
    (prep, "page_items", "range(0, len(qs), chunk)", "range(0, len(qs), chunk + 1)",
     lambda: P.test_page_items_cover_every_edge_once()),
    (prep, "arrange_for_tiles", "cost < best[0]", "cost <= best[0]",
     lambda: P.test_arrange_for_tiles_hand_trace()),
    (prep, "arrange_for_tiles", "union_size(first) + union_size(rest)", "union_size(first)",
     lambda: P.test_arrange_for_tiles_is_the_brute_force_minimum()),
    (kvcache, "e4m3fn_encode", "(hi % 2 == 0)", "(hi % 2 == 1)",
     lambda: K.test_encode_ties_go_to_even_code()),
    (kvcache, "quantize", "/ np.float32(scale)", "* np.float32(scale)",
     lambda: K.test_full_append_matches_generator_quantisation()),
    (kvcache, "_append_one", "s1 = min(last - base, ps - 1) + 1", "s1 = min(last - base, ps - 1)",
     lambda: K.test_full_append_matches_generator_quantisation()),
    (kvcache, "_append_one", "astype(np.float32) * s_old", "astype(np.float32) * s_new",
     lambda: K.test_scale_growth_reencodes_earlier_slots()),
    (kvcache, "_append_one", "if s_new > s_old:", "if s_new < s_old:",
     lambda: K.test_scale_kept_when_chunk_is_smaller()),
    (prep, "work_order", "(-max(int(union_sizes[e]), 0), e)", "(max(int(union_sizes[e]), 0), e)",
     lambda: P.test_work_order_hand_trace()),
    (prep, "work_order", "(-max(int(union_sizes[e]), 0), e)", "(-max(int(union_sizes[e]), 0), -e)",
     lambda: P.test_work_order_is_the_brute_force_order(0)),
    (prep, "work_order", "per = -(-n // ranges) if n else 0", "per = n // ranges if n else 0",
     lambda: P.test_work_order_hand_trace()),
]


@pytest.mark.parametrize("module,fn,old,new,pin", MUTATIONS,
                         ids=[f"{m[1]}:{m[3]}" for m in MUTATIONS])
def test_pin_catches_planted_mistake(monkeypatch, module, fn, old, new, pin):
    monkeypatch.setattr(module, fn, _mutant(module, fn, old, new))
    if module is numerics and fn == "e4m3fn_value":
        monkeypatch.setattr(numerics, "E4M3FN_TABLE",
                            numerics.np.array([numerics.e4m3fn_value(c) for c in range(256)]))
    with pytest.raises(AssertionError):
        pin()
