"""Pins for the oracle's preparation steps: bitsets, grouping, union tables, statistics.

The printed pin is PageWeaver's Fig. 2 caption (fixture under tests/golden);
the rest are hand traces, special cases, invariants, a brute-force optimality
check of every greedy pick and set algebra written independently of the
oracle's bit arithmetic.
"""
import itertools
import os
import random

import numpy as np
import pytest

from oracle import prep
from helpers import tiny_workload

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load_fig2():
    spec = {"support": {}}
    with open(os.path.join(GOLDEN, "fig2_regrouping.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            if key == "support":
                spec["support"][int(vals[0])] = [int(v) for v in vals[1:]]
            elif key == "regrouped_groups":
                spec[key] = [[int(x) for x in v.split(",")] for v in vals]
            else:
                spec[key] = int(vals[0])
    nq = len(spec["support"])
    topk = np.array([[spec["support"][i]] for i in range(nq)], dtype=np.int32)  # [nq, 1, 2]
    return spec, topk


def test_fig2_printed_counts():
    spec, topk = load_fig2()
    bits = prep.page_bitsets(topk, spec["n_pages"])
    nq = topk.shape[0]
    orig = [prep.group_original(nq, spec["max_group"])]
    aff = [prep.group_affinity(bits[0], spec["window"], spec["max_group"])]
    s_orig = prep.union_stats(bits, orig)
    s_aff = prep.union_stats(bits, aff)
    assert s_orig["visits"] == spec["original_visits"]
    assert s_orig["masked"] == spec["original_masked"]
    assert s_aff["visits"] == spec["regrouped_visits"]
    assert s_aff["masked"] == spec["regrouped_masked"]
    assert s_orig["selected"] == s_aff["selected"] == spec["selected_edges"]
    assert aff[0] == spec["regrouped_groups"]


def _sets(topk, g=0):
    return [frozenset(int(x) for x in row if x >= 0) for row in topk[:, g]]


def test_bitsets_match_sets_and_words():
    rng = np.random.default_rng(1)
    n_pages = 150
    topk = rng.integers(-3, n_pages, size=(40, 3, 12)).astype(np.int32)
    topk[:, :, 5] = topk[:, :, 4]                                 # duplicates collapse
    bits = prep.page_bitsets(topk, n_pages)
    words = prep.bits_to_words(bits, n_pages)
    assert words.shape == (3, 40, 3)
    for g in range(3):
        for i, s in enumerate(_sets(topk, g)):
            got = {p for p in range(n_pages) if (int(words[g, i, p // 64]) >> (p % 64)) & 1}
            assert got == set(s)


def test_bitsets_reject_out_of_range():
    topk = np.array([[[0, 5]]], dtype=np.int32)
    with pytest.raises(ValueError):
        prep.page_bitsets(topk, 5)


def test_num_groups():
    assert prep.num_groups(256, 64, 8) == 32
    assert prep.num_groups(70, 64, 8) == 8 + 1
    assert prep.num_groups(75, 64, 8) == 8 + 2
    assert prep.num_groups(5, 64, 8) == 1
    assert prep.num_groups(0, 64, 8) == 0


def _bits_of(sets):
    return [sum(1 << p for p in s) for s in sets]


def test_group_hand_trace():
    # window of 6, groups of 3.
    # 0:{1,2,3} 1:{7} 2:{2,3} 3:{1,9} 4:{7,8} 5:{3}
    # seed 0, U={1,2,3}: overlaps 1:0 2:2 3:1 4:0 5:1 -> 2; U={1,2,3}
    #   overlaps 1:0 3:1 4:0 5:1 -> 3 (tie with 5, lower ID); group (0,2,3)
    # seed 1, U={7}: 4:1 5:0 -> 4; then 5 (only one left); group (1,4,5)
    sets = [{1, 2, 3}, {7}, {2, 3}, {1, 9}, {7, 8}, {3}]
    assert prep.group_affinity(_bits_of(sets), 6, 3) == [[0, 2, 3], [1, 4, 5]]


def test_group_hand_trace_union_not_seed():
    # The score is overlap with the current union, not with the seed.
    # seed 0={1}; 1={6} 2={1,5} 3={5}: pick 2 (overlap 1), U={1,5};
    # then 3 (overlap 1 via page 5) beats 1 (0).  Scoring against the seed
    # alone would tie 1 and 3 at 0 and take 1.
    sets = [{1}, {6}, {1, 5}, {5}]
    assert prep.group_affinity(_bits_of(sets), 4, 3) == [[0, 2, 3], [1]]


def test_group_special_cases():
    same = _bits_of([{1, 2}] * 19)
    assert prep.group_affinity(same, 8, 4) == [[0, 1, 2, 3], [4, 5, 6, 7], [8, 9, 10, 11],
                                                [12, 13, 14, 15], [16, 17, 18]]
    disjoint = _bits_of([{i} for i in range(10)])
    assert prep.group_affinity(disjoint, 8, 3) == [[0, 1, 2], [3, 4, 5], [6, 7], [8, 9]]
    assert prep.group_original(10, 4) == [[0, 1, 2, 3], [4, 5, 6, 7], [8, 9]]


def _check_greedy_optimal(sets, groups, window, max_group):
    """Every pick is the argmax over the candidates still free at that moment."""
    nq = len(sets)
    for start in range(0, nq, window):
        free = list(range(start, min(start + window, nq)))
        wgroups = [g for g in groups if start <= g[0] < start + window]
        for members in wgroups:
            assert members[0] == min(free)
            free.remove(members[0])
            union = set(sets[members[0]])
            for c in members[1:]:
                best = max(len(sets[x] & union) for x in free)
                assert len(sets[c] & union) == best
                assert c == min(x for x in free if len(sets[x] & union) == best)
                free.remove(c)
                union |= sets[c]
            assert len(members) == max_group or not free
        assert not free


@pytest.mark.parametrize("seed", range(6))
def test_group_invariants_and_bruteforce(seed):
    rng = random.Random(seed)
    nq = rng.randint(1, 90)
    window = rng.choice([8, 16, 64])
    max_group = rng.choice([m for m in (1, 2, 4, 8) if window % m == 0])
    sets = [frozenset(rng.sample(range(40), rng.randint(0, 6))) for _ in range(nq)]
    groups = prep.group_affinity(_bits_of(sets), window, max_group)
    flat = sorted(q for g in groups for q in g)
    assert flat == list(range(nq))                                    # partition
    assert all(1 <= len(g) <= max_group for g in groups)
    assert all(len({q // window for q in g}) == 1 for g in groups)    # never crosses a window
    assert len(groups) == prep.num_groups(nq, window, max_group)
    _check_greedy_optimal(sets, groups, window, max_group)


def test_union_tables_set_algebra():
    rng = random.Random(3)
    hkv, nq, n_pages, mg = 2, 37, 130, 4
    S = [[frozenset(rng.sample(range(n_pages), rng.randint(0, 9))) for _ in range(nq)] for _ in range(hkv)]
    bits = [_bits_of(s) for s in S]
    groups = [prep.group_affinity(b, 16, mg) for b in bits]
    off, pages, qmask = prep.union_tables(bits, groups)
    e = 0
    for g in range(hkv):
        for members in groups[g]:
            union = sorted(frozenset().union(*(S[g][m] for m in members)))
            assert list(pages[off[e]:off[e + 1]]) == union
            for k, p in enumerate(union):
                want = sum(1 << j for j, m in enumerate(members) if p in S[g][m])
                assert qmask[off[e] + k] == want
            e += 1
    assert off[0] == 0 and off[-1] == len(pages)
    distinct = sum(len(frozenset().union(*S[g])) for g in range(hkv))
    assert off[-1] >= distinct


def test_stats_definitions():
    S = [[{0, 1}, {1, 2}, {5}]]
    bits = [_bits_of(S[0])]
    st = prep.union_stats(bits, [[[0, 1], [2]]])
    assert st == {"visits": 3 + 1, "slots": 3 * 2 + 1, "selected": 5, "masked": 2,
                  "masked_frac": 2 / 7}


def test_block_tables_union():
    rows = np.array([[[0, 3, -1]], [[3, 7, 9]], [[-1, -1, 2]]], dtype=np.int32)
    assert prep.block_tables(rows, 10) == [[0, 2, 3, 7, 9]]


def test_page_lists_hand_trace():
    # query 0: pages {0, 2}; query 1: {2}; query 2: {}; query 3: {0, 1, 2}
    bits = [0b101, 0b100, 0, 0b111]
    assert prep.page_lists(bits, 4) == [[0, 3], [3], [0, 1, 3], []]
    assert [prep.support_rank(0b111, p) for p in range(3)] == [0, 1, 2]
    assert prep.support_rank(0b101, 2) == 1


def test_page_items_hand_trace():
    bits = [[0b101, 0b100, 0, 0b111], [0b10, 0, 0, 0]]     # two KV heads, 4 queries
    items = prep.page_items(bits, 4, chunk=2, k_max=3)
    # head 0: page 0 -> [0, 3]; page 1 -> [3]; page 2 -> [0, 1] and [3]; head 1: page 1 -> [0]
    assert [(g, p, m) for g, p, m, _ in items] == [
        (0, 0, [0, 3]), (0, 1, [3]), (0, 2, [0, 1]), (0, 2, [3]), (1, 1, [0])]
    # slot = (q * hkv + g) * k_max + rank
    assert [s for *_, s in items] == [[0, 18], [19], [1, 6], [20], [3]]


def test_page_items_cover_every_edge_once():
    w = tiny_workload(hq=4, hkv=2, ps=4, kv_len=120, nq=33, k=6, seed=21)
    c = w.cfg
    bits = prep.page_bitsets(w.topk, c.n_pages)
    S = prep.supports(w.topk, c.n_pages)
    k_max = w.topk.shape[2]
    for chunk in (1, 3, 8):
        items = prep.page_items(bits, c.n_pages, chunk, k_max)
        edges = [(g, q, p) for g, p, members, _ in items for q in members]
        assert len(edges) == len(set(edges)) == sum(len(s) for Sg in S for s in Sg)
        assert set(edges) == {(g, q, p) for g in range(c.hkv) for q in range(c.nq) for p in S[g][q]}
        slots = [s for *_, sl in items for s in sl]
        assert len(set(slots)) == len(slots) and max(slots) < c.nq * c.hkv * k_max
        for g, p, members, sl in items:
            assert 1 <= len(members) <= chunk and members == sorted(members)
            for q, s in zip(members, sl):
                assert s == (q * c.hkv + g) * k_max + sorted(S[g][q]).index(p)


def test_arrange_for_tiles_hand_trace():
    # members 0..7; pages: 0,2,4,6 share page 10; 1,3,5,7 share page 11; everyone has page 0
    bits = [(1 << 0) | (1 << (10 + (q % 2))) for q in range(8)]
    members = list(range(8))
    arr = prep.arrange_for_tiles(bits, members, 4)
    assert arr == [0, 2, 4, 6, 1, 3, 5, 7]
    assert prep.tile_activations(bits, [arr], 4) == 4            # {0,10} + {0,11}
    assert prep.tile_activations(bits, [members], 4) == 6        # {0,10,11} twice
    # ties (identical supports) keep the first split in combination order: no change
    assert prep.arrange_for_tiles([5] * 8, members, 4) == members
    # small groups and other tile sizes are left alone
    assert prep.arrange_for_tiles(bits, [3, 1, 2], 4) == [3, 1, 2]
    assert prep.arrange_for_tiles(bits, members, 2) == members


def test_arrange_for_tiles_is_the_brute_force_minimum():
    import itertools
    rng = random.Random(3)
    for n in range(5, 9):
        for trial in range(20):
            bits = [rng.getrandbits(24) & rng.getrandbits(24) for _ in range(n)]
            members = list(range(n))
            arr = prep.arrange_for_tiles(bits, members, 4)
            assert sorted(arr) == members and arr[0] == 0
            best = min(prep.tile_activations(bits, [[0, *c] + [i for i in range(1, n) if i not in c]], 4)
                       for c in itertools.combinations(range(1, n), 3))
            assert prep.tile_activations(bits, [arr], 4) == best
            # relative order kept inside each tile
            assert arr[:4] == sorted(arr[:4]) and arr[4:] == sorted(arr[4:])


def test_work_order_hand_trace():
    # ranges of ceil(9 / 3) = 3: sizes (3,5,5) -> 1,2,0; (1,9,2) -> 4,5,3; (2,7,4) -> 7,8,6
    assert prep.work_order([3, 5, 5, 1, 9, 2, 2, 7, 4], ranges=3) == [1, 2, 0, 4, 5, 3, 7, 8, 6]
    assert prep.work_order([4, 1, 7, 2, 2], ranges=8) == [0, 1, 2, 3, 4]      # one item per range
    assert prep.work_order([1, 2, 3, 4], ranges=1, cap=3) == [0, 1, 2, 3]     # longer than cap
    assert prep.work_order([], ranges=8) == []


@pytest.mark.parametrize("seed", range(6))
def test_work_order_is_the_brute_force_order(seed):
    """Each range, by exhaustive search: the arrangement of its items whose size sequence is
    non-increasing with equal sizes in increasing item order is unique and is the one."""
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 30))
    ranges = int(rng.integers(1, 9))
    sizes = [int(x) for x in rng.integers(0, 4, size=n)]
    order = prep.work_order(sizes, ranges=ranges)
    assert sorted(order) == list(range(n))
    per = -(-n // ranges)
    for r in range(ranges):
        items = list(range(r * per, min(n, (r + 1) * per)))
        if not items:
            continue
        got = order[r * per:r * per + len(items)]
        if len(items) <= 6:
            valid = [p for p in itertools.permutations(items)
                     if all((sizes[a], -a) > (sizes[b], -b) for a, b in zip(p, p[1:]))]
            assert valid == [tuple(got)]
        assert sorted(got) == items
        assert all(sizes[a] > sizes[b] or (sizes[a] == sizes[b] and a < b) for a, b in zip(got, got[1:]))
