"""Preparation steps of query-union execution, in pure Python integers.

PageWeaver (abstract; Fig. 1 and Fig. 2 captions): every query keeps a fixed
TopK page set, its *support*; a bounded search over selected-page affinity
assembles query groups, identified by original query IDs; each group's page
union is loaded once, and every member keeps exactly its own support.
CompactAttention (summary, "Approach"): unions across a chunk's Q-blocks and
across the heads that share a KV head give one KV block table per KV group.

Readings where the pages are silent (each one is listed with its reason in
the design notes):
* supports are sets: negative IDs are empty slots, duplicates collapse, and an
  ID at or beyond the page count is an error;
* supports are per (query, KV head) and grouping runs per KV head;
* the search is bounded by disjoint windows of W consecutive query IDs;
  inside a window the seed is the lowest ungrouped ID, and the group grows by
  the ungrouped candidate with the largest overlap popcount(B_c & U) with the
  group's current union U (ties to the lower ID; zero overlap still joins)
  until it has ``max_group`` members or the window is exhausted;
* union pages are listed ascending; member-mask bit j marks that the j-th
  member (in pick order) selected the page;
* page visits are the sum of union sizes and masked slots are member/page
  pairs where the member did not select the page (Fig. 2's counts).
"""
from __future__ import annotations

import itertools
from typing import List, Sequence

import numpy as np


# ---------------------------------------------------------------------------
# supports and bitsets


def supports(topk: np.ndarray, n_pages: int) -> List[List[frozenset]]:
    """topk int [n_rows, hkv, K] -> S[g][row] as frozensets of page IDs."""
    topk = np.asarray(topk)
    n_rows, hkv, _ = topk.shape
    out = []
    for g in range(hkv):
        rows = []
        for r in range(n_rows):
            ids = [int(x) for x in topk[r, g] if x >= 0]
            bad = [x for x in ids if x >= n_pages]
            if bad:
                raise ValueError(f"page id {bad[0]} >= n_pages={n_pages} (row {r}, kv head {g})")
            rows.append(frozenset(ids))
        out.append(rows)
    return out


def page_bitsets(topk: np.ndarray, n_pages: int) -> List[List[int]]:
    """bits[g][row]: Python int whose bit p is set iff page p is in the support."""
    out = []
    for rows in supports(topk, n_pages):
        out.append([sum(1 << p for p in s) for s in rows])
    return out


def n_words(n_pages: int) -> int:
    return (n_pages + 63) // 64


def bits_to_words(bits: List[List[int]], n_pages: int) -> np.ndarray:
    """Python-int bitsets -> uint64 [hkv, n_rows, ceil(n_pages/64)], bit p in word p//64."""
    w = n_words(n_pages)
    hkv, n_rows = len(bits), len(bits[0]) if bits else 0
    out = np.zeros((hkv, n_rows, w), dtype=np.uint64)
    mask = (1 << 64) - 1
    for g in range(hkv):
        for r in range(n_rows):
            b = bits[g][r]
            for k in range(w):
                out[g, r, k] = (b >> (64 * k)) & mask
    return out


# ---------------------------------------------------------------------------
# grouping


def num_groups(nq: int, window: int, max_group: int) -> int:
    """Groups per KV head: each window of W IDs yields ceil(len / max_group)."""
    total = 0
    for start in range(0, nq, window):
        n = min(window, nq - start)
        total += -(-n // max_group)
    return total


def group_affinity(bits_g: Sequence[int], window: int, max_group: int) -> List[List[int]]:
    """Bounded greedy affinity grouping of one KV head's queries.

    Returns groups as lists of original query IDs in pick order, ordered by
    window and then by creation.
    """
    nq = len(bits_g)
    groups = []
    for start in range(0, nq, window):
        remaining = list(range(start, min(start + window, nq)))
        while remaining:
            seed = remaining.pop(0)
            members = [seed]
            union = bits_g[seed]
            while len(members) < max_group and remaining:
                best, best_score = None, -1
                for c in remaining:              # ascending: first max is the lowest ID
                    score = (bits_g[c] & union).bit_count()
                    if score > best_score:
                        best, best_score = c, score
                members.append(best)
                union |= bits_g[best]
                remaining.remove(best)
            groups.append(members)
    return groups


def group_original(nq: int, max_group: int) -> List[List[int]]:
    """Original-order groups [k*max_group, (k+1)*max_group)."""
    return [list(range(s, min(s + max_group, nq))) for s in range(0, nq, max_group)]


def groups_to_arrays(groups_per_g: List[List[List[int]]], max_group: int):
    """-> group_qids int32 [hkv, n_groups, max_group] (-1 padded), group_size int32 [hkv, n_groups]."""
    hkv = len(groups_per_g)
    n_groups = len(groups_per_g[0]) if hkv else 0
    qids = np.full((hkv, n_groups, max_group), -1, dtype=np.int32)
    size = np.zeros((hkv, n_groups), dtype=np.int32)
    for g, groups in enumerate(groups_per_g):
        assert len(groups) == n_groups
        for k, members in enumerate(groups):
            qids[g, k, :len(members)] = members
            size[g, k] = len(members)
    return qids, size


# ---------------------------------------------------------------------------
# union tables and statistics


def union_tables(bits: List[List[int]], groups_per_g: List[List[List[int]]], with_qmask: bool = True):
    """Per (KV head, group), in KV-head-major then group order:

    union_off  int32 [hkv * n_groups + 1]: exclusive prefix sum of union sizes
    union_pages int32 [total]: each group's union pages, ascending
    union_qmask uint8 [total]: bit j set iff member j selected that page (if with_qmask)
    """
    sizes, pages, qmask = [], [], []
    for g, groups in enumerate(groups_per_g):
        for members in groups:
            u = 0
            for m in members:
                u |= bits[g][m]
            ps = [p for p in range(u.bit_length()) if (u >> p) & 1]
            sizes.append(len(ps))
            pages.extend(ps)
            if with_qmask:
                for p in ps:
                    qm = 0
                    for j, m in enumerate(members):
                        if (bits[g][m] >> p) & 1:
                            qm |= 1 << j
                    qmask.append(qm)
    off = np.zeros(len(sizes) + 1, dtype=np.int64)
    off[1:] = np.cumsum(sizes)
    return (off.astype(np.int32), np.asarray(pages, dtype=np.int32),
            np.asarray(qmask, dtype=np.uint8) if with_qmask else None)


def union_stats(bits: List[List[int]], groups_per_g: List[List[List[int]]]) -> dict:
    """Logical page visits and masked query-page slots (PageWeaver Fig. 2, Fig. 6)."""
    visits = slots = selected = 0
    for g, groups in enumerate(groups_per_g):
        for members in groups:
            u = 0
            for m in members:
                u |= bits[g][m]
                selected += bits[g][m].bit_count()
            n = u.bit_count()
            visits += n
            slots += n * len(members)
    masked = slots - selected
    return {"visits": visits, "slots": slots, "selected": selected, "masked": masked,
            "masked_frac": (masked / slots) if slots else 0.0}


def block_tables(mask_rows: np.ndarray, n_pages: int) -> List[List[int]]:
    """CompactAttention's per-KV-group block table: the union of every mask row
    (all Q-blocks x all heads of the group) of each KV head, ascending."""
    S = supports(mask_rows, n_pages)
    return [sorted(frozenset().union(*rows)) for rows in S]


# ---------------------------------------------------------------------------
# page-major tables (direct KV-page union)


def page_lists(bits_g: Sequence[int], n_pages: int) -> List[List[int]]:
    """For one KV head: for every page P, the ascending IDs of the queries whose
    support holds P.  This is the page-major view of the same supports that
    PageWeaver's direct KV-page union visits once per page (abstract)."""
    lists: List[List[int]] = [[] for _ in range(n_pages)]
    for q, b in enumerate(bits_g):
        p = 0
        while b:
            if b & 1:
                lists[p].append(q)
            b >>= 1
            p += 1
    return lists


def support_rank(b: int, page: int) -> int:
    """Position of ``page`` among the ascending pages of the support bitset b."""
    return bin(b & ((1 << page) - 1)).count("1")


def page_items(bits: List[List[int]], n_pages: int, chunk: int, k_max: int):
    """Work items of the page-major execution, ordered by KV head, then page, then
    position in the page's query list: each item is (g, P, members, slots), where
    members are up to ``chunk`` consecutive IDs of P's list and member q's partial
    result goes to slot (q * hkv + g) * k_max + (rank of P in S(q, g))."""
    hkv = len(bits)
    items = []
    for g, bits_g in enumerate(bits):
        lists = page_lists(bits_g, n_pages)
        for p in range(n_pages):
            qs = lists[p]
            for c in range(0, len(qs), chunk):
                members = qs[c:c + chunk]
                slots = [(q * hkv + g) * k_max + support_rank(bits_g[q], p) for q in members]
                items.append((g, p, members, slots))
    return items


def page_items_to_arrays(items, chunk: int):
    """item_kvh int32 [n], union_pages int32 [n] (the item's page), group_qids and
    out_slot int32 [n, chunk] (-1 padded), group_size int32 [n]."""
    n = len(items)
    kvh = np.array([it[0] for it in items], dtype=np.int32)
    pages = np.array([it[1] for it in items], dtype=np.int32)
    qids = np.full((n, chunk), -1, dtype=np.int32)
    slots = np.full((n, chunk), -1, dtype=np.int32)
    size = np.zeros(n, dtype=np.int32)
    for i, (_, _, members, sl) in enumerate(items):
        qids[i, :len(members)] = members
        slots[i, :len(sl)] = sl
        size[i] = len(members)
    return kvh, pages, qids, slots, size


# ---------------------------------------------------------------------------
# cascaded sharing at row-tile granularity


def arrange_for_tiles(bits_g: Sequence[int], members: Sequence[int], tile_members: int) -> List[int]:
    """QUILT's cascaded sharing (summary, "Cascaded Sharing": pages shared by a whole
    group, then sharing inside smaller subgroups) read at the granularity at which the
    attention can skip work: a row tile of ``tile_members`` members.  For a group with
    more members than one tile and at most two tiles' worth (tile_members = 4: 5..8
    members), the members are split into a first tile that holds the seed (member 0)
    and the rest, choosing the split with the smallest sum over the two tiles of
    |union of the tile's supports|; ties go to the first split in the order of
    ``itertools.combinations`` over the other members' positions.  Members keep their
    relative order inside each tile.  Other shapes are returned unchanged."""
    n = len(members)
    if tile_members != 4 or n <= tile_members or n > 2 * tile_members:
        return list(members)

    def union_size(idx):
        u = 0
        for i in idx:
            u |= bits_g[members[i]]
        return bin(u).count("1")

    best = None
    for comb in itertools.combinations(range(1, n), tile_members - 1):
        first = [0, *comb]
        rest = [i for i in range(n) if i not in first]
        cost = union_size(first) + union_size(rest)
        if best is None or cost < best[0]:
            best = (cost, first + rest)
    return [members[i] for i in best[1]]


def tile_activations(bits_g: Sequence[int], groups: List[List[int]], tile_members: int) -> int:
    """Row tiles the attention computes for one KV head: for every group and every page
    of its union, the tiles (runs of tile_members members in group order) of which at
    least one member selected the page."""
    total = 0
    for members in groups:
        for t in range(0, len(members), tile_members):
            u = 0
            for m in members[t:t + tile_members]:
                u |= bits_g[m]
            total += bin(u).count("1")
    return total


# ---------------------------------------------------------------------------
# work order of the union attention (not from the pages: a scheduling aid)


def work_order(union_sizes: Sequence[int], ranges: int = 8, cap: int = 8192) -> List[int]:
    """Start order of the attention's work items.  The n items are cut into `ranges`
    consecutive ranges of ceil(n / ranges) positions; each range lists its own items by
    union size, largest first, equal sizes by lower item index.  A range longer than
    `cap` keeps item order.  Returns order[position] = item."""
    n = len(union_sizes)
    per = -(-n // ranges) if n else 0
    order: List[int] = []
    for r in range(ranges):
        items = list(range(r * per, min(n, (r + 1) * per)))
        if len(items) <= cap:
            items.sort(key=lambda e: (-max(int(union_sizes[e]), 0), e))
        order.extend(items)
    return order
