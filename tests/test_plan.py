"""The balanced split-KV schedule: the C rule against an independent Python
reading of its specification, plus the invariants any valid schedule must hold."""
import ctypes

import numpy as np
import pytest

from mla_latent_kv_04_amd import _binding as B


SEG_COST = 8   # MLA_PLAN_SEGMENT_COST


def _row_blocks(seq_lens, q_len, bs=64):
    rows = []
    for L in seq_lens:
        L = max(0, int(L))
        for m in range(q_len):
            rows.append(max(0, min(L, L - (q_len - 1 - m))))
    return rows, [(n + bs - 1) // bs for n in rows]


def greedy_starts(tiles, W, C=SEG_COST):
    """List start positions of the greedy walk with capacity W (include/mla.h)."""
    pieces = [t for t in tiles if t > 0]
    starts, pos, i, off = [], 0, 0, 0
    while i < len(pieces):
        starts.append(pos)
        cost = 0
        while i < len(pieces):
            rest = pieces[i] - off
            if cost + C + rest <= W:
                cost += C + rest
                pos += rest
                i, off = i + 1, 0
            else:
                if W - cost - C >= 1:
                    off += W - cost - C
                    pos += W - cost - C
                break
    return starts


def python_plan(seq_lens, q_len, n_h, slots, bs=64):
    """Restatement of the schedule's definition (include/mla.h)."""
    rows, tiles = _row_blocks(seq_lens, q_len, bs)
    starts = list(np.cumsum([0] + tiles[:-1])) if tiles else []
    N = sum(tiles)
    G = n_h // 64 if n_h % 64 == 0 else 1
    K = max(1, min(slots // G, N)) if N > 0 else 1
    W = SEG_COST + 1
    if N > 0:
        hi = SEG_COST + 1 + sum(SEG_COST + t for t in tiles if t > 0)
        while W < hi:
            mid = (W + hi) // 2
            if len(greedy_starts(tiles, mid)) <= K:
                hi = mid
            else:
                W = mid + 1
    bounds = (greedy_starts(tiles, W) if N > 0 else []) + [N] * (K + 1)
    bounds = bounds[:K + 1]

    def owner(pos):
        if pos >= N:
            return K - 1
        return max(k for k in range(K) if bounds[k] <= pos)

    segs, splits, parts = [], [], 0
    for r, (n, T, S) in enumerate(zip(rows, tiles, starts)):
        if T == 0:
            segs.append((owner(S), r, 0, 0, -1))
            continue
        k0, k1 = owner(S), owner(S + T - 1)
        P = k1 - k0 + 1
        if P > 1:
            splits.append((r, parts, P))
        for k in range(k0, k1 + 1):
            t0 = max(bounds[k], S) - S
            t1 = min(bounds[k + 1], S + T) - S
            segs.append((k, r, t0 * bs, min(t1 * bs, n), parts + (k - k0) if P > 1 else -1))
        if P > 1:
            parts += P
    segs.sort(key=lambda s: (s[0], s[1]))
    work = np.array([s[1:] for s in segs], dtype=np.int32).reshape(-1, 4)
    lists = np.array([sum(1 for s in segs if s[0] < k) for k in range(K + 1)], dtype=np.int32)
    return work, lists, np.array(splits, dtype=np.int32).reshape(-1, 3), parts


CASES = [
    ([4096] * 64, 1, 16, 256),
    (list(np.random.default_rng(0).integers(1024, 8193, 128)), 1, 128, 256),
    ([131072] * 4, 1, 128, 256),
    ([8192], 2048, 128, 256),
    ([0, 1, 63, 64, 65, 700], 1, 128, 7),
    ([0, 0], 3, 64, 4),
    ([300, 5000], 5, 32, 3),
    ([0, 5000, 0, 0, 130, 0], 1, 128, 8),
    ([], 1, 128, 256),
]


@pytest.mark.parametrize("lens,q_len,n_h,slots", CASES)
def test_plan_matches_specification(lens, q_len, n_h, slots):
    work, lists, split, n_parts = B.mla_plan_decode(lens, q_len, n_h, slots)
    w2, l2, s2, p2 = python_plan(lens, q_len, n_h, slots)
    np.testing.assert_array_equal(work, w2)
    np.testing.assert_array_equal(lists, l2)
    np.testing.assert_array_equal(split, s2)
    assert n_parts == p2


@pytest.mark.parametrize("lens,q_len,n_h,slots", CASES)
def test_plan_covers_every_row_exactly_once(lens, q_len, n_h, slots):
    work, lists, split, n_parts = B.mla_plan_decode(lens, q_len, n_h, slots)
    rows = len(lens) * q_len
    covered = {r: [] for r in range(rows)}
    slots_seen = []
    for row, kb, ke, slot in work.tolist():
        assert 0 <= kb <= ke
        assert kb % 64 == 0
        covered[row].append((kb, ke))
        if slot >= 0:
            slots_seen.append(slot)
    for r in range(rows):
        L = max(0, int(lens[r // q_len]))
        n = max(0, min(L, L - (q_len - 1 - r % q_len)))
        keys = sorted(j for kb, ke in covered[r] for j in range(kb, ke))
        assert keys == list(range(n))
        assert len(covered[r]) >= 1
        # a row is written straight out iff it has one segment
        assert (len(covered[r]) == 1) == all(s < 0 for rr, _, _, s in work.tolist() if rr == r)
    assert sorted(slots_seen) == list(range(n_parts))
    for row, first, count in split.tolist():
        assert count == len(covered[row]) > 1


def _list_costs(work, lists):
    costs = []
    for k in range(len(lists) - 1):
        items = work[lists[k]:lists[k + 1]]
        blk = [(ke + 63) // 64 - kb // 64 for _, kb, ke, _ in items.tolist() if ke > kb]
        costs.append(sum(blk) + SEG_COST * len(blk))
    return costs


@pytest.mark.parametrize("lens,q_len,n_h,slots", CASES)
def test_plan_lists_are_balanced(lens, q_len, n_h, slots):
    work, lists, split, n_parts = B.mla_plan_decode(lens, q_len, n_h, slots)
    G = n_h // 64 if n_h % 64 == 0 else 1
    K = len(lists) - 1
    assert 1 <= K <= max(1, slots // G) and lists[0] == 0 and lists[-1] == len(work)
    assert np.all(np.diff(lists) >= 0)
    for k in range(K):
        rows_k = work[lists[k]:lists[k + 1], 0].tolist()
        assert rows_k == sorted(rows_k) and len(set(rows_k)) == len(rows_k)
    costs = _list_costs(work, lists)
    W = max(costs)
    if W == 0:
        return
    _, tiles = _row_blocks(lens, q_len)
    N = sum(tiles)
    # no partition into K ordered lists is cheaper: one unit less of capacity
    # needs more than K lists
    if W > SEG_COST + 1:
        assert len(greedy_starts(tiles, W - 1)) > K
    # and never costlier than equal block shares (the plain split)
    eq = [k * N // K for k in range(K + 1)]
    starts = np.cumsum([0] + tiles[:-1])
    eq_costs = []
    for k in range(K):
        segs = [(s, t) for s, t in zip(starts, tiles) if t > 0 and s < eq[k + 1] and s + t > eq[k]]
        eq_costs.append(eq[k + 1] - eq[k] + SEG_COST * len(segs))
    assert W <= max(eq_costs)


def test_plan_reports_required_capacity():
    lib = B.load()
    lens = np.array([5000, 6000], dtype=np.int32)
    nw, nl, ns, npart = (ctypes.c_int32(0) for _ in range(4))
    work = np.zeros((1, 4), dtype=np.int32)
    lists = np.zeros(5, dtype=np.int32)
    split = np.zeros((1, 3), dtype=np.int32)
    st = lib.mla_plan_decode(lens.ctypes.data_as(ctypes.c_void_p), 2, 1, 64, 128, 4, 1,
                             work.ctypes.data_as(ctypes.c_void_p), ctypes.byref(nw),
                             lists.ctypes.data_as(ctypes.c_void_p), ctypes.byref(nl),
                             split.ctypes.data_as(ctypes.c_void_p), ctypes.byref(ns),
                             ctypes.byref(npart))
    assert st == 2 and nw.value > 1
