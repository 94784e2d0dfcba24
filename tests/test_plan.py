"""The balanced split-KV schedule: the C rule against an independent Python
reading of its specification, plus the invariants any valid schedule must hold."""
import ctypes

import numpy as np
import pytest

from mla_latent_kv_04_amd import _binding as B


def python_plan(seq_lens, q_len, n_h, slots, bs=64):
    """Restatement of the schedule's definition (include/mla.h)."""
    rows = []
    for L in seq_lens:
        L = max(0, int(L))
        for m in range(q_len):
            rows.append(max(0, min(L, L - (q_len - 1 - m))))
    tiles = [(n + bs - 1) // bs for n in rows]
    starts = list(np.cumsum([0] + tiles[:-1])) if tiles else []
    N = sum(tiles)
    G = n_h // 64 if n_h % 64 == 0 else 1
    K = max(1, min(slots // G, N)) if N > 0 else 1
    bounds = [k * N // K for k in range(K + 1)]

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


@pytest.mark.parametrize("lens,q_len,n_h,slots", CASES)
def test_plan_lists_are_balanced(lens, q_len, n_h, slots):
    work, lists, split, n_parts = B.mla_plan_decode(lens, q_len, n_h, slots)
    G = n_h // 64 if n_h % 64 == 0 else 1
    K = len(lists) - 1
    assert 1 <= K <= max(1, slots // G) and lists[0] == 0 and lists[-1] == len(work)
    assert np.all(np.diff(lists) >= 0)
    blocks = []
    for k in range(K):
        items = work[lists[k]:lists[k + 1]]
        rows_k = items[:, 0].tolist()
        assert rows_k == sorted(rows_k) and len(set(rows_k)) == len(rows_k)
        blocks.append(int(sum((ke + 63) // 64 - kb // 64 for _, kb, ke, _ in items.tolist())))
    if sum(blocks) > 0:
        assert max(blocks) - min(blocks) <= 1


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
