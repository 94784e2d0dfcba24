"""The balanced split-KV work plan: the C rule against an independent Python
reading of its specification, plus the invariants any valid plan must hold."""
import math

import numpy as np
import pytest

from mla_latent_kv_04_amd import _binding as B


def python_plan(seq_lens, q_len, n_h, slots, bs=64):
    """Restatement of the plan's definition (include/mla.h)."""
    rows = []
    for L in seq_lens:
        L = max(0, int(L))
        for m in range(q_len):
            rows.append(max(0, min(L, L - (q_len - 1 - m))))
    tiles = [(n + bs - 1) // bs for n in rows]
    groups = n_h // 64 if n_h % 64 == 0 else 1
    W = max(1, math.ceil(groups * sum(tiles) / slots))
    pieces, splits, slot = [], [], 0
    for r, (n, T) in enumerate(zip(rows, tiles)):
        P = max(1, math.ceil(T / W))
        if P > 1:
            splits.append((r, slot, P))
        for k in range(P):
            b0, b1 = k * T // P, (k + 1) * T // P
            pieces.append((b1 - b0, r, k, b0 * bs, min(b1 * bs, n), slot + k if P > 1 else -1))
        if P > 1:
            slot += P
    pieces.sort(key=lambda p: (-p[0], p[1], p[2]))
    work = np.array([p[1:2] + p[3:] for p in pieces], dtype=np.int32).reshape(-1, 4)
    return work, np.array(splits, dtype=np.int32).reshape(-1, 3), slot


CASES = [
    ([4096] * 64, 1, 16, 256),
    (list(np.random.default_rng(0).integers(1024, 8193, 128)), 1, 128, 256),
    ([131072] * 4, 1, 128, 256),
    ([8192], 2048, 128, 256),
    ([0, 1, 63, 64, 65, 700], 1, 128, 7),
    ([0, 0], 3, 64, 4),
    ([300, 5000], 5, 32, 3),
    ([], 1, 128, 256),
]


@pytest.mark.parametrize("lens,q_len,n_h,slots", CASES)
def test_plan_matches_specification(lens, q_len, n_h, slots):
    work, split, n_parts = B.mla_plan_decode(lens, q_len, n_h, slots)
    w2, s2, p2 = python_plan(lens, q_len, n_h, slots)
    np.testing.assert_array_equal(work, w2)
    np.testing.assert_array_equal(split, s2)
    assert n_parts == p2


@pytest.mark.parametrize("lens,q_len,n_h,slots", CASES)
def test_plan_covers_every_row_exactly_once(lens, q_len, n_h, slots):
    work, split, n_parts = B.mla_plan_decode(lens, q_len, n_h, slots)
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
    assert sorted(slots_seen) == list(range(n_parts))
    for row, first, count in split.tolist():
        assert count == len(covered[row]) > 1
    sizes = [(ke - kb + 63) // 64 for _, kb, ke, _ in work.tolist()]
    # pieces are issued longest first (sizes counted in whole blocks)
    blocks = [((ke + 63) // 64 - kb // 64) for _, kb, ke, _ in work.tolist()]
    assert blocks == sorted(blocks, reverse=True)
    del sizes


def test_plan_reports_required_capacity():
    import ctypes
    lib = B.load()
    lens = np.array([5000, 6000], dtype=np.int32)
    nw, ns, npart = ctypes.c_int32(0), ctypes.c_int32(0), ctypes.c_int32(0)
    work = np.zeros((1, 4), dtype=np.int32)
    split = np.zeros((1, 3), dtype=np.int32)
    st = lib.mla_plan_decode(lens.ctypes.data_as(ctypes.c_void_p), 2, 1, 64, 128, 4, 1,
                             work.ctypes.data_as(ctypes.c_void_p), ctypes.byref(nw),
                             split.ctypes.data_as(ctypes.c_void_p), ctypes.byref(ns),
                             ctypes.byref(npart))
    assert st == 2 and nw.value > 1
