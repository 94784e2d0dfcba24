"""C ABI checks that need no GPU: the library loads, exports every declared
entry point, rejects bad arguments before enqueuing anything, and its host
split plan matches the oracle's rule bit for bit."""
import ctypes
import os
import re

import numpy as np
import pytest

import mla_latent_kv_04_amd as pkg
from mla_latent_kv_04_amd import _binding as B
from oracle import mla_oracle as orc

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "mla.h")


@pytest.fixture(scope="module")
def lib():
    return B.load()


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int32_t|int64_t|const char\*)\s+(mla_\w+)\s*\(", text,
                                 re.M)))


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert len(names) >= 8
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(names) == sorted(B.exported_symbols())


def test_abi_version_and_status_strings(lib):
    assert lib.mla_abi_version() == 5
    for s in range(7):
        assert len(B.status_string(s)) > 0
    assert "scratch" in B.status_string(6)
    assert B.status_string(99) == "unknown status"


NULL = None
FAKE = ctypes.c_void_p(0x10000)      # aligned, never dereferenced by rejected calls
MISALIGNED = ctypes.c_void_p(0x10008)


def test_decode_rejects_bad_arguments(lib):
    call = lib.mla_decode_paged
    ok = dict(q_lat=FAKE, kv=FAKE, nblk=4, bs=64, table=FAKE, maxb=4, sl=FAKE, B=1, q_len=1,
              n_h=16, dt=1, scale=0.07, S=1, op=NULL, lp=NULL, o=FAKE, l=FAKE)

    def run(**kw):
        a = dict(ok, **kw)
        return call(a["q_lat"], a["kv"], a["nblk"], a["bs"], a["table"], a["maxb"], a["sl"],
                    a["B"], a["q_len"], a["n_h"], a["dt"], a["scale"], a["S"], a["op"], a["lp"],
                    a["o"], a["l"], None)

    assert run(dt=7) == 4
    assert run(bs=32) == 2
    assert run(n_h=48) == 2
    assert run(n_h=0) == 2
    assert run(S=0) == 2
    assert run(q_len=0) == 2
    assert run(scale=0.0) == 2
    assert run(q_lat=NULL) == 1
    assert run(o=NULL) == 1
    assert run(S=4) == 1                  # split path needs partial buffers
    assert run(q_lat=MISALIGNED) == 3
    assert run(B=0) == 0                  # nothing to do


def test_planned_decode_needs_partial_buffers_for_its_slots(lib):
    """A plan whose items write partial rows (n_parts > 0) must come with the
    partial buffers; negative counts are refused (nothing is launched)."""
    call = lib.mla_decode_paged_planned

    def run(op=FAKE, lp=FAKE, n_parts=4, n_work=3):
        return call(FAKE, FAKE, 4, 64, FAKE, 4, 2, 1, 128, 1, 0.07, FAKE, n_work, FAKE, 2,
                    op, lp, n_parts, FAKE, FAKE, None)

    assert run(op=NULL) == 1
    assert run(lp=NULL) == 1
    assert run(op=NULL, lp=NULL, n_parts=-1) == 2
    assert run(n_work=-1) == 2
    assert run(op=MISALIGNED) == 3
    assert run(n_work=0) == 0             # nothing to do


def test_noalloc_refuses_sizes_beyond_its_scratch_without_a_gpu(lib):
    """The partials of B=128, S=4, 128 heads (134 MB) exceed the fixed 64 MiB
    array: MLA_ERR_SCRATCH, decided on the host before any HIP call."""
    assert lib.mla_decode_paged_noalloc(FAKE, FAKE, 4, 64, FAKE, 4, FAKE, 128, 1, 128, 1, 0.07,
                                        4, FAKE, FAKE, None) == 6
    assert lib.mla_decode_paged_noalloc(FAKE, FAKE, 4, 64, FAKE, 4, FAKE, 1, 1, 48, 1, 0.07,
                                        2, FAKE, FAKE, None) == 2
    assert lib.mla_decode_paged_noalloc(FAKE, FAKE, 4, 64, FAKE, 4, FAKE, 1, 1, 128, 1, 0.07,
                                        2, NULL, FAKE, None) == 1


def _table(*bad):
    th = np.full(32, 0.5)
    for k, v in bad:
        th[k] = v
    return th, th.ctypes.data_as(ctypes.c_void_p)


def test_other_entry_points_reject_bad_arguments(lib):
    good, GOOD = _table()
    _, ZERO = _table((31, 0.0))
    _, NAN = _table((3, float("nan")))
    assert lib.mla_absorb_q(FAKE, FAKE, FAKE, FAKE, 4, 24, 1, 1e4, NULL, FAKE, None) == 2
    assert lib.mla_absorb_q(FAKE, FAKE, FAKE, NULL, 4, 16, 1, 1e4, NULL, FAKE, None) == 1
    assert lib.mla_absorb_q(FAKE, FAKE, FAKE, FAKE, 4, 16, 2, 1e4, NULL, FAKE, None) == 4
    assert lib.mla_absorb_q(FAKE, FAKE, MISALIGNED, FAKE, 4, 16, 1, 1e4, NULL, FAKE, None) == 3
    assert lib.mla_absorb_q(NULL, NULL, NULL, NULL, 0, 16, 1, 1e4, NULL, NULL, None) == 0
    # a table replaces the base (a bad base is then unused); a bad entry is refused
    assert lib.mla_absorb_q(NULL, NULL, NULL, NULL, 0, 16, 1, 0.0, GOOD, NULL, None) == 0
    assert lib.mla_absorb_q(NULL, NULL, NULL, NULL, 0, 16, 1, 1e4, ZERO, NULL, None) == 2
    assert lib.mla_absorb_q(NULL, NULL, NULL, NULL, 0, 16, 1, 1e4, NAN, NULL, None) == 2
    ap = lib.mla_kv_append
    assert ap(FAKE, 1, 4, 64, FAKE, 1, 4, FAKE, FAKE, FAKE, FAKE, 3, 0.0, NULL, None) == 2
    assert ap(FAKE, 1, 4, 64, NULL, 1, 4, FAKE, FAKE, FAKE, FAKE, 3, 1e4, NULL, None) == 1
    assert ap(FAKE, 1, 4, 16, FAKE, 1, 4, FAKE, FAKE, FAKE, FAKE, 3, 1e4, NULL, None) == 2
    assert ap(MISALIGNED, 1, 4, 64, FAKE, 1, 4, FAKE, FAKE, FAKE, FAKE, 3, 1e4, NULL, None) == 3
    assert ap(FAKE, 1, 4, 64, FAKE, 1, 4, FAKE, FAKE, FAKE, FAKE, 3, 1e4, ZERO, None) == 2
    assert ap(FAKE, 1, 4, 64, FAKE, 1, 4, FAKE, FAKE, FAKE, FAKE, 0, 0.0, GOOD, None) == 0
    assert lib.mla_splitkv_combine(FAKE, FAKE, 2, 0, 1, 16, FAKE, FAKE, None) == 2
    assert lib.mla_splitkv_combine(FAKE, NULL, 2, 2, 1, 16, FAKE, FAKE, None) == 1
    assert lib.mla_out_proj(FAKE, FAKE, 4, 16, 3, FAKE, None) == 4
    assert lib.mla_out_proj(NULL, FAKE, 4, 16, 1, FAKE, None) == 1
    assert lib.mla_out_proj(NULL, NULL, 0, 16, 1, NULL, None) == 0
    op = lib.mla_out_proj_planned
    assert op(FAKE, FAKE, FAKE, FAKE, 2, FAKE, 4, 16, 3, FAKE, FAKE, None) == 4   # dtype
    assert op(FAKE, FAKE, FAKE, FAKE, 5, FAKE, 4, 16, 1, FAKE, FAKE, None) == 2   # n_split > T
    assert op(FAKE, FAKE, FAKE, FAKE, -1, FAKE, 4, 16, 1, FAKE, FAKE, None) == 2
    assert op(FAKE, FAKE, FAKE, NULL, 2, FAKE, 4, 16, 1, FAKE, FAKE, None) == 1   # split
    assert op(FAKE, NULL, FAKE, FAKE, 2, FAKE, 4, 16, 1, FAKE, FAKE, None) == 1   # o_part
    assert op(FAKE, FAKE, FAKE, FAKE, 2, FAKE, 4, 16, 1, MISALIGNED, FAKE, None) == 3
    assert op(FAKE, MISALIGNED, FAKE, FAKE, 2, FAKE, 4, 16, 1, FAKE, FAKE, None) == 3
    assert op(NULL, NULL, NULL, NULL, 0, NULL, 0, 16, 1, NULL, NULL, None) == 0  # T == 0


def test_rope_theta_matches_the_oracle():
    """The library's host YaRN table against the oracle's (same float64
    formula, different code): equal to a few ulp, for DeepSeek-V2's setting and
    for settings that move every pair through the ramp."""
    for base, s, a, b, L0 in [(1e4, 40, 1, 32, 4096), (1e4, 1, 1, 32, 4096),
                              (5e5, 8, 0.5, 64, 8192), (1e4, 40, 0, 1e6, 4096)]:
        got = pkg.mla_rope_theta(base, s, a, b, L0)
        want = orc.yarn_theta(64, base, s, a, b, L0)
        np.testing.assert_allclose(got, want, rtol=4e-16, atol=0)


def test_rope_theta_rejects_bad_settings(lib):
    out = np.zeros(32)
    P = out.ctypes.data_as(ctypes.c_void_p)
    assert lib.mla_rope_theta(1e4, 40, 1, 32, 4096, NULL) == 1
    for args in [(1.0, 40, 1, 32, 4096), (1e4, 0.5, 1, 32, 4096), (1e4, 40, 32, 32, 4096),
                 (1e4, 40, -1, 32, 4096), (1e4, 40, 1, 32, 0), (float("nan"), 40, 1, 32, 4096),
                 (1e4, float("inf"), 1, 32, 4096)]:
        assert lib.mla_rope_theta(*args, P) == 2, args
    assert lib.mla_rope_theta(1e4, 40, 1, 32, 4096, P) == 0
    with pytest.raises(ValueError):
        B._theta(np.ones(31))


def test_split_plan_matches_oracle_rule():
    rng = np.random.default_rng(0)
    lens = np.concatenate([[0, 1, 63, 64, 65, 4096, 131072, 8191],
                           rng.integers(0, 9000, size=40)]).astype(np.int32)
    for S in [1, 2, 3, 7, 8, 64, 100]:
        plan = pkg.mla_split_plan(lens, S)
        for b, L in enumerate(lens):
            want = orc.split_ranges(int(L), 64, S)
            assert [tuple(x) for x in plan[b].tolist()] == want


def test_split_plan_rejects_negative_length():
    with pytest.raises(B.MLAError):
        pkg.mla_split_plan(np.array([5, -1], dtype=np.int32), 2)


def test_producers_reject_bad_arguments_and_size_their_workspace(lib):
    ws = lib.mla_kv_produce_workspace
    assert ws(128, 5120) > 0 and ws(0, 5120) == 0
    assert ws(128, 5121) == -1 and ws(-1, 5120) == -1 and ws(128, 32) == -1
    assert ws(256, 5120) >= ws(128, 5120)
    need = ws(4, 64)

    def kv(**kw):
        a = dict(h=FAKE, wd=FAKE, g=FAKE, wk=FAKE, T=4, dm=64, dt=1, eps=1e-6, base=1e4, th=NULL,
                 kv=FAKE, nb=4, bs=64, tab=FAKE, ns=1, mb=4, seq=FAKE, pos=FAKE, w=FAKE, wb=need)
        a.update(kw)
        return lib.mla_kv_produce(a["h"], a["wd"], a["g"], a["wk"], a["T"], a["dm"], a["dt"],
                                  a["eps"], a["base"], a["th"], a["kv"], a["nb"], a["bs"], a["tab"],
                                  a["ns"], a["mb"], a["seq"], a["pos"], a["w"], a["wb"], None)
    assert kv(dt=3) == 4
    assert kv(dm=48) == 2 and kv(dm=96) == 2 and kv(bs=32) == 2 and kv(eps=-1.0) == 2 and kv(base=0.0) == 2
    _, NEG = _table((0, -1.0))
    assert kv(th=NEG) == 2
    assert kv(wb=need - 1) == 2                      # workspace too small
    assert kv(h=NULL) == 1 and kv(w=NULL) == 1
    assert kv(kv=MISALIGNED) == 3
    assert kv(T=0, h=NULL, w=NULL) == 0              # nothing to do
    qws = lib.mla_q_produce_workspace
    assert qws(128, 5120, 1536, 1) > 0 and qws(128, 5120, 4096, 1) == -1
    assert qws(128, 5120, 1536, 7) == -1
    qneed = qws(4, 64, 64, 1)

    def q(**kw):
        a = dict(h=FAKE, wd=FAKE, g=FAKE, wu=FAKE, wr=FAKE, T=4, dm=64, dq=64, nh=2, dt=1,
                 eps=1e-6, qn=FAKE, qr=FAKE, w=FAKE, wb=qneed)
        a.update(kw)
        return lib.mla_q_produce(a["h"], a["wd"], a["g"], a["wu"], a["wr"], a["T"], a["dm"],
                                 a["dq"], a["nh"], a["dt"], a["eps"], a["qn"], a["qr"], a["w"],
                                 a["wb"], None)
    assert q(dt=5) == 4
    assert q(dq=40) == 2 and q(dq=96) == 2 and q(dm=160) == 2 and q(dq=4096) == 2 and q(nh=0) == 2 and q(wb=qneed - 1) == 2
    assert q(wu=NULL) == 1
    assert q(wd=MISALIGNED) == 3
    assert q(T=0, h=NULL) == 0


def test_prefill_mha_rejects_bad_arguments_and_sizes_its_workspace(lib):
    import numpy as np
    ws = lib.mla_prefill_mha_workspace
    # k^C and v^C (hi + lo) of the longest sequence, rows padded to a multiple of 256
    assert ws(8192, 128) == 3 * 128 * 128 * 8192 * 2
    assert ws(1, 16) == ws(256, 16) == 3 * 16 * 128 * 256 * 2
    assert ws(-1, 16) == -1 and ws(10, 0) == -1
    lens = np.array([300, 200], dtype=np.int32)
    need = ws(300, 16)

    def pf(**kw):
        a = dict(qn=FAKE, qr=FAKE, qp=FAKE, wk=FAKE, wv=FAKE, kv=FAKE, nb=16, bs=64, tab=FAKE,
                 mb=8, lens=lens.ctypes.data, B=2, q=100, nh=16, dt=1, sc=0.07, base=1e4,
                 th=NULL, out=FAKE, lse=FAKE, w=FAKE, wb=need)
        a.update(kw)
        return lib.mla_prefill_mha(a["qn"], a["qr"], a["qp"], a["wk"], a["wv"], a["kv"], a["nb"],
                                   a["bs"], a["tab"], a["mb"], a["lens"], a["B"], a["q"], a["nh"],
                                   a["dt"], a["sc"], a["base"], a["th"], a["out"], a["lse"], a["w"],
                                   a["wb"], None)
    assert pf(dt=0) == 4                                  # bf16 only
    _, INF = _table((7, float("inf")))
    assert pf(th=INF) == 2
    assert pf(bs=32) == 2 and pf(nh=0) == 2 and pf(sc=0.0) == 2 and pf(base=-1.0) == 2
    assert pf(mb=4) == 2                                  # 300 keys need 5 blocks of 64
    assert pf(wb=need - 1) == 2
    assert pf(nb=1 << 20) == 2                            # cache beyond 32-bit offsets
    assert pf(lens=None) == 1 and pf(wk=NULL) == 1 and pf(lse=NULL) == 1
    assert pf(out=MISALIGNED) == 3
    assert pf(B=0, lens=None) == 0 and pf(q=0) == 0       # nothing to do


def test_direct_query_producer_rejects_bad_arguments(lib):
    def q(**kw):
        a = dict(h=FAKE, wc=FAKE, wr=FAKE, T=4, dm=64, nh=2, dt=1, qn=FAKE, qr=FAKE)
        a.update(kw)
        return lib.mla_q_produce_direct(a["h"], a["wc"], a["wr"], a["T"], a["dm"], a["nh"],
                                        a["dt"], a["qn"], a["qr"], None)
    assert q(dt=9) == 4
    assert q(dm=96) == 2 and q(nh=0) == 2 and q(T=-1) == 2
    assert q(wr=NULL) == 1 and q(qn=NULL) == 1
    assert q(qr=MISALIGNED) == 3
    assert q(T=0, h=NULL) == 0


def test_o_proj_rejects_bad_arguments_and_sizes_its_workspace(lib):
    ws = lib.mla_o_proj_workspace
    assert ws(128, 128, 5120, 1) >= 128 * 128 * 128 * 2        # the bf16 copy of the outputs
    assert ws(128, 128, 5120, 7) == -1 and ws(128, 0, 5120, 1) == -1 and ws(128, 128, 100, 1) == -1
    need = ws(4, 2, 64, 1)

    def o(**kw):
        a = dict(out=FAKE, w=FAKE, T=4, nh=2, dm=64, dt=1, u=FAKE, ws=FAKE, wb=need)
        a.update(kw)
        return lib.mla_o_proj(a["out"], a["w"], a["T"], a["nh"], a["dm"], a["dt"], a["u"], a["ws"],
                              a["wb"], None)
    assert o(dt=3) == 4
    assert o(dm=96) == 2 and o(nh=0) == 2 and o(wb=need - 1) == 2
    assert o(w=NULL) == 1 and o(u=NULL) == 1
    assert o(out=MISALIGNED) == 3
    assert o(T=0, out=NULL) == 0
