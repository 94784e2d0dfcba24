"""Pins of the float64 CPU oracle against facts it does not itself compute.

Every test here runs on the CPU.  Each pin targets a plausible mistake in the
oracle: a dropped term (brute force, L = 1, q = 0), a wrong sign or pairing in
RoPE (complex-number form, relative-position property), a transposed weight
(non-square tiny shapes, absorbed == non-absorbed), a wrong scale or softmax
(library attention, rows summing to one) and a wrong merge (split combine).
"""
import cmath
import json
import math
import os

import numpy as np
import pytest

from oracle import mla_oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "deepseek_v2_dims.json")


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _tiny(seed=0, L=5, n_h=2, d_h=4, d_c=8, d_r=4, M=1):
    rng = np.random.default_rng(seed)
    return dict(
        c_kv=_rand(rng, L, d_c), k_r=_rand(rng, L, d_r),
        q_nope=_rand(rng, M, n_h, d_h), q_rope=_rand(rng, M, n_h, d_r),
        w_uk=_rand(rng, n_h, d_h, d_c) / math.sqrt(d_c),
        w_uv=_rand(rng, n_h, d_h, d_c) / math.sqrt(d_c),
    )


# --------------------------------------------------------------------------- RoPE

def _rope_complex(x, pos, base):
    """RoPE written with complex numbers: pair k is the complex number
    x[2k] + i x[2k+1], multiplied by exp(i pos theta_k), theta_k = base^(-2k/d)."""
    d = len(x)
    out = []
    for k in range(d // 2):
        z = complex(x[2 * k], x[2 * k + 1]) * cmath.exp(1j * pos * base ** (-2.0 * k / d))
        out += [z.real, z.imag]
    return np.array(out)


def test_rope_matches_complex_form():
    rng = np.random.default_rng(1)
    for pos in [0, 1, 7, 1000, 131071]:
        x = rng.standard_normal(64)
        np.testing.assert_allclose(orc.rope_rotate(x, pos, 10000.0),
                                   _rope_complex(x, pos, 10000.0), rtol=0,
                                   atol=1e-12 * max(1, pos))   # angle ulp grows with pos


def test_rope_position_zero_is_identity_and_norm_is_kept():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((3, 64))
    np.testing.assert_array_equal(orc.rope_rotate(x, np.zeros(3), 10000.0), x)
    y = orc.rope_rotate(x, np.array([5, 4096, 131071]), 10000.0)
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)


def test_rope_first_pair_turns_by_pos_radians():
    # theta_0 = base^0 = 1: the first pair of e_0 lands on (cos p, sin p).
    e0 = np.zeros(8)
    e0[0] = 1.0
    for p in [1, 2, 3, 100]:
        y = orc.rope_rotate(e0, p, 10000.0)
        np.testing.assert_allclose(y[:2], [math.cos(p), math.sin(p)], atol=1e-14)
        assert np.all(y[2:] == 0)


def test_rope_scores_depend_on_relative_position_only():
    # blog §2.2.2: (R_m q)^T (R_n k) = q^T R_{n-m} k depends on n - m only.
    rng = np.random.default_rng(3)
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    for m, n in [(0, 5), (17, 300), (1000, 999)]:
        ref = orc.rope_rotate(q, m, 10000.0) @ orc.rope_rotate(k, n, 10000.0)
        for shift in [1, 123, 65536]:
            got = orc.rope_rotate(q, m + shift, 10000.0) @ orc.rope_rotate(k, n + shift, 10000.0)
            assert abs(got - ref) < 1e-9 * (1 + abs(ref))


def test_rope_composes_additively():
    rng = np.random.default_rng(4)
    x = rng.standard_normal(64)
    np.testing.assert_allclose(orc.rope_rotate(orc.rope_rotate(x, 300, 1e4), 45, 1e4),
                               orc.rope_rotate(x, 345, 1e4), atol=1e-12)


# ------------------------------------------------------------------------ YaRN

YARN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "yarn_v2.json")))


def _yarn_v2(d=64, base=10000.0):
    return orc.yarn_theta(d, base, YARN["scale"], YARN["alpha"], YARN["beta"],
                          YARN["original_context"])


def test_yarn_fixture_is_consistent_with_the_stated_context():
    # 4K window times scale 40 is the stated 160K target (160 x 1024).
    assert YARN["original_context"] * YARN["scale"] == YARN["target_context"] == 160 * 1024
    assert YARN["trained_context"] == 128 * 1024 <= YARN["target_context"]


def test_yarn_scale_one_is_plain_rope():
    for d, base in [(64, 10000.0), (16, 500.0)]:
        np.testing.assert_allclose(orc.yarn_theta(d, base, 1.0, 1.0, 32.0, 4096),
                                   orc.rope_theta(d, base), rtol=1e-15, atol=0)
    x = np.random.default_rng(40).standard_normal(64)
    th = orc.yarn_theta(64, 1e4, 1.0, 1.0, 32.0, 4096)
    np.testing.assert_allclose(orc.rope_rotate(x, 777, 1e4, th), orc.rope_rotate(x, 777, 1e4),
                               atol=1e-12)


def test_yarn_keeps_fast_pairs_and_divides_slow_pairs_by_the_scale():
    # With base 1e4, d 64 and a 4096-token window, pair k turns
    # 4096 * 1e4^(-k/32) / (2 pi) times: 651.9 for k = 0, 0.087 for k = 31.
    d, base, L0, s = 64, 1e4, YARN["original_context"], YARN["scale"]
    th, yth = orc.rope_theta(d, base), _yarn_v2(d, base)
    turns = [L0 * base ** (-2.0 * k / d) / (2 * math.pi) for k in range(d // 2)]
    assert abs(turns[0] - 651.898646) < 1e-5 and abs(turns[31] - 0.0869) < 1e-4
    n_fast = n_slow = 0
    for k in range(d // 2):
        if turns[k] >= YARN["beta"]:
            assert yth[k] == th[k]
            n_fast += 1
        elif turns[k] <= YARN["alpha"]:
            assert abs(yth[k] - th[k] / s) <= 1e-16 * th[k]
            n_slow += 1
        else:
            assert th[k] / s < yth[k] < th[k]
    # 651.9 * 10^(-k/8) >= 32 for k <= 10 and <= 1 for k >= 23: eleven pairs
    # keep their frequency, nine are divided by s, twelve sit on the ramp
    assert (n_fast, n_slow) == (11, 9)


def test_yarn_ramp_endpoints_and_midpoint():
    # d = 2 has the single pair theta_0 = 1, which turns L0 / (2 pi) times:
    # choosing L0 puts it anywhere on the ramp between alpha and beta.
    a, b, s = 1.0, 32.0, 40.0
    for turns, want in [(a, 1.0 / s), (b, 1.0), ((a + b) / 2, 0.5 + 0.5 / s),
                        (a + 0.25 * (b - a), 0.25 + 0.75 / s), (0.5, 1.0 / s), (100.0, 1.0)]:
        got = orc.yarn_theta(2, 1e4, s, a, b, 2 * math.pi * turns)
        assert abs(got[0] - want) < 1e-15, (turns, got, want)


def test_yarn_ratio_falls_monotonically_with_the_pair_index():
    th, yth = orc.rope_theta(64, 1e4), _yarn_v2()
    ratio = yth / th
    assert np.all(np.diff(ratio) <= 1e-15) and np.any(np.diff(ratio) < -1e-3)
    assert ratio[0] == 1.0 and abs(ratio[-1] - 1.0 / YARN["scale"]) < 1e-15


def test_yarn_slow_pairs_at_scaled_position_match_plain_rope():
    # Interpolation: a pair divided by s turns at position s*p exactly as the
    # plain pair turns at p, so positions up to s * 4096 stay inside the
    # angles seen in training for those pairs.
    d, s = 64, YARN["scale"]
    th, yth = orc.rope_theta(d, 1e4), _yarn_v2(d)
    slow = np.flatnonzero(np.abs(yth - th / s) <= 1e-16 * th)
    fast = np.flatnonzero(yth == th)
    x = np.random.default_rng(41).standard_normal(d)
    for p in [1, 100, 4095]:
        y_ext = orc.rope_rotate(x, s * p, 1e4, yth).reshape(-1, 2)
        y_pln = orc.rope_rotate(x, p, 1e4).reshape(-1, 2)
        y_far = orc.rope_rotate(x, s * p, 1e4).reshape(-1, 2)
        np.testing.assert_allclose(y_ext[slow], y_pln[slow], atol=1e-10)
        np.testing.assert_allclose(y_ext[fast], y_far[fast], atol=1e-10)


def test_yarn_attention_is_shift_invariant_and_absorbs():
    # One frequency table rotates queries and keys together, so a common shift
    # of all positions leaves every output unchanged; and the absorbed chain
    # with that table equals the non-absorbed form.
    t = _tiny(seed=42, L=7, n_h=3, d_h=4, d_c=8, d_r=64, M=2)
    th = _yarn_v2()
    kp, qp, vis, sc = np.arange(7), np.array([5, 6]), np.array([6, 7]), 0.3
    o, l, _ = orc.mla_attention_naive(**t, key_pos=kp, q_pos=qp, n_visible=vis, scale=sc,
                                      base=1e4, theta=th)
    o2, l2, _ = orc.mla_attention_naive(**t, key_pos=kp + 50000, q_pos=qp + 50000, n_visible=vis,
                                     scale=sc, base=1e4, theta=th)
    np.testing.assert_allclose(o2, o, atol=1e-9)
    np.testing.assert_allclose(l2, l, atol=1e-9)
    o3, _, _ = orc.mla_attention_naive(**t, key_pos=kp, q_pos=qp, n_visible=vis, scale=sc, base=1e4)
    assert np.max(np.abs(o3 - o)) > 1e-6          # the table does change the result
    q_lat = orc.absorb_query(t["q_nope"], t["q_rope"], t["w_uk"], qp, 1e4, th)
    rows = orc.kv_cache_rows(t["c_kv"], t["k_r"], kp, 1e4, th)
    o_lat, l4 = orc.latent_attention(q_lat, rows, vis, sc, 8)
    np.testing.assert_allclose(orc.out_projection(o_lat, t["w_uv"]), o, atol=1e-12)
    np.testing.assert_allclose(l4, l, atol=1e-12)


def test_rope_rejects_a_table_of_the_wrong_length():
    with pytest.raises(ValueError):
        orc.rope_rotate(np.zeros(8), 1, 1e4, np.ones(3))


# ------------------------------------------------------------ brute-force naive MLA

def _brute_force(c_kv, k_r, q_nope, q_rope, w_uk, w_uv, key_pos, q_pos, n_vis, scale, base):
    """Scalar loops in float64: eq. 10/11 per element, RoPE in complex form,
    softmax with math.exp."""
    M, n_h, d_h = q_nope.shape
    L, d_c = c_kv.shape
    out = np.zeros((M, n_h, d_h))
    lse = np.full((M, n_h), -math.inf)
    for m in range(M):
        qr_all = [_rope_complex(q_rope[m, i], q_pos[m], base) for i in range(n_h)]
        for i in range(n_h):
            n = int(n_vis[m])
            scores, values = [], []
            for j in range(n):
                kc = [sum(w_uk[i, a, c] * c_kv[j, c] for c in range(d_c)) for a in range(d_h)]
                vc = [sum(w_uv[i, a, c] * c_kv[j, c] for c in range(d_c)) for a in range(d_h)]
                kr = _rope_complex(k_r[j], key_pos[j], base)
                dot = sum(q_nope[m, i, a] * kc[a] for a in range(d_h))
                dot += sum(qr_all[i][a] * kr[a] for a in range(len(kr)))
                scores.append(dot * scale)
                values.append(vc)
            if n == 0:
                continue
            mx = max(scores)
            es = [math.exp(s - mx) for s in scores]
            z = sum(es)
            for a in range(d_h):
                out[m, i, a] = sum(es[j] * values[j][a] for j in range(n)) / z
            lse[m, i] = mx + math.log(z)
    return out, lse


@pytest.mark.parametrize("seed,L,M", [(0, 5, 1), (1, 9, 3), (2, 1, 1)])
def test_naive_matches_brute_force(seed, L, M):
    t = _tiny(seed=seed, L=L, M=M)
    key_pos = np.arange(L)
    q_pos = np.arange(L - M, L) if M > 1 else np.array([L])
    n_vis = orc.visible_keys(L, M) if M > 1 else np.array([L])
    scale = 1 / math.sqrt(4 + 4)
    out, lse, _ = orc.mla_attention_naive(**t, key_pos=key_pos, q_pos=q_pos, n_visible=n_vis,
                                          scale=scale, base=10000.0)
    bo, bl = _brute_force(t["c_kv"], t["k_r"], t["q_nope"], t["q_rope"], t["w_uk"], t["w_uv"],
                          key_pos, q_pos, n_vis, scale, 10000.0)
    np.testing.assert_allclose(out, bo, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, bl, rtol=0, atol=1e-12)


def test_absorbed_equals_non_absorbed():
    # Associativity (blog §2.2.1.1): W^UK folds into the query, W^UV into the output.
    for seed, L, M in [(5, 37, 1), (6, 20, 4)]:
        t = _tiny(seed=seed, L=L, M=M, n_h=3, d_h=6, d_c=10, d_r=4)
        q_pos = np.arange(L - M, L) if M > 1 else np.array([L])
        n_vis = orc.visible_keys(L, M) if M > 1 else np.array([L])
        scale = 1 / math.sqrt(6 + 4)
        out, lse, o_lat = orc.mla_attention_naive(**t, key_pos=np.arange(L), q_pos=q_pos,
                                                  n_visible=n_vis, scale=scale, base=10000.0)
        rows = orc.kv_cache_rows(t["c_kv"], t["k_r"], np.arange(L), 10000.0)
        q_lat = orc.absorb_query(t["q_nope"], t["q_rope"], t["w_uk"], q_pos, 10000.0)
        o_lat2, lse2 = orc.latent_attention(q_lat, rows, n_vis, scale, d_c=10)
        out2 = orc.out_projection(o_lat2, t["w_uv"])
        np.testing.assert_allclose(out2, out, rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(lse2, lse, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(o_lat2, o_lat, rtol=1e-10, atol=1e-12)


def test_softmax_rows_sum_to_one():
    rng = np.random.default_rng(7)
    s = rng.standard_normal((4, 50)) * 10
    p, lse = orc._softmax_two_pass(s)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, atol=1e-12)
    np.testing.assert_allclose(np.exp(s - lse[:, None]).sum(axis=1), 1.0, atol=1e-12)
    assert (p >= 0).all()


# ------------------------------------------------------------- special cases

def test_identity_weights_reduce_to_library_attention():
    """W^UK = W^UV = I with d_c = d_h and no RoPE part: MQA over K = V = c^KV
    (blog §2.1.2: MQA shares one key and value head across all query heads).
    With one head it is plain scaled-dot attention, checked against torch."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(8)
    L, d = 23, 16
    c = rng.standard_normal((L, d))
    q = rng.standard_normal((1, 1, d))
    eye = np.eye(d)[None]
    out, lse, _ = orc.mla_attention_naive(
        c, np.zeros((L, 0)), q, np.zeros((1, 1, 0)), eye, eye, np.arange(L), np.array([L]),
        np.array([L]), scale=1 / math.sqrt(d), base=10000.0)
    tq = torch.tensor(q[0][None], dtype=torch.float64)            # [1, 1, d]
    tk = torch.tensor(c[None], dtype=torch.float64)               # [1, L, d]
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tk)
    np.testing.assert_allclose(out[0, 0], ref[0, 0].numpy(), rtol=1e-12, atol=1e-13)


def test_single_key_returns_its_value():
    t = _tiny(seed=9, L=1)
    out, _, _ = orc.mla_attention_naive(**t, key_pos=[0], q_pos=[1], n_visible=[1],
                                        scale=0.3, base=10000.0)
    for i in range(2):
        np.testing.assert_allclose(out[0, i], t["w_uv"][i] @ t["c_kv"][0], rtol=1e-13)


def test_zero_query_averages_values():
    t = _tiny(seed=10, L=11)
    t["q_nope"][:] = 0
    t["q_rope"][:] = 0
    out, lse, _ = orc.mla_attention_naive(**t, key_pos=np.arange(11), q_pos=[11],
                                          n_visible=[11], scale=0.3, base=10000.0)
    for i in range(2):
        np.testing.assert_allclose(out[0, i], (t["c_kv"] @ t["w_uv"][i].T).mean(axis=0),
                                   rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse, math.log(11), rtol=1e-14)


def test_causal_chunk_rows_see_their_own_position():
    # A chunk of q_len rows at positions L-q_len..L-1: row m sees keys with
    # position <= its own (eq. 7's sum over j <= t).
    L, q = 10, 4
    vis = orc.visible_keys(L, q)
    q_pos = np.arange(L - q, L)
    for m in range(q):
        assert vis[m] == q_pos[m] + 1
    assert list(orc.visible_keys(7, 1)) == [7]


def test_empty_row_gives_zero_and_minus_inf():
    t = _tiny(seed=11, L=4)
    out, lse, o_lat = orc.mla_attention_naive(**t, key_pos=np.arange(4), q_pos=[0],
                                              n_visible=[0], scale=0.3, base=1e4)
    assert np.all(out == 0) and np.all(o_lat == 0) and np.all(np.isneginf(lse))


# ---------------------------------------------------------------- split / combine

@pytest.mark.parametrize("n,S", [(1, 1), (64, 1), (65, 2), (4096, 8), (300, 16), (131072, 64),
                                 (1000, 3), (0, 4)])
def test_split_ranges_partition_the_keys(n, S):
    r = orc.split_ranges(n, 64, S)
    assert len(r) == S
    covered = [j for lo, hi in r for j in range(lo, hi)]
    assert covered == list(range(n))
    nblk = -(-n // 64)
    c = -(-nblk // S) if nblk else 0
    for lo, hi in r:
        assert hi - lo <= c * 64
        assert lo % 64 == 0 or lo == n


def test_split_ranges_against_block_walk():
    # Independent formulation: hand out blocks one by one, c to a split.
    for n in [1, 63, 64, 65, 777, 8192, 8191]:
        for S in [1, 2, 3, 5, 8, 64]:
            nblk = -(-n // 64)
            c = -(-nblk // S)
            owner = [b // c for b in range(nblk)]
            want = []
            for s in range(S):
                blocks = [b for b in range(nblk) if owner[b] == s]
                if blocks:
                    want.append((blocks[0] * 64, min((blocks[-1] + 1) * 64, n)))
                else:
                    want.append(None)
            got = orc.split_ranges(n, 64, S)
            for w, g in zip(want, got):
                if w is None:
                    assert g[0] == g[1]
                else:
                    assert w == g


def test_combine_of_splits_equals_unsplit():
    rng = np.random.default_rng(12)
    L, n_h, W, d_c = 300, 3, 12, 8
    rows = rng.standard_normal((L, W))
    q = rng.standard_normal((1, n_h, W))
    o_full, lse_full = orc.latent_attention(q, rows, [L], 0.4, d_c)
    for S in [1, 2, 5, 7]:
        parts = orc.split_ranges(L, 64, S)
        os_, ls_ = [], []
        for lo, hi in parts:
            o, l = orc.latent_attention(q, rows[lo:hi], [hi - lo], 0.4, d_c)
            os_.append(o)
            ls_.append(l)
        o, l = orc.combine_splits(np.stack(os_), np.stack(ls_))
        np.testing.assert_allclose(o, o_full, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(l, lse_full, rtol=1e-13)


def test_combine_all_empty():
    o, l = orc.combine_splits(np.zeros((3, 1, 2, 4)), np.full((3, 1, 2), -np.inf))
    assert np.all(o == 0) and np.all(np.isneginf(l))


# ------------------------------------------------------------- cache-size facts

def test_cached_row_width_is_dc_plus_dr_and_equals_gqa_225_groups():
    g = json.load(open(GOLDEN))
    v2 = g["deepseek_v2"]
    d_c, d_r, d_h, n_h = v2["d_c"], v2["d_R"], v2["d_h"], v2["n_h"]
    assert d_c == g["relations"]["d_c_over_d_h"] * d_h
    assert d_r == g["relations"]["d_R_over_d_h"] * d_h
    rng = np.random.default_rng(13)
    rows = orc.kv_cache_rows(rng.standard_normal((3, d_c)), rng.standard_normal((3, d_r)),
                             np.arange(3), 10000.0)
    per_token = rows.shape[1]
    # GQA with n_g groups caches 2 n_g d_h elements per token per layer.
    assert per_token == 2 * g["relations"]["gqa_groups_equivalent"] * d_h
    # MHA caches 2 n_h d_h (blog §2.1.1); MLA's share of it at the V2 shape:
    assert abs(per_token / (2 * n_h * d_h) - 576 / 32768) < 1e-15
    lite = g["deepseek_v2_lite"]
    assert (lite["d_c"], lite["d_R"], lite["d_h"]) == (d_c, d_r, d_h)


def test_cached_rows_keep_latent_unrotated():
    rng = np.random.default_rng(14)
    c, k = rng.standard_normal((5, 8)), rng.standard_normal((5, 4))
    rows = orc.kv_cache_rows(c, k, np.arange(5) + 100, 10000.0)
    np.testing.assert_array_equal(rows[:, :8], c)
    np.testing.assert_allclose(rows[:, 8:], orc.rope_rotate(k, np.arange(5) + 100, 1e4))


# ---------------------------------------------------------------- producers
def test_rms_norm_worked_example_and_properties():
    # [3, 4]: mean square 12.5, root 3.5355..; gain [1, 2]
    y = orc.rms_norm(np.array([[3.0, 4.0]]), np.array([1.0, 2.0]), 0.0)
    np.testing.assert_allclose(y, [[3 / np.sqrt(12.5), 8 / np.sqrt(12.5)]], rtol=1e-15)
    rng = np.random.default_rng(5)
    x = rng.standard_normal((7, 512)) * 3.0
    y = orc.rms_norm(x, np.ones(512), 0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, rtol=1e-13)
    np.testing.assert_allclose(orc.rms_norm(4.5 * x, np.ones(512), 0.0), y, rtol=1e-13)
    # eps sits inside the root: an all-zero row stays zero, a tiny row is damped
    np.testing.assert_array_equal(orc.rms_norm(np.zeros((1, 4)), np.ones(4), 1e-6), 0.0)
    t = orc.rms_norm(np.full((1, 4), 1e-3), np.ones(4), 1e-6)
    np.testing.assert_allclose(t, 1e-3 / np.sqrt(1e-6 + 1e-6), rtol=1e-13)


def test_kv_produce_identity_weights():
    """W^DKV = [I 0], W^KR = [0 I]: c^KV is the normalised first d_c features of
    h and k^R the remaining d_R, rotated in the cached row."""
    rng = np.random.default_rng(6)
    d_c, d_r, T = 8, 4, 5
    h = rng.standard_normal((T, d_c + d_r))
    w_dkv = np.hstack([np.eye(d_c), np.zeros((d_c, d_r))])
    w_kr = np.hstack([np.zeros((d_r, d_c)), np.eye(d_r)])
    pos = np.array([0, 3, 7, 100, 4096])
    c, k, rows = orc.kv_produce(h, w_dkv, np.ones(d_c), w_kr, pos, 10000.0, 0.0)
    lat = h[:, :d_c]
    np.testing.assert_allclose(c, lat / np.sqrt(np.mean(lat * lat, axis=1, keepdims=True)),
                               rtol=1e-14)
    np.testing.assert_array_equal(k, h[:, d_c:])
    np.testing.assert_array_equal(rows[:, :d_c], c)
    np.testing.assert_allclose(rows[0, d_c:], h[0, d_c:], rtol=1e-15)   # position 0
    np.testing.assert_allclose(rows[:, d_c:], orc.rope_rotate(h[:, d_c:], pos, 10000.0),
                               rtol=1e-15)


def test_producers_match_scalar_loops():
    """kv_produce and q_produce against element-by-element sums on tiny,
    non-square shapes (a transposed weight or a wrong head split fails)."""
    rng = np.random.default_rng(7)
    T, d_model, d_c, d_r, d_cq, n_h, d_h = 3, 7, 5, 4, 6, 2, 3
    h = rng.standard_normal((T, d_model))
    w_dkv = rng.standard_normal((d_c, d_model))
    w_kr = rng.standard_normal((d_r, d_model))
    g_kv = rng.standard_normal(d_c)
    w_dq = rng.standard_normal((d_cq, d_model))
    g_q = rng.standard_normal(d_cq)
    w_uq = rng.standard_normal((n_h * d_h, d_cq))
    w_qr = rng.standard_normal((n_h * d_r, d_cq))
    eps = 0.25
    c, k, _ = orc.kv_produce(h, w_dkv, g_kv, w_kr, np.zeros(T), 10000.0, eps)
    cq, qn, qr = orc.q_produce(h, w_dq, g_q, w_uq, w_qr, n_h, eps)
    for t in range(T):
        lat = [sum(w_dkv[i][j] * h[t][j] for j in range(d_model)) for i in range(d_c)]
        r = math.sqrt(sum(v * v for v in lat) / d_c + eps)
        for i in range(d_c):
            assert abs(c[t][i] - g_kv[i] * lat[i] / r) < 1e-12
        for i in range(d_r):
            assert abs(k[t][i] - sum(w_kr[i][j] * h[t][j] for j in range(d_model))) < 1e-12
        qlat = [sum(w_dq[i][j] * h[t][j] for j in range(d_model)) for i in range(d_cq)]
        rq = math.sqrt(sum(v * v for v in qlat) / d_cq + eps)
        cql = [g_q[i] * qlat[i] / rq for i in range(d_cq)]
        for i in range(d_cq):
            assert abs(cq[t][i] - cql[i]) < 1e-12
        for head in range(n_h):
            for d in range(d_h):
                want = sum(w_uq[head * d_h + d][j] * cql[j] for j in range(d_cq))
                assert abs(qn[t][head][d] - want) < 1e-12
            for d in range(d_r):
                want = sum(w_qr[head * d_r + d][j] * cql[j] for j in range(d_cq))
                assert abs(qr[t][head][d] - want) < 1e-12


def test_direct_query_producer_matches_scalar_loops():
    """q_produce_direct (reading R10) against element-by-element sums on a
    tiny non-square shape, and against q_produce when the compression is an
    identity without its norm (a transposed weight or a wrong head split
    fails one of them)."""
    rng = np.random.default_rng(11)
    T, d_model, n_h, d_h, d_r = 3, 5, 2, 4, 3
    h = rng.standard_normal((T, d_model))
    w_qc = rng.standard_normal((n_h * d_h, d_model))
    w_qr = rng.standard_normal((n_h * d_r, d_model))
    qn, qr = orc.q_produce_direct(h, w_qc, w_qr, n_h)
    assert qn.shape == (T, n_h, d_h) and qr.shape == (T, n_h, d_r)
    for t in range(T):
        for head in range(n_h):
            for d in range(d_h):
                want = sum(w_qc[head * d_h + d][j] * h[t][j] for j in range(d_model))
                assert abs(qn[t][head][d] - want) < 1e-12
            for d in range(d_r):
                want = sum(w_qr[head * d_r + d][j] * h[t][j] for j in range(d_model))
                assert abs(qr[t][head][d] - want) < 1e-12
    # q_produce with W^DQ = I and a huge eps scaled back by the gain is the
    # direct producer: RMSNorm(x) = g x / sqrt(mean(x^2) + eps) -> x when
    # g = sqrt(eps) and eps >> mean(x^2)
    eps = 1e20
    _, qn2, qr2 = orc.q_produce(h, np.eye(d_model), np.full(d_model, np.sqrt(eps)), w_qc, w_qr,
                                n_h, eps)
    np.testing.assert_allclose(qn2, qn, rtol=1e-9, atol=1e-9)
    np.testing.assert_allclose(qr2, qr, rtol=1e-9, atol=1e-9)


def test_o_projection_matches_scalar_loops():
    """eq. 8's u = W^O [o_1; ...; o_nh] against element-by-element sums (a
    head order or a transposed W^O fails), and a W^O that picks one head's
    dimension returns that output."""
    rng = np.random.default_rng(5)
    T, n_h, d_h, d_model = 3, 2, 4, 5
    out = rng.standard_normal((T, n_h, d_h))
    w_o = rng.standard_normal((d_model, n_h * d_h))
    u = orc.o_projection(out, w_o)
    for t in range(T):
        for i in range(d_model):
            want = sum(w_o[i][h * d_h + d] * out[t][h][d] for h in range(n_h) for d in range(d_h))
            assert abs(u[t][i] - want) < 1e-12
    pick = np.zeros((1, n_h * d_h))
    pick[0, 1 * d_h + 2] = 1.0                 # head 1, dimension 2
    np.testing.assert_array_equal(orc.o_projection(out, pick)[:, 0], out[:, 1, 2])


# ------------------------------------------------------- quantised latent cache

def _e4m3_table():
    """Finite E4M3 values by brute force from the bit layout (sign, 4-bit
    exponent with bias 7, 3-bit mantissa, subnormals at exponent 0, NaN at
    S.1111.111), independent of the oracle's decoder."""
    vals = {}
    for code in range(256):
        s, e, m = code >> 7, (code >> 3) & 15, code & 7
        if e == 15 and m == 7:
            continue
        mag = (m / 8) * 2.0 ** -6 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
        vals[code] = -mag if s else mag
    return vals


def test_e4m3_decoder_matches_the_bit_layout():
    table = _e4m3_table()
    v = orc.e4m3_value(np.arange(256))
    for code in range(256):
        if code in table:
            assert v[code] == table[code] and math.copysign(1, v[code]) == math.copysign(1, table[code])
        else:
            assert np.isnan(v[code])
    # landmarks of the format: 1.0, the largest value, the smallest normal and subnormal
    assert v[0x38] == 1.0 and v[0x7E] == 448.0 and v[0x08] == 2.0 ** -6 and v[0x01] == 2.0 ** -9
    assert len(table) == 254 and np.nanmax(v) == 448.0
    finite = np.array(sorted(table))
    np.testing.assert_array_equal(orc.e4m3_code(v[finite]), finite)


def test_e4m3_round_is_nearest_with_ties_to_even():
    table = _e4m3_table()
    pos = sorted({v for c, v in table.items() if v >= 0 and not (v == 0 and c & 0x80)})
    even = {v: (c & 1) == 0 for c, v in table.items() if c < 0x80}
    rng = np.random.default_rng(50)
    ys = list(rng.uniform(0, 460, 2000)) + list(2.0 ** rng.uniform(-12, 8.8, 2000))
    ys += [(a + b) / 2 for a, b in zip(pos, pos[1:])]          # every midpoint
    ys += [448.0, 455.9, 464.0, 470.0, 1e4]
    for y in ys:
        got = orc.e4m3_round(y)
        if y >= 448.0:
            assert got == 448.0                                 # clamped
            continue
        d = [abs(y - v) for v in pos]
        best = min(d)
        cands = [v for v, dv in zip(pos, d) if dv == best]
        want = cands[0] if len(cands) == 1 else [v for v in cands if even[v]][0]
        assert got == want, (y, got, want)
        assert orc.e4m3_round(-y) == -want
    # worked cases: a tie goes to the even mantissa
    assert orc.e4m3_round(1.0625) == 1.0 and orc.e4m3_round(1.1875) == 1.25
    assert orc.e4m3_round(2.0 ** -10) == 0.0 and orc.e4m3_round(1.5 * 2.0 ** -9) == 2.0 ** -8


def _fp32_rows(rng, n, scale_c=1.0, scale_r=1.0):
    rows = np.concatenate([scale_c * rng.standard_normal((n, 512)),
                           scale_r * rng.standard_normal((n, 64))], axis=1)
    return rows.astype(np.float32)


def test_quantised_rows_error_bounds_and_scale():
    rng = np.random.default_rng(51)
    rows = _fp32_rows(rng, 64, 3.0, 0.01)
    codes, scales = orc.quantize_rows(rows, 512)
    deq = orc.dequantize_rows(codes, scales, 512)
    x = rows.astype(np.float64)
    for k, (lo, hi) in enumerate([(0, 512), (512, 576)]):
        amax = np.abs(x[:, lo:hi]).max(axis=1)
        s = scales[:, k].astype(np.float64)
        assert np.all(np.abs(s * 448 / amax - 1) < 2 ** -23)     # s = amax / 448 (one rounding)
        # the largest element lands on +-448
        arg = np.abs(x[:, lo:hi]).argmax(axis=1)
        assert np.all(np.abs(orc.e4m3_value(codes[np.arange(64), lo + arg])) == 448.0)
        err = np.abs(deq[:, lo:hi] - x[:, lo:hi])
        y = np.abs(x[:, lo:hi]) / s[:, None]
        normal = y >= 2.0 ** -6
        # half a spacing: 2^-4 of the value (normal range), 2^-10 s (subnormal),
        # plus the float32 quotient's rounding
        assert np.all(err[normal] <= (2.0 ** -4 * np.abs(x[:, lo:hi]) + 1e-6 * s[:, None])[normal])
        assert np.all(err[~normal] <= (2.0 ** -10 + 1e-7) * np.broadcast_to(s[:, None], err.shape)[~normal])
    # each part has its own scale: the RoPE part, 300x smaller, is as precise
    rel = np.abs(deq - x) / np.abs(x).max(axis=1, keepdims=True)
    assert rel[:, 512:].max() < 0.05


def test_quantised_rows_special_cases():
    rows = np.zeros((3, 576), np.float32)
    rows[1, 7] = -2.5
    rows[2, 600 - 30] = 1e-30                                  # one tiny RoPE element
    codes, scales = orc.quantize_rows(rows, 512)
    assert np.all(codes[0] == 0) and np.all(scales[0] == 1.0)
    assert codes[1, 7] == 0xFE and scales[1, 0] == np.float32(2.5) / np.float32(448)
    assert np.all(codes[1, 512:] == 0) and scales[1, 1] == 1.0
    assert orc.e4m3_value(codes[2, 570]) == 448.0
    # re-quantising the dequantised rows gives the same codes
    rng = np.random.default_rng(52)
    r = _fp32_rows(rng, 16)
    c1, s1 = orc.quantize_rows(r, 512)
    c2, s2 = orc.quantize_rows(orc.dequantize_rows(c1, s1, 512).astype(np.float32), 512)
    np.testing.assert_array_equal(c1, c2)


def test_fp8_cache_rows_quantise_the_rotated_row():
    t = _tiny(seed=53, L=9, d_c=512, d_r=64)
    codes, scales = orc.kv_cache_rows_fp8(t["c_kv"], t["k_r"], np.arange(9), 1e4)
    rows = orc.kv_cache_rows(t["c_kv"], t["k_r"], np.arange(9), 1e4)
    deq = orc.dequantize_rows(codes, scales, 512)
    assert np.max(np.abs(deq - rows) / np.abs(rows).max(axis=1, keepdims=True)) < 2.0 ** -4
    # the RoPE part is quantised after the rotation: rotating the dequantised
    # unrotated key would differ
    un, su = orc.quantize_rows(np.concatenate([t["c_kv"], t["k_r"]], 1).astype(np.float32), 512)
    assert np.any(un[:, 512:] != codes[:, 512:])
