"""GPU parity of the quantised latent cache (FP8 E4M3 codes, two float32
scales per token) against the oracle's quantiser and attention.

The append must reproduce the oracle's codes and scales bit for bit (both
sides take every rounding decision in float32 on the same values; the RoPE
part is exempt only where the two float64 rotations round to different float32
values, which the test reports).  The attention is compared with the oracle's
attention over the dequantised rows at the bf16 bound, since the dequantised
values are exact in the kernel.  The quantisation error itself (against the
unquantised cache) is a property of the format and is checked on statistics.
"""
import math

import numpy as np
import pytest

from gpu_util import TOL, rel_err, say, small, to_np
from mla_latent_kv_04_amd import pipeline
from mla_latent_kv_04_amd.workloads import (BLOCK, D_C, ROPE_BASE, WORKLOADS, make_problem,
                                            softmax_scale)
from oracle import mla_oracle as orc

pytestmark = pytest.mark.gpu

F1, F2, F3, F4, F5 = ("v2lite_f32_L256", "v2lite_bf16_B64_L4096", "v2_bf16_B128_L1k-8k",
                      "v2_bf16_B4_L128k_splitkv", "v2_bf16_prefill_6144+2048")


def _host_cache(dp):
    return dp.kv_cache.cpu().numpy(), dp.kv_scale.cpu().numpy()


def _cache_rows(dp, host, b, L):
    """GPU codes [L, 576] and scales [L, 2] of sequence b's first L tokens."""
    codes, scales = host
    tab = dp.prob.block_table[b]
    j = np.arange(L)
    return codes[tab[j // BLOCK], j % BLOCK], scales[tab[j // BLOCK], j % BLOCK]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_fp8_append_reproduces_the_oracle_codes(dtype):
    """Quantise rows at ragged positions (three sequences, partial blocks) and
    compare every code and scale; untouched slots keep their poison."""
    import torch
    from mla_latent_kv_04_amd import _binding as mla
    from mla_latent_kv_04_amd.workloads import round_to_bf16
    rng = np.random.default_rng(60)
    lens = [130, 5, 64]
    nblk = sum((L + BLOCK - 1) // BLOCK for L in lens)
    table = np.full((3, 3), -1, np.int32)
    perm = rng.permutation(nblk)
    k = 0
    for b, L in enumerate(lens):
        for j in range((L + BLOCK - 1) // BLOCK):
            table[b, j] = perm[k]
            k += 1
    seq = np.concatenate([np.full(L, b) for b, L in enumerate(lens)]).astype(np.int32)
    pos = np.concatenate([np.arange(L) for L in lens]).astype(np.int32)
    n = len(seq)
    scale_c = np.exp(rng.uniform(-6, 6, (n, 1)))      # rows of very different magnitude
    c = (rng.standard_normal((n, D_C)) * scale_c).astype(np.float32)
    kr = (rng.standard_normal((n, 64)) * np.exp(rng.uniform(-6, 6, (n, 1)))).astype(np.float32)
    c[3] = 0.0                                         # an all-zero latent part
    kr[4] = 0.0                                        # an all-zero RoPE part
    if dtype == "bf16":
        c, kr = round_to_bf16(c), round_to_bf16(kr)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    cache = torch.full((nblk, BLOCK, 576), 0xFF, dtype=torch.uint8, device="cuda")
    scales = torch.full((nblk, BLOCK, 2), float("nan"), dtype=torch.float32, device="cuda")
    say(f"fp8 append {dtype} n={n}")
    mla.mla_kv_append_fp8(cache, scales, torch.from_numpy(table).cuda(),
                          torch.from_numpy(c).to(tdt).cuda(), torch.from_numpy(kr).to(tdt).cuda(),
                          torch.from_numpy(seq).cuda(), torch.from_numpy(pos).cuda(), ROPE_BASE)
    torch.cuda.synchronize()
    got_c = cache.cpu().numpy()
    got_s = scales.cpu().numpy()
    want_c, want_s = orc.kv_cache_rows_fp8(c.astype(np.float64), kr.astype(np.float64), pos,
                                           ROPE_BASE)
    blk, row = table[seq, pos // BLOCK], pos % BLOCK
    gc, gs = got_c[blk, row], got_s[blk, row]
    np.testing.assert_array_equal(gc[:, :D_C], want_c[:, :D_C])
    np.testing.assert_array_equal(gs[:, 0], want_s[:, 0])
    # RoPE part: the float32 rotated values of both sides may differ where the
    # two float64 rotations straddle a float32 rounding boundary
    rot = orc.kv_cache_rows(c.astype(np.float64), kr.astype(np.float64), pos, ROPE_BASE)[:, D_C:]
    r32 = rot.astype(np.float32).astype(np.float64)
    near = np.abs(rot - r32) > 0.5 * np.spacing(r32.astype(np.float32)).astype(np.float64) * (1 - 1e-6)
    diff_rows = np.nonzero(np.any(gc[:, D_C:] != want_c[:, D_C:], axis=1) | (gs[:, 1] != want_s[:, 1]))[0]
    print(f"[fp8] RoPE rows differing: {len(diff_rows)} of {n}", flush=True)
    for r in diff_rows:
        assert near[r].any(), r
    assert len(diff_rows) <= 2
    # all-zero parts: zero values (a rotated zero may be -0, code 0x80) and unit scales
    assert np.all(orc.e4m3_value(gc[3, :D_C]) == 0) and gs[3, 0] == 1.0
    assert np.all(orc.e4m3_value(gc[4, D_C:]) == 0) and gs[4, 1] == 1.0
    written = np.zeros(got_c.shape[:2], bool)
    written[blk, row] = True
    assert np.all(got_c[~written] == 0xFF) and np.isnan(got_s[~written]).all()


def _oracle_on_gpu_rows(dp, host, q_lat_all, b, rows=None):
    """Attention of sequence b's query rows over the dequantised GPU cache,
    with the GPU's bf16 q_lat (so that only the attention is compared)."""
    q = dp.q_len
    L = int(dp.prob.seq_lens[b])
    codes, scales = _cache_rows(dp, host, b, L)
    deq = orc.dequantize_rows(codes, scales, D_C)
    q_lat = q_lat_all[b * q:(b + 1) * q]
    vis = orc.visible_keys(L, q)
    if rows is not None:
        q_lat, vis = q_lat[rows], vis[rows]
    return orc.latent_attention(q_lat, deq, vis, softmax_scale(), D_C)


@pytest.mark.parametrize("case", [
    (F2, dict(B=4, ctx=[1000, 1, 0, 129]), 1),
    (F2, dict(B=3, ctx=[4096, 65, 700]), 4),
    (F2, dict(B=2, ctx=[700, 2000], n_h=32), 3),
    (F3, dict(B=3, ctx=[1500, 64, 333]), 2),
    (F5, dict(ctx=700, q_len=40, n_h=16), 1),
    (F5, dict(ctx=700, q_len=70), 1),
    (F2, dict(B=5, ctx=[3000, 10, 4096, 700, 1]), 0),
    (F3, dict(B=4, ctx=[2000, 1, 900, 64]), 0),
], ids=["lite-S1", "lite-S4", "h32-S3", "h128-S2", "chunk-q40", "chunk-q70-h128", "lite-planned",
        "h128-planned"])
def test_fp8_decode_matches_attention_over_the_dequantised_rows(case):
    import torch
    wl, kw, S = case
    prob = small(wl, **kw)
    say(f"fp8 decode {wl} {kw} S={S}")
    dp = pipeline.upload(prob, num_splits=S, cache="fp8")
    pipeline.append(dp)
    from mla_latent_kv_04_amd import _binding as mla
    mla.mla_absorb_q(dp.q_nope, dp.q_rope, dp.w_uk, dp.q_pos, dp.q_lat, ROPE_BASE)
    pipeline.decode(dp)
    torch.cuda.synchronize()
    o_lat, lse = to_np(dp.o_lat), to_np(dp.lse)
    host, q_lat = _host_cache(dp), to_np(dp.q_lat)
    q = prob.wl.q_len
    for b in range(prob.wl.B):
        ref, lref = _oracle_on_gpu_rows(dp, host, q_lat, b)
        got = o_lat[b * q:(b + 1) * q]
        if int(prob.seq_lens[b]) == 0:
            assert np.all(got == 0) and np.all(np.isneginf(lse[b * q:(b + 1) * q]))
            continue
        assert rel_err(got, ref) <= TOL["bf16"], b
        fin = np.isfinite(lref)
        np.testing.assert_array_equal(np.isfinite(lse[b * q:(b + 1) * q]), fin)
        assert np.max(np.abs(lse[b * q:(b + 1) * q][fin] - lref[fin])) <= TOL["bf16"] * max(
            1.0, float(np.abs(lref[fin]).max()))


@pytest.mark.parametrize("wl,kw,S", [(F2, dict(B=2, ctx=[300, 256]), 1),
                                     (F3, dict(B=2, ctx=[300, 256]), 1),
                                     (F3, dict(B=2, ctx=[300, 256]), 0)],
                         ids=["16-heads", "128-heads", "128-heads-planned"])
def test_fp8_out_of_range_block_ids_are_skipped(wl, kw, S):
    """A block id outside [0, num_blocks) drops that block's keys (their rows
    are zeroed with unit scales in LDS and masked)."""
    import torch
    prob = small(wl, **kw)
    say(f"fp8 bad block id {wl} S={S}")
    dp = pipeline.upload(prob, num_splits=S, cache="fp8")
    pipeline.append(dp)
    from mla_latent_kv_04_amd import _binding as mla
    mla.mla_absorb_q(dp.q_nope, dp.q_rope, dp.w_uk, dp.q_pos, dp.q_lat, ROPE_BASE)
    table = dp.block_table.clone()
    table[0, 1] = 10 ** 6                 # keys 64..127 of sequence 0 vanish
    table[1, 3] = -5                      # keys 192..255 of sequence 1 vanish
    dp.block_table = table
    pipeline.decode(dp)
    torch.cuda.synchronize()
    host, q_lat = _host_cache(dp), to_np(dp.q_lat)
    o_lat = to_np(dp.o_lat)
    for b, gone in ((0, range(64, 128)), (1, range(192, 256))):
        L = int(prob.seq_lens[b])
        keep = np.array([j for j in range(L) if j not in gone])
        codes, scales = _cache_rows(dp, host, b, L)
        deq = orc.dequantize_rows(codes[keep], scales[keep], D_C)
        ref, _ = orc.latent_attention(q_lat[b:b + 1], deq, [len(keep)], softmax_scale(), D_C)
        assert rel_err(o_lat[b:b + 1], ref) <= TOL["bf16"], b


@pytest.mark.timeout(600)
def test_fp8_step_full_size_lite_every_output():
    """The V2-Lite decode workload (B=64, 16 heads, L=4096) with the FP8
    cache, the benchmark's launch configuration (balanced plan, planned
    decode, merge inside the out-projection): every output against the
    oracle's out-projection of its attention over the dequantised rows."""
    import torch
    prob = make_problem(WORKLOADS[F2])
    say("fp8 full-size lite step")
    dp = pipeline.upload(prob, num_splits=0, cache="fp8")
    pipeline.step(dp)
    torch.cuda.synchronize()
    out = to_np(dp.out)
    host, q_lat = _host_cache(dp), to_np(dp.q_lat)
    refs = []
    for b in range(prob.wl.B):
        o_lat, _ = _oracle_on_gpu_rows(dp, host, q_lat, b)
        refs.append(orc.out_projection(o_lat, prob.w_uv))
    ref = np.concatenate(refs)
    err = rel_err(out, ref)
    print(f"[fp8] full-size lite: max|err|/rms = {err:.3e} over {out.size} outputs", flush=True)
    assert err <= TOL["bf16"]


@pytest.mark.timeout(900)
def test_fp8_step_full_size_v2_every_output():
    """The V2 decode workload (B=128, 128 heads, L ~ U[1024, 8192]) with the
    FP8 cache through the two-role 64-head kernel, balanced plan with lists:
    every output against the oracle's attention over the dequantised rows."""
    import torch
    prob = make_problem(WORKLOADS[F3])
    say("fp8 full-size v2 step")
    dp = pipeline.upload(prob, num_splits=0, cache="fp8")
    pipeline.step(dp)
    torch.cuda.synchronize()
    out, lse = to_np(dp.out), to_np(dp.lse)
    host, q_lat = _host_cache(dp), to_np(dp.q_lat)
    refs, lrefs = [], []
    for b in range(prob.wl.B):
        o_lat, l = _oracle_on_gpu_rows(dp, host, q_lat, b)
        refs.append(orc.out_projection(o_lat, prob.w_uv))
        lrefs.append(l)
    ref, lref = np.concatenate(refs), np.concatenate(lrefs)
    err = rel_err(out, ref)
    print(f"[fp8] full-size v2: max|err|/rms = {err:.3e} over {out.size} outputs", flush=True)
    assert err <= TOL["bf16"]
    assert np.max(np.abs(lse - lref)) <= TOL["bf16"] * max(1.0, float(np.abs(lref).max()))


def test_fp8_quantisation_error_against_the_unquantised_cache():
    """What the format costs: the same step with the bf16 cache and with the
    FP8 cache, each against the unquantised oracle.  The FP8 step's error is
    the E4M3 rounding (3 mantissa bits) seen through the softmax average: RMS
    about 3e-2 of the output RMS in a CPU evaluation of the oracle alone."""
    import torch
    prob = small(F2, B=4, ctx=[1000, 4096, 300, 64])
    say("fp8 quantisation error")
    res = {}
    for cache in ["native", "fp8"]:
        dp = pipeline.upload(prob, num_splits=1, cache=cache)
        pipeline.step(dp)
        torch.cuda.synchronize()
        res[cache] = to_np(dp.out)
    q = prob.wl.q_len
    ref = np.concatenate([
        orc.out_projection(orc.latent_attention(
            orc.absorb_query(prob.q_nope[b * q:(b + 1) * q], prob.q_rope[b * q:(b + 1) * q],
                             prob.w_uk, prob.q_pos[b * q:(b + 1) * q], ROPE_BASE),
            orc.kv_cache_rows(*[x[:int(prob.seq_lens[b])] for x in prob.seq_rows(b)],
                              np.arange(int(prob.seq_lens[b])), ROPE_BASE),
            orc.visible_keys(int(prob.seq_lens[b]), q), softmax_scale(), D_C)[0], prob.w_uv)
        for b in range(prob.wl.B)])
    rms = math.sqrt(float(np.mean(ref ** 2)))
    e_native = math.sqrt(float(np.mean((res["native"] - ref) ** 2))) / rms
    e_fp8 = math.sqrt(float(np.mean((res["fp8"] - ref) ** 2))) / rms
    print(f"[fp8] rms err/rms: bf16 cache {e_native:.3e}, fp8 cache {e_fp8:.3e}", flush=True)
    assert e_native <= 4e-3
    assert 1e-2 <= e_fp8 <= 5e-2


@pytest.mark.parametrize("wl,n_h,S", [(F3, 128, 0), (F3, 128, 1), (F2, 16, 1)],
                         ids=["h128-planned", "h128-S1", "h16-S1"])
def test_fp8_rising_scores_force_running_max_updates(wl, n_h, S):
    """Cached rows scaled up tile by tile: the running maximum keeps moving, so
    the rescale of the accumulators and (in the 64-head kernel) the rewrite of
    P and of the normaliser the score waves keep run on most tiles."""
    import torch
    from mla_latent_kv_04_amd.workloads import round_to_bf16
    prob = small(wl, B=2, ctx=[1500, 3000], n_h=n_h)
    pos = np.concatenate([np.arange(int(L)) for L in prob.seq_lens])
    f = (1.0 + pos // 32)[:, None]
    prob.c_kv = round_to_bf16(prob.c_kv * f)
    prob.k_r = round_to_bf16(prob.k_r * f)
    say(f"fp8 rising scores {wl} S={S}")
    dp = pipeline.upload(prob, num_splits=S, cache="fp8")
    pipeline.append(dp)
    from mla_latent_kv_04_amd import _binding as mla
    mla.mla_absorb_q(dp.q_nope, dp.q_rope, dp.w_uk, dp.q_pos, dp.q_lat, ROPE_BASE)
    pipeline.decode(dp)
    torch.cuda.synchronize()
    o_lat, lse = to_np(dp.o_lat), to_np(dp.lse)
    host, q_lat = _host_cache(dp), to_np(dp.q_lat)
    for b in range(2):
        ref, lref = _oracle_on_gpu_rows(dp, host, q_lat, b)
        assert rel_err(o_lat[b:b + 1], ref) <= TOL["bf16"], b
        assert np.max(np.abs(lse[b:b + 1] - lref)) <= TOL["bf16"] * max(1.0, np.abs(lref).max())


@pytest.mark.timeout(600)
def test_fp8_long_context_sampled():
    """The 128K workload with the FP8 cache (items longer than one staged
    chunk of block ids): sampled heads of every row against the oracle over
    the dequantised rows."""
    import torch
    prob = make_problem(WORKLOADS[F4])
    say("fp8 128K")
    dp = pipeline.upload(prob, num_splits=0, cache="fp8")
    pipeline.step(dp)
    torch.cuda.synchronize()
    out = to_np(dp.out)
    host, q_lat = _host_cache(dp), to_np(dp.q_lat)
    heads = [0, 63, 64, 127]
    for b in range(prob.wl.B):
        L = int(prob.seq_lens[b])
        codes, scales = _cache_rows(dp, host, b, L)
        deq = orc.dequantize_rows(codes, scales, D_C)
        o_lat, _ = orc.latent_attention(q_lat[b:b + 1][:, heads], deq, [L], softmax_scale(), D_C)
        ref = orc.out_projection(o_lat, prob.w_uv[heads])
        assert rel_err(out[b:b + 1][:, heads], ref) <= TOL["bf16"], b


def test_fp8_append_with_a_yarn_table():
    """The quantising append rotates with a given RoPE table (YaRN's): codes
    and scales equal the oracle's for the same table."""
    import torch
    from mla_latent_kv_04_amd import _binding as mla
    from mla_latent_kv_04_amd.workloads import round_to_bf16
    rng = np.random.default_rng(61)
    n = 130
    pos = np.sort(rng.choice(163840, n, replace=False)).astype(np.int32)
    used = np.unique(pos // BLOCK)
    table = np.full((1, 163840 // BLOCK), -1, np.int32)
    table[0, used] = np.arange(len(used))
    c = round_to_bf16(rng.standard_normal((n, D_C)).astype(np.float32))
    kr = round_to_bf16(rng.standard_normal((n, 64)).astype(np.float32))
    th = mla.mla_rope_theta(ROPE_BASE, 40.0, 1.0, 32.0, 4096)
    cache = torch.full((len(used), BLOCK, 576), 0xFF, dtype=torch.uint8, device="cuda")
    scales = torch.full((len(used), BLOCK, 2), float("nan"), dtype=torch.float32, device="cuda")
    say("fp8 append yarn")
    bf = torch.bfloat16
    mla.mla_kv_append_fp8(cache, scales, torch.from_numpy(table).cuda(),
                          torch.from_numpy(c).to(bf).cuda(), torch.from_numpy(kr).to(bf).cuda(),
                          torch.zeros(n, dtype=torch.int32, device="cuda"),
                          torch.from_numpy(pos).cuda(), ROPE_BASE, rope_theta=th)
    torch.cuda.synchronize()
    blk, row = table[0, pos // BLOCK], pos % BLOCK
    gc, gs = cache.cpu().numpy()[blk, row], scales.cpu().numpy()[blk, row]
    want_c, want_s = orc.kv_cache_rows_fp8(c.astype(np.float64), kr.astype(np.float64), pos,
                                           ROPE_BASE, orc.yarn_theta(64, ROPE_BASE, 40, 1, 32, 4096))
    np.testing.assert_array_equal(gc[:, :D_C], want_c[:, :D_C])
    np.testing.assert_array_equal(gs[:, 0], want_s[:, 0])
    # RoPE part: exact unless a float64 rotation lands on a float32 tie (none
    # expected among 130 rows)
    assert np.sum(np.any(gc[:, D_C:] != want_c[:, D_C:], axis=1)) <= 1
