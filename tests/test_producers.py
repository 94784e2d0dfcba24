"""GPU parity of the producers (the projections from hidden states to cache
rows and queries) against the float64 oracle, and one chain from hidden
states to the attention output."""
import math

import numpy as np
import pytest

from gpu_util import TOL, rel_err, say
from mla_latent_kv_04_amd.workloads import D_C, D_H, D_R, ROW, ROPE_BASE, round_to_bf16, softmax_scale
from oracle import mla_oracle as orc

pytestmark = pytest.mark.gpu

EPS = 1e-6


def _weights(rng, shape, fan_in, dtype):
    w = (rng.standard_normal(shape) / math.sqrt(fan_in)).astype(np.float32)
    return round_to_bf16(w) if dtype == "bf16" else w


def _dev(x, dtype):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to(torch.bfloat16 if dtype == "bf16" else torch.float32).cuda()


@pytest.mark.parametrize("dtype,d_model", [("bf16", 5120), ("bf16", 2048), ("f32", 256)])
def test_kv_produce_writes_the_oracle_rows(dtype, d_model):
    import torch
    from mla_latent_kv_04_amd import _binding as mla
    rng = np.random.default_rng(d_model)
    T = 150                                           # two row tiles, the second ragged
    h = rng.standard_normal((T, d_model)).astype(np.float32)
    if dtype == "bf16":
        h = round_to_bf16(h)
    w_dkv = _weights(rng, (D_C, d_model), d_model, dtype)
    w_kr = _weights(rng, (D_R, d_model), d_model, dtype)
    gain = (1.0 + 0.1 * rng.standard_normal(D_C)).astype(np.float32)
    # two sequences of four blocks; tokens spread over both, the last two
    # rows out of range (skipped)
    seq = np.where(np.arange(T) % 2 == 0, 0, 1).astype(np.int32)
    pos = (np.arange(T) // 2 * 3 % 256).astype(np.int32)
    pos[np.arange(T) // 2 * 3 >= 256] = 0
    order = np.unique(seq.astype(np.int64) * 1000 + pos, return_index=True)[1]
    keep = np.zeros(T, bool)
    keep[order] = True                                # one token per slot
    seq[~keep] = 7
    seq[-1] = 9
    pos[-2] = -1
    table = np.array([[5, 2, 7, 0], [1, 6, 3, 4]], dtype=np.int32)
    ref_c, ref_k, ref_rows = orc.kv_produce(h, w_dkv, gain, w_kr, pos.clip(0), ROPE_BASE, EPS)

    say(f"kv_produce {dtype} d_model={d_model}")
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    cache = torch.full((8, 64, ROW), float("nan"), dtype=tdt, device="cuda")
    ws = torch.empty(mla.mla_kv_produce_workspace(T, d_model), dtype=torch.uint8, device="cuda")
    mla.mla_kv_produce(_dev(h, dtype), _dev(w_dkv, dtype), torch.from_numpy(gain).cuda(),
                       _dev(w_kr, dtype), cache, torch.from_numpy(table).cuda(),
                       torch.from_numpy(seq).cuda(), torch.from_numpy(pos).cuda(), ROPE_BASE, EPS,
                       ws)
    torch.cuda.synchronize()
    got = cache.float().cpu().numpy().reshape(-1, ROW).astype(np.float64)
    written = np.zeros(got.shape[0], bool)
    for r in range(T):
        if not (0 <= seq[r] < 2 and 0 <= pos[r] < 256):
            continue
        slot = table[seq[r], pos[r] // 64] * 64 + pos[r] % 64
        written[slot] = True
        row, ref = got[slot], ref_rows[r]
        if dtype == "bf16":
            # fp32 products and RMSNorm, then one rounding to bf16
            assert np.all(np.abs(row - ref) <= np.abs(ref) * 2.0 ** -8 + 1e-4), r
        else:
            np.testing.assert_allclose(row, ref, rtol=2e-5, atol=2e-5 * np.abs(ref).max())
    assert np.isnan(got[~written]).all()              # nothing else was written
    assert written.sum() == int((keep & (seq < 2) & (pos >= 0)).sum())


@pytest.mark.parametrize("dtype,d_model,d_cq,n_h", [("bf16", 5120, 1536, 16), ("f32", 256, 128, 2)])
def test_q_produce_matches_oracle(dtype, d_model, d_cq, n_h):
    import torch
    from mla_latent_kv_04_amd import _binding as mla
    rng = np.random.default_rng(d_cq)
    T = 130
    h = rng.standard_normal((T, d_model)).astype(np.float32)
    if dtype == "bf16":
        h = round_to_bf16(h)
    w_dq = _weights(rng, (d_cq, d_model), d_model, dtype)
    w_uq = _weights(rng, (n_h * D_H, d_cq), d_cq, dtype)
    w_qr = _weights(rng, (n_h * D_R, d_cq), d_cq, dtype)
    gain = (1.0 + 0.1 * rng.standard_normal(d_cq)).astype(np.float32)
    c_q, ref_n, ref_r = orc.q_produce(h, w_dq, gain, w_uq, w_qr, n_h, EPS)

    say(f"q_produce {dtype} d_model={d_model} d_cq={d_cq}")
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    q_nope = torch.empty((T, n_h, D_H), dtype=tdt, device="cuda")
    q_rope = torch.empty((T, n_h, D_R), dtype=tdt, device="cuda")
    code = 1 if dtype == "bf16" else 0
    ws = torch.empty(mla.mla_q_produce_workspace(T, d_model, d_cq, code), dtype=torch.uint8,
                     device="cuda")
    mla.mla_q_produce(_dev(h, dtype), _dev(w_dq, dtype), torch.from_numpy(gain).cuda(),
                      _dev(w_uq, dtype), _dev(w_qr, dtype), q_nope, q_rope, EPS, ws)
    torch.cuda.synchronize()
    got_n = q_nope.float().cpu().numpy().astype(np.float64)
    got_r = q_rope.float().cpu().numpy().astype(np.float64)
    if dtype == "f32":
        assert rel_err(got_n, ref_n) <= 1e-5 and rel_err(got_r, ref_r) <= 1e-5
        return
    assert rel_err(got_n, ref_n) <= TOL["bf16"] and rel_err(got_r, ref_r) <= TOL["bf16"]
    # with c^Q rounded to bf16 as the kernel stores it, what is left is one
    # rounding of each output, fp32 accumulation, and the few c^Q elements
    # (about 1 in 5000) whose fp32 value rounds the other way: each moves an
    # output by a fraction of an ulp of c^Q times one weight, well under
    # 2^-9 of the output's RMS
    cq16 = round_to_bf16(c_q.astype(np.float32)).astype(np.float64)
    for got, w, d in ((got_n, w_uq, D_H), (got_r, w_qr, D_R)):
        want = (cq16 @ w.astype(np.float64).T).reshape(T, n_h, d)
        rms = np.sqrt((want ** 2).mean())
        assert np.all(np.abs(got - want) <= np.abs(want) * 2.0 ** -8 + rms * 2.0 ** -9)


@pytest.mark.parametrize("dtype,d_model,n_h", [("bf16", 2048, 16), ("f32", 256, 2)])
def test_direct_query_producer_matches_oracle(dtype, d_model, n_h):
    """Queries of a model without query compression (V2-Lite's widths in
    bf16: hidden 2048, 16 heads)."""
    import torch
    from mla_latent_kv_04_amd import _binding as mla
    rng = np.random.default_rng(d_model + n_h)
    T = 150                                           # two 128-row tiles, the second ragged
    h = rng.standard_normal((T, d_model)).astype(np.float32)
    if dtype == "bf16":
        h = round_to_bf16(h)
    w_qc = _weights(rng, (n_h * D_H, d_model), d_model, dtype)
    w_qr = _weights(rng, (n_h * D_R, d_model), d_model, dtype)
    ref_n, ref_r = orc.q_produce_direct(h, w_qc, w_qr, n_h)
    say(f"q_produce_direct {dtype} d_model={d_model} n_h={n_h}")
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    q_nope = torch.empty((T, n_h, D_H), dtype=tdt, device="cuda")
    q_rope = torch.empty((T, n_h, D_R), dtype=tdt, device="cuda")
    mla.mla_q_produce_direct(_dev(h, dtype), _dev(w_qc, dtype), _dev(w_qr, dtype), q_nope, q_rope)
    torch.cuda.synchronize()
    for got, ref in ((q_nope, ref_n), (q_rope, ref_r)):
        g = got.float().cpu().numpy().astype(np.float64)
        if dtype == "bf16":
            # fp32 products, one rounding of each output
            rms = np.sqrt(np.mean(ref ** 2))
            assert np.all(np.abs(g - ref) <= np.abs(ref) * 2.0 ** -8 + rms * 1e-4)
        else:
            assert rel_err(g, ref) <= 1e-5


@pytest.mark.parametrize("dtype,T,n_h,d_model", [("bf16", 128, 128, 5120), ("bf16", 130, 128, 5120),
                                                 ("bf16", 37, 128, 5120), ("f32", 33, 2, 192)])
def test_o_proj_matches_oracle(dtype, T, n_h, d_model):
    """eq. 8's u = W^O [o_1; ...; o_nh]: at the V2 shape (128 tokens, 128 heads,
    hidden 5120: K split over workgroups, 128-row tiles, a shorter last
    slice), with a ragged second row tile (130), with 64-row tiles (37), and a
    small fp32 case."""
    import torch
    from mla_latent_kv_04_amd import _binding as mla
    rng = np.random.default_rng(T + n_h)
    out = rng.standard_normal((T, n_h, D_H)).astype(np.float32)
    w_o = _weights(rng, (d_model, n_h * D_H), n_h * D_H, dtype)
    ref = orc.o_projection(out, w_o)
    say(f"o_proj {dtype} T={T} n_h={n_h} d_model={d_model}")
    code = 1 if dtype == "bf16" else 0
    u = torch.empty((T, d_model), dtype=torch.bfloat16 if dtype == "bf16" else torch.float32,
                    device="cuda")
    n = mla.mla_o_proj_workspace(T, n_h, d_model, code)
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device="cuda")
    mla.mla_o_proj(torch.from_numpy(out).cuda(), _dev(w_o, dtype), u, ws)
    torch.cuda.synchronize()
    got = u.float().cpu().numpy().astype(np.float64)
    assert ref.size <= 1 << 20
    if dtype == "bf16":
        # out rounded to bf16 once, fp32 accumulation, u rounded to bf16
        assert rel_err(got, ref) <= TOL["bf16"]
        cast = round_to_bf16(out).astype(np.float64)
        want = orc.o_projection(cast, w_o)
        rms = np.sqrt(np.mean(want ** 2))
        assert np.all(np.abs(got - want) <= np.abs(want) * 2.0 ** -8 + rms * 1e-4)
    else:
        assert rel_err(got, ref) <= 1e-5


def test_hidden_states_to_attention_output():
    """Cache rows and the query produced from hidden states, then absorb,
    attention and out-projection, against the oracle's producers followed by
    its non-absorbed attention."""
    import torch
    from mla_latent_kv_04_amd import _binding as mla
    rng = np.random.default_rng(11)
    d_model, d_cq, n_h, L = 1024, 512, 64, 200
    h_kv = round_to_bf16(rng.standard_normal((L, d_model)).astype(np.float32))
    h_q = round_to_bf16(rng.standard_normal((1, d_model)).astype(np.float32))
    w_dkv = _weights(rng, (D_C, d_model), d_model, "bf16")
    w_kr = _weights(rng, (D_R, d_model), d_model, "bf16")
    w_dq = _weights(rng, (d_cq, d_model), d_model, "bf16")
    w_uq = _weights(rng, (n_h * D_H, d_cq), d_cq, "bf16")
    w_qr = _weights(rng, (n_h * D_R, d_cq), d_cq, "bf16")
    w_uk = _weights(rng, (n_h, D_H, D_C), D_C, "bf16")
    w_uv = _weights(rng, (n_h, D_H, D_C), D_C, "bf16")
    g_kv = (1.0 + 0.1 * rng.standard_normal(D_C)).astype(np.float32)
    g_q = (1.0 + 0.1 * rng.standard_normal(d_cq)).astype(np.float32)

    c_kv, k_r, _ = orc.kv_produce(h_kv, w_dkv, g_kv, w_kr, np.arange(L), ROPE_BASE, EPS)
    _, q_nope, q_rope = orc.q_produce(h_q, w_dq, g_q, w_uq, w_qr, n_h, EPS)
    ref, _, _ = orc.mla_attention_naive(c_kv, k_r, q_nope, q_rope, w_uk, w_uv, np.arange(L),
                                        np.array([L]), [L], softmax_scale(), ROPE_BASE)

    say("hidden states -> attention output")
    bf = torch.bfloat16
    nblk = (L + 63) // 64
    cache = torch.full((nblk, 64, ROW), float("nan"), dtype=bf, device="cuda")
    table = torch.from_numpy(np.random.default_rng(3).permutation(nblk).astype(np.int32)[None]).cuda()
    ws = torch.empty(mla.mla_kv_produce_workspace(L, d_model), dtype=torch.uint8, device="cuda")
    mla.mla_kv_produce(_dev(h_kv, "bf16"), _dev(w_dkv, "bf16"), torch.from_numpy(g_kv).cuda(),
                       _dev(w_kr, "bf16"), cache, table,
                       torch.zeros(L, dtype=torch.int32, device="cuda"),
                       torch.arange(L, dtype=torch.int32, device="cuda"), ROPE_BASE, EPS, ws)
    qn = torch.empty((1, n_h, D_H), dtype=bf, device="cuda")
    qr = torch.empty((1, n_h, D_R), dtype=bf, device="cuda")
    wsq = torch.empty(mla.mla_q_produce_workspace(1, d_model, d_cq, 1), dtype=torch.uint8,
                      device="cuda")
    mla.mla_q_produce(_dev(h_q, "bf16"), _dev(w_dq, "bf16"), torch.from_numpy(g_q).cuda(),
                      _dev(w_uq, "bf16"), _dev(w_qr, "bf16"), qn, qr, EPS, wsq)
    q_lat = torch.empty((1, n_h, ROW), dtype=bf, device="cuda")
    mla.mla_absorb_q(qn, qr, _dev(w_uk, "bf16"), torch.tensor([L], dtype=torch.int32).cuda(),
                     q_lat, ROPE_BASE)
    o_lat = torch.empty((1, n_h, D_C), device="cuda")
    lse = torch.empty((1, n_h), device="cuda")
    mla.mla_decode_paged(q_lat, cache, table, torch.tensor([L], dtype=torch.int32).cuda(), 1,
                         softmax_scale(), 1, o_lat=o_lat, lse=lse)
    out = torch.empty((1, n_h, D_H), device="cuda")
    mla.mla_out_proj(o_lat, _dev(w_uv, "bf16"), out)
    torch.cuda.synchronize()
    assert rel_err(out.cpu().numpy(), ref) <= TOL["bf16"]
