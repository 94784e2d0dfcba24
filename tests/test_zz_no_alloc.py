"""The allocation-free entry point mla_decode_paged_noalloc against the
entry points it stands for (mla_decode_paged with split partials in a
caller-owned workspace, then mla_splitkv_combine), through the C ABI: the
same kernels run in the same order, so the results must be identical bit for
bit.  Two calls in a row, the second on a smaller problem, so that the
library's scratch array still holds the first call's partials."""
import numpy as np
import pytest

from gpu_util import say, small, to_np
from mla_latent_kv_04_amd import _binding as mla
from mla_latent_kv_04_amd import pipeline
from mla_latent_kv_04_amd.workloads import D_C, softmax_scale

pytestmark = pytest.mark.gpu


def _reference(dp, S):
    """o_lat / lse from mla_decode_paged (caller-owned partials) + combine."""
    import torch
    B, q, n_h = dp.B, dp.q_len, dp.n_h
    o_part = torch.full((B * S * q, n_h, D_C), float("nan"), device="cuda")
    lse_part = torch.full((B * S * q, n_h), float("nan"), device="cuda")
    o_lat = torch.empty((B * q, n_h, D_C), device="cuda")
    lse = torch.empty((B * q, n_h), device="cuda")
    mla.mla_decode_paged(dp.q_lat, dp.kv_cache, dp.block_table, dp.seq_lens, q,
                         softmax_scale(), S, o_part=o_part, lse_part=lse_part)
    mla.mla_splitkv_combine(o_part, lse_part, B, S, q, n_h, o_lat, lse)
    torch.cuda.synchronize()
    return to_np(o_lat), to_np(lse)


def _noalloc(dp, S):
    import torch
    B, q, n_h = dp.B, dp.q_len, dp.n_h
    o_lat = torch.full((B * q, n_h, D_C), float("nan"), device="cuda")
    lse = torch.full((B * q, n_h), float("nan"), device="cuda")
    mla.mla_decode_paged_noalloc(dp.q_lat, dp.kv_cache, dp.block_table, dp.seq_lens, q,
                                 softmax_scale(), S, o_lat, lse)
    torch.cuda.synchronize()
    return to_np(o_lat), to_np(lse)


def _prepared(name, S, **kw):
    """A problem on the device with its latent queries computed (absorb)."""
    import torch
    prob = small(name, **kw)
    dp = pipeline.upload(prob, num_splits=1)
    mla.mla_absorb_q(dp.q_nope, dp.q_rope, dp.w_uk, dp.q_pos, dp.q_lat)
    torch.cuda.synchronize()
    return dp


def test_noalloc_matches_workspace_entry_points_on_two_calls():
    # first call: 128 heads, two sequences, 6 splits (some empty: 1900 keys
    # are 30 blocks, 5 per split; 700 keys leave the last splits empty)
    big = _prepared("v2_bf16_B4_L128k_splitkv", 6, B=2, ctx=[1900, 700])
    say("noalloc call 1: B=2 n_h=128 S=6")
    got1 = _noalloc(big, 6)
    ref1 = _reference(big, 6)
    np.testing.assert_array_equal(got1[0], ref1[0])
    np.testing.assert_array_equal(got1[1], ref1[1])
    assert np.isfinite(got1[0]).all()
    # second call, smaller: one sequence, 16 heads (the other decode kernel),
    # 3 splits; the scratch still holds call 1's partials
    small_dp = _prepared("v2lite_bf16_B64_L4096", 3, B=1, ctx=[333])
    say("noalloc call 2: B=1 n_h=16 S=3")
    got2 = _noalloc(small_dp, 3)
    ref2 = _reference(small_dp, 3)
    np.testing.assert_array_equal(got2[0], ref2[0])
    np.testing.assert_array_equal(got2[1], ref2[1])
    assert np.isfinite(got2[0]).all()


def test_noalloc_refuses_problems_beyond_its_scratch():
    """B * S * q_len * n_h * 513 * 4 bytes above the fixed array: refused with
    MLA_ERR_SCRATCH before anything is enqueued."""
    big = _prepared("v2_bf16_B4_L128k_splitkv", 1, B=2, ctx=[64, 64])
    import torch
    o_lat = torch.empty((2, 128, D_C), device="cuda")
    lse = torch.empty((2, 128), device="cuda")
    S = mla.NOALLOC_SCRATCH_BYTES // (2 * 128 * 513 * 4) + 1
    with pytest.raises(mla.MLAError) as e:
        mla.mla_decode_paged_noalloc(big.q_lat, big.kv_cache, big.block_table, big.seq_lens, 1,
                                     softmax_scale(), S, o_lat, lse)
    assert e.value.status == 6
