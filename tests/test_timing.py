"""mla_time_attention through the C ABI: the attention kernel of the next
decode call records the armed events itself.  The armed launch computes the
same results bit for bit as an unarmed one (same kernel, same grid), the
events hold a plausible duration, and a call that launches nothing leaves
the events armed for the next one."""
import math

import numpy as np
import pytest

from gpu_util import say, small, to_np
from mla_latent_kv_04_amd import _binding as mla
from mla_latent_kv_04_amd import pipeline
from mla_latent_kv_04_amd.workloads import D_C, softmax_scale

pytestmark = pytest.mark.gpu

# (workload, problem overrides, cache): the four attention kernels (bf16 and
# FP8 caches, 64-head groups and 16 heads)
CASES = [
    ("v2_bf16_B4_L128k_splitkv", dict(B=2, ctx=[1900, 700]), "native"),
    ("v2lite_bf16_B64_L4096", dict(B=3, ctx=[900, 64, 333]), "native"),
    ("v2_bf16_B4_L128k_splitkv", dict(B=2, ctx=[1900, 700]), "fp8"),
    ("v2lite_bf16_B64_L4096", dict(B=3, ctx=[900, 64, 333]), "fp8"),
]


def _prepared(name, cache, **kw):
    import torch
    prob = small(name, **kw)
    dp = pipeline.upload(prob, num_splits=1, cache=cache)
    pipeline.append(dp)   # the step's own rows (poisoned until appended)
    mla.mla_absorb_q(dp.q_nope, dp.q_rope, dp.w_uk, dp.q_pos, dp.q_lat)
    torch.cuda.synchronize()
    return dp


def _attend(dp, cache, scale=None):
    import torch
    rows = dp.B * dp.q_len
    o_lat = torch.full((rows, dp.n_h, D_C), float("nan"), device="cuda")
    lse = torch.full((rows, dp.n_h), float("nan"), device="cuda")
    s = softmax_scale() if scale is None else scale
    if cache == "fp8":
        mla.mla_decode_paged_fp8(dp.q_lat, dp.kv_cache, dp.kv_scale, dp.block_table, dp.seq_lens,
                                 dp.q_len, s, 1, o_lat=o_lat, lse=lse)
    else:
        mla.mla_decode_paged(dp.q_lat, dp.kv_cache, dp.block_table, dp.seq_lens, dp.q_len, s, 1,
                             o_lat=o_lat, lse=lse)
    return o_lat, lse


@pytest.mark.parametrize("name,kw,cache", CASES,
                         ids=["h128-bf16", "h16-bf16", "h128-fp8", "h16-fp8"])
def test_armed_launch_records_its_own_duration(name, kw, cache):
    import torch
    dp = _prepared(name, cache, **kw)
    say(f"timing {name} {cache}: unarmed launch")
    o_ref, l_ref = _attend(dp, cache)
    torch.cuda.synchronize()
    timer = mla.KernelTimer()
    try:
        say(f"timing {name} {cache}: armed launch")
        timer.arm()
        o_got, l_got = _attend(dp, cache)
        ms = timer.elapsed_ms()
        torch.cuda.synchronize()
        o_ref, l_ref = to_np(o_ref), to_np(l_ref)
        assert np.isfinite(o_ref).all() and np.isfinite(l_ref).all()
        assert np.array_equal(to_np(o_got), o_ref)
        assert np.array_equal(to_np(l_got), l_ref)
        # a few thousand keys on a handful of workgroups: microseconds, not seconds
        assert math.isfinite(ms) and 0.0 < ms < 1000.0, ms
    finally:
        timer.close()


def test_call_without_launch_leaves_the_events_armed():
    import torch
    dp = _prepared("v2lite_bf16_B64_L4096", "native", B=3, ctx=[900, 64, 333])
    timer = mla.KernelTimer()
    try:
        timer.arm()
        # rejected on the host (softmax scale <= 0): nothing is launched
        with pytest.raises(mla.MLAError):
            _attend(dp, "native", scale=-1.0)
        say("timing: launch after a rejected call")
        _attend(dp, "native")
        ms = timer.elapsed_ms()
        torch.cuda.synchronize()
        assert math.isfinite(ms) and 0.0 < ms < 1000.0, ms
    finally:
        timer.close()
        mla.mla_time_attention(None, None)


def test_planned_and_noalloc_launches_record_their_events():
    """The balanced-plan entry point and the allocation-free one launch their
    attention kernel through the same armed path."""
    import torch
    prob = small("v2_bf16_B4_L128k_splitkv", B=2, ctx=[1900, 700])
    dp = pipeline.upload(prob, num_splits=0)
    pipeline.append(dp)
    mla.mla_absorb_q(dp.q_nope, dp.q_rope, dp.w_uk, dp.q_pos, dp.q_lat)
    torch.cuda.synchronize()
    timer = mla.KernelTimer()
    try:
        say("timing: planned launch")
        timer.arm()
        pipeline._attend_planned(dp)
        ms = timer.elapsed_ms()
        assert math.isfinite(ms) and 0.0 < ms < 1000.0, ms
        say("timing: allocation-free launch")
        rows = dp.B * dp.q_len
        o_lat = torch.empty((rows, dp.n_h, D_C), device="cuda")
        lse = torch.empty((rows, dp.n_h), device="cuda")
        timer.arm()
        mla.mla_decode_paged_noalloc(dp.q_lat, dp.kv_cache, dp.block_table, dp.seq_lens,
                                     dp.q_len, softmax_scale(), 3, o_lat, lse)
        ms = timer.elapsed_ms()
        torch.cuda.synchronize()
        assert math.isfinite(ms) and 0.0 < ms < 1000.0, ms
        assert torch.isfinite(o_lat).all()
    finally:
        timer.close()
        mla.mla_time_attention(None, None)
