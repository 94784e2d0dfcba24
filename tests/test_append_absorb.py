"""mla_append_absorb_q through the C ABI against mla_kv_append followed by
mla_absorb_q on the same inputs: the fused launch runs the same per-row and
per-tile code, so the cache and the latent queries must match bit for bit.
Cases cover each absorb tiling (1, 2 and 4 column tiles per workgroup), fp32
(the two launches), rows the append must skip, and either part empty."""
import numpy as np
import pytest

from gpu_util import say, small
from mla_latent_kv_04_amd import _binding as mla
from mla_latent_kv_04_amd import pipeline
from mla_latent_kv_04_amd.workloads import ROPE_BASE

pytestmark = pytest.mark.gpu

# (workload, overrides): 16 heads x 3 rows (one tile per workgroup), 128 heads
# x 2 rows (two), a 1100-row chunk of 128 heads (four, with 1100 appended rows)
# and the fp32 configuration
CASES = [
    ("v2lite_bf16_B64_L4096", dict(B=3, ctx=[900, 64, 333])),
    ("v2_bf16_B4_L128k_splitkv", dict(B=2, ctx=[1900, 700])),
    ("v2_bf16_prefill_6144+2048", dict(ctx=1200, q_len=1100)),
    ("v2lite_f32_L256", dict()),
]


def _bits(t):
    import torch
    return (t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)).cpu().numpy()


def _separate(dp, seq):
    mla.mla_kv_append(dp.kv_cache, dp.block_table, dp.new_c_kv, dp.new_k_r, seq, dp.new_pos,
                      ROPE_BASE)
    mla.mla_absorb_q(dp.q_nope, dp.q_rope, dp.w_uk, dp.q_pos, dp.q_lat, ROPE_BASE)


def _fused(dp, seq):
    mla.mla_append_absorb_q(dp.kv_cache, dp.block_table, dp.new_c_kv, dp.new_k_r, seq,
                            dp.new_pos, dp.q_nope, dp.q_rope, dp.w_uk, dp.q_pos, dp.q_lat,
                            ROPE_BASE)


@pytest.mark.parametrize("name,kw", CASES, ids=["h16", "h128", "chunk1100", "f32"])
def test_fused_launch_matches_the_two_calls(name, kw):
    import torch
    prob = small(name, **kw)
    a = pipeline.upload(prob, num_splits=1)
    b = pipeline.upload(prob, num_splits=1)
    for dp in (a, b):
        dp.q_lat.fill_(float("nan"))
    # one row aimed at a sequence that does not exist: both forms skip it
    seq = a.new_seq.clone()
    seq[seq.shape[0] // 2] = -1
    say(f"append+absorb {name}: separate calls")
    _separate(a, seq)
    say(f"append+absorb {name}: fused launch")
    _fused(b, seq)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(a.kv_cache), _bits(b.kv_cache))
    assert np.array_equal(_bits(a.q_lat), _bits(b.q_lat))
    assert not torch.isnan(b.q_lat).any()


def test_either_part_may_be_empty():
    import torch
    prob = small("v2_bf16_B4_L128k_splitkv", B=2, ctx=[1900, 700])
    a = pipeline.upload(prob, num_splits=1)
    b = pipeline.upload(prob, num_splits=1)
    empty_q = b.q_nope[:0]
    # no queries: the fused call only appends
    say("append+absorb: no queries")
    mla.mla_kv_append(a.kv_cache, a.block_table, a.new_c_kv, a.new_k_r, a.new_seq, a.new_pos,
                      ROPE_BASE)
    mla.mla_append_absorb_q(b.kv_cache, b.block_table, b.new_c_kv, b.new_k_r, b.new_seq,
                            b.new_pos, empty_q, b.q_rope[:0], b.w_uk, b.q_pos[:0], b.q_lat[:0],
                            ROPE_BASE)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(a.kv_cache), _bits(b.kv_cache))
    # no rows: the fused call only absorbs
    say("append+absorb: no rows")
    a.q_lat.fill_(float("nan"))
    b.q_lat.fill_(float("nan"))
    mla.mla_absorb_q(a.q_nope, a.q_rope, a.w_uk, a.q_pos, a.q_lat, ROPE_BASE)
    mla.mla_append_absorb_q(b.kv_cache, b.block_table, b.new_c_kv[:0], b.new_k_r[:0],
                            b.new_seq[:0], b.new_pos[:0], b.q_nope, b.q_rope, b.w_uk, b.q_pos,
                            b.q_lat, ROPE_BASE)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(a.q_lat), _bits(b.q_lat))
    assert np.array_equal(_bits(a.kv_cache), _bits(b.kv_cache))
