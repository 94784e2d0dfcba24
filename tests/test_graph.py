"""The step under HIP graph capture: the benchmark replays a graph of one step
(append, absorb, attention, merge + W^UV).  Every replay must give the eager
step's outputs bit for bit, with eager work and synchronisations between the
replays (the outputs are cleared eagerly before each replay)."""
import numpy as np
import pytest

from gpu_util import say, small, to_np
from mla_latent_kv_04_amd import pipeline

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("wl,kw,S,cache", [
    ("v2_bf16_B128_L1k-8k", dict(B=3, ctx=[1500, 64, 700]), 0, "native"),
    ("v2lite_bf16_B64_L4096", dict(B=4, ctx=[3000, 1, 900, 64]), 0, "fp8"),
    ("v2lite_bf16_B64_L4096", dict(B=3, ctx=[700, 65, 2000]), 3, "native"),
], ids=["v2-planned", "lite-fp8-planned", "lite-split3"])
def test_graph_replays_match_the_eager_step(wl, kw, S, cache):
    import torch
    prob = small(wl, **kw)
    say(f"graph {wl} {kw} S={S} cache={cache}")
    dp = pipeline.upload(prob, num_splits=S, cache=cache)
    pipeline.step(dp)
    torch.cuda.synchronize()
    want_out, want_lse = to_np(dp.out), to_np(dp.lse)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        pipeline.step(dp)
    for rep in range(4):
        dp.out.zero_()
        dp.lse.zero_()
        dp.o_lat.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(to_np(dp.out), want_out, err_msg=f"replay {rep}")
        np.testing.assert_array_equal(to_np(dp.lse), want_lse, err_msg=f"replay {rep}")
    del g
