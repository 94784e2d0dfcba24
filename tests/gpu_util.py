"""Helpers shared by the GPU parity tests (no test functions here)."""
import math
import sys

import numpy as np

from mla_latent_kv_04_amd import pipeline
from mla_latent_kv_04_amd.workloads import ROPE_BASE, make_problem, softmax_scale
from oracle import mla_oracle as orc

# Tolerances on max|gpu - oracle| / rms(oracle) for the floating-point results.
TOL = {"f32": 2e-3, "bf16": 2e-2}


def say(msg):
    """Name the case before each GPU step (flushed, so a fault still shows it)."""
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def rel_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), "non-finite GPU output"
    rms = math.sqrt(float(np.mean(ref * ref)))
    return float(np.max(np.abs(got - ref))) / max(rms, 1e-30)


def oracle_sequence(prob, b, heads=None, rows=None):
    """Non-absorbed oracle of sequence b: (out [q, h, 128], lse [q, h], o_lat)."""
    q = prob.wl.q_len
    c, k = prob.seq_rows(b)
    sl = slice(b * q, (b + 1) * q)
    qn, qr, qp = prob.q_nope[sl], prob.q_rope[sl], prob.q_pos[sl]
    L = int(prob.seq_lens[b])
    vis = orc.visible_keys(L, q)
    if rows is not None:
        rows = np.asarray(rows)
        qn, qr, qp, vis = qn[rows], qr[rows], qp[rows], vis[rows]
    wuk, wuv = prob.w_uk, prob.w_uv
    if heads is not None:
        heads = np.asarray(heads)
        qn, qr, wuk, wuv = qn[:, heads], qr[:, heads], wuk[heads], wuv[heads]
    return orc.mla_attention_naive(c[:L], k[:L], qn, qr, wuk, wuv, np.arange(L), qp, vis,
                                   softmax_scale(), ROPE_BASE)


def run_step(prob, num_splits=None):
    import torch
    dp = pipeline.upload(prob, num_splits=num_splits)
    pipeline.step(dp)
    torch.cuda.synchronize()
    return dp


def to_np(t):
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def small(name, **kw):
    from mla_latent_kv_04_amd.workloads import WORKLOADS
    return make_problem(WORKLOADS[name], **kw)
