#!/usr/bin/env python3
"""Benchmark one pass of the MLA hot path on one MI355X.

A step = append the step's new latent rows, absorb W^UK into the queries,
attend over the paged cache (split-KV), merge the splits, apply W^UV, on one
batch of seeded synthetic input already resident in HBM.  Default workload:
full DeepSeek-V2 head shape decode (B = 128 sequences, 128 heads, context
lengths uniform in [1024, 8192], paged blocks of 64 tokens, bf16).

Prints ONE JSON line.  ``value`` is query tokens per second of the whole step.
``roofline`` covers the dominant kernel (the paged attention kernel): its
algorithmic bytes (or FLOPs) per launch divided by its mean launch time,
measured with HIP events on the stream it runs on.  ``cpu_baseline`` times the
float64 CPU oracle on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0         # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
MFMA_F32_PEAK_TFLOPS = 157.3

# sources of the attention kernels; the committed HBM-traffic record is only
# used while these are unchanged
DECODE_SOURCES = ["mla_latent_kv_04_amd/csrc/decode.hip", "mla_latent_kv_04_amd/csrc/decode_h64.hip",
                  "mla_latent_kv_04_amd/csrc/mla_common.h", "mla_latent_kv_04_amd/csrc/mla_api.cpp"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_sha() -> str:
    h = hashlib.sha256()
    for p in DECODE_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def algorithmic_work(prob):
    """(bytes, flops) one attention-kernel launch must move / perform.

    Bytes: every visible cached row once (576 elements), the latent queries
    once, and the fp32 output (512 + 1 per row and head).  FLOPs: 2 * 576 for
    the score plus 2 * 512 for the weighted sum, per (query row, head, key).
    """
    import numpy as np
    wl = prob.wl
    esz = 2 if wl.dtype == "bf16" else 4
    keys_read = int(np.sum(prob.seq_lens.astype(np.int64)))          # each row read once
    pairs = 0
    for b in range(wl.B):
        L = int(prob.seq_lens[b])
        q = wl.q_len
        pairs += sum(max(0, L - (q - 1 - m)) for m in range(q))
    T = prob.T
    by = keys_read * 576 * esz + T * wl.n_h * 576 * esz + T * wl.n_h * 513 * 4
    fl = pairs * wl.n_h * (2 * 576 + 2 * 512)
    return by, fl


def load_traffic(workload: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", f"decode_traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha") != source_sha():
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(prob, budget_s: float):
    """Time the float64 oracle on whole sequences (all heads) until the budget
    is spent; returns tokens/s over the sample."""
    import numpy as np
    from oracle import mla_oracle as orc
    from mla_latent_kv_04_amd.workloads import ROPE_BASE, softmax_scale
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    wl = prob.wl
    q = wl.q_len
    done_rows = 0
    done_seqs = 0
    keys = 0
    t0 = time.perf_counter()
    rows_per_call = q if q == 1 else max(1, min(q, 16))
    for b in range(wl.B):
        c, k = prob.seq_rows(b)
        L = int(prob.seq_lens[b])
        vis = orc.visible_keys(L, q)
        sl = slice(b * q, b * q + rows_per_call)
        orc.mla_attention_naive(c[:L], k[:L], prob.q_nope[sl], prob.q_rope[sl], prob.w_uk,
                                prob.w_uv, np.arange(L), prob.q_pos[sl], vis[:rows_per_call],
                                softmax_scale(), ROPE_BASE)
        done_rows += rows_per_call
        done_seqs += 1
        keys += L
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    sample = (f"{done_seqs} of {wl.B} sequences, {done_rows} query rows x {wl.n_h} heads, "
              f"{keys} cached keys; non-absorbed float64 NumPy oracle")
    return {"value": done_rows / dt, "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle", "sample": sample, "seconds": round(dt, 2)}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    # the device needs a few hundred steps (~0.1 s) to settle its clocks and
    # caches; the timed region is then steady state
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--workload", default="v2_bf16_B128_L1k-8k")
    ap.add_argument("--splits", type=int, default=None,
                    help="split-KV partitions per row; 0 = balanced work plan (default: workload's)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="first run one plain device-to-device copy of this many bytes (a "
                         "known-size reference for hardware byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(across GPUs the attention would shard by sequence or key range).",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from mla_latent_kv_04_amd import _binding as mla
    from mla_latent_kv_04_amd import pipeline
    from mla_latent_kv_04_amd.workloads import ROPE_BASE, WORKLOADS, make_problem, softmax_scale

    wl = WORKLOADS[args.workload]
    splits = args.splits if args.splits is not None else wl.num_splits
    log(f"[bench] generating {wl.name} (splits={splits})")
    prob = make_problem(wl)
    torch.cuda.set_device(0)
    dp = pipeline.upload(prob, num_splits=splits)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    scale = softmax_scale()

    def one_step(ev=None):
        mla.mla_kv_append(dp.kv_cache, dp.block_table, dp.new_c_kv, dp.new_k_r, dp.new_seq,
                          dp.new_pos, ROPE_BASE)
        mla.mla_absorb_q(dp.q_nope, dp.q_rope, dp.w_uk, dp.q_pos, dp.q_lat, ROPE_BASE)
        if ev is not None:
            ev[0].record(stream)
        if splits == 0:
            mla.mla_decode_paged_planned(dp.q_lat, dp.kv_cache, dp.block_table, dp.B, dp.q_len,
                                         scale, dp.work, dp.o_lat, dp.lse, o_part=dp.o_part,
                                         lse_part=dp.lse_part, lists=dp.lists)
        elif splits > 1:
            mla.mla_decode_paged(dp.q_lat, dp.kv_cache, dp.block_table, dp.seq_lens, dp.q_len,
                                 scale, splits, o_part=dp.o_part, lse_part=dp.lse_part)
        else:
            mla.mla_decode_paged(dp.q_lat, dp.kv_cache, dp.block_table, dp.seq_lens, dp.q_len,
                                 scale, 1, o_lat=dp.o_lat, lse=dp.lse)
        if ev is not None:
            ev[1].record(stream)
        if splits == 0:
            # the split rows' merge runs inside the projection's loads
            mla.mla_out_proj_planned(dp.o_lat, dp.o_part, dp.lse_part, dp.split, dp.w_uv,
                                     dp.out, dp.lse)
            return
        if splits > 1:
            mla.mla_splitkv_combine(dp.o_part, dp.lse_part, dp.B, splits, dp.q_len, dp.n_h,
                                    dp.o_lat, dp.lse)
        mla.mla_out_proj(dp.o_lat, dp.w_uv, dp.out)

    if args.copy_bytes > 0:
        n = args.copy_bytes // 4
        src = torch.arange(n, dtype=torch.int32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] reference copy of {4 * n} bytes done")
        del src, dst

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()
    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        one_step(events[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    dec_ms = float(np.mean([a.elapsed_time(b) for a, b in events]))
    tokens = prob.T
    value = tokens / (ms_per_step * 1e-3)

    by, fl = algorithmic_work(prob)
    compute_bound = wl.q_len > 1
    mfma_peak = MFMA_BF16_PEAK_TFLOPS if wl.dtype == "bf16" else MFMA_F32_PEAK_TFLOPS
    gbs = by / (dec_ms * 1e-3) / 1e9
    tflops = fl / (dec_ms * 1e-3) / 1e12
    traffic = load_traffic(wl.name)
    if compute_bound:
        roof = {"bound": "mfma", "achieved": round(tflops, 2), "peak": mfma_peak,
                "unit": "TFLOP/s", "frac": round(tflops / mfma_peak, 4), "traffic": traffic}
    else:
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic}
    log(f"[bench] step {ms_per_step:.4f} ms, attention kernel {dec_ms * 1e3:.1f} us, "
        f"{gbs:.0f} GB/s, {tflops:.1f} TFLOP/s")

    cpu = None
    if not args.no_cpu_baseline:
        log(f"[bench] cpu baseline (~{args.cpu_seconds} s)")
        cpu = cpu_baseline(prob, args.cpu_seconds)

    cfg = {"workload": wl.name, "B": wl.B, "n_h": wl.n_h, "q_len": wl.q_len,
           "context": (f"U[{wl.ctx[0]},{wl.ctx[1]}]" if isinstance(wl.ctx, tuple) else wl.ctx),
           "block_size": wl.block_size,
           "split_kv": ("balanced plan" if splits == 0 else f"{splits} per row"),
           "work_items": (int(dp.work.shape[0]) if splits == 0 else dp.B * dp.q_len * splits),
           "d_c": 512, "d_R": 64, "d_h": 128}
    rec = {
        "metric": "MLA decode tokens/s (+ attention-kernel HBM GB/s and MFMA share of peak), "
                  "DeepSeek-V2 head shape",
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": wl.dtype, "data": "synthetic",
        "config": cfg, "roofline": roof,
        "attention_kernel": {"us_per_launch": round(dec_ms * 1e3, 2),
                             "algorithmic_bytes": by, "algorithmic_flops": fl,
                             "hbm_gbs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                             "mfma_tflops": round(tflops, 1),
                             "mfma_frac": round(tflops / mfma_peak, 4),
                             "source_sha": source_sha()},
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
