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
measured with HIP events on the stream it runs on, recorded by the kernel's
own dispatch (the library's mla_time_attention) over a second pass of as many
steps: the timed steps themselves carry no timing packets.  ``cpu_baseline`` times the float64
CPU oracle on a bounded sample of the same workload.
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
PRODUCER_EPS = 1e-6           # RMSNorm epsilon of the latent and query norms

# sources of the attention kernels; the committed HBM-traffic record is only
# used while these are unchanged
DECODE_SOURCES = ["mla_latent_kv_04_amd/csrc/decode.hip", "mla_latent_kv_04_amd/csrc/decode_h64.hip",
                  "mla_latent_kv_04_amd/csrc/decode_h64_fp8.hip", "mla_latent_kv_04_amd/csrc/decode_h64_common.h",
                  "mla_latent_kv_04_amd/csrc/decode_fp8.hip", "mla_latent_kv_04_amd/csrc/attention_launch.h",
                  "mla_latent_kv_04_amd/csrc/mla_common.h", "mla_latent_kv_04_amd/csrc/mla_api.cpp"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


PREFILL_MHA_SOURCES = ["mla_latent_kv_04_amd/csrc/prefill_mha.hip",
                       "mla_latent_kv_04_amd/csrc/mla_common.h",
                       "mla_latent_kv_04_amd/csrc/produce_api.cpp"]
TRAFFIC_SOURCES = {"decode": DECODE_SOURCES, "prefill_mha": PREFILL_MHA_SOURCES}


def source_sha(kind: str = "decode") -> str:
    h = hashlib.sha256()
    for p in TRAFFIC_SOURCES[kind]:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def algorithmic_work(prob, fp8=False):
    """(bytes, flops) one attention-kernel launch must move / perform.

    Bytes: every visible cached row once (576 elements; with the FP8 cache 576
    code bytes and two float32 scales), the latent queries once, and the fp32
    output (512 + 1 per row and head).  FLOPs: 2 * 576 for the score plus
    2 * 512 for the weighted sum, per (query row, head, key).
    """
    import numpy as np
    wl = prob.wl
    esz = 2 if wl.dtype == "bf16" else 4
    row_bytes = 576 + 8 if fp8 else 576 * esz
    keys_read = int(np.sum(prob.seq_lens.astype(np.int64)))          # each row read once
    pairs = 0
    for b in range(wl.B):
        L = int(prob.seq_lens[b])
        q = wl.q_len
        pairs += sum(max(0, L - (q - 1 - m)) for m in range(q))
    T = prob.T
    by = keys_read * row_bytes + T * wl.n_h * 576 * esz + T * wl.n_h * 513 * 4
    fl = pairs * wl.n_h * (2 * 576 + 2 * 512)
    return by, fl


def load_traffic(workload: str, kind: str = "decode"):
    """HBM bytes per launch of the timed attention kernel from committed
    rocprofv3 counter runs, if they were taken on the current source of that
    kernel (else None).  workload: the workload's name, with "_fp8" for the
    FP8 cache; kind: "decode" (the absorbed attention kernels) or
    "prefill_mha" (the non-absorbed prefill kernel)."""
    path = os.path.join(ROOT, "profiles", f"{kind}_traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha") != source_sha(kind):
        return None
    return rec.get("hbm_bytes_per_launch")


def non_absorbed_flops(prob):
    """FLOPs of one mla_prefill_mha call: the up-projections k^C = W^UK c^KV and
    v^C = W^UV c^KV of every key (2 * 512 * 128 per key, head and matrix),
    then 2 * 192 for the score and 2 * 128 for the weighted sum per visible
    (query row, head, key)."""
    wl = prob.wl
    keys = int(sum(int(L) for L in prob.seq_lens))
    pairs = 0
    for b in range(wl.B):
        L = int(prob.seq_lens[b])
        q = wl.q_len
        pairs += sum(max(0, L - (q - 1 - m)) for m in range(q))
    return 2 * (2 * 512 * 128) * keys * wl.n_h + pairs * wl.n_h * (2 * 192 + 2 * 128)


def producer_work(T, n_h, d_model, d_cq, esz):
    """(kv bytes, q bytes, kv flops, q flops) of the two producers for T tokens.

    Bytes: the hidden states and every weight read once, the gains, and the
    outputs written once (cache rows of 576; q^C and q^R of n_h * 192 per
    token); c^Q's round trip through the workspace is not counted.  FLOPs:
    2 per multiply-add of the projections."""
    kv_w = (512 + 64) * d_model
    if d_cq is None:                      # queries straight from h
        q_w = n_h * (128 + 64) * d_model
        q_by = (T * d_model + q_w + T * n_h * 192) * esz
    else:
        q_w = d_cq * d_model + n_h * (128 + 64) * d_cq
        q_by = (T * d_model + q_w + T * n_h * 192) * esz + d_cq * 4
    kv_by = (T * d_model + kv_w + T * 576) * esz + 512 * 4
    return kv_by, q_by, 2 * T * kv_w, 2 * T * q_w


def cpu_baseline(prob, budget_s: float, hid=None, fp8=False):
    """Time the float64 oracle on whole sequences (all heads) until the budget
    is spent; returns tokens/s over the sample.  With hidden states, each
    sequence's new row and queries come from the oracle's producers first.
    With the FP8 cache, the oracle quantises the sequence's rows and attends
    over their dequantised values (absorbed form)."""
    import numpy as np
    from oracle import mla_oracle as orc
    from mla_latent_kv_04_amd.workloads import ROPE_BASE, softmax_scale
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = None
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
        q_nope, q_rope = prob.q_nope[sl], prob.q_rope[sl]
        if hid is not None:
            # the step's rows are the last q of the sequence, its tokens b q ..
            c, k = c.copy(), k.copy()
            c[L - q:], k[L - q:], _ = orc.kv_produce(hid.h[b * q:(b + 1) * q], hid.w_dkv,
                                                     hid.kv_gain, hid.w_kr,
                                                     np.arange(L - q, L), ROPE_BASE, PRODUCER_EPS)
            if hid.w_qc is not None:
                q_nope, q_rope = orc.q_produce_direct(hid.h[sl], hid.w_qc, hid.w_qr, wl.n_h)
            else:
                _, q_nope, q_rope = orc.q_produce(hid.h[sl], hid.w_dq, hid.q_gain, hid.w_uq,
                                                  hid.w_qr, wl.n_h, PRODUCER_EPS)
        if fp8:
            codes, sc = orc.kv_cache_rows_fp8(c[:L], k[:L], np.arange(L), ROPE_BASE)
            rows = orc.dequantize_rows(codes, sc, 512)
            q_lat = orc.absorb_query(q_nope, q_rope, prob.w_uk, prob.q_pos[sl], ROPE_BASE)
            o_lat, _ = orc.latent_attention(q_lat, rows, vis[:rows_per_call], softmax_scale(),
                                            512)
            o = orc.out_projection(o_lat, prob.w_uv)
        else:
            o, _, _ = orc.mla_attention_naive(c[:L], k[:L], q_nope, q_rope, prob.w_uk,
                                              prob.w_uv, np.arange(L), prob.q_pos[sl],
                                              vis[:rows_per_call], softmax_scale(), ROPE_BASE)
        if hid is not None and hid.w_o is not None:
            orc.o_projection(o, hid.w_o)                  # eq. 8, as the step ends
        done_rows += rows_per_call
        done_seqs += 1
        keys += L
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    sample = (f"{done_seqs} of {wl.B} sequences, {done_rows} query rows x {wl.n_h} heads, "
              f"{keys} cached keys; "
              + ("float64 NumPy oracle: quantise, dequantise, absorbed attention" if fp8 else
                 "non-absorbed float64 NumPy oracle"))
    return {"value": done_rows / dt, "unit": "tokens/s", "cores": cores,
            "blas_threads": threads, "kind": "oracle", "sample": sample,
            "seconds": round(dt, 2)}


def spread(xs):
    """Mean, median, 10th and 90th percentile of a list of times (ms -> us)."""
    import numpy as np
    a = np.asarray(xs, dtype=np.float64) * 1e3
    return {"mean": round(float(a.mean()), 2), "median": round(float(np.median(a)), 2),
            "p10": round(float(np.percentile(a, 10)), 2),
            "p90": round(float(np.percentile(a, 90)), 2), "n": int(a.size)}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    # the device needs a few hundred steps (~0.1 s) to settle its clocks and
    # caches; the timed region is then steady state
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=300)
    # after the requested warm-up, untimed steps continue until this much wall
    # time has passed: a fresh device raises its clocks over the first tens of
    # milliseconds of load, and a short warm-up would time that ramp
    ap.add_argument("--settle-seconds", type=float, default=0.5)
    ap.add_argument("--cold-steps", type=int, default=20,
                    help="extra steps, each after a 1 GiB write that evicts the caches, "
                         "timed separately (reported as cold; 0 = skip)")
    ap.add_argument("--workload", default="v2_bf16_B128_L1k-8k")
    ap.add_argument("--q-len", type=int, default=None,
                    help="query rows per sequence instead of the workload's (the rows are the "
                         "last ones of each sequence; for the absorbed / non-absorbed crossover)")
    ap.add_argument("--splits", type=int, default=None,
                    help="split-KV partitions per row; 0 = balanced work plan (default: workload's)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--attention", choices=("absorbed", "non-absorbed"), default="absorbed",
                    help="chunked prefill only: non-absorbed = per-head keys and values, then "
                         "attention (mla_prefill_mha)")
    ap.add_argument("--from-hidden", action="store_true",
                    help="start the step from hidden states: the cache-row and query producers "
                         "(V2 or V2-Lite widths) replace the append and the given queries")
    ap.add_argument("--cache", choices=("native", "fp8"), default="native",
                    help="latent cache format: the workload's dtype, or FP8 E4M3 codes with two "
                         "float32 scales per row (bf16 absorbed decode workloads)")
    ap.add_argument("--launch", choices=("replay", "eager", "graph"), default="replay",
                    help="replay: the step's library calls are marshalled once and re-issued "
                         "each step without the Python wrappers' checks; eager: through the "
                         "wrappers every step; graph: the timed steps replay a HIP graph of "
                         "one step and the attention kernel is timed over replays of a graph "
                         "of that kernel alone")
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
    from mla_latent_kv_04_amd.workloads import (D_CQ_V2, D_MODEL_LITE, D_MODEL_V2, ROPE_BASE,
                                                WORKLOADS, make_hidden, make_problem,
                                                softmax_scale)

    wl = WORKLOADS[args.workload]
    if args.q_len is not None:
        import dataclasses
        wl = dataclasses.replace(wl, q_len=int(args.q_len))
    non_absorbed = args.attention == "non-absorbed"
    if non_absorbed and wl.dtype != "bf16":
        print("--attention non-absorbed is for bf16 workloads", file=sys.stderr)
        sys.exit(2)
    fp8 = args.cache == "fp8"
    if fp8 and (wl.dtype != "bf16" or non_absorbed or args.from_hidden):
        print("--cache fp8 is for bf16 workloads in the absorbed form, from latent rows",
              file=sys.stderr)
        sys.exit(2)
    # V2 (128 heads): hidden 5120, queries through c^Q (1536); V2-Lite (16
    # heads): hidden 2048, queries straight from h
    d_model, d_cq = (D_MODEL_V2, D_CQ_V2) if wl.n_h == 128 else (D_MODEL_LITE, None)
    splits = args.splits if args.splits is not None else wl.num_splits
    log(f"[bench] generating {wl.name} (splits={splits})")
    prob = make_problem(wl)
    torch.cuda.set_device(0)
    dp = pipeline.upload(prob, num_splits=splits, cache=args.cache)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    scale = softmax_scale()
    hid = hw = None
    if args.from_hidden:
        log("[bench] generating hidden states and producer weights")
        hid = make_hidden(prob, d_model, d_cq)
        hw = {k: (torch.from_numpy(v).cuda() if k.endswith("gain")
                  else pipeline._to_device(v, dp.dtype, "cuda"))
              for k, v in vars(hid).items() if v is not None}
        code = 1 if wl.dtype == "bf16" else 0
        hw["ws_kv"] = torch.empty(mla.mla_kv_produce_workspace(prob.T, d_model),
                                  dtype=torch.uint8, device="cuda")
        if d_cq is not None:
            hw["ws_q"] = torch.empty(mla.mla_q_produce_workspace(prob.T, d_model, d_cq, code),
                                     dtype=torch.uint8, device="cuda")
        hw["ws_o"] = torch.empty(max(1, mla.mla_o_proj_workspace(prob.T, wl.n_h, d_model, code)),
                                 dtype=torch.uint8, device="cuda")
        hw["u"] = torch.empty((prob.T, d_model), dtype=dp.dtype, device="cuda")
        torch.cuda.synchronize()

    pf_ws = pipeline.prefill_workspace(dp) if non_absorbed else None

    def one_step(ev=None, timer=None):
        """One step.  ev: events recorded around the step's parts (indices
        below); timer: a KernelTimer armed for the attention kernel."""
        if non_absorbed:
            mla.mla_kv_append(dp.kv_cache, dp.block_table, dp.new_c_kv, dp.new_k_r, dp.new_seq,
                              dp.new_pos, ROPE_BASE)
            if ev is not None:
                ev[0].record(stream)
            attend()
            if ev is not None:
                ev[1].record(stream)
            return
        if hw is None:
            # the step's new rows and its latent queries (one launch for the
            # native cache)
            pipeline.append_absorb(dp)
        else:
            if ev is not None:
                ev[2].record(stream)
            mla.mla_kv_produce(hw["h"], hw["w_dkv"], hw["kv_gain"], hw["w_kr"], dp.kv_cache,
                               dp.block_table, dp.new_seq, dp.new_pos, ROPE_BASE, PRODUCER_EPS,
                               hw["ws_kv"])
            if ev is not None:
                ev[3].record(stream)
            if d_cq is not None:
                mla.mla_q_produce(hw["h"], hw["w_dq"], hw["q_gain"], hw["w_uq"], hw["w_qr"],
                                  dp.q_nope, dp.q_rope, PRODUCER_EPS, hw["ws_q"])
            else:
                mla.mla_q_produce_direct(hw["h"], hw["w_qc"], hw["w_qr"], dp.q_nope, dp.q_rope)
            if ev is not None:
                ev[4].record(stream)
            mla.mla_absorb_q(dp.q_nope, dp.q_rope, dp.w_uk, dp.q_pos, dp.q_lat, ROPE_BASE)
        if ev is not None:
            ev[0].record(stream)
        if timer is not None:
            timer.arm()
        attend()
        if ev is not None:
            ev[1].record(stream)
        if splits == 0:
            # the split rows' merge runs inside the projection's loads
            mla.mla_out_proj_planned(dp.o_lat, dp.o_part, dp.lse_part, dp.split, dp.w_uv,
                                     dp.out, dp.lse)
            if hw is not None:             # eq. 8: the layer's output u = W^O [o_1; ...]
                if ev is not None:
                    ev[5].record(stream)
                mla.mla_o_proj(dp.out, hw["w_o"], hw["u"], hw["ws_o"])
                if ev is not None:
                    ev[6].record(stream)
            return
        if splits > 1:
            mla.mla_splitkv_combine(dp.o_part, dp.lse_part, dp.B, splits, dp.q_len, dp.n_h,
                                    dp.o_lat, dp.lse)
        mla.mla_out_proj(dp.o_lat, dp.w_uv, dp.out)

    def attend():
        """The attention kernel of the step (the dominant kernel)."""
        if non_absorbed:
            mla.mla_prefill_mha(dp.q_nope, dp.q_rope, dp.q_pos, dp.w_uk, dp.w_uv, dp.kv_cache,
                                dp.block_table, prob.seq_lens, dp.q_len, scale, ROPE_BASE,
                                dp.out, dp.lse, pf_ws)
        elif fp8 and splits == 0:
            mla.mla_decode_paged_planned_fp8(dp.q_lat, dp.kv_cache, dp.kv_scale, dp.block_table,
                                             dp.B, dp.q_len, scale, dp.work, dp.o_lat, dp.lse,
                                             o_part=dp.o_part, lse_part=dp.lse_part,
                                             lists=dp.lists)
        elif fp8:
            mla.mla_decode_paged_fp8(dp.q_lat, dp.kv_cache, dp.kv_scale, dp.block_table,
                                     dp.seq_lens, dp.q_len, scale, splits, o_part=dp.o_part,
                                     lse_part=dp.lse_part, o_lat=dp.o_lat, lse=dp.lse)
        elif splits == 0:
            mla.mla_decode_paged_planned(dp.q_lat, dp.kv_cache, dp.block_table, dp.B, dp.q_len,
                                         scale, dp.work, dp.o_lat, dp.lse, o_part=dp.o_part,
                                         lse_part=dp.lse_part, lists=dp.lists)
        elif splits > 1:
            mla.mla_decode_paged(dp.q_lat, dp.kv_cache, dp.block_table, dp.seq_lens, dp.q_len,
                                 scale, splits, o_part=dp.o_part, lse_part=dp.lse_part)
        else:
            mla.mla_decode_paged(dp.q_lat, dp.kv_cache, dp.block_table, dp.seq_lens, dp.q_len,
                                 scale, 1, o_lat=dp.o_lat, lse=dp.lse)

    if args.copy_bytes > 0:
        n = args.copy_bytes // 4
        src = torch.arange(n, dtype=torch.int32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] reference copy of {4 * n} bytes done")
        del src, dst

    if args.launch != "eager":
        # Checked once through the wrappers, then recorded: the timed loop
        # re-issues the marshalled calls, so that the CPU stays ahead of the
        # GPU (the wrappers' per-call checks cost more than a small step's
        # kernels and would leave the GPU idle between them, inside the
        # events that time the attention kernel).
        one_step()
        torch.cuda.synchronize()

        class _Mark:
            def __init__(self, rec, k):
                self.rec, self.k = rec, k

            def record(self, _stream):
                self.rec.calls.append(("__event__", self.k))

            def arm(self):
                self.rec.calls.append(("__arm__", None))

        with mla.recording() as rec:
            one_step(tuple(_Mark(rec, k) for k in range(7)), _Mark(rec, None))
        step_calls = rec.calls
        lib = mla.load()
        checked_step = one_step

        def one_step(ev=None, timer=None):
            for name, a in step_calls:
                if name == "__event__":
                    if ev is not None:
                        ev[a].record(stream)
                    continue
                if name == "__arm__":
                    if timer is not None:
                        lib.mla_time_attention(timer.start, timer.stop)
                    continue
                st = getattr(lib, name)(*a)
                if st != 0:
                    raise mla.MLAError(name, st, mla.status_string(st))

    log(f"[bench] warmup {args.warmup}")
    tw = time.perf_counter()
    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()
    settle = 0
    while time.perf_counter() - tw < args.settle_seconds:
        for _ in range(20):
            one_step()
        settle += 20
        torch.cuda.synchronize()
    # The timed steps carry no timing packets: an event recorded between two
    # kernels leaves the GPU idle for ~5 us, also when the kernel's own
    # dispatch records it.  The attention kernel is timed in a second pass of
    # as many identical steps, by its own dispatch (the library launches it
    # with a start / stop event pair, mla_time_attention); the non-absorbed
    # call is several kernels and is timed with events recorded around it.
    dispatch_timed = not non_absorbed

    def new_events(n):
        return tuple(torch.cuda.Event(enable_timing=True) for _ in range(n))

    def new_timers(n):
        return [mla.KernelTimer() for _ in range(n)] if dispatch_timed else [None] * n

    timers = new_timers(args.steps)
    events = [new_events(2) if non_absorbed else None for _ in range(args.steps)]
    region = new_events(2)
    log(f"[bench] {settle} settle steps; timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    region[0].record(stream)
    for i in range(args.steps):
        one_step()
    region[1].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    step_gpu_us = region[0].elapsed_time(region[1]) * 1e3 / args.steps
    for i in range(args.steps):
        one_step(events[i], timers[i])
    torch.cuda.synchronize()
    dec_times = ([t.elapsed_ms() for t in timers] if dispatch_timed
                 else [e[0].elapsed_time(e[1]) for e in events])
    for t in timers:
        if t is not None:
            t.close()
    timing = {"launch": args.launch, "warmup_steps": args.warmup, "settle_steps": settle,
              "attention_timing": (("the kernel's own dispatch events (mla_time_attention)"
                                    if dispatch_timed else "events around the call")
                                   + f", over a second pass of {args.steps} steps")}
    if args.launch == "graph":
        # Eager launches from Python cost tens of microseconds each, more than a
        # small step's kernels: the GPU then idles between them.  A graph of one
        # step is replayed instead (one launch per step); the attention kernel is
        # timed over back-to-back replays of a graph holding it alone.
        timing["unreplayed_step_ms"] = round(ms_per_step, 5)
        timing["attention_in_step_us"] = spread(dec_times)
        g_step, g_att = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_step):
            checked_step()
        with torch.cuda.graph(g_att):
            attend()
        for _ in range(20):
            g_step.replay()
            g_att.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        region[0].record(stream)
        for i in range(args.steps):
            g_step.replay()
        region[1].record(stream)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        ms_per_step = (t1 - t0) * 1e3 / args.steps
        step_gpu_us = region[0].elapsed_time(region[1]) * 1e3 / args.steps
        att_ev = [new_events(2) for _ in range(args.steps)]
        for i in range(args.steps):
            att_ev[i][0].record(stream)
            g_att.replay()
            att_ev[i][1].record(stream)
        torch.cuda.synchronize()
        dec_times = [e[0].elapsed_time(e[1]) for e in att_ev]
        del g_step, g_att
    dec_ms = float(np.mean(dec_times))
    timing["attention_us"] = spread(dec_times)
    timing["step_gpu_us"] = round(step_gpu_us, 2)   # GPU time of the timed steps / steps
    if args.cold_steps > 0:
        # each step after a 1 GiB write: the cache rows, queries and weights
        # come from HBM, not from the L2 / last-level cache
        flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
        cold_t = new_timers(args.cold_steps)
        cold_e = [new_events(2) if non_absorbed else None for _ in range(args.cold_steps)]
        for i in range(args.cold_steps):
            flush.fill_(float(i))
            one_step(cold_e[i], cold_t[i])
        torch.cuda.synchronize()
        timing["attention_cold_us"] = spread(
            [t.elapsed_ms() for t in cold_t] if dispatch_timed
            else [e[0].elapsed_time(e[1]) for e in cold_e])
        for t in cold_t:
            if t is not None:
                t.close()
        del flush
    prod_events = None
    if hw is not None:
        # the producers and W^O, timed with events around each (a separate
        # pass of as many steps, so that these events stay out of the timed
        # steps)
        prod_events = [new_events(7) for _ in range(args.steps)]
        for i in range(args.steps):
            one_step(prod_events[i])
        torch.cuda.synchronize()
    tokens = prob.T
    value = tokens / (ms_per_step * 1e-3)

    by, fl = algorithmic_work(prob, fp8)
    if non_absorbed:
        fl = non_absorbed_flops(prob)
    compute_bound = wl.q_len > 1
    mfma_peak = MFMA_BF16_PEAK_TFLOPS if wl.dtype == "bf16" else MFMA_F32_PEAK_TFLOPS
    gbs = by / (dec_ms * 1e-3) / 1e9
    tflops = fl / (dec_ms * 1e-3) / 1e12
    traffic = (load_traffic(wl.name, "prefill_mha") if non_absorbed
               else load_traffic(wl.name + ("_fp8" if fp8 else "")))
    if compute_bound:
        roof = {"bound": "mfma", "achieved": round(tflops, 2), "peak": mfma_peak,
                "unit": "TFLOP/s", "frac": round(tflops / mfma_peak, 4), "traffic": traffic}
    else:
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic}
    log(f"[bench] step {ms_per_step:.4f} ms, attention kernel {dec_ms * 1e3:.1f} us, "
        f"{gbs:.0f} GB/s, {tflops:.1f} TFLOP/s")

    producers = None
    if hw is not None:
        kv_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in prod_events]))
        q_ms = float(np.mean([e[3].elapsed_time(e[4]) for e in prod_events]))
        o_ms = (float(np.mean([e[5].elapsed_time(e[6]) for e in prod_events]))
                if splits == 0 else None)
        o_by = (prob.T * wl.n_h * 128 * 4 + d_model * wl.n_h * 128 * (2 if wl.dtype == "bf16" else 4)
                + prob.T * d_model * (2 if wl.dtype == "bf16" else 4))
        kv_by, q_by, kv_fl, q_fl = producer_work(prob.T, wl.n_h, d_model, d_cq,
                                                 2 if wl.dtype == "bf16" else 4)
        producers = {
            "d_model": d_model, "d_cq": d_cq,
            "kv_us": round(kv_ms * 1e3, 2), "q_us": round(q_ms * 1e3, 2),
            "kv_algorithmic_bytes": kv_by, "q_algorithmic_bytes": q_by,
            "kv_hbm_frac": round(kv_by / (kv_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "q_hbm_frac": round(q_by / (q_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "kv_mfma_frac": round(kv_fl / (kv_ms * 1e-3) / 1e12 / mfma_peak, 4),
            "q_mfma_frac": round(q_fl / (q_ms * 1e-3) / 1e12 / mfma_peak, 4),
            "o_proj_us": None if o_ms is None else round(o_ms * 1e3, 2),
            "o_proj_algorithmic_bytes": o_by,
            "o_proj_hbm_frac": (None if o_ms is None else
                                round(o_by / (o_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)),
        }
        log(f"[bench] producers: kv {kv_ms * 1e3:.1f} us, q {q_ms * 1e3:.1f} us"
            + ("" if o_ms is None else f"; W^O {o_ms * 1e3:.1f} us"))

    cpu = None
    if not args.no_cpu_baseline:
        log(f"[bench] cpu baseline (~{args.cpu_seconds} s)")
        cpu = cpu_baseline(prob, args.cpu_seconds, hid, fp8)

    cfg = {"workload": wl.name, "B": wl.B, "n_h": wl.n_h, "q_len": wl.q_len,
           "context": (f"U[{wl.ctx[0]},{wl.ctx[1]}]" if isinstance(wl.ctx, tuple) else wl.ctx),
           "block_size": wl.block_size,
           "split_kv": ("balanced plan" if splits == 0 else f"{splits} per row"),
           "work_items": (int(dp.work.shape[0]) if splits == 0 else dp.B * dp.q_len * splits),
           "d_c": 512, "d_R": 64, "d_h": 128,
           "attention_form": args.attention,
           "kv_cache": ("fp8 e4m3 codes + 2 fp32 scales per row" if fp8 else wl.dtype),
           "step_input": ("hidden states (cache-row and query producers in the step; the "
                          "step ends with eq. 8's W^O when the plan is balanced)"
                          if hw is not None else "new latent rows and per-head queries")}
    rec = {
        "metric": "MLA decode tokens/s (+ attention-kernel HBM GB/s and MFMA share of peak), "
                  "DeepSeek-V2 head shape",
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": wl.dtype, "data": "synthetic",
        "config": cfg, "roofline": roof, "timing": timing,
        "attention_kernel": {"scope": ("mla_prefill_mha: k^C and v^C projections, then the "
                                       "attention kernel" if non_absorbed else
                                       "the paged attention kernel"),
                             "us_per_launch": round(dec_ms * 1e3, 2),
                             "algorithmic_bytes": by, "algorithmic_flops": fl,
                             "hbm_gbs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                             "mfma_tflops": round(tflops, 1),
                             "mfma_frac": round(tflops / mfma_peak, 4),
                             "source_sha": source_sha("prefill_mha" if non_absorbed else "decode")},
        "cpu_baseline": cpu,
    }
    if producers is not None:
        rec["producers"] = producers
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
