"""One pass of the MLA hot path on device tensors.

A step is: append the step's new latent rows to the paged cache, absorb
W^UK into the queries, attend over the cache (split-KV when asked), merge the
splits and apply W^UV.  Every one of these runs in the HIP library; this
module only holds device buffers and calls the binding in order.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

from . import _binding as mla
from .workloads import BLOCK, D_C, D_H, D_R, ROPE_BASE, ROW, Problem, softmax_scale


def _torch():
    import torch
    return torch


def _to_device(x: np.ndarray, dtype, device):
    torch = _torch()
    t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to(dtype).to(device)


@dataclasses.dataclass
class DeviceProblem:
    """Device-resident inputs, cache and work buffers of one workload.

    num_splits > 0: uniform split-KV with that many splits per row.
    num_splits == 0: a load-balanced schedule from mla_plan_decode (``work``,
    ``lists``, ``split``) sized for ``num_slots`` concurrent workgroups.
    kv_scale is None for a bf16 / fp32 cache; for the FP8 cache kv_cache holds
    uint8 E4M3 codes and kv_scale the two float32 scales of every row.
    """
    prob: Problem
    num_splits: int
    dtype: object
    kv_cache: object
    block_table: object
    seq_lens: object
    new_c_kv: object
    new_k_r: object
    new_seq: object
    new_pos: object
    q_nope: object
    q_rope: object
    q_pos: object
    w_uk: object
    w_uv: object
    q_lat: object
    o_part: Optional[object]
    lse_part: Optional[object]
    o_lat: object
    lse: object
    out: object
    work: Optional[object] = None
    lists: Optional[object] = None
    split: Optional[object] = None
    n_parts: int = 0
    kv_scale: Optional[object] = None

    @property
    def B(self):
        return self.prob.wl.B

    @property
    def q_len(self):
        return self.prob.wl.q_len

    @property
    def n_h(self):
        return self.prob.wl.n_h


def new_rows(prob: Problem):
    """(sequence, position) of the rows a step appends: the last q_len keys of
    each sequence (for a decode step, the newest cached token)."""
    seqs, poss = [], []
    for b in range(prob.wl.B):
        L = int(prob.seq_lens[b])
        for p in range(max(0, L - prob.wl.q_len), L):
            seqs.append(b)
            poss.append(p)
    return np.array(seqs, dtype=np.int64), np.array(poss, dtype=np.int64)


def device_slots(device="cuda") -> int:
    """Workgroups the attention kernels run at once: one per compute unit."""
    torch = _torch()
    return int(torch.cuda.get_device_properties(torch.device(device)).multi_processor_count)


def upload(prob: Problem, num_splits: Optional[int] = None, device="cuda",
           poison: bool = True, num_slots: Optional[int] = None,
           cache: str = "native") -> DeviceProblem:
    """Copy a generated problem to the GPU and fill the cache with every row the
    step does not append itself (with the library's own append kernel).

    num_splits None -> the workload's own; 0 -> a balanced work plan.
    cache "native" keeps rows in the workload's dtype; "fp8" quantises them
    (bf16 workloads only)."""
    torch = _torch()
    wl = prob.wl
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    S = wl.num_splits if num_splits is None else int(num_splits)
    fp8 = cache == "fp8"
    if fp8 and wl.dtype != "bf16":
        raise ValueError("the FP8 cache takes bf16 queries")
    if fp8:
        # poison: 0xFF is the E4M3 NaN code
        kv_cache = torch.full((prob.num_blocks, BLOCK, ROW), 0xFF if poison else 0,
                              dtype=torch.uint8, device=device)
        kv_scale = torch.full((prob.num_blocks, BLOCK, 2), float("nan") if poison else 1.0,
                              dtype=torch.float32, device=device)
    else:
        fill = float("nan") if poison else 0.0
        kv_cache = torch.full((prob.num_blocks, BLOCK, ROW), fill, dtype=dt, device=device)
        kv_scale = None
    block_table = torch.from_numpy(prob.block_table).to(device)
    seq_lens = torch.from_numpy(prob.seq_lens).to(device)

    # Pre-fill: every key except the step's own new rows.
    step_seq, step_pos = new_rows(prob)
    is_new = np.zeros(int(prob.key_offsets[-1]), dtype=bool)
    is_new[prob.key_offsets[step_seq] + step_pos] = True
    seq_of_row = np.repeat(np.arange(wl.B), prob.seq_lens.astype(np.int64))
    pos_of_row = np.arange(int(prob.key_offsets[-1])) - prob.key_offsets[seq_of_row]
    old = np.nonzero(~is_new)[0]
    chunk = 1 << 18
    for lo in range(0, len(old), chunk):
        idx = old[lo:lo + chunk]
        args = (block_table, _to_device(prob.c_kv[idx], dt, device),
                _to_device(prob.k_r[idx], dt, device),
                torch.from_numpy(seq_of_row[idx].astype(np.int32)).to(device),
                torch.from_numpy(pos_of_row[idx].astype(np.int32)).to(device), ROPE_BASE)
        if fp8:
            mla.mla_kv_append_fp8(kv_cache, kv_scale, *args)
        else:
            mla.mla_kv_append(kv_cache, *args)
    new_idx = prob.key_offsets[step_seq] + step_pos
    T = prob.T
    work = lists = split = None
    n_parts = 0
    if S == 0:
        # the FP8 kernel runs two workgroups per compute unit below 64 heads
        per_cu = 2 if fp8 and wl.n_h < 64 else 1
        slots = per_cu * device_slots(device) if num_slots is None else int(num_slots)
        w, ls, sp, n_parts = mla.mla_plan_decode(prob.seq_lens, wl.q_len, wl.n_h, slots)
        work = torch.from_numpy(w).to(device)
        lists = torch.from_numpy(ls).to(device)
        split = torch.from_numpy(sp).to(device)
    n_part_rows = n_parts if S == 0 else (wl.B * S * wl.q_len if S > 1 else 0)
    dp = DeviceProblem(
        prob=prob, num_splits=S, dtype=dt, kv_cache=kv_cache, block_table=block_table,
        seq_lens=seq_lens,
        new_c_kv=_to_device(prob.c_kv[new_idx], dt, device),
        new_k_r=_to_device(prob.k_r[new_idx], dt, device),
        new_seq=torch.from_numpy(step_seq.astype(np.int32)).to(device),
        new_pos=torch.from_numpy(step_pos.astype(np.int32)).to(device),
        q_nope=_to_device(prob.q_nope, dt, device), q_rope=_to_device(prob.q_rope, dt, device),
        q_pos=torch.from_numpy(prob.q_pos).to(device),
        w_uk=_to_device(prob.w_uk, dt, device), w_uv=_to_device(prob.w_uv, dt, device),
        q_lat=torch.empty((T, wl.n_h, ROW), dtype=dt, device=device),
        o_part=(torch.empty((n_part_rows, wl.n_h, D_C), dtype=torch.float32, device=device)
                if n_part_rows else None),
        lse_part=(torch.empty((n_part_rows, wl.n_h), dtype=torch.float32, device=device)
                  if n_part_rows else None),
        o_lat=torch.empty((T, wl.n_h, D_C), dtype=torch.float32, device=device),
        lse=torch.empty((T, wl.n_h), dtype=torch.float32, device=device),
        out=torch.empty((T, wl.n_h, D_H), dtype=torch.float32, device=device),
        work=work, lists=lists, split=split, n_parts=n_parts, kv_scale=kv_scale,
    )
    return dp


def append(dp: DeviceProblem, stream=None):
    """The step's new rows into the cache (quantised for the FP8 cache)."""
    if dp.kv_scale is not None:
        mla.mla_kv_append_fp8(dp.kv_cache, dp.kv_scale, dp.block_table, dp.new_c_kv, dp.new_k_r,
                              dp.new_seq, dp.new_pos, ROPE_BASE, stream=stream)
    else:
        mla.mla_kv_append(dp.kv_cache, dp.block_table, dp.new_c_kv, dp.new_k_r, dp.new_seq,
                          dp.new_pos, ROPE_BASE, stream=stream)


def append_absorb(dp: DeviceProblem, stream=None):
    """The step's new rows into the cache and its latent queries: one launch
    (mla_append_absorb_q) for the native cache, the two calls for the FP8 one."""
    if dp.kv_scale is not None:
        append(dp, stream)
        mla.mla_absorb_q(dp.q_nope, dp.q_rope, dp.w_uk, dp.q_pos, dp.q_lat, ROPE_BASE,
                         stream=stream)
    else:
        mla.mla_append_absorb_q(dp.kv_cache, dp.block_table, dp.new_c_kv, dp.new_k_r,
                                dp.new_seq, dp.new_pos, dp.q_nope, dp.q_rope, dp.w_uk, dp.q_pos,
                                dp.q_lat, ROPE_BASE, stream=stream)


def step(dp: DeviceProblem, stream=None):
    """One pass of the hot path: append + absorb -> decode -> combine ->
    out-proj.  Under a balanced plan the combine runs inside the
    out-projection's loads (dp.o_lat then holds only the rows the plan did not
    split)."""
    append_absorb(dp, stream)
    if dp.num_splits == 0:
        _attend_planned(dp, stream)
        mla.mla_out_proj_planned(dp.o_lat, dp.o_part, dp.lse_part, dp.split, dp.w_uv, dp.out,
                                 dp.lse, stream=stream)
    else:
        decode(dp, stream=stream)
        mla.mla_out_proj(dp.o_lat, dp.w_uv, dp.out, stream=stream)


def prefill_workspace(dp: DeviceProblem):
    """Device workspace for step_non_absorbed (k^C and v^C of the longest sequence)."""
    torch = _torch()
    n = mla.mla_prefill_mha_workspace(int(dp.prob.seq_lens.max()), dp.n_h)
    return torch.empty(n, dtype=torch.uint8, device=dp.kv_cache.device)


def step_non_absorbed(dp: DeviceProblem, workspace, stream=None):
    """One pass of the chunked-prefill path in the non-absorbed form: append ->
    per-head keys and values -> attention, into dp.out / dp.lse (bf16 only)."""
    mla.mla_kv_append(dp.kv_cache, dp.block_table, dp.new_c_kv, dp.new_k_r, dp.new_seq,
                      dp.new_pos, ROPE_BASE, stream=stream)
    mla.mla_prefill_mha(dp.q_nope, dp.q_rope, dp.q_pos, dp.w_uk, dp.w_uv, dp.kv_cache,
                        dp.block_table, dp.prob.seq_lens, dp.q_len, softmax_scale(), ROPE_BASE,
                        dp.out, dp.lse, workspace, stream=stream)


def _attend_planned(dp: DeviceProblem, stream=None):
    if dp.kv_scale is not None:
        mla.mla_decode_paged_planned_fp8(dp.q_lat, dp.kv_cache, dp.kv_scale, dp.block_table, dp.B,
                                         dp.q_len, softmax_scale(), dp.work, dp.o_lat, dp.lse,
                                         o_part=dp.o_part, lse_part=dp.lse_part, lists=dp.lists,
                                         stream=stream)
        return
    mla.mla_decode_paged_planned(dp.q_lat, dp.kv_cache, dp.block_table, dp.B, dp.q_len,
                                 softmax_scale(), dp.work, dp.o_lat, dp.lse,
                                 o_part=dp.o_part, lse_part=dp.lse_part, lists=dp.lists,
                                 stream=stream)


def decode(dp: DeviceProblem, stream=None):
    """Attention over the cache (+ split merge) into dp.o_lat / dp.lse."""
    S = dp.num_splits
    if S == 0:
        _attend_planned(dp, stream)
        if dp.split.shape[0] > 0:
            mla.mla_combine_planned(dp.o_part, dp.lse_part, dp.split, dp.n_h, dp.o_lat, dp.lse,
                                    stream=stream)
    elif dp.kv_scale is not None:
        mla.mla_decode_paged_fp8(dp.q_lat, dp.kv_cache, dp.kv_scale, dp.block_table, dp.seq_lens,
                                 dp.q_len, softmax_scale(), S, o_part=dp.o_part,
                                 lse_part=dp.lse_part, o_lat=dp.o_lat, lse=dp.lse, stream=stream)
        if S > 1:
            mla.mla_splitkv_combine(dp.o_part, dp.lse_part, dp.B, S, dp.q_len, dp.n_h, dp.o_lat,
                                    dp.lse, stream=stream)
    elif S > 1:
        mla.mla_decode_paged(dp.q_lat, dp.kv_cache, dp.block_table, dp.seq_lens, dp.q_len,
                             softmax_scale(), S, o_part=dp.o_part, lse_part=dp.lse_part,
                             stream=stream)
        mla.mla_splitkv_combine(dp.o_part, dp.lse_part, dp.B, S, dp.q_len, dp.n_h, dp.o_lat,
                                dp.lse, stream=stream)
    else:
        mla.mla_decode_paged(dp.q_lat, dp.kv_cache, dp.block_table, dp.seq_lens, dp.q_len,
                             softmax_scale(), 1, o_lat=dp.o_lat, lse=dp.lse, stream=stream)
