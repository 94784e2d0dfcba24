"""Seeded synthetic inputs for MLA decode / chunked prefill over a paged latent cache.

This module only draws and lays out inputs.  It holds none of the attention
arithmetic: no RoPE, no projection, no softmax.  Both the CPU oracle (through
the tests and the CPU-baseline leg of the benchmark) and the HIP path consume
what it returns, so the two sides always see the same values.

Shapes follow the pages: DeepSeek-V2 uses 128 heads of width 128, a 512-wide
KV latent and a 64-wide decoupled RoPE key; V2-Lite uses 16 heads with the same
widths ([adg.csdn.net blog, part 3 §3.1.1, and the V2-Lite description in part 2]).

Recipe (one ``numpy.random.Generator(PCG64(seed))`` per workload, draws in
this order):
  1. integers that fix the shape: per-sequence context lengths (uniform
     workloads only);
  2. c_KV [sum L, 512] ~ N(0, 1), float32;
  3. raw (un-rotated) k_R [sum L, 64] ~ N(0, 1);
  4. q_nope [T, n_h, 128] ~ N(0, 1);
  5. raw q_rope [T, n_h, 64] ~ N(0, 1);
  6. W^UK [n_h, 128, 512] ~ N(0, 1/512) (fan-in 512);
  7. W^UV [n_h, 128, 512] ~ N(0, 1/512);
  8. the physical block permutation (permuted tables only).
For bf16 workloads every float draw is rounded to bf16 (round to nearest
even) and the rounded value is what both sides receive.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

D_C = 512       # KV latent width d_c
D_R = 64        # decoupled RoPE key/query width d_R
D_H = 128       # per-head width d_h
ROW = D_C + D_R # elements of one cached latent row
BLOCK = 64      # tokens per paged block
ROPE_BASE = 10000.0
D_MODEL_V2 = 5120   # DeepSeek-V2 hidden width
D_CQ_V2 = 1536      # DeepSeek-V2 query compression width d_c'
D_MODEL_LITE = 2048 # DeepSeek-V2-Lite hidden width (its queries are not compressed)


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic MLA attention problem.

    ``ctx`` is either an int (every sequence has that many keys visible to its
    last query row) or a tuple ``(lo, hi)`` for lengths uniform in [lo, hi].
    ``q_len`` > 1 is a chunked prefill: the last ``q_len`` keys of each
    sequence are the chunk's own rows, appended by the kv-append step.
    """
    name: str
    dtype: str            # "f32" or "bf16"
    B: int
    n_h: int
    ctx: object
    q_len: int = 1
    block_size: int = BLOCK
    table: str = "permuted"   # "identity" or "permuted"
    seed: int = 0
    num_splits: int = 0       # split-KV partitions of the benchmark's launch (0 = balanced plan)


# The five workloads: V2-Lite fp32 (tiny), V2-Lite bf16 paged, full V2 ragged
# decode, V2 128K split-KV decode and V2 chunked prefill.
WORKLOADS = {
    "v2lite_f32_L256": Workload("v2lite_f32_L256", "f32", B=1, n_h=16, ctx=256,
                                table="identity", seed=1001),
    "v2lite_bf16_B64_L4096": Workload("v2lite_bf16_B64_L4096", "bf16", B=64, n_h=16,
                                      ctx=4096, seed=1002),
    "v2_bf16_B128_L1k-8k": Workload("v2_bf16_B128_L1k-8k", "bf16", B=128, n_h=128,
                                    ctx=(1024, 8192), seed=1003),
    "v2_bf16_B4_L128k_splitkv": Workload("v2_bf16_B4_L128k_splitkv", "bf16", B=4, n_h=128,
                                         ctx=131072, seed=1004),
    "v2_bf16_prefill_6144+2048": Workload("v2_bf16_prefill_6144+2048", "bf16", B=1,
                                          n_h=128, ctx=8192, q_len=2048, seed=1005,
                                          num_splits=1),
}
WORKLOAD_ORDER = list(WORKLOADS)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    out = rounded.astype(np.uint32).view(np.float32)
    nan = np.isnan(x)
    if nan.any():
        out = out.copy()
        out[nan] = np.float32("nan")
    return out


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are already bf16-representable."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


@dataclasses.dataclass
class Problem:
    """Host arrays of one generated workload (float32 values, bf16-exact for bf16)."""
    wl: Workload
    seq_lens: np.ndarray      # int32 [B], keys visible to the last query row
    key_offsets: np.ndarray   # int64 [B+1], row offsets of each sequence in c_kv/k_r
    c_kv: np.ndarray          # float32 [sum L, 512]
    k_r: np.ndarray           # float32 [sum L, 64]  (before rotation)
    q_nope: np.ndarray        # float32 [T, n_h, 128], T = B * q_len
    q_rope: np.ndarray        # float32 [T, n_h, 64]  (before rotation)
    w_uk: np.ndarray          # float32 [n_h, 128, 512]
    w_uv: np.ndarray          # float32 [n_h, 128, 512]
    q_pos: np.ndarray         # int32 [T], RoPE position of each query row
    block_table: np.ndarray   # int32 [B, max_blocks]; unused entries -> guard block
    num_blocks: int           # physical blocks in the pool, guard block included
    guard_block: int          # block id that no sequence owns (kept NaN)

    @property
    def T(self) -> int:
        return self.wl.B * self.wl.q_len

    @property
    def max_blocks(self) -> int:
        return int(self.block_table.shape[1])

    def n_visible(self, b: int) -> np.ndarray:
        """Keys visible to each query row of sequence b (causal chunk rule)."""
        L = int(self.seq_lens[b])
        q = self.wl.q_len
        return np.array([L - (q - 1 - m) for m in range(q)], dtype=np.int64)

    def seq_rows(self, b: int):
        lo, hi = int(self.key_offsets[b]), int(self.key_offsets[b + 1])
        return self.c_kv[lo:hi], self.k_r[lo:hi]


def _normal(rng: np.random.Generator, shape, std: float, bf16: bool) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return round_to_bf16(x) if bf16 else x


def make_problem(wl: Workload, *, B: Optional[int] = None, n_h: Optional[int] = None,
                 ctx=None, q_len: Optional[int] = None, seed: Optional[int] = None,
                 table: Optional[str] = None) -> Problem:
    """Generate the inputs of ``wl`` (optionally with overridden sizes)."""
    if B is not None or n_h is not None or ctx is not None or q_len is not None \
            or seed is not None or table is not None:
        wl = dataclasses.replace(
            wl, B=wl.B if B is None else B, n_h=wl.n_h if n_h is None else n_h,
            ctx=wl.ctx if ctx is None else ctx, q_len=wl.q_len if q_len is None else q_len,
            seed=wl.seed if seed is None else seed, table=wl.table if table is None else table)
    bf16 = wl.dtype == "bf16"
    rng = np.random.Generator(np.random.PCG64(wl.seed))
    if isinstance(wl.ctx, tuple):
        lo, hi = wl.ctx
        seq_lens = rng.integers(lo, hi, size=wl.B, endpoint=True).astype(np.int32)
    elif isinstance(wl.ctx, (list, np.ndarray)):
        seq_lens = np.asarray(wl.ctx, dtype=np.int32)
        assert seq_lens.shape == (wl.B,)
    else:
        seq_lens = np.full(wl.B, int(wl.ctx), dtype=np.int32)
    if wl.q_len > 1 and (seq_lens < wl.q_len).any():
        raise ValueError("a prefill chunk must lie inside its sequence")
    if (seq_lens < 0).any():
        raise ValueError("negative context length")
    offsets = np.zeros(wl.B + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(seq_lens.astype(np.int64))
    total = int(offsets[-1])
    T = wl.B * wl.q_len
    c_kv = _normal(rng, (total, D_C), 1.0, bf16)
    k_r = _normal(rng, (total, D_R), 1.0, bf16)
    q_nope = _normal(rng, (T, wl.n_h, D_H), 1.0, bf16)
    q_rope = _normal(rng, (T, wl.n_h, D_R), 1.0, bf16)
    w_std = 1.0 / math.sqrt(D_C)
    w_uk = _normal(rng, (wl.n_h, D_H, D_C), w_std, bf16)
    w_uv = _normal(rng, (wl.n_h, D_H, D_C), w_std, bf16)

    bs = wl.block_size
    nblk = (seq_lens.astype(np.int64) + bs - 1) // bs
    max_blocks = max(1, int(nblk.max()))
    used = int(nblk.sum())
    if wl.table == "identity":
        phys = np.arange(used, dtype=np.int32)
    else:
        phys = rng.permutation(used).astype(np.int32)
    guard = used
    table = np.full((wl.B, max_blocks), guard, dtype=np.int32)
    pos = 0
    for b in range(wl.B):
        n = int(nblk[b])
        table[b, :n] = phys[pos:pos + n]
        pos += n
    # Query row m of sequence b sits at position seq_len - q_len + m; a decode
    # query (q_len = 1) sits right after its seq_len cached keys.
    if wl.q_len == 1:
        q_pos = seq_lens.astype(np.int32).copy()
    else:
        q_pos = np.concatenate([np.arange(int(L) - wl.q_len, int(L), dtype=np.int32)
                                for L in seq_lens])
    return Problem(wl=wl, seq_lens=seq_lens, key_offsets=offsets, c_kv=c_kv, k_r=k_r,
                   q_nope=q_nope, q_rope=q_rope, w_uk=w_uk, w_uv=w_uv, q_pos=q_pos,
                   block_table=table, num_blocks=used + 1, guard_block=guard)


def softmax_scale() -> float:
    """1/sqrt(d_h + d_R): the width of the concatenated query/key of one head."""
    return 1.0 / math.sqrt(D_H + D_R)


@dataclasses.dataclass
class HiddenInputs:
    """Hidden states of a step's tokens and the producer weights that turn
    them into cache rows and queries (float32 values, bf16-exact for bf16)."""
    h: np.ndarray        # [T, d_model]
    w_dkv: np.ndarray    # [512, d_model]
    kv_gain: np.ndarray  # [512] float32
    w_kr: np.ndarray     # [64, d_model]
    w_qr: np.ndarray     # [n_h * 64, d_cq], or [n_h * 64, d_model] without compression
    w_dq: Optional[np.ndarray] = None    # [d_cq, d_model]   (compressed queries)
    q_gain: Optional[np.ndarray] = None  # [d_cq] float32
    w_uq: Optional[np.ndarray] = None    # [n_h * 128, d_cq]
    w_qc: Optional[np.ndarray] = None    # [n_h * 128, d_model] (uncompressed queries)
    w_o: Optional[np.ndarray] = None     # [d_model, n_h * 128] (eq. 8's output projection)


def make_hidden(prob: Problem, d_model: int = D_MODEL_V2,
                d_cq: Optional[int] = D_CQ_V2) -> HiddenInputs:
    """Hidden states for the step's T tokens and random producer weights of the
    DeepSeek-V2 widths (hidden 5120, query compression 1536: adg.csdn.net blog,
    part 3 §3.1.1).

    Recipe (its own ``Generator(PCG64(seed + 7919))``, draws in this order):
    h ~ N(0, 1); W^DKV, W^KR, W^DQ ~ N(0, 1/d_model); W^UQ, W^QR ~ N(0, 1/d_cq);
    the two RMSNorm gains 1 + 0.1 N(0, 1), float32.  Weights are stored
    [d_out, d_in]; float draws are rounded to bf16 for bf16 workloads.
    d_cq None: queries without compression (V2-Lite: hidden 2048, blog, the
    V2-Lite paragraph): h; W^DKV, W^KR, W^QC, W^QR ~ N(0, 1/d_model); the
    latent gain.  Last in either case: W^O ~ N(0, 1/(n_h 128))."""
    wl = prob.wl
    bf16 = wl.dtype == "bf16"
    rng = np.random.Generator(np.random.PCG64(wl.seed + 7919))
    T, n_h = prob.T, wl.n_h
    h = _normal(rng, (T, d_model), 1.0, bf16)
    if d_cq is None:
        w_dkv = _normal(rng, (D_C, d_model), 1.0 / math.sqrt(d_model), bf16)
        w_kr = _normal(rng, (D_R, d_model), 1.0 / math.sqrt(d_model), bf16)
        w_qc = _normal(rng, (n_h * D_H, d_model), 1.0 / math.sqrt(d_model), bf16)
        w_qr = _normal(rng, (n_h * D_R, d_model), 1.0 / math.sqrt(d_model), bf16)
        kv_gain = (1.0 + 0.1 * rng.standard_normal(D_C)).astype(np.float32)
        w_o = _normal(rng, (d_model, n_h * D_H), 1.0 / math.sqrt(n_h * D_H), bf16)
        return HiddenInputs(h=h, w_dkv=w_dkv, kv_gain=kv_gain, w_kr=w_kr, w_qr=w_qr, w_qc=w_qc,
                            w_o=w_o)
    w_dkv = _normal(rng, (D_C, d_model), 1.0 / math.sqrt(d_model), bf16)
    w_kr = _normal(rng, (D_R, d_model), 1.0 / math.sqrt(d_model), bf16)
    w_dq = _normal(rng, (d_cq, d_model), 1.0 / math.sqrt(d_model), bf16)
    w_uq = _normal(rng, (n_h * D_H, d_cq), 1.0 / math.sqrt(d_cq), bf16)
    w_qr = _normal(rng, (n_h * D_R, d_cq), 1.0 / math.sqrt(d_cq), bf16)
    kv_gain = (1.0 + 0.1 * rng.standard_normal(D_C)).astype(np.float32)
    q_gain = (1.0 + 0.1 * rng.standard_normal(d_cq)).astype(np.float32)
    w_o = _normal(rng, (d_model, n_h * D_H), 1.0 / math.sqrt(n_h * D_H), bf16)
    return HiddenInputs(h=h, w_dkv=w_dkv, kv_gain=kv_gain, w_kr=w_kr, w_dq=w_dq, q_gain=q_gain,
                        w_uq=w_uq, w_qr=w_qr, w_o=w_o)

