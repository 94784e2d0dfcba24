"""Thin ctypes binding of libmla_latent_kv.so (include/mla.h).

Argument marshalling only: tensors become raw device pointers, the stream is
torch's current HIP stream, and a non-OK status raises MLAError.  Every
computation runs in the library's HIP kernels; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "_lib", "libmla_latent_kv.so")

MLA_F32, MLA_BF16 = 0, 1
MLA_OK = 0
D_C, D_R, D_H, ROW, BLOCK = 512, 64, 128, 576, 64

_EXPORTS = ("mla_status_string", "mla_abi_version", "mla_rope_theta", "mla_kv_append",
            "mla_absorb_q", "mla_decode_paged", "mla_splitkv_combine", "mla_out_proj",
            "mla_split_plan", "mla_plan_decode", "mla_decode_paged_planned", "mla_combine_planned",
            "mla_out_proj_planned", "mla_kv_produce_workspace", "mla_kv_produce",
            "mla_q_produce_workspace", "mla_q_produce", "mla_q_produce_direct",
            "mla_o_proj_workspace", "mla_o_proj",
            "mla_prefill_mha_workspace", "mla_prefill_mha", "mla_kv_append_fp8",
            "mla_decode_paged_fp8", "mla_decode_paged_planned_fp8", "mla_decode_paged_noalloc",
            "mla_time_attention", "mla_append_absorb_q")


class MLAError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn} failed with status {status}: {text}")
        self.status = status


_lib: Optional[ctypes.CDLL] = None

_P = ctypes.c_void_p
_I = ctypes.c_int32
_F = ctypes.c_float
_D = ctypes.c_double


def lib_path() -> str:
    return LIB


class _Recorder:
    """Stands in for the library while calls are recorded: every entry point
    call is kept as (name, arguments) and reports success."""

    def __init__(self, lib):
        self.lib = lib
        self.calls = []

    def __getattr__(self, name):
        fn = getattr(self.lib, name)
        if not name.startswith("mla_") or fn.restype is not _I or name == "mla_abi_version":
            return fn

        def record(*args):
            self.calls.append((name, args))
            return MLA_OK
        return record


_recorder: Optional[_Recorder] = None


class recording:
    """Context manager: the entry-point wrappers called inside it check and
    marshal their arguments as usual but enqueue nothing; ``calls`` then holds
    the marshalled calls, which ``replay`` issues again with no Python-side
    checks (for launch loops where the wrappers' overhead would leave the GPU
    idle).  The tensors and the stream the calls name must stay alive and
    unchanged in shape."""

    def __enter__(self):
        global _recorder
        _recorder = _Recorder(load())
        return _recorder

    def __exit__(self, *exc):
        global _recorder
        _recorder = None
        return False


def replay(calls):
    """Issue recorded calls in order; raises MLAError on a non-OK status."""
    lib = load()
    for name, args in calls:
        st = getattr(lib, name)(*args)
        if st != MLA_OK:
            raise MLAError(name, st, lib.mla_status_string(st).decode())


def load() -> ctypes.CDLL:
    """Load the built library (raises if it was not built)."""
    global _lib
    if _recorder is not None:
        return _recorder
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB):
        raise RuntimeError(f"{LIB} is missing: build it first "
                           "(python -m mla_latent_kv_04_amd.build)")
    lib = ctypes.CDLL(LIB)
    sig = {
        "mla_status_string": (ctypes.c_char_p, [_I]),
        "mla_abi_version": (_I, []),
        "mla_time_attention": (_I, [_P, _P]),
        "mla_append_absorb_q": (_I, [_P, _I, _I, _P, _I, _I, _P, _P, _P, _P, _I, _P, _P, _P, _P,
                                     _I, _I, _I, _F, _P, _P, _P]),
        "mla_rope_theta": (_I, [_D, _D, _D, _D, _D, _P]),
        "mla_kv_append": (_I, [_P, _I, _I, _I, _P, _I, _I, _P, _P, _P, _P, _I, _F, _P, _P]),
        "mla_absorb_q": (_I, [_P, _P, _P, _P, _I, _I, _I, _F, _P, _P, _P]),
        "mla_decode_paged": (_I, [_P, _P, _I, _I, _P, _I, _P, _I, _I, _I, _I, _F, _I,
                                  _P, _P, _P, _P, _P]),
        "mla_splitkv_combine": (_I, [_P, _P, _I, _I, _I, _I, _P, _P, _P]),
        "mla_out_proj": (_I, [_P, _P, _I, _I, _I, _P, _P]),
        "mla_split_plan": (_I, [_P, _I, _I, _I, _P]),
        "mla_plan_decode": (_I, [_P, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P]),
        "mla_decode_paged_planned": (_I, [_P, _P, _I, _I, _P, _I, _I, _I, _I, _I, _F, _P, _I,
                                          _P, _I, _P, _P, _I, _P, _P, _P]),
        "mla_combine_planned": (_I, [_P, _P, _P, _I, _I, _P, _P, _P]),
        "mla_out_proj_planned": (_I, [_P, _P, _P, _P, _I, _P, _I, _I, _I, _P, _P, _P]),
        "mla_kv_produce_workspace": (ctypes.c_int64, [_I, _I]),
        "mla_kv_produce": (_I, [_P, _P, _P, _P, _I, _I, _I, _F, _F, _P, _P, _I, _I, _P, _I, _I,
                                _P, _P, _P, ctypes.c_int64, _P]),
        "mla_q_produce_workspace": (ctypes.c_int64, [_I, _I, _I, _I]),
        "mla_q_produce": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _P, _P, _P,
                               ctypes.c_int64, _P]),
        "mla_q_produce_direct": (_I, [_P, _P, _P, _I, _I, _I, _I, _P, _P, _P]),
        "mla_o_proj_workspace": (ctypes.c_int64, [_I, _I, _I, _I]),
        "mla_o_proj": (_I, [_P, _P, _I, _I, _I, _I, _P, _P, ctypes.c_int64, _P]),
        "mla_prefill_mha_workspace": (ctypes.c_int64, [_I, _I]),
        "mla_kv_append_fp8": (_I, [_P, _P, _I, _I, _I, _P, _I, _I, _P, _P, _P, _P, _I, _F, _P,
                                   _P]),
        "mla_decode_paged_fp8": (_I, [_P, _P, _P, _I, _I, _P, _I, _P, _I, _I, _I, _F, _I, _P, _P,
                                      _P, _P, _P]),
        "mla_decode_paged_planned_fp8": (_I, [_P, _P, _P, _I, _I, _P, _I, _I, _I, _I, _F, _P, _I,
                                              _P, _I, _P, _P, _I, _P, _P, _P]),
        "mla_decode_paged_noalloc": (_I, [_P, _P, _I, _I, _P, _I, _P, _I, _I, _I, _I, _F, _I,
                                          _P, _P, _P]),
        "mla_prefill_mha": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _P, _I, _P, _I, _I, _I, _I, _F,
                                 _F, _P, _P, _P, _P, ctypes.c_int64, _P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def exported_symbols():
    return _EXPORTS


def _check(fn: str, status: int):
    if status != MLA_OK:
        raise MLAError(fn, status, load().mla_status_string(status).decode())


def status_string(status: int) -> str:
    return load().mla_status_string(status).decode()


# ---------------------------------------------------------------------------
# torch marshalling helpers
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return MLA_F32
    if t.dtype == torch.bfloat16:
        return MLA_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _dev(t, name: str, dtype=None):
    """Pointer of a contiguous CUDA(HIP) tensor, or None."""
    if t is None:
        return None
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must live on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return ctypes.c_void_p(t.data_ptr())


def _theta(rope_theta):
    """float64 host copy of a RoPE frequency table [32] (None stays None).
    The caller keeps the returned array alive across the C call."""
    if rope_theta is None:
        return None
    arr = np.ascontiguousarray(np.asarray(rope_theta, dtype=np.float64))
    if arr.shape != (D_R // 2,):
        raise ValueError("rope_theta must hold 32 pair frequencies")
    return arr


def _ptr(arr):
    return None if arr is None else arr.ctypes.data_as(ctypes.c_void_p)


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


# ---------------------------------------------------------------------------
# Entry points (same names as the C ABI)
# ---------------------------------------------------------------------------

def mla_rope_theta(base=10000.0, scale=1.0, alpha=1.0, beta=32.0, orig_ctx=4096.0):
    """RoPE pair frequencies [32] with YaRN's interpolation by parts (see mla.h).
    Host arithmetic only."""
    out = np.zeros(D_R // 2, dtype=np.float64)
    st = load().mla_rope_theta(float(base), float(scale), float(alpha), float(beta),
                               float(orig_ctx), _ptr(out))
    _check("mla_rope_theta", st)
    return out


def mla_kv_append(kv_cache, block_table, c_kv, k_rope, seq_idx, pos, rope_base=10000.0,
                  stream=None, rope_theta=None):
    """Write rows [c_kv ; R_pos k_rope] into the paged cache (see mla.h)."""
    torch = _torch()
    dt = _dtype_code(kv_cache)
    n = int(c_kv.shape[0]) if c_kv is not None else 0
    for name, t in (("c_kv", c_kv), ("k_rope", k_rope)):
        if t.dtype != kv_cache.dtype:
            raise TypeError(f"{name} dtype differs from the cache")
    if tuple(c_kv.shape) != (n, D_C) or tuple(k_rope.shape) != (n, D_R):
        raise ValueError("c_kv must be [n, 512] and k_rope [n, 64]")
    if tuple(seq_idx.shape) != (n,) or tuple(pos.shape) != (n,):
        raise ValueError("seq_idx and pos must be [n]")
    if kv_cache.dim() != 3 or kv_cache.shape[2] != ROW:
        raise ValueError("kv_cache must be [num_blocks, 64, 576]")
    th = _theta(rope_theta)
    st = load().mla_kv_append(
        _dev(kv_cache, "kv_cache"), dt, int(kv_cache.shape[0]), int(kv_cache.shape[1]),
        _dev(block_table, "block_table", torch.int32), int(block_table.shape[0]),
        int(block_table.shape[1]), _dev(c_kv, "c_kv"), _dev(k_rope, "k_rope"),
        _dev(seq_idx, "seq_idx", torch.int32), _dev(pos, "pos", torch.int32), n,
        float(rope_base), _ptr(th), _stream(stream))
    _check("mla_kv_append", st)


def mla_absorb_q(q_nope, q_rope, w_uk, q_pos, q_lat, rope_base=10000.0, stream=None,
                 rope_theta=None):
    """q_lat = [W^UK^T q_nope ; R q_rope] per row and head (see mla.h)."""
    torch = _torch()
    dt = _dtype_code(q_nope)
    T, n_h = int(q_nope.shape[0]), int(q_nope.shape[1])
    if tuple(q_nope.shape) != (T, n_h, D_H) or tuple(q_rope.shape) != (T, n_h, D_R):
        raise ValueError("q_nope must be [T, n_h, 128] and q_rope [T, n_h, 64]")
    if tuple(w_uk.shape) != (n_h, D_H, D_C) or tuple(q_lat.shape) != (T, n_h, ROW):
        raise ValueError("w_uk must be [n_h, 128, 512] and q_lat [T, n_h, 576]")
    for name, t in (("q_rope", q_rope), ("w_uk", w_uk), ("q_lat", q_lat)):
        if t.dtype != q_nope.dtype:
            raise TypeError(f"{name} dtype differs from q_nope")
    th = _theta(rope_theta)
    st = load().mla_absorb_q(_dev(q_nope, "q_nope"), _dev(q_rope, "q_rope"), _dev(w_uk, "w_uk"),
                             _dev(q_pos, "q_pos", torch.int32), T, n_h, dt, float(rope_base),
                             _ptr(th), _dev(q_lat, "q_lat"), _stream(stream))
    _check("mla_absorb_q", st)


def mla_append_absorb_q(kv_cache, block_table, c_kv, k_rope, seq_idx, pos, q_nope, q_rope, w_uk,
                        q_pos, q_lat, rope_base=10000.0, stream=None, rope_theta=None):
    """mla_kv_append and mla_absorb_q of one step in one launch (see mla.h)."""
    torch = _torch()
    dt = _dtype_code(q_nope)
    if kv_cache.dtype != q_nope.dtype:
        raise TypeError("kv_cache dtype differs from q_nope")
    n = int(c_kv.shape[0])
    for name, t in (("c_kv", c_kv), ("k_rope", k_rope)):
        if t.dtype != kv_cache.dtype:
            raise TypeError(f"{name} dtype differs from the cache")
    if tuple(c_kv.shape) != (n, D_C) or tuple(k_rope.shape) != (n, D_R):
        raise ValueError("c_kv must be [n, 512] and k_rope [n, 64]")
    if tuple(seq_idx.shape) != (n,) or tuple(pos.shape) != (n,):
        raise ValueError("seq_idx and pos must be [n]")
    if kv_cache.dim() != 3 or kv_cache.shape[2] != ROW:
        raise ValueError("kv_cache must be [num_blocks, 64, 576]")
    T, n_h = int(q_nope.shape[0]), int(q_nope.shape[1])
    if tuple(q_nope.shape) != (T, n_h, D_H) or tuple(q_rope.shape) != (T, n_h, D_R):
        raise ValueError("q_nope must be [T, n_h, 128] and q_rope [T, n_h, 64]")
    if tuple(w_uk.shape) != (n_h, D_H, D_C) or tuple(q_lat.shape) != (T, n_h, ROW):
        raise ValueError("w_uk must be [n_h, 128, 512] and q_lat [T, n_h, 576]")
    for name, t in (("q_rope", q_rope), ("w_uk", w_uk), ("q_lat", q_lat)):
        if t.dtype != q_nope.dtype:
            raise TypeError(f"{name} dtype differs from q_nope")
    th = _theta(rope_theta)
    st = load().mla_append_absorb_q(
        _dev(kv_cache, "kv_cache"), int(kv_cache.shape[0]), int(kv_cache.shape[1]),
        _dev(block_table, "block_table", torch.int32), int(block_table.shape[0]),
        int(block_table.shape[1]), _dev(c_kv, "c_kv"), _dev(k_rope, "k_rope"),
        _dev(seq_idx, "seq_idx", torch.int32), _dev(pos, "pos", torch.int32), n,
        _dev(q_nope, "q_nope"), _dev(q_rope, "q_rope"), _dev(w_uk, "w_uk"),
        _dev(q_pos, "q_pos", torch.int32), T, n_h, dt, float(rope_base), _ptr(th),
        _dev(q_lat, "q_lat"), _stream(stream))
    _check("mla_append_absorb_q", st)


def mla_decode_paged(q_lat, kv_cache, block_table, seq_lens, q_len, softmax_scale, num_splits=1,
                     o_part=None, lse_part=None, o_lat=None, lse=None, stream=None):
    """Latent attention over the paged cache (see mla.h).  q_lat is [B*q_len, n_h, 576]."""
    torch = _torch()
    dt = _dtype_code(q_lat)
    if kv_cache.dtype != q_lat.dtype:
        raise TypeError("kv_cache dtype differs from q_lat")
    B = int(seq_lens.shape[0])
    n_h = int(q_lat.shape[-2])
    if q_lat.shape[-1] != ROW or q_lat.numel() != B * q_len * n_h * ROW:
        raise ValueError("q_lat must hold [B, q_len, n_h, 576]")
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be [B, max_blocks]")
    rows = B * q_len * n_h
    if int(num_splits) > 1:
        if o_part is None or lse_part is None or o_part.numel() != rows * num_splits * D_C \
                or lse_part.numel() != rows * num_splits:
            raise ValueError("o_part / lse_part must hold [B, S, q_len, n_h, 512] / [B, S, q_len, n_h]")
    elif o_lat is None or lse is None or o_lat.numel() != rows * D_C or lse.numel() != rows:
        raise ValueError("o_lat / lse must hold [B, q_len, n_h, 512] / [B, q_len, n_h]")
    f32 = torch.float32
    st = load().mla_decode_paged(
        _dev(q_lat, "q_lat"), _dev(kv_cache, "kv_cache"), int(kv_cache.shape[0]),
        int(kv_cache.shape[1]), _dev(block_table, "block_table", torch.int32),
        int(block_table.shape[1]), _dev(seq_lens, "seq_lens", torch.int32), B, int(q_len), n_h,
        dt, float(softmax_scale), int(num_splits), _dev(o_part, "o_part", f32),
        _dev(lse_part, "lse_part", f32), _dev(o_lat, "o_lat", f32), _dev(lse, "lse", f32),
        _stream(stream))
    _check("mla_decode_paged", st)


def mla_splitkv_combine(o_part, lse_part, B, S, q_len, n_h, o_lat, lse=None, stream=None):
    """Merge split partials (see mla.h)."""
    torch = _torch()
    f32 = torch.float32
    if o_part.numel() != B * S * q_len * n_h * D_C or lse_part.numel() != B * S * q_len * n_h:
        raise ValueError("partials have the wrong size")
    if o_lat.numel() != B * q_len * n_h * D_C:
        raise ValueError("o_lat has the wrong size")
    if lse is not None and lse.numel() != B * q_len * n_h:
        raise ValueError("lse has the wrong size")
    st = load().mla_splitkv_combine(_dev(o_part, "o_part", f32), _dev(lse_part, "lse_part", f32),
                                    int(B), int(S), int(q_len), int(n_h),
                                    _dev(o_lat, "o_lat", f32), _dev(lse, "lse", f32),
                                    _stream(stream))
    _check("mla_splitkv_combine", st)


def mla_out_proj(o_lat, w_uv, out, stream=None):
    """out[t, i] = W^UV_i o_lat[t, i] (see mla.h).  o_lat [T, n_h, 512] fp32."""
    torch = _torch()
    dt = _dtype_code(w_uv)
    T, n_h = int(o_lat.shape[0]), int(o_lat.shape[1])
    if tuple(o_lat.shape) != (T, n_h, D_C) or tuple(w_uv.shape) != (n_h, D_H, D_C):
        raise ValueError("o_lat must be [T, n_h, 512] and w_uv [n_h, 128, 512]")
    if tuple(out.shape) != (T, n_h, D_H):
        raise ValueError("out must be [T, n_h, 128]")
    f32 = torch.float32
    st = load().mla_out_proj(_dev(o_lat, "o_lat", f32), _dev(w_uv, "w_uv"), T, n_h, dt,
                             _dev(out, "out", f32), _stream(stream))
    _check("mla_out_proj", st)


def mla_split_plan(seq_lens, num_splits, block_size=BLOCK) -> np.ndarray:
    """Host split plan: int32 [B, S, 2] key ranges (see mla.h)."""
    sl = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))
    B = int(sl.shape[0])
    out = np.zeros((B, int(num_splits), 2), dtype=np.int32)
    st = load().mla_split_plan(sl.ctypes.data_as(ctypes.c_void_p), B, int(block_size),
                               int(num_splits), out.ctypes.data_as(ctypes.c_void_p))
    _check("mla_split_plan", st)
    return out


def mla_plan_decode(seq_lens, q_len, n_h, num_slots, block_size=BLOCK):
    """Host schedule (see mla.h).  Returns (work int32 [n, 4], lists int32 [K + 1],
    split int32 [k, 3], n_parts)."""
    sl = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))
    B = int(sl.shape[0])
    n_work, n_lists = ctypes.c_int32(0), ctypes.c_int32(0)
    n_split, n_parts = ctypes.c_int32(0), ctypes.c_int32(0)
    lists = np.zeros(max(1, int(num_slots)) + 1, dtype=np.int32)
    cap = 16
    while True:
        work = np.zeros((cap, 4), dtype=np.int32)
        split = np.zeros((cap, 3), dtype=np.int32)
        st = load().mla_plan_decode(sl.ctypes.data_as(ctypes.c_void_p), B, int(q_len),
                                    int(block_size), int(n_h), int(num_slots), cap,
                                    work.ctypes.data_as(ctypes.c_void_p), ctypes.byref(n_work),
                                    lists.ctypes.data_as(ctypes.c_void_p), ctypes.byref(n_lists),
                                    split.ctypes.data_as(ctypes.c_void_p), ctypes.byref(n_split),
                                    ctypes.byref(n_parts))
        if st == MLA_OK:
            return (work[:n_work.value].copy(), lists[:n_lists.value + 1].copy(),
                    split[:n_split.value].copy(), int(n_parts.value))
        if st == 2 and max(n_work.value, n_split.value) > cap:
            cap = max(n_work.value, n_split.value)
            continue
        _check("mla_plan_decode", st)


def mla_decode_paged_planned(q_lat, kv_cache, block_table, B, q_len, softmax_scale, work,
                             o_lat, lse, o_part=None, lse_part=None, lists=None, stream=None):
    """Attention over a device schedule from mla_plan_decode (see mla.h); lists
    (device int32 [K + 1]) is optional."""
    torch = _torch()
    dt = _dtype_code(q_lat)
    if kv_cache.dtype != q_lat.dtype:
        raise TypeError("kv_cache dtype differs from q_lat")
    n_h = int(q_lat.shape[-2])
    rows = int(B) * int(q_len)
    if q_lat.shape[-1] != ROW or q_lat.numel() != rows * n_h * ROW:
        raise ValueError("q_lat must hold [B, q_len, n_h, 576]")
    if work.dim() != 2 or work.shape[1] != 4:
        raise ValueError("work must be [n_work, 4]")
    if lists is not None and (lists.dim() != 1 or lists.shape[0] < 2):
        raise ValueError("lists must be [n_lists + 1]")
    if o_lat.numel() != rows * n_h * D_C or lse.numel() != rows * n_h:
        raise ValueError("o_lat / lse must hold [B, q_len, n_h, 512] / [B, q_len, n_h]")
    if o_part is not None and (o_part.shape[-1] != D_C or o_part.numel() % (n_h * D_C) or
                               lse_part is None or lse_part.numel() * D_C != o_part.numel()):
        raise ValueError("o_part / lse_part must be [n_parts, n_h, 512] / [n_parts, n_h]")
    f32 = torch.float32
    st = load().mla_decode_paged_planned(
        _dev(q_lat, "q_lat"), _dev(kv_cache, "kv_cache"), int(kv_cache.shape[0]),
        int(kv_cache.shape[1]), _dev(block_table, "block_table", torch.int32),
        int(block_table.shape[1]), int(B), int(q_len), n_h, dt, float(softmax_scale),
        _dev(work, "work", torch.int32), int(work.shape[0]), _dev(lists, "lists", torch.int32),
        int(lists.shape[0]) - 1 if lists is not None else 0, _dev(o_part, "o_part", f32),
        _dev(lse_part, "lse_part", f32), int(o_part.shape[0]) if o_part is not None else 0,
        _dev(o_lat, "o_lat", f32), _dev(lse, "lse", f32), _stream(stream))
    _check("mla_decode_paged_planned", st)


def mla_combine_planned(o_part, lse_part, split, n_h, o_lat, lse=None, stream=None):
    """Merge the partials of a plan's split rows (see mla.h)."""
    torch = _torch()
    f32 = torch.float32
    if split.dim() != 2 or split.shape[1] != 3:
        raise ValueError("split must be [n_split, 3]")
    st = load().mla_combine_planned(_dev(o_part, "o_part", f32), _dev(lse_part, "lse_part", f32),
                                    _dev(split, "split", torch.int32), int(split.shape[0]),
                                    int(n_h), _dev(o_lat, "o_lat", f32), _dev(lse, "lse", f32),
                                    _stream(stream))
    _check("mla_combine_planned", st)


def mla_out_proj_planned(o_lat, o_part, lse_part, split, w_uv, out, lse=None, stream=None):
    """Merge a plan's split rows and project every row through W^UV (see mla.h).
    The split rows of o_lat are scratch; split (and o_part, lse_part) may be
    None when no row is split."""
    torch = _torch()
    f32 = torch.float32
    dt = _dtype_code(w_uv)
    T, n_h = int(o_lat.shape[0]), int(o_lat.shape[1])
    if tuple(o_lat.shape) != (T, n_h, D_C) or tuple(w_uv.shape) != (n_h, D_H, D_C):
        raise ValueError("o_lat must be [T, n_h, 512] and w_uv [n_h, 128, 512]")
    if tuple(out.shape) != (T, n_h, D_H):
        raise ValueError("out must be [T, n_h, 128]")
    if split is not None and (split.dim() != 2 or split.shape[1] != 3):
        raise ValueError("split must be [n_split, 3]")
    n_split = int(split.shape[0]) if split is not None else 0
    st = load().mla_out_proj_planned(
        _dev(o_lat, "o_lat", f32), _dev(o_part, "o_part", f32) if n_split else None,
        _dev(lse_part, "lse_part", f32) if n_split else None,
        _dev(split, "split", torch.int32) if n_split else None, n_split, _dev(w_uv, "w_uv"), T,
        n_h, dt, _dev(out, "out", f32), _dev(lse, "lse", f32), _stream(stream))
    _check("mla_out_proj_planned", st)


def mla_kv_produce_workspace(T, d_model):
    """Workspace bytes of mla_kv_produce (see mla.h)."""
    n = int(load().mla_kv_produce_workspace(int(T), int(d_model)))
    if n < 0:
        raise ValueError("invalid producer sizes")
    return n


def mla_kv_produce(h, w_dkv, kv_gain, w_kr, kv_cache, block_table, seq_idx, pos, rope_base,
                   eps, workspace, stream=None, rope_theta=None):
    """Cache rows of new tokens from their hidden states (see mla.h)."""
    torch = _torch()
    dt = _dtype_code(h)
    T, d_model = int(h.shape[0]), int(h.shape[1])
    if tuple(w_dkv.shape) != (D_C, d_model) or tuple(w_kr.shape) != (D_R, d_model):
        raise ValueError("w_dkv must be [512, d_model] and w_kr [64, d_model]")
    if tuple(kv_gain.shape) != (D_C,):
        raise ValueError("kv_gain must be [512]")
    if w_dkv.dtype != h.dtype or w_kr.dtype != h.dtype or kv_cache.dtype != h.dtype:
        raise TypeError("h, the weights and the cache must share one dtype")
    if workspace.dtype != torch.uint8:
        raise TypeError("workspace must be a uint8 tensor")
    th = _theta(rope_theta)
    st = load().mla_kv_produce(
        _dev(h, "h"), _dev(w_dkv, "w_dkv"), _dev(kv_gain, "kv_gain", torch.float32),
        _dev(w_kr, "w_kr"), T, d_model, dt, float(eps), float(rope_base), _ptr(th),
        _dev(kv_cache, "kv_cache"),
        int(kv_cache.shape[0]), int(kv_cache.shape[1]), _dev(block_table, "block_table", torch.int32),
        int(block_table.shape[0]), int(block_table.shape[1]), _dev(seq_idx, "seq_idx", torch.int32),
        _dev(pos, "pos", torch.int32), _dev(workspace, "workspace"), int(workspace.numel()),
        _stream(stream))
    _check("mla_kv_produce", st)


def mla_q_produce_workspace(T, d_model, d_cq, dtype_code):
    """Workspace bytes of mla_q_produce (see mla.h)."""
    n = int(load().mla_q_produce_workspace(int(T), int(d_model), int(d_cq), int(dtype_code)))
    if n < 0:
        raise ValueError("invalid producer sizes")
    return n


def mla_q_produce(h, w_dq, q_gain, w_uq, w_qr, q_nope, q_rope, eps, workspace, stream=None):
    """Per-head queries of tokens through the compressed query (see mla.h)."""
    torch = _torch()
    dt = _dtype_code(h)
    T, d_model = int(h.shape[0]), int(h.shape[1])
    d_cq = int(w_dq.shape[0])
    n_h = int(q_nope.shape[1])
    if tuple(w_dq.shape) != (d_cq, d_model) or tuple(q_gain.shape) != (d_cq,):
        raise ValueError("w_dq must be [d_cq, d_model] and q_gain [d_cq]")
    if tuple(w_uq.shape) != (n_h * D_H, d_cq) or tuple(w_qr.shape) != (n_h * D_R, d_cq):
        raise ValueError("w_uq must be [n_h*128, d_cq] and w_qr [n_h*64, d_cq]")
    if tuple(q_nope.shape) != (T, n_h, D_H) or tuple(q_rope.shape) != (T, n_h, D_R):
        raise ValueError("q_nope must be [T, n_h, 128] and q_rope [T, n_h, 64]")
    for name, t in (("w_dq", w_dq), ("w_uq", w_uq), ("w_qr", w_qr), ("q_nope", q_nope),
                    ("q_rope", q_rope)):
        if t.dtype != h.dtype:
            raise TypeError(f"{name} must have h's dtype")
    if workspace.dtype != torch.uint8:
        raise TypeError("workspace must be a uint8 tensor")
    st = load().mla_q_produce(
        _dev(h, "h"), _dev(w_dq, "w_dq"), _dev(q_gain, "q_gain", torch.float32), _dev(w_uq, "w_uq"),
        _dev(w_qr, "w_qr"), T, d_model, d_cq, n_h, dt, float(eps), _dev(q_nope, "q_nope"),
        _dev(q_rope, "q_rope"), _dev(workspace, "workspace"), int(workspace.numel()),
        _stream(stream))
    _check("mla_q_produce", st)


def mla_prefill_mha_workspace(max_seq_len, n_h):
    """Workspace bytes of mla_prefill_mha (see mla.h)."""
    n = int(load().mla_prefill_mha_workspace(int(max_seq_len), int(n_h)))
    if n < 0:
        raise ValueError("invalid sizes for mla_prefill_mha_workspace")
    return n


def mla_prefill_mha(q_nope, q_rope, q_pos, w_uk, w_uv, kv_cache, block_table, seq_lens, q_len,
                    softmax_scale, rope_base, out, lse, workspace, stream=None, rope_theta=None):
    """Non-absorbed chunked prefill (see mla.h).  seq_lens is a host array [B]."""
    import numpy as np
    torch = _torch()
    dt = _dtype_code(q_nope)
    lens = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))
    B = int(lens.shape[0])
    n_h = int(q_nope.shape[-2])
    T = B * int(q_len)
    if tuple(q_nope.shape) != (T, n_h, D_H) or tuple(q_rope.shape) != (T, n_h, D_R):
        raise ValueError("q_nope must be [B*q_len, n_h, 128] and q_rope [B*q_len, n_h, 64]")
    if tuple(w_uk.shape) != (n_h, D_H, D_C) or tuple(w_uv.shape) != (n_h, D_H, D_C):
        raise ValueError("w_uk and w_uv must be [n_h, 128, 512]")
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be [B, max_blocks]")
    if out.numel() != T * n_h * D_H or lse.numel() != T * n_h:
        raise ValueError("out must hold [B*q_len, n_h, 128] and lse [B*q_len, n_h]")
    for name, t in (("q_rope", q_rope), ("w_uk", w_uk), ("w_uv", w_uv), ("kv_cache", kv_cache)):
        if t.dtype != q_nope.dtype:
            raise TypeError(f"{name} must have q_nope's dtype")
    if workspace.dtype != torch.uint8:
        raise TypeError("workspace must be a uint8 tensor")
    f32 = torch.float32
    th = _theta(rope_theta)
    st = load().mla_prefill_mha(
        _dev(q_nope, "q_nope"), _dev(q_rope, "q_rope"), _dev(q_pos, "q_pos", torch.int32),
        _dev(w_uk, "w_uk"), _dev(w_uv, "w_uv"), _dev(kv_cache, "kv_cache"),
        int(kv_cache.shape[0]), int(kv_cache.shape[1]),
        _dev(block_table, "block_table", torch.int32), int(block_table.shape[1]),
        lens.ctypes.data_as(ctypes.c_void_p), B, int(q_len), n_h, dt, float(softmax_scale),
        float(rope_base), _ptr(th), _dev(out, "out", f32), _dev(lse, "lse", f32),
        _dev(workspace, "workspace"), int(workspace.numel()), _stream(stream))
    _check("mla_prefill_mha", st)


def mla_q_produce_direct(h, w_qc, w_qr, q_nope, q_rope, stream=None):
    """Per-head queries straight from hidden states (no query compression; see mla.h)."""
    dt = _dtype_code(h)
    T, d_model = int(h.shape[0]), int(h.shape[1])
    n_h = int(q_nope.shape[1])
    if tuple(w_qc.shape) != (n_h * D_H, d_model) or tuple(w_qr.shape) != (n_h * D_R, d_model):
        raise ValueError("w_qc must be [n_h*128, d_model] and w_qr [n_h*64, d_model]")
    if tuple(q_nope.shape) != (T, n_h, D_H) or tuple(q_rope.shape) != (T, n_h, D_R):
        raise ValueError("q_nope must be [T, n_h, 128] and q_rope [T, n_h, 64]")
    for name, t in (("w_qc", w_qc), ("w_qr", w_qr), ("q_nope", q_nope), ("q_rope", q_rope)):
        if t.dtype != h.dtype:
            raise TypeError(f"{name} must have h's dtype")
    st = load().mla_q_produce_direct(_dev(h, "h"), _dev(w_qc, "w_qc"), _dev(w_qr, "w_qr"), T,
                                     d_model, n_h, dt, _dev(q_nope, "q_nope"),
                                     _dev(q_rope, "q_rope"), _stream(stream))
    _check("mla_q_produce_direct", st)


def mla_o_proj_workspace(T, n_h, d_model, dtype_code):
    """Workspace bytes of mla_o_proj (see mla.h)."""
    n = int(load().mla_o_proj_workspace(int(T), int(n_h), int(d_model), int(dtype_code)))
    if n < 0:
        raise ValueError("invalid sizes for mla_o_proj_workspace")
    return n


def mla_o_proj(out, w_o, u, workspace=None, stream=None):
    """eq. 8's u = W^O [o_1; ...; o_nh] (see mla.h).  out fp32 [T, n_h, 128]."""
    torch = _torch()
    dt = _dtype_code(w_o)
    T, n_h = int(out.shape[0]), int(out.shape[1])
    d_model = int(w_o.shape[0])
    if tuple(out.shape) != (T, n_h, D_H) or out.dtype != torch.float32:
        raise ValueError("out must be fp32 [T, n_h, 128]")
    if tuple(w_o.shape) != (d_model, n_h * D_H) or tuple(u.shape) != (T, d_model):
        raise ValueError("w_o must be [d_model, n_h*128] and u [T, d_model]")
    if u.dtype != w_o.dtype:
        raise TypeError("u must have w_o's dtype")
    if workspace is not None and workspace.dtype != torch.uint8:
        raise TypeError("workspace must be a uint8 tensor")
    st = load().mla_o_proj(_dev(out, "out", torch.float32), _dev(w_o, "w_o"), T, n_h, d_model, dt,
                           _dev(u, "u"), _dev(workspace, "workspace"),
                           0 if workspace is None else int(workspace.numel()), _stream(stream))
    _check("mla_o_proj", st)


NOALLOC_SCRATCH_BYTES = 64 * 1024 * 1024


def mla_decode_paged_noalloc(q_lat, kv_cache, block_table, seq_lens, q_len, softmax_scale,
                             num_splits, o_lat, lse, stream=None):
    """mla_decode_paged (+ mla_splitkv_combine) with the split partials in the
    library's own per-device scratch array (see mla.h): no workspace argument."""
    torch = _torch()
    dt = _dtype_code(q_lat)
    if kv_cache.dtype != q_lat.dtype:
        raise TypeError("kv_cache dtype differs from q_lat")
    B = int(seq_lens.shape[0])
    n_h = int(q_lat.shape[-2])
    if q_lat.shape[-1] != ROW or q_lat.numel() != B * q_len * n_h * ROW:
        raise ValueError("q_lat must hold [B, q_len, n_h, 576]")
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be [B, max_blocks]")
    rows = B * q_len * n_h
    if o_lat.numel() != rows * D_C or lse.numel() != rows:
        raise ValueError("o_lat / lse must hold [B, q_len, n_h, 512] / [B, q_len, n_h]")
    f32 = torch.float32
    st = load().mla_decode_paged_noalloc(
        _dev(q_lat, "q_lat"), _dev(kv_cache, "kv_cache"), int(kv_cache.shape[0]),
        int(kv_cache.shape[1]), _dev(block_table, "block_table", torch.int32),
        int(block_table.shape[1]), _dev(seq_lens, "seq_lens", torch.int32), B, int(q_len), n_h,
        dt, float(softmax_scale), int(num_splits), _dev(o_lat, "o_lat", f32),
        _dev(lse, "lse", f32), _stream(stream))
    _check("mla_decode_paged_noalloc", st)


# ---------------------------------------------------------------------------
# Quantised (FP8 E4M3) latent cache
# ---------------------------------------------------------------------------

def _fp8_cache(kv_cache, kv_scale):
    torch = _torch()
    if kv_cache.dtype != torch.uint8 or kv_cache.dim() != 3 or kv_cache.shape[2] != ROW:
        raise ValueError("an FP8 kv_cache is uint8 [num_blocks, 64, 576]")
    if kv_scale.dtype != torch.float32 or tuple(kv_scale.shape) != (kv_cache.shape[0],
                                                                    kv_cache.shape[1], 2):
        raise ValueError("kv_scale must be float32 [num_blocks, 64, 2]")


def mla_kv_append_fp8(kv_cache, kv_scale, block_table, c_kv, k_rope, seq_idx, pos,
                      rope_base=10000.0, stream=None, rope_theta=None):
    """Quantise rows [c_kv ; R_pos k_rope] into the FP8 cache (see mla.h)."""
    torch = _torch()
    _fp8_cache(kv_cache, kv_scale)
    dt = _dtype_code(c_kv)
    n = int(c_kv.shape[0])
    if tuple(c_kv.shape) != (n, D_C) or tuple(k_rope.shape) != (n, D_R) or k_rope.dtype != c_kv.dtype:
        raise ValueError("c_kv must be [n, 512] and k_rope [n, 64], of one dtype")
    if tuple(seq_idx.shape) != (n,) or tuple(pos.shape) != (n,):
        raise ValueError("seq_idx and pos must be [n]")
    th = _theta(rope_theta)
    st = load().mla_kv_append_fp8(
        _dev(kv_cache, "kv_cache"), _dev(kv_scale, "kv_scale"), dt, int(kv_cache.shape[0]),
        int(kv_cache.shape[1]), _dev(block_table, "block_table", torch.int32),
        int(block_table.shape[0]), int(block_table.shape[1]), _dev(c_kv, "c_kv"),
        _dev(k_rope, "k_rope"), _dev(seq_idx, "seq_idx", torch.int32),
        _dev(pos, "pos", torch.int32), n, float(rope_base), _ptr(th), _stream(stream))
    _check("mla_kv_append_fp8", st)


def mla_decode_paged_fp8(q_lat, kv_cache, kv_scale, block_table, seq_lens, q_len, softmax_scale,
                         num_splits=1, o_part=None, lse_part=None, o_lat=None, lse=None,
                         stream=None):
    """Latent attention over the FP8 cache (see mla.h); q_lat bf16 [B*q_len, n_h, 576]."""
    torch = _torch()
    _fp8_cache(kv_cache, kv_scale)
    if q_lat.dtype != torch.bfloat16:
        raise TypeError("q_lat must be bf16")
    B = int(seq_lens.shape[0])
    n_h = int(q_lat.shape[-2])
    if q_lat.shape[-1] != ROW or q_lat.numel() != B * q_len * n_h * ROW:
        raise ValueError("q_lat must hold [B, q_len, n_h, 576]")
    rows = B * q_len * n_h
    if int(num_splits) > 1:
        if o_part is None or lse_part is None or o_part.numel() != rows * num_splits * D_C \
                or lse_part.numel() != rows * num_splits:
            raise ValueError("o_part / lse_part must hold [B, S, q_len, n_h, 512] / [B, S, q_len, n_h]")
    elif o_lat is None or lse is None or o_lat.numel() != rows * D_C or lse.numel() != rows:
        raise ValueError("o_lat / lse must hold [B, q_len, n_h, 512] / [B, q_len, n_h]")
    f32 = torch.float32
    st = load().mla_decode_paged_fp8(
        _dev(q_lat, "q_lat"), _dev(kv_cache, "kv_cache"), _dev(kv_scale, "kv_scale"),
        int(kv_cache.shape[0]), int(kv_cache.shape[1]),
        _dev(block_table, "block_table", torch.int32), int(block_table.shape[1]),
        _dev(seq_lens, "seq_lens", torch.int32), B, int(q_len), n_h, float(softmax_scale),
        int(num_splits), _dev(o_part, "o_part", f32), _dev(lse_part, "lse_part", f32),
        _dev(o_lat, "o_lat", f32), _dev(lse, "lse", f32), _stream(stream))
    _check("mla_decode_paged_fp8", st)


def mla_decode_paged_planned_fp8(q_lat, kv_cache, kv_scale, block_table, B, q_len, softmax_scale,
                                 work, o_lat, lse, o_part=None, lse_part=None, lists=None,
                                 stream=None):
    """mla_decode_paged_planned over the FP8 cache (see mla.h)."""
    torch = _torch()
    _fp8_cache(kv_cache, kv_scale)
    if q_lat.dtype != torch.bfloat16:
        raise TypeError("q_lat must be bf16")
    n_h = int(q_lat.shape[-2])
    rows = int(B) * int(q_len)
    if q_lat.shape[-1] != ROW or q_lat.numel() != rows * n_h * ROW:
        raise ValueError("q_lat must hold [B, q_len, n_h, 576]")
    if work.dim() != 2 or work.shape[1] != 4:
        raise ValueError("work must be [n_work, 4]")
    if lists is not None and (lists.dim() != 1 or lists.shape[0] < 2):
        raise ValueError("lists must be [n_lists + 1]")
    if o_lat.numel() != rows * n_h * D_C or lse.numel() != rows * n_h:
        raise ValueError("o_lat / lse must hold [B, q_len, n_h, 512] / [B, q_len, n_h]")
    if o_part is not None and (o_part.shape[-1] != D_C or o_part.numel() % (n_h * D_C) or
                               lse_part is None or lse_part.numel() * D_C != o_part.numel()):
        raise ValueError("o_part / lse_part must be [n_parts, n_h, 512] / [n_parts, n_h]")
    n_parts = int(o_part.shape[0]) if o_part is not None else 0
    f32 = torch.float32
    st = load().mla_decode_paged_planned_fp8(
        _dev(q_lat, "q_lat"), _dev(kv_cache, "kv_cache"), _dev(kv_scale, "kv_scale"),
        int(kv_cache.shape[0]), int(kv_cache.shape[1]),
        _dev(block_table, "block_table", torch.int32), int(block_table.shape[1]), int(B),
        int(q_len), n_h, float(softmax_scale), _dev(work, "work", torch.int32),
        int(work.shape[0]), _dev(lists, "lists", torch.int32),
        int(lists.shape[0]) - 1 if lists is not None else 0, _dev(o_part, "o_part", f32),
        _dev(lse_part, "lse_part", f32), n_parts, _dev(o_lat, "o_lat", f32), _dev(lse, "lse", f32),
        _stream(stream))
    _check("mla_decode_paged_planned_fp8", st)


# ---------------------------------------------------------------------------
# Kernel timing
# ---------------------------------------------------------------------------

def mla_time_attention(start_event, stop_event):
    """Arm this thread's next attention launch with two HIP event handles
    (raw hipEvent_t values, or None): the dispatch records its own start and
    end in them (see mla.h)."""
    _check("mla_time_attention", load().mla_time_attention(start_event, stop_event))


_hip_rt: Optional[ctypes.CDLL] = None


def _hip():
    """The HIP runtime the library runs on (already loaded with it)."""
    global _hip_rt
    if _hip_rt is None:
        load()
        rt = ctypes.CDLL("libamdhip64.so.7")
        rt.hipEventCreate.argtypes = [ctypes.POINTER(_P)]
        rt.hipEventDestroy.argtypes = [_P]
        rt.hipEventSynchronize.argtypes = [_P]
        rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(_F), _P, _P]
        for fn in (rt.hipEventCreate, rt.hipEventDestroy, rt.hipEventSynchronize,
                   rt.hipEventElapsedTime):
            fn.restype = ctypes.c_int
        _hip_rt = rt
    return _hip_rt


class KernelTimer:
    """A start / stop pair of HIP events (timing enabled, current device) for
    mla_time_attention: ``arm()`` before the attention call, ``elapsed_ms()``
    once the stream has passed the kernel, ``close()`` to release the events
    (not left to garbage collection, which may run after the runtime has shut
    down)."""

    def __init__(self):
        rt = _hip()
        self.start, self.stop = _P(), _P()
        for ev in (self.start, self.stop):
            if rt.hipEventCreate(ctypes.byref(ev)) != 0:
                raise RuntimeError("hipEventCreate failed")

    def arm(self):
        mla_time_attention(self.start, self.stop)

    def elapsed_ms(self) -> float:
        rt = _hip()
        if rt.hipEventSynchronize(self.stop) != 0:
            raise RuntimeError("hipEventSynchronize failed")
        ms = _F()
        st = rt.hipEventElapsedTime(ctypes.byref(ms), self.start, self.stop)
        if st != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({st}): events not recorded")
        return float(ms.value)

    def close(self):
        if _hip_rt is not None:
            for ev in (self.start, self.stop):
                if ev.value:
                    _hip_rt.hipEventDestroy(ev)
                    ev.value = None
