// Device helpers of the two-role decode kernels for 64-head groups
// (decode_h64.hip: bf16 cache; decode_h64_fp8.hip: FP8 E4M3 cache).  Both
// kernels run 8 waves per workgroup: score waves 0..3 (QK^T and the softmax
// step, the query held in AGPRs) and value waves 4..7 (PV with the
// accumulators in AGPRs, and the direct-to-LDS tile loads).
#pragma once

#include "mla_common.h"

namespace mla {

namespace {

#ifndef MLA_RESCALE_LOG2
#define MLA_RESCALE_LOG2 8.0f
#endif
constexpr float RESCALE_LOG2 = MLA_RESCALE_LOG2;  // lazy-rescale threshold (log2 units)
constexpr float NEG_BIG = -1.0e30f;   // finite "no key yet" running max

constexpr int NTHREADS = 512;                // 4 score waves + 4 value waves
constexpr int HG = 64;                       // heads per workgroup
constexpr int KSTEPS = ROW / 32;             // 18
constexpr int KSTEPS_A = 16;                 // query k-steps held in AGPRs (the rest in VGPRs)
constexpr int IDCAP = 512;                   // block ids staged per chunk of an item
#ifndef QK_REDO_STEP
#define QK_REDO_STEP 6
#endif
constexpr int QK_MID = QK_REDO_STEP;         // QK k-steps issued before the redo check

// One direct-to-LDS load, written out (scalar base + 32-bit lane offset, M0 =
// LDS destination; one wait state between the M0 write and its use): lane l's
// 16 bytes from base + lane_src land at LDS byte lds_dst + 16 l.  Left to the
// compiler, a direct-to-LDS load among LDS reads makes it wait for every
// outstanding LDS read (lgkmcnt(0)) before the next use.  The statement has no
// outputs; the loads are awaited explicitly (vm_wait) before the stage is
// read.  Nothing else in the tile loop of a value wave issues vector-memory
// instructions, so the counts given to vm_wait are exact.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // M0 is named as clobbered on purpose
__device__ __forceinline__ void dma_one(unsigned lds_dst, const char* base, unsigned lane_src) {
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %2"
      :
      : "v"(lane_src), "s"(lds_dst), "s"(base)
      : "m0");
}
#pragma clang diagnostic pop

typedef int v2i_t __attribute__((ext_vector_type(2)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v2i_t lds_v2i_t;
typedef __bf16 v2bf_t __attribute__((ext_vector_type(2)));

// 8 E4M3 codes -> the same 8 values in bf16 (exact).
__device__ __forceinline__ i16x8_t widen8(v2i_t w) {
  const v2bf_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)w[0], 1.0f, false);
  const v2bf_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)w[0], 1.0f, true);
  const v2bf_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)w[1], 1.0f, false);
  const v2bf_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)w[1], 1.0f, true);
  const u32x4_t u = {__builtin_bit_cast(unsigned, a), __builtin_bit_cast(unsigned, b),
                     __builtin_bit_cast(unsigned, c), __builtin_bit_cast(unsigned, d)};
  return __builtin_bit_cast(i16x8_t, u);
}

// s_waitcnt vmcnt(N) with the other counters untouched (gfx9 encoding).
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier for LDS traffic only (vmcnt is managed separately).
__device__ __forceinline__ void lds_sync() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// MFMAs written out so that each operand sits in the register file chosen for
// it: d = a b^T (+ d).  Score waves: the query (B operand) in AGPRs (all but
// its last two k-steps), K and the scores in VGPRs.  Value waves: the
// accumulators in AGPRs (ACC_CD form), V^T and P in VGPRs.  The two roles run
// in one kernel, whose 256 registers per wave (two waves per SIMD) the compiler
// splits into 128 VGPRs and 128 AGPRs; the query (144 registers) and the
// accumulators (128) each fill the AGPR half, the rest of either role fits the
// VGPR half.  The compiler does not see these as MFMAs, so the code adds
// the wait states it would otherwise insert: after the query is written to
// AGPRs, before VALU code reads the scores (qk_drain), and around VALU access to
// the accumulators (a redo's rescale, the epilogue).
__device__ __forceinline__ void mma_qk_first(f32x4_t& d, const i16x8_t& k, const i16x8_t& q) {
  asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(k), "a"(q));
}
template <bool Q_IN_AGPR>
__device__ __forceinline__ void mma_qk(f32x4_t& d, const i16x8_t& k, const i16x8_t& q) {
  if constexpr (Q_IN_AGPR)
    asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(k), "a"(q));
  else
    asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(k), "v"(q));
}
// FP8 scores: the K operand was widened by VALU instructions, which the
// compiler does not order against these asm MFMAs: two wait states first.
__device__ __forceinline__ void mma_qk8_first(f32x4_t& d, const i16x8_t& k, const i16x8_t& q) {
  asm("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(k), "a"(q));
}
template <bool Q_IN_AGPR, bool FIRST>
__device__ __forceinline__ void mma_qk8(f32x4_t& d, const i16x8_t& k, const i16x8_t& q) {
  if constexpr (FIRST)
    asm("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(k), "v"(q));
  else if constexpr (Q_IN_AGPR)
    asm("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(k), "a"(q));
  else
    asm("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(k), "v"(q));
}
__device__ __forceinline__ void mma_pv(f32x4_t& d, const i16x8_t& v, const i16x8_t& p) {
  d = __builtin_amdgcn_mfma_f32_16x16x32_bf16((bf16x8_t)v, (bf16x8_t)p, d, 0, 0, 0);
}
// d *= f for an accumulator held in AGPRs, one element at a time through a
// VGPR: left to the compiler, VALU arithmetic on the accumulators (rare here)
// makes it keep all of them in VGPRs across the tile loop.
__device__ __forceinline__ void scale_agpr(f32x4_t& d, float f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float x = d[i], t;
    asm volatile(
        "v_accvgpr_read_b32 %1, %0\n\t"
        "v_mul_f32 %1, %1, %2\n\t"
        "v_accvgpr_write_b32 %0, %1"
        : "+a"(x), "=&v"(t)
        : "v"(f));
    d[i] = x;
  }
}
__device__ __forceinline__ void mma_sum(f32x4_t& d, const i16x8_t& ones, const i16x8_t& p) {
  asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(ones), "v"(p));
}
// 24 wait states between the last QK MFMA writing the scores and any other
// instruction touching them (an 8-pass MFMA result needs 11 before a VALU
// read; 24 also covers 16-pass forms).
__device__ __forceinline__ void qk_drain(f32x4_t& a, f32x4_t& b, f32x4_t& c, f32x4_t& d) {
  asm volatile("s_nop 15\n\ts_nop 7" : "+v"(a), "+v"(b), "+v"(c), "+v"(d));
}
__device__ __forceinline__ void qk_drain6(f32x4_t& a, f32x4_t& b, f32x4_t& c, f32x4_t& d,
                                          f32x4_t& e, f32x4_t& f) {
  asm volatile("s_nop 15\n\ts_nop 7" : "+v"(a), "+v"(b), "+v"(c), "+v"(d), "+v"(e), "+v"(f));
}

__device__ __forceinline__ i16x8_t lds_b128(const char* p) {
  return *reinterpret_cast<const i16x8_t*>(p);
}

// Stage the block ids of blocks [blk0, blk0 + nblk) of a sequence (out-of-range
// ids become -1: a missing block).  Both barriers are workgroup-wide: the first
// waits until every wave is done with the previous chunk's buffers.  Returns
// whether any block of the chunk is missing (the same value in every thread).
__device__ __forceinline__ bool stage_ids(int* ids, const int* trow, int blk0, int nblk,
                                          int num_blocks) {
  __syncthreads();
  bool missing = false;
  for (int e = threadIdx.x; e < nblk; e += NTHREADS) {
    const int id = trow[blk0 + e];
    const bool ok = id >= 0 && id < num_blocks;
    ids[e] = ok ? id : -1;
    missing |= !ok;
  }
  return __syncthreads_or(missing) != 0;
}

// Workgroup id -> (unit, head group): a unit is one work item, or with work
// lists one list of items run in order.  The head groups of one unit sit 8 ids
// apart, so that round-robin dispatch puts them on one XCD and the second read
// of every tile is served by that XCD's L2.  Returns false for a workgroup
// past the last unit.
__device__ __forceinline__ bool h64_unit(int n_h, int n_items, const int* lists, int n_lists,
                                         int& hgrp, int& i_begin, int& i_end) {
  const int ngroups = n_h / HG;
  const int wid = blockIdx.x;
  hgrp = (wid >> 3) % ngroups;
  const int unit = (wid / (8 * ngroups)) * 8 + (wid & 7);
  if (lists != nullptr) {
    if (unit >= n_lists) return false;
    i_begin = lists[unit];
    i_end = lists[unit + 1];
  } else {
    if (unit >= n_items) return false;
    i_begin = unit;
    i_end = unit + 1;
  }
  return true;
}

}  // namespace

}  // namespace mla
