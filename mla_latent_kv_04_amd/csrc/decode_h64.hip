// Paged latent attention, bf16, for head counts that are multiples of 64
// (DeepSeek-V2 uses 128 heads).
//
// Same computation as decode.hip (eq. 7 of the DeepSeek-V2 notes,
// irregular6612.github.io, §2.1.1, on the absorbed query and the cached
// [c^KV ; k^R] rows of the DeepSeek-V2 MLA blog, adg.csdn.net, part 2 §2.2.2).
//
// One workgroup owns 64 heads of one unit of work: a work item (a row's key
// range) or a list of items run in order.  With 128 heads the two head groups
// of a unit are launched 8 workgroup ids apart, which places them on the same
// XCD so the second read of every KV tile is served by that XCD's L2.
//
// Eight waves in two roles:
//
//   score waves 0..3, (hq, th) = (w & 1, w >> 1): scores of heads
//     32hq..32hq+31 against tokens 16th..16th+15 of a tile, with the query
//     (144 registers) held in AGPRs and fed to the MFMA directly; then the
//     softmax step: scale, mask, tile maxima, P against the running max of
//     the head group, P and the maxima written to LDS.
//   value waves 4..7, wp = w - 4: output dims 128wp..128wp+127 for all 64
//     heads (128 accumulator registers, in AGPRs); each transposed V^T
//     fragment feeds four 16-head MFMAs, and one more MFMA against a ones
//     fragment sums the bf16 P of head block wp, so the softmax denominator
//     uses exactly the P of the numerator.  These waves also issue the
//     direct-to-LDS loads of the tiles.
//
// Each SIMD holds one wave of each role; the hardware interleaves the two, so
// that one role's VALU and LDS work overlaps the other's MFMAs.  Iteration a
// of the tile loop has one workgroup barrier:
//
//   barrier A(a): tile a+1 has landed; P(a), its maxima and flags are in LDS;
//                 tile a-1 is no longer read by anyone
//   score waves: QK^T of tile a+1 (36 MFMAs per wave), then its softmax step
//                (scale, mask, tile maxima, P(a+1) against the running max,
//                into the other P buffer, and the flags)
//   value waves: P(a) and V(a) into registers, PV of the first dims, loads of
//                tile a+3 into the stage of tile a-1, the rest of PV, and the
//                P row sums
//   [redo a] only if a score wave saw a score of tile a beat the running max
//            by more than 2^8 (log2 domain): the score waves agree on the new
//            max and rewrite P(a), then (one more barrier) the value waves
//            rescale their accumulators before reading P(a).
//
// P, the tile maxima and the flags alternate between two buffers by tile
// parity, so the softmax of tile a+1 never touches what the value waves read
// for tile a; a second barrier per tile between the two halves of each role's
// work (an earlier form) bought nothing and cost 1.5%.
//
// Tiles are 32 tokens (half a paged block) in four LDS stages, loaded three
// tiles ahead.
//
// LDS: four tile stages of 36,864 bytes (32 token rows of 72 16-byte chunks,
// swizzled inside 256-byte groups so that the K and V fragment reads are free
// of bank conflicts; one tile is exactly 36 direct-to-LDS instructions), two
// P buffers, two sets of tile maxima and flags, rescale factors, and the block
// ids of the current item.
#include "mla_common.h"
#include "mla_internal.h"

namespace mla {

namespace {

#ifndef MLA_RESCALE_LOG2
#define MLA_RESCALE_LOG2 8.0f
#endif
constexpr float RESCALE_LOG2 = MLA_RESCALE_LOG2;  // lazy-rescale threshold (log2 units)
constexpr float NEG_BIG = -1.0e30f;   // finite "no key yet" running max

constexpr int NTHREADS = 512;                // 4 score waves + 4 value waves
constexpr int HG = 64;                       // heads per workgroup
constexpr int TT = 32;                       // tokens per tile (half a paged block)
constexpr int NSTAGE = 4;                    // tile stages in LDS
constexpr int RSLOTS = ROW * 2 / 16;         // 72 16-byte chunks per token row
constexpr int NINST = TT * RSLOTS / 64;      // 36 direct-to-LDS instructions per tile
constexpr int STAGE = NINST * 1024;          // 36,864 bytes
constexpr int NDMA = NINST / 4;              // 9 per value wave
constexpr int KSTEPS = ROW / 32;             // 18
constexpr int KSTEPS_A = 16;                 // query k-steps held in AGPRs (the rest in VGPRs)
constexpr int IDCAP = 512;                   // block ids staged per chunk of an item
#ifndef PV_PHASE_A
#define PV_PHASE_A 4
#endif
#ifndef QK_REDO_STEP
#define QK_REDO_STEP 6
#endif

constexpr int PV_A = PV_PHASE_A;             // PV dim blocks (of 8) run before the loads of tile a+3
constexpr int QK_MID = QK_REDO_STEP;         // QK k-steps issued before the redo check

// LDS map (bytes)
constexpr int OFF_STAGE = 0;
constexpr int PBUF = 4 * 64 * 16;                     // P of one tile: [4 head blocks][64 lanes][16 B]
constexpr int OFF_P = OFF_STAGE + NSTAGE * STAGE;     // [2] P buffers
constexpr int OFF_MAX = OFF_P + 2 * PBUF;             // float [2][2 token halves][64]
constexpr int OFF_F = OFF_MAX + 2 * 2 * HG * 4;       // float [64] rescale factors
constexpr int OFF_FLAG = OFF_F + HG * 4;              // int [2][4] per score wave "my scores move the max"
constexpr int OFF_IDS = OFF_FLAG + 2 * 4 * 4;         // int [IDCAP]
constexpr int OFF_ONES = OFF_IDS + IDCAP * 4;         // 8 bf16 ones
constexpr int SMEM = OFF_ONES + 16;
static_assert(SMEM <= 163840, "LDS budget");
static_assert(TT * RSLOTS * 16 == STAGE && NINST % 4 == 0, "a tile is whole load instructions");

// FP8 E4M3 cache (codes [blocks, 64, 576] bytes and float32 scale pairs
// [blocks, 64, 2]): a tile is 32 rows of 576 code bytes, each padded to 37
// 16-byte slots in LDS (the pad slot re-reads slot 0 and is never used), in 19
// load instructions (the last one's spare lanes re-read row 0), then one
// instruction whose first 16 lanes bring the tile's 32 scale pairs.
constexpr int RSLOTS8 = ROW / 16 + 1;                 // 37
constexpr int RS8 = RSLOTS8 * 16;                     // 592-byte LDS row pitch
constexpr int NROWI8 = (TT * RSLOTS8 + 63) / 64;      // 19
constexpr int NINST8 = NROWI8 + 1;                    // 20
constexpr int SCALE_OFF8 = NROWI8 * 1024;             // scale pairs of the tile's rows
constexpr int STAGE8 = NINST8 * 1024;                 // 20,480 bytes
constexpr int NDMA8 = NINST8 / 4;                     // 5 per value wave
static_assert(NINST8 % 4 == 0 && TT * 8 <= 16 * 16, "scales fit 16 lanes of one load");

template <bool FP8> struct Lay;
template <> struct Lay<false> {
  static constexpr int STAGE_BYTES = STAGE, NDMA_W = NDMA;
};
template <> struct Lay<true> {
  static constexpr int STAGE_BYTES = STAGE8, NDMA_W = NDMA8;
};
// P buffers and what follows them sit after the stages of either layout
// (the FP8 stages are smaller; the offsets below are those of the bf16 map,
// which leaves the FP8 map's gap unused)

// ---------------------------------------------------------------------------
// Direct-to-LDS loads.  Instruction j (0..35) of a tile fills stage slots
// 64j..64j+63; slot s holds position s % 72 of token row s / 72 (72 16-byte
// chunks per 1152-byte row, no padding), and lane l of instruction j reads the
// chunk that the row's swizzle (below) places at slot 64j + l.  The swizzle
// only permutes chunks inside aligned 256-byte groups, so the 16 lanes of a
// group read one contiguous 256-byte piece of a row, which the address path
// coalesces; lanes spread over rows 1152 bytes apart would be served at about
// a quarter of the rate.  Value wave wp issues instructions j = wp + 4i.
//
// The instruction is written out (scalar base + 32-bit lane offset, M0 = LDS
// destination; one wait state between the M0 write and its use).  Left to the
// compiler, a direct-to-LDS load among LDS reads makes it wait for every
// outstanding LDS read (lgkmcnt(0)) before the next use.  The statement has no
// outputs; the loads are awaited explicitly (vm_wait) before the stage is read.
// Nothing else in the tile loop of a value wave issues vector-memory
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

// LDS layout of a tile: token row t occupies 72 consecutive 16-byte slots;
// chunk f of the row (bytes 16f .. 16f + 15 of its 1152) sits at slot
// f ^ swz(t) inside its aligned group of 16 chunks (the last, 8-chunk group
// uses swz(t) & 7).  With swz(t) = (t & 7) ^ 5 (t >> 3) neither the 16-byte K
// fragment reads (16 rows x 4 chunks per instruction) nor the transposing V
// reads (8 rows x 32 bytes per 32 lanes) hit an LDS bank twice in a cycle, as
// the LDS bank-conflict counters confirm; an unswizzled row pitch of 72 or 73
// chunks costs those reads about twice their conflict-free time.
__device__ __forceinline__ int swz(int t) { return (t & 7) ^ (5 * (t >> 3)); }
__device__ __forceinline__ int chunk_slot(int t, int f) {
  return f < 64 ? (f ^ swz(t)) : 64 + ((f - 64) ^ (swz(t) & 7));
}

// Byte offset, in the tile's half block, of the chunk that lane l of
// instruction j moves: the instruction fills stage slots 64j .. 64j + 63 in
// order, slot s = 64j + l being position s % 72 of row s / 72.  The
// swizzle permutes chunks inside aligned 256-byte groups, so the 16 lanes of
// a group still read one contiguous 256-byte piece of the row.
__device__ __forceinline__ unsigned dma_src(int j, int lane) {
  const int slot = 64 * j + lane;
  const int t = slot / RSLOTS, p = slot - t * RSLOTS;
  return (unsigned)(t * (ROW * 2) + chunk_slot(t, p) * 16);   // the slot map is an involution
}

// FP8: byte offset, from the tile's first row (or, for the scale instruction,
// from its first scale pair), of the 16 bytes that lane l of instruction j
// moves.
__device__ __forceinline__ unsigned dma_src8(int j, int lane) {
  if (j >= NROWI8) return (unsigned)((lane & 15) * 16);
  const int slot = 64 * j + lane;
  int t = slot / RSLOTS8, p = slot - t * RSLOTS8;
  if (t >= TT) t = 0, p = 0;
  if (p == RSLOTS8 - 1) p = 0;
  return (unsigned)(t * ROW + p * 16);
}

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

// One chunk of an item: tiles [c0, c1) (tile a = tokens [32a, 32a + 32) of the
// sequence, block a / 2, half a % 2), keys [kb, ke), block ids staged in ids[].
template <bool FP8>
struct Chunk {
  const int* ids;
  int c0, c1, blk0, kb, ke;
  // block id of tile a (tiles past the chunk, which the pipeline touches but
  // never uses, read the chunk's first id)
  __device__ int id(int a) const { return ids[a < c1 ? (a >> 1) - blk0 : 0]; }
  // valid rows [lo, hi) of tile a (none past the chunk or for a missing block)
  __device__ int lo(int a) const { return max(0, kb - a * TT); }
  __device__ int hi(int a) const { return hi_of(a, id(a)); }
  __device__ int hi_of(int a, int id_a) const { return (a >= c1 || id_a < 0) ? 0 : min(TT, ke - a * TT); }
  __device__ bool partial(int a) const { return lo(a) > 0 || hi(a) < TT; }
  __device__ int stage(int a) const {
    return OFF_STAGE + ((a - c0) & (NSTAGE - 1)) * Lay<FP8>::STAGE_BYTES;
  }
  __device__ int par(int a) const { return (a - c0) & 1; }
};

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

template <bool FP8>
__global__ void __launch_bounds__(NTHREADS, 1) decode_h64_kernel(
    const uint16_t* __restrict__ q_lat, const void* __restrict__ cache,
    const float* __restrict__ kv_scale, int num_blocks,
    const int* __restrict__ table, int max_blocks, const int* __restrict__ seq_lens, int q_len,
    int n_h, int n_items, int n_rows, int n_parts, float scale_log2, int S, const int4* __restrict__ work,
    const int* __restrict__ lists, int n_lists, float* __restrict__ o_lat,
    float* __restrict__ lse, float* __restrict__ o_part, float* __restrict__ lse_part) {
  __shared__ __attribute__((aligned(16))) char smem[SMEM];
  float* const maxbuf = reinterpret_cast<float*>(smem + OFF_MAX);
  float* const fbuf = reinterpret_cast<float*>(smem + OFF_F);
  int* const flags = reinterpret_cast<int*>(smem + OFF_FLAG);
  int* const ids = reinterpret_cast<int*>(smem + OFF_IDS);
  float* const l_all = reinterpret_cast<float*>(smem + OFF_P);   // epilogue: [64] denominators
  float* const mx_all = l_all + HG;                               // epilogue: [64] running maxima
  float* const l_part = mx_all + HG;   // FP8 epilogue: [2 token halves][64] normaliser parts

  // Workgroup id -> (unit, head group): a unit is one work item, or with work
  // lists one list of items run in order.  The head groups of one unit sit 8
  // ids apart so that round-robin dispatch puts them on one XCD.
  const int ngroups = n_h / HG;
  const int wid = blockIdx.x;
  const int hgrp = (wid >> 3) % ngroups;
  const int unit = (wid / (8 * ngroups)) * 8 + (wid & 7);
  int i_begin, i_end;
  if (lists != nullptr) {
    if (unit >= n_lists) return;
    i_begin = lists[unit];
    i_end = lists[unit + 1];
  } else {
    if (unit >= n_items) return;
    i_begin = unit;
    i_end = unit + 1;
  }

  const int lane = lane_id(), g = lane >> 4, r16 = lane & 15;
  // the wave index is uniform; saying so keeps the role branch and the DMA
  // addresses scalar
  const int wave = uniform((int)(threadIdx.x >> 6));
  const int hbase = hgrp * HG;                 // first head of the workgroup
  const char* const cache_bytes = reinterpret_cast<const char*>(cache);
  const unsigned lds_base = (unsigned)(uintptr_t)(__attribute__((address_space(3))) char*)smem;

  // all-ones bf16 fragment: its product with P sums P over the tile's tokens.
  // It is read from LDS rather than built from constants: the compiler would
  // rebuild a constant with VALU writes right before the MFMA that reads it,
  // without the wait states that VALU-written MFMA operands need.
  if (threadIdx.x == 0)
    *reinterpret_cast<uint4*>(smem + OFF_ONES) = uint4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  __syncthreads();

  // Both roles walk the same items, chunks and tiles and take the same
  // (workgroup-uniform) redo decisions, so they meet at every barrier.
  if (wave < 4) {
    // =========================== score waves ===========================
    const int hq = wave & 1, th = wave >> 1;
    // K fragment of k-step ks: token 16th + r16, chunk 4ks + g, at byte
    // k_addr(ks) of the stage (the swizzle leaves bits 4.. of the chunk alone)
    const int t_k = 16 * th + r16;
    int kq[4], kq2[2];
#pragma unroll
    for (int q = 0; q < 4; ++q) kq[q] = (t_k * RSLOTS + ((4 * q + g) ^ swz(t_k))) * 16;
#pragma unroll
    for (int q = 0; q < 2; ++q) kq2[q] = (t_k * RSLOTS + 64 + ((4 * q + g) ^ (swz(t_k) & 7))) * 16;
    auto k_addr = [&](int ks) { return ks < 16 ? kq[ks & 3] + 256 * (ks >> 2) : kq2[ks - 16]; };
    // FP8: 8 code bytes of token t_k at byte 32 ks + 8 g of its padded row
    const int k8 = t_k * RS8 + 8 * g;
    constexpr int KPF = 3;  // K fragments are read KPF steps ahead
    // FP8: the scale pairs of this lane's score rows 16th + 4g + i of the
    // current tile (s_lat_keep: of the tile waiting for its PV, for a redo)
    // and the running normaliser of this lane's rows (l_run: tiles done;
    // l_pend: the waiting tile, added once its redo check has passed)
    float s_lat[4] = {1.0f, 1.0f, 1.0f, 1.0f}, s_rope[4] = {1.0f, 1.0f, 1.0f, 1.0f};
    float s_lat_keep[4] = {1.0f, 1.0f, 1.0f, 1.0f};
    float l_run[2] = {0.0f, 0.0f}, l_pend[2] = {0.0f, 0.0f};

    for (int item = i_begin; item < i_end; ++item) {
      const WorkItem wi = decode_item(item, work, n_rows, n_parts, q_len, S, seq_lens, max_blocks);
      if (!uniform(wi.valid)) continue;
      const int kb = uniform(wi.kb), ke = uniform(wi.ke);
      const int* const trow = table + (long)wi.b * max_blocks;

      // Query fragments of this wave's 32 heads (B operand), placed in AGPRs.
      BF16::frag qf[2][KSTEPS];
      const long qrow = (long)(wi.b * q_len + wi.m) * n_h + hbase + hq * 32;
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks)
          qf[hb][ks] = BF16::load8(q_lat + (qrow + hb * 16 + r16) * ROW + ks * 32 + 8 * g);
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int ks = 0; ks < KSTEPS_A; ++ks) asm volatile("" : "+a"(qf[hb][ks].v));
      asm volatile("s_nop 7\n\ts_nop 7");

      float mref[2] = {NEG_BIG, NEG_BIG};  // running max of this wave's heads (log2 domain)
      if constexpr (FP8) {
        l_run[0] = l_run[1] = 0.0f;
        l_pend[0] = l_pend[1] = 0.0f;
      }

      const int t_first = kb / TT;
      const int t_last = kb < ke ? (ke + TT - 1) / TT : t_first;
      for (int c0 = t_first; c0 < t_last;) {
        const int c1 = min(t_last, (c0 & ~1) + 2 * IDCAP);
        const int blk0 = c0 >> 1;
        stage_ids(ids, trow, blk0, ((c1 - 1) >> 1) - blk0 + 1, num_blocks);
        const Chunk<FP8> ch{ids, c0, c1, blk0, kb, ke};

        // scores and maxima of the tile waiting for its PV (kept for a redo)
        f32x4_t sc_keep[2];
        float ml_keep[2];

        // P of this wave's heads and tokens: 4 bf16 per lane and head block,
        // bytes th*8 .. th*8+7 of the lane's 16 bytes of the PV B fragment of
        // head block 2hq + hb (k slots 4th .. 4th+3 of the lane's group:
        // tokens 16th + 4g + i)
        // FP8: the weight of a token carries its latent scale (rounded to
        // bf16 with it), and l_pend gets the same weights over the scale
        auto write_p = [&](int a, const f32x4_t (&sc)[2], const float (&sl)[4]) {
          char* pb = smem + OFF_P + ch.par(a) * PBUF;
#pragma unroll
          for (int hb = 0; hb < 2; ++hb) {
            uint2 w;
            if constexpr (FP8) {
              float p[4];
              l_pend[hb] = 0.0f;
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                // a masked row (score -inf) weighs exactly 0 whatever its scale
                // holds: the value waves zero such rows concurrently, so the
                // scale read here may be the stale bytes of another key
                const bool live = sc[hb][i] != -INFINITY;
                p[i] = live ? BF16::round(fast_exp2(sc[hb][i] - mref[hb]) * sl[i]) : 0.0f;
                l_pend[hb] += live ? p[i] * __builtin_amdgcn_rcpf(sl[i]) : 0.0f;
              }
              w.x = pack_bf16x2(p[0], p[1]);
              w.y = pack_bf16x2(p[2], p[3]);
            } else {
              w.x = pack_bf16x2(fast_exp2(sc[hb][0] - mref[hb]), fast_exp2(sc[hb][1] - mref[hb]));
              w.y = pack_bf16x2(fast_exp2(sc[hb][2] - mref[hb]), fast_exp2(sc[hb][3] - mref[hb]));
            }
            *reinterpret_cast<uint2*>(pb + ((hq * 2 + hb) * 64 + lane) * 16 + th * 8) = w;
          }
        };

        // QK^T of tile a in four chains (head block x k-step parity, so that no
        // MFMA waits for the one just before it), then the softmax step: P
        // against the running max both waves of a head group share.  A wave
        // whose scores would move that max raises its flag (its P, written
        // anyway, is then replaced in a redo).  Every lane of a group writes the
        // same maximum and every lane the same flag: no branches.
        auto k_first = [&](int a, i16x8_t (&kbuf)[KPF + 1]) {
          const char* kp = smem + ch.stage(a);
#pragma unroll
          for (int ks = 0; ks < KPF; ++ks) kbuf[ks] = lds_b128(kp + k_addr(ks));
        };
        auto k_first8 = [&](int a, v2i_t (&kbuf)[KPF + 1]) {
          const char* kp = smem + ch.stage(a) + k8;
#pragma unroll
          for (int ks = 0; ks < KPF; ++ks) kbuf[ks] = *reinterpret_cast<const v2i_t*>(kp + 32 * ks);
        };
        // FP8 QK^T: latent and RoPE parts in separate chains, each multiplied
        // by its token's scale; the codes are widened one k-step ahead
        auto qk8 = [&](int a, int hi, v2i_t (&kbuf)[KPF + 1], f32x4_t (&sc)[2], auto&& mid) {
          const char* kp = smem + ch.stage(a);
          float2 sp[4];
#pragma unroll
          for (int i = 0; i < 4; ++i)
            sp[i] = *reinterpret_cast<const float2*>(kp + SCALE_OFF8 + (16 * th + 4 * g + i) * 8);
          f32x4_t q4[2][2], qr[2];
          i16x8_t kf = widen8(kbuf[0]);
#pragma unroll
          for (int ks = 0; ks < KSTEPS; ++ks) {
            if (ks == QK_MID) mid();
            if (ks + KPF < KSTEPS)
              kbuf[(ks + KPF) % (KPF + 1)] = *reinterpret_cast<const v2i_t*>(kp + k8 + 32 * (ks + KPF));
            const i16x8_t kcur = kf;
            if (ks + 1 < KSTEPS) kf = widen8(kbuf[(ks + 1) % (KPF + 1)]);
#pragma unroll
            for (int hb = 0; hb < 2; ++hb) {
              if (ks < 2)
                mma_qk8_first(q4[hb][ks & 1], kcur, qf[hb][ks].v);
              else if (ks < KSTEPS_A)
                mma_qk8<true, false>(q4[hb][ks & 1], kcur, qf[hb][ks].v);
              else if (ks == KSTEPS_A)
                mma_qk8<false, true>(qr[hb], kcur, qf[hb][ks].v);
              else
                mma_qk8<false, false>(qr[hb], kcur, qf[hb][ks].v);
            }
          }
          qk_drain6(q4[0][0], q4[0][1], q4[1][0], q4[1][1], qr[0], qr[1]);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            s_lat[i] = sp[i].x;
            s_rope[i] = sp[i].y;
          }
#pragma unroll
          for (int hb = 0; hb < 2; ++hb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              sc[hb][i] = (s_lat[i] * (q4[hb][0][i] + q4[hb][1][i]) + s_rope[i] * qr[hb][i]) * scale_log2;
          const int lo = ch.lo(a);
          if (lo > 0 || hi < TT) {  // rare: rows outside [lo, hi) get no weight
#pragma unroll
            for (int hb = 0; hb < 2; ++hb)
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int row = 16 * th + 4 * g + i;
                if (row < lo || row >= hi) sc[hb][i] = -INFINITY;
              }
          }
        };
        // mid() runs after k-step QK_MID - 1 (the redo check: the scores of the
        // next tile do not depend on it, so the MFMAs start first)
        auto qk = [&](int a, int hi, i16x8_t (&kbuf)[KPF + 1], f32x4_t (&sc)[2], auto&& mid) {
          const char* kp = smem + ch.stage(a);
          f32x4_t q4[2][2];
#pragma unroll
          for (int ks = 0; ks < KSTEPS; ++ks) {
            if (ks == QK_MID) mid();
            if (ks + KPF < KSTEPS) kbuf[(ks + KPF) % (KPF + 1)] = lds_b128(kp + k_addr(ks + KPF));
#pragma unroll
            for (int hb = 0; hb < 2; ++hb) {
              if (ks < 2)
                mma_qk_first(q4[hb][ks & 1], kbuf[ks % (KPF + 1)], qf[hb][ks].v);
              else if (ks < KSTEPS_A)
                mma_qk<true>(q4[hb][ks & 1], kbuf[ks % (KPF + 1)], qf[hb][ks].v);
              else
                mma_qk<false>(q4[hb][ks & 1], kbuf[ks % (KPF + 1)], qf[hb][ks].v);
            }
          }
          qk_drain(q4[0][0], q4[0][1], q4[1][0], q4[1][1]);
#pragma unroll
          for (int hb = 0; hb < 2; ++hb) sc[hb] = (q4[hb][0] + q4[hb][1]) * scale_log2;
          const int lo = ch.lo(a);
          if (lo > 0 || hi < TT) {  // rare: rows outside [lo, hi) get no weight
#pragma unroll
            for (int hb = 0; hb < 2; ++hb)
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int row = 16 * th + 4 * g + i;
                if (row < lo || row >= hi) sc[hb][i] = -INFINITY;
              }
          }
        };
        auto softmax = [&](int a, const f32x4_t (&sc)[2]) {
          const int par = ch.par(a);
          bool need = false;
#pragma unroll
          for (int hb = 0; hb < 2; ++hb) {
            const float mx = fmaxf(fmaxf(sc[hb][0], sc[hb][1]), fmaxf(sc[hb][2], sc[hb][3]));
            ml_keep[hb] = group4_max(mx);
            need |= ml_keep[hb] > mref[hb] + RESCALE_LOG2;
            maxbuf[(par * 2 + th) * HG + hq * 32 + hb * 16 + r16] = ml_keep[hb];
          }
          write_p(a, sc, s_lat);
          flags[par * 4 + wave] = __builtin_amdgcn_ballot_w64(need) != 0 ? 1 : 0;
          sc_keep[0] = sc[0];
          sc_keep[1] = sc[1];
          if constexpr (FP8) {
#pragma unroll
            for (int i = 0; i < 4; ++i) s_lat_keep[i] = s_lat[i];
          }
        };

        lds_sync();  // tile c0 has landed
        {
          f32x4_t sc[2];
          if constexpr (FP8) {
            v2i_t kbuf[KPF + 1];
            k_first8(c0, kbuf);
            qk8(c0, ch.hi(c0), kbuf, sc, [] {});
          } else {
            i16x8_t kbuf[KPF + 1];
            k_first(c0, kbuf);
            qk(c0, ch.hi(c0), kbuf, sc, [] {});
          }
          lds_sync();
          softmax(c0, sc);
        }
        for (int a = c0; a < c1; ++a) {
          lds_sync();  // barrier A(a)
          const int par = ch.par(a);
          const int4 fl = *reinterpret_cast<const int4*>(flags + par * 4);
          const int hi_n = ch.hi(a + 1);
          auto redo = [&] {
            if (uniform(fl.x | fl.y | fl.z | fl.w) != 0) {
              // rare: agree on the new running max from both token halves,
              // record the rescale factors, rewrite P(a)
#pragma unroll
              for (int hb = 0; hb < 2; ++hb) {
                const float mx =
                    fmaxf(ml_keep[hb], maxbuf[(par * 2 + (th ^ 1)) * HG + hq * 32 + hb * 16 + r16]);
                const float mnew = mx > mref[hb] + RESCALE_LOG2 ? mx : mref[hb];
                const float f = fast_exp2(mref[hb] - mnew);
                mref[hb] = mnew;
                if (th == 0 && g == 0) fbuf[hq * 32 + hb * 16 + r16] = f;
                if constexpr (FP8) l_run[hb] *= f;
              }
              write_p(a, sc_keep, s_lat_keep);
              lds_sync();  // redone P and the factors are visible to the value waves
            }
            if constexpr (FP8) {
              // tile a's weights are final: into the normaliser
              l_run[0] += l_pend[0];
              l_run[1] += l_pend[1];
            }
          };
          // tile a+1 (past the chunk: fully masked; written but never read)
          f32x4_t sc[2];
          if constexpr (FP8) {
            v2i_t kbuf[KPF + 1];
            k_first8(a + 1, kbuf);
            qk8(a + 1, hi_n, kbuf, sc, redo);
          } else {
            i16x8_t kbuf[KPF + 1];
            k_first(a + 1, kbuf);
            qk(a + 1, hi_n, kbuf, sc, redo);
          }
          softmax(a + 1, sc);
        }
        c0 = c1;
      }

      // ---- epilogue: running maxima for the log-sum-exp -------------------
      __syncthreads();  // every wave is done with the P buffers
      if (th == 0 && g == 0) {
        mx_all[hq * 32 + r16] = mref[0];
        mx_all[hq * 32 + 16 + r16] = mref[1];
      }
      if constexpr (FP8) {
        // the normaliser: this wave's token half of each of its heads
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
          const float l = group4_sum(l_run[hb]);
          if (g == 0) l_part[th * HG + hq * 32 + hb * 16 + r16] = l;
        }
      }
      __syncthreads();  // denominators and maxima visible
      if (wave == 0) {
        const int h = lane;
        const float l = FP8 ? l_part[h] + l_part[HG + h] : l_all[h];
        float* lbase = (wi.part ? lse_part : lse) + wi.orow * n_h + hbase;
        lbase[h] = l > 0.0f ? (mx_all[h] + __log2f(l)) * LN2 : -INFINITY;
      }
    }
  } else {
    // =========================== value waves ===========================
    const int wp = wave - 4;
    const int d0 = wp * 128;                   // first output dim of this wave
    constexpr int NDMA_W = Lay<FP8>::NDMA_W;   // loads per value wave and tile
    unsigned lane_src[NDMA_W];
#pragma unroll
    for (int i = 0; i < NDMA_W; ++i)
      lane_src[i] = FP8 ? dma_src8(wp + 4 * i, lane) : dma_src(wp + 4 * i, lane);
    // V^T fragment of dims d0 + 16db ..: token t = 4g + (r16 >> 2) (and t + 16),
    // dims d0 + 16db + 4 (r16 & 3) .. +3, i.e. chunk d0 / 8 + 2db + b of the
    // row, bytes h8 .. h8 + 7 of it
    const int t_v = 4 * g + (r16 >> 2), b_v = (r16 & 3) >> 1, h8 = (r16 & 1) * 8;
    const int v_lo = t_v * RSLOTS * 16 + d0 * 2 + h8, v_hi = v_lo + 16 * RSLOTS * 16;
    const int s_lo = swz(t_v), s_hi = swz(t_v + 16);
    const i16x8_t ones = lds_b128(smem + OFF_ONES);
    // FP8: the transposing 8-bit read; lane j of each 16-lane group names row
    // T(j / 2) of its group, T(k) = 16 (k / 4) + 4 g + k % 4 (the tokens of P
    // slot k), and the 8 bytes at column d0 + 16 db + 8 (j % 2)
    const int k_v = r16 >> 1;
    const int v8 = (16 * (k_v >> 2) + 4 * g + (k_v & 3)) * RS8 + d0 + 8 * (r16 & 1);

    for (int item = i_begin; item < i_end; ++item) {
      const WorkItem wi = decode_item(item, work, n_rows, n_parts, q_len, S, seq_lens, max_blocks);
      if (!uniform(wi.valid)) continue;
      const int kb = uniform(wi.kb), ke = uniform(wi.ke);
      const int* const trow = table + (long)wi.b * max_blocks;

      // acc: 4 head blocks x this wave's 8 dim blocks; rsum: sum of P for
      // heads 16wp .. 16wp + 15
      f32x4_t acc[4][8];
#pragma unroll
      for (int hb = 0; hb < 4; ++hb)
#pragma unroll
        for (int db = 0; db < 8; ++db) acc[hb][db] = f32x4_t{0, 0, 0, 0};
      f32x4_t rsum = f32x4_t{0, 0, 0, 0};

      const int t_first = kb / TT;
      const int t_last = kb < ke ? (ke + TT - 1) / TT : t_first;
      for (int c0 = t_first; c0 < t_last;) {
        const int c1 = min(t_last, (c0 & ~1) + 2 * IDCAP);
        const int blk0 = c0 >> 1;
        const bool missing = stage_ids(ids, trow, blk0, ((c1 - 1) >> 1) - blk0 + 1, num_blocks);
        const Chunk<FP8> ch{ids, c0, c1, blk0, kb, ke};

        // loads of tile `src` into the stage of tile `dst` (src == dst except
        // past the chunk, where a valid tile is loaded into a stage nobody
        // reads, so that every tile slot issues the same number of loads and
        // the vmcnt waits stay exact).  id is src's block (load_id: a missing
        // block is read from block 0 instead; its rows are zeroed and masked).
        auto issue = [&](int dst, int src, int id) {
          const unsigned to = lds_base + (unsigned)(ch.stage(dst) + wp * 1024);
          if constexpr (FP8) {
            // instruction j = wp + 4i; the last one (j = 19) brings the scales
            const char* base = cache_bytes + (long)id * (BLOCK * ROW) + (src & 1) * (TT * ROW);
            const char* sbase = reinterpret_cast<const char*>(
                kv_scale + ((long)id * BLOCK + (src & 1) * TT) * 2);
#pragma unroll
            for (int i = 0; i < NDMA_W; ++i)
              dma_one(to + i * 4096, wp + 4 * i >= NROWI8 ? sbase : base, lane_src[i]);
          } else {
            const char* base = cache_bytes + (long)id * (BLOCK * ROW * 2) + (src & 1) * (TT * ROW * 2);
#pragma unroll
            for (int i = 0; i < NDMA; ++i) dma_one(to + i * 4096, base, lane_src[i]);
          }
        };
        // rows outside [lo, hi) of tile a hold other keys or undefined data;
        // P = 0 there, so zero them (0 * NaN would not vanish).  The score
        // waves may read these rows meanwhile: they mask them whatever they hold.
        auto zero_rows = [&](int a) {
          const int lo = ch.lo(a), hi = max(ch.hi(a), lo);
          const int nz = TT - (hi - lo);
          char* st = smem + ch.stage(a);
          if constexpr (FP8) {
            // codes 0 and unit scales (a zero scale would make the
            // normaliser's 0 / s undefined)
            for (int e = threadIdx.x - 256; e < nz * 36; e += 256) {
              const int z = e / 36, f = e % 36;
              const int r = z < lo ? z : hi + (z - lo);
              *reinterpret_cast<uint4*>(st + r * RS8 + f * 16) = uint4{0, 0, 0, 0};
              if (f == 0) *reinterpret_cast<float2*>(st + SCALE_OFF8 + r * 8) = float2{1.0f, 1.0f};
            }
          } else {
            for (int e = threadIdx.x - 256; e < nz * 72; e += 256) {
              const int z = e / 72, f = e % 72;
              const int r = z < lo ? z : hi + (z - lo);
              *reinterpret_cast<uint4*>(st + (r * RSLOTS + f) * 16) = uint4{0, 0, 0, 0};
            }
          }
        };

        auto load_id = [&](int a) { return uniform(max(ch.id(a), 0)); };
        issue(c0, c0, load_id(c0));
        issue(c0 + 1, c0 + 1 < c1 ? c0 + 1 : c0, load_id(c0 + 1 < c1 ? c0 + 1 : c0));
        issue(c0 + 2, c0 + 2 < c1 ? c0 + 2 : c0, load_id(c0 + 2 < c1 ? c0 + 2 : c0));
        vm_wait<2 * NDMA_W>();
        lds_sync();  // tile c0 has landed
        if (ch.partial(c0)) zero_rows(c0);
        lds_sync();  // the score waves' softmax of tile c0 follows
        for (int a = c0; a < c1; ++a) {
          // tile a+1 landed: its loads were issued two iterations ago; those of
          // the last iteration (tile a+2) may stay in flight
          vm_wait<NDMA_W>();
          lds_sync();  // barrier A(a)
          const int par = ch.par(a);
          // Every LDS read of the iteration is issued at once: the flags, the
          // block ids of tiles a+1 and a+3, P(a) and V(a).  P(a) changes only
          // in a redo, which reads it again.  Then PV of dims 16db.. for
          // db < PV_A, then the loads of tile a+3 (LDS reads this wave issues
          // after a direct-to-LDS load queue behind it), then the rest of PV.
          const int4 fl = *reinterpret_cast<const int4*>(flags + par * 4);
          const int src = a + 3 < c1 ? a + 3 : a;
          const int id_src = ch.id(src);
          const char* pb = smem + OFF_P + par * PBUF;
          i16x8_t pf[4];
#pragma unroll
          for (int hb = 0; hb < 4; ++hb) pf[hb] = lds_b128(pb + (hb * 64 + lane) * 16);
          i16x8_t pw = lds_b128(pb + (wp * 64 + lane) * 16);
          const char* vp = smem + ch.stage(a);
          i16x8_t vf[8];
          v2i_t vraw[8];   // FP8: codes, widened next to their MFMAs
          if constexpr (FP8) {
#pragma unroll
            for (int db = 0; db < 8; ++db)
              vraw[db] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i_t*)(vp + v8 + 16 * db));
          } else {
#pragma unroll
            for (int db = 0; db < 8; ++db) {
              const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                  (lds_i16x4_t*)(vp + v_lo + ((2 * db + b_v) ^ s_lo) * 16));
              const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                  (lds_i16x4_t*)(vp + v_hi + ((2 * db + b_v) ^ s_hi) * 16));
              vf[db] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            }
          }
          // (the block id matters only in a chunk with a missing block; reading
          // it otherwise would make this test wait for all of the reads above)
          bool zero_next = a + 1 < c1 && (ch.lo(a + 1) > 0 || ke - (a + 1) * TT < TT);
          if (missing && a + 1 < c1) zero_next = zero_next || uniform(ch.id(a + 1)) < 0;
          if (zero_next) zero_rows(a + 1);
          if (uniform(fl.x | fl.y | fl.z | fl.w) != 0) {
            lds_sync();  // the score waves have rewritten P(a) and the factors
            asm volatile("s_nop 7");  // last PV MFMA results written back
#pragma unroll
            for (int hb = 0; hb < 4; ++hb) {
              const float f = fbuf[hb * 16 + r16];
#pragma unroll
              for (int db = 0; db < 8; ++db) scale_agpr(acc[hb][db], f);
            }
            rsum *= fbuf[wp * 16 + r16];
            asm volatile("s_nop 7");  // VALU-written accumulators, then MFMA reads
#pragma unroll
            for (int hb = 0; hb < 4; ++hb) pf[hb] = lds_b128(pb + (hb * 64 + lane) * 16);
            pw = lds_b128(pb + (wp * 64 + lane) * 16);
          }
          const int nid = uniform(max(id_src, 0));
#pragma unroll
          for (int db = 0; db < PV_A; ++db) {
            const i16x8_t v = FP8 ? widen8(vraw[db]) : vf[db];
#pragma unroll
            for (int hb = 0; hb < 4; ++hb) mma_pv(acc[hb][db], v, pf[hb]);
          }
          issue(a + 3, src, nid);
#pragma unroll
          for (int db = PV_A; db < 8; ++db) {
            const i16x8_t v = FP8 ? widen8(vraw[db]) : vf[db];
#pragma unroll
            for (int hb = 0; hb < 4; ++hb) mma_pv(acc[hb][db], v, pf[hb]);
          }
          if constexpr (!FP8) mma_sum(rsum, ones, pw);   // FP8: the score waves keep the normaliser
        }
        vm_wait<0>();  // the loads past the chunk land before its stages are reused
        c0 = c1;
      }

      // ---- epilogue: normalise, write o -----------------------------------
      asm volatile("s_nop 15\n\ts_nop 15");  // last PV MFMA results written back
      __syncthreads();  // every wave is done with the P buffers
      if (g == 0) l_all[wp * 16 + r16] = rsum[0];
      __syncthreads();  // denominators and maxima visible
      float* obase = (wi.part ? o_part : o_lat) + (wi.orow * n_h + hbase) * D_C;
#pragma unroll
      for (int hb = 0; hb < 4; ++hb) {
        const int h = hb * 16 + r16;
        const float l = FP8 ? l_part[h] + l_part[HG + h] : l_all[h];
        const float inv = l > 0.0f ? 1.0f / l : 0.0f;
#pragma unroll
        for (int db = 0; db < 8; ++db)
          *reinterpret_cast<float4*>(obase + (long)h * D_C + d0 + db * 16 + 4 * g) =
              float4{acc[hb][db][0] * inv, acc[hb][db][1] * inv, acc[hb][db][2] * inv,
                     acc[hb][db][3] * inv};
      }
    }
  }
}

}  // namespace

hipError_t launch_decode_h64(const void* q_lat, const void* cache, int num_blocks,
                             const int* table, int max_blocks, const int* seq_lens, int B,
                             int q_len, int n_h, float scale, int S, const int* work, int n_work,
                             const int* lists, int n_lists, float* o_lat, float* lse,
                             float* o_part, float* lse_part, int n_parts, hipStream_t stream) {
  const long n_items = work != nullptr ? (long)n_work : (long)B * q_len * S;
  const long n_units = lists != nullptr ? (long)n_lists : n_items;
  const int ngroups = n_h / HG;
  const long wgs = (n_units + 7) / 8 * 8 * ngroups;
  if (wgs == 0 || n_items == 0) return hipSuccess;
  hipLaunchKernelGGL(decode_h64_kernel<false>, dim3((unsigned)wgs), dim3(NTHREADS), 0, stream,
                     (const uint16_t*)q_lat, cache, nullptr, num_blocks, table,
                     max_blocks, seq_lens, q_len, n_h, (int)n_items, B * q_len, n_parts, scale * LOG2E, S,
                     (const int4*)work, lists, n_lists, o_lat, lse, o_part, lse_part);
  return hipGetLastError();
}

hipError_t launch_decode_h64_fp8(const void* q_lat, const void* cache, const float* kv_scale,
                                 int num_blocks, const int* table, int max_blocks,
                                 const int* seq_lens, int B, int q_len, int n_h, float scale, int S,
                                 const int* work, int n_work, const int* lists, int n_lists,
                                 float* o_lat, float* lse, float* o_part, float* lse_part,
                                 int n_parts, hipStream_t stream) {
  const long n_items = work != nullptr ? (long)n_work : (long)B * q_len * S;
  const long n_units = lists != nullptr ? (long)n_lists : n_items;
  const int ngroups = n_h / HG;
  const long wgs = (n_units + 7) / 8 * 8 * ngroups;
  if (wgs == 0 || n_items == 0) return hipSuccess;
  hipLaunchKernelGGL(decode_h64_kernel<true>, dim3((unsigned)wgs), dim3(NTHREADS), 0, stream,
                     (const uint16_t*)q_lat, cache, kv_scale, num_blocks, table, max_blocks,
                     seq_lens, q_len, n_h, (int)n_items, B * q_len, n_parts, scale * LOG2E, S,
                     (const int4*)work, lists, n_lists, o_lat, lse, o_part, lse_part);
  return hipGetLastError();
}

}  // namespace mla
