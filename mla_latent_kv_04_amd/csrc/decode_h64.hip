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
// ids of the current item.  (The FP8 cache has a kernel of the same design
// with 64-token tiles, decode_h64_fp8.hip; the helpers both use are in
// decode_h64_common.h.)
#include "mla_common.h"
#include "attention_launch.h"
#include "mla_internal.h"
#include "decode_h64_common.h"

namespace mla {

namespace {

constexpr int TT = 32;                       // tokens per tile (half a paged block)
constexpr int NSTAGE = 4;                    // tile stages in LDS
constexpr int RSLOTS = ROW * 2 / 16;         // 72 16-byte chunks per token row
constexpr int NINST = TT * RSLOTS / 64;      // 36 direct-to-LDS instructions per tile
constexpr int STAGE = NINST * 1024;          // 36,864 bytes
constexpr int NDMA = NINST / 4;              // 9 per value wave
#ifndef PV_PHASE_A
#define PV_PHASE_A 4
#endif
constexpr int PV_A = PV_PHASE_A;             // PV dim blocks (of 8) run before the loads of tile a+3

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
// The loads are the common dma_one; nothing else in the tile loop of a value
// wave issues vector-memory instructions, so the counts given to vm_wait are
// exact.

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

// One chunk of an item: tiles [c0, c1) (tile a = tokens [32a, 32a + 32) of the
// sequence, block a / 2, half a % 2), keys [kb, ke), block ids staged in ids[].
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
    return OFF_STAGE + ((a - c0) & (NSTAGE - 1)) * STAGE;
  }
  __device__ int par(int a) const { return (a - c0) & 1; }
};

__global__ void __launch_bounds__(NTHREADS, 1) decode_h64_kernel(
    const uint16_t* __restrict__ q_lat, const void* __restrict__ cache, int num_blocks,
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

  int hgrp, i_begin, i_end;
  if (!h64_unit(n_h, n_items, lists, n_lists, hgrp, i_begin, i_end)) return;

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
    constexpr int KPF = 3;  // K fragments are read KPF steps ahead

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

      const int t_first = kb / TT;
      const int t_last = kb < ke ? (ke + TT - 1) / TT : t_first;
      for (int c0 = t_first; c0 < t_last;) {
        const int c1 = min(t_last, (c0 & ~1) + 2 * IDCAP);
        const int blk0 = c0 >> 1;
        stage_ids(ids, trow, blk0, ((c1 - 1) >> 1) - blk0 + 1, num_blocks);
        const Chunk ch{ids, c0, c1, blk0, kb, ke};

        // scores and maxima of the tile waiting for its PV (kept for a redo)
        f32x4_t sc_keep[2];
        float ml_keep[2];

        // P of this wave's heads and tokens: 4 bf16 per lane and head block,
        // bytes th*8 .. th*8+7 of the lane's 16 bytes of the PV B fragment of
        // head block 2hq + hb (k slots 4th .. 4th+3 of the lane's group:
        // tokens 16th + 4g + i)
        auto write_p = [&](int a, const f32x4_t (&sc)[2]) {
          char* pb = smem + OFF_P + ch.par(a) * PBUF;
#pragma unroll
          for (int hb = 0; hb < 2; ++hb) {
            uint2 w;
            w.x = pack_bf16x2(fast_exp2(sc[hb][0] - mref[hb]), fast_exp2(sc[hb][1] - mref[hb]));
            w.y = pack_bf16x2(fast_exp2(sc[hb][2] - mref[hb]), fast_exp2(sc[hb][3] - mref[hb]));
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
          write_p(a, sc);
          flags[par * 4 + wave] = __builtin_amdgcn_ballot_w64(need) != 0 ? 1 : 0;
          sc_keep[0] = sc[0];
          sc_keep[1] = sc[1];
        };

        lds_sync();  // tile c0 has landed
        {
          f32x4_t sc[2];
          i16x8_t kbuf[KPF + 1];
          k_first(c0, kbuf);
          qk(c0, ch.hi(c0), kbuf, sc, [] {});
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
              }
              write_p(a, sc_keep);
              lds_sync();  // redone P and the factors are visible to the value waves
            }
          };
          // tile a+1 (past the chunk: fully masked; written but never read)
          f32x4_t sc[2];
          i16x8_t kbuf[KPF + 1];
          k_first(a + 1, kbuf);
          qk(a + 1, hi_n, kbuf, sc, redo);
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
      __syncthreads();  // denominators and maxima visible
      if (wave == 0) {
        const int h = lane;
        const float l = l_all[h];
        float* lbase = (wi.part ? lse_part : lse) + wi.orow * n_h + hbase;
        lbase[h] = l > 0.0f ? (mx_all[h] + __log2f(l)) * LN2 : -INFINITY;
      }
    }
  } else {
    // =========================== value waves ===========================
    const int wp = wave - 4;
    const int d0 = wp * 128;                   // first output dim of this wave
    unsigned lane_src[NDMA];
#pragma unroll
    for (int i = 0; i < NDMA; ++i) lane_src[i] = dma_src(wp + 4 * i, lane);
    // V^T fragment of dims d0 + 16db ..: token t = 4g + (r16 >> 2) (and t + 16),
    // dims d0 + 16db + 4 (r16 & 3) .. +3, i.e. chunk d0 / 8 + 2db + b of the
    // row, bytes h8 .. h8 + 7 of it
    const int t_v = 4 * g + (r16 >> 2), b_v = (r16 & 3) >> 1, h8 = (r16 & 1) * 8;
    const int v_lo = t_v * RSLOTS * 16 + d0 * 2 + h8, v_hi = v_lo + 16 * RSLOTS * 16;
    const int s_lo = swz(t_v), s_hi = swz(t_v + 16);
    const i16x8_t ones = lds_b128(smem + OFF_ONES);

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
        const Chunk ch{ids, c0, c1, blk0, kb, ke};

        // loads of tile `src` into the stage of tile `dst` (src == dst except
        // past the chunk, where a valid tile is loaded into a stage nobody
        // reads, so that every tile slot issues the same number of loads and
        // the vmcnt waits stay exact).  id is src's block (load_id: a missing
        // block is read from block 0 instead; its rows are zeroed and masked).
        auto issue = [&](int dst, int src, int id) {
          const unsigned to = lds_base + (unsigned)(ch.stage(dst) + wp * 1024);
          const char* base = cache_bytes + (long)id * (BLOCK * ROW * 2) + (src & 1) * (TT * ROW * 2);
#pragma unroll
          for (int i = 0; i < NDMA; ++i) dma_one(to + i * 4096, base, lane_src[i]);
        };
        // rows outside [lo, hi) of tile a hold other keys or undefined data;
        // P = 0 there, so zero them (0 * NaN would not vanish).  The score
        // waves may read these rows meanwhile: they mask them whatever they hold.
        auto zero_rows = [&](int a) {
          const int lo = ch.lo(a), hi = max(ch.hi(a), lo);
          const int nz = TT - (hi - lo);
          char* st = smem + ch.stage(a);
          for (int e = threadIdx.x - 256; e < nz * 72; e += 256) {
            const int z = e / 72, f = e % 72;
            const int r = z < lo ? z : hi + (z - lo);
            *reinterpret_cast<uint4*>(st + (r * RSLOTS + f) * 16) = uint4{0, 0, 0, 0};
          }
        };

        auto load_id = [&](int a) { return uniform(max(ch.id(a), 0)); };
        issue(c0, c0, load_id(c0));
        issue(c0 + 1, c0 + 1 < c1 ? c0 + 1 : c0, load_id(c0 + 1 < c1 ? c0 + 1 : c0));
        issue(c0 + 2, c0 + 2 < c1 ? c0 + 2 : c0, load_id(c0 + 2 < c1 ? c0 + 2 : c0));
        vm_wait<2 * NDMA>();
        lds_sync();  // tile c0 has landed
        if (ch.partial(c0)) zero_rows(c0);
        lds_sync();  // the score waves' softmax of tile c0 follows
        for (int a = c0; a < c1; ++a) {
          // tile a+1 landed: its loads were issued two iterations ago; those of
          // the last iteration (tile a+2) may stay in flight
          vm_wait<NDMA>();
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
#pragma unroll
          for (int db = 0; db < 8; ++db) {
            const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_i16x4_t*)(vp + v_lo + ((2 * db + b_v) ^ s_lo) * 16));
            const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_i16x4_t*)(vp + v_hi + ((2 * db + b_v) ^ s_hi) * 16));
            vf[db] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
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
#pragma unroll
            for (int hb = 0; hb < 4; ++hb) mma_pv(acc[hb][db], vf[db], pf[hb]);
          }
          issue(a + 3, src, nid);
#pragma unroll
          for (int db = PV_A; db < 8; ++db) {
#pragma unroll
            for (int hb = 0; hb < 4; ++hb) mma_pv(acc[hb][db], vf[db], pf[hb]);
          }
          mma_sum(rsum, ones, pw);
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
        const float l = l_all[h];
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
  return launch_attention(decode_h64_kernel, dim3((unsigned)wgs), dim3(NTHREADS), stream,
                          (const uint16_t*)q_lat, cache, num_blocks, table, max_blocks, seq_lens,
                          q_len, n_h, (int)n_items, B * q_len, n_parts, scale * LOG2E, S,
                          (const int4*)work, lists, n_lists, o_lat, lse, o_part, lse_part);
}

}  // namespace mla
