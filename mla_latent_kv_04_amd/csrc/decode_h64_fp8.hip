// Paged latent attention over the FP8 E4M3 cache, for head counts that are
// multiples of 64 (DeepSeek-V2 uses 128 heads).
//
// The cache keeps each row as 576 E4M3 codes with two float32 scales, one for
// the 512 latent values and one for the 64 rotated RoPE values; a value is its
// code times its part's scale (the quantised cache of the DeepSeek-V2 MLA
// blog, adg.csdn.net, part 3 §3.1.4).  Attention is eq. 7 of the DeepSeek-V2
// notes (irregular6612.github.io, §2.1.1) over those values with the absorbed
// query, as in decode_h64.hip, whose two-role design this kernel keeps:
//
//   score waves 0..3, (hq, th) = (w & 1, w >> 1): scores of heads
//     32hq..32hq+31 against tokens 32th..32th+31 of a tile (two 16-token
//     blocks), the query (144 registers) in AGPRs.  The K codes are widened to
//     bf16 in registers one k-step ahead of their MFMAs; the latent and RoPE
//     parts of a score run in separate chains, each multiplied by its token's
//     scale.  Then the softmax step: P against the running max of the head
//     group, and the normaliser, kept here: a token's weight in P is rounded to
//     bf16 together with its latent scale (the value operand holds bare codes),
//     and the normaliser adds that rounded weight divided by the scale.
//   value waves 4..7, wp = w - 4: output dims 128wp..128wp+127 for all 64
//     heads (128 accumulators in AGPRs); V^T fragments of codes by 8-bit
//     transposing LDS reads, widened next to their MFMAs.  These waves also
//     issue the direct-to-LDS tile loads.
//
// A tile is one paged block, 64 tokens: 64 rows of 576 code bytes (592-byte
// LDS rows) and the block's 64 scale pairs come to 38 load instructions, padded
// to 40 (10 per value wave), 40 KB, about the size of a 32-token bf16 tile.
// Twice the tokens of decode_h64's tiles per workgroup barrier is the point:
// that kernel is held by its per-tile synchronisation, not by HBM.  Three
// stages fit (tile a under PV, tile a+1 under QK, tile a+2 loading), with
// the P buffers (both PV k-steps of a tile) and the tile maxima alternating by
// tile parity.  Iteration a:
//
//   barrier A(a): tile a+1 has landed; P(a), its maxima and flags are in LDS;
//                 tile a-1 is no longer read by anyone
//   value waves: loads of tile a+2 into the stage of tile a-1, then P(a) and
//                V(a) into registers and PV over the tile's two k-steps
//   score waves: QK^T of tile a+1 (72 MFMAs per wave), its softmax step into
//                the other P buffer
//   [redo a] as in decode_h64.hip: when a score of tile a beat the running
//            max by more than 2^8 (log2), the new max is agreed, P(a) and the
//            normaliser redone and the accumulators rescaled (one more barrier).
#include "mla_common.h"
#include "attention_launch.h"
#include "mla_internal.h"
#include "decode_h64_common.h"

namespace mla {

namespace {

constexpr int TT8 = BLOCK;                        // tokens per tile: one paged block
constexpr int NSTAGE8 = 3;                        // tile stages in LDS
constexpr int RSLOTS8 = ROW / 16 + 1;             // 37 16-byte slots per row (36 + pad)
constexpr int RS8 = RSLOTS8 * 16;                 // 592-byte LDS row pitch
constexpr int NROWI8 = TT8 * RSLOTS8 / 64;        // 37 row instructions
constexpr int SCALE_OFF8 = NROWI8 * 1024;         // the tile's 64 scale pairs (512 bytes)
constexpr int NINST8 = 40;                        // 37 + the scales + 2 spare
constexpr int STAGE8 = NINST8 * 1024;             // 40,960 bytes
constexpr int NDMA8 = NINST8 / 4;                 // 10 per value wave
static_assert(TT8 * RSLOTS8 % 64 == 0 && NROWI8 + 1 <= NINST8 && NINST8 % 4 == 0,
              "a tile is whole load instructions, the same number per value wave");
static_assert(TT8 * 8 == 32 * 16, "the scale pairs fill 32 lanes of one load");

// LDS map (bytes)
constexpr int PBUF8 = 2 * 4 * 64 * 16;               // P of a tile: [2 k-steps][4 head blocks][64 lanes][16 B]
constexpr int OFF_P8 = NSTAGE8 * STAGE8;             // [2] P buffers
constexpr int OFF_MAX8 = OFF_P8 + 2 * PBUF8;         // float [2][2 token halves][64]
constexpr int OFF_F8 = OFF_MAX8 + 2 * 2 * HG * 4;    // float [64] rescale factors
constexpr int OFF_FLAG8 = OFF_F8 + HG * 4;           // int [2][4] per score wave "my scores move the max"
constexpr int OFF_IDS8 = OFF_FLAG8 + 2 * 4 * 4;      // int [IDCAP]
constexpr int SMEM8 = OFF_IDS8 + IDCAP * 4;
static_assert(SMEM8 <= 163840, "LDS budget");

// Byte offset, from the block's first code row (or, for instructions past the
// rows, from its first scale pair), of the 16 bytes that lane l of load
// instruction j moves.  Instruction j fills stage slots 64j .. 64j + 63; slot s
// is slot s % 37 of row s / 37 (the pad slot re-reads slot 0 and is never
// used).  The scale instruction's lanes 32..63, and the two spare
// instructions, re-read the scale pairs into bytes nobody reads.
__device__ __forceinline__ unsigned dma_src_t64(int j, int lane) {
  if (j >= NROWI8) return (unsigned)((lane & 31) * 16);
  const int slot = 64 * j + lane;
  const int t = slot / RSLOTS8;
  int p = slot - t * RSLOTS8;
  if (p == RSLOTS8 - 1) p = 0;
  return (unsigned)(t * ROW + p * 16);
}

// One chunk of an item: tiles [c0, c1) (tile a = block a of the sequence,
// tokens [64a, 64a + 64)), keys [kb, ke), block ids of blocks c0.. in ids[].
struct Chunk64 {
  const int* ids;
  int c0, c1, kb, ke;
  // block id of tile a (tiles past the chunk, which the pipeline touches but
  // never uses, read the chunk's first id)
  __device__ int id(int a) const { return ids[a < c1 ? a - c0 : 0]; }
  // valid rows [lo, hi) of tile a (none past the chunk or for a missing block)
  __device__ int lo(int a) const { return max(0, kb - a * TT8); }
  __device__ int hi(int a) const { return hi_of(a, id(a)); }
  __device__ int hi_of(int a, int id_a) const {
    return (a >= c1 || id_a < 0) ? 0 : min(TT8, ke - a * TT8);
  }
  __device__ bool partial(int a) const { return lo(a) > 0 || hi(a) < TT8; }
  __device__ int stage(int a) const { return ((a - c0) % NSTAGE8) * STAGE8; }
  __device__ int par(int a) const { return (a - c0) & 1; }
};

__global__ void __launch_bounds__(NTHREADS, 1) decode_h64_fp8_kernel(
    const uint16_t* __restrict__ q_lat, const uint8_t* __restrict__ codes,
    const float* __restrict__ kv_scale, int num_blocks, const int* __restrict__ table,
    int max_blocks, const int* __restrict__ seq_lens, int q_len, int n_h, int n_items,
    int n_rows, int n_parts, float scale_log2, int S, const int4* __restrict__ work,
    const int* __restrict__ lists, int n_lists, float* __restrict__ o_lat,
    float* __restrict__ lse, float* __restrict__ o_part, float* __restrict__ lse_part) {
  __shared__ __attribute__((aligned(16))) char smem[SMEM8];
  float* const maxbuf = reinterpret_cast<float*>(smem + OFF_MAX8);
  float* const fbuf = reinterpret_cast<float*>(smem + OFF_F8);
  int* const flags = reinterpret_cast<int*>(smem + OFF_FLAG8);
  int* const ids = reinterpret_cast<int*>(smem + OFF_IDS8);
  float* const mx_all = reinterpret_cast<float*>(smem + OFF_P8);   // epilogue: [64] running maxima
  float* const l_part = mx_all + HG;   // epilogue: [2 token halves][64] normaliser parts

  int hgrp, i_begin, i_end;
  if (!h64_unit(n_h, n_items, lists, n_lists, hgrp, i_begin, i_end)) return;

  const int lane = lane_id(), g = lane >> 4, r16 = lane & 15;
  // the wave index is uniform; saying so keeps the role branch and the DMA
  // addresses scalar
  const int wave = uniform((int)(threadIdx.x >> 6));
  const int hbase = hgrp * HG;                 // first head of the workgroup
  const char* const cache_bytes = reinterpret_cast<const char*>(codes);
  const unsigned lds_base = (unsigned)(uintptr_t)(__attribute__((address_space(3))) char*)smem;

  // Both roles walk the same items, chunks and tiles and take the same
  // (workgroup-uniform) redo decisions, so they meet at every barrier.
  if (wave < 4) {
    // =========================== score waves ===========================
    const int hq = wave & 1, th = wave >> 1;
    // K codes of token block tb, k-step ks: 8 bytes of token 32th + 16tb + r16
    // at byte 32 ks + 8 g of its row
    const int k8 = (32 * th + r16) * RS8 + 8 * g;
    constexpr int KPF = 3;  // K fragments are read KPF steps ahead
    // the scale pairs of this lane's score rows 32th + 16tb + 4g + i of the
    // tile waiting for its PV (for a redo), and the running normaliser of
    // this lane's rows (l_run: tiles done; l_pend: the waiting tile, added once
    // its redo check has passed)
    float s_lat_keep[2][4];
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
      l_run[0] = l_run[1] = 0.0f;
      l_pend[0] = l_pend[1] = 0.0f;

      const int t_first = kb / TT8;
      const int t_last = kb < ke ? (ke + TT8 - 1) / TT8 : t_first;
      for (int c0 = t_first; c0 < t_last;) {
        const int c1 = min(t_last, c0 + IDCAP);
        stage_ids(ids, trow, c0, c1 - c0, num_blocks);
        const Chunk64 ch{ids, c0, c1, kb, ke};

        // scores and maxima of the tile waiting for its PV (kept for a redo)
        f32x4_t sc_keep[2][2];
        float ml_keep[2];

        // P of this wave's heads and tokens: the whole 16-byte B fragment of
        // PV k-step th for head block 2hq + hb, slots 0..3 from token block 0
        // (tokens 32th + 4g + i) and 4..7 from block 1 (32th + 16 + 4g + i).
        // A token's weight carries its latent scale (rounded to bf16 with
        // it); l_pend gets the same weights over the scale.
        auto write_p = [&](int a, const f32x4_t (&sc)[2][2], const float (&sl)[2][4]) {
          char* pb = smem + OFF_P8 + ch.par(a) * PBUF8;
#pragma unroll
          for (int hb = 0; hb < 2; ++hb) {
            float p[2][4];
            l_pend[hb] = 0.0f;
#pragma unroll
            for (int tb = 0; tb < 2; ++tb)
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                // a masked row (score -inf) weighs exactly 0 whatever its scale
                // holds: the value waves zero such rows concurrently, so the
                // scale read here may be the stale bytes of another key
                const bool live = sc[tb][hb][i] != -INFINITY;
                p[tb][i] = live ? BF16::round(fast_exp2(sc[tb][hb][i] - mref[hb]) * sl[tb][i]) : 0.0f;
                l_pend[hb] += live ? p[tb][i] * __builtin_amdgcn_rcpf(sl[tb][i]) : 0.0f;
              }
            *reinterpret_cast<uint4*>(pb + ((th * 4 + hq * 2 + hb) * 64 + lane) * 16) =
                uint4{pack_bf16x2(p[0][0], p[0][1]), pack_bf16x2(p[0][2], p[0][3]),
                      pack_bf16x2(p[1][0], p[1][1]), pack_bf16x2(p[1][2], p[1][3])};
          }
        };

        auto k_first = [&](int a, int tb, v2i_t (&kbuf)[KPF + 1]) {
          const char* kp = smem + ch.stage(a) + k8 + tb * 16 * RS8;
#pragma unroll
          for (int ks = 0; ks < KPF; ++ks) kbuf[ks] = *reinterpret_cast<const v2i_t*>(kp + 32 * ks);
        };
        // QK^T of token block tb of tile a: latent and RoPE parts in separate
        // chains (two for the latent part, by k-step parity, so that no MFMA
        // waits for the one just before it), each multiplied by its token's
        // scale; the codes are widened one k-step ahead.  mid() runs after
        // k-step QK_MID - 1 (the redo check: the scores of the next tile do not
        // depend on it, so the MFMAs start first).
        auto qk = [&](int a, int hi, int tb, v2i_t (&kbuf)[KPF + 1], f32x4_t (&sc)[2],
                      float (&sl)[4], auto&& mid) {
          const char* kp = smem + ch.stage(a);
          const int rbase = 32 * th + 16 * tb;   // first row of the token block
          float2 sp[4];
#pragma unroll
          for (int i = 0; i < 4; ++i)
            sp[i] = *reinterpret_cast<const float2*>(kp + SCALE_OFF8 + (rbase + 4 * g + i) * 8);
          const char* kr = kp + k8 + tb * 16 * RS8;
          f32x4_t q4[2][2], qr[2];
          i16x8_t kf = widen8(kbuf[0]);
#pragma unroll
          for (int ks = 0; ks < KSTEPS; ++ks) {
            if (ks == QK_MID) mid();
            if (ks + KPF < KSTEPS)
              kbuf[(ks + KPF) % (KPF + 1)] = *reinterpret_cast<const v2i_t*>(kr + 32 * (ks + KPF));
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
          for (int i = 0; i < 4; ++i) sl[i] = sp[i].x;
#pragma unroll
          for (int hb = 0; hb < 2; ++hb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              sc[hb][i] = (sp[i].x * (q4[hb][0][i] + q4[hb][1][i]) + sp[i].y * qr[hb][i]) * scale_log2;
          const int lo = ch.lo(a);
          if (lo > 0 || hi < TT8) {  // rare: rows outside [lo, hi) get no weight
#pragma unroll
            for (int hb = 0; hb < 2; ++hb)
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int row = rbase + 4 * g + i;
                if (row < lo || row >= hi) sc[hb][i] = -INFINITY;
              }
          }
        };
        // both token blocks of tile a; mid() inside the first
        auto qk_tile = [&](int a, int hi, f32x4_t (&sc)[2][2], float (&sl)[2][4], auto&& mid) {
          v2i_t kbuf[KPF + 1];
          k_first(a, 0, kbuf);
          qk(a, hi, 0, kbuf, sc[0], sl[0], mid);
          k_first(a, 1, kbuf);
          qk(a, hi, 1, kbuf, sc[1], sl[1], [] {});
        };
        // P against the running max both waves of a head group share.  A wave
        // whose scores would move that max raises its flag (its P, written
        // anyway, is then replaced in a redo).  Every lane of a group writes
        // the same maximum and every lane the same flag: no branches.
        auto softmax = [&](int a, const f32x4_t (&sc)[2][2], const float (&sl)[2][4]) {
          const int par = ch.par(a);
          bool need = false;
#pragma unroll
          for (int hb = 0; hb < 2; ++hb) {
            float mx = -INFINITY;
#pragma unroll
            for (int tb = 0; tb < 2; ++tb)
              mx = fmaxf(mx, fmaxf(fmaxf(sc[tb][hb][0], sc[tb][hb][1]),
                                   fmaxf(sc[tb][hb][2], sc[tb][hb][3])));
            ml_keep[hb] = group4_max(mx);
            need |= ml_keep[hb] > mref[hb] + RESCALE_LOG2;
            maxbuf[(par * 2 + th) * HG + hq * 32 + hb * 16 + r16] = ml_keep[hb];
          }
          write_p(a, sc, sl);
          flags[par * 4 + wave] = __builtin_amdgcn_ballot_w64(need) != 0 ? 1 : 0;
#pragma unroll
          for (int tb = 0; tb < 2; ++tb) {
            sc_keep[tb][0] = sc[tb][0];
            sc_keep[tb][1] = sc[tb][1];
#pragma unroll
            for (int i = 0; i < 4; ++i) s_lat_keep[tb][i] = sl[tb][i];
          }
        };

        lds_sync();  // tile c0 has landed
        {
          f32x4_t sc[2][2];
          float sl[2][4];
          qk_tile(c0, ch.hi(c0), sc, sl, [] {});
          lds_sync();
          softmax(c0, sc, sl);
        }
        for (int a = c0; a < c1; ++a) {
          lds_sync();  // barrier A(a)
          const int par = ch.par(a);
          const int4 fl = *reinterpret_cast<const int4*>(flags + par * 4);
          const int hi_n = ch.hi(a + 1);
          auto redo = [&] {
            if (uniform(fl.x | fl.y | fl.z | fl.w) != 0) {
              // rare: agree on the new running max from both token halves,
              // record the rescale factors, rewrite P(a) and its normaliser
#pragma unroll
              for (int hb = 0; hb < 2; ++hb) {
                const float mx =
                    fmaxf(ml_keep[hb], maxbuf[(par * 2 + (th ^ 1)) * HG + hq * 32 + hb * 16 + r16]);
                const float mnew = mx > mref[hb] + RESCALE_LOG2 ? mx : mref[hb];
                const float f = fast_exp2(mref[hb] - mnew);
                mref[hb] = mnew;
                if (th == 0 && g == 0) fbuf[hq * 32 + hb * 16 + r16] = f;
                l_run[hb] *= f;
              }
              write_p(a, sc_keep, s_lat_keep);
              lds_sync();  // redone P and the factors are visible to the value waves
            }
            // tile a's weights are final: into the normaliser
            l_run[0] += l_pend[0];
            l_run[1] += l_pend[1];
          };
          // tile a+1 (past the chunk: fully masked; written but never read)
          f32x4_t sc[2][2];
          float sl[2][4];
          qk_tile(a + 1, hi_n, sc, sl, redo);
          softmax(a + 1, sc, sl);
        }
        c0 = c1;
      }

      // ---- epilogue: running maxima and normalisers for the log-sum-exp ---
      __syncthreads();  // every wave is done with the P buffers
      if (th == 0 && g == 0) {
        mx_all[hq * 32 + r16] = mref[0];
        mx_all[hq * 32 + 16 + r16] = mref[1];
      }
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        const float l = group4_sum(l_run[hb]);
        if (g == 0) l_part[th * HG + hq * 32 + hb * 16 + r16] = l;
      }
      __syncthreads();  // normalisers and maxima visible
      if (wave == 0) {
        const int h = lane;
        const float l = l_part[h] + l_part[HG + h];
        float* lbase = (wi.part ? lse_part : lse) + wi.orow * n_h + hbase;
        lbase[h] = l > 0.0f ? (mx_all[h] + __log2f(l)) * LN2 : -INFINITY;
      }
    }
  } else {
    // =========================== value waves ===========================
    const int wp = wave - 4;
    const int d0 = wp * 128;                   // first output dim of this wave
    unsigned lane_src[NDMA8];
#pragma unroll
    for (int i = 0; i < NDMA8; ++i) lane_src[i] = dma_src_t64(wp + 4 * i, lane);
    // V^T fragment of k-step kk, dims d0 + 16db ..: the 8-bit transposing
    // read; lane j of each 16-lane group names row 32kk + T(j / 2) of its
    // group, T(k) = 16 (k / 4) + 4 g + k % 4 (the tokens of P slot k), and the
    // 8 bytes at column d0 + 16 db + 8 (j % 2)
    const int k_v = r16 >> 1;
    const int v8 = (16 * (k_v >> 2) + 4 * g + (k_v & 3)) * RS8 + d0 + 8 * (r16 & 1);

    for (int item = i_begin; item < i_end; ++item) {
      const WorkItem wi = decode_item(item, work, n_rows, n_parts, q_len, S, seq_lens, max_blocks);
      if (!uniform(wi.valid)) continue;
      const int kb = uniform(wi.kb), ke = uniform(wi.ke);
      const int* const trow = table + (long)wi.b * max_blocks;

      // acc: 4 head blocks x this wave's 8 dim blocks
      f32x4_t acc[4][8];
#pragma unroll
      for (int hb = 0; hb < 4; ++hb)
#pragma unroll
        for (int db = 0; db < 8; ++db) acc[hb][db] = f32x4_t{0, 0, 0, 0};

      const int t_first = kb / TT8;
      const int t_last = kb < ke ? (ke + TT8 - 1) / TT8 : t_first;
      for (int c0 = t_first; c0 < t_last;) {
        const int c1 = min(t_last, c0 + IDCAP);
        const bool missing = stage_ids(ids, trow, c0, c1 - c0, num_blocks);
        const Chunk64 ch{ids, c0, c1, kb, ke};

        // loads of tile `src` into the stage of tile `dst` (src == dst except
        // past the chunk, where a valid tile is loaded into a stage nobody
        // reads, so that every tile slot issues the same number of loads and
        // the vmcnt waits stay exact).  id is src's block (load_id: a missing
        // block is read from block 0 instead; its rows are zeroed and masked).
        auto issue = [&](int dst, int id) {
          const unsigned to = lds_base + (unsigned)(ch.stage(dst) + wp * 1024);
          const char* base = cache_bytes + (long)id * (BLOCK * ROW);
          const char* sbase = reinterpret_cast<const char*>(kv_scale + (long)id * BLOCK * 2);
#pragma unroll
          for (int i = 0; i < NDMA8; ++i)
            dma_one(to + i * 4096, wp + 4 * i >= NROWI8 ? sbase : base, lane_src[i]);
        };
        // rows outside [lo, hi) of tile a hold other keys or undefined data;
        // P = 0 there, so zero them (0 * NaN would not vanish): codes 0 and
        // unit scales (a zero scale would make the normaliser's 0 / s
        // undefined).  The score waves may read these rows meanwhile: they
        // mask them whatever they hold.
        auto zero_rows = [&](int a) {
          const int lo = ch.lo(a), hi = max(ch.hi(a), lo);
          const int nz = TT8 - (hi - lo);
          char* st = smem + ch.stage(a);
          for (int e = threadIdx.x - 256; e < nz * 36; e += 256) {
            const int z = e / 36, f = e % 36;
            const int r = z < lo ? z : hi + (z - lo);
            *reinterpret_cast<uint4*>(st + r * RS8 + f * 16) = uint4{0, 0, 0, 0};
            if (f == 0) *reinterpret_cast<float2*>(st + SCALE_OFF8 + r * 8) = float2{1.0f, 1.0f};
          }
        };

        auto load_id = [&](int a) { return uniform(max(ch.id(a), 0)); };
        issue(c0, load_id(c0));
        issue(c0 + 1, load_id(c0 + 1 < c1 ? c0 + 1 : c0));
        vm_wait<NDMA8>();
        lds_sync();  // tile c0 has landed
        if (ch.partial(c0)) zero_rows(c0);
        lds_sync();  // the score waves' softmax of tile c0 follows
        for (int a = c0; a < c1; ++a) {
          // tile a+1 landed: its loads were issued one iteration ago (or
          // before the loop)
          vm_wait<0>();
          lds_sync();  // barrier A(a)
          const int par = ch.par(a);
          // the loads of tile a+2 go into the stage of tile a-1, which nobody
          // reads any more; then every LDS read of the iteration at once: the
          // flags, P(a) and V(a) of both k-steps.  P(a) changes only in a
          // redo, which reads it again.
          issue(a + 2, load_id(a + 2 < c1 ? a + 2 : a));
          const int4 fl = *reinterpret_cast<const int4*>(flags + par * 4);
          const char* pb = smem + OFF_P8 + par * PBUF8;
          i16x8_t pf[2][4];
#pragma unroll
          for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int hb = 0; hb < 4; ++hb) pf[kk][hb] = lds_b128(pb + ((kk * 4 + hb) * 64 + lane) * 16);
          const char* vp = smem + ch.stage(a) + v8;
          v2i_t vraw[2][8];   // codes, widened next to their MFMAs
#pragma unroll
          for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int db = 0; db < 8; ++db)
              vraw[kk][db] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                  (lds_v2i_t*)(vp + kk * 32 * RS8 + 16 * db));
          // (the block id matters only in a chunk with a missing block; reading
          // it otherwise would make this test wait for all of the reads above)
          bool zero_next = a + 1 < c1 && (ch.lo(a + 1) > 0 || ke - (a + 1) * TT8 < TT8);
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
            asm volatile("s_nop 7");  // VALU-written accumulators, then MFMA reads
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
              for (int hb = 0; hb < 4; ++hb)
                pf[kk][hb] = lds_b128(pb + ((kk * 4 + hb) * 64 + lane) * 16);
          }
#pragma unroll
          for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int db = 0; db < 8; ++db) {
              const i16x8_t v = widen8(vraw[kk][db]);
#pragma unroll
              for (int hb = 0; hb < 4; ++hb) mma_pv(acc[hb][db], v, pf[kk][hb]);
            }
        }
        vm_wait<0>();  // the loads past the chunk land before its stages are reused
        c0 = c1;
      }

      // ---- epilogue: normalise, write o -----------------------------------
      asm volatile("s_nop 15\n\ts_nop 15");  // last PV MFMA results written back
      __syncthreads();  // every wave is done with the P buffers
      __syncthreads();  // normalisers and maxima visible
      float* obase = (wi.part ? o_part : o_lat) + (wi.orow * n_h + hbase) * D_C;
#pragma unroll
      for (int hb = 0; hb < 4; ++hb) {
        const int h = hb * 16 + r16;
        const float l = l_part[h] + l_part[HG + h];
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
  return launch_attention(decode_h64_fp8_kernel, dim3((unsigned)wgs), dim3(NTHREADS), stream,
                          (const uint16_t*)q_lat, (const uint8_t*)cache, kv_scale, num_blocks,
                          table, max_blocks, seq_lens, q_len, n_h, (int)n_items, B * q_len,
                          n_parts, scale * LOG2E, S, (const int4*)work, lists, n_lists, o_lat,
                          lse, o_part, lse_part);
}

}  // namespace mla
