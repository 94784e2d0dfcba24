// Paged latent attention, bf16, for head counts that are multiples of 64
// (DeepSeek-V2 uses 128 heads).
//
// Same computation as decode.hip (eq. 7 of the DeepSeek-V2 notes,
// irregular6612.github.io, §2.1.1, on the absorbed query and the cached
// [c^KV ; k^R] rows of the DeepSeek-V2 MLA blog, adg.csdn.net, part 2 §2.2.2).
//
// One workgroup (4 waves) owns 64 heads of one (sequence, query row, split).
// With 128 heads the two head halves of an item are launched 8 workgroup ids
// apart, which places them on the same XCD so the second read of every KV
// tile is served by that XCD's L2.  Inside the workgroup, per 64-token tile:
//
//   QK^T : wave (hq, th) = (w & 1, w >> 1) scores heads 32hq..32hq+31 against
//          tokens 32th..32th+31.  Its 32 query rows stay in registers (B
//          operand); each 16-token x 32-feature K fragment read from LDS feeds
//          two 16-head MFMAs.
//   softmax: the two waves sharing a head group swap their tile maxima through
//          LDS so both move the running max identically (lazy: only when a
//          score exceeds it by 2^8), then write bf16 P^T fragments to LDS.
//   PV   : wave w owns output dims 128w..128w+127 for all 64 heads; each
//          transposed V^T fragment feeds four 16-head MFMAs.
//
// LDS: two tile stages (2 x 73728 bytes) in an 8-token interleaved layout of
// 16-byte slots, slot(t, f) = ((t / 8) * 72 + f) * 8 + t % 8 (conflict-free for
// the 16-byte K reads and the transposing V reads), and an exchange buffer
// with the 8 KB of P, the tile maxima, rescale factors and flags.
#include <type_traits>

#include "mla_common.h"
#include "mla_internal.h"

namespace mla {

namespace {

constexpr float RESCALE_LOG2 = 8.0f;  // lazy-rescale threshold (log2 units)
constexpr float NEG_BIG = -1.0e30f;   // finite "no key yet" running max

constexpr int HG = 64;                       // heads per workgroup
constexpr int TT = 64;                       // tokens per tile (one paged block)
constexpr int SLOTS = TT * (ROW * 2 / 16);   // 4608 16-byte slots per tile
constexpr int STAGE = SLOTS * 16;            // 73728
constexpr int NINST = SLOTS / 64;            // 72 global->LDS instructions per tile
// Exchange buffer (a separate LDS object from the tile stages, so the compiler
// can tell its accesses apart from the in-flight direct-to-LDS loads):
constexpr int OFF_P = 0;                     // P^T fragments [2 token halves][4 head blocks][64 lanes][16 B]
constexpr int OFF_MAX = OFF_P + 2 * 4 * 64 * 16;   // float[2][64] tile maxima per token half
constexpr int OFF_F = OFF_MAX + 2 * HG * 4;  // float[64] rescale factors
constexpr int OFF_FLAG = OFF_F + HG * 4;     // int[4] (2 used) per head group "rescaled"
constexpr int XBUF = OFF_FLAG + 16;
constexpr int KSTEPS = ROW / 32;             // 18

__device__ __forceinline__ int slot_of(int t, int f) { return ((t >> 3) * 72 + f) * 8 + (t & 7); }

// Direct-to-LDS load of one 64-token block into a stage.  Instruction i fills
// slots 64i..64i+63 = 8-token group i / 9, chunks 8 (i % 9) .. 8 (i % 9) + 7,
// so lane l always reads token (l & 7) of the group, chunk (l >> 3): a per-lane
// constant byte offset plus a per-instruction uniform one (no per-lane math).
__device__ __forceinline__ void issue_tile(char* stage, const char* block_base, int lane_off,
                                           int wave) {
#pragma unroll
  for (int j = 0; j < NINST / 4; ++j) {
    const int i = wave + 4 * j;
    const int goff = (i / 9) * (8 * ROW * 2) + (i % 9) * 128;
    __builtin_amdgcn_global_load_lds(
        (const void __attribute__((address_space(1)))*)(block_base + goff + lane_off),
        (void __attribute__((address_space(3)))*)(stage + i * 1024), 16, 0, 0);
  }
}

__global__ void __launch_bounds__(256, 1) decode_h64_kernel(
    const uint16_t* __restrict__ q_lat, const uint16_t* __restrict__ cache, int num_blocks,
    const int* __restrict__ table, int max_blocks, const int* __restrict__ seq_lens, int q_len,
    int n_h, int n_items, int n_rows, float scale_log2, int S, const int4* __restrict__ work,
    float* __restrict__ o_lat, float* __restrict__ lse, float* __restrict__ o_part,
    float* __restrict__ lse_part) {
  // The two tile stages are distinct LDS objects and every tile iteration
  // names its stage at compile time, so the compiler can see that reading one
  // stage does not race the direct-to-LDS loads into the other.
  __shared__ __attribute__((aligned(16))) char stage0[STAGE];
  __shared__ __attribute__((aligned(16))) char stage1[STAGE];
  __shared__ __attribute__((aligned(16))) char xbuf[XBUF];
  char* pbuf = xbuf + OFF_P;
  float* maxbuf = reinterpret_cast<float*>(xbuf + OFF_MAX);
  float* fbuf = reinterpret_cast<float*>(xbuf + OFF_F);
  int* flags = reinterpret_cast<int*>(xbuf + OFF_FLAG);

  // Workgroup id -> (item, head group): the head groups of one item sit 8 ids
  // apart so that round-robin dispatch puts them on one XCD.
  const int ngroups = n_h / HG;
  const int wid = blockIdx.x;
  const int hgrp = (wid >> 3) % ngroups;
  const int item = (wid / (8 * ngroups)) * 8 + (wid & 7);
  if (item >= n_items) return;
  const WorkItem wi = decode_item(item, work, n_rows, q_len, S, seq_lens, max_blocks);
  if (!wi.valid) return;

  const int lane = lane_id(), wave = threadIdx.x >> 6, g = lane >> 4, r16 = lane & 15;
  const int hq = wave & 1, th = wave >> 1;
  const int b = wi.b, m = wi.m, kb = wi.kb, ke = wi.ke;
  const int hbase = hgrp * HG;                  // first head of the workgroup
  const int d0 = wave * 128;                    // first PV output dim of this wave
  const int t_begin = kb / TT, t_end = kb < ke ? (ke + TT - 1) / TT : t_begin;

  const char* cache_bytes = reinterpret_cast<const char*>(cache);
  const int* trow = table + (long)b * max_blocks;
  // per-lane constants of the tile layout (bytes)
  const int dma_off = (lane & 7) * (ROW * 2) + (lane >> 3) * 16;
  // K fragment: token rb + tb*16 + r16, chunk ks*4 + g
  const int k_off = (((th * 32) >> 3) * 576 + (r16 >> 3) * 576 + g * 8 + (r16 & 7)) * 16;
  // V^T fragment: tokens 32kh + 4g + (s4 >> 2) (+16), dims d0 + db*16 + 4 (s4 & 3)
  const int s4 = r16;
  const int v_off = ((g >> 1) * 576 + ((d0 >> 3) + ((s4 & 3) >> 1)) * 8 + 4 * (g & 1) + (s4 >> 2)) * 16 +
                    (s4 & 1) * 8;
  auto block_ptr = [&](long blk) { return cache_bytes + blk * (long)(BLOCK * ROW * 2); };
  auto tile_block = [&](int t) -> long {
    const int blk = trow[t];
    return (blk >= 0 && blk < num_blocks) ? (long)blk : -1L;
  };
  // Block ids are read one tile ahead of their DMA so the scalar load latency
  // hides behind a tile of compute.
  long blk_cur = -1, blk_nxt = -1;
  if (t_begin < t_end) {
    blk_cur = tile_block(t_begin);
    if (blk_cur >= 0) issue_tile(stage0, block_ptr(blk_cur), dma_off, wave);
    if (t_begin + 1 < t_end) blk_nxt = tile_block(t_begin + 1);
  }

  // Query fragments of this wave's 32 QK heads (B operand).
  BF16::frag qf[2][KSTEPS];
  const long qrow = (long)(b * q_len + m) * n_h + hbase + hq * 32;
#pragma unroll
  for (int hb = 0; hb < 2; ++hb)
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks)
      qf[hb][ks] = BF16::load8(q_lat + (qrow + hb * 16 + r16) * ROW + ks * 32 + 8 * g);

  // PV accumulators: 4 head blocks (64 heads) x 8 dim blocks (this wave's 128 dims).
  f32x4_t acc[4][8];
#pragma unroll
  for (int hb = 0; hb < 4; ++hb)
#pragma unroll
    for (int db = 0; db < 8; ++db) acc[hb][db] = f32x4_t{0, 0, 0, 0};
  // Running max / partial sum of this wave's QK heads (lane = head r16 of block hb).
  float mref[2] = {NEG_BIG, NEG_BIG}, lsum[2] = {0.0f, 0.0f};

  // One tile: st holds tile t, nx receives tile t + 1.
  auto tile_step = [&](auto stage_tag, int t) {
    char* st = decltype(stage_tag)::value ? stage1 : stage0;
    char* nx = decltype(stage_tag)::value ? stage0 : stage1;
    const long blk = blk_cur;
    tile_barrier();  // all loads of tile t landed; tile t-1, its P and flags consumed
    if (t + 1 < t_end) {
      if (blk_nxt >= 0) issue_tile(nx, block_ptr(blk_nxt), dma_off, wave);
      blk_cur = blk_nxt;
      blk_nxt = t + 2 < t_end ? tile_block(t + 2) : -1L;
    }
    // valid rows [lo, nv) of this tile; a missing block contributes nothing
    const int lo = max(0, kb - t * TT);
    const int nv = blk < 0 ? 0 : min(TT, ke - t * TT);
    if (nv <= lo) return;
    const bool partial = lo > 0 || nv < TT;
    if (partial) {
      // rows outside the range hold other keys or undefined data; P = 0 there,
      // so zero them
      const int nz = TT - (nv - lo);
      for (int e = threadIdx.x; e < nz * 72; e += 256) {
        const int z = e / 72, f = e % 72;
        const int r = z < lo ? z : nv + (z - lo);
        *reinterpret_cast<uint4*>(st + slot_of(r, f) * 16) = uint4{0, 0, 0, 0};
      }
      lds_barrier();
    }

    // ---- QK^T: 32 heads x this wave's 32 tokens --------------------------------
    const int rb = th * 32;
    f32x4_t sc[2][2];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) sc[hb][tb] = f32x4_t{0, 0, 0, 0};
    BF16::frag kbuf[2][2];
    const char* kp = st + k_off;
    auto load_k = [&](int ks, BF16::frag* dst) {
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
        dst[tb] = BF16::load8(reinterpret_cast<const uint16_t*>(kp + (tb * 2 * 576 + ks * 32) * 16));
    };
    load_k(0, kbuf[0]);
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      if (ks + 1 < KSTEPS) load_k(ks + 1, kbuf[(ks + 1) & 1]);
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) BF16::mma(sc[hb][tb], kbuf[ks & 1][tb], qf[hb][ks]);
      __builtin_amdgcn_sched_barrier(0);
    }
    // ---- scale, mask, local tile max -------------------------------------------
    float mloc[2];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      float mx = NEG_BIG;
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = rb + tb * 16 + 4 * g + i;
          float v = sc[hb][tb][i] * scale_log2;
          if (partial) v = (row >= lo && row < nv) ? v : -INFINITY;
          sc[hb][tb][i] = v;
          mx = fmaxf(mx, v);
        }
      mloc[hb] = group4_max(mx);
      if (g == 0) maxbuf[th * HG + hq * 32 + hb * 16 + r16] = mloc[hb];
    }
    lds_barrier();  // both token halves' maxima are visible
    // ---- running max (identical in both waves of a head group), P ---------------
    bool need = false;
    float mnew[2];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const float mx = fmaxf(mloc[hb], maxbuf[(th ^ 1) * HG + hq * 32 + hb * 16 + r16]);
      mnew[hb] = mx > mref[hb] + RESCALE_LOG2 ? mx : mref[hb];
      need |= mnew[hb] != mref[hb];
    }
    const bool resc = __builtin_amdgcn_ballot_w64(need) != 0;
    if (resc) {
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        const float f = fast_exp2(mref[hb] - mnew[hb]);
        lsum[hb] *= f;
        mref[hb] = mnew[hb];
        if (th == 0 && g == 0) fbuf[hq * 32 + hb * 16 + r16] = f;
      }
    }
    if (th == 0 && lane == 0) flags[hq] = resc ? 1 : 0;
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      float pv[8];
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int i = 0; i < 4; ++i) pv[tb * 4 + i] = BF16::round(fast_exp2(sc[hb][tb][i] - mref[hb]));
#pragma unroll
      for (int j = 0; j < 8; ++j) lsum[hb] += pv[j];
      const BF16::frag pf = BF16::from8(pv);
      *reinterpret_cast<i16x8_t*>(pbuf + ((th * 4 + hq * 2 + hb) * 64 + lane) * 16) = pf.v;
    }
    lds_barrier();  // P, factors and flags are visible
    // ---- rescale this wave's accumulators if a head group moved its max ---------
    const int2 fl = *reinterpret_cast<const int2*>(flags);
    if (fl.x | fl.y) {
#pragma unroll
      for (int hb = 0; hb < 4; ++hb) {
        const float f = (hb < 2 ? fl.x : fl.y) ? fbuf[hb * 16 + r16] : 1.0f;
#pragma unroll
        for (int db = 0; db < 8; ++db) acc[hb][db] *= f;
      }
    }
    // ---- PV: 64 heads x this wave's 128 dims x 64 tokens ------------------------
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      BF16::frag pf[4];
#pragma unroll
      for (int hb = 0; hb < 4; ++hb)
        pf[hb].v = *reinterpret_cast<const i16x8_t*>(pbuf + ((kh * 4 + hb) * 64 + lane) * 16);
      auto load_v = [&](int db) -> BF16::frag {
        // lane (dim d0 + db*16 + lane%16, group g): tokens 32kh + 4g + j and +16
        const char* p0 = st + v_off + kh * (4 * 576 * 16) + db * 256;
        i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)p0);
        i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p0 + 2 * 576 * 16));
        BF16::frag f;
        f.v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        return f;
      };
      BF16::frag vbuf[2];
      vbuf[0] = load_v(0);
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        if (db + 1 < 8) vbuf[(db + 1) & 1] = load_v(db + 1);
#pragma unroll
        for (int hb = 0; hb < 4; ++hb) BF16::mma(acc[hb][db], vbuf[db & 1], pf[hb]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  for (int t = t_begin; t < t_end; t += 2) {
    tile_step(std::integral_constant<int, 0>{}, t);
    if (t + 1 < t_end) tile_step(std::integral_constant<int, 1>{}, t + 1);
  }

  // ---- epilogue: per-head sums over both token halves, normalise, write -------
  __syncthreads();  // exchange buffer is free now
  float* mx_all = reinterpret_cast<float*>(xbuf);   // [64] running max per head
  float* l_all = mx_all + HG;                       // [2][64] partial sums per token half
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    const float l = group4_sum(lsum[hb]);
    if (g == 0) {
      l_all[th * HG + hq * 32 + hb * 16 + r16] = l;
      if (th == 0) mx_all[hq * 32 + hb * 16 + r16] = mref[hb];
    }
  }
  __syncthreads();
  float* obase = (wi.part ? o_part : o_lat) + (wi.orow * n_h + hbase) * D_C;
  float* lbase = (wi.part ? lse_part : lse) + wi.orow * n_h + hbase;
#pragma unroll
  for (int hb = 0; hb < 4; ++hb) {
    const int h = hb * 16 + r16;
    const float l = l_all[h] + l_all[HG + h];
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
#pragma unroll
    for (int db = 0; db < 8; ++db)
      *reinterpret_cast<float4*>(obase + (long)h * D_C + d0 + db * 16 + 4 * g) =
          float4{acc[hb][db][0] * inv, acc[hb][db][1] * inv, acc[hb][db][2] * inv,
                 acc[hb][db][3] * inv};
  }
  if (threadIdx.x < HG) {
    const int h = threadIdx.x;
    const float l = l_all[h] + l_all[HG + h];
    lbase[h] = l > 0.0f ? (mx_all[h] + __log2f(l)) * LN2 : -INFINITY;
  }
}

}  // namespace

hipError_t launch_decode_h64(const void* q_lat, const void* cache, int num_blocks,
                             const int* table, int max_blocks, const int* seq_lens, int B,
                             int q_len, int n_h, float scale, int S, const int* work, int n_work,
                             float* o_lat, float* lse, float* o_part, float* lse_part,
                             hipStream_t stream) {
  const long n_items = work != nullptr ? (long)n_work : (long)B * q_len * S;
  const int ngroups = n_h / HG;
  const long wgs = (n_items + 7) / 8 * 8 * ngroups;
  if (wgs == 0) return hipSuccess;
  hipLaunchKernelGGL(decode_h64_kernel, dim3((unsigned)wgs), dim3(256), 0, stream,
                     (const uint16_t*)q_lat, (const uint16_t*)cache, num_blocks, table,
                     max_blocks, seq_lens, q_len, n_h, (int)n_items, B * q_len, scale * LOG2E, S,
                     (const int4*)work, o_lat, lse, o_part, lse_part);
  return hipGetLastError();
}

}  // namespace mla
