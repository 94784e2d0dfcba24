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
//          The next tile's 18 direct-to-LDS loads of the wave ride along,
//          one per 32-feature step.
//   softmax: P^T is formed against the running max, which both waves of a head
//          group share, and written to LDS as bf16 fragments.  The max moves
//          lazily, only when a score beats it by 2^8; a wave that sees such a
//          score raises a flag instead, and after the barrier every wave redoes
//          P against the max agreed from both token halves (a second barrier
//          that only the first tile of an item normally pays).
//   PV   : wave w owns output dims 128w..128w+127 for all 64 heads; each
//          transposed V^T fragment feeds four 16-head MFMAs.
//
// LDS: two tile stages (2 x 74752 bytes), token rows of 72 16-byte slots plus
// one pad slot, slot(t, f) = 73 t + f (the 1168-byte row pitch puts the 16
// tokens of a K fragment, and the 4 tokens of a transposing V read, on
// disjoint banks), and an exchange buffer
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
constexpr int RSLOTS = ROW * 2 / 16 + 1;     // 73 16-byte slots per token row: 72 + 1 pad
constexpr int SLOTS = TT * RSLOTS;           // 4672 slots per tile
constexpr int STAGE = SLOTS * 16;            // 74752 bytes
constexpr int NINST = SLOTS / 64;            // 73 global->LDS instructions per tile
constexpr int NDMA = (NINST + 3) / 4;        // 19: instructions of wave 0 (the others issue 18)
// Exchange buffer (a separate LDS object from the tile stages, so the compiler
// can tell its accesses apart from the in-flight direct-to-LDS loads):
constexpr int OFF_P = 0;                     // P^T fragments [2 token halves][4 head blocks][64 lanes][16 B]
constexpr int OFF_MAX = OFF_P + 2 * 4 * 64 * 16;   // float[2][64] tile maxima per token half
constexpr int OFF_F = OFF_MAX + 2 * HG * 4;  // float[64] rescale factors
constexpr int OFF_FLAG = OFF_F + HG * 4;     // int[4] per wave "my scores move the max"
constexpr int XBUF = OFF_FLAG + 16;
constexpr int KSTEPS = ROW / 32;             // 18

__device__ __forceinline__ int slot_of(int t, int f) { return t * RSLOTS + f; }

// Direct-to-LDS load of one 64-token block into a stage, one instruction at a
// time.  Instruction j (0..72) fills slots 64j..64j+63 of the stage; lane l's
// slot s = 64j + l is chunk s % 73 of token s / 73, read from byte
// token * 1152 + chunk * 16 of the block (the pad slot re-reads chunk 71).
// Consecutive lanes thus read consecutive 16-byte chunks of a row, which the
// address path coalesces; lanes spread over rows (1152 bytes apart) would be
// served at about a quarter of the rate.  Wave w issues instructions
// j = w + 4i; its per-lane source offsets are computed once (lane_src).
//
// The instruction is written out (scalar base + 32-bit lane offset, M0 = LDS
// destination; one wait state between the M0 write and its use).  Left to the
// compiler, a direct-to-LDS load between the LDS reads of the QK loop makes it
// wait for every outstanding LDS read (lgkmcnt(0)) before each MFMA, which
// defeats the K prefetch.  The statement has no outputs; its completion is
// awaited explicitly (vmcnt(0) in tile_barrier) before the stage is read.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // M0 is named as clobbered on purpose
__device__ __forceinline__ void issue_one(unsigned lds_dst, const char* block_base, unsigned lane_src) {
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %2"
      :
      : "v"(lane_src), "s"(lds_dst), "s"(block_base)
      : "memory", "m0");
}
#pragma clang diagnostic pop

// Byte offset in the block of lane l's slot of instruction j.
__device__ __forceinline__ unsigned dma_src(int j, int lane) {
  const int slot = 64 * j + lane;
  const int tok = slot / RSLOTS, f = slot - tok * RSLOTS;
  return (unsigned)(tok * (ROW * 2) + min(f, RSLOTS - 2) * 16);
}

// QK^T MFMA with the query fragment read straight from an AGPR (the matrix
// unit accepts AGPR sources).  The compiler's MFMA builtin would copy each
// fragment to VGPRs first, one v_accvgpr_read per register and use, because
// the query (144 registers per wave) only fits in the AGPR file.  d = k q^T
// (+ d); the destination is the accumulator itself, so it never overlaps the
// sources.  Because the compiler does not see these as MFMAs, the callers add
// the wait states it would otherwise insert: after the query is written to
// AGPRs, and before VALU code reads the accumulators (see qk_drain).
__device__ __forceinline__ void mma_qk_first(f32x4_t& d, const i16x8_t& k, const i16x8_t& q) {
  asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(k), "a"(q));
}
__device__ __forceinline__ void mma_qk(f32x4_t& d, const i16x8_t& k, const i16x8_t& q) {
  asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(k), "a"(q));
}
// 24 wait states between the last QK MFMA writing the scores and any other
// instruction touching them (an 8-pass MFMA result needs 11 before a VALU
// read; 24 also covers 16-pass forms).
__device__ __forceinline__ void qk_drain(f32x4_t& a, f32x4_t& b, f32x4_t& c, f32x4_t& d) {
  asm volatile("s_nop 15\n\ts_nop 7" : "+v"(a), "+v"(b), "+v"(c), "+v"(d));
}

// Block-table entry read with a vector load (the address is made opaque to
// the compiler), so that no scalar load is in flight during the QK loop: an
// outstanding scalar load would also force lgkmcnt(0) before each LDS use.
// The value is consumed one tile later, after the tile barrier's vmcnt(0).
__device__ __forceinline__ int load_block_id(const int* p) {
  int z;
  asm volatile("v_mov_b32 %0, 0" : "=v"(z));
  return p[z];
}

__global__ void __launch_bounds__(256, 1) decode_h64_kernel(
    const uint16_t* __restrict__ q_lat, const uint16_t* __restrict__ cache, int num_blocks,
    const int* __restrict__ table, int max_blocks, const int* __restrict__ seq_lens, int q_len,
    int n_h, int n_items, int n_rows, float scale_log2, int S, const int4* __restrict__ work,
    const int* __restrict__ lists, int n_lists, float* __restrict__ o_lat,
    float* __restrict__ lse, float* __restrict__ o_part, float* __restrict__ lse_part) {
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

  // Workgroup id -> (unit, head group): a unit is one work item, or with work
  // lists one list of items run in order.  The head groups of one unit sit 8
  // ids apart so that round-robin dispatch puts them on one XCD, where the
  // second read of every KV tile is served by that XCD's L2.
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
  for (int item = i_begin; item < i_end; ++item) {
    const WorkItem wi = decode_item(item, work, n_rows, q_len, S, seq_lens, max_blocks);
    if (!wi.valid) continue;

    const int lane = lane_id(), g = lane >> 4, r16 = lane & 15;
    // the wave index is uniform; saying so keeps the DMA addresses scalar
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int hq = wave & 1, th = wave >> 1;
    const int b = wi.b, m = wi.m, kb = wi.kb, ke = wi.ke;
    const int hbase = hgrp * HG;                  // first head of the workgroup
    const int d0 = wave * 128;                    // first PV output dim of this wave
    const int t_begin = kb / TT, t_end = kb < ke ? (ke + TT - 1) / TT : t_begin;

    const char* cache_bytes = reinterpret_cast<const char*>(cache);
    const int* trow = table + (long)b * max_blocks;
    // per-lane constants of the tile layout (bytes)
    // source offsets of this wave's DMA instructions (i-th: j = wave + 4i)
    unsigned lane_src[NDMA];
#pragma unroll
    for (int i = 0; i < NDMA; ++i) lane_src[i] = dma_src(min(wave + 4 * i, NINST - 1), lane);
    const int n_dma = wave + 4 * (NDMA - 1) < NINST ? NDMA : NDMA - 1;   // 19 or 18
    // K fragment: token rb + tb*16 + r16, chunk ks*4 + g
    const int k_off = ((th * 32 + r16) * RSLOTS + g) * 16;
    // V^T fragment: tokens 32kh + 4g + (s4 >> 2) (+16), dims d0 + db*16 + 4 (s4 & 3)
    const int s4 = r16;
    const int v_off = (4 * g + (s4 >> 2)) * RSLOTS * 16 + (d0 + 4 * (s4 & 3)) * 2;
    // this wave's share of a block: bytes [18432 w, 18432 (w + 1)) of the block
    // land at the same offsets of the stage
    auto block_ptr = [&](long blk) { return cache_bytes + blk * (long)(BLOCK * ROW * 2); };
    // LDS address of this wave's first DMA destination in a stage
    auto lds_of = [&](char* stage) {
      return (unsigned)(uintptr_t)(__attribute__((address_space(3))) char*)stage + wave * 1024;
    };
    // all of this wave's DMA instructions for one block, back to back
    auto issue_tile = [&](unsigned lds_wave, const char* base) {
#pragma unroll
      for (int i = 0; i < NDMA; ++i)
        if (i < NDMA - 1 || n_dma == NDMA) issue_one(lds_wave + i * 4096, base, lane_src[i]);
    };
    auto tile_block = [&](int t) -> long {
      const int blk = __builtin_amdgcn_readfirstlane(load_block_id(trow + t));
      return (blk >= 0 && blk < num_blocks) ? (long)blk : -1L;
    };
    // Block ids are read one tile ahead of their DMA so the scalar load latency
    // hides behind a tile of compute.
    long blk_cur = -1, blk_nxt = -1;
    if (t_begin < t_end) {
      blk_cur = tile_block(t_begin);
      if (blk_cur >= 0) {
        issue_tile(lds_of(stage0), block_ptr(blk_cur));
      }
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
    // the QK MFMAs read the query from AGPRs: place it there once, then give
    // the AGPR writes their wait states before any MFMA reads them
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) asm volatile("" : "+a"(qf[hb][ks].v));
    asm volatile("s_nop 7\n\ts_nop 7");

    // PV accumulators: 4 head blocks (64 heads) x 8 dim blocks (this wave's 128 dims).
    f32x4_t acc[4][8];
#pragma unroll
    for (int hb = 0; hb < 4; ++hb)
#pragma unroll
      for (int db = 0; db < 8; ++db) acc[hb][db] = f32x4_t{0, 0, 0, 0};
    // Running max / partial sum of this wave's QK heads (lane = head r16 of block hb).
    // Both waves of a head group hold the same running max.
    float mref[2] = {NEG_BIG, NEG_BIG}, lsum[2] = {0.0f, 0.0f};

    // One tile: st holds tile t, nx receives tile t + 1.
    auto tile_step = [&](auto stage_tag, int t) {
      char* st = decltype(stage_tag)::value ? stage1 : stage0;
      char* nx = decltype(stage_tag)::value ? stage0 : stage1;
      const long blk = blk_cur;
      tile_barrier();  // all loads of tile t landed; tile t-1, its P and flags consumed
      // the next tile's loads are spread over this tile's QK steps
      const char* nbase = nullptr;
      if (t + 1 < t_end) {
        if (blk_nxt >= 0) nbase = block_ptr(blk_nxt);
        blk_cur = blk_nxt;
        blk_nxt = t + 2 < t_end ? tile_block(t + 2) : -1L;
      }
      // valid rows [lo, nv) of this tile; a missing block contributes nothing
      const int lo = max(0, kb - t * TT);
      const int nv = blk < 0 ? 0 : min(TT, ke - t * TT);
      if (nv <= lo) {
        if (nbase != nullptr) issue_tile(lds_of(nx), nbase);
        return;
      }
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

      // ---- QK^T: 32 heads x this wave's 32 tokens, next tile's DMA interleaved ----
      const int rb = th * 32;
      f32x4_t sc[2][2];
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) sc[hb][tb] = f32x4_t{0, 0, 0, 0};
      constexpr int KPF = 3;  // K fragments are read KPF steps ahead
      const char* kp = st + k_off;
      auto qk = [&](auto with_dma) {
        BF16::frag kbuf[KPF + 1][2];
        const unsigned nx_lds = lds_of(nx);
        auto load_k = [&](int ks, BF16::frag* dst) {
#pragma unroll
          for (int tb = 0; tb < 2; ++tb)
            dst[tb] = BF16::load8(reinterpret_cast<const uint16_t*>(kp + (tb * 16 * RSLOTS + ks * 4) * 16));
        };
#pragma unroll
        for (int ks = 0; ks < KPF; ++ks) load_k(ks, kbuf[ks]);
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
          if (ks + KPF < KSTEPS) load_k(ks + KPF, kbuf[(ks + KPF) % (KPF + 1)]);
          if (decltype(with_dma)::value) {
            issue_one(nx_lds + ks * 4096, nbase, lane_src[ks]);
            // wave 0 has a 19th instruction
            if (ks == KSTEPS - 1 && n_dma == NDMA) issue_one(nx_lds + KSTEPS * 4096, nbase, lane_src[KSTEPS]);
          }
#pragma unroll
          for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int hb = 0; hb < 2; ++hb) {
              if (ks == 0)
                mma_qk_first(sc[hb][tb], kbuf[0][tb].v, qf[hb][0].v);
              else
                mma_qk(sc[hb][tb], kbuf[ks % (KPF + 1)][tb].v, qf[hb][ks].v);
            }
          __builtin_amdgcn_sched_barrier(0);
        }
      };
      if (nbase != nullptr)
        qk(std::true_type{});
      else
        qk(std::false_type{});
      qk_drain(sc[0][0], sc[0][1], sc[1][0], sc[1][1]);
      // ---- scale, mask, tile max of this wave's tokens ----------------------------
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
          for (int i = 0; i < 4; ++i) sc[hb][tb][i] *= scale_log2;
      if (partial) {
        asm volatile("");  // keeps this a branch: full tiles skip the masking
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
#pragma unroll
          for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int row = rb + tb * 16 + 4 * g + i;
              if (row < lo || row >= nv) sc[hb][tb][i] = -INFINITY;
            }
      }
      float mloc[2];
      bool need = false;
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        float mx = NEG_BIG;
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
          for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sc[hb][tb][i]);
        mloc[hb] = group4_max(mx);
        need |= mloc[hb] > mref[hb] + RESCALE_LOG2;
        if (g == 0) maxbuf[th * HG + hq * 32 + hb * 16 + r16] = mloc[hb];
      }
      // P against the running max, which both waves of a head group share.  A
      // wave whose scores would move the max writes no P and raises its flag;
      // every wave then redoes P against the agreed max (rare: the first tile of
      // an item, and then only when a score beats the max by 2^8).
      float psum[2] = {0.0f, 0.0f};
      auto write_p = [&]() {
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
          float pv[8];
#pragma unroll
          for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int i = 0; i < 4; ++i) pv[tb * 4 + i] = BF16::round(fast_exp2(sc[hb][tb][i] - mref[hb]));
          float s = 0.0f;
#pragma unroll
          for (int j = 0; j < 8; ++j) s += pv[j];
          psum[hb] = s;
          const BF16::frag pf = BF16::from8(pv);
          *reinterpret_cast<i16x8_t*>(pbuf + ((th * 4 + hq * 2 + hb) * 64 + lane) * 16) = pf.v;
        }
      };
      const bool mine = __builtin_amdgcn_ballot_w64(need) != 0;
      if (!mine) write_p();
      if (lane == 0) flags[wave] = mine ? 1 : 0;
      lds_barrier();  // P (or the flags asking for a redo) and the tile maxima are visible
      // The flags, all P fragments and the first V fragments are read together,
      // so the common no-redo path pays one LDS round trip.
      auto load_p = [&](BF16::frag (&pf)[2][4]) {
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
          for (int hb = 0; hb < 4; ++hb)
            pf[kh][hb].v = *reinterpret_cast<const i16x8_t*>(pbuf + ((kh * 4 + hb) * 64 + lane) * 16);
      };
      auto load_v = [&](int kh, int db) -> BF16::frag {
        // lane (dim d0 + db*16 + lane%16, group g): tokens 32kh + 4g + j and +16
        const char* p0 = st + v_off + kh * (32 * RSLOTS * 16) + db * 32;
        i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)p0);
        i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p0 + 16 * RSLOTS * 16));
        BF16::frag f;
        f.v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        return f;
      };
      constexpr int VPF = 3;  // V fragments are read VPF steps ahead
      const int4 fl = *reinterpret_cast<const int4*>(flags);
      BF16::frag pf[2][4];
      load_p(pf);
      BF16::frag vbuf[VPF + 1];
#pragma unroll
      for (int s = 0; s < VPF; ++s) vbuf[s] = load_v(s >> 3, s & 7);
      if ((fl.x | fl.y | fl.z | fl.w) == 0) {
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) lsum[hb] += psum[hb];
      } else {
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
          const float mx = fmaxf(mloc[hb], maxbuf[(th ^ 1) * HG + hq * 32 + hb * 16 + r16]);
          const float mnew = mx > mref[hb] + RESCALE_LOG2 ? mx : mref[hb];
          const float f = fast_exp2(mref[hb] - mnew);
          lsum[hb] *= f;
          mref[hb] = mnew;
          if (th == 0 && g == 0) fbuf[hq * 32 + hb * 16 + r16] = f;
        }
        write_p();
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) lsum[hb] += psum[hb];
        lds_barrier();  // redone P and the rescale factors are visible
        load_p(pf);
#pragma unroll
        for (int hb = 0; hb < 4; ++hb) {
          const float f = fbuf[hb * 16 + r16];
#pragma unroll
          for (int db = 0; db < 8; ++db) acc[hb][db] *= f;
        }
      }
      // ---- PV: 64 heads x this wave's 128 dims x 64 tokens ------------------------
      // step s = (kh, db): tokens 32kh..32kh+31, dims d0 + 16db .. d0 + 16db + 15
#pragma unroll
      for (int s = 0; s < 16; ++s) {
        if (s + VPF < 16) vbuf[(s + VPF) % (VPF + 1)] = load_v((s + VPF) >> 3, (s + VPF) & 7);
#pragma unroll
        for (int hb = 0; hb < 4; ++hb) BF16::mma(acc[hb][s & 7], vbuf[s % (VPF + 1)], pf[s >> 3][hb]);
        __builtin_amdgcn_sched_barrier(0);
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
    __syncthreads();  // stages and exchange buffer are free for the next item
  }
}

}  // namespace

hipError_t launch_decode_h64(const void* q_lat, const void* cache, int num_blocks,
                             const int* table, int max_blocks, const int* seq_lens, int B,
                             int q_len, int n_h, float scale, int S, const int* work, int n_work,
                             const int* lists, int n_lists, float* o_lat, float* lse,
                             float* o_part, float* lse_part, hipStream_t stream) {
  const long n_items = work != nullptr ? (long)n_work : (long)B * q_len * S;
  const long n_units = lists != nullptr ? (long)n_lists : n_items;
  const int ngroups = n_h / HG;
  const long wgs = (n_units + 7) / 8 * 8 * ngroups;
  if (wgs == 0 || n_items == 0) return hipSuccess;
  hipLaunchKernelGGL(decode_h64_kernel, dim3((unsigned)wgs), dim3(256), 0, stream,
                     (const uint16_t*)q_lat, (const uint16_t*)cache, num_blocks, table,
                     max_blocks, seq_lens, q_len, n_h, (int)n_items, B * q_len, scale * LOG2E, S,
                     (const int4*)work, lists, n_lists, o_lat, lse, o_part, lse_part);
  return hipGetLastError();
}

}  // namespace mla
