// Paged latent attention over an FP8 E4M3 cache.
//
// Same computation as decode.hip (eq. 7 of the DeepSeek-V2 notes,
// irregular6612.github.io, §2.1.1, on the absorbed query and the cached
// [c^KV ; R k^R] rows of the DeepSeek-V2 MLA blog, adg.csdn.net, part 2
// §2.2.2), with the cache quantised as the blog's part 3 §3.1.4 serves it:
// here one E4M3 byte per element and two float32 scales per token, s_c for the
// 512 latent elements and s_r for the 64 RoPE elements.  A cached row stands
// for [s_c * c ; s_r * r] with c, r the E4M3 values.
//
// Both products stay on the bf16 MFMA: an E4M3 value is exact in bf16, so the
// codes are widened in registers (v_cvt_scalef32_pk_bf16_fp8 with scale 1)
// and the scales are applied around the products, per token:
//   score_j = s_c,j (q_c . c_j) + s_r,j (q_r . r_j)      (two accumulators)
//   o      += sum_j w_j c_j  with  w_j = bf16(P_j s_c,j)  (the MFMA operand)
//   l      += sum_j w_j / s_c,j
// so that o / l is an exact weighted mean of the dequantised latent rows.
// The value operand of P.V (dims x tokens) is read out of the token-major tile
// with ds_read_b64_tr_b8: within each 16-lane group, lane j names row T(j/2)
// and the 8 bytes at column 16 db + 8 (j % 2); lane i then receives column
// 16 db + i of rows T(0), ..., T(7).
//
// A 64-token tile is 64 rows of 576 bytes (padded to 592 in LDS) plus their
// 512 bytes of scales, 38 KB: two stages per workgroup and two workgroups per
// compute unit fit in its 160 KB of LDS (16 and 32 heads; with 64 heads per
// workgroup the registers allow one).
#include "mla_common.h"
#include "attention_launch.h"
#include "mla_internal.h"

namespace mla {

namespace {

#ifndef MLA_RESCALE_LOG2
#define MLA_RESCALE_LOG2 8.0f
#endif
constexpr float RESCALE_LOG2 = MLA_RESCALE_LOG2;   // lazy-rescale threshold in log2 units
constexpr float NEG_BIG = -1.0e30f;                 // finite "no key yet" running max

typedef int v2i_t __attribute__((ext_vector_type(2)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v2i_t lds_v2i_t;
typedef __bf16 v2bf_t __attribute__((ext_vector_type(2)));

template <int NWH_, int NWT_, int OCC_>
struct Cfg8 {
  static constexpr int NWH = NWH_, NWT = NWT_;
  static constexpr int OCC = OCC_;                  // workgroups per compute unit
  static constexpr int NW = NWH * NWT;
  static constexpr int THREADS = 64 * NW;
  static constexpr int HG = 16 * NWH;               // heads per workgroup (16 per wave)
  static constexpr int TT = BLOCK;                  // tokens per tile: one paged block
  static constexpr int TWAVE = TT / NWT;            // tokens per wave per tile
  static constexpr int CHUNKS = TWAVE >= 32 ? TWAVE / 32 : 1;
  static constexpr int CTB = TWAVE >= 32 ? 2 : 1;   // 16-token blocks per chunk
  static constexpr int RS = ROW + 16;               // padded LDS row stride (bytes)
  static constexpr int SPR = RS / 16;               // 16-byte slots per padded row
  static constexpr int NROWI = (TT * SPR + 63) / 64;
  static constexpr int SCALE_OFF = NROWI * 1024;    // the tile's scales follow its rows
  static constexpr int STAGE = SCALE_OFF + 1024;    // 512 bytes of scales, 512 unused
  static constexpr int KSTEPS = ROW / 32;           // 18 steps of 32 over 576
  static constexpr int KLAT = D_C / 32;             // the first 16 cover the latent part
  static constexpr int DBLK = D_C / 16;
  // the token slices of a head are merged through LDS, MERGE_DIMS dims at a time
  static constexpr int MERGE_BYTES_PER_DIM = NW * 16 * 4;
  static constexpr int MERGE_DIMS =
      MERGE_BYTES_PER_DIM * D_C + 2 * NW * 16 * 4 <= 2 * STAGE       ? D_C
      : MERGE_BYTES_PER_DIM * (D_C / 2) + 2 * NW * 16 * 4 <= 2 * STAGE ? D_C / 2
                                                                        : D_C / 4;
  static_assert(TWAVE >= 16 && TWAVE % 16 == 0, "token slice");
  static_assert(NWT == 1 || MERGE_BYTES_PER_DIM * MERGE_DIMS + 2 * NW * 16 * 4 <= 2 * STAGE,
                "merge space");
  static_assert(TT * SPR == NROWI * 64, "the rows fill whole load instructions");
  static_assert(2 * STAGE * OCC <= 160 * 1024, "LDS for OCC workgroups per compute unit");
};

// 8 E4M3 bytes -> the same 8 values in bf16 (exact: 3 mantissa bits and the
// E4M3 exponent range fit bf16).
__device__ __forceinline__ BF16::frag widen8(v2i_t w) {
  const v2bf_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)w[0], 1.0f, false);
  const v2bf_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)w[0], 1.0f, true);
  const v2bf_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)w[1], 1.0f, false);
  const v2bf_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)w[1], 1.0f, true);
  const u32x4_t u = {__builtin_bit_cast(unsigned, a), __builtin_bit_cast(unsigned, b),
                     __builtin_bit_cast(unsigned, c), __builtin_bit_cast(unsigned, d)};
  BF16::frag f;
  f.v = __builtin_bit_cast(i16x8_t, u);
  return f;
}

// Stage one tile: rows (slot p of the stage <- row p / SPR, piece p % SPR; the
// pad piece re-reads piece 0) and, from one wave, the 64 rows' scales.
template <class C>
__device__ __forceinline__ void issue_tile(char* stage, const uint8_t* cache,
                                           const float* kv_scale, long blk, int wave) {
  const int lane = lane_id();
  const uint8_t* base = cache + blk * BLOCK * (long)ROW;
#pragma unroll 4
  for (int i = wave; i < C::NROWI; i += C::NW) {
    const int p = i * 64 + lane;
    const int r = p / C::SPR;
    int q = p - r * C::SPR;
    if (q == C::SPR - 1) q = 0;
    __builtin_amdgcn_global_load_lds(
        (const void __attribute__((address_space(1)))*)(base + (long)r * ROW + q * 16),
        (void __attribute__((address_space(3)))*)(stage + i * 1024), 16, 0, 0);
  }
  if (wave == C::NW - 1) {
    // lanes 0..31 bring the 512 bytes of scales; lanes 32..63 repeat them into
    // the unused half
    const float* sbase = kv_scale + blk * BLOCK * 2;
    __builtin_amdgcn_global_load_lds(
        (const void __attribute__((address_space(1)))*)(sbase + 4 * (lane & 31)),
        (void __attribute__((address_space(3)))*)(stage + C::SCALE_OFF), 16, 0, 0);
  }
}

template <class C>
__global__ void __launch_bounds__(C::THREADS, C::OCC) decode_fp8_kernel(
    const uint16_t* __restrict__ q_lat, const uint8_t* __restrict__ cache,
    const float* __restrict__ kv_scale, int num_blocks, const int* __restrict__ table,
    int max_blocks, const int* __restrict__ seq_lens, int q_len, int n_h, int n_rows, int n_parts,
    float scale_log2, int S, const int4* __restrict__ work, float* __restrict__ o_lat,
    float* __restrict__ lse, float* __restrict__ o_part, float* __restrict__ lse_part) {
  __shared__ __attribute__((aligned(16))) char smem[2 * C::STAGE];
  const int lane = lane_id(), wave = threadIdx.x >> 6, g = lane >> 4, r16 = lane & 15;
  const int wh = wave % C::NWH, wt = wave / C::NWH;
  const WorkItem wi = decode_item(blockIdx.x, work, n_rows, n_parts, q_len, S, seq_lens, max_blocks);
  if (!wi.valid) return;
  const int b = wi.b, m = wi.m, kb = wi.kb, ke = wi.ke;
  const int head0 = blockIdx.y * C::HG + wh * 16;      // this wave's 16 heads
  const int t_begin = kb / C::TT, t_end = kb < ke ? (ke + C::TT - 1) / C::TT : t_begin;

  const int* trow = table + (long)b * max_blocks;
  auto tile_block = [&](int t) -> long {
    const int blk = trow[(t * C::TT) / BLOCK];
    return (blk >= 0 && blk < num_blocks) ? (long)blk : -1L;
  };

  long blk_next = -1;
  if (t_begin < t_end) {
    blk_next = tile_block(t_begin);
    if (blk_next >= 0) issue_tile<C>(smem, cache, kv_scale, blk_next, wave);
  }

  // Query fragments: B operand of QK, lane = head r16, features ks*32+8g+j.
  BF16::frag qf[C::KSTEPS];
  const long qrow = (long)(b * q_len + m) * n_h;
#pragma unroll
  for (int ks = 0; ks < C::KSTEPS; ++ks)
    qf[ks] = BF16::load8(q_lat + (qrow + head0 + r16) * ROW + ks * 32 + 8 * g);

  f32x4_t acc[C::DBLK];
#pragma unroll
  for (int db = 0; db < C::DBLK; ++db) acc[db] = f32x4_t{0, 0, 0, 0};
  float mref = NEG_BIG, lsum = 0.0f;

  for (int t = t_begin; t < t_end; ++t) {
    char* st = smem + ((t - t_begin) & 1) * C::STAGE;
    const long blk = blk_next;
    tile_barrier();  // everyone's loads of tile t landed, tile t-1 is consumed
    if (t + 1 < t_end) {
      blk_next = tile_block(t + 1);
      if (blk_next >= 0)
        issue_tile<C>(smem + ((t + 1 - t_begin) & 1) * C::STAGE, cache, kv_scale, blk_next, wave);
    }
    // valid rows [lo, nv) of this tile; a missing block contributes nothing
    const int lo = max(0, kb - t * C::TT);
    const int nv = blk < 0 ? 0 : min(C::TT, ke - t * C::TT);
    if (nv <= lo) continue;
    if (lo > 0 || nv < C::TT) {
      // Rows outside the range hold other keys or bytes that may decode to
      // NaN: zero them and give them unit scales, so that P = 0 times the row
      // stays 0.
      const int nz = C::TT - (nv - lo);
      for (int e = threadIdx.x; e < nz * (ROW / 16); e += C::THREADS) {
        const int z = e / (ROW / 16), q = e % (ROW / 16);
        const int r = z < lo ? z : nv + (z - lo);
        *reinterpret_cast<uint4*>(st + r * C::RS + q * 16) = uint4{0, 0, 0, 0};
        if (q == 0) *reinterpret_cast<float2*>(st + C::SCALE_OFF + r * 8) = float2{1.0f, 1.0f};
      }
      lds_barrier();
    }

#pragma unroll
    for (int ch = 0; ch < C::CHUNKS; ++ch) {
      const int rb = wt * C::TWAVE + ch * 32;   // first tile row of this chunk
      // ---- scores S^T[token][head], latent and RoPE parts apart --------------
      f32x4_t sl[2], sr[2];
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) { sl[tb] = f32x4_t{0, 0, 0, 0}; sr[tb] = f32x4_t{0, 0, 0, 0}; }
      v2i_t kraw[2][C::CTB];
      auto load_k = [&](int ks, v2i_t* dst) {
#pragma unroll
        for (int tb = 0; tb < C::CTB; ++tb)
          dst[tb] = *reinterpret_cast<const v2i_t*>(st + (rb + tb * 16 + r16) * C::RS + ks * 32 + 8 * g);
      };
      load_k(0, kraw[0]);
#pragma unroll
      for (int ks = 0; ks < C::KSTEPS; ++ks) {
        if (ks + 1 < C::KSTEPS) load_k(ks + 1, kraw[(ks + 1) % 2]);
#pragma unroll
        for (int tb = 0; tb < C::CTB; ++tb) {
          const BF16::frag kf = widen8(kraw[ks % 2][tb]);
          if (ks < C::KLAT) BF16::mma(sl[tb], kf, qf[ks]);
          else BF16::mma(sr[tb], kf, qf[ks]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      // ---- per-token scales and the online softmax (log2 domain) ------------
      float p[2][4], s_lat[2][4];
      float mx = NEG_BIG;
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = rb + tb * 16 + 4 * g + i;
          float v = -INFINITY;
          s_lat[tb][i] = 1.0f;
          if (tb < C::CTB) {
            const float2 sc = *reinterpret_cast<const float2*>(st + C::SCALE_OFF + row * 8);
            s_lat[tb][i] = sc.x;
            if (row >= lo && row < nv) v = (sc.x * sl[tb][i] + sc.y * sr[tb][i]) * scale_log2;
          }
          p[tb][i] = v;
          mx = fmaxf(mx, v);
        }
      mx = group4_max(mx);
      const float mnew = mx > mref + RESCALE_LOG2 ? mx : mref;
      if (__builtin_amdgcn_ballot_w64(mnew != mref)) {
        const float f = fast_exp2(mref - mnew);
        lsum *= f;
#pragma unroll
        for (int db = 0; db < C::DBLK; ++db) acc[db] *= f;
        mref = mnew;
      }
      // The weight of a token in P.V carries its latent scale and is rounded
      // to bf16; the normaliser adds that same weight over the scale.
      float pv[8];
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float w = BF16::round(fast_exp2(p[tb][i] - mref) * s_lat[tb][i]);
          pv[tb * 4 + i] = w;
          lsum += w * __builtin_amdgcn_rcpf(s_lat[tb][i]);
        }
      const BF16::frag pf = BF16::from8(pv);
      // ---- O^T[dim][head] += V^T . P^T ---------------------------------------
      // this lane names row T(k) of its group, k = (lane % 16) / 2:
      // T(k) = rb + 16 (k / 4) + 4 g + k % 4 (rows of P slot k), the upper
      // four a repeat of the lower when the chunk has one 16-token block
      const int k = r16 >> 1;
      const int vrow = rb + (C::CTB == 2 ? 16 * (k >> 2) : 0) + 4 * g + (k & 3);
      const char* vsrc = st + vrow * C::RS + 8 * (r16 & 1);
      v2i_t vraw[2];
      vraw[0] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i_t*)(vsrc));
#pragma unroll
      for (int db = 0; db < C::DBLK; ++db) {
        if (db + 1 < C::DBLK)
          vraw[(db + 1) % 2] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i_t*)(vsrc + 16 * (db + 1)));
        BF16::mma(acc[db], widen8(vraw[db % 2]), pf);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  // ---- epilogue ------------------------------------------------------------
  float* obase = (wi.part ? o_part : o_lat) + wi.orow * n_h * D_C;
  float* lbase = (wi.part ? lse_part : lse) + wi.orow * n_h;
  if constexpr (C::NWT == 1) {
    const float l = group4_sum(lsum);
    const int head = head0 + r16;
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
#pragma unroll
    for (int db = 0; db < C::DBLK; ++db)
      *reinterpret_cast<float4*>(obase + (long)head * D_C + db * 16 + 4 * g) =
          float4{acc[db][0] * inv, acc[db][1] * inv, acc[db][2] * inv, acc[db][3] * inv};
    if (g == 0) lbase[head] = l > 0.0f ? (mref + __log2f(l)) * LN2 : -INFINITY;
  } else {
    // Merge the NWT token slices of each head through LDS, MERGE_DIMS dims at
    // a time.
    constexpr int MD = C::MERGE_DIMS;
    float* mb = reinterpret_cast<float*>(smem);                   // [NW][16]
    float* lb = mb + C::NW * 16;                                  // [NW][16]
    float* ob = lb + C::NW * 16;                                  // [NW][16][MD]
    __syncthreads();  // all waves are done with the tile stages
    const float l = group4_sum(lsum);
    if (g == 0) { mb[wave * 16 + r16] = mref; lb[wave * 16 + r16] = l; }
#pragma unroll
    for (int d0 = 0; d0 < D_C; d0 += MD) {
#pragma unroll
      for (int db = d0 / 16; db < (d0 + MD) / 16; ++db)
        *reinterpret_cast<float4*>(ob + (wave * 16 + r16) * MD + (db * 16 - d0) + 4 * g) =
            float4{acc[db][0], acc[db][1], acc[db][2], acc[db][3]};
      __syncthreads();
      // thread task: one (head of the workgroup, 4 dims of this round)
      for (int e = threadIdx.x; e < C::HG * (MD / 4); e += C::THREADS) {
        const int hgl = e / (MD / 4), d4 = e % (MD / 4);
        const int whh = hgl / 16, hl = hgl % 16;
        float M = NEG_BIG;
#pragma unroll
        for (int w = 0; w < C::NWT; ++w) M = fmaxf(M, mb[(w * C::NWH + whh) * 16 + hl]);
        float Lsum = 0.0f;
        float4 o = {0, 0, 0, 0};
#pragma unroll
        for (int w = 0; w < C::NWT; ++w) {
          const int ww = w * C::NWH + whh;
          const float f = fast_exp2(mb[ww * 16 + hl] - M);
          Lsum += f * lb[ww * 16 + hl];
          const float4 x = *reinterpret_cast<const float4*>(ob + (ww * 16 + hl) * MD + 4 * d4);
          o.x += f * x.x; o.y += f * x.y; o.z += f * x.z; o.w += f * x.w;
        }
        const float inv = Lsum > 0.0f ? 1.0f / Lsum : 0.0f;
        const int head = blockIdx.y * C::HG + hgl;
        *reinterpret_cast<float4*>(obase + (long)head * D_C + d0 + 4 * d4) =
            float4{o.x * inv, o.y * inv, o.z * inv, o.w * inv};
        if (d0 == 0 && d4 == 0) lbase[head] = Lsum > 0.0f ? (M + __log2f(Lsum)) * LN2 : -INFINITY;
      }
      __syncthreads();   // the next round reuses ob
    }
  }
}

template <class C>
hipError_t launch8(const void* q_lat, const void* cache, const float* kv_scale, int num_blocks,
                   const int* table, int max_blocks, const int* seq_lens, int B, int q_len,
                   int n_h, float scale, int S, const int* work, int n_work, float* o_lat,
                   float* lse, float* o_part, float* lse_part, int n_parts, hipStream_t stream) {
  const long n_items = work != nullptr ? (long)n_work : (long)B * q_len * S;
  if (n_items == 0) return hipSuccess;
  dim3 grid((unsigned)n_items, n_h / C::HG), block(C::THREADS);
  return launch_attention(decode_fp8_kernel<C>, grid, block, stream, (const uint16_t*)q_lat,
                          (const uint8_t*)cache, kv_scale, num_blocks, table, max_blocks,
                          seq_lens, q_len, n_h, B * q_len, n_parts, scale * LOG2E, S,
                          (const int4*)work, o_lat, lse, o_part, lse_part);
}

}  // namespace

hipError_t launch_decode_fp8(const void* q_lat, const void* cache, const float* kv_scale,
                             int num_blocks, const int* table, int max_blocks,
                             const int* seq_lens, int B, int q_len, int n_h, float scale, int S,
                             const int* work, int n_work, const int* lists, int n_lists,
                             float* o_lat, float* lse, float* o_part, float* lse_part,
                             int n_parts, hipStream_t stream) {
  if (n_h % 64 == 0)
    return launch_decode_h64_fp8(q_lat, cache, kv_scale, num_blocks, table, max_blocks, seq_lens,
                                 B, q_len, n_h, scale, S, work, n_work, lists, n_lists, o_lat,
                                 lse, o_part, lse_part, n_parts, stream);
#define MLA_FP8_ARGS q_lat, cache, kv_scale, num_blocks, table, max_blocks, seq_lens, B, q_len, \
                     n_h, scale, S, work, n_work, o_lat, lse, o_part, lse_part, n_parts, stream
  if (n_h == 16) return launch8<Cfg8<1, 4, 2>>(MLA_FP8_ARGS);
  return launch8<Cfg8<2, 2, 2>>(MLA_FP8_ARGS);
#undef MLA_FP8_ARGS
}

}  // namespace mla
