// Paged latent attention: o_lat = softmax(scale * q_lat . row) . c^KV over the cache.
//
// This is eq. 7 of the DeepSeek-V2 notes (irregular6612.github.io, §2.1.1;
// standard scaled-dot softmax attention) applied to the absorbed query and the
// cached latent rows: every head of a sequence scores against the same
// [c^KV ; k^R] rows and sums the same c^KV vectors (DeepSeek-V2 MLA blog,
// adg.csdn.net, part 2 §2.2.2: only c^KV and the rotated k^R are cached, and
// W^UK / W^UV are absorbed).  Because all heads read one KV row, both products
// are dense contractions shared across heads and run on MFMA:
//   S^T[token, head] = K[token, 576] . Q^T[576, head]      (A = cache rows)
//   O^T[dim, head]  += V^T[dim, token] . P^T[token, head]  (A = c^KV transposed)
//
// Work decomposition
//   workgroup = one (sequence, query row, split) x one group of HG heads
//   wave      = HW heads (HB = HW/16 MFMA head blocks) x one token slice of each tile
//   tile      = TT consecutive tokens of one paged block, staged in LDS with
//               direct global->LDS loads, double buffered, shared by all waves.
// Softmax is online (running max / sum per head, lanes of one head reduce with
// cross-lane permutes).  The running max is only moved when a score exceeds it
// by more than RESCALE_LOG2 (log2 units), so rescaling the accumulators is
// rare.  The sum and the output use the same reference, so the result is the
// same in exact arithmetic; in rounding it is not: under a stale reference the
// key that sets the maximum gets a weight above 1 that is rounded to bf16
// like every other weight, instead of exactly 1.
#include "mla_common.h"
#include "attention_launch.h"
#include "mla_internal.h"

namespace mla {

namespace {

#ifndef MLA_RESCALE_LOG2
#define MLA_RESCALE_LOG2 8.0f
#endif
constexpr float RESCALE_LOG2 = MLA_RESCALE_LOG2;   // lazy-rescale threshold in log2 units
constexpr float NEG_BIG = -1.0e30f;    // finite "no key yet" running max

template <class E, int HW_, int NWH_, int NWT_, int TT_>
struct Cfg {
  static constexpr int HW = HW_, NWH = NWH_, NWT = NWT_, TT = TT_;
  static constexpr int HB = HW / 16;
  static constexpr int NW = NWH * NWT;
  static constexpr int THREADS = 64 * NW;
  static constexpr int HG = HW * NWH;             // heads per workgroup
  static constexpr int TWAVE = TT / NWT;          // tokens per wave per tile
  static constexpr int TBW = TWAVE / 16;          // 16-token blocks per wave per tile
  static constexpr int CHUNKS = TWAVE >= 32 ? TWAVE / 32 : 1;
  static constexpr int CTB = TWAVE >= 32 ? 2 : 1; // 16-token blocks per chunk
  static constexpr int ROWB = ROW * E::bytes;     // bytes of one cached row
  static constexpr int RS = ROWB + 16;            // padded LDS row stride
  static constexpr int SPR = RS / 16;             // 16-byte slots per padded row
  static constexpr int NINST = (TT * SPR + 63) / 64;
  static constexpr int STAGE = NINST * 64 * 16;   // bytes of one LDS stage
  static constexpr int KSTEPS = ROW / 32;         // 18 steps of 32 over 576
  static constexpr int DBLK = D_C / 16;           // 32 output blocks of 16 dims
  static_assert(TWAVE >= 16 && TWAVE % 16 == 0, "token slice");
  static_assert(BLOCK % TT == 0, "tile inside one block");
  // end-of-kernel merge of token slices needs NW * HW * 512 floats
  static_assert(NWT == 1 || NW * HW * D_C * 4 + 2 * NW * HW * 4 <= 2 * STAGE, "merge space");
};

// V^T fragment for the PV product: lane (dim = dblk + lane%16, group g) gets
// the dim-th element of tokens rb + 4g + j (slots 0..3) and rb + 16 + 4g + j
// (slots 4..7) of the staged tile; with one 16-token block the upper slots are 0.
template <class E, class C>
struct VT;

template <class C>
struct VT<BF16, C> {
  __device__ static BF16::frag load(const char* st, int rb, int dblk, bool two) {
    const int lane = lane_id(), g = lane >> 4, s = lane & 15;
    const char* p = st + (rb + 4 * g + (s >> 2)) * C::RS + (dblk + 4 * (s & 3)) * 2;
    i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)p);
    i16x4_t hi = {0, 0, 0, 0};
    if (two) hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p + 16 * C::RS));
    BF16::frag f;
    f.v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return f;
  }
};

template <class C>
struct VT<F32, C> {
  __device__ static F32::frag load(const char* st, int rb, int dblk, bool two) {
    const int lane = lane_id(), g = lane >> 4, d = dblk + (lane & 15);
    F32::frag f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      f.v[j] = *reinterpret_cast<const float*>(st + (rb + 4 * g + j) * C::RS + d * 4);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      f.v[4 + j] = two ? *reinterpret_cast<const float*>(st + (rb + 16 + 4 * g + j) * C::RS + d * 4)
                       : 0.0f;
    return f;
  }
};

template <class E, class C>
__device__ __forceinline__ void issue_tile(char* stage, const char* cache_bytes, long blk,
                                           int row0, int wave) {
  // Slot p of the stage (16 bytes) <- row p / SPR, piece p % SPR of the tile;
  // the last piece of a padded row re-reads piece 0 (never used).
  const int lane = lane_id();
  const char* base = cache_bytes + (blk * BLOCK + row0) * (long)C::ROWB;
#pragma unroll 4
  for (int i = wave; i < C::NINST; i += C::NW) {
    int p = i * 64 + lane;
    int r = p / C::SPR, q = p - r * C::SPR;
    if (q == C::SPR - 1) q = 0;
    if (r >= C::TT) { r = 0; q = 0; }
    __builtin_amdgcn_global_load_lds(
        (const void __attribute__((address_space(1)))*)(base + (long)r * C::ROWB + q * 16),
        (void __attribute__((address_space(3)))*)(stage + i * 1024), 16, 0, 0);
  }
}

template <class E, class C>
__global__ void __launch_bounds__(C::THREADS, 1) decode_kernel(
    const typename E::storage* __restrict__ q_lat, const typename E::storage* __restrict__ cache,
    int num_blocks, const int* __restrict__ table, int max_blocks, const int* __restrict__ seq_lens,
    int q_len, int n_h, int n_rows, int n_parts, float scale_log2, int S,
    const int4* __restrict__ work,
    float* __restrict__ o_lat, float* __restrict__ lse, float* __restrict__ o_part,
    float* __restrict__ lse_part) {
  __shared__ __attribute__((aligned(16))) char smem[2 * C::STAGE];
  const int lane = lane_id(), wave = threadIdx.x >> 6, g = lane >> 4, r16 = lane & 15;
  const int wh = wave % C::NWH, wt = wave / C::NWH;
  const WorkItem wi = decode_item(blockIdx.x, work, n_rows, n_parts, q_len, S, seq_lens, max_blocks);
  if (!wi.valid) return;
  const int b = wi.b, m = wi.m, kb = wi.kb, ke = wi.ke;
  const int head0 = blockIdx.y * C::HG + wh * C::HW;  // this wave's first head
  // kb is block aligned unless the range is empty or given unaligned by a plan
  const int t_begin = kb / C::TT, t_end = kb < ke ? (ke + C::TT - 1) / C::TT : t_begin;

  const char* cache_bytes = reinterpret_cast<const char*>(cache);
  const int* trow = table + (long)b * max_blocks;
  auto tile_block = [&](int t) -> long {
    int blk = trow[(t * C::TT) / BLOCK];
    return (blk >= 0 && blk < num_blocks) ? (long)blk : -1L;
  };

  long blk_next = -1;
  if (t_begin < t_end) {
    blk_next = tile_block(t_begin);
    if (blk_next >= 0)
      issue_tile<E, C>(smem, cache_bytes, blk_next, (t_begin * C::TT) % BLOCK, wave);
  }

  // Query fragments: B operand of QK, lane = head r16 of block hb, features ks*32+8g+j.
  typename E::frag qf[C::HB][C::KSTEPS];
  const long qrow = (long)(b * q_len + m) * n_h;
#pragma unroll
  for (int hb = 0; hb < C::HB; ++hb)
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks)
      qf[hb][ks] = E::load8(q_lat + (qrow + head0 + hb * 16 + r16) * ROW + ks * 32 + 8 * g);

  f32x4_t acc[C::HB][C::DBLK];
#pragma unroll
  for (int hb = 0; hb < C::HB; ++hb)
#pragma unroll
    for (int db = 0; db < C::DBLK; ++db) acc[hb][db] = f32x4_t{0, 0, 0, 0};
  float mref[C::HB], lsum[C::HB];
#pragma unroll
  for (int hb = 0; hb < C::HB; ++hb) { mref[hb] = NEG_BIG; lsum[hb] = 0.0f; }

  for (int t = t_begin; t < t_end; ++t) {
    char* st = smem + ((t - t_begin) & 1) * C::STAGE;
    const long blk = blk_next;
    tile_barrier();  // everyone's loads of tile t landed, tile t-1 is consumed
    if (t + 1 < t_end) {
      blk_next = tile_block(t + 1);
      if (blk_next >= 0)
        issue_tile<E, C>(smem + ((t + 1 - t_begin) & 1) * C::STAGE, cache_bytes, blk_next,
                         ((t + 1) * C::TT) % BLOCK, wave);
    }
    // valid rows [lo, nv) of this tile; a missing block contributes nothing
    const int lo = max(0, kb - t * C::TT);
    const int nv = blk < 0 ? 0 : min(C::TT, ke - t * C::TT);
    if (nv <= lo) continue;
    if (lo > 0 || nv < C::TT) {
      // Rows outside the range hold other keys or undefined data: zero them so
      // that P = 0 times the row stays 0.
      const int nz = C::TT - (nv - lo);
      for (int e = threadIdx.x; e < nz * (C::ROWB / 16); e += C::THREADS) {
        const int z = e / (C::ROWB / 16), q = e % (C::ROWB / 16);
        const int r = z < lo ? z : nv + (z - lo);
        *reinterpret_cast<uint4*>(st + r * C::RS + q * 16) = uint4{0, 0, 0, 0};
      }
      lds_barrier();
    }

#pragma unroll
    for (int ch = 0; ch < C::CHUNKS; ++ch) {
      const int rb = wt * C::TWAVE + ch * 32;   // first tile row of this chunk
      // ---- scores S^T[token][head] ------------------------------------------
      // K fragments are prefetched two steps ahead; the scheduling barriers
      // keep the compiler from hoisting every load (register pressure).
      f32x4_t sc[C::HB][2];
#pragma unroll
      for (int hb = 0; hb < C::HB; ++hb)
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) sc[hb][tb] = f32x4_t{0, 0, 0, 0};
      typename E::frag kbuf[2][C::CTB];
      auto load_k = [&](int ks, typename E::frag* dst) {
#pragma unroll
        for (int tb = 0; tb < C::CTB; ++tb)
          dst[tb] = E::load8(reinterpret_cast<const typename E::storage*>(
              st + (rb + tb * 16 + r16) * C::RS + (ks * 32 + 8 * g) * E::bytes));
      };
      load_k(0, kbuf[0]);
#pragma unroll
      for (int ks = 0; ks < C::KSTEPS; ++ks) {
        if (ks + 1 < C::KSTEPS) load_k(ks + 1, kbuf[(ks + 1) % 2]);
#pragma unroll
        for (int tb = 0; tb < C::CTB; ++tb)
#pragma unroll
          for (int hb = 0; hb < C::HB; ++hb) E::mma(sc[hb][tb], kbuf[ks % 2][tb], qf[hb][ks]);
        __builtin_amdgcn_sched_barrier(0);
      }
      // ---- online softmax (log2 domain) -------------------------------------
      float p[C::HB][2][4];
      bool need = false;
      float mnew[C::HB];
#pragma unroll
      for (int hb = 0; hb < C::HB; ++hb) {
        float mx = NEG_BIG;
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int row = rb + tb * 16 + 4 * g + i;
            float v = sc[hb][tb][i] * scale_log2;
            v = (tb < C::CTB && row >= lo && row < nv) ? v : -INFINITY;
            p[hb][tb][i] = v;
            mx = fmaxf(mx, v);
          }
        mx = group4_max(mx);
        mnew[hb] = mx > mref[hb] + RESCALE_LOG2 ? mx : mref[hb];
        need |= mnew[hb] != mref[hb];
      }
      if (__builtin_amdgcn_ballot_w64(need)) {
#pragma unroll
        for (int hb = 0; hb < C::HB; ++hb) {
          const float f = fast_exp2(mref[hb] - mnew[hb]);
          lsum[hb] *= f;
#pragma unroll
          for (int db = 0; db < C::DBLK; ++db) acc[hb][db] *= f;
          mref[hb] = mnew[hb];
        }
      }
      // P is rounded to the MFMA operand type; the normaliser sums the rounded
      // values so that the output is an exact weighted mean of the values.
      typename E::frag pf[C::HB];
#pragma unroll
      for (int hb = 0; hb < C::HB; ++hb) {
        float pv[8];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
          for (int i = 0; i < 4; ++i) pv[tb * 4 + i] = E::round(fast_exp2(p[hb][tb][i] - mref[hb]));
#pragma unroll
        for (int j = 0; j < 8; ++j) lsum[hb] += pv[j];
        pf[hb] = E::from8(pv);
      }
      // ---- O^T[dim][head] += V^T . P^T ---------------------------------------
      typename E::frag vbuf[2];
      vbuf[0] = VT<E, C>::load(st, rb, 0, C::CTB == 2);
#pragma unroll
      for (int db = 0; db < C::DBLK; ++db) {
        if (db + 1 < C::DBLK) vbuf[(db + 1) % 2] = VT<E, C>::load(st, rb, (db + 1) * 16, C::CTB == 2);
#pragma unroll
        for (int hb = 0; hb < C::HB; ++hb) E::mma(acc[hb][db], vbuf[db % 2], pf[hb]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  // ---- epilogue ------------------------------------------------------------
  float* obase = (wi.part ? o_part : o_lat) + wi.orow * n_h * D_C;
  float* lbase = (wi.part ? lse_part : lse) + wi.orow * n_h;
  if constexpr (C::NWT == 1) {
#pragma unroll
    for (int hb = 0; hb < C::HB; ++hb) {
      const float l = group4_sum(lsum[hb]);
      const int head = head0 + hb * 16 + r16;
      const float inv = l > 0.0f ? 1.0f / l : 0.0f;
#pragma unroll
      for (int db = 0; db < C::DBLK; ++db) {
        float4 o = {acc[hb][db][0] * inv, acc[hb][db][1] * inv, acc[hb][db][2] * inv,
                    acc[hb][db][3] * inv};
        *reinterpret_cast<float4*>(obase + (long)head * D_C + db * 16 + 4 * g) = o;
      }
      if (g == 0) lbase[head] = l > 0.0f ? (mref[hb] + __log2f(l)) * LN2 : -INFINITY;
    }
  } else {
    // Merge the NWT token slices of each head through LDS.
    __syncthreads();  // all waves are done with the tile stages
    float* ob = reinterpret_cast<float*>(smem);                  // [NW][HW][512]
    float* mb = ob + C::NW * C::HW * D_C;                        // [NW][HW]
    float* lb = mb + C::NW * C::HW;                              // [NW][HW]
#pragma unroll
    for (int hb = 0; hb < C::HB; ++hb) {
      const float l = group4_sum(lsum[hb]);
      const int hl = hb * 16 + r16;
#pragma unroll
      for (int db = 0; db < C::DBLK; ++db)
        *reinterpret_cast<float4*>(ob + ((long)wave * C::HW + hl) * D_C + db * 16 + 4 * g) =
            float4{acc[hb][db][0], acc[hb][db][1], acc[hb][db][2], acc[hb][db][3]};
      if (g == 0) { mb[wave * C::HW + hl] = mref[hb]; lb[wave * C::HW + hl] = l; }
    }
    __syncthreads();
    // Thread task: one (head of the workgroup, 4 dims).
    for (int e = threadIdx.x; e < C::HG * (D_C / 4); e += C::THREADS) {
      const int hgl = e / (D_C / 4), d4 = e % (D_C / 4);
      const int whh = hgl / C::HW, hl = hgl % C::HW;
      float M = NEG_BIG;
#pragma unroll
      for (int w = 0; w < C::NWT; ++w) M = fmaxf(M, mb[(w * C::NWH + whh) * C::HW + hl]);
      float Lsum = 0.0f;
      float4 o = {0, 0, 0, 0};
#pragma unroll
      for (int w = 0; w < C::NWT; ++w) {
        const int ww = w * C::NWH + whh;
        const float f = fast_exp2(mb[ww * C::HW + hl] - M);
        Lsum += f * lb[ww * C::HW + hl];
        const float4 x = *reinterpret_cast<const float4*>(ob + ((long)ww * C::HW + hl) * D_C + 4 * d4);
        o.x += f * x.x; o.y += f * x.y; o.z += f * x.z; o.w += f * x.w;
      }
      const float inv = Lsum > 0.0f ? 1.0f / Lsum : 0.0f;
      const int head = blockIdx.y * C::HG + hgl;
      *reinterpret_cast<float4*>(obase + (long)head * D_C + 4 * d4) =
          float4{o.x * inv, o.y * inv, o.z * inv, o.w * inv};
      if (d4 == 0) lbase[head] = Lsum > 0.0f ? (M + __log2f(Lsum)) * LN2 : -INFINITY;
    }
  }
}

template <class E, class C>
hipError_t launch(const void* q_lat, const void* cache, int num_blocks, const int* table,
                  int max_blocks, const int* seq_lens, int B, int q_len, int n_h, float scale,
                  int S, const int* work, int n_work, float* o_lat, float* lse, float* o_part,
                  float* lse_part, int n_parts, hipStream_t stream) {
  const long n_items = work != nullptr ? (long)n_work : (long)B * q_len * S;
  if (n_items == 0) return hipSuccess;
  dim3 grid((unsigned)n_items, n_h / C::HG), block(C::THREADS);
  using T = typename E::storage;
  return launch_attention(decode_kernel<E, C>, grid, block, stream, (const T*)q_lat,
                          (const T*)cache, num_blocks, table, max_blocks, seq_lens, q_len, n_h,
                          B * q_len, n_parts, scale * LOG2E, S, (const int4*)work, o_lat, lse,
                          o_part, lse_part);
}

#define MLA_DECODE_ARGS q_lat, cache, num_blocks, table, max_blocks, seq_lens, B, q_len, n_h, \
                        scale, S, work, n_work, o_lat, lse, o_part, lse_part, n_parts, stream

template <class E, int TT>
hipError_t dispatch_heads(const void* q_lat, const void* cache, int num_blocks, const int* table,
                          int max_blocks, const int* seq_lens, int B, int q_len, int n_h,
                          float scale, int S, const int* work, int n_work, float* o_lat,
                          float* lse, float* o_part, float* lse_part, int n_parts,
                          hipStream_t stream) {
  constexpr int NWT16 = TT / 16 < 4 ? TT / 16 : 4;   // token slices for a lone head block
  if (n_h == 16) return launch<E, Cfg<E, 16, 1, NWT16, TT>>(MLA_DECODE_ARGS);
  if (n_h == 32) return launch<E, Cfg<E, 16, 2, 2, TT>>(MLA_DECODE_ARGS);
  return launch<E, Cfg<E, 16, 4, 1, TT>>(MLA_DECODE_ARGS);
}

}  // namespace

hipError_t launch_decode(const void* q_lat, const void* cache, int num_blocks, const int* table,
                         int max_blocks, const int* seq_lens, int B, int q_len, int n_h,
                         int dtype, float scale, int S, const int* work, int n_work,
                         const int* lists, int n_lists, float* o_lat, float* lse, float* o_part,
                         float* lse_part, int n_parts, hipStream_t stream) {
  if (dtype == 1 && n_h % 64 == 0)
    return launch_decode_h64(q_lat, cache, num_blocks, table, max_blocks, seq_lens, B, q_len,
                             n_h, scale, S, work, n_work, lists, n_lists, o_lat, lse, o_part,
                             lse_part, n_parts, stream);
  if (dtype == 1) return dispatch_heads<BF16, 64>(MLA_DECODE_ARGS);
  return dispatch_heads<F32, 32>(MLA_DECODE_ARGS);
}

}  // namespace mla
