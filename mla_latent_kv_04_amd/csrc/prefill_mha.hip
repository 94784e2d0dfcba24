// Chunked prefill in the non-absorbed form: eq. 7 of the DeepSeek-V2 notes
// (irregular6612.github.io, §2.1.1) with eq. 10-11's per-head keys and values
// k^C_{j,i} = W^UK_i c^KV_j and v^C_{j,i} = W^UV_i c^KV_j materialised once
// per sequence, and the decoupled key / query of the DeepSeek-V2 MLA blog
// (adg.csdn.net, part 2 §2.2.2): q_i = [q^C_i ; R q^R_i], k_{j,i} = [k^C_{j,i} ;
// k^R_j].  Per (query row, head, key) this costs 2 (128 + 64) + 2 128 flops
// against 2 576 + 2 512 in the absorbed form, plus the up-projection once per
// key; the blog reserves absorption for generation, where one query row
// meets each key.
//
// Per sequence:
//   1. k^C = c^KV W^UK^T into kc [n_h][Lpad][128] and v^C transposed into
//      vt [n_h][128][Lpad] as bf16 hi + lo (hi, then lo n_h 128 Lpad
//      elements further; the tile projection of proj_tile.h, reading the
//      c^KV rows straight from the paged cache);
//   2. mha_prefill_kernel: one workgroup per (256 query rows, head); eight
//      waves of 32 rows (two per SIMD); key tiles of 64 (one paged block)
//      brought into LDS by direct global->LDS loads, one tile ahead (k^C and
//      the cached, rotated k^R of each key, and v^C^T hi and lo);
//      scores S^T = K Q^T on MFMA, an online softmax per query row, and
//      O^T += (V_hi^T + V_lo^T) P^T with P taken straight from the score
//      registers.
//
// Precision: q^R, k^C and P are rounded to bf16 as MFMA operands.  v^C is
// carried as hi + lo: rounding it too would put the largest error of a
// 2^18-output comparison at ~2.1e-2 of the output RMS (a CPU emulation of
// this arithmetic), against ~1.4e-2 without.
#include <algorithm>

#include "mla_common.h"
#include "mla_internal.h"
#include "proj_tile.h"

namespace mla {
namespace {

constexpr int NW = 8;                    // waves per workgroup (two per SIMD)
constexpr int QB = 32 * NW;              // query rows per workgroup
constexpr int KT = 64;                   // keys per tile: one paged block
constexpr int VTILE = D_H * KT * 2;      // 16 KB: v^T [128 dims][64 keys]
// one tile buffer: k^C [64][128], k^R [64][64], v^T hi, v^T lo (bytes)
constexpr int OFF_KC = 0, OFF_KR = 16384, OFF_VH = 24576, OFF_VL = OFF_VH + VTILE;
constexpr int BUF = OFF_VL + VTILE;      // 56 KB; two buffers in LDS
constexpr int NDMA = BUF / 1024 / NW;    // direct loads per wave per tile (7)
constexpr float NEG_BIG_P = -1.0e30f;    // finite "no key yet" running max

__device__ __forceinline__ int kswz(int r) { return (r & 3) | ((r >> 1) & 4); }

// LDS layouts: every row is a whole number of 16-byte pieces, and piece p of
// row r sits in slot p ^ f(r), so that the eight lanes of one ds_read_b128
// phase (eight rows, one piece) hit eight bank groups: f(r) = r & 7 for v^T
// rows (dims, read 8 consecutive at a time), kswz(r) for key rows (read as
// rows {0..3, 8..11} + 32 b + 4 c, see below).
//   k^C row (key) of 256 bytes, k^R row of 128 bytes, v^T row (dim) of 128
//   bytes whose piece p holds keys 8 p .. 8 p + 7.
// Score MFMA block a (16 keys) takes as its row 4 q + i the key
// 32 (a >> 1) + 8 q + 4 (a & 1) + i of the tile: lane (g, r16) then holds
// the scores of keys 32 (a >> 1) + 8 g + 4 (a & 1) + i, so that its eight P
// values of PV k-step ks2 (blocks 2 ks2, 2 ks2 + 1) are keys
// 32 ks2 + 8 g .. + 7, which is piece 4 ks2 + g of a v^T row.
// Direct load I (0..55) of a tile fills LDS bytes [1024 I, 1024 I + 1024) of
// the buffer: I < 16 k^C rows 4 I.., I < 24 k^R rows 8 (I - 16).., then v^T
// hi rows and v^T lo rows 8 (I - 24) % 128..; wave w issues I = 7 w .. 7 w + 6.

__global__ void __launch_bounds__(64 * NW, 1) mha_prefill_kernel(
    const uint16_t* __restrict__ q_nope, const uint16_t* __restrict__ q_rope,
    const int* __restrict__ q_pos, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vt, const uint16_t* __restrict__ cache, int num_blocks,
    const int* __restrict__ trow, int L, int q_len, int Lpad, int n_h, int row0,
    float scale_log2, RopeFreq rf, float* __restrict__ out, float* __restrict__ lse) {
  __shared__ __attribute__((aligned(16))) char smem[2 * BUF];
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int g = lane >> 4, r16 = lane & 15;
  // Workgroup (query block, head), in dispatch order wid = x + gridDim.x y.
  // Dispatch deals workgroup ids round-robin to the 8 XCDs; with n_h a
  // multiple of 8 the query blocks of one head get ids 8 apart, so they run
  // on one XCD at about the same time and read the head's k^C and v^C tiles
  // through its L2 (otherwise each XCD streams them from HBM).
  int h = blockIdx.y, qb = blockIdx.x;
  if (n_h % 8 == 0) {
    const int wid = blockIdx.x + gridDim.x * blockIdx.y, rest = wid >> 3;
    qb = rest % gridDim.x;
    h = (rest / gridDim.x) * 8 + (wid & 7);
  }
  const int m0 = qb * QB;
  const int mw = m0 + 32 * wave;                 // this wave's first query row (chunk index)
  const int shift = L - q_len + 1;               // row m sees keys j < shift + m (and j < L)
  const int m_top = min(m0 + QB, q_len) - 1;
  const int kmax = min(L, max(0, shift + m_top));
  const int ntiles = (kmax + KT - 1) / KT;
  const uint16_t* kc_h = kc + (long)h * Lpad * D_H;
  const uint16_t* vt_h = vt + (long)h * D_H * Lpad;
  const long vlo = (long)n_h * D_H * Lpad;       // v^T lo, that many elements after hi

  // Query fragments (B operand of S^T = K Q^T): q[qq][ks] holds row
  // mw + 16 qq + r16, features 32 ks + 8 g .. + 7 (ks < 4: q^C; ks = 4, 5:
  // q^R rotated at the row's position, pairs 16 (ks - 4) + 4 g .. + 3).
  i16x8_t q[2][6];
#pragma unroll
  for (int qq = 0; qq < 2; ++qq) {
    const int m = min(mw + 16 * qq + r16, q_len - 1);
    const long row = (long)(row0 + m) * n_h + h;
    const uint16_t* qn = q_nope + row * D_H;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) q[qq][ks] = *reinterpret_cast<const i16x8_t*>(qn + 32 * ks + 8 * g);
    const uint16_t* qr = q_rope + row * D_R;
    const int pos = q_pos[row0 + m];
#pragma unroll
    for (int ks = 4; ks < 6; ++ks) {
      const i16x8_t raw = *reinterpret_cast<const i16x8_t*>(qr + 32 * (ks - 4) + 8 * g);
      i16x8_t rot;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        double cs, sn;
        rope_cs(pos, rf.theta[16 * (ks - 4) + 4 * g + u], cs, sn);
        const double x = bf16_to_f32((uint16_t)raw[2 * u]), y = bf16_to_f32((uint16_t)raw[2 * u + 1]);
        rot[2 * u] = (short)f32_to_bf16((float)(x * cs - y * sn));
        rot[2 * u + 1] = (short)f32_to_bf16((float)(x * sn + y * cs));
      }
      q[qq][ks] = rot;
    }
  }

  // this wave's direct loads: lane offsets inside the tile's source rows
  unsigned loff[NDMA];
#pragma unroll
  for (int j = 0; j < NDMA; ++j) {
    const int I = NDMA * wave + j;
    if (I < 16) {                                         // k^C: 4 rows of 256 bytes
      const int r = 4 * I + (lane >> 4);
      loff[j] = (unsigned)(r * (D_H * 2) + (((lane & 15) ^ kswz(r)) * 16));
    } else if (I < 24) {                                  // k^R: 8 cache rows, bytes 1024..1151
      const int r = 8 * (I - 16) + (lane >> 3);
      loff[j] = (unsigned)(r * (ROW * 2) + (((lane & 7) ^ kswz(r)) * 16));
    } else {                                              // v^T hi / lo: 8 dims of 128 bytes
      const int d = 8 * ((I - 24) & 15) + (lane >> 3);
      loff[j] = (unsigned)(d * Lpad * 2 + (((lane & 7) ^ (d & 7)) * 16));
    }
  }
  const unsigned lds0 = (unsigned)(uintptr_t)(__attribute__((address_space(3))) char*)smem;
  auto tile_block = [&](int kt) { return __builtin_amdgcn_readfirstlane(trow[kt]); };
  auto issue = [&](int kt, int buf) __attribute__((always_inline)) {
    const int key0 = kt * KT;
    int blk = tile_block(kt);
    if (blk < 0 || blk >= num_blocks) blk = 0;           // such a tile is skipped
    const char* src_kc = reinterpret_cast<const char*>(kc_h + (long)key0 * D_H);
    const char* src_kr = reinterpret_cast<const char*>(cache + (long)blk * BLOCK * ROW + D_C);
    const char* src_vh = reinterpret_cast<const char*>(vt_h + key0);
    const char* src_vl = reinterpret_cast<const char*>(vt_h + vlo + key0);
    const unsigned dst = lds0 + (unsigned)(buf * BUF);
#pragma unroll
    for (int j = 0; j < NDMA; ++j) {
      const int I = NDMA * wave + j;
      const char* src = I < 16 ? src_kc : I < 24 ? src_kr : I < 40 ? src_vh : src_vl;
      dma16(dst + I * 1024, src, loff[j]);
    }
  };

  // O^T accumulators: acc[db][qq] lane (g, r16) holds dims 16 db + 4 g + e of
  // query row mw + 16 qq + r16; running max (log2 units) and denominator per
  // lane's row (the denominator summed over the lane's keys only: the four
  // lanes of a row are added at the end).
  f32x4_t acc[8][2];
#pragma unroll
  for (int db = 0; db < 8; ++db)
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) acc[db][qq] = f32x4_t{0, 0, 0, 0};
  float m_run[2] = {NEG_BIG_P, NEG_BIG_P}, l_run[2] = {0.0f, 0.0f};
  int lim[2];
#pragma unroll
  for (int qq = 0; qq < 2; ++qq) lim[qq] = min(L, shift + mw + 16 * qq + r16);

  if (ntiles > 0) issue(0, 0);
  for (int kt = 0; kt < ntiles; ++kt) {
    const int buf = kt & 1;
    // tile kt landed (this wave's loads, then everyone's), and every wave is
    // done with the other buffer (tile kt - 1)
    stage_barrier<0>();
    if (kt + 1 < ntiles) issue(kt + 1, buf ^ 1);
    const int blk = tile_block(kt);
    if (blk < 0 || blk >= num_blocks) continue;
    const char* tb = smem + buf * BUF;
    const int key0 = kt * KT;
    // S^T[key][row]: s[a][qq] lane (g, r16) holds keys
    // key0 + 32 (a >> 1) + 8 g + 4 (a & 1) + i
    f32x4_t s[4][2];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int qq = 0; qq < 2; ++qq) s[a][qq] = f32x4_t{0, 0, 0, 0};
#pragma unroll
    for (int ks = 0; ks < 6; ++ks) {
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int r = 32 * (a >> 1) + 8 * (r16 >> 2) + 4 * (a & 1) + (r16 & 3);
        const char* kp = ks < 4 ? tb + OFF_KC + r * (D_H * 2) + (((4 * ks + g) ^ kswz(r)) * 16)
                                : tb + OFF_KR + r * (D_R * 2) + (((4 * (ks - 4) + g) ^ kswz(r)) * 16);
        const i16x8_t kf = *reinterpret_cast<const i16x8_t*>(kp);
#pragma unroll
        for (int qq = 0; qq < 2; ++qq)
          s[a][qq] = __builtin_amdgcn_mfma_f32_16x16x32_bf16((bf16x8_t)kf, (bf16x8_t)q[qq][ks],
                                                             s[a][qq], 0, 0, 0);
      }
    }
    // online softmax per query row (the running max moves with every larger
    // score: the key that sets it then gets P = 1 exactly; a lazier max,
    // moved only past a threshold, measurably raised the largest bf16 error).
    // P (bf16) for the PV product: keys 32 ks2 + 8 g .. + 7 of k-step ks2.
    i16x8_t pf[2][2];
    // the wave's first row sees the fewest keys: if it sees the whole tile,
    // every row does and the tile needs no mask
    const bool full = key0 + KT <= min(L, shift + mw);
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) {
      float tmax = -INFINITY;
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = key0 + 32 * (a >> 1) + 8 * g + 4 * (a & 1) + i;
          const float v = full || key < lim[qq] ? s[a][qq][i] * scale_log2 : -INFINITY;
          s[a][qq][i] = v;
          tmax = fmaxf(tmax, v);
        }
      tmax = group4_max(tmax);
      const float m_new = fmaxf(m_run[qq], tmax);
      float psum = 0.0f;
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint16_t pb = f32_to_bf16(fast_exp2(s[a][qq][i] - m_new));
          psum += bf16_to_f32(pb);
          pf[qq][a >> 1][4 * (a & 1) + i] = (short)pb;
        }
      // rescale only when some row of the wave has a new maximum (otherwise
      // every factor is exactly 1)
      if (__any(m_new > m_run[qq])) {
        const float alpha = fast_exp2(m_run[qq] - m_new);
        l_run[qq] *= alpha;
#pragma unroll
        for (int db = 0; db < 8; ++db)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[db][qq][e] *= alpha;
      }
      m_run[qq] = m_new;
      l_run[qq] += psum;
    }
    // O^T[d][row] += (v^T hi + v^T lo)[d][keys] P[row][keys]
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2) {
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const int vo = (16 * db + r16) * (KT * 2) + (((4 * ks2 + g) ^ (r16 & 7)) * 16);
#pragma unroll
        for (int part = 0; part < 2; ++part) {
          const i16x8_t vf = *reinterpret_cast<const i16x8_t*>(tb + (part ? OFF_VL : OFF_VH) + vo);
#pragma unroll
          for (int qq = 0; qq < 2; ++qq)
            acc[db][qq] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                (bf16x8_t)vf, (bf16x8_t)pf[qq][ks2], acc[db][qq], 0, 0, 0);
        }
      }
    }
  }

#pragma unroll
  for (int qq = 0; qq < 2; ++qq) {
    const float l = group4_sum(l_run[qq]);
    const int m = mw + 16 * qq + r16;
    if (m >= q_len) continue;
    const long row = (long)(row0 + m) * n_h + h;
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
#pragma unroll
    for (int db = 0; db < 8; ++db)
      *reinterpret_cast<float4*>(out + row * D_H + 16 * db + 4 * g) =
          float4{acc[db][qq][0] * inv, acc[db][qq][1] * inv, acc[db][qq][2] * inv,
                 acc[db][qq][3] * inv};
    if (g == 0) lse[row] = l > 0.0f ? (m_run[qq] + __log2f(l)) * 0.69314718055994531f : -INFINITY;
  }
}

}  // namespace

long prefill_mha_workspace(int max_len, int n_h) {
  const long lpad = std::max(256L, ((long)max_len + 255) / 256 * 256);
  return 3L * n_h * D_H * lpad * 2;   // k^C, v^C^T hi, v^C^T lo
}

hipError_t launch_prefill_mha(const void* q_nope, const void* q_rope, const int* q_pos,
                              const void* w_uk, const void* w_uv, const void* cache,
                              int num_blocks, const int* table, int max_blocks,
                              const int* seq_lens, int B, int q_len, int n_h, float scale,
                              const RopeFreq& rf, float* out, float* lse, void* workspace,
                              hipStream_t stream) {
  const auto* cache16 = static_cast<const uint16_t*>(cache);
  for (int b = 0; b < B; ++b) {
    const int L = seq_lens[b];
    const int lpad = std::max(256, (L + 255) / 256 * 256);   // whole 256-key tiles
    auto* kc = static_cast<uint16_t*>(workspace);
    uint16_t* vt = kc + (long)n_h * D_H * lpad;
    const int* trow = table + (long)b * max_blocks;
    if (L > 0) {
      // 256-key tiles: the 512-long reduction makes these projections bound
      // by re-reading tiles into LDS; 256 keys per tile halve the weight
      // re-reads of 64-key tiles
      const XSrc x{cache16, ROW, trow, num_blocks};
      proj_bf16<OUT_HEADS>(x, L, D_C, D_C,
                           ProjOut{static_cast<const uint16_t*>(w_uk), n_h * D_H, kc, D_H, 0,
                                   (long)lpad * D_H},
                           ProjOut{nullptr, 0, nullptr, 0, 0, 0}, stream, 256);
      proj_bf16<OUT_HEADS_T>(x, L, D_C, D_C,
                             ProjOut{static_cast<const uint16_t*>(w_uv), n_h * D_H, vt, lpad, 0,
                                     (long)D_H * lpad, (long)n_h * D_H * lpad},
                             ProjOut{nullptr, 0, nullptr, 0, 0, 0}, stream, 256);
    }
    if (q_len == 0) continue;
    hipLaunchKernelGGL(mha_prefill_kernel, dim3((q_len + QB - 1) / QB, n_h), dim3(64 * NW), 0,
                       stream,
                       static_cast<const uint16_t*>(q_nope), static_cast<const uint16_t*>(q_rope),
                       q_pos, kc, vt, cache16, num_blocks, trow, L, q_len, lpad, n_h, b * q_len,
                       scale * 1.4426950408889634f, rf, out, lse);
  }
  return hipGetLastError();
}

}  // namespace mla
