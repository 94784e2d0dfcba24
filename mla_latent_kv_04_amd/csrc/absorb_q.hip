// Absorbed query: q_lat[t, i] = [ W^UK_i^T q_nope[t, i] ; R_{q_pos[t]} q_rope[t, i] ].
//
// W^UK folds into the query side because q . (W^UK c) = (W^UK^T q) . c
// (DeepSeek-V2 MLA blog, adg.csdn.net, part 2 §2.2.1.1 / §2.2.2; eq. 10 of
// the irregular6612.github.io DeepSeek-V2 notes, §2.1.2).
//
// Per head i this is the GEMM q_lat^T[c, t] = sum_d W^UK_i[d, c] q_nope[t, i, d]
// with M = 512 (latent c), N = T (rows), K = 128 (d).  A workgroup of four
// waves multiplies 128 rows of one head against 64-column tiles of the
// weight: each 128 x 64 tile is staged in LDS and read as the MFMA A operand
// (rows c, reduced d) with the transposing LDS read, since W^UK is stored with
// c contiguous.  The query fragments (reduced d contiguous) come straight from
// memory into registers.
//
// The A rows of the four 16-column MFMA blocks are permuted so that the
// output lands row-contiguous: block cb's row m is latent column
// 16 (m >> 2) + 4 cb + (m & 3), so after the four blocks a lane holds 16
// consecutive columns of one query row and writes them with full-width
// stores (four lanes cover a row's 64 columns).
//
// bf16 (the decode and prefill path): a workgroup owns CPW consecutive tiles
// of its head.  It loads the query fragments once for all of them and
// streams the tiles through two LDS buffers, with the next tiles already in
// flight in registers while one is multiplied and stored, so each
// workgroup's stores overlap its next loads; CPW grows with the number of
// (head, 128-row) units, from 1 for a few heads to 4 for long prefill
// chunks (where it cuts the query re-reads fourfold).  The RoPE half goes by
// whole rows: each workgroup rotates all 32 pairs of its share of the rows,
// so every 128-byte RoPE section is read and written by one workgroup.
// fp32 (the reference-precision path): one tile per workgroup, RoPE in
// float64, 4 of the 32 pairs per column tile.
#include <cmath>

#include "append_row.h"
#include "mla_common.h"
#include "mla_internal.h"

namespace mla {

namespace {

constexpr int CCH = 64;        // latent columns per weight tile

// RoPE frequencies in revolutions per position, theta_k / (2 pi), computed
// on the host in float64 from the pair frequencies theta_k.
struct RopeRev {
  double r[D_R / 2];
};
constexpr int TCH = 128;       // rows per workgroup (4 waves x 2 blocks of 16)
constexpr int KPW = (D_R / 2) / (D_C / CCH);   // RoPE pairs per fp32 workgroup

template <class E> struct AbsorbLds;
// bf16: a 136-byte row pitch puts the four rows of a transposing read on
// disjoint banks for the permuted column pattern (staged with 8-byte writes)
template <> struct AbsorbLds<BF16> { static constexpr int stride = 136; };  // bytes per d row
template <> struct AbsorbLds<F32> { static constexpr int stride = 272; };

template <class E>
__device__ __forceinline__ typename E::frag load_wt_frag(const char* lds, int d0, int c_local);

// Column of the tile that A row m of column block cb stands for.
__device__ __forceinline__ int perm_col(int m, int cb) { return 16 * (m >> 2) + 4 * cb + (m & 3); }

// bf16: two transposing reads give this lane (A row m = lane % 16)
// W[d0 + 0..3][perm_col(m, cb)] and W[d0 + 4..7][perm_col(m, cb)]: the lane
// that supplies columns 16 (s & 3) + 4 cb .. +3 of row d0 + (s >> 2) feeds
// rows m with m >> 2 == s & 3.
template <>
__device__ __forceinline__ BF16::frag load_wt_frag<BF16>(const char* lds, int d0, int cb) {
  constexpr int S = AbsorbLds<BF16>::stride;
  const int s = lane_id() & 15;
  const char* p = lds + (d0 + (s >> 2)) * S + (16 * (s & 3) + 4 * cb) * 2;
  i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p));
  i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p + 4 * S));
  BF16::frag f;
  f.v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return f;
}

template <>
__device__ __forceinline__ F32::frag load_wt_frag<F32>(const char* lds, int d0, int cb) {
  constexpr int S = AbsorbLds<F32>::stride;
  const int c = perm_col(lane_id() & 15, cb);
  F32::frag f;
#pragma unroll
  for (int j = 0; j < 8; ++j) f.v[j] = *reinterpret_cast<const float*>(lds + (d0 + j) * S + c * 4);
  return f;
}

// 16 consecutive outputs of one row, 16-byte aligned.
template <class E>
__device__ __forceinline__ void store16(typename E::storage* dst, const float (&v)[16]);
template <>
__device__ __forceinline__ void store16<BF16>(uint16_t* dst, const float (&v)[16]) {
  uint4* d = reinterpret_cast<uint4*>(dst);
  d[0] = uint4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
               pack_bf16x2(v[6], v[7])};
  d[1] = uint4{pack_bf16x2(v[8], v[9]), pack_bf16x2(v[10], v[11]), pack_bf16x2(v[12], v[13]),
               pack_bf16x2(v[14], v[15])};
}
template <>
__device__ __forceinline__ void store16<F32>(float* dst, const float (&v)[16]) {
  float4* d = reinterpret_cast<float4*>(dst);
#pragma unroll
  for (int i = 0; i < 4; ++i) d[i] = float4{v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]};
}

__global__ void __launch_bounds__(256) absorb_q_f32_kernel(
    const float* __restrict__ q_nope, const float* __restrict__ q_rope,
    const float* __restrict__ w_uk, const int* __restrict__ q_pos, int T, int n_h, RopeFreq rf,
    float* __restrict__ q_lat) {
  constexpr int S = AbsorbLds<F32>::stride;
  __shared__ __attribute__((aligned(16))) char lds[D_H * S];
  const int h = blockIdx.x;
  const int c0 = blockIdx.y * CCH;
  const int t0 = blockIdx.z * TCH;
  const int lane = lane_id(), wave = threadIdx.x >> 6, g = lane >> 4, r16 = lane & 15;

  // Query fragments (B operand): lane holds row t = tb*16 + r16, d = ks*32 + 8g + j
  // (issued first, so that they land while the weight tile is staged).
  F32::frag qf[2][4];
#pragma unroll
  for (int tb = 0; tb < 2; ++tb) {
    const int t = t0 + wave * 32 + tb * 16 + r16;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if (t < T) {
        qf[tb][ks] = F32::load8(q_nope + ((long)t * n_h + h) * D_H + ks * 32 + 8 * g);
      } else {
        float z[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        qf[tb][ks] = F32::from8(z);
      }
    }
  }
  // Stage W^UK_h[0:128, c0:c0+64] (16-byte pieces).
  constexpr int PIECES_PER_ROW = CCH / 4;
  const float* wsrc = w_uk + (long)h * D_H * D_C + c0;
  constexpr int NP = D_H * PIECES_PER_ROW / 256;   // pieces per thread
  static_assert(D_H * PIECES_PER_ROW % 256 == 0, "pieces split evenly");
  uint4 wv[NP];
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int p = i * 256 + threadIdx.x, d = p / PIECES_PER_ROW, q = p % PIECES_PER_ROW;
    wv[i] = *reinterpret_cast<const uint4*>(wsrc + (long)d * D_C + q * 4);
  }

  // Decoupled RoPE query, this column chunk's 4 of the 32 rotation pairs:
  // float64 angles and rotation (runs while the loads above are in flight).
  for (int e = threadIdx.x; e < TCH * KPW; e += 256) {
    const int t = t0 + e / KPW, k = blockIdx.y * KPW + e % KPW;
    if (t >= T) break;
    const float* src = q_rope + ((long)t * n_h + h) * D_R;
    float* dst = q_lat + ((long)t * n_h + h) * ROW + D_C;
    double c, s;
    rope_cs(q_pos[t], rf.theta[k], c, s);
    const double x = src[2 * k], y = src[2 * k + 1];
    dst[2 * k] = (float)(x * c - y * s);
    dst[2 * k + 1] = (float)(x * s + y * c);
  }

#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int p = i * 256 + threadIdx.x, d = p / PIECES_PER_ROW, q = p % PIECES_PER_ROW;
    uint2* dst = reinterpret_cast<uint2*>(lds + d * S + q * 16);
    dst[0] = uint2{wv[i].x, wv[i].y};
    dst[1] = uint2{wv[i].z, wv[i].w};
  }
  __syncthreads();

  f32x4_t acc[2][CCH / 16];
#pragma unroll
  for (int cb = 0; cb < CCH / 16; ++cb) {
    acc[0][cb] = f32x4_t{0, 0, 0, 0};
    acc[1][cb] = f32x4_t{0, 0, 0, 0};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const F32::frag wf = load_wt_frag<F32>(lds, ks * 32 + 8 * g, cb);
      F32::mma(acc[0][cb], wf, qf[0][ks]);
      F32::mma(acc[1][cb], wf, qf[1][ks]);
    }
  }
  // D[m][t] of block cb: lane holds t = r16 (+16 tb) and m = 4g + i, i.e.
  // column perm_col(4g + i, cb) = 16g + 4cb + i: columns 16g .. 16g + 15.
#pragma unroll
  for (int tb = 0; tb < 2; ++tb) {
    const int t = t0 + wave * 32 + tb * 16 + r16;
    if (t < T) {
      float v[16];
#pragma unroll
      for (int cb = 0; cb < CCH / 16; ++cb)
#pragma unroll
        for (int i = 0; i < 4; ++i) v[4 * cb + i] = acc[tb][cb][i];
      store16<F32>(q_lat + ((long)t * n_h + h) * ROW + c0 + 16 * g, v);
    }
  }
}

// bf16: workgroup (h, gy, z) owns the CPW consecutive 64-column tiles of
// head h that start at column 64 CPW gy, for rows 128 z .. 128 z + 127, and
// the RoPE part of rows 128 z + RROWS gy .. + RROWS - 1 (RROWS = 16 CPW).
// Tile c + PF is loaded into registers while tile c is multiplied; the LDS
// holds two tiles.
template <int CPW, int PF>
__device__ __forceinline__ void absorb_bf16_group(
    int h, int gy, int z, const uint16_t* __restrict__ q_nope, const uint16_t* __restrict__ q_rope,
    const uint16_t* __restrict__ w_uk, const int* __restrict__ q_pos, int T, int n_h,
    const RopeRev& rev, uint16_t* __restrict__ q_lat) {
  constexpr int S = AbsorbLds<BF16>::stride;
  constexpr int NG = (D_C / CCH) / CPW;   // column groups per head
  __shared__ __attribute__((aligned(16))) char lds[2][D_H * S];
  constexpr int TBW = TCH / 64;           // 16-row blocks per wave
  const int t0 = z * TCH;
  const int tid = threadIdx.x;
  const int lane = lane_id(), wave = tid >> 6, g = lane >> 4, r16 = lane & 15;

  // query fragments (B operand): row t = t0 + 32 wave + 16 tb + r16, d = 32 ks + 8 g + j
  BF16::frag qf[TBW][4];
#pragma unroll
  for (int tb = 0; tb < TBW; ++tb) {
    const int t = t0 + wave * 16 * TBW + tb * 16 + r16;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if (t < T) {
        qf[tb][ks] = BF16::load8(q_nope + ((long)t * n_h + h) * D_H + ks * 32 + 8 * g);
      } else {
        float z[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        qf[tb][ks] = BF16::from8(z);
      }
    }
  }
  // RoPE inputs: rows t0 + RROWS gy + 16 i + (tid >> 4), pairs 2 (tid & 15) and + 1
  constexpr int RROWS = TCH / NG, RPASS = RROWS / 16;
  static_assert(RROWS % 16 == 0, "RoPE rows split evenly");
  const int rk = 2 * (tid & 15);
  uint2 rp[RPASS];
  int rpos[RPASS];
#pragma unroll
  for (int i = 0; i < RPASS; ++i) {
    const int t = t0 + RROWS * gy + 16 * i + (tid >> 4);
    rp[i] = uint2{0, 0};
    rpos[i] = 0;
    if (t < T) {
      rp[i] = *reinterpret_cast<const uint2*>(q_rope + ((long)t * n_h + h) * D_R + 2 * rk);
      rpos[i] = q_pos[t];
    }
  }
  // weight tile c: W^UK_h[0:128, 64 (CPW gy + c) ..], four 16-byte pieces per thread
  const uint16_t* wsrc = w_uk + (long)h * D_H * D_C + CPW * gy * CCH;
  auto load_w = [&](int c, uint4 (&wv)[4]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int p = i * 256 + tid, d = p >> 3, q = p & 7;
      wv[i] = *reinterpret_cast<const uint4*>(wsrc + (long)d * D_C + c * CCH + q * 8);
    }
  };
  auto stage_w = [&](char* buf, const uint4 (&wv)[4]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int p = i * 256 + tid, d = p >> 3, q = p & 7;
      uint2* dst = reinterpret_cast<uint2*>(buf + d * S + q * 16);
      dst[0] = uint2{wv[i].x, wv[i].y};
      dst[1] = uint2{wv[i].z, wv[i].w};
    }
  };
  uint4 wv[PF][4];
#pragma unroll
  for (int c = 0; c < PF && c < CPW; ++c) load_w(c, wv[c]);

#pragma unroll
  for (int c = 0; c < CPW; ++c) {
    char* buf = lds[c & 1];
    stage_w(buf, wv[c % PF]);
    if (c + PF < CPW) load_w(c + PF, wv[c % PF]);
    __syncthreads();
    f32x4_t acc[TBW][CCH / 16];
#pragma unroll
    for (int cb = 0; cb < CCH / 16; ++cb) {
#pragma unroll
      for (int tb = 0; tb < TBW; ++tb) acc[tb][cb] = f32x4_t{0, 0, 0, 0};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const BF16::frag wf = load_wt_frag<BF16>(buf, ks * 32 + 8 * g, cb);
#pragma unroll
        for (int tb = 0; tb < TBW; ++tb) BF16::mma(acc[tb][cb], wf, qf[tb][ks]);
      }
    }
    // lane holds row t = ... + r16 and columns 16 g .. 16 g + 15 of the chunk
#pragma unroll
    for (int tb = 0; tb < TBW; ++tb) {
      const int t = t0 + wave * 16 * TBW + tb * 16 + r16;
      if (t < T) {
        float v[16];
#pragma unroll
        for (int cb = 0; cb < CCH / 16; ++cb)
#pragma unroll
          for (int i = 0; i < 4; ++i) v[4 * cb + i] = acc[tb][cb][i];
        store16<BF16>(q_lat + ((long)t * n_h + h) * ROW + (CPW * gy + c) * CCH + 16 * g, v);
      }
    }
  }
  // the angle is reduced exactly in float64 (whole turns dropped), then sine
  // and cosine in float32, far below bf16's rounding
#pragma unroll
  for (int i = 0; i < RPASS; ++i) {
    const int t = t0 + RROWS * gy + 16 * i + (tid >> 4);
    if (t >= T) continue;
    uint32_t out[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      double turns = (double)rpos[i] * rev.r[rk + j];
      turns -= rint(turns);
      float sf, cf;
      sincosf((float)(turns * 6.283185307179586), &sf, &cf);
      const uint32_t w = j == 0 ? rp[i].x : rp[i].y;
      const float x = bf16_to_f32((uint16_t)(w & 0xFFFFu)), y = bf16_to_f32((uint16_t)(w >> 16));
      out[j] = pack_bf16x2(x * cf - y * sf, x * sf + y * cf);
    }
    *reinterpret_cast<uint2*>(q_lat + ((long)t * n_h + h) * ROW + D_C + 2 * rk) = uint2{out[0], out[1]};
  }
}

template <int CPW, int PF>
__global__ void __launch_bounds__(256) absorb_q_bf16_kernel(
    const uint16_t* __restrict__ q_nope, const uint16_t* __restrict__ q_rope,
    const uint16_t* __restrict__ w_uk, const int* __restrict__ q_pos, int T, int n_h, RopeRev rev,
    uint16_t* __restrict__ q_lat) {
  absorb_bf16_group<CPW, PF>(blockIdx.x, blockIdx.y, blockIdx.z, q_nope, q_rope, w_uk, q_pos, T,
                             n_h, rev, q_lat);
}

// The step's append and absorb in one launch (bf16): workgroups 0 .. n_app-1
// append four cache rows each (one per wave), the others are the absorb's
// (h, gy, z) workgroups in the order of the plain launch's grid.  The two
// parts share no data; one launch saves a kernel boundary, and the append's
// short dependent loads run beside the absorb.
template <int CPW, int PF>
__global__ void __launch_bounds__(256) append_absorb_bf16_kernel(
    const uint16_t* __restrict__ q_nope, const uint16_t* __restrict__ q_rope,
    const uint16_t* __restrict__ w_uk, const int* __restrict__ q_pos, int T, int n_h, RopeRev rev,
    uint16_t* __restrict__ q_lat, int n_app, uint16_t* __restrict__ cache, int num_blocks,
    const int* __restrict__ table, int num_seqs, int max_blocks, const uint16_t* __restrict__ c_kv,
    const uint16_t* __restrict__ k_rope, const int* __restrict__ seq_idx,
    const int* __restrict__ pos, int n, RopeFreq rf) {
  const int wg = blockIdx.x;
  if (wg < n_app) {
    const int r = wg * 4 + (threadIdx.x >> 6);
    if (r < n)
      append_row<BF16>(cache, num_blocks, table, num_seqs, max_blocks, c_kv, k_rope, seq_idx, pos,
                       r, threadIdx.x & 63, rf);
    return;
  }
  constexpr int NG = (D_C / CCH) / CPW;
  const int a = wg - n_app;
  absorb_bf16_group<CPW, PF>(a % n_h, (a / n_h) % NG, a / (n_h * NG), q_nope, q_rope, w_uk, q_pos,
                             T, n_h, rev, q_lat);
}

// Tiles per workgroup by the number of (head, 128-row) units: measured on
// 16 x 64, 128 x 128 and 128 x 2048 (heads x rows), one tile per workgroup
// keeps a few heads spread over the chip; four, with three tiles in flight,
// suits long prefill chunks.  Returns CPW (PF follows from it).
int absorb_cpw(int n_h, int nz) {
  const int units = n_h * nz;
  return units >= 1024 ? 4 : units >= 64 ? 2 : 1;
}

RopeRev rope_rev(const RopeFreq& rf) {
  RopeRev rev;
  for (int k = 0; k < D_R / 2; ++k) rev.r[k] = rf.theta[k] / 6.283185307179586;
  return rev;
}

}  // namespace

hipError_t launch_absorb_q(const void* q_nope, const void* q_rope, const void* w_uk,
                           const int* q_pos, int T, int n_h, int dtype, const RopeFreq& rf,
                           void* q_lat, hipStream_t stream) {
  const int nz = (T + TCH - 1) / TCH;
  if (dtype != 1) {
    hipLaunchKernelGGL(absorb_q_f32_kernel, dim3(n_h, D_C / CCH, nz), dim3(256), 0, stream,
                       (const float*)q_nope, (const float*)q_rope, (const float*)w_uk, q_pos, T,
                       n_h, rf, (float*)q_lat);
    return hipGetLastError();
  }
  const RopeRev rev = rope_rev(rf);
  auto* q = (const uint16_t*)q_nope;
  auto* r = (const uint16_t*)q_rope;
  auto* w = (const uint16_t*)w_uk;
  auto* o = (uint16_t*)q_lat;
  const int cpw = absorb_cpw(n_h, nz);
  if (cpw == 4)
    hipLaunchKernelGGL((absorb_q_bf16_kernel<4, 3>), dim3(n_h, 2, nz), dim3(256), 0, stream, q, r,
                       w, q_pos, T, n_h, rev, o);
  else if (cpw == 2)
    hipLaunchKernelGGL((absorb_q_bf16_kernel<2, 2>), dim3(n_h, 4, nz), dim3(256), 0, stream, q, r,
                       w, q_pos, T, n_h, rev, o);
  else
    hipLaunchKernelGGL((absorb_q_bf16_kernel<1, 2>), dim3(n_h, 8, nz), dim3(256), 0, stream, q, r,
                       w, q_pos, T, n_h, rev, o);
  return hipGetLastError();
}

hipError_t launch_append_absorb(void* cache, int dtype, int num_blocks, const int* table,
                                int num_seqs, int max_blocks, const void* c_kv,
                                const void* k_rope, const int* seq_idx, const int* pos, int n,
                                const void* q_nope, const void* q_rope, const void* w_uk,
                                const int* q_pos, int T, int n_h, const RopeFreq& rf,
                                void* q_lat, hipStream_t stream) {
  if (dtype != 1) {
    // fp32: the two launches (the reference-precision path is not fused)
    if (n > 0) {
      const hipError_t e = launch_kv_append(cache, dtype, num_blocks, table, num_seqs,
                                            max_blocks, c_kv, k_rope, seq_idx, pos, n, rf,
                                            stream);
      if (e != hipSuccess) return e;
    }
    return T > 0 ? launch_absorb_q(q_nope, q_rope, w_uk, q_pos, T, n_h, dtype, rf, q_lat, stream)
                 : hipSuccess;
  }
  const int nz = (T + TCH - 1) / TCH;
  // append workgroups first (a multiple of 8, so that the absorb's
  // workgroups keep their XCDs), so that their dependent loads start first
  const int n_app = (n + 31) / 32 * 8;
  const int cpw = absorb_cpw(n_h, nz);
  const long n_abs = (long)n_h * (D_C / CCH / cpw) * nz;
  const long grid = n_app + n_abs;
  if (grid == 0) return hipSuccess;
  const RopeRev rev = rope_rev(rf);
  auto* q = (const uint16_t*)q_nope;
  auto* r = (const uint16_t*)q_rope;
  auto* w = (const uint16_t*)w_uk;
  auto* o = (uint16_t*)q_lat;
  auto* kc = (uint16_t*)cache;
  auto* cs = (const uint16_t*)c_kv;
  auto* kr = (const uint16_t*)k_rope;
  if (cpw == 4)
    hipLaunchKernelGGL((append_absorb_bf16_kernel<4, 3>), dim3((unsigned)grid), dim3(256), 0,
                       stream, q, r, w, q_pos, T, n_h, rev, o, n_app, kc, num_blocks, table,
                       num_seqs, max_blocks, cs, kr, seq_idx, pos, n, rf);
  else if (cpw == 2)
    hipLaunchKernelGGL((append_absorb_bf16_kernel<2, 2>), dim3((unsigned)grid), dim3(256), 0,
                       stream, q, r, w, q_pos, T, n_h, rev, o, n_app, kc, num_blocks, table,
                       num_seqs, max_blocks, cs, kr, seq_idx, pos, n, rf);
  else
    hipLaunchKernelGGL((append_absorb_bf16_kernel<1, 2>), dim3((unsigned)grid), dim3(256), 0,
                       stream, q, r, w, q_pos, T, n_h, rev, o, n_app, kc, num_blocks, table,
                       num_seqs, max_blocks, cs, kr, seq_idx, pos, n, rf);
  return hipGetLastError();
}

}  // namespace mla
