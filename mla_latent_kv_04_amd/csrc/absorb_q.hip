// Absorbed query: q_lat[t, i] = [ W^UK_i^T q_nope[t, i] ; R_{q_pos[t]} q_rope[t, i] ].
//
// W^UK folds into the query side because q . (W^UK c) = (W^UK^T q) . c
// (DeepSeek-V2 MLA blog, adg.csdn.net, part 2 §2.2.1.1 / §2.2.2; eq. 10 of
// the irregular6612.github.io DeepSeek-V2 notes, §2.1.2).
//
// Per head i this is the GEMM q_lat^T[c, t] = sum_d W^UK_i[d, c] q_nope[t, i, d]
// with M = 512 (latent c), N = T (rows), K = 128 (d).  One workgroup of four
// waves owns one head, 64 latent columns and 128 rows; the 128 x 64 weight
// tile is staged in LDS once and read as the MFMA A operand (rows c, reduced
// d) with the transposing LDS read, since W^UK is stored with c contiguous.
// The query fragments (reduced d contiguous) come straight from memory.
//
// The A rows of the four 16-column MFMA blocks are permuted so that the
// output lands row-contiguous: block cb's row m is latent column
// 16 (m >> 2) + 4 cb + (m & 3), so after the four blocks a lane holds 16
// consecutive columns of one query row and writes them with full-width
// stores (four lanes cover a row's 64 columns).  The RoPE half of q_lat is
// shared out over the eight column-chunk workgroups of a head, 4 of the 32
// rotation pairs each.
#include <cmath>

#include "mla_common.h"
#include "mla_internal.h"

namespace mla {

namespace {

constexpr int CCH = 64;        // latent columns per workgroup

// RoPE frequencies in revolutions per position, theta_k / (2 pi), computed
// on the host in float64 from the pair frequencies theta_k.
struct RopeRev {
  double r[D_R / 2];
};
constexpr int TCH = 128;       // rows per workgroup (4 waves x 2 blocks of 16)
constexpr int KPW = (D_R / 2) / (D_C / CCH);   // RoPE pairs per workgroup

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

template <class E>
__global__ void __launch_bounds__(256) absorb_q_kernel(
    const typename E::storage* __restrict__ q_nope, const typename E::storage* __restrict__ q_rope,
    const typename E::storage* __restrict__ w_uk, const int* __restrict__ q_pos, int T, int n_h,
    RopeFreq rf, RopeRev rev, typename E::storage* __restrict__ q_lat) {
  using T_ = typename E::storage;
  constexpr int S = AbsorbLds<E>::stride;
  __shared__ __attribute__((aligned(16))) char lds[D_H * S];
  const int h = blockIdx.x;
  const int c0 = blockIdx.y * CCH;
  const int t0 = blockIdx.z * TCH;
  const int lane = lane_id(), wave = threadIdx.x >> 6, g = lane >> 4, r16 = lane & 15;

  // Query fragments (B operand): lane holds row t = tb*16 + r16, d = ks*32 + 8g + j
  // (issued first, so that they land while the weight tile is staged).
  typename E::frag qf[2][4];
#pragma unroll
  for (int tb = 0; tb < 2; ++tb) {
    const int t = t0 + wave * 32 + tb * 16 + r16;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if (t < T) {
        qf[tb][ks] = E::load8(q_nope + ((long)t * n_h + h) * D_H + ks * 32 + 8 * g);
      } else {
        float z[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        qf[tb][ks] = E::from8(z);
      }
    }
  }
  // bf16 RoPE inputs (two rotation pairs per thread), loaded with the
  // fragments and rotated after the product, so their latency is hidden
  constexpr int RPT = TCH * KPW / 256;
  static_assert(TCH * KPW % 256 == 0, "rotation pairs split evenly");
  uint32_t rp[RPT];
  int rpos[RPT];
  if constexpr (E::bytes == 2) {
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int e = threadIdx.x + 256 * i;
      const int t = t0 + e / KPW, k = blockIdx.y * KPW + e % KPW;
      rp[i] = 0;
      rpos[i] = 0;
      if (t < T) {
        rp[i] = *reinterpret_cast<const uint32_t*>(q_rope + ((long)t * n_h + h) * D_R + 2 * k);
        rpos[i] = q_pos[t];
      }
    }
  }
  // Stage W^UK_h[0:128, c0:c0+64] (16-byte pieces, written as two halves:
  // the bf16 row pitch is a multiple of 8 bytes only).
  constexpr int PER16 = 16 / E::bytes;
  constexpr int PIECES_PER_ROW = CCH / PER16;
  const T_* wsrc = w_uk + (long)h * D_H * D_C + c0;
  constexpr int NP = D_H * PIECES_PER_ROW / 256;   // pieces per thread
  static_assert(D_H * PIECES_PER_ROW % 256 == 0, "pieces split evenly");
  uint4 wv[NP];
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int p = i * 256 + threadIdx.x, d = p / PIECES_PER_ROW, q = p % PIECES_PER_ROW;
    wv[i] = *reinterpret_cast<const uint4*>(wsrc + (long)d * D_C + q * PER16);
  }

  // Decoupled RoPE query, this column chunk's 4 of the 32 rotation pairs.
  if constexpr (E::bytes == 4) {
    // fp32: float64 angles and rotation (runs while the loads above are in flight)
    for (int e = threadIdx.x; e < TCH * KPW; e += 256) {
      const int t = t0 + e / KPW, k = blockIdx.y * KPW + e % KPW;
      if (t >= T) break;
      const T_* src = q_rope + ((long)t * n_h + h) * D_R;
      T_* dst = q_lat + ((long)t * n_h + h) * ROW + D_C;
      double c, s;
      rope_cs(q_pos[t], rf.theta[k], c, s);
      double x = E::to_f32(src[2 * k]), y = E::to_f32(src[2 * k + 1]);
      dst[2 * k] = E::from_f32((float)(x * c - y * s));
      dst[2 * k + 1] = E::from_f32((float)(x * s + y * c));
    }
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
      typename E::frag wf = load_wt_frag<E>(lds, ks * 32 + 8 * g, cb);
      E::mma(acc[0][cb], wf, qf[0][ks]);
      E::mma(acc[1][cb], wf, qf[1][ks]);
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
      store16<E>(q_lat + ((long)t * n_h + h) * ROW + c0 + 16 * g, v);
    }
  }
  if constexpr (E::bytes == 2) {
    // the angle is reduced exactly in float64 (whole turns dropped), then sine
    // and cosine in float32, far below bf16's rounding
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int e = threadIdx.x + 256 * i;
      const int t = t0 + e / KPW, k = blockIdx.y * KPW + e % KPW;
      if (t >= T) continue;
      double turns = (double)rpos[i] * rev.r[k];
      turns -= rint(turns);
      float sf, cf;
      sincosf((float)(turns * 6.283185307179586), &sf, &cf);
      const float x = bf16_to_f32((uint16_t)(rp[i] & 0xFFFFu)), y = bf16_to_f32((uint16_t)(rp[i] >> 16));
      *reinterpret_cast<uint32_t*>(q_lat + ((long)t * n_h + h) * ROW + D_C + 2 * k) =
          pack_bf16x2(x * cf - y * sf, x * sf + y * cf);
    }
  }

}

}  // namespace

hipError_t launch_absorb_q(const void* q_nope, const void* q_rope, const void* w_uk,
                           const int* q_pos, int T, int n_h, int dtype, const RopeFreq& rf,
                           void* q_lat, hipStream_t stream) {
  dim3 grid(n_h, D_C / CCH, (T + TCH - 1) / TCH), block(256);
  RopeRev rev;
  for (int k = 0; k < D_R / 2; ++k)
    rev.r[k] = rf.theta[k] / 6.283185307179586;
  if (dtype == 1)
    hipLaunchKernelGGL(absorb_q_kernel<BF16>, grid, block, 0, stream, (const uint16_t*)q_nope,
                       (const uint16_t*)q_rope, (const uint16_t*)w_uk, q_pos, T, n_h,
                       rf, rev, (uint16_t*)q_lat);
  else
    hipLaunchKernelGGL(absorb_q_kernel<F32>, grid, block, 0, stream, (const float*)q_nope,
                       (const float*)q_rope, (const float*)w_uk, q_pos, T, n_h, rf, rev,
                       (float*)q_lat);
  return hipGetLastError();
}

}  // namespace mla
