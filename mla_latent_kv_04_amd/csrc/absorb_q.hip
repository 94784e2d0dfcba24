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
#include "mla_common.h"
#include "mla_internal.h"

namespace mla {

namespace {

constexpr int CCH = 64;        // latent columns per workgroup
constexpr int TCH = 128;       // rows per workgroup (4 waves x 2 blocks of 16)

template <class E> struct AbsorbLds;
template <> struct AbsorbLds<BF16> { static constexpr int stride = 160; };  // bytes per d row
template <> struct AbsorbLds<F32> { static constexpr int stride = 272; };

template <class E>
__device__ __forceinline__ typename E::frag load_wt_frag(const char* lds, int d0, int c_local);

// bf16: two transposing reads give this lane W[d0 + 0..3][c] and W[d0 + 4..7][c],
// c = c_local (lane % 16 inside the 16-column block starting at c_local - lane%16).
template <>
__device__ __forceinline__ BF16::frag load_wt_frag<BF16>(const char* lds, int d0, int cblk) {
  constexpr int S = AbsorbLds<BF16>::stride;
  const int s = lane_id() & 15;
  const char* p = lds + (d0 + (s >> 2)) * S + (cblk + 4 * (s & 3)) * 2;
  i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p));
  i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p + 4 * S));
  BF16::frag f;
  f.v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return f;
}

template <>
__device__ __forceinline__ F32::frag load_wt_frag<F32>(const char* lds, int d0, int cblk) {
  constexpr int S = AbsorbLds<F32>::stride;
  const int c = cblk + (lane_id() & 15);
  F32::frag f;
#pragma unroll
  for (int j = 0; j < 8; ++j) f.v[j] = *reinterpret_cast<const float*>(lds + (d0 + j) * S + c * 4);
  return f;
}

template <class E>
__global__ void __launch_bounds__(256) absorb_q_kernel(
    const typename E::storage* __restrict__ q_nope, const typename E::storage* __restrict__ q_rope,
    const typename E::storage* __restrict__ w_uk, const int* __restrict__ q_pos, int T, int n_h,
    double base, typename E::storage* __restrict__ q_lat) {
  using T_ = typename E::storage;
  constexpr int S = AbsorbLds<E>::stride;
  __shared__ __attribute__((aligned(16))) char lds[D_H * S];
  const int h = blockIdx.x;
  const int c0 = blockIdx.y * CCH;
  const int t0 = blockIdx.z * TCH;
  const int lane = lane_id(), wave = threadIdx.x >> 6, g = lane >> 4, r16 = lane & 15;

  // Stage W^UK_h[0:128, c0:c0+64] (16-byte pieces).
  constexpr int PER16 = 16 / E::bytes;
  constexpr int PIECES_PER_ROW = CCH / PER16;
  const T_* wsrc = w_uk + (long)h * D_H * D_C + c0;
  for (int p = threadIdx.x; p < D_H * PIECES_PER_ROW; p += 256) {
    const int d = p / PIECES_PER_ROW, q = p % PIECES_PER_ROW;
    *reinterpret_cast<uint4*>(lds + d * S + q * 16) =
        *reinterpret_cast<const uint4*>(wsrc + (long)d * D_C + q * PER16);
  }
  __syncthreads();

  // Query fragments (B operand): lane holds row t = tb*16 + r16, d = ks*32 + 8g + j.
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
#pragma unroll
  for (int cb = 0; cb < CCH / 16; ++cb) {
    f32x4_t acc[2] = {{0, 0, 0, 0}, {0, 0, 0, 0}};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      typename E::frag wf = load_wt_frag<E>(lds, ks * 32 + 8 * g, cb * 16);
      E::mma(acc[0], wf, qf[0][ks]);
      E::mma(acc[1], wf, qf[1][ks]);
    }
    // D[c][t]: lane holds t = r16 (+16 tb), c = cb*16 + 4g + i.
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      const int t = t0 + wave * 32 + tb * 16 + r16;
      if (t < T) {
        T_* dst = q_lat + ((long)t * n_h + h) * ROW + c0 + cb * 16 + 4 * g;
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[i] = E::from_f32(acc[tb][i]);
      }
    }
  }

  // Decoupled RoPE query, written once per (row, head) by the first column chunk.
  if (blockIdx.y == 0) {
    for (int e = threadIdx.x; e < TCH * (D_R / 2); e += 256) {
      const int t = t0 + e / (D_R / 2), k = e % (D_R / 2);
      if (t >= T) break;
      double c, s;
      rope_cs(q_pos[t], k, base, c, s);
      const T_* src = q_rope + ((long)t * n_h + h) * D_R;
      double x = E::to_f32(src[2 * k]), y = E::to_f32(src[2 * k + 1]);
      T_* dst = q_lat + ((long)t * n_h + h) * ROW + D_C;
      dst[2 * k] = E::from_f32((float)(x * c - y * s));
      dst[2 * k + 1] = E::from_f32((float)(x * s + y * c));
    }
  }
}

}  // namespace

hipError_t launch_absorb_q(const void* q_nope, const void* q_rope, const void* w_uk,
                           const int* q_pos, int T, int n_h, int dtype, float base, void* q_lat,
                           hipStream_t stream) {
  dim3 grid(n_h, D_C / CCH, (T + TCH - 1) / TCH), block(256);
  if (dtype == 1)
    hipLaunchKernelGGL(absorb_q_kernel<BF16>, grid, block, 0, stream, (const uint16_t*)q_nope,
                       (const uint16_t*)q_rope, (const uint16_t*)w_uk, q_pos, T, n_h,
                       (double)base, (uint16_t*)q_lat);
  else
    hipLaunchKernelGGL(absorb_q_kernel<F32>, grid, block, 0, stream, (const float*)q_nope,
                       (const float*)q_rope, (const float*)w_uk, q_pos, T, n_h, (double)base,
                       (float*)q_lat);
  return hipGetLastError();
}

}  // namespace mla
