// Cache and query producers, the projections that feed the attention path,
// and eq. 8's output projection W^O, which ends an attention layer.
//
//   c^KV = RMSNorm(W^DKV h), k^R = W^KR h          (eq. 9 of the DeepSeek-V2
//   c^Q  = RMSNorm(W^DQ h),  q^C = W^UQ c^Q,        notes, irregular6612.github.io,
//   q^R  = W^QR c^Q                                 §2.1.2, eq. 12-13; the decoupled
//                                                   key / query of the DeepSeek-V2 MLA
//                                                   blog, adg.csdn.net, part 2 §2.2.2;
//                                                   the latent RMSNorm of its part 3 §3.1.1)
//
// Every projection is Y = X W^T with both operands' reduced axis contiguous
// (X [T, K] rows, W [N, K] rows as eq. 9 writes them).  For decode sizes the
// weights dominate the bytes and are read once.  In bf16 a workgroup computes
// a tile of 128 W rows x 128 (or 64) X rows with four waves of MFMA tiles;
// K advances in stages of 64 that direct global->LDS loads bring in, four
// (three) stages resident and three (two) in flight, and the two projections
// that share an input (W^DKV and W^KR; W^UQ and W^QR) run in one launch.
// Narrow projections (576 or d_cq outputs) split K over workgroups to fill
// the chip and write fp32 partial sums; one workgroup per token adds them up
// before the RMSNorm (and, for the cache row, the key rotation and the paged
// write).  A model without query compression (V2-Lite) takes both query parts
// straight from h in one launch.  W^O rounds the heads' fp32 outputs to bf16
// once, splits its long K over workgroups and sums the partials.  fp32 takes
// a plain MFMA kernel without LDS.
#include <algorithm>

#include "mla_common.h"
#include "mla_internal.h"
#include "proj_tile.h"

namespace mla {

namespace {

constexpr int GN = 64;    // fp32: outputs per workgroup
constexpr int GT = 128;   // fp32: rows per workgroup

// fp32: Y[z] = X[:, kz] W[:, kz]^T over K slice z (kz = [z kc, min(K, (z+1) kc))),
// written to columns col0 .. col0 + N - 1 of rows of ldo elements.  DIRECT:
// one slice, into out [T, ldo]; else partials into part [S, T, ldo].  Wave w
// owns outputs 16w..16w+15 (A = W rows) and all 128 rows (B = X rows).
template <class E, bool DIRECT>
__global__ void __launch_bounds__(256) gemm_nt_kernel(const typename E::storage* __restrict__ X,
                                                      const typename E::storage* __restrict__ W,
                                                      int T, int N, int K, int kc,
                                                      float* __restrict__ part, int ldo, int col0,
                                                      typename E::storage* __restrict__ out) {
  const int lane = lane_id(), wave = threadIdx.x >> 6, g = lane >> 4, r16 = lane & 15;
  const int n = blockIdx.x * GN + 16 * wave + r16;   // this lane's A row
  const int t0 = blockIdx.y * GT;
  const int z = blockIdx.z;
  const int k0 = z * kc, k1 = min(K, k0 + kc);
  const bool n_ok = n < N;
  const typename E::storage* wrow = W + (long)(n_ok ? n : 0) * K + 8 * g;
  const typename E::storage* xrow[GT / 16];
  bool t_ok[GT / 16];
#pragma unroll
  for (int tb = 0; tb < GT / 16; ++tb) {
    const int t = t0 + 16 * tb + r16;
    t_ok[tb] = t < T;
    xrow[tb] = X + (long)(t_ok[tb] ? t : 0) * K + 8 * g;
  }
  f32x4_t acc[GT / 16];
#pragma unroll
  for (int tb = 0; tb < GT / 16; ++tb) acc[tb] = f32x4_t{0, 0, 0, 0};
  const float zero8[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll 2
  for (int k = k0; k < k1; k += 32) {
    const typename E::frag a = n_ok ? E::load8(wrow + k) : E::from8(zero8);
    typename E::frag b[GT / 16];
#pragma unroll
    for (int tb = 0; tb < GT / 16; ++tb) b[tb] = t_ok[tb] ? E::load8(xrow[tb] + k) : E::from8(zero8);
#pragma unroll
    for (int tb = 0; tb < GT / 16; ++tb) E::mma(acc[tb], a, b[tb]);
  }
  // D[m][t]: lane holds outputs n0 + 4g + i (i < 4) of row t0 + 16tb + r16
  const int nb = blockIdx.x * GN + 16 * wave + 4 * g;
  if (nb >= N) return;
#pragma unroll
  for (int tb = 0; tb < GT / 16; ++tb) {
    const int t = t0 + 16 * tb + r16;
    if (t >= T) continue;
    if constexpr (DIRECT) {
      typename E::storage* o = out + (long)t * ldo + col0 + nb;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = E::from_f32(acc[tb][i]);
    } else {
      *reinterpret_cast<float4*>(part + ((long)z * T + t) * ldo + col0 + nb) =
          float4{acc[tb][0], acc[tb][1], acc[tb][2], acc[tb][3]};
    }
  }
}

// Sum over the 64 lanes of a wave.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += xor_shfl(v, m);
  return v;
}

// One workgroup per new token: wave w adds partial rows w, w + 4, .. of the
// S partial rows [576] (four at a time, all loads in flight; a row past S is
// re-read with weight 0); wave 0 adds the four sums, RMSNorms the 512 latent
// features (gain, eps), rotates the 32 key pairs at the token's position and
// writes the row into its cache slot (the slot rule and the skipping of
// out-of-range rows are those of the append).
template <class E>
__global__ void __launch_bounds__(256) kv_epilogue_kernel(
    const float* __restrict__ part, int S, int T, const float* __restrict__ gain, float eps,
    typename E::storage* __restrict__ cache, int num_blocks, const int* __restrict__ table,
    int num_seqs, int max_blocks, const int* __restrict__ seq_idx, const int* __restrict__ pos,
    RopeFreq rf) {
  using Ts = typename E::storage;
  __shared__ float red[4][ROW];
  const int r = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = lane_id();
  const int b = seq_idx[r];
  const int p = pos[r];
  if (b < 0 || b >= num_seqs || p < 0 || p / BLOCK >= max_blocks) return;
  const int blk = table[(long)b * max_blocks + p / BLOCK];
  if (blk < 0 || blk >= num_blocks) return;
  // latent features 8 lane .. 8 lane + 7; key pair lane & 31 (kept by lanes < 32)
  float y[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  float kx = 0.0f, ky = 0.0f;
  for (int z0 = wave; z0 < S; z0 += 16) {
    float4 u[4], v[4];
    float2 w[4];
    float m[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int z = z0 + 4 * q;
      m[q] = z < S ? 1.0f : 0.0f;
      const float* row = part + ((long)min(z, S - 1) * T + r) * ROW;
      u[q] = reinterpret_cast<const float4*>(row + 8 * lane)[0];
      v[q] = reinterpret_cast<const float4*>(row + 8 * lane)[1];
      w[q] = reinterpret_cast<const float2*>(row + D_C)[lane & 31];
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      y[0] += m[q] * u[q].x; y[1] += m[q] * u[q].y; y[2] += m[q] * u[q].z; y[3] += m[q] * u[q].w;
      y[4] += m[q] * v[q].x; y[5] += m[q] * v[q].y; y[6] += m[q] * v[q].z; y[7] += m[q] * v[q].w;
      kx += m[q] * w[q].x;
      ky += m[q] * w[q].y;
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) red[wave][8 * lane + j] = y[j];
  if (lane < D_R / 2) {
    red[wave][D_C + 2 * lane] = kx;
    red[wave][D_C + 2 * lane + 1] = ky;
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int c = 8 * lane + j;
    y[j] = (red[0][c] + red[1][c]) + (red[2][c] + red[3][c]);
  }
  if (lane < D_R / 2) {
    const int c = D_C + 2 * lane;
    kx = (red[0][c] + red[1][c]) + (red[2][c] + red[3][c]);
    ky = (red[0][c + 1] + red[1][c + 1]) + (red[2][c + 1] + red[3][c + 1]);
  }
  Ts* dst = cache + ((long)blk * BLOCK + (p % BLOCK)) * ROW;
  float ss = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) ss += y[j] * y[j];
  const float rs = 1.0f / sqrtf(wave_sum(ss) / (float)D_C + eps);
  float c[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) c[j] = y[j] * rs * gain[8 * lane + j];
  if constexpr (E::bytes == 2) {
    reinterpret_cast<uint4*>(dst)[lane] = uint4{pack_bf16x2(c[0], c[1]), pack_bf16x2(c[2], c[3]),
                                                pack_bf16x2(c[4], c[5]), pack_bf16x2(c[6], c[7])};
  } else {
    reinterpret_cast<float4*>(dst)[2 * lane] = float4{c[0], c[1], c[2], c[3]};
    reinterpret_cast<float4*>(dst)[2 * lane + 1] = float4{c[4], c[5], c[6], c[7]};
  }
  if (lane < D_R / 2) {
    double cs, sn;
    rope_cs(p, rf.theta[lane], cs, sn);
    const double x = kx, yv = ky;
    dst[D_C + 2 * lane] = E::from_f32((float)(x * cs - yv * sn));
    dst[D_C + 2 * lane + 1] = E::from_f32((float)(x * sn + yv * cs));
  }
}

// One workgroup per token: wave w adds partial rows w, w + 4, .. of the S
// partial rows [d] (d <= 2048, a multiple of 64; four rows at a time, all
// loads in flight, a row past S re-read with weight 0); then every thread
// adds the four sums of its features, and the token's row is RMSNormed
// (gain, eps) and stored as c^Q [T, d] in the element type.
template <class E>
__global__ void __launch_bounds__(256) q_norm_kernel(const float* __restrict__ part, int S, int T,
                                                     int d, const float* __restrict__ gain,
                                                     float eps,
                                                     typename E::storage* __restrict__ c_q) {
  __shared__ float red[4][2048];
  __shared__ float ssum[4];
  const int t = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = lane_id();
  // lane's float4 columns lane + 64 j (j < 8, below d / 4)
  const int n4 = d / 4;
  float4 y[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) y[j] = float4{0, 0, 0, 0};
  for (int z0 = wave; z0 < S; z0 += 16) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int z = z0 + 4 * q;
      const float m = z < S ? 1.0f : 0.0f;
      const float4* row = reinterpret_cast<const float4*>(part + ((long)min(z, S - 1) * T + t) * d);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (64 * j >= n4) break;
        const float4 u = row[min(lane + 64 * j, n4 - 1)];
        y[j].x += m * u.x; y[j].y += m * u.y; y[j].z += m * u.z; y[j].w += m * u.w;
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (lane + 64 * j < n4) reinterpret_cast<float4*>(red[wave])[lane + 64 * j] = y[j];
  __syncthreads();
  float v[8];
  float ss = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int i = threadIdx.x + 256 * j;
    v[j] = i < d ? (red[0][i] + red[1][i]) + (red[2][i] + red[3][i]) : 0.0f;
    ss += v[j] * v[j];
  }
  ss = wave_sum(ss);
  if (lane == 0) ssum[wave] = ss;
  __syncthreads();
  const float rs = 1.0f / sqrtf((ssum[0] + ssum[1] + ssum[2] + ssum[3]) / (float)d + eps);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int i = threadIdx.x + 256 * j;
    if (i < d) c_q[(long)t * d + i] = E::from_f32(v[j] * rs * gain[i]);
  }
}

// K slice length of a projection with N outputs for T rows: enough
// workgroups to fill the chip (about 256), each slice a multiple of 64 and
// at least 512 long, so that the fp32 partials it writes stay well below the
// weight bytes it reads.  The slice count is ceil(K / length).
int k_chunk(int T, int N, int K) {
  const int tt = t_tile(T, N);
  const long tiles = (long)((N + PN - 1) / PN) * ((T + tt - 1) / tt);
  int S = 1;
  if (tiles > 0 && tiles < 128)
    S = (int)std::max(1L, std::min((256 + tiles - 1) / tiles, (long)(K / 512)));
  return ((K + S - 1) / S + PK - 1) / PK * PK;
}
int k_slices(int T, int N, int K) {
  const int kc = k_chunk(T, N, K);
  return (K + kc - 1) / kc;
}

// fp32: one projection W [N, K] against X [T, K] into columns col0.. of rows
// of ldo, in K slices of kc (DIRECT: one slice, element-type output).
template <class E>
void gemm_f32(const void* X, const void* W, int T, int N, int K, int kc, bool direct,
              float* part, int ldo, int col0, void* out, hipStream_t stream) {
  using Ts = typename E::storage;
  const int S = (K + kc - 1) / kc;
  dim3 grid((N + GN - 1) / GN, (T + GT - 1) / GT, S), block(256);
  if (direct)
    hipLaunchKernelGGL((gemm_nt_kernel<E, true>), grid, block, 0, stream, (const Ts*)X,
                       (const Ts*)W, T, N, K, kc, nullptr, ldo, col0, (Ts*)out);
  else
    hipLaunchKernelGGL((gemm_nt_kernel<E, false>), grid, block, 0, stream, (const Ts*)X,
                       (const Ts*)W, T, N, K, kc, part, ldo, col0, nullptr);
}

template <class E>
hipError_t kv_produce(const void* h, const void* w_dkv, const float* kv_gain, const void* w_kr,
                      int T, int d_model, float eps, const RopeFreq& rf, void* cache, int num_blocks,
                      const int* table, int num_seqs, int max_blocks, const int* seq_idx,
                      const int* pos, void* workspace, hipStream_t stream) {
  float* part = static_cast<float*>(workspace);
  const int kc = k_chunk(T, ROW, d_model);
  const int S = (d_model + kc - 1) / kc;
  // the latent and the key projections fill columns 0..511 and 512..575 of
  // one partial buffer [S, T, 576]
  if constexpr (E::bytes == 2) {
    proj_bf16<OUT_PARTIAL>(XSrc{static_cast<const uint16_t*>(h), d_model, nullptr, 0}, T, d_model,
                           kc, ProjOut{static_cast<const uint16_t*>(w_dkv), D_C, part, ROW, 0, 0},
                           ProjOut{static_cast<const uint16_t*>(w_kr), D_R, part, ROW, D_C, 0},
                           stream);
  } else {
    gemm_f32<E>(h, w_dkv, T, D_C, d_model, kc, false, part, ROW, 0, nullptr, stream);
    gemm_f32<E>(h, w_kr, T, D_R, d_model, kc, false, part, ROW, D_C, nullptr, stream);
  }
  hipLaunchKernelGGL(kv_epilogue_kernel<E>, dim3(T), dim3(256), 0, stream, part, S, T, kv_gain,
                     eps, (typename E::storage*)cache, num_blocks, table, num_seqs, max_blocks,
                     seq_idx, pos, rf);
  return hipGetLastError();
}

template <class E>
hipError_t q_produce(const void* h, const void* w_dq, const float* q_gain, const void* w_uq,
                     const void* w_qr, int T, int d_model, int d_cq, int n_h, float eps,
                     void* q_nope, void* q_rope, void* workspace, hipStream_t stream) {
  const int kc = k_chunk(T, d_cq, d_model);
  const int S = (d_model + kc - 1) / kc;
  float* part = static_cast<float*>(workspace);
  const long part_bytes = ((long)S * T * d_cq * 4 + 255) / 256 * 256;
  auto* c_q = reinterpret_cast<typename E::storage*>(static_cast<char*>(workspace) + part_bytes);
  if constexpr (E::bytes == 2)
    proj_bf16<OUT_PARTIAL>(XSrc{static_cast<const uint16_t*>(h), d_model, nullptr, 0}, T, d_model,
                           kc, ProjOut{static_cast<const uint16_t*>(w_dq), d_cq, part, d_cq, 0, 0},
                           ProjOut{nullptr, 0, nullptr, 0, 0, 0}, stream);
  else
    gemm_f32<E>(h, w_dq, T, d_cq, d_model, kc, false, part, d_cq, 0, nullptr, stream);
  hipLaunchKernelGGL(q_norm_kernel<E>, dim3(T), dim3(256), 0, stream, part, S, T, d_cq, q_gain,
                     eps, c_q);
  if constexpr (E::bytes == 2) {
    proj_bf16<OUT_ROWS>(XSrc{reinterpret_cast<const uint16_t*>(c_q), d_cq, nullptr, 0}, T, d_cq, d_cq,
                        ProjOut{static_cast<const uint16_t*>(w_uq), n_h * D_H, q_nope, n_h * D_H,
                                0, 0},
                        ProjOut{static_cast<const uint16_t*>(w_qr), n_h * D_R, q_rope, n_h * D_R,
                                0, 0},
                        stream);
  } else {
    gemm_f32<E>(c_q, w_uq, T, n_h * D_H, d_cq, d_cq, true, nullptr, n_h * D_H, 0, q_nope, stream);
    gemm_f32<E>(c_q, w_qr, T, n_h * D_R, d_cq, d_cq, true, nullptr, n_h * D_R, 0, q_rope, stream);
  }
  return hipGetLastError();
}

// Queries of a model without query compression: q^C = W^QC h, q^R = W^QR h
// (both straight from the hidden states), one launch in bf16.
template <class E>
hipError_t q_direct(const void* h, const void* w_qc, const void* w_qr, int T, int d_model,
                    int n_h, void* q_nope, void* q_rope, hipStream_t stream) {
  if constexpr (E::bytes == 2) {
    proj_bf16<OUT_ROWS>(XSrc{static_cast<const uint16_t*>(h), d_model, nullptr, 0}, T, d_model,
                        d_model,
                        ProjOut{static_cast<const uint16_t*>(w_qc), n_h * D_H, q_nope, n_h * D_H,
                                0, 0},
                        ProjOut{static_cast<const uint16_t*>(w_qr), n_h * D_R, q_rope, n_h * D_R,
                                0, 0},
                        stream);
  } else {
    gemm_f32<E>(h, w_qc, T, n_h * D_H, d_model, d_model, true, nullptr, n_h * D_H, 0, q_nope,
                stream);
    gemm_f32<E>(h, w_qr, T, n_h * D_R, d_model, d_model, true, nullptr, n_h * D_R, 0, q_rope,
                stream);
  }
  return hipGetLastError();
}

// fp32 [n] -> bf16, eight elements per thread and pass (n a multiple of 8).
__global__ void __launch_bounds__(256) to_bf16_kernel(const float* __restrict__ x, long n,
                                                      uint16_t* __restrict__ y) {
  for (long i = ((long)blockIdx.x * 256 + threadIdx.x) * 8; i < n; i += (long)gridDim.x * 256 * 8) {
    const float4 a = *reinterpret_cast<const float4*>(x + i);
    const float4 b = *reinterpret_cast<const float4*>(x + i + 4);
    *reinterpret_cast<uint4*>(y + i) = uint4{pack_bf16x2(a.x, a.y), pack_bf16x2(a.z, a.w),
                                             pack_bf16x2(b.x, b.y), pack_bf16x2(b.z, b.w)};
  }
}

// y[i] = sum over z < S of part[z n + i], in the element type (n a multiple of 4).
template <class E>
__global__ void __launch_bounds__(256) sum_parts_kernel(const float* __restrict__ part, int S,
                                                        long n, typename E::storage* __restrict__ y) {
  for (long i = ((long)blockIdx.x * 256 + threadIdx.x) * 4; i < n; i += (long)gridDim.x * 256 * 4) {
    float4 v = *reinterpret_cast<const float4*>(part + i);
    for (int z = 1; z < S; ++z) {
      const float4 w = *reinterpret_cast<const float4*>(part + (long)z * n + i);
      v.x += w.x; v.y += w.y; v.z += w.z; v.w += w.w;
    }
    y[i] = E::from_f32(v.x);
    y[i + 1] = E::from_f32(v.y);
    y[i + 2] = E::from_f32(v.z);
    y[i + 3] = E::from_f32(v.w);
  }
}

// K slice length of W^O: its weights (d_model x n_h 128) dwarf the fp32
// partials of a decode batch, so slice for about 1024 workgroups while the
// partials stay within 1/8 of the weight bytes (S <= K / (16 T)), each slice
// at least 512 long and a multiple of 64.
int o_chunk(int T, int N, int K) {
  const int tt = t_tile(T, N);
  const long tiles = (long)((N + PN - 1) / PN) * ((T + tt - 1) / tt);
  const long cap = std::max(1L, std::min((long)K / 512, (long)K / (16L * std::max(T, 1))));
  const int S = (int)std::max(1L, std::min((1024 + tiles - 1) / tiles, cap));
  return ((K + S - 1) / S + PK - 1) / PK * PK;
}

// bf16 W^O: K slice length and X-row tile.  The weight stream is the bound
// and a slice's workgroups all start together, so the split fills one round
// of the chip's workgroup slots rather than several: 256 with 128-row tiles
// (one workgroup per CU, each weight tile staged once per slice) or 512 with
// 64-row tiles (two per CU, each weight tile staged twice).  128-row tiles are
// taken when T > 64 and they fill at least 3/4 of their round; the partials
// cap is as above.  V2's decode shape (T = 128, 5120 x 16384): 40 tiles x 6
// slices, 57 us against 77 us for 80 tiles x 8 slices (640 workgroups, a
// quarter of them in a second round).
int o_chunk_bf16(int T, int N, int K, int& tt) {
  constexpr long CUS = 256;
  const long cap = std::max(1L, std::min((long)K / 512, (long)K / (16L * std::max(T, 1))));
  const long ntile = (N + PN - 1) / PN;
  const long tiles128 = ntile * ((T + 127) / 128), tiles64 = ntile * ((T + 63) / 64);
  const long s128 = std::max(1L, std::min(CUS / tiles128, cap));
  const long s64 = std::max(1L, std::min(2 * CUS / tiles64, cap));
  long S;
  if (T > 64 && tiles128 * s128 * 4 >= CUS * 3) {
    tt = 128;
    S = s128;
  } else {
    tt = 64;
    S = s64;
  }
  return (int)(((K + S - 1) / S + PK - 1) / PK * PK);
}

// eq. 8: u = W^O [o_1; ...; o_nh] for T rows of the heads' fp32 outputs.  In
// bf16 the outputs are rounded to bf16 once (workspace) to feed the MFMA;
// K = n_h 128 is split over workgroups into fp32 partials when the output
// tiles alone would leave the chip idle.
template <class E>
hipError_t o_proj(const float* out, const void* w_o, int T, int n_h, int d_model, void* u,
                  void* workspace, hipStream_t stream) {
  const int K = n_h * D_H;
  int tt = 0;
  const int kc = E::bytes == 2 ? o_chunk_bf16(T, d_model, K, tt) : o_chunk(T, d_model, K);
  const int S = (K + kc - 1) / kc;
  char* ws = static_cast<char*>(workspace);
  const long xb = E::bytes == 2 ? ((long)T * K * 2 + 255) / 256 * 256 : 0;
  float* part = reinterpret_cast<float*>(ws + xb);
  const long n = (long)T * d_model;
  const int grid = (int)std::min<long>(4096, (n + 1023) / 1024);
  if constexpr (E::bytes == 2) {
    auto* xh = reinterpret_cast<uint16_t*>(ws);
    const long nx = (long)T * K;
    hipLaunchKernelGGL(to_bf16_kernel, dim3((int)std::min<long>(4096, (nx + 2047) / 2048)),
                       dim3(256), 0, stream, out, nx, xh);
    if (S == 1) {
      proj_bf16<OUT_ROWS>(XSrc{xh, K, nullptr, 0}, T, K, K,
                          ProjOut{static_cast<const uint16_t*>(w_o), d_model, u, d_model, 0, 0},
                          ProjOut{nullptr, 0, nullptr, 0, 0, 0}, stream);
      return hipGetLastError();
    }
    proj_bf16<OUT_PARTIAL>(XSrc{xh, K, nullptr, 0}, T, K, kc,
                           ProjOut{static_cast<const uint16_t*>(w_o), d_model, part, d_model, 0, 0},
                           ProjOut{nullptr, 0, nullptr, 0, 0, 0}, stream, tt);
  } else {
    if (S == 1) {
      gemm_f32<E>(out, w_o, T, d_model, K, K, true, nullptr, d_model, 0, u, stream);
      return hipGetLastError();
    }
    gemm_f32<E>(out, w_o, T, d_model, K, kc, false, part, d_model, 0, nullptr, stream);
  }
  hipLaunchKernelGGL(sum_parts_kernel<E>, dim3(grid), dim3(256), 0, stream, part, S, n,
                     static_cast<typename E::storage*>(u));
  return hipGetLastError();
}

}  // namespace

long o_proj_workspace(int T, int n_h, int d_model, int dtype) {
  const int K = n_h * D_H;
  const long xb = dtype == 1 ? ((long)T * K * 2 + 255) / 256 * 256 : 0;
  int tt = 0;
  const int kc = dtype == 1 ? o_chunk_bf16(T, d_model, K, tt) : o_chunk(T, d_model, K);
  const int S = (K + kc - 1) / kc;
  return xb + (S > 1 ? (long)S * T * d_model * 4 : 0);
}

hipError_t launch_o_proj(const float* out, const void* w_o, int T, int n_h, int d_model,
                         int dtype, void* u, void* workspace, hipStream_t stream) {
  if (dtype == 1) return o_proj<BF16>(out, w_o, T, n_h, d_model, u, workspace, stream);
  return o_proj<F32>(out, w_o, T, n_h, d_model, u, workspace, stream);
}

hipError_t launch_q_produce_direct(const void* h, const void* w_qc, const void* w_qr, int T,
                                   int d_model, int n_h, int dtype, void* q_nope, void* q_rope,
                                   hipStream_t stream) {
  if (dtype == 1) return q_direct<BF16>(h, w_qc, w_qr, T, d_model, n_h, q_nope, q_rope, stream);
  return q_direct<F32>(h, w_qc, w_qr, T, d_model, n_h, q_nope, q_rope, stream);
}

long kv_produce_workspace(int T, int d_model) {
  return (long)k_slices(T, ROW, d_model) * T * ROW * 4;
}

long q_produce_workspace(int T, int d_model, int d_cq, int dtype) {
  const long part = ((long)k_slices(T, d_cq, d_model) * T * d_cq * 4 + 255) / 256 * 256;
  return part + ((long)T * d_cq * (dtype == 1 ? 2 : 4) + 255) / 256 * 256;
}

hipError_t launch_kv_produce(const void* h, const void* w_dkv, const float* kv_gain,
                             const void* w_kr, int T, int d_model, int dtype, float eps,
                             const RopeFreq& rf, void* cache, int num_blocks, const int* table,
                             int num_seqs, int max_blocks, const int* seq_idx, const int* pos,
                             void* workspace, hipStream_t stream) {
  if (dtype == 1)
    return kv_produce<BF16>(h, w_dkv, kv_gain, w_kr, T, d_model, eps, rf, cache, num_blocks,
                            table, num_seqs, max_blocks, seq_idx, pos, workspace, stream);
  return kv_produce<F32>(h, w_dkv, kv_gain, w_kr, T, d_model, eps, rf, cache, num_blocks,
                         table, num_seqs, max_blocks, seq_idx, pos, workspace, stream);
}

hipError_t launch_q_produce(const void* h, const void* w_dq, const float* q_gain,
                            const void* w_uq, const void* w_qr, int T, int d_model, int d_cq,
                            int n_h, int dtype, float eps, void* q_nope, void* q_rope,
                            void* workspace, hipStream_t stream) {
  if (dtype == 1)
    return q_produce<BF16>(h, w_dq, q_gain, w_uq, w_qr, T, d_model, d_cq, n_h, eps, q_nope,
                           q_rope, workspace, stream);
  return q_produce<F32>(h, w_dq, q_gain, w_uq, w_qr, T, d_model, d_cq, n_h, eps, q_nope, q_rope,
                        workspace, stream);
}

}  // namespace mla
