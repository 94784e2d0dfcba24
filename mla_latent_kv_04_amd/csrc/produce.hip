// Cache and query producers: the projections that feed the attention path.
//
//   c^KV = RMSNorm(W^DKV h), k^R = W^KR h          (eq. 9 of the DeepSeek-V2
//   c^Q  = RMSNorm(W^DQ h),  q^C = W^UQ c^Q,        notes, irregular6612.github.io,
//   q^R  = W^QR c^Q                                 §2.1.2, eq. 12-13; the decoupled
//                                                   key / query of the DeepSeek-V2 MLA
//                                                   blog, adg.csdn.net, part 2 §2.2.2;
//                                                   the latent RMSNorm of its §3.1.1)
//
// Every projection is Y = X W^T with both operands' reduced axis contiguous
// (X [T, K] rows, W [N, K] rows as eq. 9 writes them), so MFMA fragments load
// straight from memory.  A workgroup of four waves computes 64 outputs for
// 128 rows over one slice of K: wave w owns outputs 16w..16w+15 (A = W rows)
// and all 128 rows (B = X rows, shared by the four waves through L1).  For the
// decode sizes the weights dominate the bytes and are read once; the narrow
// projections (576 and 1536 outputs) split K over workgroups to fill the chip,
// writing fp32 partial sums that the epilogue kernels add up before the
// RMSNorm, the key rotation and the paged write.  No LDS: occupancy hides the
// load latency.
#include <algorithm>

#include "mla_common.h"
#include "mla_internal.h"

namespace mla {

namespace {

constexpr int GN = 64;    // outputs per workgroup
constexpr int GT = 128;   // rows per workgroup

// Y[z] = X[:, kz] W[:, kz]^T over K slice z (kz = [z kc, min(K, (z+1) kc))),
// written to columns col0 .. col0 + N - 1 of rows of ldo elements.  DIRECT:
// one slice, converted to the element type into out [T, ldo]; else fp32
// partials into part [S, T, ldo].
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

// One wave per new token: add the S partial rows [576], RMSNorm the 512
// latent features (gain, eps), rotate the 32 key pairs at the token's
// position and write the row into its cache slot (the slot rule and the
// skipping of out-of-range rows are those of the append).
template <class E>
__global__ void __launch_bounds__(256) kv_epilogue_kernel(
    const float* __restrict__ part, int S, int T, const float* __restrict__ gain, float eps,
    typename E::storage* __restrict__ cache, int num_blocks, const int* __restrict__ table,
    int num_seqs, int max_blocks, const int* __restrict__ seq_idx, const int* __restrict__ pos,
    double base) {
  using Ts = typename E::storage;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = lane_id();
  if (r >= T) return;
  const int b = seq_idx[r];
  const int p = pos[r];
  if (b < 0 || b >= num_seqs || p < 0 || p / BLOCK >= max_blocks) return;
  const int blk = table[(long)b * max_blocks + p / BLOCK];
  if (blk < 0 || blk >= num_blocks) return;
  Ts* dst = cache + ((long)blk * BLOCK + (p % BLOCK)) * ROW;
  // latent features 8 lane .. 8 lane + 7
  float y[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  float kx = 0.0f, ky = 0.0f;
  for (int z = 0; z < S; ++z) {
    const float* row = part + ((long)z * T + r) * ROW;
    const float4 u = reinterpret_cast<const float4*>(row + 8 * lane)[0];
    const float4 v = reinterpret_cast<const float4*>(row + 8 * lane)[1];
    y[0] += u.x; y[1] += u.y; y[2] += u.z; y[3] += u.w;
    y[4] += v.x; y[5] += v.y; y[6] += v.z; y[7] += v.w;
    if (lane < D_R / 2) {
      const float2 w = reinterpret_cast<const float2*>(row + D_C)[lane];
      kx += w.x;
      ky += w.y;
    }
  }
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
    rope_cs(p, lane, base, cs, sn);
    const double x = kx, yv = ky;
    dst[D_C + 2 * lane] = E::from_f32((float)(x * cs - yv * sn));
    dst[D_C + 2 * lane + 1] = E::from_f32((float)(x * sn + yv * cs));
  }
}

// One workgroup per token: add the S partial rows [d], RMSNorm them (gain,
// eps) and store the compressed query c^Q [T, d] in the element type.
template <class E>
__global__ void __launch_bounds__(256) q_norm_kernel(const float* __restrict__ part, int S, int T,
                                                     int d, const float* __restrict__ gain,
                                                     float eps,
                                                     typename E::storage* __restrict__ c_q) {
  __shared__ float red[4];
  const int t = blockIdx.x;
  float ss = 0.0f;
  // d <= 256 * 8: every thread holds up to 8 features
  float y[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int i = threadIdx.x + 256 * j;
    float v = 0.0f;
    if (i < d)
      for (int z = 0; z < S; ++z) v += part[((long)z * T + t) * d + i];
    y[j] = v;
    ss += v * v;
  }
  ss = wave_sum(ss);
  if (lane_id() == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float rs = 1.0f / sqrtf((red[0] + red[1] + red[2] + red[3]) / (float)d + eps);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int i = threadIdx.x + 256 * j;
    if (i < d) c_q[(long)t * d + i] = E::from_f32(y[j] * rs * gain[i]);
  }
}

// Slices of K per projection: enough workgroups to fill the chip (about 512),
// each slice a multiple of 32 and at least 256 long.
int k_slices(int T, int N, int K) {
  const long tiles = (long)((N + GN - 1) / GN) * ((T + GT - 1) / GT);
  if (tiles == 0 || tiles >= 256) return 1;
  const int by_fill = (int)((512 + tiles - 1) / tiles);
  return std::max(1, std::min(by_fill, K / 256));
}
int k_chunk(int K, int S) { return ((K + S - 1) / S + 31) / 32 * 32; }

// One projection: W [N, K] against X [T, K] into columns col0.. of rows of
// ldo; S K-slices of fp32 partials (S > 1 or !direct) or the element type.
template <class E>
void gemm(const void* X, const void* W, int T, int N, int K, int S, bool direct, float* part,
          int ldo, int col0, void* out, hipStream_t stream) {
  using Ts = typename E::storage;
  dim3 grid((N + GN - 1) / GN, (T + GT - 1) / GT, S), block(256);
  if (direct)
    hipLaunchKernelGGL((gemm_nt_kernel<E, true>), grid, block, 0, stream, (const Ts*)X,
                       (const Ts*)W, T, N, K, k_chunk(K, S), nullptr, ldo, col0, (Ts*)out);
  else
    hipLaunchKernelGGL((gemm_nt_kernel<E, false>), grid, block, 0, stream, (const Ts*)X,
                       (const Ts*)W, T, N, K, k_chunk(K, S), part, ldo, col0, nullptr);
}

template <class E>
hipError_t kv_produce(const void* h, const void* w_dkv, const float* kv_gain, const void* w_kr,
                      int T, int d_model, float eps, float base, void* cache, int num_blocks,
                      const int* table, int num_seqs, int max_blocks, const int* seq_idx,
                      const int* pos, void* workspace, hipStream_t stream) {
  float* part = static_cast<float*>(workspace);
  const int S = k_slices(T, ROW, d_model);
  // the latent and the key projections fill columns 0..511 and 512..575 of
  // one partial buffer [S, T, 576]
  gemm<E>(h, w_dkv, T, D_C, d_model, S, false, part, ROW, 0, nullptr, stream);
  gemm<E>(h, w_kr, T, D_R, d_model, S, false, part, ROW, D_C, nullptr, stream);
  hipLaunchKernelGGL(kv_epilogue_kernel<E>, dim3((T + 3) / 4), dim3(256), 0, stream, part, S, T,
                     kv_gain, eps, (typename E::storage*)cache, num_blocks, table, num_seqs,
                     max_blocks, seq_idx, pos, (double)base);
  return hipGetLastError();
}

template <class E>
hipError_t q_produce(const void* h, const void* w_dq, const float* q_gain, const void* w_uq,
                     const void* w_qr, int T, int d_model, int d_cq, int n_h, float eps,
                     void* q_nope, void* q_rope, void* workspace, hipStream_t stream) {
  const int S = k_slices(T, d_cq, d_model);
  float* part = static_cast<float*>(workspace);
  const long part_bytes = ((long)S * T * d_cq * 4 + 255) / 256 * 256;
  auto* c_q = reinterpret_cast<typename E::storage*>(static_cast<char*>(workspace) + part_bytes);
  gemm<E>(h, w_dq, T, d_cq, d_model, S, false, part, d_cq, 0, nullptr, stream);
  hipLaunchKernelGGL(q_norm_kernel<E>, dim3(T), dim3(256), 0, stream, part, S, T, d_cq, q_gain,
                     eps, c_q);
  gemm<E>(c_q, w_uq, T, n_h * D_H, d_cq, 1, true, nullptr, n_h * D_H, 0, q_nope, stream);
  gemm<E>(c_q, w_qr, T, n_h * D_R, d_cq, 1, true, nullptr, n_h * D_R, 0, q_rope, stream);
  return hipGetLastError();
}

}  // namespace

long kv_produce_workspace(int T, int d_model) {
  return (long)k_slices(T, ROW, d_model) * T * ROW * 4;
}

long q_produce_workspace(int T, int d_model, int d_cq, int dtype) {
  const long part = ((long)k_slices(T, d_cq, d_model) * T * d_cq * 4 + 255) / 256 * 256;
  return part + ((long)T * d_cq * (dtype == 1 ? 2 : 4) + 255) / 256 * 256;
}

hipError_t launch_kv_produce(const void* h, const void* w_dkv, const float* kv_gain,
                             const void* w_kr, int T, int d_model, int dtype, float eps,
                             float base, void* cache, int num_blocks, const int* table,
                             int num_seqs, int max_blocks, const int* seq_idx, const int* pos,
                             void* workspace, hipStream_t stream) {
  if (dtype == 1)
    return kv_produce<BF16>(h, w_dkv, kv_gain, w_kr, T, d_model, eps, base, cache, num_blocks,
                            table, num_seqs, max_blocks, seq_idx, pos, workspace, stream);
  return kv_produce<F32>(h, w_dkv, kv_gain, w_kr, T, d_model, eps, base, cache, num_blocks,
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
