// KV append: write new tokens' latent rows into the paged cache.
//
// Per token the cache keeps [c^KV ; R_pos k^R]: the compressed latent unrotated
// and the decoupled RoPE key already rotated at the token's position
// (DeepSeek-V2 MLA blog, adg.csdn.net, part 2 §2.2.2).  One wave per token
// (append_row.h): the 512 latent elements are copied with 16-byte
// loads/stores, 32 lanes rotate one RoPE pair each.
//
// The FP8 variant writes the quantised row instead (DeepSeek-V2 MLA blog,
// part 3 §3.1.4: the served cache is quantised; the scheme here is OCP FP8
// E4M3 with one float32 scale for the latent part and one for the RoPE part
// of each token): per part s = amax / 448 and code = E4M3(x / s), nearest
// even, from the float32 row, both divisions correctly rounded.
#include "append_row.h"
#include "mla_common.h"
#include "mla_internal.h"

namespace mla {

template <class E>
__global__ void __launch_bounds__(256) kv_append_kernel(
    typename E::storage* __restrict__ cache, int num_blocks, const int* __restrict__ table,
    int num_seqs, int max_blocks, const typename E::storage* __restrict__ c_kv,
    const typename E::storage* __restrict__ k_rope, const int* __restrict__ seq_idx,
    const int* __restrict__ pos, int n, RopeFreq rf) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= n) return;
  append_row<E>(cache, num_blocks, table, num_seqs, max_blocks, c_kv, k_rope, seq_idx, pos, r,
                threadIdx.x & 63, rf);
}

// Largest value over the 64 lanes of the wave.
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v = fmaxf(v, xor_shfl(v, m));
  return v;
}

// E4M3 codes of a pair of quotients x / s (the hardware conversion rounds to
// nearest even; clamping to +-448 keeps a quotient just above 448 off the NaN
// code, which the format uses in place of infinity).
template <bool HIGH>
__device__ __forceinline__ int fp8_pair(float a, float b, float s, int old) {
  const float qa = fminf(fmaxf(a / s, -448.0f), 448.0f);
  const float qb = fminf(fmaxf(b / s, -448.0f), 448.0f);
  return __builtin_amdgcn_cvt_pk_fp8_f32(qa, qb, old, HIGH);
}

template <class E>
__global__ void __launch_bounds__(256) kv_append_fp8_kernel(
    uint8_t* __restrict__ cache, float* __restrict__ kv_scale, int num_blocks,
    const int* __restrict__ table, int num_seqs, int max_blocks,
    const typename E::storage* __restrict__ c_kv, const typename E::storage* __restrict__ k_rope,
    const int* __restrict__ seq_idx, const int* __restrict__ pos, int n, RopeFreq rf) {
  using T = typename E::storage;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= n) return;
  const int b = seq_idx[r];
  const int p = pos[r];
  if (b < 0 || b >= num_seqs || p < 0 || p / BLOCK >= max_blocks) return;
  const int blk = table[(long)b * max_blocks + p / BLOCK];
  if (blk < 0 || blk >= num_blocks) return;
  const long slot = (long)blk * BLOCK + p % BLOCK;
  uint8_t* dst = cache + slot * ROW;
  // latent: this lane's 8 elements
  const T* src = c_kv + (long)r * D_C + 8 * lane;
  float x[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = E::to_f32(src[j]);
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(x[j]));
  amax = wave_max(amax);
  const float sc = amax > 0.0f ? amax / 448.0f : 1.0f;
  int w0 = fp8_pair<false>(x[0], x[1], sc, 0);
  w0 = fp8_pair<true>(x[2], x[3], sc, w0);
  int w1 = fp8_pair<false>(x[4], x[5], sc, 0);
  w1 = fp8_pair<true>(x[6], x[7], sc, w1);
  *reinterpret_cast<uint2*>(dst + 8 * lane) = uint2{(unsigned)w0, (unsigned)w1};
  // RoPE part: lanes 0..31 rotate one pair each (float64, then float32)
  float kx = 0.0f, ky = 0.0f;
  if (lane < D_R / 2) {
    double c, s;
    rope_cs(p, rf.theta[lane], c, s);
    const T* kr = k_rope + (long)r * D_R;
    const double u = E::to_f32(kr[2 * lane]), v = E::to_f32(kr[2 * lane + 1]);
    kx = (float)(u * c - v * s);
    ky = (float)(u * s + v * c);
  }
  const float ramax = wave_max(fmaxf(fabsf(kx), fabsf(ky)));
  const float sr = ramax > 0.0f ? ramax / 448.0f : 1.0f;
  if (lane < D_R / 2)
    *reinterpret_cast<uint16_t*>(dst + D_C + 2 * lane) = (uint16_t)fp8_pair<false>(kx, ky, sr, 0);
  if (lane == 0) *reinterpret_cast<float2*>(kv_scale + 2 * slot) = float2{sc, sr};
}

hipError_t launch_kv_append_fp8(void* cache, float* kv_scale, int dtype, int num_blocks,
                                const int* table, int num_seqs, int max_blocks, const void* c_kv,
                                const void* k_rope, const int* seq_idx, const int* pos, int n,
                                const RopeFreq& rf, hipStream_t stream) {
  dim3 grid((n + 3) / 4), block(256);
  if (dtype == 1)
    hipLaunchKernelGGL(kv_append_fp8_kernel<BF16>, grid, block, 0, stream, (uint8_t*)cache,
                       kv_scale, num_blocks, table, num_seqs, max_blocks, (const uint16_t*)c_kv,
                       (const uint16_t*)k_rope, seq_idx, pos, n, rf);
  else
    hipLaunchKernelGGL(kv_append_fp8_kernel<F32>, grid, block, 0, stream, (uint8_t*)cache,
                       kv_scale, num_blocks, table, num_seqs, max_blocks, (const float*)c_kv,
                       (const float*)k_rope, seq_idx, pos, n, rf);
  return hipGetLastError();
}

hipError_t launch_kv_append(void* cache, int dtype, int num_blocks, const int* table,
                            int num_seqs, int max_blocks, const void* c_kv, const void* k_rope,
                            const int* seq_idx, const int* pos, int n, const RopeFreq& rf,
                            hipStream_t stream) {
  dim3 grid((n + 3) / 4), block(256);
  if (dtype == 1)
    hipLaunchKernelGGL(kv_append_kernel<BF16>, grid, block, 0, stream, (uint16_t*)cache,
                       num_blocks, table, num_seqs, max_blocks, (const uint16_t*)c_kv,
                       (const uint16_t*)k_rope, seq_idx, pos, n, rf);
  else
    hipLaunchKernelGGL(kv_append_kernel<F32>, grid, block, 0, stream, (float*)cache,
                       num_blocks, table, num_seqs, max_blocks, (const float*)c_kv,
                       (const float*)k_rope, seq_idx, pos, n, rf);
  return hipGetLastError();
}

}  // namespace mla
