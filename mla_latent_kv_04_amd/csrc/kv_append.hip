// KV append: write new tokens' latent rows into the paged cache.
//
// Per token the cache keeps [c^KV ; R_pos k^R]: the compressed latent unrotated
// and the decoupled RoPE key already rotated at the token's position
// (DeepSeek-V2 MLA blog, adg.csdn.net, part 2 §2.2.2).  One wave per token:
// the 512 latent elements are copied with 16-byte loads/stores, 32 lanes
// rotate one RoPE pair each.
#include "mla_common.h"
#include "mla_internal.h"

namespace mla {

template <class E>
__global__ void __launch_bounds__(256) kv_append_kernel(
    typename E::storage* __restrict__ cache, int num_blocks, const int* __restrict__ table,
    int num_seqs, int max_blocks, const typename E::storage* __restrict__ c_kv,
    const typename E::storage* __restrict__ k_rope, const int* __restrict__ seq_idx,
    const int* __restrict__ pos, int n, double base) {
  using T = typename E::storage;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= n) return;
  const int b = seq_idx[r];
  const int p = pos[r];
  if (b < 0 || b >= num_seqs || p < 0 || p / BLOCK >= max_blocks) return;
  const int blk = table[(long)b * max_blocks + p / BLOCK];
  if (blk < 0 || blk >= num_blocks) return;
  T* dst = cache + ((long)blk * BLOCK + (p % BLOCK)) * ROW;
  const T* src = c_kv + (long)r * D_C;
  // latent: 512 elements, 16-byte pieces
  constexpr int PER16 = 16 / E::bytes;            // elements per 16 bytes
  constexpr int PIECES = D_C / PER16;             // 64 (bf16) or 128 (fp32)
#pragma unroll
  for (int i = lane; i < PIECES; i += 64)
    reinterpret_cast<uint4*>(dst)[i] = reinterpret_cast<const uint4*>(src)[i];
  // rotated RoPE key
  if (lane < D_R / 2) {
    double c, s;
    rope_cs(p, lane, base, c, s);
    const T* kr = k_rope + (long)r * D_R;
    double x = E::to_f32(kr[2 * lane]), y = E::to_f32(kr[2 * lane + 1]);
    dst[D_C + 2 * lane] = E::from_f32((float)(x * c - y * s));
    dst[D_C + 2 * lane + 1] = E::from_f32((float)(x * s + y * c));
  }
}

hipError_t launch_kv_append(void* cache, int dtype, int num_blocks, const int* table,
                            int num_seqs, int max_blocks, const void* c_kv, const void* k_rope,
                            const int* seq_idx, const int* pos, int n, float base,
                            hipStream_t stream) {
  dim3 grid((n + 3) / 4), block(256);
  if (dtype == 1)
    hipLaunchKernelGGL(kv_append_kernel<BF16>, grid, block, 0, stream, (uint16_t*)cache,
                       num_blocks, table, num_seqs, max_blocks, (const uint16_t*)c_kv,
                       (const uint16_t*)k_rope, seq_idx, pos, n, (double)base);
  else
    hipLaunchKernelGGL(kv_append_kernel<F32>, grid, block, 0, stream, (float*)cache,
                       num_blocks, table, num_seqs, max_blocks, (const float*)c_kv,
                       (const float*)k_rope, seq_idx, pos, n, (double)base);
  return hipGetLastError();
}

}  // namespace mla
