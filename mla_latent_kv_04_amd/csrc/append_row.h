// One cache row of the KV append (kv_append.hip, and the fused append + absorb
// launch of absorb_q.hip): the cache keeps [c^KV ; R_pos k^R] per token, the
// compressed latent unrotated and the decoupled RoPE key already rotated at
// the token's position (DeepSeek-V2 MLA blog, adg.csdn.net, part 2 §2.2.2).
#pragma once

#include "mla_common.h"
#include "mla_internal.h"

namespace mla {

// Input row r (< n) by one wave: the 512 latent elements are copied with
// 16-byte loads and stores, 32 lanes rotate one RoPE pair each in float64.
// Rows whose sequence, position or block id is out of range are skipped.
template <class E>
__device__ __forceinline__ void append_row(
    typename E::storage* __restrict__ cache, int num_blocks, const int* __restrict__ table,
    int num_seqs, int max_blocks, const typename E::storage* __restrict__ c_kv,
    const typename E::storage* __restrict__ k_rope, const int* __restrict__ seq_idx,
    const int* __restrict__ pos, int r, int lane, const RopeFreq& rf) {
  using T = typename E::storage;
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
    rope_cs(p, rf.theta[lane], c, s);
    const T* kr = k_rope + (long)r * D_R;
    double x = E::to_f32(kr[2 * lane]), y = E::to_f32(kr[2 * lane + 1]);
    dst[D_C + 2 * lane] = E::from_f32((float)(x * c - y * s));
    dst[D_C + 2 * lane + 1] = E::from_f32((float)(x * s + y * c));
  }
}

}  // namespace mla
