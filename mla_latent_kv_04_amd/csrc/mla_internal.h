// Host-side launchers of the MLA kernels (one per kernel file).  They assume
// arguments were validated by the C entry points and only enqueue work.
#pragma once

#include <hip/hip_runtime.h>

namespace mla {

hipError_t launch_kv_append(void* cache, int dtype, int num_blocks, const int* table,
                            int num_seqs, int max_blocks, const void* c_kv, const void* k_rope,
                            const int* seq_idx, const int* pos, int n, float base,
                            hipStream_t stream);

hipError_t launch_absorb_q(const void* q_nope, const void* q_rope, const void* w_uk,
                           const int* q_pos, int T, int n_h, int dtype, float base, void* q_lat,
                           hipStream_t stream);

hipError_t launch_decode(const void* q_lat, const void* cache, int num_blocks, const int* table,
                         int max_blocks, const int* seq_lens, int B, int q_len, int n_h,
                         int dtype, float scale, int num_splits, float* o_out, float* lse_out,
                         hipStream_t stream);

hipError_t launch_combine(const float* o_part, const float* lse_part, int B, int S, int q_len,
                          int n_h, float* o_lat, float* lse, hipStream_t stream);

hipError_t launch_out_proj(const float* o_lat, const void* w_uv, int T, int n_h, int dtype,
                           float* out, hipStream_t stream);

}  // namespace mla
