// Host-side launchers of the MLA kernels (one per kernel file).  They assume
// arguments were validated by the C entry points and only enqueue work.
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>

namespace mla {

// Kernel timing (mla_time_attention).  The events this thread armed, taken
// (and disarmed) by its next attention launch; both null when none are armed.
struct KernelEvents {
  hipEvent_t start, stop;
};
KernelEvents take_attention_events();

// RoPE pair frequencies theta_k (radians per position) of the 64-wide
// decoupled key, k = 0..31, passed by value to the kernels that rotate.
struct RopeFreq {
  double theta[32];
};

// Plain RoPE, theta_k = base^(-2k/64), when `theta` is null; otherwise a copy
// of the caller's table (e.g. YaRN's).  False if base or an entry is not a
// finite positive number.
inline bool rope_freq(float base, const double* theta, RopeFreq& rf) {
  for (int k = 0; k < 32; ++k) {
    rf.theta[k] = theta ? theta[k] : std::pow((double)base, -(double)(2 * k) / 64.0);
    if (!(std::isfinite(rf.theta[k]) && rf.theta[k] > 0.0)) return false;
  }
  return true;
}

hipError_t launch_kv_append(void* cache, int dtype, int num_blocks, const int* table,
                            int num_seqs, int max_blocks, const void* c_kv, const void* k_rope,
                            const int* seq_idx, const int* pos, int n, const RopeFreq& rf,
                            hipStream_t stream);

// FP8 E4M3 cache: rows of 576 code bytes [num_blocks, 64, 576] and two
// float32 scales per row (latent, RoPE) [num_blocks, 64, 2].
hipError_t launch_kv_append_fp8(void* cache, float* kv_scale, int dtype, int num_blocks,
                                const int* table, int num_seqs, int max_blocks, const void* c_kv,
                                const void* k_rope, const int* seq_idx, const int* pos, int n,
                                const RopeFreq& rf, hipStream_t stream);

hipError_t launch_absorb_q(const void* q_nope, const void* q_rope, const void* w_uk,
                           const int* q_pos, int T, int n_h, int dtype, const RopeFreq& rf,
                           void* q_lat, hipStream_t stream);

// launch_kv_append and launch_absorb_q of one step, in one launch for bf16
// (absorb_q.hip); either part may be empty (n == 0 or T == 0).
hipError_t launch_append_absorb(void* cache, int dtype, int num_blocks, const int* table,
                                int num_seqs, int max_blocks, const void* c_kv,
                                const void* k_rope, const int* seq_idx, const int* pos, int n,
                                const void* q_nope, const void* q_rope, const void* w_uk,
                                const int* q_pos, int T, int n_h, const RopeFreq& rf,
                                void* q_lat, hipStream_t stream);

// Paged attention.  Uniform splits when work == nullptr (S splits per row,
// partials at row (b * S + s) * q_len + m when S > 1), else a work list of
// n_work int4 {row, key_begin, key_end, slot}; n_parts bounds the slots (an
// item with slot >= n_parts is skipped).  With lists != nullptr the
// items lists[k] .. lists[k+1]-1 (k < n_lists) are run in order by one
// workgroup per head group (a scheduling hint: kernels that do not use it run
// one item per workgroup, with the same results).
hipError_t launch_decode(const void* q_lat, const void* cache, int num_blocks, const int* table,
                         int max_blocks, const int* seq_lens, int B, int q_len, int n_h,
                         int dtype, float scale, int S, const int* work, int n_work,
                         const int* lists, int n_lists, float* o_lat, float* lse, float* o_part,
                         float* lse_part, int n_parts, hipStream_t stream);

// bf16, n_h a multiple of 64 (decode_h64.hip); same arguments.
hipError_t launch_decode_h64(const void* q_lat, const void* cache, int num_blocks,
                             const int* table, int max_blocks, const int* seq_lens, int B,
                             int q_len, int n_h, float scale, int S, const int* work, int n_work,
                             const int* lists, int n_lists, float* o_lat, float* lse,
                             float* o_part, float* lse_part, int n_parts, hipStream_t stream);

// FP8 E4M3 cache with per-row scales; queries bf16; any head count the bf16
// kernels take.  16 and 32 heads: decode_fp8.hip, one item per workgroup;
// multiples of 64: decode_h64_fp8.hip, the two-role design with 64-token tiles
// (lists as there).
hipError_t launch_decode_fp8(const void* q_lat, const void* cache, const float* kv_scale,
                             int num_blocks, const int* table, int max_blocks,
                             const int* seq_lens, int B, int q_len, int n_h, float scale, int S,
                             const int* work, int n_work, const int* lists, int n_lists,
                             float* o_lat, float* lse, float* o_part, float* lse_part,
                             int n_parts, hipStream_t stream);
hipError_t launch_decode_h64_fp8(const void* q_lat, const void* cache, const float* kv_scale,
                                 int num_blocks, const int* table, int max_blocks,
                                 const int* seq_lens, int B, int q_len, int n_h, float scale, int S,
                                 const int* work, int n_work, const int* lists, int n_lists,
                                 float* o_lat, float* lse, float* o_part, float* lse_part,
                                 int n_parts, hipStream_t stream);

hipError_t launch_combine(const float* o_part, const float* lse_part, int B, int S, int q_len,
                          int n_h, float* o_lat, float* lse, hipStream_t stream);

// Merge the partials of split rows: split[j] = {row, first_slot, count}.
hipError_t launch_combine_planned(const float* o_part, const float* lse_part, const int* split,
                                  int n_split, int n_h, float* o_lat, float* lse,
                                  hipStream_t stream);

hipError_t launch_out_proj(const float* o_lat, const void* w_uv, int T, int n_h, int dtype,
                           float* out, hipStream_t stream);

hipError_t launch_out_proj_planned(float* o_lat, const float* o_part, const float* lse_part,
                                   const int* split, int n_split, const void* w_uv, int T, int n_h,
                                   int dtype, float* out, float* lse, hipStream_t stream);

// Producers (produce.hip).  Workspace bytes as returned by the *_workspace
// functions, 256-byte aligned.
long kv_produce_workspace(int T, int d_model);
long q_produce_workspace(int T, int d_model, int d_cq, int dtype);
hipError_t launch_kv_produce(const void* h, const void* w_dkv, const float* kv_gain,
                             const void* w_kr, int T, int d_model, int dtype, float eps,
                             const RopeFreq& rf, void* cache, int num_blocks, const int* table,
                             int num_seqs, int max_blocks, const int* seq_idx, const int* pos,
                             void* workspace, hipStream_t stream);
hipError_t launch_q_produce(const void* h, const void* w_dq, const float* q_gain,
                            const void* w_uq, const void* w_qr, int T, int d_model, int d_cq,
                            int n_h, int dtype, float eps, void* q_nope, void* q_rope,
                            void* workspace, hipStream_t stream);

hipError_t launch_q_produce_direct(const void* h, const void* w_qc, const void* w_qr, int T,
                                   int d_model, int n_h, int dtype, void* q_nope, void* q_rope,
                                   hipStream_t stream);

// eq. 8's output projection (produce.hip).
long o_proj_workspace(int T, int n_h, int d_model, int dtype);
hipError_t launch_o_proj(const float* out, const void* w_o, int T, int n_h, int d_model,
                         int dtype, void* u, void* workspace, hipStream_t stream);

// Non-absorbed chunked prefill (prefill_mha.hip), bf16.  seq_lens is a host
// array; the workspace holds k^C and v^C^T of the longest sequence.
long prefill_mha_workspace(int max_len, int n_h);
hipError_t launch_prefill_mha(const void* q_nope, const void* q_rope, const int* q_pos,
                              const void* w_uk, const void* w_uv, const void* cache,
                              int num_blocks, const int* table, int max_blocks,
                              const int* seq_lens, int B, int q_len, int n_h, float scale,
                              const RopeFreq& rf, float* out, float* lse, void* workspace,
                              hipStream_t stream);

}  // namespace mla
