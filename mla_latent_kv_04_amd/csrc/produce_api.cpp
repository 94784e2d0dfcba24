// C ABI entry points of the producers (include/mla.h): host-side argument
// checks, then launch.  As for the other entry points, every check runs
// before anything is enqueued, and nothing is allocated, freed or
// synchronised: the split-K partials and c^Q live in the caller's workspace.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mla.h"
#include "mla_internal.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
bool dtype_ok(int32_t dt) { return dt == MLA_F32 || dt == MLA_BF16; }
int32_t hip_status(hipError_t e) { return e == hipSuccess ? MLA_OK : MLA_ERR_HIP; }

// A producer operand of rows x cols elements addresses its bytes with 32-bit
// offsets: rows * cols * 4 must stay below 2^31.
bool fits_2g(int64_t rows, int64_t cols) { return rows * cols * 4 < (int64_t(1) << 31); }

}  // namespace

extern "C" {

int64_t mla_kv_produce_workspace(int32_t T, int32_t d_model) {
  if (T < 0 || d_model < 64 || d_model % 64 != 0) return -1;
  return mla::kv_produce_workspace(T, d_model);
}

int32_t mla_kv_produce(const void* h, const void* w_dkv, const float* kv_gain, const void* w_kr,
                       int32_t T, int32_t d_model, int32_t dtype, float eps, float rope_base,
                       void* kv_cache, int32_t num_blocks, int32_t block_size,
                       const int32_t* block_table, int32_t num_seqs, int32_t max_blocks,
                       const int32_t* seq_idx, const int32_t* pos, void* workspace,
                       int64_t workspace_bytes, void* stream) {
  if (!dtype_ok(dtype)) return MLA_ERR_DTYPE;
  if (T < 0 || d_model < 64 || d_model % 64 != 0 || !(eps >= 0.0f) || !(rope_base > 0.0f) ||
      num_blocks < 1 || block_size != MLA_BLOCK || num_seqs < 1 || max_blocks < 1)
    return MLA_ERR_SHAPE;
  if (T == 0) return MLA_OK;
  if (!h || !w_dkv || !kv_gain || !w_kr || !kv_cache || !block_table || !seq_idx || !pos ||
      !workspace)
    return MLA_ERR_NULL;
  if (workspace_bytes < mla::kv_produce_workspace(T, d_model)) return MLA_ERR_SHAPE;
  if (!fits_2g(T, d_model)) return MLA_ERR_SHAPE;
  if (!aligned16(h) || !aligned16(w_dkv) || !aligned16(w_kr) || !aligned16(kv_cache) ||
      !aligned16(workspace) || !aligned4(kv_gain))
    return MLA_ERR_ALIGN;
  return hip_status(mla::launch_kv_produce(h, w_dkv, kv_gain, w_kr, T, d_model, dtype, eps,
                                           rope_base, kv_cache, num_blocks, block_table,
                                           num_seqs, max_blocks, seq_idx, pos, workspace,
                                           (hipStream_t)stream));
}

int64_t mla_q_produce_workspace(int32_t T, int32_t d_model, int32_t d_cq, int32_t dtype) {
  if (T < 0 || d_model < 64 || d_model % 64 != 0 || d_cq < 64 || d_cq % 64 != 0 ||
      d_cq > 2048 || !dtype_ok(dtype))
    return -1;
  return mla::q_produce_workspace(T, d_model, d_cq, dtype);
}

int32_t mla_q_produce(const void* h, const void* w_dq, const float* q_gain, const void* w_uq,
                      const void* w_qr, int32_t T, int32_t d_model, int32_t d_cq, int32_t n_h,
                      int32_t dtype, float eps, void* q_nope, void* q_rope, void* workspace,
                      int64_t workspace_bytes, void* stream) {
  if (!dtype_ok(dtype)) return MLA_ERR_DTYPE;
  if (T < 0 || d_model < 64 || d_model % 64 != 0 || d_cq < 64 || d_cq % 64 != 0 ||
      d_cq > 2048 || n_h < 1 || !(eps >= 0.0f))
    return MLA_ERR_SHAPE;
  if (T == 0) return MLA_OK;
  if (!h || !w_dq || !q_gain || !w_uq || !w_qr || !q_nope || !q_rope || !workspace)
    return MLA_ERR_NULL;
  if (workspace_bytes < mla::q_produce_workspace(T, d_model, d_cq, dtype)) return MLA_ERR_SHAPE;
  if (!fits_2g(T, d_model) || !fits_2g(T, d_cq) || !fits_2g((int64_t)n_h * 128, d_cq))
    return MLA_ERR_SHAPE;
  if (!aligned16(h) || !aligned16(w_dq) || !aligned16(w_uq) || !aligned16(w_qr) ||
      !aligned16(workspace) || !aligned4(q_gain) || !aligned16(q_nope) || !aligned16(q_rope))
    return MLA_ERR_ALIGN;
  return hip_status(mla::launch_q_produce(h, w_dq, q_gain, w_uq, w_qr, T, d_model, d_cq, n_h,
                                          dtype, eps, q_nope, q_rope, workspace,
                                          (hipStream_t)stream));
}

}  // extern "C"
