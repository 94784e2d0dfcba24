// mla_decode_paged_noalloc: split-KV attention whose split partials live in a
// device array the library holds, for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc).
//
// The array below is a file-scope device variable: every GPU the library runs
// on holds its own copy from the moment the code object is loaded until the
// process ends.  In host code its name is only a stand-in for the symbol, not
// a device address, so the entry point looks the address up once per device
// with hipGetSymbolAddress (with that device current) and passes that pointer
// to the kernels, never the name.
//
// Same kernels as mla_decode_paged followed by mla_splitkv_combine.  Every
// call on one GPU uses that GPU's one array: two calls that overlap on one GPU
// (different streams, or different host threads) race on it.  Nothing in it
// has to start at zero: each split of each row writes its partial (an empty
// split writes o = 0 and lse = -inf) before the combine reads it.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "../../include/mla.h"
#include "mla_internal.h"

namespace {

static __device__ __align__(256) char scratch[MLA_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex scratch_mutex;
void* scratch_ptr[MAX_DEVICES] = {};   // device address of `scratch`, per device

// The current device's copy of the array (nullptr if the lookup failed).
void* device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return nullptr;
  std::lock_guard<std::mutex> lock(scratch_mutex);
  if (scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    scratch_ptr[dev] = p;
  }
  return scratch_ptr[dev];
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

}  // namespace

extern "C" int32_t mla_decode_paged_noalloc(const void* q_lat, const void* kv_cache,
                                            int32_t num_blocks, int32_t block_size,
                                            const int32_t* block_table, int32_t max_blocks,
                                            const int32_t* seq_lens, int32_t B, int32_t q_len,
                                            int32_t n_h, int32_t dtype, float softmax_scale,
                                            int32_t num_splits, float* o_lat, float* lse,
                                            void* stream) {
  if (dtype != MLA_F32 && dtype != MLA_BF16) return MLA_ERR_DTYPE;
  const bool heads_ok = n_h == 16 || n_h == 32 || (n_h > 0 && n_h % 64 == 0);
  if (B < 0 || q_len < 1 || num_blocks < 1 || max_blocks < 1 || block_size != MLA_BLOCK ||
      !heads_ok || num_splits < 1 || !(softmax_scale > 0.0f))
    return MLA_ERR_SHAPE;
  const int64_t rows = (int64_t)B * q_len * num_splits;
  if (rows > 0x7fffffffLL) return MLA_ERR_SHAPE;
  // partials: o [rows, n_h, 512] then lse [rows, n_h], fp32
  const int64_t o_bytes = rows * n_h * MLA_D_C * 4;
  const int64_t need = num_splits > 1 ? o_bytes + rows * n_h * 4 : 0;
  if (need > (int64_t)MLA_NOALLOC_SCRATCH_BYTES) return MLA_ERR_SCRATCH;
  if (B == 0) return MLA_OK;
  if (!q_lat || !kv_cache || !block_table || !seq_lens || !o_lat || !lse) return MLA_ERR_NULL;
  if (!aligned16(q_lat) || !aligned16(kv_cache) || !aligned16(o_lat) || !aligned4(lse))
    return MLA_ERR_ALIGN;
  const hipStream_t st = (hipStream_t)stream;
  if (num_splits == 1)
    return mla::launch_decode(q_lat, kv_cache, num_blocks, block_table, max_blocks, seq_lens, B,
                              q_len, n_h, dtype, softmax_scale, 1, nullptr, 0, nullptr, 0, o_lat,
                              lse, nullptr, nullptr, 0, st) == hipSuccess
               ? MLA_OK
               : MLA_ERR_HIP;
  char* base = static_cast<char*>(device_scratch());
  if (base == nullptr) return MLA_ERR_HIP;
  float* o_part = reinterpret_cast<float*>(base);
  float* lse_part = reinterpret_cast<float*>(base + o_bytes);
  if (mla::launch_decode(q_lat, kv_cache, num_blocks, block_table, max_blocks, seq_lens, B, q_len,
                         n_h, dtype, softmax_scale, num_splits, nullptr, 0, nullptr, 0, o_lat, lse,
                         o_part, lse_part, (int)rows, st) != hipSuccess)
    return MLA_ERR_HIP;
  return mla::launch_combine(o_part, lse_part, B, num_splits, q_len, n_h, o_lat, lse, st) ==
                 hipSuccess
             ? MLA_OK
             : MLA_ERR_HIP;
}
