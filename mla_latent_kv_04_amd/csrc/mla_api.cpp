// C ABI entry points (include/mla.h): host-side argument checks, then launch.
//
// Every check here runs before anything is enqueued, so a rejected call has
// no effect on the stream.  No entry point allocates, frees or synchronises.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <vector>

#include "../../include/mla.h"
#include "mla_internal.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
bool dtype_ok(int32_t dt) { return dt == MLA_F32 || dt == MLA_BF16; }

// Head counts the decode kernels are built for.
bool decode_heads_ok(int32_t n_h) { return n_h == 16 || n_h == 32 || (n_h > 0 && n_h % 64 == 0); }

int32_t hip_status(hipError_t e) { return e == hipSuccess ? MLA_OK : MLA_ERR_HIP; }

// Events armed by mla_time_attention, per host thread.
thread_local mla::KernelEvents armed_events{nullptr, nullptr};

}  // namespace

mla::KernelEvents mla::take_attention_events() {
  const KernelEvents ev = armed_events;
  armed_events = KernelEvents{nullptr, nullptr};
  return ev;
}

extern "C" {

const char* mla_status_string(int32_t status) {
  switch (status) {
    case MLA_OK: return "ok";
    case MLA_ERR_NULL: return "a required pointer is NULL";
    case MLA_ERR_SHAPE: return "a size is out of range or inconsistent";
    case MLA_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case MLA_ERR_DTYPE: return "unknown dtype";
    case MLA_ERR_HIP: return "the HIP runtime refused a launch";
    case MLA_ERR_SCRATCH: return "the problem needs more than the library's fixed scratch array";
    default: return "unknown status";
  }
}

int32_t mla_abi_version(void) { return MLA_ABI_VERSION; }

int32_t mla_time_attention(void* start_event, void* stop_event) {
  armed_events = mla::KernelEvents{(hipEvent_t)start_event, (hipEvent_t)stop_event};
  return MLA_OK;
}

int32_t mla_rope_theta(double base, double scale, double alpha, double beta, double orig_ctx,
                       double* theta) {
  if (!theta) return MLA_ERR_NULL;
  if (!(base > 1.0) || !std::isfinite(base) || !(scale >= 1.0) || !std::isfinite(scale) ||
      !(alpha >= 0.0) || !(beta > alpha) || !std::isfinite(beta) || !(orig_ctx > 0.0) ||
      !std::isfinite(orig_ctx))
    return MLA_ERR_SHAPE;
  const double two_pi = 6.283185307179586;
  for (int k = 0; k < 32; ++k) {
    const double f = std::pow(base, -(double)(2 * k) / 64.0);
    // turns the pair makes over the original window, and where that lies on
    // the ramp from alpha (interpolate fully) to beta (keep as is)
    const double turns = orig_ctx * f / two_pi;
    const double keep = std::min(1.0, std::max(0.0, (turns - alpha) / (beta - alpha)));
    theta[k] = keep * f + (1.0 - keep) * (f / scale);
  }
  return MLA_OK;
}

int32_t mla_kv_append(void* kv_cache, int32_t dtype, int32_t num_blocks, int32_t block_size,
                      const int32_t* block_table, int32_t num_seqs, int32_t max_blocks,
                      const void* c_kv, const void* k_rope, const int32_t* seq_idx,
                      const int32_t* pos, int32_t n, float rope_base, const double* rope_theta,
                      void* stream) {
  if (!dtype_ok(dtype)) return MLA_ERR_DTYPE;
  mla::RopeFreq rf;
  if (n < 0 || num_blocks < 1 || num_seqs < 1 || max_blocks < 1 || block_size != MLA_BLOCK ||
      !mla::rope_freq(rope_base, rope_theta, rf))
    return MLA_ERR_SHAPE;
  if (n == 0) return MLA_OK;
  if (!kv_cache || !block_table || !c_kv || !k_rope || !seq_idx || !pos) return MLA_ERR_NULL;
  if (!aligned16(kv_cache) || !aligned16(c_kv) || !aligned4(k_rope)) return MLA_ERR_ALIGN;
  return hip_status(mla::launch_kv_append(kv_cache, dtype, num_blocks, block_table, num_seqs,
                                          max_blocks, c_kv, k_rope, seq_idx, pos, n, rf,
                                          (hipStream_t)stream));
}

int32_t mla_absorb_q(const void* q_nope, const void* q_rope, const void* w_uk,
                     const int32_t* q_pos, int32_t T, int32_t n_h, int32_t dtype,
                     float rope_base, const double* rope_theta, void* q_lat, void* stream) {
  if (!dtype_ok(dtype)) return MLA_ERR_DTYPE;
  mla::RopeFreq rf;
  if (T < 0 || n_h < 16 || n_h % 16 != 0 || !mla::rope_freq(rope_base, rope_theta, rf))
    return MLA_ERR_SHAPE;
  if (T == 0) return MLA_OK;
  if (!q_nope || !q_rope || !w_uk || !q_pos || !q_lat) return MLA_ERR_NULL;
  if (!aligned16(q_nope) || !aligned16(w_uk) || !aligned16(q_lat) || !aligned4(q_rope))
    return MLA_ERR_ALIGN;
  return hip_status(mla::launch_absorb_q(q_nope, q_rope, w_uk, q_pos, T, n_h, dtype, rf, q_lat,
                                         (hipStream_t)stream));
}

int32_t mla_append_absorb_q(void* kv_cache, int32_t num_blocks, int32_t block_size,
                            const int32_t* block_table, int32_t num_seqs, int32_t max_blocks,
                            const void* c_kv, const void* k_rope, const int32_t* seq_idx,
                            const int32_t* pos, int32_t n, const void* q_nope,
                            const void* q_rope, const void* w_uk, const int32_t* q_pos,
                            int32_t T, int32_t n_h, int32_t dtype, float rope_base,
                            const double* rope_theta, void* q_lat, void* stream) {
  if (!dtype_ok(dtype)) return MLA_ERR_DTYPE;
  mla::RopeFreq rf;
  if (n < 0 || T < 0 || !mla::rope_freq(rope_base, rope_theta, rf)) return MLA_ERR_SHAPE;
  if (n > 0) {  // the checks of mla_kv_append
    if (num_blocks < 1 || num_seqs < 1 || max_blocks < 1 || block_size != MLA_BLOCK)
      return MLA_ERR_SHAPE;
    if (!kv_cache || !block_table || !c_kv || !k_rope || !seq_idx || !pos) return MLA_ERR_NULL;
    if (!aligned16(kv_cache) || !aligned16(c_kv) || !aligned4(k_rope)) return MLA_ERR_ALIGN;
  }
  if (T > 0) {  // the checks of mla_absorb_q
    if (n_h < 16 || n_h % 16 != 0) return MLA_ERR_SHAPE;
    if (!q_nope || !q_rope || !w_uk || !q_pos || !q_lat) return MLA_ERR_NULL;
    if (!aligned16(q_nope) || !aligned16(w_uk) || !aligned16(q_lat) || !aligned4(q_rope))
      return MLA_ERR_ALIGN;
  }
  if (n == 0 && T == 0) return MLA_OK;
  return hip_status(mla::launch_append_absorb(kv_cache, dtype, num_blocks, block_table, num_seqs,
                                              max_blocks, c_kv, k_rope, seq_idx, pos, n, q_nope,
                                              q_rope, w_uk, q_pos, T, n_h, rf, q_lat,
                                              (hipStream_t)stream));
}

int32_t mla_decode_paged(const void* q_lat, const void* kv_cache, int32_t num_blocks,
                         int32_t block_size, const int32_t* block_table, int32_t max_blocks,
                         const int32_t* seq_lens, int32_t B, int32_t q_len, int32_t n_h,
                         int32_t dtype, float softmax_scale, int32_t num_splits, float* o_part,
                         float* lse_part, float* o_lat, float* lse, void* stream) {
  if (!dtype_ok(dtype)) return MLA_ERR_DTYPE;
  if (B < 0 || q_len < 1 || num_blocks < 1 || max_blocks < 1 || block_size != MLA_BLOCK ||
      !decode_heads_ok(n_h) || num_splits < 1 || !(softmax_scale > 0.0f))
    return MLA_ERR_SHAPE;
  // grid.x = B * q_len * num_splits must fit the launch limit
  if ((int64_t)B * q_len * num_splits > 0x7fffffffLL) return MLA_ERR_SHAPE;
  if (B == 0) return MLA_OK;
  if (!q_lat || !kv_cache || !block_table || !seq_lens) return MLA_ERR_NULL;
  float* o_out = o_lat;
  float* l_out = lse;
  if (num_splits > 1) {
    if (!o_part || !lse_part) return MLA_ERR_NULL;
    o_out = o_part;
    l_out = lse_part;
  } else if (!o_lat || !lse) {
    return MLA_ERR_NULL;
  }
  if (!aligned16(q_lat) || !aligned16(kv_cache) || !aligned16(o_out) || !aligned4(l_out))
    return MLA_ERR_ALIGN;
  const int64_t n_parts = num_splits > 1 ? (int64_t)B * q_len * num_splits : 0;
  if (n_parts > 0x7fffffffLL) return MLA_ERR_SHAPE;
  return hip_status(mla::launch_decode(q_lat, kv_cache, num_blocks, block_table, max_blocks,
                                       seq_lens, B, q_len, n_h, dtype, softmax_scale, num_splits,
                                       nullptr, 0, nullptr, 0, o_lat, lse, o_part, lse_part,
                                       (int)n_parts, (hipStream_t)stream));
}

int32_t mla_kv_append_fp8(void* kv_cache, float* kv_scale, int32_t dtype, int32_t num_blocks,
                          int32_t block_size, const int32_t* block_table, int32_t num_seqs,
                          int32_t max_blocks, const void* c_kv, const void* k_rope,
                          const int32_t* seq_idx, const int32_t* pos, int32_t n, float rope_base,
                          const double* rope_theta, void* stream) {
  if (!dtype_ok(dtype)) return MLA_ERR_DTYPE;
  mla::RopeFreq rf;
  if (n < 0 || num_blocks < 1 || num_seqs < 1 || max_blocks < 1 || block_size != MLA_BLOCK ||
      !mla::rope_freq(rope_base, rope_theta, rf))
    return MLA_ERR_SHAPE;
  if (n == 0) return MLA_OK;
  if (!kv_cache || !kv_scale || !block_table || !c_kv || !k_rope || !seq_idx || !pos)
    return MLA_ERR_NULL;
  if (!aligned16(kv_cache) || !aligned16(kv_scale)) return MLA_ERR_ALIGN;
  return hip_status(mla::launch_kv_append_fp8(kv_cache, kv_scale, dtype, num_blocks, block_table,
                                              num_seqs, max_blocks, c_kv, k_rope, seq_idx, pos,
                                              n, rf, (hipStream_t)stream));
}

int32_t mla_decode_paged_fp8(const void* q_lat, const void* kv_cache, const float* kv_scale,
                             int32_t num_blocks, int32_t block_size, const int32_t* block_table,
                             int32_t max_blocks, const int32_t* seq_lens, int32_t B,
                             int32_t q_len, int32_t n_h, float softmax_scale, int32_t num_splits,
                             float* o_part, float* lse_part, float* o_lat, float* lse,
                             void* stream) {
  if (B < 0 || q_len < 1 || num_blocks < 1 || max_blocks < 1 || block_size != MLA_BLOCK ||
      !decode_heads_ok(n_h) || num_splits < 1 || !(softmax_scale > 0.0f))
    return MLA_ERR_SHAPE;
  if ((int64_t)B * q_len * num_splits > 0x7fffffffLL) return MLA_ERR_SHAPE;
  if (B == 0) return MLA_OK;
  if (!q_lat || !kv_cache || !kv_scale || !block_table || !seq_lens) return MLA_ERR_NULL;
  float* o_out = o_lat;
  float* l_out = lse;
  if (num_splits > 1) {
    if (!o_part || !lse_part) return MLA_ERR_NULL;
    o_out = o_part;
    l_out = lse_part;
  } else if (!o_lat || !lse) {
    return MLA_ERR_NULL;
  }
  if (!aligned16(q_lat) || !aligned16(kv_cache) || !aligned16(kv_scale) || !aligned16(o_out) ||
      !aligned4(l_out))
    return MLA_ERR_ALIGN;
  const int64_t n_parts = num_splits > 1 ? (int64_t)B * q_len * num_splits : 0;
  return hip_status(mla::launch_decode_fp8(q_lat, kv_cache, kv_scale, num_blocks, block_table,
                                           max_blocks, seq_lens, B, q_len, n_h, softmax_scale,
                                           num_splits, nullptr, 0, nullptr, 0, o_lat, lse, o_part,
                                           lse_part, (int)n_parts, (hipStream_t)stream));
}

int32_t mla_decode_paged_planned_fp8(const void* q_lat, const void* kv_cache,
                                     const float* kv_scale, int32_t num_blocks,
                                     int32_t block_size, const int32_t* block_table,
                                     int32_t max_blocks, int32_t B, int32_t q_len, int32_t n_h,
                                     float softmax_scale, const int32_t* work, int32_t n_work,
                                     const int32_t* lists, int32_t n_lists, float* o_part,
                                     float* lse_part, int32_t n_parts, float* o_lat, float* lse,
                                     void* stream) {
  if (B < 0 || q_len < 1 || num_blocks < 1 || max_blocks < 1 || block_size != MLA_BLOCK ||
      !decode_heads_ok(n_h) || n_work < 0 || n_parts < 0 || !(softmax_scale > 0.0f) ||
      (lists && n_lists < 1))
    return MLA_ERR_SHAPE;
  if ((int64_t)B * q_len > 0x7fffffffLL) return MLA_ERR_SHAPE;
  if (n_work == 0 || B == 0) return MLA_OK;
  if (!q_lat || !kv_cache || !kv_scale || !block_table || !work || !o_lat || !lse)
    return MLA_ERR_NULL;
  if (n_parts > 0 && (!o_part || !lse_part)) return MLA_ERR_NULL;
  if (!aligned16(q_lat) || !aligned16(kv_cache) || !aligned16(kv_scale) || !aligned16(o_lat) ||
      !aligned4(lse) || !aligned16(work) || (o_part && !aligned16(o_part)) ||
      (lse_part && !aligned4(lse_part)))
    return MLA_ERR_ALIGN;
  return hip_status(mla::launch_decode_fp8(q_lat, kv_cache, kv_scale, num_blocks, block_table,
                                           max_blocks, nullptr, B, q_len, n_h, softmax_scale, 1,
                                           work, n_work, lists, lists ? n_lists : 0, o_lat, lse,
                                           o_part, lse_part, n_parts, (hipStream_t)stream));
}

int32_t mla_plan_decode(const int32_t* seq_lens, int32_t B, int32_t q_len, int32_t block_size,
                        int32_t n_h, int32_t num_slots, int32_t max_work, int32_t* work,
                        int32_t* n_work, int32_t* lists, int32_t* n_lists, int32_t* split,
                        int32_t* n_split, int32_t* n_parts) {
  if (B < 0 || q_len < 1 || block_size != MLA_BLOCK || n_h < 1 || num_slots < 1 || max_work < 0)
    return MLA_ERR_SHAPE;
  if (!n_work || !n_lists || !n_split || !n_parts) return MLA_ERR_NULL;
  if (B > 0 && !seq_lens) return MLA_ERR_NULL;
  const int64_t rows = (int64_t)B * q_len;
  if (rows > 0x7fffffffLL) return MLA_ERR_SHAPE;
  // visible keys and blocks per row, and each row's first position in the
  // concatenation of all rows' blocks
  std::vector<int64_t> nkeys(rows), tiles(rows), start(rows);
  int64_t total = 0;
  for (int64_t r = 0; r < rows; ++r) {
    const int64_t L = std::max<int64_t>(0, seq_lens[r / q_len]);
    const int64_t m = r % q_len;
    nkeys[r] = std::max<int64_t>(0, std::min<int64_t>(L, L - (q_len - 1 - m)));
    tiles[r] = (nkeys[r] + block_size - 1) / block_size;
    start[r] = total;
    total += tiles[r];
  }
  const int64_t groups = (n_h % 64 == 0) ? n_h / 64 : 1;
  const int64_t K = total > 0 ? std::max<int64_t>(1, std::min<int64_t>(num_slots / groups, total)) : 1;
  // List capacity W: the least for which the greedy walk below fills at most
  // K lists, where a list's cost is its blocks plus C per segment.
  const int64_t C = MLA_PLAN_SEGMENT_COST;
  auto walk = [&](int64_t W, std::vector<int64_t>* starts) {
    int64_t used = 0, pos = 0, r = 0;
    while (pos < total) {
      if (starts) starts->push_back(pos);
      if (++used > K && !starts) return used;
      int64_t cost = 0;
      while (pos < total) {
        while (start[r] + tiles[r] <= pos) ++r;   // the row holding block pos
        const int64_t rest = start[r] + tiles[r] - pos;
        if (cost + C + rest <= W) {
          cost += C + rest;
          pos += rest;
          continue;
        }
        if (W - cost - C >= 1) pos += W - cost - C;
        break;
      }
    }
    return used;
  };
  int64_t lo = C + 1, hi = C + 1;
  for (int64_t r = 0; r < rows; ++r) hi += tiles[r] > 0 ? C + tiles[r] : 0;
  while (lo < hi) {
    const int64_t mid = lo + (hi - lo) / 2;
    if (walk(mid, nullptr) <= K) hi = mid; else lo = mid + 1;
  }
  // list k covers concatenated blocks [bnd[k], bnd[k + 1]); unused lists are empty
  std::vector<int64_t> bnd;
  if (total > 0) walk(lo, &bnd);
  bnd.resize(K + 1, total);
  auto bound = [&](int64_t k) { return bnd[k]; };
  auto list_of = [&](int64_t pos) {  // the last list starting at or before block pos (pos < total)
    return (int64_t)(std::upper_bound(bnd.begin(), bnd.begin() + K, pos) - bnd.begin()) - 1;
  };
  struct Seg { int64_t list, row, kb, ke, slot; };
  std::vector<Seg> segs;
  std::vector<int64_t> splits;   // {row, first slot, pieces} per split row, in row order
  int64_t parts = 0;
  for (int64_t r = 0; r < rows; ++r) {
    if (tiles[r] == 0) {   // a row with no key still gets its (empty) output written
      segs.push_back({std::min(K - 1, total > 0 && start[r] < total ? list_of(start[r]) : K - 1), r,
                      0, 0, -1});
      continue;
    }
    const int64_t k0 = list_of(start[r]), k1 = list_of(start[r] + tiles[r] - 1);
    const int64_t P = k1 - k0 + 1;
    if (P > 1) splits.insert(splits.end(), {r, parts, P});
    for (int64_t k = k0; k <= k1; ++k) {
      const int64_t t0 = std::max(bound(k), start[r]) - start[r];
      const int64_t t1 = std::min(bound(k + 1), start[r] + tiles[r]) - start[r];
      segs.push_back({k, r, t0 * block_size, std::min(t1 * block_size, nkeys[r]),
                      P > 1 ? parts + (k - k0) : -1});
    }
    if (P > 1) parts += P;
  }
  const int64_t count = (int64_t)segs.size(), nsplit = (int64_t)splits.size() / 3;
  if (count > 0x7fffffffLL) return MLA_ERR_SHAPE;
  *n_work = (int32_t)count;
  *n_lists = (int32_t)K;
  *n_split = (int32_t)nsplit;
  *n_parts = (int32_t)parts;
  if (count > max_work || nsplit > max_work) return MLA_ERR_SHAPE;
  if (count > 0 && !work) return MLA_ERR_NULL;
  if (!lists) return MLA_ERR_NULL;
  if (nsplit > 0 && !split) return MLA_ERR_NULL;
  // by list, then by row: a list's segments are consecutive rows
  std::stable_sort(segs.begin(), segs.end(), [](const Seg& a, const Seg& b) {
    if (a.list != b.list) return a.list < b.list;
    return a.row < b.row;
  });
  int64_t li = 0;
  for (int64_t i = 0; i < count; ++i) {
    while (li <= segs[i].list) lists[li++] = (int32_t)i;
    work[i * 4] = (int32_t)segs[i].row;
    work[i * 4 + 1] = (int32_t)segs[i].kb;
    work[i * 4 + 2] = (int32_t)segs[i].ke;
    work[i * 4 + 3] = (int32_t)segs[i].slot;
  }
  while (li <= K) lists[li++] = (int32_t)count;
  for (int64_t i = 0; i < 3 * nsplit; ++i) split[i] = (int32_t)splits[i];
  return MLA_OK;
}

int32_t mla_decode_paged_planned(const void* q_lat, const void* kv_cache, int32_t num_blocks,
                                 int32_t block_size, const int32_t* block_table,
                                 int32_t max_blocks, int32_t B, int32_t q_len, int32_t n_h,
                                 int32_t dtype, float softmax_scale, const int32_t* work,
                                 int32_t n_work, const int32_t* lists, int32_t n_lists,
                                 float* o_part, float* lse_part, int32_t n_parts, float* o_lat,
                                 float* lse, void* stream) {
  if (!dtype_ok(dtype)) return MLA_ERR_DTYPE;
  if (B < 0 || q_len < 1 || num_blocks < 1 || max_blocks < 1 || block_size != MLA_BLOCK ||
      !decode_heads_ok(n_h) || n_work < 0 || n_parts < 0 || !(softmax_scale > 0.0f) ||
      (lists && n_lists < 1))
    return MLA_ERR_SHAPE;
  if ((int64_t)B * q_len > 0x7fffffffLL) return MLA_ERR_SHAPE;
  if (n_work == 0 || B == 0) return MLA_OK;
  if (!q_lat || !kv_cache || !block_table || !work || !o_lat || !lse) return MLA_ERR_NULL;
  if (n_parts > 0 && (!o_part || !lse_part)) return MLA_ERR_NULL;
  if (!aligned16(q_lat) || !aligned16(kv_cache) || !aligned16(o_lat) || !aligned4(lse) ||
      !aligned16(work) || (o_part && !aligned16(o_part)) || (lse_part && !aligned4(lse_part)))
    return MLA_ERR_ALIGN;
  return hip_status(mla::launch_decode(q_lat, kv_cache, num_blocks, block_table, max_blocks,
                                       nullptr, B, q_len, n_h, dtype, softmax_scale, 1, work,
                                       n_work, lists, lists ? n_lists : 0, o_lat, lse, o_part,
                                       lse_part, n_parts, (hipStream_t)stream));
}

int32_t mla_combine_planned(const float* o_part, const float* lse_part, const int32_t* split,
                            int32_t n_split, int32_t n_h, float* o_lat, float* lse, void* stream) {
  if (n_split < 0 || n_h < 1) return MLA_ERR_SHAPE;
  if (n_split == 0) return MLA_OK;
  if (!o_part || !lse_part || !split || !o_lat) return MLA_ERR_NULL;
  if (!aligned16(o_part) || !aligned16(o_lat) || !aligned4(lse_part) || (lse && !aligned4(lse)))
    return MLA_ERR_ALIGN;
  return hip_status(mla::launch_combine_planned(o_part, lse_part, split, n_split, n_h, o_lat, lse,
                                                (hipStream_t)stream));
}

int32_t mla_splitkv_combine(const float* o_part, const float* lse_part, int32_t B, int32_t S,
                            int32_t q_len, int32_t n_h, float* o_lat, float* lse, void* stream) {
  if (B < 0 || S < 1 || q_len < 1 || n_h < 1) return MLA_ERR_SHAPE;
  if ((int64_t)B * q_len > 0x7fffffffLL) return MLA_ERR_SHAPE;
  if (B == 0) return MLA_OK;
  if (!o_part || !lse_part || !o_lat) return MLA_ERR_NULL;
  if (!aligned16(o_part) || !aligned16(o_lat) || !aligned4(lse_part) || (lse && !aligned4(lse)))
    return MLA_ERR_ALIGN;
  return hip_status(mla::launch_combine(o_part, lse_part, B, S, q_len, n_h, o_lat, lse,
                                        (hipStream_t)stream));
}

int32_t mla_out_proj(const float* o_lat, const void* w_uv, int32_t T, int32_t n_h, int32_t dtype,
                     float* out, void* stream) {
  if (!dtype_ok(dtype)) return MLA_ERR_DTYPE;
  if (T < 0 || n_h < 1) return MLA_ERR_SHAPE;
  if (T == 0) return MLA_OK;
  if (!o_lat || !w_uv || !out) return MLA_ERR_NULL;
  if (!aligned16(o_lat) || !aligned16(w_uv) || !aligned16(out)) return MLA_ERR_ALIGN;
  return hip_status(mla::launch_out_proj(o_lat, w_uv, T, n_h, dtype, out, (hipStream_t)stream));
}

int32_t mla_out_proj_planned(float* o_lat, const float* o_part, const float* lse_part,
                             const int32_t* split, int32_t n_split, const void* w_uv, int32_t T,
                             int32_t n_h, int32_t dtype, float* out, float* lse, void* stream) {
  if (!dtype_ok(dtype)) return MLA_ERR_DTYPE;
  if (T < 0 || n_h < 1 || n_split < 0 || n_split > T) return MLA_ERR_SHAPE;
  if (T == 0) return MLA_OK;
  if (!o_lat || !w_uv || !out) return MLA_ERR_NULL;
  if (n_split > 0 && (!o_part || !lse_part || !split)) return MLA_ERR_NULL;
  if (!aligned16(o_lat) || !aligned16(w_uv) || !aligned16(out)) return MLA_ERR_ALIGN;
  if (n_split > 0 && (!aligned16(o_part) || !aligned4(lse_part) || (lse && !aligned4(lse))))
    return MLA_ERR_ALIGN;
  return hip_status(mla::launch_out_proj_planned(o_lat, o_part, lse_part, split, n_split, w_uv, T,
                                                 n_h, dtype, out, lse, (hipStream_t)stream));
}

int32_t mla_split_plan(const int32_t* seq_lens, int32_t B, int32_t block_size, int32_t num_splits,
                       int32_t* begin_end) {
  if (B < 0 || num_splits < 1 || block_size != MLA_BLOCK) return MLA_ERR_SHAPE;
  if (B == 0) return MLA_OK;
  if (!seq_lens || !begin_end) return MLA_ERR_NULL;
  for (int32_t b = 0; b < B; ++b)
    if (seq_lens[b] < 0) return MLA_ERR_SHAPE;
  for (int32_t b = 0; b < B; ++b) {
    const int64_t L = seq_lens[b];
    const int64_t nblk = (L + block_size - 1) / block_size;
    const int64_t c = (nblk + num_splits - 1) / num_splits;
    for (int32_t s = 0; s < num_splits; ++s) {
      int64_t lo = s * c * block_size, hi = (s + 1) * c * block_size;
      if (lo > L) lo = L;
      if (hi > L) hi = L;
      begin_end[((int64_t)b * num_splits + s) * 2] = (int32_t)lo;
      begin_end[((int64_t)b * num_splits + s) * 2 + 1] = (int32_t)hi;
    }
  }
  return MLA_OK;
}

}  // extern "C"
