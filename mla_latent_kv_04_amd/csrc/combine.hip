// Split-KV combine: merge per-split normalised outputs by their log-sum-exps.
//
// Softmax over a union of disjoint key sets is recovered exactly from the
// per-set results: LSE = log sum_s exp(lse_s), o = sum_s exp(lse_s - LSE) o_s
// (an identity of eq. 7's softmax, DeepSeek-V2 notes, irregular6612.github.io,
// §2.1.1).  Splits that saw no key carry lse = -inf and weight 0.
//
// One workgroup per (row, pair of heads); a thread owns 4 of the 512 dims.
// This pass is bandwidth bound: it reads S x 2 KB per head once.  The parts
// are read MERGE_BATCH at a time, their lse and data loads all in flight
// together, and summed in part order against a running maximum (what is
// summed so far is rescaled when a batch raises it), so a row of up to
// MERGE_BATCH parts costs one round trip to memory.
#include "merge_parts.h"
#include "mla_common.h"
#include "mla_internal.h"

namespace mla {

namespace {

__global__ void __launch_bounds__(256) combine_kernel(const float* __restrict__ o_part,
                                                      const float* __restrict__ lse_part, int S,
                                                      int q_len, int n_h, float* __restrict__ o_lat,
                                                      float* __restrict__ lse) {
  const int head = blockIdx.y * 2 + (threadIdx.x >> 7);
  const int d4 = threadIdx.x & 127;
  const int row = blockIdx.x;             // b * q_len + m
  if (head >= n_h) return;
  const int b = row / q_len, m = row % q_len;
  // partial (b, s, m, head) lives at ((b * S + s) * q_len + m) * n_h + head
  const long step = (long)q_len * n_h;    // distance between consecutive splits
  const long p0 = ((long)b * S * q_len + m) * n_h + head;
  float4 o = {0, 0, 0, 0};
  float z = 0.0f, mx = -INFINITY;
  merge_parts(o_part, lse_part, S, [&](int s) { return p0 + s * step; }, d4, o, z, mx);
  const float inv = z > 0.0f ? 1.0f / z : 0.0f;
  reinterpret_cast<float4*>(o_lat + ((long)row * n_h + head) * D_C)[d4] =
      float4{o.x * inv, o.y * inv, o.z * inv, o.w * inv};
  if (lse != nullptr && d4 == 0) lse[(long)row * n_h + head] = z > 0.0f ? mx + __logf(z) : -INFINITY;
}

// Planned merge: split[j] = {row, first_slot, count}; partial rows are
// first_slot .. first_slot + count - 1 of o_part / lse_part ([slots, n_h, ...]).
__global__ void __launch_bounds__(256) combine_planned_kernel(
    const float* __restrict__ o_part, const float* __restrict__ lse_part,
    const int* __restrict__ split, int n_h, float* __restrict__ o_lat, float* __restrict__ lse) {
  const int head = blockIdx.y * 2 + (threadIdx.x >> 7);
  const int d4 = threadIdx.x & 127;
  if (head >= n_h) return;
  const int row = split[blockIdx.x * 3], first = split[blockIdx.x * 3 + 1];
  const int count = split[blockIdx.x * 3 + 2];
  float4 o = {0, 0, 0, 0};
  float z = 0.0f, mx = -INFINITY;
  merge_parts(o_part, lse_part, count, [&](int k) { return (long)(first + k) * n_h + head; }, d4,
              o, z, mx);
  const float inv = z > 0.0f ? 1.0f / z : 0.0f;
  reinterpret_cast<float4*>(o_lat + ((long)row * n_h + head) * D_C)[d4] =
      float4{o.x * inv, o.y * inv, o.z * inv, o.w * inv};
  if (lse != nullptr && d4 == 0) lse[(long)row * n_h + head] = z > 0.0f ? mx + __logf(z) : -INFINITY;
}

}  // namespace

hipError_t launch_combine_planned(const float* o_part, const float* lse_part, const int* split,
                                  int n_split, int n_h, float* o_lat, float* lse,
                                  hipStream_t stream) {
  if (n_split == 0) return hipSuccess;
  dim3 grid((unsigned)n_split, (n_h + 1) / 2), block(256);
  hipLaunchKernelGGL(combine_planned_kernel, grid, block, 0, stream, o_part, lse_part, split, n_h,
                     o_lat, lse);
  return hipGetLastError();
}

hipError_t launch_combine(const float* o_part, const float* lse_part, int B, int S, int q_len,
                          int n_h, float* o_lat, float* lse, hipStream_t stream) {
  dim3 grid((unsigned)B * q_len, (n_h + 1) / 2), block(256);
  hipLaunchKernelGGL(combine_kernel, grid, block, 0, stream, o_part, lse_part, S, q_len, n_h, o_lat,
                     lse);
  return hipGetLastError();
}

}  // namespace mla
