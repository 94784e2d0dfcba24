// Log-sum-exp merge of split-KV partial results (combine.hip, and the
// few-row merge-and-project kernel of out_proj.hip).
//
// Softmax over a union of disjoint key sets is recovered exactly from the
// per-set results: LSE = log sum_s exp(lse_s), o = sum_s exp(lse_s - LSE) o_s
// (an identity of eq. 7's softmax, DeepSeek-V2 notes, irregular6612.github.io,
// §2.1.1).  Splits that saw no key carry lse = -inf and weight 0.
#pragma once

#include "mla_common.h"

namespace mla {

namespace {

constexpr int MERGE_BATCH = 16;

// Over parts k = 0..count-1 at p(k) (element offsets of the lse entries; the
// output row is D_C floats per lse entry): m = max_k lse_k, z = sum_k w_k and
// o = sum_k w_k x_k with w_k = exp(lse_k - m); a part with lse -inf weighs
// nothing, and m stays -inf (z = 0) when every part does.
template <class PartAt>
__device__ __forceinline__ void merge_parts(const float* __restrict__ o_part,
                                            const float* __restrict__ lse_part, int count,
                                            PartAt part_at, int d4, float4& o, float& z, float& m) {
  for (int k0 = 0; k0 < count; k0 += MERGE_BATCH) {
    float l[MERGE_BATCH];
    float4 x[MERGE_BATCH];
#pragma unroll
    for (int u = 0; u < MERGE_BATCH; ++u) {
      l[u] = -INFINITY;
      x[u] = float4{0, 0, 0, 0};
      if (k0 + u < count) {
        const long pr = part_at(k0 + u);
        l[u] = lse_part[pr];
        x[u] = reinterpret_cast<const float4*>(o_part + pr * D_C)[d4];
      }
    }
    float mb = m;
#pragma unroll
    for (int u = 0; u < MERGE_BATCH; ++u) mb = fmaxf(mb, l[u]);
    if (mb == -INFINITY) continue;
    if (mb > m) {
      const float f = m == -INFINITY ? 0.0f : __expf(m - mb);
      z *= f;
      o.x *= f; o.y *= f; o.z *= f; o.w *= f;
      m = mb;
    }
#pragma unroll
    for (int u = 0; u < MERGE_BATCH; ++u) {
      if (l[u] == -INFINITY) continue;
      const float w = __expf(l[u] - m);
      z += w;
      o.x += w * x[u].x; o.y += w * x[u].y; o.z += w * x[u].z; o.w += w * x[u].w;
    }
  }
}

}  // namespace

}  // namespace mla
