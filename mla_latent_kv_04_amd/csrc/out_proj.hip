// Output projection o[t, i] = W^UV_i o_lat[t, i] (W^UV applied after the softmax
// sum instead of to every cached latent; eq. 11 of the DeepSeek-V2 notes,
// irregular6612.github.io, §2.1.2, moved by associativity as the DeepSeek-V2
// MLA blog, adg.csdn.net, part 2 §2.2.1.1, describes).
//
// Per head: out^T[d, t] = sum_c W^UV_i[d, c] o_lat[t, i, c], M = 128 (d),
// N = T, K = 512.  Both operands have the reduced axis c contiguous, so MFMA
// fragments load straight from memory.  For bf16 weights the fp32 latent
// output is split as hi + lo with hi = bf16(x), lo = bf16(x - hi) and both
// halves are multiplied (16 significant bits of o_lat instead of 8).
// One workgroup per (head, 64 rows); wave w owns output rows d in [32w, 32w+32).
#include "mla_common.h"
#include "mla_internal.h"

namespace mla {

namespace {

constexpr int TCH = 64;

template <class E> struct LatFrag;

template <> struct LatFrag<BF16> {
  static constexpr int parts = 2;
  __device__ static void load(const float* p, bool ok, BF16::frag* f) {
    float x[8];
    if (ok) {
      const float4 a = reinterpret_cast<const float4*>(p)[0], b = reinterpret_cast<const float4*>(p)[1];
      x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = 0.0f;
    }
    float lo[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float hi = bf16_to_f32(f32_to_bf16(x[j]));
      lo[j] = x[j] - hi;
      x[j] = hi;
    }
    f[0] = BF16::from8(x);
    f[1] = BF16::from8(lo);
  }
};

template <> struct LatFrag<F32> {
  static constexpr int parts = 1;
  __device__ static void load(const float* p, bool ok, F32::frag* f) {
    if (ok) {
      f[0] = F32::load8(p);
    } else {
      float z[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      f[0] = F32::from8(z);
    }
  }
};

template <class E>
__global__ void __launch_bounds__(256) out_proj_kernel(const float* __restrict__ o_lat,
                                                       const typename E::storage* __restrict__ w_uv,
                                                       int T, int n_h, float* __restrict__ out) {
  const int h = blockIdx.x, t0 = blockIdx.y * TCH;
  const int lane = lane_id(), wave = threadIdx.x >> 6, g = lane >> 4, r16 = lane & 15;
  constexpr int P = LatFrag<E>::parts;
  f32x4_t acc[2][4];
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) acc[db][tb] = f32x4_t{0, 0, 0, 0};
  const typename E::storage* wh = w_uv + (long)h * D_H * D_C;
#pragma unroll 2
  for (int ks = 0; ks < D_C / 32; ++ks) {
    typename E::frag wf[2];
#pragma unroll
    for (int db = 0; db < 2; ++db)
      wf[db] = E::load8(wh + (long)(wave * 32 + db * 16 + r16) * D_C + ks * 32 + 8 * g);
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      const int t = t0 + tb * 16 + r16;
      typename E::frag lf[P];
      LatFrag<E>::load(o_lat + ((long)t * n_h + h) * D_C + ks * 32 + 8 * g, t < T, lf);
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int q = 0; q < P; ++q) E::mma(acc[db][tb], wf[db], lf[q]);
    }
  }
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) {
    const int t = t0 + tb * 16 + r16;
    if (t >= T) continue;
#pragma unroll
    for (int db = 0; db < 2; ++db)
      *reinterpret_cast<float4*>(out + ((long)t * n_h + h) * D_H + wave * 32 + db * 16 + 4 * g) =
          float4{acc[db][tb][0], acc[db][tb][1], acc[db][tb][2], acc[db][tb][3]};
  }
}

}  // namespace

hipError_t launch_out_proj(const float* o_lat, const void* w_uv, int T, int n_h, int dtype,
                           float* out, hipStream_t stream) {
  dim3 grid(n_h, (T + TCH - 1) / TCH), block(256);
  if (dtype == 1)
    hipLaunchKernelGGL(out_proj_kernel<BF16>, grid, block, 0, stream, o_lat,
                       (const uint16_t*)w_uv, T, n_h, out);
  else
    hipLaunchKernelGGL(out_proj_kernel<F32>, grid, block, 0, stream, o_lat, (const float*)w_uv, T,
                       n_h, out);
  return hipGetLastError();
}

}  // namespace mla
