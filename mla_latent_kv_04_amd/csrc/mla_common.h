// Device-side building blocks shared by the MLA kernels (gfx950 / CDNA4).
//
// Element types: the cache, queries and weights are either fp32 or bf16
// (stored as raw 16-bit patterns).  Accumulation is always fp32.
//
// MFMA fragments: every contraction here is cut into steps of 32 along the
// reduced axis.  In one step a lane of a 64-lane wave holds 8 consecutive
// elements of the reduced axis (lane group g = lane / 16 holds elements
// 8g..8g+7) for one row (lane % 16) of a 16-row operand.  Both operands of a
// product use the same layout, so any assignment of reduced-axis elements to
// (g, slot) is a valid dot product as long as both sides agree.
//   bf16: one v_mfma_f32_16x16x32_bf16 per step.
//   fp32: eight v_mfma_f32_16x16x4_f32 per step (slot j of every lane group
//         forms the 4-element reduction of instruction j).
// The 16x16 fp32 result: lane l holds column l % 16, rows 4*(l/16) + i, i<4.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

constexpr int D_C = 512;          // latent width
constexpr int D_R = 64;           // decoupled RoPE width
constexpr int D_H = 128;          // per-head width
constexpr int ROW = D_C + D_R;    // elements per cached row
constexpr int BLOCK = 64;         // tokens per paged block
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(8 * sizeof(short)))) short i16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(((uint32_t)h) << 16);
}

// Round to nearest even (the hardware v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(uint16_t, b);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

// ---------------------------------------------------------------------------
// Element traits.
// ---------------------------------------------------------------------------
struct F32 {
  using storage = float;
  static constexpr int bytes = 4;
  // One 8-element fragment of the reduced axis.
  struct frag { float v[8]; };
  __device__ static float load(const float* p, long i) { return p[i]; }
  __device__ static float to_f32(float x) { return x; }
  __device__ static float from_f32(float x) { return x; }
  // the value an fp32 number takes as an MFMA operand of this type
  __device__ static float round(float x) { return x; }
  __device__ static void mma(f32x4_t& acc, const frag& a, const frag& b) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[j], b.v[j], acc, 0, 0, 0);
  }
  // 8 consecutive elements from memory (LDS or global), 16-byte aligned.
  __device__ static frag load8(const float* p) {
    frag f;
    const float4* q = reinterpret_cast<const float4*>(p);
    float4 x = q[0], y = q[1];
    f.v[0] = x.x; f.v[1] = x.y; f.v[2] = x.z; f.v[3] = x.w;
    f.v[4] = y.x; f.v[5] = y.y; f.v[6] = y.z; f.v[7] = y.w;
    return f;
  }
  __device__ static frag from8(const float* x) {
    frag f;
#pragma unroll
    for (int j = 0; j < 8; ++j) f.v[j] = x[j];
    return f;
  }
};

struct BF16 {
  using storage = uint16_t;
  static constexpr int bytes = 2;
  struct frag { i16x8_t v; };
  __device__ static float load(const uint16_t* p, long i) { return bf16_to_f32(p[i]); }
  __device__ static float to_f32(uint16_t x) { return bf16_to_f32(x); }
  __device__ static uint16_t from_f32(float x) { return f32_to_bf16(x); }
  __device__ static float round(float x) { return bf16_to_f32(f32_to_bf16(x)); }
  __device__ static void mma(f32x4_t& acc, const frag& a, const frag& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16((bf16x8_t)a.v, (bf16x8_t)b.v, acc, 0, 0, 0);
  }
  __device__ static frag load8(const uint16_t* p) {
    frag f;
    f.v = *reinterpret_cast<const i16x8_t*>(p);
    return f;
  }
  __device__ static frag from8(const float* x) {
    frag f;
#pragma unroll
    for (int j = 0; j < 8; ++j) f.v[j] = (short)f32_to_bf16(x[j]);
    return f;
  }
};

// Wave-wide helpers -----------------------------------------------------------
__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63); }

__device__ __forceinline__ float xor_shfl(float v, int mask) {
  int src = (lane_id() ^ mask) << 2;
  return __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(v)));
}

// Max / sum over the four lanes that share lane % 16 (lanes l, l^16, l^32,
// l^48), without going through LDS: with both operands the same register,
// v_permlane16_swap leaves lane l holding its own value and that of lane l^16
// (one in each result), and v_permlane32_swap does the same for lane l^32.
__device__ __forceinline__ float group4_max(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float group4_sum(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Workgroup barrier for LDS traffic only.  __syncthreads() carries a memory
// fence, and the compiler then waits for every outstanding global load first,
// including direct global->LDS loads of the next tile that are meant to stay
// in flight.  Here only this wave's LDS operations are waited for.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");       // keep LDS accesses on their side of the barrier
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt untouched
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Wait for this wave's vector-memory loads (the tile's direct-to-LDS loads),
// then a full workgroup barrier.
__device__ __forceinline__ void tile_barrier() {
  __builtin_amdgcn_s_waitcnt(0xF70);   // vmcnt(0)
  __syncthreads();
}

// RoPE pair at position pos with frequency theta (radians per position):
// cos/sin of pos * theta, with the angle formed and evaluated in float64
// (fp32 angles lose ~1e-2 rad near 128K).
__device__ __forceinline__ void rope_cs(int pos, double theta, double& c, double& s) {
  sincos((double)pos * theta, &s, &c);
}

// One unit of attention work: query row (b, m) against keys [kb, ke) of
// sequence b, written to row `orow` of o_lat (part == false) or of the split
// partials (part == true).
struct WorkItem {
  int b, m, kb, ke;
  long orow;
  bool part;
  bool valid;
};

// Uniform split-KV (work == nullptr): item = (b * q_len + m) * S + s, split s of
// sequence b's blocks cut into S runs of ceil(nblk / S) blocks.  Planned
// (work != nullptr): work[item] = {row, key_begin, key_end, slot}; an item
// whose row is outside [0, n_rows) or whose slot is >= n_parts is skipped
// (nothing is written for it).
__device__ __forceinline__ WorkItem decode_item(int item, const int4* work, int n_rows,
                                                int n_parts, int q_len, int S,
                                                const int* seq_lens, int max_blocks) {
  WorkItem w;
  const int cap = max_blocks * BLOCK;
  if (work != nullptr) {
    const int4 v = work[item];
    w.valid = v.x >= 0 && v.x < n_rows && v.w < n_parts;
    const int row = w.valid ? v.x : 0;
    w.b = row / q_len;
    w.m = row % q_len;
    w.kb = max(0, min(v.y, cap));
    w.ke = max(w.kb, min(v.z, cap));
    w.part = v.w >= 0;
    w.orow = w.part ? (long)v.w : (long)row;
    return w;
  }
  const int s = item % S, bm = item / S;
  w.valid = true;
  w.m = bm % q_len;
  w.b = bm / q_len;
  const int L = max(0, min(seq_lens[w.b], cap));
  const int nvis = max(0, min(L, L - (q_len - 1 - w.m)));
  const int nblk = (L + BLOCK - 1) / BLOCK;
  const int cpb = (nblk + S - 1) / S;
  w.kb = min(s * cpb * BLOCK, nvis);
  w.ke = min((s + 1) * cpb * BLOCK, nvis);
  w.part = S > 1;
  w.orow = w.part ? ((long)(w.b * S + s) * q_len + w.m) : (long)(w.b * q_len + w.m);
  return w;
}

}  // namespace mla
