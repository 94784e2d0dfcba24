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
// One workgroup per (head, 64 rows).  bf16 weights: the head's W^UV (128 x
// 512, 128 KB at a 1040-byte row pitch, which puts the 16 rows of an MFMA
// fragment read on disjoint banks) is staged in LDS once; wave w owns query
// rows 16w .. 16w + 15 of the chunk and all 128 outputs, so every o_lat
// element is read from memory once.  fp32 weights (too large to stage):
// wave w owns output rows d in [32w, 32w+32) and reads both operands from
// memory.
//
// The planned variant also finishes a balanced split-KV schedule: a row that
// the schedule cut into several key ranges has its partial outputs merged
// with the log-sum-exp rule (each part weighted by exp(lse_k - LSE)) as the
// row's o_lat operand is loaded, so the merged row never goes to memory.
#include "merge_parts.h"
#include "mla_common.h"
#include "mla_internal.h"

namespace mla {

namespace {

constexpr int TCH = 64;

template <class E> struct LatFrag;

template <> struct LatFrag<BF16> {
  static constexpr int parts = 2;
  __device__ static void load(const float* p, bool ok, BF16::frag* f) {
    if (ok)
      split(reinterpret_cast<const float4*>(p)[0], reinterpret_cast<const float4*>(p)[1], f);
    else
      split(float4{0, 0, 0, 0}, float4{0, 0, 0, 0}, f);
  }
  __device__ static void split(const float4& a, const float4& b, BF16::frag* f) {
    float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
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

constexpr int WPITCH = D_C * 2 + 16;   // bytes per staged bf16 W^UV row

// One direct-to-LDS load: lane l's 16 bytes from base + lane_off land at LDS
// byte lds_dst + 16 l (M0 holds the LDS address; one wait state before use).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // M0 is named as clobbered on purpose
__device__ __forceinline__ void dma_row(unsigned lds_dst, const char* base, unsigned lane_off) {
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %2"
      :
      : "v"(lane_off), "s"(lds_dst), "s"(base)
      : "m0");
}
#pragma clang diagnostic pop

// A split-KV schedule's split rows: split[j] = {row, first part, parts}, in
// increasing row order; part k of row j is o_part / lse_part row first + k.
struct SplitRows {
  const float* o_part;
  const float* lse_part;
  const int* split;
  int n_split;
  float* lse;
};

// Split entry {first part, parts} of row t, or parts = 0 if row t is not
// split; tw (uniform) is the first of the 16 rows this wave loads,
// t = tw + (lane & 15).  A 64-way search finds the first entry with row >= tw
// (one round per factor of 64 entries); rows are distinct, so the wave's
// split rows are among the 16 entries from there.
struct SplitEntry {
  int first, parts;
};
__device__ __forceinline__ SplitEntry split_entry(const int* __restrict__ split, int n_split,
                                                  int tw, int t) {
  const int lane = lane_id();
  int lo = 0, len = n_split;   // the answer is lo + #{entries in [lo, lo + len) below tw}
  while (len > 0) {
    const int step = (len + 63) >> 6;
    const int off = lane * step;
    const bool below = off < len && split[3 * (lo + off)] < tw;
    const int c = __popcll(__ballot(below));   // samples are sorted: a prefix is below
    if (c == 0) break;
    const int nlo = lo + (c - 1) * step + 1;
    len = min(lo + c * step, lo + len) - nlo;
    lo = nlo;
  }
  const int j = lo + (lane & 15);
  int row_j = -1, first_j = 0, parts_j = 0;
  if (j < n_split) {
    row_j = split[3 * j];
    first_j = split[3 * j + 1];
    parts_j = split[3 * j + 2];
  }
  SplitEntry e{0, 0};
#pragma unroll
  for (int i = 0; i < 16; ++i)
    if (__builtin_amdgcn_readlane(row_j, i) == t)
      e = SplitEntry{__builtin_amdgcn_readlane(first_j, i), __builtin_amdgcn_readlane(parts_j, i)};
  return e;
}

// Workgroup (h, y) runs row chunks y, y + gridDim.y, ... of head h against
// one staged copy of W^UV_h.  PLANNED: rows listed in sp are merged from
// their partial outputs (and their log-sum-exp written to sp.lse); the other
// rows are read from o_lat.
template <bool PLANNED>
__global__ void __launch_bounds__(256) out_proj_bf16_kernel(const float* __restrict__ o_lat,
                                                            const uint16_t* __restrict__ w_uv,
                                                            int T, int n_h, float* __restrict__ out,
                                                            SplitRows sp) {
  __shared__ __attribute__((aligned(16))) char wl[D_H * WPITCH];   // [128][WPITCH]
  const int h = blockIdx.x;
  const int lane = lane_id(), wave = threadIdx.x >> 6, g = lane >> 4, r16 = lane & 15;

  // This lane's o_lat operand (query row t, columns 32ks + 8g .. +7 for all
  // 16 k-steps), loaded whole: one workgroup fits a CU, so registers are
  // plentiful, and the first chunk's loads land while W^UV is staged.
  float4 raw[D_C / 32][2];
  auto load_plain = [&](int t) __attribute__((always_inline)) {
    const bool ok = t < T;
    const float4* lrow = reinterpret_cast<const float4*>(o_lat + ((long)t * n_h + h) * D_C + 8 * g);
#pragma unroll
    for (int ks = 0; ks < D_C / 32; ++ks) {
      raw[ks][0] = ok ? lrow[ks * 8] : float4{0, 0, 0, 0};
      raw[ks][1] = ok ? lrow[ks * 8 + 1] : float4{0, 0, 0, 0};
    }
  };
  // Split row: o = sum_k exp(lse_k - LSE) o_k with LSE = log sum_k exp(lse_k);
  // parts with lse_k = -inf weigh nothing, and a row whose parts are all
  // empty gets o = 0, LSE = -inf.  Registers hold the row and half of one
  // more part: the first four lse_k, part 0 (or the o_lat row of a row that
  // is not split) and the first half of part 1 are loaded together, then one
  // half part at a time.
  float4 tmp[D_C / 64][2];
  auto load_merged = [&](int t) __attribute__((always_inline)) {
    const int tw = __builtin_amdgcn_readfirstlane(t - r16);
    const SplitEntry se = tw < T ? split_entry(sp.split, sp.n_split, tw, t) : SplitEntry{0, 0};
    const bool merged = se.parts > 0;
    const int parts = merged ? se.parts : (t < T ? 1 : 0);
    const long pstride = (long)n_h * D_C;   // floats between consecutive parts
    const float* p0 = (merged ? sp.o_part + ((long)se.first * n_h + h) * D_C
                              : o_lat + ((long)t * n_h + h) * D_C) + 8 * g;
    const float* l0 = sp.lse_part + (long)se.first * n_h + h;
    float l[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) l[k] = merged && k < parts ? l0[(long)k * n_h] : -INFINITY;
#pragma unroll
    for (int ks = 0; ks < D_C / 32; ++ks) {
      const float4* src = reinterpret_cast<const float4*>(p0 + ks * 32);
      raw[ks][0] = parts > 0 ? src[0] : float4{0, 0, 0, 0};
      raw[ks][1] = parts > 0 ? src[1] : float4{0, 0, 0, 0};
    }
    auto load_half = [&](int k, int half) __attribute__((always_inline)) {
      const float* pk = p0 + k * pstride + half * (D_C / 2);
#pragma unroll
      for (int i = 0; i < D_C / 64; ++i) {
        const float4* src = reinterpret_cast<const float4*>(pk + i * 32);
        tmp[i][0] = k < parts ? src[0] : float4{0, 0, 0, 0};
        tmp[i][1] = k < parts ? src[1] : float4{0, 0, 0, 0};
      }
    };
    load_half(1, 0);
    if (!merged) return;
    float m = -INFINITY, z = 0.0f;   // running max and sum of exp(lse_k - m)
    auto add_lse = [&](float lk) __attribute__((always_inline)) {
      if (lk == -INFINITY) return;
      if (lk > m) {
        z = z * __expf(m - lk) + 1.0f;
        m = lk;
      } else {
        z += __expf(lk - m);
      }
    };
#pragma unroll
    for (int k = 0; k < 4; ++k) add_lse(l[k]);
    for (int k = 4; k < parts; ++k) add_lse(l0[(long)k * n_h]);
    const float inv = z > 0.0f ? 1.0f / z : 0.0f;
    auto weight = [&](int k) __attribute__((always_inline)) {
      const float lk = k == 0 ? l[0] : k == 1 ? l[1] : k == 2 ? l[2] : k == 3 ? l[3]
                                                                       : l0[(long)k * n_h];
      return lk == -INFINITY ? 0.0f : __expf(lk - m) * inv;
    };
    const float w0 = weight(0);
    if (w0 == 0.0f) {
#pragma unroll
      for (int ks = 0; ks < D_C / 32; ++ks) raw[ks][0] = raw[ks][1] = float4{0, 0, 0, 0};
    } else {
#pragma unroll
      for (int ks = 0; ks < D_C / 32; ++ks)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          raw[ks][q].x *= w0;
          raw[ks][q].y *= w0;
          raw[ks][q].z *= w0;
          raw[ks][q].w *= w0;
        }
    }
    for (int k = 1; k < parts; ++k) {
      const float w = weight(k);
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        if (half == 1 || k > 1) load_half(k, half);
        if (w != 0.0f) {
#pragma unroll
          for (int i = 0; i < D_C / 64; ++i)
#pragma unroll
            for (int q = 0; q < 2; ++q) {
              float4& r = raw[half * (D_C / 64) + i][q];
              r.x += w * tmp[i][q].x;
              r.y += w * tmp[i][q].y;
              r.z += w * tmp[i][q].z;
              r.w += w * tmp[i][q].w;
            }
        }
      }
    }
    if (sp.lse != nullptr && g == 0) sp.lse[(long)t * n_h + h] = z > 0.0f ? m + __logf(z) : -INFINITY;
  };
  auto load_rows = [&](int t) __attribute__((always_inline)) {
    if constexpr (PLANNED)
      load_merged(t);
    else
      load_plain(t);
  };
  // stage W^UV_h with direct-to-LDS loads, all in flight at once: one
  // 64-lane instruction moves one 1024-byte row into its padded LDS row;
  // wave w moves rows w, w + 4, ...
  auto stage_w = [&]() __attribute__((always_inline)) {
    const char* wh = reinterpret_cast<const char*>(w_uv + (long)h * D_H * D_C);
    const unsigned wl_base = (unsigned)(uintptr_t)(__attribute__((address_space(3))) char*)wl;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
#pragma unroll 8
    for (int r = wave_u; r < D_H; r += 4)
      dma_row(wl_base + r * WPITCH, wh + (long)r * D_C * 2, lane * 16);
  };
  // (the rows first: with the weights first, measured 2% slower even where
  // the rows take a few dependent loads)
  load_rows(blockIdx.y * TCH + wave * 16 + r16);
  stage_w();
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's rows (and o_lat loads) landed
  __syncthreads();

  for (int t0 = blockIdx.y * TCH; t0 < T; t0 += gridDim.y * TCH) {
  // the weight fragments do not depend on the chunk: keep the compiler from
  // hoisting all 128 of them (512 registers) out of this loop
  asm volatile("" ::: "memory");
  const int t = t0 + wave * 16 + r16;
  // D[d][t] = sum_c W[d][c] o_lat[t][c]: A = W rows d (LDS), B = o_lat rows t
  // split into bf16 hi + lo.
  f32x4_t acc[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) acc[db] = f32x4_t{0, 0, 0, 0};
#pragma unroll
  for (int ks = 0; ks < D_C / 32; ++ks) {
    BF16::frag lf[2];
    LatFrag<BF16>::split(raw[ks][0], raw[ks][1], lf);
    const char* wp = wl + r16 * WPITCH + (ks * 32 + 8 * g) * 2;
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      BF16::frag wf;
      wf.v = *reinterpret_cast<const i16x8_t*>(wp + db * 16 * WPITCH);
      BF16::mma(acc[db], wf, lf[0]);
      BF16::mma(acc[db], wf, lf[1]);
    }
  }
  // the next chunk's rows, while this one's outputs are written
  if (t0 + gridDim.y * TCH < T) load_rows(t + gridDim.y * TCH);
  // lane holds t = r16 and d = 16db + 4g + i
  if (t < T) {
    float* orow = out + ((long)t * n_h + h) * D_H + 4 * g;
#pragma unroll
    for (int db = 0; db < 8; ++db)
      *reinterpret_cast<float4*>(orow + db * 16) =
          float4{acc[db][0], acc[db][1], acc[db][2], acc[db][3]};
  }
  }
}

// Few query rows (T <= SMALL_T, bf16 weights): one wave per (head h, 16
// outputs d0 .. d0 + 15, 16 rows t0 .. t0 + 15), so that the grid still
// spreads over the chip.  The wave's 16 rows of W^UV_h and its 16 o_lat rows
// (as bf16 hi + lo) are all loaded at once, straight from memory, then 32
// MFMAs; each W^UV row is read by T / 16 waves, each o_lat row by 8.
constexpr int SMALL_T = 64;

__global__ void __launch_bounds__(64) out_proj_small_kernel(const float* __restrict__ o_lat,
                                                            const uint16_t* __restrict__ w_uv,
                                                            int T, int n_h,
                                                            float* __restrict__ out) {
  const int h = blockIdx.x, d0 = blockIdx.y * 16, t0 = blockIdx.z * 16;
  const int lane = lane_id(), g = lane >> 4, r16 = lane & 15;
  const int t = t0 + r16;
  const uint16_t* wrow = w_uv + ((long)h * D_H + d0 + r16) * D_C + 8 * g;
  const float* lrow = o_lat + ((long)t * n_h + h) * D_C + 8 * g;
  BF16::frag wf[D_C / 32];
  float4 lat[D_C / 32][2];
#pragma unroll
  for (int ks = 0; ks < D_C / 32; ++ks) {
    wf[ks] = BF16::load8(wrow + ks * 32);
    lat[ks][0] = t < T ? reinterpret_cast<const float4*>(lrow + ks * 32)[0] : float4{0, 0, 0, 0};
    lat[ks][1] = t < T ? reinterpret_cast<const float4*>(lrow + ks * 32)[1] : float4{0, 0, 0, 0};
  }
  f32x4_t acc = {0, 0, 0, 0};
#pragma unroll
  for (int ks = 0; ks < D_C / 32; ++ks) {
    BF16::frag lf[2];
    LatFrag<BF16>::split(lat[ks][0], lat[ks][1], lf);
    BF16::mma(acc, wf[ks], lf[0]);
    BF16::mma(acc, wf[ks], lf[1]);
  }
  // lane holds row t and outputs d0 + 4g .. d0 + 4g + 3
  if (t < T)
    *reinterpret_cast<float4*>(out + ((long)t * n_h + h) * D_H + d0 + 4 * g) =
        float4{acc[0], acc[1], acc[2], acc[3]};
}

// Few rows under a split-KV plan (T <= SMALL_T, bf16 weights): merge and
// project in one launch.  Workgroup (h, SMALL_ROWS-row block): its threads
// first put the block's o_lat rows in LDS, one (row, 4 dims) each -- a split
// row merged from its parts (merge_parts, as combine_planned_kernel does; its
// LSE written to lse), any other row copied from o_lat -- then wave w
// multiplies W^UV_h rows 16w .. 16w + 15 by them with the MFMA sequence of
// out_proj_small_kernel (bf16 hi + lo).  The merged row takes the same values
// as through memory, so the outputs equal merge-then-project bit for bit.
constexpr int SMALL_ROWS = 4;
constexpr int LAT_PITCH = D_C + 4;        // floats per LDS row (rows 4 banks apart)

__global__ void __launch_bounds__(512) out_proj_small_planned_kernel(
    const float* __restrict__ o_lat, const float* __restrict__ o_part,
    const float* __restrict__ lse_part, const int* __restrict__ split, int n_split,
    const uint16_t* __restrict__ w_uv, int T, int n_h, float* __restrict__ out,
    float* __restrict__ lse) {
  static_assert(SMALL_ROWS * (D_C / 4) == 512, "one (row, 4 dims) per thread");
  __shared__ __attribute__((aligned(16))) float lat[SMALL_ROWS][LAT_PITCH];
  __shared__ int entry[SMALL_ROWS];
  const int h = blockIdx.x, t0 = blockIdx.y * SMALL_ROWS;
  const int tid = threadIdx.x;
  if (tid < SMALL_ROWS) entry[tid] = -1;
  __syncthreads();
  // split-table entries of the block's rows (rows are distinct)
  for (int j = tid; j < n_split; j += 512) {
    const int r = split[3 * j];
    if (r >= t0 && r < t0 + SMALL_ROWS) entry[r - t0] = j;
  }
  __syncthreads();
  {
    const int i = tid >> 7, d4 = tid & 127;
    const int t = t0 + i;
    float4 v = {0, 0, 0, 0};
    if (t < T) {
      const int j = entry[i];
      if (j >= 0) {
        const int first = split[3 * j + 1], count = split[3 * j + 2];
        float4 o = {0, 0, 0, 0};
        float z = 0.0f, mx = -INFINITY;
        merge_parts(o_part, lse_part, count, [&](int k) { return (long)(first + k) * n_h + h; },
                    d4, o, z, mx);
        const float inv = z > 0.0f ? 1.0f / z : 0.0f;
        v = float4{o.x * inv, o.y * inv, o.z * inv, o.w * inv};
        if (lse != nullptr && d4 == 0)
          lse[(long)t * n_h + h] = z > 0.0f ? mx + __logf(z) : -INFINITY;
      } else {
        v = reinterpret_cast<const float4*>(o_lat + ((long)t * n_h + h) * D_C)[d4];
      }
    }
    *reinterpret_cast<float4*>(&lat[i][4 * d4]) = v;
  }
  __syncthreads();
  const int lane = lane_id(), wave = tid >> 6, g = lane >> 4, r16 = lane & 15;
  const int d0 = 16 * wave;
  const uint16_t* wrow = w_uv + ((long)h * D_H + d0 + r16) * D_C + 8 * g;
  BF16::frag wf[D_C / 32];
#pragma unroll
  for (int ks = 0; ks < D_C / 32; ++ks) wf[ks] = BF16::load8(wrow + ks * 32);
  const bool row_ok = r16 < SMALL_ROWS;     // B rows past the block are zero
  f32x4_t acc = {0, 0, 0, 0};
#pragma unroll
  for (int ks = 0; ks < D_C / 32; ++ks) {
    const float* lp = &lat[row_ok ? r16 : 0][ks * 32 + 8 * g];
    const float4 a = row_ok ? reinterpret_cast<const float4*>(lp)[0] : float4{0, 0, 0, 0};
    const float4 b = row_ok ? reinterpret_cast<const float4*>(lp)[1] : float4{0, 0, 0, 0};
    BF16::frag lf[2];
    LatFrag<BF16>::split(a, b, lf);
    BF16::mma(acc, wf[ks], lf[0]);
    BF16::mma(acc, wf[ks], lf[1]);
  }
  // lane holds row t0 + r16 and outputs d0 + 4g .. d0 + 4g + 3
  const int t = t0 + r16;
  if (row_ok && t < T)
    *reinterpret_cast<float4*>(out + ((long)t * n_h + h) * D_H + d0 + 4 * g) =
        float4{acc[0], acc[1], acc[2], acc[3]};
}

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
  if (dtype == 1 && T <= SMALL_T) {
    hipLaunchKernelGGL(out_proj_small_kernel, dim3(n_h, D_H / 16, (T + 15) / 16), dim3(64), 0,
                       stream, o_lat, (const uint16_t*)w_uv, T, n_h, out);
    return hipGetLastError();
  }
  if (dtype == 1) {
    // about two workgroups per CU of (head, chunk) pairs; each stages W^UV_h
    // once for all of its chunks
    const int chunks = (T + TCH - 1) / TCH;
    const int per_wg = max(1, (chunks * n_h + 511) / 512);
    hipLaunchKernelGGL(out_proj_bf16_kernel<false>, dim3(n_h, (chunks + per_wg - 1) / per_wg),
                       block, 0, stream, o_lat, (const uint16_t*)w_uv, T, n_h, out, SplitRows{});
  } else
    hipLaunchKernelGGL(out_proj_kernel<F32>, grid, block, 0, stream, o_lat, (const float*)w_uv, T,
                       n_h, out);
  return hipGetLastError();
}

hipError_t launch_out_proj_planned(float* o_lat, const float* o_part, const float* lse_part,
                                   const int* split, int n_split, const void* w_uv, int T, int n_h,
                                   int dtype, float* out, float* lse, hipStream_t stream) {
  const long small_wgs = (long)n_h * ((T + SMALL_ROWS - 1) / SMALL_ROWS);
  if (dtype == 1 && n_split > 0 && T <= SMALL_T && small_wgs >= 256) {
    // few rows, enough (head, row block) pairs to fill the chip: merge and
    // project in one launch.  With fewer (a handful of rows cut into many
    // parts, as at 128K) the merge pass below spreads the parts over more
    // workgroups: 9.9 against 15.5 us for 4 rows x 128 heads in ~64 parts.
    hipLaunchKernelGGL(out_proj_small_planned_kernel,
                       dim3(n_h, (T + SMALL_ROWS - 1) / SMALL_ROWS), dim3(512), 0, stream, o_lat,
                       o_part, lse_part, split, n_split, (const uint16_t*)w_uv, T, n_h, out, lse);
    return hipGetLastError();
  }
  if (dtype != 1 || n_split == 0 || T <= SMALL_T) {
    // fp32 weights, no split row, or few rows on too few workgroups: merge
    // into o_lat (a pass over all split rows at once), then the plain
    // projection
    if (n_split > 0) {
      const hipError_t st =
          launch_combine_planned(o_part, lse_part, split, n_split, n_h, o_lat, lse, stream);
      if (st != hipSuccess) return st;
    }
    return launch_out_proj(o_lat, w_uv, T, n_h, dtype, out, stream);
  }
  const int chunks = (T + TCH - 1) / TCH;
  const int per_wg = max(1, (chunks * n_h + 511) / 512);
  hipLaunchKernelGGL(out_proj_bf16_kernel<true>, dim3(n_h, (chunks + per_wg - 1) / per_wg), dim3(256),
                     0, stream, o_lat, (const uint16_t*)w_uv, T, n_h, out,
                     SplitRows{o_part, lse_part, split, n_split, lse});
  return hipGetLastError();
}

}  // namespace mla
