// bf16 projection tiles shared by the producers and the non-absorbed
// prefill: Y = X W^T for X rows (contiguous, or rows of a paged cache) and
// W [N, K] rows, with the tile, staging and store layouts described below.
#pragma once

#include "mla_common.h"

namespace mla {
namespace {

constexpr int PN = 128;                        // W rows (outputs) per workgroup
constexpr int PK = 64;                         // K slices are multiples of this

// One direct global->LDS load: lane l's 16 bytes at base + lane_off land at
// LDS byte lds_dst + 16 l (M0 holds the LDS address; one wait state before
// the load reads it).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // M0 is named as clobbered on purpose
__device__ __forceinline__ void dma16(unsigned lds_dst, const char* base, unsigned lane_off) {
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %2"
      :
      : "v"(lane_off), "s"(lds_dst), "s"(base)
      : "m0");
}
#pragma clang diagnostic pop

// Wait until at most VMC of this wave's vector-memory loads are in flight
// and its LDS reads are done, then a workgroup barrier.
template <int VMC>
__device__ __forceinline__ void stage_barrier() {
  static_assert(VMC >= 0 && VMC < 64, "vmcnt field");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((VMC & 15) | ((VMC >> 4) << 14) | 0x70);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Rows of X: element k of row r at base[r' * ld + k], with r' = r, or, given
// a block table, r' = table[r / 64] * 64 + r % 64 (the rows of a paged cache,
// ld = 576; a block id outside [0, nblk) is read as block 0).  Byte offsets
// r' * ld * 2 must stay below 2^32.
struct XSrc {
  const uint16_t* base;
  int ld;
  const int* table;
  int nblk;
};

// Where a projection's outputs go (n: W row, t: X row):
//   OUT_ROWS     bf16 out[t * ldo + col0 + n]
//   OUT_PARTIAL  fp32 out[(z * T + t) * ldo + col0 + n], z the K slice
//   OUT_HEADS    bf16 out[(n / 128) * hstride + t * 128 + n % 128]
//   OUT_HEADS_T  bf16 out[(n / 128) * hstride + (n % 128) * ldo + t], every t
//                of the workgroup's tile (rows past T repeat row T - 1's
//                values, so the padding stays finite); with lo != 0 the value
//                is split into bf16 hi + lo, lo stored lo elements further
enum { OUT_ROWS = 0, OUT_PARTIAL = 1, OUT_HEADS = 2, OUT_HEADS_T = 3 };

struct ProjOut {
  const uint16_t* W;
  int N;
  void* out;
  int ldo;
  int col0;
  long hstride;
  long lo;
};

// Workgroup (x, y, z): W rows n0 .. n0 + 127 of projection p0 (x < tiles0)
// or p1, X rows TT y .. TT y + TT - 1 (of T), K slice [z kc, min(K, (z + 1) kc)),
// kc a multiple of KS.  Four waves in a 2 x 2 grid: wave (wn, wt) computes
// W rows 64 wn.. against X rows TT/2 wt.. with 4 x TT/32 MFMA tiles.
//
// A stage holds KS of K: 128 + TT rows of 2 KS bytes (the W rows, then the
// X rows); 16-byte piece q of stage row R sits in slot q ^ (R & 7), so that
// the eight lanes of one ds_read_b128 phase (eight rows, one piece) hit
// eight different bank groups.  Direct load i of a stage fills the 1024
// bytes of rows RPI i .. RPI i + RPI - 1; wave w issues loads
// w NIW .. w NIW + NIW - 1.  Rows past N or T re-read the last valid row;
// their results are dropped.  NST stages are resident, NST - 1 in flight.
template <int OUTM, int TT, int NST, int KS>
__global__ void __launch_bounds__(256, (NST * (PN + TT) * KS * 2) <= 80 * 1024 ? 2 : 1)
    proj_bf16_kernel(XSrc X, int T, int K, int kc, ProjOut p0, ProjOut p1, int tiles0) {
  constexpr int P_ROWB = KS * 2;               // bytes of one row in a stage
  constexpr int SPR = P_ROWB / 16;             // 16-byte slots per row
  constexpr int RPI = 64 / SPR;                // rows per direct load
  constexpr int STAGE = (PN + TT) * P_ROWB;
  constexpr int NIW = STAGE / 1024 / 4;
  constexpr int TB = TT / 32;                  // MFMA row tiles of X per wave
  static_assert(KS == 64 || KS == 128, "stage K");
  __shared__ __attribute__((aligned(16))) char smem[NST * STAGE];
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const bool second = (int)blockIdx.x >= tiles0;
  const ProjOut p = second ? p1 : p0;
  const int n0 = ((int)blockIdx.x - (second ? tiles0 : 0)) * PN;
  const int t0 = blockIdx.y * TT;
  const int k0 = blockIdx.z * kc;
  const int nst = (min(K, k0 + kc) - k0) / KS;

  unsigned off[NIW];
#pragma unroll
  for (int j = 0; j < NIW; ++j) {
    const int R = RPI * (wave * NIW + j) + lane / SPR;   // stage row
    const unsigned piece = (unsigned)(((lane % SPR) ^ (R & 7)) * 16);
    if (R < PN) {
      off[j] = (unsigned)min(n0 + R, p.N - 1) * (unsigned)(K * 2) + piece;
    } else {
      const int r = min(t0 + R - PN, T - 1);
      int rr = r;
      if (X.table) {
        const int blk = X.table[r >> 6];
        rr = (blk >= 0 && blk < X.nblk ? blk : 0) * 64 + (r & 63);
      }
      off[j] = (unsigned)rr * (unsigned)(X.ld * 2) + piece;
    }
  }
  const unsigned lds0 = (unsigned)(uintptr_t)(__attribute__((address_space(3))) char*)smem;
  auto issue = [&](int s) __attribute__((always_inline)) {
    const long kb = (long)(k0 + s * KS) * 2;
    const char* wb = reinterpret_cast<const char*>(p.W) + kb;
    const char* xb = reinterpret_cast<const char*>(X.base) + kb;
    const unsigned dst = lds0 + (unsigned)((s % NST) * STAGE + wave * NIW * 1024);
#pragma unroll
    for (int j = 0; j < NIW; ++j)
      dma16(dst + j * 1024, RPI * (wave * NIW + j) < PN ? wb : xb, off[j]);
  };

  // lane (g, r16) of MFMA tile (i, j) reads piece 4 ks + g of W row
  // 64 wn + 16 i + r16 and of X row TT/2 wt + 16 j + r16
  const int g = lane >> 4, r16 = lane & 15;
  const int wn = wave & 1, wt = wave >> 1;
  const int a_off = (64 * wn + r16) * P_ROWB, b_off = (PN + (TT / 2) * wt + r16) * P_ROWB;
  f32x4_t acc[4][TB];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < TB; ++j) acc[i][j] = f32x4_t{0, 0, 0, 0};
  auto compute = [&](int s) __attribute__((always_inline)) {
    const char* st = smem + (s % NST) * STAGE;
#pragma unroll
    for (int ks = 0; ks < KS / 32; ++ks) {
      const int sw = ((4 * ks + g) ^ (r16 & 7)) * 16;
      i16x8_t a[4], b[TB];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a[i] = *reinterpret_cast<const i16x8_t*>(st + a_off + 16 * i * P_ROWB + sw);
#pragma unroll
      for (int j = 0; j < TB; ++j)
        b[j] = *reinterpret_cast<const i16x8_t*>(st + b_off + 16 * j * P_ROWB + sw);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < TB; ++j) {
          if constexpr (OUTM == OUT_HEADS_T)   // D[t][n]: four rows t per lane
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16((bf16x8_t)b[j], (bf16x8_t)a[i],
                                                                acc[i][j], 0, 0, 0);
          else                                 // D[n][t]: four outputs n per lane
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16((bf16x8_t)a[i], (bf16x8_t)b[j],
                                                                acc[i][j], 0, 0, 0);
        }
    }
  };

#pragma unroll
  for (int s = 0; s < NST - 1; ++s)
    if (s < nst) issue(s);
  for (int s = 0; s < nst; ++s) {
    // stage s landed: stages s + 1 .. min(s + NST - 2, nst - 1) stay in flight
    const int ahead = min(NST - 2, nst - 1 - s);
    if constexpr (NST == 4) {
      if (ahead == 2)
        stage_barrier<2 * NIW>();
      else if (ahead == 1)
        stage_barrier<NIW>();
      else
        stage_barrier<0>();
    } else {
      static_assert(NST == 3, "three or four stages");
      if (ahead == 1)
        stage_barrier<NIW>();
      else
        stage_barrier<0>();
    }
    if (s + NST - 1 < nst) issue(s + NST - 1);   // into the slot every wave finished with
    compute(s);
  }

  if constexpr (OUTM == OUT_HEADS_T) {
    // acc[i][j][e]: output n0 + 64 wn + 16 i + r16 of row t0 + TT/2 wt + 16 j + 4 g + e
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int n = n0 + 64 * wn + 16 * i + r16;
      if (n >= p.N) continue;
      uint16_t* o = static_cast<uint16_t*>(p.out) + (long)(n >> 7) * p.hstride +
                    (long)(n & 127) * p.ldo;
#pragma unroll
      for (int j = 0; j < TB; ++j) {
        const int t = t0 + (TT / 2) * wt + 16 * j + 4 * g;
        *reinterpret_cast<uint2*>(o + t) = uint2{pack_bf16x2(acc[i][j][0], acc[i][j][1]),
                                                 pack_bf16x2(acc[i][j][2], acc[i][j][3])};
        if (p.lo != 0) {
          float r[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) r[e] = acc[i][j][e] - bf16_to_f32(f32_to_bf16(acc[i][j][e]));
          *reinterpret_cast<uint2*>(o + p.lo + t) = uint2{pack_bf16x2(r[0], r[1]),
                                                          pack_bf16x2(r[2], r[3])};
        }
      }
    }
    return;
  }
  // acc[i][j][e]: output n0 + 64 wn + 16 i + 4 g + e of row t0 + TT/2 wt + 16 j + r16
#pragma unroll
  for (int j = 0; j < TB; ++j) {
    const int t = t0 + (TT / 2) * wt + 16 * j + r16;
    if (t >= T) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int n = n0 + 64 * wn + 16 * i + 4 * g;
      if (n >= p.N) continue;
      if constexpr (OUTM == OUT_PARTIAL) {
        float* o = static_cast<float*>(p.out) + ((long)blockIdx.z * T + t) * p.ldo + p.col0 + n;
        *reinterpret_cast<float4*>(o) = float4{acc[i][j][0], acc[i][j][1], acc[i][j][2],
                                               acc[i][j][3]};
      } else {
        uint16_t* o = static_cast<uint16_t*>(p.out) +
                      (OUTM == OUT_HEADS ? (long)(n >> 7) * p.hstride + (long)t * 128 + (n & 127)
                                         : (long)t * p.ldo + p.col0 + n);
        *reinterpret_cast<uint2*>(o) = uint2{pack_bf16x2(acc[i][j][0], acc[i][j][1]),
                                             pack_bf16x2(acc[i][j][2], acc[i][j][3])};
      }
    }
  }
}

// Rows of X per bf16 workgroup: 128 (more reuse of each staged tile), or 64
// for a projection so narrow that it splits K (twice the workgroups for the
// same partial-sum bytes).  Measured on the decode shapes (T = 128): the
// W^UQ + W^QR launch of 128 heads runs 8% faster with 128-row tiles, the
// split W^DQ and W^DKV + W^KR ones 0-30% faster with 64.
inline int t_tile(int T, int N) {
  const long tiles128 = (long)((N + PN - 1) / PN) * ((T + 127) / 128);
  return tiles128 < 128 ? 64 : 128;
}

// bf16: the projections p0 and p1 (p1.N == 0: none) of X [T, K] rows, one
// launch; OUTM as in proj_bf16_kernel.
template <int OUTM>
void proj_bf16(XSrc X, int T, int K, int kc, ProjOut p0, ProjOut p1, hipStream_t stream,
               int tt_force = 0) {
  const int tiles0 = (p0.N + PN - 1) / PN, tiles1 = (p1.N + PN - 1) / PN;
  const int tt = tt_force ? tt_force : t_tile(T, p0.N + p1.N);
  dim3 grid(tiles0 + tiles1, (T + tt - 1) / tt, (K + kc - 1) / kc), block(256);
  if (tt == 64)
    hipLaunchKernelGGL((proj_bf16_kernel<OUTM, 64, 3, 64>), grid, block, 0, stream, X, T, K, kc,
                       p0, p1, tiles0);
  else if (tt == 256)
    hipLaunchKernelGGL((proj_bf16_kernel<OUTM, 256, 3, 64>), grid, block, 0, stream, X, T, K, kc,
                       p0, p1, tiles0);
  else
    hipLaunchKernelGGL((proj_bf16_kernel<OUTM, 128, 4, 64>), grid, block, 0, stream, X, T, K, kc,
                       p0, p1, tiles0);
}

}  // namespace
}  // namespace mla
