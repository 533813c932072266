// Lookup-table variant of the single-row decode projection (M = 1).
//
// bitnet.cpp's kernels follow the lookup-table method of T-MAC (TL1 on ARM)
// (thetesserapress, "Microsoft's BitNet Adds 1-Bit Embeddings...", the
// paragraphs on the repo's dependencies and on platform support): instead of
// expanding every code, precompute the partial sums that a small group of
// codes can select and index them with the packed bits.  This file is that
// method written for gfx950, as the comparison to the unpack + MFMA decode
// kernel; both compute the same int32 contraction, so the outputs are
// bit-identical.
//
// Table.  A packed byte holds the codes of k = 128t + c + 32j, j = 0..3, at
// bits 2j (unit t, byte c).  Its low nibble selects among the 16 sums
// (u0 - 1) * xq[k0] + (u1 - 1) * xq[k0 + 32] with k0 = 128t + c, u0 = bits
// 0..1, u1 = bits 2..3; the high nibble does the same for k0 = 128t + c + 64.
// (u = 3 is never stored; its entries are 0.)  So one table is 16 int16 sums
// (|sum| <= 254), 32 per unit half, 2 KB per 128-code unit.
//
// Work split.  One workgroup owns 256 * kLutCols output columns (kLutCols per
// thread, 256 apart) of one
// projection over its whole K: it quantizes the activation row into LDS
// itself (absmax scale, round half to even, clamp to 127), builds the tables
// for a chunk of kLutChunk units (32 KB) in LDS, and every thread then walks
// its column's packed bytes of those units with one LDS read per nibble.  The
// 16 entries of one table sit in 8 LDS banks and all lanes of a wave read the
// same table, so a lookup is conflict-free (lanes that pick the same dword are
// served by broadcast).  Codes are read with 16-byte non-temporal loads, a
// wave reading 64 adjacent columns' 32-byte unit slices (2 KB contiguous),
// kLutDepth units ahead.
#include <algorithm>
#include <cstring>

#include "bitnet_device.hpp"
#include "bitnet_internal.hpp"
#include "bitnet_variants.hpp"

namespace bitnet {
namespace {

#ifndef BITNET_LUT_COLS
#define BITNET_LUT_COLS 1
#endif
#ifndef BITNET_LUT_DEPTH
#define BITNET_LUT_DEPTH 4
#endif
constexpr int kLutThreads = 256;
constexpr int kLutWaves = kLutThreads / 64;
constexpr int kLutCols = BITNET_LUT_COLS;      // output columns per thread
constexpr int kLutTile = kLutThreads * kLutCols;   // output columns per workgroup
constexpr int kLutChunk = 16;                  // units per table chunk
constexpr int kLutDepth = BITNET_LUT_DEPTH;    // units of codes in flight per column
constexpr int kLutTableBytes = 32;             // 16 int16 entries
constexpr int kLutUnitBytes = 64 * kLutTableBytes;   // 2 halves x 32 bytes x 32 B
constexpr int kWeightAux = 2;                  // non-temporal

struct LutShared {
  __attribute__((aligned(16))) int8_t xq[kLutMaxK];                   // natural order
  __attribute__((aligned(16))) int16_t tab[kLutChunk * kLutUnitBytes / 2];
  float red[kLutWaves];
};

// Quantize the activation row (fp32, K) into sh.xq; returns the scale.
__device__ __forceinline__ float lut_quant_row(const float *x, int K, LutShared &sh) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n4 = K >> 2;
  const f32x4 *x4 = reinterpret_cast<const f32x4 *>(x);
  float a = 0.0f;
  for (int i = tid; i < n4; i += kLutThreads) {
    const f32x4 v = ld_global<f32x4>(x4 + i);
    a = fmaxf(a, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
  }
  a = wave_max(a);
  if (lane == 0) sh.red[wave] = a;
  __syncthreads();
  a = fmaxf(fmaxf(sh.red[0], sh.red[1]), fmaxf(sh.red[2], sh.red[3]));
  const float s = (a == 0.0f) ? 1.0f : 127.0f / a;
  for (int i = tid; i < n4; i += kLutThreads) {
    const f32x4 v = ld_global<f32x4>(x4 + i);
    *reinterpret_cast<uint32_t *>(sh.xq + 4 * i) =
        pack4_i8(quant_one(v.x, s), quant_one(v.y, s), quant_one(v.z, s), quant_one(v.w, s));
  }
  return s;
}

// Tables of units [t0, t0 + n) into sh.tab: group g = (unit * 2 + half) * 32 + c.
__device__ __forceinline__ void lut_build(int t0, int n, LutShared &sh) {
  for (int g = threadIdx.x; g < n * 64; g += kLutThreads) {
    const int ul = g >> 6, half = (g >> 5) & 1, c = g & 31;
    const int k0 = 128 * (t0 + ul) + c + 64 * half;
    const int x0 = sh.xq[k0], x1 = sh.xq[k0 + 32];
    uint32_t *dst = reinterpret_cast<uint32_t *>(sh.tab + g * 16);
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      int e[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int idx = 2 * p + q, u0 = idx & 3, u1 = idx >> 2;
        e[q] = (u0 == 3 || u1 == 3) ? 0 : (u0 - 1) * x0 + (u1 - 1) * x1;
      }
      dst[p] = (uint32_t)(e[0] & 0xffff) | ((uint32_t)e[1] << 16);
    }
  }
}

// Sum of the 64 table entries that the 32 packed bytes of one unit select.
// ubase: byte offset of the unit's tables inside sh.tab.
__device__ __forceinline__ int lut_unit(const u32x4 (&w)[2], uint32_t ubase,
                                        const LutShared &sh) {
  const char *tb = reinterpret_cast<const char *>(sh.tab);
  int acc = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t d = w[i >> 2][i & 3];   // bytes c = 4i .. 4i + 3
#pragma unroll
    for (int b = 0; b < 4; ++b) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int c = 4 * i + b, s = 8 * b + 4 * half;
        // Entry offset idx * 2 of the nibble at bit s.
        const uint32_t e2 = (s == 0 ? (d << 1) : (d >> (s - 1))) & 0x1Eu;
        acc += *reinterpret_cast<const int16_t *>(tb + (ubase | e2) +
                                                  (half * 32 + c) * kLutTableBytes);
      }
    }
  }
  return acc;
}

// Grouped: dispatch slot s of the table owns workgroups [blk_end[s-1], blk_end[s]).
__global__ void __launch_bounds__(kLutThreads)
    lut_gemv_grouped_kernel(const bitnet_problem *__restrict__ problems, GroupTable tab) {
  __shared__ LutShared sh;
  // Block b runs on XCD b % 8; unless the table deals workgroups round-robin,
  // XCD x runs its own range [xcd_first[x], xcd_first[x + 1]) of whole
  // projections.
  uint32_t b = blockIdx.x;
  if (!tab.spread) {
    const uint32_t x = b % kXcds;
    b = tab.xcd_first[x] + b / kXcds;
    if (b >= tab.xcd_first[x + 1]) return;
  }
  const SlotInfo si = find_slot(tab, b);
  const bitnet_problem pr = problems[si.problem];
  const int N = (int)pr.N, K = (int)pr.K, U = K >> 7;
  // Column r of this thread: n0 + 256 r (each wave reads 64 adjacent columns).
  const int n0 = (int)(b - si.first) * kLutTile + threadIdx.x;

  const uint32_t w_bytes = (uint32_t)((size_t)N * K / 4);
  const __amdgpu_buffer_rsrc_t w_rsrc = make_rsrc(pr.packed, w_bytes);
  const uint32_t ustride = (uint32_t)N * kUnitBytes;
  auto load_unit = [&](int t, int r, u32x4 (&w)[2]) {
    const int n = n0 + r * kLutThreads;
    const uint32_t off =
        (t < U && n < N) ? (uint32_t)t * ustride + (uint32_t)n * kUnitBytes : w_bytes;
    w[0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(w_rsrc, off, 0,
                                                                            kWeightAux));
    w[1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(w_rsrc, off + 16, 0,
                                                                            kWeightAux));
  };
  u32x4 ring[kLutDepth][kLutCols][2];
#pragma unroll
  for (int j = 0; j < kLutDepth; ++j)
#pragma unroll
    for (int r = 0; r < kLutCols; ++r) load_unit(j, r, ring[j][r]);

  const float xs = lut_quant_row(pr.x, K, sh);
  int acc[kLutCols];
#pragma unroll
  for (int r = 0; r < kLutCols; ++r) acc[r] = 0;
  for (int t0 = 0; t0 < U; t0 += kLutChunk) {
    const int nu = min(kLutChunk, U - t0);
    __syncthreads();   // the row is in LDS, and the previous chunk's lookups are done
    lut_build(t0, nu, sh);
    __syncthreads();
    // Every ring slot is refilled each step, also past K (aimed beyond the
    // buffer: no memory access), so the wait counts stay static.
    for (int base = 0; base < nu; base += kLutDepth) {
#pragma unroll
      for (int j = 0; j < kLutDepth; ++j) {
        const int ul = base + j;
#pragma unroll
        for (int r = 0; r < kLutCols; ++r) {
          if (ul < nu) acc[r] += lut_unit(ring[j][r], (uint32_t)ul * kLutUnitBytes, sh);
          load_unit(t0 + ul + kLutDepth, r, ring[j][r]);
        }
      }
    }
  }
  const float ws = ld_global<float>(pr.w_scale);
#pragma unroll
  for (int r = 0; r < kLutCols; ++r) {
    const int n = n0 + r * kLutThreads;
    if (n < N) st_global<float>(pr.y + n, dequant_exact(acc[r], ws, xs));
  }
}

}  // namespace

int lut_blocks(int64_t N) { return (int)((N + kLutTile - 1) / kLutTile); }

hipError_t launch_lut_grouped(const bitnet_problem *problems, const GroupTable &tab,
                              hipStream_t stream) {
  const unsigned grid = tab.spread ? tab.blk_end[tab.count - 1] : xcd_grid(tab.xcd_first);
  lut_gemv_grouped_kernel<<<grid, kLutThreads, 0, stream>>>(problems, tab);
  return hipGetLastError();
}

}  // namespace bitnet
