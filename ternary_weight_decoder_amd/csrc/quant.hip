// Per-row int8 absmax activation quantization.
//
// s = fl32(127 / max|x|), xq = clamp(rint(fl32(x*s)), -127, 127); an all-zero
// row gives s = 1 (and xq = 0).  The max is exact in any order, so it is reduced
// freely.  Every row is read from memory once, with all of its loads in flight
// together, and kept in registers between the absmax and the rounding pass:
//   - rows of up to 2048 values: one wave per row (four rows per workgroup),
//     wave-level reductions only;
//   - rows of up to 10240 values: one workgroup per row, reductions across its
//     four waves through LDS;
//   - longer rows: one workgroup per row, read twice.
// Besides the natural-order int8 row the kernels can write the permuted row
// used by the matmul kernels and the exact int32 row sum that removes the +1
// offset of the packed code fields.
#include "bitnet_device.hpp"
#include "bitnet_internal.hpp"

namespace bitnet {
namespace {

constexpr int kQuantThreads = 256;
constexpr int kRowsPerBlock = kQuantThreads / 64;
constexpr int kWaveVec = 8;                       // f32x4 per lane, wave per row
constexpr int kBlockVec = 10;                     // f32x4 per thread, workgroup per row
constexpr int kWaveMaxK = 64 * 4 * kWaveVec;      // 2048
constexpr int kBlockMaxK = kQuantThreads * 4 * kBlockVec;   // 10240

// Row loads.  NT: non-temporal, for the prefill-sized grouped launches
// (M > 64), whose fp32 rows are read once and would otherwise displace the
// int8 rows that the contraction launch reads next.  Decode and batched-decode
// launches (M <= 64), which stream their weights from HBM beside these rows,
// keep plain loads: they measured faster there.
template <bool NT>
__device__ __forceinline__ f32x4 ld_row(const f32x4 *p) {
  if constexpr (NT)
    return __builtin_nontemporal_load((const BITNET_GLOBAL f32x4 *)p);
  else
    return ld_global<f32x4>(p);
}

// Rows of a grouped launch from which its row loads are non-temporal.
#ifndef BITNET_QUANT_NT_MINM
#define BITNET_QUANT_NT_MINM 65
#endif

struct RowOut {
  int8_t *nat;        // natural order row, may be null
  int8_t *perm;       // permuted row, may be null
  float *scale;       // may be null
  float *scale2;      // may be null
  int32_t *rowsum;    // may be null
};

struct QuantShared {
  float red[kRowsPerBlock];
  int ired[kRowsPerBlock];
};

__device__ __forceinline__ float absmax4(f32x4 v) {
  return fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
}

__device__ __forceinline__ float scale_of(float a) { return (a == 0.0f) ? 1.0f : 127.0f / a; }

// Quantize 4 values at input index 4*i; returns their sum and stores them.
__device__ __forceinline__ int quant_store4(f32x4 v, float s, int i, const RowOut &o) {
  const int q0 = quant_one(v.x, s), q1 = quant_one(v.y, s);
  const int q2 = quant_one(v.z, s), q3 = quant_one(v.w, s);
  const uint32_t w = pack4_i8(q0, q1, q2, q3);
  if (o.nat) st_global<uint32_t>(o.nat + 4 * i, w);
  if (o.perm) st_global<uint32_t>(o.perm + perm_offset(4 * i), w);
  return q0 + q1 + q2 + q3;
}

__device__ __forceinline__ void store_row_meta(const RowOut &o, float s, int sum) {
  if (o.scale) st_global<float>(o.scale, s);
  if (o.scale2) st_global<float>(o.scale2, s);
  if (o.rowsum) st_global<int>(o.rowsum, sum);
}

// One wave, one row of K <= kWaveMaxK values (K % 4 == 0; the permuted row
// needs K % 128 == 0).
template <bool NT = false>
__device__ __forceinline__ void quant_row_wave(const float *__restrict__ xr, int K,
                                               const RowOut &o) {
  const int lane = threadIdx.x & 63;
  const f32x4 *x4 = reinterpret_cast<const f32x4 *>(xr);
  const int n4 = K >> 2;
  f32x4 v[kWaveVec];
  float a = 0.0f;
#pragma unroll
  for (int j = 0; j < kWaveVec; ++j) {
    const int i = lane + 64 * j;
    v[j] = i < n4 ? ld_row<NT>(x4 + i) : f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int j = 0; j < kWaveVec; ++j) a = fmaxf(a, absmax4(v[j]));
  const float s = scale_of(wave_max(a));
  int sum = 0;
#pragma unroll
  for (int j = 0; j < kWaveVec; ++j) {
    const int i = lane + 64 * j;
    if (i < n4) sum += quant_store4(v[j], s, i, o);
  }
  sum = wave_sum(sum);
  if (lane == 0) store_row_meta(o, s, sum);
}

__device__ __forceinline__ float block_max(float a, QuantShared &sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  a = wave_max(a);
  if (lane == 0) sh.red[wave] = a;
  __syncthreads();
  return fmaxf(fmaxf(sh.red[0], sh.red[1]), fmaxf(sh.red[2], sh.red[3]));
}

__device__ __forceinline__ void block_finish(int sum, float s, const RowOut &o, QuantShared &sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  sum = wave_sum(sum);
  if (lane == 0) sh.ired[wave] = sum;
  __syncthreads();
  if (threadIdx.x == 0) store_row_meta(o, s, sh.ired[0] + sh.ired[1] + sh.ired[2] + sh.ired[3]);
}

// One workgroup, one row of any K (K % 4 == 0; the permuted row needs
// K % 128 == 0).  Whole workgroup, uniform.
template <bool NT = false>
__device__ __forceinline__ void quant_row_block(const float *__restrict__ xr, int K,
                                                const RowOut &o, QuantShared &sh) {
  const int tid = threadIdx.x;
  const f32x4 *x4 = reinterpret_cast<const f32x4 *>(xr);
  const int n4 = K >> 2;
  int sum = 0;
  if (K <= kBlockMaxK) {
    f32x4 v[kBlockVec];
    float a = 0.0f;
#pragma unroll
    for (int j = 0; j < kBlockVec; ++j) {
      const int i = tid + kQuantThreads * j;
      v[j] = i < n4 ? ld_row<NT>(x4 + i) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int j = 0; j < kBlockVec; ++j) a = fmaxf(a, absmax4(v[j]));
    const float s = scale_of(block_max(a, sh));
#pragma unroll
    for (int j = 0; j < kBlockVec; ++j) {
      const int i = tid + kQuantThreads * j;
      if (i < n4) sum += quant_store4(v[j], s, i, o);
    }
    block_finish(sum, s, o, sh);
    return;
  }
  // Longer rows: two passes in chunks of kBlockVec loads per thread.
  float a = 0.0f;
  for (int c0 = 0; c0 < n4; c0 += kBlockVec * kQuantThreads) {
    f32x4 v[kBlockVec];
#pragma unroll
    for (int j = 0; j < kBlockVec; ++j) {
      const int i = c0 + tid + kQuantThreads * j;
      v[j] = i < n4 ? ld_row<NT>(x4 + i) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int j = 0; j < kBlockVec; ++j) a = fmaxf(a, absmax4(v[j]));
  }
  const float s = scale_of(block_max(a, sh));
  for (int c0 = 0; c0 < n4; c0 += kBlockVec * kQuantThreads) {
    f32x4 v[kBlockVec];
#pragma unroll
    for (int j = 0; j < kBlockVec; ++j) {
      const int i = c0 + tid + kQuantThreads * j;
      v[j] = i < n4 ? ld_row<NT>(x4 + i) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int j = 0; j < kBlockVec; ++j) {
      const int i = c0 + tid + kQuantThreads * j;
      if (i < n4) sum += quant_store4(v[j], s, i, o);
    }
  }
  block_finish(sum, s, o, sh);
}

__device__ __forceinline__ RowOut row_out(int8_t *xq_nat, int8_t *xq_perm, float *x_scale,
                                          float *x_scale2, int32_t *rowsum, int row, int K) {
  const size_t off = (size_t)row * K;
  return RowOut{xq_nat ? xq_nat + off : nullptr, xq_perm ? xq_perm + off : nullptr,
                x_scale ? x_scale + row : nullptr, x_scale2 ? x_scale2 + row : nullptr,
                rowsum ? rowsum + row : nullptr};
}

// WAVE_ROWS: four rows per workgroup, one per wave; otherwise one row per workgroup.
template <bool WAVE_ROWS>
__global__ void __launch_bounds__(kQuantThreads)
    quant_rows_kernel(const float *__restrict__ x, int M, int K, int8_t *__restrict__ xq_nat,
                      int8_t *__restrict__ xq_perm, float *__restrict__ x_scale,
                      float *__restrict__ x_scale2, int32_t *__restrict__ rowsum) {
  if (WAVE_ROWS) {
    const int row = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
    if (row >= M) return;
    quant_row_wave(x + (size_t)row * K, K,
                   row_out(xq_nat, xq_perm, x_scale, x_scale2, rowsum, row, K));
  } else {
    __shared__ QuantShared sh;
    const int row = blockIdx.x;
    quant_row_block(x + (size_t)row * K, K,
                    row_out(xq_nat, xq_perm, x_scale, x_scale2, rowsum, row, K), sh);
  }
}

// Already-quantized rows: copy into the permuted order and form the row sums.
__global__ void __launch_bounds__(kQuantThreads)
    permute_q8_kernel(const int8_t *__restrict__ xq, const float *__restrict__ x_scale_in, int M,
                      int K, int8_t *__restrict__ xq_perm, float *__restrict__ x_scale,
                      int32_t *__restrict__ rowsum) {
  const int row = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= M) return;
  const int lane = threadIdx.x & 63;
  const size_t off = (size_t)row * K;
  const uint32_t *src = reinterpret_cast<const uint32_t *>(xq + off);
  int sum = 0;
  for (int i = lane; i < (K >> 2); i += 64) {
    const uint32_t w = ld_global<uint32_t>(src + i);
    sum += (int)(int8_t)(w & 0xff) + (int)(int8_t)((w >> 8) & 0xff) +
           (int)(int8_t)((w >> 16) & 0xff) + (int)(int8_t)(w >> 24);
    st_global<uint32_t>(xq_perm + off + perm_offset(4 * i), w);
  }
  sum = wave_sum(sum);
  if (lane == 0) {
    st_global<float>(x_scale + row, ld_global<float>(x_scale_in + row));
    st_global<int>(rowsum + row, sum);
  }
}

// Grouped: workgroups [wg_end[s-1], wg_end[s]) quantize the M rows of problem
// order[s] into its workspace, four rows per workgroup when K <= kWaveMaxK and
// one row per workgroup otherwise.
template <bool NT>
__global__ void __launch_bounds__(kQuantThreads)
    quant_grouped_kernel(const bitnet_problem *__restrict__ problems, QuantTable tab,
                         uint8_t *__restrict__ workspace) {
  __shared__ QuantShared sh;
  const uint32_t b = blockIdx.x;
  int lo = 0, hi = tab.count - 1;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (b < tab.wg_end[mid]) hi = mid; else lo = mid + 1;
  }
  const uint32_t local = b - (lo ? tab.wg_end[lo - 1] : 0u);
  const int p = tab.order[lo];
  const int M = tab.M;
  const bitnet_problem pr = problems[p];
  const int K = (int)pr.K;
  const WsLayout L = ws_layout(M, K);
  uint8_t *ws = workspace + (size_t)tab.ws_off[p] * 256;
  int8_t *xq = reinterpret_cast<int8_t *>(ws + L.xq);
  float *xs = reinterpret_cast<float *>(ws + L.scale);
  int32_t *rs = reinterpret_cast<int32_t *>(ws + L.rowsum);
  if (K <= kWaveMaxK) {
    const int row = (int)local * kRowsPerBlock + (threadIdx.x >> 6);
    if (row >= M) return;
    quant_row_wave<NT>(pr.x + (size_t)row * K, K, row_out(nullptr, xq, xs, nullptr, rs, row, K));
  } else {
    const int row = (int)local;
    quant_row_block<NT>(pr.x + (size_t)row * K, K,
                        row_out(nullptr, xq, xs, nullptr, rs, row, K), sh);
  }
}

}  // namespace

hipError_t launch_quant_rows(const float *x, int M, int K, int8_t *xq_nat, int8_t *xq_perm,
                             float *x_scale, float *x_scale2, int32_t *rowsum,
                             hipStream_t stream) {
  if (K <= kWaveMaxK)
    quant_rows_kernel<true><<<(M + kRowsPerBlock - 1) / kRowsPerBlock, kQuantThreads, 0, stream>>>(
        x, M, K, xq_nat, xq_perm, x_scale, x_scale2, rowsum);
  else
    quant_rows_kernel<false><<<M, kQuantThreads, 0, stream>>>(x, M, K, xq_nat, xq_perm, x_scale,
                                                              x_scale2, rowsum);
  return hipGetLastError();
}

hipError_t launch_permute_q8(const int8_t *xq, const float *x_scale_in, int M, int K,
                             int8_t *xq_perm, float *x_scale, int32_t *rowsum,
                             hipStream_t stream) {
  const int blocks = (M + kRowsPerBlock - 1) / kRowsPerBlock;
  permute_q8_kernel<<<blocks, kQuantThreads, 0, stream>>>(xq, x_scale_in, M, K, xq_perm, x_scale,
                                                          rowsum);
  return hipGetLastError();
}

int64_t quant_grouped_blocks(int64_t M, int64_t K) {
  return K <= kWaveMaxK ? (M + kRowsPerBlock - 1) / kRowsPerBlock : M;
}

hipError_t launch_quant_grouped(const bitnet_problem *problems, const QuantTable &tab,
                                uint8_t *workspace, hipStream_t stream) {
  const unsigned blocks = tab.wg_end[tab.count - 1];
  if (tab.M >= BITNET_QUANT_NT_MINM)
    quant_grouped_kernel<true><<<blocks, kQuantThreads, 0, stream>>>(problems, tab, workspace);
  else
    quant_grouped_kernel<false><<<blocks, kQuantThreads, 0, stream>>>(problems, tab, workspace);
  return hipGetLastError();
}

}  // namespace bitnet
