// Per-row int8 absmax activation quantization.
//
// s = fl32(127 / max|x|), xq = clamp(rint(fl32(x*s)), -127, 127); an all-zero
// row gives s = 1 (and xq = 0).  The max is exact in any order, so a wave
// reduces it freely.  One wave quantizes one row with wave-level reductions
// only (four rows per workgroup, no barriers); rows of up to 2048 values stay
// in registers between the absmax and the rounding pass, longer rows are read
// twice.  Besides the natural-order int8 row the kernel can write the permuted
// row used by the matmul kernels and the exact int32 row sum that removes the
// +1 offset of the packed code fields.
#include "bitnet_device.hpp"
#include "bitnet_internal.hpp"

namespace bitnet {
namespace {

constexpr int kQuantThreads = 256;
constexpr int kRowsPerBlock = kQuantThreads / 64;
constexpr int kRegVec = 8;   // f32x4 per lane kept in registers: K <= 64 * 4 * 8

struct RowOut {
  int8_t *nat;        // natural order row, may be null
  int8_t *perm;       // permuted row, may be null
  float *scale;       // may be null
  float *scale2;      // may be null
  int32_t *rowsum;    // may be null
};

__device__ __forceinline__ float absmax4(f32x4 v) {
  return fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
}

// Quantize 4 values at input index 4*i; returns their sum and stores them.
__device__ __forceinline__ int quant_store4(f32x4 v, float s, int i, const RowOut &o) {
  const int q0 = quant_one(v.x, s), q1 = quant_one(v.y, s);
  const int q2 = quant_one(v.z, s), q3 = quant_one(v.w, s);
  const uint32_t w = pack4_i8(q0, q1, q2, q3);
  if (o.nat) st_global<uint32_t>(o.nat + 4 * i, w);
  if (o.perm) st_global<uint32_t>(o.perm + perm_offset(4 * i), w);
  return q0 + q1 + q2 + q3;
}

// One wave, one row of K fp32 values (K % 128 == 0).
__device__ __forceinline__ void quant_row_wave(const float *__restrict__ xr, int K,
                                               const RowOut &o) {
  const int lane = threadIdx.x & 63;
  const f32x4 *x4 = reinterpret_cast<const f32x4 *>(xr);
  const int n4 = K >> 2;
  float a = 0.0f;
  int sum = 0;
  float s;
  if (n4 <= kRegVec * 64) {
    f32x4 v[kRegVec];
#pragma unroll
    for (int j = 0; j < kRegVec; ++j) {
      const int i = lane + 64 * j;
      v[j] = i < n4 ? ld_global<f32x4>(x4 + i) : f32x4{0.f, 0.f, 0.f, 0.f};
      a = fmaxf(a, absmax4(v[j]));
    }
    a = wave_max(a);
    s = (a == 0.0f) ? 1.0f : 127.0f / a;
#pragma unroll
    for (int j = 0; j < kRegVec; ++j) {
      const int i = lane + 64 * j;
      if (i < n4) sum += quant_store4(v[j], s, i, o);
    }
  } else {
    // Longer rows: two passes, each in chunks of kRegVec loads per lane so that
    // several loads are in flight at once.
    for (int c0 = 0; c0 < n4; c0 += kRegVec * 64) {
      f32x4 v[kRegVec];
#pragma unroll
      for (int j = 0; j < kRegVec; ++j) {
        const int i = c0 + lane + 64 * j;
        v[j] = i < n4 ? ld_global<f32x4>(x4 + i) : f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int j = 0; j < kRegVec; ++j) a = fmaxf(a, absmax4(v[j]));
    }
    a = wave_max(a);
    s = (a == 0.0f) ? 1.0f : 127.0f / a;
    for (int c0 = 0; c0 < n4; c0 += kRegVec * 64) {
      f32x4 v[kRegVec];
#pragma unroll
      for (int j = 0; j < kRegVec; ++j) {
        const int i = c0 + lane + 64 * j;
        v[j] = i < n4 ? ld_global<f32x4>(x4 + i) : f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int j = 0; j < kRegVec; ++j) {
        const int i = c0 + lane + 64 * j;
        if (i < n4) sum += quant_store4(v[j], s, i, o);
      }
    }
  }
  sum = wave_sum(sum);
  if (lane == 0) {
    if (o.scale) st_global<float>(o.scale, s);
    if (o.scale2) st_global<float>(o.scale2, s);
    if (o.rowsum) st_global<int>(o.rowsum, sum);
  }
}

__global__ void __launch_bounds__(kQuantThreads)
    quant_rows_kernel(const float *__restrict__ x, int M, int K, int8_t *__restrict__ xq_nat,
                      int8_t *__restrict__ xq_perm, float *__restrict__ x_scale,
                      float *__restrict__ x_scale2, int32_t *__restrict__ rowsum) {
  const int row = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= M) return;
  const size_t off = (size_t)row * K;
  RowOut o{xq_nat ? xq_nat + off : nullptr, xq_perm ? xq_perm + off : nullptr,
           x_scale ? x_scale + row : nullptr, x_scale2 ? x_scale2 + row : nullptr,
           rowsum ? rowsum + row : nullptr};
  quant_row_wave(x + off, K, o);
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

// Grouped: wave w of workgroup b quantizes flattened row 4b + w, i.e. row
// (4b + w) % M of problem (4b + w) / M, into that problem's workspace.
__global__ void __launch_bounds__(kQuantThreads)
    quant_grouped_kernel(const bitnet_problem *__restrict__ problems, GroupTable tab,
                         uint8_t *__restrict__ workspace) {
  const int M = tab.M;
  const int flat = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (flat >= tab.count * M) return;
  const int p = flat / M;
  const int row = flat - p * M;
  const bitnet_problem pr = problems[p];
  const int K = (int)pr.K;
  const WsLayout L = ws_layout(M, K);
  uint8_t *ws = workspace + (size_t)tab.ws_off[p] * 256;
  RowOut o{nullptr, reinterpret_cast<int8_t *>(ws + L.xq) + (size_t)row * K,
           reinterpret_cast<float *>(ws + L.scale) + row, nullptr,
           reinterpret_cast<int32_t *>(ws + L.rowsum) + row};
  quant_row_wave(pr.x + (size_t)row * K, K, o);
}

}  // namespace

hipError_t launch_quant_rows(const float *x, int M, int K, int8_t *xq_nat, int8_t *xq_perm,
                             float *x_scale, float *x_scale2, int32_t *rowsum,
                             hipStream_t stream) {
  const int blocks = (M + kRowsPerBlock - 1) / kRowsPerBlock;
  quant_rows_kernel<<<blocks, kQuantThreads, 0, stream>>>(x, M, K, xq_nat, xq_perm, x_scale,
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

hipError_t launch_quant_grouped(const bitnet_problem *problems, const GroupTable &tab,
                                uint8_t *workspace, hipStream_t stream) {
  const int rows = tab.count * tab.M;
  const int blocks = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
  quant_grouped_kernel<<<blocks, kQuantThreads, 0, stream>>>(problems, tab, workspace);
  return hipGetLastError();
}

}  // namespace bitnet
