// Per-row int8 absmax activation quantization.
//
// s = fl32(127 / max|x|), xq = clamp(rint(fl32(x*s)), -127, 127); an all-zero
// row gives s = 1 (and xq = 0).  The max is exact in any order, so one
// workgroup per row reduces it freely.  Besides the natural-order int8 row the
// kernel can write the permuted row used by the matmul kernels and the exact
// int32 row sum that removes the +1 offset of the packed code fields.
#include "bitnet_device.hpp"
#include "bitnet_internal.hpp"

namespace bitnet {
namespace {

constexpr int kQuantThreads = 256;

__device__ __forceinline__ float block_max(float v, float *red) {
  v = wave_max(v);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  v = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  return v;
}

__device__ __forceinline__ int block_sum(int v, int *red) {
  v = wave_sum(v);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
}

// Quantize one row of K fp32 values (K % 128 == 0) by one 256-thread workgroup.
__device__ __forceinline__ void quant_row(const float *__restrict__ xr, int K,
                                          int8_t *__restrict__ nat, int8_t *__restrict__ perm,
                                          float *__restrict__ scale_out,
                                          float *__restrict__ scale_out2,
                                          int32_t *__restrict__ rowsum_out) {
  __shared__ float fred[4];
  __shared__ int ired[4];
  const f32x4 *x4 = reinterpret_cast<const f32x4 *>(xr);
  const int n4 = K >> 2;
  float a = 0.0f;
  for (int i = threadIdx.x; i < n4; i += kQuantThreads) {
    const f32x4 v = ld_global<f32x4>(x4 + i);
    a = fmaxf(a, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
  }
  a = block_max(a, fred);
  const float s = (a == 0.0f) ? 1.0f : 127.0f / a;
  int sum = 0;
  for (int i = threadIdx.x; i < n4; i += kQuantThreads) {
    const f32x4 v = ld_global<f32x4>(x4 + i);
    const int q0 = quant_one(v.x, s), q1 = quant_one(v.y, s);
    const int q2 = quant_one(v.z, s), q3 = quant_one(v.w, s);
    sum += q0 + q1 + q2 + q3;
    const uint32_t w = pack4_i8(q0, q1, q2, q3);
    if (nat) st_global<uint32_t>(nat + 4 * i, w);
    if (perm) st_global<uint32_t>(perm + perm_offset(4 * i), w);
  }
  sum = block_sum(sum, ired);
  if (threadIdx.x == 0) {
    if (scale_out) st_global<float>(scale_out, s);
    if (scale_out2) st_global<float>(scale_out2, s);
    if (rowsum_out) st_global<int>(rowsum_out, sum);
  }
}

__global__ void __launch_bounds__(kQuantThreads)
    quant_rows_kernel(const float *__restrict__ x, int K, int8_t *__restrict__ xq_nat,
                      int8_t *__restrict__ xq_perm, float *__restrict__ x_scale,
                      float *__restrict__ x_scale2, int32_t *__restrict__ rowsum) {
  const int row = blockIdx.x;
  const size_t off = (size_t)row * K;
  quant_row(x + off, K, xq_nat ? xq_nat + off : nullptr, xq_perm ? xq_perm + off : nullptr,
            x_scale ? x_scale + row : nullptr, x_scale2 ? x_scale2 + row : nullptr,
            rowsum ? rowsum + row : nullptr);
}

// Already-quantized rows: copy into the permuted order and form the row sums.
__global__ void __launch_bounds__(kQuantThreads)
    permute_q8_kernel(const int8_t *__restrict__ xq, const float *__restrict__ x_scale_in, int K,
                      int8_t *__restrict__ xq_perm, float *__restrict__ x_scale,
                      int32_t *__restrict__ rowsum) {
  __shared__ int ired[4];
  const int row = blockIdx.x;
  const size_t off = (size_t)row * K;
  const uint32_t *src = reinterpret_cast<const uint32_t *>(xq + off);
  int sum = 0;
  for (int i = threadIdx.x; i < (K >> 2); i += kQuantThreads) {
    const uint32_t w = ld_global<uint32_t>(src + i);
    sum += (int)(int8_t)(w & 0xff) + (int)(int8_t)((w >> 8) & 0xff) +
           (int)(int8_t)((w >> 16) & 0xff) + (int)(int8_t)(w >> 24);
    st_global<uint32_t>(xq_perm + off + perm_offset(4 * i), w);
  }
  sum = block_sum(sum, ired);
  if (threadIdx.x == 0) {
    st_global<float>(x_scale + row, ld_global<float>(x_scale_in + row));
    st_global<int>(rowsum + row, sum);
  }
}

// Grouped: workgroup b quantizes row b % M of problem b / M into its workspace.
__global__ void __launch_bounds__(kQuantThreads)
    quant_grouped_kernel(const bitnet_problem *__restrict__ problems, GroupTable tab,
                         uint8_t *__restrict__ workspace) {
  const int M = tab.M;
  const int p = blockIdx.x / M;
  const int row = blockIdx.x - p * M;
  const bitnet_problem pr = problems[p];
  const int K = (int)pr.K;
  const WsLayout L = ws_layout(M, K);
  uint8_t *ws = workspace + (size_t)tab.ws_off[p] * 256;
  quant_row(pr.x + (size_t)row * K, K, nullptr,
            reinterpret_cast<int8_t *>(ws + L.xq) + (size_t)row * K,
            reinterpret_cast<float *>(ws + L.scale) + row, nullptr,
            reinterpret_cast<int32_t *>(ws + L.rowsum) + row);
}

}  // namespace

hipError_t launch_quant_rows(const float *x, int M, int K, int8_t *xq_nat, int8_t *xq_perm,
                             float *x_scale, float *x_scale2, int32_t *rowsum,
                             hipStream_t stream) {
  quant_rows_kernel<<<M, kQuantThreads, 0, stream>>>(x, K, xq_nat, xq_perm, x_scale, x_scale2,
                                                     rowsum);
  return hipGetLastError();
}

hipError_t launch_permute_q8(const int8_t *xq, const float *x_scale_in, int M, int K,
                             int8_t *xq_perm, float *x_scale, int32_t *rowsum,
                             hipStream_t stream) {
  permute_q8_kernel<<<M, kQuantThreads, 0, stream>>>(xq, x_scale_in, K, xq_perm, x_scale,
                                                     rowsum);
  return hipGetLastError();
}

hipError_t launch_quant_grouped(const bitnet_problem *problems, const GroupTable &tab,
                                uint8_t *workspace, hipStream_t stream) {
  quant_grouped_kernel<<<tab.count * tab.M, kQuantThreads, 0, stream>>>(problems, tab,
                                                                         workspace);
  return hipGetLastError();
}

}  // namespace bitnet
