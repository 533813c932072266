// Per-tensor absmean ternarization and 2-bit packing (offline, once per weight).
//
// The method: every projection weight becomes -1, 0 or +1 with one scale per
// tensor from mean|W| (ONNX model card "multimodalart/VibeVoice-ASR-BitNet-ONNX",
// Quantization table, row "LM projections"); codes are stored at 2 bits in
// 128-code units (blog "The Paper Says ARM Support...", section "Postscript two").
//
// The mean is computed in a fixed order so that the result is bit-reproducible:
// each row in fp64 with k ascending (one thread per row), then the rows in fp64
// with n ascending (one thread), divided in fp64 and rounded once to fp32.
#include "bitnet_device.hpp"
#include "bitnet_internal.hpp"

namespace bitnet {
namespace {

// One thread per row: sum of |W[n,k]| in fp64, k ascending.
__global__ void __launch_bounds__(256) absrow_kernel(const float *__restrict__ W, int N, int K,
                                                     double *__restrict__ rowsums) {
  const int n = blockIdx.x * blockDim.x + threadIdx.x;
  if (n >= N) return;
  const f32x4 *r = reinterpret_cast<const f32x4 *>(W + (size_t)n * K);
  double s = 0.0;
  for (int i = 0; i < (K >> 2); ++i) {
    const f32x4 v = ld_global<f32x4>(r + i);
    s += fabs((double)v.x);
    s += fabs((double)v.y);
    s += fabs((double)v.z);
    s += fabs((double)v.w);
  }
  st_global<double>(rowsums + n, s);
}

// One thread: rows added with n ascending, then the mean rounded to fp32.
__global__ void absmean_final_kernel(const double *__restrict__ rowsums, int N, double count,
                                     float *__restrict__ w_scale) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  double t = 0.0;
  for (int n = 0; n < N; ++n) t += ld_global<double>(rowsums + n);
  st_global<float>(w_scale, (float)(t / count));
}

__device__ __forceinline__ uint32_t field_of(float w, float m) {
  if (m == 0.0f) return 1u;                  // all codes 0 for an all-zero tensor
  float r = __builtin_rintf(w / m);          // IEEE fp32 division, half-to-even
  r = fminf(fmaxf(r, -1.0f), 1.0f);
  return (uint32_t)((int)r + 1);
}

// One thread per packed dword: dword d of unit t of row n holds, in byte c, the
// four fields g = 0..3 of inputs k = 128t + 32g + 4d + c.
__global__ void __launch_bounds__(256) pack_kernel(const float *__restrict__ W, int N, int K,
                                                   const float *__restrict__ w_scale,
                                                   uint32_t *__restrict__ packed) {
  const int64_t total = (int64_t)N * (K >> 7) * 8;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int d = (int)(idx & 7);
  const int64_t rest = idx >> 3;
  const int n = (int)(rest % N);
  const int t = (int)(rest / N);
  const float m = ld_global<float>(w_scale);
  const float *row = W + (size_t)n * K + (size_t)t * kUnit + 4 * d;
  uint32_t out = 0;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const f32x4 v = ld_global<f32x4>(row + 32 * g);
    out |= field_of(v.x, m) << (0 + 2 * g);
    out |= field_of(v.y, m) << (8 + 2 * g);
    out |= field_of(v.z, m) << (16 + 2 * g);
    out |= field_of(v.w, m) << (24 + 2 * g);
  }
  st_global<uint32_t>(packed + idx, out);
}

}  // namespace

hipError_t launch_ternarize_pack(const float *W, int N, int K, uint8_t *packed, float *w_scale,
                                 double *rowsums, hipStream_t stream) {
  absrow_kernel<<<(N + 255) / 256, 256, 0, stream>>>(W, N, K, rowsums);
  absmean_final_kernel<<<1, 64, 0, stream>>>(rowsums, N, (double)N * (double)K, w_scale);
  const int64_t dwords = (int64_t)N * (K / kUnit) * 8;
  pack_kernel<<<(unsigned)((dwords + 255) / 256), 256, 0, stream>>>(
      W, N, K, w_scale, reinterpret_cast<uint32_t *>(packed));
  return hipGetLastError();
}

}  // namespace bitnet
