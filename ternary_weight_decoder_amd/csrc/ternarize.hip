// Per-tensor absmean ternarization and 2-bit packing (offline, once per weight).
//
// The method: every projection weight becomes -1, 0 or +1 with one scale per
// tensor from mean|W| (ONNX model card "multimodalart/VibeVoice-ASR-BitNet-ONNX",
// Quantization table, row "LM projections"); codes are stored at 2 bits in
// 128-code units (blog "The Paper Says ARM Support...", section "Postscript two").
//
// The mean is computed in a fixed order so that the result is bit-reproducible:
// each row in fp64 with k ascending (one lane per row), then the rows in fp64
// with n ascending (one lane), divided in fp64 and rounded once to fp32.  The
// order leaves only the rows to run in parallel; the reads are made coalesced
// by staging 64-row x 64-column tiles through LDS, from which every lane adds
// its own row in k order.
#include "bitnet_device.hpp"
#include "bitnet_internal.hpp"

namespace bitnet {
namespace {

constexpr int kRowsPerWave = 64;
constexpr int kTileK = 64;
constexpr int kTileStride = kTileK + 1;   // padded: lane r reads row r without bank conflicts
constexpr int kAbsWaves = 4;

// One lane per row, one wave per 64 rows: sum of |W[n,k]| in fp64, k ascending.
// Load q of a tile brings rows 4q .. 4q + 3 (16 lanes x 16 bytes = one 256-byte
// row segment each), so every load is a contiguous 1 KB read.
__global__ void __launch_bounds__(64 * kAbsWaves)
    absrow_kernel(const float *__restrict__ W, int N, int K, double *__restrict__ rowsums) {
  __shared__ float tile[kAbsWaves][kRowsPerWave * kTileStride];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n0 = (blockIdx.x * kAbsWaves + wave) * kRowsPerWave;
  if (n0 >= N) return;
  float *t = tile[wave];
  const int sub = lane & 15;        // 16-byte piece of the row segment
  double s = 0.0;
  for (int k0 = 0; k0 < K; k0 += kTileK) {
    f32x4 v[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int r = 4 * q + (lane >> 4);
      const int n = min(n0 + r, N - 1);
      v[q] = ld_global<f32x4>(W + (size_t)n * K + k0 + 4 * sub);
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      float *dst = t + (4 * q + (lane >> 4)) * kTileStride + 4 * sub;
      dst[0] = v[q].x;
      dst[1] = v[q].y;
      dst[2] = v[q].z;
      dst[3] = v[q].w;
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    const float *row = t + lane * kTileStride;
#pragma unroll 16
    for (int j = 0; j < kTileK; ++j) s += fabs((double)row[j]);
    __builtin_amdgcn_wave_barrier();
  }
  if (n0 + lane < N) st_global<double>(rowsums + n0 + lane, s);
}

// One lane: rows added with n ascending, then the mean rounded to fp32.  The
// workgroup first brings the row sums into LDS.
constexpr int kFinalChunk = 2048;
__global__ void __launch_bounds__(256)
    absmean_final_kernel(const double *__restrict__ rowsums, int N, double count,
                         float *__restrict__ w_scale) {
  __shared__ double buf[kFinalChunk];
  double t = 0.0;
  for (int c0 = 0; c0 < N; c0 += kFinalChunk) {
    const int len = min(kFinalChunk, N - c0);
    for (int i = threadIdx.x; i < len; i += blockDim.x) buf[i] = ld_global<double>(rowsums + c0 + i);
    __syncthreads();
    if (threadIdx.x == 0) {
#pragma unroll 16
      for (int i = 0; i < len; ++i) t += buf[i];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) st_global<float>(w_scale, (float)(t / count));
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
  const int rows_per_block = kRowsPerWave * kAbsWaves;
  absrow_kernel<<<(N + rows_per_block - 1) / rows_per_block, 64 * kAbsWaves, 0, stream>>>(
      W, N, K, rowsums);
  absmean_final_kernel<<<1, 256, 0, stream>>>(rowsums, N, (double)N * (double)K, w_scale);
  const int64_t dwords = (int64_t)N * (K / kUnit) * 8;
  pack_kernel<<<(unsigned)((dwords + 255) / 256), 256, 0, stream>>>(
      W, N, K, w_scale, reinterpret_cast<uint32_t *>(packed));
  return hipGetLastError();
}

}  // namespace bitnet
