// I8_S causal depthwise convolution over frames: the audio encoders' token
// mixer, in front of their pointwise (matmul + bias + ReLU) layers.
//
// The encoders run fused int8 convolution and depthwise convolution routines
// with bias (aitrends.kr summary, technical-features section), exported with
// causal padding (ONNX model card "multimodalart/VibeVoice-ASR-BitNet-ONNX",
// Provenance) and int8 per-channel weights (same card, Quantization table,
// row "VAE encoders").  Here, for x [B, T, C] (channels innermost) and an
// int8 kernel q [C, k] with one scale per channel:
//   y[b,t,c] = relu?(acc * w_scale[c] / s[b,c] + bias[c]),
//   acc      = sum_{j<k} q[c,j] * xq[b, t-(k-1)+j, c]   (frames before 0: 0),
// with xq, s the int8 quantization of x with one absmax scale per (sequence,
// channel): the sum runs over frames within a channel, so one scale per
// channel keeps it exact in int32.  The epilogue does the fp64 operations of
// the plain definition in its order (exact product, correctly rounded
// division, bias add, one rounding to fp32), so outputs are bit-exact.
//
// Launches (all HBM-bound): colmax_kernel writes the maximum |x| of each
// (sequence, 128-frame chunk, channel) to the workspace; colscale_kernel turns
// each column's chunk maxima into its scale; dwconv_kernel takes one
// sequence's 64-frame x 64-channel output tile, quantizes the tile's input
// frames (6 halo frames before it for k = 7) into LDS, and convolves from LDS.
#include <algorithm>

#include "bitnet_device.hpp"
#include "bitnet_internal.hpp"
#include "bitnet_variants.hpp"

namespace bitnet {
namespace {

constexpr int kThreads = 256;
constexpr int kChunkFrames = 128;   // frames per partial maximum
constexpr int kTileC = 64;          // channels per workgroup tile
constexpr int kTileT = 64;          // output frames per workgroup tile

struct DwParams {
  const float *x;          // [B][T][C]
  const int8_t *q;         // [C][k]
  const float *w_scale;    // [C]
  const float *bias;       // [C] or null
  float *y;                // [B][T][C]
  int32_t *acc_out;        // [B][T][C] or null
  float *x_scale_out;      // [B][C] or null
  const float *partial;    // [B][nchunk][C] chunk maxima; chunk 0 holds the scales
  int B, T, C, k, nchunk, relu;
};

// Workgroup (chunk, channel tile, b): thread (cq = tid % 16, fr = tid / 16)
// takes channels 4cq..4cq+3 of the tile and frames fr, fr + 16, ... of the
// chunk; the 16 frame lanes are then reduced through LDS.
__global__ void __launch_bounds__(kThreads) colmax_kernel(const float *x, int T, int C,
                                                          int nchunk, float *partial) {
  __shared__ f32x4 red[kThreads];
  const int chunk = blockIdx.x, c0 = blockIdx.y * kTileC, b = blockIdx.z;
  const int tid = threadIdx.x, cq = tid & 15, fr = tid >> 4;
  const int t0 = chunk * kChunkFrames;
  const f32x4 *x4 = reinterpret_cast<const f32x4 *>(x + (size_t)b * T * C + c0) + cq;
  f32x4 m = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  f32x4 v[kChunkFrames / 16];
#pragma unroll
  for (int i = 0; i < kChunkFrames / 16; ++i) {
    const int t = t0 + fr + 16 * i;
    v[i] = t < T ? ld_global<f32x4>(x4 + (size_t)t * (C / 4)) : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }
#pragma unroll
  for (int i = 0; i < kChunkFrames / 16; ++i) {
    m.x = fmaxf(m.x, fabsf(v[i].x));
    m.y = fmaxf(m.y, fabsf(v[i].y));
    m.z = fmaxf(m.z, fabsf(v[i].z));
    m.w = fmaxf(m.w, fabsf(v[i].w));
  }
  red[tid] = m;
  __syncthreads();
  if (tid < 16) {
    f32x4 a = red[tid];
    for (int r = 1; r < 16; ++r) {
      const f32x4 v = red[r * 16 + tid];
      a.x = fmaxf(a.x, v.x);
      a.y = fmaxf(a.y, v.y);
      a.z = fmaxf(a.z, v.z);
      a.w = fmaxf(a.w, v.w);
    }
    st_global<f32x4>(partial + ((size_t)b * nchunk + chunk) * C + c0 + 4 * tid, a);
  }
}

// Scales of every (sequence, channel): the maximum of its chunk maxima, one
// thread per (sequence, channel); written over chunk 0's maxima.
__global__ void __launch_bounds__(kThreads) colscale_kernel(float *partial, int B, int C,
                                                            int nchunk, float *x_scale_out) {
  const int i = blockIdx.x * kThreads + threadIdx.x;
  if (i >= B * C) return;
  const int b = i / C, c = i - b * C;
  float *col = partial + (size_t)b * nchunk * C + c;
  float a = 0.0f;
  for (int ch0 = 0; ch0 < nchunk; ch0 += 16) {   // 16 loads in flight at a time
    float m[16];
#pragma unroll
    for (int u = 0; u < 16; ++u)
      m[u] = ch0 + u < nchunk ? ld_global<float>(col + (size_t)(ch0 + u) * C) : 0.0f;
#pragma unroll
    for (int u = 0; u < 16; ++u) a = fmaxf(a, m[u]);
  }
  const float s = (a == 0.0f) ? 1.0f : 127.0f / a;
  st_global<float>(col, s);
  if (x_scale_out) st_global<float>(x_scale_out + i, s);
}

template <bool RELU>
__global__ void __launch_bounds__(kThreads) dwconv_kernel(DwParams p) {
  __shared__ float sx[kTileC], sw[kTileC], bs[kTileC];
  __shared__ int8_t qk[kTileC][kMaxDwTaps];
  // quantized input frames t0 - (k-1) .. t0 + kTileT - 1, 64 channels each
  __shared__ __attribute__((aligned(16))) int8_t xq[(kTileT + kMaxDwTaps - 1) * kTileC];
  const int tt = blockIdx.x, c0 = blockIdx.y * kTileC, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int t0 = tt * kTileT;
  const int halo = p.k - 1;

  // The tile's input frames t0 - halo .. t0 + kTileT - 1 (frames before 0 and
  // past T are zeros), all loads of a thread at once; thread (cq, fr) takes
  // channels 4cq..4cq+3 of frames fr, fr + 16, ...
  const int cq = tid & 15, fr = tid >> 4;
  const int rows = kTileT + halo;
  const f32x4 *x4 = reinterpret_cast<const f32x4 *>(p.x + (size_t)b * p.T * p.C + c0) + cq;
  constexpr int kRowLoads = (kTileT + kMaxDwTaps - 1 + 15) / 16;
  f32x4 v[kRowLoads];
#pragma unroll
  for (int i = 0; i < kRowLoads; ++i) {
    const int r = fr + 16 * i, t = t0 - halo + r;
    v[i] = (r < rows && t >= 0 && t < p.T) ? ld_global<f32x4>(x4 + (size_t)t * (p.C / 4))
                                           : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }
  // Scales (from the column-scale launch), kernel taps, bias.
  if (tid < kTileC) {
    sx[tid] = ld_global<float>(p.partial + (size_t)b * p.nchunk * p.C + c0 + tid);
    sw[tid] = ld_global<float>(p.w_scale + c0 + tid);
    bs[tid] = p.bias ? ld_global<float>(p.bias + c0 + tid) : 0.0f;
  }
  for (int i = tid; i < kTileC * p.k; i += kThreads) {
    const int c = i / p.k, j = i - c * p.k;
    qk[c][j] = p.q[(size_t)(c0 + c) * p.k + j];
  }
  __syncthreads();
  const float s0 = sx[4 * cq], s1 = sx[4 * cq + 1], s2 = sx[4 * cq + 2], s3 = sx[4 * cq + 3];
#pragma unroll
  for (int i = 0; i < kRowLoads; ++i) {
    const int r = fr + 16 * i;
    if (r < rows)
      *reinterpret_cast<uint32_t *>(&xq[r * kTileC + 4 * cq]) =
          pack4_i8(quant_one(v[i].x, s0), quant_one(v[i].y, s1), quant_one(v[i].z, s2),
                   quant_one(v[i].w, s3));
  }
  __syncthreads();

  // Output frames t0 + fr + 16 i, channels 4cq..4cq+3.
  for (int o = fr; o < kTileT; o += 16) {
    const int t = t0 + o;
    if (t >= p.T) break;
    int acc[4] = {0, 0, 0, 0};
    for (int j = 0; j < p.k; ++j) {
      const uint32_t w = *reinterpret_cast<const uint32_t *>(&xq[(o + j) * kTileC + 4 * cq]);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        acc[e] += (int)(int8_t)((w >> (8 * e)) & 0xff) * (int)qk[4 * cq + e][j];
    }
    const size_t off = ((size_t)b * p.T + t) * p.C + c0 + 4 * cq;
    f32x4 out;
    float *ov = reinterpret_cast<float *>(&out);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int c = 4 * cq + e;
      double v = (double)acc[e] * (double)sw[c] / (double)sx[c];
      if (p.bias) v += (double)bs[c];
      if (RELU && v <= 0.0) v = 0.0;
      ov[e] = (float)v;
    }
    st_global<f32x4>(p.y + off, out);
    if (p.acc_out) st_global<v4i>(p.acc_out + off, v4i{acc[0], acc[1], acc[2], acc[3]});
  }
}

// Weight quantization per channel, one thread per channel (k <= kMaxDwTaps).
__global__ void __launch_bounds__(kThreads) dw_quant_weights_kernel(const float *W, int C, int k,
                                                                    int8_t *q, float *w_scale) {
  const int c = blockIdx.x * kThreads + threadIdx.x;
  if (c >= C) return;
  float a = 0.0f;
  for (int j = 0; j < k; ++j) a = fmaxf(a, fabsf(ld_global<float>(W + (size_t)c * k + j)));
  const float s = a / 127.0f;
  st_global<float>(w_scale + c, a == 0.0f ? 0.0f : s);
  for (int j = 0; j < k; ++j) {
    int v = 0;
    if (a != 0.0f) {
      const float r = __builtin_rintf(ld_global<float>(W + (size_t)c * k + j) / s);
      v = (int)fminf(fmaxf(r, -127.0f), 127.0f);
    }
    q[(size_t)c * k + j] = (int8_t)v;
  }
}

}  // namespace

int dw_chunks(int64_t T) { return (int)((T + kChunkFrames - 1) / kChunkFrames); }

hipError_t launch_dw_quant_weights(const float *W, int64_t C, int64_t k, int8_t *q,
                                   float *w_scale, hipStream_t stream) {
  dw_quant_weights_kernel<<<(unsigned)((C + kThreads - 1) / kThreads), kThreads, 0, stream>>>(
      W, (int)C, (int)k, q, w_scale);
  return hipGetLastError();
}

hipError_t launch_dwconv(int B, int T, int C, int k, const float *x, const int8_t *q,
                         const float *w_scale, const float *bias, int relu, float *y,
                         float *partial, int32_t *acc_out, float *x_scale_out,
                         hipStream_t stream) {
  const int nchunk = dw_chunks(T);
  colmax_kernel<<<dim3(nchunk, C / kTileC, B), kThreads, 0, stream>>>(x, T, C, nchunk, partial);
  colscale_kernel<<<(unsigned)((B * C + kThreads - 1) / kThreads), kThreads, 0, stream>>>(
      partial, B, C, nchunk, x_scale_out);
  DwParams p{x, q, w_scale, bias, y, acc_out, nullptr, partial, B, T, C, k, nchunk, relu};
  const dim3 grid((T + kTileT - 1) / kTileT, C / kTileC, B);
  if (relu)
    dwconv_kernel<true><<<grid, kThreads, 0, stream>>>(p);
  else
    dwconv_kernel<false><<<grid, kThreads, 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace bitnet
