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
// Launches (both HBM-bound): colmax_kernel writes the maximum |x| of each
// (sequence, frame chunk, channel) to the workspace, with chunks of 128 frames
// or more so that a sequence has at most kMaxChunks of them; dwconv_kernel
// takes one sequence's 64-frame x 64-channel output tile, reduces its
// channels' chunk maxima to the scales, quantizes the tile's input frames (6
// halo frames before it for k = 7) into LDS, and convolves from LDS.
#include <algorithm>

#include "bitnet_device.hpp"
#include "bitnet_internal.hpp"
#include "bitnet_variants.hpp"

namespace bitnet {
namespace {

constexpr int kThreads = 256;
constexpr int kMinChunkFrames = 128;   // frames per partial maximum, at least
constexpr int kMaxChunks = 64;         // partial maxima per (sequence, channel), at most
constexpr int kTileC = 64;             // channels per workgroup tile
constexpr int kTileT = 64;             // output frames per workgroup tile
// LDS row of the quantized tile: 64 channels plus 16 bytes of padding, so the
// rows 4 apart that the 4 frame groups of a wave read together start 20 words
// apart and fall in different banks.
constexpr int kRowStride = kTileC + 16;

struct DwParams {
  const float *x;          // [B][T][C]
  const int8_t *q;         // [C][k]
  const float *w_scale;    // [C]
  const float *bias;       // [C] or null
  float *y;                // [B][T][C]
  int32_t *acc_out;        // [B][T][C] or null
  float *x_scale_out;      // [B][C] or null
  const float *partial;    // [B][nchunk][C] chunk maxima
  int B, T, C, k, nchunk, relu;
};

__host__ __device__ inline int chunk_frames(int64_t T) {
  int cf = kMinChunkFrames;
  while ((T + cf - 1) / cf > kMaxChunks) cf *= 2;
  return cf;
}

// Workgroup (chunk, channel tile, b): thread (cq = tid % 16, fr = tid / 16)
// takes channels 4cq..4cq+3 of the tile and frames fr, fr + 16, ... of the
// chunk, 8 loads in flight at a time; the 16 frame lanes are then reduced
// through LDS.
__global__ void __launch_bounds__(kThreads) colmax_kernel(const float *x, int T, int C,
                                                          int nchunk, int cf, float *partial) {
  __shared__ f32x4 red[kThreads];
  const int chunk = blockIdx.x, c0 = blockIdx.y * kTileC, b = blockIdx.z;
  const int tid = threadIdx.x, cq = tid & 15, fr = tid >> 4;
  const int t0 = chunk * cf, t1 = min(t0 + cf, T);
  const f32x4 *x4 = reinterpret_cast<const f32x4 *>(x + (size_t)b * T * C + c0) + cq;
  f32x4 m = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  for (int tb = t0; tb < t1; tb += 8 * 16) {
    f32x4 v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int t = tb + fr + 16 * i;
      v[i] = t < t1 ? ld_global<f32x4>(x4 + (size_t)t * (C / 4)) : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      m.x = fmaxf(m.x, fabsf(v[i].x));
      m.y = fmaxf(m.y, fabsf(v[i].y));
      m.z = fmaxf(m.z, fabsf(v[i].z));
      m.w = fmaxf(m.w, fabsf(v[i].w));
    }
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

__device__ __forceinline__ f32x4 max4(f32x4 a, f32x4 b) {
  return f32x4{fmaxf(a.x, b.x), fmaxf(a.y, b.y), fmaxf(a.z, b.z), fmaxf(a.w, b.w)};
}

// Byte e of w, sign-extended.
__device__ __forceinline__ int sbyte(uint32_t w, int e) { return (int)(int8_t)(w >> (8 * e)); }

template <bool RELU>
__global__ void __launch_bounds__(kThreads) dwconv_kernel(DwParams p) {
  __shared__ f32x4 red[kThreads];
  __shared__ float sx[kTileC], sw[kTileC], bs[kTileC];
  __shared__ uint32_t taps[kMaxDwTaps][kTileC / 4];   // word cq of tap j: channels 4cq..4cq+3
  // quantized input frames t0 - (k-1) .. t0 + kTileT - 1, 64 channels each
  __shared__ __attribute__((aligned(16))) int8_t xq[(kTileT + kMaxDwTaps - 1) * kRowStride];
  const int tt = blockIdx.x, c0 = blockIdx.y * kTileC, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int t0 = tt * kTileT;
  const int halo = p.k - 1;
  const int cq = tid & 15, fr = tid >> 4;

  // The tile's input frames t0 - halo .. t0 + kTileT - 1 (frames before 0 and
  // past T are zeros) and the chunk maxima of its channels (chunks fr, fr + 16,
  // fr + 32, fr + 48), all loads of a thread at once.
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
  const f32x4 *pm =
      reinterpret_cast<const f32x4 *>(p.partial + (size_t)b * p.nchunk * p.C + c0) + cq;
  f32x4 cm[kMaxChunks / 16];
#pragma unroll
  for (int i = 0; i < kMaxChunks / 16; ++i) {
    const int ch = fr + 16 * i;
    cm[i] = ch < p.nchunk ? ld_global<f32x4>(pm + (size_t)ch * (p.C / 4))
                          : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }
  if (tid < kTileC) {
    sw[tid] = ld_global<float>(p.w_scale + c0 + tid);
    bs[tid] = p.bias ? ld_global<float>(p.bias + c0 + tid) : 0.0f;
  }
  for (int i = tid; i < p.k * (kTileC / 4); i += kThreads) {
    const int j = i / (kTileC / 4), g = i - j * (kTileC / 4);
    const int8_t *qc = p.q + (size_t)(c0 + 4 * g) * p.k + j;
    taps[j][g] = pack4_i8(ld_global<int8_t>(qc), ld_global<int8_t>(qc + p.k),
                          ld_global<int8_t>(qc + 2 * p.k), ld_global<int8_t>(qc + 3 * p.k));
  }
  red[tid] = max4(max4(cm[0], cm[1]), max4(cm[2], cm[3]));
  __syncthreads();
  if (tid < 16) {
    f32x4 a = red[tid];
    for (int r = 1; r < 16; ++r) a = max4(a, red[r * 16 + tid]);
    const float *av = reinterpret_cast<const float *>(&a);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float s = (av[e] == 0.0f) ? 1.0f : 127.0f / av[e];
      sx[4 * tid + e] = s;
      if (p.x_scale_out && tt == 0)
        st_global<float>(p.x_scale_out + (size_t)b * p.C + c0 + 4 * tid + e, s);
    }
  }
  __syncthreads();
  const float s0 = sx[4 * cq], s1 = sx[4 * cq + 1], s2 = sx[4 * cq + 2], s3 = sx[4 * cq + 3];
#pragma unroll
  for (int i = 0; i < kRowLoads; ++i) {
    const int r = fr + 16 * i;
    if (r < rows)
      *reinterpret_cast<uint32_t *>(&xq[r * kRowStride + 4 * cq]) =
          pack4_i8(quant_one(v[i].x, s0), quant_one(v[i].y, s1), quant_one(v[i].z, s2),
                   quant_one(v[i].w, s3));
  }
  __syncthreads();

  // Output frames t0 + 4fr .. t0 + 4fr + 3, channels 4cq..4cq+3: a window of
  // four input rows slides over the taps, one new row and one tap word per tap.
  const int o0 = 4 * fr;
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    w[i] = *reinterpret_cast<const uint32_t *>(&xq[(o0 + i) * kRowStride + 4 * cq]);
  int acc[4][4] = {};
  for (int j = 0; j < p.k; ++j) {
    const uint32_t tw = taps[j][cq];
    int tv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) tv[e] = sbyte(tw, e);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[i][e] += sbyte(w[i], e) * tv[e];
    w[0] = w[1];
    w[1] = w[2];
    w[2] = w[3];
    if (j + 1 < p.k)
      w[3] = *reinterpret_cast<const uint32_t *>(&xq[(o0 + 4 + j) * kRowStride + 4 * cq]);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + o0 + i;
    if (t >= p.T) break;
    const size_t off = ((size_t)b * p.T + t) * p.C + c0 + 4 * cq;
    f32x4 out;
    float *ov = reinterpret_cast<float *>(&out);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int c = 4 * cq + e;
      double val = (double)acc[i][e] * (double)sw[c] / (double)sx[c];
      if (p.bias) val += (double)bs[c];
      if (RELU && val <= 0.0) val = 0.0;
      ov[e] = (float)val;
    }
    st_global<f32x4>(p.y + off, out);
    if (p.acc_out)
      st_global<v4i>(p.acc_out + off, v4i{acc[i][0], acc[i][1], acc[i][2], acc[i][3]});
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

int dw_chunks(int64_t T) {
  const int cf = chunk_frames(T);
  return (int)((T + cf - 1) / cf);
}

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
  colmax_kernel<<<dim3(nchunk, C / kTileC, B), kThreads, 0, stream>>>(x, T, C, nchunk,
                                                                      chunk_frames(T), partial);
  DwParams p{x, q, w_scale, bias, y, acc_out, x_scale_out, partial, B, T, C, k, nchunk, relu};
  const dim3 grid((T + kTileT - 1) / kTileT, C / kTileC, B);
  if (relu)
    dwconv_kernel<true><<<grid, kThreads, 0, stream>>>(p);
  else
    dwconv_kernel<false><<<grid, kThreads, 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace bitnet
