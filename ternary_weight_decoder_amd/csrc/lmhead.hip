// The decoder's 8-bit table with one scale per row: token embeddings and the
// lm_head.
//
// The ONNX build stores the embeddings and the lm_head at 8 bits with one
// scale per row / per column, where the GGUF build uses Q6_K (ONNX model card
// "multimodalart/VibeVoice-ASR-BitNet-ONNX", Quantization table, row
// "Embeddings / lm_head").  One [V, K] table serves both: row v is token v's
// embedding and, read as the lm_head weight, the weights of output column v,
// so the per-row scales are the lm_head's per-column scales.
//
//   - Quantization (offline), one wave per row: s = fl32(max|W[v,:]| / 127),
//     q = clamp(rint(fl32(W / s)), +-127); a zero row gives s = 0, q = 0.
//   - Embedding lookup: e[t,k] = fl32(q[id,k] * s[id]); an id outside [0, V)
//     gives a zero row.
//   - lm_head (M <= 16 rows): activations quantized per row (absmax int8, as
//     every projection of the decoder), acc = sum_k xq * q in int32 on
//     v_mfma_i32_16x16x64_i8, y = acc * s[v] / x_scale[m] rounded once.
//
// lm_head work split.  The table is read once per call, so the kernel is an
// HBM stream of V*K bytes (233 MB for the 151,936 x 1536 table).  Each wave
// owns a contiguous run of whole 16-column blocks, the same number for every
// wave, and walks them with a ring of items kept `D` ahead: item (b, c) is
// block b's 256 inputs [256c, 256c + 256).  Lane (col = lane % 16, h = lane
// / 16) loads, for step j = 0..3 of the item, the 16 bytes at input
// 256c + 64j + 16h of table row 16b + col; one such load instruction covers 64
// contiguous bytes of each of 16 rows.  The activation operand of MFMA j is
// the 16 bytes at the same inputs of row col of the quantized rows in LDS, so
// both operands of every MFMA agree on k.  Loads past V, past K or past the
// wave's run are aimed beyond the buffer and return zeros without a memory
// access.  The workgroup quantizes the rows into LDS itself, after issuing the
// first D items, so the first weight loads overlap the quantization.
#include <algorithm>

#include "bitnet_device.hpp"
#include "bitnet_internal.hpp"
#include "bitnet_variants.hpp"

namespace bitnet {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kItemK = 256;               // inputs per ring item
constexpr int kRowPad = 16;               // bytes between quantized rows in LDS
#ifndef BITNET_LMHEAD_DEPTH
#define BITNET_LMHEAD_DEPTH 4
#endif
#ifndef BITNET_LMHEAD_WAVES
#define BITNET_LMHEAD_WAVES 2048
#endif
constexpr int kDepth = BITNET_LMHEAD_DEPTH;       // items in flight per wave
constexpr int kTargetWaves = BITNET_LMHEAD_WAVES; // waves of a launch, before balancing
constexpr int kMaxBpw = 8;                        // blocks per wave at most
// The table is read once per call: non-temporal loads keep it from evicting
// the quantized rows and scales.
constexpr int kTableAux = 2;

struct LmShared {
  float red[kGemvMaxM][kWaves];
  float scale[kGemvMaxM];
};

struct LmParams {
  const float *x;          // [M][K]
  const int8_t *q;         // [V][K]
  const float *w_scale;    // [V]
  float *y;                // [M][V]
  int8_t *xq_out;          // optional [M][K]
  float *x_scale_out;      // optional [M]
  int32_t *acc_out;        // optional [M][V]
  int M, V, K;
  int blocks_per_wave;     // 16-column blocks of each wave
  int nblk;                // 16-column blocks of the table
};

// Quantize the M rows of x into LDS (natural order, row stride K + kRowPad):
// pass 1 takes each row's absmax, pass 2 scales, rounds and stores.
__device__ __forceinline__ void lm_quant_rows(const LmParams &p, LmShared &sh, int8_t *xq,
                                              bool write_out) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n4 = p.K >> 2;
  const int stride = p.K + kRowPad;
  for (int m = 0; m < p.M; ++m) {
    const f32x4 *x4 = reinterpret_cast<const f32x4 *>(p.x + (size_t)m * p.K);
    float a = 0.0f;
    for (int i = tid; i < n4; i += kThreads) {
      const f32x4 v = ld_global<f32x4>(x4 + i);
      a = fmaxf(a, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
    }
    a = wave_max(a);
    if (lane == 0) sh.red[m][wave] = a;
  }
  __syncthreads();
  for (int m = 0; m < p.M; ++m) {
    const float a = fmaxf(fmaxf(sh.red[m][0], sh.red[m][1]), fmaxf(sh.red[m][2], sh.red[m][3]));
    const float s = (a == 0.0f) ? 1.0f : 127.0f / a;
    const f32x4 *x4 = reinterpret_cast<const f32x4 *>(p.x + (size_t)m * p.K);
    int8_t *dst = xq + (size_t)m * stride;
    for (int i = tid; i < n4; i += kThreads) {
      const f32x4 v = ld_global<f32x4>(x4 + i);
      const uint32_t w = pack4_i8(quant_one(v.x, s), quant_one(v.y, s), quant_one(v.z, s),
                                  quant_one(v.w, s));
      *reinterpret_cast<uint32_t *>(dst + 4 * i) = w;
      if (write_out) st_global<uint32_t>(p.xq_out + (size_t)m * p.K + 4 * i, w);
    }
    if (tid == 0) {
      sh.scale[m] = s;
      if (write_out) st_global<float>(p.x_scale_out + m, s);
    }
  }
  __syncthreads();
}

// Dynamic LDS of one workgroup: the quantized rows [M][K + kRowPad], then per
// wave the column scales of its run [kMaxBpw * 16] and its int32 accumulators
// [bpw][M][16].  The outputs are dequantized and stored after the loop, so
// nothing inside the streaming loop waits on vector memory except the table
// ring itself (one counter covers a wave's loads and stores).
// (The rows region ends kItemK bytes past the last row: the operand reads of a
// last, partial item run up to that far past K.)
__host__ __device__ inline size_t lm_rows_bytes(int M, int K) {
  return (size_t)M * (K + kRowPad) + kItemK;
}
__host__ __device__ inline size_t lm_wave_bytes(int M, int bpw) {
  return (size_t)kMaxBpw * 16 * 4 + (size_t)bpw * 16 * 4 * M;
}

template <int D>
__global__ void __launch_bounds__(kThreads) lm_head_kernel(LmParams p) {
  __shared__ LmShared sh;
  extern __shared__ __attribute__((aligned(16))) int8_t lds[];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;
  const int h = lane >> 4;
  const int bpw = p.blocks_per_wave;
  const int gwave = blockIdx.x * kWaves + wave;
  const int blk0 = gwave * bpw;
  const int nb = max(0, min(bpw, p.nblk - blk0));   // blocks of this wave
  const int cpb = (p.K + kItemK - 1) / kItemK;     // items per block
  const int items = nb * cpb;
  int8_t *xq_lds = lds;
  float *wave_lds = reinterpret_cast<float *>(lds + lm_rows_bytes(p.M, p.K) +
                                              (size_t)wave * lm_wave_bytes(p.M, bpw));
  float *scale_lds = wave_lds;                                           // [kMaxBpw * 16]
  int *acc_lds = reinterpret_cast<int *>(wave_lds + kMaxBpw * 16);       // [bpw][M][16]

  const uint32_t q_bytes = (uint32_t)((size_t)p.V * p.K);
  const __amdgpu_buffer_rsrc_t q_rsrc = make_rsrc(p.q, q_bytes);
  // Next item to fetch: block fb of the wave's run, chunk fc of that block.
  int fb = 0, fc = 0, fetched = 0;
  auto load_item = [&](v4i (&w)[4]) {
    const int n = (blk0 + fb) * 16 + col;
    const bool live = fetched < items && n < p.V;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int k = fc * kItemK + 64 * j + 16 * h;
      const uint32_t off = (live && k < p.K) ? (uint32_t)n * (uint32_t)p.K + (uint32_t)k : q_bytes;
      w[j] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(q_rsrc, off, 0,
                                                                            kTableAux));
    }
    ++fetched;
    if (++fc == cpb) {
      fc = 0;
      ++fb;
    }
  };
  v4i wr[D][4];
#pragma unroll
  for (int d = 0; d < D; ++d) load_item(wr[d]);
  // The column scales of the wave's run (at most 2 per lane); the
  // quantization's waits cover their loads, and they go to LDS after it.
  float sv[kMaxBpw * 16 / 64];
#pragma unroll
  for (int t = 0; t < kMaxBpw * 16 / 64; ++t) {
    const int i = lane + 64 * t, n = blk0 * 16 + i;
    sv[t] = (i < nb * 16 && n < p.V) ? ld_global<float>(p.w_scale + n) : 0.0f;
  }

  lm_quant_rows(p, sh, xq_lds, p.xq_out != nullptr && blockIdx.x == 0);
  // (Written unconditionally: a load whose value some path leaves unused
  // would make the compiler wait for all loads at the top of the loop.)
#pragma unroll
  for (int t = 0; t < kMaxBpw * 16 / 64; ++t) scale_lds[lane + 64 * t] = sv[t];

  // Operand rows: lanes of rows past M read row M - 1 (their outputs are never
  // stored), and reads past K meet zero weights (those loads return zeros), so
  // the operand reads need no condition.
  const int stride = p.K + kRowPad;
  const int8_t *arow = xq_lds + (size_t)min(col, p.M - 1) * stride + 16 * h;
  const v4i zero4 = v4i{0, 0, 0, 0};
  v4i acc = zero4;
  int cb = 0, cc = 0;   // block and chunk of the item being consumed
  for (int base = 0; base < items; base += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      if (base + d < items) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const v4i a = *reinterpret_cast<const v4i *>(arow + cc * kItemK + 64 * j);
          acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, wr[d][j], acc, 0, 0, 0);
        }
        if (++cc == cpb) {
          // Block done: element (row = 4h + r, column 16 cb + col of the run).
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = 4 * h + r;
            if (row < p.M) acc_lds[(cb * p.M + row) * 16 + col] = acc[r];
          }
          acc = zero4;
          cc = 0;
          ++cb;
        }
      }
      load_item(wr[d]);
    }
  }
  // The run's outputs: row m of the run is 16 nb contiguous columns of y.
  const int run_cols = nb * 16;
  for (int m = 0; m < p.M; ++m) {
    const float xs = sh.scale[m];
    for (int i = lane; i < run_cols; i += 64) {
      const int n = blk0 * 16 + i;
      if (n < p.V) {
        const int a = acc_lds[((i >> 4) * p.M + m) * 16 + (i & 15)];
        if (p.acc_out) st_global<int>(p.acc_out + (size_t)m * p.V + n, a);
        st_global<float>(p.y + (size_t)m * p.V + n, dequant_exact(a, scale_lds[i], xs));
      }
    }
  }
}

// Per-row quantization, one wave per row.
__global__ void __launch_bounds__(kThreads) rowq_quant_kernel(const float *W, int N, int K,
                                                              int8_t *q, float *w_scale) {
  const int lane = threadIdx.x & 63;
  const int n = blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (n >= N) return;
  const int n4 = K >> 2;
  const f32x4 *w4 = reinterpret_cast<const f32x4 *>(W + (size_t)n * K);
  float a = 0.0f;
  for (int i = lane; i < n4; i += 64) {
    const f32x4 v = ld_global<f32x4>(w4 + i);
    a = fmaxf(a, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
  }
  a = wave_max(a);
  const float s = a / 127.0f;
  if (lane == 0) st_global<float>(w_scale + n, a == 0.0f ? 0.0f : s);
  for (int i = lane; i < n4; i += 64) {
    uint32_t packed = 0;
    if (a != 0.0f) {
      const f32x4 v = ld_global<f32x4>(w4 + i);
      int c[4] = {0, 0, 0, 0};
      const float e[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        float r = __builtin_rintf(e[t] / s);   // IEEE quotient, half to even
        c[t] = (int)fminf(fmaxf(r, -127.0f), 127.0f);
      }
      packed = pack4_i8(c[0], c[1], c[2], c[3]);
    }
    st_global<uint32_t>(q + (size_t)n * K + 4 * i, packed);
  }
}

// Embedding rows, one wave per token.
__global__ void __launch_bounds__(kThreads) embed_kernel(const int32_t *ids, int T,
                                                         const int8_t *q, const float *w_scale,
                                                         int N, int K, float *out) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (t >= T) return;
  const int id = ld_global<int>(ids + t);
  const bool live = id >= 0 && id < N;
  const float s = live ? ld_global<float>(w_scale + id) : 0.0f;
  const int n4 = K >> 2;
  for (int i = lane; i < n4; i += 64) {
    f32x4 v = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    if (live) {
      const uint32_t d = ld_global<uint32_t>(q + (size_t)id * K + 4 * i);
      v.x = (float)(int8_t)(d & 0xff) * s;
      v.y = (float)(int8_t)((d >> 8) & 0xff) * s;
      v.z = (float)(int8_t)((d >> 16) & 0xff) * s;
      v.w = (float)(int8_t)(d >> 24) * s;
    }
    st_global<f32x4>(out + (size_t)t * K + 4 * i, v);
  }
}

}  // namespace

// Blocks per wave: every wave runs the same number of whole 16-column blocks,
// ceil(nblk / kTargetWaves), at most kMaxBpw, and fewer if the workgroup's
// LDS would not fit kLmHeadMaxLds (with M * (K + 16) <= kLmHeadMaxRows one
// block per wave always fits).
int lm_bpw(int64_t M, int64_t V, int64_t K) {
  const int64_t nblk = (V + 15) / 16;
  int bpw = (int)std::min<int64_t>(kMaxBpw, (nblk + kTargetWaves - 1) / kTargetWaves);
  while (bpw > 1 && lm_rows_bytes((int)M, (int)K) + kWaves * lm_wave_bytes((int)M, bpw) >
                        kLmHeadMaxLds)
    --bpw;
  return bpw;
}

size_t lm_head_lds_bytes(int64_t M, int64_t V, int64_t K) {
  return lm_rows_bytes((int)M, (int)K) + kWaves * lm_wave_bytes((int)M, lm_bpw(M, V, K));
}

hipError_t launch_rowq_quant(const float *W, int64_t N, int64_t K, int8_t *q, float *w_scale,
                             hipStream_t stream) {
  const int64_t blocks = (N + kWaves - 1) / kWaves;
  rowq_quant_kernel<<<(unsigned)blocks, kThreads, 0, stream>>>(W, (int)N, (int)K, q, w_scale);
  return hipGetLastError();
}

hipError_t launch_embed(const int32_t *ids, int64_t T, const int8_t *q, const float *w_scale,
                        int64_t N, int64_t K, float *out, hipStream_t stream) {
  const int64_t blocks = (T + kWaves - 1) / kWaves;
  embed_kernel<<<(unsigned)blocks, kThreads, 0, stream>>>(ids, (int)T, q, w_scale, (int)N,
                                                          (int)K, out);
  return hipGetLastError();
}

// Waves get equal runs of whole blocks: bpw = ceil(nblk / target), then as
// few waves as that needs.
hipError_t launch_lm_head(int M, int V, int K, const float *x, const int8_t *q,
                          const float *w_scale, float *y, int8_t *xq_out, float *x_scale_out,
                          int32_t *acc_out, hipStream_t stream) {
  LmParams p{x, q, w_scale, y, xq_out, x_scale_out, acc_out, M, V, K, 0, 0};
  p.nblk = (V + 15) / 16;
  p.blocks_per_wave = lm_bpw(M, V, K);
  const int waves = (p.nblk + p.blocks_per_wave - 1) / p.blocks_per_wave;
  const int blocks = (waves + kWaves - 1) / kWaves;
  lm_head_kernel<kDepth><<<blocks, kThreads, lm_head_lds_bytes(M, V, K), stream>>>(p);
  return hipGetLastError();
}

}  // namespace bitnet
