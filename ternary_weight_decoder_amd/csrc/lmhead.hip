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
// Storage order.  The table is kept in 16-row x 256-input tiles of 4096
// contiguous bytes, ordered by row group and then by input chunk; inside a
// tile, input k = 64j + 16h + e of tile row r sits at byte 1024j + 256h + 16r
// + e.  Rows and inputs are padded with zero codes to multiples of 16 and 256.
//
// lm_head work split.  The table is read once per call, so the kernel is an
// HBM stream of its bytes (233 MB for the 151,936 x 1536 table).  Each wave
// owns a contiguous run of whole 16-column blocks (row groups), the same
// number for every wave, and walks them with a ring of items kept `D` ahead:
// item (b, c) is tile c of row group b.  Lane L = col + 16h loads, for step
// j = 0..3 of the item, the 16 bytes at tile byte 1024j + 16L: table row
// 16b + col, inputs 256c + 64j + 16h .. + 16.  One load instruction reads 1 KB
// contiguous, and a wave's run is one contiguous stretch of the table.  The
// activation operand of MFMA j is the 16 bytes at the same inputs of row col
// of the quantized rows in LDS, so both operands of every MFMA agree on k;
// padding inputs carry zero codes.  Loads past the wave's run are aimed beyond
// the buffer and return zeros without a memory access.  The workgroup
// quantizes the rows into LDS itself: their loads are issued before the first
// D items, so the table loads overlap the quantization, and waiting for the
// rows does not wait for the table's HBM reads.
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
#define BITNET_LMHEAD_DEPTH 6
#endif
#ifndef BITNET_LMHEAD_WAVES
#define BITNET_LMHEAD_WAVES 2048
#endif
constexpr int kDepth = BITNET_LMHEAD_DEPTH;       // items in flight per wave
constexpr int kTargetWaves = BITNET_LMHEAD_WAVES; // waves of a launch, before balancing
constexpr int kMaxBpw = 8;                        // blocks per wave at most
constexpr int kTileBytes = 16 * kItemK;   // one 16-row x 256-input tile
// Cache policy of the table loads, which are read once per call: non-temporal
// (on this storage order 36.2 us per call against 41.2 us for plain loads).
#ifndef BITNET_LMHEAD_AUX
#define BITNET_LMHEAD_AUX 2
#endif
constexpr int kTableAux = BITNET_LMHEAD_AUX;

struct LmShared {
  uint32_t amax[kGemvMaxM];   // bit patterns of the rows' absmax
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

// Quantize the M rows of x into LDS (natural order, row stride K + kRowPad).
// The rows are one flat run of M*K/4 fp32 quads; each thread takes every
// kThreads-th quad, kQuantBatch loads at a time, so a pass costs a few memory
// round trips however many rows there are.  Pass 1 takes each row's absmax
// (non-negative floats order like their bit patterns: an integer max in LDS,
// one per wave when the wave's quads lie in one row); pass 2 scales, rounds
// and stores.
constexpr int kQuantBatch = 8;

__device__ __forceinline__ void lm_quant_rows(const LmParams &p, LmShared &sh, int8_t *xq,
                                              bool write_out) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n4 = p.K >> 2;
  const int total = p.M * n4;
  const int stride = p.K + kRowPad;
  const f32x4 *x4 = reinterpret_cast<const f32x4 *>(p.x);
  if (tid < p.M) sh.amax[tid] = 0u;
  __syncthreads();
  for (int e0 = 0; e0 < total; e0 += kQuantBatch * kThreads) {
    f32x4 v[kQuantBatch];
#pragma unroll
    for (int u = 0; u < kQuantBatch; ++u) {
      const int e = e0 + u * kThreads + tid;
      v[u] = e < total ? ld_global<f32x4>(x4 + e) : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
#pragma unroll
    for (int u = 0; u < kQuantBatch; ++u) {
      const int w0 = e0 + u * kThreads + 64 * wave;   // first quad of this wave
      if (w0 >= total) break;
      const int e = w0 + lane;
      float a = fmaxf(fmaxf(fabsf(v[u].x), fabsf(v[u].y)), fmaxf(fabsf(v[u].z), fabsf(v[u].w)));
      const int m0 = w0 / n4, m1 = min(w0 + 63, total - 1) / n4;
      if (m0 == m1) {
        a = wave_max(a);
        if (lane == 0) atomicMax(&sh.amax[m0], __builtin_bit_cast(uint32_t, a));
      } else if (e < total) {
        atomicMax(&sh.amax[e / n4], __builtin_bit_cast(uint32_t, a));
      }
    }
  }
  __syncthreads();
  if (tid < p.M) {
    const float a = __builtin_bit_cast(float, sh.amax[tid]);
    const float s = (a == 0.0f) ? 1.0f : 127.0f / a;
    sh.scale[tid] = s;
    if (write_out) st_global<float>(p.x_scale_out + tid, s);
  }
  __syncthreads();
  for (int e0 = 0; e0 < total; e0 += kQuantBatch * kThreads) {
    f32x4 v[kQuantBatch];
#pragma unroll
    for (int u = 0; u < kQuantBatch; ++u) {
      const int e = e0 + u * kThreads + tid;
      v[u] = e < total ? ld_global<f32x4>(x4 + e) : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
#pragma unroll
    for (int u = 0; u < kQuantBatch; ++u) {
      const int e = e0 + u * kThreads + tid;
      if (e < total) {
        const int m = e / n4, i = e - m * n4;
        const float s = sh.scale[m];
        const uint32_t w = pack4_i8(quant_one(v[u].x, s), quant_one(v[u].y, s),
                                    quant_one(v[u].z, s), quant_one(v[u].w, s));
        *reinterpret_cast<uint32_t *>(xq + (size_t)m * stride + 4 * i) = w;
        if (write_out) st_global<uint32_t>(p.xq_out + 4 * (size_t)e, w);
      }
    }
  }
  __syncthreads();
}

// The same from rows already held in registers: the M rows as one flat run of
// M*K/4 fp32 quads, thread t holding quads t, t + kThreads, ... (NQ of them,
// zeros past the run), loaded by lm_load_rows before the workgroup's first
// table loads.  The loads of a wave complete in issue order, so rows loaded
// after the table ring could only be used once the ring's HBM reads had
// landed, and every further pass over the rows would then run with the ring
// full and the table stream stalled.  sh.amax must be zero before the call.
template <int NQ>
__device__ __forceinline__ void lm_load_rows(const LmParams &p, f32x4 (&v)[NQ]) {
  const uint32_t total = (uint32_t)p.M * (uint32_t)(p.K >> 2);
  const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(p.x, total * 16u);
#pragma unroll
  for (int u = 0; u < NQ; ++u) {
    const uint32_t e = (uint32_t)(u * kThreads) + threadIdx.x;
    v[u] = __builtin_bit_cast(
        f32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, (e < total ? e : total) * 16u, 0, 0));
  }
}

template <int NQ>
__device__ __forceinline__ void lm_quant_resident(const LmParams &p, LmShared &sh, int8_t *xq,
                                                  bool write_out, const f32x4 (&v)[NQ]) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n4 = p.K >> 2;
  const int total = p.M * n4;
  const int stride = p.K + kRowPad;
#pragma unroll
  for (int u = 0; u < NQ; ++u) {
    const int w0 = u * kThreads + 64 * wave;   // first quad of this wave
    if (w0 >= total) break;
    const int e = w0 + lane;
    float a = fmaxf(fmaxf(fabsf(v[u].x), fabsf(v[u].y)), fmaxf(fabsf(v[u].z), fabsf(v[u].w)));
    const int m0 = w0 / n4, m1 = min(w0 + 63, total - 1) / n4;
    if (m0 == m1) {
      a = wave_max(a);
      if (lane == 0) atomicMax(&sh.amax[m0], __builtin_bit_cast(uint32_t, a));
    } else if (e < total) {
      atomicMax(&sh.amax[e / n4], __builtin_bit_cast(uint32_t, a));
    }
  }
  __syncthreads();
  if (tid < p.M) {
    const float a = __builtin_bit_cast(float, sh.amax[tid]);
    const float s = (a == 0.0f) ? 1.0f : 127.0f / a;
    sh.scale[tid] = s;
    if (write_out) st_global<float>(p.x_scale_out + tid, s);
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < NQ; ++u) {
    const int e = u * kThreads + tid;
    if (e < total) {
      const int m = e / n4, i = e - m * n4;
      const float s = sh.scale[m];
      const uint32_t w = pack4_i8(quant_one(v[u].x, s), quant_one(v[u].y, s),
                                  quant_one(v[u].z, s), quant_one(v[u].w, s));
      *reinterpret_cast<uint32_t *>(xq + (size_t)m * stride + 4 * i) = w;
      if (write_out) st_global<uint32_t>(p.xq_out + 4 * (size_t)e, w);
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

// Rows held by whole waves (rows of up to kRowQuads * 256 inputs): wave w
// holds rows w, w + 4, ... (RPW of them) in registers, lane l quads l, l + 64,
// ... of each (zeros past the row and for rows past M), loaded before the
// workgroup's first table loads.  A row's absmax is then one wave reduction:
// no cross-wave atomics, no per-quad row arithmetic, and one barrier for the
// whole quantization.  At M = 16 this took the call from 53.1 to 43.8 us (a
// probe without any quantization ran 44.0 us); M = 1 and 4 are unchanged.
constexpr int kRowQuads = 6;

template <int RPW>
__device__ __forceinline__ void lm_load_wave_rows(const LmParams &p, int wave,
                                                  f32x4 (&v)[RPW][kRowQuads]) {
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t n4 = (uint32_t)(p.K >> 2);
  const uint32_t total = (uint32_t)p.M * n4;
  const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(p.x, total * 16u);
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const uint32_t m = (uint32_t)(4 * r + wave);
#pragma unroll
    for (int j = 0; j < kRowQuads; ++j) {
      const uint32_t i = 64u * j + lane;
      const uint32_t off = (m < (uint32_t)p.M && i < n4) ? (m * n4 + i) * 16u : total * 16u;
      v[r][j] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, off, 0, 0));
    }
  }
}

template <int RPW>
__device__ __forceinline__ void lm_quant_wave_rows(const LmParams &p, LmShared &sh, int8_t *xq,
                                                   bool write_out, int wave,
                                                   const f32x4 (&v)[RPW][kRowQuads]) {
  const int lane = threadIdx.x & 63;
  const int n4 = p.K >> 2;
  const int stride = p.K + kRowPad;
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const int m = 4 * r + wave;   // uniform
    if (m >= p.M) break;
    float a = 0.0f;
#pragma unroll
    for (int j = 0; j < kRowQuads; ++j)
      a = fmaxf(a, fmaxf(fmaxf(fabsf(v[r][j].x), fabsf(v[r][j].y)),
                         fmaxf(fabsf(v[r][j].z), fabsf(v[r][j].w))));
    a = wave_max(a);
    const float s = (a == 0.0f) ? 1.0f : 127.0f / a;
    if (lane == 0) {
      sh.scale[m] = s;
      if (write_out) st_global<float>(p.x_scale_out + m, s);
    }
#pragma unroll
    for (int j = 0; j < kRowQuads; ++j) {
      const int i = 64 * j + lane;
      if (i < n4) {
        const uint32_t w = pack4_i8(quant_one(v[r][j].x, s), quant_one(v[r][j].y, s),
                                    quant_one(v[r][j].z, s), quant_one(v[r][j].w, s));
        *reinterpret_cast<uint32_t *>(xq + (size_t)m * stride + 4 * i) = w;
        if (write_out) st_global<uint32_t>(p.xq_out + (size_t)m * p.K + 4 * i, w);
      }
    }
  }
  __syncthreads();
}

// RPW > 0: rows held by whole waves (lm_load_wave_rows / lm_quant_wave_rows);
// else NQ > 0: the rows as one flat run of NQ quads per thread
// (lm_load_rows / lm_quant_resident); NQ = 0: two batched passes over them.
template <int D, int NQ, int RPW>
__global__ void __launch_bounds__(kThreads) lm_head_kernel(LmParams p) {
  __shared__ LmShared sh;
  extern __shared__ __attribute__((aligned(16))) int8_t lds[];
  const int lane = threadIdx.x & 63;
  // The wave index is uniform: said so, the run's bounds and the ring's item
  // count live in scalar registers and the load addressing stays branch-free.
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
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

  const uint32_t q_bytes = (uint32_t)((size_t)p.nblk * cpb * kTileBytes);
  const __amdgpu_buffer_rsrc_t q_rsrc = make_rsrc(p.q, q_bytes);
  // Next item to fetch: the wave's run is items [blk0 * cpb, (blk0 + nb) * cpb)
  // of the table, one 4 KB tile each.
  int fetched = 0;
  const uint32_t run0 = (uint32_t)blk0 * cpb * kTileBytes + 16u * lane;
  auto load_item = [&](v4i (&w)[4]) {
    const bool live = fetched < items;
    const uint32_t base = run0 + (uint32_t)fetched * kTileBytes;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t off = live ? base + 1024u * j : q_bytes;
      w[j] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(q_rsrc, off, 0,
                                                                            kTableAux));
    }
    ++fetched;
  };
  f32x4 xv[NQ > 0 ? NQ : 1];
  f32x4 xw[RPW > 0 ? RPW : 1][kRowQuads];
  if constexpr (RPW > 0) {
    lm_load_wave_rows<RPW>(p, wave, xw);
  } else if constexpr (NQ > 0) {
    if (threadIdx.x < p.M) sh.amax[threadIdx.x] = 0u;
    lm_load_rows<NQ>(p, xv);
  }
  __builtin_amdgcn_sched_barrier(0);
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

  if constexpr (RPW > 0) {
    lm_quant_wave_rows<RPW>(p, sh, xq_lds, p.xq_out != nullptr && blockIdx.x == 0, wave, xw);
  } else if constexpr (NQ > 0) {
    __syncthreads();   // sh.amax cleared
    lm_quant_resident<NQ>(p, sh, xq_lds, p.xq_out != nullptr && blockIdx.x == 0, xv);
  } else {
    lm_quant_rows(p, sh, xq_lds, p.xq_out != nullptr && blockIdx.x == 0);
  }
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

// Byte of code (v, k) in the table's storage order; cpb = 256-input chunks
// per row group.
__device__ __forceinline__ uint32_t table_off(int v, int k, int cpb) {
  return (uint32_t)(((v >> 4) * cpb + (k >> 8)) * kTileBytes) + ((k & 255) >> 6) * 1024u +
         ((k & 63) >> 4) * 256u + (v & 15) * 16u + (k & 15);
}

// Per-row quantization, one wave per row.  TILED: write the table's storage
// order over the padded Vp x Kp table (padding rows and inputs get zero codes);
// otherwise plain row-major [N][K].
template <bool TILED>
__global__ void __launch_bounds__(kThreads) rowq_quant_kernel(const float *W, int N, int K,
                                                              int rows, int8_t *q,
                                                              float *w_scale) {
  const int lane = threadIdx.x & 63;
  const int n = blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (n >= rows) return;
  const int n4 = K >> 2;
  const int cpb = (K + kItemK - 1) / kItemK;
  const bool live = n < N;
  const f32x4 *w4 = reinterpret_cast<const f32x4 *>(W + (size_t)(live ? n : 0) * K);
  float a = 0.0f;
  if (live)
    for (int i = lane; i < n4; i += 64) {
      const f32x4 v = ld_global<f32x4>(w4 + i);
      a = fmaxf(a, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
    }
  a = wave_max(a);
  const float s = a / 127.0f;
  if (live && lane == 0) st_global<float>(w_scale + n, a == 0.0f ? 0.0f : s);
  const int nout4 = TILED ? cpb * (kItemK / 4) : n4;
  for (int i = lane; i < nout4; i += 64) {
    uint32_t packed = 0;
    if (live && a != 0.0f && i < n4) {
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
    if (TILED)
      st_global<uint32_t>(q + table_off(n, 4 * i, cpb), packed);
    else
      st_global<uint32_t>(q + (size_t)n * K + 4 * i, packed);
  }
}

// Embedding rows from the table, one wave per token; lane g takes inputs
// [16g, 16g + 16) (one 16-byte group of the storage order).
__global__ void __launch_bounds__(kThreads) embed_kernel(const int32_t *ids, int T,
                                                         const int8_t *q, const float *w_scale,
                                                         int N, int K, float *out) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (t >= T) return;
  const int id = ld_global<int>(ids + t);
  const bool live = id >= 0 && id < N;
  const float s = live ? ld_global<float>(w_scale + id) : 0.0f;
  const int cpb = (K + kItemK - 1) / kItemK;
  for (int g = lane; g < (K >> 4); g += 64) {
    v4i d = v4i{0, 0, 0, 0};
    if (live) d = ld_global<v4i>(q + table_off(id, 16 * g, cpb));
    float *o = out + (size_t)t * K + 16 * g;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t b = (uint32_t)d[w];
      f32x4 v;
      v.x = (float)(int8_t)(b & 0xff) * s;
      v.y = (float)(int8_t)((b >> 8) & 0xff) * s;
      v.z = (float)(int8_t)((b >> 16) & 0xff) * s;
      v.w = (float)(int8_t)(b >> 24) * s;
      st_global<f32x4>(o + 4 * w, v);
    }
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

size_t table_bytes(int64_t V, int64_t K) {
  return (size_t)((V + 15) / 16 * 16) * (size_t)((K + kItemK - 1) / kItemK * kItemK);
}

hipError_t launch_rowq_quant(const float *W, int64_t N, int64_t K, int8_t *q, float *w_scale,
                             bool tiled, hipStream_t stream) {
  const int64_t rows = tiled ? (N + 15) / 16 * 16 : N;
  const int64_t blocks = (rows + kWaves - 1) / kWaves;
  if (tiled)
    rowq_quant_kernel<true><<<(unsigned)blocks, kThreads, 0, stream>>>(W, (int)N, (int)K,
                                                                       (int)rows, q, w_scale);
  else
    rowq_quant_kernel<false><<<(unsigned)blocks, kThreads, 0, stream>>>(W, (int)N, (int)K,
                                                                        (int)rows, q, w_scale);
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
  // Rows of up to kRowQuads * 256 inputs are held by whole waves (M <= 16,
  // so at most 4 rows per wave); longer rows as quads of one flat run per
  // thread when they fit, else two batched passes.
  const int64_t nq = ((int64_t)M * (K >> 2) + kThreads - 1) / kThreads;
  const size_t lds = lm_head_lds_bytes(M, V, K);
  if (K <= 256 * kRowQuads && M <= 4)
    lm_head_kernel<kDepth, 0, 1><<<blocks, kThreads, lds, stream>>>(p);
  else if (K <= 256 * kRowQuads && M <= 8)
    lm_head_kernel<kDepth, 0, 2><<<blocks, kThreads, lds, stream>>>(p);
  else if (K <= 256 * kRowQuads)
    lm_head_kernel<kDepth, 0, 4><<<blocks, kThreads, lds, stream>>>(p);
  else if (nq <= 2)
    lm_head_kernel<kDepth, 2, 0><<<blocks, kThreads, lds, stream>>>(p);
  else if (nq <= 6)
    lm_head_kernel<kDepth, 6, 0><<<blocks, kThreads, lds, stream>>>(p);
  else if (nq <= 12)
    lm_head_kernel<kDepth, 12, 0><<<blocks, kThreads, lds, stream>>>(p);
  else if (nq <= 24)
    lm_head_kernel<kDepth, 24, 0><<<blocks, kThreads, lds, stream>>>(p);
  else
    lm_head_kernel<kDepth, 0, 0><<<blocks, kThreads, lds, stream>>>(p);
  return hipGetLastError();
}

}  // namespace bitnet
