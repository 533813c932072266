// I8_S: int8 weights x int8 activations, the audio encoders' linear layers.
//
// The audio tokenizer's encoders run with int8 weights and int8 activations
// and ReLU in place of GELU (ONNX model card "multimodalart/VibeVoice-ASR-
// BitNet-ONNX", Quantization table, row "VAE encoders"), in fused routines
// that combine the matmul with its bias and ReLU (aitrends.kr summary,
// technical-features section).  Here that is one library call:
//   - the activation rows are quantized (per-row absmax int8, the same
//     quantization kernel as the ternary path) into the workspace;
//   - one GEMM launch contracts them with the int8 weights on
//     v_mfma_i32_32x32x32_i8 and applies the per-row dequantization factor,
//     the bias and the ReLU in its epilogue.
// Weights are quantized once, offline, with one absmax scale per tensor.
//
// GEMM.  Workgroup tile 64 (or 128) x 128, 4 waves in a 2 x 2 arrangement,
// each wave 32 (64) x 64 as blocks of 32 x 32.  K advances KB = 128 inputs per
// step on long rows (K >= 1024, K % 128 == 0), else 64: the activation tile (BM rows x KB int8) and
// the weight tile (128 rows x KB int8) go straight from memory into LDS
// (buffer_load ... lds), into a ring of two stages issued one step ahead (KB =
// 128) or three stages issued two steps ahead (KB = 64), so 128 inputs are in
// flight either way; rows past M or N load as zeros.  With 128-input steps
// every row of a tile takes whole 128-byte lines.  Inside a stage, 16-byte chunk c of tile row r
// sits at position c ^ swz(r), so the operand reads of 16 consecutive rows hit
// 16 different bank groups.  Lane (i = lane % 32, h = lane / 32) feeds k-step s
// of a stage with chunk 2s + h of its A row and of its B row, so the k
// positions of both operands agree.
// Tiles are dealt to the eight XCDs by row block (block b runs on XCD b % 8),
// so the workgroups that read one block of activation rows share one L2.
#include <algorithm>

#include "bitnet_device.hpp"
#include "bitnet_internal.hpp"
#include "bitnet_variants.hpp"

namespace bitnet {
namespace {

// LDS stages: 0 picks 2 for 128-input steps and 3 for 64-input steps.
#ifndef BITNET_I8_RING
#define BITNET_I8_RING 0
#endif
// Steps of 128 inputs for K % 128 == 0 and K >= BITNET_I8_WIDE_MINK (else 64).
// Measured on the 8192-frame encoder layers: K = 2048 32.1 -> 30.3 us per
// call with 128-input steps, K = 512 27.9 -> 28.3 us (kept at 64).
#ifndef BITNET_I8_WIDE
#define BITNET_I8_WIDE 1
#endif
#ifndef BITNET_I8_WIDE_MINK
#define BITNET_I8_WIDE_MINK 1024
#endif
constexpr int kThreads = 256;
constexpr int kBN = 128;
template <int KB>
constexpr int ring_stages() {
  return BITNET_I8_RING > 0 ? BITNET_I8_RING : (KB == 128 ? 2 : 3);
}
constexpr int kStoreAux = 2;            // outputs are not read again here: non-temporal
typedef __attribute__((address_space(3))) void *lds_ptr_t;

// Tile height BM = 128 or 64: the 4 waves sit 2 x 2, each owning BM/2 rows
// (BM/64 blocks of 32) and 64 columns (2 blocks of 32).  KB inputs per step.
template <int BM, int KB, int kRing = ring_stages<KB>()>
struct I8Shared {
  __attribute__((aligned(16))) int8_t a[kRing][BM * KB];
  __attribute__((aligned(16))) int8_t b[kRing][kBN * KB];
  __attribute__((aligned(16))) float factor[BM];
};

// Chunk position of tile row r.  A ds_read_b128 serves 16 lanes (16
// consecutive rows, one chunk column) per cycle, and a 256-byte bank line holds
// 256 / KB rows, so the rows that share a bank line, and the line groups,
// need KB / 16 different positions.
template <int KB>
__device__ __forceinline__ int swz(int r) {
  return (r / (256 / KB)) % (KB / 16);
}

// s_waitcnt immediate: at most n vector-memory operations outstanding and no
// LDS operation (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4,
// lgkmcnt 11:8).
constexpr int vmcnt_lgkm0_wait(int n) { return (n & 0xf) | ((n >> 4) << 14) | (0x7 << 4); }

struct I8Params {
  const int8_t *xq;        // [M][K] natural order
  const float *x_scale;    // [M]
  const int8_t *q;         // [N][K]
  const float *w_scale;    // device scalar, or [N] with one scale per output channel
  const float *bias;       // [N] or null
  float *y;                // [M][N]
  int32_t *acc_out;        // [M][N] or null
  int M, N, K, relu, MB, NB;
};

// s_waitcnt for step u of the K loop: the loads of the `later` steps issued
// after it (at most kRing - 2) may stay in flight, no LDS operation may.
template <int kRing, int kDmaPerWave>
__device__ __forceinline__ void wait_for_step(int later) {
  if (kRing >= 4 && later >= 2)
    __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0_wait(2 * kDmaPerWave));
  else if (kRing >= 3 && later >= 1)
    __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0_wait(kDmaPerWave));
  else
    __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0_wait(0));
}

// Output value: relu?(fl32(fl32(acc * c) * factor) + bias), where with one
// scale per tensor c = 1 and factor = fl32(w_scale / x_scale[m]), and with one
// scale per output channel c = w_scale[n] and factor = fl32(1 / x_scale[m]).
template <bool RELU>
__device__ __forceinline__ float i8_out(float a, float c, float f, float b) {
  float v = (a * c) * f + b;
  if (RELU) v = v > 0.0f ? v : 0.0f;
  return v;
}

template <int BM, int KB, bool RELU, bool PERCOL>
__global__ void __launch_bounds__(kThreads) i8_gemm_kernel(I8Params p) {
  constexpr int RB = BM / 64;            // 32-row blocks per wave
  constexpr int kCh = KB / 16;           // 16-byte chunks per tile row
  constexpr int kRowsPerDma = 64 / kCh;  // tile rows per 1 KB load
  constexpr int kDmaA = BM / 4 / kRowsPerDma;   // activation loads per wave and step
  constexpr int kDmaB = 32 / kRowsPerDma;       // weight loads per wave and step
  constexpr int kDmaPerWave = kDmaA + kDmaB;
  constexpr int kRing = ring_stages<KB>();
  __shared__ I8Shared<BM, KB> sh;
  // Block b runs on XCD b % 8: XCD x takes row blocks x, x + 8, ... and every
  // column block of each.
  const int b = blockIdx.x, xcd = b & 7, j = b >> 3;
  const int mb = (j / p.NB) * 8 + xcd, nb = j % p.NB;
  if (mb >= p.MB) return;
  const int m0 = mb * BM, n0 = nb * kBN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 31, lh = lane >> 5;
  const int wm = wave & 1, wn = wave >> 1;
  const int steps = p.K / KB;

  // DMA: wave w fills activation rows [BM/4 w, BM/4 (w + 1)) and weight rows
  // [32w, 32w + 32) with 1 KB loads; lane L of a load lands at position
  // L % kCh of tile row r = (first row of the load) + L / kCh and so fetches
  // chunk (L % kCh) ^ swz(r).
  const uint32_t a_bytes = (uint32_t)((size_t)p.M * p.K);
  const uint32_t b_bytes = (uint32_t)((size_t)p.N * p.K);
  const __amdgpu_buffer_rsrc_t a_rsrc = make_rsrc(p.xq, a_bytes);
  const __amdgpu_buffer_rsrc_t b_rsrc = make_rsrc(p.q, b_bytes);
  uint32_t a_off[kDmaA], b_off[kDmaB];
#pragma unroll
  for (int q = 0; q < kDmaA; ++q) {
    const int r = (BM / 4) * wave + kRowsPerDma * q + lane / kCh;
    const int chunk = (lane % kCh) ^ swz<KB>(r);
    a_off[q] = m0 + r < p.M ? (uint32_t)(m0 + r) * p.K + 16 * chunk : a_bytes;
  }
#pragma unroll
  for (int q = 0; q < kDmaB; ++q) {
    const int r = 32 * wave + kRowsPerDma * q + lane / kCh;
    const int chunk = (lane % kCh) ^ swz<KB>(r);
    b_off[q] = n0 + r < p.N ? (uint32_t)(n0 + r) * p.K + 16 * chunk : b_bytes;
  }
  // The step's K offset goes in the scalar offset; rows past M or N carry a
  // vector offset at the buffer's end, so they load zeros without a memory
  // access whatever the step.  Steps past K are never issued.
  auto issue = [&](int u, int slot) {
    const uint32_t soff = (uint32_t)u * KB;
#pragma unroll
    for (int q = 0; q < kDmaA; ++q) {
      // (Through a local: a captured array element passed straight to the
      // builtin keeps this compiler's host pass from emitting the launch stub.)
      const uint32_t ao = a_off[q];
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          a_rsrc, (lds_ptr_t)(&sh.a[slot][((BM / 4) * wave + kRowsPerDma * q) * KB]), 16, ao, soff,
          0, 0);
    }
#pragma unroll
    for (int q = 0; q < kDmaB; ++q) {
      const uint32_t bo = b_off[q];
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          b_rsrc, (lds_ptr_t)(&sh.b[slot][(32 * wave + kRowsPerDma * q) * KB]), 16, bo, soff, 0, 0);
    }
  };

  // Operand reads: row (32 rb + li) of the wave's half, chunk 2s + lh.
  uint32_t rd[KB / 32];
#pragma unroll
  for (int s = 0; s < KB / 32; ++s) rd[s] = li * KB + (((2 * s + lh) ^ swz<KB>(li)) * 16);

  // Per-row dequantization factors of the tile (rows past M: any finite value).
  if (tid < BM) {
    const int row = min(m0 + tid, p.M - 1);
    const float xs = ld_global<float>(p.x_scale + row);
    sh.factor[tid] = PERCOL ? 1.0f / xs : ld_global<float>(p.w_scale) / xs;
  }

  // The bias (and channel scale) of the lane's columns, fetched now so that
  // their latency hides behind the K loop.
  float bias[2], cscale[2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int n = n0 + wn * 64 + cb * 32 + li;
    bias[cb] = (p.bias && n < p.N) ? ld_global<float>(p.bias + n) : 0.0f;
    cscale[cb] = (PERCOL && n < p.N) ? ld_global<float>(p.w_scale + n) : 1.0f;
  }

#pragma unroll
  for (int u = 0; u < kRing - 1; ++u)
    if (u < steps) issue(u, u);

  v16i acc[RB][2];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[rb][cb][e] = 0;

  for (int u = 0; u < steps; ++u) {
    const int s = u % kRing;
    // Step u's loads are this wave's oldest outstanding ones; after the
    // barrier every wave's part of stage s is in LDS and every wave is done
    // reading the stage that the next loads overwrite.  The wait also drains
    // this wave's LDS reads: the loads issued after the barrier overwrite the
    // stage read one step earlier, and a read still queued behind the barrier
    // would see the new data.  Nothing is scheduled across this point, so
    // those reads and the MFMAs that use them stay on this side.
    __builtin_amdgcn_sched_barrier(0);
    wait_for_step<kRing, kDmaPerWave>(min(kRing - 2, steps - 1 - u));
    __builtin_amdgcn_s_barrier();
    if (u + kRing - 1 < steps) issue(u + kRing - 1, (u + kRing - 1) % kRing);
    __builtin_amdgcn_sched_barrier(0);
    const int8_t *as = sh.a[s] + (wm * (BM / 2)) * KB;
    const int8_t *bs = sh.b[s] + (wn * 64) * KB;
#pragma unroll
    for (int ks = 0; ks < KB / 32; ++ks) {
      v4i av[RB], bv[2];
#pragma unroll
      for (int r = 0; r < RB; ++r) av[r] = *reinterpret_cast<const v4i *>(as + r * 32 * KB + rd[ks]);
#pragma unroll
      for (int r = 0; r < 2; ++r) bv[r] = *reinterpret_cast<const v4i *>(bs + r * 32 * KB + rd[ks]);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
          acc[rb][cb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(av[rb], bv[cb], acc[rb][cb], 0, 0, 0);
    }
  }

  // Epilogue: element e of a 32x32 block sits at row 8(e/4) + 4lh + e%4,
  // column li.  y = relu?(fl32(fl32(acc) * factor) + bias).
  const uint32_t y_bytes = (uint32_t)((size_t)p.M * p.N * 4);
  const __amdgpu_buffer_rsrc_t y_rsrc = make_rsrc(p.y, y_bytes);
  const __amdgpu_buffer_rsrc_t c_rsrc = make_rsrc(p.acc_out, p.acc_out ? y_bytes : 0);
  if (m0 + BM <= p.M && n0 + kBN <= p.N) {
    // Whole tile inside: one vector offset per column block, the row step in
    // the scalar offset.
    const uint32_t rstride = (uint32_t)p.N * 4u;
    uint32_t vo[2];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
      vo[cb] = (uint32_t)(m0 + wm * (BM / 2) + 4 * lh) * rstride +
               (uint32_t)(n0 + wn * 64 + cb * 32 + li) * 4u;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 f4 =
            *reinterpret_cast<const f32x4 *>(&sh.factor[wm * (BM / 2) + rb * 32 + 8 * g + 4 * lh]);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t so = (uint32_t)(rb * 32 + 8 * g + k) * rstride;
#pragma unroll
          for (int cb = 0; cb < 2; ++cb) {
            const int a = acc[rb][cb][4 * g + k];
            __builtin_amdgcn_raw_buffer_store_b32(
                __builtin_bit_cast(int, i8_out<RELU>((float)a, cscale[cb], f4[k], bias[cb])), y_rsrc,
                vo[cb], so, kStoreAux);
            if (p.acc_out) __builtin_amdgcn_raw_buffer_store_b32(a, c_rsrc, vo[cb], so, 0);
          }
        }
      }
    return;
  }
  // Edge tile: rows past M and columns past N are aimed beyond the buffers
  // and dropped.
  uint32_t col_off[2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int n = n0 + wn * 64 + cb * 32 + li;
    col_off[cb] = n < p.N ? (uint32_t)n * 4u : 0x80000000u;
  }
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int lrow = wm * (BM / 2) + rb * 32 + 8 * g + 4 * lh + k;
        const int row = m0 + lrow;
        const uint32_t row_off = row < p.M ? (uint32_t)row * (uint32_t)p.N * 4u : 0x80000000u;
        const float f = sh.factor[lrow];
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
          const int a = acc[rb][cb][4 * g + k];
          const uint32_t off = (row_off | col_off[cb]) >= 0x80000000u ? y_bytes
                                                                      : row_off + col_off[cb];
          __builtin_amdgcn_raw_buffer_store_b32(
              __builtin_bit_cast(int, i8_out<RELU>((float)a, cscale[cb], f, bias[cb])), y_rsrc, off,
              0, kStoreAux);
          if (p.acc_out) __builtin_amdgcn_raw_buffer_store_b32(a, c_rsrc, off, 0, 0);
        }
      }
}

// Weight quantization, one scale per tensor.  Pass 1: max |W| (non-negative
// floats order like their bit patterns, so an integer atomic max is exact and
// order-independent).  Pass 2: s = fl32(max / 127), q = clamp(rint(W / s)).
__global__ void i8_zero_kernel(uint32_t *w) {
  if (threadIdx.x == 0) w[0] = 0u;
}

__global__ void __launch_bounds__(kThreads) i8_absmax_kernel(const float *W, int64_t n4,
                                                             uint32_t *amax) {
  __shared__ float red[kThreads / 64];
  const f32x4 *w4 = reinterpret_cast<const f32x4 *>(W);
  float a = 0.0f;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n4;
       i += (int64_t)gridDim.x * kThreads) {
    const f32x4 v = ld_global<f32x4>(w4 + i);
    a = fmaxf(a, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
  }
  a = wave_max(a);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = a;
  __syncthreads();
  if (threadIdx.x == 0) {
    const float m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    atomicMax(amax, __builtin_bit_cast(uint32_t, m));
  }
}

__device__ __forceinline__ int quant_w(float w, float s) {
  float t = __builtin_rintf(w / s);
  t = fminf(fmaxf(t, -127.0f), 127.0f);
  return (int)t;
}

__global__ void __launch_bounds__(kThreads) i8_quant_weights_kernel(const float *W, int64_t n4,
                                                                    const uint32_t *amax,
                                                                    int8_t *q, float *w_scale) {
  const float a = __builtin_bit_cast(float, ld_global<uint32_t>(amax));
  const float s = a / 127.0f;
  if (blockIdx.x == 0 && threadIdx.x == 0) st_global<float>(w_scale, a == 0.0f ? 0.0f : s);
  const f32x4 *w4 = reinterpret_cast<const f32x4 *>(W);
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n4;
       i += (int64_t)gridDim.x * kThreads) {
    uint32_t packed = 0;
    if (a != 0.0f) {
      const f32x4 v = ld_global<f32x4>(w4 + i);
      packed = pack4_i8(quant_w(v.x, s), quant_w(v.y, s), quant_w(v.z, s), quant_w(v.w, s));
    }
    st_global<uint32_t>(q + 4 * i, packed);
  }
}

// 64-row tiles unless 128-row tiles are plentiful: on the encoder layers
// (1024 and 256 tiles of 128 rows) the shorter tiles, with twice the
// workgroups and four resident per compute unit, measured faster.
#ifndef BITNET_I8_TALL_MIN_TILES
#define BITNET_I8_TALL_MIN_TILES 4096
#endif
bool i8_tall_tiles(int M, int N) {
  const int64_t tiles = (int64_t)((M + 127) / 128) * ((N + kBN - 1) / kBN);
  return tiles >= BITNET_I8_TALL_MIN_TILES;
}

}  // namespace

hipError_t launch_i8_quant_weights(const float *W, int64_t N, int64_t K, int8_t *q,
                                   float *w_scale, uint32_t *amax, hipStream_t stream) {
  const int64_t n4 = N * K / 4;
  const int blocks = (int)std::min<int64_t>((n4 + kThreads - 1) / kThreads, 4096);
  i8_zero_kernel<<<1, 64, 0, stream>>>(amax);
  i8_absmax_kernel<<<blocks, kThreads, 0, stream>>>(W, n4, amax);
  i8_quant_weights_kernel<<<blocks, kThreads, 0, stream>>>(W, n4, amax, q, w_scale);
  return hipGetLastError();
}

template <int KB, bool PERCOL>
static void launch_i8_gemm_kb(const I8Params &p, bool tall, bool relu, unsigned grid,
                              hipStream_t stream) {
  if (tall && relu)
    i8_gemm_kernel<128, KB, true, PERCOL><<<grid, kThreads, 0, stream>>>(p);
  else if (tall)
    i8_gemm_kernel<128, KB, false, PERCOL><<<grid, kThreads, 0, stream>>>(p);
  else if (relu)
    i8_gemm_kernel<64, KB, true, PERCOL><<<grid, kThreads, 0, stream>>>(p);
  else
    i8_gemm_kernel<64, KB, false, PERCOL><<<grid, kThreads, 0, stream>>>(p);
}

template <bool PERCOL>
static hipError_t launch_i8_gemm_t(const I8Params &p, bool tall, bool relu, unsigned grid,
                                   hipStream_t stream) {
  if (BITNET_I8_WIDE && p.K % 128 == 0 && p.K >= BITNET_I8_WIDE_MINK)
    launch_i8_gemm_kb<128, PERCOL>(p, tall, relu, grid, stream);
  else
    launch_i8_gemm_kb<64, PERCOL>(p, tall, relu, grid, stream);
  return hipGetLastError();
}

hipError_t launch_i8_gemm(int M, int N, int K, const int8_t *xq, const float *x_scale,
                          const int8_t *q, const float *w_scale, bool per_channel,
                          const float *bias, int relu, float *y, int32_t *acc_out,
                          hipStream_t stream) {
  I8Params p{xq, x_scale, q, w_scale, bias, y, acc_out, M, N, K, relu ? 1 : 0, 0, 0};
  p.NB = (N + kBN - 1) / kBN;
  const bool tall = i8_tall_tiles(M, N);
  p.MB = (M + (tall ? 127 : 63)) / (tall ? 128 : 64);
  const int64_t grid = (int64_t)8 * ((p.MB + 7) / 8) * p.NB;
  if (grid >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  return per_channel ? launch_i8_gemm_t<true>(p, tall, relu != 0, (unsigned)grid, stream)
                     : launch_i8_gemm_t<false>(p, tall, relu != 0, (unsigned)grid, stream);
}

}  // namespace bitnet
