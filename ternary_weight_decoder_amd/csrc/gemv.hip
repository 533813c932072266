// Decode projection, M <= 16 rows: an HBM-bound stream of 2-bit packed codes.
//
// The decoder reads all of its ternary weights for every token (blog "The Paper
// Says ARM Support...", section "What the model is trying to do"), so this path
// is bound by weight bandwidth.  The contraction itself (adds and subtracts of
// activations, xujun.org article, heterogeneous-quantization section) runs on
// the int8 matrix cores: v_mfma_i32_16x16x64_i8 with the M rows padded to 16.
// That keeps the VALU work at the 2-bit unpack alone (7 ops per 16 codes per
// lane), independent of M, where a dot4 formulation would add 4*M more.
//
// Work split: each wave owns one tile of 64 columns and walks its full K, so no
// cross-wave reduction is needed; the 4 waves of a workgroup take adjacent
// tiles, which keeps their reads of one unit adjacent in memory.  In launches
// too small to fill the chip, the waves of a single-row workgroup instead share
// one tile and split its K units (S = 2 or 4 ways); their int32 partial sums
// are added through LDS.  Lane (col = lane%16, h = lane/16) loads 8 bytes =
// packed dwords 2h, 2h+1 of unit u for column col: a wave reads 512 contiguous
// bytes per unit and 16-column block.  Field values u = code+1 enter the MFMA;
// the epilogue subtracts the activation row sum.
//
// Weights are read with buffer loads kept D units ahead in a register ring.
// Loads for columns past N or units past the wave's range are aimed past the
// buffer's end: the hardware returns zeros without touching memory, so every
// ring slot issues the same instructions and the wait counts stay static.
//
// Grouped launches: the host deals whole projections to the eight XCDs (block
// b runs on XCD b % 8, and XCD x runs its own range of the table), so each
// projection's activation row, or staged int8 rows, is fetched into one L2.
//
// Activation quantization is fused when the M x K int8 rows fit in LDS: every
// workgroup quantizes the rows itself (absmax, scale, round, row sum) into LDS
// in the permuted order, so one launch does the whole projection.  Otherwise a
// separate quantization kernel writes the rows to the workspace first, and the
// workgroup streams them into LDS in chunks of kChunkUnits units (buffer_load
// ... lds, double-buffered, one barrier per chunk), so its four waves share
// one copy instead of each reading every row from L2.
#include "bitnet_device.hpp"
#include "bitnet_internal.hpp"

namespace bitnet {
namespace {

#ifndef BITNET_GEMV_C
#define BITNET_GEMV_C 4
#endif
#ifndef BITNET_GEMV_DEPTH
#define BITNET_GEMV_DEPTH 3
#endif
// Weights are read once per call: non-temporal loads keep them from evicting
// the activations and small tables that every workgroup reuses.
#ifndef BITNET_GEMV_AUX
#define BITNET_GEMV_AUX 2
#endif
constexpr int kGemvC = BITNET_GEMV_C;           // 16-column blocks per wave tile
// With the rows staged from the workspace (M > 1), a ring of 2 units and
// chunks of 4 units measured faster than 3 and 8 (M = 4: 66.9 -> 65.9 us per
// 196-projection sweep, M = 16: 85.7 -> 83.5 us); a ring of 1 unit, chunks of
// 16 units, 4-unit rings and 32-column wave tiles were slower.
#ifndef BITNET_GEMV_DEPTH_STAGED
#define BITNET_GEMV_DEPTH_STAGED 2
#endif
constexpr int kGemvDepth = BITNET_GEMV_DEPTH;   // items in flight per wave
constexpr int kGemvDepthStaged = BITNET_GEMV_DEPTH_STAGED;   // the same, rows staged
constexpr int kWeightAux = BITNET_GEMV_AUX;     // cache-policy bits of weight loads
constexpr int kWaveCols = 16 * kGemvC;          // columns of one wave tile
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
#ifndef BITNET_GEMV_CHUNK
#define BITNET_GEMV_CHUNK 4
#endif
constexpr int kChunkUnits = BITNET_GEMV_CHUNK;   // units per staged activation chunk
constexpr int kChunkBytes = kChunkUnits * kGemvMaxM * kUnit;   // 16 rows per unit
static_assert(kChunkUnits % 4 == 0, "each of the four waves stages whole units");
typedef __attribute__((address_space(3))) void *lds_ptr_t;

// 16-byte chunk position of chunk c in staged row r: pairs of rows share a
// 256-byte bank line, so the eight pairs use eight different positions and a
// 16-lane operand read (rows 0..15, one chunk) is conflict-free.
__device__ __forceinline__ int stage_pos(int c, int r) { return c ^ ((r >> 1) & 7); }

struct GemvProblem {
  const uint8_t *packed;
  const float *x;         // fused: fp32 activations [M][K]
  const int8_t *xqp;      // unfused: permuted int8 activations [M][K]
  const float *x_scale;   // unfused: [M]
  const int32_t *rowsum;  // unfused: [M]
  const float *w_scale;
  float *y;               // [M][N]
  int32_t *acc_out;       // optional [M][N]
  int8_t *xq_out;         // optional natural-order int8 rows (fused path, block 0)
  float *x_scale_out;     // optional scales (fused path, block 0)
  int N, K, M;
};

struct GemvShared {
  float red[kGemvMaxM][kWaves];
  int ired[kGemvMaxM][kWaves];
  float scale[kGemvMaxM];
  int rowsum[kGemvMaxM];
};

// Quantize the M rows of x into LDS (permuted order) with the scales and row sums,
// one grid-stride loop per pass (the form for launches that fill the chip).
__device__ __forceinline__ void quant_rows_serial(const GemvProblem &p, GemvShared &sh,
                                                  int8_t *xq_lds, bool write_out) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n4 = p.K >> 2;
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
    int8_t *dst = xq_lds + (size_t)m * p.K;
    int sum = 0;
    for (int i = tid; i < n4; i += kThreads) {
      const f32x4 v = ld_global<f32x4>(x4 + i);
      const int q0 = quant_one(v.x, s), q1 = quant_one(v.y, s);
      const int q2 = quant_one(v.z, s), q3 = quant_one(v.w, s);
      sum += q0 + q1 + q2 + q3;
      const uint32_t w = pack4_i8(q0, q1, q2, q3);
      *reinterpret_cast<uint32_t *>(dst + perm_offset(4 * i)) = w;
      if (write_out) st_global<uint32_t>(p.xq_out + (size_t)m * p.K + 4 * i, w);
    }
    sum = wave_sum(sum);
    if (lane == 0) sh.ired[m][wave] = sum;
    if (tid == 0) {
      sh.scale[m] = s;
      if (write_out) st_global<float>(p.x_scale_out + m, s);
    }
  }
  __syncthreads();
  if (tid < p.M)
    sh.rowsum[tid] = sh.ired[tid][0] + sh.ired[tid][1] + sh.ired[tid][2] + sh.ired[tid][3];
  __syncthreads();
}

// The same for small launches (K-split).  // A pass over a row issues all of a thread's loads at once (up to kQuantBatch
// 16-byte buffer loads; positions past the row are aimed beyond it and return
// zeros without a memory access), so a row costs one memory round trip per
// pass instead of one per loop iteration: on a long row (K = 8960) that is the
// difference between 2 and 18 round trips, which a small launch cannot hide
// behind other workgroups.  A single row that fits one batch stays in
// registers from the absmax pass to the quantizing pass.
constexpr int kQuantBatch = 9;   // 9 x 256 threads x 4 = 9216 inputs per batch

__device__ __forceinline__ void load_row_batch(__amdgpu_buffer_rsrc_t rsrc, int n4, int base,
                                               f32x4 (&v)[kQuantBatch]) {
#pragma unroll
  for (int j = 0; j < kQuantBatch; ++j) {
    const int i = base + j * kThreads + (int)threadIdx.x;
    const uint32_t off = (uint32_t)(i < n4 ? i : n4) * 16u;
    v[j] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, off, 0, 0));
  }
}

__device__ __forceinline__ void quant_rows_batched(const GemvProblem &p, GemvShared &sh,
                                                  int8_t *xq_lds, bool write_out) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n4 = p.K >> 2;
  constexpr int kBatch4 = kQuantBatch * kThreads;   // f32x4 elements per batch
  const bool resident = p.M == 1 && n4 <= kBatch4;
  f32x4 v[kQuantBatch];
  for (int m = 0; m < p.M; ++m) {
    const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(p.x + (size_t)m * p.K, (uint32_t)p.K * 4u);
    float a = 0.0f;
    for (int base = 0; base < n4; base += kBatch4) {
      load_row_batch(rsrc, n4, base, v);
#pragma unroll
      for (int j = 0; j < kQuantBatch; ++j)
        a = fmaxf(a, fmaxf(fmaxf(fabsf(v[j].x), fabsf(v[j].y)), fmaxf(fabsf(v[j].z), fabsf(v[j].w))));
    }
    a = wave_max(a);
    if (lane == 0) sh.red[m][wave] = a;
  }
  __syncthreads();
  for (int m = 0; m < p.M; ++m) {
    const float a = fmaxf(fmaxf(sh.red[m][0], sh.red[m][1]), fmaxf(sh.red[m][2], sh.red[m][3]));
    const float s = (a == 0.0f) ? 1.0f : 127.0f / a;
    const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(p.x + (size_t)m * p.K, (uint32_t)p.K * 4u);
    int8_t *dst = xq_lds + (size_t)m * p.K;
    int sum = 0;
    for (int base = 0; base < n4; base += kBatch4) {
      if (!resident) load_row_batch(rsrc, n4, base, v);
#pragma unroll
      for (int j = 0; j < kQuantBatch; ++j) {
        const int i = base + j * kThreads + tid;
        if (i < n4) {
          const int q0 = quant_one(v[j].x, s), q1 = quant_one(v[j].y, s);
          const int q2 = quant_one(v[j].z, s), q3 = quant_one(v[j].w, s);
          sum += q0 + q1 + q2 + q3;
          const uint32_t w = pack4_i8(q0, q1, q2, q3);
          *reinterpret_cast<uint32_t *>(dst + perm_offset(4 * i)) = w;
          if (write_out) st_global<uint32_t>(p.xq_out + (size_t)m * p.K + 4 * i, w);
        }
      }
    }
    sum = wave_sum(sum);
    if (lane == 0) sh.ired[m][wave] = sum;
    if (tid == 0) {
      sh.scale[m] = s;
      if (write_out) st_global<float>(p.x_scale_out + m, s);
    }
  }
  __syncthreads();
  if (tid < p.M)
    sh.rowsum[tid] = sh.ired[tid][0] + sh.ired[tid][1] + sh.ired[tid][2] + sh.ired[tid][3];
  __syncthreads();
}

// A single row already held in registers (loaded by load_row_batch before the
// workgroup's first weight loads): one absmax reduction, then the quantized
// row, its scale and its row sum go to LDS.  Positions past the row hold zeros.
__device__ __forceinline__ void quant_row_resident(const GemvProblem &p, GemvShared &sh,
                                                   int8_t *xq_lds, bool write_out,
                                                   const f32x4 (&v)[kQuantBatch]) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n4 = p.K >> 2;
  float a = 0.0f;
#pragma unroll
  for (int j = 0; j < kQuantBatch; ++j)
    a = fmaxf(a, fmaxf(fmaxf(fabsf(v[j].x), fabsf(v[j].y)), fmaxf(fabsf(v[j].z), fabsf(v[j].w))));
  a = wave_max(a);
  if (lane == 0) sh.red[0][wave] = a;
  __syncthreads();
  a = fmaxf(fmaxf(sh.red[0][0], sh.red[0][1]), fmaxf(sh.red[0][2], sh.red[0][3]));
  const float s = (a == 0.0f) ? 1.0f : 127.0f / a;
  int sum = 0;
#pragma unroll
  for (int j = 0; j < kQuantBatch; ++j) {
    const int i = j * kThreads + tid;
    if (i < n4) {
      const int q0 = quant_one(v[j].x, s), q1 = quant_one(v[j].y, s);
      const int q2 = quant_one(v[j].z, s), q3 = quant_one(v[j].w, s);
      sum += q0 + q1 + q2 + q3;
      const uint32_t w = pack4_i8(q0, q1, q2, q3);
      *reinterpret_cast<uint32_t *>(xq_lds + perm_offset(4 * i)) = w;
      if (write_out) st_global<uint32_t>(p.xq_out + 4 * i, w);
    }
  }
  sum = wave_sum(sum);
  if (lane == 0) sh.ired[0][wave] = sum;
  if (tid == 0) {
    sh.scale[0] = s;
    if (write_out) st_global<float>(p.x_scale_out, s);
  }
  __syncthreads();
  if (tid == 0) sh.rowsum[0] = sh.ired[0][0] + sh.ired[0][1] + sh.ired[0][2] + sh.ired[0][3];
  __syncthreads();
}

template <bool BATCHED>
__device__ __forceinline__ void quant_rows_to_lds(const GemvProblem &p, GemvShared &sh,
                                                  int8_t *xq_lds, bool write_out) {
  if (BATCHED)
    quant_rows_batched(p, sh, xq_lds, write_out);
  else
    quant_rows_serial(p, sh, xq_lds, write_out);
}

// Workgroup blk of a problem: with S = 1, wave w owns columns
// [(4 blk + w) * 64, +64) over all K units; with a K-split S (single-row fused
// launches only), wave w owns the 64 columns of group g = w % (4/S) starting at
// (blk * 4/S + g) * 64, over K units [q * units / S, (q + 1) * units / S) with
// q = w / (4/S).  FUSED: the rows are quantized into LDS here; otherwise they
// are staged into LDS from the workspace chunk by chunk.
template <bool FUSED, bool SMALL>
__device__ __forceinline__ void gemv_block(const GemvProblem &p, int blk, bool split,
                                           GemvShared &sh, int8_t *lds) {
  constexpr int C = kGemvC;
  constexpr int D = FUSED ? kGemvDepth : kGemvDepthStaged;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;
  const int h = lane >> 4;
  const int total_units = p.K >> 7;
  const int S = FUSED ? gemv_split(total_units, split) : 1;
  const int G = kWaves / S;
  const int cgrp = wave % G;
  const int kq = wave / G;
  const int u0 = kq * total_units / S;
  const int units = (kq + 1) * total_units / S - u0;   // units of this wave

  const uint32_t w_bytes = (uint32_t)((size_t)p.N * p.K / 4);
  const __amdgpu_buffer_rsrc_t w_rsrc = make_rsrc(p.packed, w_bytes);
  const uint32_t ustride = (uint32_t)p.N * kUnitBytes;
  const bool a_live = col < p.M;
  const uint32_t a_row = (uint32_t)(a_live ? col : 0) * p.K + 32 * h;
  const int lane_col0 = (blk * G + cgrp) * kWaveCols + col;   // column of block 0

  // Staging: chunk k of the rows goes to LDS buffer k % 2; wave w copies units
  // kChunkUnits / 4 * w .. + kChunkUnits / 4 - 1 of the chunk, 8 rows per
  // 1 KB load: lane i takes row
  // 8q + i / 8 of load q and lands at chunk position i % 8, so it fetches
  // chunk stage_pos(i % 8, row) of that row.  Rows past M and units past K
  // are aimed beyond the buffer and land as zeros.
  const uint32_t a_bytes = (uint32_t)((size_t)p.M * p.K);
  const __amdgpu_buffer_rsrc_t a_rsrc = make_rsrc(FUSED ? nullptr : p.xqp, FUSED ? 0 : a_bytes);
  auto stage_chunk = [&](int k) {
#pragma unroll
    for (int q = 0; q < kChunkUnits / 2; ++q) {
      const int j = (kChunkUnits / 4) * wave + (q >> 1);   // unit within the chunk
      const int row = 8 * (q & 1) + (lane >> 3);
      const int u = k * kChunkUnits + j;
      const int chunk = stage_pos(lane & 7, row);
      const uint32_t off = (u < units && row < p.M)
                               ? (uint32_t)row * p.K + (uint32_t)u * kUnit + 16 * chunk
                               : a_bytes;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          a_rsrc,
          (lds_ptr_t)(lds + (k & 1) * kChunkBytes + (j * kGemvMaxM + 8 * (q & 1)) * kUnit), 16,
          off, 0, 0, 0);
    }
  };

  int lu = 0;   // next unit to fetch, relative to u0
  u32x2 wr[D][C];
  auto load_item = [&](u32x2 *w) {
    const bool live = lu < units;
    const uint32_t ub = (uint32_t)(u0 + lu) * ustride + 8 * h;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int n = lane_col0 + 16 * c;
      const uint32_t off = (live && n < p.N) ? (uint32_t)n * kUnitBytes + ub : w_bytes;
      w[c] = __builtin_amdgcn_raw_buffer_load_b64(w_rsrc, off, 0, kWeightAux);
    }
    ++lu;
  };
  if (!FUSED) stage_chunk(0);
  // A single fused row is loaded whole before the weights: the loads of one
  // wave complete in issue order, so a row loaded after the weight ring could
  // only be used once the ring's HBM reads had landed.
  const bool resident = FUSED && p.M == 1 && (p.K >> 2) <= kQuantBatch * kThreads;
  f32x4 xv[kQuantBatch];
  if (resident)
    load_row_batch(make_rsrc(p.x, (uint32_t)p.K * 4u), p.K >> 2, 0, xv);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < D; ++j) load_item(wr[j]);

  if (FUSED) {
    const bool out = p.xq_out != nullptr && blk == 0;
    if (resident)
      quant_row_resident(p, sh, lds, out, xv);
    else
      quant_rows_to_lds<SMALL>(p, sh, lds, out);
  }

  // Dequantization inputs of accumulator element r of this lane (row 4h + r).
  const float ws = ld_global<float>(p.w_scale);
  int row_rs[4];
  float row_xs[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = min(4 * h + r, p.M - 1);
    row_rs[r] = FUSED ? sh.rowsum[row] : ld_global<int>(p.rowsum + row);
    row_xs[r] = FUSED ? sh.scale[row] : ld_global<float>(p.x_scale + row);
  }

  v4i acc[C];
#pragma unroll
  for (int c = 0; c < C; ++c) acc[c] = v4i{0, 0, 0, 0};
  const v4i zero4 = v4i{0, 0, 0, 0};
  // Staged operand reads: row col of unit j, chunks 2h and 2h + 1.
  const int s_row = col * kUnit;
  const int s_c0 = stage_pos(2 * h, col) * 16, s_c1 = stage_pos(2 * h + 1, col) * 16;

  for (int base = 0; base < units; base += D) {
#pragma unroll
    for (int j = 0; j < D; ++j) {
      const int i = base + j;
      if (!FUSED && i < units && i % kChunkUnits == 0) {
        // Chunk i / kChunkUnits begins.  This wave's copy of it was issued before the
        // code loads of the last kChunkUnits units (C each) or, for the first
        // chunk, before those of the first D units; after the barrier every
        // wave's part is in LDS and every wave is done with the other buffer,
        // which the next chunk's copy overwrites.
        if (i == 0)
          __builtin_amdgcn_s_waitcnt(vmcnt_wait(D * C));
        else
          __builtin_amdgcn_s_waitcnt(vmcnt_wait(kChunkUnits * C));
        __builtin_amdgcn_s_barrier();
        stage_chunk(i / kChunkUnits + 1);
      }
      v4i a0 = zero4, a1 = zero4;
      if (a_live && i < units) {
        if (FUSED) {
          const v4i *ap =
              reinterpret_cast<const v4i *>(lds + a_row + (uint32_t)(u0 + i) * kUnit);
          a0 = ap[0];
          a1 = ap[1];
        } else {
          const int8_t *sp = lds + ((i / kChunkUnits) & 1) * kChunkBytes +
                             (i % kChunkUnits) * kGemvMaxM * kUnit + s_row;
          a0 = *reinterpret_cast<const v4i *>(sp + s_c0);
          a1 = *reinterpret_cast<const v4i *>(sp + s_c1);
        }
      }
      // Items past the range carry zero codes: their MFMAs add nothing.
#pragma unroll
      for (int c = 0; c < C; ++c) {
        acc[c] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, unpack_fields(wr[j][c].x), acc[c],
                                                       0, 0, 0);
        acc[c] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, unpack_fields(wr[j][c].y), acc[c],
                                                       0, 0, 0);
      }
      load_item(wr[j]);
    }
  }
  // The last chunk copy (units past K) must land before the workgroup's LDS
  // can be handed on.
  if (!FUSED) __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));

  if (S > 1) {
    // K-split partials: waves q > 0 park their accumulators in LDS (over the
    // activation row, once every wave is done with it); wave q = 0 adds them.
    v4i *part = reinterpret_cast<v4i *>(lds);
    __syncthreads();
    if (kq > 0) {
#pragma unroll
      for (int c = 0; c < C; ++c) part[(((kq - 1) * G + cgrp) * C + c) * 64 + lane] = acc[c];
    }
    __syncthreads();
    if (kq > 0) return;
    for (int q = 1; q < S; ++q) {
#pragma unroll
      for (int c = 0; c < C; ++c) acc[c] += part[(((q - 1) * G + cgrp) * C + c) * 64 + lane];
    }
  }

  // Element (row = 4h + r, column col) of each 16-column block.
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int n = lane_col0 + 16 * c;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 4 * h + r;
      if (row < p.M && n < p.N) {
        const int a = acc[c][r] - row_rs[r];
        if (p.acc_out) st_global<int>(p.acc_out + (size_t)row * p.N + n, a);
        st_global<float>(p.y + (size_t)row * p.N + n, dequant_exact(a, ws, row_xs[r]));
      }
    }
  }
}

// SMALL: a launch too small to fill the chip (the K-split form), whose
// workgroups quantize their row with batched loads.  Such a launch has fewer
// than two workgroups per CU, so the register budget is that of two waves per
// SIMD (measured faster than holding it to four).
template <bool FUSED, bool SMALL>
__global__ void __launch_bounds__(kThreads, SMALL ? 2 : 1) gemv_kernel(GemvProblem p, int split) {
  __shared__ GemvShared sh;
  extern __shared__ __attribute__((aligned(16))) int8_t xq_lds[];
  gemv_block<FUSED, SMALL>(p, blockIdx.x, split != 0, sh, xq_lds);
}

// Grouped: dispatch slot s of the table owns workgroups [blk_end[s-1], blk_end[s]).
template <bool FUSED, bool SMALL>
__global__ void __launch_bounds__(kThreads, SMALL ? 2 : 1)
    gemv_grouped_kernel(const bitnet_problem *__restrict__ problems, GroupTable tab,
                        const uint8_t *__restrict__ workspace) {
  __shared__ GemvShared sh;
  extern __shared__ __attribute__((aligned(16))) int8_t xq_lds[];
  // Block b runs on XCD b % 8; unless the table deals workgroups round-robin,
  // XCD x runs its own range [xcd_first[x], xcd_first[x + 1]) of whole
  // projections, so each projection's activations are fetched into one L2.
  uint32_t b = blockIdx.x;
  if (!tab.spread) {
    const uint32_t x = b % kXcds;
    b = tab.xcd_first[x] + b / kXcds;
    if (b >= tab.xcd_first[x + 1]) return;
  }
  const SlotInfo si = find_slot(tab, b);
  const uint32_t first = si.first;
  const int pi = si.problem;
  const bitnet_problem pr = problems[pi];
  const int M = tab.M;
  GemvProblem p;
  p.packed = pr.packed;
  p.x = pr.x;
  if (!FUSED) {
    const WsLayout L = ws_layout(M, pr.K);
    const uint8_t *ws = workspace + (size_t)tab.ws_off[pi] * 256;
    p.xqp = reinterpret_cast<const int8_t *>(ws + L.xq);
    p.x_scale = reinterpret_cast<const float *>(ws + L.scale);
    p.rowsum = reinterpret_cast<const int32_t *>(ws + L.rowsum);
  } else {
    p.xqp = nullptr;
    p.x_scale = nullptr;
    p.rowsum = nullptr;
  }
  p.w_scale = pr.w_scale;
  p.y = pr.y;
  p.acc_out = nullptr;
  p.xq_out = nullptr;
  p.x_scale_out = nullptr;
  p.N = (int)pr.N;
  p.K = (int)pr.K;
  p.M = M;
  gemv_block<FUSED, SMALL>(p, (int)(b - first), tab.split != 0, sh, xq_lds);
}

}  // namespace

int gemv_blocks(int64_t N, int64_t K, bool split) {
  const int64_t cols = (int64_t)(kWaves / gemv_split((int)(K >> 7), split)) * kWaveCols;
  return (int)((N + cols - 1) / cols);
}

bool gemv_fusable(int64_t M, int64_t K) { return M * K <= kGemvFusedLdsBytes; }

// Dynamic LDS of a fused launch whose longest K is kmax: the quantized rows,
// and the K-split partials, which reuse the same space afterwards.
static size_t fused_lds_bytes(int64_t M, int64_t kmax, bool split) {
  const int S = gemv_split((int)(kmax >> 7), split);
  const size_t part = (size_t)(S - 1) * (kWaves / S) * kGemvC * 64 * sizeof(v4i);
  const size_t rows = (size_t)(M * kmax);
  return rows > part ? rows : part;
}

hipError_t launch_gemv(int M, int N, int K, const int8_t *xq_perm, const float *x_scale,
                       const int32_t *rowsum, const uint8_t *packed, const float *w_scale,
                       float *y, int32_t *acc_out, hipStream_t stream) {
  GemvProblem p{packed, nullptr, xq_perm, x_scale, rowsum, w_scale, y, acc_out,
                nullptr, nullptr, N, K, M};
  gemv_kernel<false, false><<<gemv_blocks(N, K, false), kThreads, 2 * kChunkBytes, stream>>>(p, 0);
  return hipGetLastError();
}

hipError_t launch_gemv_fused(int M, int N, int K, const float *x, const uint8_t *packed,
                             const float *w_scale, float *y, int8_t *xq_out,
                             float *x_scale_out, int32_t *acc_out, hipStream_t stream) {
  GemvProblem p{packed, x, nullptr, nullptr, nullptr, w_scale, y, acc_out,
                xq_out, x_scale_out, N, K, M};
  const bool split = gemv_blocks(N, K, false) < kGemvSplitBelow;
  if (split)
    gemv_kernel<true, true><<<gemv_blocks(N, K, true), kThreads, fused_lds_bytes(M, K, true),
                              stream>>>(p, 1);
  else
    gemv_kernel<true, false><<<gemv_blocks(N, K, false), kThreads,
                               fused_lds_bytes(M, K, false), stream>>>(p, 0);
  return hipGetLastError();
}

hipError_t launch_gemv_grouped(const bitnet_problem *problems, const GroupTable &tab,
                               const uint8_t *workspace, bool fused, int64_t kmax,
                               hipStream_t stream) {
  const unsigned blocks = tab.spread ? tab.blk_end[tab.count - 1] : xcd_grid(tab.xcd_first);
  if (fused && tab.split)
    gemv_grouped_kernel<true, true><<<blocks, kThreads, fused_lds_bytes(tab.M, kmax, true),
                                      stream>>>(problems, tab, workspace);
  else if (fused)
    gemv_grouped_kernel<true, false><<<blocks, kThreads, fused_lds_bytes(tab.M, kmax, false),
                                       stream>>>(problems, tab, workspace);
  else
    gemv_grouped_kernel<false, false><<<blocks, kThreads, 2 * kChunkBytes, stream>>>(
        problems, tab, workspace);
  return hipGetLastError();
}

}  // namespace bitnet
