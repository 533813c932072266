// Prefill projection, M > 16 rows: a dense int8 contraction on the matrix cores.
//
// With ternary weights the projection is a sum of added and subtracted
// activations (xujun.org article, heterogeneous-quantization section); over
// hundreds of token rows that is a dense contraction, done here on
// v_mfma_i32_32x32x32_i8 with int32 accumulation.
//
// Workgroup tile 128 x 256, 4 waves side by side: wave w owns all 128 rows and
// columns [64w, 64w + 64) as 4 x 2 blocks of 32 x 32.  Per 128-input unit:
//   - the activation tile (128 rows x 128 permuted int8 = 16 KB) goes straight
//     from memory into LDS (buffer_load ... lds), into a ring of three stages
//     issued two units ahead; rows past M load as zeros.  Inside a stage, the
//     16-byte chunk c of tile row r sits at chunk position c ^ (r % 8), so the
//     MFMA operand reads of 8 consecutive rows hit 8 different bank groups;
//   - each wave reads its 64 columns of packed codes (16 bytes = 64 codes per
//     lane and block) into a register ring, also two units ahead, and expands
//     the 2-bit fields to int8 in registers; every expanded operand feeds four
//     MFMAs and never touches LDS.
// The unit loop is unrolled by three so ring slots are static; units past K
// load zeros (no memory access) and add nothing, so every slot issues the same
// loads and the wait counts are exact.
// Lane (i = lane%32, h = lane/32) feeds MFMA e (0..3) of a unit with packed
// dword d = 4h + e of its column and the 16 permuted activations at 16*d of its
// row, so the k positions of both operands agree by construction.
//
// Blocks are renumbered so that consecutive logical tiles (the row blocks of
// one column tile first) stay on one XCD and share its L2.
#include "bitnet_device.hpp"
#include "bitnet_internal.hpp"

namespace bitnet {
namespace {

constexpr int BM = 128;
constexpr int BN = 256;
constexpr int WN = 64;                 // columns per wave
constexpr int RB = BM / 32;            // 32-row MFMA blocks per wave
constexpr int CB = WN / 32;            // 32-column MFMA blocks per wave
constexpr int kStages = 3;             // LDS / register ring depth (units)
constexpr int kStageBytes = BM * 128;  // one activation tile
constexpr int kThreads = 256;
constexpr int kXcds = 8;

// Two workgroups per CU: the accumulators then live in arch VGPRs, leaving room
// for a second wave per SIMD to cover the other's waits.
#ifndef BITNET_GEMM_WAVES_PER_EU
#define BITNET_GEMM_WAVES_PER_EU 2
#endif
#define BITNET_GEMM_OCCUPANCY \
  __attribute__((amdgpu_waves_per_eu(BITNET_GEMM_WAVES_PER_EU, BITNET_GEMM_WAVES_PER_EU)))

typedef __attribute__((address_space(3))) void *lds_ptr_t;

struct GemmProblem {
  const uint8_t *packed;
  const int8_t *xqp;
  const float *x_scale;
  const int32_t *rowsum;
  const float *w_scale;
  float *y;
  int32_t *acc_out;
  int M, N, K;
};

struct GemmShared {
  __attribute__((aligned(16))) int8_t a[kStages][kStageBytes];
  float factor[BM];   // w_scale / x_scale of each row of the tile
  int rowsum[BM];
};

// Logical block index.  Blocks are dealt round-robin to the XCDs (block b to
// XCD b % 8), so blocks b, b + 8, b + 16, ... share one L2.  Within each group
// of 8 * mt consecutive blocks, renumber so that the mt row blocks of one column
// tile are such a same-XCD sequence: they then read the tile's packed codes
// through one L2.  The coarse order of the launch (and with it the balance of
// long and short tiles across XCDs) is unchanged; a partial last group keeps
// its order.
__device__ __forceinline__ uint32_t xcd_logical(uint32_t b, uint32_t G, uint32_t mt) {
  const uint32_t span = kXcds * mt;
  const uint32_t base = b - b % span;
  if (base + span > G) return b;
  const uint32_t r = b - base;
  return base + (r % kXcds) * mt + r / kXcds;
}

__device__ __forceinline__ void gemm_block(const GemmProblem &p, int m0, int n0, GemmShared &sh) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int li = lane & 31, lh = lane >> 5;
  const int units = p.K >> 7;

  // Activation DMA: wave w fills tile rows [32w, 32w + 32) with 4 loads of 1 KB;
  // load j of the wave covers rows 32w + 8j .. +7, lane i lands at chunk
  // position i % 8 of row 32w + 8j + i / 8 and so fetches chunk (i % 8) ^ (i / 8).
  const uint32_t a_bytes = (uint32_t)((size_t)p.M * p.K);
  const __amdgpu_buffer_rsrc_t a_rsrc = make_rsrc(p.xqp, a_bytes);
  uint32_t dma_off[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = m0 + 32 * wave + 8 * j + (lane >> 3);
    const int chunk = (lane & 7) ^ (lane >> 3);
    dma_off[j] = row < p.M ? (uint32_t)row * p.K + 16 * chunk : a_bytes;
  }
  auto issue_dma = [&](int u, int stage) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t off = (u < units && dma_off[j] < a_bytes) ? dma_off[j] + (uint32_t)u * kUnit
                                                               : a_bytes;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          a_rsrc, (lds_ptr_t)(&sh.a[stage][(32 * wave + 8 * j) * 128]), 16, off, 0, 0, 0);
    }
  };

  // Packed codes: lane owns bytes 16*lh..16*lh+15 of each of its CB columns.
  const uint32_t w_bytes = (uint32_t)((size_t)p.N * p.K / 4);
  const __amdgpu_buffer_rsrc_t w_rsrc = make_rsrc(p.packed, w_bytes);
  const uint32_t ustride = (uint32_t)p.N * kUnitBytes;
  uint32_t w_off[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const int n = n0 + wave * WN + cb * 32 + li;
    w_off[cb] = n < p.N ? (uint32_t)n * kUnitBytes + 16 * lh : w_bytes;
  }
  auto load_b = [&](int u, v4i *dst) {
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
      dst[cb] = __builtin_amdgcn_raw_buffer_load_b128(
          w_rsrc, u < units ? w_off[cb] + (uint32_t)u * ustride : w_bytes, 0, 0);
  };

  // A operand reads: row 32rb + li, chunk 4lh + e at position (4lh + e) ^ (li % 8).
  uint32_t a_rd[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) a_rd[e] = li * 128 + (((4 * lh + e) ^ (li & 7)) * 16);

  // Per-row dequantization factors and row sums of the tile.
  if (tid < BM) {
    const int row = min(m0 + tid, p.M - 1);
    sh.factor[tid] = ld_global<float>(p.w_scale) / ld_global<float>(p.x_scale + row);
    sh.rowsum[tid] = ld_global<int>(p.rowsum + row);
  }

  v4i bq[kStages][CB];
  load_b(0, bq[0]);
  issue_dma(0, 0);
  load_b(1, bq[1]);
  issue_dma(1, 1);
  __syncthreads();

  // Accumulators start at -rowsum of their row, which removes the +1 offset of
  // the code fields: element r of a 32x32 block sits at row 8*(r/4) + 4*(lane/32)
  // + r%4, column lane%32.
  v16i acc[RB][CB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const v4i rs = *reinterpret_cast<const v4i *>(&sh.rowsum[rb * 32 + 8 * g + 4 * lh]);
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int k = 0; k < 4; ++k) acc[rb][cb][4 * g + k] = -rs[k];
    }

  for (int base = 0; base < units; base += kStages) {
#pragma unroll
    for (int s = 0; s < kStages; ++s) {
      const int u = base + s;
      // This wave's loads of unit u are its oldest outstanding ones; those of
      // unit u + 1 (4 activation loads + CB code loads) may stay in flight.
      // After the barrier every wave's part of stage s is in LDS, and every
      // wave has finished reading stage (s + 2) % 3 (its reads of unit u - 1
      // completed before the MFMAs that consumed them), which the next loads
      // overwrite.  A plain barrier: a memory fence here would drain the
      // in-flight loads of unit u + 1 as well.
      __builtin_amdgcn_s_waitcnt(vmcnt_wait(4 + CB));
      __builtin_amdgcn_s_barrier();
      load_b(u + 2, bq[(s + 2) % kStages]);
      issue_dma(u + 2, (s + 2) % kStages);
      // Operands of k-chunk e + 1 (LDS reads, code unpack) are fetched while
      // the MFMAs of chunk e run.
      const int8_t *a_stage = sh.a[s];
      v4i a_nx[RB], b_nx[CB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        a_nx[rb] = *reinterpret_cast<const v4i *>(a_stage + a_rd[0] + rb * 32 * 128);
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) b_nx[cb] = unpack_fields((uint32_t)bq[s][cb][0]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v4i a_cu[RB], b_cu[CB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) a_cu[rb] = a_nx[rb];
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) b_cu[cb] = b_nx[cb];
        if (e + 1 < 4) {
#pragma unroll
          for (int rb = 0; rb < RB; ++rb)
            a_nx[rb] = *reinterpret_cast<const v4i *>(a_stage + a_rd[e + 1] + rb * 32 * 128);
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) b_nx[cb] = unpack_fields((uint32_t)bq[s][cb][e + 1]);
        }
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int cb = 0; cb < CB; ++cb)
            acc[rb][cb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a_cu[rb], b_cu[cb], acc[rb][cb],
                                                               0, 0, 0);
      }
#if BITNET_GEMM_SCHED
      // Interleave: every MFMA is followed by part of the next chunk's LDS
      // reads and code unpacking, so they run while the matrix core is busy.
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
        __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);  // VALU
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);  // VALU
      }
#endif
    }
  }

  // Epilogue through buffer stores: the lane's column offset is fixed and the
  // row offset is uniform, both in the vector offset (the range check covers
  // it): rows past M fall beyond the buffer and are dropped, columns past N are
  // aimed beyond it.  The shape limits keep (M + 128) * N * 4 below 2^31, so no
  // offset wraps.
  const uint32_t y_bytes = (uint32_t)((size_t)p.M * p.N * 4);
  const __amdgpu_buffer_rsrc_t y_rsrc = make_rsrc(p.y, y_bytes);
  const __amdgpu_buffer_rsrc_t c_rsrc = make_rsrc(p.acc_out, p.acc_out ? y_bytes : 0);
  uint32_t col_off[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const int n = n0 + wave * WN + cb * 32 + li;
    col_off[cb] = n < p.N ? (uint32_t)(4 * lh * p.N + n) * 4u : 0x80000000u;
  }
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int lrow = rb * 32 + 8 * g + 4 * lh;     // first of 4 consecutive tile rows
      const f32x4 f = *reinterpret_cast<const f32x4 *>(&sh.factor[lrow]);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t row_off = (uint32_t)(m0 + rb * 32 + 8 * g + k) * (uint32_t)p.N * 4u;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          const int a = acc[rb][cb][4 * g + k];
          const uint32_t off = col_off[cb] + row_off;
          __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, (float)a * f[k]), y_rsrc,
                                                off, 0, 0);
          if (p.acc_out) __builtin_amdgcn_raw_buffer_store_b32(a, c_rsrc, off, 0, 0);
        }
      }
    }
  }
}

__global__ void __launch_bounds__(kThreads) BITNET_GEMM_OCCUPANCY gemm_kernel(GemmProblem p) {
  __shared__ GemmShared sh;
  const int mt = (p.M + BM - 1) / BM;
  const uint32_t L = xcd_logical(blockIdx.x, gridDim.x, mt);
  gemm_block(p, (int)(L % mt) * BM, (int)(L / mt) * BN, sh);
}

__global__ void __launch_bounds__(kThreads) BITNET_GEMM_OCCUPANCY
    gemm_grouped_kernel(const bitnet_problem *__restrict__ problems, GroupTable tab,
                        const uint8_t *__restrict__ workspace) {
  __shared__ GemmShared sh;
  const uint32_t b = xcd_logical(blockIdx.x, gridDim.x, (tab.M + BM - 1) / BM);
  const SlotInfo si = find_slot(tab, b);
  const uint32_t first = si.first;
  const int pi = si.problem;
  const bitnet_problem pr = problems[pi];
  const int M = tab.M;
  const WsLayout L = ws_layout(M, pr.K);
  const uint8_t *ws = workspace + (size_t)tab.ws_off[pi] * 256;
  GemmProblem p;
  p.packed = pr.packed;
  p.xqp = reinterpret_cast<const int8_t *>(ws + L.xq);
  p.x_scale = reinterpret_cast<const float *>(ws + L.scale);
  p.rowsum = reinterpret_cast<const int32_t *>(ws + L.rowsum);
  p.w_scale = pr.w_scale;
  p.y = pr.y;
  p.acc_out = nullptr;
  p.M = M;
  p.N = (int)pr.N;
  p.K = (int)pr.K;
  const int mt = (M + BM - 1) / BM;
  const int local = (int)(b - first);
  gemm_block(p, (local % mt) * BM, (local / mt) * BN, sh);
}

}  // namespace

int gemm_blocks(int64_t M, int64_t N) {
  return (int)(((M + BM - 1) / BM) * ((N + BN - 1) / BN));
}

hipError_t launch_gemm(int M, int N, int K, const int8_t *xq_perm, const float *x_scale,
                       const int32_t *rowsum, const uint8_t *packed, const float *w_scale,
                       float *y, int32_t *acc_out, hipStream_t stream) {
  GemmProblem p{packed, xq_perm, x_scale, rowsum, w_scale, y, acc_out, M, N, K};
  gemm_kernel<<<gemm_blocks(M, N), kThreads, 0, stream>>>(p);
  return hipGetLastError();
}

hipError_t launch_gemm_grouped(const bitnet_problem *problems, const GroupTable &tab,
                               const uint8_t *workspace, hipStream_t stream) {
  const unsigned blocks = tab.blk_end[tab.count - 1];
  gemm_grouped_kernel<<<blocks, kThreads, 0, stream>>>(problems, tab, workspace);
  return hipGetLastError();
}

}  // namespace bitnet
