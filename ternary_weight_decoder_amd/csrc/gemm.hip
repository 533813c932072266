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
// loads and the wait counts are exact.  With 128-row tiles a unit's loads go
// out between its first MFMA chunks, not all at once after its barrier.
// Lane (i = lane%32, h = lane/32) feeds MFMA e (0..3) of a unit with packed
// dword d = 4h + e of its column and the 16 permuted activations at 16*d of its
// row, so the k positions of both operands agree by construction.
//
// A grouped launch gives each XCD a set of whole projections of about equal
// work, and each projection's tiles are ordered in bands of row blocks, so the
// data an XCD needs stays in its own L2 instead of every projection's
// activations and codes being fetched by all eight.
#include <algorithm>

#include "bitnet_device.hpp"
#include "bitnet_internal.hpp"

namespace bitnet {
namespace {

constexpr int BN = 256;
constexpr int WN = 64;                 // columns per wave
constexpr int CB = WN / 32;            // 32-column MFMA blocks per wave
#ifndef BITNET_GEMM_STAGES
#define BITNET_GEMM_STAGES 3
#endif
constexpr int kStages = BITNET_GEMM_STAGES;   // LDS / register ring depth (units)
constexpr int kThreads = 256;

// Tile heights: 128 rows for prefill, 64 or 32 rows for batched decode
// (M <= 64), where a 128-row tile would mostly multiply padding.  Waves per
// SIMD: with a 128-row tile two workgroups per CU keep the accumulators in arch
// VGPRs and let each wave cover the other's waits; smaller tiles need fewer
// registers and run more waves.
template <int BM>
struct TileCfg {
  static constexpr int RB = BM / 32;             // 32-row MFMA blocks per wave
  static constexpr int kStageBytes = BM * 128;   // one activation tile
  static constexpr int kDma = BM / 32;           // 1 KB activation loads per wave and unit
  static constexpr int kWavesPerEu = BM >= 128 ? 2 : BM >= 64 ? 4 : 5;
};

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

template <int BM>
struct GemmShared {
  __attribute__((aligned(16))) int8_t a[kStages][TileCfg<BM>::kStageBytes];
  float factor[BM];   // w_scale / x_scale of each row of the tile
  int rowsum[BM];
};

// Tile order inside one projection: bands of kBand row blocks, column tiles
// one after another inside a band, the band's row blocks consecutive.  The
// tiles an XCD runs at one time then share a few activation row blocks and
// code column tiles in its L2, and a band's activation rows stay there while
// it sweeps the columns.
// Cache policy of the output stores: non-temporal, so the output stream does
// not evict the activation and code tiles that other workgroups still read.
#ifndef BITNET_GEMM_STORE_AUX
#define BITNET_GEMM_STORE_AUX 2
#endif
constexpr int kStoreAux = BITNET_GEMM_STORE_AUX;

// Tile height from which a unit's loads are issued between its MFMA chunks
// instead of right after the barrier (measured: faster with 128-row tiles,
// slower with the 32- and 64-row tiles of batched decode).
#ifndef BITNET_GEMM_SPREAD_MINBM
#define BITNET_GEMM_SPREAD_MINBM 128
#endif
#ifndef BITNET_GEMM_FENCE
#define BITNET_GEMM_FENCE 1
#endif
#ifndef BITNET_GEMM_BAND
#define BITNET_GEMM_BAND 4
#endif
constexpr int kBand = BITNET_GEMM_BAND;

__device__ __forceinline__ void band_tile(int t, int mt, int nt, int &rb, int &ct) {
  const int band = t / (kBand * nt);
  const int r0 = band * kBand;
  const int rows = min(kBand, mt - r0);
  const int tt = t - band * kBand * nt;
  ct = tt / rows;
  rb = r0 + tt % rows;
}

// Workgroups are dealt round-robin to the XCDs (block b to XCD b % 8), so
// block b runs tile b / 8 of the range owned by XCD b % 8.  Each XCD then
// works through its own projections (or, for a single projection, one compact
// piece of it) instead of every projection being spread over all eight L2s.

// Chunk swizzle of tile row r (16-byte chunks, 8 per 128-byte row).  An MFMA
// operand read (ds_read_b128) serves 16 lanes per cycle: rows li = 0..15 of one
// chunk column.  Pairs of rows share a 256-byte bank line, so rows 2i and 2i+1
// fall in different halves and the 8 pairs need 8 different chunk positions.
#ifndef BITNET_GEMM_SWZ_SHIFT
#define BITNET_GEMM_SWZ_SHIFT 1
#endif
__device__ __forceinline__ int swz(int r) { return (r >> BITNET_GEMM_SWZ_SHIFT) & 7; }

// One output tile over K units [ub, ub + nunits).  SPLIT: the tile is one of
// several K slices; its raw int32 sums (field values times activations, no
// row-sum correction) are added atomically into the output buffer, which
// holds int32 partial sums until the finishing pass.  RB: the 32-row blocks
// the tile multiplies and stores, fewer than BM / 32 for the last row block of
// a ragged M (its activation loads still cover BM rows, those past M as zeros,
// so the ring and its wait counts are the same for every tile).
template <int BM, bool SPLIT, int RB>
__device__ __forceinline__ void gemm_block(const GemmProblem &p, int m0, int n0, int ub,
                                           int nunits, GemmShared<BM> &sh) {
  static_assert(RB >= 1 && RB <= TileCfg<BM>::RB, "row blocks per tile");
  constexpr int kDma = TileCfg<BM>::kDma;
  constexpr bool kSpread = BM >= BITNET_GEMM_SPREAD_MINBM;
  // Code loads of 32- and 64-row tiles (M <= 64: one row block, so every code
  // is read once) are non-temporal and leave L2 to the activation rows that
  // every column tile re-reads; 128-row tiles re-read codes across row bands
  // and keep them cacheable.
  constexpr int kCodeAux = BM <= 64 ? 2 : 0;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int li = lane & 31, lh = lane >> 5;
  const int units = nunits;

  // Activation DMA: wave w fills tile rows [BM/4 w, BM/4 (w + 1)) with kDma
  // loads of 1 KB; load j of the wave covers rows BM/4 w + 8j .. +7, lane i
  // lands at chunk position i % 8 of row r = BM/4 w + 8j + i / 8 and so fetches
  // chunk (i % 8) ^ swz(r).
  const uint32_t a_bytes = (uint32_t)((size_t)p.M * p.K);
  const __amdgpu_buffer_rsrc_t a_rsrc = make_rsrc(p.xqp, a_bytes);
  uint32_t dma_off[kDma];
#pragma unroll
  for (int j = 0; j < kDma; ++j) {
    const int row = m0 + 8 * kDma * wave + 8 * j + (lane >> 3);
    const int chunk = (lane & 7) ^ swz(8 * kDma * wave + 8 * j + (lane >> 3));
    dma_off[j] = row < p.M ? (uint32_t)row * p.K + (uint32_t)ub * kUnit + 16 * chunk : a_bytes;
  }
  auto issue_dma = [&](int u, int stage) {
#pragma unroll
    for (int j = 0; j < kDma; ++j) {
      const uint32_t off = (u < units && dma_off[j] < a_bytes) ? dma_off[j] + (uint32_t)u * kUnit
                                                               : a_bytes;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          a_rsrc, (lds_ptr_t)(&sh.a[stage][(8 * kDma * wave + 8 * j) * 128]), 16, off, 0, 0, 0);
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
    w_off[cb] = n < p.N ? (uint32_t)ub * ustride + (uint32_t)n * kUnitBytes + 16 * lh : w_bytes;
  }
  auto load_b = [&](int u, v4i *dst) {
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
      dst[cb] = __builtin_amdgcn_raw_buffer_load_b128(
          w_rsrc, u < units ? w_off[cb] + (uint32_t)u * ustride : w_bytes, 0, kCodeAux);
  };

  // A operand reads: row 32rb + li, chunk 4lh + e at position (4lh + e) ^ swz(li).
  uint32_t a_rd[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) a_rd[e] = li * 128 + (((4 * lh + e) ^ swz(li)) * 16);

  // Per-row dequantization factors and row sums of the tile.  Their loads go
  // out first and their values go to LDS after the ring's first loads are
  // issued, so the tile start waits for one memory round trip, not two.  (A
  // wave's loads complete in issue order: waiting for these does not wait for
  // the ring.)  The publishing barrier waits for LDS only; the ring's first
  // units stay in flight until the K loop's own waits.
  float xs_row = 1.0f, ws_all = 0.0f;
  int rs_row = 0;
  if (tid < BM) {
    const int row = min(m0 + tid, p.M - 1);
    ws_all = ld_global<float>(p.w_scale);
    xs_row = ld_global<float>(p.x_scale + row);
    rs_row = ld_global<int>(p.rowsum + row);
  }
  __builtin_amdgcn_sched_barrier(0);

  v4i bq[kStages][CB];
#pragma unroll
  for (int u = 0; u < kStages - 1; ++u) {
    load_b(u, bq[u]);
    issue_dma(u, u);
  }
  __builtin_amdgcn_sched_barrier(0);
  if (tid < BM) {
    sh.factor[tid] = ws_all / xs_row;
    sh.rowsum[tid] = rs_row;
  }
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(lgkmcnt_wait(0));
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);

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
        for (int k = 0; k < 4; ++k) acc[rb][cb][4 * g + k] = SPLIT ? 0 : -rs[k];
    }

  for (int base = 0; base < units; base += kStages) {
#pragma unroll
    for (int s = 0; s < kStages; ++s) {
      const int u = base + s;
      // This wave's loads of unit u are its oldest outstanding ones; those of
      // units u + 1 .. u + kStages - 2 (kDma activation loads + CB code loads
      // each) may stay in flight.  After the barrier every wave's part of stage
      // s is in LDS, and every wave has finished reading the stage of unit
      // u - 1 (its reads completed before the MFMAs that consumed them), which
      // the next loads overwrite.  A plain barrier: a memory fence here would
      // drain the in-flight loads of the later units as well.
      // Nothing is scheduled across this point: left free, the compiler pulls
      // the next unit's code unpacking into this one, which then has to wait
      // for that unit's loads.
#if BITNET_GEMM_FENCE
      __builtin_amdgcn_sched_barrier(0);
#endif
      __builtin_amdgcn_s_waitcnt(vmcnt_wait((kStages - 2) * (kDma + CB)));
      __builtin_amdgcn_s_barrier();
      if (!kSpread) {
        load_b(u + kStages - 1, bq[(s + kStages - 1) % kStages]);
        issue_dma(u + kStages - 1, (s + kStages - 1) % kStages);
      }
#if BITNET_GEMM_FENCE
      __builtin_amdgcn_sched_barrier(0);   // (shorter tiles) the loads go out before the MFMAs
#endif
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
        // 128-row tiles: the next unit's loads go out behind this chunk's
        // MFMAs (the activation copy after chunk 0, the codes after chunk 1)
        // rather than all at once after the barrier, where the four waves'
        // 24 loads held up the first MFMAs while the address queue took them.
        if (kSpread && e == 0) {
          __builtin_amdgcn_sched_barrier(0);
          issue_dma(u + kStages - 1, (s + kStages - 1) % kStages);
          __builtin_amdgcn_sched_barrier(0);
        } else if (kSpread && e == 1) {
          __builtin_amdgcn_sched_barrier(0);
          load_b(u + kStages - 1, bq[(s + kStages - 1) % kStages]);
          __builtin_amdgcn_sched_barrier(0);
        }
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

  // The last ring slots loaded zeros into LDS; let them land before the
  // workgroup can end and its LDS be handed to another one.
  __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));

  // Epilogue through buffer stores: the lane's column offset is fixed and the
  // row offset is uniform, both in the vector offset (the range check covers
  // it): rows past M fall beyond the buffer and are dropped, columns past N are
  // aimed beyond it.  The shape limits keep (M + 128) * N * 4 below 2^31, so no
  // offset wraps.
  const uint32_t y_bytes = (uint32_t)((size_t)p.M * p.N * 4);
  const __amdgpu_buffer_rsrc_t y_rsrc = make_rsrc(p.y, y_bytes);
  if (SPLIT) {
    uint32_t col_off[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int n = n0 + wave * WN + cb * 32 + li;
      col_off[cb] = n < p.N ? (uint32_t)(4 * lh * p.N + n) * 4u : 0x80000000u;
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t row_off = (uint32_t)(m0 + rb * 32 + 8 * g + k) * (uint32_t)p.N * 4u;
#pragma unroll
          for (int cb = 0; cb < CB; ++cb)
            __builtin_amdgcn_raw_ptr_buffer_atomic_add_i32(acc[rb][cb][4 * g + k], y_rsrc,
                                                           col_off[cb] + row_off, 0, 0);
        }
    return;
  }
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
                                                off, 0, kStoreAux);
          if (p.acc_out) __builtin_amdgcn_raw_buffer_store_b32(a, c_rsrc, off, 0, 0);
        }
      }
    }
  }
}

// A tile starting at row m0: as many 32-row blocks as the rows left below M
// need, so the last row block of a ragged M does not multiply padding rows.
template <int BM, bool SPLIT, int RB = TileCfg<BM>::RB>
__device__ __forceinline__ void gemm_tile(const GemmProblem &p, int m0, int n0, int ub,
                                          int nunits, GemmShared<BM> &sh) {
  if constexpr (RB > 1) {
    if (p.M - m0 <= 32 * (RB - 1)) {
      gemm_tile<BM, SPLIT, RB - 1>(p, m0, n0, ub, nunits, sh);
      return;
    }
  }
  gemm_block<BM, SPLIT, RB>(p, m0, n0, ub, nunits, sh);
}

template <int BM>
__global__ void __launch_bounds__(kThreads)
    __attribute__((amdgpu_waves_per_eu(TileCfg<BM>::kWavesPerEu, TileCfg<BM>::kWavesPerEu)))
        gemm_kernel(GemmProblem p) {
  __shared__ GemmShared<BM> sh;
  const int mt = (p.M + BM - 1) / BM;
  const int nt = (p.N + BN - 1) / BN;
  const uint32_t tiles = (uint32_t)(mt * nt);
  const uint32_t x = blockIdx.x % kXcds;
  const uint32_t t = x * tiles / kXcds + blockIdx.x / kXcds;
  if (t >= (x + 1) * tiles / kXcds) return;
  int rb, ct;
  band_tile((int)t, mt, nt, rb, ct);
  gemm_tile<BM, false>(p, rb * BM, ct * BN, 0, p.K >> 7, sh);
}

// K-split form for launches with few tiles: block b runs K slice b % S of tile
// b / S (S consecutive blocks share a tile's rows and columns).
template <int BM>
__global__ void __launch_bounds__(kThreads)
    __attribute__((amdgpu_waves_per_eu(TileCfg<BM>::kWavesPerEu, TileCfg<BM>::kWavesPerEu)))
        gemm_split_kernel(GemmProblem p, int S) {
  __shared__ GemmShared<BM> sh;
  const int mt = (p.M + BM - 1) / BM;
  const int nt = (p.N + BN - 1) / BN;
  const int t = (int)blockIdx.x / S;
  const int q = (int)blockIdx.x % S;
  const int units = p.K >> 7;
  const int ub = q * units / S;
  int rb, ct;
  band_tile(t, mt, nt, rb, ct);
  gemm_tile<BM, true>(p, rb * BM, ct * BN, ub, (q + 1) * units / S - ub, sh);
}

// Zero the output before the K slices add into it (a fill kernel, so that the
// sequence can be captured in a graph).
__global__ void __launch_bounds__(256) zero_kernel(uint32_t *__restrict__ y, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) st_global<uint32_t>(y + i, 0u);
}

// Finish the K-split sums in place: y = (sum - rowsum) * w_scale / x_scale.
__global__ void __launch_bounds__(256)
    split_finish_kernel(float *__restrict__ y, int M, int N, const float *__restrict__ x_scale,
                        const int32_t *__restrict__ rowsum, const float *__restrict__ w_scale,
                        int32_t *__restrict__ acc_out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)M * N) return;
  const int m = (int)(i / N);
  const int a = ld_global<int>(y + i) - ld_global<int>(rowsum + m);
  const float f = ld_global<float>(w_scale) / ld_global<float>(x_scale + m);
  if (acc_out) st_global<int>(acc_out + i, a);
  st_global<float>(y + i, (float)a * f);
}

template <int BM>
__global__ void __launch_bounds__(kThreads)
    __attribute__((amdgpu_waves_per_eu(TileCfg<BM>::kWavesPerEu, TileCfg<BM>::kWavesPerEu)))
        gemm_grouped_kernel(const bitnet_problem *__restrict__ problems, GroupTable tab,
                            const uint8_t *__restrict__ workspace) {
  __shared__ GemmShared<BM> sh;
  uint32_t g = blockIdx.x;
  if (!tab.spread) {
    const uint32_t x = blockIdx.x % kXcds;
    g = tab.xcd_first[x] + blockIdx.x / kXcds;
    if (g >= tab.xcd_first[x + 1]) return;
  }
  const SlotInfo si = find_slot(tab, g);
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
  int rb, ct;
  band_tile((int)(g - si.first), (M + BM - 1) / BM, (p.N + BN - 1) / BN, rb, ct);
  gemm_tile<BM, false>(p, rb * BM, ct * BN, 0, p.K >> 7, sh);
}

}  // namespace

// Rows per tile for a launch of M rows.
#ifndef BITNET_GEMM_BM32_MAXM
#define BITNET_GEMM_BM32_MAXM 32
#endif
static int gemm_bm(int64_t M) {
  return M <= BITNET_GEMM_BM32_MAXM ? 32 : M <= 64 ? 64 : 128;
}

int gemm_blocks(int64_t M, int64_t N) {
  const int64_t bm = gemm_bm(M);
  return (int)(((M + bm - 1) / bm) * ((N + BN - 1) / BN));
}

void xcd_schedule(GroupTable &tab, const bitnet_problem *problems_host, const uint32_t *tiles) {
  // Each XCD gets a set of whole projections of about equal work (a
  // workgroup's work is its number of K units), assigned longest K first to
  // the least loaded XCD, so every XCD holds its share of the long-K
  // workgroups and starts them first, and a projection's activations and codes
  // are fetched into one L2 only.  When the projections are too few for that
  // to balance, the workgroups are dealt to the XCDs round-robin instead.
  const int count = tab.count;
  int slot[kMaxGroup];
  uint64_t work[kMaxGroup];
  for (int s = 0; s < count; ++s) {
    const int p = tab.order[s];
    slot[s] = s;
    work[s] = (uint64_t)tiles[s] * (uint64_t)(problems_host[p].K / kUnit);
  }
  std::stable_sort(slot, slot + count, [&](int a, int b) {
    const int64_t ka = problems_host[tab.order[a]].K, kb = problems_host[tab.order[b]].K;
    return ka != kb ? ka > kb : work[a] > work[b];
  });
  uint64_t load[kXcds] = {0};
  int bin[kMaxGroup];
  uint64_t total = 0;
  for (int i = 0; i < count; ++i) {
    int x = 0;
    for (int y = 1; y < kXcds; ++y)
      if (load[y] < load[x]) x = y;
    bin[slot[i]] = x;
    load[x] += work[slot[i]];
    total += work[slot[i]];
  }
  const uint64_t most = *std::max_element(load, load + kXcds);
  uint16_t order[kMaxGroup];
  uint32_t end = 0;
  int n = 0;
  tab.spread = 10 * kXcds * most > 11 * total;   // over 10% above the mean
  tab.xcd_first[0] = 0;
  for (int x = 0; x < kXcds; ++x) {
    for (int i = 0; i < count; ++i) {
      const int s = slot[i];
      if (!tab.spread && bin[s] != x) continue;
      if (tab.spread && x > 0) break;
      order[n] = tab.order[s];
      end += tiles[s];
      tab.blk_end[n] = end;
      ++n;
    }
    tab.xcd_first[x + 1] = end;
  }
  for (int i = 0; i < count; ++i) tab.order[i] = order[i];
}

unsigned xcd_grid(const uint32_t *first) {
  uint32_t most = 0;
  for (int x = 0; x < kXcds; ++x) most = std::max(most, first[x + 1] - first[x]);
  return most * kXcds;
}

// A single projection with fewer tiles than this splits K across workgroups
// (at least kSplitUnits units per slice, about kSplitTarget workgroups), as
// long as M is small enough that the slices' atomic additions into the output
// stay cheap next to the weight stream (measured: a win up to M = 256, a loss
// at M = 1800).
#ifndef BITNET_GEMM_SPLIT_BELOW
#define BITNET_GEMM_SPLIT_BELOW 256
#endif
constexpr int kSplitBelow = BITNET_GEMM_SPLIT_BELOW;
constexpr int kSplitTarget = 512;
constexpr int kSplitUnits = 6;
constexpr int kSplitMaxM = 512;

static int gemm_split_factor(int64_t M, int64_t N, int64_t K) {
  const int64_t tiles = gemm_blocks(M, N);
  if (tiles >= kSplitBelow || M > kSplitMaxM) return 1;
  const int64_t by_units = (K / kUnit) / kSplitUnits;
  const int64_t by_fill = (kSplitTarget + tiles - 1) / tiles;
  const int64_t s = std::min(by_units, by_fill);
  return s >= 2 ? (int)s : 1;
}

hipError_t launch_gemm(int M, int N, int K, const int8_t *xq_perm, const float *x_scale,
                       const int32_t *rowsum, const uint8_t *packed, const float *w_scale,
                       float *y, int32_t *acc_out, hipStream_t stream) {
  GemmProblem p{packed, xq_perm, x_scale, rowsum, w_scale, y, acc_out, M, N, K};
  const uint32_t tiles = (uint32_t)gemm_blocks(M, N);
  const int S = gemm_split_factor(M, N, K);
  if (S > 1) {
    const int64_t n = (int64_t)M * N;
    const unsigned blocks = (unsigned)((n + 255) / 256);
    zero_kernel<<<blocks, 256, 0, stream>>>(reinterpret_cast<uint32_t *>(y), n);
    switch (gemm_bm(M)) {
      case 32: gemm_split_kernel<32><<<tiles * S, kThreads, 0, stream>>>(p, S); break;
      case 64: gemm_split_kernel<64><<<tiles * S, kThreads, 0, stream>>>(p, S); break;
      default: gemm_split_kernel<128><<<tiles * S, kThreads, 0, stream>>>(p, S); break;
    }
    split_finish_kernel<<<blocks, 256, 0, stream>>>(y, M, N, x_scale, rowsum, w_scale, acc_out);
    return hipGetLastError();
  }
  uint32_t first[kXcds + 1];
  for (int x = 0; x <= kXcds; ++x) first[x] = (uint32_t)x * tiles / kXcds;
  switch (gemm_bm(M)) {
    case 32: gemm_kernel<32><<<xcd_grid(first), kThreads, 0, stream>>>(p); break;
    case 64: gemm_kernel<64><<<xcd_grid(first), kThreads, 0, stream>>>(p); break;
    default: gemm_kernel<128><<<xcd_grid(first), kThreads, 0, stream>>>(p); break;
  }
  return hipGetLastError();
}

hipError_t launch_gemm_grouped(const bitnet_problem *problems, const GroupTable &tab,
                               const uint8_t *workspace, hipStream_t stream) {
  const unsigned grid = tab.spread ? tab.blk_end[tab.count - 1] : xcd_grid(tab.xcd_first);
  switch (gemm_bm(tab.M)) {
    case 32: gemm_grouped_kernel<32><<<grid, kThreads, 0, stream>>>(problems, tab, workspace); break;
    case 64: gemm_grouped_kernel<64><<<grid, kThreads, 0, stream>>>(problems, tab, workspace); break;
    default:
      gemm_grouped_kernel<128><<<grid, kThreads, 0, stream>>>(problems, tab, workspace);
      break;
  }
  return hipGetLastError();
}

}  // namespace bitnet
