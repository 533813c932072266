// Staged decode: a sequence of dependent single-token projection stages in one
// cooperative launch.
//
// Per token the decoder streams all of its ternary weights (blog "The Paper
// Says ARM Support...", section "What the model is trying to do"), and its
// projections depend on each other: q,k,v read the layer input, o reads the
// attention output, gate and up read o's, down reads the MLP product, and the
// next layer reads down's.  Each stage is small (0.6 to 7 MB of codes), so
// its time is memory latency, not bandwidth: the tile shape here is chosen for
// one round trip per stage, not for streaming.
//
// Tile = one workgroup of 4 waves.  A wave owns one 16-column block and
// kq-th of its K units when the block's K is split S ways (S = 1, 2, 4 per
// problem, chosen on the host so that each stage fills the chip without a
// workgroup taking two tiles); the 4/S blocks of a tile are adjacent.  Every
// weight load of the wave (at most kStageItems units of 512 bytes per wave)
// is issued before the wave waits for its activations, so weight latency
// overlaps the wait.  The activation rows are read once into registers,
// quantized (absmax scale, round half to even, clamp to 127) into LDS in the
// permuted order, and contracted with v_mfma_i32_16x16x64_i8 on the field
// values u = code + 1; the epilogue subtracts the activation row sum and
// dequantizes exactly (acc * w_scale / x_scale in fp64, rounded to fp32).
//
// Dataflow between stages, without a device-wide barrier: a problem whose
// output a later stage reads also writes each output as a 64-bit pair (value
// bits, call epoch) into the workspace with one device-scope store, and the
// consumer reads those pairs with device-coherent loads, re-reading the ones
// whose tag is not yet the current epoch.  A single atomic store carries value
// and tag together, so no fence, flag or store acknowledgement sits between a
// producer and its consumers.  A consumer first polls one probe pair (the
// first one, written by the producer's first tile) so that waiting workgroups
// do not flood the memory system, then reads everything and re-reads what is
// still pending; the producer's tiles finish close together, so the full read
// mostly overlaps the last of them.  Each workgroup runs its
// tiles in stage order and the grid is co-resident, so the lowest unfinished
// tile never waits on an unfinished one.  Every wait is bounded by a
// wall-clock timeout: a wait that runs out raises the flag in workspace word 1
// instead of hanging, later waits return at once, and the outputs are then
// not valid.  The epoch (workspace word 0) is advanced by a one-thread kernel
// before each launch.
#include <algorithm>
#include <cstring>

#include "bitnet_device.hpp"
#include "bitnet_internal.hpp"

namespace bitnet {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kStageWaves = kWaves;
constexpr int kStageItems = 18;    // K units per wave: ceil(70 / 4) for K <= 8960
constexpr int kStageXVec = (int)((kGemvFusedLdsBytes / 4 + kThreads - 1) / kThreads);
constexpr int kWeightAux = 2;      // weights are read once: non-temporal

struct StageShared {
  __attribute__((aligned(16))) int8_t xq[kGemvFusedLdsBytes];   // permuted rows [M][K]
  v4i part[kStageWaves - 1][64];                                 // K-split partials
  float red[kGemvMaxM][kWaves];
  int ired[kGemvMaxM][kWaves];
  float scale[kGemvMaxM];
};

// Where a tile reads its activations and writes its tagged outputs.
struct StageIo {
  const uint64_t *x_tagged;   // producer's (value, epoch) pairs, or null: read x
  uint64_t *y_tagged;         // this problem's pairs, or null: no later reader
  uint32_t epoch;
  uint32_t *flags;            // workspace words: [0] epoch, [1] timeout flag, [2] timeout count
  uint64_t timeout;           // wall-clock ticks per wait
};

__device__ __forceinline__ uint32_t ld_agent(const uint32_t *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wave-wide max / sum with DPP row operations (lane 63 collects the result):
// swaps within quads, mirrors within 8 and 16 lanes, then row broadcasts of
// lanes 15 and 31.  Max is taken over non-negative values.
template <typename Op>
__device__ __forceinline__ int wave_reduce_dpp(int v, Op op) {
  v = op(v, __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false));    // quad_perm 1,0,3,2
  v = op(v, __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false));    // quad_perm 2,3,0,1
  v = op(v, __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false));   // row_half_mirror
  v = op(v, __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false));   // row_mirror
  v = op(v, __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false));   // row_bcast:15
  v = op(v, __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false));   // row_bcast:31
  return __builtin_amdgcn_readlane(v, 63);
}
__device__ __forceinline__ float wave_absmax_dpp(float a) {
  return __builtin_bit_cast(float, wave_reduce_dpp(__builtin_bit_cast(int, a), [](int x, int y) {
    return __builtin_bit_cast(int, fmaxf(__builtin_bit_cast(float, x), __builtin_bit_cast(float, y)));
  }));
}
__device__ __forceinline__ int wave_sum_dpp(int v) {
  return wave_reduce_dpp(v, [](int x, int y) { return x + y; });
}

// Pair i of a tagged array (uniform base, 32-bit element offset).
__device__ __forceinline__ uint64_t ld_pair(const uint64_t *base, uint32_t i) {
  const BITNET_GLOBAL uint64_t *p =
      (const BITNET_GLOBAL uint64_t *)((const BITNET_GLOBAL char *)base + (size_t)(i * 8u));
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool pair_ok(uint64_t q, uint32_t epoch) {
  return (uint32_t)(q >> 32) == epoch;
}

// Read vector e (4 activations) of every thread's share of the M x K block
// into v[]: directly from x, or from the producer's tagged pairs (one 64-bit
// atomic load per pair), waiting until every pair carries the current epoch.
// A wait ran past its bound: raise this call's flag (word 1) and, the first
// time in the call, count the call in word 2, which nothing clears (so the
// count covers every call since the workspace was zero-filled).
__device__ __forceinline__ void note_timeout(uint32_t *flags) {
  if (atomicOr(&flags[1], 1u) == 0u) atomicAdd(&flags[2], 1u);
}

__device__ __forceinline__ void stage_load_x(const float *x, const StageIo &io, int total,
                                             f32x4 (&v)[kStageXVec]) {
  const int tid = threadIdx.x;
  if (io.x_tagged == nullptr) {
    const uint32_t bytes = (uint32_t)total * 16;
    const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(x, bytes);
#pragma unroll
    for (int j = 0; j < kStageXVec; ++j) {
      const int e = tid + j * kThreads;
      const uint32_t off = e < total ? (uint32_t)e * 16 : bytes;
      v[j] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, off, 0, 0));
    }
    return;
  }
  const uint64_t *xt = io.x_tagged;
  bool expired = ld_agent(&io.flags[1]) != 0;
  uint64_t t0 = wall_clock64();
  // Probe: poll the first pair (written by the producer's first tile) first.
  while (!expired && !pair_ok(ld_pair(xt, 0u), io.epoch)) {
    if (wall_clock64() - t0 > io.timeout) {
      note_timeout(io.flags);
      expired = true;
    }
    __builtin_amdgcn_s_sleep(2);
  }
  // Vectors past the block re-read the last one (in range) and are ignored.
  uint64_t q[kStageXVec][4];
  uint32_t pending = 0;
#pragma unroll
  for (int j = 0; j < kStageXVec; ++j) {
    const int e = tid + j * kThreads;
    const uint32_t ev = (uint32_t)(e < total ? e : total - 1);
#pragma unroll
    for (int c = 0; c < 4; ++c) q[j][c] = ld_pair(xt, 4u * ev + c);
  }
#pragma unroll
  for (int j = 0; j < kStageXVec; ++j) {
    if (tid + j * kThreads < total &&
        !(pair_ok(q[j][0], io.epoch) && pair_ok(q[j][1], io.epoch) &&
          pair_ok(q[j][2], io.epoch) && pair_ok(q[j][3], io.epoch)))
      pending |= 1u << j;
  }
  t0 = wall_clock64();
  while (pending != 0 && !expired) {
    __builtin_amdgcn_s_sleep(2);
#pragma unroll
    for (int j = 0; j < kStageXVec; ++j) {
      if ((pending >> j) & 1u) {
        const int e = tid + j * kThreads;
#pragma unroll
        for (int c = 0; c < 4; ++c) q[j][c] = ld_pair(xt, 4u * e + c);
        if (pair_ok(q[j][0], io.epoch) && pair_ok(q[j][1], io.epoch) &&
            pair_ok(q[j][2], io.epoch) && pair_ok(q[j][3], io.epoch))
          pending &= ~(1u << j);
      }
    }
    if (pending != 0 && wall_clock64() - t0 > io.timeout) {
      note_timeout(io.flags);
      expired = true;
    }
  }
#pragma unroll
  for (int j = 0; j < kStageXVec; ++j)
    v[j] = f32x4{__builtin_bit_cast(float, (uint32_t)q[j][0]),
                 __builtin_bit_cast(float, (uint32_t)q[j][1]),
                 __builtin_bit_cast(float, (uint32_t)q[j][2]),
                 __builtin_bit_cast(float, (uint32_t)q[j][3])};
}

// The M rows of x (M * K <= kGemvFusedLdsBytes) into LDS as permuted int8,
// with per-row scales and per-wave row-sum partials.  Element vector e (4
// floats) of the flattened rows is held by thread e % 256 in register e / 256,
// so the whole activation block is read in one round of loads.  ONE_ROW: M = 1.
template <bool ONE_ROW>
__device__ __forceinline__ void stage_quant(const float *x, const StageIo &io, int M_, int K,
                                            StageShared &sh) {
  const int M = ONE_ROW ? 1 : M_;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n4 = K >> 2, total = M * n4;
  f32x4 v[kStageXVec];
  stage_load_x(x, io, total, v);
  int row[kStageXVec];
#pragma unroll
  for (int j = 0; j < kStageXVec; ++j) {
    const int e = tid + j * kThreads;
    row[j] = e < total ? (ONE_ROW ? 0 : e / n4) : -1;
  }
  for (int m = 0; m < M; ++m) {
    float a = 0.0f;
#pragma unroll
    for (int j = 0; j < kStageXVec; ++j) {
      if (row[j] == m)
        a = fmaxf(a, fmaxf(fmaxf(fabsf(v[j].x), fabsf(v[j].y)),
                           fmaxf(fabsf(v[j].z), fabsf(v[j].w))));
    }
    a = wave_absmax_dpp(a);
    if (lane == 0) sh.red[m][wave] = a;
  }
  __syncthreads();
  // Every thread derives the scales of the rows it holds; thread m < M also
  // publishes row m's scale for the epilogue (read after the next barrier).
  int qsum[kStageXVec];
#pragma unroll
  for (int j = 0; j < kStageXVec; ++j) {
    qsum[j] = 0;
    if (row[j] >= 0) {
      const int r = row[j];
      const float a = fmaxf(fmaxf(sh.red[r][0], sh.red[r][1]), fmaxf(sh.red[r][2], sh.red[r][3]));
      const float s = (a == 0.0f) ? 1.0f : 127.0f / a;
      const int q0 = quant_one(v[j].x, s), q1 = quant_one(v[j].y, s);
      const int q2 = quant_one(v[j].z, s), q3 = quant_one(v[j].w, s);
      qsum[j] = q0 + q1 + q2 + q3;
      const int i = tid + j * kThreads - r * n4;   // vector within the row
      *reinterpret_cast<uint32_t *>(sh.xq + r * K + perm_offset(4 * i)) = pack4_i8(q0, q1, q2, q3);
    }
  }
  if (tid < M) {
    const float a = fmaxf(fmaxf(sh.red[tid][0], sh.red[tid][1]),
                          fmaxf(sh.red[tid][2], sh.red[tid][3]));
    sh.scale[tid] = (a == 0.0f) ? 1.0f : 127.0f / a;
  }
  for (int m = 0; m < M; ++m) {
    int sum = 0;
#pragma unroll
    for (int j = 0; j < kStageXVec; ++j) sum += row[j] == m ? qsum[j] : 0;
    sum = wave_sum_dpp(sum);
    if (lane == 0) sh.ired[m][wave] = sum;
  }
  __syncthreads();
}

// Tile `tile` of problem pr with K-split S; NI >= the units of any wave.
template <int NI, bool ONE_ROW>
__device__ __forceinline__ void stage_tile(const bitnet_problem &pr, int M_, int tile, int S,
                                           StageShared &sh, const StageIo &io) {
  const int M = ONE_ROW ? 1 : M_;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, h = lane >> 4;
  const int N = (int)pr.N, K = (int)pr.K, U = K >> 7;
  const int G4 = kStageWaves / S, cgrp = wave % G4, kq = wave / G4;
  const int u0 = kq * U / S, units = (kq + 1) * U / S - u0;   // 1 <= units <= NI
  const int n = (tile * G4 + cgrp) * 16 + col;

  // Items past the wave's units are aimed past the buffer: they load zeros
  // without a memory access, and their MFMAs add nothing.
  const uint32_t w_bytes = (uint32_t)((size_t)N * K / 4);
  const __amdgpu_buffer_rsrc_t w_rsrc = make_rsrc(pr.packed, w_bytes);
  const uint32_t ustride = (uint32_t)N * kUnitBytes;
  u32x2 wr[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const uint32_t off = (i < units && n < N)
                             ? (uint32_t)(u0 + i) * ustride + (uint32_t)n * kUnitBytes + 8 * h
                             : w_bytes;
    wr[i] = __builtin_amdgcn_raw_buffer_load_b64(w_rsrc, off, 0, kWeightAux);
  }

  stage_quant<ONE_ROW>(pr.x, io, M, K, sh);

  // Four independent accumulation chains (item i feeds chain i % 4), so the
  // MFMAs of consecutive items do not wait for each other.
  constexpr int kChains = NI < 4 ? NI : 4;
  const v4i zero4 = v4i{0, 0, 0, 0};
  v4i accs[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) accs[c] = zero4;
  const bool a_live = col < M;
  const int8_t *arow = sh.xq + (a_live ? col : 0) * K + 32 * h;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int ui = u0 + (i < units ? i : units - 1);   // in range; codes are zero past units
    v4i a0 = zero4, a1 = zero4;
    if (a_live) {
      const v4i *ap = reinterpret_cast<const v4i *>(arow + ui * kUnit);
      a0 = ap[0];
      a1 = ap[1];
    }
    v4i &acc = accs[i % kChains];
    acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, unpack_fields(wr[i].x), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, unpack_fields(wr[i].y), acc, 0, 0, 0);
  }
  v4i acc = accs[0];
#pragma unroll
  for (int c = 1; c < kChains; ++c) acc += accs[c];

  if (S > 1) {
    if (kq > 0) sh.part[(kq - 1) * G4 + cgrp][lane] = acc;
    __syncthreads();
    if (kq > 0) return;
    for (int q = 1; q < S; ++q) acc += sh.part[(q - 1) * G4 + cgrp][lane];
  }

  // Element (row 4h + r, column col) of the 16-column block.
  const float ws = ld_global<float>(pr.w_scale);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int rw = 4 * h + r;
    if (rw < M && n < N) {
      const int rowsum = sh.ired[rw][0] + sh.ired[rw][1] + sh.ired[rw][2] + sh.ired[rw][3];
      const float y = dequant_exact(acc[r] - rowsum, ws, sh.scale[rw]);
      const size_t idx = (size_t)rw * N + n;
      st_global<float>(pr.y + idx, y);
      if (io.y_tagged)
        __hip_atomic_store((BITNET_GLOBAL uint64_t *)(io.y_tagged + idx),
                           (uint64_t)__builtin_bit_cast(uint32_t, y) | ((uint64_t)io.epoch << 32),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// The tile routine for the largest per-wave unit count ni of the tile.
template <bool ONE_ROW>
__device__ __forceinline__ void stage_tile_any(int ni, const bitnet_problem &pr, int M, int tile,
                                               int S, StageShared &sh, const StageIo &io) {
  if (ni <= 3)
    stage_tile<3, ONE_ROW>(pr, M, tile, S, sh, io);
  else if (ni <= 6)
    stage_tile<6, ONE_ROW>(pr, M, tile, S, sh, io);
  else if (ni <= 12)
    stage_tile<12, ONE_ROW>(pr, M, tile, S, sh, io);
  else
    stage_tile<kStageItems, ONE_ROW>(pr, M, tile, S, sh, io);
}

// Workgroup b runs tiles b, b + G, ... (G = grid size) in order; tiles are
// numbered problem by problem, and problems come in stage order.
__global__ void __launch_bounds__(kThreads, 2)
    stages_kernel(const bitnet_problem *__restrict__ problems, StageTable tab,
                  uint8_t *__restrict__ ws, uint64_t timeout) {
  __shared__ StageShared sh;
  StageIo io;
  io.flags = reinterpret_cast<uint32_t *>(ws);
  io.epoch = ld_agent(&io.flags[0]);
  io.timeout = timeout;
  for (uint32_t t = blockIdx.x; t < tab.ntiles; t += gridDim.x) {
    int lo = 0, hi = tab.count - 1;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (t < tab.blk_end[mid]) hi = mid; else lo = mid + 1;
    }
    const bitnet_problem pr = problems[lo];
    const int tile = (int)(t - (lo ? tab.blk_end[lo - 1] : 0u));
    const int src = tab.src[lo];
    io.x_tagged = src >= 0 ? reinterpret_cast<const uint64_t *>(ws + (size_t)tab.tag_off[src] * 256)
                           : nullptr;
    io.y_tagged = tab.tag_off[lo] != kNoTag
                      ? reinterpret_cast<uint64_t *>(ws + (size_t)tab.tag_off[lo] * 256)
                      : nullptr;
    const int S = (int)tab.split[lo];
    const int ni = ((int)(pr.K >> 7) + S - 1) / S;
    // Every wave is done with the previous tile's LDS before this one starts.
    __syncthreads();
    if (tab.M == 1)
      stage_tile_any<true>(ni, pr, 1, tile, S, sh, io);
    else
      stage_tile_any<false>(ni, pr, tab.M, tile, S, sh, io);
  }
}

// Advance the call epoch (never 0, the value of a zero-filled workspace) and
// clear the timeout flag.
__global__ void stage_epoch_kernel(uint32_t *__restrict__ w) {
  if (threadIdx.x == 0) {
    uint32_t e = w[0] + 1u;
    w[0] = e == 0u ? 1u : e;
    w[1] = 0u;
  }
}

// Tiles of one problem at K-split S.
int64_t stage_tiles(int64_t N, int S) {
  const int64_t blocks = (N + 15) / 16;
  const int64_t per = kStageWaves / S;
  return (blocks + per - 1) / per;
}

// K-split of a problem for a stage-wide choice S: at least what keeps a
// wave's units within kStageItems, at most what leaves every wave a unit.
int problem_split(int64_t K, int S) {
  const int64_t U = K >> 7;
  const int need = U <= kStageItems ? 1 : U <= 2 * kStageItems ? 2 : 4;
  const int most = U >= 4 ? 4 : U >= 2 ? 2 : 1;
  return std::max(need, std::min(S, most));
}

}  // namespace

size_t stages_workspace_bytes(int64_t M, const bitnet_problem *problems_host, int count) {
  size_t total = kStageHeaderBytes;
  for (int i = 0; i < count; ++i) total += align256((size_t)(M * problems_host[i].N) * 8);
  return total;
}

hipError_t launch_stages(const bitnet_problem *problems_dev, const bitnet_problem *problems_host,
                         int count, const int32_t *stage_end, int nstages, int M,
                         const int16_t *src, uint8_t *ws, hipStream_t stream) {
  int dev = 0, per_cu = 0, cus = 0, clock_khz = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&clock_khz, hipDeviceAttributeWallClockRate, dev);
  if (e != hipSuccess) return e;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, stages_kernel, kThreads, 0);
  if (e != hipSuccess) return e;
  if (per_cu < 1 || cus < 1) return hipErrorInvalidConfiguration;

  StageTable tab;
  std::memset(&tab, 0, sizeof(tab));
  tab.count = count;
  tab.M = M;
  // Tagged outputs: only for problems that a later one reads.
  bool consumed[kMaxGroup] = {};
  for (int i = 0; i < count; ++i)
    if (src[i] >= 0) consumed[src[i]] = true;
  size_t off = kStageHeaderBytes;
  for (int i = 0; i < count; ++i) {
    tab.src[i] = src[i];
    tab.tag_off[i] = consumed[i] ? (uint32_t)(off / 256) : kNoTag;
    off += align256((size_t)((int64_t)M * problems_host[i].N) * 8);
  }
  // Per stage, the largest K-split (more, shorter waves) whose tiles still fit
  // the resident grid at once; if none fits, the smallest.
  const int64_t resident = std::min<int64_t>((int64_t)per_cu * cus, kMaxStageGrid);
  int64_t total = 0;
  int first = 0;
  for (int s = 0; s < nstages; ++s) {
    const int last = stage_end[s];
    int chosen = 1;
    for (int S : {4, 2, 1}) {
      int64_t tiles = 0;
      for (int i = first; i < last; ++i)
        tiles += stage_tiles(problems_host[i].N, problem_split(problems_host[i].K, S));
      chosen = S;
      if (tiles <= resident) break;
    }
    for (int i = first; i < last; ++i) {
      const int Si = problem_split(problems_host[i].K, chosen);
      tab.split[i] = (uint8_t)Si;
      total += stage_tiles(problems_host[i].N, Si);
      if (total >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
      tab.blk_end[i] = (uint32_t)total;
    }
    first = last;
  }
  tab.ntiles = (uint32_t)total;
  // As many workgroups as can be resident: a workgroup that finishes early
  // starts its next tile's weight loads while that tile's inputs are made.
  const unsigned grid = (unsigned)std::min<int64_t>(resident, total);
  // Bound each wait at 200 ms of the wall clock.
  uint64_t timeout = (uint64_t)std::max(clock_khz, 1) * 200u;
  stage_epoch_kernel<<<1, 64, 0, stream>>>(reinterpret_cast<uint32_t *>(ws));
  void *args[] = {(void *)&problems_dev, (void *)&tab, (void *)&ws, (void *)&timeout};
  return hipLaunchCooperativeKernel((const void *)stages_kernel, dim3(grid), dim3(kThreads), args,
                                    0, stream);
}

}  // namespace bitnet
