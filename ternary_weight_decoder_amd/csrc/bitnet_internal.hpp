// Host-side launchers shared between the kernel files and the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "bitnet_tm.h"

namespace bitnet {

constexpr int kMaxGroup = BITNET_MAX_GROUP;
constexpr int kXcds = 8;   // accelerator complex dies, each with its own L2

// Workspace of one problem: permuted int8 activations [M][K], fp32 scales [M],
// int32 row sums [M]; each region 256-byte aligned.
struct WsLayout {
  size_t xq, scale, rowsum, total;
};

__host__ __device__ inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

__host__ __device__ inline WsLayout ws_layout(int64_t M, int64_t K) {
  WsLayout w;
  w.xq = 0;
  w.scale = align256((size_t)(M * K));
  w.rowsum = w.scale + align256((size_t)M * 4);
  w.total = w.rowsum + align256((size_t)M * 4);
  return w;
}

// Per-launch table of a grouped call, passed by value as a kernel argument.
struct GroupTable {
  int32_t count;
  int32_t M;
  int32_t split;                 // decode only: K-split of single-row projections
  uint32_t blk_end[kMaxGroup];   // inclusive prefix sum of workgroups, in dispatch order
  uint16_t order[kMaxGroup];     // problem index of each dispatch slot
  uint32_t ws_off[kMaxGroup];    // workspace offset of each problem, in 256-byte units
  // spread == 0: the workgroups are one list in slot order, cut into kXcds
  // contiguous ranges of whole projections of about equal work; XCD x runs
  // [xcd_first[x], xcd_first[x + 1]).  spread != 0: workgroup b runs entry b.
  int32_t spread;
  uint32_t xcd_first[kXcds + 1];
};

// Per-launch table of a grouped quantization: workgroups [wg_end[s-1], wg_end[s])
// quantize the rows of problem order[s].
struct QuantTable {
  int32_t count;
  int32_t M;
  uint32_t wg_end[kMaxGroup];
  uint16_t order[kMaxGroup];
  uint32_t ws_off[kMaxGroup];
};

// Per-launch table of a staged decode launch: problem i owns tiles
// [blk_end[i-1], blk_end[i]) of one list in problem (= stage) order, each tile
// one workgroup whose waves share 4 / split[i] 16-column blocks and split
// their K units split[i] ways.  src[i]: the earlier problem whose output is
// problem i's x, or -1 for an input written before the call.  tag_off[i]:
// workspace offset (256-byte units) of problem i's tagged outputs, kNoTag if
// no later problem reads them.
constexpr int kMaxStages = BITNET_MAX_STAGES;
constexpr size_t kStageHeaderBytes = 256;   // [0] epoch, [1] timeout flag
constexpr uint32_t kNoTag = 0xffffffffu;
constexpr int kMaxStageGrid = 2048;   // workgroups of one staged launch
struct StageTable {
  int32_t count;
  int32_t M;
  uint32_t ntiles;
  uint32_t blk_end[kMaxGroup];
  uint32_t tag_off[kMaxGroup];
  int16_t src[kMaxGroup];
  uint8_t split[kMaxGroup];
};

// Dispatch slot of workgroup b in a grouped launch (binary search over the
// block ranges; the index is uniform, so the table is read through the scalar
// cache), the first workgroup of that slot and its problem index.
struct SlotInfo {
  int slot;
  uint32_t first;
  int problem;
};

__device__ __forceinline__ SlotInfo find_slot(const GroupTable &tab, uint32_t b) {
  int lo = 0, hi = tab.count - 1;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (b < tab.blk_end[mid]) hi = mid; else lo = mid + 1;
  }
  return SlotInfo{lo, lo ? tab.blk_end[lo - 1] : 0u, (int)tab.order[lo]};
}

// ternarize.hip
hipError_t launch_ternarize_pack(const float *W, int N, int K, uint8_t *packed, float *w_scale,
                                 double *rowsums, hipStream_t stream);

// quant.hip
hipError_t launch_quant_rows(const float *x, int M, int K, int8_t *xq_nat, int8_t *xq_perm,
                             float *x_scale, float *x_scale2, int32_t *rowsum,
                             hipStream_t stream);
hipError_t launch_permute_q8(const int8_t *xq, const float *x_scale_in, int M, int K,
                             int8_t *xq_perm, float *x_scale, int32_t *rowsum,
                             hipStream_t stream);
int64_t quant_grouped_blocks(int64_t M, int64_t K);
hipError_t launch_quant_grouped(const bitnet_problem *problems, const QuantTable &tab,
                                uint8_t *workspace, hipStream_t stream);

// gemv.hip  (M <= 16)
constexpr int kGemvMaxM = 16;
// Largest M*K whose int8 rows the decode kernel quantizes into LDS itself
// (one row of the longest projection).  Beyond it a separate quantization
// launch and staged rows are faster: per-workgroup quantization of several
// long rows costs more than it saves, and its LDS limits occupancy.
#ifndef BITNET_GEMV_FUSED_MAX
#define BITNET_GEMV_FUSED_MAX 8960
#endif
constexpr int64_t kGemvFusedLdsBytes = BITNET_GEMV_FUSED_MAX;
hipError_t launch_gemv(int M, int N, int K, const int8_t *xq_perm, const float *x_scale,
                       const int32_t *rowsum, const uint8_t *packed, const float *w_scale,
                       float *y, int32_t *acc_out, hipStream_t stream);
hipError_t launch_gemv_fused(int M, int N, int K, const float *x, const uint8_t *packed,
                             const float *w_scale, float *y, int8_t *xq_out,
                             float *x_scale_out, int32_t *acc_out, hipStream_t stream);
// K-split of the single-row decode kernel in small launches: with fewer than
// kGemvSplitBelow workgroups the chip is not filled, and a long-K projection's
// waves are latency-bound chains, so the waves of a workgroup then share one
// 64-column tile and split its K units (at least kGemvUnitsPerWave each).
#ifndef BITNET_GEMV_SPLIT_BELOW
#define BITNET_GEMV_SPLIT_BELOW 512
#endif
#ifndef BITNET_GEMV_UNITS_PER_WAVE
#define BITNET_GEMV_UNITS_PER_WAVE 6
#endif
constexpr int kGemvSplitBelow = BITNET_GEMV_SPLIT_BELOW;
__host__ __device__ inline int gemv_split(int units, bool split) {
  if (!split) return 1;
  const int s = units / BITNET_GEMV_UNITS_PER_WAVE;
  return s >= 4 ? 4 : s >= 2 ? 2 : 1;
}
int gemv_blocks(int64_t N, int64_t K, bool split);
bool gemv_fusable(int64_t M, int64_t K);
hipError_t launch_gemv_grouped(const bitnet_problem *problems, const GroupTable &tab,
                               const uint8_t *workspace, bool fused, int64_t kmax,
                               hipStream_t stream);

// stages.hip: dependent decode stages in one cooperative launch.  src[i]: the
// earlier problem whose y is problem i's x, or -1.  ws: the workspace
// (stages_workspace_bytes), zero-filled before its first use.
size_t stages_workspace_bytes(int64_t M, const bitnet_problem *problems_host, int count);
hipError_t launch_stages(const bitnet_problem *problems_dev, const bitnet_problem *problems_host,
                         int count, const int32_t *stage_end, int nstages, int M,
                         const int16_t *src, uint8_t *ws, hipStream_t stream);

// gemm.hip  (M > 16)
hipError_t launch_gemm(int M, int N, int K, const int8_t *xq_perm, const float *x_scale,
                       const int32_t *rowsum, const uint8_t *packed, const float *w_scale,
                       float *y, int32_t *acc_out, hipStream_t stream);
int gemm_blocks(int64_t M, int64_t N);
// Prefill launch schedule: reorders the slots (tab.order, tab.blk_end) and
// fills tab.spread / tab.xcd_first.
// Deal whole projections to the XCDs (sets tab.order, blk_end, spread and
// xcd_first); tiles[s] = workgroups of dispatch slot s in the current order.
void xcd_schedule(GroupTable &tab, const bitnet_problem *problems_host, const uint32_t *tiles);
// Grid of an XCD-scheduled launch: eight times the largest per-XCD range.
unsigned xcd_grid(const uint32_t *first);
hipError_t launch_gemm_grouped(const bitnet_problem *problems, const GroupTable &tab,
                               const uint8_t *workspace, hipStream_t stream);

}  // namespace bitnet
