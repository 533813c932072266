// C ABI of the ternary projection library: argument checks, workspace layout
// and dispatch to the gfx950 kernels.  Nothing is launched unless every check
// passes; no device memory is allocated here.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstring>
#include <mutex>
#include <utility>

#include "bitnet_internal.hpp"
#include "bitnet_variants.hpp"
#include "bitnet_tm.h"

using namespace bitnet;

// Built-in workspace of bitnet_ternary_matmul_noalloc, for callers that cannot
// allocate.  Every device the library runs on holds its own copy from module
// load until the process ends.  In host code `scratch` only names the symbol:
// its device address on the current device comes from hipGetSymbolAddress,
// looked up once per device (scratch_address) and passed to the kernels.
static __device__ __align__(256) uint8_t scratch[BITNET_SCRATCH_BYTES];

namespace {

constexpr int64_t kLimit = (int64_t)1 << 31;  // M*K, N*K, M*N must stay below this

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

bool shape_ok(int64_t M, int64_t N, int64_t K) {
  if (M < 1 || N < 1 || K < 1) return false;
  if (K % 128 != 0) return false;  // 128 codes per packing unit
  if (M >= kLimit || N >= kLimit || K >= kLimit) return false;
  if (M * K >= kLimit || N * K >= kLimit || M * N >= kLimit) return false;
  // Byte offsets of the fp32 output, including a 128-row tile past M, stay 32-bit.
  if ((M + 128) * N * 4 >= kLimit) return false;
  return true;
}

// Per-device record of the architecture check: 0 unknown, 1 gfx950, 2 other.
constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_ok[kMaxDevices];

bitnet_status device_check() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return BITNET_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return BITNET_ERR_DEVICE;
  int v = g_arch_ok[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return BITNET_ERR_HIP;
    v = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_arch_ok[dev].store(v, std::memory_order_relaxed);
  }
  return v == 1 ? BITNET_OK : BITNET_ERR_DEVICE;
}

bitnet_status from_hip(hipError_t e) { return e == hipSuccess ? BITNET_OK : BITNET_ERR_HIP; }

// Device address of `scratch` on each device (see its definition above).
constexpr size_t kScratchBytes = BITNET_SCRATCH_BYTES;
std::atomic<void *> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

bitnet_status scratch_address(void **out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return BITNET_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return BITNET_ERR_DEVICE;
  void *p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return BITNET_ERR_HIP;
      if (!aligned(p, 256)) return BITNET_ERR_HIP;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return BITNET_OK;
}

hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

bitnet_status check_problem(int64_t M, const bitnet_problem &p) {
  if (!p.x || !p.packed || !p.w_scale || !p.y) return BITNET_ERR_NULL;
  if (!shape_ok(M, p.N, p.K)) return BITNET_ERR_SHAPE;
  if (!aligned(p.x, 16) || !aligned(p.packed, 16) || !aligned(p.w_scale, 4) ||
      !aligned(p.y, 4))
    return BITNET_ERR_ALIGN;
  return BITNET_OK;
}

// owner[i]: the lowest index of the problems with the same x and K as
// problem i (i itself when there is none).  Such problems read the same rows,
// so they share one quantized copy: a decoder's q, k and v read one input, as
// do its gate and up.  count <= kMaxGroup.
void input_owners(const bitnet_problem *ph, int32_t count, int32_t *owner) {
  int32_t ix[kMaxGroup];
  for (int32_t i = 0; i < count; ++i) ix[i] = i;
  const auto key = [&](int32_t i) {
    return std::make_pair(reinterpret_cast<uintptr_t>(ph[i].x), ph[i].K);
  };
  std::sort(ix, ix + count, [&](int32_t a, int32_t b) {
    return key(a) != key(b) ? key(a) < key(b) : a < b;
  });
  for (int32_t r = 0; r < count;) {
    int32_t e = r;
    while (e < count && key(ix[e]) == key(ix[r])) owner[ix[e++]] = ix[r];
    r = e;
  }
}

// Workspace offsets (256-byte units) of each problem of a group; problems that
// share their input share its region.  count <= kMaxGroup.
size_t group_ws(int64_t M, const bitnet_problem *ph, int32_t count, uint32_t *off,
                int32_t *owner_out = nullptr) {
  int32_t owner_buf[kMaxGroup];
  int32_t *owner = owner_out ? owner_out : owner_buf;
  input_owners(ph, count, owner);
  uint32_t own[kMaxGroup];
  size_t total = 0;
  for (int32_t i = 0; i < count; ++i) {
    if (owner[i] == i) {
      own[i] = (uint32_t)(total / 256);
      total += align256(ws_layout(M, ph[i].K).total);
    } else {
      own[i] = own[owner[i]];
    }
    if (off) off[i] = own[i];
  }
  return total;
}

}  // namespace

extern "C" {

const char *bitnet_status_string(bitnet_status s) {
  switch (s) {
    case BITNET_OK: return "ok";
    case BITNET_ERR_NULL: return "required pointer is NULL";
    case BITNET_ERR_SHAPE: return "shape out of range (M,N,K >= 1, K % 128 == 0, products < 2^31)";
    case BITNET_ERR_ALIGN: return "pointer not aligned as required";
    case BITNET_ERR_WORKSPACE: return "workspace missing or too small";
    case BITNET_ERR_HIP: return "HIP runtime or launch error";
    case BITNET_ERR_DEVICE: return "current device is not a gfx950";
    case BITNET_ERR_ALIAS: return "outputs overlap each other or an input";
    case BITNET_ERR_SCRATCH:
      return "problem needs more workspace than the built-in scratch (bitnet_scratch_bytes())";
    default: return "unknown status";
  }
}

size_t bitnet_packed_bytes(int64_t N, int64_t K) {
  if (N < 1 || K < 1) return 0;
  return (size_t)(N * K / 4);
}

size_t bitnet_ternarize_workspace_bytes(int64_t N) {
  if (N < 1) return 0;
  return (size_t)N * sizeof(double);
}

bitnet_status bitnet_ternarize_pack(const float *W, int64_t N, int64_t K, uint8_t *packed,
                                    float *w_scale, void *workspace, size_t workspace_bytes,
                                    void *stream) {
  if (!W || !packed || !w_scale) return BITNET_ERR_NULL;
  if (!shape_ok(1, N, K)) return BITNET_ERR_SHAPE;
  if (!aligned(W, 16) || !aligned(packed, 16) || !aligned(w_scale, 4)) return BITNET_ERR_ALIGN;
  if (!workspace || workspace_bytes < bitnet_ternarize_workspace_bytes(N))
    return BITNET_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return BITNET_ERR_ALIGN;
  bitnet_status st = device_check();
  if (st != BITNET_OK) return st;
  return from_hip(launch_ternarize_pack(W, (int)N, (int)K, packed, w_scale,
                                        reinterpret_cast<double *>(workspace),
                                        as_stream(stream)));
}

bitnet_status bitnet_quant_act(const float *x, int64_t M, int64_t K, int8_t *xq,
                               float *x_scale, void *stream) {
  if (!x || !xq || !x_scale) return BITNET_ERR_NULL;
  if (!shape_ok(M, 1, K)) return BITNET_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(xq, 16) || !aligned(x_scale, 4)) return BITNET_ERR_ALIGN;
  bitnet_status st = device_check();
  if (st != BITNET_OK) return st;
  return from_hip(launch_quant_rows(x, (int)M, (int)K, xq, nullptr, x_scale, nullptr, nullptr,
                                    as_stream(stream)));
}

size_t bitnet_matmul_workspace_bytes(int64_t M, int64_t K) {
  if (M < 1 || K < 1) return 0;
  return ws_layout(M, K).total;
}

static bitnet_status matmul_from_ws(int64_t M, int64_t N, int64_t K, const uint8_t *packed,
                                    const float *w_scale, float *y, uint8_t *ws,
                                    int32_t *acc_out, hipStream_t s) {
  const WsLayout L = ws_layout(M, K);
  const int8_t *xqp = reinterpret_cast<const int8_t *>(ws + L.xq);
  const float *xs = reinterpret_cast<const float *>(ws + L.scale);
  const int32_t *rs = reinterpret_cast<const int32_t *>(ws + L.rowsum);
  if (M <= kGemvMaxM)
    return from_hip(launch_gemv((int)M, (int)N, (int)K, xqp, xs, rs, packed, w_scale, y,
                                acc_out, s));
  return from_hip(
      launch_gemm((int)M, (int)N, (int)K, xqp, xs, rs, packed, w_scale, y, acc_out, s));
}

// Argument checks of the single projection, apart from the workspace.
static bitnet_status matmul_args_ok(int64_t M, int64_t N, int64_t K, const float *x,
                                    const uint8_t *packed, const float *w_scale, float *y,
                                    int8_t *xq_out, float *x_scale_out, int32_t *acc_out) {
  if (!x || !packed || !w_scale || !y) return BITNET_ERR_NULL;
  if (!shape_ok(M, N, K)) return BITNET_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(packed, 16) || !aligned(w_scale, 4) || !aligned(y, 4) ||
      (xq_out && !aligned(xq_out, 16)) || (x_scale_out && !aligned(x_scale_out, 4)) ||
      (acc_out && !aligned(acc_out, 4)))
    return BITNET_ERR_ALIGN;
  return BITNET_OK;
}

// The single projection once its arguments are checked; `workspace` holds at
// least bitnet_matmul_workspace_bytes(M, K) bytes, 256-byte aligned.
static bitnet_status matmul_run(int64_t M, int64_t N, int64_t K, const float *x,
                                const uint8_t *packed, const float *w_scale, float *y,
                                void *workspace, int8_t *xq_out, float *x_scale_out,
                                int32_t *acc_out, hipStream_t s) {
  bitnet_status st;
  if (M <= kGemvMaxM && gemv_fusable(M, K))
    return from_hip(launch_gemv_fused((int)M, (int)N, (int)K, x, packed, w_scale, y, xq_out,
                                      x_scale_out, acc_out, s));
  uint8_t *ws = reinterpret_cast<uint8_t *>(workspace);
  const WsLayout L = ws_layout(M, K);
  st = from_hip(launch_quant_rows(x, (int)M, (int)K, xq_out,
                                  reinterpret_cast<int8_t *>(ws + L.xq),
                                  reinterpret_cast<float *>(ws + L.scale), x_scale_out,
                                  reinterpret_cast<int32_t *>(ws + L.rowsum), s));
  if (st != BITNET_OK) return st;
  return matmul_from_ws(M, N, K, packed, w_scale, y, ws, acc_out, s);
}

bitnet_status bitnet_ternary_matmul(int64_t M, int64_t N, int64_t K, const float *x,
                                    const uint8_t *packed, const float *w_scale, float *y,
                                    void *workspace, size_t workspace_bytes, int8_t *xq_out,
                                    float *x_scale_out, int32_t *acc_out, void *stream) {
  bitnet_status st = matmul_args_ok(M, N, K, x, packed, w_scale, y, xq_out, x_scale_out, acc_out);
  if (st != BITNET_OK) return st;
  if (!workspace || workspace_bytes < bitnet_matmul_workspace_bytes(M, K))
    return BITNET_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return BITNET_ERR_ALIGN;
  st = device_check();
  if (st != BITNET_OK) return st;
  return matmul_run(M, N, K, x, packed, w_scale, y, workspace, xq_out, x_scale_out, acc_out,
                    as_stream(stream));
}

size_t bitnet_scratch_bytes(void) { return kScratchBytes; }

bitnet_status bitnet_ternary_matmul_noalloc(int64_t M, int64_t N, int64_t K, const float *x,
                                            const uint8_t *packed, const float *w_scale,
                                            float *y, int8_t *xq_out, float *x_scale_out,
                                            int32_t *acc_out, void *stream) {
  bitnet_status st = matmul_args_ok(M, N, K, x, packed, w_scale, y, xq_out, x_scale_out, acc_out);
  if (st != BITNET_OK) return st;
  if (bitnet_matmul_workspace_bytes(M, K) > kScratchBytes) return BITNET_ERR_SCRATCH;
  st = device_check();
  if (st != BITNET_OK) return st;
  void *ws = nullptr;
  st = scratch_address(&ws);
  if (st != BITNET_OK) return st;
  return matmul_run(M, N, K, x, packed, w_scale, y, ws, xq_out, x_scale_out, acc_out,
                    as_stream(stream));
}

bitnet_status bitnet_ternary_matmul_q8(int64_t M, int64_t N, int64_t K, const int8_t *xq,
                                       const float *x_scale, const uint8_t *packed,
                                       const float *w_scale, float *y, void *workspace,
                                       size_t workspace_bytes, int32_t *acc_out,
                                       void *stream) {
  if (!xq || !x_scale || !packed || !w_scale || !y) return BITNET_ERR_NULL;
  if (!shape_ok(M, N, K)) return BITNET_ERR_SHAPE;
  if (!aligned(xq, 16) || !aligned(x_scale, 4) || !aligned(packed, 16) ||
      !aligned(w_scale, 4) || !aligned(y, 4) || (acc_out && !aligned(acc_out, 4)))
    return BITNET_ERR_ALIGN;
  if (!workspace || workspace_bytes < bitnet_matmul_workspace_bytes(M, K))
    return BITNET_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return BITNET_ERR_ALIGN;
  bitnet_status st = device_check();
  if (st != BITNET_OK) return st;
  hipStream_t s = as_stream(stream);
  uint8_t *ws = reinterpret_cast<uint8_t *>(workspace);
  const WsLayout L = ws_layout(M, K);
  st = from_hip(launch_permute_q8(xq, x_scale, (int)M, (int)K,
                                  reinterpret_cast<int8_t *>(ws + L.xq),
                                  reinterpret_cast<float *>(ws + L.scale),
                                  reinterpret_cast<int32_t *>(ws + L.rowsum), s));
  if (st != BITNET_OK) return st;
  return matmul_from_ws(M, N, K, packed, w_scale, y, ws, acc_out, s);
}

size_t bitnet_grouped_workspace_bytes(int64_t M, const bitnet_problem *problems_host,
                                      int32_t count) {
  if (M < 1 || !problems_host || count < 1 || count > kMaxGroup) return 0;
  return group_ws(M, problems_host, count, nullptr);
}

bitnet_status bitnet_ternary_matmul_grouped(int64_t M, const bitnet_problem *problems_dev,
                                            int32_t count, const bitnet_problem *problems_host,
                                            void *workspace, size_t workspace_bytes,
                                            void *stream) {
  if (!problems_dev || !problems_host) return BITNET_ERR_NULL;
  if (count < 1 || count > kMaxGroup) return BITNET_ERR_SHAPE;
  if (!aligned(problems_dev, 8)) return BITNET_ERR_ALIGN;
  for (int32_t i = 0; i < count; ++i) {
    bitnet_status st = check_problem(M, problems_host[i]);
    if (st != BITNET_OK) return st;
  }
  GroupTable tab;
  std::memset(&tab, 0, sizeof(tab));
  tab.count = count;
  tab.M = (int32_t)M;
  int32_t owner[kMaxGroup];
  const size_t need = group_ws(M, problems_host, count, tab.ws_off, owner);
  if (!workspace || workspace_bytes < need) return BITNET_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return BITNET_ERR_ALIGN;
  bitnet_status st = device_check();
  if (st != BITNET_OK) return st;

  // Dispatch order: longest K first, so the longest-running workgroups start
  // early and the tail of the launch is made of short ones.
  int32_t idx[kMaxGroup];
  for (int32_t i = 0; i < count; ++i) idx[i] = i;
  std::stable_sort(idx, idx + count, [&](int32_t a, int32_t b) {
    return problems_host[a].K > problems_host[b].K;
  });
  const bool gemv = M <= kGemvMaxM;
  int64_t kmax = 0;
  for (int32_t i = 0; i < count; ++i) kmax = std::max(kmax, problems_host[i].K);
  const bool fused = gemv && gemv_fusable(M, kmax);
  auto fill_blocks = [&](bool split) -> uint64_t {
    uint64_t total = 0;
    for (int32_t s = 0; s < count; ++s) {
      const bitnet_problem &p = problems_host[idx[s]];
      total += gemv ? (uint64_t)gemv_blocks(p.N, p.K, split) : (uint64_t)gemm_blocks(M, p.N);
      tab.blk_end[s] = (uint32_t)std::min<uint64_t>(total, UINT32_MAX);
      tab.order[s] = (uint16_t)idx[s];
    }
    return total;
  };
  uint64_t total = fill_blocks(false);
  if (total >= ((uint64_t)1 << 31)) return BITNET_ERR_SHAPE;
  // A single-row launch too small to fill the chip splits K across waves.
  if (fused && total < (uint64_t)kGemvSplitBelow) {
    tab.split = 1;
    total = fill_blocks(true);
  }
  hipStream_t hs = as_stream(stream);
  uint8_t *ws = reinterpret_cast<uint8_t *>(workspace);
  // Workgroups of each dispatch slot, for the XCD schedule of the main launch.
  auto schedule = [&]() {
    uint32_t tiles[kMaxGroup];
    for (int32_t s = 0; s < count; ++s) {
      const bitnet_problem &p = problems_host[tab.order[s]];
      tiles[s] = gemv ? (uint32_t)gemv_blocks(p.N, p.K, tab.split != 0)
                      : (uint32_t)gemm_blocks(M, p.N);
    }
    xcd_schedule(tab, problems_host, tiles);
  };
  if (fused) {
    schedule();
    return from_hip(launch_gemv_grouped(problems_dev, tab, ws, true, kmax, hs));
  }
  QuantTable qt;
  std::memset(&qt, 0, sizeof(qt));
  qt.count = 0;
  qt.M = (int32_t)M;
  // One quantization per distinct input.
  uint64_t qtotal = 0;
  for (int32_t s = 0; s < count; ++s) {
    if (owner[idx[s]] != idx[s]) continue;
    qtotal += (uint64_t)quant_grouped_blocks(M, problems_host[idx[s]].K);
    if (qtotal >= ((uint64_t)1 << 31)) return BITNET_ERR_SHAPE;
    qt.wg_end[qt.count] = (uint32_t)qtotal;
    qt.order[qt.count] = (uint16_t)idx[s];
    ++qt.count;
  }
  std::memcpy(qt.ws_off, tab.ws_off, sizeof(qt.ws_off));
  st = from_hip(launch_quant_grouped(problems_dev, qt, ws, hs));
  if (st != BITNET_OK) return st;
  schedule();
  if (gemv) return from_hip(launch_gemv_grouped(problems_dev, tab, ws, false, kmax, hs));
  return from_hip(launch_gemm_grouped(problems_dev, tab, ws, hs));
}

// The prefill part of a grouped call over problems sub[0..n) (indices into
// the whole problem array, whose workspace offsets and input owners are
// given): the quantization launch of the inputs owned inside sub goes on qs,
// the GEMM launch on gs; with ev, gs waits for qs through it in between.
static bitnet_status prefill_chunk(int64_t M, const bitnet_problem *problems_dev,
                                   const bitnet_problem *ph, const int32_t *sub, int32_t n,
                                   const uint32_t *ws_off, const int32_t *owner, uint8_t *ws,
                                   hipStream_t qs, hipStream_t gs, hipEvent_t ev) {
  int32_t idx[kMaxGroup];
  std::copy(sub, sub + n, idx);
  std::stable_sort(idx, idx + n, [&](int32_t a, int32_t b) { return ph[a].K > ph[b].K; });
  GroupTable tab;
  std::memset(&tab, 0, sizeof(tab));
  tab.count = n;
  tab.M = (int32_t)M;
  std::memcpy(tab.ws_off, ws_off, sizeof(tab.ws_off));
  uint32_t tiles[kMaxGroup];
  uint64_t total = 0;
  for (int32_t s = 0; s < n; ++s) {
    tiles[s] = (uint32_t)gemm_blocks(M, ph[idx[s]].N);
    total += tiles[s];
    if (total >= ((uint64_t)1 << 31)) return BITNET_ERR_SHAPE;
    tab.blk_end[s] = (uint32_t)total;
    tab.order[s] = (uint16_t)idx[s];
  }
  QuantTable qt;
  std::memset(&qt, 0, sizeof(qt));
  qt.M = (int32_t)M;
  uint64_t qtotal = 0;
  for (int32_t s = 0; s < n; ++s) {
    if (owner[idx[s]] != idx[s]) continue;   // owned in this chunk or an earlier one
    qtotal += (uint64_t)quant_grouped_blocks(M, ph[idx[s]].K);
    if (qtotal >= ((uint64_t)1 << 31)) return BITNET_ERR_SHAPE;
    qt.wg_end[qt.count] = (uint32_t)qtotal;
    qt.order[qt.count] = (uint16_t)idx[s];
    ++qt.count;
  }
  std::memcpy(qt.ws_off, ws_off, sizeof(qt.ws_off));
  if (qt.count > 0) {
    bitnet_status st = from_hip(launch_quant_grouped(problems_dev, qt, ws, qs));
    if (st != BITNET_OK) return st;
  }
  if (ev) {
    if (hipEventRecord(ev, qs) != hipSuccess || hipStreamWaitEvent(gs, ev, 0) != hipSuccess)
      return BITNET_ERR_HIP;
  }
  xcd_schedule(tab, ph, tiles);
  return from_hip(launch_gemm_grouped(problems_dev, tab, ws, gs));
}

bitnet_status bitnet_ternary_matmul_grouped_overlap(int64_t M, const bitnet_problem *problems_dev,
                                                    int32_t count,
                                                    const bitnet_problem *problems_host,
                                                    int32_t nchunks, void *workspace,
                                                    size_t workspace_bytes, void *stream,
                                                    void *aux_stream) {
  if (M <= kGemvMaxM || nchunks <= 1 || aux_stream == stream)
    return bitnet_ternary_matmul_grouped(M, problems_dev, count, problems_host, workspace,
                                         workspace_bytes, stream);
  if (!problems_dev || !problems_host) return BITNET_ERR_NULL;
  if (count < 1 || count > kMaxGroup || nchunks > count || nchunks > BITNET_MAX_CHUNKS)
    return BITNET_ERR_SHAPE;
  if (!aligned(problems_dev, 8)) return BITNET_ERR_ALIGN;
  for (int32_t i = 0; i < count; ++i) {
    bitnet_status st = check_problem(M, problems_host[i]);
    if (st != BITNET_OK) return st;
  }
  uint32_t ws_off[kMaxGroup] = {0};
  int32_t owner[kMaxGroup];
  const size_t need = group_ws(M, problems_host, count, ws_off, owner);
  if (!workspace || workspace_bytes < need) return BITNET_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return BITNET_ERR_ALIGN;
  bitnet_status st = device_check();
  if (st != BITNET_OK) return st;
  // Chunks: contiguous runs of problems of about equal contraction work.
  uint64_t work_total = 0;
  for (int32_t i = 0; i < count; ++i)
    work_total += (uint64_t)problems_host[i].N * (uint64_t)problems_host[i].K;
  int32_t first[BITNET_MAX_CHUNKS + 1];
  int32_t c = 0;
  uint64_t acc = 0;
  first[0] = 0;
  for (int32_t i = 0; i < count && c + 1 < nchunks; ++i) {
    acc += (uint64_t)problems_host[i].N * (uint64_t)problems_host[i].K;
    if (acc * (uint64_t)nchunks >= work_total * (uint64_t)(c + 1) && i + 1 < count)
      first[++c] = i + 1;
  }
  const int32_t chunks = c + 1;
  first[chunks] = count;
  // Launch sizes over the whole call: every chunk's launches are smaller, so
  // no chunk can fail its own size check once some chunks are queued.
  uint64_t gemm_total = 0, quant_total = 0;
  for (int32_t i = 0; i < count; ++i) {
    gemm_total += (uint64_t)gemm_blocks(M, problems_host[i].N);
    if (owner[i] == i) quant_total += (uint64_t)quant_grouped_blocks(M, problems_host[i].K);
  }
  if (gemm_total >= ((uint64_t)1 << 31) || quant_total >= ((uint64_t)1 << 31))
    return BITNET_ERR_SHAPE;
  // Every event is created before the first launch, so a failure to create
  // one leaves nothing queued.  Events are released after use; HIP frees them
  // once their pending work completes.
  hipEvent_t ev[BITNET_MAX_CHUNKS + 1];
  int32_t made = 0;
  for (; made <= chunks; ++made)
    if (hipEventCreateWithFlags(&ev[made], hipEventDisableTiming) != hipSuccess) break;
  if (made <= chunks) {
    for (int32_t k = 0; k < made; ++k) hipEventDestroy(ev[k]);
    return BITNET_ERR_HIP;
  }
  hipStream_t gs = as_stream(stream), qs = as_stream(aux_stream);
  uint8_t *ws = reinterpret_cast<uint8_t *>(workspace);
  // The auxiliary stream starts after everything already queued on the main
  // stream (the inputs, and an earlier call's contractions over the same
  // workspace).
  st = (hipEventRecord(ev[chunks], gs) == hipSuccess &&
        hipStreamWaitEvent(qs, ev[chunks], 0) == hipSuccess)
           ? BITNET_OK
           : BITNET_ERR_HIP;
  int32_t sub[kMaxGroup];
  for (int32_t k = 0; k < chunks && st == BITNET_OK; ++k) {
    const int32_t n = first[k + 1] - first[k];
    for (int32_t i = 0; i < n; ++i) sub[i] = first[k] + i;
    st = prefill_chunk(M, problems_dev, problems_host, sub, n, ws_off, owner, ws, qs, gs, ev[k]);
  }
  for (int32_t k = 0; k <= chunks; ++k) hipEventDestroy(ev[k]);
  return st;
}

// I8_S shapes: K a multiple of 64 (one GEMM step), the same size limits as the
// ternary path.
static bool i8_shape_ok(int64_t M, int64_t N, int64_t K) {
  if (M < 1 || N < 1 || K < 64 || K % 64 != 0) return false;
  if (M >= kLimit || N >= kLimit || K >= kLimit) return false;
  if (M * K >= kLimit || N * K >= kLimit || M * N >= kLimit) return false;
  if ((M + 128) * N * 4 >= kLimit) return false;
  return true;
}

size_t bitnet_i8_quant_workspace_bytes(void) { return 256; }

bitnet_status bitnet_i8_quant_weights(const float *W, int64_t N, int64_t K, int8_t *q,
                                      float *w_scale, void *workspace, size_t workspace_bytes,
                                      void *stream) {
  if (!W || !q || !w_scale) return BITNET_ERR_NULL;
  if (!i8_shape_ok(1, N, K)) return BITNET_ERR_SHAPE;
  if (!aligned(W, 16) || !aligned(q, 16) || !aligned(w_scale, 4)) return BITNET_ERR_ALIGN;
  if (!workspace || workspace_bytes < bitnet_i8_quant_workspace_bytes())
    return BITNET_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return BITNET_ERR_ALIGN;
  bitnet_status st = device_check();
  if (st != BITNET_OK) return st;
  return from_hip(launch_i8_quant_weights(W, N, K, q, w_scale,
                                          reinterpret_cast<uint32_t *>(workspace),
                                          as_stream(stream)));
}

size_t bitnet_i8_linear_workspace_bytes(int64_t M, int64_t K) {
  if (M < 1 || K < 1) return 0;
  return align256((size_t)(M * K)) + align256((size_t)M * 4);
}

static bitnet_status i8_linear_common(int64_t M, int64_t N, int64_t K, const float *x,
                                      const int8_t *q, const float *w_scale, bool per_channel,
                                      const float *bias, int32_t relu, float *y, void *workspace,
                                      size_t workspace_bytes, int32_t *acc_out, void *stream) {
  if (!x || !q || !w_scale || !y) return BITNET_ERR_NULL;
  if (!i8_shape_ok(M, N, K)) return BITNET_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(q, 16) || !aligned(w_scale, 4) || !aligned(y, 4) ||
      (bias && !aligned(bias, 4)) || (acc_out && !aligned(acc_out, 4)))
    return BITNET_ERR_ALIGN;
  if (!workspace || workspace_bytes < bitnet_i8_linear_workspace_bytes(M, K))
    return BITNET_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return BITNET_ERR_ALIGN;
  bitnet_status st = device_check();
  if (st != BITNET_OK) return st;
  hipStream_t s = as_stream(stream);
  uint8_t *ws = reinterpret_cast<uint8_t *>(workspace);
  int8_t *xq = reinterpret_cast<int8_t *>(ws);
  float *xs = reinterpret_cast<float *>(ws + align256((size_t)(M * K)));
  st = from_hip(launch_quant_rows(x, (int)M, (int)K, xq, nullptr, xs, nullptr, nullptr, s));
  if (st != BITNET_OK) return st;
  return from_hip(launch_i8_gemm((int)M, (int)N, (int)K, xq, xs, q, w_scale, per_channel, bias,
                                 relu != 0 ? 1 : 0, y, acc_out, s));
}

bitnet_status bitnet_i8_linear(int64_t M, int64_t N, int64_t K, const float *x, const int8_t *q,
                               const float *w_scale, const float *bias, int32_t relu, float *y,
                               void *workspace, size_t workspace_bytes, int32_t *acc_out,
                               void *stream) {
  return i8_linear_common(M, N, K, x, q, w_scale, false, bias, relu, y, workspace,
                          workspace_bytes, acc_out, stream);
}

bitnet_status bitnet_i8_linear_rows(int64_t M, int64_t N, int64_t K, const float *x,
                                    const int8_t *q, const float *w_scale, const float *bias,
                                    int32_t relu, float *y, void *workspace,
                                    size_t workspace_bytes, int32_t *acc_out, void *stream) {
  return i8_linear_common(M, N, K, x, q, w_scale, true, bias, relu, y, workspace,
                          workspace_bytes, acc_out, stream);
}

bitnet_status bitnet_i8_quant_weights_rows(const float *W, int64_t N, int64_t K, int8_t *q,
                                           float *w_scale, void *stream) {
  if (!W || !q || !w_scale) return BITNET_ERR_NULL;
  if (!i8_shape_ok(1, N, K)) return BITNET_ERR_SHAPE;
  if (!aligned(W, 16) || !aligned(q, 16) || !aligned(w_scale, 4)) return BITNET_ERR_ALIGN;
  bitnet_status st = device_check();
  if (st != BITNET_OK) return st;
  return from_hip(launch_rowq_quant(W, N, K, q, w_scale, false, as_stream(stream)));
}

size_t bitnet_table_bytes(int64_t V, int64_t K) {
  if (!i8_shape_ok(1, V, K)) return 0;
  return table_bytes(V, K);
}

bitnet_status bitnet_table_quant(const float *W, int64_t V, int64_t K, int8_t *table,
                                 float *w_scale, void *stream) {
  if (!W || !table || !w_scale) return BITNET_ERR_NULL;
  if (!i8_shape_ok(1, V, K) || table_bytes(V, K) >= (size_t)kLimit) return BITNET_ERR_SHAPE;
  if (!aligned(W, 16) || !aligned(table, 16) || !aligned(w_scale, 4)) return BITNET_ERR_ALIGN;
  bitnet_status st = device_check();
  if (st != BITNET_OK) return st;
  return from_hip(launch_rowq_quant(W, V, K, table, w_scale, true, as_stream(stream)));
}

bitnet_status bitnet_embed_lookup(const int32_t *ids, int64_t T, const int8_t *q,
                                  const float *w_scale, int64_t N, int64_t K, float *out,
                                  void *stream) {
  if (T == 0) return BITNET_OK;
  if (!ids || !q || !w_scale || !out) return BITNET_ERR_NULL;
  if (T < 0 || T >= kLimit || T * K >= kLimit || !i8_shape_ok(1, N, K) ||
      table_bytes(N, K) >= (size_t)kLimit)
    return BITNET_ERR_SHAPE;
  if (!aligned(ids, 4) || !aligned(q, 16) || !aligned(w_scale, 4) || !aligned(out, 16))
    return BITNET_ERR_ALIGN;
  bitnet_status st = device_check();
  if (st != BITNET_OK) return st;
  return from_hip(launch_embed(ids, T, q, w_scale, N, K, out, as_stream(stream)));
}

bitnet_status bitnet_lm_head(int64_t M, int64_t N, int64_t K, const float *x, const int8_t *q,
                             const float *w_scale, float *y, int8_t *xq_out, float *x_scale_out,
                             int32_t *acc_out, void *stream) {
  if (!x || !q || !w_scale || !y) return BITNET_ERR_NULL;
  if (!i8_shape_ok(M, N, K) || M > kGemvMaxM || M * (K + 16) > kLmHeadMaxRows ||
      table_bytes(N, K) >= (size_t)kLimit)
    return BITNET_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(q, 16) || !aligned(w_scale, 4) || !aligned(y, 4) ||
      (xq_out && !aligned(xq_out, 16)) || (x_scale_out && !aligned(x_scale_out, 4)) ||
      (acc_out && !aligned(acc_out, 4)))
    return BITNET_ERR_ALIGN;
  bitnet_status st = device_check();
  if (st != BITNET_OK) return st;
  return from_hip(launch_lm_head((int)M, (int)N, (int)K, x, q, w_scale, y, xq_out, x_scale_out,
                                 acc_out, as_stream(stream)));
}

static bool dw_shape_ok(int64_t B, int64_t T, int64_t C, int64_t k) {
  if (B < 1 || T < 1 || C < 64 || C % 64 != 0 || k < 1 || k > kMaxDwTaps) return false;
  if (B > 65535 || C >= kLimit || T >= kLimit || B * T * C >= kLimit / 4) return false;
  return true;
}

bitnet_status bitnet_i8_dwconv_quant_weights(const float *W, int64_t C, int64_t k, int8_t *q,
                                             float *w_scale, void *stream) {
  if (!W || !q || !w_scale) return BITNET_ERR_NULL;
  if (!dw_shape_ok(1, 1, C, k)) return BITNET_ERR_SHAPE;
  if (!aligned(W, 4) || !aligned(w_scale, 4)) return BITNET_ERR_ALIGN;
  bitnet_status st = device_check();
  if (st != BITNET_OK) return st;
  return from_hip(launch_dw_quant_weights(W, C, k, q, w_scale, as_stream(stream)));
}

size_t bitnet_i8_dwconv_workspace_bytes(int64_t B, int64_t T, int64_t C) {
  if (!dw_shape_ok(B, T, C, 1)) return 0;
  return (size_t)B * dw_chunks(T) * C * sizeof(float);
}

bitnet_status bitnet_i8_dwconv(int64_t B, int64_t T, int64_t C, int64_t k, const float *x,
                               const int8_t *q, const float *w_scale, const float *bias,
                               int32_t relu, float *y, void *workspace, size_t workspace_bytes,
                               int32_t *acc_out, float *x_scale_out, void *stream) {
  if (!x || !q || !w_scale || !y) return BITNET_ERR_NULL;
  if (!dw_shape_ok(B, T, C, k)) return BITNET_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(w_scale, 4) || !aligned(y, 16) ||
      (bias && !aligned(bias, 4)) || (acc_out && !aligned(acc_out, 16)) ||
      (x_scale_out && !aligned(x_scale_out, 4)))
    return BITNET_ERR_ALIGN;
  if (!workspace || workspace_bytes < bitnet_i8_dwconv_workspace_bytes(B, T, C))
    return BITNET_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return BITNET_ERR_ALIGN;
  bitnet_status st = device_check();
  if (st != BITNET_OK) return st;
  return from_hip(launch_dwconv((int)B, (int)T, (int)C, (int)k, x, q, w_scale, bias,
                                relu != 0 ? 1 : 0, y, reinterpret_cast<float *>(workspace),
                                acc_out, x_scale_out, as_stream(stream)));
}

bitnet_status bitnet_ternary_matmul_lut_grouped(const bitnet_problem *problems_dev,
                                                int32_t count,
                                                const bitnet_problem *problems_host,
                                                void *stream) {
  if (!problems_dev || !problems_host) return BITNET_ERR_NULL;
  if (count < 1 || count > kMaxGroup) return BITNET_ERR_SHAPE;
  if (!aligned(problems_dev, 8)) return BITNET_ERR_ALIGN;
  for (int32_t i = 0; i < count; ++i) {
    bitnet_status st = check_problem(1, problems_host[i]);
    if (st != BITNET_OK) return st;
    if (problems_host[i].K > kLutMaxK) return BITNET_ERR_SHAPE;
  }
  bitnet_status st = device_check();
  if (st != BITNET_OK) return st;
  // Longest K first, as in the grouped call.
  int32_t idx[kMaxGroup];
  for (int32_t i = 0; i < count; ++i) idx[i] = i;
  std::stable_sort(idx, idx + count, [&](int32_t a, int32_t b) {
    return problems_host[a].K > problems_host[b].K;
  });
  GroupTable tab;
  std::memset(&tab, 0, sizeof(tab));
  tab.count = count;
  tab.M = 1;
  uint64_t total = 0;
  uint32_t tiles[kMaxGroup];
  for (int32_t s = 0; s < count; ++s) {
    tiles[s] = (uint32_t)lut_blocks(problems_host[idx[s]].N);
    total += tiles[s];
    if (total >= ((uint64_t)1 << 31)) return BITNET_ERR_SHAPE;
    tab.blk_end[s] = (uint32_t)total;
    tab.order[s] = (uint16_t)idx[s];
  }
  // Whole projections to the XCDs, as in the grouped call.
  xcd_schedule(tab, problems_host, tiles);
  return from_hip(launch_lut_grouped(problems_dev, tab, as_stream(stream)));
}

size_t bitnet_stages_workspace_bytes(int64_t M, const bitnet_problem *problems_host,
                                     int32_t count) {
  if (!problems_host || count < 1 || count > kMaxGroup || M < 1 || M > kGemvMaxM) return 0;
  for (int32_t i = 0; i < count; ++i)
    if (!shape_ok(M, problems_host[i].N, problems_host[i].K)) return 0;
  return stages_workspace_bytes(M, problems_host, count);
}

bitnet_status bitnet_ternary_matmul_stages(int64_t M, const bitnet_problem *problems_dev,
                                           int32_t count, const int32_t *stage_end,
                                           int32_t nstages, const bitnet_problem *problems_host,
                                           void *workspace, size_t workspace_bytes,
                                           void *stream) {
  if (!problems_dev || !problems_host || !stage_end) return BITNET_ERR_NULL;
  if (count < 1 || count > kMaxGroup || nstages < 1 || nstages > kMaxStages)
    return BITNET_ERR_SHAPE;
  if (M < 1 || M > kGemvMaxM) return BITNET_ERR_SHAPE;
  if (!aligned(problems_dev, 8)) return BITNET_ERR_ALIGN;
  for (int32_t i = 0; i < count; ++i) {
    bitnet_status st = check_problem(M, problems_host[i]);
    if (st != BITNET_OK) return st;
    if (!gemv_fusable(M, problems_host[i].K)) return BITNET_ERR_SHAPE;
  }
  int32_t prev = 0;
  int32_t stage_of[kMaxGroup];
  for (int32_t s = 0; s < nstages; ++s) {
    if (stage_end[s] <= prev || stage_end[s] > count) return BITNET_ERR_SHAPE;
    for (int32_t i = prev; i < stage_end[s]; ++i) stage_of[i] = s;
    prev = stage_end[s];
  }
  if (prev != count) return BITNET_ERR_SHAPE;
  // Producers: an x equal to the y of a problem of an earlier stage.  Every
  // other x is an input and must not overlap any y; y ranges are disjoint.
  int16_t src[kMaxGroup];
  auto y_lo = [&](int32_t j) { return reinterpret_cast<uintptr_t>(problems_host[j].y); };
  auto y_hi = [&](int32_t j) { return y_lo(j) + (uintptr_t)(M * problems_host[j].N) * 4; };
  for (int32_t i = 0; i < count; ++i) {
    src[i] = -1;
    for (int32_t j = 0; j < count; ++j)
      if (stage_of[j] < stage_of[i] && (const void *)problems_host[j].y == problems_host[i].x)
        src[i] = (int16_t)j;
    if (src[i] >= 0) {
      if (problems_host[src[i]].N != problems_host[i].K) return BITNET_ERR_SHAPE;
      continue;
    }
    const uintptr_t lo = reinterpret_cast<uintptr_t>(problems_host[i].x);
    const uintptr_t hi = lo + (uintptr_t)(M * problems_host[i].K) * 4;
    for (int32_t j = 0; j < count; ++j)
      if (lo < y_hi(j) && y_lo(j) < hi) return BITNET_ERR_ALIAS;
  }
  for (int32_t i = 0; i < count; ++i)
    for (int32_t j = i + 1; j < count; ++j)
      if (y_lo(i) < y_hi(j) && y_lo(j) < y_hi(i)) return BITNET_ERR_ALIAS;
  if (!workspace || workspace_bytes < stages_workspace_bytes(M, problems_host, count))
    return BITNET_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return BITNET_ERR_ALIGN;
  bitnet_status st = device_check();
  if (st != BITNET_OK) return st;

  return from_hip(launch_stages(problems_dev, problems_host, count, stage_end, nstages, (int)M,
                                src, reinterpret_cast<uint8_t *>(workspace), as_stream(stream)));
}

}  // extern "C"
