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
// Work split: a workgroup (4 waves) owns 16*C output columns; its 4 waves split
// the K units evenly and add their int32 partials through LDS (exact in any
// order).  Lane (col = lane%16, h = lane/16) loads 8 bytes = packed dwords
// 2h, 2h+1 of unit u for column col, so a wave reads 512 contiguous bytes per
// unit and column tile.  Field values u = code+1 enter the MFMA; the epilogue
// subtracts the activation row sum.
//
// Activation quantization is fused when the M x K int8 rows fit in LDS: every
// workgroup quantizes the rows itself (absmax, scale, round, row sum) into LDS
// in the permuted order, so one launch does the whole projection.  Otherwise a
// separate quantization kernel writes the rows to the workspace first.
#include "bitnet_device.hpp"
#include "bitnet_internal.hpp"

namespace bitnet {
namespace {

constexpr int kGemvC = 4;                       // 16-column tiles per workgroup
constexpr int kGemvCols = 16 * kGemvC;
constexpr int kThreads = 256;

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
  v4i part[4][kGemvC][64];
  float red[kGemvMaxM][4];
  int ired[kGemvMaxM][4];
  float scale[kGemvMaxM];
  int rowsum[kGemvMaxM];
};

// Quantize the M rows of x into LDS (permuted order) with the scales and row sums.
__device__ __forceinline__ void quant_rows_to_lds(const GemvProblem &p, GemvShared &sh,
                                                  int8_t *xq_lds, bool write_out) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n4 = p.K >> 2;
  for (int m = 0; m < p.M; ++m) {
    const float4 *x4 = reinterpret_cast<const float4 *>(p.x + (size_t)m * p.K);
    float a = 0.0f;
    for (int i = tid; i < n4; i += kThreads) {
      const float4 v = x4[i];
      a = fmaxf(a, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
    }
    a = wave_max(a);
    if (lane == 0) sh.red[m][wave] = a;
  }
  __syncthreads();
  for (int m = 0; m < p.M; ++m) {
    const float a = fmaxf(fmaxf(sh.red[m][0], sh.red[m][1]), fmaxf(sh.red[m][2], sh.red[m][3]));
    const float s = (a == 0.0f) ? 1.0f : 127.0f / a;
    const float4 *x4 = reinterpret_cast<const float4 *>(p.x + (size_t)m * p.K);
    int8_t *dst = xq_lds + (size_t)m * p.K;
    int sum = 0;
    for (int i = tid; i < n4; i += kThreads) {
      const float4 v = x4[i];
      const int q0 = quant_one(v.x, s), q1 = quant_one(v.y, s);
      const int q2 = quant_one(v.z, s), q3 = quant_one(v.w, s);
      sum += q0 + q1 + q2 + q3;
      const uint32_t w = pack4_i8(q0, q1, q2, q3);
      *reinterpret_cast<uint32_t *>(dst + perm_offset(4 * i)) = w;
      if (write_out) reinterpret_cast<uint32_t *>(p.xq_out + (size_t)m * p.K)[i] = w;
    }
    sum = wave_sum(sum);
    if (lane == 0) sh.ired[m][wave] = sum;
    if (tid == 0) {
      sh.scale[m] = s;
      if (write_out) p.x_scale_out[m] = s;
    }
  }
  __syncthreads();
  if (tid < p.M)
    sh.rowsum[tid] = sh.ired[tid][0] + sh.ired[tid][1] + sh.ired[tid][2] + sh.ired[tid][3];
  __syncthreads();
}

template <bool FUSED>
__device__ __forceinline__ void gemv_block(const GemvProblem &p, int n_base, GemvShared &sh,
                                           int8_t *xq_lds) {
  constexpr int C = kGemvC;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;
  const int h = lane >> 4;
  const int units = p.K >> 7;
  const int u0 = (wave * units) >> 2;
  const int u1 = ((wave + 1) * units) >> 2;

  if (FUSED) quant_rows_to_lds(p, sh, xq_lds, p.xq_out != nullptr && n_base == 0);

  v4i acc[C];
#pragma unroll
  for (int c = 0; c < C; ++c) acc[c] = v4i{0, 0, 0, 0};

  const bool a_live = col < p.M;
  const int8_t *a_ptr = (FUSED ? xq_lds : p.xqp) + (size_t)col * p.K + 32 * h;
  const size_t ustride = (size_t)p.N * kUnitBytes;
  const uint8_t *w_ptr[C];
  bool n_live[C];
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int n = n_base + 16 * c + col;
    n_live[c] = n < p.N;
    w_ptr[c] = p.packed + (size_t)n * kUnitBytes + 8 * h;
  }

  uint2 w_cur[C], w_nxt[C];
  v4i a0 = v4i{0, 0, 0, 0}, a1 = v4i{0, 0, 0, 0};
  if (u0 < u1) {
#pragma unroll
    for (int c = 0; c < C; ++c)
      w_cur[c] = n_live[c] ? *reinterpret_cast<const uint2 *>(w_ptr[c] + (size_t)u0 * ustride)
                           : make_uint2(0u, 0u);
  }
  for (int u = u0; u < u1; ++u) {
    if (u + 1 < u1) {
#pragma unroll
      for (int c = 0; c < C; ++c)
        w_nxt[c] = n_live[c]
                       ? *reinterpret_cast<const uint2 *>(w_ptr[c] + (size_t)(u + 1) * ustride)
                       : make_uint2(0u, 0u);
    }
    if (a_live) {
      const v4i *ap = reinterpret_cast<const v4i *>(a_ptr + (size_t)u * kUnit);
      a0 = ap[0];
      a1 = ap[1];
    }
#pragma unroll
    for (int c = 0; c < C; ++c) {
      acc[c] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, unpack_fields(w_cur[c].x), acc[c],
                                                     0, 0, 0);
      acc[c] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, unpack_fields(w_cur[c].y), acc[c],
                                                     0, 0, 0);
    }
#pragma unroll
    for (int c = 0; c < C; ++c) w_cur[c] = w_nxt[c];
  }

#pragma unroll
  for (int c = 0; c < C; ++c) sh.part[wave][c][lane] = acc[c];
  __syncthreads();

  const float ws = *p.w_scale;
  // Output element (row = 4*(l/16) + r, column = l%16) of each 16x16 tile.
  for (int i = threadIdx.x; i < C * 64; i += kThreads) {
    const int c = i >> 6, l = i & 63;
    const int n = n_base + 16 * c + (l & 15);
    if (n >= p.N) continue;
    const v4i s = sh.part[0][c][l] + sh.part[1][c][l] + sh.part[2][c][l] + sh.part[3][c][l];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 4 * (l >> 4) + r;
      if (row < p.M) {
        const int rs = FUSED ? sh.rowsum[row] : p.rowsum[row];
        const float xs = FUSED ? sh.scale[row] : p.x_scale[row];
        const int a = s[r] - rs;
        if (p.acc_out) p.acc_out[(size_t)row * p.N + n] = a;
        p.y[(size_t)row * p.N + n] = dequant(a, ws, xs);
      }
    }
  }
}

template <bool FUSED>
__global__ void __launch_bounds__(kThreads) gemv_kernel(GemvProblem p) {
  __shared__ GemvShared sh;
  extern __shared__ __attribute__((aligned(16))) int8_t xq_lds[];
  gemv_block<FUSED>(p, blockIdx.x * kGemvCols, sh, xq_lds);
}

// Grouped: dispatch slot s of the table owns workgroups [blk_end[s-1], blk_end[s]).
template <bool FUSED>
__global__ void __launch_bounds__(kThreads)
    gemv_grouped_kernel(const bitnet_problem *__restrict__ problems, GroupTable tab,
                        const uint8_t *__restrict__ workspace) {
  __shared__ GemvShared sh;
  extern __shared__ __attribute__((aligned(16))) int8_t xq_lds[];
  const uint32_t b = blockIdx.x;
  int lo = 0, hi = tab.count - 1;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (b < tab.blk_end[mid]) hi = mid; else lo = mid + 1;
  }
  const int slot = lo;
  const uint32_t first = slot ? tab.blk_end[slot - 1] : 0u;
  const int pi = tab.order[slot];
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
  gemv_block<FUSED>(p, (int)(b - first) * kGemvCols, sh, xq_lds);
}

}  // namespace

int gemv_blocks(int64_t N) { return (int)((N + kGemvCols - 1) / kGemvCols); }

bool gemv_fusable(int64_t M, int64_t K) { return M * K <= kGemvFusedLdsBytes; }

hipError_t launch_gemv(int M, int N, int K, const int8_t *xq_perm, const float *x_scale,
                       const int32_t *rowsum, const uint8_t *packed, const float *w_scale,
                       float *y, int32_t *acc_out, hipStream_t stream) {
  GemvProblem p{packed, nullptr, xq_perm, x_scale, rowsum, w_scale, y, acc_out,
                nullptr, nullptr, N, K, M};
  gemv_kernel<false><<<gemv_blocks(N), kThreads, 0, stream>>>(p);
  return hipGetLastError();
}

hipError_t launch_gemv_fused(int M, int N, int K, const float *x, const uint8_t *packed,
                             const float *w_scale, float *y, int8_t *xq_out,
                             float *x_scale_out, int32_t *acc_out, hipStream_t stream) {
  GemvProblem p{packed, x, nullptr, nullptr, nullptr, w_scale, y, acc_out,
                xq_out, x_scale_out, N, K, M};
  gemv_kernel<true><<<gemv_blocks(N), kThreads, (size_t)M * K, stream>>>(p);
  return hipGetLastError();
}

hipError_t launch_gemv_grouped(const bitnet_problem *problems, const GroupTable &tab,
                               const uint8_t *workspace, bool fused, size_t lds_bytes,
                               hipStream_t stream) {
  const unsigned blocks = tab.blk_end[tab.count - 1];
  if (fused)
    gemv_grouped_kernel<true><<<blocks, kThreads, lds_bytes, stream>>>(problems, tab, workspace);
  else
    gemv_grouped_kernel<false><<<blocks, kThreads, 0, stream>>>(problems, tab, workspace);
  return hipGetLastError();
}

}  // namespace bitnet
