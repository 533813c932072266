// Prefill projection, M > 16 rows: a dense int8 contraction on the matrix cores.
//
// Output tile 128 x 256 per workgroup; 4 waves in a 2 x 2 grid, each owning
// 64 x 128 outputs as 2 x 4 blocks of v_mfma_i32_32x32x32_i8 (int32 accumulate).
// Per 128-input unit:
//   - the activation tile (128 rows x 128 permuted int8) is staged through LDS,
//     double buffered, rows beyond M zero-filled;
//   - each wave loads its 128 columns of packed codes straight from global
//     memory (16 bytes = 64 codes per lane) and expands the 2-bit fields to
//     int8 in registers; the expanded codes never touch LDS.
// Lane (i = lane%32, h = lane/32) feeds MFMA e (0..3) of a unit with packed
// dword d = 4h + e of its column and the 16 permuted activations at 16*d of
// its row, so the k positions of both operands agree by construction.
#include "bitnet_device.hpp"
#include "bitnet_internal.hpp"

namespace bitnet {
namespace {

constexpr int BM = 128;
constexpr int BN = 256;
constexpr int WM = 64;               // rows per wave
constexpr int WN = 128;              // columns per wave
constexpr int RB = WM / 32;          // 32-row MFMA blocks per wave
constexpr int CB = WN / 32;          // 32-column MFMA blocks per wave
constexpr int LDS_STRIDE = 128 + 16; // bytes per staged activation row (padded)

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

__device__ __forceinline__ void gemm_block(const GemmProblem &p, int m0, int n0) {
  __shared__ __attribute__((aligned(16))) int8_t a_lds[2][BM * LDS_STRIDE];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int li = lane & 31, lh = lane >> 5;
  const int units = p.K >> 7;

  // Global -> LDS staging of the activation tile: thread owns 64 bytes of a row.
  const int st_row = tid >> 1, st_half = tid & 1;
  const bool st_live = (m0 + st_row) < p.M;
  const int8_t *st_src = p.xqp + (size_t)(m0 + st_row) * p.K + 64 * st_half;
  const int st_dst = st_row * LDS_STRIDE + 64 * st_half;

  // Packed-code loads: lane owns bytes 16*lh..16*lh+15 of each of its CB columns.
  const size_t ustride = (size_t)p.N * kUnitBytes;
  const uint8_t *w_ptr[CB];
  bool n_live[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const int n = n0 + wn * WN + cb * 32 + li;
    n_live[cb] = n < p.N;
    w_ptr[cb] = p.packed + (size_t)n * kUnitBytes + 16 * lh;
  }

  v16i acc[RB][CB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[rb][cb][r] = 0;

  v4i st_reg[4];
  u32x4 w_cur[CB], w_nxt[CB];
  const v4i zero4 = v4i{0, 0, 0, 0};

  // Prologue: unit 0.
  {
    const v4i *src = reinterpret_cast<const v4i *>(st_src);
#pragma unroll
    for (int i = 0; i < 4; ++i) st_reg[i] = st_live ? ld_global<v4i>(src + i) : zero4;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<v4i *>(&a_lds[0][st_dst + 16 * i]) = st_reg[i];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
      w_cur[cb] = n_live[cb] ? ld_global<u32x4>(w_ptr[cb]) : u32x4{0u, 0u, 0u, 0u};
  }
  __syncthreads();

  for (int u = 0; u < units; ++u) {
    const int buf = u & 1;
    const bool more = (u + 1) < units;
    if (more) {
      const v4i *src = reinterpret_cast<const v4i *>(st_src + (size_t)(u + 1) * kUnit);
#pragma unroll
      for (int i = 0; i < 4; ++i) st_reg[i] = st_live ? ld_global<v4i>(src + i) : zero4;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
        w_nxt[cb] = n_live[cb]
                        ? ld_global<u32x4>(w_ptr[cb] + (size_t)(u + 1) * ustride)
                        : u32x4{0u, 0u, 0u, 0u};
    }
    const int8_t *a_base = &a_lds[buf][(wm * WM + li) * LDS_STRIDE + 64 * lh];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v4i a[RB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        a[rb] = *reinterpret_cast<const v4i *>(a_base + rb * 32 * LDS_STRIDE + 16 * e);
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const uint32_t d = e == 0 ? w_cur[cb].x : e == 1 ? w_cur[cb].y : e == 2 ? w_cur[cb].z : w_cur[cb].w;
        const v4i b = unpack_fields(d);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          acc[rb][cb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[rb], b, acc[rb][cb], 0, 0, 0);
      }
    }
    if (more) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<v4i *>(&a_lds[buf ^ 1][st_dst + 16 * i]) = st_reg[i];
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) w_cur[cb] = w_nxt[cb];
    }
    __syncthreads();
  }

  // Epilogue: element r of a 32x32 block sits at row 8*(r/4) + 4*(lane/32) + r%4,
  // column lane%32.
  const float ws = ld_global<float>(p.w_scale);
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = m0 + wm * WM + rb * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
      if (row >= p.M) continue;
      const int rs = ld_global<int>(p.rowsum + row);
      const float xs = ld_global<float>(p.x_scale + row);
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const int n = n0 + wn * WN + cb * 32 + li;
        if (n < p.N) {
          const int a = acc[rb][cb][r] - rs;
          if (p.acc_out) st_global<int>(p.acc_out + (size_t)row * p.N + n, a);
          st_global<float>(p.y + (size_t)row * p.N + n, dequant(a, ws, xs));
        }
      }
    }
  }
}

__global__ void __launch_bounds__(256) gemm_kernel(GemmProblem p) {
  const int nt = (p.N + BN - 1) / BN;
  gemm_block(p, (int)(blockIdx.x / nt) * BM, (int)(blockIdx.x % nt) * BN);
}

__global__ void __launch_bounds__(256)
    gemm_grouped_kernel(const bitnet_problem *__restrict__ problems, GroupTable tab,
                        const uint8_t *__restrict__ workspace) {
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
  const int nt = (p.N + BN - 1) / BN;
  const int local = (int)(b - first);
  gemm_block(p, (local / nt) * BM, (local % nt) * BN);
}

}  // namespace

int gemm_blocks(int64_t M, int64_t N) {
  return (int)(((M + BM - 1) / BM) * ((N + BN - 1) / BN));
}

hipError_t launch_gemm(int M, int N, int K, const int8_t *xq_perm, const float *x_scale,
                       const int32_t *rowsum, const uint8_t *packed, const float *w_scale,
                       float *y, int32_t *acc_out, hipStream_t stream) {
  GemmProblem p{packed, xq_perm, x_scale, rowsum, w_scale, y, acc_out, M, N, K};
  gemm_kernel<<<gemm_blocks(M, N), 256, 0, stream>>>(p);
  return hipGetLastError();
}

hipError_t launch_gemm_grouped(const bitnet_problem *problems, const GroupTable &tab,
                               const uint8_t *workspace, hipStream_t stream) {
  const unsigned blocks = tab.blk_end[tab.count - 1];
  gemm_grouped_kernel<<<blocks, 256, 0, stream>>>(problems, tab, workspace);
  return hipGetLastError();
}

}  // namespace bitnet
