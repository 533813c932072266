// Host-side launchers of the comparison and adjacent paths (lookup-table
// decode, I8_S int8 x int8 layers), shared between their kernel files and the
// C ABI layer.  Kept apart from bitnet_internal.hpp, which the decode kernels
// build from.
#pragma once

#include "bitnet_internal.hpp"

namespace bitnet {

// lut.hip: lookup-table variant of the single-row decode (M = 1, K <= kLutMaxK).
constexpr int kLutMaxK = 16384;
int lut_blocks(int64_t N);
hipError_t launch_lut_grouped(const bitnet_problem *problems, const GroupTable &tab,
                              hipStream_t stream);

// i8.hip: I8_S int8 weights x int8 activations.  amax: one zero-filled word of
// workspace (filled here).
hipError_t launch_i8_quant_weights(const float *W, int64_t N, int64_t K, int8_t *q,
                                   float *w_scale, uint32_t *amax, hipStream_t stream);
// per_channel: w_scale holds one scale per output channel [N] instead of one
// device scalar.
hipError_t launch_i8_gemm(int M, int N, int K, const int8_t *xq, const float *x_scale,
                          const int8_t *q, const float *w_scale, bool per_channel,
                          const float *bias, int relu, float *y, int32_t *acc_out,
                          hipStream_t stream);

// lmhead.hip: the decoder's 8-bit table with one scale per row (embeddings,
// lm_head).  lm_head: M <= kGemvMaxM and M * (K + 16) <= kLmHeadMaxRows; the
// workgroup's dynamic LDS then stays within kLmHeadMaxLds.
constexpr size_t kLmHeadMaxLds = 64512;    // with the static LDS, under 64 KB
constexpr int64_t kLmHeadMaxRows = 57344;  // quantized rows in LDS
size_t lm_head_lds_bytes(int64_t M, int64_t V, int64_t K);
// Bytes of the table in its storage order (16-row x 256-input tiles, padded).
size_t table_bytes(int64_t V, int64_t K);
// tiled: write the table's storage order (embeddings, lm_head); otherwise
// row-major [N][K] (per-channel I8_S weights).
hipError_t launch_rowq_quant(const float *W, int64_t N, int64_t K, int8_t *q, float *w_scale,
                             bool tiled, hipStream_t stream);
hipError_t launch_embed(const int32_t *ids, int64_t T, const int8_t *q, const float *w_scale,
                        int64_t N, int64_t K, float *out, hipStream_t stream);
hipError_t launch_lm_head(int M, int V, int K, const float *x, const int8_t *q,
                          const float *w_scale, float *y, int8_t *xq_out, float *x_scale_out,
                          int32_t *acc_out, hipStream_t stream);

// dwconv.hip: I8_S causal depthwise convolution over frames, x [B][T][C],
// C % 64 == 0, 1 <= k <= kMaxDwTaps.  partial: workspace of
// B * dw_chunks(T) * C floats (per-chunk column maxima).
constexpr int kMaxDwTaps = 64;
int dw_chunks(int64_t T);
hipError_t launch_dw_quant_weights(const float *W, int64_t C, int64_t k, int8_t *q,
                                   float *w_scale, hipStream_t stream);
hipError_t launch_dwconv(int B, int T, int C, int k, const float *x, const int8_t *q,
                         const float *w_scale, const float *bias, int relu, float *y,
                         float *partial, int32_t *acc_out, float *x_scale_out,
                         hipStream_t stream);

}  // namespace bitnet
