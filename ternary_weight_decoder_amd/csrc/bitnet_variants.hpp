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
hipError_t launch_i8_gemm(int M, int N, int K, const int8_t *xq, const float *x_scale,
                          const int8_t *q, const float *w_scale, const float *bias, int relu,
                          float *y, int32_t *acc_out, hipStream_t stream);

}  // namespace bitnet
