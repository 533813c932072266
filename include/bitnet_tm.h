/*
 * bitnet_tm.h -- C ABI of the MI355X (gfx950) ternary-weight x int8-activation
 * projection library.
 *
 * The operation is the linear projection of a BitNet b1.58 ("I2_S") decoder:
 *   - every projection weight is one of -1, 0, +1, with one floating scale per
 *     tensor taken from the mean absolute weight (ONNX model card
 *     "multimodalart/VibeVoice-ASR-BitNet-ONNX", Quantization table, row "LM
 *     projections"; blog "The Paper Says ARM Support. I Might Be the First to
 *     Actually Compile It", section "What the model is trying to do");
 *   - codes are stored at 2 bits in units of 128 inputs (same blog, section
 *     "Postscript two");
 *   - with ternary weights the products reduce to adding and subtracting
 *     activations (xujun.org AIGCPanel article, section on heterogeneous
 *     quantization; aitrends.kr model summary, sections on technical features and
 *     differentiators).
 *
 * Numeric definitions (the pages leave these open; this library fixes them):
 *   m        = mean|W| over all N*K weights: each row summed in fp64 with k
 *              ascending, rows added in fp64 with n ascending, divided by N*K in
 *              fp64, rounded once to fp32.  w_scale = m.
 *   code     = clamp(rint(fl32(W / m)), -1, 1), rint = round half to even,
 *              fl32(W/m) = IEEE fp32 division.  m == 0 gives all codes 0.
 *   x_scale  = fl32(127 / max_k |x[m,k]|) per row; xq = clamp(rint(fl32(x*s)), -127, 127).
 *              An all-zero row gives xq = 0 and x_scale = 1.
 *   acc      = sum_k xq[m,k] * code[n,k]   (exact, int32; |acc| <= 127*K)
 *   y[m,n]   = acc * w_scale / x_scale[m], rounded to fp32.  The reference
 *              value is the product in fp64 (exact), divided in fp64 (correctly
 *              rounded) and rounded once more to fp32.  Decode calls (M <= 16)
 *              return exactly that value; prefill calls (M > 16) are within
 *              1e-6 relative of it (one fp32 factor w_scale / x_scale per row).
 *              acc == 0 gives exactly 0.
 *   NaN/Inf inputs and rows whose 127/absmax overflows are outside the contract.
 *
 * Packed layout (2 bits per code, N*K/4 bytes, K a multiple of 128):
 *   field value u = code + 1 in {0,1,2}; the value 3 never occurs.
 *   For code (n,k): t = k/128, r = k%128,
 *     byte  = (t*N + n)*32 + (r % 32)
 *     bits  = [2*(r/32)+1 : 2*(r/32)]
 *   i.e. unit t of row n is a 32-byte block; all N blocks of unit t are
 *   contiguous ("unit-column-major").  This bit placement is this library's
 *   own; the pages fix only the unit size and the 2-bit width.
 *
 * Workspaces.  Every entry point that needs temporary device memory takes it
 * as a caller-provided workspace argument with a size helper
 * (bitnet_*_workspace_bytes), so the library itself never allocates; that is
 * why the ternarization, the q8 matmul and the grouped calls carry workspace
 * arguments, and why the matmul's size helper is named for the matmul
 * (bitnet_matmul_workspace_bytes).  The one exception, for callers that
 * cannot allocate at all, is bitnet_ternary_matmul_noalloc.
 *
 * Conventions for every entry point:
 *   - All data pointers are DEVICE pointers on the current HIP device, which
 *     must be a gfx950 (MI355X).  `stream` is a hipStream_t passed as void*
 *     (NULL = the default stream).  Every call is asynchronous on `stream`.
 *   - The library never allocates device memory; callers own every buffer,
 *     except the fixed scratch array of bitnet_ternary_matmul_noalloc, which
 *     each device holds from module load to process exit.  Its only mutable
 *     host state is per-device caches (the architecture check and that
 *     array's device address), filled on first use under a lock.  Calls on
 *     different streams are independent as long as their buffers do not
 *     overlap.
 *   - Arguments are checked on the host before anything is launched.  On any
 *     error nothing is launched and nothing is written.  Faults inside kernels
 *     surface at the caller's next synchronization.
 *   - Pointers that are read or written with vector loads must be 16-byte
 *     aligned (x, W, packed, xq, xq_out, workspace); others need their natural
 *     alignment.
 *   - Size limits: M, N, K >= 1, K % 128 == 0, M*K and N*K below 2^31, and
 *     (M + 128) * N * 4 below 2^31 (the fp32 output is addressed with 32-bit
 *     byte offsets).
 */
#ifndef BITNET_TM_H
#define BITNET_TM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t bitnet_status;

#define BITNET_OK            0
#define BITNET_ERR_NULL      1  /* a required pointer is NULL                      */
#define BITNET_ERR_SHAPE     2  /* M,N,K out of range or K % 128 != 0              */
#define BITNET_ERR_ALIGN     3  /* a pointer is not aligned as required            */
#define BITNET_ERR_WORKSPACE 4  /* workspace missing or smaller than required      */
#define BITNET_ERR_HIP       5  /* a HIP call or kernel launch reported an error   */
#define BITNET_ERR_DEVICE    6  /* the current device is not a gfx950             */
#define BITNET_ERR_ALIAS     7  /* outputs overlap each other or an input          */
#define BITNET_ERR_SCRATCH   8  /* needs more than the built-in scratch (noalloc)  */

/* Maximum number of problems in one grouped call. */
#define BITNET_MAX_GROUP     256

/* Human-readable name of a status code (static string, never NULL). */
const char *bitnet_status_string(bitnet_status s);

/* Bytes of the packed code buffer for an N x K weight: N*K/4. */
size_t bitnet_packed_bytes(int64_t N, int64_t K);

/* ------------------------------------------------------------------------
 * Ternarization and packing (offline, once per weight tensor).
 *
 * W        [N,K] fp32 row-major master weights (out x in), 16-byte aligned.
 * packed   [N*K/4] bytes, 16-byte aligned, fully overwritten.
 * w_scale  one fp32 written on the device: mean|W| (see definitions above).
 * workspace: at least bitnet_ternarize_workspace_bytes(N) bytes, 16-byte
 *          aligned; holds the fp64 row sums.  Contents on return are unspecified.
 * Passage: ONNX model card, Quantization table, row "LM projections" (per-tensor
 * absmean scale, ternary values); same card, note under that table (ternarize
 * the master weights right before export); blog, "Postscript two" (128-code
 * units).
 * ------------------------------------------------------------------------ */
size_t bitnet_ternarize_workspace_bytes(int64_t N);

bitnet_status bitnet_ternarize_pack(const float *W, int64_t N, int64_t K, uint8_t *packed,
                                    float *w_scale, void *workspace, size_t workspace_bytes,
                                    void *stream);

/* ------------------------------------------------------------------------
 * Per-row int8 absmax activation quantization.
 *
 * x        [M,K] fp32 row-major, 16-byte aligned.
 * xq       [M,K] int8 row-major (natural k order), 16-byte aligned.
 * x_scale  [M] fp32: 127/absmax of each row (1.0 for an all-zero row).
 * Passage: int8 activations with absmax scaling appear on the pages for the
 * audio encoder's I8_S path (ONNX model card, Quantization table, row "VAE
 * encoders"); the formula above is this library's definition for the LM.
 * ------------------------------------------------------------------------ */
bitnet_status bitnet_quant_act(const float *x, int64_t M, int64_t K, int8_t *xq,
                               float *x_scale, void *stream);

/* ------------------------------------------------------------------------
 * The projection: y[M,N] = dequant( quant(x) . codes^T ).
 *
 * x        [M,K] fp32 row-major, 16-byte aligned.
 * packed   codes of W [N,K] in the packed layout, 16-byte aligned.
 * w_scale  device pointer to the fp32 tensor scale written by
 *          bitnet_ternarize_pack.
 * y        [M,N] fp32 row-major output, 4-byte aligned.
 * workspace: at least bitnet_matmul_workspace_bytes(M, K) bytes, 256-byte
 *          aligned (quantized activations, scales and row sums).
 * xq_out, x_scale_out, acc_out: optional (may be NULL) copies of the int8
 *          activations [M,K], their scales [M] and the int32 accumulators [M,N],
 *          for parity checks.
 * M <= 16 runs the decode GEMV (HBM-bound weight stream), M > 16 the prefill
 * GEMM (int8 MFMA); results are identical either way.
 * Passage: the add/subtract contraction (xujun.org article, heterogeneous
 * quantization section; aitrends.kr summary, technical-features section); the
 * decoder reads all of its weights for every token (blog, "What the model is
 * trying to do").
 * ------------------------------------------------------------------------ */
size_t bitnet_matmul_workspace_bytes(int64_t M, int64_t K);

bitnet_status bitnet_ternary_matmul(int64_t M, int64_t N, int64_t K, const float *x,
                                    const uint8_t *packed, const float *w_scale, float *y,
                                    void *workspace, size_t workspace_bytes, int8_t *xq_out,
                                    float *x_scale_out, int32_t *acc_out, void *stream);

/* Same projection for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * no workspace argument; the quantized rows, scales and row sums go to a
 * built-in scratch array of BITNET_SCRATCH_BYTES (= bitnet_scratch_bytes())
 * per device.  Problems whose bitnet_matmul_workspace_bytes(M, K) exceeds it
 * are rejected with BITNET_ERR_SCRATCH (M = 1800 fits up to K = 18560).
 * Allocates nothing (no hipMalloc, no library allocation); the first call on
 * a device looks up the array's address.  Every call on one device shares
 * that array and leaves its contents behind: calls that overlap in time on
 * one device (different streams, or host threads) race and must be ordered
 * by the caller.  Outputs are identical to bitnet_ternary_matmul's. */
#define BITNET_SCRATCH_BYTES ((size_t)32 << 20)

size_t bitnet_scratch_bytes(void);

bitnet_status bitnet_ternary_matmul_noalloc(int64_t M, int64_t N, int64_t K, const float *x,
                                            const uint8_t *packed, const float *w_scale,
                                            float *y, int8_t *xq_out, float *x_scale_out,
                                            int32_t *acc_out, void *stream);

/* Same projection from already-quantized activations (xq natural order, as
 * written by bitnet_quant_act): the prefill GEMM proper, separable from the
 * quantization.  workspace: bitnet_matmul_workspace_bytes(M, K) (the rows
 * permuted to the packed order, and their sums).  Passage: as for
 * bitnet_ternary_matmul; the pages' own interface also keeps the quantized
 * tensors apart from the matmul node that consumes them (ONNX model card,
 * Quantization table, row "LM projections": MatMulNBits over packed blocks). */
bitnet_status bitnet_ternary_matmul_q8(int64_t M, int64_t N, int64_t K, const int8_t *xq,
                                       const float *x_scale, const uint8_t *packed,
                                       const float *w_scale, float *y, void *workspace,
                                       size_t workspace_bytes, int32_t *acc_out,
                                       void *stream);

/* ------------------------------------------------------------------------
 * Grouped projections: `count` independent problems with the same M, one
 * quantization launch and one matmul launch for all of them.  A decoder layer
 * (7 projections) or a whole decoder (196) fits in one call.
 *
 * problems_dev  device copy of the problem array (read by the kernels).
 * problems_host host copy of the same array (read by the host to check shapes
 *               and size the launch); both must hold identical values.
 * workspace     at least bitnet_grouped_workspace_bytes(M, problems_host, count)
 *               bytes, 256-byte aligned (that function returns 0 for M < 1,
 *               a NULL array or count outside 1..BITNET_MAX_GROUP).
 * count         1..BITNET_MAX_GROUP.
 * Every problem obeys the single-problem rules above.  Problems with the same
 * x pointer and the same K (a decoder's q, k and v, or its gate and up) share
 * one quantized copy of their rows: it is made once per call and takes
 * workspace once.  The outputs are the same as with separate copies.
 * Passage: the decoder has 196 such matrices and reads all of them for every
 * token (blog, "What the model is trying to do"; ONNX model card, Quantization
 * table, row "LM projections (196 mats)"), so one token's projections are a
 * stream of independent problems that one launch can cover.
 * ------------------------------------------------------------------------ */
typedef struct bitnet_problem {
    const float *x;          /* [M,K] fp32 activations                     */
    const uint8_t *packed;   /* packed codes of W [N,K]                    */
    const float *w_scale;    /* device fp32 tensor scale                   */
    float *y;                /* [M,N] fp32 output                          */
    int64_t N;
    int64_t K;
} bitnet_problem;

size_t bitnet_grouped_workspace_bytes(int64_t M, const bitnet_problem *problems_host,
                                      int32_t count);

bitnet_status bitnet_ternary_matmul_grouped(int64_t M, const bitnet_problem *problems_dev,
                                            int32_t count, const bitnet_problem *problems_host,
                                            void *workspace, size_t workspace_bytes,
                                            void *stream);

/* The same grouped projections at prefill (M > 16) with the activation
 * quantization overlapped with the contraction: the problems are cut into
 * `nchunks` contiguous runs of about equal work; the quantization launch of
 * run c + 1 goes on aux_stream while the GEMM launch of run c runs on
 * `stream` (the two kernels fit on a compute unit together: the GEMM leaves
 * register room for a quantization wave), ordered by events the call creates
 * and releases.  aux_stream first waits for the work already queued on
 * `stream`; after the call, `stream` holds the whole result, and later work
 * on aux_stream is ordered after the quantizations only.  Outputs are those of
 * bitnet_ternary_matmul_grouped (the same kernels).  With M <= 16, nchunks <=
 * 1 or aux_stream == stream this is the plain grouped call on `stream`.
 * nchunks <= count and <= BITNET_MAX_CHUNKS; workspace as for the grouped
 * call.  Use distinct, default-priority streams.  Shapes, sizes and the
 * events are all checked or created before the first launch, so those errors
 * leave nothing queued; a HIP error while the chunks are being queued
 * (BITNET_ERR_HIP) can leave the earlier chunks queued.  The call is meant
 * for prefill-sized steps: each chunk adds launches and an event hand-off
 * between the streams. */
#define BITNET_MAX_CHUNKS 32

bitnet_status bitnet_ternary_matmul_grouped_overlap(int64_t M, const bitnet_problem *problems_dev,
                                                    int32_t count,
                                                    const bitnet_problem *problems_host,
                                                    int32_t nchunks, void *workspace,
                                                    size_t workspace_bytes, void *stream,
                                                    void *aux_stream);

/* ------------------------------------------------------------------------
 * I8_S: int8 weights x int8 activations, the audio encoders' linear layers.
 * The encoders run with int8 weights and activations and ReLU in place of
 * GELU (ONNX model card "multimodalart/VibeVoice-ASR-BitNet-ONNX",
 * Quantization table, row "VAE encoders"), in fused matmul + bias + ReLU
 * routines (aitrends.kr summary, technical-features section).  The pages give
 * no scale granularity; this library uses one absmax scale per weight tensor
 * (as I2_S has one scale per tensor) and the per-row activation quantization
 * of bitnet_quant_act.
 *
 * bitnet_i8_quant_weights: W fp32 [N,K] row-major -> q int8 [N,K] and the
 *   device scalar w_scale = fl32(max|W| / 127); q = clamp(rint(fl32(W /
 *   w_scale)), -127, 127), half to even; a zero tensor gives w_scale 0 and
 *   q 0.  Bit-exact.  K >= 64, K % 64 == 0; W, q 16-byte aligned; workspace
 *   bitnet_i8_quant_workspace_bytes() bytes, 256-byte aligned (scratch).
 *   Three small launches.
 *
 * bitnet_i8_linear: y[m,n] = relu?(acc[m,n] * w_scale / x_scale[m] + bias[n])
 *   with xq, x_scale the per-row quantization of x (as bitnet_quant_act) and
 *   acc = sum_k xq[m,k] * q[n,k] in int32 (bit-exact).  The epilogue is fp32:
 *   fl32(fl32(acc) * fl32(w_scale / x_scale)) + bias, then max(., 0) when
 *   relu != 0; its error is below 4 * 2^-24 * (|acc * w_scale / x_scale| +
 *   |bias|).  x fp32 [M,K], q int8 [N,K] (16-byte aligned), bias fp32 [N] or
 *   NULL, y fp32 [M,N]; acc_out int32 [M,N] or NULL.  K >= 64, K % 64 == 0.
 *   workspace: bitnet_i8_linear_workspace_bytes(M, K) bytes, 256-byte
 *   aligned (the int8 rows and their scales).  Two launches.
 * ------------------------------------------------------------------------ */
size_t bitnet_i8_quant_workspace_bytes(void);

bitnet_status bitnet_i8_quant_weights(const float *W, int64_t N, int64_t K, int8_t *q,
                                      float *w_scale, void *workspace, size_t workspace_bytes,
                                      void *stream);

size_t bitnet_i8_linear_workspace_bytes(int64_t M, int64_t K);

/* bitnet_i8_linear_rows: the same layer with one weight scale per output
 *   channel, as the ONNX build stores the encoders ("int8 per-channel
 *   weights": ONNX model card, Quantization table, row "VAE encoders"):
 *   q and w_scale [N] come from bitnet_i8_quant_weights_rows, and
 *   y[m,n] = relu?(acc[m,n] * w_scale[n] / x_scale[m] + bias[n]).  The
 *   epilogue is fp32: fl32(fl32(fl32(acc) * w_scale[n]) * fl32(1 / x_scale[m]))
 *   + bias, then ReLU; its error is below 5 * 2^-24 * (|acc * w_scale[n] /
 *   x_scale[m]| + |bias|).  Same arguments, workspace, limits and launches as
 *   bitnet_i8_linear; w_scale 4-byte aligned. */
bitnet_status bitnet_i8_linear_rows(int64_t M, int64_t N, int64_t K, const float *x,
                                    const int8_t *q, const float *w_scale, const float *bias,
                                    int32_t relu, float *y, void *workspace,
                                    size_t workspace_bytes, int32_t *acc_out, void *stream);

bitnet_status bitnet_i8_linear(int64_t M, int64_t N, int64_t K, const float *x, const int8_t *q,
                               const float *w_scale, const float *bias, int32_t relu, float *y,
                               void *workspace, size_t workspace_bytes, int32_t *acc_out,
                               void *stream);

/* ------------------------------------------------------------------------
 * I8_S causal depthwise convolution over frames: the encoders' token mixer.
 * The encoders fuse int8 convolution and depthwise convolution with bias
 * (aitrends.kr summary, technical-features section), padded causally in the
 * ONNX export (ONNX model card, Provenance), with int8 per-channel weights
 * (same card, Quantization table, row "VAE encoders").  The pages give no
 * formula; this library's:
 *   y[b,t,c] = relu?(acc * w_scale[c] / x_scale[b,c] + bias[c]), rounded
 *              once to fp32 from fp64 (exact product, correctly rounded
 *              division, then the bias add), bit-exact;
 *   acc      = sum_{j<k} q[c,j] * xq[b, t-(k-1)+j, c] (frames before 0 count
 *              as 0), int32;
 *   xq, x_scale: x quantized with one absmax scale per (sequence, channel),
 *              x_scale = fl32(127 / max_t |x[b,t,c]|), round half to even,
 *              clamp +-127; an all-zero column gives xq = 0, x_scale = 1.
 *
 * bitnet_i8_dwconv_quant_weights: W fp32 [C,k] -> q int8 [C,k] and w_scale
 *   fp32 [C], per channel as the table rows (bitnet_table_quant's formula).
 *   C % 64 == 0, 1 <= k <= 64.  One launch.
 * bitnet_i8_dwconv: x fp32 [B,T,C] (channels innermost, 16-byte aligned),
 *   y fp32 [B,T,C] (16-byte aligned), bias [C] or NULL, acc_out int32
 *   [B,T,C] (16-byte aligned) and x_scale_out fp32 [B,C] optional.
 *   B <= 65535, C % 64 == 0, 1 <= k <= 64, B*T*C < 2^29.  workspace:
 *   bitnet_i8_dwconv_workspace_bytes(B, T, C) bytes, 16-byte aligned (the
 *   column maxima of each frame chunk: chunks of 128 frames, or of a larger
 *   power of two so that a sequence has at most 64).  Two launches: the
 *   chunk maxima, then the convolution, whose workgroups reduce them to the
 *   scales of their channels.
 * ------------------------------------------------------------------------ */
bitnet_status bitnet_i8_dwconv_quant_weights(const float *W, int64_t C, int64_t k, int8_t *q,
                                             float *w_scale, void *stream);

size_t bitnet_i8_dwconv_workspace_bytes(int64_t B, int64_t T, int64_t C);

bitnet_status bitnet_i8_dwconv(int64_t B, int64_t T, int64_t C, int64_t k, const float *x,
                               const int8_t *q, const float *w_scale, const float *bias,
                               int32_t relu, float *y, void *workspace, size_t workspace_bytes,
                               int32_t *acc_out, float *x_scale_out, void *stream);

/* ------------------------------------------------------------------------
 * The decoder's 8-bit table with one scale per row: token embeddings and the
 * lm_head.  The ONNX build stores both at 8 bits, "per-row / per-column", where
 * the GGUF build uses Q6_K (ONNX model card "multimodalart/VibeVoice-ASR-
 * BitNet-ONNX", Quantization table, row "Embeddings / lm_head"; xujun.org
 * article, heterogeneous-quantization section: I2_S plus Q6_K embeddings).
 * One table (V vocabulary rows x K hidden inputs) serves both: row v is
 * token v's embedding and, read as the lm_head weight, the weights of logit v,
 * so its per-row scales are the lm_head's per-column scales.  The Q6_K block
 * format is not on the pages; this 8-bit form is the card's ONNX one.
 *
 * Table storage order (this library's own; the pages fix only 8 bits per code
 * and one scale per row): rows are grouped by 16 and inputs by 256; each
 * 16-row x 256-input tile is 4096 contiguous bytes, tiles ordered by row group
 * and then by input chunk; inside a tile, input k = 64j + 16h + e (j, h < 4,
 * e < 16) of tile row r sits at byte 1024j + 256h + 16r + e.  The table is
 * padded with zero codes to Vp = 16*ceil(V/16) rows and Kp = 256*ceil(K/256)
 * inputs: bitnet_table_bytes(V, K) = Vp * Kp bytes (0 for shapes outside the
 * limits).
 *
 * bitnet_table_quant: W fp32 [V,K] row-major master weights -> the table in
 *   the storage order above (all Vp * Kp bytes written, padding 0) and
 *   w_scale fp32 [V]: per row v, w_scale[v] = fl32(max_k |W[v,k]| / 127),
 *   code = clamp(rint(fl32(W / w_scale[v])), -127, 127), half to even; a zero
 *   row gives w_scale[v] = 0 and codes 0.  Bit-exact.  V >= 1, K >= 64,
 *   K % 64 == 0, V*K and Vp*Kp < 2^31; W and table 16-byte aligned, w_scale
 *   4-byte.  One launch, no workspace.
 *
 * bitnet_i8_quant_weights_rows: the same per-row quantization into plain
 *   row-major q int8 [N,K], for the per-channel I8_S layer
 *   (bitnet_i8_linear_rows).  Same limits; N*K < 2^31.
 *
 * bitnet_embed_lookup: out[t,k] = fl32(code[ids[t],k] * w_scale[ids[t]]) for
 *   t < T, from a table made by bitnet_table_quant (V rows); an id outside
 *   [0, V) gives a zero row (ids are device data and are not checked on the
 *   host).  ids int32 [T] (4-byte aligned), table and out fp32 [T,K] 16-byte
 *   aligned.  T == 0 launches nothing and returns BITNET_OK.  K >= 64,
 *   K % 64 == 0, T*K < 2^31.  Bit-exact.
 *
 * bitnet_lm_head: y[m,v] = acc[m,v] * w_scale[v] / x_scale[m], rounded once to
 *   fp32 (the product in fp64, exact; the division in fp64, correctly rounded),
 *   with xq, x_scale the per-row quantization of x (as bitnet_quant_act) and
 *   acc = sum_k xq[m,k] * code[v,k] in int32; the table as made by
 *   bitnet_table_quant.  Decode only: 1 <= M <= 16 and M * (K + 16) <= 57344
 *   (the quantized rows stay in LDS); K >= 64, K % 64 == 0, M*V*4 < 2^31.
 *   x fp32 [M,K] and table 16-byte aligned, w_scale fp32 [V], y fp32 [M,V]
 *   4-byte aligned.  xq_out [M,K] (16-byte aligned), x_scale_out [M] and
 *   acc_out [M,V] are optional copies for parity checks.  One launch, no
 *   workspace; an HBM stream of the table.
 * ------------------------------------------------------------------------ */
size_t bitnet_table_bytes(int64_t V, int64_t K);

bitnet_status bitnet_table_quant(const float *W, int64_t V, int64_t K, int8_t *table,
                                 float *w_scale, void *stream);

bitnet_status bitnet_i8_quant_weights_rows(const float *W, int64_t N, int64_t K, int8_t *q,
                                           float *w_scale, void *stream);

bitnet_status bitnet_embed_lookup(const int32_t *ids, int64_t T, const int8_t *table,
                                  const float *w_scale, int64_t V, int64_t K, float *out,
                                  void *stream);

bitnet_status bitnet_lm_head(int64_t M, int64_t V, int64_t K, const float *x,
                             const int8_t *table, const float *w_scale, float *y, int8_t *xq_out,
                             float *x_scale_out, int32_t *acc_out, void *stream);

/* ------------------------------------------------------------------------
 * Lookup-table variant of the single-row decode, for comparison with the
 * unpack + matrix-core path.  bitnet.cpp's kernels use the lookup-table method
 * of T-MAC (thetesserapress, "Microsoft's BitNet Adds 1-Bit Embeddings...",
 * the paragraphs on the repo's dependencies and on platform support): each
 * workgroup quantizes the activation row, tabulates the 16 signed sums that a
 * 4-bit pair of packed codes can select, and adds one table entry per pair.
 * The int32 sums, and so the outputs, equal the grouped call's at M = 1
 * (exactly rounded).
 *
 * problems      as for the grouped call, with M = 1 (x is [1, K]);
 *               1 <= K <= 16384, K % 128 == 0.
 * No workspace; one launch.  Same status codes as the grouped call.
 * ------------------------------------------------------------------------ */
bitnet_status bitnet_ternary_matmul_lut_grouped(const bitnet_problem *problems_dev,
                                                int32_t count,
                                                const bitnet_problem *problems_host,
                                                void *stream);

/* ------------------------------------------------------------------------
 * Dependent decode stages in one launch.  The decoder reads all of its
 * weights for every token (blog "The Paper Says ARM Support...", section
 * "What the model is trying to do"), and its projections depend on each
 * other in order: q,k,v, then o, then gate,up, then down, layer after layer.
 * This call runs such a sequence of stages: problems [stage_end[s-1],
 * stage_end[s]) form stage s (stage_end[-1] = 0), in order.  A problem whose
 * x pointer equals the y pointer of a problem of an earlier stage reads that
 * problem's output (its K must equal that problem's N); every other x is an
 * input written before the call.  Outputs are those of the single calls
 * (decode: exactly rounded).
 *
 * M             1..16, and M*K <= 8960 for every problem (rows quantized in
 *               the same workgroup; one row of the longest projection).
 * count         1..BITNET_MAX_GROUP problems in stage order; nstages
 *               1..BITNET_MAX_STAGES; stage_end (host) strictly increasing,
 *               stage_end[nstages-1] == count.
 * problems_dev / problems_host as for the grouped call.
 * y ranges      must not overlap each other nor any input x (one written
 *               before the call): BITNET_ERR_ALIAS.
 * workspace     bitnet_stages_workspace_bytes(M, problems_host, count)
 *               bytes, 256-byte aligned, ZERO-FILLED before its first use
 *               and written by nothing else afterwards (it carries a call
 *               counter and the outputs that later stages read, each tagged
 *               with that counter; later calls may reuse it).  Word 1 (uint32) is nonzero after the call
 *               completes if a wait for a producer ran past its bound (200 ms
 *               of the device's wall clock; once one wait has run out the
 *               later ones return at once); the outputs are then not valid.
 *               Word 2 (uint32) counts the calls in which that happened since
 *               the workspace was zero-filled; the library never clears it.
 *               The call never waits without bound.
 * One one-thread kernel (advances the counter), then one cooperative launch
 * (all workgroups resident at once); no device-wide barrier: each tile waits
 * only for the outputs it reads.  BITNET_ERR_HIP if the device cannot run
 * the workgroups together.  Calls that share a workspace must not overlap.
 * ------------------------------------------------------------------------ */
#define BITNET_MAX_STAGES 256

size_t bitnet_stages_workspace_bytes(int64_t M, const bitnet_problem *problems_host,
                                     int32_t count);

bitnet_status bitnet_ternary_matmul_stages(int64_t M, const bitnet_problem *problems_dev,
                                           int32_t count, const int32_t *stage_end,
                                           int32_t nstages, const bitnet_problem *problems_host,
                                           void *workspace, size_t workspace_bytes,
                                           void *stream);

#ifdef __cplusplus
}
#endif

#endif /* BITNET_TM_H */
