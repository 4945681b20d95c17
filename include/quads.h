/*
 * quads.h -- C ABI of the QUADS rollout hot path on MI355X (gfx950).
 *
 * The method is "QUADS: Stabilizing NVFP4 Reinforcement Learning for MoE via
 * QUantization-error Alignment across Dual Sides" (arXiv 2607.15810): NVFP4
 * activation quantization (section 2.2, "FP4" paragraph; Eq. (9)), Residual
 * Activation Compensation (section 3.3, Eq. (20)-(24)) and the W4A4 product
 * (Eq. (6), (21)), here for MoE expert layers.
 *
 * Conventions shared by every call
 *  - Pointers are device pointers unless stated.  bf16 tensors are passed as
 *    uint16_t bit patterns.  Every tensor is dense and row-major.  Every
 *    pointer must be 16-byte aligned.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *    stream).  No call synchronizes with the host, allocates memory or keeps
 *    a pointer after it returns (quads_rac_quantize_noalloc keeps its own
 *    static scratch).  Scalars produced on the device (tensor
 *    scales, selected channels, expert offsets) stay on the device.
 *  - Scratch memory is caller-owned: `ws` must hold at least the bytes the
 *    matching *_ws() query returns for the same sizes (NULL is allowed when
 *    that is 0).  Calls that share a workspace must be ordered on one stream.
 *  - Argument checks run on the host before any launch.  A failed check
 *    returns QUADS_EINVAL (null or misaligned pointer, bad enum),
 *    QUADS_ESHAPE (a size rule below), QUADS_EWORKSPACE or QUADS_ESCRATCH
 *    (input too large for a no-allocation call's static scratch); nothing is
 *    launched then.  A failed launch returns QUADS_EHIP; quads_status_string
 *    then describes the HIP error of the calling thread.
 *  - Inputs must be finite.  Size-0 tensors (M, T or rows = 0) are a no-op
 *    that returns QUADS_OK (tensor scales are still written as 0 where an
 *    output scale is requested).
 *
 * NVFP4 layout (arXiv 2607.15810, section 2.2 "FP4")
 *  - Element: 4-bit E2M1 code, bit 3 = sign, bits 2..0 = magnitude code
 *    0..7 for 0, 0.5, 1, 1.5, 2, 3, 4, 6.  Two codes per byte; the even
 *    channel is the low nibble.  `nib` of a [rows, K] tensor is [rows, K/2].
 *  - Block scale: one OCP E4M3FN byte (max 448, section 2.2 "FP8") per 16
 *    consecutive channels of a row; `scale` is [rows, K/16].
 *  - Tensor scale: one fp32.  Value of an element = v * s_b * s_t.
 *  - Quantization: s_t = RN32(max|x| / 2688); s_b = min(448, RNE_E4M3(
 *    amax_block / (6 s_t))); code = RNE_E2M1(|x| / (s_b s_t)) saturating at
 *    6, ties to even, sign bit copied from x; s_t = 0 or s_b = 0 give
 *    magnitude 0.  RNE is taken on the exact real quotient.
 */
#ifndef QUADS_H
#define QUADS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    QUADS_OK = 0,
    QUADS_EINVAL = -1,
    QUADS_ESHAPE = -2,
    QUADS_EWORKSPACE = -3,
    QUADS_EHIP = -4,
    QUADS_ESCRATCH = -5
} quads_status;

typedef enum { QUADS_OUT_F32 = 0, QUADS_OUT_BF16 = 1 } quads_out_dtype;
typedef enum { QUADS_EPI_NONE = 0, QUADS_EPI_SWIGLU = 1 } quads_epilogue;
/* MX element formats (the comparator GEMM); the values are the block-scaled
   MFMA's own format codes. */
typedef enum { QUADS_MX_FP8 = 0, QUADS_MX_FP4 = 4 } quads_mx_format;

/* Human-readable text for a status code (thread-local detail for QUADS_EHIP). */
const char* quads_status_string(int status);

/* Library version string, e.g. "quads-mi355x 0.1 gfx950". Host pointer. */
const char* quads_version(void);

/*
 * NVFP4 activation quantization, Q_A of Eq. (9) (section 3.1) with the
 * format of section 2.2.
 *   x       bf16 [M, K], K % 16 == 0
 *   ts_in   NULL: dynamic tensor scale from max|x|;  else a device fp32 used
 *           as s_t (must be finite and >= 0; blocks then saturate at 448 and
 *           codes at 6)
 *   nib     out uint8 [M, K/2];  scale out uint8 [M, K/16]
 *   ts_out  out fp32 [1]: the tensor scale used
 */
size_t quads_nvfp4_quantize_ws(int64_t M, int64_t K);
int quads_nvfp4_quantize(const uint16_t* x, int64_t M, int64_t K, const float* ts_in,
                         uint8_t* nib, uint8_t* scale, float* ts_out,
                         void* ws, size_t ws_bytes, void* stream);

/*
 * quads_nvfp4_quantize with the dynamic tensor scale of Eq. (9) taken from
 * a producer's partial maxima of |x| instead of a max pass over x (one pass
 * over x instead of two), e.g. the ones quads_moe_w4a4_gemm_amax writes for
 * its SwiGLU output.
 *   amax_part  uint32 [groups] (4-byte aligned), groups >= 1: bf16
 *              magnitude bit patterns (|x| as bf16 bits & 0x7FFF) whose
 *              maximum is that of every element of x; nib, scale and ts_out
 *              are then those of quads_nvfp4_quantize(ts_in = NULL) bit for
 *              bit
 * No workspace.  M == 0 writes ts_out = 0.
 */
int quads_nvfp4_quantize_partials(const uint16_t* x, int64_t M, int64_t K,
                                  const uint32_t* amax_part, int64_t groups, uint8_t* nib,
                                  uint8_t* scale, float* ts_out, void* stream);

/*
 * Per-row (per-token) variant of the NVFP4 activation quantization: each
 * row of x is quantized as a tensor of its own, with its own dynamic tensor
 * scale s_t[m] = RN32(max_j |x[m, j]| / 2688) and then the block and element
 * rules of section 2.2's "FP4" paragraph unchanged.  The pages define one
 * FP32 scale per tensor; this form keeps one FP32 value per row so that rows
 * of very different magnitude each use the full E4M3 block-scale range.
 *   x       bf16 [M, K], K % 16 == 0
 *   nib     out uint8 [M, K/2];  scale out uint8 [M, K/16]
 *   ts      out fp32 [M]: the row scales (0 for an all-zero row)
 * No workspace.  M == 0 is a no-op.
 */
int quads_nvfp4_quantize_rows(const uint16_t* x, int64_t M, int64_t K, uint8_t* nib,
                              uint8_t* scale, float* ts, void* stream);

/*
 * Residual Activation Compensation (section 3.3).
 *   x        bf16 [M, K], K % 16 == 0;  k % 16 == 0, 0 <= k <= K
 *   nib, scale, ts    main NVFP4 of x, identical to quads_nvfp4_quantize
 *                     with a dynamic tensor scale
 *   sel      out int32 [k]: S of Eq. (24), the k channels with the largest
 *            score s_j = sum_t r_tj^2 (Eq. (23) squared), ties to the lower
 *            index, ascending.  r = RN32(x - DQ(Q(x))) is the negated error
 *            of Eq. (20).  The sum runs in fp64 in a fixed order: tokens in
 *            groups of 64 summed in order from +0, then those sums in groups
 *            of 64, and so on.
 *   r_nib, r_scale, r_ts  out: NVFP4 of the gathered residual R[t,i] =
 *            r[t, sel[i]] ([M, k/2], [M, k/16], fp32 [1]), quantized like x
 *            with its own dynamic tensor scale.  Then
 *            X~ = DQ(x) + scatter_sel(DQ(R)) is Eq. (21).
 *   score_out  NULL or out fp64 [K]: the channel scores
 * With k == 0 no residual output is written except r_ts = 0 (r_nib,
 * r_scale and sel may then be NULL).
 */
size_t quads_rac_quantize_ws(int64_t M, int64_t K, int32_t k);
int quads_rac_quantize(const uint16_t* x, int64_t M, int64_t K, int32_t k,
                       uint8_t* nib, uint8_t* scale, float* ts,
                       int32_t* sel, uint8_t* r_nib, uint8_t* r_scale, float* r_ts,
                       double* score_out, void* ws, size_t ws_bytes, void* stream);

/*
 * quads_rac_quantize with max|x| (the tensor scale of the main NVFP4 pass)
 * from a producer's partial maxima, as in quads_nvfp4_quantize_partials:
 * the max pass over x is skipped.  amax_part [groups] must have the maximum
 * of |x| (bf16 magnitude bits); every output is then that of
 * quads_rac_quantize bit for bit (inputs of at most 64 rows and 16384
 * elements take the one-launch path, which reads the maximum from x
 * itself).  Workspace and other arguments as quads_rac_quantize.
 */
int quads_rac_quantize_partials(const uint16_t* x, int64_t M, int64_t K, int32_t k,
                                const uint32_t* amax_part, int64_t groups,
                                uint8_t* nib, uint8_t* scale, float* ts,
                                int32_t* sel, uint8_t* r_nib, uint8_t* r_scale, float* r_ts,
                                double* score_out, void* ws, size_t ws_bytes, void* stream);

/*
 * quads_rac_quantize without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Arguments, outputs and results are
 * those of quads_rac_quantize; the workspace is a static device array of
 * QUADS_RAC_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs
 * on until the process ends.  Sizes whose quads_rac_quantize_ws exceeds it
 * return QUADS_ESCRATCH before any launch (the other argument checks come
 * first).  The call runs on the calling thread's current device; `stream`
 * must belong to it.  All calls on one GPU share that GPU's array: calls
 * that may overlap in time on one GPU (different streams, or threads without
 * ordering) race and give undefined results.  The first call on a device
 * looks up the array's address there (no allocation).
 */
#define QUADS_RAC_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int quads_rac_quantize_noalloc(const uint16_t* x, int64_t M, int64_t K, int32_t k,
                               uint8_t* nib, uint8_t* scale, float* ts,
                               int32_t* sel, uint8_t* r_nib, uint8_t* r_scale, float* r_ts,
                               double* score_out, void* stream);

/*
 * RAC with one channel selection per expert (a variant of section 3.3; the
 * paper lists more adaptive residual-channel selection as future work), for
 * activations already in packed expert order (the down-projection input).
 * The main NVFP4 (nib, scale, ts) is that of quads_rac_quantize.  Expert e's
 * rows offsets[e] .. offsets[e+1]-1 are then a tensor of their own for the
 * scores (the same fixed-order sum over its rows alone), the selection S_e
 * (k largest, ties to the lower index, ascending) and the second pass of
 * r[rows_e][:, S_e] with its own dynamic tensor scale.  An expert without
 * rows gets S_e = 0 .. k-1 and a residual scale of 0.
 *   x        bf16 [M, K] in packed order, M <= 64^3, K % 16 == 0, K <= 8192;
 *            E <= 4096
 *   offsets  int32 [E+1], offsets[0] = 0, offsets[E] = M, non-decreasing
 *   sel      out int32 [E, k];  r_ts out fp32 [E]
 *   r_nib, r_scale  out [M, k/2], [M, k/16]: row p in its expert's S_e order
 *   score_out  NULL or out fp64 [E, K]
 */
size_t quads_rac_quantize_experts_ws(int64_t M, int64_t K, int32_t k, int32_t E);
int quads_rac_quantize_experts(const uint16_t* x, int64_t M, int64_t K, int32_t k,
                               const int32_t* offsets, int32_t E,
                               uint8_t* nib, uint8_t* scale, float* ts,
                               int32_t* sel, uint8_t* r_nib, uint8_t* r_scale, float* r_ts,
                               double* score_out, void* ws, size_t ws_bytes, void* stream);

/*
 * Shared NVFP4 weight QDQ, Q_W of Eq. (7) / QDQ_W of Eq. (12): each expert
 * matrix W_e [N, K] (rows = output features, blocks along K) is quantized
 * with its own dynamic tensor scale.
 *   w       bf16 [E, N, K], K % 16 == 0, E >= 1
 *   w_nib   out [E, N, K/2];  w_scale out [E, N, K/16];  w_ts out fp32 [E]
 *   w_dq    NULL or out bf16 [E, N, K]: RNE_bf16 of the exact v*s_b*s_t
 */
size_t quads_nvfp4_weight_qdq_ws(int64_t E, int64_t N, int64_t K);
int quads_nvfp4_weight_qdq(const uint16_t* w, int64_t E, int64_t N, int64_t K,
                           uint8_t* w_nib, uint8_t* w_scale, float* w_ts, uint16_t* w_dq,
                           void* ws, size_t ws_bytes, void* stream);

/*
 * Token-to-expert packing: stable counting sort of the (token, slot) pairs
 * by expert id.  Packed order: experts ascending, then t*topk + slot
 * ascending.
 *   topk_ids  int32 [T, topk], every id in [0, E)
 *   offsets   out int32 [E+1]: rows of expert e are offsets[e] .. offsets[e+1]-1
 *   row_token out int32 [T*topk]: token feeding each packed row
 *   pos       out int32 [T*topk]: packed row of (t, slot) at index t*topk+slot
 */
size_t quads_moe_pack_ws(int64_t T, int32_t topk, int32_t E);
int quads_moe_pack(const int32_t* topk_ids, int64_t T, int32_t topk, int32_t E,
                   int32_t* offsets, int32_t* row_token, int32_t* pos,
                   void* ws, size_t ws_bytes, void* stream);

/*
 * Grouped W4A4 GEMM with the RAC compensation term in the same accumulator
 * (Eq. (6) applied to X~ of Eq. (21)).  For packed row p of expert e and
 * output feature n:
 *   Y[p,n] = s_tA s_tW[e] sum_{j<K} a[row(p), j] w_e[n, j]
 *          + s_tR s_tW[e] sum_{i<k} r[row(p), i] w_e[n, sel[i]]
 * with a, r, w the exact v*s_b values (computed on bf16/fp16-exact MFMA
 * operands, fp32 accumulation).
 *   a_nib, a_scale, a_ts   activation NVFP4 [Ta, K/2], [Ta, K/16], fp32 [1]
 *   row_token  NULL: row(p) = p (Ta = rows);  else int32 [rows], row(p) =
 *              row_token[p] < Ta
 *   r_nib, r_scale, r_ts, sel, k   second pass (quads_rac_quantize layout);
 *              sel must be strictly ascending in [0, K) (as quads_rac_quantize
 *              writes it; other values give undefined results, never
 *              out-of-bounds accesses); k == 0 gives plain W4A4 and these may
 *              be NULL
 *   w_nib, w_scale, w_ts   weights [E, N, K/2], [E, N, K/16], fp32 [E]
 *   offsets    int32 [E+1] with offsets[0] = 0, offsets[E] = rows,
 *              non-decreasing; NULL only when E == 1 (all rows, expert 0)
 *   epilogue   QUADS_EPI_NONE: out [rows, N];
 *              QUADS_EPI_SWIGLU: N even, gate = features [0, N/2), up =
 *              [N/2, N), out bf16 [rows, N/2] = RNE_bf16(silu(g) * u)
 *   out_dtype  QUADS_OUT_F32 or QUADS_OUT_BF16 (SWIGLU requires BF16)
 *   ws         quads_moe_w4a4_gemm_ws bytes: 0 except for contractions with
 *              K % 128 == 0, K <= 8192, K + k > 1152 and k > 256 a multiple
 *              of 128 (such as k = K/2), where it holds W[:, S] of every
 *              expert as fp16 (E * N * k * 2 bytes), gathered by the call
 * The error is below (142 + (K + k)/1024 + 6) 2^-24 sum |a w| per output
 * element, whatever the data: the accumulators restart at least every 1024
 * channels (gfx950's f16 MFMA rounds each group of 8 products once).
 */
size_t quads_moe_w4a4_gemm_ws(int64_t rows, int64_t K, int32_t k, int32_t E, int64_t N);
int quads_moe_w4a4_gemm(const uint8_t* a_nib, const uint8_t* a_scale, const float* a_ts,
                        const int32_t* row_token, int64_t rows, int64_t K,
                        const uint8_t* r_nib, const uint8_t* r_scale, const float* r_ts,
                        const int32_t* sel, int32_t k,
                        const uint8_t* w_nib, const uint8_t* w_scale, const float* w_ts,
                        const int32_t* offsets, int32_t E, int64_t N,
                        int epilogue, int out_dtype, void* out,
                        void* ws, size_t ws_bytes, void* stream);

/*
 * The SwiGLU form of quads_moe_w4a4_gemm (epilogue QUADS_EPI_SWIGLU, bf16
 * out) that also hands the next quantizer the maximum of its output h, so
 * that quantizing h (the down projection's input, Eq. (9) or section 3.3 at
 * the second site) needs no separate max pass: every work-group of the
 * call writes the largest |h| it stored, as bf16 magnitude bits, into its
 * own slot of amax_part (no atomics), and slots no work-group takes are
 * written 0.  The maximum over amax_part[0 .. amax_groups) is then
 * max |h| exactly; pass (amax_part, amax_groups) to
 * quads_nvfp4_quantize_partials or quads_rac_quantize_partials.
 *   amax_part    out uint32 [amax_groups] (4-byte aligned), amax_groups >=
 *                quads_moe_w4a4_gemm_amax_groups for the call's sizes
 *                (QUADS_EWORKSPACE if smaller)
 *   every other argument, the workspace and the error bound as in
 *   quads_moe_w4a4_gemm with epilogue = QUADS_EPI_SWIGLU and out_dtype =
 *   QUADS_OUT_BF16.  rows == 0 writes nothing.
 * quads_moe_w4a4_gemm_amax_groups: the slot count for these sizes (the
 * work-groups of the call's launches, the largest over calls with or
 * without offsets and workspace), or 0 for sizes the GEMM rejects.
 */
int64_t quads_moe_w4a4_gemm_amax_groups(int64_t rows, int64_t K, int32_t k, int32_t E,
                                        int64_t N);
int quads_moe_w4a4_gemm_amax(const uint8_t* a_nib, const uint8_t* a_scale, const float* a_ts,
                             const int32_t* row_token, int64_t rows, int64_t K,
                             const uint8_t* r_nib, const uint8_t* r_scale, const float* r_ts,
                             const int32_t* sel, int32_t k,
                             const uint8_t* w_nib, const uint8_t* w_scale, const float* w_ts,
                             const int32_t* offsets, int32_t E, int64_t N, void* out,
                             uint32_t* amax_part, int64_t amax_groups,
                             void* ws, size_t ws_bytes, void* stream);

/*
 * Grouped W4A4 GEMM with per-row activation tensor scales (the activations
 * of quads_nvfp4_quantize_rows), no compensation term:
 *   Y[p,n] = s_tA[row(p)] s_tW[e] sum_{j<K} a[row(p), j] w_e[n, j]
 *   a_ts_rows  fp32 [Ta]: the scale of each A row
 *   every other argument, the workspace and the rules as in
 *   quads_moe_w4a4_gemm with k == 0 (query quads_moe_w4a4_gemm_ws with k = 0)
 */
int quads_moe_w4a4_gemm_rowscale(const uint8_t* a_nib, const uint8_t* a_scale,
                                 const float* a_ts_rows, const int32_t* row_token,
                                 int64_t rows, int64_t K,
                                 const uint8_t* w_nib, const uint8_t* w_scale, const float* w_ts,
                                 const int32_t* offsets, int32_t E, int64_t N,
                                 int epilogue, int out_dtype, void* out,
                                 void* ws, size_t ws_bytes, void* stream);

/*
 * Grouped W4A4 GEMM with the per-expert compensation of
 * quads_rac_quantize_experts: packed row p of expert e takes
 *   s_tR[e] s_tW[e] sum_{i<k} r[p, i] w_e[n, sel[e, i]]
 * as its second term.  Activations in packed order (no row_token; row p is
 * activation row p); sel int32 [E, k], each row strictly ascending in
 * [0, K); r_ts fp32 [E]; offsets required.  Everything else as in
 * quads_moe_w4a4_gemm (same workspace query).
 */
int quads_moe_w4a4_gemm_sel_experts(const uint8_t* a_nib, const uint8_t* a_scale,
                                    const float* a_ts, int64_t rows, int64_t K,
                                    const uint8_t* r_nib, const uint8_t* r_scale,
                                    const float* r_ts, const int32_t* sel, int32_t k,
                                    const uint8_t* w_nib, const uint8_t* w_scale,
                                    const float* w_ts, const int32_t* offsets, int32_t E,
                                    int64_t N, int epilogue, int out_dtype, void* out,
                                    void* ws, size_t ws_bytes, void* stream);

/*
 * MoE combine: out[t, n] = sum over slots in order of topk_w[t, slot] *
 * y[pos[t*topk + slot], n], accumulated in fp32.
 *   y        [T*topk, N], fp32 (y_dtype QUADS_OUT_F32) or bf16 (QUADS_OUT_BF16)
 *   topk_w   fp32 [T, topk];  out fp32 [T, N];  N % 8 == 0
 */
int quads_moe_combine(const void* y, int y_dtype, const int32_t* pos, const float* topk_w,
                      int64_t T, int32_t topk, int64_t N, float* out, void* stream);

/*
 * MX block-scaled comparator (the FP8 W8A8 baseline of section 4.4.2 and
 * Fig. 9(a), with the fine-grained block scaling of section 2.2's "FP8"
 * paragraph in the form gfx950's block-scaled MFMA takes).  Not part of the
 * NVFP4 method: it exists so the method's GEMM can be measured against FP8
 * on the same hardware.
 *
 * MX quantization of bf16 x [M, K] (K % 32 == 0), per row, blocks of 32:
 * E = floor(log2 max|x|) - emax (emax 8 for FP8 E4M3, 2 for FP4 E2M1),
 * clamped to [-127, 127], -127 for an all-zero block; scale byte E + 127;
 * element = RNE(x / 2^E) on the element grid, saturated (448 / 6), sign of
 * x kept.
 *   fmt     QUADS_MX_FP8: codes uint8 [M, K] (OCP E4M3FN bytes);
 *           QUADS_MX_FP4: codes uint8 [M, K/2] (even element in the low nibble)
 *   scales  uint8 [M, K/32]
 */
int quads_mx_quantize(const uint16_t* x, int64_t M, int64_t K, int fmt, uint8_t* codes,
                      uint8_t* scales, void* stream);

/*
 * Grouped MX GEMM: Y[p, n] = sum_k a[row(p), k] w_e[n, k] with a and w the
 * decoded MX values (products exact, fp32 accumulation in the MFMA).
 *   a_codes, a_scale   quads_mx_quantize layout, [Ta, ...], [Ta, K/32]
 *   row_token, rows, offsets, E, N, epilogue, out_dtype, out   as in
 *              quads_moe_w4a4_gemm (same packed-row and output conventions)
 *   w_codes, w_scale   [E, N, ...], [E, N, K/32]
 *   fmt        QUADS_MX_FP8 or QUADS_MX_FP4 (both operands)
 *   K % 128 == 0.  No workspace.
 */
int quads_moe_mx_gemm(const uint8_t* a_codes, const uint8_t* a_scale, const int32_t* row_token,
                      int64_t rows, int64_t K, const uint8_t* w_codes, const uint8_t* w_scale,
                      const int32_t* offsets, int32_t E, int64_t N, int fmt, int epilogue,
                      int out_dtype, void* out, void* stream);

/*
 * RAC on the MX FP4 mode (section 3.3 with the MX FP4 format that the "FP4"
 * paragraph of section 2.2 sets beside NVFP4).
 *   x        bf16 [M, K], K % 32 == 0, K <= 8192;  k % 32 == 0, 0 <= k <= K
 *   codes, scales   MX FP4 of x, identical to quads_mx_quantize
 *   sel      out int32 [k]: the k channels with the largest sum over rows of
 *            r^2, r = x - DQ(Q(x)) (exact in fp32), in the fixed order and with
 *            the tie rule of quads_rac_quantize; ascending
 *   r_codes, r_scales   out: MX FP4 of the gathered residual R[t, i] =
 *            r[t, sel[i]] ([M, k/2], [M, k/32]: 32-element blocks along the
 *            compacted index).  X~ = DQ(Q(x)) + scatter_sel(DQ(R)) is Eq. (21).
 *   score_out  NULL or out fp64 [K]: the channel scores
 * Workspace: quads_mx_rac_quantize_ws bytes.  With k == 0 only the codes
 * (and the scores, when asked) are written; sel, r_codes, r_scales may be NULL.
 */
size_t quads_mx_rac_quantize_ws(int64_t M, int64_t K, int32_t k);
int quads_mx_rac_quantize(const uint16_t* x, int64_t M, int64_t K, int32_t k,
                          uint8_t* codes, uint8_t* scales, int32_t* sel,
                          uint8_t* r_codes, uint8_t* r_scales, double* score_out,
                          void* ws, size_t ws_bytes, void* stream);

/*
 * Grouped MX FP4 GEMM with the RAC compensation term (Eq. (21) into Eq. (6)
 * on the MX FP4 mode): for packed row p of expert e and feature n
 *   Y[p,n] = sum_{j<K} a[row(p), j] w_e[n, j] + sum_{i<k} r[row(p), i] w_e[n, sel[i]]
 * with a, r, w the decoded MX FP4 values.  The main sum runs on the
 * block-scaled FP4 MFMA, the compensation on bf16 MFMAs (MX FP4 values are
 * exact in bf16) into the same fp32 accumulators.
 *   a_codes, a_scale, r_codes, r_scale, sel, k   quads_mx_rac_quantize's
 *              outputs (sel strictly ascending in [0, K)); k == 0 is
 *              quads_moe_mx_gemm with QUADS_MX_FP4
 *   the other arguments as in quads_moe_mx_gemm (K % 128 == 0)
 *   ws         quads_moe_mx_rac_gemm_ws bytes (W[:, S] as bf16, E * N * k * 2)
 */
size_t quads_moe_mx_rac_gemm_ws(int32_t E, int64_t N, int32_t k);
int quads_moe_mx_rac_gemm(const uint8_t* a_codes, const uint8_t* a_scale,
                          const int32_t* row_token, int64_t rows, int64_t K,
                          const uint8_t* r_codes, const uint8_t* r_scale, const int32_t* sel,
                          int32_t k, const uint8_t* w_codes, const uint8_t* w_scale,
                          const int32_t* offsets, int32_t E, int64_t N, int epilogue,
                          int out_dtype, void* out, void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QUADS_H */
