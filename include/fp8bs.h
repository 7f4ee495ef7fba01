/*
 * fp8bs.h -- C ABI of the block-scaled FP8 library for AMD MI355X (gfx950).
 *
 * The method (DeepSeek-V3 style FP8 training, as described in the codingmall
 * knowledge-base pages "How online quantization in DeepSeek-V3 differs from
 * delayed quantization", "How the unified E4M3 format adds to DeepSeek-V3's
 * efficiency" and "Advantages of using FP8 for GEMM operations in
 * DeepSeek-V3"):
 *   - activations are quantized to E4M3 per 1x128 tile and weights per
 *     128x128 block, each group with its own scale computed on the fly from
 *     the group's current maximum magnitude (no history of maxima);
 *   - the FP8 GEMM promotes its partial sums to FP32 once per 128-wide K
 *     group and applies the activation-tile and weight-block scales there.
 *
 * Numerics (identical on every entry point):
 *   E4M3 is the OCP E4M3FN format (bias 7, max 448, no infinities).
 *   For a group with largest magnitude amax:  a = max(amax, 2^-64),
 *   s = RN32(a / 448) (stored scale), r = RN32(448 / a),
 *   q = E4M3_RNE_saturating(RN32(x * r)).
 *   GEMM:  C[m][n] = sum_kb S_A(m,kb) * S_W(n/128,kb) * P(m,n,kb), where
 *   P is the FP8 x FP8 dot product over the 128 K values of group kb,
 *   accumulated in FP32; the promotion is an FP32 multiply-add.
 *   Inputs are finite.  A NaN or infinite input element is outside the
 *   contract: the codes and scale of the group that holds it are unspecified
 *   (no fault, and every other group is quantized as usual).
 *
 * Conventions for every call:
 *   - All tensor pointers are DEVICE memory owned by the caller.  The library
 *     never allocates or frees device memory.  Its state is a thread-local
 *     record of the last HIP error and a per-device cache of the compute-unit
 *     count (filled on first use by whichever thread calls; safe under
 *     concurrent calls).
 *   - FP8BS_ERR_HIP reports the failure of a launch made by this call only:
 *     an error that an earlier, unrelated HIP call left pending is neither
 *     returned nor cleared.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t passed as
 *     void*; NULL means the default stream).  The return value is a
 *     synchronous status: FP8BS_OK means "validated and enqueued"; a device
 *     fault surfaces at the caller's next synchronisation.  On any other
 *     status nothing has been enqueued.
 *   - Matrices are row-major with K contiguous (A is [M][K], W/B is [N][K],
 *     C is [M][N]); leading dimensions are in elements.
 *   - K must be a positive multiple of 128.  M and N may be any value >= 0
 *     (partial tiles at the edges are handled); a call with M == 0 or N == 0
 *     returns FP8BS_OK and launches nothing.
 *   - Leading dimensions must be >= the row length and multiples of 16;
 *     tensor pointers must be 16-byte aligned.  The GEMMs' lda and ldb must
 *     also be at most 2^24 elements, because the tile copies use 32-bit byte
 *     offsets.  Otherwise FP8BS_ERR_LAYOUT.
 *   - Outputs must not alias inputs.  Calls are thread-safe.
 */
#ifndef FP8BS_H
#define FP8BS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
enum {
  FP8BS_OK = 0,
  FP8BS_ERR_NULL = 1,      /* a required pointer is NULL                     */
  FP8BS_ERR_SHAPE = 2,     /* negative size, K not a multiple of 128, ...    */
  FP8BS_ERR_LAYOUT = 3,    /* leading dimension or alignment not supported   */
  FP8BS_ERR_DTYPE = 4,     /* unknown a_kind / out_kind                      */
  FP8BS_ERR_WORKSPACE = 5, /* workspace missing or smaller than required     */
  FP8BS_ERR_HIP = 6        /* a HIP launch failed (see fp8bs_last_hip_error) */
};

/* out_kind: element type of C. */
enum { FP8BS_OUT_F32 = 0, FP8BS_OUT_BF16 = 1 };

/* a_kind: element type of A in fp8_block_gemm. */
enum { FP8BS_A_E4M3 = 0, FP8BS_A_BF16 = 1 };

/* mode of fp8_quant_act_1x128_delayed: granularity of the history. */
enum { FP8BS_DELAY_TILE = 0, FP8BS_DELAY_TENSOR = 1 };
/* op ids for fp8bs_workspace_bytes. */
enum {
  FP8BS_OP_QUANT_ACT = 0,
  FP8BS_OP_QUANT_W = 1,
  FP8BS_OP_GEMM_E4M3 = 2,
  FP8BS_OP_GEMM_BF16 = 3,
  FP8BS_OP_GROUPED_GEMM = 4
};

/*
 * Online activation quantization, one scale per 1x128 tile.
 * Pages: "How online quantization in DeepSeek-V3 differs from delayed
 * quantization", item 1 (scale per 1x128 activation tile, computed on the
 * fly); "How the unified E4M3 format adds to DeepSeek-V3's efficiency",
 * sections "Fine-grained quantization strategy" and "Dynamic scaling and
 * online quantization".
 *
 *   x   [in]  bf16 bit patterns, [M][ldx]; columns 0..K-1 are read.
 *   q   [out] E4M3 codes, [M][ldq].
 *   s   [out] fp32 scales: s(m, kb) is stored at s[kb*lds + m], lds >= M,
 *             for kb = 0..K/128-1 (layout M-contiguous per K group, the order
 *             in which the GEMM reads them).
 * Errors: NULL pointer -> ERR_NULL; M < 0, K <= 0, K % 128 -> ERR_SHAPE;
 *         ldx/ldq < K or not multiples of 16, lds < M, misaligned pointer
 *         -> ERR_LAYOUT.
 */
int fp8_quant_act_1x128(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                        uint8_t* q, int64_t ldq, float* s, int64_t lds,
                        void* stream);

/*
 * Delayed (history-based) scaling of 1x128 activation tiles: the baseline
 * that online scaling is compared against, for measurement.
 * Pages: "How online quantization in DeepSeek-V3 differs from delayed
 * quantization", items 2-4 (delayed quantization takes its scales from the
 * maxima of earlier iterations, kept in a stored history).
 *
 * Step `step` (t >= 0) scales each tile from the largest magnitude over
 * steps t-H .. t-1 (its window) by the online rule above, with
 * a = max(window maximum, 2^-64); a tile whose window maximum is 0 (no
 * history yet) is scaled from its own current maximum.  Values pushed past
 * the format saturate to +-448.
 *   mode  FP8BS_DELAY_TILE:   one history per tile position.  hist is a
 *                             ring of H slots; slot h holds the maxima of a
 *                             step u with u % H == h, tile (m, kb) at
 *                             hist[(h*(K/128) + kb)*ldh + m], ldh >= M.
 *                             The call reads the H slots, then writes this
 *                             step's maxima into slot t % H.
 *         FP8BS_DELAY_TENSOR: one history for the whole tensor.  hist is a
 *                             ring of H + 2 floats; step u in slot
 *                             u % (H + 2).  The call reads the H window
 *                             slots, raises slot t % (H + 2) to this step's
 *                             tensor maximum (atomic max: the slot must hold
 *                             0 or less) and sets slot (t + 1) % (H + 2) to 0
 *                             for the next step.  ldh is ignored.
 *         A history starts as all zeros and is passed to the steps
 *         t = 0, 1, 2, ... in order, on one stream.
 *   x, q, s  as fp8_quant_act_1x128 (s receives the scales used).
 *   stats [in/out] optional uint32[2] (NULL: not counted), accumulated with
 *         atomic adds: [0] += values clipped by saturation (|x*r| > 464,
 *         where round-to-nearest would leave the format), [1] += non-zero
 *         values quantized to a zero code.
 * M == 0 launches nothing and leaves the history unchanged.
 * Errors: as fp8_quant_act_1x128; unknown mode -> ERR_DTYPE; H outside
 *         [1, 4096] or step < 0 -> ERR_SHAPE; hist NULL -> ERR_NULL;
 *         per-tile ldh < M -> ERR_LAYOUT.
 */
int fp8_quant_act_1x128_delayed(const uint16_t* x, int64_t M, int64_t K,
                                int64_t ldx, uint8_t* q, int64_t ldq,
                                float* s, int64_t lds, int mode, float* hist,
                                int64_t ldh, int64_t H, int64_t step,
                                uint32_t* stats, void* stream);
/*
 * Online weight quantization, one scale per 128x128 block.
 * Pages: "How online quantization in DeepSeek-V3 differs from delayed
 * quantization", item 1 (scale per 128x128 weight block); "How the unified
 * E4M3 format adds to DeepSeek-V3's efficiency", section "Fine-grained
 * quantization strategy".
 *
 *   w   [in]  bf16 bit patterns, [N][ldw].
 *   q   [out] E4M3 codes, [N][ldq].
 *   s   [out] fp32 scales, row-major [ceil(N/128)][K/128]:
 *             s(nb, kb) at s[nb*(K/128) + kb].  A partial last band (N not a
 *             multiple of 128) takes its maximum over its valid rows.
 * Errors: as fp8_quant_act_1x128.
 */
int fp8_quant_w_128x128(const uint16_t* w, int64_t N, int64_t K, int64_t ldw,
                        uint8_t* q, int64_t ldq, float* s, void* stream);

/*
 * Both operands of a forward linear layer, y = x . W^T, quantized in one
 * launch: exactly fp8_quant_act_1x128 on x and fp8_quant_w_128x128 on W
 * (same codes, scales and layouts), with one launch's ramp and drain instead
 * of two.  Pages: as those two calls (the activation and the weight are both
 * quantized online, on every step).
 *
 *   x, q, s, ldx, ldq, lds  as fp8_quant_act_1x128 (M rows).
 *   w, qw, sw, ldw, ldqw    as fp8_quant_w_128x128's w, q, s, ldw, ldq
 *                           (N rows).
 *   K is shared.  M == 0 or N == 0 skips that operand (its pointers are not
 *   read); both zero launches nothing.
 * Errors: K not a positive multiple of 128, M < 0 or N < 0 -> ERR_SHAPE;
 *         a NULL pointer of a non-empty operand -> ERR_NULL; that operand's
 *         layout or alignment as in the single calls -> ERR_LAYOUT.
 */
int fp8_quant_linear(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                     uint8_t* q, int64_t ldq, float* s, int64_t lds,
                     const uint16_t* w, int64_t N, int64_t ldw, uint8_t* qw,
                     int64_t ldqw, float* sw, void* stream);

/*
 * Quantization in groups of 128 consecutive rows per column, with the codes
 * written transposed: the operands of the weight-gradient GEMM
 * dW[N][K] = dY^T . X of the backward pass, which contracts over the M
 * tokens (both dY [M][N] and X [M][K] go through this call).
 * Pages: "How the unified E4M3 format adds to DeepSeek-V3's efficiency",
 * section "Fine-grained quantization strategy" (E4M3 with fine-grained
 * groups in every stage of training); reading: groups of 128 along the
 * GEMM's contraction dimension, so these are the 1x128 tiles of x^T,
 * quantized by the online rule.
 *
 *   x   [in]  bf16 bit patterns [M][ldx], ldx >= N.
 *   qt  [out] E4M3 codes of x^T, [N][ldqt] (row n holds x[0..M-1][n]);
 *             ldqt >= M, a multiple of 16; 16-byte aligned.
 *   st  [out] fp32 scales: st(n, mb) at st[mb*ldst + n], ldst >= N (the
 *             activation-scale layout for a GEMM whose rows are the n).
 * Errors: M or N not a multiple of 128 -> ERR_SHAPE; as
 *         fp8_quant_act_1x128 otherwise.
 */
int fp8_quant_act_128x1_t(const uint16_t* x, int64_t M, int64_t N,
                          int64_t ldx, uint8_t* qt, int64_t ldqt, float* st,
                          int64_t ldst, void* stream);
/*
 * fp8_quant_w_128x128 that also writes the codes transposed, the B operand
 * of the data-gradient GEMM dX = dY . W of the backward pass (there the
 * contraction runs over N).  The 128x128 blocks and their scales are the same
 * for W and W^T; only the layouts change.
 * Pages: "How the unified E4M3 format adds to DeepSeek-V3's efficiency",
 * section "Fine-grained quantization strategy" (E4M3 with the same
 * fine-grained groups in every stage of training, the backward pass
 * included); reading: the groups stay 128x128 blocks of W.
 *
 *   w, q, s  as fp8_quant_w_128x128 (N must be a multiple of 128).
 *   qt  [out] E4M3 codes of W^T, [K][ldqt] (row k holds W[0..N-1][k]);
 *             ldqt >= N, a multiple of 16; 16-byte aligned.
 *   st  [out] fp32 scales of W^T's blocks, row-major [K/128][N/128]:
 *             st[kb*(N/128) + nb] = s[nb*(K/128) + kb].
 *   (qt, st) is the (b, sb) of fp8_block_gemm for dX[M][K] = dY[M][N] . W,
 *   with the GEMM's contraction length N.
 * Errors: as fp8_quant_w_128x128; N % 128 != 0 -> ERR_SHAPE.
 */
int fp8_quant_w_128x128_t(const uint16_t* w, int64_t N, int64_t K,
                          int64_t ldw, uint8_t* q, int64_t ldq, float* s,
                          uint8_t* qt, int64_t ldqt, float* st, void* stream);
/*
 * Block-scaled FP8 GEMM with FP32 promotion every 128 K:  C = A . B^T.
 * Pages: "Advantages of using FP8 for GEMM operations in DeepSeek-V3",
 * items 1, 5 and 8 (FP8 GEMM; partial sums promoted to FP32 registers at
 * fixed intervals); "How the unified E4M3 format adds to DeepSeek-V3's
 * efficiency", section "Enhanced numerical stability".
 *
 *   a_kind  FP8BS_A_E4M3: a is E4M3 codes [M][lda] and sa (input) holds the
 *                         activation scales, sa(m,kb) at sa[kb*ldsa + m].
 *           FP8BS_A_BF16: a is bf16 bit patterns [M][lda], quantized per
 *                         1x128 tile inside the call exactly as
 *                         fp8_quant_act_1x128 would; sa may be NULL, else the
 *                         computed scales are written there (same layout).
 *                         Needs a workspace of
 *                         fp8bs_workspace_bytes(FP8BS_OP_GEMM_BF16, M, N, K, 0).
 *   b, sb   E4M3 weight codes [N][ldb] and block scales
 *           [ceil(N/128)][K/128] (layout of fp8_quant_w_128x128).
 *   c       output [M][ldc], fp32 or bf16 (round-to-nearest-even) by out_kind.
 * Errors: as above; unknown a_kind/out_kind -> ERR_DTYPE; workspace too
 *         small -> ERR_WORKSPACE.
 */
int fp8_block_gemm(int a_kind, const void* a, int64_t lda, float* sa,
                   int64_t ldsa, const uint8_t* b, int64_t ldb,
                   const float* sb, void* c, int64_t ldc, int out_kind,
                   int64_t M, int64_t N, int64_t K, void* workspace,
                   size_t workspace_bytes, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * fp8_block_gemm with a bf16 A (a_kind FP8BS_A_BF16) whose in-call E4M3
 * codes and scales go to a fixed device buffer of the library instead of a
 * caller workspace.  The buffer, FP8BS_NOALLOC_SCRATCH_BYTES bytes, is a
 * static device array: every GPU that loads the library holds its own copy
 * until the process ends.  The call allocates nothing (no hipMalloc or
 * hipFree, no allocating library routine).
 *
 *   a       [in]  bf16 [M][lda]; sa [out, may be NULL] fp32 scales
 *                 sa(m, kb) at sa[kb*ldsa + m], ldsa >= M.
 *   b, sb, c, ldc, out_kind, M, N, K, stream  as fp8_block_gemm.
 * Sizes: needs fp8bs_workspace_bytes(FP8BS_OP_GEMM_BF16, M, N, K, 0) <=
 *   FP8BS_NOALLOC_SCRATCH_BYTES (M <= 1134 rows at K = 7168);
 *   larger -> FP8BS_ERR_WORKSPACE, before any HIP call.
 * Sharing: every call on one GPU uses that GPU's one buffer, which keeps the
 *   last call's contents.  Calls ordered on one stream are safe; calls that
 *   overlap on one GPU (several streams, or threads without ordering) race
 *   and give undefined results.
 * Errors: as fp8_block_gemm (FP8BS_ERR_HIP also if the buffer's device
 *   address cannot be looked up).
 */
#define FP8BS_NOALLOC_SCRATCH_BYTES (8u * 1024u * 1024u)
int fp8_block_gemm_bf16_noalloc(const uint16_t* a, int64_t lda, float* sa,
                                int64_t ldsa, const uint8_t* b, int64_t ldb,
                                const float* sb, void* c, int64_t ldc,
                                int out_kind, int64_t M, int64_t N, int64_t K,
                                void* stream);

/*
 * fp8_block_gemm with the output quantized for the next FP8 GEMM: C is
 * computed exactly as by fp8_block_gemm (FP32 accumulator) and then
 * quantized per 1x128 tile along N by the online rule above, inside the
 * GEMM, so that (qc, sc) can be passed on as the E4M3 activation (a, sa) of
 * a following GEMM with K' = N.
 * Pages: "Advantages of using FP8 for GEMM operations in DeepSeek-V3",
 * items 1 and 8 (FP8 GEMMs throughout the layers); "How online quantization
 * in DeepSeek-V3 differs from delayed quantization", item 1 (activations
 * quantized per 1x128 tile from their current values); "How the unified
 * E4M3 format adds to DeepSeek-V3's efficiency", section "Fine-grained
 * quantization strategy".
 *
 *   a, sa, b, sb, workspace  as fp8_block_gemm.
 *   qc   [out] E4M3 codes [M][ldqc]; ldqc >= N, a multiple of 16; 16-byte
 *              aligned.
 *   sc   [out] fp32 scales: sc(m, nb) at sc[nb*ldsc + m] for
 *              nb = 0..N/128-1, ldsc >= M (the layout of sa).
 * Errors: as fp8_block_gemm; N not a multiple of 128 -> ERR_SHAPE; sc NULL
 *         -> ERR_NULL; ldsc < M -> ERR_LAYOUT.
 */
int fp8_block_gemm_e4m3_out(int a_kind, const void* a, int64_t lda, float* sa,
                            int64_t ldsa, const uint8_t* b, int64_t ldb,
                            const float* sb, uint8_t* qc, int64_t ldqc,
                            float* sc, int64_t ldsc, int64_t M, int64_t N,
                            int64_t K, void* workspace,
                            size_t workspace_bytes, void* stream);
/*
 * Block-scaled FP8 GEMM with one scale per row and 128-K group on both
 * operands:  C[m][n] = sum_kb sa(m,kb) * sb(n,kb) * P(m,n,kb), P the FP8 x FP8
 * dot product of group kb accumulated in FP32, promoted with one FP32
 * multiply-add per group.  This is the weight-gradient GEMM
 * dW[N][K] = dY^T . X: a = dY^T and b = X^T from fp8_quant_act_128x1_t,
 * the GEMM's K being the token count.
 * Pages: "Advantages of using FP8 for GEMM operations in DeepSeek-V3",
 * items 1 and 5 (FP8 GEMMs with FP32 promotion at fixed intervals); "How
 * the unified E4M3 format adds to DeepSeek-V3's efficiency", section
 * "Fine-grained quantization strategy" (the same format in the backward
 * pass).
 *
 *   a, sa   E4M3 codes [M][lda], sa(m,kb) at sa[kb*ldsa + m], ldsa >= M.
 *   b, sb   E4M3 codes [N][ldb], sb(n,kb) at sb[kb*ldsb + n], ldsb >= N.
 *   c       [M][ldc], fp32 or bf16 by out_kind.
 * Errors: as fp8_block_gemm.
 */
int fp8_block_gemm_rowscaled(const uint8_t* a, int64_t lda, const float* sa,
                             int64_t ldsa, const uint8_t* b, int64_t ldb,
                             const float* sb, int64_t ldsb, void* c,
                             int64_t ldc, int out_kind, int64_t M, int64_t N,
                             int64_t K, void* stream);
/*
 * MoE weight gradients in one launch: for every expert g,
 *   C_g[M][N] = A[:, t0:t1] . B[:, t0:t1]^T,  [t0, t1) = [off[g], off[g+1]),
 * the row-scaled GEMM of fp8_block_gemm_rowscaled over the expert's token
 * columns.  A = dY^T and B = X^T of all experts' tokens, each expert's tokens
 * zero-padded to a multiple of 128 (zero rows raise no maximum and add
 * nothing), both quantized by fp8_quant_act_128x1_t.
 * Pages: "Advantages of using FP8 for GEMM operations in DeepSeek-V3",
 * items 5 and 8 (FP8 GEMMs with FP32 promotion, for dense and MoE layers);
 * "How the unified E4M3 format adds to DeepSeek-V3's efficiency", section
 * "Fine-grained quantization strategy" (the same format in the backward
 * pass).
 *
 *   a, sa   codes [M][lda] (lda >= K_total), sa(m, j) at sa[j*ldsa + m] for
 *           the 128-token groups j = 0 .. K_total/128 - 1.
 *   b, sb   codes [N][ldb], sb(n, j) at sb[j*ldsb + n].
 *   c       outputs: C_g starts at c + g*c_group_stride (elements), rows of
 *           ldc; fp32 or bf16 by out_kind.  An expert without tokens gets
 *           C_g = 0.
 *   group_offsets DEVICE int32 [G+1], 0 = off[0] <= ... <= off[G] = K_total,
 *           every offset a multiple of 128.  Not validated (read on the
 *           device): each range is clamped to [0, K_total] with its end at
 *           least its start, and an offset that is not a multiple of 128 is
 *           rounded down; results for such offsets are unspecified but no
 *           access leaves the operands.
 * Errors: as fp8_block_gemm_rowscaled; G outside [1, 4096] or K_total not a
 *         multiple of 128 -> ERR_SHAPE; c_group_stride < (M-1)*ldc + N ->
 *         ERR_LAYOUT.
 */
int fp8_block_kgrouped_gemm_rowscaled(const uint8_t* a, int64_t lda,
                                      const float* sa, int64_t ldsa,
                                      const uint8_t* b, int64_t ldb,
                                      const float* sb, int64_t ldsb, void* c,
                                      int64_t ldc, int64_t c_group_stride,
                                      int out_kind,
                                      const int32_t* group_offsets, int64_t G,
                                      int64_t M, int64_t N, int64_t K_total,
                                      void* stream);
/*
 * Grouped (MoE) block-scaled FP8 GEMM: rows group_offsets[g] ..
 * group_offsets[g+1]-1 of A are multiplied by expert g's weight.
 * Pages: "Advantages of using FP8 for GEMM operations in DeepSeek-V3",
 * item 8 (the FP8 GEMM serves dense and MoE layers).
 *
 *   a, sa         E4M3 codes [M_total][lda], scales sa(m,kb) at
 *                 sa[kb*ldsa + m] (rows sorted by expert).
 *   b             expert weights: expert g's [N][ldb] codes start at
 *                 b + g*b_group_stride (bytes; multiple of 16).
 *   sb            block scales sb(g,nb,kb) at
 *                 sb[(g*ceil(N/128) + nb)*(K/128) + kb].
 *   group_offsets DEVICE int32 [G+1], 0 = off[0] <= off[1] <= ... <=
 *                 off[G] = M_total.  Read on the device (no host
 *                 synchronisation), so not validated: the kernel clamps each
 *                 group's range to [0, M_total] (and its end to at least its
 *                 start), so offsets outside this contract give unspecified
 *                 results but no access outside the operands.  Empty groups
 *                 are allowed and write nothing.
 * Errors: as above; G < 1 or G > 4096 -> ERR_SHAPE.
 */
int fp8_block_grouped_gemm(const uint8_t* a, int64_t lda, const float* sa,
                           int64_t ldsa, const uint8_t* b, int64_t ldb,
                           int64_t b_group_stride, const float* sb, void* c,
                           int64_t ldc, int out_kind,
                           const int32_t* group_offsets, int64_t G,
                           int64_t M_total, int64_t N, int64_t K,
                           void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * fp8_block_grouped_gemm with E4M3 output quantized per 1x128 tile along N,
 * as fp8_block_gemm_e4m3_out (same pages).  qc [M_total][ldqc] codes and
 * sc(m, nb) at sc[nb*ldsc + m], ldsc >= M_total; every row 0..M_total-1
 * gets its codes and scales.
 * Errors: as fp8_block_grouped_gemm; N not a multiple of 128 -> ERR_SHAPE;
 *         sc NULL -> ERR_NULL; ldsc < M_total -> ERR_LAYOUT.
 */
int fp8_block_grouped_gemm_e4m3_out(const uint8_t* a, int64_t lda,
                                    const float* sa, int64_t ldsa,
                                    const uint8_t* b, int64_t ldb,
                                    int64_t b_group_stride, const float* sb,
                                    uint8_t* qc, int64_t ldqc, float* sc,
                                    int64_t ldsc, const int32_t* group_offsets,
                                    int64_t G, int64_t M_total, int64_t N,
                                    int64_t K, void* workspace,
                                    size_t workspace_bytes, void* stream);
/* Workspace bytes an entry point needs for the given sizes (0 if none). */
size_t fp8bs_workspace_bytes(int op, int64_t M, int64_t N, int64_t K,
                             int64_t G);

/* Static description of a status code. */
const char* fp8bs_status_string(int status);

/* hipError_t of the last failed HIP call on this thread (0 if none). */
int fp8bs_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FP8BS_H */
