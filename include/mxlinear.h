/*
 * mxlinear.h -- C ABI of libmxlinear.so, the MI355X (gfx950) library for the
 * W4A4 microscaling linear layer:
 *
 *   (a) round-to-nearest weight packing to MXFP4 (E2M1 elements, one E8M0
 *       scale per 32 elements, EVEN scale rule),
 *   (b) dynamic per-token activation quantization to MXFP4 (CEIL rule),
 *   (c) the block-scaled FP4 x FP4 GEMM with fp32 accumulation and a bf16
 *       output,
 * and the same path for MXFP8 (E4M3 elements, E8M0 per 32) and NVFP4 (E2M1
 * elements, an E4M3 scale per 16, a per-tensor fp32 global scale).
 *
 * Passages defining the operations (model-card pages):
 *  - Qwen3.5-27B-MXFP4-QAD-W4A4-LR1e-5-s1000, "How this checkpoint was
 *    produced": MXFP4 weights are E2M1 in blocks of 32 with EVEN-rule E8M0
 *    scales; activations are quantized dynamically.
 *  - Qwen3.5-9B-MXFP4-QAD-W4A4-LR1e-5-s3000, "Training mode": activations are
 *    quantized per token in blocks of 32 to E2M1 with CEIL-rule UE8M0 scales,
 *    a rule distinct from the weights' EVEN rule; "Serving": the packed format
 *    (E2M1 weights, block-32 E8M0 scales) and the W4A4 FP4 GEMM with
 *    activations quantized per token at run time.
 *  - Qwen3.5-27B-NVFP4-RTN-weight-only (introduction, "How this checkpoint was
 *    produced") and Qwen3.5-27B-NVFP4-GPTQ (introduction): NVFP4 weights
 *    rounded to the lattice, per-tensor input global scales.
 *  - Qwen3.8-27B-MXFP8Attn-MXFP4MLP-lmheadMXFP4, introduction and sections 1,
 *    2 and 7: MXFP8 = E4M3 + E8M0 per group of 32, MXFP4 = E2M1 + E8M0,
 *    symmetric, dynamic activations, OCP Microscaling formats; the prior FP8
 *    kernel rejected N < 128, which this library does not.
 *
 * Conventions for every entry point:
 *  - All tensors are dense, row-major, contiguous device buffers owned by the
 *    caller.  The library never allocates, frees or keeps a pointer after the
 *    call returns, and keeps no per-call state.
 *  - bf16 tensors are arrays of uint16_t bit patterns.
 *  - Block layout: a block is 32 (MX) or 16 (NVFP4) consecutive elements
 *    along K of one row.  E2M1 codes are packed two per byte, element 2j in
 *    the low nibble of byte j: a [rows, K] tensor occupies rows * K/2 bytes.
 *    E4M3 codes take one byte each.  Scales form a [rows, K/32] (E8M0) or
 *    [rows, K/16] (E4M3) byte plane.
 *  - GEMM orientation: Y[M, N] = A[M, K] * W[N, K]^T (W as nn.Linear stores
 *    it), fp32 accumulation, Y written as bf16 (or fp32 with MX_OUT_F32).
 *  - Every call only enqueues work on `stream` (0 = the null stream) and never
 *    synchronizes the host.
 *  - Arguments are validated before any HIP call.  On an error nothing is
 *    enqueued and a status code comes back.  Kernels never trap; non-finite
 *    inputs are outside the contract (unspecified output, no crash).
 *  - Functions are thread-safe.
 *  - GEMM error bound and its domain.  Every GEMM meets, per output element,
 *        |y - y_exact| <= 1e-4 * S + F + (K/16 + 1) * 2^-126
 *    (plus half a bf16 ulp of the result when Y is bf16), where S =
 *    sum_k |a_k w_k| over the dequantized operands and F is the part of S
 *    contributed by terms with an operand value below 2^-126, the smallest
 *    normal fp32.  For operands in the normal fp32 range (F = 0) and results
 *    above 2^-126 * K this is the 1e-4 * S bound.  Below that range values
 *    are rounded: the dequantizing kernels hold operands in bf16, so MXFP8
 *    values below 2^-126 (blocks with scales below 2^-117) become the
 *    nearest bf16 subnormal (ties to even), and an fp32 accumulator may lose
 *    sums below 2^-126, at most once per 16-wide step.
 *  - Workspaces.  A GEMM that can use device scratch takes (workspace,
 *    ws_bytes); NULL/0 is always valid and selects the variant that needs
 *    none, except for mx_gemm_fused with a mixed pair.  A non-NULL workspace
 *    smaller than the size query's answer for the same arguments returns
 *    MX_ERR_WORKSPACE.  Calls sharing a workspace must not overlap in time.
 */
#ifndef MXLINEAR_H
#define MXLINEAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* A HIP stream handle (hipStream_t); declared opaque so that callers need no
 * HIP headers. */
typedef void* mx_stream_t;

/* Each enum carries two range markers so that its type holds every int:
 * a caller may pass any int where an enum is expected, and the functions
 * reject unknown values with MX_ERR_INVALID_ARG (or describe them, for
 * mx_status_string) instead of reading an out-of-range enum value. */
typedef enum {
    MX_OK = 0,
    MX_ERR_INVALID_ARG = 1, /* null pointer, unknown enum, bad format/rule pair */
    MX_ERR_SHAPE = 2,       /* m, n or k < 1; k not a multiple of the block */
    MX_ERR_ALIGN = 3,       /* a pointer is not 16-byte aligned (256 for the quantize-once workspace) */
    MX_ERR_WORKSPACE = 4,   /* a non-NULL workspace smaller than the call needs, or none where one is required */
    MX_ERR_UNSUPPORTED = 5, /* device is not gfx950, or the selected kernel cannot address operands this large */
    MX_ERR_HIP = 6,         /* a HIP runtime call or launch failed */
    MX_STATUS_RANGE_MIN_ = -2147483647 - 1, MX_STATUS_RANGE_MAX_ = 2147483647
} mx_status;

typedef enum {
    MX_FMT_MXFP4 = 0, /* E2M1 elements, E8M0 scale per 32 */
    MX_FMT_MXFP8 = 1, /* E4M3 elements, E8M0 scale per 32 */
    MX_FMT_NVFP4 = 2, /* E2M1 elements, E4M3 scale per 16, fp32 global scale */
    MX_FMT_RANGE_MIN_ = -2147483647 - 1, MX_FMT_RANGE_MAX_ = 2147483647
} mx_format;

typedef enum {
    MX_RULE_FLOOR = 0, /* e = floor(log2 amax) - emax (OCP MX v1.0) */
    MX_RULE_CEIL = 1,  /* smallest e with amax <= max_elem * 2^e (activations) */
    MX_RULE_EVEN = 2,  /* amax rounded to the element's mantissa width, then FLOOR (weights) */
    MX_RULE_RANGE_MIN_ = -2147483647 - 1, MX_RULE_RANGE_MAX_ = 2147483647
} mx_scale_rule;

/* GEMM flags */
#define MX_OUT_F32 0x1u  /* write Y as fp32 instead of bf16 */
#define MX_FP8_FAST 0x2u /* pairs with an MXFP8 operand: contract on the block-scaled FP8
                          * (or FP8 x FP4) matrix cores (about 2x the throughput); their
                          * internal accumulation is inexact, with errors measured up to
                          * ~2e-4 * sum|a*b|, so this opts out of the 1e-4 bound that the
                          * default path meets (documented bound 5e-4 * sum|a*b|) */
#define MX_DEBUG_DUMP_AQ 0x4u /* mx_gemm_fused only: also write the prologue's A codes and scales
                                 to the workspace (see mx_gemm_fused) */
#define MX_FUSED_IN_GEMM 0x8u /* mx_gemm_fused only: on the quantize-once shapes, quantize A inside
                                 the GEMM's own launches (see mx_gemm_fused) */

/* ABI version of this header (bumped on any signature change). */
#define MXLINEAR_ABI_VERSION 8
int mx_abi_version(void);

/* Static text for a status code; never NULL. */
const char* mx_status_string(mx_status status);

/*
 * mx_quantize_act -- dynamic per-token activation quantization: per token
 * row, blocks of 32 along k to E2M1 with a CEIL-rule UE8M0 scale, computed
 * at run time with no calibration state (Qwen3.5-9B-MXFP4-QAD-W4A4-LR1e-5-
 * s3000, "Training mode"); MXFP8 activations are dynamic too
 * (Qwen3.8-27B-MXFP8Attn-MXFP4MLP-lmheadMXFP4, section 2); NVFP4 uses the
 * static per-tensor input global scale (Qwen3.5-27B-NVFP4-GPTQ,
 * introduction).
 * a_bf16: [m, k] bf16.  Outputs a_q and a_s in the block layout above.
 *  fmt MXFP4 or MXFP8: one E8M0 scale per 32 along k, chosen by `rule`
 *    (CEIL is the activation rule); element = RNE(x * 2^-e), ties to the even
 *    code, saturating at the largest magnitude (6 or 448); the sign bit copies
 *    the input's sign; an all-zero block gets scale byte 0.
 *  fmt NVFP4: `global_scale` g is the tensor's encode scale (see
 *    mx_nv_global_scale); per 16 along k: s = RNE_E4M3(amax * g / 6),
 *    element = RNE_E2M1(x * g / s), both of the exact real values; `rule` is
 *    ignored.
 * Requires k % 32 == 0 (MX) or k % 16 == 0 (NVFP4) and 16-byte aligned
 * pointers.  Each block is quantized independently, so the result does not
 * depend on how rows are batched.
 */
mx_status mx_quantize_act(mx_format fmt, mx_scale_rule rule, const void* a_bf16, int64_t m,
                          int64_t k, float global_scale, void* a_q, void* a_s,
                          mx_stream_t stream);

/*
 * mx_pack_weights -- round-to-nearest weight packing, once per weight tensor
 * (the exporter step): E2M1 in blocks of 32 with EVEN-rule E8M0 scales
 * (Qwen3.5-27B-MXFP4-QAD-W4A4-LR1e-5-s1000, "How this checkpoint was
 * produced"), each weight rounded to the lattice with no scale search
 * (Qwen3.5-27B-NVFP4-RTN-weight-only, introduction).  Same kernel, layouts
 * and errors as mx_quantize_act with the [n, k] weight matrix.
 */
mx_status mx_pack_weights(mx_format fmt, mx_scale_rule rule, const void* w_bf16, int64_t n,
                          int64_t k, float global_scale, void* w_q, void* w_s,
                          mx_stream_t stream);

/*
 * mx_gemm -- block-scaled GEMM on MX operands: the W4A4 FP4 GEMM that serves
 * the MXFP4 checkpoints (Qwen3.5-9B-MXFP4-QAD-W4A4-LR1e-5-s3000, "Serving":
 * block-32 E2M1 weights with E8M0 scales times activations quantized per
 * token at run time), and the MXFP8 W8A8 projections of the mixed recipe
 * (Qwen3.8-27B-MXFP8Attn-MXFP4MLP-lmheadMXFP4, introduction and section 2:
 * E4M3 with E8M0 per group of 32 for attention, MXFP4 for the MLP and
 * lm_head).
 * a_fmt, w_fmt in {MXFP4, MXFP8}, equal or mixed.  a_q/a_s are [m, k] codes
 * and [m, k/32] E8M0 scales, w_q/w_s are [n, k] codes and [n, k/32] scales
 * (codes: E2M1 two per byte, E4M3 one per byte).  y is [m, n] bf16 (RNE of
 * the fp32 accumulator) or fp32 with MX_OUT_F32.  Requires k % 32 == 0; any
 * m, n >= 1 (no lower limit on n).  All pointers 16-byte aligned.
 * Kernels:
 *  - MXFP4 x MXFP4 runs on the block-scaled FP4 matrix cores, whose block
 *    sums are exact.
 *  - MXFP8 x MXFP8 and the mixed pairs by default dequantize each operand
 *    exactly to bf16 (element times its power-of-two block scale) and run on
 *    bf16 matrix cores.  MX_FP8_FAST selects the block-scaled FP8 (and
 *    FP8 x FP4) matrix cores instead, whose internal accumulation is inexact
 *    (bound 5e-4 * S instead of 1e-4 * S).
 * Result: the GEMM error bound above (1e-4 * S on normal-range operands).
 * workspace/ws_bytes: optional split-K scratch (mx_gemm_workspace_size).
 * When the output tiles alone cannot occupy the GPU (small m or n) and a
 * workspace is given, K is split across workgroups: each writes an fp32
 * partial product into the workspace and a second kernel sums the partials
 * in split order (deterministic) and rounds once.  Without one the call runs
 * unsplit.  Both meet the bound; they are not bitwise equal to each other.
 * Errors: MX_ERR_INVALID_ARG (NVFP4, null pointer, unknown flag),
 * MX_ERR_SHAPE, MX_ERR_ALIGN, MX_ERR_WORKSPACE (workspace too small),
 * MX_ERR_UNSUPPORTED (not gfx950; or the tile/decode kernels, which use
 * 32-bit offsets, would see an operand of 2 GiB or more), MX_ERR_HIP.
 */
mx_status mx_gemm(mx_format a_fmt, mx_format w_fmt, const void* a_q, const void* a_s,
                  const void* w_q, const void* w_s, int64_t m, int64_t n, int64_t k, void* y,
                  void* workspace, size_t ws_bytes, unsigned flags, mx_stream_t stream);

/*
 * mx_gemm_noalloc -- mx_gemm for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same arguments without the workspace.  Where mx_gemm
 * would split K, the fp32 partials go to a scratch array of
 * MX_NOALLOC_SCRATCH_BYTES that the library holds in device memory on every
 * GPU it runs on, for the life of the process; the call itself allocates
 * nothing.  The result is bitwise equal to mx_gemm with a workspace.  Split-K
 * runs only while the output tiles cannot fill the GPU twice over (at most
 * 384 tile-splits of 128 x 128 fp32: one per CU up to 128 tiles, two per
 * tile from 129 to 192 tiles of the dequantizing kernel), so every shape fits
 * the scratch; a need beyond it would return MX_ERR_WORKSPACE.  All calls on
 * one GPU share its scratch (nothing in it needs clearing between calls):
 * calls that overlap in time on one GPU, on different streams, race and must
 * be ordered by the caller.
 * Errors as mx_gemm.
 */
#define MX_NOALLOC_SCRATCH_BYTES (24u << 20)
mx_status mx_gemm_noalloc(mx_format a_fmt, mx_format w_fmt, const void* a_q, const void* a_s,
                          const void* w_q, const void* w_s, int64_t m, int64_t n, int64_t k, void* y,
                          unsigned flags, mx_stream_t stream);

/*
 * mx_gemm_fused -- mx_gemm with the per-token activation quantization done
 * inside the GEMM from bf16 A ([m, k]) with scale rule a_rule (CEIL is the
 * activation rule: Qwen3.5-9B-MXFP4-QAD-W4A4-LR1e-5-s3000, "Training mode").
 * The result equals mx_quantize_act followed by an unsplit mx_gemm, bit for
 * bit.  Workspace (mx_gemm_fused_workspace_size):
 *  - same-format pairs on the quantize-once shapes (large MXFP4 shapes: m,
 *    n >= 1024, k % 128 == 0; exact MXFP8 on its 128 x 128 kernel: k % 128
 *    == 0, n > 256): optional.  With a workspace, A is quantized into it by
 *    mx_quantize_act's kernel (codes [m, k * bits / 8], then scales [m,
 *    k/32]) and mx_gemm's kernel reads it there: two launches, the same work
 *    as the standalone pair.  With MX_FUSED_IN_GEMM instead, each 256-row
 *    (MXFP4) or 128-row (MXFP8) block of A is quantized once into it inside
 *    the GEMM's own launches.  That layout, from a 256-byte aligned base
 *    (MX_ERR_ALIGN): A codes; E8M0 scales [m, k/32] at the next 256-byte
 *    boundary (both as mx_quantize_act writes them); at the next 256-byte
 *    boundary the int32 state: a chunk pool counter, one done counter per
 *    block and an error word.  The error word is nonzero after the call if
 *    a tile's bounded wait for its block gave up; that tile's part of Y is
 *    then NaN.  Without a workspace (or with MX_FP8_FAST) each tile
 *    quantizes its own rows of A instead.
 *  - other same-format shapes without MX_DEBUG_DUMP_AQ: none used (each
 *    tile quantizes its own rows of A; one launch).
 *  - mixed pairs, and exact MXFP8 on the shapes of its large-tile kernel
 *    (k % 128 == 0 and at least 256 tiles of 256 x 256): required
 *    (MX_ERR_WORKSPACE without it).  A is quantized into it (codes [m, k *
 *    bits(a_fmt) / 8], then scales [m, k/32]) and mx_gemm's kernel reads it
 *    there.
 *  - with MX_DEBUG_DUMP_AQ (same-format pairs), the codes and scales that
 *    the in-tile prologue computed are also written to the workspace, A
 *    codes [m, k * bits / 8] followed by E8M0 scales [m, k/32], so they can
 *    be checked bit for bit; the workspace must hold both.
 * Errors as mx_gemm; MX_ERR_INVALID_ARG also for an unknown rule.
 */
mx_status mx_gemm_fused(mx_format a_fmt, mx_format w_fmt, const void* a_bf16, mx_scale_rule a_rule,
                        const void* w_q, const void* w_s, int64_t m, int64_t n, int64_t k, void* y,
                        void* workspace, size_t ws_bytes, unsigned flags, mx_stream_t stream);

/*
 * mx_gemm_fused_workspace_size -- bytes of workspace mx_gemm_fused uses on
 * this shape, pair and flags (0: none): the codes and scales of A, or with
 * MX_FUSED_IN_GEMM on a quantize-once shape that layout with its state.
 * Same argument checks as mx_gemm_fused.
 */
mx_status mx_gemm_fused_workspace_size(mx_format a_fmt, mx_format w_fmt, int64_t m, int64_t n, int64_t k,
                                       unsigned flags, size_t* bytes);

/*
 * nv_gemm -- NVFP4 x NVFP4 GEMM, the W4A4 path of the NVFP4 checkpoints
 * (Qwen3.5-27B-NVFP4-GPTQ and Qwen3.5-27B-NVFP4-RTN-weight-only,
 * introductions: E2M1 elements with block scales and per-tensor global
 * scales for weights and inputs).  a_q [m, k/2] E2M1, a_s [m, k/16] E4M3,
 * w_q [n, k/2], w_s [n, k/16].  Y = alpha * sum_k (e2m1_a * s_a) *
 * (e2m1_w * s_w), with alpha = 1 / (g_a * g_w) supplied by the caller.
 * Requires k % 16 == 0.  The block products are exact in f16, so the
 * contraction runs on f16 matrix cores with fp32 accumulation: the GEMM
 * error bound above with F = 0.  workspace: split-K scratch as for mx_gemm
 * (alpha is applied after the partial sums).  Errors as mx_gemm, plus
 * MX_ERR_INVALID_ARG for a non-finite alpha.
 */
mx_status nv_gemm(const void* a_q, const void* a_s, const void* w_q, const void* w_s, int64_t m,
                  int64_t n, int64_t k, float alpha, void* y, void* workspace, size_t ws_bytes,
                  unsigned flags, mx_stream_t stream);

/*
 * mx_gemm_w4a16 -- weight-only quantized linear (W4A16): bf16 activations,
 * used as they are, times packed 4-bit weights.  One packed artifact serves
 * both W4A4 and W4A16 (Qwen3.5-27B-MXFP4-QAD-W4A4-LR1e-5-s1000,
 * introduction); the NVFP4 weight-only checkpoint keeps activations in bf16
 * with weight bytes identical to the W4A4 sibling
 * (Qwen3.5-27B-NVFP4-RTN-weight-only, introduction).
 *
 * a_bf16 [m, k] bf16; w_q [n, k/2] E2M1 (element 2j in the low nibble of
 * byte j); w_s [n, k/32] E8M0 for w_fmt == MX_FMT_MXFP4 or [n, k/16] E4M3
 * for MX_FMT_NVFP4.  y [m, n] bf16 (RNE of the fp32 result) or fp32 with
 * MX_OUT_F32:
 *   Y = alpha * sum_k a * dq(w),  dq(w) = e2m1 * 2^(s - 127)  (MXFP4)
 *                                 dq(w) = e2m1 * s_e4m3       (NVFP4),
 * alpha = 1 / g_w for NVFP4 weights (their global scale), normally 1 for
 * MXFP4.  A weight element times its block scale is exact in bf16, so the
 * contraction runs on bf16 matrix cores with fp32 accumulation: the GEMM
 * error bound above (1e-4 * sum_k |a_k dq(w)_k| on normal-range operands;
 * MXFP4 weight values and bf16 activations below 2^-126 may be flushed).
 * Requires k % 32 == 0 (MXFP4) or k % 16 == 0 (NVFP4); any m, n >= 1.
 * Errors: MX_ERR_INVALID_ARG for null pointers, unknown flags, a
 * non-finite alpha or a w_fmt other than MXFP4/NVFP4 (MXFP8:
 * MX_ERR_UNSUPPORTED); MX_ERR_SHAPE, MX_ERR_ALIGN (16-byte alignment of
 * every pointer) and MX_ERR_HIP as for mx_gemm.  workspace: split-K scratch
 * as for mx_gemm (see mx_gemm_w4a16_workspace_size), used by the general
 * kernel only.
 */
mx_status mx_gemm_w4a16(mx_format w_fmt, const void* a_bf16, const void* w_q, const void* w_s, int64_t m,
                        int64_t n, int64_t k, float alpha, void* y, void* workspace, size_t ws_bytes,
                        unsigned flags, mx_stream_t stream);

/*
 * mx_gemm_workspace_size / mx_gemm_w4a16_workspace_size -- *bytes = the
 * workspace with which mx_gemm (MX pairs, equal or mixed, with the given
 * flags; NVFP4 with NVFP4 for nv_gemm) or mx_gemm_w4a16 splits K on this
 * shape; 0 when it never does.  Pure host logic; errors as the GEMM's own
 * argument checks.
 */
mx_status mx_gemm_workspace_size(mx_format a_fmt, mx_format w_fmt, int64_t m, int64_t n, int64_t k,
                                 unsigned flags, size_t* bytes);
mx_status mx_gemm_w4a16_workspace_size(mx_format w_fmt, int64_t m, int64_t n, int64_t k, size_t* bytes);

/*
 * mx_gemm_w4a16_plan -- writes into `name` (capacity `len`) the kernel that
 * mx_gemm_w4a16 would launch for this shape.  Pure host logic.
 */
mx_status mx_gemm_w4a16_plan(mx_format w_fmt, int64_t m, int64_t n, int64_t k, char* name, size_t len);

/*
 * mx_gemm_swiglu_quant -- the gate_up projection of the gated MLP with the
 * SwiGLU activation and the down projection's activation quantization fused
 * into the GEMM's epilogue, so h never exists in bf16 in memory.  The MLP
 * weights are MXFP4 and vLLM fuses gate_proj and up_proj into one
 * gate_up_proj (Qwen3.8-27B-MXFP8Attn-MXFP4MLP-lmheadMXFP4, section 2); h is
 * the down projection's input, quantized per token with the CEIL rule
 * (Qwen3.5-9B-MXFP4-QAD-W4A4-LR1e-5-s3000, "Training mode").
 *
 * a_q/a_s: [m, k] MXFP4 activations.  w_q/w_s: the [2*inter, k] MXFP4 gate_up
 * weights with rows alternating 32 gate and 32 up rows: row 64c + r is gate
 * row 32c + r and row 64c + 32 + r is up row 32c + r (a row permutation of
 * the [gate; up] weight, applied before or after packing, since packing is
 * row-local).  Outputs h_q [m, inter/2] codes and h_s [m, inter/32] E8M0
 * scales, the layout of mx_quantize_act, ready for mx_gemm with the down
 * projection's weights.
 * Per element: gate and up are the fp32 accumulators rounded to bf16 (as a
 * bf16 Y would hold them); h = bf16(gate * rcp(1 + exp2(-gate * log2 e)) * up)
 * in fp32 on the hardware exp2 and reciprocal; then CEIL-rule MXFP4
 * quantization of each 32-column block of h.  mx_swiglu_quant applies the
 * same arithmetic to a stored [gate | up] Y, so the fused and unfused paths
 * agree bit for bit whenever their GEMMs accumulate alike (both run the
 * prefill kernel on these shapes).
 * Requires inter % 32 == 0 and k % 32 == 0 (MX_ERR_SHAPE); the fused kernel
 * needs k % 128 == 0 and operands below 2 GiB (else MX_ERR_UNSUPPORTED:
 * use mx_gemm and mx_swiglu_quant).  16-byte aligned pointers.
 */
mx_status mx_gemm_swiglu_quant(const void* a_q, const void* a_s, const void* w_q, const void* w_s, int64_t m,
                               int64_t inter, int64_t k, void* h_q, void* h_s, mx_stream_t stream);

/* mx_gemm_swiglu_quant_plan -- names the kernel mx_gemm_swiglu_quant would
 * launch for this shape, or returns its error.  Pure host logic. */
mx_status mx_gemm_swiglu_quant_plan(int64_t m, int64_t inter, int64_t k, char* name, size_t len);

/*
 * mx_swiglu_quant -- the same SwiGLU + CEIL MXFP4 quantization as the fused
 * epilogue above, from a stored bf16 gate_up output x_bf16 [m, 2*inter]
 * whose columns [0, inter) are gate and [inter, 2*inter) up (the output of
 * mx_gemm with the [gate; up] weight).  h_q [m, inter/2], h_s [m, inter/32].
 * Requires inter % 32 == 0 and 16-byte aligned pointers.
 */
mx_status mx_swiglu_quant(const void* x_bf16, int64_t m, int64_t inter, void* h_q, void* h_s,
                          mx_stream_t stream);

/*
 * mx_fake_quant -- training-time fake quantization: the quantize ->
 * dequantize round trip written back as bf16.  Quantization-aware
 * distillation runs it in the student's forward on every quantized linear,
 * weights with the EVEN rule and per-token activations with the CEIL rule
 * (Qwen3.5-27B-MXFP4-QAD-W4A4-LR1e-5-s1000, "How this checkpoint was
 * produced", Training row), and its activation quantizer is bit-identical to
 * the serving one (Qwen3.5-9B-MXFP4-QAD-W4A4-LR1e-5-s3000, "Training mode").
 *
 * x_bf16 [rows, k] bf16 in; y_bf16 [rows, k] bf16 out, which must not
 * overlap x (MX_ERR_INVALID_ARG).  The codes and scales are exactly those
 * that mx_quantize_act computes for the same fmt, rule and global_scale; each
 * output is the bf16 nearest to the dequantized value, ties to even:
 * code * 2^(e) for MXFP4/MXFP8 (exact in bf16 unless it passes the largest
 * finite bf16, which gives infinity), code * s / g for NVFP4 (one rounding
 * of the exact quotient).  A zero keeps the input's sign.  The straight-
 * through gradient of the op is the identity and needs no call.
 * Requirements and errors as mx_quantize_act.
 */
mx_status mx_fake_quant(mx_format fmt, mx_scale_rule rule, const void* x_bf16, int64_t rows, int64_t k,
                        float global_scale, void* y_bf16, mx_stream_t stream);

/*
 * mx_tensor_amax -- largest |x| of a bf16 tensor of `count` elements, written
 * as fp32 to *amax_dev (device memory).  The NVFP4 global scales come from it
 * (activations: the running maximum over calibration batches).
 */
mx_status mx_tensor_amax(const void* x_bf16, int64_t count, float* amax_dev, mx_stream_t stream);

/*
 * mx_nv_global_scale -- host helper: g = RNE_fp32(448 * 6 / amax), correctly
 * rounded; 1 when amax <= 0; the largest finite fp32 when the quotient
 * leaves the fp32 range.
 */
float mx_nv_global_scale(float amax);

/*
 * mx_gemm_plan -- writes into `name` (capacity `len`) the kernel and tile
 * configuration that mx_gemm with these flags (fused != 0: mx_gemm_fused;
 * a_fmt == NVFP4: nv_gemm) would launch for this shape, so callers can
 * confirm which path runs.  Pure host logic; makes no HIP call.
 */
mx_status mx_gemm_plan(mx_format a_fmt, mx_format w_fmt, int64_t m, int64_t n, int64_t k,
                       int fused, unsigned flags, char* name, size_t len);

#ifdef __cplusplus
}
#endif

#endif /* MXLINEAR_H */
