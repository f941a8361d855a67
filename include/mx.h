/*
 * mx.h -- C ABI of libmx, block-scaled quantize-then-GEMM for MI355X (gfx950).
 *
 * What the library computes (lightly-train README "DINOv3 + EoMT on RTX 5090"):
 *   - section 2, number formats table: MXFP8 = E4M3 elements with a UE8M0
 *     (power-of-two) scale per 1x32 block; MXFP4 = E2M1 elements with a
 *     UE8M0 scale per 1x32; NVFP4 = E2M1 elements with an E4M3 scale per
 *     1x16 plus one fp32 scale for the whole tensor.
 *   - section 4.3: the quantized GEMMs of a ViT block are qkv, proj, fc1 and
 *     fc2, each C = A * W^T (+ bias).
 *   - section 5.5: every low-precision GEMM is "TN" (both operands K-major);
 *     the weight-gradient GEMM needs a copy of its operands quantized along
 *     the token axis and stored transposed (MX_AXIS_COL below).
 *
 * Conventions the pages leave open, fixed by this library:
 *   - MX shared exponent e = floor(log2(block amax)) - emax, emax = 8 (E4M3)
 *     or 2 (E2M1), clamped to [-127, 127]; an all-zero block has e = -127.
 *     Scale byte = e + 127. Elements are x * 2^-e rounded to nearest, ties
 *     to even, saturating at +-448 (E4M3) / +-6 (E2M1).
 *   - NVFP4 tensor scale s_t = fp32 round-to-nearest-even(tensor amax / 2688),
 *     2688 = 448 * 6; block byte = E4M3 RNE(block amax / (6 s_t)) of the exact
 *     quotient; element = E2M1 RNE(x / (dec(byte) * s_t)) of the exact
 *     quotient. If that scale is zero, the block's codes are signed zeros.
 *   - The sign bit of a code is the sign bit of its input (-0.0 -> 0x80 / 0x8).
 *   - Inputs must be finite; NaN / Inf inputs are outside the contract.
 *
 * Storage (all row-major, no swizzle):
 *   Quantizing X [rows, cols] (bf16, leading dimension ld >= cols elements):
 *     axis ROW: blocks run along cols.  L = cols, R = rows.
 *     axis COL: blocks run along rows; the result is the ROW quantization of
 *               X^T, i.e. stored as R = cols rows of L = rows elements.
 *   K_pad = round_up(L, 128).
 *   codes : R x K_pad bytes (MXFP8), R x K_pad/2 bytes (MXFP4, NVFP4; element
 *           2i in the low nibble of byte i, 2i+1 in the high nibble).
 *           Codes past L are 0.
 *   scales: R x K_pad/bs bytes (bs = 32 for MX, 16 for NVFP4), scale bytes past
 *           the last real block are 0. NVFP4 appends a 16-byte trailer at
 *           byte offset round_up(R * K_pad/16, 16): {float s_t; float amax;
 *           uint32 0; uint32 0}; bytes between the last scale and the
 *           trailer are 0.
 *   Use mx_codes_bytes / mx_scales_bytes for the sizes.
 *
 * GEMM: C[M, N] = A[M, K] * B[N, K]^T (+ bias[N]), A and B the outputs of
 *   mx_quantize in the same format (A: M rows, B: N rows, both of length K).
 *   fp32 accumulation; the bias (bf16) is added in fp32; NVFP4 multiplies by
 *   s_tA * s_tB before the bias; the result is stored as bf16 (round to
 *   nearest even) or fp32, row-major with leading dimension N.
 *   Accuracy: |C - exact| <= 2^-12 * (sum_k |a_k b_k| + |bias|) before the
 *   final bf16 rounding, "exact" being the sum of the dequantized values.
 *
 * Memory: every pointer is a device pointer owned by the caller; the library
 *   never allocates, frees or synchronizes. Codes, scales and C must be
 *   16-byte aligned; src and bias 2-byte aligned. Calls are asynchronous on
 *   the given HIP stream (NULL = the default stream) and are reentrant; two
 *   calls writing the same buffers must be ordered by the caller.
 *
 * Errors: invalid arguments are detected on the host before any launch and
 *   leave every output untouched (MX_ERR_INVALID_ARG, MX_ERR_ALIGNMENT,
 *   MX_ERR_UNSUPPORTED). A failed launch returns MX_ERR_HIP. The message of
 *   the last non-OK status of the calling thread is in mx_last_error().
 *
 * Size limits (MX_ERR_UNSUPPORTED beyond them): every count (rows, cols, M,
 *   N, K) is at most 2^31 - 256, so that K_pad stays below 2^31; every code
 *   or scale buffer, and a quantizer's input span rows * ld, stays below
 *   2 GiB (the kernels address them with 32-bit offsets).
 */
#ifndef MX_H_
#define MX_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { MX_FMT_MXFP8 = 1, MX_FMT_MXFP4 = 2, MX_FMT_NVFP4 = 3 } mx_fmt;
typedef enum { MX_AXIS_ROW = 0, MX_AXIS_COL = 1 } mx_axis;
typedef enum { MX_OUT_BF16 = 0, MX_OUT_F32 = 1 } mx_dtype;
typedef enum {
  MX_OK = 0,
  MX_ERR_INVALID_ARG = 1,
  MX_ERR_UNSUPPORTED = 2,
  MX_ERR_ALIGNMENT = 3,
  MX_ERR_HIP = 4
} mx_status;

/* Library version as major*10000 + minor*100 + patch. */
int mx_version(void);

/* K_pad = round_up(length, 128): the stored length of a quantized row. */
int64_t mx_k_pad(int64_t length);

/* Bytes of the codes / scales buffers for X [rows, cols] quantized along
 * axis in fmt. 0 if an argument is invalid (rows or cols < 1, unknown enum). */
size_t mx_codes_bytes(int64_t rows, int64_t cols, mx_fmt fmt, mx_axis axis);
size_t mx_scales_bytes(int64_t rows, int64_t cols, mx_fmt fmt, mx_axis axis);

/* Quantize X [rows, cols] (bf16, row-major, leading dimension ld elements)
 * along axis into codes / scales (layouts above). README section 2 (formats)
 * and section 5.5 (the transposed, token-axis copy for weight gradients).
 * NVFP4 first reduces the tensor amax (stored in the scales trailer), then
 * quantizes; the whole call is stream-ordered. */
mx_status mx_quantize(const void* src, int64_t rows, int64_t cols, int64_t ld,
                      void* codes, void* scales, mx_fmt fmt, mx_axis axis,
                      void* hip_stream);

/* Both copies a training step needs, from one read of X (README section
 * 5.5: a fused quantizer reads the tensor once and writes the row copy and
 * the transposed copy): row_codes / row_scales receive exactly the bytes of
 * mx_quantize(..., MX_AXIS_ROW) and col_codes / col_scales those of
 * mx_quantize(..., MX_AXIS_COL) (sizes from mx_codes_bytes /
 * mx_scales_bytes with the respective axis).
 * NVFP4 tensor scale (README section 5.5, delayed amax):
 *   amax_prev == NULL: s_t from this tensor's amax, as mx_quantize (one
 *     extra read of X for the amax); both trailers get {s_t, amax}.
 *   amax_prev != NULL: a device pointer to one fp32 value, typically the
 *     amax field of a trailer from the previous step (it may be a trailer
 *     this call writes: the value is read before anything is written);
 *     s_t = fp32 RNE of fp64(fp64(headroom * amax_prev) / 2688), no extra
 *     read; blocks whose amax exceeds 2688 s_t saturate. Both trailers get
 *     {s_t, this tensor's amax}, for the next call. headroom must be finite
 *     and > 0 (the pages' study suggests 32 for gradients).
 *   MX formats ignore amax_prev and headroom.
 * Errors and memory rules as for mx_quantize; the four outputs must not
 * overlap. */
mx_status mx_quantize_dual(const void* src, int64_t rows, int64_t cols, int64_t ld,
                           void* row_codes, void* row_scales, void* col_codes, void* col_scales,
                           mx_fmt fmt, const float* amax_prev, float headroom, void* hip_stream);

/* mx_quantize_dual with stochastically rounded NVFP4 elements, for
 * gradients (README section 5.3: the P3 recipe rounds dY stochastically;
 * section 5.5: in software, with draws from Philox).
 * Block scale bytes, s_t and the trailers are exactly mx_quantize_dual's;
 * only the element codes differ:
 *   draws: Philox4x64 with 10 rounds (Salmon et al., SC 2011), key
 *     (seed0, seed1), counter (q, 0, 0, 0) for group q of eight elements;
 *     element i = r * cols + c of X takes 32 bits of output word
 *     (i mod 8) / 2, the low half for even i. Both copies use the draw of
 *     the element, so the draws do not depend on the axis.
 *   element: S32 = fp32(dec(byte) * s_t); y = fp32(|x| / S32) (IEEE round
 *     to nearest); y >= 6 gives 6; else with E2M1 neighbours lo <= y < hi,
 *     frac = (y - lo) / (hi - lo), the code is hi iff u < ceil(frac * 2^32),
 *     u the element's draw, else lo; S32 == 0 gives signed zeros; the sign
 *     is x's.
 * fmt must be MX_FMT_NVFP4 and cols a multiple of 8 (else
 * MX_ERR_UNSUPPORTED); other arguments, errors and memory rules as for
 * mx_quantize_dual. Calls with the same inputs and seeds write the same
 * bytes. */
mx_status mx_quantize_dual_sr(const void* src, int64_t rows, int64_t cols, int64_t ld,
                              void* row_codes, void* row_scales, void* col_codes, void* col_scales,
                              mx_fmt fmt, const float* amax_prev, float headroom,
                              uint64_t seed0, uint64_t seed1, void* hip_stream);

/* LayerNorm fused with quantization (README section 4.3: in the MXFP8
 * stack LayerNorm and quantization are one kernel; the residual stream and
 * the LayerNorm statistics stay fp32). x: fp32 [rows, cols], leading
 * dimension ld elements (the residual stream); gamma, beta: fp32 [cols];
 * eps finite and > 0 (so that a constant row, var = 0, gives y = beta).
 * Each row becomes
 *   y = (x - mu) / sqrt(var + eps) * gamma + beta   (mu, var: the row's mean
 *       and biased variance, computed in fp32),
 * rounded to bf16, and codes / scales receive what mx_quantize of that bf16
 * tensor (axis MX_AXIS_ROW) would write (sizes mx_codes_bytes /
 * mx_scales_bytes of (rows, cols, fmt, MX_AXIS_ROW)), so they serve directly
 * as the A operand of the next mx_gemm (K = cols). The bf16 LayerNorm output
 * itself is never stored. y lies within 2^-16 (|gamma| r (max|x - mu| +
 * |x - mu| + |mu|) + |beta| + |y|) of the exact value, r = 1/sqrt(var + eps).
 * cols is at most 8192 (MX_ERR_UNSUPPORTED beyond: the fp32 row sums of
 * longer rows could exceed that accuracy statement).
 * fmt: MX_FMT_MXFP8 or MX_FMT_MXFP4 (NVFP4 would need the output's tensor
 * amax before the first block: MX_ERR_UNSUPPORTED). x, gamma and beta must be
 * 4-byte aligned (16 bytes, with ld % 4 == 0, takes the vector loads), codes
 * and scales 16-byte aligned. Errors and memory rules as for mx_quantize. */
mx_status mx_layernorm_quantize(const void* x, int64_t rows, int64_t cols, int64_t ld,
                                const void* gamma, const void* beta, float eps,
                                void* codes, void* scales, mx_fmt fmt, void* hip_stream);

/* One tensor of mx_quantize_batch: X [rows, cols] (bf16, leading dimension
 * ld elements) and its row-axis outputs, sized by mx_codes_bytes /
 * mx_scales_bytes with MX_AXIS_ROW. */
typedef struct {
  const void* src;
  int64_t rows;
  int64_t cols;
  int64_t ld;
  void* codes;
  void* scales;
} mx_quant_item;

/* Most items one mx_quantize_batch call takes. */
#define MX_QUANT_BATCH_MAX 32

/* Row quantization (README section 2 formats, along K as for mx_quantize
 * with MX_AXIS_ROW) of n independent tensors in ONE launch: item i's codes
 * and scales are byte for byte those of mx_quantize(item i, fmt,
 * MX_AXIS_ROW). Meant for many small tensors quantized together, such as
 * every weight matrix at the start of a training step, where one launch per
 * tensor would cost more than the work.
 *   items: host array of n entries, read during the call only; n in
 *          [1, MX_QUANT_BATCH_MAX].
 *   fmt:   MX_FMT_MXFP8 or MX_FMT_MXFP4. NVFP4 needs a tensor-amax pass per
 *          item and is MX_ERR_UNSUPPORTED here (use mx_quantize).
 * Every item is validated as mx_quantize validates its arguments (and each
 * item's input must also satisfy rows * ld < 2^31 elements) before anything
 * is launched; on an error nothing is written and the message names the
 * item. Outputs of different items must not overlap. */
mx_status mx_quantize_batch(const mx_quant_item* items, int n, mx_fmt fmt, void* hip_stream);

/* Words per tensor of the amax accumulators of mx_quantize_batch_amax, and
 * the most words mx_quantize_amax reduces. */
#define MX_AMAX_WORDS 256
#define MX_AMAX_MAX_WORDS 256

/* mx_quantize_batch that also reduces each item's tensor amax (the largest
 * |x|, as the fp32 bit pattern of the bf16 magnitude). README section 5.3:
 * the P3 recipe quantizes activations and weights in MXFP8 for the forward
 * GEMMs and again in NVFP4 for the backward ones, whose tensor scale needs
 * the tensor amax (section 2); the forward quantization reads every element
 * anyway, so a later mx_quantize_amax of the same tensor needs no amax pass.
 *   amax: device array of n * MX_AMAX_WORDS fp32 words, 4-byte aligned,
 *     owned by the caller. The call zeroes it, then item i's amax is the
 *     largest of words i * MX_AMAX_WORDS .. (i + 1) * MX_AMAX_WORDS - 1
 *     (partial maxima, spread over words on separate cache lines so that
 *     the reductions of many workgroups do not queue on one); pass those
 *     words to mx_quantize_amax. Stream-ordered like the codes.
 * Codes and scales are byte for byte those of mx_quantize_batch; other
 * arguments, errors (also: amax NULL or misaligned) and memory rules as for
 * mx_quantize_batch; amax must not overlap an output. */
mx_status mx_quantize_batch_amax(const mx_quant_item* items, int n, mx_fmt fmt, float* amax, void* hip_stream);

/* mx_quantize with the NVFP4 tensor amax given instead of reduced from X
 * (README sections 5.3 and 5.5: the backward copy of a tensor whose amax
 * the forward quantization found). amax: device pointer to nslots fp32
 * words, nslots in [1, MX_AMAX_MAX_WORDS], 4-byte aligned; the tensor amax
 * is the largest magnitude among them (e.g. the MX_AMAX_WORDS words of an
 * item of mx_quantize_batch_amax, or, with nslots 1, the amax field of a
 * scales trailer). s_t = fp32 RNE of fp64(amax) / 2688 as mx_quantize derives
 * it, blocks whose amax exceeds 2688 s_t saturate, and the trailer gets
 * {s_t, the given amax}. With X's own amax the bytes are mx_quantize's.
 * fmt must be MX_FMT_NVFP4 (MX_ERR_UNSUPPORTED otherwise: the MX formats
 * have no tensor scale); other arguments, errors and memory rules as for
 * mx_quantize; amax must not overlap an output. */
mx_status mx_quantize_amax(const void* src, int64_t rows, int64_t cols, int64_t ld,
                           void* codes, void* scales, mx_fmt fmt, mx_axis axis,
                           const float* amax, int nslots, void* hip_stream);

/* C = A * B^T (+ bias) from quantized operands (README section 4.3 GEMMs,
 * section 5.5 TN layout). A / As: codes and scales of an M-row operand,
 * B / Bs: of an N-row operand, both of logical length K. bias: bf16[N] or
 * NULL. out_dtype selects bf16 or fp32 C. */
mx_status mx_gemm(const void* A, const void* As, const void* B, const void* Bs,
                  void* C, int64_t M, int64_t N, int64_t K, mx_fmt fmt,
                  const void* bias, mx_dtype out_dtype, void* hip_stream);

/* Weight-gradient GEMMs contract over the tokens (README section 5.4: the
 * dgrad / wgrad GEMMs of every block; section 5.5: wgrad takes the token-axis
 * copies), so K is long while C has few tiles. mx_gemm_ws may then split K
 * into S <= 16 ranges, each written as an fp32 partial C to `workspace`
 * (S * M * N * 4 bytes), and sum the partials in the fixed order 0, 1, ...,
 * S - 1 before the bias and the final rounding, so the result does not
 * depend on timing. It picks the fastest plan whose partials fit in
 * workspace_bytes; with workspace == NULL (or too small for any split) it
 * runs exactly what mx_gemm runs. Accuracy as for mx_gemm (S - 1 more fp32
 * additions). workspace: caller-owned device memory, 16-byte aligned, not
 * overlapping any other argument; its contents are scratch (overwritten,
 * nothing read from a previous call). Other arguments, errors and memory
 * rules as for mx_gemm. */
mx_status mx_gemm_ws(const void* A, const void* As, const void* B, const void* Bs,
                     void* C, int64_t M, int64_t N, int64_t K, mx_fmt fmt,
                     const void* bias, mx_dtype out_dtype, void* workspace,
                     size_t workspace_bytes, void* hip_stream);

/* Workspace bytes with which mx_gemm_ws runs its fastest plan for these sizes
 * (0 when that plan does not split K, or when an argument is invalid). */
size_t mx_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, mx_fmt fmt);

/* Bytes of device scratch the library holds per GPU for mx_gemm_scratch. */
#define MX_SCRATCH_BYTES ((size_t)64 << 20)

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * mx_gemm_ws with the library's own device scratch in place of a caller
 * workspace. It runs the plan mx_gemm_ws runs with
 * mx_gemm_workspace_bytes(M, N, K, fmt) bytes of workspace (the same
 * kernels, the same result bit for bit) and allocates and frees nothing.
 * The scratch is a device array of MX_SCRATCH_BYTES in the library; each GPU
 * the library runs on holds its own copy from the library's load until the
 * process ends, and the first call on a GPU looks up its address once (with
 * that GPU current). Every plan fits: a split plan has at most one work item
 * per resident workgroup, so S * M * N * 4 <= MX_SCRATCH_BYTES; a plan that
 * did not would return MX_ERR_UNSUPPORTED. The partials are fully written
 * by each call before they are read, so nothing has to start at zero. Every
 * call on one GPU shares that GPU's scratch: calls that can overlap on one
 * GPU (on two streams, or from two threads) race, and the caller must order
 * them. Other arguments, errors and memory rules as for mx_gemm. */
mx_status mx_gemm_scratch(const void* A, const void* As, const void* B, const void* Bs,
                          void* C, int64_t M, int64_t N, int64_t K, mx_fmt fmt,
                          const void* bias, mx_dtype out_dtype, void* hip_stream);

/* fc1 writing fc2's operand (README section 4.3, MXFP8 row of the block
 * table: fc1's epilogue quantizes the GELU output straight into fc2's E4M3
 * operand). Computes H = A * B^T (+ bias) as mx_gemm with bf16 output
 * would, applies the exact GELU, GELU(h) = h/2 * erfc(-h / sqrt 2), in fp32
 * to each bf16 h and rounds it to bf16, and writes the row quantization of
 * that [M, N] tensor in the operand format fmt: out_codes / out_scales
 * receive what mx_quantize(GELU tensor, fmt, MX_AXIS_ROW) would write
 * (sizes mx_codes_bytes / mx_scales_bytes of (M, N, fmt, MX_AXIS_ROW)), so
 * they serve directly as the A operand of the next mx_gemm (K = N). H itself
 * is never stored. The accumulation follows mx_gemm's accuracy rule, and the
 * fp32 GELU lies within 2^-14 |GELU| + 2^-126 of the exact value and has the
 * sign of h (-0 for a negative h whose GELU vanishes in fp32).
 * fmt: MX_FMT_MXFP8 or MX_FMT_MXFP4 (NVFP4 would need the tensor amax of H
 * first: MX_ERR_UNSUPPORTED). N must be a multiple of 8. Other arguments,
 * errors and memory rules as for mx_gemm. */
mx_status mx_gemm_gelu_quantize(const void* A, const void* As, const void* B, const void* Bs,
                                int64_t M, int64_t N, int64_t K, mx_fmt fmt, const void* bias,
                                void* out_codes, void* out_scales, void* hip_stream);

/* Name of the kernel configuration mx_gemm launches for these sizes and
 * format (for example "gemm_mx_kernel<mxfp8, 256x256>"), so profiles can be
 * matched to calls; a static string, or NULL if an argument is invalid. */
const char* mx_gemm_plan(int64_t M, int64_t N, int64_t K, mx_fmt fmt);

/* The same for mx_gemm_ws with workspace_bytes of workspace (a split plan
 * is named "<kernel>+splitk<S>"). */
const char* mx_gemm_ws_plan(int64_t M, int64_t N, int64_t K, mx_fmt fmt, size_t workspace_bytes);

/* Message for the last non-OK status returned on the calling thread. */
const char* mx_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MX_H_ */
