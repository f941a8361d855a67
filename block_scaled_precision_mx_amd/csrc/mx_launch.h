// Launch wrappers called by the C ABI layer (host code, no validation here).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mx {

// NVFP4: amax NULL -> the tensor amax is reduced first; else it is the
// largest magnitude among the nslots fp32 words at amax (device).
hipError_t launch_quantize(const uint16_t* src, int64_t rows, int64_t cols, int64_t ld, uint8_t* codes,
                           uint8_t* scales, int fmt, int axis, const uint32_t* amax, int nslots, hipStream_t stream);

// Amax accumulators of a batched quantization: kAmaxWords words per tensor,
// of which the words kAmaxStride apart (one per 128-byte line) take partial
// maxima; the others stay zero.
constexpr int kAmaxWords = 256, kAmaxStride = 32, kAmaxLines = kAmaxWords / kAmaxStride;

// One tensor of a batched row quantization (MX formats): its source, sizes,
// outputs and K_pad = round_up(cols, 128).
struct QuantBatchItem {
  const uint16_t* src;
  uint8_t* codes;
  uint8_t* scales;
  int rows, cols, ld, kpad;
  uint32_t* amax;   // kAmaxWords accumulator words, or NULL (set by the launcher)
};
constexpr int kQuantBatchMax = 32;
// Passed by value as the kernel argument (about 1.4 KB).
struct QuantBatch {
  QuantBatchItem items[kQuantBatchMax];
  int first_wg[kQuantBatchMax + 1];
  int n;
};

// Row quantization of n <= kQuantBatchMax MXFP8 / MXFP4 tensors in one launch.
// amax non-NULL: n * kAmaxWords words, zeroed here, into which each item's
// tensor amax is reduced (item i: words i * kAmaxWords ..).
hipError_t launch_quantize_batch(const QuantBatchItem* items, int n, int fmt, uint32_t* amax, hipStream_t stream);

// Both quantized copies (row, and column stored transposed) from one read.
// NVFP4: amax_prev NULL -> tensor scale from this tensor; else delayed scale
// fp32(fp64(headroom * *amax_prev) / 2688). sr (NVFP4, cols % 8 == 0):
// elements rounded stochastically with Philox4x64-10 draws keyed by
// (seed0, seed1).
// LayerNorm of fp32 rows (gamma, beta fp32, eps) rounded to bf16 and
// row-quantized (MXFP8 / MXFP4).
hipError_t launch_layernorm_quantize(const float* x, int64_t rows, int64_t cols, int64_t ld, const float* gamma,
                                     const float* beta, float eps, uint8_t* codes, uint8_t* scales, int fmt,
                                     hipStream_t stream);

hipError_t launch_quantize_dual(const uint16_t* src, int64_t rows, int64_t cols, int64_t ld, uint8_t* rcodes,
                                uint8_t* rscales, uint8_t* ccodes, uint8_t* cscales, int fmt, const float* amax_prev,
                                float headroom, int sr, uint64_t seed0, uint64_t seed1, hipStream_t stream);

// MXFP8 / MXFP4: scaled-MFMA GEMM. C = A * B^T (+ bias), fp32 accumulate.
// ws / ws_bytes: a device workspace the plan may use for split-K partials
// (S M N fp32 values, S <= 16); NULL / 0 runs the unsplit plan.
hipError_t launch_gemm_mx(const uint8_t* A, const uint8_t* As, const uint8_t* B, const uint8_t* Bs,
                          void* C, int64_t M, int64_t N, int64_t K, int fmt, const uint16_t* bias,
                          int out_f32, float* ws, int64_t ws_bytes, hipStream_t stream);

// NVFP4 GEMM on the MX kernel's data path, in one of its tile shapes.
enum NvTile { NV_TILE_192x256 = 0, NV_TILE_128x128 = 1, NV_TILE_128x256 = 2 };
hipError_t run_gemm_nvfp4_mx(int tile, int splits, const uint8_t* A, const uint8_t* As, const uint8_t* B,
                             const uint8_t* Bs, void* C, int64_t M, int64_t N, int64_t K, const uint16_t* bias,
                             int out_f32, float* ws, hipStream_t stream);

// MXFP8 / MXFP4 GEMM whose output is GELU(bf16(A B^T + bias)) rounded to
// bf16 and quantized along N in the same format (rows of K_pad(N)
// elements): fc1 writing fc2's A operand. N % 8 == 0.
hipError_t launch_gemm_mx_gelu_quant(const uint8_t* A, const uint8_t* As, const uint8_t* B, const uint8_t* Bs,
                                     int64_t M, int64_t N, int64_t K, int fmt, const uint16_t* bias, uint8_t* qcodes,
                                     uint8_t* qscales, hipStream_t stream);

// NVFP4: E2M1 x E4M3 operands dequantized exactly to fp16 on the way into
// LDS, fp16 MFMA with fp32 accumulate, s_tA * s_tB applied in the epilogue.
// ws / ws_bytes as for launch_gemm_mx.
hipError_t launch_gemm_nvfp4(const uint8_t* A, const uint8_t* As, const uint8_t* B, const uint8_t* Bs,
                             void* C, int64_t M, int64_t N, int64_t K, const uint16_t* bias, int out_f32,
                             float* ws, int64_t ws_bytes, hipStream_t stream);

// C = sum_{s < splits} P[s] (+ bias) for split-K partials P[s] = ws + s M N
// (fp32, in order s = 0, 1, ...), stored as bf16 or fp32.
hipError_t launch_splitk_reduce(const float* ws, int splits, int64_t M, int64_t N, const uint16_t* bias, void* C,
                                int out_f32, hipStream_t stream);

// Workspace bytes of the fastest plan for a shape (0 if it does not split K).
int64_t gemm_mx_workspace_bytes(int64_t M, int64_t N, int64_t K, int fmt);
int64_t gemm_nvfp4_workspace_bytes(int64_t M, int64_t N, int64_t K);

// Size of the library's device scratch (csrc/scratch.hip): the largest
// split-K workspace any plan needs (S M N 4 bytes with at most one item per
// resident workgroup: 256 items of a 256x256 tile).
constexpr size_t kScratchBytes = (size_t)64 << 20;
// Device address of the current device's scratch (taken once per device).
hipError_t scratch_buffer(void** ptr);

// Name of the kernel configuration the launchers above pick for a shape
// given ws_bytes of workspace.
const char* plan_gemm_mx(int64_t M, int64_t N, int64_t K, int fmt, int64_t ws_bytes);
const char* plan_gemm_nvfp4(int64_t M, int64_t N, int64_t K, int64_t ws_bytes);

}  // namespace mx
