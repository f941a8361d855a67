// C ABI of libmx: argument validation on the host, then dispatch to the
// launch wrappers. Every check happens before the first launch, so a call
// that returns an argument error has not touched any output.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "../../include/mx.h"
#include "mx_launch.h"

namespace {

thread_local std::string g_last_error;

mx_status fail(mx_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
mx_status fail(mx_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

bool valid_fmt(int f) { return f == MX_FMT_MXFP8 || f == MX_FMT_MXFP4 || f == MX_FMT_NVFP4; }
bool valid_axis(int a) { return a == MX_AXIS_ROW || a == MX_AXIS_COL; }
int64_t k_pad(int64_t len) { return (len + 127) / 128 * 128; }
int64_t code_row_bytes(int64_t kpad, int fmt) { return fmt == MX_FMT_MXFP8 ? kpad : kpad / 2; }
int block_elems(int fmt) { return fmt == MX_FMT_NVFP4 ? 16 : 32; }
bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Buffer offsets inside the kernels are 32-bit, and the launchers pass
// counts (rows, columns, K_pad) as int: every one of them stays below 2^31.
constexpr int64_t kMaxBytes = (int64_t)1 << 31;
constexpr int64_t kMaxCount = ((int64_t)1 << 31) - 256;   // K_pad = round_up(count, 128) stays below 2^31 too

// LayerNorm rows longer than this would let the fp32 row sums (cols / 64
// values added in sequence per lane) exceed the accuracy the header states.
constexpr int64_t kMaxLayerNormCols = 8192;

int64_t scales_total(int64_t R, int64_t kpad, int fmt) {
  int64_t n = R * (kpad / block_elems(fmt));
  if (fmt == MX_FMT_NVFP4) n = (n + 15) / 16 * 16 + 16;
  return n;
}

}  // namespace

extern "C" {

int mx_version(void) { return 10000; }

int64_t mx_k_pad(int64_t length) { return length < 1 ? 0 : k_pad(length); }

size_t mx_codes_bytes(int64_t rows, int64_t cols, mx_fmt fmt, mx_axis axis) {
  if (rows < 1 || cols < 1 || !valid_fmt(fmt) || !valid_axis(axis)) return 0;
  const int64_t R = axis == MX_AXIS_ROW ? rows : cols, L = axis == MX_AXIS_ROW ? cols : rows;
  return (size_t)(R * code_row_bytes(k_pad(L), fmt));
}

size_t mx_scales_bytes(int64_t rows, int64_t cols, mx_fmt fmt, mx_axis axis) {
  if (rows < 1 || cols < 1 || !valid_fmt(fmt) || !valid_axis(axis)) return 0;
  const int64_t R = axis == MX_AXIS_ROW ? rows : cols, L = axis == MX_AXIS_ROW ? cols : rows;
  return (size_t)scales_total(R, k_pad(L), fmt);
}

// mx_quantize and mx_quantize_amax: `name` prefixes the messages; amax NULL
// reduces the NVFP4 tensor amax from X.
static mx_status quantize_impl(const char* name, const void* src, int64_t rows, int64_t cols, int64_t ld, void* codes,
                               void* scales, mx_fmt fmt, mx_axis axis, const float* amax, int nslots,
                               void* hip_stream) {
  if (!valid_fmt(fmt)) return fail(MX_ERR_INVALID_ARG, "%s: unknown format %d", name, (int)fmt);
  if (!valid_axis(axis)) return fail(MX_ERR_INVALID_ARG, "%s: unknown axis %d", name, (int)axis);
  if (rows < 1 || cols < 1) return fail(MX_ERR_INVALID_ARG, "%s: empty tensor (%lld x %lld)", name, (long long)rows, (long long)cols);
  if (ld < cols) return fail(MX_ERR_INVALID_ARG, "%s: ld %lld < cols %lld", name, (long long)ld, (long long)cols);
  if (!src || !codes || !scales) return fail(MX_ERR_INVALID_ARG, "%s: null pointer", name);
  if (!aligned(src, 2)) return fail(MX_ERR_ALIGNMENT, "%s: src must be 2-byte aligned", name);
  if (!aligned(codes, 16) || !aligned(scales, 16))
    return fail(MX_ERR_ALIGNMENT, "%s: codes and scales must be 16-byte aligned", name);
  if (rows > kMaxCount || cols > kMaxCount)
    return fail(MX_ERR_UNSUPPORTED, "%s: rows and cols must be below 2^31 - 256", name);
  const int64_t R = axis == MX_AXIS_ROW ? rows : cols, L = axis == MX_AXIS_ROW ? cols : rows;
  const int64_t kpad = k_pad(L);
  if (R * code_row_bytes(kpad, fmt) >= kMaxBytes || scales_total(R, kpad, fmt) >= kMaxBytes)
    return fail(MX_ERR_UNSUPPORTED, "%s: output larger than 2 GiB", name);
  if (ld >= ((int64_t)1 << 31) || rows > ((int64_t)1 << 40) / ld)
    return fail(MX_ERR_UNSUPPORTED, "%s: input too large (ld must be below 2^31)", name);
  hipError_t e = mx::launch_quantize(static_cast<const uint16_t*>(src), rows, cols, ld, static_cast<uint8_t*>(codes),
                                     static_cast<uint8_t*>(scales), (int)fmt, (int)axis,
                                     reinterpret_cast<const uint32_t*>(amax), nslots,
                                     static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return fail(MX_ERR_HIP, "%s: launch failed: %s", name, hipGetErrorString(e));
  return MX_OK;
}

mx_status mx_quantize(const void* src, int64_t rows, int64_t cols, int64_t ld, void* codes, void* scales,
                      mx_fmt fmt, mx_axis axis, void* hip_stream) {
  return quantize_impl("mx_quantize", src, rows, cols, ld, codes, scales, fmt, axis, nullptr, 0, hip_stream);
}

mx_status mx_quantize_amax(const void* src, int64_t rows, int64_t cols, int64_t ld, void* codes, void* scales,
                           mx_fmt fmt, mx_axis axis, const float* amax, int nslots, void* hip_stream) {
  if (fmt != MX_FMT_NVFP4) {
    if (!valid_fmt(fmt)) return fail(MX_ERR_INVALID_ARG, "mx_quantize_amax: unknown format %d", (int)fmt);
    return fail(MX_ERR_UNSUPPORTED, "mx_quantize_amax: only NVFP4 has a tensor scale");
  }
  if (!amax) return fail(MX_ERR_INVALID_ARG, "mx_quantize_amax: null amax");
  if (!aligned(amax, 4)) return fail(MX_ERR_ALIGNMENT, "mx_quantize_amax: amax must be 4-byte aligned");
  if (nslots < 1 || nslots > MX_AMAX_MAX_WORDS)
    return fail(MX_ERR_INVALID_ARG, "mx_quantize_amax: nslots = %d outside [1, %d]", nslots, MX_AMAX_MAX_WORDS);
  return quantize_impl("mx_quantize_amax", src, rows, cols, ld, codes, scales, fmt, axis, amax, nslots, hip_stream);
}

mx_status mx_layernorm_quantize(const void* x, int64_t rows, int64_t cols, int64_t ld, const void* gamma,
                                const void* beta, float eps, void* codes, void* scales, mx_fmt fmt,
                                void* hip_stream) {
  if (fmt != MX_FMT_MXFP8 && fmt != MX_FMT_MXFP4) {
    if (fmt == MX_FMT_NVFP4)
      return fail(MX_ERR_UNSUPPORTED, "mx_layernorm_quantize: NVFP4 needs the output's tensor amax first");
    return fail(MX_ERR_INVALID_ARG, "mx_layernorm_quantize: unknown format %d", (int)fmt);
  }
  if (rows < 1 || cols < 1)
    return fail(MX_ERR_INVALID_ARG, "mx_layernorm_quantize: empty tensor (%lld x %lld)", (long long)rows, (long long)cols);
  if (ld < cols)
    return fail(MX_ERR_INVALID_ARG, "mx_layernorm_quantize: ld %lld < cols %lld", (long long)ld, (long long)cols);
  if (!x || !gamma || !beta || !codes || !scales) return fail(MX_ERR_INVALID_ARG, "mx_layernorm_quantize: null pointer");
  if (cols > kMaxLayerNormCols)
    return fail(MX_ERR_UNSUPPORTED, "mx_layernorm_quantize: rows longer than %lld columns are not supported",
                (long long)kMaxLayerNormCols);
  // eps > 0 keeps var + eps positive: a constant row (var = 0) then gives
  // y = beta instead of 0 * inf
  if (!(eps > 0.0f) || !(eps < 3.0e38f))
    return fail(MX_ERR_INVALID_ARG, "mx_layernorm_quantize: eps must be finite and > 0");
  if (!aligned(x, 4) || !aligned(gamma, 4) || !aligned(beta, 4))
    return fail(MX_ERR_ALIGNMENT, "mx_layernorm_quantize: x, gamma and beta must be 4-byte aligned");
  if (!aligned(codes, 16) || !aligned(scales, 16))
    return fail(MX_ERR_ALIGNMENT, "mx_layernorm_quantize: codes and scales must be 16-byte aligned");
  const int64_t kpad = k_pad(cols);
  if (rows * code_row_bytes(kpad, fmt) >= kMaxBytes || scales_total(rows, kpad, fmt) >= kMaxBytes)
    return fail(MX_ERR_UNSUPPORTED, "mx_layernorm_quantize: output larger than 2 GiB");
  if (ld >= ((int64_t)1 << 31) || rows >= ((int64_t)1 << 31))
    return fail(MX_ERR_UNSUPPORTED, "mx_layernorm_quantize: ld and rows must be below 2^31");
  hipError_t e = mx::launch_layernorm_quantize(static_cast<const float*>(x), rows, cols, ld,
                                               static_cast<const float*>(gamma), static_cast<const float*>(beta), eps,
                                               static_cast<uint8_t*>(codes), static_cast<uint8_t*>(scales), (int)fmt,
                                               static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return fail(MX_ERR_HIP, "mx_layernorm_quantize: launch failed: %s", hipGetErrorString(e));
  return MX_OK;
}

// mx_quantize_batch and mx_quantize_batch_amax (amax NULL: no reduction).
static mx_status quantize_batch_impl(const char* name, const mx_quant_item* items, int n, mx_fmt fmt, float* amax,
                                     void* hip_stream) {
  if (fmt != MX_FMT_MXFP8 && fmt != MX_FMT_MXFP4) {
    if (fmt == MX_FMT_NVFP4)
      return fail(MX_ERR_UNSUPPORTED, "%s: NVFP4 needs a tensor amax per item; use mx_quantize", name);
    return fail(MX_ERR_INVALID_ARG, "%s: unknown format %d", name, (int)fmt);
  }
  if (amax && !aligned(amax, 4)) return fail(MX_ERR_ALIGNMENT, "%s: amax must be 4-byte aligned", name);
  if (!items) return fail(MX_ERR_INVALID_ARG, "%s: null item array", name);
  if (n < 1 || n > MX_QUANT_BATCH_MAX)
    return fail(MX_ERR_INVALID_ARG, "%s: n = %d outside [1, %d]", name, n, MX_QUANT_BATCH_MAX);
  static_assert(MX_QUANT_BATCH_MAX == mx::kQuantBatchMax, "batch size of the header and the launcher");
  mx::QuantBatchItem q[MX_QUANT_BATCH_MAX];
  for (int i = 0; i < n; ++i) {
    const mx_quant_item& it = items[i];
    if (it.rows < 1 || it.cols < 1)
      return fail(MX_ERR_INVALID_ARG, "%s: item %d: empty tensor (%lld x %lld)", name, i, (long long)it.rows,
                  (long long)it.cols);
    if (it.ld < it.cols)
      return fail(MX_ERR_INVALID_ARG, "%s: item %d: ld %lld < cols %lld", name, i, (long long)it.ld,
                  (long long)it.cols);
    if (!it.src || !it.codes || !it.scales) return fail(MX_ERR_INVALID_ARG, "%s: item %d: null pointer", name, i);
    if (!aligned(it.src, 2)) return fail(MX_ERR_ALIGNMENT, "%s: item %d: src must be 2-byte aligned", name, i);
    if (!aligned(it.codes, 16) || !aligned(it.scales, 16))
      return fail(MX_ERR_ALIGNMENT, "%s: item %d: codes and scales must be 16-byte aligned", name, i);
    if (it.rows > kMaxCount || it.cols > kMaxCount)
      return fail(MX_ERR_UNSUPPORTED, "%s: item %d: rows and cols must be below 2^31 - 256", name, i);
    const int64_t kpad = k_pad(it.cols);
    if (it.rows * code_row_bytes(kpad, fmt) >= kMaxBytes || scales_total(it.rows, kpad, fmt) >= kMaxBytes)
      return fail(MX_ERR_UNSUPPORTED, "%s: item %d: output larger than 2 GiB", name, i);
    if (it.ld >= ((int64_t)1 << 31) || it.rows > (((int64_t)1 << 31) - 1) / it.ld)
      return fail(MX_ERR_UNSUPPORTED, "%s: item %d: input too large (rows * ld must be below 2^31)", name, i);
    q[i] = mx::QuantBatchItem{static_cast<const uint16_t*>(it.src), static_cast<uint8_t*>(it.codes),
                              static_cast<uint8_t*>(it.scales), (int)it.rows, (int)it.cols, (int)it.ld, (int)kpad,
                              nullptr};
  }
  hipError_t e = mx::launch_quantize_batch(q, n, (int)fmt, reinterpret_cast<uint32_t*>(amax),
                                           static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return fail(MX_ERR_HIP, "%s: launch failed: %s", name, hipGetErrorString(e));
  return MX_OK;
}

mx_status mx_quantize_batch(const mx_quant_item* items, int n, mx_fmt fmt, void* hip_stream) {
  return quantize_batch_impl("mx_quantize_batch", items, n, fmt, nullptr, hip_stream);
}

mx_status mx_quantize_batch_amax(const mx_quant_item* items, int n, mx_fmt fmt, float* amax, void* hip_stream) {
  if (!amax) return fail(MX_ERR_INVALID_ARG, "mx_quantize_batch_amax: null amax");
  return quantize_batch_impl("mx_quantize_batch_amax", items, n, fmt, amax, hip_stream);
}

mx_status mx_quantize_dual(const void* src, int64_t rows, int64_t cols, int64_t ld, void* row_codes,
                           void* row_scales, void* col_codes, void* col_scales, mx_fmt fmt, const float* amax_prev,
                           float headroom, void* hip_stream) {
  if (!valid_fmt(fmt)) return fail(MX_ERR_INVALID_ARG, "mx_quantize_dual: unknown format %d", (int)fmt);
  if (rows < 1 || cols < 1)
    return fail(MX_ERR_INVALID_ARG, "mx_quantize_dual: empty tensor (%lld x %lld)", (long long)rows, (long long)cols);
  if (ld < cols) return fail(MX_ERR_INVALID_ARG, "mx_quantize_dual: ld %lld < cols %lld", (long long)ld, (long long)cols);
  if (!src || !row_codes || !row_scales || !col_codes || !col_scales)
    return fail(MX_ERR_INVALID_ARG, "mx_quantize_dual: null pointer");
  const bool delayed = fmt == MX_FMT_NVFP4 && amax_prev != nullptr;
  if (delayed && !(headroom > 0.0f && headroom <= 3.0e38f))
    return fail(MX_ERR_INVALID_ARG, "mx_quantize_dual: headroom must be finite and > 0");
  if (!aligned(src, 2)) return fail(MX_ERR_ALIGNMENT, "mx_quantize_dual: src must be 2-byte aligned");
  if (!aligned(row_codes, 16) || !aligned(row_scales, 16) || !aligned(col_codes, 16) || !aligned(col_scales, 16))
    return fail(MX_ERR_ALIGNMENT, "mx_quantize_dual: codes and scales must be 16-byte aligned");
  if (delayed && !aligned(amax_prev, 4)) return fail(MX_ERR_ALIGNMENT, "mx_quantize_dual: amax_prev must be 4-byte aligned");
  if (rows > kMaxCount || cols > kMaxCount)
    return fail(MX_ERR_UNSUPPORTED, "mx_quantize_dual: rows and cols must be below 2^31 - 256");
  const int64_t rkpad = k_pad(cols), ckpad = k_pad(rows);
  if (rows * code_row_bytes(rkpad, fmt) >= kMaxBytes || scales_total(rows, rkpad, fmt) >= kMaxBytes ||
      cols * code_row_bytes(ckpad, fmt) >= kMaxBytes || scales_total(cols, ckpad, fmt) >= kMaxBytes)
    return fail(MX_ERR_UNSUPPORTED, "mx_quantize_dual: output larger than 2 GiB");
  if (ld >= ((int64_t)1 << 31) || rows > ((int64_t)1 << 40) / ld)
    return fail(MX_ERR_UNSUPPORTED, "mx_quantize_dual: input too large (ld must be below 2^31)");
  hipError_t e = mx::launch_quantize_dual(
      static_cast<const uint16_t*>(src), rows, cols, ld, static_cast<uint8_t*>(row_codes),
      static_cast<uint8_t*>(row_scales), static_cast<uint8_t*>(col_codes), static_cast<uint8_t*>(col_scales), (int)fmt,
      delayed ? amax_prev : nullptr, headroom, 0, 0, 0, static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return fail(MX_ERR_HIP, "mx_quantize_dual: launch failed: %s", hipGetErrorString(e));
  return MX_OK;
}

mx_status mx_quantize_dual_sr(const void* src, int64_t rows, int64_t cols, int64_t ld, void* row_codes,
                              void* row_scales, void* col_codes, void* col_scales, mx_fmt fmt, const float* amax_prev,
                              float headroom, uint64_t seed0, uint64_t seed1, void* hip_stream) {
  if (!valid_fmt(fmt)) return fail(MX_ERR_INVALID_ARG, "mx_quantize_dual_sr: unknown format %d", (int)fmt);
  if (fmt != MX_FMT_NVFP4)
    return fail(MX_ERR_UNSUPPORTED, "mx_quantize_dual_sr: stochastic rounding is implemented for NVFP4 only");
  if (rows < 1 || cols < 1)
    return fail(MX_ERR_INVALID_ARG, "mx_quantize_dual_sr: empty tensor (%lld x %lld)", (long long)rows, (long long)cols);
  if (ld < cols) return fail(MX_ERR_INVALID_ARG, "mx_quantize_dual_sr: ld %lld < cols %lld", (long long)ld, (long long)cols);
  if (cols % 8 != 0)
    return fail(MX_ERR_UNSUPPORTED, "mx_quantize_dual_sr: cols (%lld) must be a multiple of 8", (long long)cols);
  if (!src || !row_codes || !row_scales || !col_codes || !col_scales)
    return fail(MX_ERR_INVALID_ARG, "mx_quantize_dual_sr: null pointer");
  const bool delayed = amax_prev != nullptr;
  if (delayed && !(headroom > 0.0f && headroom <= 3.0e38f))
    return fail(MX_ERR_INVALID_ARG, "mx_quantize_dual_sr: headroom must be finite and > 0");
  if (!aligned(src, 2)) return fail(MX_ERR_ALIGNMENT, "mx_quantize_dual_sr: src must be 2-byte aligned");
  if (!aligned(row_codes, 16) || !aligned(row_scales, 16) || !aligned(col_codes, 16) || !aligned(col_scales, 16))
    return fail(MX_ERR_ALIGNMENT, "mx_quantize_dual_sr: codes and scales must be 16-byte aligned");
  if (delayed && !aligned(amax_prev, 4))
    return fail(MX_ERR_ALIGNMENT, "mx_quantize_dual_sr: amax_prev must be 4-byte aligned");
  if (rows > kMaxCount || cols > kMaxCount)
    return fail(MX_ERR_UNSUPPORTED, "mx_quantize_dual_sr: rows and cols must be below 2^31 - 256");
  const int64_t rkpad = k_pad(cols), ckpad = k_pad(rows);
  if (rows * code_row_bytes(rkpad, fmt) >= kMaxBytes || scales_total(rows, rkpad, fmt) >= kMaxBytes ||
      cols * code_row_bytes(ckpad, fmt) >= kMaxBytes || scales_total(cols, ckpad, fmt) >= kMaxBytes)
    return fail(MX_ERR_UNSUPPORTED, "mx_quantize_dual_sr: output larger than 2 GiB");
  if (ld >= ((int64_t)1 << 31) || rows > ((int64_t)1 << 40) / ld)
    return fail(MX_ERR_UNSUPPORTED, "mx_quantize_dual_sr: input too large (ld must be below 2^31)");
  hipError_t e = mx::launch_quantize_dual(
      static_cast<const uint16_t*>(src), rows, cols, ld, static_cast<uint8_t*>(row_codes),
      static_cast<uint8_t*>(row_scales), static_cast<uint8_t*>(col_codes), static_cast<uint8_t*>(col_scales), (int)fmt,
      delayed ? amax_prev : nullptr, headroom, 1, seed0, seed1, static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return fail(MX_ERR_HIP, "mx_quantize_dual_sr: launch failed: %s", hipGetErrorString(e));
  return MX_OK;
}

}  // extern "C"

namespace {

// Shared by mx_gemm and mx_gemm_ws: every check before the launch.
mx_status gemm_checked(const char* fn, const void* A, const void* As, const void* B, const void* Bs, void* C,
                       int64_t M, int64_t N, int64_t K, mx_fmt fmt, const void* bias, mx_dtype out_dtype,
                       void* workspace, size_t workspace_bytes, void* hip_stream, bool validate_only = false) {
  if (!valid_fmt(fmt)) return fail(MX_ERR_INVALID_ARG, "%s: unknown format %d", fn, (int)fmt);
  if (out_dtype != MX_OUT_BF16 && out_dtype != MX_OUT_F32)
    return fail(MX_ERR_INVALID_ARG, "%s: unknown output dtype %d", fn, (int)out_dtype);
  if (M < 1 || N < 1 || K < 1)
    return fail(MX_ERR_INVALID_ARG, "%s: M, N, K must be >= 1 (got %lld, %lld, %lld)", fn, (long long)M, (long long)N,
                (long long)K);
  if (!A || !As || !B || !Bs || !C) return fail(MX_ERR_INVALID_ARG, "%s: null pointer", fn);
  if (!aligned(A, 16) || !aligned(As, 16) || !aligned(B, 16) || !aligned(Bs, 16) || !aligned(C, 16))
    return fail(MX_ERR_ALIGNMENT, "%s: A, As, B, Bs and C must be 16-byte aligned", fn);
  if (bias && !aligned(bias, 2)) return fail(MX_ERR_ALIGNMENT, "%s: bias must be 2-byte aligned", fn);
  if (workspace && !aligned(workspace, 16)) return fail(MX_ERR_ALIGNMENT, "%s: workspace must be 16-byte aligned", fn);
  if (M > kMaxCount || N > kMaxCount || K > kMaxCount)
    return fail(MX_ERR_UNSUPPORTED, "%s: M, N and K must be below 2^31 - 256", fn);
  const int64_t kpad = k_pad(K);
  const int64_t rb = code_row_bytes(kpad, fmt);
  if (M * rb >= kMaxBytes || N * rb >= kMaxBytes || scales_total(M, kpad, fmt) >= kMaxBytes ||
      scales_total(N, kpad, fmt) >= kMaxBytes)
    return fail(MX_ERR_UNSUPPORTED, "%s: operand larger than 2 GiB", fn);
  if (validate_only) return MX_OK;
  hipError_t e;
  const int out_f32 = out_dtype == MX_OUT_F32;
  const hipStream_t s = static_cast<hipStream_t>(hip_stream);
  float* ws = static_cast<float*>(workspace);
  const int64_t ws_bytes = workspace ? (int64_t)std::min<size_t>(workspace_bytes, (size_t)INT64_MAX) : 0;
  if (fmt == MX_FMT_NVFP4) {
    e = mx::launch_gemm_nvfp4(static_cast<const uint8_t*>(A), static_cast<const uint8_t*>(As),
                              static_cast<const uint8_t*>(B), static_cast<const uint8_t*>(Bs), C, M, N, K,
                              static_cast<const uint16_t*>(bias), out_f32, ws, ws_bytes, s);
  } else {
    e = mx::launch_gemm_mx(static_cast<const uint8_t*>(A), static_cast<const uint8_t*>(As),
                           static_cast<const uint8_t*>(B), static_cast<const uint8_t*>(Bs), C, M, N, K, (int)fmt,
                           static_cast<const uint16_t*>(bias), out_f32, ws, ws_bytes, s);
  }
  if (e != hipSuccess) return fail(MX_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return MX_OK;
}

}  // namespace

extern "C" {

mx_status mx_gemm(const void* A, const void* As, const void* B, const void* Bs, void* C, int64_t M, int64_t N,
                  int64_t K, mx_fmt fmt, const void* bias, mx_dtype out_dtype, void* hip_stream) {
  return gemm_checked("mx_gemm", A, As, B, Bs, C, M, N, K, fmt, bias, out_dtype, nullptr, 0, hip_stream);
}

mx_status mx_gemm_ws(const void* A, const void* As, const void* B, const void* Bs, void* C, int64_t M, int64_t N,
                     int64_t K, mx_fmt fmt, const void* bias, mx_dtype out_dtype, void* workspace,
                     size_t workspace_bytes, void* hip_stream) {
  return gemm_checked("mx_gemm_ws", A, As, B, Bs, C, M, N, K, fmt, bias, out_dtype, workspace, workspace_bytes,
                      hip_stream);
}

mx_status mx_gemm_scratch(const void* A, const void* As, const void* B, const void* Bs, void* C, int64_t M,
                          int64_t N, int64_t K, mx_fmt fmt, const void* bias, mx_dtype out_dtype, void* hip_stream) {
  static_assert(MX_SCRATCH_BYTES == mx::kScratchBytes, "scratch size of the header and the library");
  const size_t need = mx_gemm_workspace_bytes(M, N, K, fmt);
  if (need > mx::kScratchBytes)
    return fail(MX_ERR_UNSUPPORTED, "mx_gemm_scratch: the plan needs %zu bytes of scratch, more than the %zu the "
                "library holds", need, mx::kScratchBytes);
  void* ws = nullptr;
  if (need > 0) {
    // arguments first: a call that fails validation must not take the address
    const mx_status st = gemm_checked("mx_gemm_scratch", A, As, B, Bs, C, M, N, K, fmt, bias, out_dtype, nullptr, 0,
                                      nullptr, /*validate_only=*/true);
    if (st != MX_OK) return st;
    const hipError_t e = mx::scratch_buffer(&ws);
    if (e != hipSuccess)
      return fail(MX_ERR_HIP, "mx_gemm_scratch: no device address for the scratch: %s", hipGetErrorString(e));
  }
  return gemm_checked("mx_gemm_scratch", A, As, B, Bs, C, M, N, K, fmt, bias, out_dtype, ws, need, hip_stream);
}

size_t mx_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, mx_fmt fmt) {
  if (!valid_fmt(fmt) || M < 1 || N < 1 || K < 1 || M > kMaxCount || N > kMaxCount || K > kMaxCount) return 0;
  return (size_t)(fmt == MX_FMT_NVFP4 ? mx::gemm_nvfp4_workspace_bytes(M, N, K)
                                      : mx::gemm_mx_workspace_bytes(M, N, K, (int)fmt));
}

mx_status mx_gemm_gelu_quantize(const void* A, const void* As, const void* B, const void* Bs, int64_t M, int64_t N,
                                int64_t K, mx_fmt fmt, const void* bias, void* out_codes, void* out_scales,
                                void* hip_stream) {
  if (!valid_fmt(fmt)) return fail(MX_ERR_INVALID_ARG, "mx_gemm_gelu_quantize: unknown format %d", (int)fmt);
  if (fmt == MX_FMT_NVFP4)
    return fail(MX_ERR_UNSUPPORTED, "mx_gemm_gelu_quantize: MXFP8 and MXFP4 only");
  if (M < 1 || N < 1 || K < 1)
    return fail(MX_ERR_INVALID_ARG, "mx_gemm_gelu_quantize: M, N, K must be >= 1 (got %lld, %lld, %lld)",
                (long long)M, (long long)N, (long long)K);
  if (N % 8 != 0) return fail(MX_ERR_UNSUPPORTED, "mx_gemm_gelu_quantize: N (%lld) must be a multiple of 8", (long long)N);
  if (!A || !As || !B || !Bs || !out_codes || !out_scales)
    return fail(MX_ERR_INVALID_ARG, "mx_gemm_gelu_quantize: null pointer");
  if (!aligned(A, 16) || !aligned(As, 16) || !aligned(B, 16) || !aligned(Bs, 16) || !aligned(out_codes, 16) ||
      !aligned(out_scales, 16))
    return fail(MX_ERR_ALIGNMENT, "mx_gemm_gelu_quantize: operands and outputs must be 16-byte aligned");
  if (bias && !aligned(bias, 2)) return fail(MX_ERR_ALIGNMENT, "mx_gemm_gelu_quantize: bias must be 2-byte aligned");
  if (M > kMaxCount || N > kMaxCount || K > kMaxCount)
    return fail(MX_ERR_UNSUPPORTED, "mx_gemm_gelu_quantize: M, N and K must be below 2^31 - 256");
  const int64_t kpad = k_pad(K), rb = code_row_bytes(kpad, fmt);
  if (M * rb >= kMaxBytes || N * rb >= kMaxBytes || scales_total(M, kpad, fmt) >= kMaxBytes ||
      scales_total(N, kpad, fmt) >= kMaxBytes)
    return fail(MX_ERR_UNSUPPORTED, "mx_gemm_gelu_quantize: operand larger than 2 GiB");
  const int64_t npad = k_pad(N);
  if (M * code_row_bytes(npad, fmt) >= kMaxBytes || scales_total(M, npad, fmt) >= kMaxBytes)
    return fail(MX_ERR_UNSUPPORTED, "mx_gemm_gelu_quantize: output larger than 2 GiB");
  hipError_t e = mx::launch_gemm_mx_gelu_quant(
      static_cast<const uint8_t*>(A), static_cast<const uint8_t*>(As), static_cast<const uint8_t*>(B),
      static_cast<const uint8_t*>(Bs), M, N, K, (int)fmt, static_cast<const uint16_t*>(bias),
      static_cast<uint8_t*>(out_codes), static_cast<uint8_t*>(out_scales), static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return fail(MX_ERR_HIP, "mx_gemm_gelu_quantize: launch failed: %s", hipGetErrorString(e));
  return MX_OK;
}

const char* mx_gemm_plan(int64_t M, int64_t N, int64_t K, mx_fmt fmt) {
  if (!valid_fmt(fmt) || M < 1 || N < 1 || K < 1) return nullptr;
  return fmt == MX_FMT_NVFP4 ? mx::plan_gemm_nvfp4(M, N, K, 0) : mx::plan_gemm_mx(M, N, K, (int)fmt, 0);
}

const char* mx_gemm_ws_plan(int64_t M, int64_t N, int64_t K, mx_fmt fmt, size_t workspace_bytes) {
  if (!valid_fmt(fmt) || M < 1 || N < 1 || K < 1) return nullptr;
  const int64_t ws = (int64_t)std::min<size_t>(workspace_bytes, (size_t)INT64_MAX);
  return fmt == MX_FMT_NVFP4 ? mx::plan_gemm_nvfp4(M, N, K, ws) : mx::plan_gemm_mx(M, N, K, (int)fmt, ws);
}

const char* mx_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
