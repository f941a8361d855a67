// Device-side helpers shared by the quantizer and GEMM kernels (gfx950).
//
// Element and scale encodings (lightly-train README "DINOv3 + EoMT on RTX
// 5090", section 2 table; largest E4M3 value 448 per "2x, not 16x", section
// 5.4). Rounding is to nearest with ties to the even code, magnitudes past
// the largest finite value saturate, and the sign bit is copied from the
// input. Every encoder here is exact: it either works on integer bit fields
// or compares against thresholds that are exactly representable.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mx {

enum : int { FMT_MXFP8 = 1, FMT_MXFP4 = 2, FMT_NVFP4 = 3 };

constexpr int kAlignK = 128;   // stored row length is a multiple of this

__host__ __device__ inline int64_t round_up(int64_t n, int64_t m) { return (n + m - 1) / m * m; }

// bf16 bits -> fp32 (exact).
__device__ __forceinline__ float bf16_to_f32(uint32_t bits) { return __uint_as_float(bits << 16); }

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Two fp32 values -> two bf16 (lo in bits 0-15), round to nearest even:
// one V_CVT_PK_BF16_F32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float v2f_t __attribute__((ext_vector_type(2)));
  typedef __bf16 v2bf_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f_t{lo, hi}), v2bf_t));
}

// MX shared exponent from the magnitude bits of the block's largest bf16
// element: e = floor(log2 amax) - emax, clamped to [-127, 127]; a zero or
// subnormal amax gives -127 (for subnormals floor(log2) - emax < -127).
__device__ __forceinline__ int mx_shared_exp(uint32_t amax_mag_bits, int emax) {
  int E = (int)((amax_mag_bits >> 7) & 0xFFu);
  if (E == 0) return -127;
  int e = E - 127 - emax;
  return e < -127 ? -127 : e;   // upper clamp cannot trigger for bf16 input
}

// MX elements are x * 2^-e rounded to nearest even onto the element grid,
// saturating, sign copied. gfx950's scaled conversions do exactly that: they
// divide by the power of two held in the exponent field of their fp32 scale
// operand (the E8M0 byte; mantissa ignored, field 0 = 2^-127) and round to
// nearest even; the E2M1 form saturates at 6, the E4M3 form turns magnitudes
// past 448 into NaN, so its inputs are clamped to +-448 * 2^e first (exact).
// Checked on the chip against exact software encoders for every finite bf16
// input and every e in [-127, 126] (bf16 inputs give e <= 119 / 125).

// The scale operand for scale byte sb = e + 127.
__device__ __forceinline__ float mx_scale_operand(uint32_t sb) { return __uint_as_float(sb << 23); }

// 4 values -> 4 E4M3FN codes of v * 2^-e (byte i = value i).
__device__ __forceinline__ uint32_t e4m3x4_scaled(float a, float b, float c, float d, uint32_t sb) {
  typedef short v2s __attribute__((ext_vector_type(2)));
  // 448 * 2^e = 1.75 * 2^(e + 8): a normal float for every e >= -127
  const float lim = __uint_as_float((min(sb + 8u, 254u) << 23) | 0x600000u);
  const float s = mx_scale_operand(sb);
  a = __builtin_amdgcn_fmed3f(a, -lim, lim);
  b = __builtin_amdgcn_fmed3f(b, -lim, lim);
  c = __builtin_amdgcn_fmed3f(c, -lim, lim);
  d = __builtin_amdgcn_fmed3f(d, -lim, lim);
  v2s r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(v2s{0, 0}, a, b, s, false);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, c, d, s, true);
  return __builtin_bit_cast(uint32_t, r);
}

// 8 values -> 8 E2M1 codes of v * 2^-e (nibble i = value i).
__device__ __forceinline__ uint32_t e2m1x8_scaled(const float* x, uint32_t sb) {
  const float s = mx_scale_operand(sb);
  uint32_t r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, x[0], x[1], s, 0);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, x[2], x[3], s, 1);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, x[4], x[5], s, 2);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, x[6], x[7], s, 3);
  return r;
}

// E4M3 code (sign 0) of a non-negative double q, RNE + saturation. Used for
// the NVFP4 block scale q = block_amax / (6 s_t): the exact quotient is never
// within 2^-53 relative of an E4M3 rounding boundary unless it lies on it
// (then the double quotient is exact), so rounding the double is the same
// as rounding the exact quotient.
__device__ __forceinline__ uint32_t e4m3_encode_pos_f64(double q) {
  if (q >= 448.0) return 0x7Eu;
  if (q >= 0.015625) {
    uint64_t u = (uint64_t)__double_as_longlong(q);
    uint64_t r = (u + 0x0000FFFFFFFFFFFFull + ((u >> 49) & 1ull)) >> 49;
    return (uint32_t)(r - (1016ull << 3));
  }
  return (uint32_t)__builtin_rint(q * 512.0);
}

// Value of a non-negative E4M3 byte as double (exact).
__device__ __forceinline__ double e4m3_value(uint32_t b) {
  uint32_t e = (b >> 3) & 15u, m = b & 7u;
  if (e == 0) return (double)m * 0.001953125;   // m * 2^-9
  return (double)(8u + m) * (double)__uint_as_float((e - 10u + 127u) << 23);  // (8+m) * 2^(e-10)
}

// Smallest fp32 value >= T (T a positive double).
__device__ __forceinline__ float ceil_to_f32(double T, bool* exact) {
  float f = (float)T;                    // round to nearest
  double back = (double)f;
  if (back < T) f = __uint_as_float(__float_as_uint(f) + 1u);
  *exact = (back == T);
  return f;
}

// NVFP4 per-block E2M1 decision thresholds. With S = dec(byte) * s_t and the
// E2M1 midpoints M = {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5}, T_i = M_i * S is
// exact in double (<= 3 + 28 significant bits). For a bf16 input x (exact in
// fp32) the code magnitude is the number of i with |x| >= t_i, where t_i is
// the smallest fp32 value that rounds up across midpoint i: ceil(T_i), or
// the next fp32 above T_i when T_i is exact and ties go down (i even).
struct Nv4Thresholds {
  float t[7];
};

__device__ __forceinline__ Nv4Thresholds nvfp4_thresholds(double S) {
  Nv4Thresholds th;
  const double mids[7] = {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0};
#pragma unroll
  for (int i = 0; i < 7; ++i) {
    if (S == 0.0) {
      th.t[i] = __builtin_inff();
    } else {
      bool exact;
      float f = ceil_to_f32(mids[i] * S, &exact);
      if (exact && (i % 2 == 0)) f = __uint_as_float(__float_as_uint(f) + 1u);
      th.t[i] = f;
    }
  }
  return th;
}

__device__ __forceinline__ uint32_t nvfp4_encode(float x, const Nv4Thresholds& th) {
  uint32_t sign = (__float_as_uint(x) >> 28) & 8u;
  float a = __builtin_fabsf(x);
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 7; ++i) m += (uint32_t)(a >= th.t[i]);
  return sign | m;
}

// NVFP4 tensor scale from the tensor amax (fp32 bits of a bf16 magnitude):
// fp32 RNE of amax / 2688. The double quotient of an 8-significant-bit value
// by 21 * 2^7 is never within 2^-53 of an fp32 rounding boundary, so one
// rounding of the double quotient equals one rounding of the exact quotient.
__device__ __forceinline__ float nvfp4_tensor_scale(uint32_t amax_f32_bits) {
  return (float)((double)__uint_as_float(amax_f32_bits) / 2688.0);
}

}  // namespace mx
