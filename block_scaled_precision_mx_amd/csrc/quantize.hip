// Block-scaled quantizers for gfx950: bf16 -> MXFP8 / MXFP4 / NVFP4 codes
// and scales, along the contiguous axis (row) or along the first axis with a
// transposed store (col).
//
// lightly-train README "DINOv3 + EoMT on RTX 5090": section 2 (formats and
// their block sizes), section 5.5 (the weight-gradient GEMM takes a copy
// quantized along the token axis and stored transposed; a stand-alone
// quantizer that made that copy ran 6-10x below the read-bandwidth bound).
//
// The work is HBM-bound (2 bytes read, 0.5-1.03 bytes written per element),
// so the kernels are shaped for coalescing and bytes in flight, and keep all
// index arithmetic in 32 bits (a 64-bit division is a long software routine
// on this GPU):
//  * row: a row of the stored operand is split over TPR = K_pad / 16 threads;
//    thread j of a row handles 8-element groups j and j + TPR (two 16-byte
//    loads in flight). The 4 lanes of a 32-element MX block (2 lanes of a
//    16-element NVFP4 block) are adjacent and combine their amax with
//    cross-lane shuffles; each lane stores its 8 codes next to its
//    neighbours'.
//  * col: a workgroup stages a 128 x 64 bf16 tile through LDS with 16-byte
//    row loads; each wave then owns 32 consecutive rows (one MX block, two
//    NVFP4 blocks) of 64 columns and each lane emits its column's 32 codes
//    as one contiguous 32- or 16-byte store of the transposed output.
//  * NVFP4 first reduces the tensor amax (bf16 magnitude bits, which order
//    like the values) into the scale trailer with one atomic max per wave;
//    the quantizer derives s_t from it.
#include "mx_device.h"
#include "mx_launch.h"

#include <algorithm>
#include <mutex>
#include <utility>
#include <vector>

namespace mx {

// Output buffers are written with raw buffer stores: a lane with nothing to
// store gives an offset past the end (kDropped), which the buffer's range
// check discards. The stores are then unconditional, so the compiler knows
// how many are in flight and can wait for a tile's prefetched loads without
// waiting for the stores issued after them.
constexpr uint32_t kDropped = 0x80000000u;   // outputs are < 2 GiB

__device__ __forceinline__ __amdgpu_buffer_rsrc_t out_rsrc(void* p, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, (int)bytes, 0x00020000);
}

// 16-byte streaming load (the source is read once).
__device__ __forceinline__ uint4 load16_stream(const void* p) {
  typedef unsigned v4 __attribute__((ext_vector_type(4)));
  const v4 v = __builtin_nontemporal_load(reinterpret_cast<const v4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

struct NvTrailer {
  float s_t;
  uint32_t amax_bits;   // fp32 bits of the tensor amax
  uint32_t pad[2];
};

// ------------------------------------------------------------ amax (NVFP4)

// Zeroes the trailer and the (< 16) padding bytes between the last scale
// byte and the trailer, so the whole scale buffer is defined.
__global__ void nv_trailer_init_kernel(uint8_t* gap, int gap_bytes, NvTrailer* tr) {
  if ((int)threadIdx.x < gap_bytes) gap[threadIdx.x] = 0;
  if (threadIdx.x == 0) {
    tr->s_t = 0.0f;
    tr->amax_bits = 0u;
    tr->pad[0] = 0u;
    tr->pad[1] = 0u;
  }
}

// An NVFP4 quantization whose amax is given (mx_quantize_amax): the amax is
// the largest magnitude among `nslots` (<= 256) fp32 words. Each workgroup
// reduces them itself, one word per thread of its 4 waves, then a wave max
// and a max over the waves through LDS; s_t derives from the result as from
// a reduced amax, and workgroup 0 writes the trailer and zeroes the padding
// before it, so no separate launch precedes the encode. Called by every
// thread of a 256-thread workgroup in uniform control flow.
struct NvGiven {
  const uint32_t* words;   // nullptr: the amax is in the trailer already
  int nslots;
  uint8_t* gap;
  int gap_bytes;
};

__device__ __forceinline__ uint32_t nv_given_amax(const NvGiven& gv, NvTrailer* tr) {
  __shared__ uint32_t wave_max[4];
  const int t = threadIdx.x;
  uint32_t b = t < gv.nslots ? gv.words[t] & 0x7FFFFFFFu : 0u;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) b = max(b, (uint32_t)__shfl_xor((int)b, off));
  if ((t & 63) == 0) wave_max[t >> 6] = b;
  __syncthreads();
  b = max(max(wave_max[0], wave_max[1]), max(wave_max[2], wave_max[3]));
  if (blockIdx.x == 0) {
    if (t < gv.gap_bytes) gv.gap[t] = 0;
    if (t == 0) {
      tr->amax_bits = b;
      tr->pad[0] = 0u;
      tr->pad[1] = 0u;
    }
  }
  return b;
}

// The tensor scale an NVFP4 encode uses: from the given words, or from the
// amax already reduced into the trailer; workgroup 0 records it there.
__device__ __forceinline__ float nv_kernel_s_t(const NvGiven& gv, NvTrailer* tr) {
  const uint32_t b = gv.words != nullptr ? nv_given_amax(gv, tr) : tr->amax_bits;
  const float s_t = nvfp4_tensor_scale(b);
  if (blockIdx.x == 0 && threadIdx.x == 0) tr->s_t = s_t;
  return s_t;
}

// Largest |x| of X [rows, cols]: 8-element groups, gpr per row. A grid of
// about one workgroup per CU walks the tensor with 4 loads in flight per
// thread; waves reduce through LDS and each workgroup issues one atomic
// (many atomics on one address serialize in the L2).
constexpr int kAmaxUnroll = 4;

__global__ __launch_bounds__(256) void amax_kernel(const uint16_t* __restrict__ src, int rows, int cols, int ld,
                                                   int gpr, NvTrailer* tr) {
  __shared__ uint32_t wave_max[4];
  const int total = rows * gpr;
  const bool vec_ok = (ld % 8) == 0 && ((uintptr_t)src % 16) == 0;
  const int stride = gridDim.x * blockDim.x;
  uint32_t m = 0;
  for (int base = blockIdx.x * blockDim.x + threadIdx.x; base < total; base += stride * kAmaxUnroll) {
    uint4 v[kAmaxUnroll];
    bool full[kAmaxUnroll];
#pragma unroll
    for (int u = 0; u < kAmaxUnroll; ++u) {
      const int i = base + u * stride;
      v[u] = make_uint4(0u, 0u, 0u, 0u);
      full[u] = false;
      if (i < total) {
        const int r = i / gpr;
        const int c = (i - r * gpr) * 8;
        const uint16_t* p = src + (int64_t)r * ld + c;
        if (vec_ok && c + 8 <= cols) {
          v[u] = load16_stream(p);
          full[u] = true;
        } else {
          uint32_t mm = 0;
          for (int k = 0; k < 8 && c + k < cols; ++k) mm = max(mm, (uint32_t)p[k] & 0x7FFFu);
          m = max(m, mm);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kAmaxUnroll; ++u) {
      if (!full[u]) continue;
      const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        m = max(m, w[k] & 0x7FFFu);
        m = max(m, (w[k] >> 16) & 0x7FFFu);
      }
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
  if ((threadIdx.x & 63) == 0) wave_max[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t b = max(max(wave_max[0], wave_max[1]), max(wave_max[2], wave_max[3]));
    if (b != 0) atomicMax(&tr->amax_bits, b << 16);
  }
}

// ------------------------------------------------------------ shared encode

// Per-block scale of one lane's block given the block's amax bits; returns
// the scale byte and, for NVFP4, sets the element thresholds.
template <int FMT>
__device__ __forceinline__ uint32_t block_scale(uint32_t amax_bits, float s_t, Nv4Thresholds& th) {
  if (FMT == FMT_NVFP4) {
    const double q = (s_t == 0.0f) ? 0.0 : (double)bf16_to_f32(amax_bits) / (6.0 * (double)s_t);
    const uint32_t b = e4m3_encode_pos_f64(q);
    th = nvfp4_thresholds(e4m3_value(b) * (double)s_t);
    return b;
  }
  const int e = mx_shared_exp(amax_bits, FMT == FMT_MXFP8 ? 8 : 2);
  return (uint32_t)(e + 127);
}

// ------------------------------------------------------------ NVFP4 encode
//
// The NVFP4 element code is the E2M1 rounding (nearest, ties to the even
// code, saturating at 6) of the real quotient |x| / S with S = E4M3(byte) *
// s_t, sign copied. The threshold form (nvfp4_thresholds / nvfp4_encode)
// compares |x| with the fp32 ceilings of the seven midpoints times S: seven
// compares per element and fp64 work per block. The fast form below gets the
// same codes with gfx950's scaled E2M1 conversion, which at scale 2^0 rounds
// an fp32 value to nearest even, saturates at 6 and keeps the sign: it
// converts x * r_lo and x * r_hi, where r_lo < 1 / S < r_hi bracket the
// reciprocal within 2^-19 (relative). The two products then bracket the
// quotient and the conversion is monotone, so two equal codes are the
// quotient's code; they differ only when a midpoint lies within about 2^-19
// of the quotient (an exact tie or a near one), and then by one step, which
// an exact fp64 comparison with that midpoint settles. Both forms compute the
// same function; the fast one needs a finite block amax and an s_t for which
// S and 1 / S stay normal fp32.
//
// Error budget of the bracket: S32 = fp32(S) (2^-24), v_rcp_f32 (1 ulp,
// 2^-23), r_lo / r_hi rounded (2^-24) and the product rounded (2^-24): under
// 2^-21.5 in all, well inside the 2^-19 offsets.

struct Nv4Tensor {
  float s_t;
  float inv6;      // fp32(1 / (6 s_t)) when `fast`
  bool fast;       // s_t in [2^-96, 2^96] (false for 0, inf, NaN)
};

__device__ __forceinline__ Nv4Tensor nv4_tensor(float s_t) {
  Nv4Tensor t;
  t.s_t = s_t;
  t.fast = s_t >= 0x1p-96f && s_t <= 0x1p96f;
  t.inv6 = t.fast ? (float)(1.0 / (6.0 * (double)s_t)) : 0.0f;
  return t;
}

// E4M3 byte (RNE, saturating at 448) of a q >= 0 known through qf, an fp32
// value within 2^-22 (relative) of it. False when qf is too close to a
// rounding midpoint for its rounding to be the rounding of q.
__device__ __forceinline__ bool e4m3_from_near(float qf, uint32_t& b) {
  if (qf >= 448.0f) {                   // q > 447.9: 448 (the midpoint below it is 432)
    b = 0x7Eu;
    return true;
  }
  if (qf >= 0x1p-6f) {                  // normal E4M3: keep 3 of the 23 fraction bits
    const uint32_t u = __float_as_uint(qf);
    const uint32_t low = u & 0xFFFFFu;  // the midpoint is low == 0x80000
    if (low - 0x7FFF0u < 0x21u) return false;
    b = ((u + 0x7FFFFu + ((u >> 20) & 1u)) >> 20) - (120u << 3);
    return true;
  }
  const float t = qf * 512.0f;          // subnormal E4M3: multiples of 2^-9 (t < 8, exact)
  const float fl = floorf(t);
  const float fr = t - fl;
  if (fabsf(fr - 0.5f) < 0x1p-16f) return false;
  b = (uint32_t)fl + (fr > 0.5f ? 1u : 0u);
  return true;
}

struct Nv4Block {
  uint32_t sb;     // E4M3 scale byte
  bool fast;       // the bracket below is valid
  float r_lo, r_hi;
};

// Block scale byte of q = amax / (6 s_t) and the reciprocal bracket of S.
__device__ __forceinline__ Nv4Block nv4_block(uint32_t amax_bits, const Nv4Tensor& T) {
  Nv4Block B;
  const bool finite = amax_bits < 0x7F80u;
  uint32_t b = 0u;
  if (!(T.fast && finite && e4m3_from_near(bf16_to_f32(amax_bits) * T.inv6, b))) {
    const double q = (T.s_t == 0.0f) ? 0.0 : (double)bf16_to_f32(amax_bits) / (6.0 * (double)T.s_t);
    b = e4m3_encode_pos_f64(q);
  }
  B.sb = b;
  B.fast = T.fast && finite;
  const float r = b ? __builtin_amdgcn_rcpf((float)e4m3_value(b) * T.s_t) : 0.0f;   // S = 0: codes are signs
  B.r_lo = r * (1.0f - 0x1p-19f);
  B.r_hi = r * (1.0f + 0x1p-19f);
  return B;
}

// 8 NVFP4 codes (nibble i = x[i]) of one block's elements.
__device__ __forceinline__ uint32_t nv4_encode8(const float (&x)[8], const Nv4Block& B, const Nv4Tensor& T) {
  const float one = 1.0f;               // scale operand 2^0
  uint32_t lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, x[0] * B.r_lo, x[1] * B.r_lo, one, 0);
  uint32_t hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, x[0] * B.r_hi, x[1] * B.r_hi, one, 0);
  lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo, x[2] * B.r_lo, x[3] * B.r_lo, one, 1);
  hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi, x[2] * B.r_hi, x[3] * B.r_hi, one, 1);
  lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo, x[4] * B.r_lo, x[5] * B.r_lo, one, 2);
  hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi, x[4] * B.r_hi, x[5] * B.r_hi, one, 2);
  lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo, x[6] * B.r_lo, x[7] * B.r_lo, one, 3);
  hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi, x[6] * B.r_hi, x[7] * B.r_hi, one, 3);
  if (B.fast) {
    if (lo == hi) return lo;
    // Elements whose bracket straddles a midpoint (ties are common: with s_t
    // from a bf16 amax the quotients are ratios of short integers): their
    // two codes are c and c + 1 around the midpoint m_c, and the code is c +
    // 1 when |x| > m_c S, or |x| == m_c S with c odd (ties to even). In fp64
    // both sides are exact (m_c S has at most 33 significant bits).
    const double S = e4m3_value(B.sb) * (double)T.s_t;
    const uint32_t diff = lo ^ hi;
    uint32_t word = lo;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if ((diff >> (4 * i)) & 0xFu) {
        const uint32_t c = (lo >> (4 * i)) & 7u;
        const double m = c < 4u ? 0.25 + 0.5 * (double)c : (c == 6u ? 5.0 : (double)c - 1.5);
        const double a = fabs((double)x[i]), t = m * S;
        if (a > t || (a == t && (c & 1u))) word += 1u << (4 * i);   // c <= 6: the sign bit is untouched
      }
    }
    return word;
  }
  const Nv4Thresholds th = nvfp4_thresholds(e4m3_value(B.sb) * (double)T.s_t);
  uint32_t word = 0u;
#pragma unroll
  for (int i = 0; i < 8; ++i) word |= nvfp4_encode(x[i], th) << (4 * i);
  return word;
}

// Encode 8 values with MX scale byte sb; packed codes in the low 64 (fp8) or
// 32 (fp4) bits. (NVFP4 goes through nv4_encode8.)
template <int FMT>
__device__ __forceinline__ uint64_t encode8(const float (&x)[8], uint32_t sb, const Nv4Thresholds&) {
  static_assert(FMT != FMT_NVFP4, "NVFP4 elements are encoded by nv4_encode8");
  if (FMT == FMT_MXFP8)
    return (uint64_t)e4m3x4_scaled(x[0], x[1], x[2], x[3], sb) | ((uint64_t)e4m3x4_scaled(x[4], x[5], x[6], x[7], sb) << 32);
  return e2m1x8_scaled(x, sb);
}

// ------------------------------------------------------------ row quantizer

// Groups of 8 elements per thread: four loads in flight per thread for
// large tensors, two for tensors of fewer than 2^20 groups (a few million
// elements), which then spread over more workgroups and finish sooner.
constexpr int kRowGroupsPerThread = 4;
constexpr int kRowGroupsSmall = 2;
constexpr int64_t kRowSmallGroups = 1 << 20;

// Row quantization of one tensor by threads first_tid, first_tid + stride,
// ... of the threads given to it (each thread: U groups of 8 elements of one
// stored row).
template <int FMT, int U>
__device__ __forceinline__ uint32_t quant_rows(const uint16_t* __restrict__ src, int rows, int cols, int ld,
                                               uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, int kpad,
                                               float s_t, int first_tid, int stride) {
  constexpr int BS = (FMT == FMT_NVFP4) ? 16 : 32;
  constexpr int LANES_PER_BLOCK = BS / 8;
  static_assert(U == 1 || U == 2 || U == 4, "kpad / 8 (a multiple of 16) / U must stay a multiple of 4");
  const int gpr = kpad / 8;                       // groups per stored row (multiple of 16)
  const int tpr = gpr / U;                        // threads per row: a multiple of 4, so the lanes of a block
                                                  // are adjacent, aligned and in one row
  const int total = rows * tpr;
  const bool vec_ok = (ld % 8) == 0 && ((uintptr_t)src % 16) == 0;
  [[maybe_unused]] const Nv4Tensor nt = nv4_tensor(s_t);
  uint32_t own_max = 0u;                          // largest |x| bits this thread saw
  for (int tid = first_tid; tid < total; tid += stride) {
    const int r = tid / tpr;
    const int j = tid - r * tpr;
    const uint16_t* row = src + (int64_t)r * ld;
    uint32_t w[U][4];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = (j + tpr * u) * 8;
      w[u][0] = w[u][1] = w[u][2] = w[u][3] = 0u;
      if (vec_ok && c + 8 <= cols) {
        const uint4 v = load16_stream(row + c);
        w[u][0] = v.x; w[u][1] = v.y; w[u][2] = v.z; w[u][3] = v.w;
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (c + i < cols) w[u][i / 2] |= (uint32_t)row[c + i] << (16 * (i % 2));
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = (j + tpr * u) * 8;
      float x[8];
      uint32_t m = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t b = (w[u][i / 2] >> (16 * (i % 2))) & 0xFFFFu;
        x[i] = bf16_to_f32(b);
        m = max(m, b & 0x7FFFu);
      }
      own_max = max(own_max, m);
      // block amax across the adjacent lanes of this block
#pragma unroll
      for (int off = 1; off < LANES_PER_BLOCK; off <<= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
      uint32_t sb;
      uint64_t packed;
      if constexpr (FMT == FMT_NVFP4) {
        const Nv4Block B = nv4_block(m, nt);
        sb = B.sb;
        packed = nv4_encode8(x, B, nt);
      } else {
        Nv4Thresholds th;
        sb = block_scale<FMT>(m, s_t, th);
        packed = encode8<FMT>(x, sb, th);
      }
      if (FMT == FMT_MXFP8) {
        *reinterpret_cast<uint2*>(codes + (int64_t)r * kpad + c) = make_uint2((uint32_t)packed, (uint32_t)(packed >> 32));
      } else {
        *reinterpret_cast<uint32_t*>(codes + (int64_t)r * (kpad / 2) + c / 2) = (uint32_t)packed;
      }
      if ((j % LANES_PER_BLOCK) == 0) scales[(int64_t)r * (kpad / BS) + c / BS] = (uint8_t)sb;
    }
  }
  return own_max;
}

template <int FMT, int U>
__global__ __launch_bounds__(256) void quant_row_kernel(const uint16_t* __restrict__ src, int rows, int cols, int ld,
                                                        uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                                        int kpad, NvTrailer* tr, NvGiven gv) {
  float s_t = 0.0f;
  if (FMT == FMT_NVFP4) s_t = nv_kernel_s_t(gv, tr);
  quant_rows<FMT, U>(src, rows, cols, ld, codes, scales, kpad, s_t, blockIdx.x * blockDim.x + threadIdx.x,
                  gridDim.x * blockDim.x);
}

// Several MX tensors in one launch: workgroups first_wg[i] .. first_wg[i+1]-1
// quantize item i (the search is over a handful of kernel-argument entries,
// uniform per workgroup).
// AMAX: each item's tensor amax (bf16 magnitude bits, as fp32 bits) is also
// reduced, one atomic max per workgroup into one of kAmaxLines words of the
// item's accumulators, each on its own 128-byte line. Atomics on one line
// are served one after another (about 9 ns each, measured): thousands of
// workgroups on one line cost 50 us on an 11235 x 4096 tensor; spread over
// lines, and finishing throughout the launch, they do not queue.
template <int FMT, bool AMAX>
__global__ __launch_bounds__(256) void quant_row_batch_kernel(const QuantBatch batch) {
  __shared__ uint32_t wave_max[4];
  int i = 0;
  while (i + 1 < batch.n && (int)blockIdx.x >= batch.first_wg[i + 1]) ++i;
  const QuantBatchItem& it = batch.items[i];
  const int wg = (int)blockIdx.x - batch.first_wg[i];
  const int nwg = batch.first_wg[i + 1] - batch.first_wg[i];
  uint32_t m = quant_rows<FMT, kRowGroupsPerThread>(it.src, it.rows, it.cols, it.ld, it.codes, it.scales, it.kpad,
                                                    0.0f, wg * 256 + (int)threadIdx.x, nwg * 256);
  if constexpr (AMAX) {
    const int t = threadIdx.x;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
    if ((t & 63) == 0) wave_max[t >> 6] = m;
    __syncthreads();
    if (t == 0) {
      const uint32_t b = max(max(wave_max[0], wave_max[1]), max(wave_max[2], wave_max[3]));
      if (b != 0) atomicMax(&it.amax[(blockIdx.x % kAmaxLines) * kAmaxStride], b << 16);
    }
  }
}

// Zeroes n words (the amax accumulators of mx_quantize_batch_amax).
__global__ void zero_words_kernel(uint32_t* w, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) w[i] = 0u;
}

// ------------------------------------------------------------ col quantizer

constexpr int kColTileR = 128;   // rows of X (the block axis) per tile
constexpr int kColTileC = 64;    // columns of X per tile
constexpr int kColLdsLd = kColTileC + 8;   // padded LDS row (elements), keeps 16-B alignment

// Column-copy output of one 128 x 64 tile, staged through LDS so that the
// stores are whole row segments. col_stage_write: lane j of wave w hands in
// the codes of output row c0 + j, elements r0 + 32 w .. + 31 (CB bytes: 32
// for MXFP8, 16 for the fp4 formats) and their scale bytes (NVFP4: two, in
// the low 16 bits; MX: one); they go to `stage` as rows of 4 CB bytes (+16
// bytes of padding, which keeps a wave's 16-byte writes on distinct banks)
// followed by 64 rows of scale bytes. col_stage_flush, after a barrier:
// each output row is stored as 16-byte chunks by adjacent lanes and its
// scale bytes by one lane (one write request per row segment instead of one
// per lane and chunk); output rows at or past `cols` are dropped. Every
// thread of the workgroup calls both.
template <int FMT>
struct ColStage {
  static constexpr int CB = (FMT == FMT_MXFP8) ? 32 : 16;   // code bytes per lane
  static constexpr int ROW = 4 * CB;                         // code bytes per output row of the tile
  static constexpr int CS = ROW + 16;                        // staged row stride
  static constexpr int BS = (FMT == FMT_NVFP4) ? 16 : 32;
  static constexpr int NSB = 128 / BS;                       // scale bytes per output row of the tile
  static constexpr int SC_OFF = 64 * CS;
  static constexpr int BYTES = SC_OFF + 64 * NSB;
};

template <int FMT>
__device__ __forceinline__ void col_stage_write(uint8_t* stage, int t, const uint32_t (&words)[8], uint32_t sbytes) {
  using C = ColStage<FMT>;
  const int w = t / 64, j = t % 64;
  uint8_t* dst = stage + j * C::CS + w * C::CB;
  *reinterpret_cast<uint4*>(dst) = make_uint4(words[0], words[1], words[2], words[3]);
  if (C::CB == 32) *reinterpret_cast<uint4*>(dst + 16) = make_uint4(words[4], words[5], words[6], words[7]);
  if (FMT == FMT_NVFP4) {
    *reinterpret_cast<uint16_t*>(stage + C::SC_OFF + j * C::NSB + 2 * w) = (uint16_t)sbytes;
  } else {
    stage[C::SC_OFF + j * C::NSB + w] = (uint8_t)sbytes;
  }
}

template <int FMT>
__device__ __forceinline__ void col_stage_flush(const uint8_t* stage, int t, __amdgpu_buffer_rsrc_t codes,
                                                __amdgpu_buffer_rsrc_t scales, int kpad, int r0, int c0, int cols) {
  using C = ColStage<FMT>;
  constexpr int RC = C::ROW / 16;                            // 16-byte chunks per output row
  static_assert((64 * RC) % 256 == 0, "every thread stores the same number of chunks");
  typedef unsigned v4u __attribute__((ext_vector_type(4)));
  typedef unsigned v2u __attribute__((ext_vector_type(2)));
  const int out_row = (FMT == FMT_MXFP8) ? kpad : kpad / 2;
  const int first = (FMT == FMT_MXFP8) ? r0 : r0 / 2;        // byte offset of the tile in an output row
#pragma unroll
  for (int q = t; q < 64 * RC; q += 256) {
    const int row = q / RC, k = q % RC;
    const uint4 c = *reinterpret_cast<const uint4*>(stage + row * C::CS + 16 * k);
    const uint32_t off = c0 + row < cols ? (uint32_t)((c0 + row) * out_row + first + 16 * k) : kDropped;
    __builtin_amdgcn_raw_buffer_store_b128(v4u{c.x, c.y, c.z, c.w}, codes, off, 0, 0);
  }
  // scale bytes: row t of the tile, by the first wave (the others drop theirs)
  const int srow = t % 64;
  const uint32_t soff = (t < 64 && c0 + srow < cols) ? (uint32_t)((c0 + srow) * (kpad / C::BS) + r0 / C::BS) : kDropped;
  if (C::NSB == 8) {
    const uint2 sv = *reinterpret_cast<const uint2*>(stage + C::SC_OFF + srow * C::NSB);
    __builtin_amdgcn_raw_buffer_store_b64(v2u{sv.x, sv.y}, scales, soff, 0, 0);
  } else {
    __builtin_amdgcn_raw_buffer_store_b32(*reinterpret_cast<const uint32_t*>(stage + C::SC_OFF + srow * C::NSB), scales,
                                          soff, 0, 0);
  }
}

// ------------------------------------------------------------ stochastic rounding

// Philox4x64-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as
// easy as 1, 2, 3", SC 2011): ten rounds of the four-word round function,
// the key bumped by the Weyl constants between rounds.
// 128-bit product m * c as (hi, lo), from four 32 x 32 -> 64 multiply-adds
// (V_MAD_U64_U32); no partial sum overflows 64 bits.
__device__ __forceinline__ void mul_64x64(uint64_t m, uint64_t c, uint64_t& hi, uint64_t& lo) {
  const uint32_t m0 = (uint32_t)m, m1 = (uint32_t)(m >> 32), c0 = (uint32_t)c, c1 = (uint32_t)(c >> 32);
  const uint64_t p00 = (uint64_t)m0 * c0;
  const uint64_t p01 = (uint64_t)m0 * c1 + (p00 >> 32);
  const uint64_t p10 = (uint64_t)m1 * c0 + (uint32_t)p01;
  hi = (uint64_t)m1 * c1 + (p01 >> 32) + (p10 >> 32);
  lo = (p10 << 32) | (uint32_t)p00;
}

__device__ __forceinline__ void philox4x64_10(uint64_t (&c)[4], uint64_t k0, uint64_t k1) {
  constexpr uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  constexpr uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    uint64_t hi0, lo0, hi1, lo1;
    mul_64x64(M0, c[0], hi0, lo0);
    mul_64x64(M1, c[2], hi1, lo1);
    const uint64_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
    k0 += W0;
    k1 += W1;
  }
}

// The eight 32-bit draws of elements 8q .. 8q + 7 of X (row-major element
// order): Philox4x64-10 of counter (q, 0, 0, 0), each word split low half
// first.
__device__ __forceinline__ void sr_draws8(uint64_t q, uint64_t k0, uint64_t k1, uint32_t (&d)[8]) {
  uint64_t c[4] = {q, 0ull, 0ull, 0ull};
  philox4x64_10(c, k0, k1);
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    d[2 * w] = (uint32_t)c[w];
    d[2 * w + 1] = (uint32_t)(c[w] >> 32);
  }
}

// E2M1 magnitude code of y >= 0 rounded stochastically with draw u: between
// the grid neighbours lo <= y < hi, hi iff u < ceil(frac * 2^32), frac =
// (y - lo) / (hi - lo) (exact); y >= 6 saturates.
// Without branches: the grid spacing is 2^(e - 1) with e = clamp(floor(log2
// y), 0, 2), so s = y / spacing is exact, floor(s) + 2e is the code of lo and
// s - floor(s) the exact fraction.
__device__ __forceinline__ uint32_t e2m1_sr(float y, uint32_t u) {
  const int E = (int)(__float_as_uint(y) >> 23) - 127;     // y >= 0
  const int e = min(max(E, 0), 2);
  const float s = y * __uint_as_float((uint32_t)(128 - e) << 23);   // y * 2^(1 - e), exact
  const float f = floorf(s);
  const float frac = s - f;                                // exact
  const uint32_t T = (uint32_t)ceilf(frac * 4294967296.0f); // < 2^32 - 255: exact
  const uint32_t code = (uint32_t)f + 2u * (uint32_t)e + (u < T ? 1u : 0u);
  return y < 6.0f ? code : 7u;                             // 6 and above (inf, NaN too): 6
}

// fp64 reciprocal of a block's S32 = fp32(dec(byte) * s_t) for
// nvfp4_encode_sr (0 when S32 is not positive).
__device__ __forceinline__ double sr_inv_scale(float S32) { return S32 > 0.0f ? 1.0 / (double)S32 : 0.0; }

// NVFP4 code of x with scale S32 > 0, rounded stochastically with draw u:
// y = fp32(|x| / S32), the correctly rounded quotient, sign copied from x
// (S32 = 0: a zero code). y comes from fp64 instead of an fp32 division:
// |x| (a bf16 value, at most 8 significant bits) over S32 (24 bits) is never
// an fp32 rounding midpoint and lies at least 2^-25 ulp from every one (the
// difference |x| - m S32 for a midpoint m is a nonzero multiple of
// ulp(m) S32 / 2^25 or coarser), while |x| * RN64(1 / S32) in fp64 is within
// 2^-52 of the quotient (relative; also for fp32-subnormal results, whose
// midpoints are as far apart in ulps). Rounding that product to fp32 is
// therefore the rounding of the quotient itself.
__device__ __forceinline__ uint32_t nvfp4_encode_sr(float x, double inv_S, uint32_t u) {
  const uint32_t sign = (__float_as_uint(x) >> 28) & 8u;
  const float y = (float)((double)fabsf(x) * inv_S);
  return sign | (inv_S > 0.0 ? e2m1_sr(y, u) : 0u);
}

// Tile walk of a persistent grid (gridDim.x a multiple of 8). Workgroups are
// dealt to the 8 XCDs round-robin, so workgroup b runs on XCD b % 8; each XCD
// takes a contiguous range of tile numbers and its workgroups interleave over
// it (number start + b / 8 + i * gridDim.x / 8). A workgroup walks several
// tiles and loads the next one while it encodes the current one: with one
// tile per workgroup, loads were only in flight between encodes, too few
// bytes to cover HBM latency.
struct TileWalk {
  int first, step, end;
};

__device__ __forceinline__ TileWalk tile_walk(int ntiles) {
  const int x = (int)blockIdx.x % 8, nb = (int)gridDim.x / 8;
  const int q = ntiles / 8, r = ntiles % 8;
  const int start = x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q;
  return {start + (int)blockIdx.x / 8, nb, start + q + (x < r ? 1 : 0)};
}

// Tile (row, column) of tile number n: super-rows of 8 tile rows, numbered
// down each column of tiles, then across. Tiles that share output lines then
// get numbers close together (one XCD, the same step of the walk): the column
// copy's scale bytes of 8 tiles down a column fill one 64-byte segment, and
// its codes of 2 tiles one 128-byte line; the row copy's codes of 4 tiles
// across fill a line (scale bytes: 16). Lines written in parts by different
// L2s, or evicted between parts, cost extra partial writes to HBM.
__device__ __forceinline__ void tile_coords(int n, int tiles_r, int tiles_c, int& r0, int& c0) {
  const int band = n / (8 * tiles_c);
  const int h = min(8, tiles_r - 8 * band);
  const int rem = n - band * 8 * tiles_c;
  const int tc = rem / h;
  r0 = (8 * band + rem - tc * h) * kColTileR;
  c0 = tc * kColTileC;
}

// Thread t's share of the 128 x 64 tile at (r0, c0): 8 columns of rows
// t / 8 + 32 p (16-byte loads), zeros outside X.
__device__ __forceinline__ void load_tile(uint4 (&v)[4], const uint16_t* __restrict__ src, int rows, int cols, int ld,
                                          bool vec_ok, int r0, int c0, int t) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int r = r0 + t / 8 + 32 * p, c = c0 + (t % 8) * 8;
    v[p] = make_uint4(0u, 0u, 0u, 0u);
    if (r < rows && c < cols) {
      const uint16_t* q = src + (int64_t)r * ld + c;
      if (vec_ok && c + 8 <= cols) {
        v[p] = load16_stream(q);
      } else {
        uint32_t w[4] = {0u, 0u, 0u, 0u};
        for (int i = 0; i < 8; ++i)
          if (c + i < cols) w[i / 2] |= (uint32_t)q[i] << (16 * (i % 2));
        v[p] = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
  }
}

__device__ __forceinline__ void stage_tile(uint16_t* tile, const uint4 (&v)[4], int t) {
#pragma unroll
  for (int p = 0; p < 4; ++p) *reinterpret_cast<uint4*>(&tile[(t / 8 + 32 * p) * kColLdsLd + (t % 8) * 8]) = v[p];
}

// Elements 8g .. 8g + 7 of a lane's column, from the packed bf16 pairs.
__device__ __forceinline__ void unpack8(const uint32_t (&h)[16], int g, float (&x)[8]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    x[2 * k] = __uint_as_float(h[4 * g + k] << 16);
    x[2 * k + 1] = __uint_as_float(h[4 * g + k] & 0xFFFF0000u);
  }
}

// Column pass of a staged tile: wave w owns tile rows 32 w .. 32 w + 31, lane
// j column j (output row c0 + j; lanes past `cols` encode zeros that are
// never stored). The 32 values are kept as 16 packed bf16 pairs: block amax
// first, then the codes 8 at a time. NVFP4: two 16-row blocks, their scale
// bytes in the low 16 bits of sbytes; stochastic rounding takes element k's
// draw from draw[(32 w + k) * 64 + j]. MX: one 32-row block.
template <int FMT, bool SR>
__device__ __forceinline__ void col_encode(const uint16_t* tile, const uint32_t* draw, int w, int j,
                                           const Nv4Tensor& nt, uint32_t (&words)[8], uint32_t& sbytes) {
  uint32_t h[16];
  uint32_t m2[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t lo = tile[(32 * w + 2 * i) * kColLdsLd + j];
    const uint32_t hi = tile[(32 * w + 2 * i + 1) * kColLdsLd + j];
    h[i] = lo | (hi << 16);
    m2[i / 8] = max(m2[i / 8], max(lo & 0x7FFFu, hi & 0x7FFFu));
  }
#pragma unroll
  for (int q = 0; q < 8; ++q) words[q] = 0u;
  sbytes = 0u;
  if constexpr (FMT == FMT_NVFP4) {
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const Nv4Block B = nv4_block(m2[hb], nt);
      [[maybe_unused]] double inv_S = 0.0;
      if constexpr (SR) inv_S = sr_inv_scale(__fmul_rn((float)e4m3_value(B.sb), nt.s_t));
#pragma unroll
      for (int q2 = 0; q2 < 2; ++q2) {
        float x[8];
        unpack8(h, 2 * hb + q2, x);
        if constexpr (SR) {
          uint32_t word = 0u;
#pragma unroll
          for (int i = 0; i < 8; ++i)
            word |= nvfp4_encode_sr(x[i], inv_S, draw[(32 * w + 16 * hb + 8 * q2 + i) * kColTileC + j]) << (4 * i);
          words[2 * hb + q2] = word;
        } else {
          words[2 * hb + q2] = nv4_encode8(x, B, nt);
        }
      }
      sbytes |= B.sb << (8 * hb);
    }
  } else {
    Nv4Thresholds th;
    const uint32_t sb = block_scale<FMT>(max(m2[0], m2[1]), 0.0f, th);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      float x[8];
      unpack8(h, g, x);
      if (FMT == FMT_MXFP8) {
        words[2 * g] = e4m3x4_scaled(x[0], x[1], x[2], x[3], sb);
        words[2 * g + 1] = e4m3x4_scaled(x[4], x[5], x[6], x[7], sb);
      } else {
        words[g] = e2m1x8_scaled(x, sb);
      }
    }
    sbytes = sb;
  }
}

// X [rows, cols] -> codes of X^T: [cols, kpad] with kpad = round_up(rows, 128).
template <int FMT>
__global__ __launch_bounds__(256) void quant_col_kernel(const uint16_t* __restrict__ src, int rows, int cols, int ld,
                                                        uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                                        int kpad, NvTrailer* tr, NvGiven gv) {
  __shared__ __align__(16) uint16_t tile[kColTileR * kColLdsLd];
  uint8_t* const stage = reinterpret_cast<uint8_t*>(tile);   // the staged output reuses the tile
  static_assert(ColStage<FMT>::BYTES <= (int)sizeof(tile), "staged output fits in the tile buffer");
  const int tiles_c = (cols + kColTileC - 1) / kColTileC;
  const int tiles_r = kpad / kColTileR;
  const int ntiles = tiles_c * tiles_r;
  const bool vec_ok = (ld % 8) == 0 && ((uintptr_t)src % 16) == 0;
  const int t = threadIdx.x;
  // NVFP4: s_t is read once, after the first tile's loads are issued, so
  // that its loads and theirs are in flight together
  [[maybe_unused]] Nv4Tensor nt = nv4_tensor(0.0f);
  bool nt_ready = FMT != FMT_NVFP4;
  constexpr int BS = (FMT == FMT_NVFP4) ? 16 : 32;
  const __amdgpu_buffer_rsrc_t c_rs = out_rsrc(codes, (int64_t)cols * (FMT == FMT_MXFP8 ? kpad : kpad / 2));
  const __amdgpu_buffer_rsrc_t s_rs = out_rsrc(scales, (int64_t)cols * (kpad / BS));
  // one tile per workgroup when the grid covers the tiles (the launch does);
  // many workgroups resident per CU keep the loads in flight
  const TileWalk tw = tile_walk(ntiles);
  for (int n = tw.first; n < tw.end; n += tw.step) {
    int r0, c0;
    tile_coords(n, tiles_r, tiles_c, r0, c0);
    uint4 v[4];
    load_tile(v, src, rows, cols, ld, vec_ok, r0, c0, t);
    if (!nt_ready) {                          // uniform: the walk is per workgroup
      nt = nv4_tensor(nv_kernel_s_t(gv, tr));
      nt_ready = true;
    }
    stage_tile(tile, v, t);
    __syncthreads();                          // tile staged
    uint32_t words[8], sbytes;
    col_encode<FMT, false>(tile, nullptr, t / 64, t % 64, nt, words, sbytes);
    __syncthreads();                          // tile read
    col_stage_write<FMT>(stage, t, words, sbytes);
    __syncthreads();                          // output staged
    col_stage_flush<FMT>(stage, t, c_rs, s_rs, kpad, r0, c0, cols);
    __syncthreads();                          // staged output read
  }
  if (!nt_ready) nv_kernel_s_t(gv, tr);       // a workgroup without tiles still records the trailer
}

// ------------------------------------------------------------ fused row + col

// README section 5.5: the weight-gradient GEMM needs each operand twice,
// quantized along its rows and along its columns (stored transposed); one
// kernel reads X once and writes both copies. A 128 x 64 tile is loaded as
// in quant_col_kernel: thread t holds 8 consecutive elements of rows
// t / 8 + 32 p, which the 4 (MX) or 2 (NVFP4) adjacent lanes of a row block
// quantize straight from registers into the row copy, while the tile goes
// through LDS for the column copy. The tiles cover round_up(cols, 128)
// columns so that the row copy's padding is written too, and round_up(rows,
// 128) rows for the column copy's.
//
// NVFP4 tensor scale: either from this tensor's amax (reduced first into the
// row copy's trailer, as mx_quantize does), or delayed (README section 5.5):
// set before this kernel from an earlier amax times a headroom, in which case
// this kernel reduces the tensor's own amax into both trailers on the side
// (one atomic max per workgroup), for the next call.

// Trailers of both copies and the padding before them; with `delayed`,
// s_t = fp32(fp64(headroom * *amax_prev) / 2688), read before anything is
// written (amax_prev may be the amax field of either trailer).
__global__ void nv_dual_init_kernel(uint8_t* rgap, int rgap_bytes, NvTrailer* rtr, uint8_t* cgap, int cgap_bytes,
                                    NvTrailer* ctr, const float* amax_prev, float headroom, int delayed) {
  const int t = threadIdx.x;
  if (t == 0) {
    float s_t = 0.0f;
    if (delayed) s_t = (float)(((double)headroom * (double)*amax_prev) / 2688.0);
    rtr->s_t = s_t;
    ctr->s_t = s_t;
    rtr->amax_bits = ctr->amax_bits = 0u;
    rtr->pad[0] = rtr->pad[1] = ctr->pad[0] = ctr->pad[1] = 0u;
  }
  if (t < rgap_bytes) rgap[t] = 0;
  if (t < cgap_bytes) cgap[t] = 0;
}

// Row copy of 8 consecutive elements of tile row t / 8 + 32 p (thread t;
// the lanes of a row block are adjacent): block amax across the lanes, scale
// byte, codes, stores (dropped past the last row). Stochastic rounding draws
// the 8 elements' numbers here and leaves them in `draw` for the column copy.
template <int FMT, bool SR>
__device__ __forceinline__ void row_encode_store(const uint4 vv, int p, int t, int r0, int c0, int rows, int cols,
                                                 int rkpad, const Nv4Tensor& nt, uint32_t* draw, uint64_t seed0,
                                                 uint64_t seed1, __amdgpu_buffer_rsrc_t rc_rs,
                                                 __amdgpu_buffer_rsrc_t rs_rs, uint32_t& own_max) {
  constexpr int BS = (FMT == FMT_NVFP4) ? 16 : 32;
  constexpr int LANES_PER_BLOCK = BS / 8;
  typedef unsigned v2u __attribute__((ext_vector_type(2)));
  const int r = r0 + t / 8 + 32 * p, c = c0 + (t % 8) * 8;
  const uint32_t w[4] = {vv.x, vv.y, vv.z, vv.w};
  float x[8];
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t b = (w[i / 2] >> (16 * (i % 2))) & 0xFFFFu;
    x[i] = bf16_to_f32(b);
    m = max(m, b & 0x7FFFu);
  }
  own_max = max(own_max, m);
#pragma unroll
  for (int off = 1; off < LANES_PER_BLOCK; off <<= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
  uint32_t sb;
  uint64_t packed;
  if constexpr (SR) {
    sb = nv4_block(m, nt).sb;
    // draws of elements (r, c .. c + 7): one Philox block when the element
    // index r * cols + c is a multiple of 8 (cols % 8 == 0 is a
    // precondition); tile padding never reaches a code (its x is 0)
    uint32_t d[8];
    sr_draws8(((uint64_t)r * (uint64_t)cols + (uint64_t)c) >> 3, seed0, seed1, d);
    *reinterpret_cast<uint4*>(&draw[(t / 8 + 32 * p) * kColTileC + (t % 8) * 8]) = make_uint4(d[0], d[1], d[2], d[3]);
    *reinterpret_cast<uint4*>(&draw[(t / 8 + 32 * p) * kColTileC + (t % 8) * 8 + 4]) = make_uint4(d[4], d[5], d[6], d[7]);
    const double inv_S = sr_inv_scale(__fmul_rn((float)e4m3_value(sb), nt.s_t));
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) word |= nvfp4_encode_sr(x[i], inv_S, d[i]) << (4 * i);
    packed = word;
  } else if constexpr (FMT == FMT_NVFP4) {
    const Nv4Block B = nv4_block(m, nt);
    sb = B.sb;
    packed = nv4_encode8(x, B, nt);
  } else {
    Nv4Thresholds th;
    sb = block_scale<FMT>(m, 0.0f, th);
    packed = encode8<FMT>(x, sb, th);
  }
  if (FMT == FMT_MXFP8) {
    const uint32_t off = r < rows ? (uint32_t)(r * rkpad + c) : kDropped;
    __builtin_amdgcn_raw_buffer_store_b64(v2u{(uint32_t)packed, (uint32_t)(packed >> 32)}, rc_rs, off, 0, 0);
  } else {
    const uint32_t off = r < rows ? (uint32_t)(r * (rkpad / 2) + c / 2) : kDropped;
    __builtin_amdgcn_raw_buffer_store_b32((uint32_t)packed, rc_rs, off, 0, 0);
  }
  const uint32_t soff = (r < rows && ((t % 8) % LANES_PER_BLOCK) == 0) ? (uint32_t)(r * (rkpad / BS) + c / BS) : kDropped;
  __builtin_amdgcn_raw_buffer_store_b8((uint8_t)sb, rs_rs, soff, 0, 0);
}

// WALK: a persistent grid walks the tiles, loading the next one while it
// encodes the current one (the staged column output gets a buffer of its
// own: it is stored while the next tile is already staged); pays off where
// encoding is long (NVFP4). Otherwise one tile per workgroup, the many
// resident workgroups keeping loads in flight, and the output staged in the
// tile buffer.
template <int FMT, bool SR, bool WALK>
__global__ __launch_bounds__(256) void quant_dual_kernel(const uint16_t* __restrict__ src, int rows, int cols, int ld,
                                                         uint8_t* __restrict__ rcodes, uint8_t* __restrict__ rscales,
                                                         int rkpad, uint8_t* __restrict__ ccodes,
                                                         uint8_t* __restrict__ cscales, int ckpad, NvTrailer* rtr,
                                                         NvTrailer* ctr, int delayed, uint64_t seed0, uint64_t seed1) {
  constexpr int BS = (FMT == FMT_NVFP4) ? 16 : 32;
  static_assert(!SR || FMT == FMT_NVFP4, "stochastic rounding is an NVFP4 option");
  __shared__ __align__(16) uint16_t tile[kColTileR * kColLdsLd];
  // stochastic rounding: the draw of every element of the tile, written by
  // the row pass and read by the column pass (one draw per element of X).
  // WALK: the staged column output, which shares the draws' space (it is
  // written after the column pass has read them and stored before the next
  // row pass writes them).
  constexpr int kDrawWords = kColTileR * kColTileC, kStageWords = (ColStage<FMT>::BYTES + 3) / 4;
  __shared__ __align__(16) uint32_t draw[SR ? kDrawWords : (WALK ? kStageWords : 4)];
  uint8_t* const stage = WALK ? reinterpret_cast<uint8_t*>(draw) : reinterpret_cast<uint8_t*>(tile);
  static_assert(ColStage<FMT>::BYTES <= (int)sizeof(tile) && (!WALK || kStageWords * 4 <= (int)sizeof(draw)),
                "staged output fits");
  __shared__ uint32_t wave_max[4];
  const int tiles_c = rkpad / kColTileC;
  const int tiles_r = ckpad / kColTileR;
  const int ntiles = tiles_c * tiles_r;
  const bool vec_ok = (ld % 8) == 0 && ((uintptr_t)src % 16) == 0;
  const int t = threadIdx.x;
  float s_t = 0.0f;
  if (FMT == FMT_NVFP4) {
    if (delayed) {
      s_t = rtr->s_t;
    } else {
      s_t = nvfp4_tensor_scale(rtr->amax_bits);
      if (blockIdx.x == 0 && t == 0) {
        rtr->s_t = s_t;
        ctr->s_t = s_t;
        ctr->amax_bits = rtr->amax_bits;
      }
    }
  }
  [[maybe_unused]] const Nv4Tensor nt = nv4_tensor(s_t);
  const __amdgpu_buffer_rsrc_t rc_rs = out_rsrc(rcodes, (int64_t)rows * (FMT == FMT_MXFP8 ? rkpad : rkpad / 2));
  const __amdgpu_buffer_rsrc_t rs_rs = out_rsrc(rscales, (int64_t)rows * (rkpad / BS));
  const __amdgpu_buffer_rsrc_t cc_rs = out_rsrc(ccodes, (int64_t)cols * (FMT == FMT_MXFP8 ? ckpad : ckpad / 2));
  const __amdgpu_buffer_rsrc_t cs_rs = out_rsrc(cscales, (int64_t)cols * (ckpad / BS));
  uint32_t own_max = 0u;                      // largest |x| bits this thread saw (delayed NVFP4)
  const TileWalk tw = tile_walk(ntiles);
  if constexpr (WALK) {
    uint4 v[4];
    int nr0 = 0, nc0 = 0;                     // the tile in v
    if (tw.first < tw.end) {
      tile_coords(tw.first, tiles_r, tiles_c, nr0, nc0);
      load_tile(v, src, rows, cols, ld, vec_ok, nr0, nc0, t);
    }
    // Per tile: stage it, store the previous tile's staged column output,
    // load the next tile, then encode both copies (the row copy's stores go
    // out during the encode). The loop head waits for every memory operation
    // in flight (loads and stores share one counter), which were then all
    // issued an encode earlier.
    int pr0 = -1, pc0 = 0;
    for (int n = tw.first; n < tw.end; n += tw.step) {
      const int r0 = nr0, c0 = nc0;
      stage_tile(tile, v, t);
      if (pr0 >= 0) col_stage_flush<FMT>(stage, t, cc_rs, cs_rs, ckpad, pr0, pc0, cols);
      if (n + tw.step < tw.end) {
        tile_coords(n + tw.step, tiles_r, tiles_c, nr0, nc0);
        load_tile(v, src, rows, cols, ld, vec_ok, nr0, nc0, t);
      }
      __syncthreads();                        // tile staged; staged output read
#pragma unroll
      for (int p = 0; p < 4; ++p)
        row_encode_store<FMT, SR>(*reinterpret_cast<const uint4*>(&tile[(t / 8 + 32 * p) * kColLdsLd + (t % 8) * 8]), p, t,
                                  r0, c0, rows, cols, rkpad, nt, draw, seed0, seed1, rc_rs, rs_rs, own_max);
      if constexpr (SR) __syncthreads();     // draws written before the column pass reads them
      uint32_t words[8], sbytes;
      col_encode<FMT, SR>(tile, draw, t / 64, t % 64, nt, words, sbytes);
      if constexpr (SR) __syncthreads();     // draws read before the staged output overwrites them
      col_stage_write<FMT>(stage, t, words, sbytes);
      __syncthreads();                        // output staged; tile read
      pr0 = r0;
      pc0 = c0;
    }
    if (pr0 >= 0) col_stage_flush<FMT>(stage, t, cc_rs, cs_rs, ckpad, pr0, pc0, cols);
  } else {
    for (int n = tw.first; n < tw.end; n += tw.step) {
      int r0, c0;
      tile_coords(n, tiles_r, tiles_c, r0, c0);
      uint4 v[4];
      load_tile(v, src, rows, cols, ld, vec_ok, r0, c0, t);
      stage_tile(tile, v, t);
#pragma unroll
      for (int p = 0; p < 4; ++p)
        row_encode_store<FMT, SR>(v[p], p, t, r0, c0, rows, cols, rkpad, nt, draw, seed0, seed1, rc_rs, rs_rs, own_max);
      __syncthreads();                        // tile staged (and draws written)
      uint32_t words[8], sbytes;
      col_encode<FMT, SR>(tile, draw, t / 64, t % 64, nt, words, sbytes);
      __syncthreads();                        // tile read
      col_stage_write<FMT>(stage, t, words, sbytes);
      __syncthreads();                        // output staged
      col_stage_flush<FMT>(stage, t, cc_rs, cs_rs, ckpad, r0, c0, cols);
      __syncthreads();                        // staged output read
    }
  }
  if (FMT == FMT_NVFP4 && delayed) {          // this tensor's amax, for the next call
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) own_max = max(own_max, (uint32_t)__shfl_xor((int)own_max, off));
    if ((t & 63) == 0) wave_max[t >> 6] = own_max;
    __syncthreads();
    if (t == 0) {
      const uint32_t b = max(max(wave_max[0], wave_max[1]), max(wave_max[2], wave_max[3]));
      if (b != 0) {
        atomicMax(&rtr->amax_bits, b << 16);
        atomicMax(&ctr->amax_bits, b << 16);
      }
    }
  }
}

// ------------------------------------------------------------ launchers

// Resident workgroups of 256 threads of `kernel` on the current device
// (occupancy x CUs), cached per kernel and device.
static int resident_wgs(const void* kernel) {
  static std::mutex mu;
  static std::vector<std::pair<std::pair<const void*, int>, int>> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  std::lock_guard<std::mutex> lock(mu);
  for (const auto& e : cache)
    if (e.first.first == kernel && e.first.second == dev) return e.second;
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 256, 0) != hipSuccess || per_cu < 1) per_cu = 1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 8) cus = 8;
  cache.push_back({{kernel, dev}, per_cu * cus});
  return per_cu * cus;
}

// Grid of a tile-walking kernel (tile_walk): at most one resident round of
// workgroups, no more than the tiles need, and a multiple of 8 so that each
// XCD gets the same share; every workgroup of an XCD walks the same number
// of tiles, give or take one.
static int walk_grid(int64_t ntiles, const void* kernel) {
  const int64_t per_xcd = std::max<int64_t>(1, resident_wgs(kernel) / 8);
  const int64_t tiles_xcd = std::max<int64_t>(1, (ntiles + 7) / 8);
  const int64_t rounds = (tiles_xcd + per_xcd - 1) / per_xcd;
  return (int)(8 * ((tiles_xcd + rounds - 1) / rounds));
}

// One workgroup per tile, rounded up to a multiple of 8 (tile_walk).
static int one_tile_grid(int64_t ntiles) { return (int)(8 * std::max<int64_t>(1, (ntiles + 7) / 8)); }

static int grid_for(int64_t work_items, int per_block, int cap) {
  int64_t g = (work_items + per_block - 1) / per_block;
  if (g < 1) g = 1;
  if (g > cap) g = cap;
  return (int)g;
}

template <int U>
static void launch_row(const uint16_t* src, int ir, int ic, int ild, uint8_t* codes, uint8_t* scales, int ikp,
                       NvTrailer* tr, NvGiven gv, int64_t R, int fmt, hipStream_t stream) {
  const int g = grid_for(R * (ikp / 8 / U), 256, 1 << 20);
  switch (fmt) {
    case FMT_MXFP8:
      quant_row_kernel<FMT_MXFP8, U><<<g, 256, 0, stream>>>(src, ir, ic, ild, codes, scales, ikp, tr, gv);
      break;
    case FMT_MXFP4:
      quant_row_kernel<FMT_MXFP4, U><<<g, 256, 0, stream>>>(src, ir, ic, ild, codes, scales, ikp, tr, gv);
      break;
    default:
      quant_row_kernel<FMT_NVFP4, U><<<g, 256, 0, stream>>>(src, ir, ic, ild, codes, scales, ikp, tr, gv);
      break;
  }
}

hipError_t launch_quantize(const uint16_t* src, int64_t rows, int64_t cols, int64_t ld, uint8_t* codes,
                           uint8_t* scales, int fmt, int axis, const uint32_t* amax, int nslots, hipStream_t stream) {
  // The C ABI bounds every size so that element, group and byte counts fit
  // in 32 bits (outputs < 2 GiB, input < 2^40 bytes is checked per row).
  const int64_t R = axis == 0 ? rows : cols;        // stored rows
  const int64_t L = axis == 0 ? cols : rows;        // stored length (block axis)
  const int64_t kpad = round_up(L, kAlignK);
  const int bs = fmt == FMT_NVFP4 ? 16 : 32;
  const int ir = (int)rows, ic = (int)cols, ild = (int)ld, ikp = (int)kpad;
  NvTrailer* tr = nullptr;
  NvGiven gv{nullptr, 0, nullptr, 0};
  if (fmt == FMT_NVFP4) {
    const int64_t nscale = R * (kpad / bs);
    tr = reinterpret_cast<NvTrailer*>(scales + round_up(nscale, 16));
    if (amax) {
      gv = NvGiven{amax, nslots, scales + nscale, (int)(round_up(nscale, 16) - nscale)};   // the encode derives s_t
    } else {
      nv_trailer_init_kernel<<<1, 64, 0, stream>>>(scales + nscale, (int)(round_up(nscale, 16) - nscale), tr);
      const int gpr = (int)((cols + 7) / 8);
      amax_kernel<<<grid_for(rows * gpr, 256 * kAmaxUnroll, 512), 256, 0, stream>>>(src, ir, ic, ild, gpr, tr);
    }
  }
  if (axis == 0) {
    if (R * (kpad / 8) >= kRowSmallGroups)
      launch_row<kRowGroupsPerThread>(src, ir, ic, ild, codes, scales, ikp, tr, gv, R, fmt, stream);
    else
      launch_row<kRowGroupsSmall>(src, ir, ic, ild, codes, scales, ikp, tr, gv, R, fmt, stream);
  } else {
    const int64_t ntiles = ((cols + kColTileC - 1) / kColTileC) * (kpad / kColTileR);
    switch (fmt) {
      case FMT_MXFP8: {
        const int g = one_tile_grid(ntiles);
        quant_col_kernel<FMT_MXFP8><<<g, 256, 0, stream>>>(src, ir, ic, ild, codes, scales, ikp, tr, gv);
        break;
      }
      case FMT_MXFP4: {
        const int g = one_tile_grid(ntiles);
        quant_col_kernel<FMT_MXFP4><<<g, 256, 0, stream>>>(src, ir, ic, ild, codes, scales, ikp, tr, gv);
        break;
      }
      default: {
        const int g = one_tile_grid(ntiles);
        quant_col_kernel<FMT_NVFP4><<<g, 256, 0, stream>>>(src, ir, ic, ild, codes, scales, ikp, tr, gv);
        break;
      }
    }
  }
  return hipGetLastError();
}

hipError_t launch_quantize_batch(const QuantBatchItem* items, int n, int fmt, uint32_t* amax, hipStream_t stream) {
  QuantBatch batch{};
  batch.n = n;
  int64_t wg = 0;
  for (int i = 0; i < n; ++i) {
    batch.items[i] = items[i];
    batch.items[i].amax = amax ? amax + (int64_t)i * kAmaxWords : nullptr;
    batch.first_wg[i] = (int)wg;
    const int64_t threads = (int64_t)items[i].rows * (items[i].kpad / 8 / kRowGroupsPerThread);
    wg += grid_for(threads, 256, 1 << 16);
  }
  batch.first_wg[n] = (int)wg;
  if (amax) {
    zero_words_kernel<<<1, 256, 0, stream>>>(amax, n * kAmaxWords);
    if (fmt == FMT_MXFP8) quant_row_batch_kernel<FMT_MXFP8, true><<<(int)wg, 256, 0, stream>>>(batch);
    else quant_row_batch_kernel<FMT_MXFP4, true><<<(int)wg, 256, 0, stream>>>(batch);
  } else {
    if (fmt == FMT_MXFP8) quant_row_batch_kernel<FMT_MXFP8, false><<<(int)wg, 256, 0, stream>>>(batch);
    else quant_row_batch_kernel<FMT_MXFP4, false><<<(int)wg, 256, 0, stream>>>(batch);
  }
  return hipGetLastError();
}

// ------------------------------------------------------------ LayerNorm + quantize

// README section 4.3: the MXFP8 stack computes LayerNorm and quantization in
// one kernel, with the residual stream and the LayerNorm statistics in fp32.
// The output is what an LN kernel with bf16 output followed by the row
// quantizer would write: y = (x - mu) / sqrt(var + eps) * gamma + beta in
// fp32 (mu, var: the row's mean and biased variance), rounded to bf16, then
// MX-quantized along the row. One wave per row: pass 1 sums the row, pass 2
// sums the squares of the centred values (the row is read again, from the
// caches), pass 3 normalizes, rounds and quantizes 8 consecutive values per
// lane, the 4 adjacent lanes of a 32-element block combining their amax.
__device__ __forceinline__ void load8_f32(const float* row, int c, int cols, bool vec_ok, float (&v)[8]) {
  if (vec_ok && c + 8 <= cols) {
    const float4 a = *reinterpret_cast<const float4*>(row + c), b = *reinterpret_cast<const float4*>(row + c + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (c + i < cols) ? row[c + i] : 0.0f;
  }
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

template <int FMT>
__global__ __launch_bounds__(256) void ln_quant_kernel(const float* __restrict__ x, int rows, int cols, int ld,
                                                       const float* __restrict__ gamma, const float* __restrict__ beta,
                                                       float eps, uint8_t* __restrict__ codes,
                                                       uint8_t* __restrict__ scales, int kpad) {
  static_assert(FMT != FMT_NVFP4, "NVFP4 needs the tensor amax of the output first");
  const int lane = threadIdx.x & 63;
  const bool vec_ok = (ld % 4) == 0 && ((uintptr_t)x % 16) == 0;
  const bool pvec_ok = ((uintptr_t)gamma % 16) == 0 && ((uintptr_t)beta % 16) == 0;
  for (int r = blockIdx.x * 4 + (threadIdx.x >> 6); r < rows; r += gridDim.x * 4) {   // one row per wave
    const float* xr = x + (int64_t)r * ld;
    float s = 0.0f;
    for (int c0 = 0; c0 < cols; c0 += 512) {
      float v[8];
      load8_f32(xr, c0 + 8 * lane, cols, vec_ok, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) s += v[i];
    }
    const float mu = wave_sum(s) / (float)cols;
    float q = 0.0f;
    for (int c0 = 0; c0 < cols; c0 += 512) {
      const int c = c0 + 8 * lane;
      float v[8];
      load8_f32(xr, c, cols, vec_ok, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float d = (c + i < cols) ? v[i] - mu : 0.0f;
        q = fmaf(d, d, q);
      }
    }
    const float rstd = 1.0f / sqrtf(wave_sum(q) / (float)cols + eps);
    for (int c0 = 0; c0 < kpad; c0 += 512) {
      const int c = c0 + 8 * lane;
      float v[8], gm[8], bt[8];
      load8_f32(xr, c, cols, vec_ok, v);
      load8_f32(gamma, c, cols, pvec_ok, gm);
      load8_f32(beta, c, cols, pvec_ok, bt);
      float y[8];
      uint32_t m = 0;
#pragma unroll
      for (int i = 0; i < 8; i += 2) {
        // columns past cols are padding: code 0 (they do not raise the amax)
        const float y0 = (c + i < cols) ? fmaf((v[i] - mu) * rstd, gm[i], bt[i]) : 0.0f;
        const float y1 = (c + i + 1 < cols) ? fmaf((v[i + 1] - mu) * rstd, gm[i + 1], bt[i + 1]) : 0.0f;
        const uint32_t p = pack_bf16x2(y0, y1);   // RNE to bf16
        y[i] = __uint_as_float(p << 16);
        y[i + 1] = __uint_as_float(p & 0xFFFF0000u);
        m = max(m, max(p & 0x7FFFu, (p >> 16) & 0x7FFFu));
      }
      m = max(m, (uint32_t)__shfl_xor((int)m, 1));
      m = max(m, (uint32_t)__shfl_xor((int)m, 2));
      Nv4Thresholds th;
      const uint32_t sb = block_scale<FMT>(m, 0.0f, th);
      const uint64_t packed = encode8<FMT>(y, sb, th);
      if (c < kpad) {
        if (FMT == FMT_MXFP8) {
          *reinterpret_cast<uint2*>(codes + (int64_t)r * kpad + c) = make_uint2((uint32_t)packed, (uint32_t)(packed >> 32));
        } else {
          *reinterpret_cast<uint32_t*>(codes + (int64_t)r * (kpad / 2) + c / 2) = (uint32_t)packed;
        }
        if ((lane & 3) == 0) scales[(int64_t)r * (kpad / 32) + c / 32] = (uint8_t)sb;
      }
    }
  }
}

// Rows of at most 512 NCH elements (NCH <= 4): each wave keeps its row in
// registers (8 NCH values per lane), so the row is read from memory once
// instead of three times, holds gamma and beta for its columns across all
// its rows, and issues the loads of its next row before reducing the
// current one. Same arithmetic in the same order as ln_quant_kernel (the
// outputs are identical byte for byte); 1.3-1.5x faster on ViT rows.
template <int FMT, int NCH>
__global__ __launch_bounds__(256) void ln_quant_reg_kernel(const float* __restrict__ x, int rows, int cols, int ld,
                                                           const float* __restrict__ gamma,
                                                           const float* __restrict__ beta, float eps,
                                                           uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                                           int kpad) {
  static_assert(FMT != FMT_NVFP4, "NVFP4 needs the tensor amax of the output first");
  const int lane = threadIdx.x & 63;
  const bool vec_ok = (ld % 4) == 0 && ((uintptr_t)x % 16) == 0;
  const bool pvec_ok = ((uintptr_t)gamma % 16) == 0 && ((uintptr_t)beta % 16) == 0;
  float gm[NCH][8], bt[NCH][8];
#pragma unroll
  for (int k = 0; k < NCH; ++k) {
    load8_f32(gamma, 512 * k + 8 * lane, cols, pvec_ok, gm[k]);
    load8_f32(beta, 512 * k + 8 * lane, cols, pvec_ok, bt[k]);
  }
  const int step = gridDim.x * 4;
  int r = blockIdx.x * 4 + (threadIdx.x >> 6);    // one row per wave at a time
  float v[NCH][8];
  if (r < rows) {
#pragma unroll
    for (int k = 0; k < NCH; ++k) load8_f32(x + (int64_t)r * ld, 512 * k + 8 * lane, cols, vec_ok, v[k]);
  }
  for (; r < rows; r += step) {
    float vn[NCH][8];
    if (r + step < rows) {
#pragma unroll
      for (int k = 0; k < NCH; ++k) load8_f32(x + (int64_t)(r + step) * ld, 512 * k + 8 * lane, cols, vec_ok, vn[k]);
    }
    float s = 0.0f;
#pragma unroll
    for (int k = 0; k < NCH; ++k)
#pragma unroll
      for (int i = 0; i < 8; ++i) s += v[k][i];               // columns past cols were loaded as 0
    const float mu = wave_sum(s) / (float)cols;
    float q = 0.0f;
#pragma unroll
    for (int k = 0; k < NCH; ++k)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float d = (512 * k + 8 * lane + i < cols) ? v[k][i] - mu : 0.0f;
        q = fmaf(d, d, q);
      }
    const float rstd = 1.0f / sqrtf(wave_sum(q) / (float)cols + eps);
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
      const int c = 512 * k + 8 * lane;
      float y[8];
      uint32_t m = 0;
#pragma unroll
      for (int i = 0; i < 8; i += 2) {
        const float y0 = (c + i < cols) ? fmaf((v[k][i] - mu) * rstd, gm[k][i], bt[k][i]) : 0.0f;
        const float y1 = (c + i + 1 < cols) ? fmaf((v[k][i + 1] - mu) * rstd, gm[k][i + 1], bt[k][i + 1]) : 0.0f;
        const uint32_t p = pack_bf16x2(y0, y1);   // RNE to bf16
        y[i] = __uint_as_float(p << 16);
        y[i + 1] = __uint_as_float(p & 0xFFFF0000u);
        m = max(m, max(p & 0x7FFFu, (p >> 16) & 0x7FFFu));
      }
      m = max(m, (uint32_t)__shfl_xor((int)m, 1));
      m = max(m, (uint32_t)__shfl_xor((int)m, 2));
      Nv4Thresholds th;
      const uint32_t sb = block_scale<FMT>(m, 0.0f, th);
      const uint64_t packed = encode8<FMT>(y, sb, th);
      if (c < kpad) {
        if (FMT == FMT_MXFP8) {
          *reinterpret_cast<uint2*>(codes + (int64_t)r * kpad + c) = make_uint2((uint32_t)packed, (uint32_t)(packed >> 32));
        } else {
          *reinterpret_cast<uint32_t*>(codes + (int64_t)r * (kpad / 2) + c / 2) = (uint32_t)packed;
        }
        if ((lane & 3) == 0) scales[(int64_t)r * (kpad / 32) + c / 32] = (uint8_t)sb;
      }
    }
    if (r + step < rows) {
#pragma unroll
      for (int k = 0; k < NCH; ++k)
#pragma unroll
        for (int i = 0; i < 8; ++i) v[k][i] = vn[k][i];
    }
  }
}

template <int FMT>
static void launch_ln_quant(const float* x, int rows, int cols, int ld, const float* gamma, const float* beta,
                            float eps, uint8_t* codes, uint8_t* scales, int kpad, hipStream_t stream) {
  // one row per wave up to 2^18 rows (a persistent grid of 4 or 8
  // workgroups per CU, each wave walking rows, measured 5-10% slower on the
  // 11235-row ViT-L stream); beyond that the waves walk the rows with the
  // next one in flight
  const int g = grid_for(rows, 4, 1 << 16);
  if (cols <= 512)
    ln_quant_reg_kernel<FMT, 1><<<g, 256, 0, stream>>>(x, rows, cols, ld, gamma, beta, eps, codes, scales, kpad);
  else if (cols <= 1024)
    ln_quant_reg_kernel<FMT, 2><<<g, 256, 0, stream>>>(x, rows, cols, ld, gamma, beta, eps, codes, scales, kpad);
  else if (cols <= 2048)
    ln_quant_reg_kernel<FMT, 4><<<g, 256, 0, stream>>>(x, rows, cols, ld, gamma, beta, eps, codes, scales, kpad);
  else
    ln_quant_kernel<FMT><<<grid_for(rows, 4, 1 << 16), 256, 0, stream>>>(x, rows, cols, ld, gamma, beta, eps, codes,
                                                                         scales, kpad);
}

hipError_t launch_layernorm_quantize(const float* x, int64_t rows, int64_t cols, int64_t ld, const float* gamma,
                                     const float* beta, float eps, uint8_t* codes, uint8_t* scales, int fmt,
                                     hipStream_t stream) {
  const int kpad = (int)round_up(cols, kAlignK);
  if (fmt == FMT_MXFP8)
    launch_ln_quant<FMT_MXFP8>(x, (int)rows, (int)cols, (int)ld, gamma, beta, eps, codes, scales, kpad, stream);
  else
    launch_ln_quant<FMT_MXFP4>(x, (int)rows, (int)cols, (int)ld, gamma, beta, eps, codes, scales, kpad, stream);
  return hipGetLastError();
}


hipError_t launch_quantize_dual(const uint16_t* src, int64_t rows, int64_t cols, int64_t ld, uint8_t* rcodes,
                                uint8_t* rscales, uint8_t* ccodes, uint8_t* cscales, int fmt, const float* amax_prev,
                                float headroom, int sr, uint64_t seed0, uint64_t seed1, hipStream_t stream) {
  const int64_t rkpad = round_up(cols, kAlignK);    // row copy: rows x rkpad
  const int64_t ckpad = round_up(rows, kAlignK);    // column copy: cols x ckpad
  const int ir = (int)rows, ic = (int)cols, ild = (int)ld;
  NvTrailer *rtr = nullptr, *ctr = nullptr;
  const int delayed = (fmt == FMT_NVFP4 && amax_prev != nullptr) ? 1 : 0;
  if (fmt == FMT_NVFP4) {
    const int64_t rn = rows * (rkpad / 16), cn = cols * (ckpad / 16);
    rtr = reinterpret_cast<NvTrailer*>(rscales + round_up(rn, 16));
    ctr = reinterpret_cast<NvTrailer*>(cscales + round_up(cn, 16));
    nv_dual_init_kernel<<<1, 64, 0, stream>>>(rscales + rn, (int)(round_up(rn, 16) - rn), rtr, cscales + cn,
                                              (int)(round_up(cn, 16) - cn), ctr, amax_prev, headroom, delayed);
    if (!delayed) {
      const int gpr = (int)((cols + 7) / 8);
      amax_kernel<<<grid_for(rows * gpr, 256 * kAmaxUnroll, 512), 256, 0, stream>>>(src, ir, ic, ild, gpr, rtr);
    }
  }
  const int64_t ntiles = (rkpad / kColTileC) * (ckpad / kColTileR);
  const int g = one_tile_grid(ntiles);
  const int rk = (int)rkpad, ck = (int)ckpad;
  switch (fmt) {
    case FMT_MXFP8:
      quant_dual_kernel<FMT_MXFP8, false, false><<<g, 256, 0, stream>>>(src, ir, ic, ild, rcodes, rscales, rk, ccodes,
                                                                        cscales, ck, rtr, ctr, delayed, 0, 0);
      break;
    case FMT_MXFP4:
      quant_dual_kernel<FMT_MXFP4, false, false><<<g, 256, 0, stream>>>(src, ir, ic, ild, rcodes, rscales, rk, ccodes,
                                                                        cscales, ck, rtr, ctr, delayed, 0, 0);
      break;
    default:
      if (sr) {
        quant_dual_kernel<FMT_NVFP4, true, false><<<g, 256, 0, stream>>>(src, ir, ic, ild, rcodes, rscales, rk, ccodes,
                                                                         cscales, ck, rtr, ctr, delayed, seed0, seed1);
      } else {
        const int gw = walk_grid(ntiles, reinterpret_cast<const void*>(&quant_dual_kernel<FMT_NVFP4, false, true>));
        quant_dual_kernel<FMT_NVFP4, false, true><<<gw, 256, 0, stream>>>(src, ir, ic, ild, rcodes, rscales, rk, ccodes,
                                                                          cscales, ck, rtr, ctr, delayed, 0, 0);
      }
      break;
  }
  return hipGetLastError();
}

}  // namespace mx
