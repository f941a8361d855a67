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
// so the kernels are shaped for coalescing, not arithmetic:
//  * row: each lane reads 8 consecutive bf16 (one 16-byte load), the 4 lanes
//    of a 32-element MX block (2 lanes of a 16-element NVFP4 block) combine
//    their amax with cross-lane shuffles, and each lane stores its 8 codes
//    (8 bytes fp8 / 4 bytes fp4) next to its neighbours'.
//  * col: a workgroup stages a 128 x 64 bf16 tile through LDS with 16-byte
//    row loads; each wave then owns 32 consecutive rows (one MX block, two
//    NVFP4 blocks) of 64 columns and each lane emits its column's 32 codes
//    as one contiguous 32- or 16-byte store of the transposed output.
//  * NVFP4 first reduces the tensor amax (bf16 magnitude bits, which order
//    like the values) into the scale trailer with one atomic max per
//    workgroup; the quantizer derives s_t from it.
#include "mx_device.h"
#include "mx_launch.h"

namespace mx {

struct NvTrailer {
  float s_t;
  uint32_t amax_bits;   // fp32 bits of the tensor amax
  uint32_t pad[2];
};

// ------------------------------------------------------------ amax (NVFP4)

// Zeroes the trailer and the (< 16) padding bytes between the last scale
// byte and the trailer, so the whole scale buffer is defined.
__global__ void nv_trailer_init_kernel(uint8_t* gap, int gap_bytes, NvTrailer* tr) {
  if (threadIdx.x < gap_bytes) gap[threadIdx.x] = 0;
  if (threadIdx.x == 0) {
    tr->s_t = 0.0f;
    tr->amax_bits = 0u;
    tr->pad[0] = 0u;
    tr->pad[1] = 0u;
  }
}

__global__ __launch_bounds__(256) void amax_kernel(const uint16_t* __restrict__ src, int64_t rows,
                                                   int64_t cols, int64_t ld, NvTrailer* tr) {
  const int64_t gpr = (cols + 7) / 8;          // 8-element groups per row
  const int64_t total = rows * gpr;
  const bool vec_ok = (ld % 8) == 0 && ((uintptr_t)src % 16) == 0;
  uint32_t m = 0;
  for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < total;
       g += (int64_t)gridDim.x * blockDim.x) {
    int64_t r = g / gpr;
    int64_t c = (g - r * gpr) * 8;
    const uint16_t* p = src + r * ld + c;
    if (vec_ok && c + 8 <= cols) {
      uint4 v = *reinterpret_cast<const uint4*>(p);
      uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        m = max(m, w[i] & 0x7FFFu);
        m = max(m, (w[i] >> 16) & 0x7FFFu);
      }
    } else {
      for (int i = 0; i < 8 && c + i < cols; ++i) m = max(m, (uint32_t)p[i] & 0x7FFFu);
    }
  }
  // wave reduction, then one atomic per wave
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
  if ((threadIdx.x & 63) == 0 && m != 0) atomicMax(&tr->amax_bits, m << 16);
}

// ------------------------------------------------------------ row quantizer

// Encode the 8 values of one lane. `mul` is 2^-e (MX); `th` the NVFP4
// thresholds. Returns packed codes in the low 64 (fp8) or 32 (fp4) bits.
template <int FMT>
__device__ __forceinline__ uint64_t encode8(const float (&x)[8], float mul, const Nv4Thresholds& th) {
  uint64_t out = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t c;
    if (FMT == FMT_MXFP8) {
      c = e4m3_encode(x[i] * mul);
      out |= (uint64_t)c << (8 * i);
    } else if (FMT == FMT_MXFP4) {
      c = e2m1_encode(x[i] * mul);
      out |= (uint64_t)c << (4 * i);
    } else {
      c = nvfp4_encode(x[i], th);
      out |= (uint64_t)c << (4 * i);
    }
  }
  return out;
}

template <int FMT>
__global__ __launch_bounds__(256) void quant_row_kernel(const uint16_t* __restrict__ src, int64_t rows,
                                                        int64_t cols, int64_t ld,
                                                        uint8_t* __restrict__ codes,
                                                        uint8_t* __restrict__ scales, int64_t kpad,
                                                        NvTrailer* tr) {
  constexpr int BS = (FMT == FMT_NVFP4) ? 16 : 32;
  constexpr int LANES_PER_BLOCK = BS / 8;
  const int64_t gpr = kpad / 8;                 // groups per stored row (multiple of 16)
  const int64_t total = rows * gpr;
  const bool vec_ok = (ld % 8) == 0 && ((uintptr_t)src % 16) == 0;
  float s_t = 0.0f;
  if (FMT == FMT_NVFP4) {
    s_t = nvfp4_tensor_scale(tr->amax_bits);
    if (blockIdx.x == 0 && threadIdx.x == 0) tr->s_t = s_t;
  }
  for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < total;
       g += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = g / gpr;
    const int64_t c = (g - r * gpr) * 8;
    const uint16_t* p = src + r * ld + c;
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    if (vec_ok && c + 8 <= cols) {
      uint4 v = *reinterpret_cast<const uint4*>(p);
      w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (c + i < cols) w[i / 2] |= (uint32_t)p[i] << (16 * (i % 2));
    }
    float x[8];
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t b = (w[i / 2] >> (16 * (i % 2))) & 0xFFFFu;
      x[i] = bf16_to_f32(b);
      m = max(m, b & 0x7FFFu);
    }
    // block amax across the lanes of this block (lane groups are aligned)
#pragma unroll
    for (int off = 1; off < LANES_PER_BLOCK; off <<= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
    uint32_t scale_byte;
    float mul = 1.0f;
    Nv4Thresholds th;
    if (FMT == FMT_NVFP4) {
      double q = (s_t == 0.0f) ? 0.0 : (double)bf16_to_f32(m) / (6.0 * (double)s_t);
      scale_byte = e4m3_encode_pos_f64(q);
      th = nvfp4_thresholds(e4m3_value(scale_byte) * (double)s_t);
    } else {
      int e = mx_shared_exp(m, FMT == FMT_MXFP8 ? 8 : 2);
      scale_byte = (uint32_t)(e + 127);
      mul = pow2_neg(e);
    }
    uint64_t packed = encode8<FMT>(x, mul, th);
    if (FMT == FMT_MXFP8) {
      *reinterpret_cast<uint2*>(codes + r * kpad + c) = make_uint2((uint32_t)packed, (uint32_t)(packed >> 32));
    } else {
      *reinterpret_cast<uint32_t*>(codes + r * (kpad / 2) + c / 2) = (uint32_t)packed;
    }
    if ((threadIdx.x % LANES_PER_BLOCK) == 0) scales[r * (kpad / BS) + c / BS] = (uint8_t)scale_byte;
  }
}

// ------------------------------------------------------------ col quantizer

constexpr int kColTileR = 128;   // rows of X (the block axis) per tile
constexpr int kColTileC = 64;    // columns of X per tile
constexpr int kColLdsLd = kColTileC + 8;   // padded LDS row (elements), keeps 16-B alignment

// X [rows, cols] -> codes of X^T: [cols, kpad] with kpad = round_up(rows, 128).
template <int FMT>
__global__ __launch_bounds__(256) void quant_col_kernel(const uint16_t* __restrict__ src, int64_t rows,
                                                        int64_t cols, int64_t ld,
                                                        uint8_t* __restrict__ codes,
                                                        uint8_t* __restrict__ scales, int64_t kpad,
                                                        NvTrailer* tr) {
  constexpr int BS = (FMT == FMT_NVFP4) ? 16 : 32;
  __shared__ __align__(16) uint16_t tile[kColTileR * kColLdsLd];
  const int64_t tiles_c = (cols + kColTileC - 1) / kColTileC;
  const int64_t tiles_r = kpad / kColTileR;
  const int64_t ntiles = tiles_c * tiles_r;
  const bool vec_ok = (ld % 8) == 0 && ((uintptr_t)src % 16) == 0;
  const int t = threadIdx.x;
  float s_t = 0.0f;
  if (FMT == FMT_NVFP4) {
    s_t = nvfp4_tensor_scale(tr->amax_bits);
    if (blockIdx.x == 0 && t == 0) tr->s_t = s_t;
  }
  for (int64_t tile_id = blockIdx.x; tile_id < ntiles; tile_id += gridDim.x) {
    const int64_t tr_ = tile_id / tiles_c;
    const int64_t tc = tile_id - tr_ * tiles_c;
    const int64_t r0 = tr_ * kColTileR, c0 = tc * kColTileC;
    // stage: 128 rows x 64 cols; thread t loads 8 columns of rows t/8 + 32 p
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int lr = t / 8 + 32 * p;
      const int lc = (t % 8) * 8;
      const int64_t r = r0 + lr, c = c0 + lc;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (r < rows) {
        const uint16_t* q = src + r * ld + c;
        if (vec_ok && c + 8 <= cols) {
          v = *reinterpret_cast<const uint4*>(q);
        } else {
          uint32_t w[4] = {0u, 0u, 0u, 0u};
          for (int i = 0; i < 8; ++i)
            if (c + i < cols) w[i / 2] |= (uint32_t)q[i] << (16 * (i % 2));
          v = make_uint4(w[0], w[1], w[2], w[3]);
        }
      }
      *reinterpret_cast<uint4*>(&tile[lr * kColLdsLd + lc]) = v;
    }
    __syncthreads();
    // wave w owns tile rows 32w .. 32w+31; lane j owns column j
    const int w = t / 64, j = t % 64;
    const int64_t oc = c0 + j;                // output row (a column of X)
    float x[32];
    uint32_t m[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      uint32_t b = tile[(32 * w + i) * kColLdsLd + j];
      x[i] = bf16_to_f32(b);
      m[i / 16] = max(m[i / 16], b & 0x7FFFu);
    }
    if (oc < cols) {
      const int64_t orow = r0 + 32 * w;       // first element index along the block axis
      if (FMT == FMT_NVFP4) {
        uint32_t packed[4];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          double q = (s_t == 0.0f) ? 0.0 : (double)bf16_to_f32(m[h]) / (6.0 * (double)s_t);
          uint32_t sb = e4m3_encode_pos_f64(q);
          Nv4Thresholds th = nvfp4_thresholds(e4m3_value(sb) * (double)s_t);
#pragma unroll
          for (int q2 = 0; q2 < 2; ++q2) {
            uint32_t word = 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) word |= nvfp4_encode(x[16 * h + 8 * q2 + i], th) << (4 * i);
            packed[2 * h + q2] = word;
          }
          scales[oc * (kpad / 16) + orow / 16 + h] = (uint8_t)sb;
        }
        *reinterpret_cast<uint4*>(codes + oc * (kpad / 2) + orow / 2) =
            make_uint4(packed[0], packed[1], packed[2], packed[3]);
      } else {
        const uint32_t mm = max(m[0], m[1]);
        const int e = mx_shared_exp(mm, FMT == FMT_MXFP8 ? 8 : 2);
        const float mul = pow2_neg(e);
        if (FMT == FMT_MXFP8) {
          uint32_t words[8];
#pragma unroll
          for (int q2 = 0; q2 < 8; ++q2) {
            uint32_t word = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) word |= e4m3_encode(x[4 * q2 + i] * mul) << (8 * i);
            words[q2] = word;
          }
          uint4* dst = reinterpret_cast<uint4*>(codes + oc * kpad + orow);
          dst[0] = make_uint4(words[0], words[1], words[2], words[3]);
          dst[1] = make_uint4(words[4], words[5], words[6], words[7]);
        } else {
          uint32_t words[4];
#pragma unroll
          for (int q2 = 0; q2 < 4; ++q2) {
            uint32_t word = 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) word |= e2m1_encode(x[8 * q2 + i] * mul) << (4 * i);
            words[q2] = word;
          }
          *reinterpret_cast<uint4*>(codes + oc * (kpad / 2) + orow / 2) =
              make_uint4(words[0], words[1], words[2], words[3]);
        }
        scales[oc * (kpad / 32) + orow / 32] = (uint8_t)(e + 127);
      }
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------ launchers

static int grid_for(int64_t work_items, int per_block) {
  int64_t g = (work_items + per_block - 1) / per_block;
  if (g < 1) g = 1;
  if (g > 65536) g = 65536;
  return (int)g;
}

hipError_t launch_quantize(const uint16_t* src, int64_t rows, int64_t cols, int64_t ld, uint8_t* codes,
                           uint8_t* scales, int fmt, int axis, hipStream_t stream) {
  const int64_t R = axis == 0 ? rows : cols;        // stored rows
  const int64_t L = axis == 0 ? cols : rows;        // stored length (block axis)
  const int64_t kpad = round_up(L, kAlignK);
  const int bs = fmt == FMT_NVFP4 ? 16 : 32;
  NvTrailer* tr = nullptr;
  if (fmt == FMT_NVFP4) {
    const int64_t nscale = R * (kpad / bs);
    tr = reinterpret_cast<NvTrailer*>(scales + round_up(nscale, 16));
    nv_trailer_init_kernel<<<1, 64, 0, stream>>>(scales + nscale, (int)(round_up(nscale, 16) - nscale), tr);
    const int64_t groups = rows * ((cols + 7) / 8);
    int g = grid_for(groups, 256 * 8);
    if (g > 2048) g = 2048;
    amax_kernel<<<g, 256, 0, stream>>>(src, rows, cols, ld, tr);
  }
  if (axis == 0) {
    const int64_t groups = R * (kpad / 8);
    const int g = grid_for(groups, 256 * 2);
    switch (fmt) {
      case FMT_MXFP8: quant_row_kernel<FMT_MXFP8><<<g, 256, 0, stream>>>(src, rows, cols, ld, codes, scales, kpad, tr); break;
      case FMT_MXFP4: quant_row_kernel<FMT_MXFP4><<<g, 256, 0, stream>>>(src, rows, cols, ld, codes, scales, kpad, tr); break;
      default:        quant_row_kernel<FMT_NVFP4><<<g, 256, 0, stream>>>(src, rows, cols, ld, codes, scales, kpad, tr); break;
    }
  } else {
    const int64_t ntiles = ((cols + kColTileC - 1) / kColTileC) * (kpad / kColTileR);
    const int g = grid_for(ntiles, 1);
    switch (fmt) {
      case FMT_MXFP8: quant_col_kernel<FMT_MXFP8><<<g, 256, 0, stream>>>(src, rows, cols, ld, codes, scales, kpad, tr); break;
      case FMT_MXFP4: quant_col_kernel<FMT_MXFP4><<<g, 256, 0, stream>>>(src, rows, cols, ld, codes, scales, kpad, tr); break;
      default:        quant_col_kernel<FMT_NVFP4><<<g, 256, 0, stream>>>(src, rows, cols, ld, codes, scales, kpad, tr); break;
    }
  }
  return hipGetLastError();
}

}  // namespace mx
