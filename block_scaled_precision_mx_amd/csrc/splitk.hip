// Split-K reduction for the GEMMs whose K is long and whose output is small
// (the weight-gradient GEMMs of training contract over the tokens, lightly-
// train README "DINOv3 + EoMT on RTX 5090", sections 5.4 and 5.5): the GEMM
// kernel splits K into S ranges and writes each range's fp32 partial tile to
// a workspace P[S][M][N]; this kernel forms
//   C[m, n] = ((P[0] + P[1]) + ...) + P[S-1] + bias[n]
// in fp32, in that fixed order (so the result does not depend on which
// partial finished first), and stores it as bf16 (one round to nearest even)
// or fp32. HBM-bound: S M N 4 bytes read, M N 2 or 4 written.
#include "gemm_common.h"
#include "mx_launch.h"

#include <algorithm>

namespace mx {

typedef float v4f __attribute__((ext_vector_type(4)));

// N % 8 == 0: each thread sums 8 consecutive outputs of one row (two 16-byte
// loads per partial) and writes them with one 16-byte (bf16) or two 16-byte
// (fp32) stores. The partials are read once, with non-temporal loads.
__global__ __launch_bounds__(256) void splitk_reduce8_kernel(const float* __restrict__ ws, int splits, int64_t mn,
                                                             int N, const uint16_t* __restrict__ bias,
                                                             void* __restrict__ C, int out_f32) {
  const int64_t stride = (int64_t)gridDim.x * 256 * 8;
  for (int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8; i < mn; i += stride) {
    const v4f* p = reinterpret_cast<const v4f*>(ws + i);
    v4f lo = __builtin_nontemporal_load(p), hi = __builtin_nontemporal_load(p + 1);
    for (int s = 1; s < splits; ++s) {
      const v4f* q = reinterpret_cast<const v4f*>(ws + (int64_t)s * mn + i);
      lo = lo + __builtin_nontemporal_load(q);
      hi = hi + __builtin_nontemporal_load(q + 1);
    }
    if (bias != nullptr) {
      const int n = (int)(i % N);
      uint16_t b[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) b[j] = bias[n + j];
      lo = lo + v4f{bf16_to_f32(b[0]), bf16_to_f32(b[1]), bf16_to_f32(b[2]), bf16_to_f32(b[3])};
      hi = hi + v4f{bf16_to_f32(b[4]), bf16_to_f32(b[5]), bf16_to_f32(b[6]), bf16_to_f32(b[7])};
    }
    if (out_f32) {
      v4f* c = reinterpret_cast<v4f*>(static_cast<float*>(C) + i);
      c[0] = lo;
      c[1] = hi;
    } else {
      *reinterpret_cast<uint4*>(static_cast<uint16_t*>(C) + i) =
          make_uint4(pack_bf16x2(lo.x, lo.y), pack_bf16x2(lo.z, lo.w), pack_bf16x2(hi.x, hi.y),
                     pack_bf16x2(hi.z, hi.w));
    }
  }
}

// Any N: one output per thread and iteration.
__global__ __launch_bounds__(256) void splitk_reduce1_kernel(const float* __restrict__ ws, int splits, int64_t mn,
                                                             int N, const uint16_t* __restrict__ bias,
                                                             void* __restrict__ C, int out_f32) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < mn; i += stride) {
    float v = ws[i];
    for (int s = 1; s < splits; ++s) v += ws[(int64_t)s * mn + i];
    if (bias != nullptr) v += bf16_to_f32(bias[i % N]);
    if (out_f32) static_cast<float*>(C)[i] = v;
    else static_cast<uint16_t*>(C)[i] = (uint16_t)f32_to_bf16_rne(v);
  }
}

hipError_t launch_splitk_reduce(const float* ws, int splits, int64_t M, int64_t N, const uint16_t* bias, void* C,
                                int out_f32, hipStream_t stream) {
  const int64_t mn = M * N;
  const int per_thread = (N % 8 == 0) ? 8 : 1;
  const int64_t threads = (mn + per_thread - 1) / per_thread;
  const int grid = (int)std::min<int64_t>((threads + 255) / 256, (int64_t)cu_count() * 8);
  if (per_thread == 8)
    splitk_reduce8_kernel<<<grid, 256, 0, stream>>>(ws, splits, mn, (int)N, bias, C, out_f32);
  else
    splitk_reduce1_kernel<<<grid, 256, 0, stream>>>(ws, splits, mn, (int)N, bias, C, out_f32);
  return hipGetLastError();
}

}  // namespace mx
