// MXFP8 / MXFP4 GEMM on CDNA4's scaled matrix cores:
//   C[M, N] = sum_k (a_k 2^ea)(b_k 2^eb) (+ bias[n]),  fp32 accumulate.
//
// lightly-train README "DINOv3 + EoMT on RTX 5090": section 2 (MXFP8 = E4M3
// + UE8M0 per 1x32, MXFP4 = E2M1 + UE8M0 per 1x32), section 4.3 (qkv / proj
// / fc1 / fc2 are the quantized GEMMs, with their bias in the epilogue),
// section 5.5 (TN: both operands K-major). The page's kernels target an
// RTX 5090's block-scaled mma.sync; on gfx950 the same arithmetic is one
// V_MFMA_SCALE_F32_16X16X128_F8F6F4 per 16 x 16 x 128 sub-tile, which takes
// the E8M0 scale bytes of both operands directly, so no dequantization
// happens outside the matrix core.
//
// Operand layout inside the instruction (measured on gfx950):
//   FP8:  lane l holds row l%16; bytes 0-15 are K 16g..16g+15 and bytes
//         16-31 are K 64+16g..64+16g+15, g = l/16; the scale of K-block kb
//         of row r comes from lane r + 16 kb.
//   FP4:  lane l holds row l%16, K 32g..32g+31 (low nibble first) in its
//         first four registers; its scale is its own block g.
//   Out:  lane l holds D[4g + v][l%16], v = 0..3.
// The kernel feeds the B tile as the instruction's first operand, so each
// lane ends up with 4 consecutive output columns of one output row (one
// 8-byte bf16 store).
//
// Tiling: a workgroup computes a BM x BN tile; 128 K-elements per stage
// (128 bytes of fp8 / 64 bytes of fp4 per row) are copied global -> LDS with
// 16-byte loads, double-buffered, with an XOR swizzle of the 16-byte chunks
// so that the 16 lanes reading one chunk column hit distinct banks. Scale
// bytes go straight from global memory (L2) to registers, one dword per
// lane per 16-row fragment per stage. Workgroups are renumbered so that each
// XCD (own L2) gets a contiguous range of tiles, grouped 8 tile-rows deep.
#include "mx_device.h"
#include "mx_launch.h"

namespace mx {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

template <int FMT_, int BM_, int BN_, int WAVES_M_, int WAVES_N_, int SWZ_>
struct MxCfg {
  static constexpr int FMT = FMT_, BM = BM_, BN = BN_, WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
  static constexpr int SWZ = SWZ_;
  static constexpr int KB = (FMT == FMT_MXFP8) ? 128 : 64;   // code bytes per row per stage
  static constexpr int CHUNKS = KB / 16;
  static constexpr int NT = 64 * WAVES_M * WAVES_N;
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  static constexpr int FM = WM / 16, FN = WN / 16;
  static constexpr int A_STAGE = BM * KB, B_STAGE = BN * KB;
  static constexpr int A_LOADS = BM * CHUNKS / NT;
  static constexpr int B_LOADS = BN * CHUNKS / NT;
  static constexpr int MFMA_FMT = (FMT == FMT_MXFP8) ? 0 : 4;   // E4M3 / E2M1 selector
  static_assert(A_LOADS * NT == BM * CHUNKS && B_LOADS * NT == BN * CHUNKS, "tile/threads mismatch");
  static_assert(WM % 16 == 0 && WN % 16 == 0, "wave tile");
};

__device__ __forceinline__ int swz_chunk(int r, int c, int chunks, int shift) {
  return c ^ ((r >> shift) & (chunks - 1));
}

// Tile coordinates of this workgroup: XCD-contiguous renumbering, then
// groups of 8 tile-rows walked column by column.
__device__ __forceinline__ void tile_coords(int tiles_m, int tiles_n, int& tm, int& tn) {
  const int nwg = tiles_m * tiles_n;
  const int i = blockIdx.x;
  const int q = nwg / 8, r = nwg % 8;
  const int xcd = i % 8, local = i / 8;
  const int wg = (xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q) + local;
  constexpr int GROUP = 8;
  const int group_size = GROUP * tiles_n;
  const int gid = wg / group_size;
  const int first_m = gid * GROUP;
  const int gm = min(tiles_m - first_m, GROUP);
  const int in_group = wg - gid * group_size;
  tm = first_m + in_group % gm;
  tn = in_group / gm;
}

// Epilogue store of one fragment: 4 consecutive columns n..n+3 of row m.
__device__ __forceinline__ void store4(void* C, int M, int N, int m, int n, v4f acc, float scale,
                                      const uint16_t* bias, int out_f32) {
  if (m >= M) return;
  float v[4] = {acc[0] * scale, acc[1] * scale, acc[2] * scale, acc[3] * scale};
  const bool full = ((N & 3) == 0) && (n + 3 < N);
  if (bias) {
    if (full && (reinterpret_cast<uintptr_t>(bias) & 7) == 0) {
      uint2 b = *reinterpret_cast<const uint2*>(bias + n);
      v[0] += bf16_to_f32(b.x & 0xFFFFu); v[1] += bf16_to_f32(b.x >> 16);
      v[2] += bf16_to_f32(b.y & 0xFFFFu); v[3] += bf16_to_f32(b.y >> 16);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (n + j < N) v[j] += bf16_to_f32(bias[n + j]);
    }
  }
  const int64_t off = (int64_t)m * N + n;
  if (out_f32) {
    float* c = reinterpret_cast<float*>(C) + off;
    if (full) {
      *reinterpret_cast<float4*>(c) = make_float4(v[0], v[1], v[2], v[3]);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (n + j < N) c[j] = v[j];
    }
  } else {
    uint16_t* c = reinterpret_cast<uint16_t*>(C) + off;
    if (full) {
      uint2 w;
      w.x = f32_to_bf16_rne(v[0]) | (f32_to_bf16_rne(v[1]) << 16);
      w.y = f32_to_bf16_rne(v[2]) | (f32_to_bf16_rne(v[3]) << 16);
      *reinterpret_cast<uint2*>(c) = w;
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (n + j < N) c[j] = (uint16_t)f32_to_bf16_rne(v[j]);
    }
  }
}

// One 16-byte-per-lane copy global -> LDS: lane l's 16 bytes land at
// lds_base + 16 l (lds_base is wave-uniform).
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rs, uint8_t* lds_base, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds_base, 16, voff, soff, 0, 0);
}

template <class Cfg>
__global__ __launch_bounds__(Cfg::NT) void gemm_mx_kernel(const uint8_t* __restrict__ A,
                                                          const uint8_t* __restrict__ As,
                                                          const uint8_t* __restrict__ B,
                                                          const uint8_t* __restrict__ Bs, void* __restrict__ C,
                                                          int M, int N, int kpad,
                                                          const uint16_t* __restrict__ bias, int out_f32,
                                                          int tiles_m, int tiles_n) {
  constexpr int KB = Cfg::KB, CH = Cfg::CHUNKS, NW = Cfg::NT / 64;
  constexpr int BM = Cfg::BM, BN = Cfg::BN, WM = Cfg::WM, WN = Cfg::WN, FM = Cfg::FM, FN = Cfg::FN;
  constexpr int A_DMA = Cfg::A_STAGE / (1024 * NW);    // 1-KB wave copies per stage
  constexpr int B_DMA = Cfg::B_STAGE / (1024 * NW);
  static_assert(A_DMA * 1024 * NW == Cfg::A_STAGE && B_DMA * 1024 * NW == Cfg::B_STAGE, "dma split");
  __shared__ __align__(16) uint8_t lds[2 * (Cfg::A_STAGE + Cfg::B_STAGE)];

  int tm, tn;
  tile_coords(tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave / Cfg::WAVES_N, wn = wave % Cfg::WAVES_N;
  const int row_bytes = (FMT_MXFP8 == Cfg::FMT) ? kpad : kpad / 2;
  const int srow = kpad / 32;               // scale bytes per row
  const int nk = kpad / 128;
  const int g = lane >> 4, r16 = lane & 15;

  // Buffer resources: reads past the last row return zeros (tail tiles).
  const __amdgpu_buffer_rsrc_t a_rs = __builtin_amdgcn_make_buffer_rsrc((void*)A, 0, M * row_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t b_rs = __builtin_amdgcn_make_buffer_rsrc((void*)B, 0, N * row_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t as_rs = __builtin_amdgcn_make_buffer_rsrc((void*)As, 0, M * srow, 0x00020000);
  const __amdgpu_buffer_rsrc_t bs_rs = __builtin_amdgcn_make_buffer_rsrc((void*)Bs, 0, N * srow, 0x00020000);

  // Direct global -> LDS copies: copy j of this wave fills LDS chunks
  // P = (j * NW + wave) * 64 + lane, i.e. row P / CH, swizzled position
  // P % CH, which holds global chunk (P % CH) ^ swizzle(row).
  int a_voff[A_DMA], b_voff[B_DMA];
#pragma unroll
  for (int j = 0; j < A_DMA; ++j) {
    const int P = (j * NW + wave) * 64 + lane, r = P / CH, p = P % CH;
    a_voff[j] = (m0 + r) * row_bytes + swz_chunk(r, p, CH, Cfg::SWZ) * 16;
  }
#pragma unroll
  for (int j = 0; j < B_DMA; ++j) {
    const int P = (j * NW + wave) * 64 + lane, r = P / CH, p = P % CH;
    b_voff[j] = (n0 + r) * row_bytes + swz_chunk(r, p, CH, Cfg::SWZ) * 16;
  }
  // scale dwords (4 K-blocks per stage): one per fragment and lane
  const int sa_voff = (m0 + wm * WM + r16) * srow;
  const int sb_voff = (n0 + wn * WN + r16) * srow;
  const int sshift = 8 * g;
  // LDS read offsets of this lane's fragment 0 (chunk g and, for fp8, 4+g);
  // fragment f adds 16 f rows, which keeps the swizzle (it uses row bits < 4).
  const int ra = wm * WM + r16, rb = wn * WN + r16;
  const int a_off0 = ra * KB + swz_chunk(ra, g, CH, Cfg::SWZ) * 16;
  const int a_off1 = ra * KB + swz_chunk(ra, (4 + g) & (CH - 1), CH, Cfg::SWZ) * 16;
  const int b_off0 = rb * KB + swz_chunk(rb, g, CH, Cfg::SWZ) * 16;
  const int b_off1 = rb * KB + swz_chunk(rb, (4 + g) & (CH - 1), CH, Cfg::SWZ) * 16;

  auto issue_stage = [&](int ks, int buf) {
    uint8_t* a_dst = lds + buf * Cfg::A_STAGE;
    uint8_t* b_dst = lds + 2 * Cfg::A_STAGE + buf * Cfg::B_STAGE;
#pragma unroll
    for (int j = 0; j < A_DMA; ++j)
      dma16(a_rs, a_dst + (j * NW + wave) * 1024, a_voff[j], ks * KB);
#pragma unroll
    for (int j = 0; j < B_DMA; ++j)
      dma16(b_rs, b_dst + (j * NW + wave) * 1024, b_voff[j], ks * KB);
  };

  v4f acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  uint32_t sa_cur[FM], sb_cur[FN], sa_nxt[FM], sb_nxt[FN];
  issue_stage(0, 0);
#pragma unroll
  for (int f = 0; f < FM; ++f) sa_cur[f] = __builtin_amdgcn_raw_buffer_load_b32(as_rs, sa_voff + 16 * f * srow, 0, 0) >> sshift;
#pragma unroll
  for (int f = 0; f < FN; ++f) sb_cur[f] = __builtin_amdgcn_raw_buffer_load_b32(bs_rs, sb_voff + 16 * f * srow, 0, 0) >> sshift;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  for (int ks = 0; ks < nk; ++ks) {
    const int cur = ks & 1;
    const bool more = ks + 1 < nk;
    if (more) {
      issue_stage(ks + 1, cur ^ 1);
#pragma unroll
      for (int f = 0; f < FM; ++f)
        sa_nxt[f] = __builtin_amdgcn_raw_buffer_load_b32(as_rs, sa_voff + 16 * f * srow, 4 * (ks + 1), 0) >> sshift;
#pragma unroll
      for (int f = 0; f < FN; ++f)
        sb_nxt[f] = __builtin_amdgcn_raw_buffer_load_b32(bs_rs, sb_voff + 16 * f * srow, 4 * (ks + 1), 0) >> sshift;
    }
    const uint8_t* a_buf = lds + cur * Cfg::A_STAGE;
    const uint8_t* b_buf = lds + 2 * Cfg::A_STAGE + cur * Cfg::B_STAGE;
    v8i bfrag[FN];
#pragma unroll
    for (int f = 0; f < FN; ++f) {
      uint4 lo = *reinterpret_cast<const uint4*>(b_buf + b_off0 + 16 * f * KB);
      uint4 hi = make_uint4(0u, 0u, 0u, 0u);
      if (Cfg::FMT == FMT_MXFP8) hi = *reinterpret_cast<const uint4*>(b_buf + b_off1 + 16 * f * KB);
      bfrag[f] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      uint4 lo = *reinterpret_cast<const uint4*>(a_buf + a_off0 + 16 * fm * KB);
      uint4 hi = make_uint4(0u, 0u, 0u, 0u);
      if (Cfg::FMT == FMT_MXFP8) hi = *reinterpret_cast<const uint4*>(a_buf + a_off1 + 16 * fm * KB);
      const v8i afrag = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        acc[fm][fn] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            bfrag[fn], afrag, acc[fm][fn], Cfg::MFMA_FMT, Cfg::MFMA_FMT, 0, (int)sb_cur[fn], 0, (int)sa_cur[fm]);
      }
    }
    // the copies into the other buffer (and the next scales) must land
    // before any wave reads them after the barrier
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (more) {
#pragma unroll
      for (int f = 0; f < FM; ++f) sa_cur[f] = sa_nxt[f];
#pragma unroll
      for (int f = 0; f < FN; ++f) sb_cur[f] = sb_nxt[f];
    }
  }

  // epilogue: lane holds C[m][n..n+3]
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
    const int m = m0 + wm * WM + 16 * fm + r16;
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
      const int n = n0 + wn * WN + 16 * fn + 4 * g;
      store4(C, M, N, m, n, acc[fm][fn], 1.0f, bias, out_f32);
    }
  }
}

template <class Cfg>
static hipError_t run_mx(const uint8_t* A, const uint8_t* As, const uint8_t* B, const uint8_t* Bs, void* C,
                         int64_t M, int64_t N, int64_t K, const uint16_t* bias, int out_f32, hipStream_t stream) {
  const int64_t kpad = round_up(K, kAlignK);
  const int tiles_m = (int)((M + Cfg::BM - 1) / Cfg::BM);
  const int tiles_n = (int)((N + Cfg::BN - 1) / Cfg::BN);
  gemm_mx_kernel<Cfg><<<tiles_m * tiles_n, Cfg::NT, 0, stream>>>(A, As, B, Bs, C, (int)M, (int)N, (int)kpad, bias,
                                                                  out_f32, tiles_m, tiles_n);
  return hipGetLastError();
}

hipError_t launch_gemm_mx(const uint8_t* A, const uint8_t* As, const uint8_t* B, const uint8_t* Bs, void* C,
                          int64_t M, int64_t N, int64_t K, int fmt, const uint16_t* bias, int out_f32,
                          hipStream_t stream) {
  // Large problems: 256 x 256 tiles, 8 waves of 128 x 64. Small ones:
  // 128 x 128 tiles, 4 waves of 64 x 64, so more workgroups fill the chip.
  const int64_t big_tiles = ((M + 255) / 256) * ((N + 255) / 256);
  const bool big = big_tiles >= 256;
  if (fmt == FMT_MXFP8) {
    if (big) return run_mx<MxCfg<FMT_MXFP8, 256, 256, 2, 2, 0>>(A, As, B, Bs, C, M, N, K, bias, out_f32, stream);
    return run_mx<MxCfg<FMT_MXFP8, 128, 128, 2, 2, 0>>(A, As, B, Bs, C, M, N, K, bias, out_f32, stream);
  }
  if (big) return run_mx<MxCfg<FMT_MXFP4, 256, 256, 2, 2, 1>>(A, As, B, Bs, C, M, N, K, bias, out_f32, stream);
  return run_mx<MxCfg<FMT_MXFP4, 128, 128, 2, 2, 1>>(A, As, B, Bs, C, M, N, K, bias, out_f32, stream);
}

}  // namespace mx
