// MXFP8 / MXFP4 GEMM on CDNA4's scaled matrix cores:
//   C[M, N] = sum_k (a_k 2^ea)(b_k 2^eb) (+ bias[n]),  fp32 accumulate.
//
// lightly-train README "DINOv3 + EoMT on RTX 5090": section 2 (MXFP8 = E4M3
// + UE8M0 per 1x32, MXFP4 = E2M1 + UE8M0 per 1x32), section 4.3 (qkv / proj
// / fc1 / fc2 are the quantized GEMMs, with their bias in the epilogue),
// section 5.5 (TN: both operands K-major). The page's kernels target an
// RTX 5090's block-scaled mma.sync; on gfx950 the same arithmetic is one
// V_MFMA_SCALE_F32_32X32X64_F8F6F4 per 32 x 32 x 64 sub-tile, which takes the
// E8M0 scale bytes of both operands directly, so no dequantization happens
// outside the matrix core. (The 16x16x128 form runs FP4 at only the FP8 rate
// on this chip; the 32x32x64 form runs FP4 at twice the FP8 rate.)
//
// Operand layout inside the instruction (measured on gfx950), lane l,
// r = l % 32, g = l / 32:
//   FP8:  row r; bytes 0-15 are K 16g..16g+15, bytes 16-31 are K 32+16g..+15;
//         the scale of K-block kb of row r comes from lane r + 32 kb.
//   FP4:  row r, K 32g..32g+31 (low nibble first) in the first 4 registers;
//         its scale is its own block g.
//   Out:  register 4q + v holds D[8q + 4g + v][r].
// The B tile is fed as the instruction's first operand, so each lane ends up
// with runs of 4 consecutive output columns of one output row.
//
// Pipeline: a K-stage is 64 bytes of codes per row (64 fp8 / 128 fp4
// elements) plus the aligned scale dword holding that stage's blocks (fp8:
// the 4 blocks of stages 2j, 2j+1; fp4: the 4 blocks of the stage). NST
// stages are in flight: each wave copies its share of a stage global -> LDS
// with buffer_load ... lds (16 bytes of codes or one scale dword per lane,
// rows past the tensor read as zero), waits with vmcnt for its own copies of
// the stage about to be used, then a workgroup barrier makes every wave's
// copies visible. The copies are issued from inline assembly so that the
// compiler does not conservatively wait for all of them before each LDS
// read; the kernel does its own counting. Code rows are XOR-swizzled in
// 16-byte chunks so the 32 lanes reading one chunk column hit distinct
// banks. Tiles are renumbered so each XCD (own L2) gets a contiguous range,
// walked in groups of 8 tile-rows.
#include "mx_device.h"
#include "mx_launch.h"

namespace mx {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));

template <int FMT_, int BM_, int BN_, int WAVES_M_, int WAVES_N_, int NST_>
struct MxCfg {
  static constexpr int FMT = FMT_, BM = BM_, BN = BN_, WAVES_M = WAVES_M_, WAVES_N = WAVES_N_, NST = NST_;
  static constexpr int NT = 64 * WAVES_M * WAVES_N, NW = NT / 64;
  static constexpr int RB = 64;                               // code bytes per row per stage
  static constexpr int KS = (FMT == FMT_MXFP8) ? 64 : 128;    // K elements per stage
  static constexpr int SB = 4;                                // scale bytes per row in a stage slot
                                                              // (fp8: blocks of 2 stages; fp4: of 1 stage)
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  static constexpr int FM = WM / 32, FN = WN / 32;
  static constexpr int CODE_BYTES = (BM + BN) * RB;            // per stage
  static constexpr int SCALE_BYTES = (BM + BN) * SB;
  static constexpr int STAGE = CODE_BYTES + SCALE_BYTES;
  static constexpr int LDS = NST * STAGE;
  static constexpr int CODE_DMA = CODE_BYTES / 1024 / NW;     // 1-KB copies per wave per stage
  static constexpr int SCALE_DMA = (BM + BN) / 64 / NW;       // 64-row scale copies per wave per stage
  static constexpr int OPS = CODE_DMA + SCALE_DMA;            // vector memory ops per wave per stage
  static constexpr int MFMA_FMT = (FMT == FMT_MXFP8) ? 0 : 4;  // E4M3 / E2M1 operand selector
  static_assert(CODE_DMA * 1024 * NW == CODE_BYTES, "code copies must split evenly over waves");
  static_assert(SCALE_DMA * 64 * NW == BM + BN && SCALE_DMA >= 1, "scale copies must split evenly");
  static_assert((BM * RB) % 1024 == 0 && BM % 64 == 0 && BN % 64 == 0, "tile");
  static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile");
  static_assert(LDS <= 160 * 1024, "LDS");
};

// Row r keeps 16-byte chunk c at position c ^ ((r >> 1) & 3).
__device__ __forceinline__ int swz4(int r, int c) { return c ^ ((r >> 1) & 3); }

__device__ __forceinline__ v4u buffer_rsrc(const void* p, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  v4u r;
  r.x = __builtin_amdgcn_readfirstlane((uint32_t)a);
  r.y = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  r.z = __builtin_amdgcn_readfirstlane(bytes);
  r.w = 0x00020000u;   // raw buffer, 32-bit data format: out-of-range reads return 0
  return r;
}

// One wave-wide copy global -> LDS: lane l's SIZE (16 or 4) bytes at `voff`
// land at lds_addr + SIZE * l. M0 is saved and restored around the copy.
template <int SIZE>
__device__ __forceinline__ void dma(v4u rs, uint32_t lds_addr, uint32_t voff, uint32_t soff) {
  uint32_t saved;
  if (SIZE == 16)
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\tbuffer_load_dwordx4 %2, %3, %4 offen lds\n\ts_mov_b32 m0, %0"
                 : "=&s"(saved) : "s"(lds_addr), "v"(voff), "s"(rs), "s"(soff) : "memory");
  else
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\tbuffer_load_dword %2, %3, %4 offen lds\n\ts_mov_b32 m0, %0"
                 : "=&s"(saved) : "s"(lds_addr), "v"(voff), "s"(rs), "s"(soff) : "memory");
}

// Wait until at most N of this wave's vector memory operations are pending.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
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

template <class Cfg>
__global__ __launch_bounds__(Cfg::NT) void gemm_mx_kernel(const uint8_t* __restrict__ A,
                                                          const uint8_t* __restrict__ As,
                                                          const uint8_t* __restrict__ B,
                                                          const uint8_t* __restrict__ Bs, void* __restrict__ C,
                                                          int M, int N, int kpad,
                                                          const uint16_t* __restrict__ bias, int out_f32,
                                                          int tiles_m, int tiles_n) {
  constexpr int BM = Cfg::BM, WM = Cfg::WM, WN = Cfg::WN, FM = Cfg::FM, FN = Cfg::FN;
  constexpr int RB = Cfg::RB, SB = Cfg::SB, NW = Cfg::NW, NST = Cfg::NST;
  __shared__ __align__(16) uint8_t lds[Cfg::LDS];

  int tm, tn;
  tile_coords(tiles_m, tiles_n, tm, tn);
  const int m0 = tm * Cfg::BM, n0 = tn * Cfg::BN;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / Cfg::WAVES_N, wn = wave % Cfg::WAVES_N;
  const int row_bytes = (Cfg::FMT == FMT_MXFP8) ? kpad : kpad / 2;
  const int srow = kpad / 32;               // scale bytes per row
  const int nk = kpad / Cfg::KS;            // stages
  const int g = lane >> 5, r32 = lane & 31;

  const v4u a_rs = buffer_rsrc(A, (uint32_t)(M * row_bytes));
  const v4u b_rs = buffer_rsrc(B, (uint32_t)(N * row_bytes));
  const v4u as_rs = buffer_rsrc(As, (uint32_t)(M * srow));
  const v4u bs_rs = buffer_rsrc(Bs, (uint32_t)(N * srow));
  const uint32_t lds_base = (uint32_t)reinterpret_cast<uintptr_t>(lds);

  // Copy j of this wave fills the stage's 1-KB code block J = j * NW + wave:
  // 16-byte chunk P = 64 J + lane, A rows first (4 chunks per row), then B.
  uint32_t code_voff[Cfg::CODE_DMA];
  bool code_is_a[Cfg::CODE_DMA];
#pragma unroll
  for (int j = 0; j < Cfg::CODE_DMA; ++j) {
    const int J = j * NW + wave;
    const int P = J * 64 + lane;
    const bool isa = P < BM * 4;
    const int Pr = isa ? P : P - BM * 4;
    const int r = Pr >> 2, p = Pr & 3;
    code_is_a[j] = J * 64 < BM * 4;       // uniform per copy
    code_voff[j] = (uint32_t)(((isa ? m0 : n0) + r) * row_bytes + swz4(r, p) * 16);
  }
  // Scale copy j of this wave covers rows 64 J' .. 64 J' + 63 of [A rows, B rows].
  uint32_t scale_voff[Cfg::SCALE_DMA];
  bool scale_is_a[Cfg::SCALE_DMA];
#pragma unroll
  for (int j = 0; j < Cfg::SCALE_DMA; ++j) {
    const int J = j * NW + wave;
    const int row = J * 64 + lane;
    scale_is_a[j] = J * 64 < BM;
    const int r = scale_is_a[j] ? row : row - BM;
    scale_voff[j] = (uint32_t)(((scale_is_a[j] ? m0 : n0) + r) * srow);
  }

  auto issue_stage = [&](int ks) {
    const uint32_t st = lds_base + (uint32_t)((ks % NST) * Cfg::STAGE);
#pragma unroll
    for (int j = 0; j < Cfg::CODE_DMA; ++j) {
      const uint32_t dst = st + (uint32_t)((j * NW + wave) * 1024);
      dma<16>(code_is_a[j] ? a_rs : b_rs, dst, code_voff[j], (uint32_t)(ks * RB));
    }
#pragma unroll
    for (int j = 0; j < Cfg::SCALE_DMA; ++j) {
      const uint32_t dst = st + Cfg::CODE_BYTES + (uint32_t)((j * NW + wave) * 64 * SB);
      const uint32_t sdw = (uint32_t)((Cfg::FMT == FMT_MXFP8 ? (ks >> 1) : ks) * 4);
      dma<4>(scale_is_a[j] ? as_rs : bs_rs, dst, scale_voff[j], sdw);
    }
  };

  // LDS read offsets (within a stage) of this lane's fragments.
  const int ra = wm * WM + r32, rb = wn * WN + r32;     // fragment 0 rows; +32 per fragment keeps the swizzle
  const int a_code = ra * RB, b_code = BM * RB + rb * RB;
  const int a_c0 = swz4(ra, g) * 16, a_c1 = swz4(ra, 2 + g) * 16;     // fp8: chunks g, 2+g; fp4: 2t+g
  const int b_c0 = swz4(rb, g) * 16, b_c1 = swz4(rb, 2 + g) * 16;
  const int a_sc = Cfg::CODE_BYTES + ra * SB, b_sc = Cfg::CODE_BYTES + (BM + rb) * SB;

  // bias of this lane's output columns, loaded once (consumed after the loop)
  uint2 bias_v[FN][4];
#pragma unroll
  for (int fn = 0; fn < FN; ++fn)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int n = n0 + wn * WN + 32 * fn + 8 * q + 4 * g;
      bias_v[fn][q] = make_uint2(0u, 0u);
      if (bias) {
        if (((N & 3) == 0) && n + 3 < N && (reinterpret_cast<uintptr_t>(bias) & 7) == 0) {
          bias_v[fn][q] = *reinterpret_cast<const uint2*>(bias + n);
        } else {
          uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
          for (int v = 0; v < 4; ++v)
            if (n + v < N) w[v] = bias[n + v];
          bias_v[fn][q] = make_uint2(w[0] | (w[1] << 16), w[2] | (w[3] << 16));
        }
      }
    }

  v16f acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = v16f{};

  // prologue: stages 0 .. NST-2 in flight
#pragma unroll
  for (int s = 0; s < NST - 1; ++s)
    if (s < nk) issue_stage(s);

  for (int ks = 0; ks < nk; ++ks) {
    // this wave's copies of stage ks have landed when at most the copies of
    // the (up to NST-2) later stages already issued are still pending
    const int later = min(nk - 1 - ks, NST - 2);
    if (later >= 2) wait_vm<2 * Cfg::OPS>();
    else if (later == 1) wait_vm<Cfg::OPS>();
    else wait_vm<0>();
    __syncthreads();                        // every wave's copies of stage ks are visible, and
                                            // every wave is done with the slot reused below
    if (ks + NST - 1 < nk) issue_stage(ks + NST - 1);

    const uint8_t* st = lds + (ks % NST) * Cfg::STAGE;
    if (Cfg::FMT == FMT_MXFP8) {
      v8i bf[FN], af[FM];
      int sbv[FN], sav[FM];
      const int sh = 8 * (2 * (ks & 1) + g);   // this lane's block within the stage pair's dword
#pragma unroll
      for (int f = 0; f < FN; ++f) {
        const uint4 lo = *reinterpret_cast<const uint4*>(st + b_code + 32 * f * RB + b_c0);
        const uint4 hi = *reinterpret_cast<const uint4*>(st + b_code + 32 * f * RB + b_c1);
        bf[f] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        sbv[f] = (int)(*reinterpret_cast<const uint32_t*>(st + b_sc + 32 * f * SB) >> sh);
      }
#pragma unroll
      for (int f = 0; f < FM; ++f) {
        const uint4 lo = *reinterpret_cast<const uint4*>(st + a_code + 32 * f * RB + a_c0);
        const uint4 hi = *reinterpret_cast<const uint4*>(st + a_code + 32 * f * RB + a_c1);
        af[f] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        sav[f] = (int)(*reinterpret_cast<const uint32_t*>(st + a_sc + 32 * f * SB) >> sh);
      }
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
          acc[fm][fn] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bf[fn], af[fm], acc[fm][fn], 0, 0, 0, sbv[fn],
                                                                        0, sav[fm]);
    } else {
      int sbv[FN], sav[FM];
#pragma unroll
      for (int f = 0; f < FN; ++f)
        sbv[f] = (int)(*reinterpret_cast<const uint32_t*>(st + b_sc + 32 * f * SB) >> (8 * g));
#pragma unroll
      for (int f = 0; f < FM; ++f)
        sav[f] = (int)(*reinterpret_cast<const uint32_t*>(st + a_sc + 32 * f * SB) >> (8 * g));
#pragma unroll
      for (int t = 0; t < 2; ++t) {         // two 64-element sub-steps; scale byte 2t (after the shift)
        v8i bf[FN], af[FM];
#pragma unroll
        for (int f = 0; f < FN; ++f) {
          const uint4 lo = *reinterpret_cast<const uint4*>(st + b_code + 32 * f * RB + (t ? b_c1 : b_c0));
          bf[f] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, 0, 0, 0, 0};
        }
#pragma unroll
        for (int f = 0; f < FM; ++f) {
          const uint4 lo = *reinterpret_cast<const uint4*>(st + a_code + 32 * f * RB + (t ? a_c1 : a_c0));
          af[f] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, 0, 0, 0, 0};
        }
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
          for (int fn = 0; fn < FN; ++fn) {
            if (t == 0)
              acc[fm][fn] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bf[fn], af[fm], acc[fm][fn], 4, 4, 0,
                                                                            sbv[fn], 0, sav[fm]);
            else
              acc[fm][fn] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bf[fn], af[fm], acc[fm][fn], 4, 4, 2,
                                                                            sbv[fn], 2, sav[fm]);
          }
      }
    }
  }

  // epilogue: register 4q + v of acc[fm][fn] is C[m][n + v] with
  // m = m0 + wm WM + 32 fm + r32, n = n0 + wn WN + 32 fn + 8 q + 4 g
  const bool vec = ((N & 3) == 0);
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
    const int m = m0 + wm * WM + 32 * fm + r32;
    if (m >= M) continue;
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = n0 + wn * WN + 32 * fn + 8 * q + 4 * g;
        if (n >= N) continue;
        const uint2 bb = bias_v[fn][q];
        float v[4];
        v[0] = acc[fm][fn][4 * q + 0] + bf16_to_f32(bb.x & 0xFFFFu);
        v[1] = acc[fm][fn][4 * q + 1] + bf16_to_f32(bb.x >> 16);
        v[2] = acc[fm][fn][4 * q + 2] + bf16_to_f32(bb.y & 0xFFFFu);
        v[3] = acc[fm][fn][4 * q + 3] + bf16_to_f32(bb.y >> 16);
        const int64_t off = (int64_t)m * N + n;
        if (out_f32) {
          float* c = reinterpret_cast<float*>(C) + off;
          if (vec && n + 3 < N) {
            *reinterpret_cast<float4*>(c) = make_float4(v[0], v[1], v[2], v[3]);
          } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
              if (n + j < N) c[j] = v[j];
          }
        } else {
          uint16_t* c = reinterpret_cast<uint16_t*>(C) + off;
          if (vec && n + 3 < N) {
            *reinterpret_cast<uint2*>(c) = make_uint2(f32_to_bf16_rne(v[0]) | (f32_to_bf16_rne(v[1]) << 16),
                                                      f32_to_bf16_rne(v[2]) | (f32_to_bf16_rne(v[3]) << 16));
          } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
              if (n + j < N) c[j] = (uint16_t)f32_to_bf16_rne(v[j]);
          }
        }
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
  // 256 x 256 tiles (8 waves of 128 x 64) when they fill the chip, else
  // 128 x 128 tiles (4 waves of 64 x 64, two workgroups per CU).
  const int64_t big_tiles = ((M + 255) / 256) * ((N + 255) / 256);
  const bool big = big_tiles >= 256;
  if (fmt == FMT_MXFP8) {
    if (big) return run_mx<MxCfg<FMT_MXFP8, 256, 256, 2, 4, 4>>(A, As, B, Bs, C, M, N, K, bias, out_f32, stream);
    return run_mx<MxCfg<FMT_MXFP8, 128, 128, 2, 2, 4>>(A, As, B, Bs, C, M, N, K, bias, out_f32, stream);
  }
  if (big) return run_mx<MxCfg<FMT_MXFP4, 256, 256, 2, 4, 4>>(A, As, B, Bs, C, M, N, K, bias, out_f32, stream);
  return run_mx<MxCfg<FMT_MXFP4, 128, 128, 2, 2, 4>>(A, As, B, Bs, C, M, N, K, bias, out_f32, stream);
}

}  // namespace mx
