// NVFP4 GEMM for gfx950: C = s_tA s_tB sum_k (a_k dA)(b_k dB) (+ bias[n]).
//
// lightly-train README "DINOv3 + EoMT on RTX 5090", section 2: NVFP4 is
// E2M1 elements with an E4M3 scale per 1x16 block plus an fp32 scale per
// tensor; section 5.3-5.5 use it for the dgrad / wgrad GEMMs of training.
//
// CDNA4's scaled matrix instructions take power-of-two (E8M0) scales per 32
// elements, which cannot express an E4M3 scale per 16. Folding the E4M3
// scale into the element instead is exact in fp16: a_k * dA has at most
// 2 + 4 significant bits and lies in [2^-10, 2688] (normal fp16), so the
// product of two such values (<= 12 bits) is exact in the fp32 matrix
// accumulator too. The kernel therefore dequantizes each operand tile to
// fp16 while staging it into LDS (one pass per tile, shared by all waves):
// nibble -> fp16 via a byte-permute table, times the block scale as a packed
// fp16 multiply; then runs V_MFMA_F32_16X16X32_F16 with fp32 accumulation
// and applies s_tA * s_tB in the epilogue. The roof of this path is the fp16
// matrix rate, a quarter of the FP4 rate; the accuracy is that of the exact
// method (fp32 accumulation only).
//
// fp16 operand layout (measured on gfx950): lane l holds row l%16, K
// 8g..8g+7, g = l/16; output as in the MX kernel (lane: D[4g + v][l%16]).
#include "mx_device.h"
#include "mx_launch.h"

namespace mx {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

template <int BM_, int BN_, int WAVES_M_, int WAVES_N_, int SWZ_>
struct NvCfg {
  static constexpr int BM = BM_, BN = BN_, WAVES_M = WAVES_M_, WAVES_N = WAVES_N_, SWZ = SWZ_;
  static constexpr int NT = 64 * WAVES_M * WAVES_N;
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  static constexpr int FM = WM / 16, FN = WN / 16;
  static constexpr int KS = 64;                  // K elements per stage
  static constexpr int ROWB = KS * 2;            // fp16 bytes per LDS row
  static constexpr int CH = ROWB / 16;           // 16-byte chunks per LDS row (8)
  static constexpr int A_STAGE = BM * ROWB, B_STAGE = BN * ROWB;
  static constexpr int A_ITEMS = BM * 2 / NT;    // 16-byte code chunks (32 elements) per thread
  static constexpr int B_ITEMS = BN * 2 / NT;
  static_assert(A_ITEMS * NT == BM * 2 && B_ITEMS * NT == BN * 2, "items");
};

__device__ __forceinline__ int nv_swz(int r, int c, int shift) { return c ^ ((r >> shift) & 7); }

// fp16 bits of a non-negative E4M3 scale byte, replicated into both halves.
__device__ __forceinline__ uint32_t e4m3_to_h2(uint32_t b) {
  const uint32_t e = (b >> 3) & 15u, m = b & 7u;
  float f = e ? (float)(8u + m) * __uint_as_float((e - 10u + 127u) << 23) : (float)m * 0.001953125f;
  _Float16 h = (_Float16)f;   // exact: E4M3 values are fp16 values
  uint32_t hb = (uint32_t)__builtin_bit_cast(uint16_t, h);
  return hb | (hb << 16);
}

// 8 E2M1 codes (one dword, element j in nibble j) times a scale (half2 bits)
// -> 8 fp16 values in 4 dwords, element order preserved.
__device__ __forceinline__ uint4 dequant8(uint32_t x, uint32_t scale_h2) {
  // fp16 high byte of each E2M1 magnitude: 0, 0.5, 1, 1.5 | 2, 3, 4, 6
  constexpr uint32_t LUT_LO = 0x3E3C3800u, LUT_HI = 0x46444240u;
  const uint32_t lo = x & 0x0F0F0F0Fu;            // elements 0, 2, 4, 6 (byte k = element 2k)
  const uint32_t hi = (x >> 4) & 0x0F0F0F0Fu;     // elements 1, 3, 5, 7
  const uint32_t plo = __builtin_amdgcn_perm(LUT_HI, LUT_LO, lo & 0x07070707u) | ((lo & 0x08080808u) << 4);
  const uint32_t phi = __builtin_amdgcn_perm(LUT_HI, LUT_LO, hi & 0x07070707u) | ((hi & 0x08080808u) << 4);
  uint32_t h[4];
  h[0] = __builtin_amdgcn_perm(phi, plo, 0x040C000Cu);   // {elem0, elem1}
  h[1] = __builtin_amdgcn_perm(phi, plo, 0x050C010Cu);
  h[2] = __builtin_amdgcn_perm(phi, plo, 0x060C020Cu);
  h[3] = __builtin_amdgcn_perm(phi, plo, 0x070C030Cu);
  const v2h s = __builtin_bit_cast(v2h, scale_h2);
  uint4 out;
  out.x = __builtin_bit_cast(uint32_t, __builtin_bit_cast(v2h, h[0]) * s);
  out.y = __builtin_bit_cast(uint32_t, __builtin_bit_cast(v2h, h[1]) * s);
  out.z = __builtin_bit_cast(uint32_t, __builtin_bit_cast(v2h, h[2]) * s);
  out.w = __builtin_bit_cast(uint32_t, __builtin_bit_cast(v2h, h[3]) * s);
  return out;
}

// Same tile numbering as the MX kernel.
__device__ __forceinline__ void nv_tile_coords(int tiles_m, int tiles_n, int& tm, int& tn) {
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

__device__ __forceinline__ void nv_store4(void* C, int M, int N, int m, int n, v4f acc, float scale,
                                         const uint16_t* bias, int out_f32) {
  if (m >= M) return;
  float v[4] = {acc[0] * scale, acc[1] * scale, acc[2] * scale, acc[3] * scale};
  const bool full = ((N & 3) == 0) && (n + 3 < N);
  if (bias) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (n + j < N) v[j] += bf16_to_f32(bias[n + j]);
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

template <class Cfg>
__global__ __launch_bounds__(Cfg::NT) void gemm_nv_kernel(const uint8_t* __restrict__ A,
                                                          const uint8_t* __restrict__ As,
                                                          const uint8_t* __restrict__ B,
                                                          const uint8_t* __restrict__ Bs, void* __restrict__ C,
                                                          int M, int N, int kpad,
                                                          const uint16_t* __restrict__ bias, int out_f32,
                                                          int tiles_m, int tiles_n, int a_trailer, int b_trailer) {
  constexpr int NT = Cfg::NT, ROWB = Cfg::ROWB;
  constexpr int BM = Cfg::BM, BN = Cfg::BN, WM = Cfg::WM, WN = Cfg::WN, FM = Cfg::FM, FN = Cfg::FN;
  __shared__ __align__(16) uint8_t lds[2 * (Cfg::A_STAGE + Cfg::B_STAGE)];

  int tm, tn;
  nv_tile_coords(tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave / Cfg::WAVES_N, wn = wave % Cfg::WAVES_N;
  const int row_bytes = kpad / 2;           // code bytes per row
  const int srow = kpad / 16;               // scale bytes per row
  const int nk = kpad / Cfg::KS;
  const int g = lane >> 4, r16 = lane & 15;

  const __amdgpu_buffer_rsrc_t a_rs = __builtin_amdgcn_make_buffer_rsrc((void*)A, 0, M * row_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t b_rs = __builtin_amdgcn_make_buffer_rsrc((void*)B, 0, N * row_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t as_rs = __builtin_amdgcn_make_buffer_rsrc((void*)As, 0, M * srow, 0x00020000);
  const __amdgpu_buffer_rsrc_t bs_rs = __builtin_amdgcn_make_buffer_rsrc((void*)Bs, 0, N * srow, 0x00020000);

  // staging items: item q covers row q/2, code bytes 16 (q%2) .. +15 of the
  // stage (elements 32 (q%2) .. +31, two 16-element scale blocks)
  int a_coff[Cfg::A_ITEMS], a_soff[Cfg::A_ITEMS], a_lds[Cfg::A_ITEMS][4];
#pragma unroll
  for (int i = 0; i < Cfg::A_ITEMS; ++i) {
    const int q = t + NT * i, r = q / 2, h = q % 2;
    a_coff[i] = (m0 + r) * row_bytes + 16 * h;
    a_soff[i] = (m0 + r) * srow + 2 * h;
#pragma unroll
    for (int d = 0; d < 4; ++d) a_lds[i][d] = r * ROWB + nv_swz(r, 4 * h + d, Cfg::SWZ) * 16;
  }
  int b_coff[Cfg::B_ITEMS], b_soff[Cfg::B_ITEMS], b_lds[Cfg::B_ITEMS][4];
#pragma unroll
  for (int i = 0; i < Cfg::B_ITEMS; ++i) {
    const int q = t + NT * i, r = q / 2, h = q % 2;
    b_coff[i] = (n0 + r) * row_bytes + 16 * h;
    b_soff[i] = (n0 + r) * srow + 2 * h;
#pragma unroll
    for (int d = 0; d < 4; ++d) b_lds[i][d] = r * ROWB + nv_swz(r, 4 * h + d, Cfg::SWZ) * 16;
  }
  const int ra = wm * WM + r16, rb = wn * WN + r16;
  const int a_off0 = ra * ROWB + nv_swz(ra, g, Cfg::SWZ) * 16;
  const int a_off1 = ra * ROWB + nv_swz(ra, 4 + g, Cfg::SWZ) * 16;
  const int b_off0 = rb * ROWB + nv_swz(rb, g, Cfg::SWZ) * 16;
  const int b_off1 = rb * ROWB + nv_swz(rb, 4 + g, Cfg::SWZ) * 16;

  uint4 a_code[Cfg::A_ITEMS], b_code[Cfg::B_ITEMS];
  uint32_t a_sc[Cfg::A_ITEMS], b_sc[Cfg::B_ITEMS];

  auto load_stage = [&](int ks) {
#pragma unroll
    for (int i = 0; i < Cfg::A_ITEMS; ++i) {
      a_code[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(a_rs, a_coff[i], ks * 32, 0));
      a_sc[i] = __builtin_amdgcn_raw_buffer_load_b16(as_rs, a_soff[i], ks * 4, 0);
    }
#pragma unroll
    for (int i = 0; i < Cfg::B_ITEMS; ++i) {
      b_code[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(b_rs, b_coff[i], ks * 32, 0));
      b_sc[i] = __builtin_amdgcn_raw_buffer_load_b16(bs_rs, b_soff[i], ks * 4, 0);
    }
  };
  auto store_stage = [&](int buf) {
    uint8_t* a_dst = lds + buf * Cfg::A_STAGE;
    uint8_t* b_dst = lds + 2 * Cfg::A_STAGE + buf * Cfg::B_STAGE;
#pragma unroll
    for (int i = 0; i < Cfg::A_ITEMS; ++i) {
      const uint32_t s0 = e4m3_to_h2(a_sc[i] & 0xFFu), s1 = e4m3_to_h2((a_sc[i] >> 8) & 0xFFu);
      *reinterpret_cast<uint4*>(a_dst + a_lds[i][0]) = dequant8(a_code[i].x, s0);
      *reinterpret_cast<uint4*>(a_dst + a_lds[i][1]) = dequant8(a_code[i].y, s0);
      *reinterpret_cast<uint4*>(a_dst + a_lds[i][2]) = dequant8(a_code[i].z, s1);
      *reinterpret_cast<uint4*>(a_dst + a_lds[i][3]) = dequant8(a_code[i].w, s1);
    }
#pragma unroll
    for (int i = 0; i < Cfg::B_ITEMS; ++i) {
      const uint32_t s0 = e4m3_to_h2(b_sc[i] & 0xFFu), s1 = e4m3_to_h2((b_sc[i] >> 8) & 0xFFu);
      *reinterpret_cast<uint4*>(b_dst + b_lds[i][0]) = dequant8(b_code[i].x, s0);
      *reinterpret_cast<uint4*>(b_dst + b_lds[i][1]) = dequant8(b_code[i].y, s0);
      *reinterpret_cast<uint4*>(b_dst + b_lds[i][2]) = dequant8(b_code[i].z, s1);
      *reinterpret_cast<uint4*>(b_dst + b_lds[i][3]) = dequant8(b_code[i].w, s1);
    }
  };

  v4f acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  load_stage(0);
  store_stage(0);
  __syncthreads();

  for (int ks = 0; ks < nk; ++ks) {
    const int cur = ks & 1;
    const bool more = ks + 1 < nk;
    if (more) load_stage(ks + 1);
    const uint8_t* a_buf = lds + cur * Cfg::A_STAGE;
    const uint8_t* b_buf = lds + 2 * Cfg::A_STAGE + cur * Cfg::B_STAGE;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      v8h bfrag[FN];
#pragma unroll
      for (int f = 0; f < FN; ++f)
        bfrag[f] = __builtin_bit_cast(v8h, *reinterpret_cast<const uint4*>(b_buf + (sub ? b_off1 : b_off0) + 16 * f * ROWB));
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) {
        const v8h afrag =
            __builtin_bit_cast(v8h, *reinterpret_cast<const uint4*>(a_buf + (sub ? a_off1 : a_off0) + 16 * fm * ROWB));
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
          acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bfrag[fn], afrag, acc[fm][fn], 0, 0, 0);
      }
    }
    if (more) store_stage(cur ^ 1);
    __syncthreads();
  }

  // epilogue: the two tensor scales live in the scale buffers' trailers
  const float sta = *reinterpret_cast<const float*>(As + a_trailer);
  const float stb = *reinterpret_cast<const float*>(Bs + b_trailer);
  const float scale = sta * stb;
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
    const int m = m0 + wm * WM + 16 * fm + r16;
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
      const int n = n0 + wn * WN + 16 * fn + 4 * g;
      nv_store4(C, M, N, m, n, acc[fm][fn], scale, bias, out_f32);
    }
  }
}

template <class Cfg>
static hipError_t run_nv(const uint8_t* A, const uint8_t* As, const uint8_t* B, const uint8_t* Bs, void* C,
                         int64_t M, int64_t N, int64_t K, const uint16_t* bias, int out_f32, hipStream_t stream) {
  const int64_t kpad = round_up(K, kAlignK);
  const int tiles_m = (int)((M + Cfg::BM - 1) / Cfg::BM);
  const int tiles_n = (int)((N + Cfg::BN - 1) / Cfg::BN);
  const int a_tr = (int)round_up(M * (kpad / 16), 16);
  const int b_tr = (int)round_up(N * (kpad / 16), 16);
  gemm_nv_kernel<Cfg><<<tiles_m * tiles_n, Cfg::NT, 0, stream>>>(A, As, B, Bs, C, (int)M, (int)N, (int)kpad, bias,
                                                                  out_f32, tiles_m, tiles_n, a_tr, b_tr);
  return hipGetLastError();
}

const char* plan_gemm_nvfp4(int64_t, int64_t) { return "gemm_nv_kernel<nvfp4, 128x128>"; }

hipError_t launch_gemm_nvfp4(const uint8_t* A, const uint8_t* As, const uint8_t* B, const uint8_t* Bs, void* C,
                             int64_t M, int64_t N, int64_t K, const uint16_t* bias, int out_f32,
                             hipStream_t stream) {
  return run_nv<NvCfg<128, 128, 2, 2, 0>>(A, As, B, Bs, C, M, N, K, bias, out_f32, stream);
}

}  // namespace mx
