// NVFP4 GEMM for gfx950: C = s_tA s_tB sum_k (a_k dA)(b_k dB) (+ bias[n]).
//
// lightly-train README "DINOv3 + EoMT on RTX 5090", section 2: NVFP4 is
// E2M1 elements with an E4M3 scale per 1x16 block plus an fp32 scale per
// tensor; sections 5.3-5.5 use it for the dgrad / wgrad GEMMs of training.
//
// CDNA4's scaled matrix instructions take power-of-two (E8M0) scales per 32
// elements, which cannot express an E4M3 scale per 16. Folding the E4M3
// scale into the element instead is exact in fp16: a_k * dA has at most
// 2 + 4 significant bits and lies in [2^-10, 2688] (normal fp16), so the
// product of two such values (<= 12 bits) is exact in the fp32 matrix
// accumulator too. The kernel therefore dequantizes each operand tile to
// fp16 while staging it into LDS (once per tile row, shared by all waves):
// two codes -> fp16 pair by the hardware conversion, times the block scale
// as a packed fp16 multiply; then runs V_MFMA_F32_32X32X16_F16 with fp32 accumulation
// and applies s_tA * s_tB in the epilogue. The roof of this path is the fp16
// matrix rate; the accuracy is that of the exact method (fp32 accumulation
// only).
//
// Structure (as in the MX kernel): a persistent walk over output tiles with
// XCD-contiguous numbering, 8 waves of 128 x 64 (or 96 x 64) outputs, two
// LDS stages of 64 K elements (128 fp16 bytes per row, chunk-swizzled) and
// the LDS-staged bf16 epilogue. Staging goes through registers: after a
// stage's barrier every thread loads one tile row's 32 code bytes and 4
// scale bytes of the next stage (global -> VGPR), the stage's matrix
// instructions run, then the thread writes that row, dequantized, into the
// other LDS buffer before the next barrier.
//
// fp16 operand layout of the 32x32x16 instruction (measured on gfx950):
// lane l holds row l % 32, K 8 (l / 32) .. + 7; output as in the MX kernel.
#include "gemm_common.h"
#include "mx_launch.h"

#include <algorithm>
#include <cstdio>
#include <mutex>
#include <type_traits>

namespace mx {

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

template <int BM_, int BN_, int WAVES_M_, int WAVES_N_, int OCC_>
struct NvCfg {
  static constexpr int BM = BM_, BN = BN_, WAVES_M = WAVES_M_, WAVES_N = WAVES_N_, OCC = OCC_;
  static constexpr int NT = 64 * WAVES_M * WAVES_N, NW = NT / 64;
  static constexpr int RB = 128;                              // fp16 bytes per LDS row per stage
  static constexpr int KS = 64;                               // K elements per stage
  static constexpr int SUB = KS / 16;                         // 32x32x16 sub-steps per stage
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  static constexpr int FM = WM / 32, FN = WN / 32;
  static constexpr int STAGE = (BM + BN) * RB;
  static constexpr int BIAS_OFF = 2 * STAGE;                  // two 1-KB bias slots (tile parity)
  static constexpr int SCRATCH_OFF = BIAS_OFF + 2 * 1024;     // rows of threads past BM + BN
  static constexpr int LDS = SCRATCH_OFF + (NT - BM - BN) * RB;
  static constexpr int CPR = BN / 8;
  static constexpr int EPI_STORES = WM * CPR / NT;
  static_assert(BM + BN <= NT, "one staged row per thread");
  static_assert(BM % 64 == 0 && BN % 64 == 0 && WM % 32 == 0 && WN % 32 == 0, "tile");
  static_assert(LDS * OCC <= 160 * 1024, "LDS");
  static_assert(WM * BN * 2 <= STAGE, "one wave-row of the bf16 C tile must fit in a stage buffer");
  static_assert(EPI_STORES * NT == WM * CPR, "epilogue stores must split evenly over threads");
  static_assert(BN * 2 <= 1024 && BN / 8 <= NT, "a tile's bias must fit one bias slot");
};

// E4M3 scale byte j of `scales` (sign ignored) placed as fp16 bits into both
// halves of a dword, read as fp16 it is 2^-8 times the E4M3 value: the 4
// exponent and 3 mantissa bits land in the low bits of fp16's 5-bit exponent
// and the top of its mantissa, which rebiases the exponent by 8 for normal
// values and turns E4M3 subnormals into fp16 subnormals of the same
// significand. The factor 2^8 is carried by the element conversion below.
template <int J>
__device__ __forceinline__ uint32_t e4m3_h2_div256(uint32_t scales) {
  // bytes {J, 0, J, 0} -> two 16-bit copies of the byte, then shift into place
  constexpr uint32_t sel = 0x0C000C00u | (J << 16) | J;
  return __builtin_amdgcn_perm(0u, scales & 0x7F7F7F7Fu, sel) << 7;
}

// 8 E2M1 codes (one dword, element j in nibble j) times a scale (fp16 pair
// from e4m3_h2_div256) -> 8 fp16 values in 4 dwords, element order kept.
// The hardware conversion turns the two codes of one byte into fp16 (low
// nibble -> low half) times a power of two taken from its fp32 scale
// operand (only the exponent is used); with 2^8 there, the packed multiply
// by the E4M3 scale / 2^8 gives the exact element values (products of at
// most 6 significant bits, between 2^-10 and 2688 in magnitude: normal fp16).
__device__ __forceinline__ uint4 dequant8(uint32_t x, uint32_t scale_h2) {
  const v2h s = __builtin_bit_cast(v2h, scale_h2);
  uint4 out;
  out.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 256.0f, 0) * s);
  out.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 256.0f, 1) * s);
  out.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 256.0f, 2) * s);
  out.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 256.0f, 3) * s);
  return out;
}

// fp16 fragment of sub-step t for tile row `row`: chunk 2t + g (K 16t + 8g ..).
template <class Cfg>
__device__ __forceinline__ v8h nv_frag(const uint8_t* st, int row, int t, int g) {
  return __builtin_bit_cast(v8h, *reinterpret_cast<const uint4*>(st + row * Cfg::RB + swz(row, 2 * t + g) * 16));
}

// STAGED: bf16 output written through LDS in 16-byte rows (N % 8 == 0 and
// M N < 2^30); otherwise each lane writes its own outputs. The two are
// separate kernels so that the waits of a tile's first stage are the same on
// every path into it.
template <class Cfg, bool STAGED>
__global__ __launch_bounds__(Cfg::NT, Cfg::OCC) void gemm_nv_kernel(const uint8_t* __restrict__ A,
                                                                    const uint8_t* __restrict__ As,
                                                                    const uint8_t* __restrict__ B,
                                                                    const uint8_t* __restrict__ Bs,
                                                                    void* __restrict__ C, int M, int N, int kpad,
                                                                    const uint16_t* __restrict__ bias, int out_f32,
                                                                    int tiles_m, int tiles_n, int a_trailer,
                                                                    int b_trailer, int splits,
                                                                    float* __restrict__ ws) {
  constexpr int BM = Cfg::BM, BN = Cfg::BN, WM = Cfg::WM, WN = Cfg::WN, FM = Cfg::FM, FN = Cfg::FN;
  constexpr int RB = Cfg::RB, SUB = Cfg::SUB, CPR = Cfg::CPR;
  __shared__ __align__(16) uint8_t lds[Cfg::LDS];

  // work items: (tile, split) pairs; with splits > 1 an item covers the K
  // stages [k0, k1) of its split (an even number: stages come in pairs) and
  // writes its fp32 partial tile, times s_tA s_tB, to ws + split M N (no
  // bias), summed by the split-K reduction afterwards
  const int tiles = tiles_m * tiles_n * splits;
  const int tid = (int)threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / Cfg::WAVES_N, wn = wave % Cfg::WAVES_N;
  const int row_bytes = kpad / 2;            // code bytes per row
  const int srow = kpad / 16;                // scale bytes per row
  const int nk = kpad / Cfg::KS;             // K_pad is a multiple of 128
  const int g = lane >> 5, r32 = lane & 31;
  constexpr bool staged = STAGED;
  auto item = [&](int t, int& tm, int& tn, int& sp, int& k0, int& k1) {
    int tnv;
    tile_coords(t, tiles_m, tiles_n * splits, tm, tnv);
    tn = tnv % tiles_n;
    sp = tnv / tiles_n;
    k0 = 2 * ((sp * (nk / 2)) / splits);
    k1 = 2 * (((sp + 1) * (nk / 2)) / splits);
  };

  const __amdgpu_buffer_rsrc_t a_rs = __builtin_amdgcn_make_buffer_rsrc((void*)A, (short)0, M * row_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t b_rs = __builtin_amdgcn_make_buffer_rsrc((void*)B, (short)0, N * row_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t as_rs = __builtin_amdgcn_make_buffer_rsrc((void*)As, (short)0, M * srow, 0x00020000);
  const __amdgpu_buffer_rsrc_t bs_rs = __builtin_amdgcn_make_buffer_rsrc((void*)Bs, (short)0, N * srow, 0x00020000);
  const __amdgpu_buffer_rsrc_t c_rs =
      __builtin_amdgcn_make_buffer_rsrc(C, (short)0, staged ? M * N * 2 : 0, 0x00020000);
  // a 16-byte aligned bias with N % 8 == 0 is loaded 8 columns per thread;
  // otherwise element by element
  const bool bias_vec = bias != nullptr && (N & 7) == 0 && (reinterpret_cast<uintptr_t>(bias) & 15) == 0;
  const __amdgpu_buffer_rsrc_t bias_rs =
      __builtin_amdgcn_make_buffer_rsrc((void*)bias, (short)0, bias_vec ? N * 2 : 0, 0x00020000);

  // Staging: thread tid stages row tid of the stage, i.e. A row tid (waves
  // below BM / 64) or B row tid - BM; threads past BM + BN write their
  // (zero) rows into a scratch area. Loader cursor: tile lt, its stage lks,
  // ltc tiles begun. The loads of a stage run two stages ahead of the
  // matrix instructions, into one of two register sets, so that each stage
  // dequantizes the next stage's rows (loaded a full stage earlier) in the
  // same instruction stream as its own matrix instructions. Every stage
  // issues exactly 4 loads per wave (2 x 16 code bytes, 4 scale bytes, 16
  // bias bytes); those with nothing to load use an offset past the buffer's
  // range and read zero.
  const bool stager = tid < BM + BN;
  const bool st_is_a = wave < BM / 64;       // wave-uniform: BM is a multiple of 64
  const int st_row = st_is_a ? tid : tid - BM;
  uint8_t* const st_dst = stager ? lds + tid * RB : lds + Cfg::SCRATCH_OFF + (tid - BM - BN) * RB;
  const int st_buf_stride = stager ? Cfg::STAGE : 0;
  int lt = blockIdx.x, lks = 0, lk0 = 0, lk1 = nk, ltc = 0;
  int code_off = 0, scale_off = 0, bias_col = 0;
  auto set_load_tile = [&](int t) {
    int tm, tn, sp;
    item(t, tm, tn, sp, lk0, lk1);
    lks = lk0;
    const int r = (st_is_a ? tm * BM : tn * BN) + st_row;
    code_off = r * row_bytes;                // rows past the operand read as zero (range-checked)
    scale_off = r * srow;
    bias_col = tn * BN + 8 * tid;            // first bias column of threads tid < BN / 8
  };
  struct Raw {
    uint4 c0, c1, bias;
    uint32_t sc;
    int first, slot;                         // wave-uniform: first stage of a tile, its bias slot
  };
  constexpr int OOB = (int)0x80000000u;
  auto load = [&](Raw& R) {                  // global -> registers, then advance the cursor
    const bool loading = lt < tiles;
    const __amdgpu_buffer_rsrc_t crs = st_is_a ? a_rs : b_rs;
    const __amdgpu_buffer_rsrc_t srs = st_is_a ? as_rs : bs_rs;
    const bool row_live = stager && loading;
    const int co = row_live ? code_off + lks * 32 : OOB;
    const int so = row_live ? scale_off + lks * 4 : OOB;
    const int bo = (loading && lks == lk0 && bias_vec && tid < BN / 8) ? bias_col * 2 : OOB;
    R.c0 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(crs, co, 0, 0));
    R.c1 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(crs, co, 16, 0));
    R.sc = __builtin_amdgcn_raw_buffer_load_b32(srs, so, 0, 0);
    R.bias = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(bias_rs, bo, 0, 0));
    R.first = loading && lks == lk0;
    R.slot = ltc & 1;
    if (loading && ++lks == lk1) {
      lks = lk0;
      ++ltc;
      lt += gridDim.x;
      if (lt < tiles) set_load_tile(lt);
    }
  };
  // registers -> dequantized fp16 row in LDS buffer `buf` (one 16-byte
  // chunk per call, chunk c covers K 8c .. 8c + 7 of the stage)
  auto dequant_chunk = [&](const Raw& R, int buf, int c) {
    const uint32_t w = c < 4 ? (&R.c0.x)[c] : (&R.c1.x)[c - 4];
    uint32_t sh;
    switch (c / 2) {
      case 0: sh = e4m3_h2_div256<0>(R.sc); break;
      case 1: sh = e4m3_h2_div256<1>(R.sc); break;
      case 2: sh = e4m3_h2_div256<2>(R.sc); break;
      default: sh = e4m3_h2_div256<3>(R.sc); break;
    }
    *reinterpret_cast<uint4*>(st_dst + buf * st_buf_stride + swz(tid, c) * 16) = dequant8(w, sh);
  };
  auto store_bias = [&](const Raw& R) {      // a tile's bias, into bias slot R.slot
    if (R.first && bias != nullptr && tid < BN / 8) {
      uint4 v = R.bias;
      if (!bias_vec) {
        uint32_t e[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (bias_col + i < N) e[i] = bias[bias_col + i];
        v = make_uint4(e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16), e[6] | (e[7] << 16));
      }
      *reinterpret_cast<uint4*>(lds + Cfg::BIAS_OFF + R.slot * 1024 + 16 * tid) = v;
    }
  };

  const int ra = wm * WM + r32, rb = wn * WN + r32;
  const float tensor_scale = *reinterpret_cast<const float*>(As + a_trailer) *
                             *reinterpret_cast<const float*>(Bs + b_trailer);

  Raw R0, R1;
  set_load_tile(lt);
  load(R0);
  load(R1);
  wait_vm<4>();                              // R0 has landed
#pragma unroll
  for (int c = 0; c < 8; ++c) dequant_chunk(R0, 0, c);
  store_bias(R0);
  if (STAGED) {
    // as many (discarded) stores as a tile's epilogue issues, so that the
    // first stage finds the same operations in flight on every path
#pragma unroll
    for (int j = 0; j < Cfg::WAVES_M * Cfg::EPI_STORES; ++j)
      __builtin_amdgcn_raw_buffer_store_b128(v4u{0u, 0u, 0u, 0u}, c_rs, OOB + 16 * j, 0, 0);   // distinct: kept
  }
  int ctc = 0;

  // One stage: matrix instructions on LDS buffer P while the other register
  // set's rows are dequantized into buffer 1 - P; LS receives the loads of
  // the stage after next. Every tile has an even number of stages, so its
  // stages use buffers 0, 1, 0, ..., 1.
  v16f acc[FM][FN];
  // DS's loads are waited for by the compiler's own bookkeeping, which
  // leaves the previous tile's stores and LS's loads in flight.
  auto stage = [&](auto parity, Raw& LS, Raw& DS) {
    constexpr int P = decltype(parity)::value;
    block_sync();                            // buffer P is complete; nobody reads buffer 1 - P
    load(LS);
    const uint8_t* st = lds + P * Cfg::STAGE;
    constexpr int TOTAL = SUB * FM * FN;
    v8h b_cur[FN], b_nxt[FN], a_cur, a_nxt;
#pragma unroll
    for (int f = 0; f < FN; ++f) b_cur[f] = nv_frag<Cfg>(st, BM + rb + 32 * f, 0, g);
    a_cur = nv_frag<Cfg>(st, ra, 0, g);
#pragma unroll
    for (int t = 0; t < SUB; ++t) {
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) {
        if (fm + 1 < FM) a_nxt = nv_frag<Cfg>(st, ra + 32 * (fm + 1), t, g);
        else if (t + 1 < SUB) a_nxt = nv_frag<Cfg>(st, ra, t + 1, g);
        if (fm == 0 && t + 1 < SUB) {
#pragma unroll
          for (int f = 0; f < FN; ++f) b_nxt[f] = nv_frag<Cfg>(st, BM + rb + 32 * f, t + 1, g);
        }
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
          acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_f16(b_cur[fn], a_cur, acc[fm][fn], 0, 0, 0);
          const int i = (t * FM + fm) * FN + fn;            // matrix instruction index in the stage
#pragma unroll
          for (int c = 0; c < 8; ++c)
            if (i == c * TOTAL / 8) dequant_chunk(DS, 1 - P, c);
        }
        if (fm + 1 < FM || t + 1 < SUB) a_cur = a_nxt;
      }
      if (t + 1 < SUB) {
#pragma unroll
        for (int f = 0; f < FN; ++f) b_cur[f] = b_nxt[f];
      }
    }
    store_bias(DS);
  };

  for (int ct = blockIdx.x; ct < tiles; ct += gridDim.x) {
    int tm, tn, sp, k0, k1;
    item(ct, tm, tn, sp, k0, k1);
    const int m0 = tm * BM, n0 = tn * BN;
    // a split item's partial goes to its slice of the workspace, in fp32
    void* const Ct = splits > 1 ? static_cast<void*>(ws + (int64_t)sp * M * N) : C;
    const int out_f32_t = splits > 1 ? 1 : out_f32;

#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = v16f{};

    // the first pair is peeled: its predecessors are the prologue and the
    // previous tile's epilogue, not the loop's back edge
    stage(std::integral_constant<int, 0>{}, R0, R1);
    stage(std::integral_constant<int, 1>{}, R1, R0);
    for (int ks = k0 + 2; ks < k1; ks += 2) {
      stage(std::integral_constant<int, 0>{}, R0, R1);
      stage(std::integral_constant<int, 1>{}, R1, R0);
    }

    // epilogue: register 4q + v of acc[fm][fn] is C[m][n + v] with
    // m = m0 + wm WM + 32 fm + r32, n = n0 + wn WN + 32 fn + 8 q + 4 g; the
    // tile's bias is in bias slot ctc & 1 (written with its first stage)
    const uint8_t* lds_bias = lds + Cfg::BIAS_OFF + (ctc & 1) * 1024;
    auto bias4 = [&](int nl) -> uint2 {
      if (bias == nullptr) return make_uint2(0u, 0u);
      return *reinterpret_cast<const uint2*>(lds_bias + 2 * nl);
    };
    if constexpr (STAGED) {
      uint8_t* stg = lds + Cfg::STAGE;     // buffer 1: the last stage's, just consumed
#pragma unroll
      for (int h = 0; h < Cfg::WAVES_M; ++h) {
        block_sync();                        // previous readers of the buffer are done
        if (wm == h) {
#pragma unroll
          for (int fn = 0; fn < FN; ++fn) {
            uint2 bb[4];                     // bias of this lane's columns of fragment column fn
#pragma unroll
            for (int q = 0; q < 4; ++q) bb[q] = bias4(wn * WN + 32 * fn + 8 * q + 4 * g);
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) {
              const int lr = 32 * fm + r32;
              uint32_t P[4][2];
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const float v0 = acc[fm][fn][4 * q + 0] * tensor_scale + bf16_to_f32(bb[q].x & 0xFFFFu);
                const float v1 = acc[fm][fn][4 * q + 1] * tensor_scale + bf16_to_f32(bb[q].x >> 16);
                const float v2 = acc[fm][fn][4 * q + 2] * tensor_scale + bf16_to_f32(bb[q].y & 0xFFFFu);
                const float v3 = acc[fm][fn][4 * q + 3] * tensor_scale + bf16_to_f32(bb[q].y >> 16);
                P[q][0] = pack_bf16x2(v0, v1);
                P[q][1] = pack_bf16x2(v2, v3);
              }
#pragma unroll
              for (int p = 0; p < 2; ++p) {
                // lane g = 0 ends with columns 16p .. 16p + 7 of the fragment,
                // lane g = 1 with 16p + 8 .. + 15
                const auto s0 = __builtin_amdgcn_permlane32_swap(P[2 * p][0], P[2 * p + 1][0], false, false);
                const auto s1 = __builtin_amdgcn_permlane32_swap(P[2 * p][1], P[2 * p + 1][1], false, false);
                const int chunk = (wn * WN + 32 * fn + 16 * p + 8 * g) >> 3;
                *reinterpret_cast<uint4*>(stg + lr * (BN * 2) + ((chunk ^ (lr & (CPR - 1))) * 16)) =
                    make_uint4(s0[0], s1[0], s0[1], s1[1]);
              }
            }
          }
        }
        block_sync();
#pragma unroll
        for (int j = 0; j < Cfg::EPI_STORES; ++j) {
          const int id = tid + j * Cfg::NT;
          const int row = id / CPR, c = id % CPR;
          const int m = m0 + h * WM + row, n = n0 + 8 * c;
          const uint4 w = *reinterpret_cast<const uint4*>(stg + row * (BN * 2) + ((c ^ (row & (CPR - 1))) * 16));
          const int off = (m < M && n < N) ? (m * N + n) * 2 : (int)0x80000000u;
          __builtin_amdgcn_raw_buffer_store_b128(v4u{w.x, w.y, w.z, w.w}, c_rs, off, 0, kStoreDeviceScope);
        }
      }
    } else {
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
            const uint2 bb = bias4(n - n0);
            float v[4];
            v[0] = acc[fm][fn][4 * q + 0] * tensor_scale + bf16_to_f32(bb.x & 0xFFFFu);
            v[1] = acc[fm][fn][4 * q + 1] * tensor_scale + bf16_to_f32(bb.x >> 16);
            v[2] = acc[fm][fn][4 * q + 2] * tensor_scale + bf16_to_f32(bb.y & 0xFFFFu);
            v[3] = acc[fm][fn][4 * q + 3] * tensor_scale + bf16_to_f32(bb.y >> 16);
            const int64_t off = (int64_t)m * N + n;
            if (out_f32_t) {
              float* c = reinterpret_cast<float*>(Ct) + off;
              if (vec && n + 3 < N) {
                *reinterpret_cast<float4*>(c) = make_float4(v[0], v[1], v[2], v[3]);
              } else {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                  if (n + j < N) c[j] = v[j];
              }
            } else {
              uint16_t* c = reinterpret_cast<uint16_t*>(Ct) + off;
              if (vec && n + 3 < N) {
                *reinterpret_cast<uint2*>(c) = make_uint2(pack_bf16x2(v[0], v[1]),
                                                          pack_bf16x2(v[2], v[3]));
              } else {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                  if (n + j < N) c[j] = (uint16_t)f32_to_bf16_rne(v[j]);
              }
            }
          }
      }
    }
    ++ctc;
  }
  wait_vm<0>();                              // the drained loader's zero loads and the last stores
}

template <class Cfg>
static hipError_t run_nv(const uint8_t* A, const uint8_t* As, const uint8_t* B, const uint8_t* Bs, void* C,
                         int64_t M, int64_t N, int64_t K, const uint16_t* bias, int out_f32, int splits, float* ws,
                         hipStream_t stream) {
  const int64_t kpad = round_up(K, kAlignK);
  const int tiles_m = (int)((M + Cfg::BM - 1) / Cfg::BM);
  const int tiles_n = (int)((N + Cfg::BN - 1) / Cfg::BN);
  const int items = tiles_m * tiles_n * splits;
  const int a_tr = (int)round_up(M * (kpad / 16), 16);
  const int b_tr = (int)round_up(N * (kpad / 16), 16);
  // persistent grid: one slot per resident workgroup, a multiple of 8
  const int slots = std::max(8, (Cfg::OCC * cu_count()) / 8 * 8);
  const int grid = items <= slots ? items : slots;
  const bool staged = splits == 1 && !out_f32 && (N & 7) == 0 && M * N < ((int64_t)1 << 30);
  const uint16_t* kbias = splits > 1 ? nullptr : bias;
  if (staged)
    gemm_nv_kernel<Cfg, true><<<grid, Cfg::NT, 0, stream>>>(A, As, B, Bs, C, (int)M, (int)N, (int)kpad, kbias,
                                                            out_f32, tiles_m, tiles_n, a_tr, b_tr, splits, ws);
  else
    gemm_nv_kernel<Cfg, false><<<grid, Cfg::NT, 0, stream>>>(A, As, B, Bs, C, (int)M, (int)N, (int)kpad, kbias,
                                                             out_f32, tiles_m, tiles_n, a_tr, b_tr, splits, ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || splits == 1) return e;
  return launch_splitk_reduce(ws, splits, M, N, bias, C, out_f32, stream);
}

struct NvPlan {
  bool small;                                // 128x128 (two workgroups per CU) instead of 192x256
  int splits;
};

// Tile shape with the least work per CU lost to a partly filled last round:
// rounds of resident workgroups x tile area x workgroups per CU. 128x128 (4
// waves of 64x64, two workgroups per CU) fills the chip on the weight-
// gradient shapes (4096 x 1024 outputs, K = tokens), where 192x256 tiles
// leave most CUs idle; on ties the larger tiles win (less dequantization
// and LDS traffic per output).
static bool nv_small_tiles(int64_t M, int64_t N) {
  auto cost = [&](int bm, int bn, int occ) {
    const int64_t tiles = ((M + bm - 1) / bm) * ((N + bn - 1) / bn);
    const int64_t slots = std::max(8, occ * cu_count() / 8 * 8);
    return (double)((tiles + slots - 1) / slots) * bm * bn * occ;
  };
  return cost(128, 128, 2) < cost(192, 256, 1);
}

// Estimated time of a plan (us): rounds x stages per item x stage time (a
// 64-K stage of one workgroup with every CU busy, measured on MI355X on the
// training shapes; two 128x128 workgroups sharing a CU split its throughput,
// the dequantization being VALU and LDS work), plus the split-K partials
// (about 3 us + 0.25 us per MB, measured).
static double nv_plan_us(int64_t M, int64_t N, int64_t K, NvPlan p) {
  const int64_t nk = round_up(K, kAlignK) / 64;
  const int bm = p.small ? 128 : 192, bn = p.small ? 128 : 256, occ = p.small ? 2 : 1;
  const int64_t cus = cu_count();
  const int64_t items = ((M + bm - 1) / bm) * ((N + bn - 1) / bn) * p.splits;
  const int64_t rounds = (items + occ * cus - 1) / (occ * cus);
  const double stage = p.small ? 0.73 * (items > cus ? 2.0 : 1.0) : 1.7;
  double t = (double)rounds * (double)(2 * ((nk / 2 + p.splits - 1) / p.splits)) * stage;
  if (p.splits > 1) t += 3.0 + 0.25 * (double)(p.splits * 4) * (double)(M * N) / 1.0e6;
  return t;
}

// As for the MX GEMM: a split plan only if the workspace holds its partials
// and the estimate beats the unsplit plan by 5%.
static NvPlan nv_choose_plan(int64_t M, int64_t N, int64_t K, int64_t ws_bytes) {
  NvPlan best{nv_small_tiles(M, N), 1};
  if (ws_bytes < 2 * M * N * 4) return best;
  double best_us = nv_plan_us(M, N, K, best);
  const int64_t pairs = round_up(K, kAlignK) / 128;
  for (bool small : {false, true}) {
    const int bm = small ? 128 : 192, bn = small ? 128 : 256, occ = small ? 2 : 1;
    const int64_t tiles = ((M + bm - 1) / bm) * ((N + bn - 1) / bn);
    for (int s = 2; s <= 16 && tiles * s <= occ * cu_count() && pairs >= 2 * s && s * M * N * 4 <= ws_bytes; ++s) {
      const double us = nv_plan_us(M, N, K, NvPlan{small, s});
      if (us < 0.95 * best_us) {
        best_us = us;
        best = NvPlan{small, s};
      }
    }
  }
  return best;
}

int64_t gemm_nvfp4_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  const NvPlan p = nv_choose_plan(M, N, K, INT64_MAX);
  return p.splits > 1 ? (int64_t)p.splits * M * N * 4 : 0;
}

const char* plan_gemm_nvfp4(int64_t M, int64_t N, int64_t K, int64_t ws_bytes) {
  static const char* names[2] = {"gemm_nv_kernel<nvfp4, 192x256>", "gemm_nv_kernel<nvfp4, 128x128>"};
  static char split_names[2][17][48];
  static std::once_flag once;
  std::call_once(once, [] {
    for (int t = 0; t < 2; ++t)
      for (int sp = 2; sp <= 16; ++sp) snprintf(split_names[t][sp], 48, "%s+splitk%d", names[t], sp);
  });
  const NvPlan p = nv_choose_plan(M, N, K, ws_bytes);
  return p.splits > 1 ? split_names[p.small][p.splits] : names[p.small];
}

hipError_t launch_gemm_nvfp4(const uint8_t* A, const uint8_t* As, const uint8_t* B, const uint8_t* Bs, void* C,
                             int64_t M, int64_t N, int64_t K, const uint16_t* bias, int out_f32, float* ws,
                             int64_t ws_bytes, hipStream_t stream) {
  const NvPlan p = nv_choose_plan(M, N, K, ws != nullptr ? ws_bytes : 0);
  if (p.small)
    return run_nv<NvCfg<128, 128, 2, 2, 2>>(A, As, B, Bs, C, M, N, K, bias, out_f32, p.splits, ws, stream);
  return run_nv<NvCfg<192, 256, 2, 4, 1>>(A, As, B, Bs, C, M, N, K, bias, out_f32, p.splits, ws, stream);
}

}  // namespace mx
