// MXFP8 / MXFP4 GEMM on CDNA4's scaled matrix cores, and NVFP4 on its fp16
// matrix cores:
//   C[M, N] = sum_k (a_k 2^ea)(b_k 2^eb) (+ bias[n]),  fp32 accumulate
//   (NVFP4: s_tA s_tB sum_k (a_k dA)(b_k dB) (+ bias[n])).
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
// NVFP4 (section 2: E2M1 + E4M3 per 1x16 + an fp32 scale per tensor;
// sections 5.3-5.5 use it for training's dgrad / wgrad GEMMs) runs on the
// same data path: its codes are staged exactly like MXFP4's, its scale bytes
// (one per 16 K) like MX scales, but an E4M3 scale is no power of two, so the
// scaled instructions cannot take it. Each wave instead folds the scale into
// its fp4 fragments, exactly, as fp16 (an E2M1 value times an E4M3 scale has
// at most 6 significant bits and lies in [2^-10, 2688], inside fp16's normal
// range; the product of two such values has at most 12 bits, exact in the
// fp32 accumulator) and runs V_MFMA_F32_32X32X16_F16 (fp16 operand: lane l
// holds row l % 32, K 8 (l / 32) .. + 7, measured on gfx950). s_tA s_tB
// multiplies the fp32 sums before the epilogue. This path's roof is the fp16
// matrix rate, and the conversions are VALU work beside it.
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
// Persistent schedule. One workgroup per CU (two for the small tile) walks
// tiles blockIdx.x, blockIdx.x + gridDim.x, ...; tiles are renumbered so each
// XCD (own L2) works through a contiguous range, in groups of 8 tile-rows.
// The copy cursor runs one K-stage ahead of the compute cursor across tile
// boundaries, so the next tile's first stage is in flight while the current
// tile finishes and while its epilogue runs.
//
// Data movement. A K-stage is 128 bytes of codes per row (128 fp8 / 256 fp4
// elements); two stages are double-buffered in LDS. Scales travel in chunks
// of 16 bytes per row (16 blocks, i.e. 512 K elements), double-buffered in
// their own LDS slots. Both are copied global -> LDS with
// buffer_load ... lds (16 bytes per lane; rows past the tensor read as
// zero), issued from inline assembly with the kernel's own waits, so the
// compiler does not stall every LDS read on copies that are still in
// flight. A stage's 1-KB wave copies cover 8 rows x 128 bytes, the shape the
// L2 serves fastest. Code rows are XOR-swizzled in 16-byte chunks so the 8
// lanes of one LDS read cycle hit distinct banks. Inside a stage each wave
// reads the next A fragment (and the next sub-step's B fragments) while the
// matrix instructions of the current one run.
//
// Who issues the copies. A wave issues its instructions in order, so one
// stalled on a copy (the load path accepts about 64 bytes per clock per CU)
// issues no matrix instruction meanwhile. In MXFP8 only waves 0-3 copy, all
// of a stage's code copies in one burst after the stage barrier, while
// waves 4-7 (one per SIMD) go straight to their fragment reads and matrix
// instructions: 6-8% faster than every wave copying on every ViT shape
// (192 x 256 and 256 x 256 alike), with outputs unchanged. MXFP4 (twice the
// flops per copied byte) measured no difference and keeps every wave copying,
// spread over the stage's matrix-instruction blocks.
//
// Epilogue. For bf16 output with one workgroup per CU each wave stages its
// own sub-tile through an LDS area of its own, 32 rows at a time: bias
// added, rounded to bf16, written with 16-byte chunks XOR-swizzled by row,
// read back as whole row segments (128 or 256 bytes) and stored with
// range-checked buffer stores (rows and columns outside C are dropped by the
// buffer's bounds). No workgroup barrier separates the waves there, which
// measured 2-8% faster on the ViT shapes than staging whole tile rows
// through the stage buffer; the two-workgroup 128 x 128 tile and the
// quantized output keep that tile-row staging. Every wave issues the same
// number of stores, so the next tile's first wait lets exactly those stores
// stay in flight. fp32 output (or N % 8 != 0) is stored straight from
// registers and drained before the next tile.
#include "gemm_common.h"
#include "mx_launch.h"

#include <algorithm>
#include <cstdio>
#include <mutex>

namespace mx {

// Table of RNE_bf16(GELU(h)) for the quantized-output epilogue: bf16 h with
// biased exponent 111 .. 130 (|h| in [2^-16, 16)), both signs.
constexpr int kGeluTabExp0 = 111, kGeluTabExps = 20;
constexpr int kGeluTabEntries = 2 * kGeluTabExps * 128;     // sign x exponent x mantissa
constexpr int kGeluTabBytes = 2 * kGeluTabEntries;           // bf16 entries

// EPI_ = 0: C (bf16 / fp32) out. EPI_ = 1: the output is GELU-activated and
// quantized along N in the operand format (fc1 -> fc2's A operand).
// PF_: L2 prefetch (see the kernel's `prefetch`). CPW_: the number of waves
// that issue the stage's code copies (0: every wave).
template <int FMT_, int BM_, int BN_, int WAVES_M_, int WAVES_N_, int OCC_, bool SPREAD_, int EPI_ = 0, bool PF_ = false,
          int CPW_ = 0>
struct MxCfg {
  static constexpr int FMT = FMT_, BM = BM_, BN = BN_, WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
  static constexpr int EPI = EPI_;
  static constexpr bool PF = PF_;
  static constexpr int PF_OPS = PF_ ? 1 : 0;                  // prefetch instructions per wave per stage
  static constexpr int OCC = OCC_;                            // workgroups per CU (LDS-limited)
  static constexpr bool SPREAD = SPREAD_;                     // spread code copies over the stage
  static constexpr int NT = 64 * WAVES_M * WAVES_N, NW = NT / 64;
  static constexpr int RB = 128;                              // code bytes per row per stage
  static constexpr int CH = RB / 16;                          // 16-byte chunks per row
  static constexpr int KS = (FMT == FMT_MXFP8) ? RB : 2 * RB; // K elements per stage
  static constexpr int SUB = KS / 64;                         // 64-K sub-steps per stage
  // K elements per scale byte: MX blocks of 32, NVFP4 blocks of 16
  static constexpr int BSZ = (FMT == FMT_NVFP4) ? 16 : 32;
  static constexpr int SPC = 16 * BSZ / KS;                   // stages per 16-byte scale chunk
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  static constexpr int FM = WM / 32, FN = WN / 32;
  static constexpr int STAGE = (BM + BN) * RB;                 // code bytes per stage
  static constexpr int SCHUNK = (BM + BN) * 16;                // bytes per scale slot
  static constexpr int BIAS_OFF = 2 * STAGE + 2 * SCHUNK;     // two 1-KB bias slots (tile parity)
  // quantized output: RNE_bf16(GELU(h)) of every bf16 h with |h| in
  // [2^-16, 16) as a table in LDS, where the LDS budget leaves room for it
  static constexpr int GTAB_OFF = BIAS_OFF + 2 * 1024;
  static constexpr bool GTAB = EPI_ == 1 && (GTAB_OFF + kGeluTabBytes) * OCC_ <= 160 * 1024;
  // bf16 C out with one workgroup per CU: each wave stages 32 rows of its
  // WM x WN sub-tile at a time in a WAREA-byte area of its own and stores
  // them as whole 2 WN-byte row segments, with no workgroup barrier between
  // the waves (mx_epilogue_wave). The areas sit past the bias slots where
  // the LDS has room for them (WAVE_OWN), otherwise in the stage buffer just
  // consumed, after one barrier.
  static constexpr int WAREA = 64 * WN;
  static constexpr bool WAVE_EPI = EPI_ == 0 && OCC_ == 1 && (WN == 64 || WN == 128) && NW * WAREA <= STAGE;
  static constexpr bool WAVE_OWN = WAVE_EPI && GTAB_OFF + NW * WAREA <= 160 * 1024;
  static constexpr int WAREA_OFF = GTAB_OFF;
  static constexpr int LDS = GTAB_OFF + (GTAB ? kGeluTabBytes : 0) + (WAVE_OWN ? NW * WAREA : 0);
  static constexpr int CPW = CPW_ ? CPW_ : NW;                // copy waves: waves 0 .. CPW - 1
  static constexpr int CODE_DMA = STAGE / 1024 / CPW;         // 1-KB code copies per copy wave per stage
  static constexpr int SCALE_COPIES = (BM + BN) / 64;         // 1-KB copies per scale chunk
  static constexpr int SCALE_DMA = (SCALE_COPIES + NW - 1) / NW;  // per wave (some may be idle)
  static constexpr int MFMA_FMT = (FMT == FMT_MXFP8) ? 0 : 4;  // E4M3 / E2M1 operand selector
  // NVFP4: the software-pipelined stage where a SIMD runs one wave (no other
  // wave's conversions to fill its matrix instructions' shadow), with
  // NV_VALU VALU instructions scheduled after each fp16 matrix instruction
  static constexpr bool NV_PIPED = NW * OCC == 4;
  static constexpr int NV_VALU = 6;
  static constexpr int CPR = BN / 8;                          // 16-byte bf16 chunks per C row
  static constexpr int EPI_STORES = WM * CPR / NT;            // stores per thread per epilogue pass
  // stores per thread per tile: one per 16-byte chunk of C, or a code store
  // and a scale-byte store per chunk of the quantized output
  static constexpr int EPI_TOTAL = WAVE_EPI ? FM * (WN / 16) : WAVES_M * EPI_STORES * (EPI_ == 1 ? 2 : 1);
  static_assert(CODE_DMA * 1024 * CPW == STAGE, "code copies must split evenly over the copy waves");
  static_assert(BM % (8 * CPW) == 0, "every copy wave's copies split into A rows, then B rows");
  static_assert(CPW % 2 == 0 && CPW <= NW, "copy blocks of one wave share the parity of the wave");
  static_assert(BM % 64 == 0 && BN % 64 == 0 && WM % 32 == 0 && WN % 32 == 0, "tile");
  static_assert(LDS * OCC <= 160 * 1024, "LDS");
  static_assert(WM * BN * 2 <= STAGE, "one wave-row of the bf16 C tile must fit in a stage buffer");
  static_assert(EPI_STORES * NT == WM * CPR, "epilogue stores must split evenly over threads");
  static_assert(EPI_TOTAL <= 48, "stores left in flight must stay within the vmcnt range");
  static_assert(BN * 2 <= 1024, "a tile's bias must fit one bias slot");
  static_assert(!PF_ || BN * 2 <= 512, "the prefetch's dummy LDS target is the second half of bias slot 0");
};

// fp8: A or B fragment of sub-step t for tile row `row` of a stage: 16-byte
// chunks 4t+g and 4t+2+g (K 16g.. and 32+16g.. of the sub-step).
// fp4: chunk 2t+g (K 32g.. of the sub-step) in the first 4 registers.
template <class Cfg>
__device__ __forceinline__ v8i load_frag(const uint8_t* st, int row, int t, int g) {
  const uint8_t* p = st + row * Cfg::RB;
  if (Cfg::FMT == FMT_MXFP8) {
    const uint4 lo = *reinterpret_cast<const uint4*>(p + swz(row, 4 * t + g) * 16);
    const uint4 hi = *reinterpret_cast<const uint4*>(p + swz(row, 4 * t + 2 + g) * 16);
    return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  } else {
    const uint4 lo = *reinterpret_cast<const uint4*>(p + swz(row, 2 * t + g) * 16);
    return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, 0, 0, 0, 0};
  }
}

// Scale bytes of one stage for tile row `row`, shifted right by 8g so that
// the block sub-step t needs from this lane (2t + g within the stage) sits
// in byte 2t (fp8: one word, 4 blocks) or byte 2(t%2) of word t/2 (fp4: 8
// blocks).
template <class Cfg>
__device__ __forceinline__ uint2 load_stage_scales(const uint8_t* sc, int row, int sj, int g) {
  if (Cfg::FMT == FMT_MXFP8) {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(sc + row * 16 + 4 * sj);
    return make_uint2(w >> (8 * g), 0u);
  } else {
    const uint2 w = *reinterpret_cast<const uint2*>(sc + row * 16 + 8 * sj);
    return make_uint2(w.x >> (8 * g), w.y >> (8 * g));
  }
}

template <class Cfg>
__device__ __forceinline__ int substep_scale(uint2 s, int t) {
  const uint32_t w = (Cfg::FMT == FMT_MXFP8 || t < 2) ? s.x : s.y;
  return (int)(w >> (16 * (t & 1)));
}

// All sub-steps of one stage for one wave. after_block(i) runs after the
// matrix instructions of the i-th (sub-step, A fragment) block, i = 0 ..
// SUB * FM - 1 (a compile-time value once unrolled): the kernel spreads the
// next stage's copies over these points instead of issuing them in a burst.
template <class Cfg, class AfterBlock>
__device__ __forceinline__ void mma_stage(v16f (&acc)[Cfg::FM][Cfg::FN], const uint8_t* st, const uint8_t* sc,
                                          int sj, int g, int ra, int rb, AfterBlock&& after_block) {
  constexpr int FM = Cfg::FM, FN = Cfg::FN, SUB = Cfg::SUB;
  uint2 sa[FM], sb[FN];
#pragma unroll
  for (int f = 0; f < FN; ++f) sb[f] = load_stage_scales<Cfg>(sc, Cfg::BM + rb + 32 * f, sj, g);
#pragma unroll
  for (int f = 0; f < FM; ++f) sa[f] = load_stage_scales<Cfg>(sc, ra + 32 * f, sj, g);
  v8i b_cur[FN], b_nxt[FN], a_cur, a_nxt;
#pragma unroll
  for (int f = 0; f < FN; ++f) b_cur[f] = load_frag<Cfg>(st, Cfg::BM + rb + 32 * f, 0, g);
  a_cur = load_frag<Cfg>(st, ra, 0, g);
#pragma unroll
  for (int t = 0; t < SUB; ++t) {
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      if (fm + 1 < FM) a_nxt = load_frag<Cfg>(st, ra + 32 * (fm + 1), t, g);
      else if (t + 1 < SUB) a_nxt = load_frag<Cfg>(st, ra, t + 1, g);
      if (fm == 0 && t + 1 < SUB) {
#pragma unroll
        for (int f = 0; f < FN; ++f) b_nxt[f] = load_frag<Cfg>(st, Cfg::BM + rb + 32 * f, t + 1, g);
      }
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
        acc[fm][fn] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            b_cur[fn], a_cur, acc[fm][fn], Cfg::MFMA_FMT, Cfg::MFMA_FMT, 0, substep_scale<Cfg>(sb[fn], t), 0,
            substep_scale<Cfg>(sa[fm], t));
      after_block(t * FM + fm);
      if (fm + 1 < FM || t + 1 < SUB) a_cur = a_nxt;
    }
    if (t + 1 < SUB) {
#pragma unroll
      for (int f = 0; f < FN; ++f) b_cur[f] = b_nxt[f];
    }
  }
}

// NVFP4 (E2M1 codes with an E4M3 scale per 16 elements): the E4M3 scale is
// not a power of two, so the scaled matrix instructions cannot take it;
// instead each wave dequantizes its fp4 fragments, read from the stage as
// for MXFP4, exactly to fp16 (nv_dequant8: an element times its scale has at
// most 6 significant bits within fp16's normal range) and runs
// V_MFMA_F32_32X32X16_F16. The fp4 fragment of sub-step t holds K 64t + 32g
// .. + 31 of its row (dword k: K 64t + 32g + 8k ..), so its 4 dwords feed 4
// fp16 instructions: instruction k pairs, in A and B alike, K 64t + 8k + i
// (lanes g = 0) and 64t + 32 + 8k + i (lanes g = 1), i < 8; over k = 0..3
// that is every K of the sub-step once. The scale of K 64t + 32g + 8k is
// byte 4t + 2g + k / 2 of the row's 16 scale bytes of the stage.

// E4M3 byte j (0 or 1) of the 16-bit value in the low half of `s`, placed as
// fp16 bits into both halves: 2^-8 times its value (the exponent rebiased by
// 8, E4M3 subnormals as fp16 subnormals); the factor 2^8 is carried by the
// element conversion.
template <int J>
__device__ __forceinline__ uint32_t nv_scale_h2(uint32_t s) {
  constexpr uint32_t sel = 0x0C000C00u | (J << 16) | J;
  return __builtin_amdgcn_perm(0u, s & 0x7F7F7F7Fu, sel) << 7;
}

typedef _Float16 v8h_t __attribute__((ext_vector_type(8)));
typedef _Float16 v2h_t __attribute__((ext_vector_type(2)));

// 8 E2M1 codes (element j in nibble j) times an fp16 scale pair -> 8 fp16:
// the hardware conversion at scale operand 2^8 (only its exponent is used),
// then one packed multiply per pair.
__device__ __forceinline__ v8h_t nv_dequant8(uint32_t x, uint32_t scale_h2) {
  const v2h_t s = __builtin_bit_cast(v2h_t, scale_h2);
  const v2h_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 256.0f, 0) * s;
  const v2h_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 256.0f, 1) * s;
  const v2h_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 256.0f, 2) * s;
  const v2h_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 256.0f, 3) * s;
  return v8h_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// Dequantized fragment: 4 x 8 fp16 from the fp4 fragment `f` (first 4
// dwords) with the scale bytes of its two blocks in the low 16 bits of `s`.
__device__ __forceinline__ void nv_dequant_frag(const v8i& f, uint32_t s, v8h_t (&out)[4]) {
  const uint32_t s0 = nv_scale_h2<0>(s), s1 = nv_scale_h2<1>(s);
  out[0] = nv_dequant8((uint32_t)f[0], s0);
  out[1] = nv_dequant8((uint32_t)f[1], s0);
  out[2] = nv_dequant8((uint32_t)f[2], s1);
  out[3] = nv_dequant8((uint32_t)f[3], s1);
}

// This lane's two scale bytes of sub-step t for tile row `row` (in the low
// 16 bits): bytes 4t + 2g, 4t + 2g + 1 of the row's 16 bytes of the stage.
template <class Cfg>
__device__ __forceinline__ uint32_t nv_substep_scales(const uint8_t* sc, int row, int t, int g) {
  return *reinterpret_cast<const uint32_t*>(sc + row * 16 + 4 * t) >> (16 * g);
}

template <class Cfg, class AfterBlock>
__device__ __forceinline__ void nv_mma_stage(v16f (&acc)[Cfg::FM][Cfg::FN], const uint8_t* st, const uint8_t* sc,
                                             int g, int ra, int rb, AfterBlock&& after_block) {
  constexpr int FM = Cfg::FM, FN = Cfg::FN, SUB = Cfg::SUB;
  v8i b_cur[FN], b_nxt[FN], a_cur, a_nxt;
#pragma unroll
  for (int f = 0; f < FN; ++f) b_cur[f] = load_frag<Cfg>(st, Cfg::BM + rb + 32 * f, 0, g);
  a_cur = load_frag<Cfg>(st, ra, 0, g);
#pragma unroll
  for (int t = 0; t < SUB; ++t) {
    v8h_t bd[FN][4];
#pragma unroll
    for (int f = 0; f < FN; ++f) nv_dequant_frag(b_cur[f], nv_substep_scales<Cfg>(sc, Cfg::BM + rb + 32 * f, t, g), bd[f]);
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      if (fm + 1 < FM) a_nxt = load_frag<Cfg>(st, ra + 32 * (fm + 1), t, g);
      else if (t + 1 < SUB) a_nxt = load_frag<Cfg>(st, ra, t + 1, g);
      if (fm == 0 && t + 1 < SUB) {
#pragma unroll
        for (int f = 0; f < FN; ++f) b_nxt[f] = load_frag<Cfg>(st, Cfg::BM + rb + 32 * f, t + 1, g);
      }
      v8h_t ad[4];
      nv_dequant_frag(a_cur, nv_substep_scales<Cfg>(sc, ra + 32 * fm, t, g), ad);
#pragma unroll
      for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
          acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bd[fn][k], ad[k], acc[fm][fn], 0, 0, 0);
      after_block(t * FM + fm);
      if (fm + 1 < FM || t + 1 < SUB) a_cur = a_nxt;
    }
    if (t + 1 < SUB) {
#pragma unroll
      for (int f = 0; f < FN; ++f) b_cur[f] = b_nxt[f];
    }
  }
}

// The same stage, software-pipelined: the 4 * FN fp16 instructions of block
// (t, fm) use A dequantized during the previous block and B dequantized
// during sub-step t - 1, so the conversions that run beside them (the next
// block's A fragment and a share of sub-step t + 1's B fragments) do not
// feed them, and the schedule alternates one matrix instruction with a few
// conversions. B's raw fragments for t + 1 are read from LDS at block
// (t, 0) and converted in the blocks fm >= 1 (all of them at fm = 0 when
// FM = 1); A's raw fragment is read two blocks ahead.
template <class Cfg, class AfterBlock>
__device__ __forceinline__ void nv_mma_stage_piped(v16f (&acc)[Cfg::FM][Cfg::FN], const uint8_t* st,
                                                   const uint8_t* sc, int g, int ra, int rb,
                                                   AfterBlock&& after_block) {
  constexpr int FM = Cfg::FM, FN = Cfg::FN, SUB = Cfg::SUB, NB = SUB * FM;
  auto a_frag = [&](int b) { return load_frag<Cfg>(st, ra + 32 * (b % FM), b / FM, g); };
  auto a_scales = [&](int b) { return nv_substep_scales<Cfg>(sc, ra + 32 * (b % FM), b / FM, g); };
  auto b_scales = [&](int f, int t) { return nv_substep_scales<Cfg>(sc, Cfg::BM + rb + 32 * f, t, g); };
  auto b_block = [](int f) { return FM > 1 ? 1 + f * (FM - 1) / FN : 0; };   // block fm that converts B frag f
  v8i b_raw[FN], a_raw1, a_raw2;
  uint32_t b_sc[FN], a_sc1, a_sc2;
  v8h_t bd[FN][4], bdn[FN][4], ad[4], adn[4];
#pragma unroll
  for (int f = 0; f < FN; ++f) {
    b_raw[f] = load_frag<Cfg>(st, Cfg::BM + rb + 32 * f, 0, g);
    b_sc[f] = b_scales(f, 0);
  }
  const v8i a_raw0 = a_frag(0);
  const uint32_t a_sc0 = a_scales(0);
  if (NB > 1) {
    a_raw1 = a_frag(1);
    a_sc1 = a_scales(1);
  }
  // before the first instruction only B fragment 0 and A are converted; the
  // other B fragments of sub-step 0 are converted beside block 0's
  // instructions, which run fragment by fragment (each accumulator still
  // takes its 4 instructions in K order)
  nv_dequant_frag(b_raw[0], b_sc[0], bd[0]);
  nv_dequant_frag(a_raw0, a_sc0, ad);
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int t = b / FM, fm = b % FM;
    if (b == 0) {
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        if (fn + 1 < FN) nv_dequant_frag(b_raw[fn + 1], b_sc[fn + 1], bd[fn + 1]);
#pragma unroll
        for (int k = 0; k < 4; ++k)
          acc[0][fn] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bd[fn][k], ad[k], acc[0][fn], 0, 0, 0);
      }
    }
    if (b + 2 < NB) {
      a_raw2 = a_frag(b + 2);
      a_sc2 = a_scales(b + 2);
    }
    if (fm == 0 && t + 1 < SUB) {
#pragma unroll
      for (int f = 0; f < FN; ++f) {
        b_raw[f] = load_frag<Cfg>(st, Cfg::BM + rb + 32 * f, t + 1, g);
        b_sc[f] = b_scales(f, t + 1);
      }
    }
    if (b + 1 < NB) nv_dequant_frag(a_raw1, a_sc1, adn);
    if (t + 1 < SUB) {
#pragma unroll
      for (int f = 0; f < FN; ++f)
        if (b_block(f) == fm) nv_dequant_frag(b_raw[f], b_sc[f], bdn[f]);
    }
    if (b > 0) {
#pragma unroll
      for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
          acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bd[fn][k], ad[k], acc[fm][fn], 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4 * FN; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);             // one matrix instruction
      __builtin_amdgcn_sched_group_barrier(0x002, Cfg::NV_VALU, 0);  // then a few VALU
    }
    after_block(b);
#pragma unroll
    for (int k = 0; k < 4; ++k) ad[k] = adn[k];
    a_raw1 = a_raw2;
    a_sc1 = a_sc2;
    if (fm == FM - 1 && t + 1 < SUB) {
#pragma unroll
      for (int f = 0; f < FN; ++f)
#pragma unroll
        for (int k = 0; k < 4; ++k) bd[f][k] = bdn[f][k];
    }
  }
}

// GELU(h) = h Phi(h) in fp32. With z = |h|, Q(z) = Phi(-z) = exp(-z^2/2) R(z)
// and R a degree-7 polynomial in t = 1 / (1 + 0.35 z), fitted for relative
// error on z in [0, 14] (csrc/gelu_fit.py derives the constants): Q's
// relative error is below 2^-20 in this fp32 evaluation, plus the exp2
// argument's rounding in the far tail (about 2^-16 at z = 13). Phi(h) is
// 1 - Q for h >= 0 and Q for h < 0. One v_rcp_f32, one v_exp_f32 and about a
// dozen multiply-adds, against several dozen operations for erfcf. Far out
// (z in the hundreds, t near 0) the polynomial tends to its negative constant
// term while the exp2 factor has long flushed to zero; R is clamped at 0 so
// that Q stays +0 there and the result keeps the sign of h (-0 for h < 0).
__device__ __forceinline__ float gelu_f32(float h) {
  const float z = fabsf(h);
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3499999940395355f, z, 1.0f));
  float r = 0.04894101619720459f;
  r = fmaf(r, t, -0.2021145224571228f);
  r = fmaf(r, t, 0.24063429236412048f);
  r = fmaf(r, t, -0.017018629238009453f);
  r = fmaf(r, t, 0.1559593826532364f);
  r = fmaf(r, t, 0.13335564732551575f);
  r = fmaf(r, t, 0.14027026295661926f);
  r = fmaf(r, t, -2.7310272344038822e-05f);
  const float q = __builtin_amdgcn_exp2f(-0.7213475204444817f * z * z) * fmaxf(r, 0.0f);   // 2^(-z^2 / (2 ln 2))
  return h >= 0.0f ? fmaf(-h, q, h) : h * q;
}

// RNE_bf16(GELU(h)) depends only on the 16 bits of the bf16 h. For |h| in
// [2^-16, 16), biased exponents 111 .. 130, it is read from a table that each
// workgroup fills once with gelu_f32, so the table path gives exactly the
// values gelu_f32 gives. Outside that range gelu_f32 rounds to closed forms:
// for exponents 2 .. 110 (|h| < 2^-16) GELU(h) = h/2 (1 + O(h)) and its fp32
// value is within 2^-15 of h/2 relative, so the bf16 result is h/2 exactly
// (the exponent minus one); for |h| >= 16 the tail factor exp2(-z^2 / (2 ln 2))
// underflows, so the result is h for h > 0 and -0 for h < 0 (the exact
// rounding of a negative value far below the bf16 range, which gelu_f32 gives
// there too). Only exponents 0, 1 (zero, values below 2^-125) and 255 are
// evaluated directly.
__device__ __forceinline__ uint32_t gelu_bf16_direct(uint32_t b) {
  return pack_bf16x2(gelu_f32(__uint_as_float(b << 16)), 0.0f) & 0xFFFFu;
}

__device__ __forceinline__ void fill_gelu_table(uint16_t* tab, int tid, int nt) {
  for (int i = tid; i < kGeluTabEntries; i += nt) {
    const uint32_t sign = (uint32_t)(i / (kGeluTabExps * 128)), r = (uint32_t)(i % (kGeluTabExps * 128));
    tab[i] = (uint16_t)gelu_bf16_direct((sign << 15) | ((kGeluTabExp0 + r / 128) << 7) | (r % 128));
  }
}

// RNE_bf16(GELU(h)) of the 8 bf16 values in w (element 2k in the low half of
// word k): table reads, the closed forms for lanes holding a value outside
// the table's range (selects, under one branch), and gelu_f32 for exponents 0,
// 1 and 255 (a second, rarer branch).
__device__ __forceinline__ void gelu_bf16_lookup8(const uint32_t (&words)[4], const uint16_t* tab, uint32_t (&gb)[8]) {
  constexpr uint32_t SPAN = kGeluTabExps * 128;
  uint32_t b[8];
  bool all_in = true;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    b[i] = (words[i / 2] >> (16 * (i % 2))) & 0xFFFFu;
    const uint32_t off = (b[i] & 0x7FFFu) - ((uint32_t)kGeluTabExp0 << 7);   // wraps for small |h|
    const bool in = off < SPAN;
    all_in = all_in && in;
    gb[i] = tab[in ? off + (b[i] >> 15) * SPAN : 0u];
  }
  if (!all_in) {
    bool special = false;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t e = (b[i] >> 7) & 0xFFu;
      const bool in = e - (uint32_t)kGeluTabExp0 < (uint32_t)kGeluTabExps;
      const bool small = e - 2u < (uint32_t)(kGeluTabExp0 - 2);                         // exponents 2 .. 110
      const bool big = e - (uint32_t)(kGeluTabExp0 + kGeluTabExps) < (uint32_t)(255 - kGeluTabExp0 - kGeluTabExps);
      const uint32_t closed = small ? b[i] - 0x80u : ((b[i] & 0x8000u) ? 0x8000u : b[i]);
      gb[i] = in ? gb[i] : closed;
      special = special || !(in || small || big);
    }
    if (special) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t e = (b[i] >> 7) & 0xFFu;
        if (e < 2u || e == 255u) gb[i] = gelu_bf16_direct(b[i]);
      }
    }
  }
}

// The quantized-output epilogue for one 16-byte chunk (8 consecutive
// columns n .. n + 7 of row m, bf16 h = RNE(acc + bias)): g = RNE_bf16(GELU(h))
// with gelu_f32 above, two values per V_CVT_PK_BF16_F32; the four lanes
// holding one 32-column block (adjacent lanes, one row) combine their amax
// bits; the MX scale byte and the codes follow as in the row quantizer. Every
// lane issues both stores (rows past M, columns past the output's K_pad and
// the scale bytes of three of the four lanes go to an offset past the buffer).
template <int FMT, bool TAB>
__device__ __forceinline__ void gelu_quant_store(uint4 w, bool scale_lane, bool in, int code_off, int scale_off,
                                                 __amdgpu_buffer_rsrc_t q_rs, __amdgpu_buffer_rsrc_t qs_rs,
                                                 const uint16_t* tab) {
  typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
  const uint32_t words[4] = {w.x, w.y, w.z, w.w};
  uint32_t gb[8];
  if constexpr (TAB) gelu_bf16_lookup8(words, tab, gb);
  float g[8];
  u16x2 mag = {0, 0};                        // largest |g| bits of each half
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    // element 2k in the low half of word k, 2k + 1 in the high half
    const uint32_t gp =
        TAB ? gb[2 * k] | (gb[2 * k + 1] << 16)
            : pack_bf16x2(gelu_f32(__uint_as_float(words[k] << 16)), gelu_f32(__uint_as_float(words[k] & 0xFFFF0000u)));
    g[2 * k] = __uint_as_float(gp << 16);
    g[2 * k + 1] = __uint_as_float(gp & 0xFFFF0000u);
    mag = __builtin_elementwise_max(mag, __builtin_bit_cast(u16x2, gp & 0x7FFF7FFFu));
  }
  uint32_t amax = max((uint32_t)mag.x, (uint32_t)mag.y);
  amax = max(amax, (uint32_t)__shfl_xor((int)amax, 1));
  amax = max(amax, (uint32_t)__shfl_xor((int)amax, 2));
  const uint32_t sb = (uint32_t)(mx_shared_exp(amax, FMT == FMT_MXFP8 ? 8 : 2) + 127);
  const int coff = in ? code_off : (int)0x80000000u;
  if constexpr (FMT == FMT_MXFP8) {
    const uint32_t lo = e4m3x4_scaled(g[0], g[1], g[2], g[3], sb), hi = e4m3x4_scaled(g[4], g[5], g[6], g[7], sb);
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(v2u, make_uint2(lo, hi)), q_rs, coff, 0, kStoreDeviceScope);
  } else {
    __builtin_amdgcn_raw_buffer_store_b32(e2m1x8_scaled(g, sb), q_rs, coff, 0, kStoreDeviceScope);
  }
  __builtin_amdgcn_raw_buffer_store_b8((uint8_t)sb, qs_rs, (in && scale_lane) ? scale_off : (int)0x80000000u, 0, kStoreDeviceScope);
}

// The epilogue of one tile. acc register 4q + v of fragment [fm][fn] is
// C[m][n + v] with m = m0 + wm WM + 32 fm + r32, n = n0 + wn WN + 32 fn + 8 q + 4 g;
// lds_bias holds the tile's BN bias values (zeros without a bias). With
// `staged` (bf16 C below 2 GiB with N % 8 == 0, or the quantized output) the
// tile goes through LDS one wave-row at a time, row lr of the staging area at
// row_ptr(lr) (BN * 2 bytes, free for the whole epilogue): bias added,
// rounded to bf16, written as 16-byte chunks XOR-swizzled by row, then stored
// as whole rows with range-checked buffer stores (every thread issues
// EPI_STORES of them, or twice that for the quantized output). Otherwise it
// is stored from registers (fp32, or the element-wise fallback).
template <class Cfg, class RowPtr>
__device__ __forceinline__ void mx_epilogue(const v16f (&acc)[Cfg::FM][Cfg::FN], const uint8_t* lds_bias, bool staged,
                                            int M, int N, int m0, int n0, int wm, int wn, int g, int r32, void* Ct,
                                            int out_f32_t, __amdgpu_buffer_rsrc_t c_rs, __amdgpu_buffer_rsrc_t q_rs,
                                            __amdgpu_buffer_rsrc_t qs_rs, int qld, int q_row_bytes,
                                            const uint16_t* gtab, RowPtr row_ptr) {
  constexpr int FM = Cfg::FM, FN = Cfg::FN, WM = Cfg::WM, WN = Cfg::WN, CPR = Cfg::CPR;
  auto bias4 = [&](int nl) -> uint2 { return *reinterpret_cast<const uint2*>(lds_bias + 2 * nl); };
  if (staged) {
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
              const float v0 = acc[fm][fn][4 * q + 0] + bf16_to_f32(bb[q].x & 0xFFFFu);
              const float v1 = acc[fm][fn][4 * q + 1] + bf16_to_f32(bb[q].x >> 16);
              const float v2 = acc[fm][fn][4 * q + 2] + bf16_to_f32(bb[q].y & 0xFFFFu);
              const float v3 = acc[fm][fn][4 * q + 3] + bf16_to_f32(bb[q].y >> 16);
              P[q][0] = pack_bf16x2(v0, v1);
              P[q][1] = pack_bf16x2(v2, v3);
            }
#pragma unroll
            for (int p = 0; p < 2; ++p) {
              // the two lanes holding adjacent 4-column runs of a row swap
              // halves across the wave: lane g = 0 ends with columns
              // 16p .. 16p + 7 of the fragment, lane g = 1 with 16p + 8 .. + 15
              const auto s0 = __builtin_amdgcn_permlane32_swap(P[2 * p][0], P[2 * p + 1][0], false, false);
              const auto s1 = __builtin_amdgcn_permlane32_swap(P[2 * p][1], P[2 * p + 1][1], false, false);
              const int chunk = (wn * WN + 32 * fn + 16 * p + 8 * g) >> 3;
              *reinterpret_cast<uint4*>(row_ptr(lr) + ((chunk ^ (lr & (CPR - 1))) * 16)) =
                  make_uint4(s0[0], s1[0], s0[1], s1[1]);
            }
          }
        }
      }
      block_sync();
      // LDS reads in batches of up to 4, each batch ahead of its stores
      constexpr int E = Cfg::EPI_STORES;
      constexpr int BATCH = E % 4 == 0 ? 4 : E % 3 == 0 ? 3 : E % 2 == 0 ? 2 : 1;
      static_assert(Cfg::EPI_STORES % BATCH == 0, "store batches");
#pragma unroll
      for (int j0 = 0; j0 < Cfg::EPI_STORES; j0 += BATCH) {
        uint4 w[BATCH];
#pragma unroll
        for (int j = 0; j < BATCH; ++j) {
          const int id = (int)threadIdx.x + (j0 + j) * Cfg::NT;
          const int row = id / CPR, c = id % CPR;
          w[j] = *reinterpret_cast<const uint4*>(row_ptr(row) + ((c ^ (row & (CPR - 1))) * 16));
        }
#pragma unroll
        for (int j = 0; j < BATCH; ++j) {
          const int id = (int)threadIdx.x + (j0 + j) * Cfg::NT;
          const int row = id / CPR, c = id % CPR;
          const int m = m0 + h * WM + row, n = n0 + 8 * c;
          if constexpr (Cfg::EPI == 0) {
            const int off = (m < M && n < N) ? (m * N + n) * 2 : (int)0x80000000u;
            __builtin_amdgcn_raw_buffer_store_b128(v4u{w[j].x, w[j].y, w[j].z, w[j].w}, c_rs, off, 0, kStoreDeviceScope);
          } else {
            gelu_quant_store<Cfg::FMT, Cfg::GTAB>(w[j], (c & 3) == 0, m < M && n < qld,
                                                  m * q_row_bytes + ((Cfg::FMT == FMT_MXFP8) ? n : n / 2),
                                                  m * (qld / 32) + n / 32, q_rs, qs_rs, gtab);
          }
        }
      }
    }
  } else {
    block_sync();
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
          v[0] = acc[fm][fn][4 * q + 0] + bf16_to_f32(bb.x & 0xFFFFu);
          v[1] = acc[fm][fn][4 * q + 1] + bf16_to_f32(bb.x >> 16);
          v[2] = acc[fm][fn][4 * q + 2] + bf16_to_f32(bb.y & 0xFFFFu);
          v[3] = acc[fm][fn][4 * q + 3] + bf16_to_f32(bb.y >> 16);
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
}

// The bf16 epilogue of one wave (Cfg::WAVE_EPI, C staged): for each of
// its FM fragment rows (32 rows of C), bias added and rounded to bf16 as in
// mx_epilogue, the 16-byte chunks written to the wave's area `wst` (rows of
// 2 WN bytes, chunks XOR-swizzled by row), read back as whole row segments
// (WN / 8 lanes per row) and stored with range-checked buffer stores: WN / 16
// stores per fragment row, FM WN / 16 = EPI_TOTAL in all. Only this wave
// touches its area, so no workgroup barrier is needed; the LDS returns a
// wave's reads and writes in order.
template <class Cfg, int POLICY>
__device__ __forceinline__ void mx_epilogue_wave(const v16f (&acc)[Cfg::FM][Cfg::FN], const uint8_t* lds_bias,
                                                 int M, int N, int m0, int n0, int wm, int wn, int g, int r32,
                                                 int lane, __amdgpu_buffer_rsrc_t c_rs, uint8_t* wst) {
  constexpr int FM = Cfg::FM, FN = Cfg::FN, WM = Cfg::WM, WN = Cfg::WN;
  constexpr int CW = WN / 8;            // 16-byte chunks per row segment
  constexpr int RPS = 64 / CW;          // rows per store
  static_assert(Cfg::WAVE_EPI && Cfg::WAREA == 32 * 2 * WN, "an area holds 32 row segments");
  auto bias4 = [&](int nl) -> uint2 { return *reinterpret_cast<const uint2*>(lds_bias + 2 * nl); };
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
      uint2 bb[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) bb[q] = bias4(wn * WN + 32 * fn + 8 * q + 4 * g);
      uint32_t P[4][2];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float v0 = acc[fm][fn][4 * q + 0] + bf16_to_f32(bb[q].x & 0xFFFFu);
        const float v1 = acc[fm][fn][4 * q + 1] + bf16_to_f32(bb[q].x >> 16);
        const float v2 = acc[fm][fn][4 * q + 2] + bf16_to_f32(bb[q].y & 0xFFFFu);
        const float v3 = acc[fm][fn][4 * q + 3] + bf16_to_f32(bb[q].y >> 16);
        P[q][0] = pack_bf16x2(v0, v1);
        P[q][1] = pack_bf16x2(v2, v3);
      }
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        // as in mx_epilogue: lane g = 0 ends with columns 16p .. 16p + 7 of
        // the fragment, lane g = 1 with 16p + 8 .. + 15 (chunk 4 fn + 2 p + g
        // of the wave's row segment)
        const auto s0 = __builtin_amdgcn_permlane32_swap(P[2 * p][0], P[2 * p + 1][0], false, false);
        const auto s1 = __builtin_amdgcn_permlane32_swap(P[2 * p][1], P[2 * p + 1][1], false, false);
        const int c = 4 * fn + 2 * p + g;
        *reinterpret_cast<uint4*>(wst + r32 * (2 * WN) + ((c ^ (r32 & (CW - 1))) * 16)) =
            make_uint4(s0[0], s1[0], s0[1], s1[1]);
      }
    }
#pragma unroll
    for (int k = 0; k < 32 / RPS; ++k) {
      const int row = RPS * k + lane / CW, c = lane % CW;
      const uint4 w = *reinterpret_cast<const uint4*>(wst + row * (2 * WN) + ((c ^ (row & (CW - 1))) * 16));
      const int m = m0 + wm * WM + 32 * fm + row, n = n0 + wn * WN + 8 * c;
      const int off = (m < M && n < N) ? (m * N + n) * 2 : (int)0x80000000u;
      __builtin_amdgcn_raw_buffer_store_b128(v4u{w.x, w.y, w.z, w.w}, c_rs, off, 0, POLICY);
    }
  }
}

template <class Cfg>
__global__ __launch_bounds__(Cfg::NT, Cfg::OCC) void gemm_mx_kernel(const uint8_t* __restrict__ A,
                                                          const uint8_t* __restrict__ As,
                                                          const uint8_t* __restrict__ B,
                                                          const uint8_t* __restrict__ Bs, void* __restrict__ C,
                                                          int M, int N, int kpad,
                                                          const uint16_t* __restrict__ bias, int out_f32,
                                                          int tiles_m, int tiles_n, uint8_t* __restrict__ qcodes,
                                                          uint8_t* __restrict__ qscales, int qld, int splits,
                                                          float* __restrict__ ws) {
  constexpr int BM = Cfg::BM, BN = Cfg::BN, WM = Cfg::WM, WN = Cfg::WN, FM = Cfg::FM, FN = Cfg::FN;
  constexpr int RB = Cfg::RB, CH = Cfg::CH, NW = Cfg::NW, CPR = Cfg::CPR;
  __shared__ __align__(16) uint8_t lds[Cfg::LDS];

  // work items: (tile, split) pairs; with splits > 1 an item covers the K
  // stages [k0, k1) of its split and writes an fp32 partial tile to
  // ws + split M N (no bias), summed by the split-K reduction afterwards
  const int tiles = tiles_m * tiles_n * splits;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / Cfg::WAVES_N, wn = wave % Cfg::WAVES_N;
  const int row_bytes = (Cfg::FMT == FMT_MXFP8) ? kpad : kpad / 2;
  const int srow = kpad / Cfg::BSZ;         // scale bytes per row
  // stages per tile; with fp4 a stage holds 256 elements while K_pad is a
  // multiple of 128, so the last stage may hold only its first 64 bytes
  const int nk = (kpad + Cfg::KS - 1) / Cfg::KS;
  const int g = lane >> 5, r32 = lane & 31;
  // bf16 output goes through LDS and 32-bit buffer offsets when C is below
  // 2 GiB; anything else is stored from registers with 64-bit addresses
  // (the quantized output always goes through LDS; the host ensures N % 8 == 0)
  const bool staged = Cfg::EPI == 1 || (splits == 1 && !out_f32 && (N & 7) == 0 && (int64_t)M * N < ((int64_t)1 << 30));
  // the coordinates and K-stage range of work item t
  auto item = [&](int t, int& tm, int& tn, int& sp, int& k0, int& k1) {
    int tnv;
    tile_coords(t, tiles_m, tiles_n * splits, tm, tnv);
    tn = tnv % tiles_n;
    sp = tnv / tiles_n;
    k0 = (sp * nk) / splits;
    k1 = ((sp + 1) * nk) / splits;
  };
  // quantized output: rows of qld elements (K_pad of N), codes and scale bytes
  const int q_row_bytes = (Cfg::FMT == FMT_MXFP8) ? qld : qld / 2;
  const __amdgpu_buffer_rsrc_t q_rs =
      __builtin_amdgcn_make_buffer_rsrc(qcodes, (short)0, Cfg::EPI == 1 ? M * q_row_bytes : 0, 0x00020000);
  const __amdgpu_buffer_rsrc_t qs_rs =
      __builtin_amdgcn_make_buffer_rsrc(qscales, (short)0, Cfg::EPI == 1 ? M * (qld / 32) : 0, 0x00020000);

  const v4u a_rs = buffer_rsrc(A, (uint32_t)(M * row_bytes));
  const v4u b_rs = buffer_rsrc(B, (uint32_t)(N * row_bytes));
  const v4u as_rs = buffer_rsrc(As, (uint32_t)(M * srow));
  const v4u bs_rs = buffer_rsrc(Bs, (uint32_t)(N * srow));
  const __amdgpu_buffer_rsrc_t c_rs =
      __builtin_amdgcn_make_buffer_rsrc(C, (short)0, staged ? M * N * 2 : 0, 0x00020000);
  // a 16-byte aligned bias with N % 8 == 0 is copied to LDS with each tile's
  // first stage; otherwise the epilogue reads it from global memory
  const bool bias_dma = bias != nullptr && (N & 7) == 0 && (reinterpret_cast<uintptr_t>(bias) & 15) == 0;
  const v4u bias_rs = buffer_rsrc(bias, bias_dma ? (uint32_t)(N * 2) : 0u);
  const uint32_t lds_base = (uint32_t)reinterpret_cast<uintptr_t>(lds);
  const uint32_t sc_base = lds_base + 2 * Cfg::STAGE;

  // Code copy j of copy wave `wave` (< CPW) fills the stage's 1-KB block
  // J = j CPW + wave: rows 8 J .. 8 J + 7 of [A rows, B rows] (A iff
  // 8 J < BM, uniform per copy), lane l taking row 8 J + l / 8 and logical
  // chunk l % 8, which lands at swizzled position (l % 8) ^ (row / 2 % 8):
  // with CPW even, (row / 2) % 8 = (4 (wave % 2) + l / 16) % 8
  const uint32_t code_byte = (uint32_t)(((lane & 7) ^ ((4 * (wave & 1) + (lane >> 4)) & 7)) * 16);
  // this lane's row within its wave's first copy: 8 wave + lane / 8
  // (offsets of rows past the operand may wrap; they only feed rows and
  // columns of C that are never stored, and every read is range-checked)
  const uint32_t code_lane = (uint32_t)(8 * wave + (lane >> 3)) * (uint32_t)row_bytes + code_byte;
  const uint32_t copy_stride = (uint32_t)(8 * Cfg::CPW) * (uint32_t)row_bytes;   // rows between copy j and j + 1
  const bool copy_wave = wave < Cfg::CPW;
  // Scale copy j of this wave fills rows 64 J .. 64 J + 63 of [A rows, B rows]
  // with 16 bytes each (copies J >= SCALE_COPIES are skipped). When K_pad is
  // not a multiple of 512 the last chunk of the last row runs past the end of
  // the scale buffer; the buffer range check applies to each dword of a load,
  // the scalar offset included (probed on gfx950), so those dwords read as
  // zero and nothing past the buffer is touched.
  const uint32_t scale_lane = (uint32_t)lane * (uint32_t)srow;

  // copy cursor: tile lt (rows m0l / n0l), its stage lks; lgs / lgc count
  // stages / scale chunks issued so far (they pick the LDS buffer and slot)
  // copy cursor: tile lt (first rows m0l / n0l; a_base / b_base are the byte
  // offsets of its A rows and of its B rows shifted down by BM), its stage
  // lks; lgs / lgc / ltc count stages / scale chunks / tiles issued so far
  int lt = blockIdx.x, lks = 0, lk0 = 0, lk1 = nk, lgs = 0, lgc = 0, ltc = 0, m0l = 0, n0l = 0;
  uint32_t a_base = 0, b_base = 0;
  auto set_copy_tile = [&](int t) {
    int tm, tn, sp;
    item(t, tm, tn, sp, lk0, lk1);
    lks = lk0;
    m0l = tm * BM;
    n0l = tn * BN;
    a_base = (uint32_t)m0l * (uint32_t)row_bytes;
    b_base = (uint32_t)(n0l - BM) * (uint32_t)row_bytes;
  };
  // Copies of the copy cursor's stage. open_copy_stage issues the tile's bias
  // (first stage) and a new scale chunk (every SPC stages) and fixes where
  // the stage's code copies go; issue_code(j) issues code copy j of this
  // wave; close_copy_stage advances the cursor.
  uint32_t cp_st = 0, cp_soff = 0;
  bool cp_in_row = false;
  auto open_copy_stage = [&]() {
    if (lks == lk0 && bias_dma && wave == 0) {  // the tile's bias, into bias slot ltc & 1
      const uint32_t voff = lane < BN / 8 ? (uint32_t)((n0l + 8 * lane) * 2) : 0x80000000u;
      dma16(bias_rs, lds_base + (uint32_t)(Cfg::BIAS_OFF + (ltc & 1) * 1024), voff, 0u);
    }
    if (lks == lk0 || lks % Cfg::SPC == 0) {  // first stage of a scale chunk: bring the chunk too
      const uint32_t dst = sc_base + (uint32_t)((lgc & 1) * Cfg::SCHUNK);
      const uint32_t soff = (uint32_t)(16 * (lks / Cfg::SPC));
#pragma unroll
      for (int j = 0; j < Cfg::SCALE_DMA; ++j) {
        const int J = j * NW + wave;
        if (J < Cfg::SCALE_COPIES) {
          const bool isa = J * 64 < BM;
          const int row0 = (isa ? m0l : n0l - BM) + J * 64;
          dma16(isa ? as_rs : bs_rs, dst + (uint32_t)(J * 1024), scale_lane + (uint32_t)row0 * (uint32_t)srow, soff);
        }
      }
      ++lgc;
    }
    cp_st = lds_base + (uint32_t)((lgs & 1) * Cfg::STAGE);
    cp_soff = (uint32_t)(lks * RB);
    // bytes past the end of the row (last fp4 stage) read as zero: offset
    // beyond the buffer
    cp_in_row = code_byte < (uint32_t)(row_bytes - lks * RB);
  };
  // copy j of a copy wave fills 1-KB block J = j CPW + wave of the stage:
  // rows 8 J .. 8 J + 7 of [A rows, B rows]; the first BM / (8 CPW) copies
  // of every copy wave are A rows
  auto issue_code = [&](int j) {
    constexpr int A_COPIES = BM / (8 * Cfg::CPW);
    const bool isa = j < A_COPIES;
    const uint32_t voff = cp_in_row ? code_lane + (isa ? a_base : b_base) + (uint32_t)j * copy_stride : 0x80000000u;
    dma16(isa ? a_rs : b_rs, cp_st + (uint32_t)((j * Cfg::CPW + wave) * 1024), voff, cp_soff);
  };
  auto close_copy_stage = [&]() {
    ++lgs;
    if (++lks == lk1) {
      lks = lk0;
      ++ltc;
      lt += gridDim.x;
      if (lt < tiles) set_copy_tile(lt);
    }
  };
  // L2 prefetch (Cfg::PF), issued after the last code copy of each stage:
  // the stage after the one just copied, within the same work item, is
  // touched with one 4-byte LDS copy per 128-byte row segment, so that its
  // lines are in the L2 by the time the stage copy reads them. The tile walk
  // runs about 4 tiles of a tile-row and 8 of a tile-column at once on an
  // XCD, so a workgroup touches a quarter of its A rows (by tile column) and
  // an eighth of its B rows (by tile row), waves 0 and 1; the data lands in
  // the unused second half of bias slot 0. Every wave issues exactly one such
  // instruction per stage (the others out of range: nothing is read), so the
  // stage waits allow PF_OPS of them in flight. It pays only where the
  // operands miss the L2 at every stage of long tiles (measured: MXFP8 fc2,
  // K = 4096, 8% faster; 1-3% slower on the K = 1024 shapes and on MXFP4).
  // Wave 1's copy reads B, the others' A; the buffer resource goes through
  // readfirstlane so that the compiler keeps it in scalar registers.
  v4u pf_rs = a_rs;
  if constexpr (Cfg::PF) {
    const v4u r = wave == 1 ? b_rs : a_rs;
    pf_rs = v4u{(unsigned)__builtin_amdgcn_readfirstlane(r.x), (unsigned)__builtin_amdgcn_readfirstlane(r.y),
                (unsigned)__builtin_amdgcn_readfirstlane(r.z), (unsigned)__builtin_amdgcn_readfirstlane(r.w)};
  }
  auto prefetch = [&]() {
    if constexpr (Cfg::PF) {
      const int ps = lks + 1;
      const int tm = m0l / BM, tn = n0l / BN;
      const uint32_t pa = (uint32_t)(m0l + (BM / 4) * (tn & 3) + lane) * (uint32_t)row_bytes;
      const uint32_t pb = (uint32_t)(n0l + (BN / 8) * (tm & 7) + lane) * (uint32_t)row_bytes;
      const bool in = ps < lk1;
      const uint32_t voff = (in && wave == 0 && lane < BM / 4) ? pa : (in && wave == 1 && lane < BN / 8) ? pb : 0x80000000u;
      dma4(pf_rs, lds_base + (uint32_t)(Cfg::BIAS_OFF + 512), voff, (uint32_t)(ps * RB));
    }
  };
  // The whole next stage in one burst. Everything it needs is local, which
  // keeps the register budget of the 256 x 256 tile within 256.
  auto issue_next = [&]() {
    if (lks == lk0 && bias_dma && wave == 0) {
      const uint32_t voff = lane < BN / 8 ? (uint32_t)((n0l + 8 * lane) * 2) : 0x80000000u;
      dma16(bias_rs, lds_base + (uint32_t)(Cfg::BIAS_OFF + (ltc & 1) * 1024), voff, 0u);
    }
    if (lks == lk0 || lks % Cfg::SPC == 0) {
      const uint32_t dst = sc_base + (uint32_t)((lgc & 1) * Cfg::SCHUNK);
      const uint32_t soff = (uint32_t)(16 * (lks / Cfg::SPC));
#pragma unroll
      for (int j = 0; j < Cfg::SCALE_DMA; ++j) {
        const int J = j * NW + wave;
        if (J < Cfg::SCALE_COPIES) {
          const bool isa = J * 64 < BM;
          const int row0 = (isa ? m0l : n0l - BM) + J * 64;
          dma16(isa ? as_rs : bs_rs, dst + (uint32_t)(J * 1024), scale_lane + (uint32_t)row0 * (uint32_t)srow, soff);
        }
      }
      ++lgc;
    }
    const uint32_t st = lds_base + (uint32_t)((lgs & 1) * Cfg::STAGE);
    const bool in_row = code_byte < (uint32_t)(row_bytes - lks * RB);
    if (copy_wave) {
#pragma unroll
      for (int j = 0; j < Cfg::CODE_DMA; ++j) {
        constexpr int A_COPIES = BM / (8 * Cfg::CPW);
        const bool isa = j < A_COPIES;
        const uint32_t voff = in_row ? code_lane + (isa ? a_base : b_base) + (uint32_t)j * copy_stride : 0x80000000u;
        dma16(isa ? a_rs : b_rs, st + (uint32_t)((j * Cfg::CPW + wave) * 1024), voff, (uint32_t)(lks * RB));
      }
    }
    prefetch();
    close_copy_stage();
  };

  const int ra = wm * WM + r32, rb = wn * WN + r32;     // this lane's fragment-0 rows in the tile
  // NVFP4: s_tA s_tB, the fp32 words at the start of the scale buffers'
  // trailers (16-byte aligned after the scale bytes)
  [[maybe_unused]] float tensor_scale = 1.0f;
  if constexpr (Cfg::FMT == FMT_NVFP4)
    tensor_scale = *reinterpret_cast<const float*>(As + (((int64_t)M * srow + 15) & ~(int64_t)15)) *
                   *reinterpret_cast<const float*>(Bs + (((int64_t)N * srow + 15) & ~(int64_t)15));

  // the GELU table; the first stage barrier orders it before every reader
  if constexpr (Cfg::GTAB) fill_gelu_table(reinterpret_cast<uint16_t*>(lds + Cfg::GTAB_OFF), (int)threadIdx.x, Cfg::NT);
  set_copy_tile(lt);
  issue_next();
  int gs = 0, gc = 0, ctc = 0;              // compute cursor: stages / scale chunks / tiles consumed

  for (int ct = blockIdx.x; ct < tiles; ct += gridDim.x) {
    int tm, tn, sp, k0, k1;
    item(ct, tm, tn, sp, k0, k1);
    const int m0 = tm * BM, n0 = tn * BN;
    // a split item's partial goes to its slice of the workspace, in fp32
    void* const Ct = splits > 1 ? static_cast<void*>(ws + (int64_t)sp * M * N) : C;
    const int out_f32_t = splits > 1 ? 1 : out_f32;

    v16f acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = v16f{};
    int slot = 0;

    for (int ks = k0; ks < k1; ++ks) {
      // this stage's copies are done (with PF, the prefetch issued after
      // them may still be in flight); after the previous tile's LDS-staged
      // epilogue its EPI_TOTAL stores (issued after them) may still be in
      // flight. The register epilogue drains its stores itself, so there the
      // count must be 0: an allowance would let this stage's own copies
      // (fewer than EPI_TOTAL per wave) still be in flight.
      if (ks == k0 && ctc > 0 && staged) wait_vm<Cfg::EPI_TOTAL + Cfg::PF_OPS>();
      else wait_vm<Cfg::PF_OPS>();
      block_sync();                         // everyone's copies are visible, and everyone is done
                                            // with the buffers the next copies overwrite
      // The next stage's copies. SPREAD: bias and scales now, code copies
      // spread over the stage's matrix-instruction blocks (copy j after
      // block j * BLOCKS / CODE_DMA); past this workgroup's last tile the
      // cursor keeps copying the last tile's rows into the buffer, scale
      // slot and bias slot no later stage reads, so no branch splits the
      // blocks. Otherwise: all of them now, in one burst (code copies from
      // the copy waves only).
      if (Cfg::SPREAD) open_copy_stage();
      else if (lt < tiles) issue_next();
      if (ks == k0 || ks % Cfg::SPC == 0) slot = gc++ & 1;   // a new scale chunk (as on the copy side)
      auto after_block = [&](int blk) {
        constexpr int BLOCKS = Cfg::SUB * FM;
        if (Cfg::SPREAD) {
#pragma unroll
          for (int j = 0; j < Cfg::CODE_DMA; ++j)
            if (j * BLOCKS / Cfg::CODE_DMA == blk) {
              if (copy_wave) issue_code(j);
              if (j == Cfg::CODE_DMA - 1) prefetch();
            }
        }
      };
      const uint8_t* const st_codes = lds + (gs & 1) * Cfg::STAGE;
      const uint8_t* const st_scales = lds + 2 * Cfg::STAGE + slot * Cfg::SCHUNK;
      if constexpr (Cfg::FMT == FMT_NVFP4 && Cfg::NV_PIPED)
        nv_mma_stage_piped<Cfg>(acc, st_codes, st_scales, g, ra, rb, after_block);
      else if constexpr (Cfg::FMT == FMT_NVFP4)
        nv_mma_stage<Cfg>(acc, st_codes, st_scales, g, ra, rb, after_block);
      else
        mma_stage<Cfg>(acc, st_codes, st_scales, ks % Cfg::SPC, g, ra, rb, after_block);
      if (Cfg::SPREAD) close_copy_stage();
      ++gs;
    }

    if constexpr (Cfg::FMT == FMT_NVFP4) {   // the two tensor scales, from the scale buffers' trailers
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] *= tensor_scale;
    }
    // epilogue: register 4q + v of acc[fm][fn] is C[m][n + v] with
    // m = m0 + wm WM + 32 fm + r32, n = n0 + wn WN + 32 fn + 8 q + 4 g.
    // The tile's bias sits in bias slot ctc & 1 (copied with the tile's first
    // stage); without that copy it is written here (zeros if there is no
    // bias), ordered before its readers by the next barrier.
    uint8_t* lds_bias = lds + Cfg::BIAS_OFF + (ctc & 1) * 1024;
    if (!bias_dma) {
      for (int i = (int)threadIdx.x; i < BN; i += Cfg::NT)
        reinterpret_cast<uint16_t*>(lds_bias)[i] = (bias != nullptr && n0 + i < N) ? bias[n0 + i] : (uint16_t)0;
    }
    bool wave_done = false;
    if constexpr (Cfg::WAVE_EPI) {
      if (staged) {
        // a bias written just above must be visible; an area in the stage
        // buffer just consumed is free once every wave is done reading it
        if (!Cfg::WAVE_OWN || !bias_dma) block_sync();
        uint8_t* const area =
            (Cfg::WAVE_OWN ? lds + Cfg::WAREA_OFF : lds + ((gs - 1) & 1) * Cfg::STAGE) + wave * Cfg::WAREA;
        // tiles before a workgroup's last one: streaming stores as well
        if (ct + (int)gridDim.x < tiles)
          mx_epilogue_wave<Cfg, kStoreStreamDeviceScope>(acc, lds_bias, M, N, m0, n0, wm, wn, g, r32, lane, c_rs, area);
        else
          mx_epilogue_wave<Cfg, kStoreDeviceScope>(acc, lds_bias, M, N, m0, n0, wm, wn, g, r32, lane, c_rs, area);
        wave_done = true;
      }
    }
    if (!wave_done)
      mx_epilogue<Cfg>(acc, lds_bias, staged, M, N, m0, n0, wm, wn, g, r32, Ct, out_f32_t, c_rs, q_rs, qs_rs, qld,
                       q_row_bytes, reinterpret_cast<const uint16_t*>(lds + Cfg::GTAB_OFF),
                       [&](int lr) { return lds + ((gs - 1) & 1) * Cfg::STAGE + lr * (BN * 2); });
    if (!staged) wait_vm<0>();               // nothing but the next stage's copies stays in flight
    ++ctc;
  }
  wait_vm<0>();                              // no copy into LDS outlives the workgroup
}

template <class Cfg>
static hipError_t run_mx(const uint8_t* A, const uint8_t* As, const uint8_t* B, const uint8_t* Bs, void* C,
                         int64_t M, int64_t N, int64_t K, const uint16_t* bias, int out_f32, int splits, float* ws,
                         hipStream_t stream) {
  const int64_t kpad = round_up(K, kAlignK);
  const int tiles_m = (int)((M + Cfg::BM - 1) / Cfg::BM);
  const int tiles_n = (int)((N + Cfg::BN - 1) / Cfg::BN);
  const int items = tiles_m * tiles_n * splits;
  // persistent grid: one slot per resident workgroup, a multiple of 8 so a
  // workgroup's items all map to its own XCD; smaller problems get one
  // workgroup per item
  const int slots = std::max(8, (Cfg::OCC * cu_count()) / 8 * 8);
  const int grid = items <= slots ? items : slots;
  gemm_mx_kernel<Cfg><<<grid, Cfg::NT, 0, stream>>>(A, As, B, Bs, C, (int)M, (int)N, (int)kpad,
                                                    splits > 1 ? nullptr : bias, out_f32, tiles_m, tiles_n, nullptr,
                                                    nullptr, 0, splits, ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || splits == 1) return e;
  return launch_splitk_reduce(ws, splits, M, N, bias, C, out_f32, stream);
}

template <class Cfg>
static hipError_t run_mx_q(const uint8_t* A, const uint8_t* As, const uint8_t* B, const uint8_t* Bs, int64_t M,
                           int64_t N, int64_t K, const uint16_t* bias, uint8_t* qcodes, uint8_t* qscales,
                           hipStream_t stream) {
  const int64_t kpad = round_up(K, kAlignK);
  const int tiles_m = (int)((M + Cfg::BM - 1) / Cfg::BM);
  const int tiles_n = (int)((N + Cfg::BN - 1) / Cfg::BN);
  const int tiles = tiles_m * tiles_n;
  const int slots = std::max(8, (Cfg::OCC * cu_count()) / 8 * 8);
  const int grid = tiles <= slots ? tiles : slots;
  gemm_mx_kernel<Cfg><<<grid, Cfg::NT, 0, stream>>>(A, As, B, Bs, qcodes, (int)M, (int)N, (int)kpad, bias, 0, tiles_m,
                                                    tiles_n, qcodes, qscales, (int)round_up(N, kAlignK), 1, nullptr);
  return hipGetLastError();
}

// NVFP4 through the MX kernel's data path (fp4 stages, dequantized per
// wave to fp16). Tiles: 192x256 (4 waves of 96x128, one wave per SIMD, so
// the pipelined stage), 128x128 (4 waves of 64x64, two workgroups per CU)
// or 128x256 (4 waves of 64x128, one workgroup per CU, pipelined; the
// split weight gradients). Four waves of 96x128 convert 7 fragments per 48
// matrix instructions where eight of 96x64 convert 5 per 24, and the
// conversions are this path's VALU limit.
hipError_t run_gemm_nvfp4_mx(int tile, int splits, const uint8_t* A, const uint8_t* As, const uint8_t* B,
                             const uint8_t* Bs, void* C, int64_t M, int64_t N, int64_t K, const uint16_t* bias,
                             int out_f32, float* ws, hipStream_t stream) {
  if (tile == NV_TILE_128x128)
    return run_mx<MxCfg<FMT_NVFP4, 128, 128, 2, 2, 2, true>>(A, As, B, Bs, C, M, N, K, bias, out_f32, splits, ws,
                                                               stream);
  if (tile == NV_TILE_128x256)
    return run_mx<MxCfg<FMT_NVFP4, 128, 256, 2, 2, 1, true>>(A, As, B, Bs, C, M, N, K, bias, out_f32, splits, ws,
                                                               stream);
  return run_mx<MxCfg<FMT_NVFP4, 192, 256, 2, 2, 1, true>>(A, As, B, Bs, C, M, N, K, bias, out_f32, splits, ws,
                                                             stream);
}

enum MxTile { TILE_128x128 = 0, TILE_192x256 = 1, TILE_256x256 = 2 };

// 256x256 and 192x256 tiles (8 waves of 128x64 / 96x64) are LDS-bound to
// one workgroup per CU; 128x128 (4 waves of 64x64) fits two per CU and
// serves problems too small to fill the chip with the large tiles. The
// 192x256 tile spreads its copies over the stage (the 256x256 tile has no
// registers left for that), which makes it the faster one on equal cost, and
// for FP4 (half the bytes per MFMA) on every ViT shape measured.
static MxTile choose_tile(int64_t M, int64_t N, int fmt) {
  const int64_t big = ((M + 255) / 256) * ((N + 255) / 256);
  if (big < 128) return TILE_128x128;
  const double c192 = tiling_cost(M, N, 192, 256), c256 = tiling_cost(M, N, 256, 256);
  if (fmt == FMT_MXFP4 ? c192 <= c256 : c192 < c256) return TILE_192x256;
  return TILE_256x256;
}

struct MxPlan {
  MxTile tile;
  int splits;
  bool pf;        // L2 prefetch: MXFP8 192 x 256 tiles of at least 32 stages
};

// Time of one K-stage of one workgroup with every CU busy (us), measured on
// MI355X on the ViT training shapes: fp8 stages hold 128 K elements, fp4
// stages 256. A 128x128 workgroup sharing its CU with a second one runs its
// stages 1.36x (fp8) / 1.6x (fp4) slower, so two per CU still nearly double
// the CU's throughput. The large fp4 tiles are bound by the L2 -> LDS copies
// once every CU runs them.
static double mx_stage_us(MxTile t, int fmt, bool shared_cu) {
  const bool f8 = fmt == FMT_MXFP8;
  switch (t) {
    case TILE_128x128: return f8 ? 0.92 * (shared_cu ? 1.36 : 1.0) : 0.98 * (shared_cu ? 1.6 : 1.0);
    case TILE_192x256: return f8 ? 1.7 : 2.4;
    default: return f8 ? 2.35 : 3.5;
  }
}

static int mx_tile_m(MxTile t) { return t == TILE_128x128 ? 128 : t == TILE_192x256 ? 192 : 256; }
static int mx_tile_n(MxTile t) { return t == TILE_128x128 ? 128 : 256; }

// Estimated time of a plan: rounds of resident workgroups x stages per work
// item x stage time, plus for a split plan the partials' cost (written by the
// GEMM, read back by the reduction: about 3 us + 0.25 us per MB, measured).
static double mx_plan_us(int64_t M, int64_t N, int64_t K, int fmt, MxPlan p) {
  const int64_t kpad = round_up(K, kAlignK);
  const int ks = fmt == FMT_MXFP8 ? 128 : 256;
  const int64_t nk = (kpad + ks - 1) / ks;
  const int occ = p.tile == TILE_128x128 ? 2 : 1;
  const int64_t cus = cu_count();
  const int64_t items = ((M + mx_tile_m(p.tile) - 1) / mx_tile_m(p.tile)) *
                        ((N + mx_tile_n(p.tile) - 1) / mx_tile_n(p.tile)) * p.splits;
  const int64_t rounds = (items + occ * cus - 1) / (occ * cus);
  const bool shared = occ == 2 && items > cus;
  double t = (double)rounds * (double)((nk + p.splits - 1) / p.splits) * mx_stage_us(p.tile, fmt, shared);
  if (p.splits > 1) t += 3.0 + 0.25 * (double)(p.splits * 4) * (double)(M * N) / 1.0e6;
  return t;
}

// The plan a GEMM runs: the tile above, or -- when the caller's workspace holds
// the partials (S M N fp32 values) and the output has too few tiles to fill
// the chip while K is long (the weight-gradient GEMMs) -- a tile with K split
// into up to 16 ranges, whichever the estimate says is fastest; a split plan
// must win by 5% to be taken.
static MxPlan choose_plan(int64_t M, int64_t N, int64_t K, int fmt, int64_t ws_bytes) {
  const int64_t kpad = round_up(K, kAlignK);
  const int64_t nk = (kpad + (fmt == FMT_MXFP8 ? 127 : 255)) / (fmt == FMT_MXFP8 ? 128 : 256);
  MxPlan best{choose_tile(M, N, fmt), 1, false};
  // the L2 prefetch variant for long MXFP8 tiles (measured faster only there)
  best.pf = fmt == FMT_MXFP8 && best.tile == TILE_192x256 && nk >= 32;
  if (ws_bytes < 2 * M * N * 4) return best;
  double best_us = mx_plan_us(M, N, K, fmt, best);
  for (MxTile t : {TILE_256x256, TILE_192x256, TILE_128x128}) {
    const int occ = t == TILE_128x128 ? 2 : 1;
    const int64_t tiles = ((M + mx_tile_m(t) - 1) / mx_tile_m(t)) * ((N + mx_tile_n(t) - 1) / mx_tile_n(t));
    for (int s = 2; s <= 16 && tiles * s <= occ * cu_count() && nk >= 4 * s && s * M * N * 4 <= ws_bytes; ++s) {
      const double us = mx_plan_us(M, N, K, fmt, MxPlan{t, s, false});
      if (us < 0.95 * best_us) {
        best_us = us;
        best = MxPlan{t, s, false};
      }
    }
  }
  return best;
}

template <int FMT>
static hipError_t dispatch_mx(const uint8_t* A, const uint8_t* As, const uint8_t* B, const uint8_t* Bs, void* C,
                              int64_t M, int64_t N, int64_t K, const uint16_t* bias, int out_f32, MxPlan p, float* ws,
                              hipStream_t stream) {
  switch (p.tile) {
    case TILE_128x128:
      return run_mx<MxCfg<FMT, 128, 128, 2, 2, 2, true>>(A, As, B, Bs, C, M, N, K, bias, out_f32, p.splits, ws, stream);
    case TILE_192x256:
      if constexpr (FMT == FMT_MXFP8) {
        // MXFP8: each stage's copies in one burst from waves 0-3 (see the
        // kernel's copy notes)
        if (p.pf)
          return run_mx<MxCfg<FMT, 192, 256, 2, 4, 1, false, 0, true, 4>>(A, As, B, Bs, C, M, N, K, bias, out_f32,
                                                                         p.splits, ws, stream);
        return run_mx<MxCfg<FMT, 192, 256, 2, 4, 1, false, 0, false, 4>>(A, As, B, Bs, C, M, N, K, bias, out_f32,
                                                                        p.splits, ws, stream);
      } else {
        return run_mx<MxCfg<FMT, 192, 256, 2, 4, 1, true>>(A, As, B, Bs, C, M, N, K, bias, out_f32, p.splits, ws,
                                                           stream);
      }
    default:
      if constexpr (FMT == FMT_MXFP8)
        return run_mx<MxCfg<FMT, 256, 256, 2, 4, 1, false, 0, false, 4>>(A, As, B, Bs, C, M, N, K, bias, out_f32,
                                                                        p.splits, ws, stream);
      else
        return run_mx<MxCfg<FMT, 256, 256, 2, 4, 1, false>>(A, As, B, Bs, C, M, N, K, bias, out_f32, p.splits, ws,
                                                            stream);
  }
}

template <int FMT>
static hipError_t dispatch_mx_q(const uint8_t* A, const uint8_t* As, const uint8_t* B, const uint8_t* Bs, int64_t M,
                                int64_t N, int64_t K, const uint16_t* bias, uint8_t* qcodes, uint8_t* qscales,
                                hipStream_t stream) {
  switch (choose_tile(M, N, FMT)) {
    case TILE_128x128:
      return run_mx_q<MxCfg<FMT, 128, 128, 2, 2, 2, true, 1>>(A, As, B, Bs, M, N, K, bias, qcodes, qscales, stream);
    case TILE_192x256:
      return run_mx_q<MxCfg<FMT, 192, 256, 2, 4, 1, true, 1>>(A, As, B, Bs, M, N, K, bias, qcodes, qscales, stream);
    default:
      return run_mx_q<MxCfg<FMT, 256, 256, 2, 4, 1, false, 1>>(A, As, B, Bs, M, N, K, bias, qcodes, qscales, stream);
  }
}

hipError_t launch_gemm_mx_gelu_quant(const uint8_t* A, const uint8_t* As, const uint8_t* B, const uint8_t* Bs,
                                     int64_t M, int64_t N, int64_t K, int fmt, const uint16_t* bias, uint8_t* qcodes,
                                     uint8_t* qscales, hipStream_t stream) {
  if (fmt == FMT_MXFP8) return dispatch_mx_q<FMT_MXFP8>(A, As, B, Bs, M, N, K, bias, qcodes, qscales, stream);
  return dispatch_mx_q<FMT_MXFP4>(A, As, B, Bs, M, N, K, bias, qcodes, qscales, stream);
}

int64_t gemm_mx_workspace_bytes(int64_t M, int64_t N, int64_t K, int fmt) {
  const MxPlan p = choose_plan(M, N, K, fmt, INT64_MAX);
  return p.splits > 1 ? (int64_t)p.splits * M * N * 4 : 0;
}

hipError_t launch_gemm_mx(const uint8_t* A, const uint8_t* As, const uint8_t* B, const uint8_t* Bs, void* C,
                          int64_t M, int64_t N, int64_t K, int fmt, const uint16_t* bias, int out_f32, float* ws,
                          int64_t ws_bytes, hipStream_t stream) {
  const MxPlan p = choose_plan(M, N, K, fmt, ws != nullptr ? ws_bytes : 0);
  if (fmt == FMT_MXFP8) return dispatch_mx<FMT_MXFP8>(A, As, B, Bs, C, M, N, K, bias, out_f32, p, ws, stream);
  return dispatch_mx<FMT_MXFP4>(A, As, B, Bs, C, M, N, K, bias, out_f32, p, ws, stream);
}

const char* plan_gemm_mx(int64_t M, int64_t N, int64_t K, int fmt, int64_t ws_bytes) {
  static const char* names[2][3] = {
      {"gemm_mx_kernel<mxfp8, 128x128>", "gemm_mx_kernel<mxfp8, 192x256>", "gemm_mx_kernel<mxfp8, 256x256>"},
      {"gemm_mx_kernel<mxfp4, 128x128>", "gemm_mx_kernel<mxfp4, 192x256>", "gemm_mx_kernel<mxfp4, 256x256>"}};
  // split plans: "<kernel>+splitk<S>", one static string per (format, tile, S)
  static char split_names[2][3][17][48];
  static std::once_flag once;
  std::call_once(once, [] {
    for (int f = 0; f < 2; ++f)
      for (int t = 0; t < 3; ++t)
        for (int sp = 2; sp <= 16; ++sp) snprintf(split_names[f][t][sp], 48, "%s+splitk%d", names[f][t], sp);
  });
  const MxPlan p = choose_plan(M, N, K, fmt, ws_bytes);
  const int f = fmt == FMT_MXFP8 ? 0 : 1;
  if (p.pf) return "gemm_mx_kernel<mxfp8, 192x256, l2pf>";
  return p.splits > 1 ? split_names[f][p.tile][p.splits] : names[f][p.tile];
}

}  // namespace mx
