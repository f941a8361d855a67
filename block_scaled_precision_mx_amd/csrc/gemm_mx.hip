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
// Data movement. A K-stage is 128 bytes of codes per row (128 fp8 / 256 fp4
// elements); two stages are double-buffered in LDS. Scales travel in chunks
// of 16 bytes per row (16 blocks, i.e. 512 K elements), double-buffered in
// their own LDS slots. Both are copied global -> LDS with
// buffer_load ... lds (16 bytes per lane; rows past the tensor read as
// zero), issued from inline assembly with the kernel's own waits, so the
// compiler does not stall every LDS read on copies that are still in
// flight. A stage's 1-KB wave copies cover 8 rows x 128 bytes, the shape the
// L2 serves fastest. Code rows are XOR-swizzled in 16-byte chunks so the 8
// lanes of one LDS read cycle hit distinct banks. Each sub-step's fragments
// are read into registers before the matrix instructions of the previous
// sub-step are issued. Tiles are renumbered so each XCD (own L2) gets a
// contiguous range, walked in groups of 8 tile-rows.
//
// Epilogue: the bias is loaded before the K loop. For bf16 output the tile
// is converted and written to LDS (16-byte chunks XOR-swizzled by row), then
// stored as whole rows of 16-byte lanes; fp32 output (or N % 8 != 0) is
// stored straight from registers.
#include "mx_device.h"
#include "mx_launch.h"

namespace mx {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));

template <int FMT_, int BM_, int BN_, int WAVES_M_, int WAVES_N_>
struct MxCfg {
  static constexpr int FMT = FMT_, BM = BM_, BN = BN_, WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
  static constexpr int NT = 64 * WAVES_M * WAVES_N, NW = NT / 64;
  static constexpr int RB = 128;                              // code bytes per row per stage
  static constexpr int CH = RB / 16;                          // 16-byte chunks per row
  static constexpr int KS = (FMT == FMT_MXFP8) ? RB : 2 * RB; // K elements per stage
  static constexpr int SUB = KS / 64;                         // 32x32x64 sub-steps per stage
  static constexpr int SPC = 512 / KS;                        // stages per scale chunk
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  static constexpr int FM = WM / 32, FN = WN / 32;
  static constexpr int STAGE = (BM + BN) * RB;                 // code bytes per stage
  static constexpr int SCHUNK = (BM + BN) * 16;                // bytes per scale slot
  static constexpr int LDS = 2 * STAGE + 2 * SCHUNK;
  static constexpr int CODE_DMA = STAGE / 1024 / NW;          // 1-KB code copies per wave per stage
  static constexpr int SCALE_COPIES = (BM + BN) / 64;         // 1-KB copies per scale chunk
  static constexpr int SCALE_DMA = (SCALE_COPIES + NW - 1) / NW;  // per wave (some may be idle)
  static constexpr int MFMA_FMT = (FMT == FMT_MXFP8) ? 0 : 4;  // E4M3 / E2M1 operand selector
  static_assert(CODE_DMA * 1024 * NW == STAGE, "code copies must split evenly over waves");
  static_assert(BM % 64 == 0 && BN % 64 == 0 && WM % 32 == 0 && WN % 32 == 0, "tile");
  static_assert(LDS <= 160 * 1024, "LDS");
  static_assert(BM * BN * 2 <= LDS, "the bf16 C tile must fit in LDS");
};

// Row r keeps 16-byte chunk c of a 128-byte row at position c ^ (r & 7).
__device__ __forceinline__ int swz(int r, int c) { return c ^ (r & 7); }

__device__ __forceinline__ v4u buffer_rsrc(const void* p, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  v4u r;
  r.x = __builtin_amdgcn_readfirstlane((uint32_t)a);
  r.y = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  r.z = __builtin_amdgcn_readfirstlane(bytes);
  r.w = 0x00020000u;   // raw buffer, 32-bit data format: out-of-range reads return 0
  return r;
}

// One wave-wide copy global -> LDS: lane l's 16 bytes at `voff` (+ soff)
// land at lds_addr + 16 l. M0 is saved and restored around the copy.
__device__ __forceinline__ void dma16(v4u rs, uint32_t lds_addr, uint32_t voff, uint32_t soff) {
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\tbuffer_load_dwordx4 %2, %3, %4 offen lds\n\ts_mov_b32 m0, %0"
               : "=&s"(saved) : "s"(lds_addr), "v"(voff), "s"(rs), "s"(soff) : "memory");
}

// Wait until every vector memory operation of this wave has completed.
__device__ __forceinline__ void wait_vm_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

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

// One sub-step's operands for one wave: FM A fragments, FN B fragments and
// their scales, shifted so that this lane's scale byte is byte 0.
template <class Cfg>
struct Frags {
  v8i a[Cfg::FM], b[Cfg::FN];
  int sa[Cfg::FM], sb[Cfg::FN];
};

// Sub-step t of the stage held at `st` (codes) whose scales are in the
// chunk at `sc`, chunk-relative stage index `sj`. fp8: lane chunks 4t+g and
// 4t+2+g (K 16g.. and 32+16g.. of the sub-step); fp4: chunk 2t+g. This
// lane's scale byte is block (KS/32) sj + 2t + g of the row's 16-byte chunk.
template <class Cfg>
__device__ __forceinline__ void load_frags(Frags<Cfg>& fr, const uint8_t* st, const uint8_t* sc, int t, int sj,
                                           int g, int ra, int rb) {
  constexpr int RB = Cfg::RB;
  const int blk = (Cfg::KS / 32) * sj + 2 * t + g;
  const int sdw = blk >> 2, sh = 8 * (blk & 3);
#pragma unroll
  for (int f = 0; f < Cfg::FN; ++f) {
    const int r = rb + 32 * f;
    const uint8_t* row = st + (Cfg::BM + r) * RB;
    fr.sb[f] = (int)(*reinterpret_cast<const uint32_t*>(sc + (Cfg::BM + r) * 16 + 4 * sdw) >> sh);
    if (Cfg::FMT == FMT_MXFP8) {
      const uint4 lo = *reinterpret_cast<const uint4*>(row + swz(r, 4 * t + g) * 16);
      const uint4 hi = *reinterpret_cast<const uint4*>(row + swz(r, 4 * t + 2 + g) * 16);
      fr.b[f] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    } else {
      const uint4 lo = *reinterpret_cast<const uint4*>(row + swz(r, 2 * t + g) * 16);
      fr.b[f] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, 0, 0, 0, 0};
    }
  }
#pragma unroll
  for (int f = 0; f < Cfg::FM; ++f) {
    const int r = ra + 32 * f;
    const uint8_t* row = st + r * RB;
    fr.sa[f] = (int)(*reinterpret_cast<const uint32_t*>(sc + r * 16 + 4 * sdw) >> sh);
    if (Cfg::FMT == FMT_MXFP8) {
      const uint4 lo = *reinterpret_cast<const uint4*>(row + swz(r, 4 * t + g) * 16);
      const uint4 hi = *reinterpret_cast<const uint4*>(row + swz(r, 4 * t + 2 + g) * 16);
      fr.a[f] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    } else {
      const uint4 lo = *reinterpret_cast<const uint4*>(row + swz(r, 2 * t + g) * 16);
      fr.a[f] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, 0, 0, 0, 0};
    }
  }
}

template <class Cfg>
__global__ __launch_bounds__(Cfg::NT) void gemm_mx_kernel(const uint8_t* __restrict__ A,
                                                          const uint8_t* __restrict__ As,
                                                          const uint8_t* __restrict__ B,
                                                          const uint8_t* __restrict__ Bs, void* __restrict__ C,
                                                          int M, int N, int kpad,
                                                          const uint16_t* __restrict__ bias, int out_f32,
                                                          int tiles_m, int tiles_n) {
  constexpr int BM = Cfg::BM, BN = Cfg::BN, WM = Cfg::WM, WN = Cfg::WN, FM = Cfg::FM, FN = Cfg::FN;
  constexpr int RB = Cfg::RB, CH = Cfg::CH, NW = Cfg::NW;
  __shared__ __align__(16) uint8_t lds[Cfg::LDS];

  int tm, tn;
  tile_coords(tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / Cfg::WAVES_N, wn = wave % Cfg::WAVES_N;
  const int row_bytes = (Cfg::FMT == FMT_MXFP8) ? kpad : kpad / 2;
  const int srow = kpad / 32;               // scale bytes per row
  // stages; with fp4 a stage holds 256 elements while K_pad is a multiple
  // of 128, so the last stage may hold only its first 64 bytes
  const int nk = (kpad + Cfg::KS - 1) / Cfg::KS;
  const int g = lane >> 5, r32 = lane & 31;

  const v4u a_rs = buffer_rsrc(A, (uint32_t)(M * row_bytes));
  const v4u b_rs = buffer_rsrc(B, (uint32_t)(N * row_bytes));
  const v4u as_rs = buffer_rsrc(As, (uint32_t)(M * srow));
  const v4u bs_rs = buffer_rsrc(Bs, (uint32_t)(N * srow));
  const uint32_t lds_base = (uint32_t)reinterpret_cast<uintptr_t>(lds);
  const uint32_t sc_base = lds_base + 2 * Cfg::STAGE;

  // Code copy j of this wave fills the stage's 1-KB block J = j NW + wave,
  // i.e. 16-byte chunks 64 J + lane: A rows first (CH chunks per row), then B.
  uint32_t code_voff[Cfg::CODE_DMA];
  int code_byte[Cfg::CODE_DMA];             // byte of the stage this lane copies
  bool code_is_a[Cfg::CODE_DMA];
#pragma unroll
  for (int j = 0; j < Cfg::CODE_DMA; ++j) {
    const int J = j * NW + wave;
    const int P = J * 64 + lane;
    const bool isa = P < BM * CH;
    const int Pr = isa ? P : P - BM * CH;
    const int r = Pr / CH, p = Pr % CH;
    code_is_a[j] = J * 64 < BM * CH;           // uniform per copy
    code_byte[j] = swz(r, p) * 16;
    code_voff[j] = (uint32_t)(((isa ? m0 : n0) + r) * row_bytes + code_byte[j]);
  }
  // Scale copy j of this wave fills rows 64 J .. 64 J + 63 of [A rows, B rows]
  // with 16 bytes each (copies J >= SCALE_COPIES are skipped).
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
    if (ks % Cfg::SPC == 0) {               // first stage of a scale chunk: bring the chunk too
      const int c = ks / Cfg::SPC;
      const uint32_t dst = sc_base + (uint32_t)((c & 1) * Cfg::SCHUNK);
#pragma unroll
      for (int j = 0; j < Cfg::SCALE_DMA; ++j) {
        const int J = j * NW + wave;
        if (J < Cfg::SCALE_COPIES) dma16(scale_is_a[j] ? as_rs : bs_rs, dst + (uint32_t)(J * 1024), scale_voff[j],
                                         (uint32_t)(16 * c));
      }
    }
    const uint32_t st = lds_base + (uint32_t)((ks & 1) * Cfg::STAGE);
    const int rem = row_bytes - ks * RB;    // bytes of each row left from this stage on
#pragma unroll
    for (int j = 0; j < Cfg::CODE_DMA; ++j) {
      // bytes past the end of the row read as zero (offset beyond the buffer)
      const uint32_t voff = code_byte[j] < rem ? code_voff[j] : 0x80000000u;
      dma16(code_is_a[j] ? a_rs : b_rs, st + (uint32_t)((j * NW + wave) * 1024), voff, (uint32_t)(ks * RB));
    }
  };

  const int ra = wm * WM + r32, rb = wn * WN + r32;     // this lane's fragment-0 rows in the tile

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

  issue_stage(0);
  for (int ks = 0; ks < nk; ++ks) {
    wait_vm_all();                          // this wave's copies of stage ks (and its scale chunk)
    __syncthreads();                        // everyone's copies are visible, and everyone is done
                                            // with the buffers the next copies overwrite
    if (ks + 1 < nk) issue_stage(ks + 1);

    const uint8_t* st = lds + (ks & 1) * Cfg::STAGE;
    const uint8_t* sc = lds + 2 * Cfg::STAGE + ((ks / Cfg::SPC) & 1) * Cfg::SCHUNK;
    const int sj = ks % Cfg::SPC;
    Frags<Cfg> cur_f, nxt_f;
    load_frags<Cfg>(cur_f, st, sc, 0, sj, g, ra, rb);
#pragma unroll
    for (int t = 0; t < Cfg::SUB; ++t) {
      if (t + 1 < Cfg::SUB) load_frags<Cfg>(nxt_f, st, sc, t + 1, sj, g, ra, rb);
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
          acc[fm][fn] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(cur_f.b[fn], cur_f.a[fm], acc[fm][fn],
                                                                        Cfg::MFMA_FMT, Cfg::MFMA_FMT, 0, cur_f.sb[fn],
                                                                        0, cur_f.sa[fm]);
      if (t + 1 < Cfg::SUB) cur_f = nxt_f;
    }
  }

  // epilogue: register 4q + v of acc[fm][fn] is C[m][n + v] with
  // m = m0 + wm WM + 32 fm + r32, n = n0 + wn WN + 32 fn + 8 q + 4 g.
  if (!out_f32 && (N & 7) == 0) {
    constexpr int CPR = BN / 8;                          // 16-byte chunks per tile row
    __syncthreads();                                     // every wave is done reading the last stage
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      const int ml = wm * WM + 32 * fm + r32;
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int nl = wn * WN + 32 * fn + 8 * q + 4 * g;
          const uint2 bb = bias_v[fn][q];
          const float v0 = acc[fm][fn][4 * q + 0] + bf16_to_f32(bb.x & 0xFFFFu);
          const float v1 = acc[fm][fn][4 * q + 1] + bf16_to_f32(bb.x >> 16);
          const float v2 = acc[fm][fn][4 * q + 2] + bf16_to_f32(bb.y & 0xFFFFu);
          const float v3 = acc[fm][fn][4 * q + 3] + bf16_to_f32(bb.y >> 16);
          const int chunk = (nl >> 3) ^ (ml & (CPR - 1));
          *reinterpret_cast<uint2*>(lds + ml * (BN * 2) + chunk * 16 + (nl & 7) * 2) =
              make_uint2(f32_to_bf16_rne(v0) | (f32_to_bf16_rne(v1) << 16),
                         f32_to_bf16_rne(v2) | (f32_to_bf16_rne(v3) << 16));
        }
    }
    __syncthreads();
    constexpr int TOTAL = BM * CPR;
#pragma unroll 4
    for (int id = threadIdx.x; id < TOTAL; id += Cfg::NT) {
      const int row = id / CPR, c = id % CPR;
      const int m = m0 + row, n = n0 + 8 * c;
      if (m < M && n < N) {
        const uint4 w = *reinterpret_cast<const uint4*>(lds + row * (BN * 2) + ((c ^ (row & (CPR - 1))) * 16));
        *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(C) + (int64_t)m * N + n) = w;
      }
    }
    return;
  }
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

// Rounds of workgroups a tiling needs on the 256 CUs (one 256x256 or
// 192x256 workgroup per CU, LDS-limited), weighted by tile area: the shape
// with the least MFMA time lost to idle CUs in the last round wins.
static double tiling_cost(int64_t M, int64_t N, int bm, int bn) {
  const int64_t tiles = ((M + bm - 1) / bm) * ((N + bn - 1) / bn);
  const int64_t rounds = (tiles + 255) / 256;
  return (double)rounds * bm * bn;
}

enum MxTile { TILE_128x128 = 0, TILE_192x256 = 1, TILE_256x256 = 2 };

// 256x256 and 192x256 tiles (8 waves of 128x64 / 96x64) are LDS-bound to
// one workgroup per CU; 128x128 (4 waves of 64x64) fits two per CU and
// serves problems too small to fill the chip with the large tiles.
static MxTile choose_tile(int64_t M, int64_t N) {
  const int64_t big = ((M + 255) / 256) * ((N + 255) / 256);
  if (big < 128) return TILE_128x128;
  if (tiling_cost(M, N, 192, 256) < tiling_cost(M, N, 256, 256)) return TILE_192x256;
  return TILE_256x256;
}

template <int FMT>
static hipError_t dispatch_mx(const uint8_t* A, const uint8_t* As, const uint8_t* B, const uint8_t* Bs, void* C,
                              int64_t M, int64_t N, int64_t K, const uint16_t* bias, int out_f32,
                              hipStream_t stream) {
  switch (choose_tile(M, N)) {
    case TILE_128x128: return run_mx<MxCfg<FMT, 128, 128, 2, 2>>(A, As, B, Bs, C, M, N, K, bias, out_f32, stream);
    case TILE_192x256: return run_mx<MxCfg<FMT, 192, 256, 2, 4>>(A, As, B, Bs, C, M, N, K, bias, out_f32, stream);
    default:           return run_mx<MxCfg<FMT, 256, 256, 2, 4>>(A, As, B, Bs, C, M, N, K, bias, out_f32, stream);
  }
}

hipError_t launch_gemm_mx(const uint8_t* A, const uint8_t* As, const uint8_t* B, const uint8_t* Bs, void* C,
                          int64_t M, int64_t N, int64_t K, int fmt, const uint16_t* bias, int out_f32,
                          hipStream_t stream) {
  if (fmt == FMT_MXFP8) return dispatch_mx<FMT_MXFP8>(A, As, B, Bs, C, M, N, K, bias, out_f32, stream);
  return dispatch_mx<FMT_MXFP4>(A, As, B, Bs, C, M, N, K, bias, out_f32, stream);
}

const char* plan_gemm_mx(int64_t M, int64_t N, int fmt) {
  static const char* names[2][3] = {
      {"gemm_mx_kernel<mxfp8, 128x128>", "gemm_mx_kernel<mxfp8, 192x256>", "gemm_mx_kernel<mxfp8, 256x256>"},
      {"gemm_mx_kernel<mxfp4, 128x128>", "gemm_mx_kernel<mxfp4, 192x256>", "gemm_mx_kernel<mxfp4, 256x256>"}};
  return names[fmt == FMT_MXFP8 ? 0 : 1][choose_tile(M, N)];
}

}  // namespace mx
