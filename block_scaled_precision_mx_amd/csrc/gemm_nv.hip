// NVFP4 GEMM plans: C = s_tA s_tB sum_k (a_k dA)(b_k dB) (+ bias[n]).
//
// lightly-train README "DINOv3 + EoMT on RTX 5090", section 2: NVFP4 is
// E2M1 elements with an E4M3 scale per 1x16 block plus an fp32 scale per
// tensor; sections 5.3-5.5 use it for the dgrad / wgrad GEMMs of training.
// The kernel is gemm_mx_kernel's NVFP4 mode (exact dequantization to fp16
// per wave, fp16 matrix instructions); this file picks its tile shape and
// split-K factor per GEMM shape.
#include "gemm_common.h"
#include "mx_launch.h"

#include <algorithm>
#include <cstdio>
#include <mutex>

namespace mx {

struct NvPlan {
  int tile;                                  // NvTile
  int splits;
};

struct NvTileShape {
  int bm, bn, occ;                           // rows, columns, workgroups per CU
  double step_us;                            // one 64-K step of one workgroup, every CU busy (see nv_plan_us)
};

static NvTileShape nv_tile_shape(int tile) {
  switch (tile) {
    case NV_TILE_128x128: return {128, 128, 2, 0.73};
    case NV_TILE_128x256: return {128, 256, 1, 1.12};
    default:              return {192, 256, 1, 1.7};
  }
}

// Tile shape with the least work per CU lost to a partly filled last round:
// rounds of resident workgroups x tile area x workgroups per CU. 128x128 (4
// waves of 64x64, two workgroups per CU) fills the chip on the weight-
// gradient shapes (4096 x 1024 outputs, K = tokens), where 192x256 tiles
// leave most CUs idle; on ties the larger tiles win (less dequantization
// and LDS traffic per output).
static int nv_unsplit_tile(int64_t M, int64_t N) {
  auto cost = [&](int bm, int bn, int occ) {
    const int64_t tiles = ((M + bm - 1) / bm) * ((N + bn - 1) / bn);
    const int64_t slots = std::max(8, occ * cu_count() / 8 * 8);
    return (double)((tiles + slots - 1) / slots) * bm * bn * occ;
  };
  return cost(128, 128, 2) < cost(192, 256, 1) ? NV_TILE_128x128 : NV_TILE_192x256;
}

// Estimated time of a plan (us): rounds x 64-K steps per item x the time of
// one 64-K step of one workgroup with every CU busy (measured on MI355X on
// the training shapes: about 1.7 us for 192x256, 1.1 us for 128x256, 0.7 us
// for 128x128, whose two workgroups per CU split the CU's throughput, the
// dequantization being VALU work), plus the split-K partials (about 3 us +
// 0.25 us per MB, measured). The kernel stages 256 K at a time; the model
// counts in 64 K.
static double nv_plan_us(int64_t M, int64_t N, int64_t K, NvPlan p) {
  const NvTileShape t = nv_tile_shape(p.tile);
  const int64_t nk = round_up(K, kAlignK) / 64;
  const int64_t cus = cu_count();
  const int64_t items = ((M + t.bm - 1) / t.bm) * ((N + t.bn - 1) / t.bn) * p.splits;
  const int64_t rounds = (items + t.occ * cus - 1) / (t.occ * cus);
  const double step = t.occ == 2 && items > cus ? 2.0 * t.step_us : t.step_us;
  double us = (double)rounds * (double)(2 * ((nk / 2 + p.splits - 1) / p.splits)) * step;
  if (p.splits > 1) us += 3.0 + 0.25 * (double)(p.splits * 4) * (double)(M * N) / 1.0e6;
  return us;
}

// As for the MX GEMM: a split plan only if the workspace holds its partials
// and the estimate beats the unsplit plan by 5%. Split plans may also take
// 128x256 tiles (4 waves of 64x128): with one workgroup per CU and fewer
// conversions per matrix instruction than 128x128, they fill the chip on
// the 4096 x 1024 weight gradients with two splits.
static NvPlan nv_choose_plan(int64_t M, int64_t N, int64_t K, int64_t ws_bytes) {
  NvPlan best{nv_unsplit_tile(M, N), 1};
  if (ws_bytes < 2 * M * N * 4) return best;
  double best_us = nv_plan_us(M, N, K, best);
  const int64_t pairs = round_up(K, kAlignK) / 128;
  for (int tile : {NV_TILE_192x256, NV_TILE_128x128, NV_TILE_128x256}) {
    const NvTileShape t = nv_tile_shape(tile);
    const int64_t tiles = ((M + t.bm - 1) / t.bm) * ((N + t.bn - 1) / t.bn);
    for (int s = 2; s <= 16 && tiles * s <= t.occ * cu_count() && pairs >= 2 * s && s * M * N * 4 <= ws_bytes; ++s) {
      const double us = nv_plan_us(M, N, K, NvPlan{tile, s});
      if (us < 0.95 * best_us) {
        best_us = us;
        best = NvPlan{tile, s};
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
  static const char* names[3] = {"gemm_mx_kernel<nvfp4, 192x256>", "gemm_mx_kernel<nvfp4, 128x128>",
                                 "gemm_mx_kernel<nvfp4, 128x256>"};
  static char split_names[3][17][48];
  static std::once_flag once;
  std::call_once(once, [] {
    for (int t = 0; t < 3; ++t)
      for (int sp = 2; sp <= 16; ++sp) snprintf(split_names[t][sp], 48, "%s+splitk%d", names[t], sp);
  });
  const NvPlan p = nv_choose_plan(M, N, K, ws_bytes);
  return p.splits > 1 ? split_names[p.tile][p.splits] : names[p.tile];
}

hipError_t launch_gemm_nvfp4(const uint8_t* A, const uint8_t* As, const uint8_t* B, const uint8_t* Bs, void* C,
                             int64_t M, int64_t N, int64_t K, const uint16_t* bias, int out_f32, float* ws,
                             int64_t ws_bytes, hipStream_t stream) {
  const NvPlan p = nv_choose_plan(M, N, K, ws != nullptr ? ws_bytes : 0);
  return run_gemm_nvfp4_mx(p.tile, p.splits, A, As, B, Bs, C, M, N, K, bias, out_f32, ws, stream);
}

}  // namespace mx
