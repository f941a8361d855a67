// Pieces shared by the two GEMM kernels (gfx950): buffer resources, the
// LDS copy instruction, explicit waits and barriers, the XCD-aware tile
// numbering, the LDS row swizzle, and host-side launch sizing.
#pragma once

#include "mx_device.h"

#include <atomic>

namespace mx {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));

// Row r keeps 16-byte chunk c of a 128-byte row at position c ^ ((r / 2) % 8).
// A 128-byte row covers half of the LDS's 64 four-byte banks, so rows
// alternate bank halves; a 16-byte read is served 16 lanes at a time, and the
// 16 consecutive rows those lanes read (same logical chunk) then land on 16
// distinct 16-byte bank groups.
__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r >> 1) & 7); }

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

// One wave-wide 4-byte-per-lane copy global -> LDS, used only to touch a
// line so that the L2 holds it when the stage copy that reads it comes.
__device__ __forceinline__ void dma4(v4u rs, uint32_t lds_addr, uint32_t voff, uint32_t soff) {
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\tbuffer_load_dword %2, %3, %4 offen lds\n\ts_mov_b32 m0, %0"
               : "=&s"(saved) : "s"(lds_addr), "v"(voff), "s"(rs), "s"(soff) : "memory");
}

// Wait until at most N vector memory operations of this wave are in flight
// (they complete in issue order). Issued through the builtin so the
// compiler's own wait bookkeeping sees it too.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Cache policy of the GEMMs' output stores: device scope (sc1). The XCD's L2
// then writes them through rather than holding them dirty until the release
// at the end of the kernel, which otherwise writes the last tiles' output
// back after the matrix work is done (measured on gfx950: about 1.5 us less
// on launches of one round of tiles, no change on longer ones).
constexpr int kStoreDeviceScope = 16;
// The same with the non-temporal hint as well (streaming: the line is not
// kept for reuse). Used for the output tiles a GEMM workgroup stores before
// its last one: they then displace less of the operand panels the L2 holds
// for the following tiles (measured on gfx950: 2-10% faster GEMMs of three
// rounds of tiles on the ViT shapes; on launches of one round of tiles the
// hint alone made no difference or cost up to 3%, so a workgroup's last
// tile keeps the plain device-scope store).
constexpr int kStoreStreamDeviceScope = 16 | 2;

// Workgroup barrier after this wave's LDS operations have completed. Global
// stores still in flight are deliberately not waited for. The LDS wait goes
// through the builtin so the compiler knows every earlier LDS read is done
// (otherwise it re-waits for them, counting later reads in between).
__device__ __forceinline__ void block_sync() {
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));   // lgkmcnt(0)
  asm volatile("s_barrier" ::: "memory");
}

// Coordinates of tile t: XCD-contiguous renumbering (tile t runs on XCD
// t % 8 because the grid is a multiple of 8 or covers every tile once), then
// groups of 8 tile-rows walked column by column.
__device__ __forceinline__ void tile_coords(int t, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int nwg = tiles_m * tiles_n;
  const int q = nwg / 8, r = nwg % 8;
  const int xcd = t % 8, local = t / 8;
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

// Compute units of the current device (cached per device).
inline int cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
  cache[dev].store(v, std::memory_order_relaxed);
  return v;
}

// Rounds of workgroups a tiling needs on the 256 CUs (one 256x256 or
// 192x256 workgroup per CU, LDS-limited), weighted by tile area: the shape
// with the least MFMA time lost to idle CUs in the last round wins.
inline double tiling_cost(int64_t M, int64_t N, int bm, int bn) {
  const int64_t tiles = ((M + bm - 1) / bm) * ((N + bn - 1) / bn);
  const int64_t rounds = (tiles + 255) / 256;
  return (double)rounds * bm * bn;
}

}  // namespace mx
