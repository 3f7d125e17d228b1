// Device helpers shared by the GEMM kernels (gfx950): direct global->LDS
// transfers, wait-count control, the LDS chunk swizzle of the 256-row stage
// layouts and the grouped, XCD-contiguous tile order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

constexpr uint32_t kGroupM = 4;  // tile rows per group of the tile order

// 16-byte chunk swizzle of a row of a stage: chunk c of row r is stored at
// chunk c ^ swz(r), which spreads the ds_read_b128 of 32 consecutive rows at
// one chunk index over all LDS banks
__device__ __forceinline__ uint32_t swz(uint32_t r) { return ((r >> 1) ^ (r >> 3)) & 3u; }

typedef __attribute__((address_space(3))) void lds_void_t;
__device__ __forceinline__ uint32_t lds_addr(const void *p) { return (uint32_t)(size_t)(lds_void_t *)p; }

// one wave-wide direct transfer: lane l's 16 (4) bytes at base + voff land at
// LDS byte lds + 16 l (4 l)
__device__ __forceinline__ void dma16(const void *base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds), "v"(voff), "s"(base) : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void *base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2" ::"s"(lds), "v"(voff), "s"(base) : "memory", "m0");
}

// a pointer the caller knows to be wave-uniform, in scalar registers (the
// transfers take their base address from SGPRs).  The NVFP4 fast path moves
// this base by the K-tile offset; the MXFP4 kernel, which issues its ten
// transfers back to back, was 14 % slower that way and adds the offset per lane.
__device__ __forceinline__ const uint8_t *uniform_ptr(const uint8_t *p) {
  const uint64_t v = (uint64_t)p;
  return (const uint8_t *)(((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(v >> 32)) << 32) |
                           (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)v));
}

// vmcnt <= n (other counters untouched)
#define NVFP4_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))

// lgkmcnt <= 0 (LDS reads of this wave complete; other counters untouched)
#define NVFP4_WAIT_LGKM0() __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4))

// Origin of tile t of the grouped order for a 256x256-tiled M x N output:
// groups of kGroupM tile rows, walked column by column, so that consecutive
// tiles (one XCD's range under xcd_tile) cover a compact block of C and share
// the operand K-slices in that XCD's L2.
__device__ __forceinline__ void tile_origin(int64_t M, int64_t N, uint32_t tile, int64_t &m0, int64_t &n0) {
  const uint32_t tiles_m = (uint32_t)(M / 256), tiles_n = (uint32_t)(N / 256);
  const uint32_t group = tile / (kGroupM * tiles_n), first_m = group * kGroupM;
  const uint32_t gm = tiles_m - first_m < kGroupM ? tiles_m - first_m : kGroupM;
  const uint32_t local = tile - group * kGroupM * tiles_n;
  m0 = (int64_t)(first_m + local % gm) * 256;
  n0 = (int64_t)(local / gm) * 256;
}

}  // namespace nvfp4
