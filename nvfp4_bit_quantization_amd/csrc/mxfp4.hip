// MXFP4 for gfx950: quantisation, dequantisation and the GEMM on the native
// block-scaled FP4 matrix instruction (v_mfma_scale_f32_32x32x64_f8f6f4).
//
// MXFP4 is the earlier 4-bit microscaling format the NVFP4 pretraining news
// page (zubnet.ai) sets NVFP4 against in paragraph 3; the page does not define
// it, so the definition is the OCP Microscaling Formats (MX) specification
// v1.0: blocks of 32 elements along K share one E8M0 scale X = 2^e with
// e = floor(log2(max |v|)) - 2 (clamped to [-127, 127]; code e + 127, an
// all-zero block code 0), and the elements are v / X rounded to nearest-even
// onto E2M1, clamped at 6.  There is no per-tensor scale, so quantisation is a
// single pass, and the 32-element E8M0 blocks are exactly what the matrix
// instruction applies itself: the GEMM feeds packed codes and scale bytes to
// the MFMA with no expansion.
#include "gemm_device.hpp"
#include "quantize_device.hpp"

#include <stdlib.h>

namespace nvfp4 {

typedef int int8v __attribute__((ext_vector_type(8)));
typedef float float16v __attribute__((ext_vector_type(16)));

// E8M0 code of a block maximum m >= 0 (finite): with E the binary32 biased
// exponent of m, floor(log2 m) = E - 127 for normal m, so the code is
// (E - 129) + 127 = E - 2, clamped at 0 (which also covers zero and subnormal
// maxima, whose exponent would be below -127).
__device__ __forceinline__ uint32_t mx_scale_code(float m) {
  const uint32_t E = __float_as_uint(m) >> 23;
  return E > 2u ? E - 2u : 0u;
}
// 1 / X = 2^(127 - code) as binary32 (2^127 .. 2^-127 for codes 0 .. 254)
__device__ __forceinline__ float mx_inv_scale(uint32_t code) { return __uint_as_float((254u - code) << 23); }

// ------------------------------------------------------------------------
// quantisation: one 16-row x 8-column micro-tile per lane (the lane/tile
// decomposition of the NVFP4 kernels).  Row blocks of 32 columns span the
// lanes cc, cc^1, cc^2, cc^3 (lane bits 3-4), column blocks of 32 rows the
// lanes cg and cg^1 (lane bit 0).  Every lane takes part in the cross-lane
// maxima; lanes past the tensor hold zeros and store nothing.
// ------------------------------------------------------------------------
template <int G>
__global__ __launch_bounds__(kQThreads) void mx_quantize_kernel(MxQuantArgs a) {
  const Lane L = lane_coords(blockIdx.x, a.R, a.C);  // row-major tile order, as for NVFP4
  const uint32_t lane = threadIdx.x & 63;
  uint4 raw[16];
  if (L.valid) {
    load_micro_tile(a.x, a.ld, L, raw);
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) raw[i] = make_uint4(0u, 0u, 0u, 0u);
  }
  if (G == G_ROW) {
    const bool first = ((lane >> 3) & 3u) == 0u;  // cc % 4 == 0: first lane of its block
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float v[8];
      float m = 0.0f;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        v[k] = bf16_at(raw[i], k);
        m = fmaxf(m, fabsf(v[k]));
      }
      m = fmaxf(m, swap8(m));                 // lane ^ 8
      m = fmaxf(m, __shfl_xor(m, 16, 64));    // lane ^ 16
      const uint32_t code = mx_scale_code(m);
      const uint32_t word = pack8_rtn(v, mx_inv_scale(code));
      if (L.valid) {
        const int64_t r = L.r0 + i;
        *reinterpret_cast<uint32_t *>(a.codes + r * (a.C / 2) + L.c0 / 2) = word;
        if (first) a.scales[r * (a.C / 32) + L.c0 / 32] = (uint8_t)code;
      }
    }
  } else {
    const bool first = (lane & 1u) == 0u;  // even row group: first half of its block
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float v[16];
      float m = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        v[i] = bf16_at(raw[i], j);
        m = fmaxf(m, fabsf(v[i]));
      }
      m = fmaxf(m, __shfl_xor(m, 1, 64));  // lane ^ 1
      const uint32_t code = mx_scale_code(m);
      const float inv = mx_inv_scale(code);
      uint2 words;
      words.x = pack8_rtn(v, inv);
      words.y = pack8_rtn(v + 8, inv);
      if (L.valid) {
        const int64_t c = L.c0 + j;
        *reinterpret_cast<uint2 *>(a.codes + c * (a.R / 2) + L.r0 / 2) = words;
        if (first) a.scales[c * (a.R / 32) + L.r0 / 32] = (uint8_t)code;
      }
    }
  }
}

// ------------------------------------------------------------------------
// dequantisation: one 32-element block per thread, y = e(code) * 2^(s - 127)
// (exact in binary32 for the codes a finite bf16 input produces)
// ------------------------------------------------------------------------
__global__ __launch_bounds__(256) void mx_dequant_kernel(MxDequantArgs a) {
  const int64_t nb = a.rows * (a.cols / 32);
  for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nb; b += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = b / (a.cols / 32), cb = b % (a.cols / 32);
    const uint4 q = *reinterpret_cast<const uint4 *>(a.codes + r * (a.cols / 2) + cb * 16);
    const uint32_t code = a.scales[r * (a.cols / 32) + cb];
    // X = 2^(code - 127): the bit pattern code << 23, except code 0, 2^-127 (subnormal)
    const float s = code ? __uint_as_float(code << 23) : 5.877471754111438e-39f;
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
    float4 *dst = reinterpret_cast<float4 *>(a.y + r * a.ld_y + cb * 32);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const auto e0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[d], 1.0f, 0);
      const auto e1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[d], 1.0f, 1);
      const auto e2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[d], 1.0f, 2);
      const auto e3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[d], 1.0f, 3);
      dst[2 * d] = make_float4(e0[0] * s, e0[1] * s, e1[0] * s, e1[1] * s);
      dst[2 * d + 1] = make_float4(e2[0] * s, e2[1] * s, e3[0] * s, e3[1] * s);
    }
  }
}

// ------------------------------------------------------------------------
// GEMM.  MFMA operand mapping (32x32x64, FP4 A and B, E8M0 scales): lane l
// supplies row (A) / column (B) l % 32 and the 32 consecutive k of block
// 32 (l / 32) within the 64-wide K-step, as 16 bytes of packed codes (the
// instruction reads four registers for FP4), plus that block's scale in byte 0
// of its scale operand.  A and B use the same k assignment, so every k of the
// step is summed once.  Output: the usual 32x32 fp32 accumulator layout.
// ------------------------------------------------------------------------
__device__ __forceinline__ float16v mx_mfma(const uint4 &a, const uint4 &b, uint32_t sa, uint32_t sb,
                                            const float16v &c) {
  const int8v A = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
  const int8v B = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, B, c, 4, 4, 0, (int)sa, 0, (int)sb);
}

__device__ __forceinline__ void mx_store(const MxGemmArgs &g, int64_t m, int64_t n, float v) {
  if (g.c_bf16) {
    const uint32_t u = __float_as_uint(v);
    reinterpret_cast<uint16_t *>(g.c)[m * g.ldc + n] = (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
  } else {
    reinterpret_cast<float *>(g.c)[m * g.ldc + n] = v;
  }
}

// Any shape (K a multiple of 32): 128x128 tiles, 4 waves as 2 x 2, each wave
// 64x64 as 2 x 2 MFMA blocks; fragments are read straight from global memory,
// rows past M/N and k past K read as zero codes.
__global__ __launch_bounds__(256) void mx_gemm_generic_kernel(MxGemmArgs g) {
  const int64_t tiles_n = (g.N + 127) / 128;
  const int64_t m0 = (int64_t)(blockIdx.x / tiles_n) * 128, n0 = (int64_t)(blockIdx.x % tiles_n) * 128;
  const uint32_t wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const uint32_t wm = wave >> 1, wn = wave & 1, lr = lane & 31, h = lane >> 5;
  float16v acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  for (int64_t k0 = 0; k0 < g.K; k0 += 64) {
    const int64_t kk = k0 + 32 * h;
    uint4 qa[2], qb[2];
    uint32_t sa[2], sb[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int64_t m = m0 + wm * 64 + i * 32 + lr;
      const bool ok = m < g.M && kk < g.K;
      qa[i] = ok ? *reinterpret_cast<const uint4 *>(g.a_codes + m * (g.K / 2) + kk / 2) : make_uint4(0u, 0u, 0u, 0u);
      sa[i] = ok ? g.a_scales[m * (g.K / 32) + kk / 32] : 127u;
      const int64_t n = n0 + wn * 64 + i * 32 + lr;
      const bool okb = n < g.N && kk < g.K;
      qb[i] = okb ? *reinterpret_cast<const uint4 *>(g.b_codes + n * (g.K / 2) + kk / 2) : make_uint4(0u, 0u, 0u, 0u);
      sb[i] = okb ? g.b_scales[n * (g.K / 32) + kk / 32] : 127u;
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = mx_mfma(qa[i], qb[j], sa[i], sb[j], acc[i][j]);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t n = n0 + wn * 64 + j * 32 + lr;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + wm * 64 + i * 32 + (r >> 2) * 8 + h * 4 + (r & 3);
        if (m < g.M && n < g.N) mx_store(g, m, n, acc[i][j][r]);
      }
    }
}

// ===========================================================================
// Fast path (M, N multiples of 256, K a multiple of 128): 256x256x128 tiles,
// four LDS stages filled by direct global->LDS transfers, up to three K-tiles
// ahead of the MFMAs.
//
// Stage layout (34 KiB): codes of the 256 A rows then the 256 B rows, 64
// bytes per row (one 128-wide K slice) in four 16-byte chunks stored at
// chunk ^ swz(row); then one dword of scales per row (the slice's four E8M0
// bytes, byte b = k-block b).  K-step s (0, 1) of a tile: lane-half h reads
// chunk 2s + h of its row and scale byte 2s + h.
//
// Each wave issues exactly ten transfers per K-tile (8 x 1 KiB of codes,
// 2 x 256 B of scales): waves 0-1 the A half of the stage, waves 2-3 the B
// half; the vmcnt waits of the main loop count on that.
// ===========================================================================
constexpr int kMxStageCodes = 512 * 64;
constexpr int kMxStageBytes = kMxStageCodes + 512 * 4;
constexpr int kMxStages = 4;

struct MxDma {
  const uint8_t *cbase, *sbase;
  uint32_t coff[8];  // per-lane global byte offsets at kt = 0
  uint32_t soff[2];
};

__device__ __forceinline__ void mx_issue(const MxDma &c, uint32_t lds_stage, uint32_t kt, uint32_t wave) {
#pragma unroll
  for (int t = 0; t < 8; ++t)
    dma16(c.cbase, c.coff[t] + kt * 64u, __builtin_amdgcn_readfirstlane(lds_stage + (wave * 8 + t) * 1024u));
#pragma unroll
  for (int t = 0; t < 2; ++t)
    dma4(c.sbase, c.soff[t] + kt * 4u,
         __builtin_amdgcn_readfirstlane(lds_stage + kMxStageCodes + (wave * 2 + t) * 256u));
}

// one K-step's fragments: codes of 4 A and 4 B row blocks
struct MxFrags {
  uint4 a[4], b[4];
};

__global__ __launch_bounds__(256) void mx_gemm_fast_kernel(MxGemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kMxStages * kMxStageBytes];
  int64_t m0, n0;
  tile_origin(g.M, g.N, xcd_tile(blockIdx.x, gridDim.x), m0, n0);
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const uint32_t wm = wave >> 1, wn = wave & 1, lr = lane & 31, h = lane >> 5;
  const uint32_t kbytes = (uint32_t)(g.K / 2), kblocks = (uint32_t)(g.K / 32);
  const uint32_t KT = (uint32_t)(g.K / 128);

  MxDma c;
  c.cbase = wave < 2 ? g.a_codes : g.b_codes;
  c.sbase = wave < 2 ? g.a_scales : g.b_scales;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const uint32_t q = (wave * 8 + t) * 64 + lane;  // 16-byte slot of the stage
    const uint32_t row = q >> 2;                      // 0..511: A rows then B rows
    const uint32_t chunk = (q & 3u) ^ swz(row);
    const uint32_t grow = (uint32_t)(row < 256 ? m0 + row : n0 + (row - 256));
    c.coff[t] = grow * kbytes + chunk * 16u;
  }
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const uint32_t row = (wave * 2 + t) * 64 + lane;  // scale dword slot = row
    const uint32_t grow = (uint32_t)(row < 256 ? m0 + row : n0 + (row - 256));
    c.soff[t] = grow * kblocks;
  }
  // this lane's fragment offsets within a stage
  uint32_t aoff[4][2], boff[4][2], asoff[4], bsoff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t ra = wm * 128 + i * 32 + lr, rb = 256 + wn * 128 + i * 32 + lr;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      aoff[i][s] = (ra * 4 + ((2 * s + h) ^ swz(ra))) * 16;
      boff[i][s] = (rb * 4 + ((2 * s + h) ^ swz(rb))) * 16;
    }
    asoff[i] = kMxStageCodes + ra * 4;
    bsoff[i] = kMxStageCodes + rb * 4;
  }

  float16v acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const uint32_t lds0 = lds_addr(lds), klast = KT - 1;
  mx_issue(c, lds0, 0, wave);
  mx_issue(c, lds0 + kMxStageBytes, 1 < klast ? 1 : klast, wave);
  mx_issue(c, lds0 + 2 * kMxStageBytes, 2 < klast ? 2 : klast, wave);
  NVFP4_WAIT_VMCNT(20);  // this wave's transfers of tile 0 are done
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");

  MxFrags f0, f1;
  uint32_t sw_a[4], sw_b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f0.a[i] = *reinterpret_cast<const uint4 *>(lds + aoff[i][0]);
    f0.b[i] = *reinterpret_cast<const uint4 *>(lds + boff[i][0]);
    sw_a[i] = *reinterpret_cast<const uint32_t *>(lds + asoff[i]);
    sw_b[i] = *reinterpret_cast<const uint32_t *>(lds + bsoff[i]);
  }

  for (uint32_t kt = 0; kt < KT; ++kt) {
    const uint8_t *base = lds + (kt & 3u) * kMxStageBytes;
    // K-step 1 of this tile: its codes are read while K-step 0 multiplies
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f1.a[i] = *reinterpret_cast<const uint4 *>(base + aoff[i][1]);
      f1.b[i] = *reinterpret_cast<const uint4 *>(base + boff[i][1]);
    }
    uint32_t s0a[4], s0b[4], s1a[4], s1b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s0a[i] = sw_a[i] >> (8 * h);
      s1a[i] = sw_a[i] >> (8 * (2 + h));
      s0b[i] = sw_b[i] >> (8 * h);
      s1b[i] = sw_b[i] >> (8 * (2 + h));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mx_mfma(f0.a[i], f0.b[j], s0a[i], s0b[j], acc[i][j]);

    NVFP4_WAIT_LGKM0();    // this wave's reads of the tile are complete
    NVFP4_WAIT_VMCNT(10);  // this wave's transfers of tile kt+1 are done (kt+2's may be in flight)
    __builtin_amdgcn_s_barrier();  // every wave's: tile kt+1 is in LDS, stage (kt+3)%4 is free
    asm volatile("" ::: "memory");
    mx_issue(c, lds0 + ((kt + 3) & 3u) * kMxStageBytes, kt + 3 < klast ? kt + 3 : klast, wave);
    // K-step 0 of tile kt+1 (on the last tile from a stale stage; not used)
    const uint8_t *nbase = lds + ((kt + 1) & 3u) * kMxStageBytes;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f0.a[i] = *reinterpret_cast<const uint4 *>(nbase + aoff[i][0]);
      f0.b[i] = *reinterpret_cast<const uint4 *>(nbase + boff[i][0]);
      sw_a[i] = *reinterpret_cast<const uint32_t *>(nbase + asoff[i]);
      sw_b[i] = *reinterpret_cast<const uint32_t *>(nbase + bsoff[i]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mx_mfma(f1.a[i], f1.b[j], s1a[i], s1b[j], acc[i][j]);
  }
  NVFP4_WAIT_VMCNT(0);  // the clamped transfers of the last iterations

  // Non-temporal C stores, as in the NVFP4 GEMM: C goes to HBM while this
  // MFMA-bound kernel runs, so the next kernel does not pay for write-back.
  uint32_t ldc = (uint32_t)g.ldc;
  asm volatile("" : "+s"(ldc));
  if (g.c_bf16) {
    uint16_t *ct = reinterpret_cast<uint16_t *>(g.c) + m0 * g.ldc + n0;
    asm volatile("" : "+s"(ct));
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const uint32_t m = wm * 128 + i * 32 + (r >> 2) * 8 + h * 4 + (r & 3), n = wn * 128 + j * 32 + lr;
          const uint32_t u = __float_as_uint(acc[i][j][r]);
          __builtin_nontemporal_store((uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16), &ct[m * ldc + n]);
        }
  } else {
    float *ct = reinterpret_cast<float *>(g.c) + m0 * g.ldc + n0;
    asm volatile("" : "+s"(ct));
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const uint32_t m = wm * 128 + i * 32 + (r >> 2) * 8 + h * 4 + (r & 3), n = wn * 128 + j * 32 + lr;
          __builtin_nontemporal_store(acc[i][j][r], &ct[m * ldc + n]);
        }
  }
}

// ------------------------------------------------------------------------
// host launchers
// ------------------------------------------------------------------------
hipError_t launch_mx_quantize(const MxQuantArgs &a, int geom, hipStream_t s) {
  const dim3 grid(quant_tiles(a.R, a.C)), block(kQThreads);
  if (geom == G_ROW)
    hipLaunchKernelGGL((mx_quantize_kernel<G_ROW>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((mx_quantize_kernel<G_COL>), grid, block, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_mx_dequantize(const MxDequantArgs &a, hipStream_t s) {
  int64_t blocks = (a.rows * (a.cols / 32) + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(mx_dequant_kernel, dim3((uint32_t)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

// 256-aligned M and N, K a multiple of 128, and operands whose byte offsets
// fit the 32-bit transfer offsets
static bool mx_gemm_fast_ok(const MxGemmArgs &g) {
  return g.M % 256 == 0 && g.N % 256 == 0 && g.K % 128 == 0 && g.K >= 128 &&
         g.M * (g.K / 2) + g.K < ((int64_t)1 << 32) && g.N * (g.K / 2) + g.K < ((int64_t)1 << 32);
}

hipError_t launch_mx_gemm(const MxGemmArgs &g, hipStream_t s) {
  if (mx_gemm_fast_ok(g) && !getenv("NVFP4_GEMM_GENERIC")) {
    const uint32_t tiles = (uint32_t)((g.M / 256) * (g.N / 256));
    hipLaunchKernelGGL(mx_gemm_fast_kernel, dim3(tiles), dim3(256), 0, s, g);
  } else {
    const int64_t tiles = ((g.M + 127) / 128) * ((g.N + 127) / 128);
    hipLaunchKernelGGL(mx_gemm_generic_kernel, dim3((uint32_t)tiles), dim3(256), 0, s, g);
  }
  return hipGetLastError();
}

}  // namespace nvfp4
