// NVFP4 quantisation kernels for gfx950: the per-tensor amax pass and the
// fused (RHT +) block-scale + round + pack pass with one or two outputs from a
// single read of the input; dequantisation; the codec self-test kernel.  Their
// device code is in quantize_device.hpp.
//
// Method: NVFP4 pretraining news page (zubnet.ai), paragraph 2.
#include "quantize_device.hpp"

namespace nvfp4 {

// amax pass: workgroup `part` of `nparts` takes tiles part, part + nparts, ...
// and writes its partial maxima to slot `part`
template <bool PLAIN, bool RC, bool RR>
__device__ __forceinline__ void amax_body(const AmaxArgs &a, uint32_t part, uint32_t nparts) {
  const int64_t ntiles = ((a.R + kQTileR - 1) / kQTileR) * ((a.C + kQTileC - 1) / kQTileC);
  float m_plain = 0.0f, m_rc = 0.0f, m_rr = 0.0f;
  for (int64_t t = part; t < ntiles; t += nparts) {
    const Lane L = lane_coords((uint32_t)t, a.R, a.C);
    if (!L.valid) continue;  // pairs of lanes are valid together (C % 16 == 0)
    uint4 raw[16];
    load_micro_tile(a.x, a.ld, L, raw);
    tile_maxes<PLAIN, RC, RR>(raw, L, a.mask_rows, a.mask_cols, m_plain, m_rc, m_rr);
  }
  write_partials<PLAIN, RC, RR>(m_plain, m_rc, m_rr, a.partials, part);
}

template <bool PLAIN, bool RC, bool RR>
__global__ __launch_bounds__(kQThreads) void amax_kernel(AmaxArgs a) {
  amax_body<PLAIN, RC, RR>(a, blockIdx.x, gridDim.x);
}

// The RHT-column amax passes of two tensors in one launch: the first na
// workgroups serve a, the rest b.
__global__ __launch_bounds__(kQThreads) void amax_batch2_kernel(AmaxArgs a, AmaxArgs b, uint32_t na) {
  if (blockIdx.x < na)
    amax_body<false, true, false>(a, blockIdx.x, na);
  else
    amax_body<false, true, false>(b, blockIdx.x - na, gridDim.x - na);
}

// Quantise pass: one micro-tile per lane, global scales from the partial
// maxima of the amax pass.  Instantiations with a column output in the RHT
// domain are held to five waves per SIMD (at most 102 VGPRs), or four (128)
// when stochastic rounding is involved: they fit without spilling, and the
// extra waves hide more load latency than the larger register budget the
// compiler would otherwise take buys (measured); the others keep their
// allocation, which some of them need to avoid spills.
template <int G0, bool RHT0, bool SR0, int G1, bool RHT1, bool SR1, bool STAGE>
constexpr int quant_waves_per_simd() {
  return ((G0 == G_COL && RHT0) || (G1 == G_COL && RHT1)) ? ((SR0 || SR1 || STAGE) ? 4 : 5) : 1;
}
// With STAGE (row + column pairs of at least 512 tiles) the row output goes
// through LDS and is stored as whole 128-byte row segments (row_stage_flush);
// measured faster on every such pair (activation row + column 44.85 -> 43.17
// us; 16384 x 5120 row + column with the RHT 87.7 -> 84.7 us), although the
// stage's registers hold the RHT-column RTN pairs to four waves per SIMD.  On
// small tensors the extra barrier costs more than it saves.
// quantise pass for one tile of the tensor (in the order of quant_tiles)
template <int G0, bool RHT0, bool SR0, int G1, bool RHT1, bool SR1, bool STAGE = false>
__device__ __forceinline__ void quantize_body(const QuantArgs &a, uint32_t tile) {
  constexpr int NOUT = (G1 == G_NONE) ? 1 : 2;
  __shared__ float s_lut[2][128];
  __shared__ float s_S[2];
  // tiles in row-major order (see quant_tiles); 256 x 128 ones for a single column output
  constexpr bool TALL = G0 == G_COL && G1 == G_NONE;
  const Lane L = TALL ? lane_coords_tall(tile, a.R, a.C) : lane_coords(tile, a.R, a.C);
  float pm[2][4];
  load_partials<NOUT>(a, (uint32_t)a.nparts, pm);
  uint4 raw[16];
  load_micro_tile_any(a.x, a.ld, L, raw);
  quant_setup<NOUT>(a, pm, s_S, s_lut, tile == 0);
  if constexpr (STAGE) {
    __shared__ RowStage st;
    if (L.valid) quant_tile<G0, RHT0, SR0, G1, RHT1, SR1>(raw, L, a, s_S, s_lut, &st);
    __syncthreads();  // every lane's row codes and scales are in the stage
    const int64_t ntc = (a.C + kQTileC - 1) / kQTileC;
    row_stage_flush(&st, a.o[0], (int64_t)(tile / ntc) * kQTileR, (int64_t)(tile % ntc) * kQTileC, a.R, a.C);
  } else {
    if (!L.valid) return;
    quant_tile<G0, RHT0, SR0, G1, RHT1, SR1>(raw, L, a, s_S, s_lut);
  }
}

template <int G0, bool RHT0, bool SR0, int G1, bool RHT1, bool SR1, bool STAGE = false>
__global__ __launch_bounds__(kQThreads) __attribute__((amdgpu_waves_per_eu(
    quant_waves_per_simd<G0, RHT0, SR0, G1, RHT1, SR1, STAGE>()))) void quantize_kernel(QuantArgs a) {
  quantize_body<G0, RHT0, SR0, G1, RHT1, SR1, STAGE>(a, blockIdx.x);
}

// The quantise passes of two tensors, each with one RHT column output (the
// Wgrad operands), in one launch.  Workgroups alternate between the two
// (the first 2 min(ta, tb) block indices), the larger one's remaining tiles
// come last, so every CU runs both at once.  Measured on dY (SR) and X (RTN)
// of 8192 x 5120, the pass takes about as long as the two separate ones: the
// RTN input's workgroups run at four waves per SIMD here (five alone), which
// takes back what running beside the ALU-bound SR pass gains.  The batch
// saves the two kernel boundaries and runs both amax passes as one launch.
template <bool SRA, bool SRB>
__global__ __launch_bounds__(kQThreads) __attribute__((amdgpu_waves_per_eu(
    quant_waves_per_simd<G_COL, true, SRA || SRB, G_NONE, false, false, false>()))) void quantize_batch2_kernel(
    QuantArgs a, QuantArgs b, uint32_t ta, uint32_t tb) {
  const uint32_t i = blockIdx.x, m = ta < tb ? ta : tb;
  bool second;
  uint32_t t;
  if (i < 2 * m) {
    second = (i & 1u) != 0;
    t = i >> 1;
  } else {
    second = tb > ta;
    t = i - m;
  }
  if (!second)
    quantize_body<G_COL, true, SRA, G_NONE, false, false>(a, t);
  else
    quantize_body<G_COL, true, SRB, G_NONE, false, false>(b, t);
}

// 2D and 2D_T outputs, both rounded to nearest, from the same maximum (so
// under the same global scale): the codes are computed once per element.
// With STAGE (from 512 tiles up) the 2D codes go through LDS as the row output
// of the row + column kernels does (weight 2D + 2D_T 98.0 -> 92.9 us).
template <bool STAGE>
__global__ __launch_bounds__(kQThreads) void quantize_tile_pair_kernel(QuantArgs a) {
  __shared__ float s_lut[2][128];
  __shared__ float s_S[2];
  const Lane L = lane_coords(blockIdx.x, a.R, a.C);
  float pm[2][4];
  load_partials<2>(a, (uint32_t)a.nparts, pm);
  uint4 raw[16];
  load_micro_tile_any(a.x, a.ld, L, raw);
  quant_setup<2>(a, pm, s_S, s_lut, blockIdx.x == 0);
  if constexpr (STAGE) {
    __shared__ RowStage st;
    if (L.valid) tile_pair_rtn(raw, L, a.o[0], a.o[1], s_S[0], s_lut[0], a.R, a.C, &st);
    __syncthreads();  // every lane's 2D codes are in the stage
    const int64_t ntc = (a.C + kQTileC - 1) / kQTileC;
    row_stage_flush<false>(&st, a.o[0], (int64_t)(blockIdx.x / ntc) * kQTileR, (int64_t)(blockIdx.x % ntc) * kQTileC,
                           a.R, a.C);
  } else {
    if (!L.valid) return;
    tile_pair_rtn(raw, L, a.o[0], a.o[1], s_S[0], s_lut[0], a.R, a.C);
  }
}

// ------------------------------------------------------------------------
// dequantisation: one 16-element block per thread
// ------------------------------------------------------------------------
// 8 codes (nibble k = element k) -> (e * s) / S; the product is exact and the
// division rounds once
__device__ __forceinline__ void dequant8(uint32_t word, float s, float S, float out[8]) {
  const auto e0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 0);
  const auto e1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 1);
  const auto e2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 2);
  const auto e3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 3);
  const float e[8] = {e0[0], e0[1], e1[0], e1[1], e2[0], e2[1], e3[0], e3[1]};
#pragma unroll
  for (int k = 0; k < 8; ++k) out[k] = (e[k] * s) / S;
}

__global__ __launch_bounds__(256) void dequant_kernel(DequantArgs a) {
  const int64_t nb = a.rows * (a.cols / 16);
  const float S = *a.S;
  for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nb; b += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = b / (a.cols / 16), cb = b % (a.cols / 16);
    const uint2 q = *reinterpret_cast<const uint2 *>(a.codes + r * (a.cols / 2) + cb * 8);
    const uint8_t sc = a.scale_kind == 0 ? a.scales[r * (a.cols / 16) + cb] : a.scales[(r / 16) * (a.cols / 16) + cb];
    const float s = e4m3_value(sc);
    float out[16];
    dequant8(q.x, s, S, out);
    dequant8(q.y, s, S, out + 8);
    float4 *dst = reinterpret_cast<float4 *>(a.y + r * a.ld_y + cb * 16);
#pragma unroll
    for (int k = 0; k < 4; ++k) dst[k] = make_float4(out[4 * k], out[4 * k + 1], out[4 * k + 2], out[4 * k + 3]);
  }
}

// ------------------------------------------------------------------------
// codec self-test
// ------------------------------------------------------------------------
__global__ void codec_selftest_kernel(int which, const float *in, const uint16_t *u16, uint8_t *out, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const float v = in[i];
    uint32_t c;
    if (which == 0)
      c = NVFP4_CVT_PK_FP4(0u, v, 0.0f, 0) & 0xFu;
    else if (which == 1)
      c = e2m1_sr_hw(v, u16[i], (int)(i & 1));
    else
      c = e4m3_encode(v);
    out[i] = (uint8_t)c;
  }
}

// ------------------------------------------------------------------------
// host launchers
// ------------------------------------------------------------------------
// Quantise workgroups take their tiles in row-major order, one per block
// index.  The tiles share no input, so dealing them to the XCDs in contiguous
// ranges (as the GEMM does, for L2 reuse) gains nothing here; measured, it was
// up to 5 % slower (2D + 2D_T outputs of a 5120 x 20480 weight), and other
// orders (column-major, bands of 4-16 tile rows or columns) were no faster.
int quant_tiles(int64_t R, int64_t C) {
  return (int)(((R + kQTileR - 1) / kQTileR) * ((C + kQTileC - 1) / kQTileC));
}

hipError_t launch_amax(const AmaxArgs &a, bool plain, bool rc, bool rr, int nparts, hipStream_t s) {
  const dim3 grid(nparts), block(kQThreads);
  const int key = (plain ? 1 : 0) | (rc ? 2 : 0) | (rr ? 4 : 0);
  switch (key) {
    case 1: hipLaunchKernelGGL((amax_kernel<true, false, false>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((amax_kernel<false, true, false>), grid, block, 0, s, a); break;
    case 3: hipLaunchKernelGGL((amax_kernel<true, true, false>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((amax_kernel<false, false, true>), grid, block, 0, s, a); break;
    case 5: hipLaunchKernelGGL((amax_kernel<true, false, true>), grid, block, 0, s, a); break;
    case 6: hipLaunchKernelGGL((amax_kernel<false, true, true>), grid, block, 0, s, a); break;
    case 7: hipLaunchKernelGGL((amax_kernel<true, true, true>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int G0, bool RHT0, bool SR0, int G1, bool RHT1, bool SR1>
static hipError_t launch_q(const QuantArgs &a, hipStream_t s) {
  if constexpr (G0 == G_ROW && G1 == G_COL) {
    if (quant_tiles(a.R, a.C) >= 512) {
      hipLaunchKernelGGL((quantize_kernel<G0, RHT0, SR0, G1, RHT1, SR1, true>), dim3(quant_tiles(a.R, a.C)),
                         dim3(kQThreads), 0, s, a);
      return hipGetLastError();
    }
  }
  const int tiles = (G0 == G_COL && G1 == G_NONE)
                        ? (int)(((a.R + kQTallR - 1) / kQTallR) * ((a.C + kQTallC - 1) / kQTallC))
                        : quant_tiles(a.R, a.C);
  hipLaunchKernelGGL((quantize_kernel<G0, RHT0, SR0, G1, RHT1, SR1>), dim3(tiles), dim3(kQThreads), 0, s, a);
  return hipGetLastError();
}

template <int G, bool RHT>
static hipError_t dispatch_single(const QuantArgs &a, bool sr, hipStream_t s) {
  return sr ? launch_q<G, RHT, true, G_NONE, false, false>(a, s) : launch_q<G, RHT, false, G_NONE, false, false>(a, s);
}

// {ROW, COL} pairs: g0 = ROW, g1 = COL
template <bool RHT0, bool RHT1>
static hipError_t dispatch_row_col(const QuantArgs &a, bool sr0, bool sr1, hipStream_t s) {
  if (!sr0 && !sr1) return launch_q<G_ROW, RHT0, false, G_COL, RHT1, false>(a, s);
  if (!sr0 && sr1) return launch_q<G_ROW, RHT0, false, G_COL, RHT1, true>(a, s);
  if (sr0 && !sr1) return launch_q<G_ROW, RHT0, true, G_COL, RHT1, false>(a, s);
  return launch_q<G_ROW, RHT0, true, G_COL, RHT1, true>(a, s);
}

hipError_t launch_quantize(const QuantArgs &a, int g0, bool rht0, bool sr0, int g1, bool rht1, bool sr1,
                           hipStream_t s, bool *supported) {
  *supported = true;
  if (g1 == G_NONE) {
    if (g0 == G_ROW) return rht0 ? dispatch_single<G_ROW, true>(a, sr0, s) : dispatch_single<G_ROW, false>(a, sr0, s);
    if (g0 == G_COL) return rht0 ? dispatch_single<G_COL, true>(a, sr0, s) : dispatch_single<G_COL, false>(a, sr0, s);
    if (g0 == G_TILE && !rht0) return dispatch_single<G_TILE, false>(a, sr0, s);
    if (g0 == G_TILE_T && !rht0) return dispatch_single<G_TILE_T, false>(a, sr0, s);
  } else if (g0 == G_ROW && g1 == G_COL) {
    if (!rht0 && !rht1) return dispatch_row_col<false, false>(a, sr0, sr1, s);
    if (!rht0 && rht1) return dispatch_row_col<false, true>(a, sr0, sr1, s);
    if (rht0 && !rht1) return dispatch_row_col<true, false>(a, sr0, sr1, s);
    return dispatch_row_col<true, true>(a, sr0, sr1, s);
  } else if (g0 == G_TILE && g1 == G_TILE_T && !rht0 && !rht1) {
    if (!sr0 && !sr1 && a.o[0].amax_in == a.o[1].amax_in && a.o[0].amax_mode == a.o[1].amax_mode) {
      if (quant_tiles(a.R, a.C) >= 512)
        hipLaunchKernelGGL(quantize_tile_pair_kernel<true>, dim3(quant_tiles(a.R, a.C)), dim3(kQThreads), 0, s, a);
      else
        hipLaunchKernelGGL(quantize_tile_pair_kernel<false>, dim3(quant_tiles(a.R, a.C)), dim3(kQThreads), 0, s, a);
      return hipGetLastError();
    }
    if (!sr0 && !sr1) return launch_q<G_TILE, false, false, G_TILE_T, false, false>(a, s);
    if (!sr0 && sr1) return launch_q<G_TILE, false, false, G_TILE_T, false, true>(a, s);
    if (sr0 && !sr1) return launch_q<G_TILE, false, true, G_TILE_T, false, false>(a, s);
    return launch_q<G_TILE, false, true, G_TILE_T, false, true>(a, s);
  }
  *supported = false;
  return hipErrorInvalidValue;
}

// The Wgrad operand pair: one amax launch (a's nparts workgroups, then b's)
// and one quantise launch (quantize_batch2_kernel).
hipError_t launch_quantize_batch2(const AmaxArgs &aa, const QuantArgs &qa, bool sra, const AmaxArgs &ab,
                                  const QuantArgs &qb, bool srb, hipStream_t s) {
  hipLaunchKernelGGL(amax_batch2_kernel, dim3((uint32_t)(qa.nparts + qb.nparts)), dim3(kQThreads), 0, s, aa, ab,
                     (uint32_t)qa.nparts);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const uint32_t ta = (uint32_t)(((qa.R + kQTallR - 1) / kQTallR) * ((qa.C + kQTallC - 1) / kQTallC));
  const uint32_t tb = (uint32_t)(((qb.R + kQTallR - 1) / kQTallR) * ((qb.C + kQTallC - 1) / kQTallC));
  const dim3 grid(ta + tb), block(kQThreads);
  if (sra && srb)
    hipLaunchKernelGGL((quantize_batch2_kernel<true, true>), grid, block, 0, s, qa, qb, ta, tb);
  else if (sra)
    hipLaunchKernelGGL((quantize_batch2_kernel<true, false>), grid, block, 0, s, qa, qb, ta, tb);
  else if (srb)
    hipLaunchKernelGGL((quantize_batch2_kernel<false, true>), grid, block, 0, s, qa, qb, ta, tb);
  else
    hipLaunchKernelGGL((quantize_batch2_kernel<false, false>), grid, block, 0, s, qa, qb, ta, tb);
  return hipGetLastError();
}

hipError_t launch_dequantize(const DequantArgs &a, hipStream_t s) {
  const int64_t nb = a.rows * (a.cols / 16);
  int64_t blocks = (nb + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(dequant_kernel, dim3((uint32_t)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_codec_selftest(int which, const float *in, const uint16_t *u16, uint8_t *out, int64_t n,
                                 hipStream_t s) {
  if (n == 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  hipLaunchKernelGGL(codec_selftest_kernel, dim3((uint32_t)blocks), dim3(256), 0, s, which, in, u16, out, n);
  return hipGetLastError();
}
}  // namespace nvfp4
