// Kernel argument blocks and launch helpers shared by the host API and the
// kernel translation units of libnvfp4.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

// Geometry of one quantised output (block shape and storage orientation).
enum Geom : int {
  G_NONE = 0,
  G_ROW = 1,    // 1D blocks of 16 along the contiguous dim, stored [R][C/2]
  G_COL = 2,    // 1D blocks of 16 along rows, stored transposed [C][R/2]
  G_TILE = 3,   // 16x16 tiles, stored [R][C/2], scales [R/16][C/16]
  G_TILE_T = 4  // 16x16 tiles, stored [C][R/2], scales [C/16][R/16]
};

// Which maximum an output's global scale is taken over.
enum AmaxMode : int {
  AM_PLAIN = 0,    // max |x|
  AM_RHT_COL = 1,  // max |RHT along rows (groups of 16 rows)|: column-blocked outputs
  AM_RHT_ROW = 2   // max |RHT along cols (groups of 16 cols)|: row-blocked outputs
};

constexpr int kQTileR = 128;  // rows per quantise workgroup tile
constexpr int kQTileC = 256;  // cols per quantise workgroup tile
constexpr int kQThreads = 256;
constexpr int kMaxParts = 1024;  // partial maxima per amax mode

// Quantise workspace: partial maxima [3][kMaxParts] floats.
constexpr size_t kWsBytes = sizeof(float) * 3 * kMaxParts;

struct OutArgs {
  uint8_t *codes;
  uint8_t *scales;
  float *S_out;
  float *amax_out;
  const float *amax_in;  // the output's maximum when given by the caller, else null (partials are reduced)
  uint64_t sr_seed;
  int amax_mode;
  int pad;
};

struct QuantArgs {
  const uint16_t *x;
  int64_t R, C, ld;
  const float *partials;  // [3][kMaxParts]
  int nparts;
  uint32_t mask_rows;  // RHT sign mask for transforms along rows (column blocks)
  uint32_t mask_cols;  // RHT sign mask for transforms along cols (row blocks)
  OutArgs o[2];
};

struct AmaxArgs {
  const uint16_t *x;
  int64_t R, C, ld;
  float *partials;  // [3][kMaxParts]
  uint32_t mask_rows;
  uint32_t mask_cols;
};

struct DequantArgs {
  const uint8_t *codes;
  const uint8_t *scales;
  const float *S;
  float *y;
  int64_t rows, cols, ld_y;
  int scale_kind;
};

struct GemmArgs {
  const uint8_t *a_codes;
  const uint8_t *a_scales;
  const float *a_S;
  const uint8_t *b_codes;
  const uint8_t *b_scales;
  const float *b_S;
  void *c;
  int64_t M, N, K, ldc;
  int a_kind, b_kind;  // 0 = 1D scales, 1 = 2D scales
  int c_bf16;
  // producer-fused maxima of the bf16 output (null: not wanted); bit patterns
  // of non-negative floats, combined with atomic maxima
  unsigned int *amax_plain;
  unsigned int *amax_rht;
  uint32_t rht_mask;  // RHT sign mask of the 16-row groups (amax_rht)
};

// MXFP4 (OCP MX v1.0): 32-element blocks with an E8M0 scale, no per-tensor scale
struct MxQuantArgs {
  const uint16_t *x;
  int64_t R, C, ld;
  uint8_t *codes;   // ROW: [R][C/2]; COL: [C][R/2]
  uint8_t *scales;  // ROW: [R][C/32]; COL: [C][R/32]
};

struct MxDequantArgs {
  const uint8_t *codes;
  const uint8_t *scales;
  float *y;
  int64_t rows, cols, ld_y;
};

struct MxGemmArgs {
  const uint8_t *a_codes;
  const uint8_t *a_scales;
  const uint8_t *b_codes;
  const uint8_t *b_scales;
  void *c;
  int64_t M, N, K, ldc;
  int c_bf16;
};

hipError_t launch_mx_quantize(const MxQuantArgs &a, int geom, hipStream_t s);
hipError_t launch_mx_dequantize(const MxDequantArgs &a, hipStream_t s);
hipError_t launch_mx_gemm(const MxGemmArgs &g, hipStream_t s);

// host launchers (one per translation unit); return hipError_t of the launch
hipError_t launch_amax(const AmaxArgs &a, bool plain, bool rht_col, bool rht_row, int nparts, hipStream_t s);
hipError_t launch_quantize(const QuantArgs &a, int g0, bool rht0, bool sr0, int g1, bool rht1, bool sr1,
                           hipStream_t s, bool *supported);
// two quantise calls, each with one RHT column output (sra, srb: stochastic
// rounding), as one amax launch and one quantise launch
hipError_t launch_quantize_batch2(const AmaxArgs &aa, const QuantArgs &qa, bool sra, const AmaxArgs &ab,
                                  const QuantArgs &qb, bool srb, hipStream_t s);
int quant_tiles(int64_t R, int64_t C);
hipError_t launch_dequantize(const DequantArgs &a, hipStream_t s);
// GEMM workspace (stream-K path): kGemmMaxCUs flag words, an error word, then
// from byte kGemmWsSlots one fp32 256x256 partial per compute unit.
constexpr int kGemmMaxCUs = 1024;
constexpr size_t kGemmWsSlots = 8192;
constexpr size_t kGemmSlotBytes = 256 * 256 * 4;
size_t gemm_workspace_bytes(int cus);
hipError_t launch_gemm(const GemmArgs &a, void *workspace, size_t workspace_bytes, hipStream_t s);
hipError_t launch_codec_selftest(int which, const float *in, const uint16_t *u16, uint8_t *out, int64_t n,
                                 hipStream_t s);

}  // namespace nvfp4
