// NVFP4-operand GEMM for gfx950: C[m][n] = (sum_k A^[m][k] B^[n][k]) / (S_A S_B)
// with A^ = e(code) * s_b, both operands stored K-contiguous ("TN").
//
// Method: NVFP4 pretraining news page (zubnet.ai), paragraphs 1-2 -- the 4-bit
// GEMMs consume E2M1 codes with E4M3 block scales and FP32 per-tensor scales.
//
// Design.  Packed codes (4 bits/element) and scale bytes are staged in LDS, so
// a K-tile costs 0.5625 B/element of global and LDS traffic.  Each wave reads
// its MFMA fragments straight from the packed tile and expands them in
// registers: the gfx950 FP4->FP16 conversion gives e(code), one packed FP16
// multiply applies the block scale.  e * s_b has at most 6 significant bits
// and lies in [2^-10, 2688], so the FP16 operand is exact and the
// v_mfma_f32_32x32x16_f16 products are exact; accumulation is FP32 and the
// per-tensor scales are applied once in the epilogue.
//
// Fragment/K mapping: within a 64-wide K-tile, lane-half h (lane / 32) of an
// MFMA in sub-step s holds the 8 consecutive k = 32h + 8s + [0, 8), i.e. one
// dword of codes at byte 16h + 4s of the row's 32-byte K-tile slice, under the
// block scale of k-block 2h + s/2.  A and B use the same mapping, so every k
// of the tile is summed exactly once.
#include "nvfp4_device.hpp"
#include "nvfp4_kernels.hpp"

namespace nvfp4 {

typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef _Float16 half8v __attribute__((ext_vector_type(8)));
typedef float float16v __attribute__((ext_vector_type(16)));

constexpr int kGThreads = 256;  // 4 waves as 2 x 2
constexpr int kBK = 64;         // K per tile
constexpr int kRowBytes = 48;   // LDS bytes per row: 32 bytes of codes + 16 pad (bank spread)

// 8 codes in `q` with block scale `s` -> 8 exact fp16 operand values
__device__ __forceinline__ half8v expand8(uint32_t q, _Float16 s) {
  const half2v sv = {s, s};
  const half2v p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, 1.0f, 0) * sv;
  const half2v p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, 1.0f, 1) * sv;
  const half2v p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, 1.0f, 2) * sv;
  const half2v p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, 1.0f, 3) * sv;
  half8v r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

__device__ __forceinline__ _Float16 scale_f16(uint32_t scales4, int blk) {
  // E4M3 byte -> fp32 (exact) -> fp16 (exact: 2^-9 .. 448 are fp16 normals)
  const uint32_t b = (scales4 >> (8 * blk)) & 0xFFu;
  return (_Float16)e4m3_value(b);
}

template <int TM, int TN>
struct GemmTile {
  static constexpr int BM = 64 * TM;
  static constexpr int BN = 64 * TN;
  static constexpr int ROWS = BM + BN;
};

// Global -> register staging of one K-tile: 32 bytes of codes and 4 scale bytes
// for each of the BM + BN rows.  Rows past M/N and k-blocks past K read as 0.
template <int TM, int TN>
struct Stage {
  static constexpr int ROWS = GemmTile<TM, TN>::ROWS;
  static constexpr int CHUNKS = ROWS * 4;  // 8-byte chunks of codes
  static constexpr int CPT = CHUNKS / kGThreads;
  static constexpr int SPT = (ROWS + kGThreads - 1) / kGThreads;
  uint2 code[CPT];
  uint32_t scale[SPT];
};

template <int TM, int TN>
__device__ __forceinline__ void stage_load(const GemmArgs &g, int64_t m0, int64_t n0, int64_t kt, Stage<TM, TN> &st) {
  constexpr int BM = GemmTile<TM, TN>::BM, ROWS = GemmTile<TM, TN>::ROWS;
  const int64_t kblocks = g.K / 16;
#pragma unroll
  for (int i = 0; i < Stage<TM, TN>::CPT; ++i) {
    const int c = threadIdx.x + i * kGThreads;
    const int row = c >> 2, part = c & 3;  // part = k-block within the tile
    const bool isA = row < BM;
    const int64_t grow = isA ? m0 + row : n0 + (row - BM);
    const int64_t lim = isA ? g.M : g.N;
    const int64_t kb = kt * 4 + part;
    uint2 v = make_uint2(0u, 0u);
    if (grow < lim && kb < kblocks) {
      const uint8_t *base = isA ? g.a_codes : g.b_codes;
      v = *reinterpret_cast<const uint2 *>(base + grow * (g.K / 2) + kb * 8);
    }
    st.code[i] = v;
  }
#pragma unroll
  for (int i = 0; i < Stage<TM, TN>::SPT; ++i) {
    const int row = threadIdx.x + i * kGThreads;
    uint32_t w = 0;
    if (row < ROWS) {
      const bool isA = row < BM;
      const int64_t grow = isA ? m0 + row : n0 + (row - BM);
      const int64_t lim = isA ? g.M : g.N;
      if (grow < lim) {
        const uint8_t *sc = isA ? g.a_scales : g.b_scales;
        const int kind = isA ? g.a_kind : g.b_kind;
        const uint8_t *p = kind == 0 ? sc + grow * kblocks : sc + (grow / 16) * kblocks;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int64_t kb = kt * 4 + b;
          if (kb < kblocks) w |= (uint32_t)p[kb] << (8 * b);
        }
      }
    }
    st.scale[i] = w;
  }
}

template <int TM, int TN>
__device__ __forceinline__ void stage_store(uint8_t *lcodes, uint32_t *lscales, const Stage<TM, TN> &st) {
  constexpr int ROWS = GemmTile<TM, TN>::ROWS;
#pragma unroll
  for (int i = 0; i < Stage<TM, TN>::CPT; ++i) {
    const int c = threadIdx.x + i * kGThreads;
    const int row = c >> 2, part = c & 3;
    *reinterpret_cast<uint2 *>(lcodes + row * kRowBytes + part * 8) = st.code[i];
  }
#pragma unroll
  for (int i = 0; i < Stage<TM, TN>::SPT; ++i) {
    const int row = threadIdx.x + i * kGThreads;
    if (row < ROWS) lscales[row] = st.scale[i];
  }
}

template <int TM, int TN>
__global__ __launch_bounds__(kGThreads) void gemm_kernel(GemmArgs g) {
  constexpr int BM = GemmTile<TM, TN>::BM, BN = GemmTile<TM, TN>::BN, ROWS = GemmTile<TM, TN>::ROWS;
  __shared__ __attribute__((aligned(16))) uint8_t lcodes[2][ROWS * kRowBytes];
  __shared__ uint32_t lscales[2][ROWS];

  const int64_t tiles_n = (g.N + BN - 1) / BN;
  const uint32_t tile = xcd_tile(blockIdx.x, gridDim.x);
  const int64_t m0 = (int64_t)(tile / tiles_n) * BM;
  const int64_t n0 = (int64_t)(tile % tiles_n) * BN;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int lrow = lane & 31, half = lane >> 5;

  float16v acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int64_t KT = (g.K + kBK - 1) / kBK;
  Stage<TM, TN> st;
  stage_load<TM, TN>(g, m0, n0, 0, st);
  stage_store<TM, TN>(lcodes[0], lscales[0], st);
  __syncthreads();

  for (int64_t kt = 0; kt < KT; ++kt) {
    const int buf = (int)(kt & 1);
    if (kt + 1 < KT) stage_load<TM, TN>(g, m0, n0, kt + 1, st);

    // fragments of this wave for the whole K-tile: 16 bytes of codes per row tile
    uint4 qa[TM], qb[TN];
    uint32_t sa[TM], sb[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int row = wm * (TM * 32) + i * 32 + lrow;
      qa[i] = *reinterpret_cast<const uint4 *>(&lcodes[buf][row * kRowBytes + half * 16]);
      sa[i] = lscales[buf][row];
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int row = BM + wn * (TN * 32) + j * 32 + lrow;
      qb[j] = *reinterpret_cast<const uint4 *>(&lcodes[buf][row * kRowBytes + half * 16]);
      sb[j] = lscales[buf][row];
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int blk = 2 * half + (s >> 1);
      half8v fa[TM], fb[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const uint32_t q = s == 0 ? qa[i].x : s == 1 ? qa[i].y : s == 2 ? qa[i].z : qa[i].w;
        fa[i] = expand8(q, scale_f16(sa[i], blk));
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const uint32_t q = s == 0 ? qb[j].x : s == 1 ? qb[j].y : s == 2 ? qb[j].z : qb[j].w;
        fb[j] = expand8(q, scale_f16(sb[j], blk));
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }

    if (kt + 1 < KT) stage_store<TM, TN>(lcodes[buf ^ 1], lscales[buf ^ 1], st);
    __syncthreads();
  }

  // epilogue: C = acc / (S_A S_B)
  const float inv = 1.0f / (*g.a_S * *g.b_S);
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int64_t n = n0 + wn * (TN * 32) + j * 32 + lrow;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + wm * (TM * 32) + i * 32 + (r >> 2) * 8 + half * 4 + (r & 3);
        if (m < g.M && n < g.N) {
          const float v = acc[i][j][r] * inv;
          if (g.c_bf16) {
            const uint32_t u = __float_as_uint(v);
            const uint16_t h = (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);  // nearest-even
            reinterpret_cast<uint16_t *>(g.c)[m * g.ldc + n] = h;
          } else {
            reinterpret_cast<float *>(g.c)[m * g.ldc + n] = v;
          }
        }
      }
    }
}

hipError_t launch_gemm(const GemmArgs &g, hipStream_t s) {
  constexpr int TM = 4, TN = 4;
  constexpr int BM = GemmTile<TM, TN>::BM, BN = GemmTile<TM, TN>::BN;
  const int64_t tiles = ((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN);
  hipLaunchKernelGGL((gemm_kernel<TM, TN>), dim3((uint32_t)tiles), dim3(kGThreads), 0, s, g);
  return hipGetLastError();
}

}  // namespace nvfp4
