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
#include "gemm_device.hpp"
#include "nvfp4_device.hpp"
#include "nvfp4_kernels.hpp"

#include <stdlib.h>

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

// The epilogue's division by S_A S_B, without forming that product in
// binary32: it overflows when both per-tensor maxima are small (about 1e-16
// each) and underflows when both are large, although C itself is
// representable.  S_A S_B = m 2^e with m = ma mb in [1/4, 1) (frexp), so
// C = ldexp(acc * (1/m), -e): one rounded multiply (1/m lies in (1, 4]), then
// an exact power-of-two scaling whenever C is a normal binary32.
struct EpiScale {
  float inv_m;
  int neg_e;
};

__device__ __forceinline__ EpiScale epi_scale(const GemmArgs &g) {
  int ea, eb;
  const float ma = frexpf(*g.a_S, &ea), mb = frexpf(*g.b_S, &eb);
  EpiScale s;
  s.inv_m = 1.0f / (ma * mb);
  s.neg_e = -(ea + eb);
  return s;
}

__device__ __forceinline__ float epi_apply(float acc, const EpiScale &s) { return ldexpf(acc * s.inv_m, s.neg_e); }

__device__ __forceinline__ _Float16 scale_f16(uint32_t scales4, int blk) {
  // E4M3 byte -> fp32 (exact) -> fp16 (exact: 2^-9 .. 448 are fp16 normals)
  const uint32_t b = (scales4 >> (8 * blk)) & 0xFFu;
  return (_Float16)e4m3_value(b);
}

// ---------------------------------------------------------------------------
// Producer-fused maxima of a bf16 output (nvfp4_gemm_amax): the per-tensor
// maxima the quantisation of C needs, taken from the rounded outputs while
// they are in registers, so that the quantiser need not read C for them.
//   plain: max |c| over the stored bf16 values;
//   RHT along rows: max |H16 D c| / 4 over the aligned 16-row groups (the
//   transform a column-blocked quantisation of C applies; D from the mask).
// The transform of a 32x32 accumulator block is one product Z = T C on the
// bf16 MFMA (two 16-deep K-steps), T block-diagonal with two copies of H16 D.
// The accumulator layout (lane half h holds rows (r >> 2) 8 + 4h + (r & 3))
// serves directly as the K order of the B operand: K-step s takes r = 8s ..
// 8s + 7, i.e. the rows rho(k) = (k & 3) | (h << 2) | ((k >> 2) << 3) of
// group s, k = 8h + kk, and T's columns are permuted to match.  Products with
// +-1 are exact; the sums are fp32.  Each wave folds its maxima with one
// device-scope atomic maximum per tensor (bit patterns of non-negative floats
// order like the values).
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));

__device__ __forceinline__ uint32_t bf16_rne_bits(float v) {
  const uint32_t u = __float_as_uint(v);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// A operand of K-step s: lane l supplies row i = l % 32 of Z and k = 8 (l/32) + kk
__device__ __forceinline__ bf16x8v rht_rows_operand(uint32_t mask, uint32_t s, uint32_t lane) {
  const uint32_t i = lane & 31u, hh = lane >> 5;
  uint32_t w[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t pair = 0;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const uint32_t kk = 2 * q + e;
      const uint32_t rho = (kk & 3u) | (hh << 2) | ((kk >> 2) << 3);  // row of the 16-row group
      const uint32_t neg = (__builtin_popcount((i & 15u) & rho) + ((mask >> rho) & 1u)) & 1u;
      const uint32_t v = (i >> 4) == s ? (neg ? 0xBF80u : 0x3F80u) : 0u;
      pair |= v << (16 * e);
    }
    w[q] = pair;
  }
  return __builtin_bit_cast(bf16x8v, make_uint4(w[0], w[1], w[2], w[3]));
}

struct FusedMax {
  bf16x8v t0, t1;     // the transform's A operands (K-steps 0 and 1)
  uint32_t plain;     // max of |c| as bf16 magnitude bits
  float rht;          // max |H16 D c| (unnormalised)
};

__device__ __forceinline__ void fused_max_init(FusedMax &f, const GemmArgs &g, uint32_t lane) {
  f.plain = 0;
  f.rht = 0.0f;
  if (g.amax_rht) {
    f.t0 = rht_rows_operand(g.rht_mask, 0, lane);
    f.t1 = rht_rows_operand(g.rht_mask, 1, lane);
  }
}

// fold one 32x32 block's 16 rounded values (bf16 bit patterns) of this lane
__device__ __forceinline__ void fused_max_block(FusedMax &f, const GemmArgs &g, const uint32_t hb[16]) {
#pragma unroll
  for (int r = 0; r < 16; ++r) f.plain = max(f.plain, hb[r] & 0x7FFFu);
  if (g.amax_rht) {
    const bf16x8v b0 = __builtin_bit_cast(
        bf16x8v, make_uint4(hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16), hb[4] | (hb[5] << 16), hb[6] | (hb[7] << 16)));
    const bf16x8v b1 = __builtin_bit_cast(bf16x8v, make_uint4(hb[8] | (hb[9] << 16), hb[10] | (hb[11] << 16),
                                                              hb[12] | (hb[13] << 16), hb[14] | (hb[15] << 16)));
    float16v z;
#pragma unroll
    for (int r = 0; r < 16; ++r) z[r] = 0.0f;
    z = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.t0, b0, z, 0, 0, 0);
    z = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.t1, b1, z, 0, 0, 0);
#pragma unroll
    for (int r = 0; r < 16; ++r) f.rht = fmaxf(f.rht, fabsf(z[r]));
  }
}

__device__ __forceinline__ void fused_max_flush(const FusedMax &f, const GemmArgs &g) {
  uint32_t mp = f.plain;
  float mr = f.rht;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    mp = max(mp, (uint32_t)__shfl_xor((int)mp, off, 64));
    mr = fmaxf(mr, __shfl_xor(mr, off, 64));
  }
  if ((threadIdx.x & 63u) == 0) {
    if (g.amax_plain) atomicMax(g.amax_plain, mp << 16);
    if (g.amax_rht) atomicMax(g.amax_rht, __float_as_uint(mr * 0.25f));  // the exact 1/4 of the transform
  }
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
__global__ __launch_bounds__(kGThreads) void gemm_generic_kernel(GemmArgs g) {
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

  // epilogue: C = acc / (S_A S_B); outputs past M or N are zero (zero
  // operands), so they do not change the fused maxima
  const EpiScale es = epi_scale(g);
  const bool fused = g.c_bf16 && (g.amax_plain || g.amax_rht);
  FusedMax fm;
  if (fused) fused_max_init(fm, g, lane);
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int64_t n = n0 + wn * (TN * 32) + j * 32 + lrow;
      uint32_t hb[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + wm * (TM * 32) + i * 32 + (r >> 2) * 8 + half * 4 + (r & 3);
        const float v = epi_apply(acc[i][j][r], es);
        hb[r] = bf16_rne_bits(v);
        if (m < g.M && n < g.N) {
          if (g.c_bf16)
            reinterpret_cast<uint16_t *>(g.c)[m * g.ldc + n] = (uint16_t)hb[r];
          else
            reinterpret_cast<float *>(g.c)[m * g.ldc + n] = v;
        }
      }
      if (fused) fused_max_block(fm, g, hb);
    }
  if (fused) fused_max_flush(fm, g);
}

// ===========================================================================
// Fast path (M, N multiples of 256, K a multiple of 128): 256x256x128 tiles,
// three LDS stages filled by direct global->LDS transfers.
//
// LDS stage layout (36 KiB): codes of the 256 A rows then the 256 B rows,
// 64 bytes (one 128-wide K slice) per row in four 16-byte chunks stored in
// the order chunk ^ swz(row), then 8 scale bytes per row as two dwords stored
// in the order half ^ ((row >> 4) & 1).  The swizzles make the fragment reads
// (ds_read_b128 of one row per lane, ds_read_b32 of its scales) free of bank
// conflicts for 32- and 64-bank LDS.  The transfers write consecutive 16-byte
// (4-byte for scales) slots per lane, so the swizzle is applied by choosing
// which global chunk each lane fetches.
//
// K mapping inside a 128-wide K-tile: lane-half h of the MFMA in sub-step s
// (0..7) holds k = 64h + 8s + [0, 8): dword s of the 32 bytes at byte 32h of
// the row slice, under block scale 4h + s/2 (byte s/2 of scale dword h).
// ===========================================================================
constexpr int kFBK = 128;
constexpr int kFStageCodes = 512 * 64;         // bytes of codes per stage
constexpr int kFStageBytes = kFStageCodes + 512 * 8;
constexpr int kFStages = 3;

struct FastCtx {
  const uint8_t *cbase;  // codes of the operand this wave transfers (A: waves 0-1, B: waves 2-3)
  const uint8_t *sbase;  // its scales
  // per-lane global offsets (bytes) of this lane's 8 code chunks and 4 scale dwords at kt = 0
  uint32_t coff[8];
  uint32_t soff[4];
};

// Each wave issues exactly 12 transfers per K-tile (8 x 1 KiB of codes, 4 x
// 256 B of scales), which the vmcnt waits of the main loop count on.  Waves 0-1
// fill the A half of the stage (code slots 0..1023, scale slots 0..511), waves
// 2-3 the B half.  Transfers [FIRST, FIRST + COUNT) of the 12 are issued here
// (0-7 codes, 8-11 scales), so that a tile's transfers can be spread over
// several MFMA sub-steps.  `wave` must be wave-uniform.
// The K-tile's offset moves the scalar base address (two scalar adds per
// operand), so the per-lane offsets stay fixed: adding it to each transfer's
// per-lane offset took twelve VALU adds per K-tile from the MFMA shadow
// (measured: the 5120 x 5120 x 8192 GEMM 1.5 % faster this way).
template <int FIRST, int COUNT>
__device__ __forceinline__ void fast_issue(const FastCtx &c, uint32_t lds_stage, uint32_t kt, uint32_t wave) {
  const uint8_t *cb = uniform_ptr(c.cbase + (uint64_t)kt * 64u), *sb = uniform_ptr(c.sbase + (uint64_t)kt * 8u);
#pragma unroll
  for (int t = FIRST; t < FIRST + COUNT; ++t) {
    if (t < 8)
      dma16(cb, c.coff[t], __builtin_amdgcn_readfirstlane(lds_stage + (wave * 8 + t) * 1024u));
    else
      dma4(sb, c.soff[t - 8], __builtin_amdgcn_readfirstlane(lds_stage + kFStageCodes + (wave * 4 + (t - 8)) * 256u));
  }
}

// The fp16 MFMA operands of one sub-step (16 k): 4 A and 4 B fragments.
struct Frags {
  half8v a[4], b[4];
};

// Expand sub-step s (0..3) of one half of a K-tile: dword s of this lane's
// 16 code bytes of each row, under block scale element s/2 of the pair.
template <int S>
__device__ __forceinline__ void expand_step(Frags &f, const uint4 qa[4], const uint4 qb[4], const half2v sa[4],
                                            const half2v sb[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w = S == 0 ? qa[i].x : S == 1 ? qa[i].y : S == 2 ? qa[i].z : qa[i].w;
    f.a[i] = expand8(w, (S >> 1) ? sa[i][1] : sa[i][0]);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t w = S == 0 ? qb[j].x : S == 1 ? qb[j].y : S == 2 ? qb[j].z : qb[j].w;
    f.b[j] = expand8(w, (S >> 1) ? sb[j][1] : sb[j][0]);
  }
}

__device__ __forceinline__ void mfma_step(float16v acc[4][4], const Frags &f) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
}

// Instruction order of one sub-step: each MFMA followed by four VALU
// instructions of the next sub-step's expansion (64 of them per 16 MFMAs), so
// the expansion runs in the shadow of the 8-pass MFMAs instead of between them.
__device__ __forceinline__ void interleave_step() {
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // VALU
  }
}

// Accumulate K-tiles [ka, kb) of the 256x256 C tile at (m0, n0) into acc.
// Every wave of the workgroup calls it with the same arguments; it owns the
// whole LDS pipeline while it runs (it starts with a barrier, so the stages
// may be reused from one call to the next, and ends with no transfer in
// flight).
__device__ __forceinline__ void fast_tile(const GemmArgs &g, int64_t m0, int64_t n0, uint32_t ka, uint32_t kb,
                                          float16v acc[4][4], uint8_t *lds) {
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const uint32_t lr = lane & 31, h = lane >> 5;
  const uint32_t kbytes = (uint32_t)(g.K / 2), kblocks = (uint32_t)(g.K / 16);

  // which global bytes this lane transfers (the same for every K-tile up to the K offset)
  FastCtx c;
  c.cbase = wave < 2 ? g.a_codes : g.b_codes;
  c.sbase = wave < 2 ? g.a_scales : g.b_scales;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t q = (wave * 8 + i) * 64 + lane;  // 16-byte slot of the stage
    const uint32_t row = q >> 2;                      // 0..511: A rows then B rows
    const uint32_t chunk = (q & 3u) ^ swz(row);
    const uint32_t grow = (uint32_t)(row < 256 ? m0 + row : n0 + (row - 256));
    c.coff[i] = grow * kbytes + chunk * 16u;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t d = (wave * 4 + i) * 64 + lane;  // scale dword slot
    const uint32_t row = d >> 1;
    const uint32_t half = (d & 1u) ^ ((row >> 4) & 1u);
    const uint32_t grow = (uint32_t)(row < 256 ? m0 + row : n0 + (row - 256));
    const int kind = row < 256 ? g.a_kind : g.b_kind;
    const uint32_t srow = kind == 0 ? grow : (grow >> 4);
    c.soff[i] = srow * kblocks + half * 4u;
  }

  // LDS byte offsets (within a stage) of this lane's fragments: [i][0] holds
  // the k of the first half of the K-tile (sub-steps 0-3), [i][1] the second
  uint32_t aoff[4][2], boff[4][2], asoff[4], bsoff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t r = wm * 128 + i * 32 + lr;
    aoff[i][0] = (r * 4 + ((2 * h) ^ swz(r))) * 16;
    aoff[i][1] = (r * 4 + ((2 * h + 1) ^ swz(r))) * 16;
    asoff[i] = kFStageCodes + (r * 2 + (h ^ ((r >> 4) & 1u))) * 4;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t r = 256 + wn * 128 + j * 32 + lr;
    boff[j][0] = (r * 4 + ((2 * h) ^ swz(r))) * 16;
    boff[j][1] = (r * 4 + ((2 * h + 1) ^ swz(r))) * 16;
    bsoff[j] = kFStageCodes + (r * 2 + (h ^ ((r >> 4) & 1u))) * 4;
  }

  // Pipeline.  Transfers run up to three K-tiles ahead of the MFMAs; every
  // iteration issues exactly one tile's transfers (the index clamped to the
  // last tile, so the vmcnt bookkeeping is the same in every iteration; the
  // clamped copies land in stages nobody reads again), two per sub-step: the
  // first six of tile kt+3 after the barrier of iteration kt, the other six
  // in the first half of iteration kt+1, before its barrier.  The barrier of tile
  // kt+1 sits between the two halves of tile kt, and the fp16 fragments are
  // expanded one MFMA sub-step ahead, so MFMAs are ready on both sides of it.
  const uint32_t lds0 = lds_addr(lds);
  const uint32_t klast = kb - 1;
  NVFP4_WAIT_LGKM0();
  __builtin_amdgcn_s_barrier();  // no wave still reads the stages (a previous tile's)
  asm volatile("" ::: "memory");
  fast_issue<0, 12>(c, lds0, ka, wave);
  fast_issue<0, 12>(c, lds0 + kFStageBytes, ka + 1 < klast ? ka + 1 : klast, wave);
  fast_issue<0, 6>(c, lds0 + 2 * kFStageBytes, ka + 2 < klast ? ka + 2 : klast, wave);
  NVFP4_WAIT_VMCNT(18);  // this wave's transfers of tile ka are done
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");

  // first-half codes and the tile's scales (E4M3 -> fp16 pairs: lo = blocks
  // (4h, 4h+1) of the first half, hi = (4h+2, 4h+3) of the second)
  uint4 qlo_a[4], qlo_b[4];
  half2v sal[4], sah[4], sbl[4], sbh[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    qlo_a[i] = *reinterpret_cast<const uint4 *>(lds + aoff[i][0]);
    const uint32_t sw = *reinterpret_cast<const uint32_t *>(lds + asoff[i]);
    sal[i] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sw, 1.0f, false);
    sah[i] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sw, 1.0f, true);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    qlo_b[j] = *reinterpret_cast<const uint4 *>(lds + boff[j][0]);
    const uint32_t sw = *reinterpret_cast<const uint32_t *>(lds + bsoff[j]);
    sbl[j] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sw, 1.0f, false);
    sbh[j] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sw, 1.0f, true);
  }
  Frags f, fn;
  expand_step<0>(f, qlo_a, qlo_b, sal, sbl);

  uint32_t stage = 0;
  for (uint32_t kt = ka; kt < kb; ++kt) {
    // Each sub-step is a scheduling region of its own (sched_barrier), in
    // which the MFMAs of one sub-step interleave with the expansion of the next.
    const uint8_t *base = lds + stage * kFStageBytes;
    const uint32_t pstage = stage == 0 ? 2 : stage - 1;  // (kt + 2) % 3
    const uint32_t plds = lds0 + pstage * kFStageBytes, ptile = kt + 2 < klast ? kt + 2 : klast;
    uint4 qhi_a[4], qhi_b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) qhi_a[i] = *reinterpret_cast<const uint4 *>(base + aoff[i][1]);
#pragma unroll
    for (int j = 0; j < 4; ++j) qhi_b[j] = *reinterpret_cast<const uint4 *>(base + boff[j][1]);

    // first half: sub-steps 0-3 (sub-step 0's fragments are ready)
    expand_step<1>(fn, qlo_a, qlo_b, sal, sbl);
    mfma_step(acc, f);
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);  // the second-half code reads first
    interleave_step();
    fast_issue<6, 2>(c, plds, ptile, wave);
    __builtin_amdgcn_sched_barrier(0);
    expand_step<2>(f, qlo_a, qlo_b, sal, sbl);
    mfma_step(acc, fn);
    interleave_step();
    fast_issue<8, 2>(c, plds, ptile, wave);
    __builtin_amdgcn_sched_barrier(0);
    expand_step<3>(fn, qlo_a, qlo_b, sal, sbl);
    mfma_step(acc, f);
    interleave_step();
    fast_issue<10, 2>(c, plds, ptile, wave);
    __builtin_amdgcn_sched_barrier(0);
    expand_step<0>(f, qhi_a, qhi_b, sah, sbh);
    mfma_step(acc, fn);
    interleave_step();
    __builtin_amdgcn_sched_barrier(0);

    half2v cah[4], cbh[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) cah[i] = sah[i];
#pragma unroll
    for (int j = 0; j < 4; ++j) cbh[j] = sbh[j];

    NVFP4_WAIT_LGKM0();    // this wave's reads of the stage are complete
    NVFP4_WAIT_VMCNT(12);  // this wave's transfers of tile kt+1 are done (kt+2's may be in flight)
    __builtin_amdgcn_s_barrier();  // every wave's: tile kt+1 is in LDS, this stage is free
    asm volatile("" ::: "memory");
    const uint32_t dlds = lds_addr(base), dtile = kt + 3 < klast ? kt + 3 : klast;
    const uint32_t nstage = stage == 2 ? 0 : stage + 1;
    const uint8_t *nbase = lds + nstage * kFStageBytes;
    uint32_t swa[4], swb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      qlo_a[i] = *reinterpret_cast<const uint4 *>(nbase + aoff[i][0]);
      swa[i] = *reinterpret_cast<const uint32_t *>(nbase + asoff[i]);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      qlo_b[j] = *reinterpret_cast<const uint4 *>(nbase + boff[j][0]);
      swb[j] = *reinterpret_cast<const uint32_t *>(nbase + bsoff[j]);
    }
    stage = nstage;

    // second half: sub-steps 4-7, then sub-step 0 of tile kt+1 is expanded
    // (on the last tile from a stale stage; those fragments are not used)
    expand_step<1>(fn, qhi_a, qhi_b, cah, cbh);
    mfma_step(acc, f);
    interleave_step();
    fast_issue<0, 2>(c, dlds, dtile, wave);
    __builtin_amdgcn_sched_barrier(0);
    expand_step<2>(f, qhi_a, qhi_b, cah, cbh);
    mfma_step(acc, fn);
    interleave_step();
    fast_issue<2, 2>(c, dlds, dtile, wave);
    __builtin_amdgcn_sched_barrier(0);
    expand_step<3>(fn, qhi_a, qhi_b, cah, cbh);
    mfma_step(acc, f);
    interleave_step();
    fast_issue<4, 2>(c, dlds, dtile, wave);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sal[i] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(swa[i], 1.0f, false);
      sah[i] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(swa[i], 1.0f, true);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      sbl[j] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(swb[j], 1.0f, false);
      sbh[j] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(swb[j], 1.0f, true);
    }
    expand_step<0>(f, qlo_a, qlo_b, sal, sbl);
    mfma_step(acc, fn);
    interleave_step();
    __builtin_amdgcn_sched_barrier(0);
  }
  NVFP4_WAIT_VMCNT(0);  // the clamped transfers of the last iterations

}

// C tile = acc / (S_A S_B), 32-bit offsets from the tile origin
// C is written with non-temporal stores.  Written back through the caches,
// a large C leaves dirty lines in the memory-side cache, and the next kernel
// pays for their write-back while it reads: a 20480x5120 weight quantise
// took 110 us right after a 16384x20480 bf16 GEMM output against 88 us
// alone.  With non-temporal stores C reaches HBM while the GEMM, which is
// bound by the MFMA and not by HBM, still runs (the quantise then took 95 us,
// the GEMM's own time unchanged), and the Wgrad step ran 1 % faster.
__device__ __forceinline__ void fast_store_c(const GemmArgs &g, int64_t m0, int64_t n0, const float16v acc[4][4]) {
  const uint32_t wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const uint32_t lr = lane & 31, h = lane >> 5;
  const EpiScale es = epi_scale(g);
  uint32_t ldc = (uint32_t)g.ldc;
  asm volatile("" : "+s"(ldc));  // per-element offsets are formed here, not hoisted and kept live
  if (g.c_bf16) {
    uint16_t *ct = reinterpret_cast<uint16_t *>(g.c) + m0 * g.ldc + n0;
    asm volatile("" : "+s"(ct));  // keep the address arithmetic in the epilogue
    const bool fused = g.amax_plain || g.amax_rht;
    FusedMax fm;
    if (fused) fused_max_init(fm, g, lane);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t hb[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const uint32_t m = wm * 128 + i * 32 + (r >> 2) * 8 + h * 4 + (r & 3);
          const uint32_t n = wn * 128 + j * 32 + lr;
          hb[r] = bf16_rne_bits(epi_apply(acc[i][j][r], es));
          __builtin_nontemporal_store((uint16_t)hb[r], &ct[m * ldc + n]);
        }
        if (fused) fused_max_block(fm, g, hb);
      }
    if (fused) fused_max_flush(fm, g);
  } else {
    float *ct = reinterpret_cast<float *>(g.c) + m0 * g.ldc + n0;
    asm volatile("" : "+s"(ct));  // keep the address arithmetic in the epilogue
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const uint32_t m = wm * 128 + i * 32 + (r >> 2) * 8 + h * 4 + (r & 3);
          const uint32_t n = wn * 128 + j * 32 + lr;
          __builtin_nontemporal_store(epi_apply(acc[i][j][r], es), &ct[m * ldc + n]);
        }
  }
}

template <int TM, int TN>
__global__ __launch_bounds__(kGThreads) void gemm_fast_kernel(GemmArgs g) {
  static_assert(TM == 4 && TN == 4, "fast path is laid out for 256x256 tiles");
  __shared__ __attribute__((aligned(16))) uint8_t lds[kFStages * kFStageBytes];
  // Each XCD takes a contiguous range of the tile sequence, and the sequence
  // runs down groups of kGroupM tile rows column by column, so the workgroups
  // that one XCD runs at a time cover a compact block of C: they share the A
  // and B K-slices in that XCD's L2 instead of each streaming its own.
  int64_t m0, n0;
  tile_origin(g.M, g.N, xcd_tile(blockIdx.x, gridDim.x), m0, n0);
  float16v acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  fast_tile(g, m0, n0, 0, (uint32_t)(g.K / kFBK), acc, lds);
  fast_store_c(g, m0, n0, acc);
}

// ===========================================================================
// Stream-K (fast path shapes whose tile count leaves compute units idle in
// the last round): one persistent workgroup per compute unit, all resident
// (the LDS admits one per CU).  The first dp_tiles tiles (whole rounds) are done
// as whole tiles, round by round, so that the workgroups of one XCD start
// their tiles together and share K-slices in L2.  The remaining tiles' units
// (tile, K-tile) are numbered tile by tile in the grouped order and dealt out
// as G contiguous ranges.  A workgroup whose range starts inside a tile
// computes that part first, writes its fp32 partial to workspace slot w and
// raises flag w.  The workgroup that holds the tile's first K-tile (the head,
// at the end of its range) computes its part last, then for each following
// workgroup whose range starts inside the tile waits for its flag (normally
// long raised), adds its partial (in workgroup order, so the sum does not
// depend on timing) and lowers the flag, leaving every flag zero for the next
// launch; then it writes C.  Partials and flags use device-coherent (sc1)
// accesses; a partial's writes complete (vmcnt) before its flag is raised.
// Each wait is bounded (about a second); on time-out `err` is set, that
// tile's result is invalid and the late partial is neither added nor its flag
// lowered, but the launch always ends.
// ===========================================================================
struct StreamK {
  uint32_t *flags;  // [G]
  uint32_t *err;
  float *slots;     // [G][65536]
  uint32_t tiles, KT;
  uint32_t dp_tiles;  // tiles done whole before the stream-K part (a multiple of G)
};

// The partial moves 64 values at a time (a compiler memory barrier between
// groups): four round trips to memory for the loads, and no more than 64
// extra registers live next to the 256 accumulators.
__device__ __forceinline__ void store_partial(float *slot, const float16v acc[4][4]) {
  asm volatile("" : "+s"(slot));  // keep the address arithmetic here (not hoisted and kept live)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        __hip_atomic_store(slot + ((i * 4 + j) * 16 + r) * kGThreads + threadIdx.x, acc[i][j][r], __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    asm volatile("" ::: "memory");
  }
}

__device__ __forceinline__ void add_partial(float16v acc[4][4], const float *slot) {
  asm volatile("" : "+s"(slot));  // keep the address arithmetic here (not hoisted and kept live)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float p[4][16];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        p[j][r] = __hip_atomic_load(slot + ((i * 4 + j) * 16 + r) * kGThreads + threadIdx.x, __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT);
    asm volatile("" ::: "memory");
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] += p[j][r];
  }
}

__device__ __forceinline__ void zero_acc(float16v acc[4][4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
}

__global__ __launch_bounds__(kGThreads) void gemm_streamk_kernel(GemmArgs g, StreamK sk) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kFStages * kFStageBytes];
  const uint32_t G = gridDim.x, w = xcd_tile(blockIdx.x, G);
  float16v acc[4][4];
  int64_t m0, n0;

  for (uint32_t t = w; t < sk.dp_tiles; t += G) {  // whole tiles, round by round
    tile_origin(g.M, g.N, t, m0, n0);
    zero_acc(acc);
    fast_tile(g, m0, n0, 0, sk.KT, acc, lds);
    fast_store_c(g, m0, n0, acc);
  }

  const uint64_t U = (uint64_t)(sk.tiles - sk.dp_tiles) * sk.KT;
  uint64_t u = U * w / G;
  const uint64_t uend = U * (w + 1) / G;
  while (u < uend) {
    const uint32_t ts = (uint32_t)(u / sk.KT), ka = (uint32_t)(u - (uint64_t)ts * sk.KT);
    const uint64_t tend = (uint64_t)(ts + 1) * sk.KT;
    const uint32_t kb = (uint32_t)((uend < tend ? uend : tend) - (uint64_t)ts * sk.KT);
    tile_origin(g.M, g.N, sk.dp_tiles + ts, m0, n0);
    zero_acc(acc);
    fast_tile(g, m0, n0, ka, kb, acc, lds);
    if (ka > 0) {  // this range starts inside the tile: hand the partial to its head
      store_partial(sk.slots + (size_t)w * 65536, acc);
      NVFP4_WAIT_VMCNT(0);
      __syncthreads();
      if (threadIdx.x == 0) __hip_atomic_store(sk.flags + w, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      // head: add the partials of the following workgroups whose (non-empty)
      // ranges start inside the tile
      __shared__ uint32_t timed_out;
      for (uint32_t v = w + 1; v < G && U * v / G < tend; ++v) {
        if (U * (v + 1) / G == U * v / G) continue;  // an empty range wrote no partial
        if (threadIdx.x == 0) {
          uint32_t late = 0;
          for (uint32_t spins = 0;
               __hip_atomic_load(sk.flags + v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u;) {
            __builtin_amdgcn_s_sleep(8);
            if (++spins == (1u << 22)) {
              __hip_atomic_store(sk.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              late = 1;
              break;
            }
          }
          timed_out = late;
        }
        __syncthreads();
        // On a time-out the slot holds no finished partial and the flag is
        // left alone (workgroup v raises it later): the tile is invalid, the
        // error word says so, and the caller zero-fills the workspace again
        // before its next use.
        if (!timed_out) {
          add_partial(acc, sk.slots + (size_t)v * 65536);
          __syncthreads();
          if (threadIdx.x == 0) __hip_atomic_store(sk.flags + v, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();  // timed_out is read by every thread before it is written again
      }
      fast_store_c(g, m0, n0, acc);
    }
    u += kb - ka;
  }
}

bool gemm_fast_ok(const GemmArgs &g) {
  return g.M % 256 == 0 && g.N % 256 == 0 && g.K % kFBK == 0 && g.K / 2 * (g.M > g.N ? g.M : g.N) < (1ll << 32) &&
         g.ldc * 256 < (1ll << 31);
}

size_t gemm_workspace_bytes(int cus) { return kGemmWsSlots + (size_t)cus * kGemmSlotBytes; }

hipError_t launch_gemm(const GemmArgs &g, void *workspace, size_t workspace_bytes, hipStream_t s) {
  constexpr int TM = 4, TN = 4;
  constexpr int BM = GemmTile<TM, TN>::BM, BN = GemmTile<TM, TN>::BN;
  const int64_t tiles = ((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN);
  if (!gemm_fast_ok(g) || getenv("NVFP4_GEMM_GENERIC")) {
    hipLaunchKernelGGL((gemm_generic_kernel<TM, TN>), dim3((uint32_t)tiles), dim3(kGThreads), 0, s, g);
    return hipGetLastError();
  }
  // Stream-K when a workspace is given, there are more than two rounds of
  // tiles and the last round would leave more than a tenth of the compute
  // units idle.  (With fewer rounds the split tiles' pipeline refills and
  // partial sums cost more than the idle units of one short last round, which
  // also runs at a higher clock: measured on 5120x5120x8192.)
  // A stream being captured into a graph gets whole tiles: a replay must not
  // depend on every workgroup of the persistent grid being resident.
  hipStreamCaptureStatus capture = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &capture) != hipSuccess) {
    (void)hipGetLastError();
    capture = hipStreamCaptureStatusActive;  // unknown: take the whole-tile path
  }
  int dev = 0, cus = 0;
  if (workspace && capture == hipStreamCaptureStatusNone && !getenv("NVFP4_GEMM_DATA_PARALLEL") &&
      hipGetDevice(&dev) == hipSuccess &&
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cus > 0 &&
      cus <= kGemmMaxCUs && tiles > 2 * (int64_t)cus && workspace_bytes >= gemm_workspace_bytes(cus)) {
    const int64_t rounds = (tiles + cus - 1) / cus;
    if (10 * tiles < 9 * rounds * cus) {
      StreamK sk;
      sk.flags = (uint32_t *)workspace;
      sk.err = (uint32_t *)workspace + kGemmMaxCUs;
      sk.slots = (float *)((char *)workspace + kGemmWsSlots);
      sk.tiles = (uint32_t)tiles;
      sk.KT = (uint32_t)(g.K / kFBK);
      sk.dp_tiles = (uint32_t)((tiles / cus) * cus);  // whole rounds first
      // One workgroup per compute unit, launched as an ordinary kernel: its
      // 108 KiB of LDS admits one per CU, so on a GPU that runs nothing
      // else all are resident together.  A workgroup only ever waits for
      // workgroups with a larger index, and each wait is bounded, so the
      // launch ends even if some were held back (then the error word is set).
      // (A cooperative launch would guarantee residency but costs 15-22 us
      // per call, measured on the Wgrad and linear-step shapes.)
      int per_cu = 0;
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, gemm_streamk_kernel, kGThreads, 0) == hipSuccess &&
          per_cu >= 1) {
        hipLaunchKernelGGL(gemm_streamk_kernel, dim3((uint32_t)cus), dim3(kGThreads), 0, s, g, sk);
        return hipGetLastError();
      }
      (void)hipGetLastError();  // occupancy unknown: whole tiles
    }
  }
  hipLaunchKernelGGL((gemm_fast_kernel<TM, TN>), dim3((uint32_t)tiles), dim3(kGThreads), 0, s, g);
  return hipGetLastError();
}

}  // namespace nvfp4
