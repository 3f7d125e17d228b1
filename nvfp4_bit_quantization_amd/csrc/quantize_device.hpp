// Device code of the quantisation kernels:
// the lane/tile decomposition, the RHT butterflies on a lane's micro-tile, the
// per-tile maxima, the block-scale and element encoders, one output of one
// micro-tile, and the global-scale setup.
//
// Method: NVFP4 pretraining news page (zubnet.ai), paragraph 2 -- blocks of
// 16 E2M1 values share one E4M3 scale, under one FP32 scale per tensor; 1D
// blocks for activations/gradients, 16x16 blocks for weights; stochastic
// rounding for gradients; a 16-point Hadamard transform with a random +-1
// sign vector on the weight-gradient inputs.
//
// Work decomposition.  A workgroup (4 waves) owns a 128 x 256 tile of the
// bf16 input.  Each lane owns a 16-row x 8-column micro-tile, loaded as 16
// 16-byte vectors; inside a wave the lanes form an 8 (column chunks) x 8
// (row groups) grid, so one load instruction reads 128 contiguous bytes from
// each of 8 rows.  A 16-element row block spans lanes l and l^8 (combined
// with one DPP row rotate), a 16-element column block and the 16-point
// Hadamard transform along rows live entirely inside one lane.
#pragma once

#include "nvfp4_device.hpp"
#include "nvfp4_kernels.hpp"

namespace nvfp4 {

struct Lane {
  int64_t r0, c0;  // top-left element of this lane's 16x8 micro-tile
  uint32_t hi;     // 1 if the micro-tile is the right half of a 16-col block
  bool valid;
};

__device__ __forceinline__ Lane lane_coords(uint32_t tile, int64_t R, int64_t C) {
  const int64_t ntc = (C + kQTileC - 1) / kQTileC;
  const int64_t tr = tile / ntc, tc = tile % ntc;
  const uint32_t w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const uint32_t cg = lane & 7, cc = lane >> 3;
  Lane L;
  L.r0 = tr * kQTileR + cg * 16;
  L.c0 = tc * kQTileC + w * 64 + cc * 8;
  L.hi = cc & 1;
  L.valid = (L.r0 < R) && (L.c0 < C);
  return L;
}

// A single column output takes 256 x 128 workgroup tiles instead (waves
// 2 x 2): each workgroup then writes 128 bytes of every output row it touches,
// a whole line, instead of 64.  Measured 2 % faster on 8192 x 5120 column
// quantisations (X: 38.0 -> 37.2 us); outputs identical.
constexpr int kQTallR = 256, kQTallC = 128;
__device__ __forceinline__ Lane lane_coords_tall(uint32_t tile, int64_t R, int64_t C) {
  const int64_t ntc = (C + kQTallC - 1) / kQTallC;
  const int64_t tr = tile / ntc, tc = tile % ntc;
  const uint32_t w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const uint32_t cg = lane & 7, cc = lane >> 3;
  Lane L;
  L.r0 = tr * kQTallR + (w >> 1) * 128 + cg * 16;
  L.c0 = tc * kQTallC + (w & 1) * 64 + cc * 8;
  L.hi = cc & 1;
  L.valid = (L.r0 < R) && (L.c0 < C);
  return L;
}

__device__ __forceinline__ void load_micro_tile(const uint16_t *x, int64_t ld, const Lane &L, uint4 raw[16]) {
  const uint16_t *p = x + L.r0 * ld + L.c0;
#pragma unroll
  for (int i = 0; i < 16; ++i) raw[i] = *reinterpret_cast<const uint4 *>(p + i * ld);
}
// The same without a branch: a lane past the tensor loads the micro-tile at
// (0, 0), which always exists (both sizes are at least 16), and ignores it.
// Without the branch the loads issued before the tile's (the partial maxima)
// can be waited for alone.
__device__ __forceinline__ void load_micro_tile_any(const uint16_t *x, int64_t ld, const Lane &L, uint4 raw[16]) {
  Lane M = L;
  M.r0 = L.valid ? L.r0 : 0;
  M.c0 = L.valid ? L.c0 : 0;
  load_micro_tile(x, ld, M, raw);
}

// An empty asm that claims to change the raw words: a later pass over the
// micro-tile then unpacks bf16 -> fp32 again instead of keeping the 128
// unpacked values of an earlier pass live, which would take 128 VGPRs and
// cost waves per SIMD.
__device__ __forceinline__ void opaque_raw(uint4 raw[16]) {
#pragma unroll
  for (int i = 0; i < 16; ++i) asm volatile("" : "+v"(raw[i].x), "+v"(raw[i].y), "+v"(raw[i].z), "+v"(raw[i].w));
}

// maximum over the wave, returned in every lane: DPP within each row of 16
// lanes, then the four row maxima read as scalars (no LDS round trips)
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float wave_max(float m) {
  m = fmaxf(m, dpp_f<0xB1>(m));   // quad_perm [1,0,3,2]
  m = fmaxf(m, dpp_f<0x4E>(m));   // quad_perm [2,3,0,1]
  m = fmaxf(m, dpp_f<0x124>(m));  // row_ror:4
  m = fmaxf(m, dpp_f<0x128>(m));  // row_ror:8
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// ------------------------------------------------------------------------
// RHT: the random signs flip sign bits, then the butterflies
// ------------------------------------------------------------------------
// element k of a micro-tile row as fp32, its sign bit flipped when s is
// 0x80000000 (s = 0 or 0x80000000): the flip costs nothing beyond the
// unpacking (a shift-add for the low half, since adding 2^31 flips bit 31,
// and a three-input logic op for the high half)
__device__ __forceinline__ float bf16_at_signed(const uint4 &q, int k, uint32_t s) {
  const uint32_t w = (k >> 1) == 0 ? q.x : (k >> 1) == 1 ? q.y : (k >> 1) == 2 ? q.z : q.w;
  return __uint_as_float((k & 1) ? ((w & 0xFFFF0000u) ^ s) : ((w << 16) + s));
}
// along columns: column j = 8 hi + k of the 16-column block gets d_j
__device__ __forceinline__ void flip_cols(uint4 raw[16], uint32_t mask, uint32_t hi) {
  const uint32_t m = mask >> (8 * hi);
  uint32_t f[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) f[p] = (((m >> (2 * p)) & 1u) << 15) | (((m >> (2 * p + 1)) & 1u) << 31);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    raw[i].x ^= f[0];
    raw[i].y ^= f[1];
    raw[i].z ^= f[2];
    raw[i].w ^= f[3];
  }
}

// column j (16 rows; row i of the 16-row group gets d_i, bit i of mask):
// H D v in binary32 (the 1/4 is applied later)
__device__ __forceinline__ void fwht_column(const uint4 raw[16], int j, uint32_t mask, float d[16]) {
#pragma unroll
  for (int i = 0; i < 16; ++i) d[i] = bf16_at_signed(raw[i], j, ((mask >> i) & 1u) << 31);
  fwht16(d);
}

// row i of a 16-column block held by lanes l (cols 0..7) and l^8 (cols 8..15),
// signs applied: butterflies on j bits 0-2 inside the lane, bit 3 across lanes
__device__ __forceinline__ void fwht_row(const uint4 &row, uint32_t hi, float d[8]) {
#pragma unroll
  for (int k = 0; k < 8; ++k) d[k] = bf16_at(row, k);
#pragma unroll
  for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if ((k & h) == 0) {
        const float a = d[k], b = d[k + h];
        d[k] = a + b;
        d[k + h] = a - b;
      }
    }
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float other = swap8(d[k]);
    d[k] = hi ? (other - d[k]) : (d[k] + other);
  }
}

// ------------------------------------------------------------------------
// amax: per-workgroup partial maxima for up to three modes
// ------------------------------------------------------------------------
// maxima of one micro-tile: |x|, |H d x| along rows (column blocks) and along
// columns (row blocks), the latter two without the exact factor 1/4
template <bool PLAIN, bool RC, bool RR>
__device__ __forceinline__ void tile_maxes(const uint4 raw[16], const Lane &L, uint32_t mask_rows,
                                           uint32_t mask_cols, float &m_plain, float &m_rc, float &m_rr) {
  if (PLAIN && !RC) {
#pragma unroll
    for (int i = 0; i < 16; ++i)
#pragma unroll
      for (int k = 0; k < 8; ++k) m_plain = fmaxf(m_plain, fabsf(bf16_at(raw[i], k)));
  }
  if (RC) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float d[16];
      if (PLAIN) {  // the plain maximum from the same unpacked values: a sign flip keeps |x|
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          d[i] = bf16_at_signed(raw[i], j, ((mask_rows >> i) & 1u) << 31);
          m_plain = fmaxf(m_plain, fabsf(d[i]));
        }
        fwht16(d);
      } else {
        fwht_column(raw, j, mask_rows, d);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) m_rc = fmaxf(m_rc, fabsf(d[i]));
    }
  }
  if (RR) {
    uint4 r[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) r[i] = raw[i];
    flip_cols(r, mask_cols, L.hi);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float d[8];
      fwht_row(r[i], L.hi, d);
#pragma unroll
      for (int k = 0; k < 8; ++k) m_rr = fmaxf(m_rr, fabsf(d[k]));
    }
  }
}

// workgroup maxima -> partials[mode * kMaxParts + slot] (the quarter of the
// Hadamard normalisation is exact, a power of two)
template <bool PLAIN, bool RC, bool RR>
__device__ __forceinline__ void write_partials(float m_plain, float m_rc, float m_rr, float *partials,
                                               uint32_t slot) {
  __shared__ float red[3][kQThreads / 64];
  const uint32_t w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const float v0 = wave_max(m_plain);
  const float v1 = wave_max(m_rc * 0.25f);
  const float v2 = wave_max(m_rr * 0.25f);
  if (lane == 0) {
    red[0][w] = v0;
    red[1][w] = v1;
    red[2][w] = v2;
  }
  __syncthreads();
  if (threadIdx.x < 3) {
    float m = red[threadIdx.x][0];
    for (int i = 1; i < kQThreads / 64; ++i) m = fmaxf(m, red[threadIdx.x][i]);
    const bool want = threadIdx.x == 0 ? PLAIN : threadIdx.x == 1 ? RC : RR;
    if (want) partials[threadIdx.x * kMaxParts + slot] = m;
  }
}

// ------------------------------------------------------------------------
// element encoders over a lane's values
// ------------------------------------------------------------------------
// 8 values -> one 32-bit word of codes (value k in nibble k), RTN
__device__ __forceinline__ uint32_t pack8_rtn(const float v[8], float rb) {
  uint32_t w = NVFP4_CVT_PK_FP4(0u, v[0] * rb, v[1] * rb, 0);
  w = NVFP4_CVT_PK_FP4(w, v[2] * rb, v[3] * rb, 1);
  w = NVFP4_CVT_PK_FP4(w, v[4] * rb, v[5] * rb, 2);
  w = NVFP4_CVT_PK_FP4(w, v[6] * rb, v[7] * rb, 3);
  return w;
}

// 8 values -> word, SR with the uniforms of draw w[] (value k uses u16_of(w, k)),
// on the hardware conversion (e2m1_sr_hw): word j of the draw holds the
// uniforms of values 2j (low half) and 2j+1 (high half).  The even and the
// odd values each go through the conversion's first slot, into the low
// nibbles of bytes 0..3 of their own word; the odd word is moved up a nibble
// when the two are merged.  (The first slot in both chains lets every call
// take its value in one fixed register pair whose second half is zero, and
// the odd values' random operand is one OR.)
template <int J>
__device__ __forceinline__ void sr_pair(const float v[8], float rb, const uint32_t w[4], uint32_t &lo, uint32_t &hi) {
  const uint32_t nw = ~w[J];
  lo = cvt_sr_fp4<J>(lo, sr_hw_prepare(v[2 * J] * rb), 0.0f, sr_hw_rand_lo(nw));
  hi = cvt_sr_fp4<J>(hi, sr_hw_prepare(v[2 * J + 1] * rb), 0.0f, sr_hw_rand_hi(nw));
}
__device__ __forceinline__ uint32_t pack8_sr(const float v[8], float rb, const uint32_t w[4]) {
  uint32_t lo = 0u, hi = 0u;
  sr_pair<0>(v, rb, w, lo, hi);
  sr_pair<1>(v, rb, w, lo, hi);
  sr_pair<2>(v, rb, w, lo, hi);
  sr_pair<3>(v, rb, w, lo, hi);
  return lo | (hi << 4);  // the high nibbles of both words are 0 (the +0 slot)
}

// bmax / 6 correctly rounded (binary32).  From 2^-120 up, the product with
// the rounded reciprocal and one fused correction step give the correctly
// rounded quotient for every input (checked over all non-negative binary32
// values); below, where the quotient is near or in the subnormal range, the
// division itself is used.
__device__ __forceinline__ float div6(float x) {
  const float r = 1.0f / 6.0f;
  const float q0 = x * r;
  float t = __builtin_fmaf(__builtin_fmaf(-q0, 6.0f, x), r, q0);
  const bool slow = x < 0x1p-120f;
  if (__builtin_amdgcn_ballot_w64(slow) != 0) {  // a wave-uniform branch: rarely taken
    float xs = x;
    asm volatile("" : "+v"(xs));  // keeps the division inside the branch (not computed speculatively)
    if (slow) t = xs / 6.0f;
  }
  return t;
}

__device__ __forceinline__ float block_scale(float bmax, float S, const float *lut, uint32_t *code) {
  const float t = div6(bmax);
  const float sb = t * S;
  const uint32_t c = e4m3_encode(sb);
  *code = c;
  return lut[c];
}

// ------------------------------------------------------------------------
// row-layout output staged in LDS: the workgroup's 128 rows x 128 bytes of
// codes and 128 x 16 scale bytes, written out afterwards as whole row segments
// (a lane's own stores write 8 rows x 32 bytes per instruction)
// ------------------------------------------------------------------------
struct __align__(16) RowStage {
  uint32_t codes[kQTileR * 32];  // dword d of row r at stage_dword(r, d)
  uint8_t scales[kQTileR * 16];
};
// the 8 row groups of a wave write the same dword columns: an XOR of the
// column by the row group spreads them over the LDS banks
__device__ __forceinline__ uint32_t stage_dword(uint32_t r, uint32_t d) { return r * 32u + (d ^ (((r >> 4) & 3u) * 8u)); }

// all threads of the workgroup, after a barrier; (tr0, tc0) is the tile origin
template <bool SCALES = true>
__device__ __forceinline__ void row_stage_flush(const RowStage *st, const OutArgs &o, int64_t tr0, int64_t tc0,
                                                int64_t R, int64_t C) {
  const uint32_t t = threadIdx.x;
#pragma unroll
  for (int k = 0; k < 4; ++k) {  // codes: thread t stores 16 bytes (32 elements) of row t/8 + 32k
    const uint32_t row = (t >> 3) + 32u * k, chunk = t & 7u;
    const int64_t r = tr0 + row, c = tc0 + chunk * 32;
    if (r < R && c < C) {
      const uint4 v = *reinterpret_cast<const uint4 *>(st->codes + stage_dword(row, chunk * 4));
      uint8_t *dst = o.codes + r * (C / 2) + c / 2;
      if ((C & 31) == 0) {
        *reinterpret_cast<uint4 *>(dst) = v;
      } else {  // rows start 8-byte aligned only; the last chunk may hold 16 elements
        *reinterpret_cast<uint2 *>(dst) = make_uint2(v.x, v.y);
        if (c + 32 <= C) *reinterpret_cast<uint2 *>(dst + 8) = make_uint2(v.z, v.w);
      }
    }
  }
  if (SCALES) {  // scales: thread t stores the 8 block scales of half t&1 of row t/2
    const uint32_t row = t >> 1, h = t & 1u;
    const int64_t r = tr0 + row, nbc = C / 16, b0 = tc0 / 16 + h * 8;
    if (r < R && b0 < nbc) {
      const uint2 v = *reinterpret_cast<const uint2 *>(st->scales + row * 16 + h * 8);
      uint8_t *dst = o.scales + r * nbc + b0;
      const int64_t n = nbc - b0 < 8 ? nbc - b0 : 8;
      if (n == 8 && (reinterpret_cast<uintptr_t>(dst) & 7u) == 0) {
        *reinterpret_cast<uint2 *>(dst) = v;
      } else {
        const uint64_t w = ((uint64_t)v.y << 32) | v.x;
        for (int64_t q = 0; q < n; ++q) dst[q] = (uint8_t)(w >> (8 * q));
      }
    }
  }
}

// ------------------------------------------------------------------------
// one output of the quantise pass
// ------------------------------------------------------------------------
// (mask_rows: the RHT signs of a column-block output, applied while
// unpacking; a row-block output's signs are already in raw)
template <int G, bool RHT, bool SR>
__device__ __forceinline__ void quantize_output(uint4 raw[16], const Lane &L, const OutArgs &o, float S,
                                                const float *lut, int64_t R, int64_t C, uint32_t mask_rows,
                                                RowStage *st = nullptr) {
  if (G == G_ROW) {
    const int64_t nbc = C / 16;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      // with the RHT, v holds the unnormalised sums H d x; the exact factor
      // 1/4 is applied to the block maximum and folded into the element factor
      float v[8];
      if (RHT) {
        fwht_row(raw[i], L.hi, v);
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = bf16_at(raw[i], k);
      }
      float m = 0.0f;
#pragma unroll
      for (int k = 0; k < 8; ++k) m = fmaxf(m, fabsf(v[k]));
      m = fmaxf(m, swap8(m));
      if (RHT) m *= 0.25f;
      uint32_t sc;
      float rb = block_scale(m, S, lut, &sc);
      if (RHT) rb *= 0.25f;
      const int64_t r = L.r0 + i;
      const uint32_t blk = (uint32_t)(r * nbc + L.c0 / 16);
      // with a stage: the row within the tile and the dword column within its 128 bytes
      const uint32_t lrow = (threadIdx.x & 7u) * 16u + i;
      const uint32_t ldw = (threadIdx.x >> 6) * 8u + ((threadIdx.x & 63u) >> 3);
      if (!L.hi) {
        if (st)
          st->scales[lrow * 16 + ldw / 2] = (uint8_t)sc;
        else
          o.scales[blk] = (uint8_t)sc;
      }
      uint32_t word;
      if (SR) {
        uint32_t w[4];
        sr_draw(o.sr_seed, blk, L.hi, w);
        word = pack8_sr(v, rb, w);
      } else {
        word = pack8_rtn(v, rb);
      }
      if (st)
        st->codes[stage_dword(lrow, ldw)] = word;
      else
        *reinterpret_cast<uint32_t *>(o.codes + r * (C / 2) + L.c0 / 2) = word;
    }
  } else if (G == G_COL) {
    const int64_t nbr = R / 16;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float v[16];  // with the RHT: unnormalised sums, 1/4 folded as for rows
      if (RHT) {
        fwht_column(raw, j, mask_rows, v);
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = bf16_at(raw[i], j);
      }
      float m = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(v[i]));
      if (RHT) m *= 0.25f;
      uint32_t sc;
      float rb = block_scale(m, S, lut, &sc);
      if (RHT) rb *= 0.25f;
      const int64_t c = L.c0 + j;
      const uint32_t blk = (uint32_t)(c * nbr + L.r0 / 16);
      o.scales[blk] = (uint8_t)sc;
      uint2 words;
      if (SR) {
        uint32_t w[4];
        sr_draw(o.sr_seed, blk, 0u, w);
        words.x = pack8_sr(v, rb, w);
        sr_draw(o.sr_seed, blk, 1u, w);
        words.y = pack8_sr(v + 8, rb, w);
      } else {
        words.x = pack8_rtn(v, rb);
        words.y = pack8_rtn(v + 8, rb);
      }
      *reinterpret_cast<uint2 *>(o.codes + c * (R / 2) + L.r0 / 2) = words;
    }
  } else {  // G_TILE or G_TILE_T: one scale per 16x16 tile (this lane and lane^8)
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i)
#pragma unroll
      for (int k = 0; k < 8; ++k) m = fmaxf(m, fabsf(bf16_at(raw[i], k)));
    m = fmaxf(m, swap8(m));
    opaque_raw(raw);
    uint32_t sc;
    const float rb = block_scale(m, S, lut, &sc);
    const int64_t nbc = C / 16, nbr = R / 16;
    if (G == G_TILE) {
      if (!L.hi) o.scales[(L.r0 / 16) * nbc + L.c0 / 16] = (uint8_t)sc;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = bf16_at(raw[i], k);
        const int64_t r = L.r0 + i;
        uint32_t word;
        if (SR) {
          uint32_t w[4];
          sr_draw(o.sr_seed, (uint32_t)(r * nbc + L.c0 / 16), L.hi, w);
          word = pack8_sr(v, rb, w);
        } else {
          word = pack8_rtn(v, rb);
        }
        *reinterpret_cast<uint32_t *>(o.codes + r * (C / 2) + L.c0 / 2) = word;
      }
    } else {
      if (!L.hi) o.scales[(L.c0 / 16) * nbr + L.r0 / 16] = (uint8_t)sc;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float v[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = bf16_at(raw[i], j);
        uint2 words;
        if (SR) {
          // the uniforms follow the row-blocked numbering of the untransposed tensor
          uint32_t lo = 0, hi = 0;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            uint32_t w[4];
            sr_draw(o.sr_seed, (uint32_t)((L.r0 + i) * nbc + L.c0 / 16), L.hi, w);
            const uint32_t code = e2m1_sr_hw(v[i] * rb, u16_of(w, j), 0);
            if (i < 8)
              lo |= code << (4 * i);
            else
              hi |= code << (4 * (i - 8));
          }
          words.x = lo;
          words.y = hi;
        } else {
          words.x = pack8_rtn(v, rb);
          words.y = pack8_rtn(v + 8, rb);
        }
        *reinterpret_cast<uint2 *>(o.codes + (L.c0 + j) * (R / 2) + L.r0 / 2) = words;
      }
    }
  }
}

// Transpose of an 8x8 matrix of nibbles held as 8 words (word i, nibble k) in
// three steps: the off-diagonal 4x4 blocks (16-bit halves), then the 2x2
// blocks inside each 4x4 (bytes), then single nibbles inside each 2x2.
__device__ __forceinline__ void nibble_transpose8(uint32_t a[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t x = a[i], y = a[i + 4];
    a[i] = (x & 0x0000FFFFu) | (y << 16);
    a[i + 4] = (x >> 16) | (y & 0xFFFF0000u);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (i & 2) continue;
    const uint32_t x = a[i], y = a[i + 2];
    a[i] = (x & 0x00FF00FFu) | ((y & 0x00FF00FFu) << 8);
    a[i + 2] = ((x >> 8) & 0x00FF00FFu) | (y & 0xFF00FF00u);
  }
#pragma unroll
  for (int i = 0; i < 8; i += 2) {
    const uint32_t x = a[i], y = a[i + 1];
    a[i] = (x & 0x0F0F0F0Fu) | ((y & 0x0F0F0F0Fu) << 4);
    a[i + 1] = ((x >> 4) & 0x0F0F0F0Fu) | (y & 0xF0F0F0F0u);
  }
}

// The 2D and 2D_T outputs under one global scale, both rounded to nearest:
// every element gets the same code in both, so the codes are computed once,
// row-packed for 2D, and the 2D_T words come from transposing the lane's two
// 8x8 nibble matrices in registers.
__device__ __forceinline__ void tile_pair_rtn(uint4 raw[16], const Lane &L, const OutArgs &o0,
                                              const OutArgs &o1, float S, const float *lut, int64_t R, int64_t C,
                                              RowStage *st = nullptr) {
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i)
#pragma unroll
    for (int k = 0; k < 8; ++k) m = fmaxf(m, fabsf(bf16_at(raw[i], k)));
  m = fmaxf(m, swap8(m));
  opaque_raw(raw);
  uint32_t sc;
  const float rb = block_scale(m, S, lut, &sc);
  const int64_t nbc = C / 16, nbr = R / 16;
  if (!L.hi) {
    o0.scales[(L.r0 / 16) * nbc + L.c0 / 16] = (uint8_t)sc;
    o1.scales[(L.c0 / 16) * nbr + L.r0 / 16] = (uint8_t)sc;
  }
  uint32_t w[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = bf16_at(raw[i], k);
    w[i] = pack8_rtn(v, rb);
    if (st)
      st->codes[stage_dword((threadIdx.x & 7u) * 16u + i, (threadIdx.x >> 6) * 8u + ((threadIdx.x & 63u) >> 3))] = w[i];
    else
      *reinterpret_cast<uint32_t *>(o0.codes + (L.r0 + i) * (C / 2) + L.c0 / 2) = w[i];
  }
  nibble_transpose8(w);
  nibble_transpose8(w + 8);
#pragma unroll
  for (int j = 0; j < 8; ++j)
    *reinterpret_cast<uint2 *>(o1.codes + (L.c0 + j) * (R / 2) + L.r0 / 2) = make_uint2(w[j], w[8 + j]);
}

// This thread's share of the nparts partial maxima of each output's amax mode
// (written by the amax pass), or the maximum the caller gave (thread 0).  The
// loads are independent and are issued before the micro-tile's, so that
// waiting for them does not wait for the tile.
static_assert(kMaxParts <= 4 * kQThreads, "four partial maxima per thread at most");
template <int NOUT>
__device__ __forceinline__ void load_partials(const QuantArgs &a, uint32_t nparts, float pm[2][4]) {
#pragma unroll
  for (int o = 0; o < NOUT; ++o) {
    const float *part = a.partials + a.o[o].amax_mode * kMaxParts;
    const bool given = a.o[o].amax_in != nullptr;  // producer-fused
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t p = threadIdx.x + k * kQThreads;
      pm[o][k] = (!given && p < nparts) ? part[p] : 0.0f;
    }
    if (given && threadIdx.x == 0) pm[o][0] = *a.o[o].amax_in;
  }
}

// Global scale of each output from its partial maxima (load_partials), and
// the table r(c) = S / E4M3(c) of element factors (0 for the zero scale).
// Threads 0-127 build output 0's table, threads 128-255 output 1's; each
// thread derives its output's S itself from the wave maxima, so two barriers
// serve both outputs.  The workgroup with `writer` set (the one that holds
// the tensor's first tile) also stores S and amax.
static_assert(kQThreads == 256, "one half of the workgroup per output table");
template <int NOUT>
__device__ __forceinline__ void quant_setup(const QuantArgs &a, const float pm[2][4], float s_S[2],
                                            float s_lut[2][128], bool writer) {
  __shared__ float s_red[2][kQThreads / 64];
  const uint32_t w = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 0; o < NOUT; ++o) {
    const float m = wave_max(fmaxf(fmaxf(pm[o][0], pm[o][1]), fmaxf(pm[o][2], pm[o][3])));
    if (lane == 0) s_red[o][w] = m;
  }
  __syncthreads();
  const uint32_t o = (NOUT == 2) ? (threadIdx.x >> 7) : 0u, c = threadIdx.x & 127u;
  float amax = s_red[o][0];
#pragma unroll
  for (int i = 1; i < kQThreads / 64; ++i) amax = fmaxf(amax, s_red[o][i]);
  float S = 2688.0f / amax;  // 448 * 6
  if (amax == 0.0f || !__builtin_isfinite(S)) S = 1.0f;
  if (threadIdx.x == 128u * o) {
    s_S[o] = S;
    if (writer) {
      *a.o[o].S_out = S;
      *a.o[o].amax_out = amax;
    }
  }
  if (c < 127u && (NOUT == 2 || threadIdx.x < 128u)) {
    const float val = e4m3_value(c);
    s_lut[o][c] = (val == 0.0f) ? 0.0f : S / val;
  }
  __syncthreads();
}

// All outputs of one micro-tile: outputs without the RHT first, then the RHT
// ones.  A column-block output applies its signs while unpacking; a row-block
// output has its signs XORed into the raw bf16 values (undone if another
// output follows).  Between passes raw is either changed by such a flip or
// fenced by opaque_raw, so that the compiler does not keep one pass's
// unpacked values live for the next.  (A fence before the first pass would
// make every load land before any work starts, so there is none.)
template <int G0, bool RHT0, bool SR0, int G1, bool RHT1, bool SR1>
__device__ __forceinline__ void quant_tile(uint4 raw[16], const Lane &L, const QuantArgs &a, const float s_S[2],
                                           const float s_lut[2][128], RowStage *st = nullptr) {
  constexpr int NOUT = (G1 == G_NONE) ? 1 : 2;
  if (!RHT0) quantize_output<G0, false, SR0>(raw, L, a.o[0], s_S[0], s_lut[0], a.R, a.C, 0u, st);
  if (NOUT == 2 && !RHT0 && !RHT1) opaque_raw(raw);
  if (NOUT == 2 && !RHT1) quantize_output<G1, false, SR1>(raw, L, a.o[1], s_S[1], s_lut[1], a.R, a.C, 0u);
  if (RHT0) {
    if (G0 == G_COL) {
      if (NOUT == 2 && !RHT1) opaque_raw(raw);  // the non-RHT output went first
    } else {
      flip_cols(raw, a.mask_cols, L.hi);
    }
    quantize_output<G0, true, SR0>(raw, L, a.o[0], s_S[0], s_lut[0], a.R, a.C, a.mask_rows);
    if (NOUT == 2 && RHT1 && G0 != G_COL) flip_cols(raw, a.mask_cols, L.hi);  // undo
  }
  if (NOUT == 2 && RHT1) {
    if (G1 == G_COL)
      opaque_raw(raw);  // another pass went first
    else
      flip_cols(raw, a.mask_cols, L.hi);
    quantize_output<G1, true, SR1>(raw, L, a.o[1], s_S[1], s_lut[1], a.R, a.C, a.mask_rows);
  }
}

}  // namespace nvfp4
