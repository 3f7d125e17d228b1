// Device helpers for the NVFP4 kernels (gfx950): bf16 unpacking, the E4M3
// block-scale codec, the E2M1 element encoders, Philox4x32-10 and the 16-point
// Hadamard butterfly.
//
// Method: NVFP4 pretraining news page (zubnet.ai), paragraph 2 -- blocks of 16
// E2M1 values with an E4M3 scale each, an FP32 scale per tensor, stochastic
// rounding for gradients, a 16-point randomised Hadamard transform on the
// weight-gradient inputs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

constexpr int kWave = 64;

// ---------------------------------------------------------------- bf16 ----
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// element k (0..7) of 8 bf16 packed in a uint4
__device__ __forceinline__ float bf16_at(const uint4 &q, int k) {
  uint32_t w = (k >> 1) == 0 ? q.x : (k >> 1) == 1 ? q.y : (k >> 1) == 2 ? q.z : q.w;
  return (k & 1) ? bf16_hi(w) : bf16_lo(w);
}

// ---------------------------------------------------------------- E4M3 ----
// OCP E4M3FN, nearest-even, saturating at 448, subnormals m * 2^-9 kept.
// s must be finite and >= 0.  The gfx950 FP8 conversion (OCP E4M3FN,
// nearest-even, subnormals kept) of min(s, 448): clamping first gives the
// saturation (values from 448 up encode as 448, code 0x7E).
__device__ __forceinline__ uint32_t e4m3_encode(float s) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(fminf(s, 448.0f), 0.0f, 0, false) & 0xFFu;
}

__device__ __forceinline__ float e4m3_value(uint32_t c) {
  uint32_t e = (c >> 3) & 15u, m = c & 7u;
  return e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
}

// ---------------------------------------------------------------- E2M1 ----
// Nearest-even onto {0,.5,1,1.5,2,3,4,6}, saturating, sign kept: the gfx950
// conversion instruction with a unit scale (its scale operand only contributes
// an exponent; with 1.0 it is the plain conversion).  Two values -> one byte
// (first value in the low nibble) placed in byte `sel` of `old`.
#define NVFP4_CVT_PK_FP4(old, a, b, sel) __builtin_amdgcn_cvt_scalef32_pk_fp4_f32((old), (a), (b), 1.0f, (sel))

// Stochastic rounding with a 16-bit uniform u16: a' = min(|y|, 6) lies between
// grid neighbours lo <= a' <= hi, and the magnitude rounds up iff
// u16 < 65536 (a' - lo) / (hi - lo).
// Stochastic rounding on the gfx950 conversion instruction
// v_cvt_scalef32_sr_pk_fp4_f32 (two values -> one byte; the scale operand
// divides, contributing its exponent only).  For each value it computes the
// position f of |x| between its two E2M1 neighbours, truncated to 22 bits,
// and rounds the magnitude up iff (R >> 10) + floor(2^22 f) >= 2^22 (R the
// 32-bit random operand; the pair's second value uses R rotated left by one).
// That equals the 16-bit rule above once
//   * |y| is first rounded up to a multiple of 2^-23: f then has 22 bits
//     (from 1 upwards it always has; below 1 the rounding-up changes
//     ceil(65536 f), the count of rounding-up u16, not at all), and
//   * R >> 10 = 2^22 - 1 - 64 u16, i.e. R = ~(u16 << 16) | 0xFFFF, since then
//     the instruction rounds up iff floor(2^22 f) > 64 u16, i.e. u16 < 65536 f.
// The rounding-up of |y| is done at scale 2^23 (t = y * 2^23 is exact; the
// ceiling is of |t|, with y's sign put back), and the instruction's scale
// operand 2^23 divides it back exactly.  The sign is handled by the instruction (sign-magnitude,
// -0 gives code 8).  Each call converts one value, in the first slot (so R is
// used unrotated); the second slot gets +0, whose code is 0 under any R.
__device__ __forceinline__ float sr_hw_prepare(float y) {
  const float t = y * 8388608.0f;  // 2^23
  return __builtin_copysignf(__builtin_ceilf(__builtin_fabsf(t)), t);
}
// the random operand R = ~(u16 << 16) | 0xFFFF for a uniform held in bits
// 0..15 of a word w (lo) or in bits 16..31 (hi, where ~u16 already sits in
// bits 31..16 of ~w); nw = ~w
__device__ __forceinline__ uint32_t sr_hw_rand_lo(uint32_t nw) { return __builtin_amdgcn_alignbit(nw, 0xFFFFFFFFu, 16); }
__device__ __forceinline__ uint32_t sr_hw_rand_hi(uint32_t nw) { return nw | 0xFFFFu; }
typedef float nvfp4_float2 __attribute__((ext_vector_type(2)));
// The conversion writes byte `SEL` of its destination and keeps the other
// three (probed on the device).  The compiler's builtin for it does not tie
// the destination to the `old` operand, so chained calls would lose the
// earlier bytes; the instruction is written here with the destination tied
// explicitly (scale 2^23: it divides the pre-rounded value back exactly).
template <int SEL>
__device__ __forceinline__ uint32_t cvt_sr_fp4(uint32_t dst, float a, float b, uint32_t rnd) {
  const nvfp4_float2 v = {a, b};
  const float scale = 8388608.0f;
  if constexpr (SEL == 0)
    asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, %3" : "+v"(dst) : "v"(v), "v"(rnd), "v"(scale));
  else if constexpr (SEL == 1)
    asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, %3 op_sel:[0,0,1,0]" : "+v"(dst) : "v"(v), "v"(rnd), "v"(scale));
  else if constexpr (SEL == 2)
    asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, %3 op_sel:[0,0,0,1]" : "+v"(dst) : "v"(v), "v"(rnd), "v"(scale));
  else
    asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, %3 op_sel:[0,0,1,1]" : "+v"(dst) : "v"(v), "v"(rnd), "v"(scale));
  return dst;
}

// one element: code of y under uniform u16, with the random operand built as
// the kernels build it for an element of that parity (even: u16 in the low
// half of its Philox word, odd: in the high half)
__device__ __forceinline__ uint32_t e2m1_sr_hw(float y, uint32_t u16, int odd) {
  const float c = sr_hw_prepare(y);
  if (!odd) return cvt_sr_fp4<0>(0u, c, 0.0f, sr_hw_rand_lo(~u16)) & 0xFu;
  return cvt_sr_fp4<0>(0u, c, 0.0f, sr_hw_rand_hi(~(u16 << 16))) & 0xFu;
}

// -------------------------------------------------------------- Philox ----
// Philox4x32-10 (Salmon et al., SC'11).  c[] in: counter, out: 4 random words.
__device__ __forceinline__ void philox4x32_10(uint32_t k0, uint32_t k1, uint32_t c[4]) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c[0];
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c[2];
    uint32_t n0, n2;
    if (r < 2) {  // the first rounds see the zero counter words: left to constant folding
      n0 = (uint32_t)(p1 >> 32) ^ c[1] ^ k0;
      n2 = (uint32_t)(p0 >> 32) ^ c[3] ^ k1;
    } else {  // three-way XOR in one instruction
      n0 = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c[1], k0, 0x96);
      n2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c[3], k1, 0x96);
    }
    c[1] = (uint32_t)p1;
    c[3] = (uint32_t)p0;
    c[0] = n0;
    c[2] = n2;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
}

// The 8 words of the two Philox draws that serve one 16-element block:
// draw g = 2*block + half, counter (g, 0, 0, 0) -- block indices stay below
// 2^31 (checked on the host), so the counter's high word is 0.  Element j of
// the block uses word (j & 7) >> 1 of draw j >> 3, 16-bit half j & 1.
__device__ __forceinline__ void sr_draw(uint64_t seed, uint32_t block, uint32_t half, uint32_t w[4]) {
  w[0] = 2u * block + half;
  w[1] = 0u;
  w[2] = 0u;
  w[3] = 0u;
  philox4x32_10((uint32_t)seed, (uint32_t)(seed >> 32), w);
}

__device__ __forceinline__ uint32_t u16_of(const uint32_t w[4], int k) {  // k = j & 7
  const uint32_t word = (k >> 1) == 0 ? w[0] : (k >> 1) == 1 ? w[1] : (k >> 1) == 2 ? w[2] : w[3];
  return (k & 1) ? (word >> 16) : (word & 0xFFFFu);
}

// ------------------------------------------------------------ Hadamard ----
// In-place 16-point fast Walsh-Hadamard transform in binary32 (Sylvester
// order: out_i = sum_j (-1)^popcount(i&j) in_j).  Each butterfly addition is
// rounded, so a result can differ from the exactly rounded sum by a few units
// in the last place when the 16 inputs span many binades; the quantised
// outputs of the RHT paths are compared with a tolerance for that reason.
__device__ __forceinline__ void fwht16(float v[16]) {
#pragma unroll
  for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if ((i & h) == 0) {
        const float a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
    }
  }
}

// ------------------------------------------------------------- lanes ------
// value of lane (lane ^ 8) -- rotate by 8 inside each row of 16 lanes
__device__ __forceinline__ float swap8(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x128, 0xF, 0xF, false));  // row_ror:8
}
// ------------------------------------------------------------- XCDs -------
// Workgroups are dealt round-robin to the 8 XCDs; remap so that each XCD works
// on one contiguous range of tiles (neighbouring tiles share its L2).
__device__ __forceinline__ uint32_t xcd_tile(uint32_t b, uint32_t n) {
  const uint32_t per = n / 8u, rem = n % 8u, x = b % 8u, i = b / 8u;
  return x < rem ? x * (per + 1u) + i : rem * (per + 1u) + (x - rem) * per + i;
}

}  // namespace nvfp4
