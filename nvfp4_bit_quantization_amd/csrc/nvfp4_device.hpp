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
// s must be finite and >= 0.  Branch-free: both the normal and the subnormal
// encodings are formed and the right one selected.
__device__ __forceinline__ uint32_t e4m3_encode(float s) {
  const uint32_t u = __float_as_uint(s);
  // normal range: round the 23-bit mantissa to 3 bits (ties to even), rebias 127 -> 7
  const uint32_t normal = ((u + 0x7FFFFu + ((u >> 20) & 1u)) >> 20) - (120u << 3);
  // below the smallest normal 2^-6: multiples of 2^-9 (exact scaling, then RNE)
  const uint32_t sub = (uint32_t)__builtin_rintf(s * 512.0f);
  const uint32_t c = s < 0.015625f ? sub : normal;
  return s >= 448.0f ? 0x7Eu : c;
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
// grid neighbours lo <= a' <= hi, and rounds up iff u16 < 65536 (a' - lo) /
// (hi - lo).  With an integer u16 that is the same as u16 < ceil(65536 f)
// for the exact fraction f, i.e. a carry out of (ceil(65536 f) + 65535 - u16)
// into bit 16.  Two exact forms of the sum, each valid on part of the range:
//   * a' < 2, where the grid ordinal is 2a' (steps of 1/2):
//     T = ceil(2^17 a') is computed exactly in binary32 (a power-of-two
//     scaling, then a ceiling), and the code is (T + 65535 - u16) >> 16;
//   * a' >= 1, where every grid point is a binary32 value with one mantissa
//     bit: a step is one unit of bit 22 of the bit pattern, the low 22 bits d
//     give f = d / 2^22, and the code is (bits(a') + 2^22 - 1 - 64 u16) >> 22
//     less the ordinal offset of 1.0 (the carry also crosses binades).
// Both sums are formed at the scale of bit 22 (the first as 64 T), offset so
// that one constant finishes either: X_lo = 64 T + bits(2^16) and X_hi =
// bits(2^17 a') = bits(a') + 17 * 2^23.  For a' < 1, X_hi <= X_lo <= bits(2^17);
// for a' >= 1, bits(2^17) <= X_hi <= X_lo; so the median of the three picks
// the right one (compared as positive binary32 values, i.e. as integers).
// Then (u16 << 6) ^ 0xB8BFFFFF = 2^22 - 1 - 64 u16 - bits(2^16) (mod 2^32) is
// added and bits 22.. give the magnitude code 0..7.
__device__ __forceinline__ uint32_t e2m1_sr_mag(float y, uint32_t u16) {
  const float a17 = fminf(fabsf(y * 131072.0f), 786432.0f);  // 2^17 a', exact
  const uint32_t t = (uint32_t)__builtin_ceilf(a17);
  const uint32_t x_lo = (t << 6) + 0x47800000u;
  const float x = __builtin_amdgcn_fmed3f(__uint_as_float(x_lo), 131072.0f, a17);
  return (((u16 << 6) ^ 0xB8BFFFFFu) + __float_as_uint(x)) >> 22;
}

// the full code: magnitude plus the sign bit of y (-0 gives 0x8)
__device__ __forceinline__ uint32_t e2m1_sr(float y, uint32_t u16) {
  return e2m1_sr_mag(y, u16) | ((__float_as_uint(y) >> 28) & 8u);
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
