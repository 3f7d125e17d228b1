// Device helpers for the NVFP4 kernels (gfx950): bf16 unpacking, the E4M3
// block-scale codec, the E2M1 element encoders, Philox4x32-10 and the 16-point
// Hadamard butterfly.
//
// Method: NVFP4 pretraining news page (zubnet.ai), paragraph 2 -- E2M1 elements
// in 16-element blocks, E4M3 block scales, FP32 per-tensor scale, stochastic
// rounding for gradients, 16x16 random Hadamard transforms on Wgrad inputs.
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

// Stochastic rounding with a 16-bit uniform: a' = min(|y|, 6) lies between grid
// neighbours lo <= a' <= hi; round up iff u16 < 65536 * (a' - lo) / (hi - lo).
// For a' >= 1 the grid points are the binary32 values with one mantissa bit:
// a step is one unit of bit 22, and the low 22 bits d give the fraction d / 2^22,
// so rounding up (d > 64 u16) is exactly a carry into bit 22 when 2^22 - 1 -
// 64 u16 is added; the carry also crosses binades (1.5 -> 2, 3 -> 4).  Below 1
// the spacing is 1/2: t = 2a' is exact and its fraction t - floor(t) is
// compared in binary32 (exact).  Both forms are evaluated and one selected.
__device__ __forceinline__ uint32_t e2m1_sr(float y, uint32_t u16) {
  const uint32_t sign = (__float_as_uint(y) >> 28) & 8u;
  const float a = fminf(fabsf(y), 6.0f);
  const uint32_t code_hi = ((__float_as_uint(a) + (0x3FFFFFu - (u16 << 6))) >> 22) - 252u;
  const float t = a * 2.0f;
  const float fr = __builtin_amdgcn_fractf(t);
  const uint32_t code_lo = (uint32_t)t + (((float)u16 < fr * 65536.0f) ? 1u : 0u);
  return (a >= 1.0f ? code_hi : code_lo) | sign;
}

// -------------------------------------------------------------- Philox ----
// Philox4x32-10 (Salmon et al., SC'11).  c[] in: counter, out: 4 random words.
__device__ __forceinline__ void philox4x32_10(uint32_t k0, uint32_t k1, uint32_t c[4]) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c[0];
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c[2];
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c[1] ^ k0;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c[3] ^ k1;
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
