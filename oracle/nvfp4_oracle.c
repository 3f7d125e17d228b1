/*
 * nvfp4_oracle.c -- plain, slow CPU oracle for the NVFP4 quantisation pipeline
 * and the NVFP4-operand GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark do.  It shares no code, header, table or constant generator
 * with the HIP path.
 *
 * Source of the method: "NVIDIA NVFP4 paper: 4-bit pretrain hits FP8 parity"
 * (zubnet.ai news page, en/pt/fr/hi), paragraph 2 (the stabilising
 * techniques and the number format): blocks of 16 E2M1 values with an E4M3
 * scale each, under one FP32 scale per tensor; a 16x16 randomised Hadamard
 * transform (random +/-1 signs) on the weight-gradient inputs; 16x16 scale
 * blocks for weights; stochastic rounding for gradients and for nothing else.
 * The page gives no
 * formulas; the arithmetic convention below (global scale 448*6/amax, block
 * scale E4M3(amax_b/6 * S), elements scaled onto the E2M1 grid
 * {0,.5,1,1.5,2,3,4,6}) is the fixed convention of this project, and every
 * point the page leaves open is a reading of this project, named where the
 * code takes it.
 *
 * Precision: the page fixes the per-tensor scale as FP32, so the scale chain
 * (S, block scale, per-block factor, scaled element) is evaluated as single
 * IEEE-754 binary32 operations with round-to-nearest-even, one operation per
 * statement (build with -ffp-contract=off).  The Hadamard sums are evaluated in
 * binary64 (exact for 16 bf16 terms whose exponents span fewer than 41
 * binades) and rounded once to binary32.  Grid searches (E2M1, E4M3) compare
 * against exact binary64 midpoints.
 *
 * Loops over independent rows or blocks run in parallel (OpenMP); every value
 * is produced by the same sequence of operations at any thread count, and the
 * per-tensor maximum does not depend on the order of comparisons.
 *
 * Parity pins: every function here is checked by the tests under tests/
 * against enumeration, brute force, closed forms, a library routine or
 * invariants (see each function's comment).  The storage conventions (nibble
 * order, code/scale layouts, Philox counter assignment, block order) are a
 * choice of this project with no value on the page to check them against:
 * parity unpinned beyond their own definition.
 */
#include <stdint.h>
#include <string.h>
#include <math.h>
#include <stddef.h>
#ifdef _OPENMP
#include <omp.h>
#endif
#include <stdlib.h>

/* ---- enumerations (the library's C header defines the same numbers) ---- */
#define OR_ROW_1D 0 /* 1D 16-element blocks along the contiguous dim, output [R][C] */
#define OR_COL_1D 1 /* 1D 16-element blocks along rows, output is x^T [C][R] */
#define OR_2D 2     /* aligned 16x16 tiles, output [R][C] */
#define OR_2D_T 3   /* the same per-element results as OR_2D, stored as [C][R] */
#define OR_RTN 0
#define OR_SR 1
#define OR_SCALE_1D16 0
#define OR_SCALE_2D16 1

/* ------------------------------------------------------------------------ */
/* bf16 / fp32 helpers                                                        */
/* ------------------------------------------------------------------------ */
/* Threads the parallel loops use (1 in a build without OpenMP). */
int oracle_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Set the threads of the parallel loops (n >= 1; no effect without OpenMP).
 * Results do not depend on it: every loop writes disjoint outputs, and the
 * one reduction is a maximum. */
void oracle_set_threads(int n) {
#ifdef _OPENMP
  if (n >= 1) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

static float bf16_bits_to_float(uint16_t h) {
  uint32_t u = (uint32_t)h << 16; /* bf16 is the top half of a binary32 */
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* ------------------------------------------------------------------------ */
/* E2M1 element code.  Reading: bit3 = sign, bits 2:1 = exponent (bias 1),    */
/* bit0 = mantissa; magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6 for codes 0..7.      */
/* Pinned by enumeration of all 16 codes against the grid.                    */
/* ------------------------------------------------------------------------ */
static const double E2M1_GRID[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double oracle_e2m1_value(uint8_t code) {
  double m = E2M1_GRID[code & 7];
  return (code & 8) ? -m : m;
}

/* Round-to-nearest onto the E2M1 grid, ties to the even mantissa bit (code & 1
 * == 0), magnitudes above 6 saturate to 6, the sign is kept (so -0 -> 0x8).
 * Pinned by brute force over fp32 bit patterns against an exact-rational
 * nearest-even search and by the hand-derived threshold list. */
uint8_t oracle_e2m1_encode_rtn(float y) {
  uint8_t sign = signbit(y) ? 8 : 0;
  double a = fabs((double)y);
  if (a >= 6.0) return sign | 7;
  int i = 0;
  while (i < 7 && E2M1_GRID[i + 1] <= a) i++; /* grid[i] <= a < grid[i+1] */
  if (E2M1_GRID[i] == a) return sign | (uint8_t)i;
  double mid = 0.5 * (E2M1_GRID[i] + E2M1_GRID[i + 1]); /* exact dyadic */
  int pick;
  if (a < mid)
    pick = i;
  else if (a > mid)
    pick = i + 1;
  else
    pick = ((i & 1) == 0) ? i : i + 1; /* tie: even mantissa bit */
  return sign | (uint8_t)pick;
}

/* Stochastic rounding onto the E2M1 grid with a 16-bit uniform u16.
 * a' = min(|y|, 6); lo <= a' <= hi are the neighbouring grid points;
 * frac = (a' - lo)/(hi - lo) (exact: both differences are dyadic and hi - lo
 * is a power of two); round away from zero iff u16 < frac * 65536.
 * Pinned by enumerating all 65536 u16 (exactly ceil(frac*65536) round-ups)
 * and by unbiasedness over 1e5 Philox draws. */
uint8_t oracle_e2m1_encode_sr(float y, uint16_t u16) {
  uint8_t sign = signbit(y) ? 8 : 0;
  double a = fabs((double)y);
  if (a > 6.0) a = 6.0;
  int i = 0;
  while (i < 7 && E2M1_GRID[i + 1] <= a) i++;
  if (E2M1_GRID[i] == a) return sign | (uint8_t)i;
  double frac = (a - E2M1_GRID[i]) / (E2M1_GRID[i + 1] - E2M1_GRID[i]);
  double threshold = frac * 65536.0;
  int up = ((double)u16 < threshold) ? 1 : 0;
  return sign | (uint8_t)(i + up);
}

/* ------------------------------------------------------------------------ */
/* E4M3 block scale (OCP E4M3FN: bias 7, max 448 = 0x7E, 0x7F = NaN,          */
/* subnormals m * 2^-9).  Pinned by enumeration of all 256 codes and by an    */
/* exhaustive comparison with torch's float8_e4m3fn cast (after a clamp).     */
/* ------------------------------------------------------------------------ */
float oracle_e4m3_value(uint8_t code) {
  int e = (code >> 3) & 15, m = code & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = m * ldexp(1.0, -9);
  else
    v = (1.0 + m / 8.0) * ldexp(1.0, e - 7);
  return (float)((code & 0x80) ? -v : v);
}

/* Nearest non-negative finite E4M3 value, ties to even mantissa bit, values at
 * or above 448 saturate to 448 (satfinite).  Input must be finite and >= 0;
 * the block scales are never negative. */
uint8_t oracle_e4m3_encode(float x) {
  double a = (double)x;
  if (!(a > 0.0)) return 0;
  if (a >= 448.0) return 0x7E;
  /* codes 0x00..0x7E are increasing in value: binary search for the last
   * code whose value is <= a */
  int lo = 0, hi = 0x7E;
  while (lo < hi) {
    int mid = (lo + hi + 1) / 2;
    if ((double)oracle_e4m3_value((uint8_t)mid) <= a)
      lo = mid;
    else
      hi = mid - 1;
  }
  double vlo = oracle_e4m3_value((uint8_t)lo);
  if (vlo == a) return (uint8_t)lo;
  double vhi = oracle_e4m3_value((uint8_t)(lo + 1));
  double mid = 0.5 * (vlo + vhi);
  if (a < mid) return (uint8_t)lo;
  if (a > mid) return (uint8_t)(lo + 1);
  return (lo & 1) == 0 ? (uint8_t)lo : (uint8_t)(lo + 1);
}

/* ------------------------------------------------------------------------ */
/* Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as    */
/* easy as 1, 2, 3", SC'11): 10 rounds of two 32x32->64 multiplications, key  */
/* incremented by the Weyl constants between rounds.  Pinned against the      */
/* open-source rocRAND engine and a second pure-Python implementation.        */
/* ------------------------------------------------------------------------ */
void oracle_philox4x32_10(const uint32_t key_in[2], const uint32_t ctr_in[4], uint32_t out[4]) {
  uint32_t k0 = key_in[0], k1 = key_in[1];
  uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
  for (int round = 0; round < 10; round++) {
    if (round > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    uint32_t n0 = hi1 ^ c1 ^ k0;
    uint32_t n1 = lo1;
    uint32_t n2 = hi0 ^ c3 ^ k1;
    uint32_t n3 = lo0;
    c0 = n0;
    c1 = n1;
    c2 = n2;
    c3 = n3;
  }
  out[0] = c0;
  out[1] = c1;
  out[2] = c2;
  out[3] = c3;
}

/* 16-bit uniform for element j (0..15) of output-order block b under seed:
 * counter = (g lo, g hi, 0, 0) with g = 2b + (j >> 3); the element takes the
 * 16-bit half (j & 1) of word (j & 7) >> 1.  Counter word 2 = 0 keeps this
 * stream apart from the sign-vector draw (word 2 = 1). */
uint16_t oracle_sr_uniform(uint64_t seed, uint64_t block, int j) {
  uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  uint64_t g = 2 * block + (uint64_t)(j >> 3);
  uint32_t ctr[4] = {(uint32_t)g, (uint32_t)(g >> 32), 0u, 0u};
  uint32_t w[4];
  oracle_philox4x32_10(key, ctr, w);
  uint32_t word = w[(j & 7) >> 1];
  return (uint16_t)((word >> (16 * (j & 1))) & 0xFFFFu);
}

/* ------------------------------------------------------------------------ */
/* Random Hadamard transform on one 16-group: z_i = 1/4 sum_j H[i][j] d_j v_j,  */
/* H[i][j] = (-1)^popcount(i & j) (Sylvester order), d_j = -1 iff bit j of    */
/* the sign mask.  The 1/4 makes the transform orthonormal.                   */
/* Pinned by H H^T = 16 I, exact inversion and (QA)^T(QB) = A^T B.            */
/* ------------------------------------------------------------------------ */
uint16_t oracle_rht_sign_mask(uint64_t rht_seed) {
  uint32_t key[2] = {(uint32_t)rht_seed, (uint32_t)(rht_seed >> 32)};
  uint32_t ctr[4] = {0u, 0u, 1u, 0u};
  uint32_t w[4];
  oracle_philox4x32_10(key, ctr, w);
  return (uint16_t)(w[0] & 0xFFFFu);
}

static int popcount4(int v) { return (v & 1) + ((v >> 1) & 1) + ((v >> 2) & 1) + ((v >> 3) & 1); }

/* in: 16 values; out: 16 binary64 exact(-ish) sums before the final rounding */
void oracle_rht16_f64(const double v[16], uint16_t sign_mask, double z[16]) {
  for (int i = 0; i < 16; i++) {
    double s = 0.0;
    for (int j = 0; j < 16; j++) {
      double h = (popcount4(i & j) & 1) ? -1.0 : 1.0;
      double d = ((sign_mask >> j) & 1) ? -1.0 : 1.0;
      s += h * d * v[j];
    }
    z[i] = 0.25 * s;
  }
}

/* ------------------------------------------------------------------------ */
/* Quantisation of one output orientation.                                    */
/* x: bf16 bit patterns, [R][C] row-major with row stride ld (elements).      */
/* layout OR_ROW_1D / OR_2D / OR_2D_T: output rows = R, cols = C              */
/* layout OR_COL_1D:                   output rows = C, cols = R (x^T)        */
/* OR_2D_T stores the OR_2D results transposed: codes [C][R/2], scales        */
/* [C/16][R/16].                                                              */
/* codes: [out_rows][out_cols/2], element 2i in the low nibble.               */
/* scales: 1D [out_rows][out_cols/16]; 2D [out_rows/16][out_cols/16].         */
/* Returns 0, or -1 for an unsupported combination (shapes not multiples of   */
/* 16, RHT with a 2D layout, unknown enums).                                  */
/* ------------------------------------------------------------------------ */
static float v_at(const uint16_t *x, int64_t ld, int64_t r, int64_t c) {
  return bf16_bits_to_float(x[r * ld + c]);
}

int oracle_quantize_at(const uint16_t *x, int64_t R, int64_t C, int64_t ld, int layout, int rounding, int rht,
                       uint64_t sr_seed, uint64_t rht_seed, uint64_t block_offset, uint8_t *codes, uint8_t *scales,
                       float *S_out, float *amax_out);

int oracle_quantize(const uint16_t *x, int64_t R, int64_t C, int64_t ld, int layout, int rounding, int rht,
                    uint64_t sr_seed, uint64_t rht_seed, uint8_t *codes, uint8_t *scales, float *S_out,
                    float *amax_out) {
  return oracle_quantize_at(x, R, C, ld, layout, rounding, rht, sr_seed, rht_seed, 0, codes, scales, S_out,
                            amax_out);
}

/* As oracle_quantize, for a slice of a larger tensor: the stochastic-rounding
 * block index is block_offset + the slice's own block index (block_offset =
 * the blocks that precede the slice in output order, e.g. rows x cols/16 for
 * a slice starting at that output row).  Everything else is unchanged. */
int oracle_quantize_at(const uint16_t *x, int64_t R, int64_t C, int64_t ld, int layout, int rounding, int rht,
                       uint64_t sr_seed, uint64_t rht_seed, uint64_t block_offset, uint8_t *codes, uint8_t *scales,
                       float *S_out, float *amax_out) {
  if (R <= 0 || C <= 0 || (R % 16) || (C % 16) || ld < C) return -1;
  if (layout < OR_ROW_1D || layout > OR_2D_T) return -1;
  if (rounding != OR_RTN && rounding != OR_SR) return -1;
  if (rht && (layout == OR_2D || layout == OR_2D_T)) return -1;

  /* Step 1: the values to quantise, v, in the working orientation
   * (rows x cols).  2D and 2D_T work on x itself; the transpose of 2D_T is
   * applied only when storing. */
  int transposed_input = (layout == OR_COL_1D);
  int64_t rows = transposed_input ? C : R;
  int64_t cols = transposed_input ? R : C;
  size_t n = (size_t)rows * (size_t)cols;
  float *v = (float *)malloc(n * sizeof(float));
  if (!v) return -2;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; r++)
    for (int64_t c = 0; c < cols; c++)
      v[r * cols + c] = transposed_input ? v_at(x, ld, c, r) : v_at(x, ld, r, c);

  /* Step 2: optional 16x16 RHT along the block dimension (the columns of the
   * working orientation: hidden for ROW_1D, tokens for COL_1D). */
  if (rht) {
    uint16_t mask = oracle_rht_sign_mask(rht_seed);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++)
      for (int64_t g = 0; g < cols; g += 16) {
        double in[16], z[16];
        for (int j = 0; j < 16; j++) in[j] = (double)v[r * cols + g + j];
        oracle_rht16_f64(in, mask, z);
        for (int j = 0; j < 16; j++) v[r * cols + g + j] = (float)z[j];
      }
  }

  /* Step 3: per-tensor amax and Step 4: the FP32 global (encode) scale. */
  float amax = 0.0f;
#pragma omp parallel for schedule(static) reduction(max : amax)
  for (size_t i = 0; i < n; i++) {
    float a = fabsf(v[i]);
    if (a > amax) amax = a;
  }
  float S = 2688.0f / amax; /* 2688 = 448 * 6 */
  if (amax == 0.0f || !isfinite(S)) S = 1.0f;
  *S_out = S;
  *amax_out = amax;

  /* Steps 5-6: per block, the E4M3 scale, then each element. */
  int is2d = (layout == OR_2D || layout == OR_2D_T);
  int64_t bh = is2d ? 16 : 1; /* block height in the working orientation */
  int64_t nbc = cols / 16;
#pragma omp parallel for schedule(static)
  for (int64_t br = 0; br < rows; br += bh)
    for (int64_t bc = 0; bc < nbc; bc++) {
      float amax_b = 0.0f;
      for (int64_t r = br; r < br + bh; r++)
        for (int64_t c = bc * 16; c < bc * 16 + 16; c++) {
          float a = fabsf(v[r * cols + c]);
          if (a > amax_b) amax_b = a;
        }
      float t = amax_b / 6.0f;
      float sb = t * S;
      uint8_t sb_code = oracle_e4m3_encode(sb);
      float sb_val = oracle_e4m3_value(sb_code);
      float rb = (sb_val == 0.0f) ? 0.0f : S / sb_val;

      /* store the scale */
      if (!is2d) {
        scales[br * nbc + bc] = sb_code;
      } else if (layout == OR_2D) {
        scales[(br / 16) * nbc + bc] = sb_code;
      } else { /* OR_2D_T: transposed scale grid [C/16][R/16] */
        scales[bc * (rows / 16) + br / 16] = sb_code;
      }

      for (int64_t r = br; r < br + bh; r++)
        for (int j = 0; j < 16; j++) {
          int64_t c = bc * 16 + j;
          float y = v[r * cols + c] * rb;
          uint8_t code;
          if (rounding == OR_RTN) {
            code = oracle_e2m1_encode_rtn(y);
          } else {
            /* block order: row-major 1D block index of the working
             * orientation (2D uses its row blocks too) */
            uint64_t b = block_offset + (uint64_t)r * (uint64_t)nbc + (uint64_t)bc;
            code = oracle_e2m1_encode_sr(y, oracle_sr_uniform(sr_seed, b, j));
          }
          /* store the code */
          int64_t orow = r, ocol = c, ocols = cols;
          if (layout == OR_2D_T) {
            orow = c;
            ocol = r;
            ocols = rows;
          }
          size_t byte = (size_t)orow * (size_t)(ocols / 2) + (size_t)(ocol / 2);
          if ((ocol & 1) == 0)
            codes[byte] = (uint8_t)((codes[byte] & 0xF0) | code);
          else
            codes[byte] = (uint8_t)((codes[byte] & 0x0F) | (code << 4));
        }
    }
  free(v);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Dequantisation: x^ = (e(code) * s_b) / S, the product exact in binary32,   */
/* one rounding in the division.  Pinned by the closed form and round trips.  */
/* ------------------------------------------------------------------------ */
static uint8_t code_at(const uint8_t *codes, int64_t cols, int64_t r, int64_t c) {
  uint8_t b = codes[r * (cols / 2) + c / 2];
  return (c & 1) ? (uint8_t)(b >> 4) : (uint8_t)(b & 15);
}

static uint8_t scale_at(const uint8_t *scales, int64_t cols, int scale_kind, int64_t r, int64_t c) {
  if (scale_kind == OR_SCALE_1D16) return scales[r * (cols / 16) + c / 16];
  return scales[(r / 16) * (cols / 16) + c / 16];
}

int oracle_dequantize(const uint8_t *codes, const uint8_t *scales, int64_t rows, int64_t cols, int scale_kind,
                      float S, float *y) {
  if (rows <= 0 || cols <= 0 || (rows % 16) || (cols % 16)) return -1;
  if (scale_kind != OR_SCALE_1D16 && scale_kind != OR_SCALE_2D16) return -1;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; r++)
    for (int64_t c = 0; c < cols; c++) {
      float e = (float)oracle_e2m1_value(code_at(codes, cols, r, c));
      float s = oracle_e4m3_value(scale_at(scales, cols, scale_kind, r, c));
      float p = e * s; /* exact: at most 6 significant bits */
      y[r * cols + c] = p / S;
    }
  return 0;
}

/* Exact operand values e(code) * s_b (no global scale), as binary64. */
int oracle_decode_products(const uint8_t *codes, const uint8_t *scales, int64_t rows, int64_t cols, int scale_kind,
                           double *out) {
  if (rows <= 0 || cols <= 0 || (rows % 16) || (cols % 16)) return -1;
  if (scale_kind != OR_SCALE_1D16 && scale_kind != OR_SCALE_2D16) return -1;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; r++)
    for (int64_t c = 0; c < cols; c++)
      out[r * cols + c] = oracle_e2m1_value(code_at(codes, cols, r, c)) *
                          (double)oracle_e4m3_value(scale_at(scales, cols, scale_kind, r, c));
  return 0;
}

/* ------------------------------------------------------------------------ */
/* GEMM: C[m][n] = (sum_k A^[m][k] * B^[n][k]) / (S_A * S_B), A^ = e * s_b,    */
/* both operands K-contiguous.  Plain triple loop in binary64; the caller     */
/* rounds to the output dtype.  Pinned by brute-force agreement with a BLAS   */
/* float64 matmul and a single-block closed form.                             */
/* ------------------------------------------------------------------------ */
int oracle_gemm_f64(const uint8_t *a_codes, const uint8_t *a_scales, int a_kind, float a_S, const uint8_t *b_codes,
                    const uint8_t *b_scales, int b_kind, float b_S, int64_t M, int64_t N, int64_t K, double *c) {
  if (M <= 0 || N <= 0 || K <= 0 || (M % 16) || (N % 16) || (K % 16)) return -1;
  double denom = (double)a_S * (double)b_S; /* exact product of two binary32 */
#pragma omp parallel for schedule(static)
  for (int64_t m = 0; m < M; m++)
    for (int64_t nn = 0; nn < N; nn++) {
      double acc = 0.0;
      for (int64_t k = 0; k < K; k++) {
        double av = oracle_e2m1_value(code_at(a_codes, K, m, k)) *
                    (double)oracle_e4m3_value(scale_at(a_scales, K, a_kind, m, k));
        double bv = oracle_e2m1_value(code_at(b_codes, K, nn, k)) *
                    (double)oracle_e4m3_value(scale_at(b_scales, K, b_kind, nn, k));
        acc += av * bv;
      }
      c[m * N + nn] = acc / denom;
    }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* MXFP4, the earlier 4-bit microscaling format the page sets NVFP4 against  */
/* (paragraph 3).  The page gives no definition of it; the one followed here  */
/* is the OCP Microscaling Formats (MX) specification v1.0 (section 5: MX     */
/* block of k = 32 elements, E8M0 shared scale, FP4 E2M1 elements; section    */
/* 6.3: conversion).  Per block of 32 consecutive elements along the          */
/* contiguous (K) dimension of the output orientation:                        */
/*   e = floor(log2(max |v|)) - 2  (2 = exponent of 4, the largest power of    */
/*       two of E2M1), clamped to the E8M0 range [-127, 127];                 */
/*   X = 2^e, stored as the E8M0 code e + 127;                                */
/*   element = v / X rounded to the nearest E2M1 value, ties to even, values  */
/*       above 6 clamped to 6 (the E2M1 RTN encoder above), sign kept.       */
/* Readings: an all-zero block takes the smallest scale 2^-127 (code 0); the  */
/* code 0xFF (NaN) is never produced (inputs are finite).                     */
/* Pinned by hand-computed codes, brute-force scale and grid searches, the    */
/* block-maximum invariant and an exact rational GEMM on small inputs.        */
/* ------------------------------------------------------------------------ */
uint8_t oracle_e8m0_scale_code(double amax) {
  if (!(amax > 0.0)) return 0;
  int fe;
  frexp(amax, &fe); /* amax = f 2^fe, f in [0.5, 1): floor(log2 amax) = fe - 1 */
  int e = fe - 1 - 2;
  if (e < -127) e = -127;
  if (e > 127) e = 127;
  return (uint8_t)(e + 127);
}

double oracle_e8m0_value(uint8_t code) { return ldexp(1.0, (int)code - 127); }

/* layout OR_ROW_1D: blocks along C, output [R][C]; OR_COL_1D: blocks along R,
 * output x^T [C][R].  codes [orow][ocol/2] (element 2i in the low nibble),
 * scales [orow][ocol/32].  The blocked dimension must be a multiple of 32.
 * Returns 0, or -1 for unsupported arguments. */
int oracle_mx_quantize(const uint16_t *x, int64_t R, int64_t C, int64_t ld, int layout, uint8_t *codes,
                       uint8_t *scales) {
  if (R <= 0 || C <= 0 || ld < C) return -1;
  if (layout != OR_ROW_1D && layout != OR_COL_1D) return -1;
  const int64_t orow = layout == OR_ROW_1D ? R : C, ocol = layout == OR_ROW_1D ? C : R;
  if (ocol % 32) return -1;
  memset(codes, 0, (size_t)(orow * (ocol / 2)));
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < orow; r++)
    for (int64_t b = 0; b < ocol / 32; b++) {
      double v[32], amax = 0.0;
      for (int j = 0; j < 32; j++) {
        const int64_t c = b * 32 + j;
        v[j] = layout == OR_ROW_1D ? (double)v_at(x, ld, r, c) : (double)v_at(x, ld, c, r);
        if (fabs(v[j]) > amax) amax = fabs(v[j]);
      }
      const uint8_t sc = oracle_e8m0_scale_code(amax);
      scales[r * (ocol / 32) + b] = sc;
      const double X = oracle_e8m0_value(sc);
      for (int j = 0; j < 32; j++) {
        /* v / X is exact in binary64; in binary32 it can only lose bits when
         * it is below 2^-126, where every value encodes to a signed zero */
        const uint8_t code = oracle_e2m1_encode_rtn((float)(v[j] / X));
        const int64_t c = b * 32 + j;
        codes[r * (ocol / 2) + c / 2] |= (uint8_t)((c & 1) ? (code << 4) : code);
      }
    }
  return 0;
}

/* x^ = e(code) * X, exact in binary64 */
int oracle_mx_decode(const uint8_t *codes, const uint8_t *scales, int64_t rows, int64_t cols, double *out) {
  if (rows <= 0 || cols <= 0 || (cols % 32)) return -1;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; r++)
    for (int64_t c = 0; c < cols; c++)
      out[r * cols + c] = oracle_e2m1_value(code_at(codes, cols, r, c)) * oracle_e8m0_value(scales[r * (cols / 32) + c / 32]);
  return 0;
}

/* C[m][n] = sum_k A^[m][k] B^[n][k], both operands K-contiguous; binary64
 * triple loop (every product exact) */
int oracle_mx_gemm_f64(const uint8_t *a_codes, const uint8_t *a_scales, const uint8_t *b_codes,
                       const uint8_t *b_scales, int64_t M, int64_t N, int64_t K, double *c) {
  if (M <= 0 || N <= 0 || K <= 0 || (K % 32)) return -1;
#pragma omp parallel for schedule(static)
  for (int64_t m = 0; m < M; m++)
    for (int64_t nn = 0; nn < N; nn++) {
      double acc = 0.0;
      for (int64_t k = 0; k < K; k++)
        acc += oracle_e2m1_value(code_at(a_codes, K, m, k)) * oracle_e8m0_value(a_scales[m * (K / 32) + k / 32]) *
               oracle_e2m1_value(code_at(b_codes, K, nn, k)) * oracle_e8m0_value(b_scales[nn * (K / 32) + k / 32]);
      c[m * N + nn] = acc;
    }
  return 0;
}

/* Round a binary64 value to the nearest bf16 (ties to even), returning the
 * bit pattern; one rounding straight from binary64. */
uint16_t oracle_f64_to_bf16(double x) {
  uint16_t sign = signbit(x) ? 0x8000 : 0;
  double a = fabs(x);
  if (isnan(x)) return 0x7FC0;
  if (a == 0.0) return sign;
  int e;
  frexp(a, &e); /* a = f * 2^e, f in [0.5, 1) -> a in [2^(e-1), 2^e) */
  int E = e - 1; /* a in [2^E, 2^(E+1)) */
  if (E < -126) E = -126; /* bf16 subnormal range: fixed quantum 2^-133 */
  double q = ldexp(a, 7 - E); /* significand scaled to [128, 256) for normals */
  double qi = nearbyint(q);   /* default rounding mode: nearest, ties to even */
  int64_t iq = (int64_t)qi;
  if (iq >= 256) { /* rounded up into the next binade */
    iq >>= 1;
    E += 1;
  }
  if (iq < 128) { /* subnormal (E == -126 only) */
    return sign | (uint16_t)iq;
  }
  if (E > 127) return sign | 0x7F80; /* overflow to infinity */
  uint16_t expf = (uint16_t)(E + 127);
  return sign | (uint16_t)(expf << 7) | (uint16_t)(iq & 0x7F);
}

/* Bulk helpers for the tests (loops over the scalar functions above). */
void oracle_e2m1_encode_rtn_array(const float *y, int64_t n, uint8_t *out) {
  for (int64_t i = 0; i < n; i++) out[i] = oracle_e2m1_encode_rtn(y[i]);
}
void oracle_e2m1_encode_sr_array(const float *y, const uint16_t *u, int64_t n, uint8_t *out) {
  for (int64_t i = 0; i < n; i++) out[i] = oracle_e2m1_encode_sr(y[i], u[i]);
}
void oracle_e4m3_encode_array(const float *x, int64_t n, uint8_t *out) {
  for (int64_t i = 0; i < n; i++) out[i] = oracle_e4m3_encode(x[i]);
}
/* all fp32 bit patterns in [start, start + count): RTN codes */
void oracle_e2m1_encode_rtn_bits(uint32_t start, uint32_t count, uint8_t *out) {
  for (uint32_t i = 0; i < count; i++) {
    uint32_t u = start + i;
    float f;
    memcpy(&f, &u, 4);
    out[i] = isfinite(f) ? oracle_e2m1_encode_rtn(f) : 0xFF;
  }
}
/* all fp32 bit patterns in [start, start + count): E4M3 codes (0xFF for
 * negative, NaN or Inf patterns, which the encoder does not take) */
void oracle_e4m3_encode_bits(uint32_t start, uint32_t count, uint8_t *out) {
  for (uint32_t i = 0; i < count; i++) {
    uint32_t u = start + i;
    float f;
    memcpy(&f, &u, 4);
    out[i] = (isfinite(f) && !signbit(f)) ? oracle_e4m3_encode(f) : 0xFF;
  }
}
/* all fp32 bit patterns in [start, start + count): the stochastic-rounding
 * step of each value, i.e. the smallest u16 whose code equals the code at
 * u16 = 65535 (0 when every u16 gives the same code), found by bisection on
 * oracle_e2m1_encode_sr (the round-up set is a prefix of the u16 range);
 * 0xFFFFFFFF for NaN or Inf patterns */
void oracle_e2m1_sr_step_bits(uint32_t start, uint32_t count, uint32_t *out) {
  for (uint32_t i = 0; i < count; i++) {
    uint32_t u = start + i;
    float f;
    memcpy(&f, &u, 4);
    if (!isfinite(f)) {
      out[i] = 0xFFFFFFFFu;
      continue;
    }
    const uint8_t last = oracle_e2m1_encode_sr(f, 0xFFFF);
    uint32_t lo = 0, hi = 0xFFFF; /* the answer lies in [lo, hi] */
    while (lo < hi) {
      uint32_t mid = (lo + hi) / 2;
      if (oracle_e2m1_encode_sr(f, (uint16_t)mid) == last)
        hi = mid;
      else
        lo = mid + 1;
    }
    out[i] = lo;
  }
}
void oracle_philox_array(const uint32_t *keys, const uint32_t *ctrs, int64_t n, uint32_t *out) {
  for (int64_t i = 0; i < n; i++) oracle_philox4x32_10(keys + 2 * i, ctrs + 4 * i, out + 4 * i);
}
void oracle_f64_to_bf16_array(const double *x, int64_t n, uint16_t *out) {
  for (int64_t i = 0; i < n; i++) out[i] = oracle_f64_to_bf16(x[i]);
}
void oracle_sr_uniform_array(uint64_t seed, const uint64_t *blocks, const int32_t *js, int64_t n, uint16_t *out) {
  for (int64_t i = 0; i < n; i++) out[i] = oracle_sr_uniform(seed, blocks[i], js[i]);
}
