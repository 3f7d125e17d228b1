/*
 * nvfp4.h -- C ABI of libnvfp4.so: NVFP4 tensor quantisation and the
 * NVFP4-operand GEMM on AMD Instinct MI355X (gfx950).
 *
 * The method follows the NVFP4 pretraining news page (zubnet.ai,
 * "nvidia-nvfp4-paper-4-bit-pretrain-hits-fp8-parity-12b-10t-tokens"),
 * paragraph 2: E2M1 elements in blocks of 16, one E4M3 scale per block, an
 * FP32 per-tensor scale over the whole tensor; 1D blocks for activations and
 * gradients, 16x16 2D blocks for weights (so a weight and its transpose
 * quantise identically), stochastic rounding for gradients only, and a 16x16
 * random Hadamard transform (RHT) with random +/-1 signs on the inputs of the
 * weight-gradient GEMM.  Paragraph 1 gives the GEMM's role (the 4-bit matrix
 * products that replace FP8 ones).
 *
 * Arithmetic convention (all binary32, round-to-nearest-even, no FMA):
 *   amax  = max |v| over the tensor (v = the RHT output when rht is set)
 *   S     = 2688 / amax  (2688 = 448 * 6); S = 1 if amax == 0 or S is not finite
 *   per block b: sb = (amax_b / 6) * S; s_b = E4M3(sb), nearest-even, saturating
 *   at 448, subnormals kept; r_b = S / s_b (0 if s_b == 0)
 *   per element: y = v * r_b, then E2M1 nearest-even (saturating at 6) or
 *   stochastic rounding with a 16-bit Philox4x32-10 uniform
 *   dequantised value = (e(code) * s_b) / S.
 *
 * Storage:
 *   codes  : packed E2M1, [rows][cols/2] bytes, element 2i in the low nibble;
 *            code bit 3 = sign, codes 0..7 = 0, .5, 1, 1.5, 2, 3, 4, 6
 *   scales : E4M3 (OCP E4M3FN) bytes, 1D: [rows][cols/16]; 2D: [rows/16][cols/16]
 *   "rows x cols" is the stored orientation; cols is the blocked (K) dimension.
 *
 * Conventions common to every entry point:
 *   - every data pointer is a DEVICE pointer owned by the caller; the library
 *     allocates nothing, keeps no state and is reentrant;
 *   - work is enqueued on `stream` (a hipStream_t; NULL = the default stream)
 *     and nothing synchronises the host; outputs are valid once the stream
 *     reaches that point, and inputs must not change before then;
 *   - arguments are validated on the host before anything is enqueued; on an
 *     error nothing is written and a negative status is returned;
 *   - inputs must be finite (NaN/Inf give unspecified outputs); with the RHT,
 *     |x| < 2^124, so that the binary32 sums of 16 terms stay finite;
 *   - debugging: with the environment variable NVFP4_SYNC_CHECK=1 (read once
 *     per process) every call also waits for its stream and returns
 *     NVFP4_E_HIP if a kernel failed.
 */
#ifndef NVFP4_H
#define NVFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define NVFP4_OK 0
#define NVFP4_E_NULL (-1)        /* a required pointer is NULL */
#define NVFP4_E_SHAPE (-2)       /* a size <= 0, not a multiple of 16, or inconsistent */
#define NVFP4_E_LD (-3)          /* a leading dimension smaller than the row length */
#define NVFP4_E_ALIGN (-4)       /* x, codes or y not 16-byte aligned, or ld not a multiple of 8 */
#define NVFP4_E_UNSUPPORTED (-5) /* unknown enum, RHT with a 2D layout, bad n_outs, K mismatch */
#define NVFP4_E_WORKSPACE (-6)   /* workspace NULL or smaller than nvfp4_workspace_bytes() */
#define NVFP4_E_HIP (-7)         /* a HIP launch failed */

/* layouts of one quantised output of an input x[rows][cols] */
#define NVFP4_ROW_1D 0 /* 1D blocks of 16 along cols; stored [rows][cols] */
#define NVFP4_COL_1D 1 /* 1D blocks of 16 along rows; stored transposed [cols][rows] */
#define NVFP4_2D 2     /* 16x16 tiles; stored [rows][cols], scales [rows/16][cols/16] */
#define NVFP4_2D_T 3   /* the NVFP4_2D results stored transposed [cols][rows], scales [cols/16][rows/16] */

/* output flags (nvfp4_quant_output.flags) */
#define NVFP4_AMAX_GIVEN 1 /* out.amax already holds the output's maximum (e.g. from nvfp4_gemm_amax) */

/* rounding */
#define NVFP4_RTN 0 /* nearest, ties to even mantissa bit */
#define NVFP4_SR 1  /* stochastic, Philox4x32-10 keyed by sr_seed */

/* scale kinds of a quantised tensor */
#define NVFP4_SCALE_1D16 0
#define NVFP4_SCALE_2D16 1

/* GEMM output dtypes */
#define NVFP4_F32 0
#define NVFP4_BF16 1

/* A quantised tensor in its stored orientation (rows x cols, cols = K). */
typedef struct {
  uint8_t *codes;       /* [rows][cols/2] packed E2M1 */
  uint8_t *scales;      /* E4M3: 1D [rows][cols/16]; 2D [rows/16][cols/16] */
  float *global_scale;  /* 1 float: S = 2688 / amax */
  float *amax;          /* 1 float: amax of what was quantised (after the RHT if any) */
  int64_t rows;
  int64_t cols;
  int32_t scale_kind;   /* NVFP4_SCALE_1D16 or NVFP4_SCALE_2D16 */
  int32_t rht;          /* 1 if the codes hold RHT-domain values (informational) */
} nvfp4_tensor;

/* One requested output of nvfp4_quantize.  `out` must describe buffers of the
 * shape implied by `layout` (rows/cols in the stored orientation, scale_kind
 * matching the layout). */
typedef struct {
  int32_t layout;     /* NVFP4_ROW_1D, NVFP4_COL_1D, NVFP4_2D, NVFP4_2D_T */
  int32_t rounding;   /* NVFP4_RTN or NVFP4_SR */
  int32_t rht;        /* 1: 16x16 RHT along the blocked dim; 1D layouts only */
  int32_t flags;      /* 0 or NVFP4_AMAX_GIVEN */
  uint64_t sr_seed;   /* Philox key of the stochastic rounding */
  uint64_t rht_seed;  /* Philox key of the RHT sign vector */
  nvfp4_tensor out;
} nvfp4_quant_output;

/*
 * nvfp4_quantize -- quantise x (bf16, [rows][cols], row stride ld_x elements)
 * into one or two outputs from a single pass over x.
 *
 * Defines: page paragraph 2 (format, 1D/2D block scaling, stochastic rounding
 * on gradients, RHT on Wgrad inputs).
 *   x          device, bf16, 16-byte aligned, ld_x >= cols, ld_x % 8 == 0
 *   rows, cols multiples of 16, rows/16 * cols < 2^31
 *   outs       host array of n_outs (1 or 2) output descriptors.  With two
 *              outputs the pair must be {ROW_1D, COL_1D} (either order, any
 *              rounding/RHT each) or {2D, 2D_T}; two outputs sharing RHT
 *              settings share the amax.
 *   workspace  device scratch of at least nvfp4_workspace_bytes() bytes,
 *              16-byte aligned (per-workgroup partial maxima of the amax pass;
 *              no initialisation needed).  Calls that may run concurrently
 *              (different streams) need separate workspaces.
 * Enqueues two kernels (amax pass, quantise pass) on `stream`.  With
 * flags = NVFP4_AMAX_GIVEN, *out.amax must already hold max |v| of what that
 * output quantises (the RHT-domain maximum for an RHT output, as
 * nvfp4_gemm_amax produces it); the amax pass skips that output's maximum and
 * is not launched at all when no output needs it (one kernel).
 * Writes codes, scales, *global_scale and *amax of every output.
 * RHT signs: d_j = -1 iff bit (j mod 16) of nvfp4_rht_sign_mask(rht_seed),
 * j the index along the blocked dimension.
 * Returns NVFP4_OK or a negative status (nothing enqueued).
 */
int nvfp4_quantize(const void *x, int64_t rows, int64_t cols, int64_t ld_x, const nvfp4_quant_output *outs,
                   int n_outs, void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of device workspace nvfp4_quantize needs (a small constant: partial
 * maxima of up to 1024 workgroups per amax mode). */
size_t nvfp4_workspace_bytes(void);

/* One job of nvfp4_quantize_batch: the arguments of one nvfp4_quantize call
 * without its workspace. */
typedef struct {
  const void *x;                   /* device bf16 [rows][cols], row stride ld_x */
  int64_t rows;
  int64_t cols;
  int64_t ld_x;
  const nvfp4_quant_output *outs;  /* host array of n_outs (1 or 2) descriptors */
  int32_t n_outs;
} nvfp4_quant_job;

/*
 * nvfp4_quantize_batch -- several independent quantisations, each with
 * exactly the outputs nvfp4_quantize gives for the same job (bit for bit),
 * enqueued together on `stream`.
 *
 * Defines: page paragraph 2 (the quantisation of each job as for
 * nvfp4_quantize; the weight-gradient GEMM's two inputs are quantised with
 * the 16x16 RHT along the token dimension).
 *   jobs       host array of n_jobs >= 1 job descriptors, each checked as
 *              nvfp4_quantize checks its arguments.  Jobs must not write the
 *              same output buffers.
 *   workspace  device scratch of at least n_jobs * nvfp4_workspace_bytes()
 *              bytes, 16-byte aligned (job j uses the j-th slice).
 * Two jobs that each have a single NVFP4_COL_1D output with the RHT and
 * flags 0 (the weight-gradient operand pair; either rounding for each) run as
 * one amax launch and one quantise launch whose workgroups alternate between
 * the two inputs (two kernel launches instead of four).  Any other batch
 * enqueues its jobs one after another, as nvfp4_quantize would.
 * Returns NVFP4_OK or a negative status: NVFP4_E_NULL for jobs == NULL,
 * NVFP4_E_UNSUPPORTED for n_jobs < 1, NVFP4_E_WORKSPACE or NVFP4_E_ALIGN for
 * the workspace, else the first failing job's status.  Every job is checked
 * before anything is enqueued.
 */
int nvfp4_quantize_batch(const nvfp4_quant_job *jobs, int n_jobs, void *workspace, size_t workspace_bytes,
                         void *stream);

/*
 * nvfp4_quantize_noalloc -- nvfp4_quantize without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation).  The partial maxima
 * live in a static device buffer of the library, 12 KiB
 * (nvfp4_workspace_bytes()) on each GPU it runs on, held until the process
 * ends; its device address is looked up on the first call for a device (the
 * stream's device, or the current one for a NULL stream).  The buffer's size
 * does not depend on the input (the amax pass writes at most 1024 partial
 * maxima per mode), so every input nvfp4_quantize accepts fits; the call
 * allocates nothing.
 *   x, rows, cols, ld_x, outs, n_outs, stream: as nvfp4_quantize.
 * Every call on one GPU shares that GPU's buffer, which keeps the last call's
 * partial maxima (each call writes the ones it reads before reading them):
 * calls that may overlap on one GPU (different streams, or host threads)
 * race and can produce wrong global scales -- order them on one stream.
 * Returns as nvfp4_quantize, or NVFP4_E_HIP if the buffer's device address
 * cannot be obtained.
 */
int nvfp4_quantize_noalloc(const void *x, int64_t rows, int64_t cols, int64_t ld_x, const nvfp4_quant_output *outs,
                           int n_outs, void *stream);

/*
 * nvfp4_dequantize -- y[r][c] = (e(code) * s_b) / S for the stored
 * orientation of q, as fp32 with row stride ld_y elements.
 * Defines: page paragraph 2 (block scale times element, over the per-tensor
 * scale).  q->codes, q->scales, q->global_scale and y are device pointers;
 * y 16-byte aligned, ld_y >= q->cols, ld_y % 4 == 0.
 */
int nvfp4_dequantize(const nvfp4_tensor *q, float *y, int64_t ld_y, void *stream);

/*
 * nvfp4_gemm -- C[m][n] = (sum_k A^[m][k] * B^[n][k]) / (S_A * S_B), where
 * A^ = e(code) * s_b is the exact operand value.
 * Defines: page paragraph 1 (the 4-bit GEMMs) with the scales of paragraph 2.
 *   a : M x K quantised tensor (a->rows = M, a->cols = K)
 *   b : N x K quantised tensor (b->rows = N, b->cols = K); a->cols == b->cols
 *   c : device, [M][N] with row stride ldc elements, fp32 or bf16 (RNE)
 *   workspace : NULL, or device memory of at least nvfp4_gemm_workspace_bytes()
 *              bytes, 16-byte aligned, ZERO-FILLED before its first use (every
 *              call leaves its flag words at zero again).  With a workspace,
 *              shapes with more than two rounds of 256x256 tiles whose last
 *              round would leave more than a tenth of the compute units idle
 *              run as stream-K: whole tiles for the full rounds, then the
 *              remaining tiles' K-tiles spread evenly over one
 *              persistent workgroup per compute unit (the kernel's LDS use
 *              admits one per CU, so on an otherwise idle GPU all are
 *              resident), the fp32 partial sums of a split tile added in the
 *              workspace.  Without one every workgroup computes whole
 *              tiles.  The environment variable NVFP4_GEMM_DATA_PARALLEL
 *              forces whole tiles, and so does a stream that is being
 *              captured into a graph.  Calls that may run concurrently need
 *              separate workspaces.  The stream-K wait is bounded: if it ever
 *              times out, the word at byte offset 4096 of the workspace becomes
 *              non-zero and stays so, that call's output is invalid, and the
 *              workspace must be zero-filled again before it is used again
 *              (a late partial's flag may still be raised).
 * Operands are expanded exactly to fp16 in registers and multiplied on MFMA
 * with fp32 accumulation; the per-tensor scales are applied in the epilogue.
 */
int nvfp4_gemm(const nvfp4_tensor *a, const nvfp4_tensor *b, void *c, int32_t c_dtype, int64_t ldc, void *workspace,
               size_t workspace_bytes, void *stream);

/*
 * nvfp4_gemm_amax -- nvfp4_gemm with bf16 output that also produces the
 * per-tensor maxima the quantisation of C needs (producer-fused amax: the
 * quantiser can then skip its read of C for the amax).
 * Defines: page paragraph 2 (the FP32 per-tensor scale, whose amax this is,
 * and the RHT on Wgrad inputs: C's column quantisation along its rows).
 *   a, b, c, ldc, workspace, workspace_bytes: as nvfp4_gemm, c bf16 (RNE)
 *   amax_plain    device float or NULL: becomes max(*amax_plain, max |c|)
 *                 over the stored bf16 values -- the amax of a ROW_1D, COL_1D,
 *                 2D or 2D_T quantisation of C without RHT;
 *   amax_rht_col  device float or NULL: becomes max(*amax_rht_col, max |z|)
 *                 with z the 16x16 RHT (signs from rht_seed) of every aligned
 *                 16-row group of C -- the amax of a COL_1D + RHT quantisation
 *                 of C (rows are its blocked dimension).  Summed on the bf16
 *                 MFMA, so it may differ from the quantiser's own binary32
 *                 butterflies in the last bits (RHT tolerance).
 * Both maxima are combined with device-scope atomic maxima, so the caller
 * initialises them (0 for a fresh tensor).  At least one must be non-NULL;
 * both 4-byte aligned.
 */
int nvfp4_gemm_amax(const nvfp4_tensor *a, const nvfp4_tensor *b, void *c, int64_t ldc, void *workspace,
                    size_t workspace_bytes, float *amax_plain, float *amax_rht_col, uint64_t rht_seed, void *stream);

/* Bytes of GEMM workspace for the current device (8 KiB of flags plus one
 * 256 KiB fp32 tile per compute unit; 0 if no device is visible). */
size_t nvfp4_gemm_workspace_bytes(void);

/* Host: the 16-bit RHT sign mask for a seed (bit j set => d_j = -1):
 * the low 16 bits of word 0 of Philox4x32-10(key = seed, counter = (0,0,1,0)).
 * Defines: page paragraph 2 (the random +/-1 signs of the 16-point randomised
 * Hadamard transform); the counter and the bits taken are this library's
 * convention.  One mask serves every 16-group of a tensor and both operands
 * of a weight-gradient GEMM, so that the transforms cancel in the product. */
uint16_t nvfp4_rht_sign_mask(uint64_t rht_seed);

/* Host: a static description of a status code. */
const char *nvfp4_status_string(int status);

/* ------------------------------------------------------------------------
 * MXFP4, the earlier 4-bit microscaling format the page sets NVFP4 against
 * (paragraph 3: its loss gap to BF16 and the extra tokens it needs).  The page
 * does not define it; these entry points follow the OCP Microscaling Formats
 * (MX) specification v1.0 (section 5: blocks of 32 elements sharing an E8M0
 * scale, FP4 E2M1 elements; section 6.3: conversion):
 *   per block of 32 along the blocked (K) dimension:
 *     e = floor(log2(max |v|)) - 2, clamped to [-127, 127]; X = 2^e, stored as
 *     the E8M0 byte e + 127 (an all-zero block: byte 0);
 *     element = v / X rounded to nearest, ties to even, onto the E2M1 grid,
 *     values above 6 clamped to 6, sign kept (-0 gives code 8).
 *   dequantised value = e(code) * X.  There is no per-tensor scale: one pass.
 * Storage: codes as for NVFP4 ([rows][cols/2], element 2i in the low nibble);
 * scales [rows][cols/32] E8M0 bytes.  The GEMM runs on the gfx950 block-scaled
 * FP4 matrix instruction, which applies the 32-element E8M0 scales itself.
 * ------------------------------------------------------------------------ */
typedef struct {
  uint8_t *codes;   /* [rows][cols/2] packed E2M1 */
  uint8_t *scales;  /* [rows][cols/32] E8M0 */
  int64_t rows;
  int64_t cols;     /* blocked (K) dimension, a multiple of 32 */
} mxfp4_tensor;

/*
 * mxfp4_quantize -- quantise x (bf16, [rows][cols], row stride ld_x) into out.
 * Defines: page paragraph 3 names the format; the OCP MX specification v1.0
 * defines it (see above).
 *   x       device, bf16, 16-byte aligned, ld_x >= cols, ld_x % 8 == 0
 *   layout  NVFP4_ROW_1D (blocks along cols; out is rows x cols) or
 *           NVFP4_COL_1D (blocks along rows; out is x^T, cols x rows)
 *   rows, cols  the blocked dimension a multiple of 32, the other of 16
 *   out     device buffers of the stored shape; codes 16-byte aligned
 * Enqueues one kernel; writes out->codes and out->scales.
 */
int mxfp4_quantize(const void *x, int64_t rows, int64_t cols, int64_t ld_x, int32_t layout, const mxfp4_tensor *out,
                   void *stream);

/*
 * mxfp4_dequantize -- y[r][c] = e(code) * X for the stored orientation of q,
 * fp32 with row stride ld_y (y 16-byte aligned, ld_y >= q->cols,
 * ld_y % 4 == 0; q->codes 16-byte aligned; q->cols a multiple of 32).
 */
int mxfp4_dequantize(const mxfp4_tensor *q, float *y, int64_t ld_y, void *stream);

/*
 * mxfp4_gemm -- C[m][n] = sum_k A^[m][k] * B^[n][k], A^ = e(code) * X.
 *   a : M x K, b : N x K (a->cols == b->cols = K, a multiple of 32)
 *   c : device, [M][N] with row stride ldc >= N, fp32 or bf16 (RNE)
 *   codes 16-byte aligned, scales 4-byte aligned, c 16-byte aligned
 * FP4 codes and E8M0 scales go to the MFMA unchanged; fp32 accumulation.
 * M, N multiples of 256 and K of 128 take the LDS-pipelined 256x256 kernel;
 * other shapes a direct kernel with zero-filled edges.
 */
int mxfp4_gemm(const mxfp4_tensor *a, const mxfp4_tensor *b, void *c, int32_t c_dtype, int64_t ldc, void *stream);

/*
 * Codec self-test hooks (for the exhaustive hardware checks in the tests):
 * run the device's element/scale encoders exactly as the quantise kernels use
 * them.  which = 0: E2M1 round-to-nearest of in_f32[i] -> out_u8[i];
 * which = 1: E2M1 stochastic rounding of in_f32[i] with uniform in_u16[i];
 * which = 2: E4M3 of the non-negative in_f32[i].  in_u16 is read for which = 1
 * only.  n >= 0; all pointers device.
 */
int nvfp4_codec_selftest(int which, const float *in_f32, const uint16_t *in_u16, uint8_t *out_u8, int64_t n,
                         void *stream);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_H */
