"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The C oracle, compiled with gcc and both sanitizers (aborting on the first
  report), driven by a small C program through every entry point: the
  codecs over dense value ranges, Philox, the RHT, quantisation in every
  layout, rounding and RHT combination on ragged shapes (and a slice with a
  block offset), dequantisation, the binary64 GEMM, the MXFP4 functions, the
  bf16 rounding and the bulk helpers.
* The C ABI's host-side validation (api.cpp), compiled with both sanitizers on
  its host code, linked with stand-ins for the kernel launchers, and called
  with the invalid arguments that must be rejected before anything is
  enqueued, plus the host-only helpers (sign mask, status strings, workspace
  size).  No GPU is touched.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_C = os.path.join(ROOT, "oracle", "nvfp4_oracle.c")
CSRC = os.path.join(ROOT, "nvfp4_bit_quantization_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")

ORACLE_DRIVER = r"""
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include <math.h>
double oracle_e2m1_value(uint8_t); uint8_t oracle_e2m1_encode_rtn(float); uint8_t oracle_e2m1_encode_sr(float, uint16_t);
float oracle_e4m3_value(uint8_t); uint8_t oracle_e4m3_encode(float);
void oracle_philox4x32_10(const uint32_t*, const uint32_t*, uint32_t*);
uint16_t oracle_sr_uniform(uint64_t, uint64_t, int); uint16_t oracle_rht_sign_mask(uint64_t);
void oracle_rht16_f64(const double*, uint16_t, double*);
int oracle_quantize_at(const uint16_t*, int64_t, int64_t, int64_t, int, int, int, uint64_t, uint64_t, uint64_t,
                       uint8_t*, uint8_t*, float*, float*);
int oracle_dequantize(const uint8_t*, const uint8_t*, int64_t, int64_t, int, float, float*);
int oracle_decode_products(const uint8_t*, const uint8_t*, int64_t, int64_t, int, double*);
int oracle_gemm_f64(const uint8_t*, const uint8_t*, int, float, const uint8_t*, const uint8_t*, int, float,
                    int64_t, int64_t, int64_t, double*);
uint8_t oracle_e8m0_scale_code(double); double oracle_e8m0_value(uint8_t);
int oracle_mx_quantize(const uint16_t*, int64_t, int64_t, int64_t, int, uint8_t*, uint8_t*);
int oracle_mx_decode(const uint8_t*, const uint8_t*, int64_t, int64_t, double*);
int oracle_mx_gemm_f64(const uint8_t*, const uint8_t*, const uint8_t*, const uint8_t*, int64_t, int64_t, int64_t, double*);
uint16_t oracle_f64_to_bf16(double);
void oracle_e2m1_encode_rtn_bits(uint32_t, uint32_t, uint8_t*); void oracle_e4m3_encode_bits(uint32_t, uint32_t, uint8_t*);
void oracle_sr_uniform_array(uint64_t, const uint64_t*, const int32_t*, int64_t, uint16_t*);

static uint32_t rs = 12345u;
static uint32_t rnd(void) { rs ^= rs << 13; rs ^= rs >> 17; rs ^= rs << 5; return rs; }
static uint16_t bf16_of(float f) { uint32_t u; memcpy(&u, &f, 4); return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16); }
#define CHECK(c) do { if (!(c)) { printf("check failed line %d\n", __LINE__); return 1; } } while (0)

int main(void) {
  unsigned acc = 0;
  for (int c = 0; c < 256; ++c) { acc += (unsigned)oracle_e2m1_value((uint8_t)c); acc += (unsigned)(oracle_e4m3_value((uint8_t)c) == oracle_e4m3_value((uint8_t)c)); }
  for (uint32_t u = 0; u < (1u << 20); ++u) {
    uint32_t b = rnd(); float f; memcpy(&f, &b, 4);
    if (!isfinite(f)) continue;
    acc += oracle_e2m1_encode_rtn(f) + oracle_e2m1_encode_sr(f, (uint16_t)rnd());
    acc += oracle_e4m3_encode(fabsf(f));
  }
  uint8_t *buf = malloc(1 << 20);
  oracle_e2m1_encode_rtn_bits(0x3E000000u, 1u << 20, buf);
  oracle_e4m3_encode_bits(0x3C000000u, 1u << 20, buf);
  uint32_t key[2] = {1, 2}, ctr[4] = {3, 4, 5, 6}, out[4];
  oracle_philox4x32_10(key, ctr, out);
  acc += out[0] + oracle_sr_uniform(77, 5, 15) + oracle_rht_sign_mask(1234);
  double v[16], z[16];
  for (int j = 0; j < 16; ++j) v[j] = (double)(int)(rnd() % 200) - 100.0;
  oracle_rht16_f64(v, 0xA5A5, z);
  /* quantisation: ragged shapes, a padded leading dimension, all combinations */
  const int64_t shapes[4][2] = {{16, 16}, {48, 80}, {96, 32}, {32, 272}};
  for (int s = 0; s < 4; ++s) {
    const int64_t R = shapes[s][0], C = shapes[s][1], ld = C + 8;
    uint16_t *x = malloc(sizeof(uint16_t) * R * ld);
    for (int64_t i = 0; i < R * ld; ++i) x[i] = bf16_of(((float)(int)(rnd() % 2001) - 1000.0f) * 1e-3f);
    x[3] = bf16_of(50.0f);
    uint8_t *codes = malloc(R * C / 2), *scales = malloc(R * C / 16);
    float S, amax;
    for (int layout = 0; layout < 4; ++layout)
      for (int rounding = 0; rounding < 2; ++rounding)
        for (int rht = 0; rht < 2; ++rht) {
          int rc = oracle_quantize_at(x, R, C, ld, layout, rounding, rht, 9, 10, 7, codes, scales, &S, &amax);
          CHECK(rc == 0 || (rht && layout >= 2));
          if (rc) continue;
          const int64_t orow = (layout == 1 || layout == 3) ? C : R, ocol = (layout == 1 || layout == 3) ? R : C;
          const int kind = layout >= 2;
          float *y = malloc(sizeof(float) * orow * ocol);
          double *d = malloc(sizeof(double) * orow * ocol);
          CHECK(oracle_dequantize(codes, scales, orow, ocol, kind, S, y) == 0);
          CHECK(oracle_decode_products(codes, scales, orow, ocol, kind, d) == 0);
          double *c = malloc(sizeof(double) * orow * orow);
          CHECK(oracle_gemm_f64(codes, scales, kind, S, codes, scales, kind, S, orow, orow, ocol, c) == 0);
          acc += (unsigned)(y[0] != 0) + (unsigned)(c[0] != 0);
          free(y); free(d); free(c);
        }
    CHECK(oracle_quantize_at(x, R, C, ld, 9, 0, 0, 0, 0, 0, codes, scales, &S, &amax) != 0);
    CHECK(oracle_quantize_at(x, R + 1, C, ld, 0, 0, 0, 0, 0, 0, codes, scales, &S, &amax) != 0);
    free(codes); free(scales);
    if (C % 32 == 0) {
      uint8_t *mc = malloc(R * C / 2), *ms = malloc(R * C / 32);
      CHECK(oracle_mx_quantize(x, R, C, ld, 0, mc, ms) == 0);
      double *md = malloc(sizeof(double) * R * C), *mg = malloc(sizeof(double) * R * R);
      CHECK(oracle_mx_decode(mc, ms, R, C, md) == 0);
      CHECK(oracle_mx_gemm_f64(mc, ms, mc, ms, R, R, C, mg) == 0);
      free(mc); free(ms); free(md); free(mg);
    }
    free(x);
  }
  acc += oracle_e8m0_scale_code(0.0) + oracle_e8m0_scale_code(1e300) + (unsigned)oracle_e8m0_value(130);
  const double bvals[] = {0.0, -0.0, 1e-45, 3e38, 3.5e38, -1e300, 1.0 + 1.0 / 256.0, NAN};
  for (int i = 0; i < 8; ++i) acc += oracle_f64_to_bf16(bvals[i]);
  uint64_t blocks[64]; int32_t js[64]; uint16_t us[64];
  for (int i = 0; i < 64; ++i) { blocks[i] = (uint64_t)rnd() << 20; js[i] = i & 15; }
  oracle_sr_uniform_array(5, blocks, js, 64, us);
  free(buf);
  printf("ok %u\n", acc);
  return 0;
}
"""

ABI_DRIVER = r"""
#include <stdio.h>
#include <stdint.h>
#include <string.h>
#include "nvfp4.h"
#include "nvfp4_kernels.hpp"
// stand-ins for the kernel launchers: the validation paths must return
// before any of them is reached
namespace nvfp4 {
static int launched = 0;
hipError_t launch_amax(const AmaxArgs &, bool, bool, bool, int, hipStream_t) { ++launched; return hipErrorInvalidValue; }
hipError_t launch_quantize(const QuantArgs &, int, bool, bool, int, bool, bool, hipStream_t, bool *s) { ++launched; *s = true; return hipErrorInvalidValue; }
hipError_t launch_quantize_batch2(const AmaxArgs &, const QuantArgs &, bool, const AmaxArgs &, const QuantArgs &, bool, hipStream_t) { ++launched; return hipErrorInvalidValue; }
int quant_tiles(int64_t R, int64_t C) { return (int)(((R + 127) / 128) * ((C + 255) / 256)); }
hipError_t launch_dequantize(const DequantArgs &, hipStream_t) { ++launched; return hipErrorInvalidValue; }
size_t gemm_workspace_bytes(int cus) { return kGemmWsSlots + (size_t)cus * kGemmSlotBytes; }
hipError_t launch_gemm(const GemmArgs &, void *, size_t, hipStream_t) { ++launched; return hipErrorInvalidValue; }
hipError_t launch_codec_selftest(int, const float *, const uint16_t *, uint8_t *, int64_t, hipStream_t) { ++launched; return hipErrorInvalidValue; }
hipError_t launch_mx_quantize(const MxQuantArgs &, int, hipStream_t) { ++launched; return hipErrorInvalidValue; }
hipError_t launch_mx_dequantize(const MxDequantArgs &, hipStream_t) { ++launched; return hipErrorInvalidValue; }
hipError_t launch_mx_gemm(const MxGemmArgs &, hipStream_t) { ++launched; return hipErrorInvalidValue; }
}
#define FAKE ((void *)0x10000)
#define CHECK(c) do { if (!(c)) { printf("check failed line %d\n", __LINE__); return 1; } } while (0)
static nvfp4_tensor T(int64_t r, int64_t c, int kind, void *codes = FAKE) {
  nvfp4_tensor t; memset(&t, 0, sizeof t);
  t.codes = (uint8_t *)codes; t.scales = (uint8_t *)FAKE; t.global_scale = (float *)FAKE; t.amax = (float *)FAKE;
  t.rows = r; t.cols = c; t.scale_kind = kind; return t;
}
static nvfp4_quant_output O(int layout, int64_t r, int64_t c, int kind, int rounding = 0, int rht = 0, int flags = 0) {
  nvfp4_quant_output o; memset(&o, 0, sizeof o);
  o.layout = layout; o.rounding = rounding; o.rht = rht; o.flags = flags; o.sr_seed = 1; o.rht_seed = 2;
  o.out = T(r, c, kind); return o;
}
int main() {
  nvfp4_quant_output row = O(NVFP4_ROW_1D, 64, 32, NVFP4_SCALE_1D16), col = O(NVFP4_COL_1D, 32, 64, NVFP4_SCALE_1D16);
  nvfp4_quant_output pair[3] = {row, col, row};
  const size_t wsb = nvfp4_workspace_bytes();
  CHECK(nvfp4_quantize(nullptr, 64, 32, 32, &row, 1, FAKE, wsb, nullptr) == NVFP4_E_NULL);
  CHECK(nvfp4_quantize(FAKE, 24, 32, 32, &row, 1, FAKE, wsb, nullptr) == NVFP4_E_SHAPE);
  CHECK(nvfp4_quantize(FAKE, 64, 32, 16, &row, 1, FAKE, wsb, nullptr) == NVFP4_E_LD);
  CHECK(nvfp4_quantize((char *)FAKE + 8, 64, 32, 32, &row, 1, FAKE, wsb, nullptr) == NVFP4_E_ALIGN);
  CHECK(nvfp4_quantize(FAKE, 64, 32, 32, pair, 3, FAKE, wsb, nullptr) == NVFP4_E_UNSUPPORTED);
  CHECK(nvfp4_quantize(FAKE, 64, 32, 32, &row, 1, nullptr, wsb, nullptr) == NVFP4_E_WORKSPACE);
  CHECK(nvfp4_quantize(FAKE, 64, 32, 32, &row, 1, FAKE, 16, nullptr) == NVFP4_E_WORKSPACE);
  nvfp4_quant_output bad = O(NVFP4_2D, 64, 32, NVFP4_SCALE_2D16, 0, 1);
  CHECK(nvfp4_quantize(FAKE, 64, 32, 32, &bad, 1, FAKE, wsb, nullptr) == NVFP4_E_UNSUPPORTED);
  bad = O(NVFP4_ROW_1D, 32, 64, NVFP4_SCALE_1D16);
  CHECK(nvfp4_quantize(FAKE, 64, 32, 32, &bad, 1, FAKE, wsb, nullptr) == NVFP4_E_SHAPE);
  nvfp4_quant_output rr[2] = {row, row};
  CHECK(nvfp4_quantize(FAKE, 64, 32, 32, rr, 2, FAKE, wsb, nullptr) == NVFP4_E_UNSUPPORTED);
  CHECK(nvfp4_quantize(FAKE, (int64_t)1 << 20, (int64_t)1 << 15, (int64_t)1 << 15, &row, 1, FAKE, wsb, nullptr) == NVFP4_E_SHAPE);
  nvfp4_quant_output colr = O(NVFP4_COL_1D, 32, 64, NVFP4_SCALE_1D16, 0, 1);
  nvfp4_quant_job jobs[2];
  memset(jobs, 0, sizeof jobs);
  jobs[0].x = FAKE; jobs[0].rows = 64; jobs[0].cols = 32; jobs[0].ld_x = 32; jobs[0].outs = &colr; jobs[0].n_outs = 1;
  jobs[1] = jobs[0];
  CHECK(nvfp4_quantize_batch(nullptr, 1, FAKE, wsb, nullptr) == NVFP4_E_NULL);
  CHECK(nvfp4_quantize_batch(jobs, 0, FAKE, wsb, nullptr) == NVFP4_E_UNSUPPORTED);
  CHECK(nvfp4_quantize_batch(jobs, 2, FAKE, 2 * wsb - 1, nullptr) == NVFP4_E_WORKSPACE);
  CHECK(nvfp4_quantize_batch(jobs, 2, (char *)FAKE + 8, 2 * wsb, nullptr) == NVFP4_E_ALIGN);
  jobs[1].rows = 24;
  CHECK(nvfp4_quantize_batch(jobs, 2, FAKE, 2 * wsb, nullptr) == NVFP4_E_SHAPE);
  jobs[1].rows = 64; jobs[1].n_outs = 3;
  CHECK(nvfp4_quantize_batch(jobs, 2, FAKE, 2 * wsb, nullptr) == NVFP4_E_UNSUPPORTED);
  jobs[1].n_outs = 1; jobs[1].outs = nullptr;
  CHECK(nvfp4_quantize_batch(jobs, 2, FAKE, 2 * wsb, nullptr) == NVFP4_E_NULL);
  CHECK(nvfp4_quantize_noalloc(nullptr, 64, 32, 32, &row, 1, nullptr) == NVFP4_E_NULL);
  CHECK(nvfp4_quantize_noalloc(FAKE, 64, 32, 16, &row, 1, nullptr) == NVFP4_E_LD);
  CHECK(nvfp4_quantize_noalloc(FAKE, 64, 32, 32, rr, 2, nullptr) == NVFP4_E_UNSUPPORTED);
  nvfp4_tensor a = T(64, 32, 0), b = T(48, 32, 0), b2 = T(48, 48, 0);
  CHECK(nvfp4_dequantize(nullptr, (float *)FAKE, 32, nullptr) == NVFP4_E_NULL);
  CHECK(nvfp4_dequantize(&a, (float *)FAKE, 16, nullptr) == NVFP4_E_LD);
  CHECK(nvfp4_gemm(&a, &b2, FAKE, NVFP4_F32, 48, nullptr, 0, nullptr) == NVFP4_E_UNSUPPORTED);
  CHECK(nvfp4_gemm(&a, &b, FAKE, 7, 48, nullptr, 0, nullptr) == NVFP4_E_UNSUPPORTED);
  CHECK(nvfp4_gemm(&a, &b, FAKE, NVFP4_F32, 32, nullptr, 0, nullptr) == NVFP4_E_LD);
  CHECK(nvfp4_gemm(&a, &b, (char *)FAKE + 4, NVFP4_F32, 48, nullptr, 0, nullptr) == NVFP4_E_ALIGN);
  CHECK(nvfp4_gemm_amax(&a, &b, FAKE, 48, nullptr, 0, nullptr, nullptr, 0, nullptr) == NVFP4_E_NULL);
  CHECK(nvfp4_gemm_amax(&a, &b, FAKE, 48, nullptr, 0, (float *)((char *)FAKE + 2), nullptr, 0, nullptr) == NVFP4_E_ALIGN);
  mxfp4_tensor m; memset(&m, 0, sizeof m); m.codes = (uint8_t *)FAKE; m.scales = (uint8_t *)FAKE; m.rows = 64; m.cols = 48;
  CHECK(mxfp4_quantize(FAKE, 64, 48, 48, NVFP4_ROW_1D, &m, nullptr) == NVFP4_E_SHAPE);
  CHECK(mxfp4_gemm(&m, &m, FAKE, NVFP4_F32, 64, nullptr) == NVFP4_E_SHAPE);
  CHECK(nvfp4_codec_selftest(5, nullptr, nullptr, nullptr, 0, nullptr) == NVFP4_E_UNSUPPORTED);
  CHECK(nvfp4_codec_selftest(0, nullptr, nullptr, nullptr, -1, nullptr) == NVFP4_E_SHAPE);
  unsigned acc = 0;
  for (uint64_t s = 0; s < 1000; ++s) acc += nvfp4_rht_sign_mask(s);
  for (int st = -8; st <= 1; ++st) acc += (unsigned)strlen(nvfp4_status_string(st));
  CHECK(nvfp4::launched == 0);
  printf("ok %u\n", acc);
  return 0;
}
"""


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, "%s\n%s\n%s" % (" ".join(cmd), r.stdout[-3000:], r.stderr[-6000:])
    return r


def test_oracle_under_asan_and_ubsan(tmp_path):
    if not shutil.which("gcc"):
        pytest.skip("gcc not available")
    drv = tmp_path / "drv.c"
    drv.write_text(ORACLE_DRIVER)
    exe = tmp_path / "oracle_san"
    _run(["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off", "-fopenmp",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-o", str(exe), ORACLE_C, str(drv), "-lm"])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1",
               OMP_NUM_THREADS="4")
    r = _run([str(exe)], env=env, timeout=600)
    assert r.stdout.startswith("ok"), r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-3000:]


def test_abi_validation_under_asan_and_ubsan(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    drv = tmp_path / "drv.cpp"
    drv.write_text(ABI_DRIVER)
    exe = tmp_path / "abi_san"
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all"]
    _run([hipcc, "-x", "hip", "--offload-arch=gfx950", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer"] + san +
         ["-I", INCLUDE, "-I", CSRC, "-o", str(exe), os.path.join(CSRC, "api.cpp"), str(drv)])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = _run([str(exe)], env=env, timeout=300)
    assert r.stdout.startswith("ok"), r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-3000:]
