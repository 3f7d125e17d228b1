// C ABI of libnvfp4.so: argument validation on the host, then kernel launches
// on the caller's stream.  The entry points and their contracts are declared
// and documented in include/nvfp4.h.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include <atomic>
#include <mutex>

#include "nvfp4.h"
#include "nvfp4_kernels.hpp"

using namespace nvfp4;

// Partial maxima of nvfp4_quantize_noalloc: the library's own copy of the
// quantise workspace, one per GPU (each device holds its own instance until
// the process ends).  In host code this name is not a device address; the
// kernels get the address hipGetSymbolAddress returns for the device.
static __device__ __align__(256) float scratch[3 * kMaxParts];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
std::atomic<void *> g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on device dev (looked up once per device, with
// that device current; the caller's current device is restored).
int scratch_address(int dev, void **out) {
  if (dev < 0 || dev >= kMaxDevices) return NVFP4_E_UNSUPPORTED;
  void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) {
    *out = p;
    return NVFP4_OK;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
  if (!p) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return NVFP4_E_HIP;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return NVFP4_E_HIP;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) (void)hipSetDevice(cur);
    if (e != hipSuccess || !p) {
      (void)hipGetLastError();
      return NVFP4_E_HIP;
    }
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return NVFP4_OK;
}

// Philox4x32-10 on the host, for the RHT sign mask (same published algorithm
// as the device copy: Salmon et al., SC'11).
uint32_t host_philox_word0(uint64_t seed, const uint32_t ctr_in[4]) {
  uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
  uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
    c1 = (uint32_t)p1;
    c3 = (uint32_t)p0;
    c0 = n0;
    c2 = n2;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return c0;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

bool sync_check_enabled() {
  static int v = -1;
  if (v < 0) {
    const char *e = getenv("NVFP4_SYNC_CHECK");
    v = (e && e[0] == '1') ? 1 : 0;
  }
  return v == 1;
}

int finish(hipError_t e, hipStream_t s) {
  if (e != hipSuccess) return NVFP4_E_HIP;
  if (sync_check_enabled()) {
    if (hipStreamSynchronize(s) != hipSuccess) return NVFP4_E_HIP;
    if (hipGetLastError() != hipSuccess) return NVFP4_E_HIP;
  }
  return NVFP4_OK;
}

struct OutPlan {
  int geom;
  bool rht, sr;
  int amax_mode;
};

// validate one output descriptor against the input shape; fill its plan
int plan_output(const nvfp4_quant_output &o, int64_t R, int64_t C, OutPlan *p) {
  if (o.flags != 0 && o.flags != NVFP4_AMAX_GIVEN) return NVFP4_E_UNSUPPORTED;
  if (o.rounding != NVFP4_RTN && o.rounding != NVFP4_SR) return NVFP4_E_UNSUPPORTED;
  if (o.rht != 0 && o.rht != 1) return NVFP4_E_UNSUPPORTED;
  const nvfp4_tensor &t = o.out;
  if (!t.codes || !t.scales || !t.global_scale || !t.amax) return NVFP4_E_NULL;
  if (!aligned16(t.codes)) return NVFP4_E_ALIGN;
  int64_t rows, cols;
  int kind;
  switch (o.layout) {
    case NVFP4_ROW_1D: p->geom = G_ROW; rows = R; cols = C; kind = NVFP4_SCALE_1D16; break;
    case NVFP4_COL_1D: p->geom = G_COL; rows = C; cols = R; kind = NVFP4_SCALE_1D16; break;
    case NVFP4_2D: p->geom = G_TILE; rows = R; cols = C; kind = NVFP4_SCALE_2D16; break;
    case NVFP4_2D_T: p->geom = G_TILE_T; rows = C; cols = R; kind = NVFP4_SCALE_2D16; break;
    default: return NVFP4_E_UNSUPPORTED;
  }
  if (o.rht && (p->geom == G_TILE || p->geom == G_TILE_T)) return NVFP4_E_UNSUPPORTED;
  if (t.rows != rows || t.cols != cols || t.scale_kind != kind) return NVFP4_E_SHAPE;
  p->rht = o.rht != 0;
  p->sr = o.rounding == NVFP4_SR;
  p->amax_mode = !p->rht ? AM_PLAIN : (p->geom == G_COL ? AM_RHT_COL : AM_RHT_ROW);
  return NVFP4_OK;
}

// host-side validation shared by nvfp4_gemm and nvfp4_gemm_amax
int gemm_check(const nvfp4_tensor *a, const nvfp4_tensor *b, const void *c, int32_t c_dtype, int64_t ldc,
               const void *workspace) {
  if (!a || !b || !c) return NVFP4_E_NULL;
  if (!a->codes || !a->scales || !a->global_scale || !b->codes || !b->scales || !b->global_scale) return NVFP4_E_NULL;
  if (a->rows <= 0 || b->rows <= 0 || a->cols <= 0 || (a->rows % 16) || (b->rows % 16) || (a->cols % 16))
    return NVFP4_E_SHAPE;
  if (a->cols != b->cols) return NVFP4_E_UNSUPPORTED;
  if (c_dtype != NVFP4_F32 && c_dtype != NVFP4_BF16) return NVFP4_E_UNSUPPORTED;
  if ((a->scale_kind != NVFP4_SCALE_1D16 && a->scale_kind != NVFP4_SCALE_2D16) ||
      (b->scale_kind != NVFP4_SCALE_1D16 && b->scale_kind != NVFP4_SCALE_2D16))
    return NVFP4_E_UNSUPPORTED;
  if (ldc < b->rows) return NVFP4_E_LD;
  if (!aligned16(a->codes) || !aligned16(b->codes) || !aligned16(c)) return NVFP4_E_ALIGN;
  if (workspace && !aligned16(workspace)) return NVFP4_E_ALIGN;
  if (a->rows > ((int64_t)1 << 31) || b->rows > ((int64_t)1 << 31)) return NVFP4_E_SHAPE;
  // one workgroup per 256x256 tile of C: the grid size is a 32-bit count
  if (((a->rows + 255) / 256) * ((b->rows + 255) / 256) >= ((int64_t)1 << 31)) return NVFP4_E_SHAPE;
  return NVFP4_OK;
}

GemmArgs gemm_args(const nvfp4_tensor *a, const nvfp4_tensor *b, void *c, int32_t c_dtype, int64_t ldc) {
  GemmArgs g;
  g.a_codes = a->codes;
  g.a_scales = a->scales;
  g.a_S = a->global_scale;
  g.b_codes = b->codes;
  g.b_scales = b->scales;
  g.b_S = b->global_scale;
  g.c = c;
  g.M = a->rows;
  g.N = b->rows;
  g.K = a->cols;
  g.ldc = ldc;
  g.a_kind = a->scale_kind;
  g.b_kind = b->scale_kind;
  g.c_bf16 = c_dtype == NVFP4_BF16 ? 1 : 0;
  return g;
}

OutArgs out_args(const nvfp4_quant_output &o, int amax_mode) {
  OutArgs a;
  a.codes = o.out.codes;
  a.scales = o.out.scales;
  a.S_out = o.out.global_scale;
  a.amax_out = o.out.amax;
  a.amax_in = (o.flags & NVFP4_AMAX_GIVEN) ? o.out.amax : nullptr;
  a.sr_seed = o.sr_seed;
  a.amax_mode = amax_mode;
  a.pad = 0;
  return a;
}

}  // namespace

extern "C" {

size_t nvfp4_workspace_bytes(void) { return kWsBytes; }

uint16_t nvfp4_rht_sign_mask(uint64_t rht_seed) {
  const uint32_t ctr[4] = {0u, 0u, 1u, 0u};
  return (uint16_t)(host_philox_word0(rht_seed, ctr) & 0xFFFFu);
}

const char *nvfp4_status_string(int status) {
  switch (status) {
    case NVFP4_OK: return "ok";
    case NVFP4_E_NULL: return "a required pointer is NULL";
    case NVFP4_E_SHAPE: return "size <= 0, not a multiple of 16, or inconsistent with the layout";
    case NVFP4_E_LD: return "leading dimension smaller than the row length";
    case NVFP4_E_ALIGN: return "pointer not 16-byte aligned or leading dimension not a multiple of 8";
    case NVFP4_E_UNSUPPORTED: return "unsupported combination of arguments";
    case NVFP4_E_WORKSPACE: return "workspace missing or too small";
    case NVFP4_E_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

}  // extern "C"

namespace {

// One quantise call, planned: its kernel arguments and what it launches.
struct QuantCall {
  QuantArgs qa;
  AmaxArgs aa;
  OutPlan p0, p1;        // the outputs in kernel order (ROW before COL, TILE before TILE_T)
  bool plain, rc, rr;    // maxima the amax pass must produce
};

// nvfp4_quantize's argument checks, in this order: pointers and counts,
// shape, leading dimension, alignment, the workspace (only with check_ws),
// the outputs.  With `call`, also its kernel arguments (partial maxima in the
// workspace).
int plan_quantize(const void *x, int64_t rows, int64_t cols, int64_t ld_x, const nvfp4_quant_output *outs,
                  int n_outs, bool check_ws, void *workspace, size_t workspace_bytes, QuantCall *call) {
  if (!x || !outs) return NVFP4_E_NULL;
  if (n_outs != 1 && n_outs != 2) return NVFP4_E_UNSUPPORTED;
  if (rows <= 0 || cols <= 0 || (rows % 16) || (cols % 16)) return NVFP4_E_SHAPE;
  if (rows > (int64_t)1 << 31 || cols > (int64_t)1 << 31) return NVFP4_E_SHAPE;
  // 16-element blocks are numbered in 31 bits (the stochastic-rounding counters)
  if ((rows / 16) * cols >= ((int64_t)1 << 31)) return NVFP4_E_SHAPE;
  if (ld_x < cols) return NVFP4_E_LD;
  if (!aligned16(x) || (ld_x % 8)) return NVFP4_E_ALIGN;
  if (check_ws) {
    if (!workspace) return NVFP4_E_WORKSPACE;
    if (workspace_bytes < kWsBytes) return NVFP4_E_WORKSPACE;
    if (!aligned16(workspace)) return NVFP4_E_ALIGN;
  }

  OutPlan p[2];
  for (int i = 0; i < n_outs; ++i) {
    const int st = plan_output(outs[i], rows, cols, &p[i]);
    if (st != NVFP4_OK) return st;
  }
  int order[2] = {0, 1};
  if (n_outs == 2) {
    // canonical pair order: ROW before COL, TILE before TILE_T
    if ((p[0].geom == G_COL && p[1].geom == G_ROW) || (p[0].geom == G_TILE_T && p[1].geom == G_TILE)) {
      order[0] = 1;
      order[1] = 0;
    }
    const int g0 = p[order[0]].geom, g1 = p[order[1]].geom;
    if (!((g0 == G_ROW && g1 == G_COL) || (g0 == G_TILE && g1 == G_TILE_T))) return NVFP4_E_UNSUPPORTED;
  }
  if (!call) return NVFP4_OK;

  uint32_t mask_rows = 0, mask_cols = 0;
  for (int i = 0; i < n_outs; ++i) {
    if (!p[i].rht) continue;
    const uint32_t m = nvfp4_rht_sign_mask(outs[i].rht_seed);
    if (p[i].geom == G_COL)
      mask_rows = m;
    else
      mask_cols = m;
  }
  const int tiles = quant_tiles(rows, cols);
  float *partials = (float *)workspace;
  QuantArgs &qa = call->qa;
  qa.x = (const uint16_t *)x;
  qa.R = rows;
  qa.C = cols;
  qa.ld = ld_x;
  qa.partials = partials;
  qa.nparts = tiles < kMaxParts ? tiles : kMaxParts;
  qa.mask_rows = mask_rows;
  qa.mask_cols = mask_cols;
  call->p0 = p[order[0]];
  qa.o[0] = out_args(outs[order[0]], call->p0.amax_mode);
  call->p1 = OutPlan{G_NONE, false, false, AM_PLAIN};
  if (n_outs == 2) {
    call->p1 = p[order[1]];
    qa.o[1] = out_args(outs[order[1]], call->p1.amax_mode);
  } else {
    qa.o[1] = qa.o[0];
  }
  AmaxArgs &aa = call->aa;
  aa.x = (const uint16_t *)x;
  aa.R = rows;
  aa.C = cols;
  aa.ld = ld_x;
  aa.partials = partials;
  aa.mask_rows = mask_rows;
  aa.mask_cols = mask_cols;
  call->plain = call->rc = call->rr = false;
  for (int i = 0; i < n_outs; ++i) {
    if (outs[i].flags & NVFP4_AMAX_GIVEN) continue;
    call->plain |= p[i].amax_mode == AM_PLAIN;
    call->rc |= p[i].amax_mode == AM_RHT_COL;
    call->rr |= p[i].amax_mode == AM_RHT_ROW;
  }
  return NVFP4_OK;
}

// enqueue a planned call: the amax pass (when a maximum is needed), then the
// quantise pass
int launch_call(const QuantCall &c, hipStream_t s) {
  if (c.plain || c.rc || c.rr) {
    if (launch_amax(c.aa, c.plain, c.rc, c.rr, c.qa.nparts, s) != hipSuccess) return NVFP4_E_HIP;
  }
  bool supported = true;
  const hipError_t e = launch_quantize(c.qa, c.p0.geom, c.p0.rht, c.p0.sr, c.p1.geom, c.p1.rht, c.p1.sr, s, &supported);
  if (!supported) return NVFP4_E_UNSUPPORTED;
  return e == hipSuccess ? NVFP4_OK : NVFP4_E_HIP;
}

// nvfp4_quantize; with check_only, the argument checks that do not concern
// the workspace, and nothing else (nvfp4_quantize_noalloc runs them before it
// looks up its scratch)
int quantize_impl(bool check_only, const void *x, int64_t rows, int64_t cols, int64_t ld_x,
                  const nvfp4_quant_output *outs, int n_outs, void *workspace, size_t workspace_bytes, void *stream) {
  QuantCall c;
  const int st = plan_quantize(x, rows, cols, ld_x, outs, n_outs, !check_only, workspace, workspace_bytes,
                               check_only ? nullptr : &c);
  if (st != NVFP4_OK || check_only) return st;
  hipStream_t s = (hipStream_t)stream;
  const int lst = launch_call(c, s);
  if (lst != NVFP4_OK) return lst;
  return finish(hipSuccess, s);
}

// a job of the Wgrad operand kind: one RHT column output, its maximum from
// the amax pass
bool wgrad_operand(const nvfp4_quant_job &j) {
  return j.n_outs == 1 && j.outs[0].layout == NVFP4_COL_1D && j.outs[0].rht == 1 && j.outs[0].flags == 0;
}

}  // namespace

extern "C" {

int nvfp4_quantize(const void *x, int64_t rows, int64_t cols, int64_t ld_x, const nvfp4_quant_output *outs,
                   int n_outs, void *workspace, size_t workspace_bytes, void *stream) {
  return quantize_impl(false, x, rows, cols, ld_x, outs, n_outs, workspace, workspace_bytes, stream);
}

int nvfp4_quantize_batch(const nvfp4_quant_job *jobs, int n_jobs, void *workspace, size_t workspace_bytes,
                         void *stream) {
  if (!jobs) return NVFP4_E_NULL;
  if (n_jobs < 1) return NVFP4_E_UNSUPPORTED;
  if (!workspace || workspace_bytes / kWsBytes < (size_t)n_jobs) return NVFP4_E_WORKSPACE;
  if (!aligned16(workspace)) return NVFP4_E_ALIGN;
  for (int j = 0; j < n_jobs; ++j) {  // every job is checked before anything is enqueued
    const nvfp4_quant_job &b = jobs[j];
    const int st = plan_quantize(b.x, b.rows, b.cols, b.ld_x, b.outs, b.n_outs, false, nullptr, 0, nullptr);
    if (st != NVFP4_OK) return st;
  }
  hipStream_t s = (hipStream_t)stream;
  char *ws = (char *)workspace;  // job j's partial maxima in the j-th slice of kWsBytes
  QuantCall c[2];
  if (n_jobs == 2 && wgrad_operand(jobs[0]) && wgrad_operand(jobs[1])) {
    for (int j = 0; j < 2; ++j) {
      const nvfp4_quant_job &b = jobs[j];
      const int st = plan_quantize(b.x, b.rows, b.cols, b.ld_x, b.outs, b.n_outs, true, ws + j * kWsBytes, kWsBytes,
                                   &c[j]);
      if (st != NVFP4_OK) return st;
    }
    return finish(launch_quantize_batch2(c[0].aa, c[0].qa, c[0].p0.sr, c[1].aa, c[1].qa, c[1].p0.sr, s), s);
  }
  for (int j = 0; j < n_jobs; ++j) {
    const nvfp4_quant_job &b = jobs[j];
    int st = plan_quantize(b.x, b.rows, b.cols, b.ld_x, b.outs, b.n_outs, true, ws + j * kWsBytes, kWsBytes, &c[0]);
    if (st == NVFP4_OK) st = launch_call(c[0], s);
    if (st != NVFP4_OK) return st;
  }
  return finish(hipSuccess, s);
}

int nvfp4_quantize_noalloc(const void *x, int64_t rows, int64_t cols, int64_t ld_x, const nvfp4_quant_output *outs,
                           int n_outs, void *stream) {
  static_assert(sizeof(scratch) >= kWsBytes, "the static scratch holds a whole quantise workspace");
  // the arguments first, with nvfp4_quantize's checks; the scratch address is
  // looked up only for a call that will be launched
  const int chk = quantize_impl(true, x, rows, cols, ld_x, outs, n_outs, nullptr, 0, stream);
  if (chk != NVFP4_OK) return chk;
  hipStream_t s = (hipStream_t)stream;
  int dev = -1;
  if (s) {
    if (hipStreamGetDevice(s, &dev) != hipSuccess) {
      (void)hipGetLastError();
      return NVFP4_E_HIP;
    }
  } else if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return NVFP4_E_HIP;
  }
  void *ws = nullptr;
  const int st = scratch_address(dev, &ws);
  if (st != NVFP4_OK) return st;
  return quantize_impl(false, x, rows, cols, ld_x, outs, n_outs, ws, sizeof(scratch), stream);
}

int nvfp4_dequantize(const nvfp4_tensor *q, float *y, int64_t ld_y, void *stream) {
  if (!q || !y || !q->codes || !q->scales || !q->global_scale) return NVFP4_E_NULL;
  if (q->rows <= 0 || q->cols <= 0 || (q->rows % 16) || (q->cols % 16)) return NVFP4_E_SHAPE;
  if (q->scale_kind != NVFP4_SCALE_1D16 && q->scale_kind != NVFP4_SCALE_2D16) return NVFP4_E_UNSUPPORTED;
  if (ld_y < q->cols) return NVFP4_E_LD;
  if (!aligned16(y) || (ld_y % 4) || !aligned16(q->codes)) return NVFP4_E_ALIGN;
  DequantArgs a;
  a.codes = q->codes;
  a.scales = q->scales;
  a.S = q->global_scale;
  a.y = y;
  a.rows = q->rows;
  a.cols = q->cols;
  a.ld_y = ld_y;
  a.scale_kind = q->scale_kind;
  hipStream_t s = (hipStream_t)stream;
  return finish(launch_dequantize(a, s), s);
}

size_t nvfp4_gemm_workspace_bytes(void) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                                              hipSuccess || cus <= 0)
    return 0;
  return gemm_workspace_bytes(cus < kGemmMaxCUs ? cus : kGemmMaxCUs);
}

int nvfp4_gemm(const nvfp4_tensor *a, const nvfp4_tensor *b, void *c, int32_t c_dtype, int64_t ldc, void *workspace,
               size_t workspace_bytes, void *stream) {
  const int st = gemm_check(a, b, c, c_dtype, ldc, workspace);
  if (st != NVFP4_OK) return st;
  GemmArgs g = gemm_args(a, b, c, c_dtype, ldc);
  g.amax_plain = nullptr;
  g.amax_rht = nullptr;
  g.rht_mask = 0;
  hipStream_t s = (hipStream_t)stream;
  return finish(launch_gemm(g, workspace, workspace_bytes, s), s);
}

int nvfp4_gemm_amax(const nvfp4_tensor *a, const nvfp4_tensor *b, void *c, int64_t ldc, void *workspace,
                    size_t workspace_bytes, float *amax_plain, float *amax_rht_col, uint64_t rht_seed, void *stream) {
  if (!amax_plain && !amax_rht_col) return NVFP4_E_NULL;
  if (((uintptr_t)amax_plain & 3u) || ((uintptr_t)amax_rht_col & 3u)) return NVFP4_E_ALIGN;
  // the validation of nvfp4_gemm, without enqueueing anything
  const int st = gemm_check(a, b, c, NVFP4_BF16, ldc, workspace);
  if (st != NVFP4_OK) return st;
  GemmArgs g = gemm_args(a, b, c, NVFP4_BF16, ldc);
  g.amax_plain = reinterpret_cast<unsigned int *>(amax_plain);
  g.amax_rht = reinterpret_cast<unsigned int *>(amax_rht_col);
  g.rht_mask = nvfp4_rht_sign_mask(rht_seed);
  hipStream_t s = (hipStream_t)stream;
  return finish(launch_gemm(g, workspace, workspace_bytes, s), s);
}

// ---------------------------------------------------------------- MXFP4 ----
int mxfp4_quantize(const void *x, int64_t rows, int64_t cols, int64_t ld_x, int32_t layout, const mxfp4_tensor *out,
                   void *stream) {
  if (!x || !out || !out->codes || !out->scales) return NVFP4_E_NULL;
  if (layout != NVFP4_ROW_1D && layout != NVFP4_COL_1D) return NVFP4_E_UNSUPPORTED;
  const int64_t orow = layout == NVFP4_ROW_1D ? rows : cols, ocol = layout == NVFP4_ROW_1D ? cols : rows;
  if (rows <= 0 || cols <= 0 || (ocol % 32) || (orow % 16)) return NVFP4_E_SHAPE;
  if (out->rows != orow || out->cols != ocol) return NVFP4_E_SHAPE;
  if (ld_x < cols) return NVFP4_E_LD;
  if (!aligned16(x) || (ld_x % 8) || !aligned16(out->codes)) return NVFP4_E_ALIGN;
  if ((rows / 128 + 1) * (cols / 256 + 1) >= ((int64_t)1 << 31)) return NVFP4_E_SHAPE;
  MxQuantArgs a;
  a.x = static_cast<const uint16_t *>(x);
  a.R = rows;
  a.C = cols;
  a.ld = ld_x;
  a.codes = out->codes;
  a.scales = out->scales;
  hipStream_t s = (hipStream_t)stream;
  return finish(launch_mx_quantize(a, layout == NVFP4_ROW_1D ? G_ROW : G_COL, s), s);
}

int mxfp4_dequantize(const mxfp4_tensor *q, float *y, int64_t ld_y, void *stream) {
  if (!q || !y || !q->codes || !q->scales) return NVFP4_E_NULL;
  if (q->rows <= 0 || q->cols <= 0 || (q->cols % 32)) return NVFP4_E_SHAPE;
  if (ld_y < q->cols) return NVFP4_E_LD;
  if (!aligned16(y) || (ld_y % 4) || !aligned16(q->codes)) return NVFP4_E_ALIGN;
  MxDequantArgs a;
  a.codes = q->codes;
  a.scales = q->scales;
  a.y = y;
  a.rows = q->rows;
  a.cols = q->cols;
  a.ld_y = ld_y;
  hipStream_t s = (hipStream_t)stream;
  return finish(launch_mx_dequantize(a, s), s);
}

int mxfp4_gemm(const mxfp4_tensor *a, const mxfp4_tensor *b, void *c, int32_t c_dtype, int64_t ldc, void *stream) {
  if (!a || !b || !c || !a->codes || !a->scales || !b->codes || !b->scales) return NVFP4_E_NULL;
  if (a->rows <= 0 || b->rows <= 0 || a->cols <= 0 || (a->cols % 32)) return NVFP4_E_SHAPE;
  if (a->cols != b->cols) return NVFP4_E_UNSUPPORTED;
  if (c_dtype != NVFP4_F32 && c_dtype != NVFP4_BF16) return NVFP4_E_UNSUPPORTED;
  if (ldc < b->rows) return NVFP4_E_LD;
  if (!aligned16(a->codes) || !aligned16(b->codes) || !aligned16(c) || ((uintptr_t)a->scales & 3u) ||
      ((uintptr_t)b->scales & 3u))
    return NVFP4_E_ALIGN;
  if (a->rows > ((int64_t)1 << 31) || b->rows > ((int64_t)1 << 31)) return NVFP4_E_SHAPE;
  if (((a->rows + 127) / 128) * ((b->rows + 127) / 128) >= ((int64_t)1 << 31)) return NVFP4_E_SHAPE;
  MxGemmArgs g;
  g.a_codes = a->codes;
  g.a_scales = a->scales;
  g.b_codes = b->codes;
  g.b_scales = b->scales;
  g.c = c;
  g.M = a->rows;
  g.N = b->rows;
  g.K = a->cols;
  g.ldc = ldc;
  g.c_bf16 = c_dtype == NVFP4_BF16 ? 1 : 0;
  hipStream_t s = (hipStream_t)stream;
  return finish(launch_mx_gemm(g, s), s);
}

int nvfp4_codec_selftest(int which, const float *in_f32, const uint16_t *in_u16, uint8_t *out_u8, int64_t n,
                         void *stream) {
  if (which < 0 || which > 2) return NVFP4_E_UNSUPPORTED;
  if (n < 0) return NVFP4_E_SHAPE;
  if (n > 0 && (!in_f32 || !out_u8 || (which == 1 && !in_u16))) return NVFP4_E_NULL;
  hipStream_t s = (hipStream_t)stream;
  return finish(launch_codec_selftest(which, in_f32, in_u16, out_u8, n, s), s);
}

}  // extern "C"
