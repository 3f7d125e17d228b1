"""Python binding of libnvfp4.so: NVFP4 quantisation and the NVFP4 GEMM on
MI355X (gfx950).

The functions named like the C ABI (``nvfp4_quantize``, ``nvfp4_dequantize``,
``nvfp4_gemm``, ...) only marshal arguments: torch supplies device memory and
the current HIP stream, every step of the computation runs in the library's
HIP kernels.  Importing this package fails loudly when the library has not
been built (``python -m nvfp4_bit_quantization_amd.build``); there is no CPU
fallback.

Method: NVFP4 pretraining news page (zubnet.ai), paragraph 2 -- blocks of 16
E2M1 values with an E4M3 scale each, an FP32 scale per tensor, 1D blocks for
activations/gradients and 16x16 blocks for weights, stochastic rounding for
gradients, a 16-point randomised Hadamard transform on the weight-gradient
inputs.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import List, Optional, Sequence

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libnvfp4.so")

# enums (include/nvfp4.h)
NVFP4_OK = 0
ROW_1D, COL_1D, TWO_D, TWO_D_T = 0, 1, 2, 3
RTN, SR = 0, 1
AMAX_GIVEN = 1  # nvfp4_quant_output.flags
SCALE_1D16, SCALE_2D16 = 0, 1
F32, BF16 = 0, 1
LAYOUTS = {"row": ROW_1D, "col": COL_1D, "2d": TWO_D, "2d_t": TWO_D_T}
ROUNDINGS = {"rtn": RTN, "sr": SR}


class Nvfp4Error(RuntimeError):
    pass


class nvfp4_tensor(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("global_scale", ctypes.c_void_p),
                ("amax", ctypes.c_void_p), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("scale_kind", ctypes.c_int32), ("rht", ctypes.c_int32)]


class mxfp4_tensor(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("rows", ctypes.c_int64),
                ("cols", ctypes.c_int64)]


class nvfp4_quant_output(ctypes.Structure):
    _fields_ = [("layout", ctypes.c_int32), ("rounding", ctypes.c_int32), ("rht", ctypes.c_int32),
                ("flags", ctypes.c_int32), ("sr_seed", ctypes.c_uint64), ("rht_seed", ctypes.c_uint64),
                ("out", nvfp4_tensor)]


class nvfp4_quant_job(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64), ("ld_x", ctypes.c_int64),
                ("outs", ctypes.POINTER(nvfp4_quant_output)), ("n_outs", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libnvfp4.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError("libnvfp4.so is not built: run `python -m nvfp4_bit_quantization_amd.build` "
                          "(expected at %s)" % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    P, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    L.nvfp4_quantize.restype = i32
    L.nvfp4_quantize.argtypes = [P, i64, i64, i64, ctypes.POINTER(nvfp4_quant_output), i32, P, ctypes.c_size_t, P]
    L.nvfp4_quantize_batch.restype = i32
    L.nvfp4_quantize_batch.argtypes = [ctypes.POINTER(nvfp4_quant_job), i32, P, ctypes.c_size_t, P]
    L.nvfp4_quantize_noalloc.restype = i32
    L.nvfp4_quantize_noalloc.argtypes = [P, i64, i64, i64, ctypes.POINTER(nvfp4_quant_output), i32, P]
    L.nvfp4_workspace_bytes.restype = ctypes.c_size_t
    L.nvfp4_workspace_bytes.argtypes = []
    L.nvfp4_dequantize.restype = i32
    L.nvfp4_dequantize.argtypes = [ctypes.POINTER(nvfp4_tensor), P, i64, P]
    L.nvfp4_gemm.restype = i32
    L.nvfp4_gemm.argtypes = [ctypes.POINTER(nvfp4_tensor), ctypes.POINTER(nvfp4_tensor), P, ctypes.c_int32, i64, P,
                             ctypes.c_size_t, P]
    L.nvfp4_gemm_amax.restype = i32
    L.nvfp4_gemm_amax.argtypes = [ctypes.POINTER(nvfp4_tensor), ctypes.POINTER(nvfp4_tensor), P, i64, P,
                                  ctypes.c_size_t, P, P, ctypes.c_uint64, P]
    L.nvfp4_gemm_workspace_bytes.restype = ctypes.c_size_t
    L.nvfp4_gemm_workspace_bytes.argtypes = []
    L.nvfp4_rht_sign_mask.restype = ctypes.c_uint16
    L.nvfp4_rht_sign_mask.argtypes = [ctypes.c_uint64]
    L.nvfp4_status_string.restype = ctypes.c_char_p
    L.nvfp4_status_string.argtypes = [i32]
    L.nvfp4_codec_selftest.restype = i32
    L.nvfp4_codec_selftest.argtypes = [i32, P, P, P, i64, P]
    L.mxfp4_quantize.restype = i32
    L.mxfp4_quantize.argtypes = [P, i64, i64, i64, ctypes.c_int32, ctypes.POINTER(mxfp4_tensor), P]
    L.mxfp4_dequantize.restype = i32
    L.mxfp4_dequantize.argtypes = [ctypes.POINTER(mxfp4_tensor), P, i64, P]
    L.mxfp4_gemm.restype = i32
    L.mxfp4_gemm.argtypes = [ctypes.POINTER(mxfp4_tensor), ctypes.POINTER(mxfp4_tensor), P, ctypes.c_int32, i64, P]
    _lib = L
    return L


def _check(status: int, what: str):
    if status != NVFP4_OK:
        raise Nvfp4Error("%s failed: %d (%s)" % (what, status, lib().nvfp4_status_string(status).decode()))


def _stream(stream):
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _on_stream(stream):
    """Context under which the conveniences allocate: the stream the library
    will launch on.  torch's caching allocator then hands a freed block (the
    temporary quantise workspace) to later allocations on that same stream
    only, i.e. after the kernels that use it; memory taken on another stream
    could be reused while those kernels still run."""
    import contextlib
    import torch
    if stream is None:
        return contextlib.nullcontext()
    if isinstance(stream, int):
        stream = torch.cuda.ExternalStream(stream)
    return torch.cuda.stream(stream)


# ---------------------------------------------------------------------------
# quantised tensors held in torch device memory
# ---------------------------------------------------------------------------
@dataclass
class QTensor:
    codes: "object"         # torch.uint8 [rows][cols/2]
    scales: "object"        # torch.uint8, 1D [rows][cols/16] or 2D [rows/16][cols/16]
    global_scale: "object"  # torch.float32 [1]
    amax: "object"          # torch.float32 [1]
    rows: int
    cols: int
    scale_kind: int
    rht: int = 0

    def c_struct(self) -> nvfp4_tensor:
        return nvfp4_tensor(self.codes.data_ptr(), self.scales.data_ptr(), self.global_scale.data_ptr(),
                            self.amax.data_ptr(), self.rows, self.cols, self.scale_kind, self.rht)


def empty_qtensor(rows: int, cols: int, scale_kind: int, device="cuda", rht: int = 0) -> QTensor:
    import torch
    sshape = (rows, cols // 16) if scale_kind == SCALE_1D16 else (rows // 16, cols // 16)
    return QTensor(codes=torch.empty((rows, cols // 2), dtype=torch.uint8, device=device),
                   scales=torch.empty(sshape, dtype=torch.uint8, device=device),
                   global_scale=torch.empty(1, dtype=torch.float32, device=device),
                   amax=torch.empty(1, dtype=torch.float32, device=device),
                   rows=rows, cols=cols, scale_kind=scale_kind, rht=rht)


@dataclass
class QuantSpec:
    """One requested output of nvfp4_quantize."""
    layout: int = ROW_1D
    rounding: int = RTN
    rht: bool = False
    sr_seed: int = 0
    rht_seed: int = 0
    amax_given: bool = False  # the output's amax tensor already holds its maximum (nvfp4_gemm_amax)

    @staticmethod
    def of(layout="row", rounding="rtn", rht=False, sr_seed=0, rht_seed=0, amax_given=False) -> "QuantSpec":
        return QuantSpec(LAYOUTS.get(layout, layout), ROUNDINGS.get(rounding, rounding), bool(rht), sr_seed, rht_seed,
                         bool(amax_given))


def output_shape(rows: int, cols: int, layout: int):
    """(rows, cols, scale_kind) of the stored output for an input [rows][cols]."""
    if layout == ROW_1D:
        return rows, cols, SCALE_1D16
    if layout == COL_1D:
        return cols, rows, SCALE_1D16
    if layout == TWO_D:
        return rows, cols, SCALE_2D16
    if layout == TWO_D_T:
        return cols, rows, SCALE_2D16
    raise ValueError(layout)


def new_workspace(device="cuda", jobs=1):
    """A quantise workspace (one per stream), for `jobs` jobs of a batch."""
    import torch
    return torch.empty(jobs * lib().nvfp4_workspace_bytes() // 4, dtype=torch.float32, device=device)


# ---------------------------------------------------------------------------
# C ABI entry points (argument marshalling only)
# ---------------------------------------------------------------------------
def nvfp4_quantize(x, specs: Sequence[QuantSpec], outs: Sequence[QTensor], workspace, stream=None) -> List[QTensor]:
    """Quantise the bf16 device tensor x [rows][cols] (row stride x.stride(0))
    into 1 or 2 outputs (see include/nvfp4.h)."""
    assert len(specs) == len(outs) and 1 <= len(specs) <= 2
    import torch
    assert x.dtype == torch.bfloat16 and x.dim() == 2 and x.stride(1) == 1
    arr = (nvfp4_quant_output * len(specs))()
    for i, (s, o) in enumerate(zip(specs, outs)):
        arr[i] = nvfp4_quant_output(s.layout, s.rounding, int(s.rht), AMAX_GIVEN if s.amax_given else 0, s.sr_seed,
                                    s.rht_seed, o.c_struct())
    st = lib().nvfp4_quantize(ctypes.c_void_p(x.data_ptr()), x.shape[0], x.shape[1], x.stride(0), arr, len(specs),
                              ctypes.c_void_p(workspace.data_ptr()), workspace.numel() * workspace.element_size(),
                              _stream(stream))
    _check(st, "nvfp4_quantize")
    return list(outs)


def nvfp4_quantize_batch(jobs, workspace, stream=None):
    """Several independent nvfp4_quantize calls enqueued together (see
    include/nvfp4.h).  jobs: a sequence of (x, specs, outs); workspace: at
    least len(jobs) * nvfp4_workspace_bytes() bytes (new_workspace(len(jobs)))."""
    import torch
    arrs = []
    jarr = (nvfp4_quant_job * len(jobs))()
    for j, (x, specs, outs) in enumerate(jobs):
        assert len(specs) == len(outs) and 1 <= len(specs) <= 2
        assert x.dtype == torch.bfloat16 and x.dim() == 2 and x.stride(1) == 1
        arr = (nvfp4_quant_output * len(specs))()
        for i, (s, o) in enumerate(zip(specs, outs)):
            arr[i] = nvfp4_quant_output(s.layout, s.rounding, int(s.rht), AMAX_GIVEN if s.amax_given else 0,
                                        s.sr_seed, s.rht_seed, o.c_struct())
        arrs.append(arr)  # kept alive until the call returns
        jarr[j] = nvfp4_quant_job(x.data_ptr(), x.shape[0], x.shape[1], x.stride(0),
                                  ctypes.cast(arr, ctypes.POINTER(nvfp4_quant_output)), len(specs))
    st = lib().nvfp4_quantize_batch(jarr, len(jobs), ctypes.c_void_p(workspace.data_ptr()),
                                    workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "nvfp4_quantize_batch")
    return [list(outs) for _, _, outs in jobs]


def nvfp4_quantize_noalloc(x, specs: Sequence[QuantSpec], outs: Sequence[QTensor], stream=None) -> List[QTensor]:
    """nvfp4_quantize with the library's static scratch instead of a
    workspace (allocates nothing; calls overlapping on one GPU race)."""
    assert len(specs) == len(outs) and 1 <= len(specs) <= 2
    import torch
    assert x.dtype == torch.bfloat16 and x.dim() == 2 and x.stride(1) == 1
    arr = (nvfp4_quant_output * len(specs))()
    for i, (s, o) in enumerate(zip(specs, outs)):
        arr[i] = nvfp4_quant_output(s.layout, s.rounding, int(s.rht), AMAX_GIVEN if s.amax_given else 0, s.sr_seed,
                                    s.rht_seed, o.c_struct())
    st = lib().nvfp4_quantize_noalloc(ctypes.c_void_p(x.data_ptr()), x.shape[0], x.shape[1], x.stride(0), arr,
                                      len(specs), _stream(stream))
    _check(st, "nvfp4_quantize_noalloc")
    return list(outs)


def nvfp4_dequantize(q: QTensor, y, stream=None):
    """y[r][c] = (e(code) * s_b) / S for the stored orientation of q (fp32)."""
    import torch
    assert y.dtype == torch.float32 and y.stride(1) == 1
    t = q.c_struct()
    _check(lib().nvfp4_dequantize(ctypes.byref(t), ctypes.c_void_p(y.data_ptr()), y.stride(0), _stream(stream)),
           "nvfp4_dequantize")
    return y


def nvfp4_gemm(a: QTensor, b: QTensor, c, workspace=None, stream=None):
    """C[M][N] = A^ B^T / (S_A S_B) into the fp32 or bf16 device tensor c.
    `workspace` (from new_gemm_workspace) enables the stream-K path."""
    import torch
    dt = F32 if c.dtype == torch.float32 else BF16 if c.dtype == torch.bfloat16 else None
    if dt is None:
        raise TypeError("c must be float32 or bfloat16")
    assert c.stride(1) == 1
    ta, tb = a.c_struct(), b.c_struct()
    wp = ctypes.c_void_p(workspace.data_ptr()) if workspace is not None else ctypes.c_void_p(0)
    wb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().nvfp4_gemm(ctypes.byref(ta), ctypes.byref(tb), ctypes.c_void_p(c.data_ptr()), dt, c.stride(0),
                            wp, wb, _stream(stream)), "nvfp4_gemm")
    return c


def nvfp4_gemm_amax(a: QTensor, b: QTensor, c, amax_plain=None, amax_rht_col=None, rht_seed: int = 0,
                    workspace=None, stream=None):
    """nvfp4_gemm into the bf16 tensor c that also folds max |c| into the
    float32 device tensor amax_plain[0] and the RHT-domain maximum of c's
    16-row groups (signs from rht_seed) into amax_rht_col[0] (atomic maxima:
    initialise them, e.g. to 0)."""
    import torch
    if c.dtype != torch.bfloat16:
        raise TypeError("c must be bfloat16")
    assert c.stride(1) == 1
    ta, tb = a.c_struct(), b.c_struct()
    p = (lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0))
    wb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().nvfp4_gemm_amax(ctypes.byref(ta), ctypes.byref(tb), ctypes.c_void_p(c.data_ptr()), c.stride(0),
                                 p(workspace), wb, p(amax_plain), p(amax_rht_col), rht_seed, _stream(stream)),
           "nvfp4_gemm_amax")
    return c


def nvfp4_gemm_workspace_bytes() -> int:
    return lib().nvfp4_gemm_workspace_bytes()


def new_gemm_workspace(device="cuda"):
    """A zero-filled GEMM workspace (one per stream)."""
    import torch
    return torch.zeros(lib().nvfp4_gemm_workspace_bytes(), dtype=torch.uint8, device=device)


def gemm_workspace_timed_out(workspace) -> bool:
    """True if a stream-K call on this workspace hit its wait limit (the
    outputs of that call are invalid; reset_gemm_workspace before reuse)."""
    return bool(workspace[4096:4100].view(__import__("torch").int32).item() != 0)


def reset_gemm_workspace(workspace):
    """Zero-fill a GEMM workspace again (needed after a timed-out call)."""
    workspace.zero_()
    return workspace


def nvfp4_workspace_bytes() -> int:
    return lib().nvfp4_workspace_bytes()


def nvfp4_rht_sign_mask(seed: int) -> int:
    return lib().nvfp4_rht_sign_mask(seed)


def nvfp4_status_string(status: int) -> str:
    return lib().nvfp4_status_string(status).decode()


def nvfp4_codec_selftest(which: int, x, u16, out, stream=None):
    p = (lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0))
    _check(lib().nvfp4_codec_selftest(which, p(x), p(u16), p(out), out.numel(), _stream(stream)),
           "nvfp4_codec_selftest")
    return out


# ---------------------------------------------------------------------------
# conveniences (allocation + one call)
# ---------------------------------------------------------------------------
def quantize(x, specs: Sequence[QuantSpec], workspace=None, stream=None) -> List[QTensor]:
    """Allocate the outputs for `specs` (and, if none is given, a workspace)
    on the stream the call runs on, and quantise x into them."""
    with _on_stream(stream):
        if workspace is None:
            workspace = new_workspace(x.device)
        outs = []
        for s in specs:
            r, c, k = output_shape(x.shape[0], x.shape[1], s.layout)
            outs.append(empty_qtensor(r, c, k, x.device, rht=int(s.rht)))
    return nvfp4_quantize(x, specs, outs, workspace, stream)


def dequantize(q: QTensor, stream=None):
    import torch
    with _on_stream(stream):
        y = torch.empty((q.rows, q.cols), dtype=torch.float32, device=q.codes.device)
    return nvfp4_dequantize(q, y, stream)


def gemm(a: QTensor, b: QTensor, out_dtype="f32", workspace=None, stream=None):
    import torch
    dt = torch.float32 if out_dtype == "f32" else torch.bfloat16
    with _on_stream(stream):
        c = torch.empty((a.rows, b.rows), dtype=dt, device=a.codes.device)
    return nvfp4_gemm(a, b, c, workspace, stream)


# ---------------------------------------------------------------------------
# MXFP4 (OCP MX v1.0: 32-element blocks, E8M0 scales, no per-tensor scale)
# ---------------------------------------------------------------------------
@dataclass
class MXTensor:
    codes: "object"   # torch.uint8 [rows][cols/2]
    scales: "object"  # torch.uint8 [rows][cols/32] (E8M0)
    rows: int
    cols: int

    def c_struct(self) -> mxfp4_tensor:
        return mxfp4_tensor(self.codes.data_ptr(), self.scales.data_ptr(), self.rows, self.cols)


def empty_mxtensor(rows: int, cols: int, device="cuda") -> MXTensor:
    import torch
    return MXTensor(codes=torch.empty((rows, cols // 2), dtype=torch.uint8, device=device),
                    scales=torch.empty((rows, cols // 32), dtype=torch.uint8, device=device), rows=rows, cols=cols)


def mxfp4_quantize(x, layout, out: MXTensor, stream=None) -> MXTensor:
    """MXFP4-quantise the bf16 device tensor x [rows][cols] into out
    (layout ROW_1D: out is rows x cols; COL_1D: out is x^T)."""
    import torch
    assert x.dtype == torch.bfloat16 and x.dim() == 2 and x.stride(1) == 1
    t = out.c_struct()
    _check(lib().mxfp4_quantize(ctypes.c_void_p(x.data_ptr()), x.shape[0], x.shape[1], x.stride(0),
                                LAYOUTS.get(layout, layout), ctypes.byref(t), _stream(stream)), "mxfp4_quantize")
    return out


def mxfp4_dequantize(q: MXTensor, y, stream=None):
    """y = e(code) * 2^(scale - 127) as fp32."""
    import torch
    assert y.dtype == torch.float32 and y.stride(1) == 1
    t = q.c_struct()
    _check(lib().mxfp4_dequantize(ctypes.byref(t), ctypes.c_void_p(y.data_ptr()), y.stride(0), _stream(stream)),
           "mxfp4_dequantize")
    return y


def mxfp4_gemm(a: MXTensor, b: MXTensor, c, stream=None):
    """C[M][N] = A^ B^T into the fp32 or bf16 device tensor c."""
    import torch
    dt = F32 if c.dtype == torch.float32 else BF16 if c.dtype == torch.bfloat16 else None
    if dt is None:
        raise TypeError("c must be float32 or bfloat16")
    assert c.stride(1) == 1
    ta, tb = a.c_struct(), b.c_struct()
    _check(lib().mxfp4_gemm(ctypes.byref(ta), ctypes.byref(tb), ctypes.c_void_p(c.data_ptr()), dt, c.stride(0),
                            _stream(stream)), "mxfp4_gemm")
    return c


def mx_quantize(x, layout="row", stream=None) -> MXTensor:
    """Allocate the output and MXFP4-quantise x."""
    layout = LAYOUTS.get(layout, layout)
    r, c = (x.shape[0], x.shape[1]) if layout == ROW_1D else (x.shape[1], x.shape[0])
    with _on_stream(stream):
        out = empty_mxtensor(r, c, x.device)
    return mxfp4_quantize(x, layout, out, stream)


def mx_gemm(a: MXTensor, b: MXTensor, out_dtype="f32", stream=None):
    import torch
    dt = torch.float32 if out_dtype == "f32" else torch.bfloat16
    with _on_stream(stream):
        c = torch.empty((a.rows, b.rows), dtype=dt, device=a.codes.device)
    return mxfp4_gemm(a, b, c, stream)
