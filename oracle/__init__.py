"""CPU oracle for the NVFP4 quantisation pipeline and the NVFP4 GEMM.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use this package; the product library
and its Python binding never import it.  The arithmetic lives in the plain C
file ``nvfp4_oracle.c`` (built with gcc, no fast-math, no FP contraction);
this module is ctypes marshalling plus the large-GEMM route, which multiplies
the exactly decoded operands with a float64 BLAS matmul (a library primitive
standing in for the triple loop of ``oracle_gemm_f64``, which the tests check
it against on small shapes).

Method source: the NVFP4 pretraining news page (zubnet.ai,
"nvidia-nvfp4-paper-4-bit-pretrain-hits-fp8-parity-12b-10t-tokens", en/pt/fr/hi
versions), paragraph 2: blocks of 16 E2M1 values, each with an E4M3 scale,
under one FP32 scale per tensor; a 16x16 RHT with random signs on the
weight-gradient inputs; 16x16 scale blocks for weights; stochastic rounding for
gradients.

MXFP4 (the earlier microscaling format the page compares NVFP4 with, paragraph
3) follows the OCP Microscaling Formats (MX) specification v1.0, since the page
does not define it: 32-element blocks, E8M0 scale 2^(floor(log2 amax) - 2),
E2M1 elements rounded to nearest-even and clamped at 6.

Parity unpinned (conventions with no value on the page to pin them): nibble
order, code and scale layouts, the Philox counter assignment for stochastic
rounding and for the sign vector, and the block order.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Dict

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nvfp4_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle_nvfp4.so")

ROW_1D, COL_1D, TWO_D, TWO_D_T = 0, 1, 2, 3
RTN, SR = 0, 1
SCALE_1D16, SCALE_2D16 = 0, 1
LAYOUTS = {"row": ROW_1D, "col": COL_1D, "2d": TWO_D, "2d_t": TWO_D_T}
ROUNDINGS = {"rtn": RTN, "sr": SR}

_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc into ``oracle/liboracle_nvfp4.so``."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-ffp-contract=off", "-fno-fast-math",
               "-fexcess-precision=standard", "-fopenmp", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build(force=True)
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    i64, i32, u64, u32 = ctypes.c_int64, ctypes.c_int, ctypes.c_uint64, ctypes.c_uint32
    f32, f64 = ctypes.c_float, ctypes.c_double
    sig = {
        "oracle_threads": (i32, []),
        "oracle_set_threads": (None, [i32]),
        "oracle_e2m1_value": (f64, [ctypes.c_uint8]),
        "oracle_e2m1_encode_rtn": (ctypes.c_uint8, [f32]),
        "oracle_e2m1_encode_sr": (ctypes.c_uint8, [f32, ctypes.c_uint16]),
        "oracle_e4m3_value": (f32, [ctypes.c_uint8]),
        "oracle_e4m3_encode": (ctypes.c_uint8, [f32]),
        "oracle_philox4x32_10": (None, [P, P, P]),
        "oracle_sr_uniform": (ctypes.c_uint16, [u64, u64, i32]),
        "oracle_rht_sign_mask": (ctypes.c_uint16, [u64]),
        "oracle_rht16_f64": (None, [P, ctypes.c_uint16, P]),
        "oracle_quantize": (i32, [P, i64, i64, i64, i32, i32, i32, u64, u64, P, P, P, P]),
        "oracle_quantize_at": (i32, [P, i64, i64, i64, i32, i32, i32, u64, u64, u64, P, P, P, P]),
        "oracle_dequantize": (i32, [P, P, i64, i64, i32, f32, P]),
        "oracle_decode_products": (i32, [P, P, i64, i64, i32, P]),
        "oracle_gemm_f64": (i32, [P, P, i32, f32, P, P, i32, f32, i64, i64, i64, P]),
        "oracle_f64_to_bf16": (ctypes.c_uint16, [f64]),
        "oracle_e2m1_encode_rtn_array": (None, [P, i64, P]),
        "oracle_e2m1_encode_sr_array": (None, [P, P, i64, P]),
        "oracle_e4m3_encode_array": (None, [P, i64, P]),
        "oracle_e2m1_encode_rtn_bits": (None, [u32, u32, P]),
        "oracle_e4m3_encode_bits": (None, [u32, u32, P]),
        "oracle_e2m1_sr_step_bits": (None, [u32, u32, P]),
        "oracle_philox_array": (None, [P, P, i64, P]),
        "oracle_f64_to_bf16_array": (None, [P, i64, P]),
        "oracle_sr_uniform_array": (None, [u64, P, P, i64, P]),
        "oracle_e8m0_scale_code": (ctypes.c_uint8, [f64]),
        "oracle_e8m0_value": (f64, [ctypes.c_uint8]),
        "oracle_mx_quantize": (i32, [P, i64, i64, i64, i32, P, P]),
        "oracle_mx_decode": (i32, [P, P, i64, i64, P]),
        "oracle_mx_gemm_f64": (i32, [P, P, P, P, i64, i64, i64, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


# --------------------------------------------------------------------------
# scalar / array codecs
# --------------------------------------------------------------------------
def threads() -> int:
    """Threads the oracle's parallel loops use."""
    return int(_load().oracle_threads())


def set_threads(n: int) -> None:
    """Set the threads of the oracle's parallel loops (results do not depend on it)."""
    _load().oracle_set_threads(int(n))


def e2m1_value(code: int) -> float:
    return _load().oracle_e2m1_value(code)


def e4m3_value_array(codes) -> np.ndarray:
    """E4M3 decode of an array of codes (the scalar decoder, tabulated)."""
    table = np.array([e4m3_value(c) for c in range(256)], dtype=np.float32)
    return table[np.asarray(codes, dtype=np.uint8)]


def e4m3_value(code: int) -> float:
    return _load().oracle_e4m3_value(code)


def e2m1_encode_rtn(y) -> np.ndarray:
    y = np.ascontiguousarray(y, dtype=np.float32)
    out = np.empty(y.shape, dtype=np.uint8)
    _load().oracle_e2m1_encode_rtn_array(_ptr(y), y.size, _ptr(out))
    return out


def e2m1_encode_sr(y, u16) -> np.ndarray:
    y = np.ascontiguousarray(y, dtype=np.float32)
    u16 = np.ascontiguousarray(np.broadcast_to(u16, y.shape), dtype=np.uint16)
    out = np.empty(y.shape, dtype=np.uint8)
    _load().oracle_e2m1_encode_sr_array(_ptr(y), _ptr(u16), y.size, _ptr(out))
    return out


def e4m3_encode(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint8)
    _load().oracle_e4m3_encode_array(_ptr(x), x.size, _ptr(out))
    return out


def e2m1_encode_rtn_bits(start: int, count: int) -> np.ndarray:
    """RTN codes for the fp32 bit patterns start .. start+count-1 (0xFF for NaN/Inf)."""
    out = np.empty(count, dtype=np.uint8)
    _load().oracle_e2m1_encode_rtn_bits(start, count, _ptr(out))
    return out


def e4m3_encode_bits(start: int, count: int) -> np.ndarray:
    """E4M3 codes for the fp32 bit patterns start .. start+count-1 (0xFF for
    negative, NaN or Inf patterns)."""
    out = np.empty(count, dtype=np.uint8)
    _load().oracle_e4m3_encode_bits(start, count, _ptr(out))
    return out


def e2m1_sr_step_bits(start: int, count: int) -> np.ndarray:
    """For the fp32 bit patterns start .. start+count-1: the smallest u16 whose
    stochastic-rounding code equals the code at u16 = 65535 (0 if all u16 give
    one code); 0xFFFFFFFF for NaN/Inf patterns."""
    out = np.empty(count, dtype=np.uint32)
    _load().oracle_e2m1_sr_step_bits(start, count, _ptr(out))
    return out


def philox4x32_10(key, ctr) -> np.ndarray:
    """Philox4x32-10 for arrays of keys [n,2] and counters [n,4] (uint32)."""
    key = np.ascontiguousarray(np.atleast_2d(key), dtype=np.uint32)
    ctr = np.ascontiguousarray(np.atleast_2d(ctr), dtype=np.uint32)
    n = ctr.shape[0]
    assert key.shape == (n, 2) and ctr.shape == (n, 4)
    out = np.empty((n, 4), dtype=np.uint32)
    _load().oracle_philox_array(_ptr(key), _ptr(ctr), n, _ptr(out))
    return out


def sr_uniform(seed: int, block: int, j: int) -> int:
    return _load().oracle_sr_uniform(seed, block, j)


def sr_uniform_array(seed: int, blocks, js) -> np.ndarray:
    blocks = np.ascontiguousarray(blocks, dtype=np.uint64)
    js = np.ascontiguousarray(np.broadcast_to(js, blocks.shape), dtype=np.int32)
    out = np.empty(blocks.shape, dtype=np.uint16)
    _load().oracle_sr_uniform_array(seed, _ptr(blocks), _ptr(js), blocks.size, _ptr(out))
    return out


def rht_sign_mask(seed: int) -> int:
    return _load().oracle_rht_sign_mask(seed)


def rht16(v, sign_mask: int) -> np.ndarray:
    """One 16-group of the RHT in binary64 (before the final fp32 rounding)."""
    v = np.ascontiguousarray(v, dtype=np.float64)
    assert v.shape == (16,)
    z = np.empty(16, dtype=np.float64)
    _load().oracle_rht16_f64(_ptr(v), sign_mask, _ptr(z))
    return z


def f64_to_bf16_bits(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    _load().oracle_f64_to_bf16_array(_ptr(x), x.size, _ptr(out))
    return out


def bf16_bits_to_f32(b) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------
# tensor-level operations
# --------------------------------------------------------------------------
def out_shape(rows: int, cols: int, layout: int):
    """(out_rows, out_cols) of the stored codes for an input [rows][cols]."""
    if layout in (COL_1D, TWO_D_T):
        return cols, rows
    return rows, cols


def scale_shape(rows: int, cols: int, layout: int):
    orow, ocol = out_shape(rows, cols, layout)
    if layout in (TWO_D, TWO_D_T):
        return orow // 16, ocol // 16
    return orow, ocol // 16


def quantize(x_bits: np.ndarray, layout="row", rounding="rtn", rht=False, sr_seed=0, rht_seed=0,
             block_offset=0) -> Dict:
    """Quantise a bf16 tensor given as uint16 bit patterns [R][C].

    ``block_offset`` numbers the stochastic-rounding blocks of a slice of a
    larger tensor as in the whole (the blocks before the slice in output order).
    Returns dict(codes [orow][ocol/2] uint8, scales uint8, S float32,
    amax float32, rows, cols, scale_kind)."""
    layout = LAYOUTS.get(layout, layout)
    rounding = ROUNDINGS.get(rounding, rounding)
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    R, C = x_bits.shape
    orow, ocol = out_shape(R, C, layout)
    codes = np.zeros((orow, ocol // 2), dtype=np.uint8)
    scales = np.zeros(scale_shape(R, C, layout), dtype=np.uint8)
    S = np.zeros(1, dtype=np.float32)
    amax = np.zeros(1, dtype=np.float32)
    rc = _load().oracle_quantize_at(_ptr(x_bits), R, C, C, layout, rounding, int(bool(rht)), sr_seed, rht_seed,
                                    int(block_offset), _ptr(codes), _ptr(scales), _ptr(S), _ptr(amax))
    if rc != 0:
        raise ValueError("oracle_quantize rejected the arguments (rc=%d)" % rc)
    kind = SCALE_2D16 if layout in (TWO_D, TWO_D_T) else SCALE_1D16
    return dict(codes=codes, scales=scales, S=np.float32(S[0]), amax=np.float32(amax[0]), rows=orow, cols=ocol,
                scale_kind=kind)


def dequantize(q: Dict) -> np.ndarray:
    codes = np.ascontiguousarray(q["codes"], dtype=np.uint8)
    scales = np.ascontiguousarray(q["scales"], dtype=np.uint8)
    y = np.empty((q["rows"], q["cols"]), dtype=np.float32)
    rc = _load().oracle_dequantize(_ptr(codes), _ptr(scales), q["rows"], q["cols"], q["scale_kind"],
                                   float(q["S"]), _ptr(y))
    if rc != 0:
        raise ValueError("oracle_dequantize rejected the arguments (rc=%d)" % rc)
    return y


def decode_products(q: Dict) -> np.ndarray:
    """Exact operand values e(code) * s_b as float64 (no global scale)."""
    codes = np.ascontiguousarray(q["codes"], dtype=np.uint8)
    scales = np.ascontiguousarray(q["scales"], dtype=np.uint8)
    out = np.empty((q["rows"], q["cols"]), dtype=np.float64)
    rc = _load().oracle_decode_products(_ptr(codes), _ptr(scales), q["rows"], q["cols"], q["scale_kind"],
                                        _ptr(out))
    if rc != 0:
        raise ValueError("oracle_decode_products rejected the arguments (rc=%d)" % rc)
    return out


def gemm_f64_loop(qa: Dict, qb: Dict) -> np.ndarray:
    """C = (A^ B^T)/(S_A S_B) by the plain triple loop in binary64 (small shapes)."""
    M, K = qa["rows"], qa["cols"]
    N, Kb = qb["rows"], qb["cols"]
    assert K == Kb
    c = np.empty((M, N), dtype=np.float64)
    rc = _load().oracle_gemm_f64(_ptr(np.ascontiguousarray(qa["codes"])), _ptr(np.ascontiguousarray(qa["scales"])),
                                 qa["scale_kind"], float(qa["S"]),
                                 _ptr(np.ascontiguousarray(qb["codes"])), _ptr(np.ascontiguousarray(qb["scales"])),
                                 qb["scale_kind"], float(qb["S"]), M, N, K, _ptr(c))
    if rc != 0:
        raise ValueError("oracle_gemm_f64 rejected the arguments (rc=%d)" % rc)
    return c


def gemm_f64(qa: Dict, qb: Dict, rows_a=None) -> np.ndarray:
    """C = (A^ B^T)/(S_A S_B) in binary64 via a float64 BLAS matmul on the
    exactly decoded operands.  ``rows_a`` optionally restricts to a subset of
    rows of A (sampled parity at full size)."""
    A = decode_products(qa)
    if rows_a is not None:
        A = A[np.asarray(rows_a)]
    B = decode_products(qb)
    return (A @ B.T) / (np.float64(qa["S"]) * np.float64(qb["S"]))


def round_output(c64: np.ndarray, out_dtype: str) -> np.ndarray:
    """Round the binary64 GEMM result once to the output dtype ('f32' or 'bf16');
    bf16 results are returned as float32 values of the bf16 bit patterns."""
    if out_dtype == "f32":
        return c64.astype(np.float32)
    if out_dtype == "bf16":
        return bf16_bits_to_f32(f64_to_bf16_bits(c64))
    raise ValueError(out_dtype)


# --------------------------------------------------------------------------
# MXFP4 (OCP MX v1.0): 32-element blocks with an E8M0 scale
# --------------------------------------------------------------------------
def e8m0_scale_code(amax: float) -> int:
    return int(_load().oracle_e8m0_scale_code(float(amax)))


def e8m0_value(code: int) -> float:
    return float(_load().oracle_e8m0_value(code))


def mx_quantize(x_bits: np.ndarray, layout="row") -> Dict:
    """MXFP4 quantisation of a bf16 tensor (uint16 bit patterns [R][C]); layout
    'row' (blocks along C, output [R][C]) or 'col' (blocks along R, output
    [C][R]).  Returns dict(codes [orow][ocol/2], scales [orow][ocol/32] E8M0,
    rows, cols)."""
    layout = LAYOUTS.get(layout, layout)
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    R, C = x_bits.shape
    orow, ocol = out_shape(R, C, layout)
    codes = np.zeros((orow, ocol // 2), dtype=np.uint8)
    scales = np.zeros((orow, max(ocol // 32, 1)), dtype=np.uint8)
    rc = _load().oracle_mx_quantize(_ptr(x_bits), R, C, C, layout, _ptr(codes), _ptr(scales))
    if rc != 0:
        raise ValueError("oracle_mx_quantize rejected the arguments (rc=%d)" % rc)
    return dict(codes=codes, scales=scales, rows=orow, cols=ocol)


def mx_decode(q: Dict) -> np.ndarray:
    """Exact element values e(code) * 2^(scale - 127) as float64."""
    codes = np.ascontiguousarray(q["codes"], dtype=np.uint8)
    scales = np.ascontiguousarray(q["scales"], dtype=np.uint8)
    out = np.empty((q["rows"], q["cols"]), dtype=np.float64)
    rc = _load().oracle_mx_decode(_ptr(codes), _ptr(scales), q["rows"], q["cols"], _ptr(out))
    if rc != 0:
        raise ValueError("oracle_mx_decode rejected the arguments (rc=%d)" % rc)
    return out


def mx_gemm_f64_loop(qa: Dict, qb: Dict) -> np.ndarray:
    """C = A^ B^T by the plain triple loop in binary64 (small shapes)."""
    M, K = qa["rows"], qa["cols"]
    N = qb["rows"]
    assert qb["cols"] == K
    c = np.empty((M, N), dtype=np.float64)
    rc = _load().oracle_mx_gemm_f64(_ptr(np.ascontiguousarray(qa["codes"])), _ptr(np.ascontiguousarray(qa["scales"])),
                                    _ptr(np.ascontiguousarray(qb["codes"])), _ptr(np.ascontiguousarray(qb["scales"])),
                                    M, N, K, _ptr(c))
    if rc != 0:
        raise ValueError("oracle_mx_gemm_f64 rejected the arguments (rc=%d)" % rc)
    return c


def mx_gemm_f64(qa: Dict, qb: Dict, rows_a=None) -> np.ndarray:
    """C = A^ B^T in binary64 via a float64 BLAS matmul on the exactly decoded
    operands (optionally only the rows ``rows_a`` of A)."""
    A = mx_decode(qa)
    if rows_a is not None:
        A = A[np.asarray(rows_a)]
    return A @ mx_decode(qb).T
