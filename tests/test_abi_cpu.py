"""CPU-only checks of the C ABI: the library loads, exports every function
include/nvfp4.h declares, and rejects invalid arguments on the host before
anything is enqueued (no GPU is touched by these calls)."""
import ctypes
import os
import re
import subprocess

import pytest

import nvfp4_bit_quantization_amd as nv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(nv.LIB_PATH):
        from nvfp4_bit_quantization_amd import build
        build.build()
    return nv.lib()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w \*]*?\b((?:nv|mx)fp4_\w+)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("nvfp4_quantize", "nvfp4_quantize_batch", "nvfp4_quantize_noalloc", "nvfp4_dequantize", "nvfp4_gemm", "nvfp4_workspace_bytes",
              "nvfp4_rht_sign_mask",
              "nvfp4_status_string", "nvfp4_codec_selftest", "mxfp4_quantize", "mxfp4_dequantize", "mxfp4_gemm"):
        assert n in names


def test_library_exports_every_declared_symbol(L):
    for n in declared_functions():
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", nv.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (\w+)", out))
    assert set(declared_functions()) <= exported


def test_header_compiles_as_c():
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-fsyntax-only", "-x", "c", HEADER],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


FAKE = 0x10000  # a 16-byte aligned non-null address; never dereferenced on the error paths


def _tensor(rows, cols, kind, codes=FAKE):
    return nv.nvfp4_tensor(codes, FAKE, FAKE, FAKE, rows, cols, kind, 0)


def _out(layout, rows, cols, kind, rounding=0, rht=0, flags=0, codes=FAKE):
    return nv.nvfp4_quant_output(layout, rounding, rht, flags, 1, 2, _tensor(rows, cols, kind, codes))


def _q(L, outs, x=FAKE, rows=64, cols=32, ld=32, ws=FAKE, wsb=None):
    arr = (nv.nvfp4_quant_output * max(1, len(outs)))(*outs)
    if wsb is None:
        wsb = L.nvfp4_workspace_bytes()
    return L.nvfp4_quantize(ctypes.c_void_p(x), rows, cols, ld, arr, len(outs), ctypes.c_void_p(ws), wsb, None)


def test_quantize_argument_validation(L):
    row = _out(nv.ROW_1D, 64, 32, nv.SCALE_1D16)
    col = _out(nv.COL_1D, 32, 64, nv.SCALE_1D16)
    assert _q(L, [row], x=0) == -1                                    # NULL x
    assert _q(L, [row], rows=24) == -2                                 # rows % 16
    assert _q(L, [row], cols=0) == -2
    assert _q(L, [row], ld=16) == -3                                   # ld < cols
    assert _q(L, [row], x=FAKE + 8) == -4                              # misaligned x
    assert _q(L, [row], ld=36) == -4                                   # ld % 8
    assert _q(L, [row, col, row]) == -5                                # n_outs
    assert _q(L, [row], ws=0) == -6
    assert _q(L, [row], wsb=16) == -6
    assert _q(L, [_out(nv.TWO_D, 64, 32, nv.SCALE_2D16, rht=1)]) == -5  # RHT with 2D
    assert _q(L, [_out(nv.ROW_1D, 64, 32, nv.SCALE_1D16, rounding=7)]) == -5
    assert _q(L, [_out(9, 64, 32, nv.SCALE_1D16)]) == -5
    assert _q(L, [_out(nv.ROW_1D, 64, 32, nv.SCALE_1D16, flags=2)]) == -5     # unknown flag
    assert _q(L, [_out(nv.ROW_1D, 32, 64, nv.SCALE_1D16)]) == -2        # descriptor shape mismatch
    assert _q(L, [_out(nv.ROW_1D, 64, 32, nv.SCALE_2D16)]) == -2        # wrong scale kind
    assert _q(L, [_out(nv.ROW_1D, 64, 32, nv.SCALE_1D16, codes=0)]) == -1
    assert _q(L, [_out(nv.ROW_1D, 64, 32, nv.SCALE_1D16, codes=FAKE + 4)]) == -4
    assert _q(L, [row, row]) == -5                                     # unsupported pair
    assert _q(L, [_out(nv.TWO_D, 64, 32, nv.SCALE_2D16), col]) == -5
    # 16-element blocks are numbered in 31 bits: rows/16 * cols < 2^31
    big_r, big_c = 1 << 20, 1 << 15
    assert _q(L, [_out(nv.ROW_1D, big_r, big_c, nv.SCALE_1D16)], rows=big_r, cols=big_c, ld=big_c) == -2


def _qn(L, outs, x=FAKE, rows=64, cols=32, ld=32):
    arr = (nv.nvfp4_quant_output * max(1, len(outs)))(*outs)
    return L.nvfp4_quantize_noalloc(ctypes.c_void_p(x), rows, cols, ld, arr, len(outs), None)


def test_quantize_noalloc_argument_validation(L):
    """The allocation-free entry point checks its arguments as nvfp4_quantize
    does, before it looks up its scratch (no GPU is needed for these)."""
    row = _out(nv.ROW_1D, 64, 32, nv.SCALE_1D16)
    col = _out(nv.COL_1D, 32, 64, nv.SCALE_1D16)
    assert _qn(L, [row], x=0) == -1
    assert _qn(L, [row], rows=24) == -2
    assert _qn(L, [row], ld=16) == -3
    assert _qn(L, [row], x=FAKE + 8) == -4
    assert _qn(L, [row, col, row]) == -5
    assert _qn(L, [_out(nv.TWO_D, 64, 32, nv.SCALE_2D16, rht=1)]) == -5
    assert _qn(L, [_out(nv.ROW_1D, 32, 64, nv.SCALE_1D16)]) == -2
    assert _qn(L, [row, row]) == -5
    arr = (nv.nvfp4_quant_output * 1)(row)
    assert L.nvfp4_quantize_noalloc(None, 64, 32, 32, arr, 1, None) == -1
    assert L.nvfp4_quantize_noalloc(ctypes.c_void_p(FAKE), 64, 32, 32, None, 1, None) == -1


def _job(outs, x=FAKE, rows=64, cols=32, ld=32):
    arr = (nv.nvfp4_quant_output * max(1, len(outs)))(*outs)
    return nv.nvfp4_quant_job(x, rows, cols, ld, ctypes.cast(arr, ctypes.POINTER(nv.nvfp4_quant_output)),
                              len(outs)), arr


def test_quantize_batch_argument_validation(L):
    """The batch entry point rejects a bad batch, or any bad job in it, with
    that job's nvfp4_quantize status, before anything is enqueued."""
    row = _out(nv.ROW_1D, 64, 32, nv.SCALE_1D16)
    colr = _out(nv.COL_1D, 32, 64, nv.SCALE_1D16, rht=1)
    wsb = L.nvfp4_workspace_bytes()

    def batch(specs, n=None, ws=FAKE, nbytes=None):
        made = [_job(*s) if isinstance(s, tuple) else _job(s) for s in specs]
        arr = (nv.nvfp4_quant_job * max(1, len(made)))(*[m[0] for m in made])
        n = len(made) if n is None else n
        nbytes = n * wsb if nbytes is None else nbytes
        return L.nvfp4_quantize_batch(arr, n, ctypes.c_void_p(ws), nbytes, None)

    assert L.nvfp4_quantize_batch(None, 1, ctypes.c_void_p(FAKE), wsb, None) == -1
    assert batch([[row]], n=0) == -5
    assert batch([[row]], ws=0) == -6
    assert batch([[colr], [colr]], nbytes=2 * wsb - 1) == -6          # one slice per job
    assert batch([[row]], ws=FAKE + 8) == -4
    assert batch([([row], 0)]) == -1                                  # NULL x in the only job
    assert batch([[colr], ([colr], FAKE, 24)]) == -2                  # the second job's shape
    assert batch([[colr], ([colr], FAKE, 64, 32, 16)]) == -3          # the second job's ld
    assert batch([[colr], [row, row]]) == -5                          # unsupported pair in a job
    assert batch([[colr], []]) == -5                                  # a job without outputs


def test_dequantize_and_gemm_validation(L):
    t = _tensor(64, 32, nv.SCALE_1D16)
    y = ctypes.c_void_p(FAKE)
    assert L.nvfp4_dequantize(None, y, 32, None) == -1
    assert L.nvfp4_dequantize(ctypes.byref(t), None, 32, None) == -1
    assert L.nvfp4_dequantize(ctypes.byref(_tensor(60, 32, 0)), y, 32, None) == -2
    assert L.nvfp4_dequantize(ctypes.byref(t), y, 16, None) == -3
    assert L.nvfp4_dequantize(ctypes.byref(t), ctypes.c_void_p(FAKE + 4), 32, None) == -4
    assert L.nvfp4_dequantize(ctypes.byref(_tensor(64, 32, 5)), y, 32, None) == -5
    a = _tensor(64, 32, nv.SCALE_1D16)
    b = _tensor(48, 32, nv.SCALE_2D16)
    bk = _tensor(48, 48, nv.SCALE_1D16)
    c = ctypes.c_void_p(FAKE)
    assert L.nvfp4_gemm(ctypes.byref(a), ctypes.byref(bk), c, 0, 48, None, 0, None) == -5   # K mismatch
    assert L.nvfp4_gemm(ctypes.byref(a), ctypes.byref(b), c, 3, 48, None, 0, None) == -5    # dtype
    assert L.nvfp4_gemm(ctypes.byref(a), ctypes.byref(b), c, 0, 40, None, 0, None) == -3    # ldc < N
    assert L.nvfp4_gemm(ctypes.byref(a), ctypes.byref(b), None, 0, 48, None, 0, None) == -1
    assert L.nvfp4_gemm(ctypes.byref(_tensor(64, 40, 0)), ctypes.byref(_tensor(48, 40, 0)), c, 0, 48, None, 0,
                        None) == -2
    ws = ctypes.c_void_p(FAKE + 8)                                                         # misaligned workspace
    assert L.nvfp4_gemm(ctypes.byref(a), ctypes.byref(b), c, 0, 48, ws, 1 << 20, None) == -4
    big = (1 << 31) - 16                                       # 2^46 tiles of C: more than the 32-bit grid holds
    assert L.nvfp4_gemm(ctypes.byref(_tensor(big, 32, 0)), ctypes.byref(_tensor(big, 32, 0)), c, 0, big, None, 0,
                        None) == -2
    # producer-fused maxima: at least one target, 4-byte aligned, plus the GEMM's own checks
    am = ctypes.c_void_p(FAKE)
    assert L.nvfp4_gemm_amax(ctypes.byref(a), ctypes.byref(b), c, 48, None, 0, None, None, 0, None) == -1
    assert L.nvfp4_gemm_amax(ctypes.byref(a), ctypes.byref(b), c, 48, None, 0, ctypes.c_void_p(FAKE + 2), None, 0,
                             None) == -4
    assert L.nvfp4_gemm_amax(ctypes.byref(a), ctypes.byref(bk), c, 48, None, 0, am, am, 0, None) == -5
    assert L.nvfp4_gemm_amax(ctypes.byref(a), ctypes.byref(b), c, 40, None, 0, am, None, 0, None) == -3
    assert L.nvfp4_codec_selftest(3, None, None, None, 0, None) == -5
    assert L.nvfp4_codec_selftest(0, None, None, None, -1, None) == -2
    assert L.nvfp4_codec_selftest(0, None, None, None, 5, None) == -1


def _mx(rows, cols, codes=FAKE, scales=FAKE):
    return nv.mxfp4_tensor(codes, scales, rows, cols)


def test_mxfp4_argument_validation(L):
    x = ctypes.c_void_p(FAKE)
    q = lambda out, rows=64, cols=96, ld=96, layout=nv.ROW_1D, xx=x: L.mxfp4_quantize(  # noqa: E731
        xx, rows, cols, ld, layout, ctypes.byref(out), None)
    assert q(_mx(64, 96), xx=None) == -1
    assert q(_mx(64, 96, codes=0)) == -1
    assert q(_mx(40, 96), rows=40) == -2                       # rows % 16 (row layout)
    assert q(_mx(96, 48), rows=48, layout=nv.COL_1D) == -2     # blocked rows % 32 (column layout)
    assert q(_mx(64, 80), cols=80, ld=80) == -2                # cols % 32
    assert q(_mx(96, 64)) == -2                                # descriptor is not the stored shape
    assert q(_mx(64, 96), ld=64) == -3
    assert q(_mx(64, 96), ld=100) == -4                        # ld % 8
    assert q(_mx(64, 96), xx=ctypes.c_void_p(FAKE + 2)) == -4
    assert q(_mx(64, 96, codes=FAKE + 8)) == -4
    assert q(_mx(64, 96), layout=nv.TWO_D) == -5
    y = ctypes.c_void_p(FAKE)
    assert L.mxfp4_dequantize(None, y, 96, None) == -1
    assert L.mxfp4_dequantize(ctypes.byref(_mx(64, 80)), y, 96, None) == -2
    assert L.mxfp4_dequantize(ctypes.byref(_mx(64, 96)), y, 64, None) == -3
    assert L.mxfp4_dequantize(ctypes.byref(_mx(64, 96)), y, 98, None) == -4
    a, b, c = _mx(64, 96), _mx(48, 96), ctypes.c_void_p(FAKE)
    g = lambda a_, b_, c_=c, dt=0, ldc=48: L.mxfp4_gemm(ctypes.byref(a_), ctypes.byref(b_), c_, dt, ldc, None)  # noqa
    assert g(a, b, c_=None) == -1
    assert g(a, _mx(48, 64)) == -5                             # K mismatch
    assert g(_mx(64, 80), _mx(48, 80)) == -2                   # K % 32
    assert g(a, b, dt=2) == -5
    assert g(a, b, ldc=40) == -3
    assert g(a, _mx(48, 96, scales=FAKE + 2)) == -4            # scales 4-byte aligned
    assert g(_mx(64, 96, codes=FAKE + 4), b) == -4


def test_status_strings(L):
    for s in range(-7, 1):
        assert nv.nvfp4_status_string(s)
    assert nv.nvfp4_status_string(-99) == "unknown status"


def test_workspace_bytes_is_small(L):
    assert 0 < nv.nvfp4_workspace_bytes() <= 64 * 1024


def test_rht_sign_mask_matches_oracle(L):
    import oracle
    for seed in (0, 1, 1234, 4321, 2**40 + 3, 2**64 - 1):
        assert nv.nvfp4_rht_sign_mask(seed) == oracle.rht_sign_mask(seed)


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    monkeypatch.setattr(nv, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(nv, "_lib", None)
    with pytest.raises(ImportError):
        nv.lib()
