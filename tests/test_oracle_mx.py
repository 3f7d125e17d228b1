"""Pins of the MXFP4 oracle (the earlier 4-bit microscaling format the NVFP4
news page sets NVFP4 against, paragraph 3; defined by the OCP Microscaling
Formats (MX) specification v1.0, sections 5 and 6.3, since the page gives no
definition): hand-worked blocks, brute-force scale and grid searches written
independently of the oracle's closed forms, the block-maximum invariant, and an
exact rational GEMM."""
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
GRID = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def bf16_bits(v) -> np.ndarray:
    f = np.asarray(v, dtype=np.float32)
    b = f.view(np.uint32)
    assert np.all((b & 0xFFFF) == 0), "values must be bf16-exact"
    return (b >> 16).astype(np.uint16)


def unpack(codes: np.ndarray) -> np.ndarray:
    lo, hi = codes & 15, codes >> 4
    return np.stack([lo, hi], axis=-1).reshape(codes.shape[0], -1)


def test_e8m0_scale_closed_forms():
    # exponent floor(log2 amax) - 2, code = exponent + 127, clamped; zero -> code 0
    cases = {6.0: 127, 4.0: 127, 7.99: 127, 8.0: 128, 1.0: 125, 0.001: 115, 0.0: 0,
             2.0 ** -133: 0, 2.0 ** -125: 0, 2.0 ** -124: 1, 2.0 ** -120: 5, 3.3895e38: 252, 2.0 ** 127: 252}
    for amax, code in cases.items():
        assert oracle.e8m0_scale_code(amax) == code, amax
    for code in (0, 1, 126, 127, 128, 254):
        assert oracle.e8m0_value(code) == 2.0 ** (code - 127)


def test_golden_blocks():
    rows, want_s, want_c = [], [], []
    for line in open(os.path.join(GOLDEN, "mxfp4_blocks.txt")):
        if line.startswith("#") or not line.strip():
            continue
        v, s, c = line.split("|")
        rows.append([float(t) for t in v.split()])
        want_s.append(int(s))
        want_c.append([int(t, 16) for t in c.split()])
    x = bf16_bits(np.array(rows, dtype=np.float64).astype(np.float32))
    q = oracle.mx_quantize(x, "row")
    assert q["scales"][:, 0].tolist() == want_s
    assert unpack(q["codes"]).tolist() == want_c
    # the same blocks along the other dimension (column layout of x^T)
    qc = oracle.mx_quantize(np.ascontiguousarray(x.T), "col")
    assert qc["scales"][:, 0].tolist() == want_s
    assert unpack(qc["codes"]).tolist() == want_c


def brute_force_block(v: np.ndarray):
    """Scale: the largest power of two X = 2^e, e in [-127, 127], with
    max |v| / X >= 4 (so that max |v| / X lies in [4, 8)), found by search;
    elements: the grid value nearest to |v| / X (ties to the even code
    index), clamped at 6, with the sign bit of v."""
    amax = float(np.max(np.abs(v)))
    e = -127
    if amax > 0:
        for cand in range(127, -128, -1):
            if amax / 2.0 ** cand >= 4.0:
                e = cand
                break
        else:
            e = -127
    X = 2.0 ** e
    codes = []
    for val in v:
        a = min(abs(float(val)) / X, 6.0)
        d = [abs(a - g) for g in GRID]
        best = min(range(8), key=lambda i: (d[i], i % 2))  # nearest, then even code
        codes.append(best | (8 if np.signbit(val) else 0))
    return e + 127, codes


@pytest.mark.parametrize("layout", ["row", "col"])
def test_brute_force_small(layout):
    rng = np.random.default_rng(5)
    R, C = 32, 96
    vals = rng.normal(size=(R, C)) * np.exp2(rng.integers(-20, 20, size=(R, 1)))
    vals[3, :] = 0.0
    vals[4, 5] = -0.0
    vals[7, :32] = rng.choice(np.array(GRID + [-g for g in GRID]), size=32) * 2.0 ** -3  # on-grid values
    vals[9, :] = rng.normal(size=C) * 2.0 ** -130  # bf16 subnormals: clamped scale
    x = (vals.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)  # truncation to bf16
    xf = oracle.bf16_bits_to_f32(x).astype(np.float64)
    q = oracle.mx_quantize(x, layout)
    src = xf if layout == "row" else xf.T
    codes = unpack(q["codes"])
    for r in range(src.shape[0]):
        for b in range(src.shape[1] // 32):
            s, c = brute_force_block(src[r, 32 * b:32 * b + 32])
            assert q["scales"][r, b] == s, (r, b)
            assert codes[r, 32 * b:32 * b + 32].tolist() == c, (r, b)


def test_block_max_invariant():
    """The largest magnitude of every non-zero block decodes to 4 X or 6 X
    (max |v| / X lies in [4, 8)), and every element is within half a grid
    step of v / X (or clamped at 6)."""
    rng = np.random.default_rng(11)
    vals = rng.standard_t(3, size=(64, 256)) * np.exp2(rng.integers(-30, 30, size=(64, 1)))
    x = (vals.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    xf = oracle.bf16_bits_to_f32(x).astype(np.float64)
    q = oracle.mx_quantize(x, "row")
    d = oracle.mx_decode(q)
    X = np.exp2(q["scales"].astype(np.float64) - 127).repeat(32, axis=1)
    bm = np.abs(d).reshape(64, 8, 32).max(axis=2) / X[:, ::32]
    assert np.all((bm == 4.0) | (bm == 6.0))
    a = np.abs(xf) / X
    step = np.where(a < 2, 0.5, np.where(a < 4, 1.0, 2.0))
    err = np.abs(np.abs(d) / X - np.minimum(a, 6.0))
    assert np.all(err <= step / 2 + 1e-12)


def test_gemm_exact_rational():
    """C = A^ B^T with every product and sum exact in rationals, against the
    oracle's binary64 triple loop and its BLAS route."""
    rng = np.random.default_rng(3)
    M, N, K = 16, 16, 96
    qa = dict(codes=rng.integers(0, 256, (M, K // 2), dtype=np.uint8),
              scales=rng.integers(120, 135, (M, K // 32), dtype=np.uint8), rows=M, cols=K)
    qb = dict(codes=rng.integers(0, 256, (N, K // 2), dtype=np.uint8),
              scales=rng.integers(120, 135, (N, K // 32), dtype=np.uint8), rows=N, cols=K)
    mag = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3), Fraction(4), Fraction(6)]

    def val(q, r, k):
        b = int(q["codes"][r, k // 2])
        c = (b >> 4) if k & 1 else (b & 15)
        v = mag[c & 7] * Fraction(2) ** (int(q["scales"][r, k // 32]) - 127)
        return -v if c & 8 else v

    A = [[val(qa, m, k) for k in range(K)] for m in range(M)]
    B = [[val(qb, n, k) for k in range(K)] for n in range(N)]
    exact = np.array([[float(sum(A[m][k] * B[n][k] for k in range(K))) for n in range(N)] for m in range(M)])
    assert np.array_equal(oracle.mx_gemm_f64_loop(qa, qb), exact)
    assert np.array_equal(oracle.mx_gemm_f64(qa, qb), exact)


def test_rejects_bad_shapes():
    x = np.zeros((16, 48), dtype=np.uint16)
    with pytest.raises(ValueError):
        oracle.mx_quantize(x, "row")  # 48 is not a multiple of 32
    with pytest.raises(ValueError):
        oracle.mx_quantize(np.zeros((48, 32), dtype=np.uint16), "col")
    with pytest.raises(ValueError):
        oracle.mx_quantize(x, "2d")
