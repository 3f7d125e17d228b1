"""GPU parity of the MXFP4 path (the earlier 4-bit microscaling format the
NVFP4 news page compares against, paragraph 3; defined by the OCP MX
specification v1.0) against the oracle: codes and E8M0 scales bit-exact,
dequantised values bit-exact, and the GEMM on the block-scaled FP4 MFMA within
relative Frobenius error 1e-5 of the oracle's binary64 result (fp32
accumulation of exact products) -- at several tiles with ragged edges, on both
kernels, and at the Wgrad shape 5120x5120x8192 on sampled rows."""
import numpy as np
import pytest

import oracle
from nvfp4_bit_quantization_amd import synthetic as syn

from gpu_util import dev_bf16, host, rel_frobenius, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def nv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import nvfp4_bit_quantization_amd as nv
    nv.lib()
    return nv


def gpu_mx(q) -> dict:
    return dict(codes=host(q.codes), scales=host(q.scales), rows=q.rows, cols=q.cols)


def mixed_bits(R, C, seed):
    """Channel-scaled normals with outliers, an all-zero block row, negative
    zeros, bf16 subnormals and a few huge values."""
    b = syn.activation(R, C, seed=seed)
    rng = np.random.default_rng(seed + 1)
    b[0, :64] = 0
    b[1, 32:64] = 0x8000  # -0
    b[2, :] = syn.f32_to_bf16_bits((rng.normal(size=C) * 2.0 ** -130).astype(np.float32))
    b[3, 5] = syn.f32_to_bf16_bits(np.float32([3.0e38]))[0]
    return b


QCASES = [(32, 32), (96, 160), (128, 256), (160, 352), (416, 608)]  # multiples of 32: both layouts


@pytest.mark.parametrize("layout", ["row", "col"])
@pytest.mark.parametrize("shape", QCASES, ids=lambda s: "%dx%d" % s)
def test_mx_quantize_bit_exact(nv, shape, layout):
    R, C = shape
    say("mx quantize", shape, layout)
    bits = mixed_bits(R, C, seed=R + C)
    q = nv.mx_quantize(dev_bf16(bits), layout)
    torch.cuda.synchronize()
    g, o = gpu_mx(q), oracle.mx_quantize(bits, layout)
    assert g["scales"].shape == o["scales"].shape and g["codes"].shape == o["codes"].shape
    assert np.count_nonzero(g["scales"] != o["scales"]) == 0
    assert np.count_nonzero(g["codes"] != o["codes"]) == 0


@pytest.mark.parametrize("layout", ["row", "col"])
def test_mx_quantize_wgrad_operands_full(nv, layout):
    """The full 8192x5120 Wgrad operands (dY Laplace, X normal), whole tensors."""
    dy, xx = syn.wgrad_8192x5120()
    for name, bits in (("dY", dy), ("X", xx)):
        say("mx quantize full", name, layout)
        q = nv.mx_quantize(dev_bf16(bits), layout)
        torch.cuda.synchronize()
        g, o = gpu_mx(q), oracle.mx_quantize(bits, layout)
        assert np.count_nonzero(g["scales"] != o["scales"]) == 0, name
        assert np.count_nonzero(g["codes"] != o["codes"]) == 0, name


def test_mx_dequantize_bit_exact(nv):
    bits = mixed_bits(96, 320, seed=9)
    say("mx dequantize")
    q = nv.mx_quantize(dev_bf16(bits), "row")
    y = torch.empty((96, 320), dtype=torch.float32, device="cuda")
    nv.mxfp4_dequantize(q, y)
    torch.cuda.synchronize()
    want = oracle.mx_decode(gpu_mx(q)).astype(np.float32)
    assert np.array_equal(host(y).view(np.uint32), want.view(np.uint32))


GCASES = [  # (M, N, K, out dtype)
    (32, 32, 32, "f32"),
    (48, 80, 96, "f32"),
    (208, 144, 224, "bf16"),
    (256, 256, 128, "f32"),        # fast path, one K-tile
    (512, 768, 384, "bf16"),       # fast path
    (768, 512, 1280, "f32"),       # fast path, ten K-tiles
    (304, 272, 1056, "f32"),       # direct kernel, ragged in M, N and K % 64 == 32
]


@pytest.mark.parametrize("case", GCASES, ids=lambda c: "x".join(map(str, c[:3])) + "-" + c[3])
def test_mx_gemm_small(nv, case):
    M, N, K, dt = case
    say("mx gemm", case)
    a_bits = syn.activation(M, K, seed=M + K)
    b_bits = syn.normal(N, K, seed=N + 3 * K, std=0.02)
    qa, qb = nv.mx_quantize(dev_bf16(a_bits), "row"), nv.mx_quantize(dev_bf16(b_bits), "row")
    c = host(nv.mx_gemm(qa, qb, dt).float())
    torch.cuda.synchronize()
    ga, gb = gpu_mx(qa), gpu_mx(qb)
    ref = oracle.round_output(oracle.mx_gemm_f64(ga, gb), dt)
    err = rel_frobenius(c, ref)
    assert err <= (1e-5 if dt == "f32" else 1e-3), err


def test_mx_fast_and_direct_kernels_agree(nv, monkeypatch):
    M, N, K = 512, 512, 1024
    say("mx gemm fast vs direct")
    qa = nv.mx_quantize(dev_bf16(syn.activation(M, K, seed=11)), "row")
    qb = nv.mx_quantize(dev_bf16(syn.normal(N, K, seed=12, std=0.02)), "row")
    c_fast = host(nv.mx_gemm(qa, qb, "f32"))
    torch.cuda.synchronize()
    monkeypatch.setenv("NVFP4_GEMM_GENERIC", "1")
    c_gen = host(nv.mx_gemm(qa, qb, "f32"))
    torch.cuda.synchronize()
    assert rel_frobenius(c_fast, c_gen) <= 1e-6


def test_mx_wgrad_8192x5120_sampled(nv):
    """dW = dY^T X with both operands MXFP4-quantised along tokens (the
    transposed, column layout), C fp32 5120x5120, 256 sampled rows."""
    dy, xx = syn.wgrad_8192x5120()
    say("mx wgrad quantize")
    qa, qb = nv.mx_quantize(dev_bf16(dy), "col"), nv.mx_quantize(dev_bf16(xx), "col")
    say("mx wgrad gemm")
    c = nv.mx_gemm(qa, qb, "f32")
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(7).choice(5120, size=256, replace=False))
    ref = oracle.round_output(oracle.mx_gemm_f64(gpu_mx(qa), gpu_mx(qb), rows_a=rows), "f32")
    err = rel_frobenius(host(c)[rows], ref)
    say("mx wgrad sampled rel err", err)
    assert err <= 1e-5


def test_mx_gemm_fast_path_at_its_offset_limit(nv):
    """The largest operands the MX 256x256 fast path takes: M = N = 4096 and
    K = 2096000 (M * K/2 + K just under 2^32), so its 32-bit transfer offsets
    reach their top range.  A 16x16 sample of C over the first and last rows
    and columns against the oracle on the GPU's own operand rows."""
    M = N = 4096
    K = 2096000
    assert M * (K // 2) + K < 2 ** 32
    if torch.cuda.get_device_properties(0).total_memory < 80 * 2**30:
        pytest.skip("needs about 45 GB of device memory")
    say("mx offset limit: draw and quantise", M, N, K)
    xa = syn.normal_device(M, K, seed=83)
    qa = nv.mx_quantize(xa, "row")
    del xa
    xb = syn.normal_device(N, K, seed=84)
    qb = nv.mx_quantize(xb, "row")
    del xb
    torch.cuda.empty_cache()
    say("mx offset limit: gemm")
    c = nv.mx_gemm(qa, qb, "f32")
    torch.cuda.synchronize()
    rows = np.array([0, 1, 255, 256, 1023, 2047, 2048, 3071, 3839, 3840, 4000, 4090, 4092, 4093, 4094, 4095])
    cols = np.array([0, 7, 128, 255, 256, 1000, 2047, 2049, 3000, 3583, 3584, 3900, 4064, 4093, 4094, 4095])

    def sub(q, idx):
        t = torch.as_tensor(idx, device="cuda")
        return dict(codes=host(q.codes[t]), scales=host(q.scales[t]), rows=len(idx), cols=K)

    say("mx offset limit: oracle sample")
    ref = oracle.round_output(oracle.mx_gemm_f64(sub(qa, rows), sub(qb, cols)), "f32")
    got = host(c)[np.ix_(rows, cols)]
    del qa, qb, c
    torch.cuda.empty_cache()
    err = rel_frobenius(got, ref)
    say("mx offset limit rel err", err)
    assert err <= 1e-5
