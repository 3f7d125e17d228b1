"""GPU parity of the NVFP4 GEMM against the oracle's binary64 GEMM on the same
(GPU-quantised) operands: relative Frobenius error at most 1e-3 -- for fp32
outputs the observed error is at the level of fp32 accumulation.  The operands
are first checked bit-exact against the oracle's quantisation, so the GEMM is
compared in isolation.  The Wgrad case is the 5120x5120x8192 weight-gradient
GEMM of the 5120-hidden model (NVFP4 pretraining news page, zubnet.ai,
paragraph 1), compared on sampled output rows.
"""
import numpy as np
import pytest

import oracle
from nvfp4_bit_quantization_amd import synthetic as syn

from gpu_util import assert_bit_exact, assert_rht_tolerance, dev_bf16, gpu_q_as_dict, host, rel_frobenius, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def nv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import nvfp4_bit_quantization_amd as nv
    nv.lib()
    return nv


def quant(nv, bits, layout, rounding="rtn", rht=False, sr_seed=0, rht_seed=0):
    x = dev_bf16(bits)
    q = nv.quantize(x, [nv.QuantSpec.of(layout, rounding, rht, sr_seed, rht_seed)])[0]
    return q


CASES = [  # (M, N, K, a layout, b layout, out dtype)
    (16, 16, 16, "row", "row", "f32"),
    (48, 80, 112, "row", "row", "f32"),
    (48, 80, 112, "row", "2d", "bf16"),
    (256, 256, 64, "row", "row", "f32"),
    (304, 272, 576, "2d", "row", "f32"),
    (512, 384, 1024, "row", "2d", "bf16"),
    (272, 528, 2048, "row", "row", "f32"),
    # shapes on the 256x256x128 fast path
    (256, 256, 128, "row", "row", "f32"),
    (512, 768, 384, "row", "2d", "bf16"),
    (768, 512, 1280, "2d", "row", "f32"),
    (1024, 1024, 2048, "col", "col", "f32"),
    # both operands with 16x16 (weight) scales, fast path and direct kernel
    (512, 512, 1024, "2d", "2d", "bf16"),
    (304, 272, 576, "2d", "2d", "f32"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c[:3])) + "-" + "-".join(c[3:]))
def test_gemm_small(nv, case):
    M, N, K, la, lb, dt = case
    say("gemm", case)
    a_bits = syn.activation(M, K, seed=M + K)
    b_bits = syn.normal(N, K, seed=N + 3 * K, std=0.02)
    qa, qb = quant(nv, a_bits, la), quant(nv, b_bits, lb)
    c = host(nv.gemm(qa, qb, dt).float())
    torch.cuda.synchronize()
    ga, gb = gpu_q_as_dict(qa), gpu_q_as_dict(qb)
    assert_bit_exact(ga, oracle.quantize(a_bits, la), "A")
    assert_bit_exact(gb, oracle.quantize(b_bits, lb), "B")
    ref = oracle.round_output(oracle.gemm_f64(ga, gb), dt)
    err = rel_frobenius(c, ref)
    assert err <= 1e-3, err
    if dt == "f32":
        assert err <= 1e-5, err  # fp32 accumulation of exact products


def test_fast_and_generic_kernels_agree(nv, monkeypatch):
    """The 256x256x128 fast path and the generic kernel compute the same sums."""
    M, N, K = 512, 512, 1024
    say("gemm fast vs generic")
    qa = quant(nv, syn.activation(M, K, seed=11), "row")
    qb = quant(nv, syn.normal(N, K, seed=12, std=0.02), "2d")
    c_fast = host(nv.gemm(qa, qb, "f32"))
    torch.cuda.synchronize()
    monkeypatch.setenv("NVFP4_GEMM_GENERIC", "1")
    c_gen = host(nv.gemm(qa, qb, "f32"))
    torch.cuda.synchronize()
    assert rel_frobenius(c_fast, c_gen) <= 1e-6


def test_gemm_ldc_and_zero_operand(nv):
    M, N, K = 64, 48, 96
    say("gemm ldc")
    qa = quant(nv, syn.activation(M, K, seed=1), "row")
    qb = quant(nv, np.zeros((N, K), np.uint16), "row")  # S = 1, all-zero codes
    c = torch.full((M, 64), 3.0, dtype=torch.float32, device="cuda")
    nv.nvfp4_gemm(qa, qb, c[:, :N])
    torch.cuda.synchronize()
    ch = host(c)
    assert np.all(ch[:, :N] == 0.0) and np.all(ch[:, N:] == 3.0)


def test_wgrad_8192x5120_sampled(nv):
    """dW = dY^T X: A = column-quantised dY (RHT + SR), B = column-quantised X
    (RHT + RTN), both 5120 x 8192 stored; C fp32 5120x5120 (with a workspace:
    the stream-K launch the benchmark times).  256 sampled rows of C against
    the oracle on the GPU's own operands."""
    dy, xx = syn.wgrad_8192x5120()
    say("wgrad quantize")
    qa = quant(nv, dy, "col", "sr", True, 1234, 1234)
    qb = quant(nv, xx, "col", "rtn", True, 0, 1234)
    say("wgrad gemm")
    c = nv.gemm(qa, qb, "f32", workspace=nv.new_gemm_workspace())
    torch.cuda.synchronize()
    ga, gb = gpu_q_as_dict(qa), gpu_q_as_dict(qb)
    rows = np.sort(np.random.default_rng(7).choice(5120, size=256, replace=False))
    ref = oracle.round_output(oracle.gemm_f64(ga, gb, rows_a=rows), "f32")
    got = host(c)[rows]
    err = rel_frobenius(got, ref)
    say("wgrad sampled rel err", err)
    assert err <= 1e-3
    # the operands themselves against the oracle (RHT tolerance)
    say("wgrad operand parity")
    assert_rht_tolerance(ga, oracle.quantize(dy, "col", "sr", True, 1234, 1234), "dY")
    assert_rht_tolerance(gb, oracle.quantize(xx, "col", "rtn", True, 0, 1234), "X")


# ------------------------------------------------------------------ stream-K
@pytest.fixture(scope="module")
def gws(nv):
    return nv.new_gemm_workspace()


def _random_operands(M, N, K, seed):
    g = torch.Generator(device="cpu").manual_seed(seed)
    def q(rows):
        codes = torch.randint(0, 256, (rows, K // 2), dtype=torch.uint8, generator=g).cuda()
        scales = torch.randint(0x20, 0x50, (rows, K // 16), dtype=torch.uint8, generator=g).cuda()
        S = torch.tensor([0.75], dtype=torch.float32, device="cuda")
        amax = torch.tensor([1.0], dtype=torch.float32, device="cuda")
        return codes, scales, S, amax
    import nvfp4_bit_quantization_amd as nvm
    a, b = q(M), q(N)
    qa = nvm.QTensor(a[0], a[1], a[2], a[3], M, K, nvm.SCALE_1D16)
    qb = nvm.QTensor(b[0], b[1], b[2], b[3], N, K, nvm.SCALE_1D16)
    return qa, qb


@pytest.mark.parametrize("shape", [(4352, 8448, 1024), (5376, 6400, 512), (8192, 5120, 2048), (5376, 6400, 128)],
                         ids=lambda s: "x".join(map(str, s)))
def test_streamk_matches_whole_tiles(nv, gws, shape, monkeypatch):
    """More than two rounds of tiles with an ill-filled last round (561, 525
    and 640 tiles on 256 compute units) take the stream-K path when a
    workspace is given: whole tiles for the full rounds, then the remaining
    K-tiles spread over every workgroup, split tiles' partial sums added in
    the workspace (up to several parts per tile, and workgroups with empty
    ranges when the remainder has fewer K-tiles than there are workgroups).
    The result equals the whole-tile path's up to fp32 reassociation, is the
    same bit for bit on every run, matches the oracle on sampled rows, and
    leaves the workspace's flag and error words at zero.  K = 128 (one K-tile)
    splits no tile."""
    M, N, K = shape
    qa, qb = _random_operands(M, N, K, seed=M + N + K)
    say("stream-K", shape)
    monkeypatch.delenv("NVFP4_GEMM_DATA_PARALLEL", raising=False)
    c1 = nv.gemm(qa, qb, "f32", workspace=gws)
    c2 = nv.gemm(qa, qb, "f32", workspace=gws)
    monkeypatch.setenv("NVFP4_GEMM_DATA_PARALLEL", "1")
    cd = nv.gemm(qa, qb, "f32", workspace=gws)
    torch.cuda.synchronize()
    assert torch.equal(c1.view(torch.int32), c2.view(torch.int32))
    rel = (torch.linalg.norm((c1 - cd).double()) / torch.linalg.norm(cd.double())).item()
    say("stream-K vs whole tiles rel", rel)
    assert rel < 1e-6
    words = host(gws[:4100].view(torch.int32))
    assert not words.any() and not nv.gemm_workspace_timed_out(gws)
    if K <= 1024:
        ga, gb = gpu_q_as_dict(qa), gpu_q_as_dict(qb)
        rows = np.sort(np.random.default_rng(M).choice(M, size=48, replace=False))
        ref = oracle.round_output(oracle.gemm_f64(ga, gb, rows_a=rows), "f32")
        err = rel_frobenius(host(c1)[rows], ref)
        say("stream-K vs oracle", err)
        assert err <= 1e-3


def test_gemm_fast_path_at_its_offset_limit(nv):
    """The largest operands the 256x256 fast path takes: M = N = 4096 and
    K = 2097024, so K/2 * 4096 = 2^32 - 262144 bytes of codes per operand and
    the 32-bit transfer offsets reach their top range (the transfers add them,
    zero-extended, to a 64-bit base).  A 16x16 sample of C, spread over the
    first and last rows and columns, against the oracle's binary64 GEMM on the
    GPU's own operand rows."""
    M = N = 4096
    K = 2097024
    if torch.cuda.get_device_properties(0).total_memory < 80 * 2**30:
        pytest.skip("needs about 45 GB of device memory")
    say("offset limit: draw and quantise", M, N, K)
    xa = syn.normal_device(M, K, seed=81)
    qa = nv.quantize(xa, [nv.QuantSpec.of("row")])[0]
    del xa
    xb = syn.normal_device(N, K, seed=82)
    qb = nv.quantize(xb, [nv.QuantSpec.of("row")])[0]
    del xb
    torch.cuda.empty_cache()
    say("offset limit: gemm")
    c = nv.gemm(qa, qb, "f32")
    torch.cuda.synchronize()
    rows = np.array([0, 1, 255, 256, 1023, 2047, 2048, 3071, 3839, 3840, 4000, 4090, 4092, 4093, 4094, 4095])
    cols = np.array([0, 7, 128, 255, 256, 1000, 2047, 2049, 3000, 3583, 3584, 3900, 4064, 4093, 4094, 4095])

    def sub(q, idx):
        return dict(codes=host(q.codes[torch.as_tensor(idx, device="cuda")]),
                    scales=host(q.scales[torch.as_tensor(idx, device="cuda")]),
                    S=np.float32(host(q.global_scale)[0]), rows=len(idx), cols=K, scale_kind=q.scale_kind)

    say("offset limit: oracle sample")
    ref = oracle.round_output(oracle.gemm_f64(sub(qa, rows), sub(qb, cols)), "f32")
    got = host(c)[np.ix_(rows, cols)]
    del qa, qb, c
    torch.cuda.empty_cache()
    err = rel_frobenius(got, ref)
    say("offset limit rel err", err)
    assert err <= 1e-3


# ------------------------------------------------------- extreme tensor scales
# The per-tensor scales S_A = 2688 / amax_A and S_B = 2688 / amax_B enter C only
# through the division by S_A S_B (page paragraph 2: the FP32 per-tensor scale
# over the E4M3 block scales).  That product overflows binary32 once
# amax_A amax_B < 2688^2 / FLT_MAX (about 2e-32), e.g. two gradient-like tensors
# with maxima near 1e-16, although C itself (about K amax_A amax_B) is an
# ordinary binary32 number; and it underflows once amax_A amax_B exceeds about
# 5e51, where every non-zero C overflows binary32 but the zero entries must stay
# zero.
EXTREME_SHAPES = [(256, 256, 512), (48, 80, 112)]  # fast path, direct kernel


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("shape", EXTREME_SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("stds", [(1e-17, 1e-17), (3e-20, 2e-15)], ids=["both-1e-17", "3e-20-and-2e-15"])
def test_gemm_tiny_tensor_maxima(nv, shape, dt, stds):
    M, N, K = shape
    say("gemm tiny maxima", shape, dt, stds)
    a_bits = syn.normal(M, K, seed=M + 5 * K, std=stds[0])
    b_bits = syn.normal(N, K, seed=N + 7 * K, std=stds[1])
    qa, qb = quant(nv, a_bits, "row"), quant(nv, b_bits, "row")
    c = host(nv.gemm(qa, qb, dt).float())
    torch.cuda.synchronize()
    ga, gb = gpu_q_as_dict(qa), gpu_q_as_dict(qb)
    assert_bit_exact(ga, oracle.quantize(a_bits, "row"), "A")
    assert_bit_exact(gb, oracle.quantize(b_bits, "row"), "B")
    # the case this test is about: S_A S_B is not a finite binary32
    with np.errstate(over="ignore"):
        assert not np.isfinite(np.float32(ga["S"]) * np.float32(gb["S"]))
    ref = oracle.round_output(oracle.gemm_f64(ga, gb), dt)
    assert np.all(np.isfinite(ref)) and np.count_nonzero(ref) > 0.9 * ref.size
    err = rel_frobenius(c, ref)
    say("rel err", err)
    assert err <= (1e-5 if dt == "f32" else 1e-3), err


def test_gemm_tiny_maxima_wgrad_operands(nv):
    """A Wgrad product of two gradient-sized tensors along tokens, both with
    the RHT (signs from seed 77), the first with stochastic rounding: maxima
    around 1e-17 and 1e-16."""
    tokens, h1, h2 = 512, 256, 256
    say("gemm tiny maxima, RHT operands")
    dy = syn.laplace(tokens, h1, seed=61, scale=2e-18)
    xx = syn.normal(tokens, h2, seed=62, std=3e-17)
    qa = quant(nv, dy, "col", "sr", True, 99, 77)
    qb = quant(nv, xx, "col", "rtn", True, 0, 77)
    c = host(nv.gemm(qa, qb, "f32"))
    torch.cuda.synchronize()
    ga, gb = gpu_q_as_dict(qa), gpu_q_as_dict(qb)
    assert_rht_tolerance(ga, oracle.quantize(dy, "col", "sr", True, 99, 77), "dY")
    assert_rht_tolerance(gb, oracle.quantize(xx, "col", "rtn", True, 0, 77), "X")
    with np.errstate(over="ignore"):
        assert not np.isfinite(np.float32(ga["S"]) * np.float32(gb["S"]))
    ref = oracle.round_output(oracle.gemm_f64(ga, gb), "f32")
    err = rel_frobenius(c, ref)
    say("rel err", err)
    assert err <= 1e-5, err


def _block_sparse_positive(rows, K, seed, std, shift):
    """|N(0, std)| values; row r keeps only its 16-wide k-block (r + shift) mod (K/16)."""
    bits = syn.normal(rows, K, seed=seed, std=std) & np.uint16(0x7FFF)
    blk = (np.arange(K)[None, :] // 16) == ((np.arange(rows)[:, None] + shift) % (K // 16))
    return np.where(blk, bits, np.uint16(0)).astype(np.uint16)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [(256, 256, 128), (48, 80, 112)], ids=lambda s: "x".join(map(str, s)))
def test_gemm_huge_tensor_maxima(nv, shape, dt):
    """Maxima near 1e26 on both operands: S_A S_B underflows binary32.  The
    operands are block-sparse and non-negative, so C is exactly zero wherever
    the rows' k-blocks differ and far beyond the binary32 range wherever they
    match: the oracle's once-rounded C is 0 or +inf, and the GPU must give the
    same (no NaN from 0 times an infinite factor)."""
    M, N, K = shape
    say("gemm huge maxima", shape, dt)
    a_bits = _block_sparse_positive(M, K, seed=M + K, std=1e26, shift=0)
    b_bits = _block_sparse_positive(N, K, seed=N + 3 * K, std=1e26, shift=1)
    qa, qb = quant(nv, a_bits, "row"), quant(nv, b_bits, "row")
    c = host(nv.gemm(qa, qb, dt).float())
    torch.cuda.synchronize()
    ga, gb = gpu_q_as_dict(qa), gpu_q_as_dict(qb)
    assert_bit_exact(ga, oracle.quantize(a_bits, "row"), "A")
    assert_bit_exact(gb, oracle.quantize(b_bits, "row"), "B")
    with np.errstate(under="ignore"):
        assert np.float32(ga["S"]) * np.float32(gb["S"]) == 0.0
    with np.errstate(over="ignore"):
        ref = oracle.round_output(oracle.gemm_f64(ga, gb), dt)
    assert np.count_nonzero(ref == 0) > 0 and np.count_nonzero(np.isinf(ref)) > 0
    assert not np.isnan(c).any()
    assert np.array_equal(c, ref), (np.count_nonzero(c != ref), c.size)
