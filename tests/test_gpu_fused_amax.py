"""Producer-fused per-tensor maxima (nvfp4_gemm_amax) and quantisation with
a given maximum (NVFP4_AMAX_GIVEN).

The per-tensor amax is the one global reduction of the recipe on the NVFP4
news page (zubnet.ai, paragraph 2: the FP32 per-tensor scale); when the tensor
is a GEMM output (H and dH of the linear step) the GEMM's epilogue can take it
from the outputs in registers, and the quantiser skips its amax pass.  The
plain maximum must equal max |C| of the stored bf16 output exactly; the
RHT-domain maximum (16x16 transform of every 16-row group, the amax of C's
column quantisation with the RHT) must agree with the oracle's exact one within
2^-20 relative, the tolerance of the RHT paths.  Shapes cover the direct
kernel, the 256x256 fast path and a stream-K launch."""
import numpy as np
import pytest

import oracle
from nvfp4_bit_quantization_amd import synthetic as syn

from gpu_util import assert_bit_exact, assert_rht_tolerance, dev_bf16, gpu_q_as_dict, host, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

SEED = 4321


@pytest.fixture(scope="module")
def nv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import nvfp4_bit_quantization_amd as nv
    nv.lib()
    return nv


def bf16_bits(t):
    return host(t.contiguous().view(torch.int16)).view(np.uint16)


CASES = [(48, 80, 112, False), (512, 768, 384, False), (4352, 8448, 1024, True)]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c[:3])) + ("-streamk" if c[3] else ""))
def test_gemm_amax_matches_definitions(nv, case):
    M, N, K, sk = case
    say("gemm amax", case)
    S = nv.QuantSpec.of
    qa = nv.quantize(dev_bf16(syn.activation(M, K, seed=M + K)), [S("row")])[0]
    qb = nv.quantize(dev_bf16(syn.normal(N, K, seed=N + K, std=0.02)), [S("row")])[0]
    ws = nv.new_gemm_workspace() if sk else None
    c = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    am = torch.zeros(2, dtype=torch.float32, device="cuda")
    nv.nvfp4_gemm_amax(qa, qb, c, am[0:1], am[1:2], SEED, workspace=ws)
    c_ref = nv.gemm(qa, qb, "bf16", workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(c.view(torch.int16), c_ref.view(torch.int16))  # the output itself is unchanged
    cb = bf16_bits(c)
    got_plain, got_rht = host(am)
    want_plain = np.abs(oracle.bf16_bits_to_f32(cb)).max()
    assert np.float32(got_plain).view(np.uint32) == np.float32(want_plain).view(np.uint32)
    o = oracle.quantize(cb, "col", "rtn", True, 0, SEED)  # amax of C's column quantisation with the RHT
    say("rht amax fused / oracle", got_rht, o["amax"])
    assert abs(float(got_rht) - float(o["amax"])) <= 2.0 ** -20 * float(o["amax"])
    # the GPU's own amax pass over C agrees as well
    g = gpu_q_as_dict(nv.quantize(c, [S("col", "rtn", True, 0, SEED)])[0])
    assert abs(float(got_rht) - float(g["amax"])) <= 2.0 ** -20 * float(g["amax"])
    if sk:
        assert not nv.gemm_workspace_timed_out(ws)


def test_gemm_amax_keeps_a_larger_value(nv):
    """The maxima are atomic maxima: a larger initial value survives, and a
    NULL target is skipped."""
    S = nv.QuantSpec.of
    qa = nv.quantize(dev_bf16(syn.activation(256, 256, seed=1)), [S("row")])[0]
    qb = nv.quantize(dev_bf16(syn.normal(256, 256, seed=2, std=0.02)), [S("row")])[0]
    c = torch.empty((256, 256), dtype=torch.bfloat16, device="cuda")
    am = torch.full((1,), 1.0e30, dtype=torch.float32, device="cuda")
    nv.nvfp4_gemm_amax(qa, qb, c, am, None, SEED)
    torch.cuda.synchronize()
    assert float(host(am)[0]) == np.float32(1.0e30)


def test_2d_pair_with_given_amax(nv):
    """The 2D + 2D_T pair computes each code once only when both outputs take
    their maximum from the same source; with a given maximum on one or both
    outputs the library runs the general kernel instead.  Both routes give the
    oracle's outputs bit for bit."""
    bits = syn.normal(272, 528, seed=78, std=0.02)
    o2, o2t = oracle.quantize(bits, "2d"), oracle.quantize(bits, "2d_t")
    x = dev_bf16(bits)
    S = nv.QuantSpec.of
    for given in ((False, False), (True, True), (True, False), (False, True)):
        say("2d pair, given amax =", given)
        specs = [S("2d", amax_given=given[0]), S("2d_t", amax_given=given[1])]
        outs = [nv.empty_qtensor(272, 528, nv.SCALE_2D16), nv.empty_qtensor(528, 272, nv.SCALE_2D16)]
        for q, g in zip(outs, given):
            q.amax.fill_(float(o2["amax"]) if g else -1.0)  # ignored when not given
        nv.nvfp4_quantize(x, specs, outs, nv.new_workspace())
        torch.cuda.synchronize()
        assert_bit_exact(gpu_q_as_dict(outs[0]), o2, "2d")
        assert_bit_exact(gpu_q_as_dict(outs[1]), o2t, "2d_t")


def test_quantize_with_given_amax(nv):
    """Given the oracle's maxima, the quantiser reproduces the oracle: the row
    output bit for bit, the RHT column output within the RHT tolerance, S
    exactly; also with one maximum given and the other from the amax pass."""
    bits = syn.activation(256, 512, seed=77)
    x = dev_bf16(bits)
    o_row = oracle.quantize(bits, "row")
    o_col = oracle.quantize(bits, "col", "rtn", True, 0, SEED)
    S = nv.QuantSpec.of
    for both in (True, False):
        say("given amax, both =", both)
        specs = [S("row", amax_given=True), S("col", "rtn", True, 0, SEED, amax_given=both)]
        outs = [nv.empty_qtensor(256, 512, nv.SCALE_1D16), nv.empty_qtensor(512, 256, nv.SCALE_1D16, rht=1)]
        outs[0].amax.fill_(float(o_row["amax"]))
        outs[1].amax.fill_(float(o_col["amax"]) if both else -1.0)  # ignored when not given
        nv.nvfp4_quantize(x, specs, outs, nv.new_workspace())
        torch.cuda.synchronize()
        g0, g1 = gpu_q_as_dict(outs[0]), gpu_q_as_dict(outs[1])
        assert_bit_exact(g0, o_row, "row")
        assert_rht_tolerance(g1, o_col, "col-rht")
        if both:
            assert np.float32(g1["S"]).view(np.uint32) == np.float32(o_col["S"]).view(np.uint32)
