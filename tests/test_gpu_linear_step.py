"""Stage-wise parity of a full linear-layer step (Fprop, Dgrad and Wgrad of
the up- and down-projection of a 5120 -> 20480 -> 5120 FFN) on the GPU.

The per-role recipe follows paragraph 2 of the NVFP4 pretraining news page
(zubnet.ai): activations 1D round-to-nearest, weights 2D (the transposed copy
serves Dgrad), gradients 1D with stochastic rounding, and the 16x16 RHT with
shared signs on both Wgrad inputs.  Hidden 5120 and FFN 20480 are the real
sizes; the step runs with 512 tokens and with the full 16384 (the shapes the
benchmark times).  Each quantisation is checked against the oracle on the
GPU's own bf16 input (bit-exact, or the RHT tolerance), each GEMM on 64
sampled output rows against the oracle's binary64 product of the GPU's
operands.
"""
import numpy as np
import pytest

import oracle
from nvfp4_bit_quantization_amd import synthetic as syn

from gpu_util import assert_bit_exact, assert_rht_tolerance, gpu_q_as_dict, host, rel_frobenius, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

HID, FFN = 5120, 20480


@pytest.fixture(scope="module")
def nv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import nvfp4_bit_quantization_amd as nv
    nv.lib()
    return nv


def bf16_bits(t):
    return host(t.contiguous().view(torch.int16)).view(np.uint16)


def check_quant(outs, bits, specs, what):
    for q, s in zip(outs, specs):
        o = oracle.quantize(bits, s[0], s[1], s[2], s[3], s[4])
        g = gpu_q_as_dict(q)
        if s[2]:
            assert_rht_tolerance(g, o, what + "-" + s[0])
        else:
            assert_bit_exact(g, o, what + "-" + s[0])


def check_gemm(qa, qb, c, what, dt):
    ga, gb = gpu_q_as_dict(qa), gpu_q_as_dict(qb)
    rows = np.sort(np.random.default_rng(sum(what.encode())).choice(qa.rows, size=64, replace=False))
    ref = oracle.round_output(oracle.gemm_f64(ga, gb, rows_a=rows), dt)
    got = host(c.float())[rows]
    err = rel_frobenius(got, ref)
    say(what, "rel err", err)
    assert err <= 1e-3, (what, err)


def run_step(nv, T, fused=False):
    """fused: the H and dH GEMMs produce the maxima of their outputs'
    quantisations (nvfp4_gemm_amax), which then skip their amax pass."""
    say("linear step", T, "tokens", "fused amax" if fused else "")
    d = syn.linear_step_16384(T, HID, FFN)
    dev = {k: torch.from_numpy(v.view(np.int16)).view(torch.bfloat16).cuda() for k, v in d.items()}
    S = nv.QuantSpec.of
    sX = [S("row"), S("col", "rtn", True, 0, 4321)]
    sW = [S("2d"), S("2d_t")]
    sdY = [S("row", "sr", False, 1234), S("col", "sr", True, 1235, 4321)]
    sdH = [S("row", "sr", False, 1236), S("col", "sr", True, 1237, 4321)]
    oX = [("row", "rtn", False, 0, 0), ("col", "rtn", True, 0, 4321)]
    oW = [("2d", "rtn", False, 0, 0), ("2d_t", "rtn", False, 0, 0)]
    odY = [("row", "sr", False, 1234, 0), ("col", "sr", True, 1235, 4321)]
    odH = [("row", "sr", False, 1236, 0), ("col", "sr", True, 1237, 4321)]

    say("forward")
    gws = nv.new_gemm_workspace()
    qX = nv.quantize(dev["X"], sX)
    qW1 = nv.quantize(dev["W1"], sW)
    if fused:
        H = torch.empty((T, FFN), dtype=torch.bfloat16, device="cuda")
        qH = [nv.empty_qtensor(T, FFN, nv.SCALE_1D16), nv.empty_qtensor(FFN, T, nv.SCALE_1D16, rht=1)]
        for q in qH:
            q.amax.zero_()
        nv.nvfp4_gemm_amax(qX[0], qW1[0], H, qH[0].amax, qH[1].amax, 4321, workspace=gws)
        sH = [S("row", amax_given=True), S("col", "rtn", True, 0, 4321, amax_given=True)]
        nv.nvfp4_quantize(H, sH, qH, nv.new_workspace())
    else:
        H = nv.gemm(qX[0], qW1[0], "bf16", workspace=gws)         # H = X W1^T   [T][FFN]
        qH = nv.quantize(H, sX)
    qW2 = nv.quantize(dev["W2"], sW)
    Y = nv.gemm(qH[0], qW2[0], "bf16", workspace=gws)             # Y = H W2^T   [T][HID]
    say("backward")
    qdY = nv.quantize(dev["dY"], sdY)
    if fused:
        dH = torch.empty((T, FFN), dtype=torch.bfloat16, device="cuda")
        qdH = [nv.empty_qtensor(T, FFN, nv.SCALE_1D16), nv.empty_qtensor(FFN, T, nv.SCALE_1D16, rht=1)]
        for q in qdH:
            q.amax.zero_()
        nv.nvfp4_gemm_amax(qdY[0], qW2[1], dH, qdH[0].amax, qdH[1].amax, 4321, workspace=gws)
        sdHf = [S("row", "sr", False, 1236, amax_given=True), S("col", "sr", True, 1237, 4321, amax_given=True)]
        nv.nvfp4_quantize(dH, sdHf, qdH, nv.new_workspace())
    else:
        dH = nv.gemm(qdY[0], qW2[1], "bf16", workspace=gws)       # dH = dY W2   [T][FFN]
        qdH = nv.quantize(dH, sdH)
    dX = nv.gemm(qdH[0], qW1[1], "bf16", workspace=gws)           # dX = dH W1   [T][HID]
    dW2 = nv.gemm(qdY[1], qH[1], "f32", workspace=gws)            # dW2 = dY^T H [HID][FFN]
    dW1 = nv.gemm(qdH[1], qX[1], "f32", workspace=gws)            # dW1 = dH^T X [FFN][HID]
    torch.cuda.synchronize()

    say("quantisation parity")
    check_quant(qX, d["X"], oX, "X")
    check_quant(qW1, d["W1"], oW, "W1")
    check_quant(qW2, d["W2"], oW, "W2")
    check_quant(qdY, d["dY"], odY, "dY")
    check_quant(qH, bf16_bits(H), oX, "H")
    check_quant(qdH, bf16_bits(dH), odH, "dH")

    say("GEMM parity")
    check_gemm(qX[0], qW1[0], H, "fprop-H", "bf16")
    check_gemm(qH[0], qW2[0], Y, "fprop-Y", "bf16")
    check_gemm(qdY[0], qW2[1], dH, "dgrad-dH", "bf16")
    check_gemm(qdH[0], qW1[1], dX, "dgrad-dX", "bf16")
    check_gemm(qdY[1], qH[1], dW2, "wgrad-dW2", "f32")
    check_gemm(qdH[1], qX[1], dW1, "wgrad-dW1", "f32")

    # the RHT-domain Wgrad estimates the plain product: compare with the
    # binary64 dY^T H of the bf16 tensors on a few rows
    dy = syn.bf16_bits_to_f32(d["dY"]).astype(np.float64)
    h = syn.bf16_bits_to_f32(bf16_bits(H)).astype(np.float64)
    rows = np.arange(0, HID, 640)
    ref = dy[:, rows].T @ h
    rel = rel_frobenius(host(dW2)[rows], ref)
    say("dW2 vs unquantised product", rel)
    assert rel < 0.2


def test_linear_step_stagewise(nv):
    run_step(nv, 512)


def test_linear_step_16384_full(nv):
    run_step(nv, 16384)


def test_linear_step_fused_amax(nv):
    run_step(nv, 512, fused=True)
