"""Tensor-level ablations of the recipe's techniques on synthetic data, run
through the HIP path.

The NVFP4 pretraining news page (zubnet.ai), paragraph 2, motivates three of
its techniques by what they do to the quantised tensors: random Hadamard
transforms on the Wgrad inputs (outliers), stochastic rounding on gradients
(bias), and 16x16 2D weight scaling (the forward and backward passes see the
same quantised weight).  These tests measure each effect on seeded synthetic
tensors, print the numbers, and assert what the arithmetic guarantees:

- stochastic rounding is unbiased: averaged over 1000 seeds the dequantised
  values converge to the input at the 1/sqrt(N) rate, except on elements the
  method saturates (scaled values above 6 when the E4M3 block scale rounds
  down), where the clamp is the bias;
- 2D weight scaling gives bit-identical forward and backward weights, 1D
  row/column scaling does not;
- NVFP4 quantises activation- and gradient-like tensors, and their Wgrad
  product, more accurately than MXFP4 (paragraph 3's comparison);
- the RHT-domain Wgrad estimates the plain product as well as the direct one
  (on i.i.d. synthetic inputs the RHT neither helps nor hurts much: the
  benefit the page reports is on real training tensors, which these inputs do
  not model; the numbers are printed, not asserted beyond that).
"""
import numpy as np
import pytest

import oracle
from nvfp4_bit_quantization_amd import synthetic as syn

from gpu_util import dev_bf16, host, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def nv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import nvfp4_bit_quantization_amd as nv
    nv.lib()
    return nv


def test_sr_unbiased_over_seeds(nv):
    """1000 stochastic-rounding draws of a 4096x512 N(0,1) tensor: the mean
    dequantised value's error on unsaturated elements shrinks like
    1/sqrt(1000) of one draw's, far below the round-to-nearest error."""
    bits = syn.normal(4096, 512, 21)
    x = dev_bf16(bits)
    xf = x.float()
    ws = nv.new_workspace()
    S = nv.QuantSpec.of
    n = 1000
    acc = torch.zeros_like(xf)
    for s in range(n):
        acc += nv.dequantize(nv.quantize(x, [S("row", "sr", False, 1000 + s)], workspace=ws)[0])
    mean_sr = acc / n
    one = nv.dequantize(nv.quantize(x, [S("row", "sr", False, 5)], workspace=ws)[0])
    q_rtn = nv.quantize(x, [S("row")], workspace=ws)[0]
    rtn = nv.dequantize(q_rtn)
    # scaled values y = x * S / s_b (the same for every seed): saturated where |y| > 6
    sb = oracle.e4m3_value_array(host(q_rtn.scales).reshape(-1)).reshape(4096, 32)
    Sg = float(host(q_rtn.global_scale)[0])
    y = np.abs(host(xf)) * Sg / np.repeat(sb, 16, axis=1)
    sat = y > 6.0
    e_sr, e_one, e_rtn = host(mean_sr - xf), host(one - xf), host(rtn - xf)
    ok = ~sat
    rms = lambda e: float(np.sqrt(np.mean(e.astype(np.float64) ** 2)))
    say("SR mean of %d draws: rms err %.3e unsaturated, %.3e saturated (%d elements); one draw %.3e; RTN %.3e"
        % (n, rms(e_sr[ok]), rms(e_sr[sat]) if sat.any() else 0.0, int(sat.sum()), rms(e_one[ok]), rms(e_rtn[ok])))
    assert rms(e_sr[ok]) < 1.5 * rms(e_one[ok]) / np.sqrt(n)
    assert rms(e_sr[ok]) < 0.1 * rms(e_rtn[ok])
    # the global mean of the unsaturated errors is zero within its noise
    m = float(np.mean(e_sr[ok].astype(np.float64)))
    assert abs(m) < 5 * rms(e_sr[ok]) / np.sqrt(ok.sum())


def test_2d_weight_scaling_forward_backward_consistent(nv):
    """A 1024x4096 N(0, 0.02) weight: 16x16 2D scaling gives the forward
    (2D) and backward (2D_T, transposed) operands the same dequantised
    values bit for bit; 1D row blocks (forward) and column blocks (backward)
    disagree by about the quantisation error itself."""
    w = dev_bf16(syn.normal(1024, 4096, 31, std=0.02))
    wf = w.float()
    S = nv.QuantSpec.of
    qr, qc = nv.quantize(w, [S("row"), S("col")])
    q2, q2t = nv.quantize(w, [S("2d"), S("2d_t")])
    d_r, d_c = nv.dequantize(qr), nv.dequantize(qc).t()
    d_2, d_2t = nv.dequantize(q2), nv.dequantize(q2t).t()
    rel = lambda a, b: float((a - b).norm() / wf.norm())
    say("1D fwd vs bwd rel diff %.4f (errors %.4f / %.4f); 2D fwd vs bwd max |diff| %.1e (error %.4f)"
        % (rel(d_r, d_c), rel(d_r, wf), rel(d_c, wf), float((d_2 - d_2t).abs().max()), rel(d_2, wf)))
    assert torch.equal(d_2.contiguous().view(torch.int32), d_2t.contiguous().view(torch.int32))
    assert rel(d_r, d_c) > 0.01


@pytest.mark.parametrize("case", ["laplace_dY_normal_X", "laplace_dY_activation_X"])
def test_rht_wgrad_error(nv, case):
    """Wgrad dW = dY^T X (8192 tokens, 2048 channels) from NVFP4 operands
    with and without the 16x16 RHT along tokens, against the binary64
    product of the bf16 inputs.  Both estimates are within the error the
    4-bit operands allow, and within 25 % of each other."""
    T, H = 8192, 2048
    dy_bits = syn.laplace(T, H, 11, 1e-3)
    x_bits = syn.normal(T, H, 12) if case == "laplace_dY_normal_X" else syn.activation(T, H, 14)
    dy, x = dev_bf16(dy_bits), dev_bf16(x_bits)
    ref = syn.bf16_bits_to_f32(dy_bits).astype(np.float64).T @ syn.bf16_bits_to_f32(x_bits).astype(np.float64)
    S = nv.QuantSpec.of
    gws = nv.new_gemm_workspace()
    errs = {}
    for rht in (True, False):
        qa = nv.quantize(dy, [S("col", "sr", rht, 77, 1234)])[0]
        qb = nv.quantize(x, [S("col", "rtn", rht, 0, 1234)])[0]
        c = host(nv.gemm(qa, qb, "f32", workspace=gws)).astype(np.float64)
        errs[rht] = float(np.linalg.norm(c - ref) / np.linalg.norm(ref))
    say(case, "Wgrad rel error: RHT %.4f, no RHT %.4f" % (errs[True], errs[False]))
    assert 0.05 < errs[True] < 0.3 and 0.05 < errs[False] < 0.3
    assert 0.8 < errs[True] / errs[False] < 1.25


@pytest.mark.parametrize("case", ["outlier_tokens_x30", "sparse_outliers_x3e4"])
def test_rht_wgrad_error_with_structured_outliers(nv, case):
    """The regimes the RHT (page, paragraph 2: on the weight-gradient inputs
    only) is meant for: dY with outliers.  dW = dY^T X over 8192 tokens, X
    N(0,1) with 1024 channels, against the binary64 product of the bf16 inputs.
    * outlier_tokens_x30: in every 16-token group one token, across all 2048
      channels, is 30 times larger.  The outlier tokens dominate dW, and
      without the RHT each sits at its block's maximum with near-FP8
      precision; spread over 16 tokens by the RHT it gets 4-bit precision, so
      the RHT does not lower the error here (recorded, not asserted better).
    * sparse_outliers_x3e4: 256 entries 3e4 times the bulk.  The tensor
      maximum then pushes almost every ordinary block's E4M3 scale into the
      subnormal range (fewer scale bits); the RHT spreads each outlier over
      16 tokens, the maximum drops about 4 times and the scales move back
      into the normal range.  The Wgrad error is then no worse with the RHT
      (the oracle gives 0.1055 against 0.1078 on these inputs)."""
    T, H, HX = 8192, 2048, 1024
    if case == "outlier_tokens_x30":
        dy_bits = syn.token_outlier_gradient(T, H, 21, 1e-3, 30.0, 1)
    else:
        dy_bits = syn.sparse_outlier_gradient(T, H, 22, 1e-3, 3e4, 256)
    x_bits = syn.normal(T, HX, 23)
    dy, x = dev_bf16(dy_bits), dev_bf16(x_bits)
    ref = syn.bf16_bits_to_f32(dy_bits).astype(np.float64).T @ syn.bf16_bits_to_f32(x_bits).astype(np.float64)
    S = nv.QuantSpec.of
    gws = nv.new_gemm_workspace()
    errs, subn = {}, {}
    for rht in (True, False):
        qa = nv.quantize(dy, [S("col", "sr", rht, 77, 1234)])[0]
        qb = nv.quantize(x, [S("col", "rtn", rht, 0, 1234)])[0]
        c = host(nv.gemm(qa, qb, "f32", workspace=gws)).astype(np.float64)
        errs[rht] = float(np.linalg.norm(c - ref) / np.linalg.norm(ref))
        sc = host(qa.scales)
        subn[rht] = float(np.mean((sc > 0) & (sc < 8)))  # E4M3 subnormal block scales of dY
    say(case, "Wgrad rel error: RHT %.4f, no RHT %.4f; dY subnormal block scales: RHT %.3f, no RHT %.3f"
        % (errs[True], errs[False], subn[True], subn[False]))
    assert 0.03 < errs[True] < 0.3 and 0.03 < errs[False] < 0.3
    if case == "sparse_outliers_x3e4":
        assert subn[False] > 0.5 and subn[True] < subn[False] / 10
        assert errs[True] < 1.01 * errs[False]


def test_nvfp4_against_mxfp4(nv):
    """Paragraph 3 of the page sets NVFP4 against MXFP4 (MXFP4's loss ends
    2.5 % above BF16's, NVFP4's 1.5 %).  At tensor level the difference is the block: 16 elements
    with an E4M3 scale (plus the FP32 per-tensor scale) against 32 elements
    with a power-of-two E8M0 scale, whose block maximum lands anywhere in
    [4, 8) before rounding -- so MXFP4 both rounds its largest elements more
    coarsely and clamps the ones above 6.  Measured here: the dequantisation
    error of activation-like and gradient-like tensors, and the error of the
    Wgrad product dY^T X, in both formats (round-to-nearest, no RHT, column
    layout along tokens); NVFP4 must be the more accurate in every case."""
    S = nv.QuantSpec.of
    T, H = 4096, 1024
    xa = dev_bf16(syn.activation(T, H, seed=31))
    dy = dev_bf16(syn.laplace(T, H, seed=32, scale=1e-3))
    res = {}
    for name, x in (("activation", xa), ("gradient", dy)):
        xf = x.float()
        q = nv.quantize(x, [S("row")])[0]
        e_nv = (torch.linalg.norm(nv.dequantize(q) - xf) / torch.linalg.norm(xf)).item()
        m = nv.mx_quantize(x, "row")
        ym = torch.empty((T, H), dtype=torch.float32, device="cuda")
        nv.mxfp4_dequantize(m, ym)
        e_mx = (torch.linalg.norm(ym - xf) / torch.linalg.norm(xf)).item()
        res[name] = (e_nv, e_mx)
        say("dequantisation error", name, "NVFP4 %.4f  MXFP4 %.4f" % (e_nv, e_mx))
        assert e_nv < e_mx
    # Wgrad dW = dY^T X over the 4096 tokens (both operands quantised along tokens)
    ref = dy.float().t().contiguous() @ xa.float()
    qa, qb = nv.quantize(dy, [S("col")])[0], nv.quantize(xa, [S("col")])[0]
    c_nv = nv.gemm(qa, qb, "f32")
    c_mx = nv.mx_gemm(nv.mx_quantize(dy, "col"), nv.mx_quantize(xa, "col"), "f32")
    e_nv = (torch.linalg.norm(c_nv - ref) / torch.linalg.norm(ref)).item()
    e_mx = (torch.linalg.norm(c_mx - ref) / torch.linalg.norm(ref)).item()
    say("Wgrad error", "NVFP4 %.4f  MXFP4 %.4f" % (e_nv, e_mx))
    assert e_nv < e_mx
