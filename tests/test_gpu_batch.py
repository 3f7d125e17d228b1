"""nvfp4_quantize_batch: several independent quantisations enqueued together.

Each job's outputs must be exactly those of nvfp4_quantize on the same job
(codes, scales, S and amax, bit for bit), whether the batch runs as the grouped
launches of the weight-gradient operand pair (two single RHT column outputs:
one amax launch, one quantise launch whose workgroups alternate between the
two inputs) or job after job.  The pair is also checked against the oracle
directly (RHT tolerance; the stochastic-rounding output of the pair under the
oracle's own Philox streams).  The quantisation follows the NVFP4 news page
(zubnet.ai), paragraph 2: the RHT on the weight-gradient GEMM's inputs,
stochastic rounding on gradients."""
import numpy as np
import pytest

import oracle
from nvfp4_bit_quantization_amd import synthetic as syn

from gpu_util import assert_bit_exact, assert_rht_tolerance, dev_bf16, gpu_q_as_dict, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def nv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import nvfp4_bit_quantization_amd as nv
    nv.lib()
    return nv


def _outs(nv, R, C, specs):
    outs = []
    for s in specs:
        r, c, k = nv.output_shape(R, C, s.layout)
        outs.append(nv.empty_qtensor(r, c, k, rht=int(s.rht)))
    return outs


def _separate(nv, jobs):
    """the same jobs through nvfp4_quantize, one call each"""
    res = []
    for x, specs, _ in jobs:
        outs = _outs(nv, x.shape[0], x.shape[1], specs)
        nv.nvfp4_quantize(x, specs, outs, nv.new_workspace())
        res.append(outs)
    return res


def _batched(nv, jobs, ws=None):
    if ws is None:
        ws = nv.new_workspace(jobs=len(jobs))
    nv.nvfp4_quantize_batch(jobs, ws)
    torch.cuda.synchronize()
    return [outs for _, _, outs in jobs]


def _assert_same(nv, batched, separate, what):
    for j, (bo, so) in enumerate(zip(batched, separate)):
        for i, (b, s) in enumerate(zip(bo, so)):
            assert_bit_exact(gpu_q_as_dict(b), gpu_q_as_dict(s), "%s job %d output %d" % (what, j, i))


def _wgrad_pair(nv, dy_bits, x_bits, sr_dy, sr_x):
    S = nv.QuantSpec.of
    s_dy = [S("col", "sr" if sr_dy else "rtn", True, 1234 if sr_dy else 0, 1234)]
    s_x = [S("col", "sr" if sr_x else "rtn", True, 77 if sr_x else 0, 1234)]
    dy, x = dev_bf16(dy_bits), dev_bf16(x_bits)
    return [(dy, s_dy, _outs(nv, *dy_bits.shape, s_dy)), (x, s_x, _outs(nv, *x_bits.shape, s_x))]


@pytest.mark.parametrize("sr_dy,sr_x", [(True, False), (False, True), (True, True), (False, False)])
def test_wgrad_pair_matches_single_calls_and_oracle(nv, sr_dy, sr_x):
    """the grouped launches on two ragged inputs of different shapes (so the
    alternating workgroups run out for one of them first)"""
    say("batch wgrad pair", sr_dy, sr_x)
    dy_bits = syn.laplace(1040, 784, 31, 1e-3)
    x_bits = syn.normal(528, 1296, 32)
    jobs = _wgrad_pair(nv, dy_bits, x_bits, sr_dy, sr_x)
    sep = _separate(nv, jobs)
    got = _batched(nv, jobs)
    _assert_same(nv, got, sep, "wgrad pair")
    for (bits, specs, outs) in ((dy_bits, jobs[0][1], got[0]), (x_bits, jobs[1][1], got[1])):
        s = specs[0]
        o = oracle.quantize(bits, "col", "sr" if s.rounding == nv.SR else "rtn", True, s.sr_seed, s.rht_seed)
        assert_rht_tolerance(gpu_q_as_dict(outs[0]), o, "batch vs oracle")


def test_wgrad_pair_full_size(nv):
    """the Wgrad operands of the 8192-token, 5120-hidden layer: dY with SR, X
    with RTN, both with the RHT along tokens"""
    say("batch wgrad pair 8192x5120")
    dy_bits, x_bits = syn.wgrad_8192x5120(8192, 5120)
    jobs = _wgrad_pair(nv, dy_bits, x_bits, True, False)
    sep = _separate(nv, jobs)
    _assert_same(nv, _batched(nv, jobs), sep, "wgrad 8192x5120")


def test_other_batches_run_job_after_job(nv):
    """batches the grouped kernels do not cover: three jobs, a two-output job,
    a given maximum, and a pair with a row output"""
    say("batch fallback")
    S = nv.QuantSpec.of
    a_bits = syn.activation(1024, 768, 202)
    w_bits = syn.normal(512, 1024, 5, 0.02)
    g_bits = syn.laplace(784, 528, 6, 1e-3)
    a, w, g = dev_bf16(a_bits), dev_bf16(w_bits), dev_bf16(g_bits)
    s_a = [S("row"), S("col", "rtn", True, 0, 4321)]
    s_w = [S("2d"), S("2d_t")]
    s_g = [S("col", "sr", True, 9, 4321)]
    jobs = [(a, s_a, _outs(nv, 1024, 768, s_a)), (w, s_w, _outs(nv, 512, 1024, s_w)), (g, s_g, _outs(nv, 784, 528, s_g))]
    _assert_same(nv, _batched(nv, jobs), _separate(nv, jobs), "three jobs")
    # a pair that is not the operand kind: one row output
    s_r = [S("row", "sr", False, 3)]
    jobs = [(g, s_g, _outs(nv, 784, 528, s_g)), (a, s_r, _outs(nv, 1024, 768, s_r))]
    _assert_same(nv, _batched(nv, jobs), _separate(nv, jobs), "col + row pair")
    # a given maximum on one job of an otherwise eligible pair
    ref = _separate(nv, [(g, s_g, None)])[0][0]
    given = [S("col", "sr", True, 9, 4321, amax_given=True)]
    out_given = _outs(nv, 784, 528, given)
    out_given[0].amax.copy_(ref.amax)
    s_x = [S("col", "rtn", True, 0, 4321)]
    jobs = [(g, given, out_given), (a, s_x, _outs(nv, 1024, 768, s_x))]
    got = _batched(nv, jobs)
    assert_bit_exact(gpu_q_as_dict(got[0][0]), gpu_q_as_dict(ref), "given maximum")
    _assert_same(nv, [got[1]], _separate(nv, [jobs[1]]), "the other job")


def test_batches_in_a_row_reuse_the_workspace(nv):
    """two grouped calls in a row on one workspace, the second on smaller
    inputs: nothing of the first call's partial maxima is carried over"""
    say("batch twice")
    ws = nv.new_workspace(jobs=2)
    big = _wgrad_pair(nv, syn.laplace(2048, 1024, 41, 1e-3), syn.normal(2048, 1024, 42), True, False)
    _assert_same(nv, _batched(nv, big, ws), _separate(nv, big), "first call")
    small = _wgrad_pair(nv, syn.laplace(272, 144, 43, 1e-4), syn.normal(272, 144, 44), True, False)
    _assert_same(nv, _batched(nv, small, ws), _separate(nv, small), "second call")


def test_batch_rejects_before_enqueuing(nv):
    """a bad job anywhere in the batch: its status, and the other jobs' outputs
    untouched"""
    say("batch rejects")
    S = nv.QuantSpec.of
    x = dev_bf16(syn.normal(256, 256, 8))
    s_c = [S("col", "rtn", True, 0, 5)]
    good = _outs(nv, 256, 256, s_c)
    for o in good:
        o.codes.fill_(0xAB)
    bad_x = dev_bf16(syn.normal(256, 256, 9))[:, :248]  # cols % 16 != 0
    jobs = [(x, s_c, good), (bad_x, s_c, _outs(nv, 256, 256, s_c))]
    with pytest.raises(RuntimeError):
        nv.nvfp4_quantize_batch(jobs, nv.new_workspace(jobs=2))
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(good[0].codes != 0xAB)) == 0
    with pytest.raises(RuntimeError):
        nv.nvfp4_quantize_batch([(x, s_c, good), (x, s_c, _outs(nv, 256, 256, s_c))], nv.new_workspace(jobs=1))
