"""The library's calls captured in a HIP graph (torch.cuda.CUDAGraph): every
entry point only enqueues kernels on the caller's stream -- no allocation, no
memset, no host synchronisation -- so a step of them can be captured once and
replayed.  Each replay, with eager work and synchronisations in between, must
reproduce the eager results bit for bit (stochastic rounding is keyed by the
seed and block index, so it is deterministic too).  The step is the Wgrad path
of the NVFP4 pretraining news page (zubnet.ai), paragraph 2, at a small shape,
plus a row/column quantisation and a dequantisation; the Wgrad operands are
quantised by two calls, or by one batch call (the bench's form)."""
import numpy as np
import pytest

from nvfp4_bit_quantization_amd import synthetic as syn

from gpu_util import dev_bf16, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def nv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import nvfp4_bit_quantization_amd as nv
    nv.lib()
    return nv


@pytest.mark.parametrize("batch", [False, True])
def test_step_replays_from_a_graph(nv, batch):
    T, H1, H2 = 2048, 768, 512
    dy = dev_bf16(syn.laplace(T, H1, seed=51, scale=1e-3))
    x = dev_bf16(syn.normal(T, H2, seed=52))
    a = dev_bf16(syn.activation(T, H2, seed=53))
    ws_dy, ws_x, ws_a = nv.new_workspace(), nv.new_workspace(), nv.new_workspace()
    ws_b = nv.new_workspace(jobs=2)
    s_dy = [nv.QuantSpec.of("col", "sr", True, 1234, 1234)]
    s_x = [nv.QuantSpec.of("col", "rtn", True, 0, 1234)]
    s_a = [nv.QuantSpec.of("row"), nv.QuantSpec.of("col")]
    q_dy = [nv.empty_qtensor(H1, T, nv.SCALE_1D16, rht=1)]
    q_x = [nv.empty_qtensor(H2, T, nv.SCALE_1D16, rht=1)]
    q_a = [nv.empty_qtensor(T, H2, nv.SCALE_1D16), nv.empty_qtensor(H2, T, nv.SCALE_1D16)]
    c = torch.empty((H1, H2), dtype=torch.float32, device="cuda")
    y = torch.empty((T, H2), dtype=torch.float32, device="cuda")

    def step():
        if batch:
            nv.nvfp4_quantize_batch([(dy, s_dy, q_dy), (x, s_x, q_x)], ws_b)
        else:
            nv.nvfp4_quantize(dy, s_dy, q_dy, ws_dy)
            nv.nvfp4_quantize(x, s_x, q_x, ws_x)
        nv.nvfp4_gemm(q_dy[0], q_x[0], c)
        nv.nvfp4_quantize(a, s_a, q_a, ws_a)
        nv.nvfp4_dequantize(q_a[0], y)

    outs = [q_dy[0].codes, q_dy[0].scales, q_dy[0].global_scale, q_x[0].codes, q_x[0].scales, c,
            q_a[0].codes, q_a[1].codes, q_a[1].scales, y]
    say("graph: eager step, batch", batch)
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]

    say("graph: capture")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm-up on a side stream, as capture requires
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    for i in range(4):
        for t in outs:
            t.zero_()  # eager work between replays
        torch.cuda.synchronize()
        say("graph: replay", i)
        g.replay()
        torch.cuda.synchronize()
        for k, (t, r) in enumerate(zip(outs, ref)):
            assert torch.equal(t, r), "replay %d output %d differs from the eager step" % (i, k)


def test_streamk_shape_captured_takes_whole_tiles(nv):
    """A GEMM with a workspace on a shape that runs as stream-K when launched
    eagerly (4352x8448, K = 1024: 4.3 rounds of tiles) is captured as whole
    tiles; its replays equal an eager whole-tile launch bit for bit and the
    eager stream-K result to fp32 accumulation-order level."""
    M, N, K = 4352, 8448, 1024
    qa = nv.quantize(dev_bf16(syn.normal(M, K, seed=61)), [nv.QuantSpec.of("row")])[0]
    qb = nv.quantize(dev_bf16(syn.normal(N, K, seed=62)), [nv.QuantSpec.of("row")])[0]
    gws = nv.new_gemm_workspace()
    gws.zero_()
    c = torch.empty((M, N), dtype=torch.float32, device="cuda")
    say("graph stream-K shape: eager")
    nv.nvfp4_gemm(qa, qb, c, gws)
    torch.cuda.synchronize()
    c_sk = c.clone()
    import os
    os.environ["NVFP4_GEMM_DATA_PARALLEL"] = "1"
    try:
        nv.nvfp4_gemm(qa, qb, c, gws)
        torch.cuda.synchronize()
    finally:
        del os.environ["NVFP4_GEMM_DATA_PARALLEL"]
    c_dp = c.clone()
    say("graph stream-K shape: capture")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        nv.nvfp4_gemm(qa, qb, c, gws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        nv.nvfp4_gemm(qa, qb, c, gws)
    torch.cuda.synchronize()
    for i in range(3):
        c.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(c, c_dp), "replay %d differs from the eager whole-tile launch" % i
    assert not nv.gemm_workspace_timed_out(gws)
    rel = float((c - c_sk).norm() / c_sk.norm())
    assert rel <= 1e-6, rel
