"""nvfp4_quantize_noalloc -- the quantise entry point that allocates nothing
(its partial maxima live in the library's static device scratch), for callers
that cannot allocate device memory -- against nvfp4_quantize with a caller
workspace, through the C ABI, bit for bit on every output (codes, scales, S,
amax).  The same kernels run in both, so any difference would come from the
scratch: a wrong device address, or stale partial maxima of an earlier call.
Two calls in a row, the second on a smaller input (fewer partial maxima than
the first wrote), check the second; the small cases are also checked against
the oracle (bit-exact for RTN/SR without the RHT, the RHT tolerance with it).
"""
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


def _outs(nv, rows, cols, specs):
    outs = []
    for s in specs:
        r, c, k = nv.output_shape(rows, cols, s.layout)
        outs.append(nv.empty_qtensor(r, c, k, rht=int(s.rht)))
    return outs


def _same(a, b, what):
    for name in ("codes", "scales", "global_scale", "amax"):
        ta, tb = getattr(a, name), getattr(b, name)
        assert torch.equal(ta.view(torch.uint8), tb.view(torch.uint8)), "%s: %s differs" % (what, name)


CASES = [  # (name, bits, specs)
    ("wgrad dY 8192x5120 col RHT SR", lambda: syn.laplace(8192, 5120, seed=404, scale=1e-3),
     [("col", "sr", True, 1234, 1234)]),
    ("act 512x768 row+col RTN", lambda: syn.activation(512, 768, seed=9),
     [("row", "rtn", False, 0, 0), ("col", "rtn", False, 0, 0)]),
    ("weight 256x512 2D+2D_T RTN", lambda: syn.normal(256, 512, seed=10, std=0.02),
     [("2d", "rtn", False, 0, 0), ("2d_t", "rtn", False, 0, 0)]),
    ("grad 96x160 row SR + col RHT SR", lambda: syn.laplace(96, 160, seed=11, scale=1e-3),
     [("row", "sr", False, 5, 0), ("col", "sr", True, 6, 7)]),
]


def test_noalloc_matches_the_workspace_entry_point(nv):
    data = [(name, make(), [nv.QuantSpec.of(*s) for s in specs]) for name, make, specs in CASES]
    xs = [dev_bf16(bits) for _, bits, _ in data]
    # reference: the existing entry point, each call with its own workspace
    ref = []
    for (name, bits, specs), x in zip(data, xs):
        outs = _outs(nv, bits.shape[0], bits.shape[1], specs)
        nv.nvfp4_quantize(x, specs, outs, nv.new_workspace())
        ref.append(outs)
    torch.cuda.synchronize()
    # the allocation-free entry point: all calls back to back on one stream
    # (each later call smaller than the first), no synchronisation between them
    got = []
    for (name, bits, specs), x in zip(data, xs):
        say("noalloc", name)
        outs = _outs(nv, bits.shape[0], bits.shape[1], specs)
        got.append(outs)
    before = torch.cuda.memory_allocated()
    for (name, bits, specs), x, outs in zip(data, xs, got):
        nv.nvfp4_quantize_noalloc(x, specs, outs)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    for (name, bits, specs), r, g in zip(data, ref, got):
        for i, (ro, go) in enumerate(zip(r, g)):
            _same(ro, go, "%s output %d" % (name, i))
    # the small cases against the oracle
    for (name, bits, specs), g in list(zip(data, got))[1:]:
        for s, go in zip(specs, g):
            layout = {nv.ROW_1D: "row", nv.COL_1D: "col", nv.TWO_D: "2d", nv.TWO_D_T: "2d_t"}[s.layout]
            o = oracle.quantize(bits, layout, "sr" if s.rounding == nv.SR else "rtn", s.rht, s.sr_seed, s.rht_seed)
            if s.rht:
                assert_rht_tolerance(gpu_q_as_dict(go), o, name)
            else:
                assert_bit_exact(gpu_q_as_dict(go), o, name)


def test_noalloc_repeated_calls_keep_no_state(nv):
    """A large call, then a small one, then the large one again: every result
    equals the workspace entry point's, so nothing an earlier call left in the
    shared scratch leaks into a later one."""
    big = dev_bf16(syn.normal(4096, 4096, seed=21))
    small = dev_bf16(syn.normal(64, 128, seed=22, std=1e-3))
    spec = [nv.QuantSpec.of("row")]
    want_big = nv.quantize(big, spec)[0]
    want_small = nv.quantize(small, spec)[0]
    seq = [(big, want_big), (small, want_small), (big, want_big), (small, want_small)]
    outs = [_outs(nv, x.shape[0], x.shape[1], spec)[0] for x, _ in seq]
    say("noalloc big/small/big/small")
    for (x, _), o in zip(seq, outs):
        nv.nvfp4_quantize_noalloc(x, spec, [o])
    torch.cuda.synchronize()
    for k, ((x, w), o) in enumerate(zip(seq, outs)):
        _same(w, o, "call %d" % k)


def test_noalloc_rejects_bad_arguments_before_anything_else(nv):
    x = dev_bf16(syn.normal(64, 64, seed=1))
    outs = _outs(nv, 64, 64, [nv.QuantSpec.of("row")])
    with pytest.raises(nv.Nvfp4Error):
        nv.nvfp4_quantize_noalloc(x[:, :48], [nv.QuantSpec.of("row")], outs)  # shape mismatch with outs
