"""The device encoders against the oracle's codecs.

The E2M1 round-to-nearest path uses gfx950's FP32->FP4 conversion instruction,
so it is checked exhaustively over all 2^32 binary32 bit patterns (NaN/Inf
excluded).  The E4M3 block-scale encoder (gfx950's FP32->FP8 conversion after
a clamp at 448) is checked exhaustively over every non-negative finite
binary32 pattern, the only inputs it takes.
The stochastic-rounding encoder (the gfx950 SR conversion after an exact
pre-rounding) is checked at every step point of every y with
2^-17 <= |y| < 8, on random (y, u16) pairs and on structured grids (every
u16 against grid points, midpoints and neighbours).
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import oracle

from gpu_util import host, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def nv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import nvfp4_bit_quantization_amd as nv
    nv.lib()
    return nv


def test_e2m1_rtn_exhaustive(nv):
    chunk = 1 << 28
    out = torch.empty(chunk, dtype=torch.uint8, device="cuda")
    pool = ThreadPoolExecutor(16)
    sub = 1 << 24
    for start in range(0, 1 << 32, chunk):
        say("e2m1 exhaustive chunk", hex(start))
        bits = torch.arange(start, start + chunk, dtype=torch.int64, device="cuda").to(torch.int32)
        x = bits.view(torch.float32)
        nv.nvfp4_codec_selftest(0, x, None, out)
        got = host(out)
        del bits, x
        parts = list(pool.map(lambda s: oracle.e2m1_encode_rtn_bits(s, sub), range(start, start + chunk, sub)))
        want = np.concatenate(parts)
        finite = want != 0xFF
        bad = np.flatnonzero((got != want) & finite)
        assert bad.size == 0, "first mismatching pattern 0x%08x: gpu %x oracle %x" % (
            start + bad[0], got[bad[0]], want[bad[0]])


def test_e4m3_encoder_exhaustive(nv):
    """Every non-negative finite binary32 pattern (0 to 0x7F7FFFFF, 2^31 - 2^23
    values): the device's block-scale encoder against the oracle's."""
    chunk = 1 << 28
    limit = 0x7F800000  # +Inf: the first pattern that is not a finite non-negative value
    out = torch.empty(chunk, dtype=torch.uint8, device="cuda")
    pool = ThreadPoolExecutor(16)
    sub = 1 << 24
    for start in range(0, limit, chunk):
        n = min(chunk, limit - start)
        say("e4m3 exhaustive chunk", hex(start), n)
        bits = torch.arange(start, start + n, dtype=torch.int64, device="cuda").to(torch.int32)
        x = bits.view(torch.float32)
        nv.nvfp4_codec_selftest(2, x, None, out[:n])
        got = host(out[:n])
        del bits, x
        parts = list(pool.map(lambda s0: oracle.e4m3_encode_bits(s0, min(sub, start + n - s0)),
                              range(start, start + n, sub)))
        want = np.concatenate(parts)
        assert np.count_nonzero(want == 0xFF) == 0
        bad = np.flatnonzero(got != want)
        assert bad.size == 0, "first mismatching pattern 0x%08x: gpu %x oracle %x" % (
            start + bad[0], got[bad[0]], want[bad[0]])


def test_e2m1_sr_encoder(nv):
    rng = np.random.default_rng(1)
    n = 1 << 22
    y = np.concatenate([rng.uniform(-7, 7, n // 2).astype(np.float32),
                        rng.integers(0, 2 ** 32, n // 2, dtype=np.uint64).astype(np.uint32).view(np.float32)])
    y = y[np.isfinite(y)]
    u = rng.integers(0, 65536, y.size, dtype=np.uint16)
    # structured: every u16 against values at and around grid points and midpoints
    grid = np.array([0, .25, .5, .75, 1, 1.25, 1.5, 1.75, 2, 2.5, 3, 3.5, 4, 5, 6, 6.5], np.float32)
    gpts = np.concatenate([grid, np.nextafter(grid, np.float32(9)), np.nextafter(grid, np.float32(-1)),
                           grid * np.float32(1.37), np.float32([1e-40, 3e-39, 0.1])])
    gpts = np.concatenate([gpts, -gpts])
    ys = np.concatenate([y, np.repeat(gpts, 65536)]).astype(np.float32)
    us = np.concatenate([u, np.tile(np.arange(65536, dtype=np.uint16), gpts.size)])
    say("e2m1 sr", ys.size)
    out = torch.empty(ys.size, dtype=torch.uint8, device="cuda")
    x = torch.from_numpy(ys).cuda()
    uu = torch.from_numpy(us.view(np.int16)).cuda()
    nv.nvfp4_codec_selftest(1, x, uu, out)
    got = host(out)
    want = oracle.e2m1_encode_sr(ys, us)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, (ys[bad[:5]], us[bad[:5]], got[bad[:5]], want[bad[:5]])


def _sr_points(nv, pool, start, n, stride=1):
    """Device against oracle stochastic rounding for the fp32 patterns
    start, start + stride, ... (n of them), each at u16 = 0, step - 1, step
    and 65535, step being where the oracle's rounding switches from up to
    down.  Returns the number of (y, u16) pairs compared."""
    sub = 1 << 22
    if stride == 1:
        bits = np.arange(start, start + n, dtype=np.uint64).astype(np.uint32)
        steps = np.concatenate(list(pool.map(lambda s0: oracle.e2m1_sr_step_bits(s0, min(sub, start + n - s0)),
                                             range(start, start + n, sub))))
    else:
        bits = (start + stride * np.arange(n, dtype=np.uint64)).astype(np.uint32)
        steps = np.array([oracle.e2m1_sr_step_bits(int(b), 1)[0] for b in bits], dtype=np.uint32)
    y = bits.view(np.float32)
    keep = steps != 0xFFFFFFFF
    y, steps = y[keep], steps[keep]
    u = np.stack([np.zeros_like(steps), np.maximum(steps, 1) - 1, np.minimum(steps, 65535),
                  np.full_like(steps, 65535)], axis=1).astype(np.uint16)
    ys = np.repeat(y, 4)
    us = u.reshape(-1)
    # the element index decides the instruction slot (even: first, odd: second);
    # run every pair twice, shifted by one, so that both slots see every case
    ys2, us2 = np.concatenate([ys, ys[:1], ys]), np.concatenate([us, us[:1], us])
    x = torch.from_numpy(ys2).cuda()
    uu = torch.from_numpy(us2.view(np.int16)).cuda()
    out = torch.empty(ys2.size, dtype=torch.uint8, device="cuda")
    nv.nvfp4_codec_selftest(1, x, uu, out)
    got = host(out)
    want = np.concatenate(list(pool.map(lambda i: oracle.e2m1_encode_sr(ys[i:i + sub], us[i:i + sub]),
                                        range(0, ys.size, sub))))
    for part, off in (("even slot", 0), ("odd slot", ys.size + 1)):
        g = got[off:off + ys.size]
        bad = np.flatnonzero(g != want)
        assert bad.size == 0, "%s: y=%r u16=%d gpu %x oracle %x (%d mismatches)" % (
            part, float(ys[bad[0]]), int(us[bad[0]]), g[bad[0]], want[bad[0]], bad.size)
    return 2 * ys.size


def test_e2m1_sr_hardware_path_at_every_step(nv):
    """The stochastic-rounding encoder the kernels use (gfx950 conversion
    instruction, after rounding |y| up to a multiple of 2^-23) against the
    oracle's, for every binary32 y with 2^-17 <= |y| < 8, both signs: for each
    y the oracle's round-up set is a prefix [0, step) of the u16 range, and
    the device is checked at u16 = 0, step - 1, step and 65535, in both slots
    of the instruction.  Below 2^-17 only u16 = 0 rounds up (a sampled check),
    and 8 and above saturate like 6 (sampled)."""
    pool = ThreadPoolExecutor(16)
    lo, hi = 0x37000000, 0x41000000  # 2^-17 .. 8
    chunk = 1 << 24
    total = 0
    for sign in (0, 0x80000000):
        for start in range(lo, hi, chunk):
            say("sr steps", hex(sign | start))
            total += _sr_points(nv, pool, sign | start, min(chunk, hi - start))
        total += _sr_points(nv, pool, sign | 0x00000001, 200000, stride=(lo - 1) // 200000)
        total += _sr_points(nv, pool, sign | hi, 100000, stride=(0x7F7FFFFF - hi) // 100000)
    say("sr steps: pairs compared", total)
    assert total > 8 * (hi - lo)


def test_sync_check_mode_in_a_child_process():
    """NVFP4_SYNC_CHECK=1 (read once per process) makes every call wait for
    its stream: the same quantise and GEMM calls succeed and give the same
    codes and product as without it."""
    import os
    import subprocess
    import sys
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    prog = (
        "import sys, hashlib; sys.path.insert(0, %r)\n"
        "import numpy as np, torch\n"
        "import nvfp4_bit_quantization_amd as nv\n"
        "from nvfp4_bit_quantization_amd import synthetic as syn\n"
        "x = torch.from_numpy(syn.laplace(256, 512, seed=3).view(np.int16)).view(torch.bfloat16).cuda()\n"
        "qa = nv.quantize(x, [nv.QuantSpec.of('row', 'sr', False, 5)])[0]\n"
        "c = nv.gemm(qa, qa, 'f32')\n"
        "torch.cuda.synchronize()\n"
        "print(hashlib.sha256(qa.codes.cpu().numpy().tobytes() + c.cpu().numpy().tobytes()).hexdigest())\n"
    ) % root
    outs = []
    for flag in ("0", "1"):
        env = dict(os.environ, NVFP4_SYNC_CHECK=flag)
        r = subprocess.run([sys.executable, "-c", prog], env=env, capture_output=True, text=True, timeout=240)
        assert r.returncode == 0, r.stderr[-2000:]
        outs.append(r.stdout.strip().splitlines()[-1])
    assert outs[0] == outs[1]
