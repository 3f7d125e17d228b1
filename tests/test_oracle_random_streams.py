"""Statistical pins of the oracle's two random streams.

The page asks for random +/-1 sign vectors on the RHT (paragraph 2, the
16-point randomised Hadamard transform on the weight-gradient inputs) and for
stochastic rounding of gradients (same paragraph).  Which Philox counter and
which bits of its output feed each element is a convention of this project, so
no value on the page pins it; what the mathematics does fix is that the draws
are fair and independent.  These tests check exactly that, on the oracle's own
outputs, so that a structural slip in the convention code (a truncated mask, a
16-bit half read twice, overlapping counters between neighbouring blocks, two
elements of a 2D tile sharing a uniform) fails here even though it would pass
the tests that only restate the convention:

* sign mask: over 10^5 seeds each of the 16 bits is fair, every pair of bits
  is uncorrelated, and the number of distinct masks matches the occupancy of
  65536 equally likely values;
* SR uniforms: over 10^5 blocks every one of the 256 bits (16 elements x 16
  bits) is fair and every pair of bits belonging to different elements is
  uncorrelated, within a block and across neighbouring blocks; each element's
  uniform has the mean and variance of a discrete uniform on [0, 65536);
* quantised tensors: on an input where every non-maximal element sits exactly
  halfway between two E2M1 values, the round-up decisions of ROW, COL and 2D
  outputs are fair and no two rows or columns of decisions are correlated.

Bounds are 6 standard deviations of the statistic under independence (the
family-wise false-alarm rate of the largest test, 2^15 correlations, is below
1e-4).
"""
import numpy as np
import pytest

import oracle

N_SEEDS = 100_000
N_BLOCKS = 100_000
SIGMAS = 6.0


def _pm1_bits(words: np.ndarray, nbits: int) -> np.ndarray:
    """[n] unsigned integers -> [n, nbits] float32 matrix of +/-1 (bit set -> -1)."""
    b = (words[:, None].astype(np.uint64) >> np.arange(nbits, dtype=np.uint64)[None, :]) & np.uint64(1)
    return (1.0 - 2.0 * b).astype(np.float32)


def _sign_masks(seeds) -> np.ndarray:
    return np.array([oracle.rht_sign_mask(int(s)) for s in seeds], dtype=np.uint32)


@pytest.fixture(scope="module")
def masks():
    rng = np.random.default_rng(2024)
    seeds = np.concatenate([np.arange(N_SEEDS // 2, dtype=np.uint64),  # consecutive seeds
                            rng.integers(0, 2 ** 63, N_SEEDS // 2, dtype=np.uint64)])
    return _sign_masks(seeds)


def test_sign_mask_bits_are_fair(masks):
    b = _pm1_bits(masks, 16)
    mean = b.mean(axis=0)  # each +/-1 bit: mean 0, standard deviation 1/sqrt(N)
    bound = SIGMAS / np.sqrt(b.shape[0])
    assert np.all(np.abs(mean) < bound), (np.abs(mean).max(), bound)


def test_sign_mask_bits_are_pairwise_uncorrelated(masks):
    b = _pm1_bits(masks, 16)
    c = (b.T @ b) / b.shape[0]
    off = c[~np.eye(16, dtype=bool)]
    bound = SIGMAS / np.sqrt(b.shape[0])
    assert np.all(np.abs(off) < bound), (np.abs(off).max(), bound)


def test_sign_mask_occupancy(masks):
    # n draws of 65536 equally likely masks: the number of distinct values has
    # mean 65536 (1 - (1 - 1/65536)^n) and a standard deviation below 100
    n, m = masks.size, 65536.0
    expected = m * (1.0 - (1.0 - 1.0 / m) ** n)
    distinct = np.unique(masks).size
    assert abs(distinct - expected) < 600, (distinct, expected)


@pytest.fixture(scope="module")
def uniforms():
    """u16 of the 16 elements of N_BLOCKS blocks (consecutive and random block
    indices) and of the block after each: arrays [N_BLOCKS, 16]."""
    rng = np.random.default_rng(77)
    seed = 0x5EED_1234_ABCD
    blocks = np.concatenate([np.arange(N_BLOCKS // 2, dtype=np.uint64),
                             rng.integers(0, 2 ** 40, N_BLOCKS // 2, dtype=np.uint64)])
    js = np.arange(16, dtype=np.int32)
    u = oracle.sr_uniform_array(seed, np.repeat(blocks, 16), np.tile(js, blocks.size)).reshape(-1, 16)
    un = oracle.sr_uniform_array(seed, np.repeat(blocks + 1, 16), np.tile(js, blocks.size)).reshape(-1, 16)
    return u, un


def test_sr_uniform_moments(uniforms):
    u = uniforms[0].astype(np.float64)
    n = u.shape[0]
    mu, var = 32767.5, (65536.0 ** 2 - 1) / 12.0
    assert np.all(np.abs(u.mean(axis=0) - mu) < SIGMAS * np.sqrt(var / n))
    # sample variance: standard deviation of the estimate sqrt((m4 - var^2) / n), m4 = 65536^4 / 80
    sd_var = np.sqrt((65536.0 ** 4 / 80 - var ** 2) / n)
    assert np.all(np.abs(u.var(axis=0) - var) < SIGMAS * sd_var)


def _bit_matrix(u):  # [n, 16 elements] u16 -> [n, 256] +/-1 bits (element-major)
    return np.concatenate([_pm1_bits(u[:, j].astype(np.uint32), 16) for j in range(16)], axis=1)


def test_sr_uniform_bits_fair_and_independent_within_a_block(uniforms):
    b = _bit_matrix(uniforms[0])
    n = b.shape[0]
    bound = SIGMAS / np.sqrt(n)
    assert np.all(np.abs(b.mean(axis=0)) < bound)
    c = (b.T @ b) / n
    elem = np.arange(256) // 16
    other = elem[:, None] != elem[None, :]  # bit pairs of different elements
    assert np.all(np.abs(c[other]) < bound), (np.abs(c[other]).max(), bound)


def test_sr_uniform_bits_independent_across_neighbouring_blocks(uniforms):
    b0, b1 = _bit_matrix(uniforms[0]), _bit_matrix(uniforms[1])
    n = b0.shape[0]
    c = (b0.T @ b1) / n  # every bit of block b against every bit of block b + 1
    bound = SIGMAS / np.sqrt(n)
    assert np.all(np.abs(c) < bound), (np.abs(c).max(), bound)


# ------------------------------------------------------------------------------
def _halfway_tensor(R, C, layout):
    """bf16 bit patterns: 2.5 everywhere except one 6.0 per scale block (its
    first element in the stored orientation), so that S = 448, every block
    scale is 448 and every other element scales to exactly 2.5, halfway
    between the E2M1 values 2 and 3."""
    x = np.full((R, C), 2.5, dtype=np.float32)
    if layout == "row":
        x[:, ::16] = 6.0
    elif layout == "col":
        x[::16, :] = 6.0
    else:  # 2d
        x[::16, ::16] = 6.0
    from nvfp4_bit_quantization_amd.synthetic import f32_to_bf16_bits
    return f32_to_bf16_bits(x)


def _round_up_decisions(q):
    codes = q["codes"]
    nib = np.stack([codes & 15, codes >> 4], axis=-1).reshape(codes.shape[0], -1)
    return nib


@pytest.mark.parametrize("layout", ["row", "col", "2d"])
def test_sr_decisions_fair_and_uncorrelated_in_quantised_tensors(layout):
    R = C = 1024
    q = oracle.quantize(_halfway_tensor(R, C, layout), layout, "sr", False, 31337)
    assert q["S"] == np.float32(448.0)
    nib = _round_up_decisions(q).astype(np.int32)
    stored_max = np.zeros(nib.shape, dtype=bool)
    if layout == "2d":
        stored_max[::16, ::16] = True
    else:  # the block maximum is the first element of each stored 16-block
        stored_max[:, ::16] = True
    assert np.all(nib[stored_max] == 7)  # 6.0 at scale 448 is exactly the top code
    mid = nib[~stored_max]
    assert np.all((mid == 4) | (mid == 5))  # 2.0 or 3.0, never anything else
    up = np.where(stored_max, 0.0, (nib == 5) * 2.0 - 1.0)  # +/-1 decisions, 0 at the maxima
    n = np.count_nonzero(~stored_max)
    # fair: P(up) = ceil(0.5 * 65536) / 65536 = 1/2 exactly under O17
    assert abs(up.sum()) < SIGMAS * np.sqrt(n)
    for mat in (up, up.T):  # rows of decisions, then columns
        k = mat.shape[1]
        c = (mat @ mat.T) / k
        off = c[~np.eye(c.shape[0], dtype=bool)]
        assert np.all(np.abs(off) < SIGMAS / np.sqrt(k * 15 / 16)), np.abs(off).max()
