"""The integer-weight split of the 4-bit scan's MFMA operand, checked in fp32 on the CPU.

The scan forms each weight a~ = rint(q kscale / alpha) (round half to even; q and kscale
fp16, alpha = 2^(x - 11) the block's grid step with |q kscale| < 2^x) as one fused
multiply-add of q kscale and the constant (1.5 2^23 + 128) alpha, and takes two signed
int8 digits from the bits of the fp32 sum: byte 1 is a1 and byte 0 with its top bit
flipped is a0, with a~ = 256 a1 + a0.  Here the product of two fp16 values is exact in
fp32, so the FMA equals the fp32 sum of the product and the constant, which numpy
reproduces; the test checks the digit identity against the exact rounding (computed in
fp64, where q kscale / alpha is exact) over random operands, ties and both signs.
"""

import numpy as np


def _digits(q16, k16, alpha):
    """The scan's two digits (a1, a0) for fp16 arrays q16, k16 and fp32 grid steps alpha."""
    magic = np.float32(1.5 * 2.0**23 + 128.0)
    c = np.where(alpha > 0, magic * alpha, magic).astype(np.float32)
    prod = q16.astype(np.float32) * k16.astype(np.float32)      # exact: 11 x 11 bits
    t = (prod + c).astype(np.float32)                           # the FMA's single rounding
    bits = t.view(np.uint32)
    a1 = ((bits >> 8) & 0xFF).astype(np.uint8).view(np.int8).astype(np.int64)
    a0 = ((bits & 0xFF) ^ 0x80).astype(np.uint8).view(np.int8).astype(np.int64)
    return a1, a0


def _grid(qmax, ksmax):
    m = np.float32(qmax) * np.float32(ksmax)
    if m == 0:
        return np.float32(0.0)
    _, x = np.frexp(np.float64(m))
    return np.float32(np.ldexp(1.0, int(x) - 11))


def test_digits_reproduce_the_rounded_weight():
    rng = np.random.default_rng(20261202)
    for trial in range(200):
        n = 4096
        qs = np.float16(rng.choice([1e-3, 0.05, 1.0, 30.0, 2000.0]))
        ks_scale = np.float16(rng.choice([1e-4, 0.01, 0.3, 8.0]))
        q16 = (rng.standard_normal(n) * np.float32(qs)).astype(np.float16)
        k16 = np.abs(rng.standard_normal(n) * np.float32(ks_scale)).astype(np.float16)
        alpha = _grid(np.abs(q16.astype(np.float32)).max(), k16.astype(np.float32).max())
        a1, a0 = _digits(q16, k16, alpha)
        exact = q16.astype(np.float64) * k16.astype(np.float64) / np.float64(alpha)
        want = np.rint(exact).astype(np.int64)                    # half to even
        assert np.all(np.abs(want) <= 2048), trial
        assert np.array_equal(256 * a1 + a0, want), trial
        assert a1.min() >= -8 and a1.max() <= 8
        assert a0.min() >= -128 and a0.max() <= 127


def test_ties_go_to_even():
    # products that land exactly halfway between two integers of the grid
    alpha = np.float32(1.0)
    q16 = np.array([0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 127.5, -128.5, 255.5, -255.5], dtype=np.float16)
    k16 = np.ones_like(q16)
    a1, a0 = _digits(q16, k16, np.full(q16.shape, alpha, dtype=np.float32))
    want = np.rint(q16.astype(np.float64)).astype(np.int64)
    assert np.array_equal(256 * a1 + a0, want)


def test_zero_grid_gives_zero_weights():
    # a zero query group (or zero scales): alpha = 0 and every weight must be 0
    q16 = np.zeros(8, dtype=np.float16)
    k16 = np.linspace(0, 3, 8).astype(np.float16)
    a1, a0 = _digits(q16, k16, np.zeros(8, dtype=np.float32))
    assert np.all(256 * a1 + a0 == 0)


def test_extreme_weights():
    # |q kscale| just below 2^x gives the largest weights, +-2048 after rounding
    q16 = np.array([65504.0, -65504.0, 1.0, -1.0], dtype=np.float16)
    k16 = np.array([1.0, 1.0, 0.99951171875, 0.99951171875], dtype=np.float16)
    for i in range(4):
        alpha = _grid(abs(float(q16[i])), float(k16[i]))
        a1, a0 = _digits(q16[i:i + 1], k16[i:i + 1], np.full(1, alpha, dtype=np.float32))
        want = int(np.rint(float(q16[i]) * float(k16[i]) / float(alpha)))
        assert 256 * int(a1[0]) + int(a0[0]) == want
        assert abs(want) <= 2048
