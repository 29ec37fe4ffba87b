"""Exp(1) perturbations from hashed uniforms (test infrastructure only).

[S] Methodology > Algorithm Components item 1: each pool key gets E_i = -ln u_i, the
uniform u_i taken from 53 bits of a hash; [A] and [S] Results > CPU Speed: fresh
perturbations at every decoding step.  The hash itself is not given.  Reading
taken: a chain of the SplitMix64 generator's output function (Steele, Lea and
Flood, "Fast splittable pseudorandom number generators", OOPSLA 2014, with the
"Mix13" finalizer of Vigna's public reference version) over
(seed, step, layer, kv_head, position):

    h0 = mix(seed), h1 = mix(h0 ^ step), h2 = mix(h1 ^ layer),
    h3 = mix(h2 ^ kv_head), h_i = mix(h3 ^ position),

where mix(x) adds the golden-ratio increment to x and applies the finalizer.
u_i = ((h_i >> 11) + 1) * 2^-53 lies in (0, 1], so E_i = -ln u_i is finite.  E_i
has no query-head index: the whole GQA group shares it.

ln is evaluated by one written specification, the algorithm of fdlibm's e_log.c
(Sun Microsystems, 1993: x = 2^k (1 + f), s = f / (2 + f), a degree-14 odd
polynomial in s with coefficients Lg1..Lg7, ln 2 split in two parts), in fp64
without fused operations, so that every implementation of it gives the same bits.
"""

import numpy as np

GAMMA = 0x9E3779B97F4A7C15
M1 = 0xBF58476D1CE4E5B9
M2 = 0x94D049BB133111EB
MASK = (1 << 64) - 1


def splitmix64_mix(x: int) -> int:
    """One SplitMix64 step applied to state x: returns the generator's output."""
    z = (x + GAMMA) & MASK
    z = ((z ^ (z >> 30)) * M1) & MASK
    z = ((z ^ (z >> 27)) * M2) & MASK
    return z ^ (z >> 31)


def hash_prefix(seed: int, step: int, layer: int, kv_head: int) -> int:
    h = splitmix64_mix(seed & MASK)
    h = splitmix64_mix(h ^ (step & MASK))
    h = splitmix64_mix(h ^ (layer & MASK))
    return splitmix64_mix(h ^ (kv_head & MASK))


def _mix_vec(z: np.ndarray) -> np.ndarray:
    z = z + np.uint64(GAMMA)
    z = (z ^ (z >> np.uint64(30))) * np.uint64(M1)
    z = (z ^ (z >> np.uint64(27))) * np.uint64(M2)
    return z ^ (z >> np.uint64(31))


def uniforms(seed: int, step: int, layer: int, kv_head: int, positions) -> np.ndarray:
    """u_i in (0, 1] for the given token positions (fp64, exact)."""
    pre = np.uint64(hash_prefix(seed, step, layer, kv_head))
    pos = np.asarray(positions, dtype=np.uint64)
    with np.errstate(over="ignore"):
        h = _mix_vec(pre ^ pos)
    return ((h >> np.uint64(11)) + np.uint64(1)).astype(np.float64) * 2.0 ** -53


# The steps and constants of log_spec follow fdlibm's e_log.c, which carries this notice:
#   Copyright (C) 1993 by Sun Microsystems, Inc. All rights reserved.
#   Developed at SunPro, a Sun Microsystems, Inc. business.
#   Permission to use, copy, modify, and distribute this software is freely granted,
#   provided that this notice is preserved.


def _f64(bits: int) -> float:
    return float(np.array([bits], dtype=np.uint64).view(np.float64)[0])


LN2_HI = _f64(0x3FE62E42FEE00000)
LN2_LO = _f64(0x3DEA39EF35793C76)
LG1 = _f64(0x3FE5555555555593)
LG2 = _f64(0x3FD999999997FA04)
LG3 = _f64(0x3FD2492494229359)
LG4 = _f64(0x3FCC71C51D8E78AF)
LG5 = _f64(0x3FC7466496CB03DE)
LG6 = _f64(0x3FC39A09D078C69F)
LG7 = _f64(0x3FC2F112DF3E5244)


def log_spec(x) -> np.ndarray:
    """ln x for normal positive fp64 x by the fdlibm e_log steps (vectorised)."""
    x = np.asarray(x, dtype=np.float64)
    bits = x.view(np.uint64)
    hx = (bits >> np.uint64(32)).astype(np.int64)
    lx = bits & np.uint64(0xFFFFFFFF)
    k = (hx >> 20) - 1023
    hx = hx & 0x000FFFFF
    i = (hx + 0x95F64) & 0x100000
    hi_new = (hx | (i ^ 0x3FF00000)).astype(np.uint64)
    xn = ((hi_new << np.uint64(32)) | lx).view(np.float64)
    k = k + (i >> 20)
    f = xn - 1.0
    dk = k.astype(np.float64)
    # |f| < 2^-20
    small = (0x000FFFFF & (2 + hx)) < 3
    r_small = f * f * (0.5 - 0.33333333333333333 * f)
    res_small = np.where(f == 0.0,
                         np.where(k == 0, 0.0, dk * LN2_HI + dk * LN2_LO),
                         np.where(k == 0, f - r_small, dk * LN2_HI - ((r_small - dk * LN2_LO) - f)))
    s = f / (2.0 + f)
    z = s * s
    ii = hx - 0x6147A
    w = z * z
    j = 0x6B851 - hx
    t1 = w * (LG2 + w * (LG4 + w * LG6))
    t2 = z * (LG1 + w * (LG3 + w * (LG5 + w * LG7)))
    ii = ii | j
    R = t2 + t1
    hfsq = 0.5 * f * f
    res_a = np.where(k == 0, f - (hfsq - s * (hfsq + R)),
                     dk * LN2_HI - ((hfsq - (s * (hfsq + R) + dk * LN2_LO)) - f))
    res_b = np.where(k == 0, f - s * (f - R), dk * LN2_HI - ((s * (f - R) - dk * LN2_LO) - f))
    return np.where(small, res_small, np.where(ii > 0, res_a, res_b))


def perturbations(seed: int, step: int, layer: int, kv_head: int, positions) -> np.ndarray:
    """E_i = -ln u_i (fp64, ln by the written specification above)."""
    return -log_spec(uniforms(seed, step, layer, kv_head, positions))
