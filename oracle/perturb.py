"""Exp(1) perturbations from a 53-bit uniform hash (test infrastructure only).

[S] Methodology > Algorithm Components item 1: each pool key gets E_i = -ln u_i with
u_i from a 53-bit uniform hash; [A] and [S] Results > CPU Speed: fresh
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


def perturbations(seed: int, step: int, layer: int, kv_head: int, positions) -> np.ndarray:
    """E_i = -ln u_i (fp64)."""
    return -np.log(uniforms(seed, step, layer, kv_head, positions))
