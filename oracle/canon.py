"""Canonical fp64 arithmetic rules of the oracle (test infrastructure only).

The HIP path follows the same *written* rules; no code is shared.

R1  Every fp64 sum over the 128 channels of a head uses one order: eight
    sequential partial sums over channels 16p .. 16p+15 (starting from channel
    16p), combined as ((p0+p1)+(p2+p3))+((p4+p5)+(p6+p7)).
R2  No fused multiply-add; IEEE round-to-nearest-even in the order written.
R3  fp16 x fp16 products are exact in fp64 (and in fp32).
R4  Constants below.  LOGTAU[j] = (-j * LN2) / r in fp64.
R5  "The first level where x passes" is first(x) = min{ j in [0, J] : x >= LOGTAU[j] },
    J + 1 when there is none (inclusive comparison).

The grid tau_j = 2^(-j/r) and the threshold test s - c* + E >= log tau come from
[S] Methodology > Algorithm Components items 1 and 3.
"""

import numpy as np

LN2 = 0.6931471805599453          # fp64 rounding of ln 2
RSQRT_D = 0.08838834764831845     # fp64 rounding of 1/sqrt(128) = 2^-3.5
PADF = 2.0 ** -40                 # relative pad that dominates fp64 rounding
D = 128


def csum128(x):
    """Sum over the last axis (128 channels) in the R1 order."""
    x = np.asarray(x, dtype=np.float64)
    if x.shape[-1] != D:
        raise ValueError("csum128 expects 128 channels on the last axis")
    parts = []
    for p in range(8):
        acc = x[..., 16 * p].copy()
        for t in range(1, 16):
            acc = acc + x[..., 16 * p + t]
        parts.append(acc)
    return ((parts[0] + parts[1]) + (parts[2] + parts[3])) + ((parts[4] + parts[5]) + (parts[6] + parts[7]))


def logtau(r: int, J: int) -> np.ndarray:
    """LOGTAU[j] = log tau_j = (-j ln 2)/r for j = 0..J (R4)."""
    return np.array([(-float(j) * LN2) / float(r) for j in range(J + 1)], dtype=np.float64)


def tau_table(r: int, J: int) -> np.ndarray:
    """tau_j = exp(LOGTAU[j]): the HT weight that matches the threshold test exactly."""
    return np.exp(logtau(r, J))


def first_level(x, LT: np.ndarray) -> np.ndarray:
    """R5: index of the first grid level whose log-threshold x reaches; J+1 if none.

    LT is strictly decreasing, so the levels x fails are exactly 0..first-1 and
    their count is the answer.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.int32)
    flat_x = x.reshape(-1)
    flat_o = out.reshape(-1)
    step = 1 << 20
    for a in range(0, flat_x.shape[0], step):
        flat_o[a:a + step] = (flat_x[a:a + step, None] < LT[None, :]).sum(axis=1)
    return out


def fp16_sqrt_up(T):
    """Smallest fp16 value h >= 0 with h*h >= T, h*h evaluated exactly in fp64.

    Used for the per-token norm bounds (kerr, vnorm): the result is a valid upper
    bound on sqrt(T) whatever the rounding of any sqrt used to find it.
    """
    T = np.asarray(T, dtype=np.float64)
    with np.errstate(over="ignore"):
        h = np.sqrt(T).astype(np.float16)
    inf16 = np.float16(np.inf)
    while True:
        low = h.astype(np.float64) ** 2 < T
        if not low.any():
            break
        with np.errstate(over="ignore"):
            h = np.where(low, np.nextafter(h, inf16), h)
    while True:
        prev = np.nextafter(h, np.float16(0.0))
        down = (h > 0) & (prev.astype(np.float64) ** 2 >= T)
        if not down.any():
            break
        h = np.where(down, prev, h)
    return h


def fp32_sqrt_up(T):
    """Smallest fp32 value y >= 0 with y*y >= T, y*y evaluated exactly in fp64."""
    T = np.asarray(T, dtype=np.float64)
    y = np.sqrt(T).astype(np.float32)
    inf32 = np.float32(np.inf)
    while True:
        low = y.astype(np.float64) ** 2 < T
        if not low.any():
            break
        y = np.where(low, np.nextafter(y, inf32), y)
    while True:
        prev = np.nextafter(y, np.float32(0.0))
        down = (y > 0) & (prev.astype(np.float64) ** 2 >= T)
        if not down.any():
            break
        y = np.where(down, prev, y)
    return y
