"""Dense attention, the plain definition (test infrastructure only).

[S] Methodology > Problem Setup: s_i = q.k_i / sqrt(d), c* = max_i s_i,
w_i = exp(s_i - c*), D = sum w_i, N = sum w_i v_i, o = N / D, a_i = w_i / D and the
value scale M^2 = sum_i a_i |v_i|^2.
"""

import numpy as np

from .canon import RSQRT_D, csum128


def exact_scores(q16: np.ndarray, K16: np.ndarray, chunk: int = 8192) -> np.ndarray:
    """s_i = (R1 sum of q_t k_it in fp64) * RSQRT_D for every row of K16 [n][128]."""
    qd = q16.astype(np.float64)
    n = K16.shape[0]
    out = np.empty(n, dtype=np.float64)
    for a in range(0, n, chunk):
        out[a:a + chunk] = csum128(qd[None, :] * K16[a:a + chunk].astype(np.float64)) * RSQRT_D
    return out


def dense_attention(q16: np.ndarray, K16: np.ndarray, V16: np.ndarray, n: int) -> dict:
    """Exact attention of one query over the first n cached keys of one KV head."""
    s = exact_scores(q16, K16[:n])
    cstar = float(s.max())
    w = np.exp(s - cstar)
    Vd = V16[:n].astype(np.float64)
    Dn = float(w.sum())
    N = w @ Vd
    o = N / Dn
    vsq = (Vd * Vd).sum(axis=1)
    M = float(np.sqrt((w @ vsq) / Dn))
    return {"s": s, "c_star": cstar, "w": w, "D": Dn, "N": N, "o": o, "M": M}


def dense_attention_heads(Q16: np.ndarray, K16: np.ndarray, V16: np.ndarray, n: int,
                          K64: np.ndarray | None = None, V64: np.ndarray | None = None) -> dict:
    """The same definition for several queries Q16 [G][128] of one KV head at once, with
    the scores and sums taken by fp64 matrix products (for many decode steps; the
    summation order differs from ``exact_scores`` by rounding only).

    K64 / V64 may pass the first n rows already in fp64.
    """
    Kd = K16[:n].astype(np.float64) if K64 is None else K64[:n]
    Vd = V16[:n].astype(np.float64) if V64 is None else V64[:n]
    s = (Kd @ Q16.astype(np.float64).T) * RSQRT_D             # [n][G]
    cstar = s.max(axis=0)
    w = np.exp(s - cstar[None, :])
    Dn = w.sum(axis=0)
    N = w.T @ Vd                                             # [G][128]
    o = N / Dn[:, None]
    vsq = (Vd * Vd).sum(axis=1)
    M = np.sqrt((w.T @ vsq) / Dn)
    return {"c_star": cstar, "D": Dn, "N": N, "o": o, "M": M}
