"""Deterministic lower and upper score bounds from the 4-bit keys (the scan).

[S] Methodology > Algorithm Components item 4: the 4-bit keys give deterministic
upper bounds u_i >= s_i for all scores, and the scan that computes them is integer
dot-product work; [A]: the scan is shared across a GQA group and reads every key.
The pages do not give the bound's formula.  Reading taken (test infrastructure
only; the HIP scan follows the same written rules):

For KV head h, block b, query g of the group (q fp16), channel t:

1. a_gt = q_gt * kscale_bt, exact in fp32 (fp16 x fp16).
2. One power-of-two step per (h, b), shared by the group: m_b = qmax_h * ksmax_b
   (fp32, exact) with qmax_h = max |q| over the group and ksmax_b = max_t kscale_bt.
   If m_b = 0 then alpha_b = 0 and every weight is 0; otherwise m_b = f 2^x with
   f in [0.5, 1) and alpha_b = 2^(x-11).
3. Integer weights a~_gt = rint_half_even(a_gt * 2^(11-x)) in [-2048, 2048]; then
   |a_gt - alpha_b a~_gt| <= alpha_b / 2 for every channel.
4. Per key: I_gi = sum_t a~_gt c_it and C_i = sum_t c_it (exact integers).
5. base_gb = R1-sum_t q_gt kmin_bt (fp64, exact products).
6. qn_g = smallest fp32 y with y^2 >= R1-sum_t q_gt^2 * (1 + 2^-40) (so qn_g >= |q_g|),
   qnp_g = qn_g * (1 + 2^-40); qabs_g = R1-sum_t |q_gt|;
   Kmax_b = max_t (|kmin_bt| + 15 kscale_bt); pad_gb = (2^-40 * qabs_g) * Kmax_b.
7. shat_i = (base_gb + alpha_b I_gi) * RSQRT_D,
   slack_i = ((alpha_b/2 * C_i + qnp_g * kerr_i) + pad_gb) * RSQRT_D,
   UB_i = shat_i + slack_i,  LB_i = shat_i - slack_i   (fp64, in this order).

Validity: q.k = q.k~ + q.(k - k~); q.k~ = base + sum_t a_t c_t; the quantization of
a_t moves that by at most alpha/2 * C_i, Cauchy-Schwarz bounds |q.(k - k~)| by
|q| kerr_i, and the pad terms dominate every fp64 rounding of this computation and
of the exact score's, so LB_i <= s_i <= UB_i holds for the fp64 values.
"""

import numpy as np

from .canon import PADF, RSQRT_D, csum128, fp32_sqrt_up


def query_constants(q16: np.ndarray) -> dict:
    """Per-query constants of step 6 for an array of queries [G][128]."""
    qd = q16.astype(np.float64)
    qn = fp32_sqrt_up(csum128(qd * qd) * (1.0 + PADF)).astype(np.float64)
    qnp = qn * (1.0 + PADF)
    qabs = csum128(np.abs(qd))
    return {"qn": qn, "qnp": qnp, "qabs": qabs}


def block_constants(q16: np.ndarray, kmin16: np.ndarray, kscale16: np.ndarray) -> dict:
    """Steps 1-3, 5 and the block part of 6 for one KV head.

    q16 [G][128]; kmin16, kscale16 [nb][128].  Returns alpha [nb], integer weights
    wts [G][nb][128] (int64), base [G][nb], pad [G][nb].
    """
    G = q16.shape[0]
    qf = q16.astype(np.float32)
    ksf = kscale16.astype(np.float32)
    qmax = np.float32(np.abs(qf).max())
    ksmax = ksf.max(axis=1)                                   # [nb]
    m = (qmax * ksmax).astype(np.float32)                     # exact
    _, x = np.frexp(m)                                        # m = f 2^x, f in [0.5, 1)
    x = x.astype(np.int64)
    alpha = np.where(m > 0, np.ldexp(1.0, x - 11), 0.0)       # fp64, exact powers of two
    a = qf[:, None, :] * ksf[None, :, :]                      # [G][nb][128] fp32, exact
    scale = np.where(m > 0, np.ldexp(np.float32(1.0), (11 - x).astype(np.int32)), np.float32(0.0))
    scaled = (a * scale[None, :, None].astype(np.float32)).astype(np.float32)
    wts = np.rint(scaled).astype(np.int64)
    qd = q16.astype(np.float64)
    kmind = kmin16.astype(np.float64)
    base = csum128(qd[:, None, :] * kmind[None, :, :])       # [G][nb]
    qc = query_constants(q16)
    kmax_b = (np.abs(kmind) + 15.0 * kscale16.astype(np.float64)).max(axis=1)  # [nb]
    pad = (PADF * qc["qabs"])[:, None] * kmax_b[None, :]
    return {"alpha": alpha, "wts": wts, "base": base, "pad": pad, **qc}


def scan_bounds(q16: np.ndarray, packed: dict, h: int, npool: int) -> dict:
    """UB and LB [G][npool] for the pool keys 0..npool-1 of KV head h (step 7)."""
    nb = (npool + 31) // 32
    codes = packed["codes"][h, :32 * nb].astype(np.int64).reshape(nb, 32, 128)
    bc = block_constants(q16, packed["kmin"][h, :nb], packed["kscale"][h, :nb])
    I = np.einsum("gbt,bit->gbi", bc["wts"], codes)          # exact int64
    C = codes.sum(axis=2)                                     # [nb][32]
    kerr = packed["kerr"][h, :32 * nb].astype(np.float64).reshape(nb, 32)
    alpha = bc["alpha"][None, :, None]
    shat = (bc["base"][:, :, None] + alpha * I.astype(np.float64)) * RSQRT_D
    slack = (((alpha / 2.0) * C[None, :, :].astype(np.float64)
              + bc["qnp"][:, None, None] * kerr[None, :, :])
             + bc["pad"][:, :, None]) * RSQRT_D
    UB = (shat + slack).reshape(q16.shape[0], 32 * nb)[:, :npool]
    LB = (shat - slack).reshape(q16.shape[0], 32 * nb)[:, :npool]
    return {"UB": UB, "LB": LB, "I": I.reshape(q16.shape[0], -1)[:, :npool],
            "C": C.reshape(-1)[:npool], "consts": bc}
