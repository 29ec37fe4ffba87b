"""Deterministic lower and upper score bounds from the 4-bit keys (the scan).

[S] Methodology > Algorithm Components item 4: the 4-bit keys give deterministic
upper bounds u_i >= s_i for all scores, and the scan that computes them is integer
dot-product work; [A]: the scan is shared across a GQA group and reads every key.
The pages do not give the bound's formula.  Reading taken (test infrastructure
only; the HIP scan's exact pass follows the same written rules, and its streaming pass
uses fp32 values that can only widen these bounds):

Per call, query g (fp16 q_g):
  Q1. qa_g = max_t |q_gt|; beta_g = 2^(e-11) with qa_g = f 2^e, f in [0.5, 1)
      (beta_g = 0 and q~ = 0 when qa_g = 0); q~_gt = rint_half_even(q_gt / beta_g)
      in [-2048, 2048], so |q_gt - beta_g q~_gt| <= beta_g / 2.
  Q2. qn_g = smallest fp32 y with y^2 >= R1-sum_t q_gt^2 * (1 + 2^-40) (so qn_g >= |q_g|),
      qnp_g = qn_g * (1 + 2^-40); qabs_g = R1-sum_t |q_gt|.
Per KV head h, block b (kappa_b = 2^kexp_b, integer zero points z_bt, kscale_bt):
  B1. One power-of-two step shared by the group: m_b = qmax_h * ksmax_b (fp32, exact)
      with qmax_h = max |q| over the group and ksmax_b = max_t kscale_bt; alpha_b = 0
      when m_b = 0, else alpha_b = 2^(x-11) with m_b = f 2^x, f in [0.5, 1).
  B2. Integer weights a~_gbt = rint_half_even(fp32(q_gt * kscale_bt) * 2^(11-x)) in
      [-2048, 2048]; |q_gt kscale_bt - alpha_b a~_gbt| <= alpha_b / 2.
  B3. base_gb = (beta_g kappa_b) * sum_t q~_gt z_bt (exact integer times a power of two);
      eb_gb = (beta_g / 2) kappa_b sum_t |z_bt| (exact).
  B4. Kmax_b = smallest fp32 value >= max_t (|kappa_b z_bt| + 15 kscale_bt);
      pad_gb = (2^-40 qabs_g) Kmax_b.
Per key i of block b:
  K1. I_gi = sum_t a~_gbt c_it and C_i = sum_t c_it (exact integers).
  K2. shat_i = (base_gb + alpha_b I_gi) * RSQRT_D,
      slack_i = (((alpha_b/2 * C_i + qnp_g * kerr_i) + eb_gb) + pad_gb) * RSQRT_D,
      UB_i = shat_i + slack_i,  LB_i = shat_i - slack_i   (fp64, in this order).

Validity: q.k = q.k~ + q.(k - k~) with q.k~ = sum_t q_t kappa z_t + sum_t q_t kscale_t c_t.
The first sum is base up to eb (Q1), the second is alpha I up to alpha/2 C (B2),
Cauchy-Schwarz bounds |q.(k - k~)| by |q| kerr_i, and the pad dominates every fp64
rounding here and in the exact score, so LB_i <= s_i <= UB_i for the fp64 values.
"""

import numpy as np

from .canon import PADF, RSQRT_D, csum128, fp32_sqrt_up


def fp32_up(x):
    """Smallest fp32 value >= x, as fp64."""
    x = np.asarray(x, dtype=np.float64)
    f = x.astype(np.float32)
    low = f.astype(np.float64) < x
    f = np.where(low, np.nextafter(f, np.float32(np.inf)), f)
    return f.astype(np.float64)


def query_constants(q16: np.ndarray) -> dict:
    """Q1 and Q2 for an array of queries [G][128]."""
    qd = q16.astype(np.float64)
    qn = fp32_sqrt_up(csum128(qd * qd) * (1.0 + PADF)).astype(np.float64)
    qnp = qn * (1.0 + PADF)
    qabs = csum128(np.abs(qd))
    qa = np.abs(qd).max(axis=1)
    _, e = np.frexp(qa)
    beta = np.where(qa > 0, np.ldexp(1.0, e - 11), 0.0)
    qint = np.where(qa[:, None] > 0, np.rint(qd / np.where(beta > 0, beta, 1.0)[:, None]), 0.0)
    return {"qn": qn, "qnp": qnp, "qabs": qabs, "qbeta": beta, "qint": qint.astype(np.int64)}


def block_constants(q16: np.ndarray, packed: dict, h: int, nb: int) -> dict:
    """B1-B4 for blocks 0..nb-1 of KV head h and the group's queries q16 [G][128]."""
    qc = query_constants(q16)
    qf = q16.astype(np.float32)
    ks16 = packed["kscale"][h, :nb]
    ksf = ks16.astype(np.float32)
    qmax = np.float32(np.abs(qf).max())
    ksmax = ksf.max(axis=1)                                   # [nb]
    m = (qmax * ksmax).astype(np.float32)                     # exact
    _, x = np.frexp(m)
    x = x.astype(np.int64)
    alpha = np.where(m > 0, np.ldexp(1.0, x - 11), 0.0)
    scale = np.where(m > 0, np.ldexp(np.float32(1.0), (11 - x).astype(np.int32)), np.float32(0.0))
    a = qf[:, None, :] * ksf[None, :, :]                      # [G][nb][128] fp32, exact
    wts = np.rint((a * scale[None, :, None].astype(np.float32)).astype(np.float32)).astype(np.int64)
    z = packed["z"][h, :nb].astype(np.int64)                  # [nb][128]
    kappa = np.ldexp(1.0, packed["kexp"][h, :nb])             # [nb]
    Bint = qc["qint"] @ z.T                                   # [G][nb] exact
    base = (qc["qbeta"][:, None] * kappa[None, :]) * Bint.astype(np.float64)
    Z1 = np.abs(z).sum(axis=1)
    eb = ((qc["qbeta"][:, None] / 2.0) * kappa[None, :]) * Z1[None, :].astype(np.float64)
    kmin = kappa[:, None] * z.astype(np.float64)
    kmax_b = fp32_up((np.abs(kmin) + 15.0 * ks16.astype(np.float64)).max(axis=1))
    pad = (PADF * qc["qabs"])[:, None] * kmax_b[None, :]
    return {"alpha": alpha, "wts": wts, "base": base, "eb": eb, "pad": pad, "Bint": Bint,
            "Kmax": kmax_b, "Z1": Z1, **qc}


def scan_bounds(q16: np.ndarray, packed: dict, h: int, npool: int) -> dict:
    """UB and LB [G][npool] for the pool keys 0..npool-1 of KV head h (K1, K2)."""
    nb = (npool + 31) // 32
    codes = packed["codes"][h, :32 * nb].astype(np.int64).reshape(nb, 32, 128)
    bc = block_constants(q16, packed, h, nb)
    I = np.einsum("gbt,bit->gbi", bc["wts"], codes)          # exact int64
    C = codes.sum(axis=2)                                     # [nb][32]
    kerr = packed["kerr"][h, :32 * nb].astype(np.float64).reshape(nb, 32)
    alpha = bc["alpha"][None, :, None]
    shat = (bc["base"][:, :, None] + alpha * I.astype(np.float64)) * RSQRT_D
    slack = ((((alpha / 2.0) * C[None, :, :].astype(np.float64)
               + bc["qnp"][:, None, None] * kerr[None, :, :])
              + bc["eb"][:, :, None])
             + bc["pad"][:, :, None]) * RSQRT_D
    G = q16.shape[0]
    UB = (shat + slack).reshape(G, 32 * nb)[:, :npool]
    LB = (shat - slack).reshape(G, 32 * nb)[:, :npool]
    return {"UB": UB, "LB": LB, "I": I.reshape(G, -1)[:, :npool],
            "C": C.reshape(-1)[:npool], "consts": bc}


def refine_bounds8(q16: np.ndarray, packed: dict, h: int, positions) -> dict:
    """8-bit refinement bounds UB8, LB8 [G][len(positions)] of the given keys of KV head h.

    [S] Methodology > Algorithm Components item 4 (8-bit refinement before exact reads).
    Reading taken (the HIP path follows the same written rules):
      S8_gi    = R1-sum_t q_gt * (s8_i * k8_it)   (every product exact in fp64)
      slack8   = (qnp_g * kerr8_i) + 2^-40 * ((128 * s8_i) * qabs_g)
      UB8 = (S8 + slack8) * RSQRT_D,  LB8 = (S8 - slack8) * RSQRT_D   (fp64, this order).
    Validity: q.k = q.k~8 + q.(k - k~8); Cauchy-Schwarz bounds the second term by
    |q| kerr8_i <= qnp kerr8_i; the pad exceeds every fp64 rounding of S8, of the slack
    and of the exact score, all relative to sum_t |q_t| |k_it| <= qabs * 128 s8_i.
    """
    pos = np.asarray(positions, dtype=np.int64)
    qc = query_constants(q16)
    qd = q16.astype(np.float64)
    s8 = packed["s8"][h, pos].astype(np.float64)
    kt = s8[:, None] * packed["k8"][h, pos].astype(np.float64)          # exact
    kerr8 = packed["kerr8"][h, pos].astype(np.float64)
    G = q16.shape[0]
    S8 = np.empty((G, pos.size), dtype=np.float64)
    for g in range(G):
        S8[g] = csum128(qd[g][None, :] * kt) if pos.size else np.empty(0)
    slack = (qc["qnp"][:, None] * kerr8[None, :]) + PADF * ((128.0 * s8)[None, :] * qc["qabs"][:, None])
    return {"UB8": (S8 + slack) * RSQRT_D, "LB8": (S8 - slack) * RSQRT_D, "S8": S8}
