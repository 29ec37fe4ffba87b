"""Per-level certificates (test infrastructure only).

[S] Methodology > Algorithm Components item 3 fixes the shape: on the grid
tau_j = 2^(-j/r) with a per-level failure budget, a Chernoff interval for the number
of light samples, a sum of independent Bernoulli draws (denominator), a Bernstein-type
concentration bound for vectors in a Hilbert space on
Z_c = sum_{i in A} (tau X_i - w_i)(v_i - c) (numerator), the output bound
beta = (zeta + |o^ - c| dD) / (D^ - dD), and a stop at the first certified level.
[S] Theorem 4: validity per head and per error measure, uniformly over levels.
[S] Problem Setup: the three error scales (denominator, output norm, value scale).

Readings taken where the pages leave the completion open:

* Budget: each level spends delta/(J+1), split evenly over its one-sided tails;
  L = ln(T (J+1) / delta) with T = 6 tails for the value scale (2 for the count,
  2 for the Pinelis bound, 1 for the variance proxy, 1 for the lower bound on M),
  T = 5 for the output norm and T = 2 for the denominator.
* kl(x, mu) = mu - x + x ln(x / mu) (0 ln 0 = 0): the Chernoff exponent of a sum of
  independent [0, 1] variables with mean mu (Poisson-dominated moment bound).
  mu_hi is the root above x and mu_lo the root below x (0 when x = 0).
* Denominator: dD = tau max(k - mu_lo, mu_hi - k), D_hi = D_det + tau mu_hi.
* Centre c = N_det / D_det (fixed before sampling); R_c = Vmax + |c|.
* Variance proxy: y = (P - 2 c.V + k |c|^2) / R_c^2 clamped at 0, mu_G the root
  above y, sigma^2 = tau^2 R_c^2 mu_G, b = tau R_c.
* Pinelis: zeta = sqrt(2 sigma^2 L) + (2/3) b L.
* beta_abs = (zeta + |o^ - c| dD) / (D^ - dD), +inf when D^ <= dD.
* Value scale: mu_Q the root below P / Vmax^2, Q_lo = Q_det + tau Vmax^2 mu_Q,
  M_lo = max(|o^| - beta_abs, sqrt(Q_lo / D_hi)), beta = beta_abs / M_lo.
  Output norm: beta = beta_abs / (|o^| - beta_abs).  Denominator:
  beta = dD / (D^ - dD).  Non-positive denominators give +inf.
"""

import math

import numpy as np

MEASURE_DENOM, MEASURE_OUTNORM, MEASURE_VALUE = 0, 1, 2


def tails_per_level(measure: int) -> int:
    return {MEASURE_DENOM: 2, MEASURE_OUTNORM: 5, MEASURE_VALUE: 6}[measure]


def budget_L(J: int, delta: float, measure: int) -> float:
    return math.log(tails_per_level(measure) * (J + 1) / delta)


def kl(x, mu):
    """Poisson-form Chernoff exponent kl(x, mu) = mu - x + x ln(x/mu), 0 ln 0 = 0."""
    x = np.asarray(x, dtype=np.float64)
    mu = np.asarray(mu, dtype=np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        t = np.where(x > 0, x * np.log(x / mu), 0.0)
    return mu - x + t


def kl_upper_root(x, L):
    """Smallest representable mu >= root of kl(x, mu) = L above x (bisection)."""
    x = np.atleast_1d(np.asarray(x, dtype=np.float64)).copy()
    lo = x.copy()
    hi = np.maximum(2.0 * x, x + 1.0)
    while True:
        short = kl(x, hi) < L
        if not short.any():
            break
        hi = np.where(short, 2.0 * hi, hi)
    for _ in range(2000):
        mid = 0.5 * (lo + hi)
        moved = (mid > lo) & (mid < hi)
        if not moved.any():
            break
        above = kl(x, mid) >= L
        hi = np.where(moved & above, mid, hi)
        lo = np.where(moved & ~above, mid, lo)
    return hi


def kl_lower_root(x, L):
    """Largest representable mu <= root of kl(x, mu) = L below x; 0 when x = 0."""
    x = np.atleast_1d(np.asarray(x, dtype=np.float64)).copy()
    lo = np.zeros_like(x)
    hi = x.copy()
    for _ in range(2000):
        mid = 0.5 * (lo + hi)
        moved = (mid > lo) & (mid < hi)
        if not moved.any():
            break
        above = kl(x, mid) >= L          # mid at or below the root
        lo = np.where(moved & above, mid, lo)
        hi = np.where(moved & ~above, mid, hi)
    return np.where(x > 0, lo, 0.0)


def _root_inputs(D_det, N_det, k, Vs, Ps, Vmax, measure):
    """What the level's four KL roots are taken of: the light-sample count k (denominator
    interval), y (variance proxy) and P / Vmax^2 (lower bound on Q)."""
    k = float(k)
    pre = {"k": k}
    if measure == MEASURE_DENOM:
        return pre
    c = N_det / D_det
    cn = float(np.sqrt(c @ c))
    Rc = Vmax + cn
    if Rc > 0:
        y = max((Ps - 2.0 * float(c @ Vs) + k * cn * cn) / (Rc * Rc), 0.0)
    else:
        y = 0.0
    pre.update({"c": c, "Rc": Rc, "y": y})
    if measure == MEASURE_VALUE:
        pre["yq"] = Ps / (Vmax * Vmax) if Vmax > 0 else 0.0
    return pre


def _certificate_from_roots(*, D_det, N_det, Q_det, Vs, tau, L, Vmax, measure, pre, roots):
    """The level's bound once its roots are known (the arithmetic of one level)."""
    k = pre["k"]
    D_hat = D_det + tau * k
    N_hat = N_det + tau * Vs
    o_hat = N_hat / D_hat
    mu_hi, mu_lo = roots["mu_hi"], roots["mu_lo"]
    dD = tau * max(k - mu_lo, mu_hi - k)
    D_hi = D_det + tau * mu_hi
    out = {"D_hat": D_hat, "N_hat": N_hat, "o_hat": o_hat, "dD": dD, "mu_hi": mu_hi, "mu_lo": mu_lo}
    if measure == MEASURE_DENOM:
        out["beta"] = dD / (D_hat - dD) if D_hat > dD else math.inf
        return out
    c, Rc, y = pre["c"], pre["Rc"], pre["y"]
    mu_G = roots["mu_G"]
    sigma2 = tau * tau * Rc * Rc * mu_G
    b = tau * Rc
    zeta = math.sqrt(2.0 * sigma2 * L) + (2.0 / 3.0) * b * L
    diff = o_hat - c
    dn = float(np.sqrt(diff @ diff))
    beta_abs = (zeta + dn * dD) / (D_hat - dD) if D_hat > dD else math.inf
    on = float(np.sqrt(o_hat @ o_hat))
    out.update({"c": c, "Rc": Rc, "y": y, "mu_G": mu_G, "zeta": zeta, "beta_abs": beta_abs})
    if measure == MEASURE_OUTNORM:
        out["beta"] = beta_abs / (on - beta_abs) if on > beta_abs else math.inf
        return out
    mu_Q = roots["mu_Q"]
    Q_lo = Q_det + tau * Vmax * Vmax * mu_Q
    M_lo = max(on - beta_abs, math.sqrt(Q_lo / D_hi))
    out.update({"mu_Q": mu_Q, "Q_lo": Q_lo, "M_lo": M_lo})
    out["beta"] = beta_abs / M_lo if (M_lo > 0 and math.isfinite(beta_abs)) else math.inf
    return out


def _roots(pres, L, measure):
    """The KL roots of several levels at once (the bisections run elementwise, so each
    level's roots are the same as when it is solved alone)."""
    k = np.array([p["k"] for p in pres], dtype=np.float64)
    cols = {"mu_hi": kl_upper_root(k, L), "mu_lo": kl_lower_root(k, L)}
    if measure != MEASURE_DENOM:
        cols["mu_G"] = kl_upper_root(np.array([p["y"] for p in pres], dtype=np.float64), L)
    if measure == MEASURE_VALUE:
        cols["mu_Q"] = kl_lower_root(np.array([p["yq"] for p in pres], dtype=np.float64), L)
    return [{name: float(v[i]) for name, v in cols.items()} for i in range(len(pres))]


def level_certificate(*, D_det, N_det, Q_det, k, Vs, Ps, tau, L, Vmax, measure=MEASURE_VALUE):
    """Certificate at one level from the deterministic and sampled sums.

    D_det, Q_det, Ps scalars; N_det, Vs vectors [128]; k the light-sample count.
    """
    pre = _root_inputs(D_det, N_det, k, Vs, Ps, Vmax, measure)
    roots = _roots([pre], L, measure)[0]
    return _certificate_from_roots(D_det=D_det, N_det=N_det, Q_det=Q_det, Vs=Vs, tau=tau, L=L, Vmax=Vmax,
                                   measure=measure, pre=pre, roots=roots)


def level_certificates(stats, taus, L, Vmax, measure=MEASURE_VALUE):
    """``level_certificate`` of every level in ``stats`` (dicts with D_det, N_det, Q_det,
    k, Vs, Ps) at thresholds ``taus``; the roots of all levels are solved together."""
    pres = [_root_inputs(st["D_det"], st["N_det"], st["k"], st["Vs"], st["Ps"], Vmax, measure) for st in stats]
    roots = _roots(pres, L, measure) if pres else []
    return [_certificate_from_roots(D_det=st["D_det"], N_det=st["N_det"], Q_det=st["Q_det"], Vs=st["Vs"],
                                    tau=float(tau), L=L, Vmax=Vmax, measure=measure, pre=pre, roots=rt)
            for st, tau, pre, rt in zip(stats, taus, pres, roots)]
