"""Pins of the certificate for each error measure and of Theorem 4.

Sources: the summary page "Certified Sparse Attention via Perturbed Retrieval",
Methodology > Problem Setup (the three error scales: denominator, output norm, value
scale), Methodology > Algorithm Components item 3 (Chernoff interval, Hilbert-space
Bernstein bound, beta, per-level budget) and Theorem 4 (validity per head and per
measure, uniformly over the levels).

What fixes each expected value (none of it is the oracle's own formula typed again):

* the union bound: each level's budget L = ln(T (J+1) / delta) must count every
  one-sided tail the level's bound relies on; the test counts the KL roots the
  certificate actually solves (one tail each) plus the two of Pinelis's inequality;
* Pinelis's tail 2 exp(-t^2 / (2 sigma^2 + 2 b t / 3)) evaluated at the relaxed root;
* each measure's definition, evaluated by brute force over every outcome its event
  allows: the worst case must not exceed beta (and, for the output norm, beta must be
  that worst case);
* closed forms when no light key is sampled (kl(0, mu) = mu, so the count's roots
  are 0 and L exactly), worked by hand below;
* the empirical failure rate of the whole method per measure against exact
  attention, at a loose level (<= the number of tails times e^-L) and at the real
  delta over 1000 seeds on the 4096-token and 32768-token shapes (Theorem 4), with a
  planted mistake in the oracle that must fail the same test.
"""

import math
import multiprocessing as mp
import os

import numpy as np
import pytest

import oracle
import synth
import oracle.certify as cf
from oracle.canon import first_level, logtau
from oracle.decode import level_sums
from oracle.perturb import perturbations

DENOM, OUTNORM, VALUE = cf.MEASURE_DENOM, cf.MEASURE_OUTNORM, cf.MEASURE_VALUE


def _level_inputs(seed=3, k=37):
    """A level with light samples: sums of k random value rows, a heavy part and a window."""
    rng = np.random.default_rng(seed)
    Vs = rng.standard_normal(128) * math.sqrt(k)
    Ps = float(k * 128 + rng.standard_normal() * 10)
    N_det = rng.standard_normal(128) * 0.7
    return dict(D_det=1.7, N_det=N_det, Q_det=1.7 * 130.0, k=k, Vs=Vs, Ps=Ps, tau=2.0 ** -6, Vmax=12.5)


# ---------------------------------------------------------------- budget and Pinelis
@pytest.mark.parametrize("measure", [DENOM, OUTNORM, VALUE])
def test_tail_budget_counts_the_events_each_measure_uses(monkeypatch, measure):
    """T in L = ln(T (J+1)/delta) equals the one-sided tails the level's bound uses."""
    calls = {"n": 0}
    real_u, real_l = cf.kl_upper_root, cf.kl_lower_root

    def upper(x, L):
        calls["n"] += np.atleast_1d(x).size
        return real_u(x, L)

    def lower(x, L):
        calls["n"] += np.atleast_1d(x).size
        return real_l(x, L)

    monkeypatch.setattr(cf, "kl_upper_root", upper)
    monkeypatch.setattr(cf, "kl_lower_root", lower)
    lv = _level_inputs()
    cert = cf.level_certificate(**lv, L=9.0, measure=measure)
    pinelis = 2 if "zeta" in cert else 0          # Pr[|Z| >= t] <= 2 exp(...): two units of e^-L
    events = calls["n"] + pinelis
    assert events == {DENOM: 2, OUTNORM: 5, VALUE: 6}[measure]
    assert cf.tails_per_level(measure) == events
    for J, delta in ((30, 0.01), (48, 0.01), (40, 0.2)):
        L = cf.budget_L(J, delta, measure)
        # J + 1 levels, each failing with probability at most events * e^-L, spend delta
        assert abs((J + 1) * events * math.exp(-L) - delta) <= 1e-12 * delta


@pytest.mark.parametrize("k", [0, 1, 37, 5000])
def test_pinelis_tail_at_the_relaxed_root(k):
    """zeta = sqrt(2 sigma^2 L) + (2/3) b L makes Pinelis's tail at most 2 e^-L."""
    lv = _level_inputs(k=k)
    for L in (math.log(10.0), 9.83, 10.29):
        c = cf.level_certificate(**lv, L=L, measure=VALUE)
        sigma2 = lv["tau"] ** 2 * c["Rc"] ** 2 * c["mu_G"]
        b = lv["tau"] * c["Rc"]
        z = c["zeta"]
        exponent = z * z / (2.0 * sigma2 + 2.0 * b * z / 3.0)
        assert exponent >= L * (1.0 - 1e-12)


# ---------------------------------------------------------------- worst case of each measure
def _denominator_grid():
    for tau in (2.0 ** -3, 2.0 ** -10):
        for D_det in (0.5, 1.0, 10.0, 1000.0):
            for k in (0, 1, 5, 40, 300, 10000):
                yield tau, D_det, k


def test_denominator_beta_covers_the_worst_case_of_its_event():
    """|D^ - D| <= beta D for every D the count's interval allows: D = D_det + tau mu,
    mu in [mu_lo, mu_hi] (the expected light count is D_A / tau)."""
    L = cf.budget_L(40, 0.01, DENOM)
    checked = tight = 0
    for tau, D_det, k in _denominator_grid():
        c = cf.level_certificate(D_det=D_det, N_det=np.zeros(128), Q_det=0.0, k=k, Vs=np.zeros(128), Ps=0.0,
                                 tau=tau, L=L, Vmax=1.0, measure=DENOM)
        if not math.isfinite(c["beta"]):
            assert D_det + tau * k <= c["dD"]
            continue
        mu = np.concatenate([np.linspace(c["mu_lo"], c["mu_hi"], 4001), [c["mu_lo"], c["mu_hi"], float(k)]])
        D = D_det + tau * mu
        worst = float(np.max(np.abs(c["D_hat"] - D) / D))
        assert worst <= c["beta"] * (1.0 + 1e-12), (tau, D_det, k, worst, c["beta"])
        checked += 1
        tight += worst >= c["beta"] * (1.0 - 0.05)
    assert checked >= 30 and tight >= 5


def test_output_norm_beta_covers_the_worst_case_of_its_event():
    """On the event |o^ - o| <= beta_abs (the identity behind beta), |o^ - o| <= beta |o|
    for every such o, and some o on the event's boundary attains beta."""
    for seed, k in ((1, 37), (2, 400), (3, 5)):
        lv = _level_inputs(seed=seed, k=k)
        centre = np.random.default_rng(seed).standard_normal(128)
        lv.update(D_det=20.0, N_det=20.0 * 4.0 * centre / np.linalg.norm(centre), tau=2.0 ** -9)
        c = cf.level_certificate(**lv, L=9.5, measure=OUTNORM)
        ba, on = c["beta_abs"], float(np.linalg.norm(c["o_hat"]))
        assert on > ba and math.isfinite(c["beta"])
        # o = o^ + a e_par + b e_perp: the ratio depends only on (a, b)
        rho = np.linspace(0.0, ba, 401)[:, None]
        th = np.linspace(0.0, 2.0 * math.pi, 721)[None, :]
        a, b = rho * np.cos(th), rho * np.sin(th)
        ratio = np.sqrt(a * a + b * b) / np.sqrt((on + a) ** 2 + b * b)
        worst = float(ratio.max())
        assert worst <= c["beta"] * (1.0 + 1e-12)
        assert worst >= c["beta"] * (1.0 - 1e-9)


# ---------------------------------------------------------------- hand-computed closed forms
def test_certificate_closed_forms_when_no_light_key_is_sampled():
    """k = 0, no light sums.  kl(0, mu) = mu, so mu_lo = 0 and mu_hi = L; y = 0 gives
    mu_G = L; P = 0 gives mu_Q = 0.  o^ = c = N_det / D_det.  Worked by hand:
      dD = tau L;  beta_denom = tau L / (D_det - tau L)
      zeta = sqrt(2 tau^2 Rc^2 L * L) + (2/3) tau Rc L = tau Rc L (sqrt 2 + 2/3)
      beta_abs = zeta / (D_det - tau L)
      beta_outnorm = beta_abs / (|c| - beta_abs)
      M_lo = max(|c| - beta_abs, sqrt(Q_det / (D_det + tau L))), beta_value = beta_abs / M_lo
    with T = 2, 5 and 6 tails in L = ln(T (J+1) / delta)."""
    J, delta, tau = 30, 0.01, 2.0 ** -10
    D_det, Q_det, Vmax = 2.0, 3.0, 2.4
    N_det = np.zeros(128)
    N_det[5] = 0.6 * D_det                     # c = 0.6 e_5, |c| = 0.6, Rc = 3.0
    kw = dict(D_det=D_det, N_det=N_det, Q_det=Q_det, k=0, Vs=np.zeros(128), Ps=0.0, tau=tau, Vmax=Vmax)
    L2, L5, L6 = (math.log(T * (J + 1) / delta) for T in (2, 5, 6))

    c = cf.level_certificate(**kw, L=cf.budget_L(J, delta, DENOM), measure=DENOM)
    assert c["mu_lo"] == 0.0 and c["mu_hi"] == pytest.approx(L2, rel=1e-15)
    assert c["beta"] == pytest.approx(tau * L2 / (D_det - tau * L2), rel=1e-12)

    c = cf.level_certificate(**kw, L=cf.budget_L(J, delta, OUTNORM), measure=OUTNORM)
    beta_abs = tau * 3.0 * L5 * (math.sqrt(2.0) + 2.0 / 3.0) / (D_det - tau * L5)
    assert c["beta_abs"] == pytest.approx(beta_abs, rel=1e-12)
    assert c["beta"] == pytest.approx(beta_abs / (0.6 - beta_abs), rel=1e-12)

    c = cf.level_certificate(**kw, L=cf.budget_L(J, delta, VALUE), measure=VALUE)
    beta_abs = tau * 3.0 * L6 * (math.sqrt(2.0) + 2.0 / 3.0) / (D_det - tau * L6)
    M_lo = max(0.6 - beta_abs, math.sqrt(Q_det / (D_det + tau * L6)))
    assert c["mu_Q"] == 0.0
    assert c["beta"] == pytest.approx(beta_abs / M_lo, rel=1e-12)


# ---------------------------------------------------------------- coverage at a loose level
@pytest.fixture(scope="module")
def small_case():
    w = synth.peaked_head(256, seed=5, G=1, heavy=4, q_mix=0.3)
    d = oracle.dense_attention(w.q[0], w.K[0], w.V[0], w.n)
    npool = w.n - w.window
    V = w.V[0, :w.n].astype(np.float64)
    vsq = (V * V).sum(axis=1)
    wR = d["w"][npool:]
    return {"d": d, "npool": npool, "V": V, "vsq": vsq, "D_R": float(wR.sum()), "N_R": wR @ V[npool:],
            "Q_R": float(wR @ vsq[npool:])}


@pytest.mark.parametrize("measure", [DENOM, OUTNORM, VALUE])
def test_each_measure_covers_at_a_loose_level(small_case, measure):
    """At L = ln 20 (e^-L = 0.05) a level's bound fails at most T e^-L of the time,
    T the measure's tail count; the denominator's event is not vacuous there."""
    N, j, r, J = 4000, 8, 2, 30
    L = math.log(20.0)
    LT = logtau(r, J)
    tau = float(np.exp(LT[j]))
    c, npool, d = small_case, small_case["npool"], small_case["d"]
    s = d["s"][:npool]
    w_pool = d["w"][:npool]
    h = first_level(s - d["c_star"], LT)
    Vmax = float(np.sqrt(c["vsq"][:npool]).max())
    fails = 0
    dens = []
    for sd in range(N):
        E = perturbations(sd, 0, 0, 0, np.arange(npool))
        ll = first_level((s + E) - d["c_star"], LT)
        st = level_sums(j, h, ll, w_pool, c["V"][:npool], c["vsq"][:npool], c["D_R"], c["N_R"], c["Q_R"])
        cert = cf.level_certificate(D_det=st["D_det"], N_det=st["N_det"], Q_det=st["Q_det"], k=st["k"],
                                    Vs=st["Vs"], Ps=st["Ps"], tau=tau, L=L, Vmax=Vmax, measure=measure)
        if measure == DENOM:
            err, scale = abs(cert["D_hat"] - d["D"]), d["D"]
            dens.append(err / d["D"])
        else:
            err = float(np.linalg.norm(cert["o_hat"] - d["o"]))
            scale = float(np.linalg.norm(d["o"])) if measure == OUTNORM else d["M"]
        fails += err > cert["beta"] * scale
    T = cf.tails_per_level(measure)
    bound = T * math.exp(-L)
    assert fails / N <= bound + 4 * math.sqrt(bound * (1 - bound) / N), (fails, N)
    if measure == DENOM:
        assert max(dens) > 0.0          # the estimate is random at this level


# ---------------------------------------------------------------- Theorem 4 at delta
_P12 = {}


def _p12_worker(seeds):
    from threadpoolctl import threadpool_limits
    with threadpool_limits(1):          # one thread per worker process
        return _p12_run(seeds)


def _p12_run(seeds):
    st = _P12
    fails = trials = certified = 0
    for sd in seeds:
        for sc, dense in zip(st["scans"], st["dense"]):
            res = oracle.sample_stage(sc, eps=st["eps"], delta=st["delta"], r=st["r"], J=st["J"], seed=sd,
                                      step=st["step"], layer=0, measure=st["measure"], with_dense=False)
            for g, rr in enumerate(res):
                trials += 1
                if rr["stop_level"] > st["J"]:
                    continue
                certified += 1
                d = dense[g]
                if st["measure"] == DENOM:
                    err = abs(rr["trace"]["levels"][rr["stop_level"]]["D_hat"] - d["D"])
                    scale = d["D"]
                else:
                    err = float(np.linalg.norm(rr["o_hat"] - d["o"]))
                    scale = float(np.linalg.norm(d["o"])) if st["measure"] == OUTNORM else d["M"]
                fails += err > st["eps"] * scale
    return fails, trials, certified


def _failure_rate(w, heads, measure, seeds, shrink=1.0):
    """Rate of (certified and error > eps x the measure's scale) over seeds x query heads,
    the seed-independent scan done once per KV head.  ``shrink`` plants a mistake in the
    oracle: every level's beta divided by it."""
    packed = oracle.pack_kv_4bit(w.K, w.V, w.n // 32)
    scans, dense = [], []
    for h in heads:
        qh = w.q[h * w.G:(h + 1) * w.G]
        scans.append(oracle.scan_stage(qh, w.K[h], w.V[h], packed, h, w.n, window=w.window))
        dense.append([oracle.dense_attention(qh[g], w.K[h], w.V[h], w.n) for g in range(w.G)])
    _P12.clear()
    _P12.update(scans=scans, dense=dense, eps=w.eps, delta=w.delta, r=w.r, J=w.J, step=w.step,
                measure=measure)
    real = oracle.decode.level_certificates
    if shrink != 1.0:
        def shrunk(*a, **kw):
            out = real(*a, **kw)
            for c in out:
                c["beta"] = c["beta"] / shrink
            return out
        oracle.decode.level_certificates = shrunk
    try:
        seeds = list(seeds)
        nproc = max(1, min(8, os.cpu_count() or 1, len(seeds)))
        parts = [seeds[i::nproc] for i in range(nproc)]
        if nproc == 1:
            out = [_p12_worker(parts[0])]
        else:
            with mp.get_context("fork").Pool(nproc) as pool:
                out = pool.map(_p12_worker, parts)
    finally:
        oracle.decode.level_certificates = real
    return tuple(sum(x[i] for x in out) for i in range(3))


def _bar(delta, trials):
    return delta + 4.0 * math.sqrt(delta * (1.0 - delta) / trials)


@pytest.mark.parametrize("measure", [DENOM, OUTNORM, VALUE])
def test_theorem4_per_measure_config1_shape(cfg1, measure):
    """1000 seeds x 4 query heads of the 4096-token parity shape: failure rate <= delta
    (+ 4 standard errors, which is below 2 delta here)."""
    fails, trials, certified = _failure_rate(cfg1, [0], measure, range(1000))
    assert trials == 4000 and _bar(0.01, trials) <= 0.02
    assert certified >= 0.9 * trials
    assert fails / trials <= _bar(0.01, trials), (fails, trials)


def test_theorem4_32k_layer_shape():
    """1000 seeds x the 4 query heads of one KV head of the 32768-token layer."""
    w = synth.config2()
    fails, trials, certified = _failure_rate(w, [0], VALUE, range(1000))
    assert trials == 4000
    assert certified >= 0.9 * trials
    assert fails / trials <= _bar(0.01, trials), (fails, trials)


@pytest.mark.parametrize("measure", [DENOM, OUTNORM, VALUE])
def test_theorem4_detects_a_planted_mistake_per_measure(cfg1, measure):
    """The same test with every beta divided by 30 in the oracle must fail."""
    fails, trials, _ = _failure_rate(cfg1, [0], measure, range(100), shrink=30.0)
    assert fails / trials > _bar(0.01, trials), (fails, trials)
