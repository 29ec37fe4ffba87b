"""Pins of the oracle's sampling, estimation and certificate steps.

What fixes each expected value: the exact dense maximum (brute force), the
threshold-sampling law Pr[i in S(tau)] = min(1, w_i/tau) (Theoretical Foundation),
Theorem 1 (unbiasedness, Var D^ = sum_A w(tau - w) <= tau D_A), nesting of the
samples, the tau -> 0 limit, the algebraic identity behind beta, a library root
finder for the KL roots, nominal coverage of each tail at a loose level and
Theorem 2 (samples and keys read bounded independently of n).  Theorem 4 and the
per-measure pins are in test_oracle_measures.py.
"""

import math

import numpy as np
import pytest

import oracle
import synth
from oracle.canon import first_level, logtau
from oracle.certify import level_certificate
from oracle.decode import level_sums
from oracle.perturb import perturbations


def _decode(w, packed=None, **over):
    packed = oracle.pack_kv_4bit(w.K, w.V, w.n // 32) if packed is None else packed
    kw = dict(eps=w.eps, delta=w.delta, r=w.r, J=w.J, window=w.window, seed=w.seed,
              step=w.step, layer=w.layer)
    kw.update(over)
    return oracle.certified_decode_layer(w.q, w.K, w.V, packed, w.n, w.G, **kw)


# ---------------------------------------------------------------- P5, P6
def test_exact_max_and_no_false_negatives(cfg1, cfg1_packed):
    res = _decode(cfg1, cfg1_packed)
    npool = cfg1.n - cfg1.window
    LT = logtau(cfg1.r, cfg1.J)
    for g, r in enumerate(res):
        tr, d = r["trace"], r["dense"]
        assert tr["c_star"] == d["c_star"]                     # P5: exact maximum
        s_pool = d["s"][:npool]
        if s_pool.max() >= tr["c_R"]:
            assert int(np.argmax(s_pool)) in set(tr["cmax_pos"].tolist())
        l_all = first_level((s_pool + tr["E"]) - tr["c_star"], LT)
        h_all = first_level(s_pool - tr["c_star"], LT)
        assert np.all(tr["lub"] <= l_all)                      # l^ub <= l for every key
        assert np.all(l_all <= h_all)                          # B_j subset of S_j
        cand = set(tr["cand"].tolist())
        assert set(np.nonzero(l_all <= cfg1.J)[0].tolist()) <= cand
        # levels recomputed on the candidates agree with brute force
        np.testing.assert_array_equal(tr["l"], l_all[tr["cand"]])
        np.testing.assert_array_equal(tr["h"], h_all[tr["cand"]])
        assert r["stop_level"] <= cfg1.J and r["beta"] <= cfg1.eps


def test_nesting_and_small_tau_limit():
    """S_j grows with j; with tau_J below every weight, A_J is empty and o^_J = o."""
    w = synth.peaked_head(256, seed=21, G=2)
    res = _decode(w, r=1, J=60, eps=1e-300)                     # never certifies: all levels kept
    for r in res:
        lv = r["trace"]["levels"]
        assert len(lv) == 61 and r["stop_level"] == 61
        ns = [x["n_sample"] for x in lv]
        nh = [x["n_heavy"] for x in lv]
        assert ns == sorted(ns) and nh == sorted(nh)
        assert all(h <= s for h, s in zip(nh, ns))
        last = lv[-1]
        assert last["k"] == 0 and last["n_heavy"] == w.n - w.window
        np.testing.assert_allclose(last["o_hat"], r["dense"]["o"], rtol=1e-12, atol=1e-13)
        assert abs(last["D_hat"] - r["dense"]["D"]) <= 1e-12 * r["dense"]["D"]


# ---------------------------------------------------------------- P7, P8 (threshold sampling)
@pytest.fixture(scope="module")
def small_case():
    w = synth.peaked_head(256, seed=5, G=1, heavy=4, q_mix=0.3)
    d = oracle.dense_attention(w.q[0], w.K[0], w.V[0], w.n)
    npool = w.n - w.window
    s = d["s"]
    V = w.V[0, :w.n].astype(np.float64)
    vsq = (V * V).sum(axis=1)
    wR = d["w"][npool:]
    return {"w": w, "d": d, "npool": npool, "s": s, "V": V, "vsq": vsq,
            "D_R": float(wR.sum()), "N_R": wR @ V[npool:], "Q_R": float(wR @ vsq[npool:])}


def _samples(case, seeds, j, r=2, J=30):
    LT = logtau(r, J)
    npool, s, c = case["npool"], case["s"], case["d"]["c_star"]
    h = first_level(s[:npool] - c, LT)
    out = []
    for sd in seeds:
        E = perturbations(sd, 0, 0, 0, np.arange(npool))
        ll = first_level((s[:npool] + E) - c, LT)
        out.append((ll, h))
    return out, float(np.exp(LT[j]))


def test_inclusion_frequency_matches_pps(small_case):
    N, j = 10000, 6
    samp, tau = _samples(small_case, range(N), j)
    freq = np.mean([ll <= j for ll, _ in samp], axis=0)
    p = np.minimum(1.0, small_case["d"]["w"][:small_case["npool"]] / tau)
    se = np.sqrt(np.maximum(p * (1 - p), 1.0 / N) / N)
    assert np.all(np.abs(freq - p) <= 4 * se + 1e-12)
    assert 0.05 < p.mean() < 0.95 or np.any((p > 0.05) & (p < 0.95))


def test_ht_unbiased_with_theorem1_variance(small_case):
    N = 10000
    npool = small_case["npool"]
    w_pool = small_case["d"]["w"][:npool]
    Vp, vsqp = small_case["V"][:npool], small_case["vsq"][:npool]
    D_true, N_true = small_case["d"]["D"], small_case["d"]["N"]
    for j in (0, 4, 8, 12, 16):
        samp, tau = _samples(small_case, range(N), j)
        Dh, Nh = [], []
        for ll, h in samp:
            st = level_sums(j, h, ll, w_pool, Vp, vsqp, small_case["D_R"], small_case["N_R"],
                            small_case["Q_R"])
            Dh.append(st["D_det"] + tau * st["k"])
            Nh.append(st["N_det"] + tau * st["Vs"])
        Dh, Nh = np.array(Dh), np.array(Nh)
        light = w_pool < tau
        var_th = float((w_pool[light] * (tau - w_pool[light])).sum())
        assert var_th <= tau * float(w_pool[light].sum()) + 1e-15     # Theorem 1's bound
        if var_th == 0:
            assert np.all(Dh == Dh[0]) and abs(Dh[0] - D_true) <= 1e-12 * D_true
            continue
        assert abs(Dh.mean() - D_true) <= 4 * math.sqrt(var_th / N)
        assert abs(Dh.var() - var_th) <= 6 * var_th * math.sqrt(2.0 / N) + 1e-15
        se = Nh.std(axis=0) / math.sqrt(N) + 1e-15
        assert np.all(np.abs(Nh.mean(axis=0) - N_true) <= 4.5 * se)


# ---------------------------------------------------------------- P10 identity behind beta
def test_beta_identity(cfg1, cfg1_packed):
    """o^ - o = [Z_c + (o^ - c)(D - D^)] / D with Z_c = sum_A (tau X - w)(v - c)."""
    res = _decode(cfg1, cfg1_packed, eps=1e-300)
    npool = cfg1.n - cfg1.window
    LT = logtau(cfg1.r, cfg1.J)
    V = cfg1.V[0, :npool].astype(np.float64)
    for r in res[:2]:
        tr, d = r["trace"], r["dense"]
        s_pool = d["s"][:npool]
        w_pool = np.exp(s_pool - d["c_star"])
        l_all = first_level((s_pool + tr["E"]) - d["c_star"], LT)
        h_all = first_level(s_pool - d["c_star"], LT)
        for j in (3, 9, 15, 24):
            lv = tr["levels"][j]
            tau = float(np.exp(LT[j]))
            A = h_all > j
            X = (l_all <= j).astype(np.float64)
            c = lv["c"]
            Zc = ((tau * X[A] - w_pool[A])[:, None] * (V[A] - c)).sum(axis=0)
            lhs = lv["o_hat"] - d["o"]
            rhs = (Zc + (lv["o_hat"] - c) * (d["D"] - lv["D_hat"])) / d["D"]
            np.testing.assert_allclose(lhs, rhs, atol=1e-10 * d["M"], rtol=0)
            # the deterministic parts are the sums over R and B_j
            np.testing.assert_allclose(lv["D_det"], tr["D_R"] + w_pool[~A].sum(), rtol=1e-12)


# ---------------------------------------------------------------- KL roots
def test_kl_roots_match_library_root_finder():
    from scipy.optimize import brentq
    for L in (math.log(10.0), 9.83, 10.29):
        for x in (0.0, 1e-3, 0.5, 1.0, 7.0, 123.0, 8000.0):
            f = lambda mu: oracle.kl(x, mu) - L  # noqa: E731
            hi = brentq(f, x if x > 0 else 1e-300, x + 10 * L + 10 * math.sqrt(x * L) + 10,
                        xtol=1e-14, rtol=1e-15)
            got = float(oracle.kl_upper_root(x, L)[0])
            assert got >= hi * (1 - 1e-13) and got <= hi * (1 + 1e-12)
            lo = float(oracle.kl_lower_root(x, L)[0])
            if x == 0:
                assert lo == 0.0
            elif oracle.kl(x, 1e-300) > L:
                want = brentq(f, 1e-300, x, xtol=1e-300, rtol=1e-15)
                assert lo <= want * (1 + 1e-13) and lo >= want * (1 - 1e-12)
    assert float(oracle.kl_upper_root(0.0, 3.0)[0]) == pytest.approx(3.0, rel=1e-14)


# ---------------------------------------------------------------- P11 tail coverage
def test_certificate_tails_cover_at_loose_level(small_case):
    """At L = ln 10 each tail fails at most at its nominal rate (2e^-L or e^-L)."""
    N, j = 10000, 8
    L = math.log(10.0)
    npool = small_case["npool"]
    w_pool = small_case["d"]["w"][:npool]
    Vp, vsqp = small_case["V"][:npool], small_case["vsq"][:npool]
    vnorm = np.sqrt(vsqp)
    Vmax = float(vnorm.max())
    samp, tau = _samples(small_case, range(N), j)
    miss_mu = miss_z = miss_g = miss_q = 0
    A = w_pool < tau
    mu_true = float(w_pool[A].sum()) / tau
    Q_A = float((w_pool[A] * vsqp[A]).sum())
    for ll, h in samp:
        st = level_sums(j, h, ll, w_pool, Vp, vsqp, small_case["D_R"], small_case["N_R"],
                        small_case["Q_R"])
        cert = level_certificate(D_det=st["D_det"], N_det=st["N_det"], Q_det=st["Q_det"], k=st["k"],
                                 Vs=st["Vs"], Ps=st["Ps"], tau=tau, L=L, Vmax=Vmax)
        miss_mu += not (cert["mu_lo"] <= mu_true <= cert["mu_hi"])
        c = cert["c"]
        X = (ll <= j).astype(np.float64)
        Zc = ((tau * X[A] - w_pool[A])[:, None] * (Vp[A] - c)).sum(axis=0)
        G_A = float((w_pool[A] * ((Vp[A] - c) ** 2).sum(axis=1)).sum())
        zeta_true = math.sqrt(2 * tau * G_A * L) + (2.0 / 3.0) * tau * cert["Rc"] * L
        miss_z += float(np.sqrt(Zc @ Zc)) > zeta_true
        miss_g += G_A > tau * cert["Rc"] ** 2 * cert["mu_G"]
        miss_q += Q_A < tau * Vmax * Vmax * cert["mu_Q"]
    for miss, nominal in ((miss_mu, 0.2), (miss_z, 0.2), (miss_g, 0.1), (miss_q, 0.1)):
        rate = miss / N
        assert rate <= nominal + 4 * math.sqrt(nominal * (1 - nominal) / N), (miss_mu, miss_z, miss_g, miss_q)
    assert miss_mu > 0                     # the interval is not vacuous at this level


# ---------------------------------------------------------------- P13 Theorem 2
def _p13_layer(n):
    """One KV head (4 queries) of the 32768-token layer's recipe at context n: sink of
    3.5 nats on tokens 0-3 and 1 % power-law heavy hitters along the mean query."""
    rng = np.random.default_rng(2)
    _, q, K, V = synth.recipe_layer(rng, 1, 4, n, sink=3.5)
    return synth.Workload(f"p13.{n}", q, K, V, n, 4, window=64, r=2, J=40, eps=0.05, delta=0.01)


@pytest.mark.slow
def test_keys_read_flat_in_context_length():
    """Theorem 2 on the 32768-token layer's generator at n = 16K..128K: the median keys
    read grows by at most 1.3x while n grows 4x (32K -> 128K), and the values read stay
    within a fixed multiple of m = 2 L eps^-2."""
    from oracle.certify import budget_L
    m = 2.0 * budget_L(40, 0.01, 2) / 0.05 ** 2
    keys = {}
    for n in (16384, 32768, 65536, 131072):
        w = _p13_layer(n)
        res = _decode(w, with_dense=False)
        assert all(r["stop_level"] <= w.J for r in res)
        keys[n] = float(np.median([r["keys_read"] for r in res]))
        assert max(r["values_read"] - w.window for r in res) <= 3.0 * m
    assert keys[131072] / keys[32768] <= 1.3, keys


@pytest.mark.slow
def test_light_samples_bounded_independent_of_context_length():
    """Theorem 2 where all keys are light-ish (no heavy hitters, scores spread by a
    query of twice the usual norm): the light samples k at the stop level never exceed
    3 m, m = 2 L eps^-2, at any n, and the keys read stay within a fixed multiple of the
    values read (the 4-bit candidates around each sampled key).

    On this generator the sample itself still grows with n over 16K..128K, because the
    light share of the attention mass rises (about 0.45 -> 0.75) and k approaches its
    n-free ceiling from below; the keys read follow it (about 1.9x from 32K to 128K).
    """
    from oracle.certify import budget_L
    eps = 0.1
    m = 2.0 * budget_L(30, 0.01, 2) / eps ** 2
    for n in (16384, 32768, 65536, 131072):
        w = synth.peaked_head(n, seed=9, G=4, heavy=0, eps=eps, q_scale=2.0)
        res = _decode(w, eps=eps, with_dense=False)
        for r in res:
            assert r["stop_level"] <= w.J
            lv = r["trace"]["levels"][r["stop_level"]]
            assert lv["k"] <= 3.0 * m, (n, lv["k"], m)
            assert r["values_read"] - w.window <= 3.0 * m
            assert r["keys_read"] <= 6.0 * r["values_read"], (n, r["keys_read"], r["values_read"])
