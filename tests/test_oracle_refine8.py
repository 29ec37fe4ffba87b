"""Pins of the 8-bit refinement tier (summary page "Certified Sparse Attention via
Perturbed Retrieval", Methodology > Algorithm Components item 4: an 8-bit tier narrows
the candidates before any exact 16-bit key is read).

What fixes each expected value: exact rational arithmetic (the residual norm bound),
the rounding property of the codes, brute-force exact scores of every pool key (bound
validity, no false negatives of the refined level), and the set relations the reading
implies (the sample and the heavy keys are read exactly; the 8-bit reads contain the
exact ones).
"""

from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from oracle.bounds import refine_bounds8
from oracle.canon import first_level, logtau


def _cases():
    yield synth.config1()
    yield synth.peaked_head(5000, seed=31, G=3)
    yield synth.peaked_head(2100, seed=32, G=7, J=20)
    rng = np.random.default_rng(2)
    _, q, K, V = synth.recipe_layer(rng, 2, 4, 8192, sink=3.5)
    yield synth.Workload("layer2x4", q, K, V, 8192, 4, window=64, r=2, J=40, eps=0.05, delta=0.01)


@pytest.fixture(scope="module")
def cases():
    out = []
    for w in _cases():
        out.append((w, oracle.pack_kv_4bit(w.K, w.V, w.n // 32)))
    return out


def test_pack8_codes_scale_and_residual_bound(cases):
    w, pk = cases[0]
    K = w.K[0].astype(np.float64)
    k8 = pk["k8"][0].astype(np.float64)
    s8 = pk["s8"][0].astype(np.float64)
    assert k8.min() >= -127 and k8.max() <= 127
    # the largest channel of a token uses (almost) the full code range
    assert np.all(np.abs(k8).max(axis=1)[s8 > 0] >= 126)
    # rounding: every channel within half a step (the scale is a rounded fp32 value)
    err = np.abs(K - s8[:, None] * k8)
    assert np.all(err <= 0.5 * s8[:, None] * (1 + 2.0 ** -20))
    # kerr8 >= |k - k~8| exactly, and it is the smallest fp16 that is
    kerr8 = pk["kerr8"][0]
    for i in range(0, K.shape[0], 4):
        res = sum((Fraction(float(K[i, t])) - Fraction(float(s8[i])) * int(k8[i, t])) ** 2 for t in range(128))
        h = Fraction(float(kerr8[i]))
        assert h * h >= res
        prev = np.nextafter(kerr8[i], np.float16(0.0))
        assert Fraction(float(prev)) ** 2 < res or kerr8[i] == 0
    # the 8-bit copy is far finer than the 4-bit one
    assert np.median(pk["kerr8"][0].astype(np.float64)) <= 0.2 * np.median(pk["kerr"][0].astype(np.float64))


def test_bounds8_hold_for_every_key(cases):
    """LB8 <= s <= UB8 for every pool key of every case (brute force), and UB8 is the
    tighter bound on most keys."""
    for w, pk in cases:
        npool = w.n - w.window
        for h in range(w.H_kv):
            qh = w.q[h * w.G:(h + 1) * w.G]
            b8 = refine_bounds8(qh, pk, h, np.arange(npool))
            b4 = oracle.scan_bounds(qh, pk, h, npool)
            for g in range(w.G):
                s = oracle.exact_scores(qh[g], w.K[h, :npool])
                assert np.all(b8["LB8"][g] <= s) and np.all(s <= b8["UB8"][g]), (w.name, h, g)
                assert np.median(b8["UB8"][g] - s) <= 0.2 * np.median(b4["UB"][g] - s)


def test_refined_levels_have_no_false_negatives(cases):
    """For every pool key: l^ub <= l8 <= l, so every key that can be sampled at some
    level up to J is read exactly, and S_j is inside {l8 <= j} inside {l^ub <= j}."""
    for w, pk in cases:
        res = oracle.certified_decode_layer(w.q, w.K, w.V, pk, w.n, w.G, eps=w.eps, delta=w.delta, r=w.r,
                                            J=w.J, window=w.window, seed=w.seed)
        npool = w.n - w.window
        LT = logtau(w.r, w.J)
        for hq, r in enumerate(res):
            t = r["trace"]
            h = hq // w.G
            s = oracle.exact_scores(w.q[hq], w.K[h, :npool])
            l_all = first_level((s + t["E"]) - t["c_star"], LT)
            h_all = first_level(s - t["c_star"], LT)
            cand = t["cand"]
            assert np.all(t["lub"][cand] <= t["l8"])
            assert np.all(t["l8"] <= l_all[cand])
            # keys read exactly carry their true levels; the others can never be sampled
            ex = t["l8"] <= w.J
            np.testing.assert_array_equal(t["l"][ex], l_all[cand][ex])
            np.testing.assert_array_equal(t["h"][ex], h_all[cand][ex])
            assert np.all(l_all[cand][~ex] > w.J)
            assert np.all(t["h"][~ex] == w.J + 1) and np.all(t["l"][~ex] == w.J + 1)
            assert set(np.nonzero(l_all <= w.J)[0].tolist()) <= set(cand[ex].tolist())


def test_keys_read_counts_the_exact_reads(cases):
    """keys read = window + |C_max union {l8 <= j*}|: at least the window plus every key
    sampled or heavy at the stop level, at most the 8-bit reads (l^ub <= j*) plus C_max."""
    fewer = 0
    for w, pk in cases:
        res = oracle.certified_decode_layer(w.q, w.K, w.V, pk, w.n, w.G, eps=w.eps, delta=w.delta, r=w.r,
                                            J=w.J, window=w.window, seed=w.seed)
        for r in res:
            if r["stop_level"] > w.J:
                continue
            t = r["trace"]
            js = r["stop_level"]
            sampled = set(t["cand"][t["l"] <= js].tolist())
            exact = set(t["cand"][t["l8"] <= js].tolist()) | set(t["cmax_pos"].tolist())
            assert sampled <= exact
            assert r["keys_read"] == w.window + len(exact)
            four = set(t["cand"][t["lub"][t["cand"]] <= js].tolist()) | set(t["cmax_pos"].tolist())
            assert exact <= four
            assert r["values_read"] <= r["keys_read"] <= w.window + len(four)
            fewer += r["keys_read"] < w.window + len(four)
    assert fewer > 0
