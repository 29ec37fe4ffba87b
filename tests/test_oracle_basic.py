"""Pins of the oracle's deterministic parts against things other than itself.

Each test names what fixes the expected value: a library routine, exact rational
arithmetic, brute force over every key, published generator outputs, or a
statistical law.
"""

import os
import subprocess
import sys
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle.bounds import block_constants
from oracle.canon import fp16_sqrt_up, fp32_sqrt_up
from oracle.pack import zero_points

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


# ---------------------------------------------------------------- P1 dense attention
def test_dense_matches_library_softmax(cfg1):
    """Problem Setup's o = N/D and M^2 = sum a |v|^2 against torch's fp64 softmax."""
    q = torch.from_numpy(cfg1.q.astype(np.float64))
    K = torch.from_numpy(cfg1.K[0].astype(np.float64))
    V = torch.from_numpy(cfg1.V[0].astype(np.float64))
    a = torch.softmax((q @ K.T) / np.sqrt(128.0), dim=-1)
    o_ref = (a @ V).numpy()
    M_ref = torch.sqrt(a @ (V * V).sum(dim=1)).numpy()
    for g in range(cfg1.G):
        d = oracle.dense_attention(cfg1.q[g], cfg1.K[0], cfg1.V[0], cfg1.n)
        np.testing.assert_allclose(d["o"], o_ref[g], rtol=1e-12, atol=1e-13)
        assert abs(d["M"] - M_ref[g]) <= 1e-12 * M_ref[g]
        s_ref = ((q[g] @ K.T) / np.sqrt(128.0)).numpy()
        np.testing.assert_allclose(d["s"], s_ref, rtol=1e-13, atol=1e-13)
        assert d["c_star"] == d["s"].max()


def test_dense_ragged_n(cfg1):
    """Only the first n keys count: a key appended after n must not change o."""
    for n in (1, 33, 100, 4095):
        d = oracle.dense_attention(cfg1.q[0], cfg1.K[0], cfg1.V[0], n)
        q = torch.from_numpy(cfg1.q[0].astype(np.float64))
        K = torch.from_numpy(cfg1.K[0, :n].astype(np.float64))
        V = torch.from_numpy(cfg1.V[0, :n].astype(np.float64))
        o_ref = (torch.softmax(K @ q / np.sqrt(128.0), dim=0) @ V).numpy()
        np.testing.assert_allclose(d["o"], o_ref, rtol=1e-12, atol=1e-13)


def test_dense_heads_matches_library_softmax(cfg1):
    """The several-queries form of the same definition against torch's fp64 softmax,
    at full length and at a ragged n."""
    q = torch.from_numpy(cfg1.q.astype(np.float64))
    for n in (cfg1.n, 1001):
        K = torch.from_numpy(cfg1.K[0, :n].astype(np.float64))
        V = torch.from_numpy(cfg1.V[0, :n].astype(np.float64))
        a = torch.softmax((q @ K.T) / np.sqrt(128.0), dim=-1)
        d = oracle.dense_attention_heads(cfg1.q, cfg1.K[0], cfg1.V[0], n)
        np.testing.assert_allclose(d["o"], (a @ V).numpy(), rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(d["M"], torch.sqrt(a @ (V * V).sum(dim=1)).numpy(), rtol=1e-12)


# ---------------------------------------------------------------- P2 pack
def test_pack_codes_and_block_metadata(cfg1, cfg1_packed):
    pk = cfg1_packed
    K = cfg1.K[0].astype(np.float64).reshape(-1, 32, 128)
    codes = pk["codes"][0].reshape(-1, 32, 128).astype(np.float64)
    kmin = zero_points(pk)[0]
    kappa = np.ldexp(1.0, pk["kexp"][0])[:, None]
    ks = pk["kscale"][0].astype(np.float64)
    assert codes.min() >= 0 and codes.max() <= 15
    z = pk["z"][0].astype(np.int64)
    assert z.min() >= -2048 and z.max() <= 2047
    # zero point: the block minimum rounded down onto the block's power-of-two grid
    mn = K.min(axis=1)
    assert np.all(kmin <= mn) and np.all(mn - kmin < kappa)
    # the grid is as fine as 12 bits allow: the largest |min| needs more than 10 bits
    assert np.all(np.abs(mn).max(axis=1) >= 1024 * kappa[:, 0])
    # kscale is the fp16 value nearest to (max - kmin)/15: within 15 half-ulps
    span = K.max(axis=1) - kmin
    ulp = np.spacing(pk["kscale"][0]).astype(np.float64)
    assert np.all(np.abs(15.0 * ks - span) <= 15.0 * ulp / 2 + 1e-30)
    # Every code is a nearest grid point: |k - k~| <= kscale/2 unless clamped at an end.
    ktil = kmin[:, None, :] + ks[:, None, :] * codes
    err = np.abs(K - ktil)
    inner = (codes > 0) & (codes < 15)
    assert np.all(err[inner] <= ks[:, None, :].repeat(32, 1)[inner] / 2 * (1 + 1e-12))


def test_pack_norm_bounds_exact_rational(cfg1, cfg1_packed):
    """kerr >= |k - k~| and vnorm >= |v| in exact rational arithmetic, and tight."""
    pk = cfg1_packed
    rng = np.random.default_rng(11)
    toks = rng.choice(cfg1.n, size=1000, replace=False)
    for i in toks:
        b = i // 32
        k = [Fraction(float(x)) for x in cfg1.K[0, i]]
        kappa = Fraction(2) ** int(pk["kexp"][0, b])
        kmin = [kappa * int(x) for x in pk["z"][0, b]]
        ks = [Fraction(float(x)) for x in pk["kscale"][0, b]]
        c = [int(x) for x in pk["codes"][0, i]]
        res2 = sum((k[t] - kmin[t] - ks[t] * c[t]) ** 2 for t in range(128))
        kerr = Fraction(float(pk["kerr"][0, i]))
        assert kerr * kerr >= res2
        prev = Fraction(float(np.nextafter(pk["kerr"][0, i], np.float16(0))))
        if kerr > 0:
            assert prev * prev < res2 * (1 + Fraction(1, 2 ** 30))
        v2 = sum(Fraction(float(x)) ** 2 for x in cfg1.V[0, i])
        vn = Fraction(float(pk["vnorm"][0, i]))
        assert vn * vn >= v2
        prev = Fraction(float(np.nextafter(pk["vnorm"][0, i], np.float16(0))))
        assert prev * prev < v2 * (1 + Fraction(1, 2 ** 30))


def test_pack_degenerate_blocks():
    """A constant block gives kscale 0, codes 0 and kerr 0; a two-valued block is exact."""
    K = np.zeros((1, 64, 128), dtype=np.float16)
    K[0, :32] = np.float16(0.75)
    K[0, 32:] = np.float16(-1.5)
    K[0, 40, 5] = np.float16(2.25)
    V = np.ones((1, 64, 128), dtype=np.float16)
    pk = oracle.pack_kv_4bit(K, V, 2)
    assert np.all(pk["kscale"][0, 0] == 0) and np.all(pk["codes"][0, :32] == 0)
    assert np.all(pk["kerr"][0, :32] == 0)
    assert pk["kscale"][0, 1, 5] == np.float16(3.75 / 15)
    assert pk["codes"][0, 40, 5] == 15 and np.all(pk["kerr"][0, 32:] == 0)
    # sqrt(128) = 11.3137...; the next fp16 value above it is 11.3203125 (ulp 2^-7)
    assert np.all(pk["vnorm"][0] == np.float16(11.3203125))


def test_sqrt_up_helpers_are_minimal():
    rng = np.random.default_rng(3)
    T = np.concatenate([rng.exponential(200.0, 5000), [0.0, 1.0, 2.0, 65504.0 ** 2, 1e12]])
    h = fp16_sqrt_up(T).astype(np.float64)
    assert np.all(h * h >= T)
    prev = np.nextafter(fp16_sqrt_up(T), np.float16(0)).astype(np.float64)
    assert np.all((h == 0) | (prev * prev < T))
    y = fp32_sqrt_up(T[:-1]).astype(np.float64)
    assert np.all(y * y >= T[:-1])


# ---------------------------------------------------------------- P3 score bounds
def _check_bounds(w, packed, max_heads=None):
    npool = w.n - w.window
    for h in range(w.H_kv if max_heads is None else max_heads):
        qg = w.q[h * w.G:(h + 1) * w.G]
        b = oracle.scan_bounds(qg, packed, h, npool)
        for g in range(w.G):
            s = oracle.exact_scores(qg[g], w.K[h, :npool])
            assert np.all(b["LB"][g] <= s), (h, g)
            assert np.all(s <= b["UB"][g]), (h, g)
            yield float(np.mean(b["UB"][g] - s))


def test_bounds_hold_for_every_key_config1(cfg1, cfg1_packed):
    slack = list(_check_bounds(cfg1, cfg1_packed))
    assert max(slack) < 2.0          # not vacuous: about a nat on N(0,1) keys


def test_bounds_hold_for_every_key_config2():
    w = synth.config2()
    pk = oracle.pack_kv_4bit(w.K, w.V, w.n // 32)
    slack = list(_check_bounds(w, pk))
    assert len(slack) == 32 and max(slack) < 2.5


def test_bounds_integer_weights(cfg1, cfg1_packed):
    """|q*kscale - alpha*w| <= alpha/2 with |w| <= 2048; |q - beta*q~| <= beta/2."""
    qg = cfg1.q
    nb = cfg1.n // 32
    bc = block_constants(qg, cfg1_packed, 0, nb)
    a = qg.astype(np.float64)[:, None, :] * cfg1_packed["kscale"][0].astype(np.float64)[None]
    alpha = bc["alpha"][None, :, None]
    assert np.abs(bc["wts"]).max() <= 2048
    assert np.all(np.abs(a - alpha * bc["wts"]) <= alpha / 2)
    assert np.abs(bc["wts"]).max() >= 512       # the step is not needlessly coarse
    qd = qg.astype(np.float64)
    beta = bc["qbeta"][:, None]
    assert np.all(np.abs(qd - beta * bc["qint"]) <= beta / 2)
    assert np.all(np.abs(bc["qint"]).max(axis=1) >= 1024)
    # the offset term is exact: base equals q~ . kmin times beta, in exact arithmetic
    kmin = zero_points(cfg1_packed)[0]
    for g in range(cfg1.G):
        for b in (0, 7, nb - 1):
            exact = sum(Fraction(int(bc["qint"][g, t])) * Fraction(float(kmin[b, t])) for t in range(128))
            assert Fraction(float(bc["base"][g, b])) == exact * Fraction(float(bc["qbeta"][g]))


def test_bounds_planted_mistake_is_caught(cfg1, cfg1_packed):
    """Dropping the Cauchy-Schwarz term (kerr = 0) must make the brute-force check fail."""
    pk = dict(cfg1_packed)
    pk["kerr"] = np.zeros_like(pk["kerr"])
    with pytest.raises(AssertionError):
        list(_check_bounds(cfg1, pk))


# ---------------------------------------------------------------- P4 hash
def _golden_splitmix():
    out = {}
    with open(os.path.join(ROOT, "tests", "golden", "splitmix64.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            parts = line.split()
            out[int(parts[0], 0)] = [int(x, 0) for x in parts[1:]]
    return out


def test_splitmix64_published_outputs():
    from oracle.perturb import GAMMA, MASK, splitmix64_mix
    for seed, want in _golden_splitmix().items():
        x, got = seed, []
        for _ in want:
            got.append(splitmix64_mix(x))
            x = (x + GAMMA) & MASK
        assert got == want


def test_vectorised_hash_matches_scalar():
    from oracle.perturb import hash_prefix, splitmix64_mix, uniforms
    pre = hash_prefix(0x5EED, 7, 3, 5)
    pos = np.array([0, 1, 2, 31, 4095, 131071, 2 ** 31 - 1])
    u = uniforms(0x5EED, 7, 3, 5, pos)
    for p, uu in zip(pos, u):
        h = splitmix64_mix(pre ^ int(p))
        assert uu == ((h >> 11) + 1) * 2.0 ** -53


def test_hash_independent_of_python_hash_seed():
    code = ("import sys; sys.path.insert(0, %r); import numpy as np; from oracle.perturb import perturbations;"
            "print(perturbations(0x5EED, 3, 2, 1, np.arange(1000)).tobytes().hex()[:4000])" % ROOT)
    outs = []
    for hs in ("0", "12345"):
        env = dict(os.environ, PYTHONHASHSEED=hs)
        outs.append(subprocess.run([sys.executable, "-c", code], env=env, capture_output=True,
                                   text=True, check=True).stdout)
    assert outs[0] == outs[1] and len(outs[0]) > 100


def test_hash_uniform_and_exponential():
    from scipy import stats
    from oracle.perturb import uniforms
    u = uniforms(0x5EED, 0, 0, 0, np.arange(200000))
    assert u.min() > 0 and u.max() <= 1
    assert stats.kstest(u, "uniform").pvalue > 1e-3
    E = -np.log(u)
    assert abs(E.mean() - 1) < 4 * 1 / np.sqrt(u.size)
    assert abs(E.var() - 1) < 4 * np.sqrt(8 / u.size)
    # different steps, heads and layers give unrelated streams
    u2 = uniforms(0x5EED, 1, 0, 0, np.arange(200000))
    assert abs(np.corrcoef(u, u2)[0, 1]) < 0.02


def test_log_spec_within_one_ulp_of_exact():
    """ln by the written specification vs 40-digit decimal logarithms (correctly rounded)."""
    from decimal import Decimal, getcontext
    from oracle.perturb import log_spec, uniforms
    getcontext().prec = 40
    u = np.concatenate([uniforms(0x5EED, 0, 0, 0, np.arange(3000)),
                        [1.0, 0.5, 0.25, 2.0 ** -53, 1 - 2.0 ** -53, 0.75, 1 - 2.0 ** -21, 1 - 2.0 ** -19]])
    got = log_spec(u)
    for x, g in zip(u, got):
        exact = float(Decimal(float(x)).ln())          # correctly rounded to the nearest double
        assert abs(g - exact) <= np.spacing(abs(exact)) or g == exact, (x, g, exact)
    assert log_spec(np.array([1.0]))[0] == 0.0
    assert log_spec(np.array([0.5]))[0] == -0.6931471805599453
    # the Exp(1) law: mean and variance of E = -ln u stay 1 with this ln
    E = -log_spec(uniforms(0x5EED, 0, 0, 0, np.arange(200000)))
    assert abs(E.mean() - 1) < 4 / np.sqrt(E.size)
