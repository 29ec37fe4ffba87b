"""Batched certified calls: every kernel of the path launched once for several items.

Items are requests with their own context length, target and hash inputs, or layers of
one request, each reading its own slot of one cache tensor ([S] Results > CPU Speed:
fresh perturbations per step; [S] Algorithm Components item 1: the hash inputs).  Each
item is compared with the oracle (the single-call bar: stop levels and keys read exact,
beta within 1e-4, o_hat within 1e-3 M) and with a single call on the same item (the same
stop levels and keys read; floats equal up to the order of the level sums).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from test_gpu_parity import _to

pytestmark = pytest.mark.gpu

D = 128


def _csa():
    import certified_sparse_attention_amd as csa
    return csa


def _say(msg):
    import sys
    print(f"[batch] {msg}", file=sys.stderr, flush=True)


def _build(specs, H_kv, G, n_cap, slots, J=40, seed0=900):
    """specs: (n, eps, q_scale, step, layer) per item; slots: the item's cache slot (items
    sharing a slot share its keys and values).  Returns the cache, queries and items."""
    S = max(slots) + 1
    K = np.zeros((S, H_kv, n_cap, D), dtype=np.float16)
    V = np.zeros((S, H_kv, n_cap, D), dtype=np.float16)
    made = {}
    items, qs = [], []
    for i, ((n, eps, q_scale, step, layer), s) in enumerate(zip(specs, slots)):
        rng = np.random.default_rng(seed0 + i)
        _, q, Ks, Vs = synth.recipe_layer(rng, H_kv, G, n, n_cap=n_cap, sink=3.0, q_scale=q_scale)
        if s not in made:
            K[s], V[s] = Ks, Vs
            made[s] = True
        qs.append(q)
        items.append(dict(n=n, slot=s, eps=eps, seed=seed0 + 7 * i, step=step, layer=layer))
    return K, V, np.stack(qs), items


def _oracle_item(K, V, q, it, G, J, pk_cache):
    s = it["slot"]
    if s not in pk_cache:
        pk_cache[s] = oracle.pack_kv_4bit(K[s], V[s], K.shape[2] // 32)
    return oracle.certified_decode_layer(q, K[s], V[s], pk_cache[s], it["n"], G, eps=it["eps"], delta=0.01, r=2,
                                         J=J, window=64, seed=it["seed"], step=it["step"], layer=it["layer"])


def _run_batch(K, V, q, items, G, J, **kw):
    csa = _csa()
    S, H_kv, n_cap, _ = K.shape
    Kd, Vd = _to(K), _to(V)
    packed = csa.pack_kv_4bit(Kd.view(S * H_kv, n_cap, D), Vd.view(S * H_kv, n_cap, D))
    out = csa.certified_decode_attention_batch(_to(q), Kd, Vd, packed, items, delta=0.01, r=2, J=J, window=64, **kw)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in out], (Kd, Vd, packed)


def _check_item(b, res, ref, J):
    o_hat, beta, stop, keys = (x[b] for x in res)
    for hq, r in enumerate(ref):
        M = r["dense"]["M"]
        assert int(stop[hq]) == r["stop_level"], (b, hq, int(stop[hq]), r["stop_level"])
        assert int(keys[hq]) == r["keys_read"], (b, hq, int(keys[hq]), r["keys_read"])
        assert np.linalg.norm(o_hat[hq].astype(np.float64) - r["o_hat"]) <= 1e-3 * M, (b, hq)
        if r["stop_level"] <= J:
            assert abs(beta[hq] - r["beta"]) <= 1e-4 * abs(r["beta"]), (b, hq)
        else:
            assert beta[hq] == 0.0


def _check_against_single(res, dev, q, items, G, J):
    """Each item of the batch against a single call on its own slot."""
    csa = _csa()
    Kd, Vd, packed = dev
    S, H_kv, n_cap, _ = Kd.shape
    for b, it in enumerate(items):
        s = it["slot"]
        sub = packed.slot(S, s)
        one = csa.certified_decode_attention(_to(q[b]), Kd[s], Vd[s], sub, it["n"], eps=it["eps"], delta=0.01, r=2,
                                             J=J, window=64, seed=it["seed"], step=it["step"], layer=it["layer"])
        torch.cuda.synchronize()
        o1, b1, s1, k1 = (t.cpu().numpy() for t in one)
        np.testing.assert_array_equal(res[2][b], s1, err_msg=f"stop levels of item {b}")
        np.testing.assert_array_equal(res[3][b], k1, err_msg=f"keys read of item {b}")
        np.testing.assert_allclose(res[1][b], b1, rtol=1e-9, atol=0, err_msg=f"beta of item {b}")
        np.testing.assert_allclose(res[0][b], o1, rtol=1e-5, atol=1e-6, err_msg=f"o_hat of item {b}")


SMALL_SPECS = [
    # (n, eps, q_scale, step, layer)
    (3001, 0.05, 1.0, 0, 0),
    (5990, 0.02, 0.1, 3, 1),     # near-flat
    (40, 0.1, 1.0, 0, 2),        # n <= window: exact
    (4500, 0.1, 1.0, 7, 3),
    (2300, 0.05, 0.1, 1, 4),     # near-flat
    (64, 0.05, 1.0, 0, 5),       # n = window
    (65, 0.05, 1.0, 2, 6),       # one pool key
    (6000, 0.05, 1.0, 9, 7),
    (3001, 0.05, 1.0, 1, 0),     # the first item's slot at the next step
]
SMALL_SLOTS = [3, 0, 5, 1, 7, 2, 6, 4, 3]


@pytest.fixture(scope="module")
def small_batch():
    G, J = 4, 40
    K, V, q, items = _build(SMALL_SPECS, 2, G, 6016, SMALL_SLOTS, J=J)
    pk_cache = {}
    refs = [_oracle_item(K, V, q[b], it, G, J, pk_cache) for b, it in enumerate(items)]
    return K, V, q, items, refs, G, J


def test_ragged_batch_matches_oracle(small_batch):
    K, V, q, items, refs, G, J = small_batch
    _say(f"{len(items)} items, n = {[it['n'] for it in items]}")
    res, _ = _run_batch(K, V, q, items, G, J)
    for b, ref in enumerate(refs):
        _check_item(b, res, ref, J)


def test_ragged_batch_matches_single_calls(small_batch):
    K, V, q, items, refs, G, J = small_batch
    res, dev = _run_batch(K, V, q, items, G, J)
    _check_against_single(res, dev, q, items, G, J)


@pytest.mark.parametrize("budgets", [(1, 0), (4, 40), (300, 0)])
def test_ragged_batch_budgets_do_not_change_results(small_batch, budgets):
    K, V, q, items, refs, G, J = small_batch
    base, _ = _run_batch(K, V, q, items, G, J)
    res, _ = _run_batch(K, V, q, items, G, J, cand_budget=budgets[0], cand_budget2=budgets[1])
    np.testing.assert_array_equal(res[2], base[2])
    np.testing.assert_array_equal(res[3], base[3])
    for b, ref in enumerate(refs):
        _check_item(b, res, ref, J)


def test_batch_of_windows_only():
    G, J = 3, 20
    specs = [(1, 0.05, 1.0, 0, 0), (33, 0.1, 1.0, 1, 1), (64, 0.02, 1.0, 2, 2)]
    K, V, q, items = _build(specs, 2, G, 128, [0, 1, 2], J=J)
    res, _ = _run_batch(K, V, q, items, G, J)
    pk_cache = {}
    for b, it in enumerate(items):
        ref = _oracle_item(K, V, q[b], it, G, J, pk_cache)
        _check_item(b, res, ref, J)
        assert np.all(res[2][b] == 0) and np.all(res[3][b] == it["n"])


def test_layers_of_one_step_in_one_call():
    """Four layers of one decode step (8 KV heads x GQA 4, n = 8192), each its own slot
    and layer index: one call, each layer against the oracle."""
    G, J, n = 4, 40, 8192
    specs = [(n, 0.05, 1.0, 5, layer) for layer in range(4)]
    K, V, q, items = _build(specs, 8, G, n, list(range(4)), J=J, seed0=1200)
    res, _ = _run_batch(K, V, q, items, G, J)
    pk_cache = {}
    for b, it in enumerate(items):
        _say(f"layer {b}")
        _check_item(b, res, _oracle_item(K, V, q[b], it, G, J, pk_cache), J)


def test_batch_is_deterministic(small_batch):
    K, V, q, items, refs, G, J = small_batch
    a, _ = _run_batch(K, V, q, items, G, J)
    b, _ = _run_batch(K, V, q, items, G, J)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)
