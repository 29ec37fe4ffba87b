"""Full-size parity: the HIP path against the oracle at the workloads' real sizes.

* the 128K Llama-shaped layer the bench times (8 KV heads x GQA 4), layers 0 and 31,
  every query head;
* all 16 requests of the ragged batch (n from 16K to 128K, per-request epsilon, odd
  requests near-flat), every query head, as 16 single calls and as one batched call; the
  oracle side of each request runs in CPU worker processes while the GPU side runs;
* the appending Qwen-shaped layer (4 KV heads x GQA 7, n = 131072 + t) with fresh
  perturbations each step, packing each block as an append completes it: parity at
  steps 0, 1, 33 and 255, and over all 256 steps the rate of certified heads whose
  error exceeds eps M against the oracle's fp64 exact attention.

The same call the bench times is used, with the trace on; sets, counts, stop levels
and keys read are compared bit for bit, floats to the stated tolerances.
"""
import math
import multiprocessing as mp
import os
import sys
from concurrent.futures import ProcessPoolExecutor

import numpy as np
import pytest
import torch

import oracle
import synth
from test_gpu_parity import DEV, _compare_decode, _kw, _to, pad_cache

pytestmark = pytest.mark.gpu


def _csa():
    import certified_sparse_attention_amd as csa
    return csa


def _say(msg):
    print(f"[fullsize] {msg}", file=sys.stderr, flush=True)


def _gpu_call(w, **over):
    q, K, V = _to(w.q), _to(w.K), _to(w.V)
    packed = _csa().pack_kv_4bit(K, V)
    kw = _kw(w, **over)
    out = _csa().certified_decode_attention(q, K, V, packed, w.n, trace=True, **kw)
    torch.cuda.synchronize()
    return out, kw


def _run_layer(w, **over):
    _say(f"{w.name}: n={w.n} H_kv={w.H_kv} G={w.G} eps={w.eps} J={w.J}")
    w = pad_cache(w)
    pk_ref = oracle.pack_kv_4bit(w.K, w.V, w.n_cap // 32)
    out, kw = _gpu_call(w, **over)
    return _compare_decode(w, pk_ref, out[:4], out[4], **kw)


@pytest.mark.parametrize("layer", [0, 31])
def test_llama_layer_128k(layer):
    ref = _run_layer(synth.config3_layer(layer), step=3)
    assert len(ref) == 32


# ---------------------------------------------------------------- the ragged batch
@pytest.fixture(scope="module")
def ragged_refs():
    import _oracle_jobs
    workers = max(1, min(8, os.cpu_count() or 1))
    ex = ProcessPoolExecutor(max_workers=workers, mp_context=mp.get_context("spawn"))
    futs = {b: ex.submit(_oracle_jobs.ragged_request_reference, b) for b in range(16)}
    yield futs
    ex.shutdown(wait=False, cancel_futures=True)


@pytest.mark.parametrize("b", list(range(16)))
def test_ragged_request(b, ragged_refs):
    w = pad_cache(synth.config4_request(b))
    _say(f"{w.name}: n={w.n} eps={w.eps} flat={w.extra['flat']}")
    out, kw = _gpu_call(w)
    ref = ragged_refs[b].result()
    _compare_decode(w, None, out[:4], out[4], ref=ref, **kw)
    assert len(ref) == w.H_q


def test_ragged_batch_in_one_call(ragged_refs):
    """All 16 requests in one batched call (each its own cache slot, n, eps and seed),
    every request's heads against the oracle."""
    csa = _csa()
    ws = [pad_cache(synth.config4_request(b)) for b in range(16)]
    n_cap = max(w.n_cap for w in ws)
    K = torch.zeros((16, 8, n_cap, 128), dtype=torch.float16, device=DEV)
    V = torch.zeros_like(K)
    for b, w in enumerate(ws):
        K[b, :, :w.n_cap] = _to(w.K)
        V[b, :, :w.n_cap] = _to(w.V)
    q = _to(np.stack([w.q for w in ws]))
    packed = csa.pack_kv_4bit(K.view(16 * 8, n_cap, 128), V.view(16 * 8, n_cap, 128))
    items = [dict(n=w.n, slot=b, eps=w.eps, seed=w.seed, step=w.step, layer=w.layer) for b, w in enumerate(ws)]
    _say(f"ragged batch: n = {[w.n for w in ws]}")
    out = csa.certified_decode_attention_batch(q, K, V, packed, items, delta=0.01, r=2, J=48, window=64)
    torch.cuda.synchronize()
    o_hat, beta, stop, keys = (t.cpu().numpy() for t in out)
    for b, w in enumerate(ws):
        ref = ragged_refs[b].result()
        for hq, r in enumerate(ref):
            assert int(stop[b, hq]) == r["stop_level"], (b, hq)
            assert int(keys[b, hq]) == r["keys_read"], (b, hq)
            assert np.linalg.norm(o_hat[b, hq].astype(np.float64) - r["o_hat"]) <= 1e-3 * r["dense"]["M"], (b, hq)
            if r["stop_level"] <= 48:
                assert abs(beta[b, hq] - r["beta"]) <= 1e-4 * abs(r["beta"]), (b, hq)
    del K, V, packed


# ---------------------------------------------------------------- the appending layer
STEPS = 256


@pytest.fixture(scope="module")
def appending():
    """The Qwen-shaped layer with room for 256 appends, on the GPU, packed up to n0."""
    w = pad_cache(synth.config5_base(steps=STEPS))
    n0 = w.n
    K, V = _to(w.K), _to(w.V)
    packed = _csa().pack_kv_4bit(K, V, block_end=n0 // 32)
    torch.cuda.synchronize()
    return {"w": w, "n0": n0, "K": K, "V": V, "packed": packed, "nb": n0 // 32}


def _advance(app, t):
    """Pack the blocks the appends up to step t have completed (and only those)."""
    while (app["n0"] + t) // 32 > app["nb"]:
        _csa().pack_kv_4bit(app["K"], app["V"], app["packed"], block_begin=app["nb"], block_end=app["nb"] + 1)
        app["nb"] += 1


def _step_call(app, t, trace):
    w = app["w"]
    n = app["n0"] + t
    q16 = synth.config5_step_query(w, t)
    wt = synth.Workload(f"config5.t{t}", q16, w.K, w.V, n, w.G, window=w.window, r=w.r, J=w.J,
                        eps=w.eps, delta=w.delta, step=t)
    kw = _kw(wt)
    out = _csa().certified_decode_attention(_to(q16), app["K"], app["V"], app["packed"], n, trace=trace, **kw)
    return wt, kw, out


def test_appending_gqa7_layer_parity(appending):
    """Parity at steps 0, 1, 33 and 255: the block of tokens n0..n0+31 is packed when step
    32 completes it, so later steps scan it from the packed cache."""
    app = appending
    w = app["w"]
    for t in (0, 1, 33, 255):
        _advance(app, t)
        pk_ref = oracle.pack_kv_4bit(w.K, w.V, app["nb"])
        _say(f"config5 step {t}: n={app['n0'] + t}, packed blocks {app['nb']}")
        wt, kw, out = _step_call(app, t, True)
        torch.cuda.synchronize()
        _compare_decode(wt, pk_ref, out[:4], out[4], **kw)


def test_appending_gqa7_256_steps_failure_rate(appending):
    """All 256 steps: #(certified and |o^ - o| > eps M) / (256 x 28) <= delta (+ 4 standard
    errors), o and M from the oracle's fp64 exact attention of each step."""
    app = appending
    w = app["w"]
    H_q, J = w.H_q, w.J
    o_all = torch.empty((STEPS, H_q, 128), dtype=torch.float32, device=app["K"].device)
    stop_all = torch.empty((STEPS, H_q), dtype=torch.int32, device=app["K"].device)
    for t in range(STEPS):
        _advance(app, t)
        _, _, out = _step_call(app, t, False)
        o_all[t].copy_(out[0])
        stop_all[t].copy_(out[2])
        if t % 64 == 63:
            torch.cuda.synchronize()
            _say(f"config5 256-step run: {t + 1} steps done")
    torch.cuda.synchronize()
    o_all, stop_all = o_all.cpu().numpy().astype(np.float64), stop_all.cpu().numpy()
    n_last = app["n0"] + STEPS - 1
    K64 = [w.K[h, :n_last + 1].astype(np.float64) for h in range(w.H_kv)]
    V64 = [w.V[h, :n_last + 1].astype(np.float64) for h in range(w.H_kv)]
    fails = certified = 0
    for t in range(STEPS):
        n = app["n0"] + t
        q16 = synth.config5_step_query(w, t)
        for h in range(w.H_kv):
            d = oracle.dense_attention_heads(q16[h * w.G:(h + 1) * w.G], w.K[h], w.V[h], n, K64[h], V64[h])
            for g in range(w.G):
                hq = h * w.G + g
                if stop_all[t, hq] <= J:
                    certified += 1
                    fails += float(np.linalg.norm(o_all[t, hq] - d["o"][g])) > w.eps * d["M"][g]
    trials = STEPS * H_q
    _say(f"config5: {certified} of {trials} heads certified, {fails} above eps M")
    assert certified > 0.9 * trials
    assert fails / trials <= w.delta + 4 * math.sqrt(w.delta * (1 - w.delta) / trials)
