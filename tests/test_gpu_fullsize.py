"""Full-size parity: the HIP path against the oracle at the workloads' real sizes.

* the 128K Llama-shaped layer the bench times (8 KV heads x GQA 4), layers 0 and 31,
  every query head;
* four requests of the ragged batch (n from 16K to 128K, per-request epsilon, odd
  requests near-flat), every query head;
* the appending Qwen-shaped layer (4 KV heads x GQA 7, n = 131072 + t) over decode
  steps with fresh perturbations, packing each block as an append completes it.

The same call the bench times is used, with the trace on; sets, counts, stop levels
and keys read are compared bit for bit, floats to the stated tolerances.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from test_gpu_parity import _compare_decode, _kw, _to, pad_cache

pytestmark = pytest.mark.gpu


def _csa():
    import certified_sparse_attention_amd as csa
    return csa


def _run_layer(w, **over):
    print(f"[fullsize] {w.name}: n={w.n} H_kv={w.H_kv} G={w.G} eps={w.eps} J={w.J}", file=sys.stderr, flush=True)
    w = pad_cache(w)
    pk_ref = oracle.pack_kv_4bit(w.K, w.V, w.n_cap // 32)
    q, K, V = _to(w.q), _to(w.K), _to(w.V)
    packed = _csa().pack_kv_4bit(K, V)
    kw = _kw(w, **over)
    out = _csa().certified_decode_attention(q, K, V, packed, w.n, trace=True, **kw)
    torch.cuda.synchronize()
    return _compare_decode(w, pk_ref, out[:4], out[4], **kw)


@pytest.mark.parametrize("layer", [0, 31])
def test_llama_layer_128k(layer):
    ref = _run_layer(synth.config3_layer(layer), step=3)
    assert len(ref) == 32


@pytest.mark.parametrize("b", [0, 1, 2, 3])
def test_ragged_request(b):
    w = synth.config4_request(b)
    ref = _run_layer(w)
    assert len(ref) == w.H_q


def test_appending_gqa7_layer():
    """Decode steps t of the appending layer: n = n0 + t, query AR(1), step = t in the hash.
    The block of tokens n0..n0+31 is packed when step 32 completes it (and only then), on
    the GPU by a block-range pack call, so later steps scan it from the packed cache."""
    steps = 72
    w = synth.config5_base(steps=steps)
    n0 = w.n
    w = pad_cache(w)
    K, V = _to(w.K), _to(w.V)
    csa = _csa()
    packed = csa.pack_kv_4bit(K, V, block_end=n0 // 32)
    nb_packed = n0 // 32
    pk_ref = oracle.pack_kv_4bit(w.K, w.V, nb_packed)
    certified = 0
    for t in (0, 1, 33, 70):
        while (n0 + t) // 32 > nb_packed:          # blocks completed by the appends so far
            csa.pack_kv_4bit(K, V, packed, block_begin=nb_packed, block_end=nb_packed + 1)
            nb_packed += 1
            pk_ref = oracle.pack_kv_4bit(w.K, w.V, nb_packed)
        n = n0 + t
        q16 = synth.config5_step_query(w, t)
        print(f"[fullsize] config5 step {t}: n={n}, packed blocks {nb_packed}", file=sys.stderr, flush=True)
        wt = synth.Workload(f"config5.t{t}", q16, w.K, w.V, n, w.G, window=w.window, r=w.r, J=w.J,
                            eps=w.eps, delta=w.delta, step=t)
        kw = _kw(wt)
        out = csa.certified_decode_attention(_to(q16), K, V, packed, n, trace=True, **kw)
        torch.cuda.synchronize()
        ref = _compare_decode(wt, pk_ref, out[:4], out[4], **kw)
        # the guarantee itself on these draws: a certified head is within eps M of exact
        o_hat = out[0].cpu().numpy().astype(np.float64)
        for hq, r in enumerate(ref):
            if r["stop_level"] <= w.J:
                certified += 1
                d = r["dense"]
                assert np.linalg.norm(o_hat[hq] - d["o"]) <= w.eps * d["M"], (t, hq)
    assert certified > 0
