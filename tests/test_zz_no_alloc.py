"""The allocation-free entry point against the workspace entry point, through the C ABI.

Two allocation-free calls in a row, the second on a smaller input (fewer heads, a
shorter context), so that the second runs on scratch the first left behind; each is
compared with the workspace entry point on the same input: the kernels are the same,
so every output must be bit-identical.  A shape whose scratch need exceeds the static
array is rejected before anything is launched.
"""

import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _csa():
    import certified_sparse_attention_amd as csa
    return csa


def _setup(w):
    q = torch.from_numpy(np.ascontiguousarray(w.q)).to(DEV)
    K = torch.from_numpy(np.ascontiguousarray(w.K)).to(DEV)
    V = torch.from_numpy(np.ascontiguousarray(w.V)).to(DEV)
    packed = _csa().pack_kv_4bit(K, V)
    kw = dict(eps=w.eps, delta=w.delta, r=w.r, J=w.J, window=w.window, seed=w.seed, step=w.step, layer=w.layer)
    return q, K, V, packed, kw


def _outs(H_q):
    return (torch.full((H_q, 128), float("nan"), dtype=torch.float32, device=DEV),
            torch.full((H_q,), float("nan"), dtype=torch.float64, device=DEV),
            torch.full((H_q,), -7, dtype=torch.int32, device=DEV),
            torch.full((H_q,), -7, dtype=torch.int64, device=DEV))


def _large():
    rng = np.random.default_rng(71)
    _, q, K, V = synth.recipe_layer(rng, 2, 4, 24576, sink=3.5)
    return synth.Workload("noalloc.large", q, K, V, 24576, 4, window=64, r=2, J=40, eps=0.05, delta=0.01)


def test_noalloc_matches_workspace_entry_point():
    csa = _csa()
    small = synth.peaked_head(3032, seed=72, G=3)
    pad = ((0, 0), (0, (-small.n_cap) % 32), (0, 0))
    small.K, small.V = np.pad(small.K, pad), np.pad(small.V, pad)
    cases = [_large(), small]
    prepared = [_setup(w) for w in cases]
    got = []
    for w, (q, K, V, packed, kw) in zip(cases, prepared):          # two calls in a row
        out = _outs(w.H_q)
        csa.certified_decode_attention_noalloc(q, K, V, packed, w.n, out, **kw)
        got.append(out)
    torch.cuda.synchronize()
    for w, (q, K, V, packed, kw), out in zip(cases, prepared, got):
        ref = csa.certified_decode_attention(q, K, V, packed, w.n, **kw)
        torch.cuda.synchronize()
        for a, b in zip(out, ref):
            assert torch.equal(a, b), w.name
        assert int(out[2].max()) <= w.J and int(out[3].min()) >= w.window


def test_noalloc_rejects_shapes_beyond_its_scratch():
    csa = _csa()
    w = synth.peaked_head(4096, seed=73, G=4)
    q, K, V, packed, kw = _setup(w)
    big = torch.zeros((8, 131072, 128), dtype=torch.float16, device=DEV)
    qb = torch.zeros((32, 128), dtype=torch.float16, device=DEV)
    pb = csa.PackedKV.allocate(8, 131072)
    out = _outs(32)
    with pytest.raises(RuntimeError, match="static scratch"):
        csa.certified_decode_attention_noalloc(qb, big, big, pb, 131072, out, **kw)
    torch.cuda.synchronize()
    assert int(out[2][0]) == -7          # nothing was launched
