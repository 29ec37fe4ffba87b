"""Oracle runs for the full-size GPU parity tests, executed in CPU worker processes
(they import numpy only, never the GPU library) while the GPU side runs."""

import numpy as np


def _pad(w):
    cap = -(-w.n_cap // 32) * 32
    if cap != w.n_cap:
        pad = ((0, 0), (0, cap - w.n_cap), (0, 0))
        w.K = np.pad(w.K, pad)
        w.V = np.pad(w.V, pad)
    return w


_TRACE_KEEP = ("c_R", "c_lo", "c_star", "cmax_pos", "lub", "cand", "h", "l", "l8", "levels")
_LEVEL_KEEP = ("k", "D_hat", "beta")


def _slim(res):
    """Only what the comparison reads (the per-key bounds and perturbations stay behind)."""
    out = []
    for r in res:
        s = {k: r[k] for k in ("o_hat", "beta", "stop_level", "keys_read")}
        s["dense"] = {"M": r["dense"]["M"], "o": r["dense"]["o"]}
        if "trace" in r:
            t = r["trace"]
            s["trace"] = {k: t[k] for k in _TRACE_KEEP if k != "levels"}
            s["trace"]["levels"] = [{k: lv[k] for k in _LEVEL_KEEP} for lv in t["levels"]]
        out.append(s)
    return out


def ragged_request_reference(b):
    """The oracle's result for request b of the 16-request ragged batch."""
    from threadpoolctl import threadpool_limits
    import oracle
    import synth
    with threadpool_limits(1):
        w = _pad(synth.config4_request(b))
        pk = oracle.pack_kv_4bit(w.K, w.V, w.n_cap // 32)
        res = oracle.certified_decode_layer(w.q, w.K, w.V, pk, w.n, w.G, eps=w.eps, delta=w.delta, r=w.r,
                                            J=w.J, window=w.window, seed=w.seed, step=w.step, layer=w.layer)
    return _slim(res)
