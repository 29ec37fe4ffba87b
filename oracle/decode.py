"""One certified decode step for one layer (test infrastructure only).

Follows the method's steps in the pages' order:

1. Window / pool split: the last ``window`` tokens R are read exactly, the rest is
   the pool P ([S] Algorithm Components item 1).
2. Deterministic score bounds from the 4-bit keys, shared by the GQA group
   (``bounds.scan_bounds``; [S] item 4, [A]).
3. Exact maximum over a small set: c_lo = max(c_R, max_P LB); C_max = {UB >= c_lo};
   c* = max(c_R, max over C_max of s) ([S] item 4, "exact maximum").
4. Perturbations E_i (``perturb``), and each pool key's earliest possible level
   l^ub = first((UB + E) - c*) ([S] item 4: candidates are grouped by the first level
   at which they could be sampled).  Reading: buckets are taken relative to the exact c*.
5. The 8-bit refinement of every candidate (l^ub <= J): UB8 from the 8-bit copy
   (``bounds.refine_bounds8``) and the refined level l8 = first((min(UB, UB8) + E) - c*)
   ([S] item 4: an 8-bit tier narrows the candidates before any 16-bit key is read).
   Exact 16-bit reads only for candidates with l8 <= J: s_i, the heavy level
   h = first(s - c*) and the entry level l = first((s + E) - c*) (so l <= h, and
   l^ub <= l8 <= l because min(UB, UB8) >= s); the others have h = l = J + 1.
6. Per level j (tau_j = exp(LOGTAU[j])): B_j = {h <= j} (w >= tau, always in),
   A_j = P \\ B_j, S_j = {l <= j}, k = |S_j & A_j|,
   D^ = D_R + D_B + tau k, N^ = N_R + N_B + tau sum_{S&A} v ([S] item 2); the
   letters R, B, A, k are read so that [S] Theorem 1's Var D^ <= tau D_A holds.
7. Certificate per level (``certify``) and the stop at the first level with
   beta <= eps ([S] item 3); if none, the exact fallback ([S] Results > Certificate
   Validity mentions heads falling back to exact attention): o exact, beta = 0,
   stop level J + 1, keys read n.  With n <= window every key is in the window:
   o exact, beta = 0, stop level 0, keys read n.

keys_read counts exact 16-bit key reads: window + |C_max union {l8 <= j*}|
(reading of "keys read", [S] Summary and Table 1's caption); the trace also gives the
8-bit reads, |{l^ub <= j*}|.
"""

import numpy as np

from .canon import LN2, csum128, first_level, logtau  # noqa: F401
from .bounds import refine_bounds8, scan_bounds
from .certify import MEASURE_VALUE, budget_L, level_certificates
from .dense import dense_attention, exact_scores
from .perturb import perturbations


def level_sums(j, hl, ll, w, Vr, vsq, D_R, N_R, Q_R):
    """Deterministic and sampled sums at level j over the rescored keys.

    Heavy keys B_j = {h <= j} add (w, w v, w |v|^2); light sampled keys
    S_j & A_j = {l <= j < h} add (1, v, |v|^2).  Keys never rescored have l > J and
    contribute nothing at any level.
    """
    heavy = hl <= j
    light = (ll <= j) & ~heavy
    return {
        "D_det": D_R + float(w[heavy].sum()),
        "N_det": N_R + w[heavy] @ Vr[heavy],
        "Q_det": Q_R + float(w[heavy] @ vsq[heavy]),
        "k": int(light.sum()),
        "Vs": Vr[light].sum(axis=0),
        "Ps": float(vsq[light].sum()),
        "n_heavy": int(heavy.sum()),
        "n_sample": int((ll <= j).sum()),
    }


def _exact_result(q16, K16, V16, n, stop_level):
    d = dense_attention(q16, K16, V16, n)
    return {"o_hat": d["o"], "beta": 0.0, "stop_level": stop_level, "keys_read": n,
            "values_read": n, "dense": d}


def scan_stage(q16, K16, V16, packed, h, n, *, window=64):
    """Steps 1-3 for the G queries q16 [G][128] of KV head h: everything that does not
    depend on the perturbations (window scores, bounds, c_lo, C_max and c*).

    Returns None when n <= window (every key is exact); otherwise a dict with the
    per-query values in lists indexed by g.
    """
    G = q16.shape[0]
    W = window
    if n <= W:
        return None
    npool = n - W
    Vd_all = V16[:n].astype(np.float64)
    vsq_all = csum128(Vd_all * Vd_all)
    Vmax = float(packed["vnorm"][h, :npool].astype(np.float64).max())
    bnd = scan_bounds(q16, packed, h, npool)
    per = []
    for g in range(G):
        s_R = exact_scores(q16[g], K16[npool:n])
        c_R = float(s_R.max())
        UB, LB = bnd["UB"][g], bnd["LB"][g]
        c_lo = max(c_R, float(LB.max()))
        cmax_pos = np.nonzero(UB >= c_lo)[0]
        s_cm = exact_scores(q16[g], K16[cmax_pos])
        c_star = max(c_R, float(s_cm.max())) if cmax_pos.size else c_R
        w_R = np.exp(s_R - c_star)
        per.append({"s_R": s_R, "c_R": c_R, "UB": UB, "LB": LB, "c_lo": c_lo, "cmax_pos": cmax_pos,
                    "c_star": c_star, "D_R": float(w_R.sum()), "N_R": w_R @ Vd_all[npool:n],
                    "Q_R": float(w_R @ vsq_all[npool:n])})
    return {"q16": q16, "K16": K16, "V16": V16, "h": h, "n": n, "W": W, "npool": npool,
            "Vd_all": Vd_all, "vsq_all": vsq_all, "Vmax": Vmax, "per": per, "packed": packed}


def sample_stage(sc, *, eps, delta, r, J, seed=0x5EED, step=0, layer=0, measure=MEASURE_VALUE,
                 with_dense=True):
    """Steps 4-7 for every query of a ``scan_stage`` result, with the perturbations of
    (seed, step, layer, KV head): buckets, exact rescoring of the candidates, the level
    sums, the certificate of every level and the stop at the first certified one."""
    q16, K16, V16, h, n, W, npool = sc["q16"], sc["K16"], sc["V16"], sc["h"], sc["n"], sc["W"], sc["npool"]
    LT = logtau(r, J)
    TAU = np.exp(LT)
    L = budget_L(J, delta, measure)
    Vd_all, vsq_all, Vmax = sc["Vd_all"], sc["vsq_all"], sc["Vmax"]
    E = perturbations(seed, step, layer, h, np.arange(npool))
    results = []
    for g, pg in enumerate(sc["per"]):
        c_star, UB = pg["c_star"], pg["UB"]
        p = UB + E
        lub = first_level(p - c_star, LT)
        cand = np.nonzero(lub <= J)[0]
        UB8 = refine_bounds8(q16[g:g + 1], sc["packed"], h, cand)["UB8"][0]
        l8 = first_level((np.minimum(UB[cand], UB8) + E[cand]) - c_star, LT)
        ex = l8 <= J                                        # exact 16-bit reads
        s_c = np.full(cand.size, np.nan)
        s_c[ex] = exact_scores(q16[g], K16[cand[ex]])
        hl = np.full(cand.size, J + 1, dtype=np.int32)
        ll = np.full(cand.size, J + 1, dtype=np.int32)
        hl[ex] = first_level(s_c[ex] - c_star, LT)
        ll[ex] = first_level((s_c[ex] + E[cand[ex]]) - c_star, LT)
        w_c = np.zeros(cand.size)
        w_c[ex] = np.exp(s_c[ex] - c_star)
        Vc = Vd_all[cand]
        vsq_c = vsq_all[cand]
        stats = [level_sums(j, hl, ll, w_c, Vc, vsq_c, pg["D_R"], pg["N_R"], pg["Q_R"]) for j in range(J + 1)]
        certs = level_certificates(stats, TAU, L, Vmax, measure)
        levels = []
        stop = None
        for st, cert in zip(stats, certs):
            cert.update(st)
            levels.append(cert)
            if cert["beta"] <= eps:
                stop = len(levels) - 1
                break
        trace = {"c_R": pg["c_R"], "c_lo": pg["c_lo"], "c_star": c_star, "cmax_pos": pg["cmax_pos"],
                 "lub": lub, "cand": cand, "UB8": UB8, "l8": l8, "s_c": s_c, "h": hl, "l": ll, "E": E,
                 "UB": UB, "LB": pg["LB"], "levels": levels, "L": L, "Vmax": Vmax, "D_R": pg["D_R"]}
        if stop is None:
            res = _exact_result(q16[g], K16, V16, n, J + 1)
            res["trace"] = trace
            results.append(res)
            continue
        read_set = np.union1d(pg["cmax_pos"], cand[l8 <= stop])
        trace["keys_read_8bit"] = int((lub[cand] <= stop).sum())
        res = {"o_hat": levels[stop]["o_hat"], "beta": float(levels[stop]["beta"]),
               "stop_level": stop, "keys_read": int(W + read_set.size),
               "values_read": int(W + int((ll <= stop).sum())), "trace": trace}
        if with_dense:
            res["dense"] = dense_attention(q16[g], K16, V16, n)
        results.append(res)
    return results


def certified_decode(q16, K16, V16, packed, h, n, *, eps, delta, r, J, window=64,
                     seed=0x5EED, step=0, layer=0, measure=MEASURE_VALUE, with_dense=True):
    """Certified decode for the G queries q16 [G][128] of KV head h.

    K16, V16: fp16 [n_cap][128] of this KV head.  Returns a list (one entry per
    query) of dicts with o_hat, beta, stop_level, keys_read and a trace.
    """
    sc = scan_stage(q16, K16, V16, packed, h, n, window=window)
    if sc is None:
        return [_exact_result(q16[g], K16, V16, n, 0) for g in range(q16.shape[0])]
    return sample_stage(sc, eps=eps, delta=delta, r=r, J=J, seed=seed, step=step, layer=layer,
                        measure=measure, with_dense=with_dense)


def certified_decode_layer(q16, K16, V16, packed, n, G, **kw):
    """All KV heads of one layer: q16 [H_q][128], K16/V16 [H_kv][n_cap][128]."""
    out = []
    for h in range(K16.shape[0]):
        out.extend(certified_decode(q16[h * G:(h + 1) * G], K16[h], V16[h], packed, h, n, **kw))
    return out
