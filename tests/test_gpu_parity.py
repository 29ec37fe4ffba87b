"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Bit-exact: packed codes and metadata, score bounds UB/LB, perturbations E, c_lo,
c*, |C_max|, buckets l^ub, the candidate set, the heavy and entry levels (h, l) of
every rescored candidate and hence the sample S_j = {l <= j} and the heavy set
B_j = {h <= j} at every level up to the stop, candidate counts, stop levels and keys
read.  Floating point: beta and D^ at every level up to the stop within 1e-4
relative, |o^_gpu - o^_cpu| <= 1e-3 M.

Shapes: GQA groups of 1 to 7 queries, 1 to 8 KV heads, grids r = 1, 2, 3, deepest
levels J = 20 to 60, windows of 32, 64 and 128 tokens, contexts that are not
multiples of 32.
"""

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _csa():
    import certified_sparse_attention_amd as csa
    return csa


def _to(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def decode_codes(codes: np.ndarray) -> np.ndarray:
    """GPU code layout (include/csa.h) -> logical codes [H][nb*32][128]."""
    H, nb, _ = codes.shape
    a = codes.reshape(H, nb, 2, 4, 16, 16)            # T, g, n, j
    lo, hi = a & 15, a >> 4
    out = np.zeros((H, nb, 2, 16, 128), dtype=np.uint8)
    for g in range(4):
        out[:, :, :, :, 32 * g:32 * g + 16] = lo[:, :, :, g]
        out[:, :, :, :, 32 * g + 16:32 * g + 32] = hi[:, :, :, g]
    return out.reshape(H, nb * 32, 128)


def _packed_numpy(p):
    bm = p.bmeta.cpu().numpy().reshape(p.bmeta.shape[0], p.bmeta.shape[1], 16)
    return {
        "codes": decode_codes(p.codes.cpu().numpy()),
        "kscale": p.kscale.cpu().numpy(),
        "z": (128 * p.zq[:, :, 0].to(torch.int32) + p.zq[:, :, 1].to(torch.int32)).cpu().numpy(),
        "ksmax": bm[..., 0:4].copy().view(np.float32)[..., 0],
        "kexp": bm[..., 4:8].copy().view(np.int32)[..., 0],
        "z1sum": bm[..., 8:12].copy().view(np.int32)[..., 0],
        "kmax": bm[..., 12:16].copy().view(np.float32)[..., 0],
        "kerr": p.kerr.cpu().numpy(),
        "vnorm": p.vnorm.cpu().numpy(),
        "codes8": p.codes8.cpu().numpy(),
        "scale8": p.scale8.cpu().numpy(),
        "kerr8": p.kerr8.cpu().numpy(),
    }


def _with(w, **kw):
    for k, v in kw.items():
        setattr(w, k, v)
    return w


def _multi_head(n, H_kv, G, seed, q_scale=1.0):
    rng = np.random.default_rng(seed)
    _, q, K, V = synth.recipe_layer(rng, H_kv, G, n, sink=2.5, q_scale=q_scale)
    return synth.Workload(f"layer{H_kv}x{G}", q, K, V, n, G, window=64, r=2, J=40, eps=0.05, delta=0.01)


WORKLOADS = {
    "config1": synth.config1,
    "config2": synth.config2,
    "ragged_5000": lambda: synth.peaked_head(5000, seed=31, G=3),
    "ragged_g7": lambda: synth.peaked_head(2100, seed=32, G=7, J=20),
    "g1": lambda: synth.peaked_head(3001, seed=51, G=1),
    "g2": lambda: synth.peaked_head(3500, seed=52, G=2),
    "g5": lambda: synth.peaked_head(4003, seed=53, G=5),
    "g6": lambda: synth.peaked_head(2650, seed=54, G=6),
    "r1": lambda: _with(synth.peaked_head(3100, seed=55, G=4, J=25), r=1),
    "r3": lambda: _with(synth.peaked_head(3100, seed=56, G=4, J=60), r=3),
    "window32": lambda: synth.peaked_head(3077, seed=57, G=4, window=32),
    "window128": lambda: synth.peaked_head(3200, seed=58, G=4, window=128),
    "J60": lambda: synth.peaked_head(2999, seed=59, G=4, J=60, eps=0.02),
    "kv3_g5": lambda: _multi_head(6000, 3, 5, seed=60),
    "kv2_g4_flat": lambda: _multi_head(5000, 2, 4, seed=61, q_scale=0.1),
}


def pad_cache(w):
    """Give the cache a capacity that is a multiple of 32 (n itself stays ragged)."""
    cap = -(-w.n_cap // 32) * 32
    if cap != w.n_cap:
        pad = ((0, 0), (0, cap - w.n_cap), (0, 0))
        w.K = np.pad(w.K, pad)
        w.V = np.pad(w.V, pad)
    return w


@pytest.fixture(scope="module", params=list(WORKLOADS))
def case(request):
    w = pad_cache(WORKLOADS[request.param]())
    nb = w.n_cap // 32
    pk_ref = oracle.pack_kv_4bit(w.K, w.V, nb)
    q, K, V = _to(w.q), _to(w.K), _to(w.V)
    packed = _csa().pack_kv_4bit(K, V)
    torch.cuda.synchronize()
    return {"w": w, "pk_ref": pk_ref, "q": q, "K": K, "V": V, "packed": packed, "name": request.param}


def test_pack_bit_exact(case):
    w, ref = case["w"], case["pk_ref"]
    got = _packed_numpy(case["packed"])
    np.testing.assert_array_equal(got["codes"], ref["codes"])
    np.testing.assert_array_equal(got["kscale"].view(np.uint16), ref["kscale"].view(np.uint16))
    np.testing.assert_array_equal(got["z"], ref["z"].astype(np.int32))
    np.testing.assert_array_equal(got["kexp"], ref["kexp"])
    np.testing.assert_array_equal(got["kerr"].view(np.uint16), ref["kerr"].view(np.uint16))
    np.testing.assert_array_equal(got["vnorm"].view(np.uint16), ref["vnorm"].view(np.uint16))
    np.testing.assert_array_equal(got["codes8"], ref["k8"])
    np.testing.assert_array_equal(got["scale8"].view(np.uint32), ref["s8"].view(np.uint32))
    np.testing.assert_array_equal(got["kerr8"].view(np.uint16), ref["kerr8"].view(np.uint16))
    from oracle.bounds import block_constants
    for h in range(w.H_kv):
        bc = block_constants(w.q[h * w.G:(h + 1) * w.G], ref, h, w.n_cap // 32)
        np.testing.assert_array_equal(got["z1sum"][h], bc["Z1"])
        np.testing.assert_array_equal(got["kmax"][h].astype(np.float64), bc["Kmax"])
        np.testing.assert_array_equal(got["ksmax"][h], ref["kscale"][h].astype(np.float32).max(axis=1))


def test_scan_bounds_bit_exact(case):
    w = case["w"]
    UB, LB, E = _csa().scan_bounds(case["q"], case["K"], case["packed"], w.n, J=w.J, r=w.r,
                                   window=w.window, seed=w.seed, step=w.step, layer=w.layer)
    UB, LB, E = UB.cpu().numpy(), LB.cpu().numpy(), E.cpu().numpy()
    npool = w.n - w.window
    for h in range(w.H_kv):
        b = oracle.scan_bounds(w.q[h * w.G:(h + 1) * w.G], case["pk_ref"], h, npool)
        np.testing.assert_array_equal(UB[h * w.G:(h + 1) * w.G], b["UB"])
        np.testing.assert_array_equal(LB[h * w.G:(h + 1) * w.G], b["LB"])
        e_ref = oracle.perturbations(w.seed, w.step, w.layer, h, np.arange(npool))
        np.testing.assert_array_equal(E[h], e_ref)


def _compare_decode(w, pk_ref, res, tr, ref=None, **kw):
    """Compare a GPU call (outputs ``res``, trace ``tr``) with the oracle's result ``ref``
    (computed here from the packed reference when not given)."""
    o_hat, beta, stop, keys = (t.cpu().numpy() for t in res)
    if ref is None:
        ref = oracle.certified_decode_layer(w.q, w.K, w.V, pk_ref, w.n, w.G, **kw)
    trn = {k: v.cpu().numpy() for k, v in tr.items()}
    for hq, r in enumerate(ref):
        M = r["dense"]["M"]
        t = r.get("trace")
        assert int(stop[hq]) == r["stop_level"], (hq, int(stop[hq]), r["stop_level"])
        assert int(keys[hq]) == r["keys_read"], (hq, int(keys[hq]), r["keys_read"])
        assert np.linalg.norm(o_hat[hq].astype(np.float64) - r["o_hat"]) <= 1e-3 * M
        if r["stop_level"] <= kw["J"]:
            assert abs(beta[hq] - r["beta"]) <= 1e-4 * abs(r["beta"])
        else:
            assert beta[hq] == 0.0
        if t is None:
            continue
        assert trn["c_R"][hq] == t["c_R"]
        assert trn["c_lo"][hq] == t["c_lo"]
        assert trn["c_star"][hq] == t["c_star"]
        assert trn["cmax_count"][hq] == t["cmax_pos"].size
        npool = w.n - kw["window"]
        np.testing.assert_array_equal(trn["lub"][hq, :npool], t["lub"])
        np.testing.assert_array_equal(trn["bucket_count"][hq],
                                      np.bincount(t["lub"], minlength=kw["J"] + 2))
        assert trn["cand_count"][hq] == t["cand"].size
        _compare_samples(hq, trn, t, r["stop_level"], kw["J"])
        for j, lv in enumerate(t["levels"]):
            assert trn["k_level"][hq, j] == lv["k"], (hq, j)
            assert abs(trn["dhat_level"][hq, j] - lv["D_hat"]) <= 1e-4 * lv["D_hat"]
            b_ref = lv["beta"]
            if np.isfinite(b_ref):
                assert abs(trn["beta_level"][hq, j] - b_ref) <= 1e-4 * b_ref, (hq, j)
            else:
                assert not np.isfinite(trn["beta_level"][hq, j])
    return ref


def _compare_samples(hq, trn, t, stop, J):
    """The candidate list, the refined level l8 and the (h, l) of every rescored candidate,
    and S_j, B_j at every level up to the stop (up to J on the exact fallback), element by
    element."""
    cc = int(trn["cand_count"][hq])
    pos = trn["cand_pos"][hq, :cc]
    np.testing.assert_array_equal(np.sort(pos), t["cand"])     # the same set, no repeats
    nres = int(trn["rescored_count"][hq])
    assert 0 <= nres <= cc
    hl = trn["cand_hl"][hq, :cc]
    assert np.all(hl[:nres] >= 0) and np.all(hl[nres:] == -1)
    rpos = pos[:nres]
    idx = np.searchsorted(t["cand"], rpos)
    gh, gl = hl[:nres] & 0xFF, hl[:nres] >> 8
    np.testing.assert_array_equal(gh, t["h"][idx])
    np.testing.assert_array_equal(gl, t["l"][idx])
    l8 = trn["cand_l8"][hq, :cc]
    assert np.all(l8[nres:] == -1)
    np.testing.assert_array_equal(l8[:nres], t["l8"][idx])
    for j in range(min(stop, J) + 1):
        np.testing.assert_array_equal(np.sort(rpos[gl <= j]), t["cand"][t["l"] <= j], err_msg=f"S_{j} of {hq}")
        np.testing.assert_array_equal(np.sort(rpos[gh <= j]), t["cand"][t["h"] <= j], err_msg=f"B_{j} of {hq}")


def _check_list_order(trn, H_q, J, budget=0, budget2=0):
    """The candidate list is the first range (l^ub <= j1), then the second (j1 < l^ub <= j2),
    then the third (j2 < l^ub <= J), each in position order, where j1 is the deepest level
    whose cumulative bucket count fits the first budget (32 unless given, at most 2048) and
    j2 > j1 the deepest one within the second (no limit unless given)."""
    b1 = min(budget, 2048) if budget > 0 else 32
    b2 = budget2 if budget2 > 0 else np.iinfo(np.int64).max
    for hq in range(H_q):
        cum = np.cumsum(trn["bucket_count"][hq][:J + 1])
        j1 = int(np.sum(cum <= b1)) - 1
        j2 = min(J, max(j1 + 1, int(np.sum(cum <= b2)) - 1))
        npool = trn["lub"].shape[1]
        lub = trn["lub"][hq, :npool].astype(np.int64)
        at = np.arange(npool)
        want = np.concatenate([at[lub <= j1], at[(lub > j1) & (lub <= j2)], at[(lub > j2) & (lub <= J)]])
        cc = int(trn["cand_count"][hq])
        np.testing.assert_array_equal(trn["cand_pos"][hq, :cc], want, err_msg=f"candidate list of {hq}")


def _kw(w, **over):
    kw = dict(eps=w.eps, delta=w.delta, r=w.r, J=w.J, window=w.window, seed=w.seed, step=w.step,
              layer=w.layer)
    kw.update(over)
    return kw


def test_certified_decode_parity(case):
    w = case["w"]
    kw = _kw(w)
    out = _csa().certified_decode_attention(case["q"], case["K"], case["V"], case["packed"], w.n,
                                            trace=True, **kw)
    torch.cuda.synchronize()
    _compare_decode(w, case["pk_ref"], out[:4], out[4], **kw)
    trn = {k: v.cpu().numpy() for k, v in out[4].items()}
    _check_list_order(trn, w.H_q, w.J)
    lt = out[4]["logtau"].cpu().numpy()
    np.testing.assert_array_equal(lt, oracle.logtau(w.r, w.J))


def test_certified_decode_is_deterministic(case):
    w = case["w"]
    kw = _kw(w)
    a = _csa().certified_decode_attention(case["q"], case["K"], case["V"], case["packed"], w.n, **kw)
    a = [t.clone() for t in a]
    b = _csa().certified_decode_attention(case["q"], case["K"], case["V"], case["packed"], w.n, **kw)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("measure", ["denominator", "output_norm"])
def test_other_measures(case, measure):
    w = case["w"]
    kw = _kw(w)
    out = _csa().certified_decode_attention(case["q"], case["K"], case["V"], case["packed"], w.n,
                                            trace=True, measure=measure, **kw)
    torch.cuda.synchronize()
    m = {"denominator": 0, "output_norm": 1}[measure]
    _compare_decode(w, case["pk_ref"], out[:4], out[4], measure=m, **kw)


def test_ragged_n_and_window_edges():
    """n just above the window, n not a multiple of 32, and n inside the window."""
    w = synth.peaked_head(4096, seed=41, G=4)
    pk_ref = oracle.pack_kv_4bit(w.K, w.V, w.n_cap // 32)
    q, K, V = _to(w.q), _to(w.K), _to(w.V)
    packed = _csa().pack_kv_4bit(K, V)
    for n in (1, 40, 64, 65, 97, 1000, 4095):
        kw = _kw(w)
        out = _csa().certified_decode_attention(q, K, V, packed, n, trace=(n > 64), **kw)
        torch.cuda.synchronize()
        if n <= 64:
            o_hat, beta, stop, keys = (t.cpu().numpy() for t in out)
            for g in range(w.G):
                d = oracle.dense_attention(w.q[g], w.K[0], w.V[0], n)
                assert stop[g] == 0 and beta[g] == 0.0 and keys[g] == n
                assert np.linalg.norm(o_hat[g] - d["o"]) <= 1e-6 * d["M"]
        else:
            w2 = synth.Workload(w.name, w.q, w.K, w.V, n, w.G, window=w.window, r=w.r, J=w.J,
                                eps=w.eps, delta=w.delta)
            _compare_decode(w2, pk_ref, out[:4], out[4], **kw)


def test_fallback_paths():
    """J = 0 or a tiny eps: no level certifies and the exact output comes back."""
    w = synth.config1()
    pk_ref = oracle.pack_kv_4bit(w.K, w.V, w.n_cap // 32)
    q, K, V = _to(w.q), _to(w.K), _to(w.V)
    packed = _csa().pack_kv_4bit(K, V)
    for over in (dict(J=0), dict(eps=1e-9)):
        kw = _kw(w, **over)
        out = _csa().certified_decode_attention(q, K, V, packed, w.n, trace=True, **kw)
        torch.cuda.synchronize()
        ref = _compare_decode(w, pk_ref, out[:4], out[4], **kw)
        o_hat = out[0].cpu().numpy()
        for hq, r in enumerate(ref):
            assert r["stop_level"] == kw["J"] + 1
            assert np.linalg.norm(o_hat[hq] - r["dense"]["o"]) <= 1e-6 * r["dense"]["M"]


def test_fresh_perturbations_per_step():
    """Another step gives other perturbations (and still matches the oracle)."""
    w = synth.config1()
    pk_ref = oracle.pack_kv_4bit(w.K, w.V, w.n_cap // 32)
    q, K, V = _to(w.q), _to(w.K), _to(w.V)
    packed = _csa().pack_kv_4bit(K, V)
    kw = _kw(w, step=7, layer=3)
    out = _csa().certified_decode_attention(q, K, V, packed, w.n, trace=True, **kw)
    torch.cuda.synchronize()
    _compare_decode(w, pk_ref, out[:4], out[4], **kw)


def test_dense_decode_matches_oracle(case):
    w = case["w"]
    o = _csa().dense_decode_attention(case["q"], case["K"], case["V"], w.n).cpu().numpy()
    for hq in range(w.H_q):
        h = hq // w.G
        d = oracle.dense_attention(w.q[hq], w.K[h], w.V[h], w.n)
        assert np.linalg.norm(o[hq] - d["o"]) <= 1e-4 * d["M"], hq


def test_level_zero_over_the_budget():
    """A near-flat head whose level-0 bucket alone holds more candidates than the fused
    first pass takes: the first pass is empty and the second pass takes every level."""
    rng = np.random.default_rng(77)
    _, q, K, V = synth.recipe_layer(rng, 1, 4, 12288, sink=3.5, q_scale=0.1)
    w = pad_cache(synth.Workload("flat12k", q, K, V, 12288, 4, window=64, r=2, J=30, eps=0.1, delta=0.01))
    pk_ref = oracle.pack_kv_4bit(w.K, w.V, w.n_cap // 32)
    qg, Kg, Vg = _to(w.q), _to(w.K), _to(w.V)
    packed = _csa().pack_kv_4bit(Kg, Vg)
    kw = _kw(w)
    out = _csa().certified_decode_attention(qg, Kg, Vg, packed, w.n, trace=True, **kw)
    torch.cuda.synchronize()
    ref = _compare_decode(w, pk_ref, out[:4], out[4], **kw)
    level0 = [int((r["trace"]["lub"] == 0).sum()) for r in ref]
    assert max(level0) > 2048, level0


@pytest.mark.parametrize("cluster,budget,crowd", [(40, 64, 8), (120, 200, 64)])
def test_clustered_first_range(cluster, budget, crowd):
    """A run of strong keys inside one bucket tile puts more of the first range in that tile
    than the entries the certificate kernel reads ahead per tile (40 keys), or than a
    tile's level-ordered list holds (120 keys): the list, its order and every result stay
    oracle-exact."""
    rng = np.random.default_rng(91)
    q32, q, K, V = synth.recipe_layer(rng, 1, 4, 12288, heavy_frac=0.0)
    qbar = q.astype(np.float64).mean(axis=0)
    dirv = np.sqrt(128.0) * qbar / float(qbar @ qbar)
    K = K.astype(np.float32)
    K[0, 3000:3000 + cluster] += (10.0 * dirv).astype(np.float32)
    K = K.astype(np.float16)
    w = pad_cache(synth.Workload("cluster12k", q, K, V, 12288, 4, window=64, r=2, J=30, eps=0.1, delta=0.01))
    pk_ref = oracle.pack_kv_4bit(w.K, w.V, w.n_cap // 32)
    qg, Kg, Vg = _to(w.q), _to(w.K), _to(w.V)
    packed = _csa().pack_kv_4bit(Kg, Vg)
    kw = _kw(w)
    out = _csa().certified_decode_attention(qg, Kg, Vg, packed, w.n, trace=True, cand_budget=budget, **kw)
    torch.cuda.synchronize()
    _compare_decode(w, pk_ref, out[:4], out[4], **kw)
    trn = {k: v.cpu().numpy() for k, v in out[4].items()}
    _check_list_order(trn, w.H_q, w.J, budget)
    # the first range does crowd one tile
    most = 0
    for hq in range(w.H_q):
        cum = np.cumsum(trn["bucket_count"][hq][:w.J + 1])
        tot1 = int(cum[int(np.sum(cum <= budget)) - 1]) if cum[0] <= budget else 0
        if tot1:
            most = max(most, int(np.bincount(trn["cand_pos"][hq, :tot1] // 2048).max()))
    assert most > crowd, most


def test_stream_read_checksum():
    """The read helper visits every 32-bit word once: per-workgroup XORs match the host's."""
    rng = np.random.default_rng(5)
    for nbytes, wgs in ((16 * 1000, 7), (1 << 20, 64), (16 * 4097, 300)):
        host = rng.integers(0, 2**32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
        sink = _csa().stream_read(torch.from_numpy(host.view(np.int32)).to(DEV), workgroups=wgs)
        torch.cuda.synchronize()
        got = sink.cpu().numpy().view(np.uint32)
        n16 = nbytes // 16
        per = -(-n16 // wgs)
        for w in range(wgs):
            part = host[4 * min(n16, w * per):4 * min(n16, (w + 1) * per)]
            assert got[w] == (np.bitwise_xor.reduce(part) if part.size else 0), (nbytes, wgs, w)


@pytest.mark.parametrize("budget,budget2", [(1, 0), (16, 0), (300, 0), (1, 3), (4, 40)])
def test_speculative_budget_does_not_change_results(case, budget, budget2):
    """Small candidate budgets force the second and third passes; results stay oracle-exact."""
    w = case["w"]
    kw = _kw(w)
    out = _csa().certified_decode_attention(case["q"], case["K"], case["V"], case["packed"], w.n,
                                            trace=True, cand_budget=budget, cand_budget2=budget2, **kw)
    torch.cuda.synchronize()
    _compare_decode(w, case["pk_ref"], out[:4], out[4], **kw)
    _check_list_order({k: v.cpu().numpy() for k, v in out[4].items()}, w.H_q, w.J, budget, budget2)
