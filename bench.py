"""Benchmark: certified decode-attention steps/s at 128K context, 8 KV heads, d = 128.

One step is one certified decode step of one layer: all 8 KV heads x GQA 4 query
heads at n = 131072 over a 16-bit cache (window and exact reads, the 4-bit scan,
the exact maximum, buckets, exact rescoring, level sums, certificates, the stop).
The timed loop rotates over the 32 layers of a Llama-3.1-8B-shaped decode step
(synthetic sink + power-law heavy-hitter caches, 16 GiB of K/V resident in HBM) so
that no layer's data is still in the 256 MB Infinity Cache when it is read again.

Beside the headline line the same JSON object carries, per workload (the 128K layer,
all 32 layers of the step in one batched call, the 32K layer, the 16-request ragged
batch as one batched call and as 16 single calls, the appending GQA-7 layer over 256
steps): the median and p10/p90 over timed iterations of the certified call, of its
4-bit scan kernel and of the library's dense decode; keys read and stop levels; and the
CPU legs (the oracle on one core and on a process per KV head, a CPU fp64 dense
attention, and the appending layer's failure rate against the oracle's exact
attention).

Prints one JSON line.  Only one GPU is used: --gpus above 1 exits.
"""

import argparse
import hashlib
import json
import os
import platform
import sys
import time
from concurrent.futures import ThreadPoolExecutor

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

HBM_PEAK_GBS = 8000.0
N_CTX = 131072
H_KV, GQA, D = 8, 4, 128
WINDOW = 64
SCAN_BYTES_PER_TOKEN = 84.5   # codes 64 + kscale 8 + zero points 8 + block record 0.5 + kerr 2 + vnorm 2
DENSE_BYTES_PER_TOKEN = 512   # K and V rows, fp16
EVENT_EVERY = 4
STATS_ITERS = 100


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=64)
    p.add_argument("--warmup", type=int, default=8)
    p.add_argument("--layers", type=int, default=32)
    p.add_argument("--stats-iters", type=int, default=STATS_ITERS)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--headline-only", action="store_true",
                   help="only the 128K layer (no 32K, ragged-batch or appending legs)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain 1 GiB device-to-device copy 4 times (reference for "
                        "scaling the FETCH_SIZE / WRITE_SIZE counters)")
    return p.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def copy_calibration():
    import torch
    nbytes = 1 << 30
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(4):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read_per_launch": nbytes, "copy_bytes_written_per_launch": nbytes,
                      "launches": 4}))


def scan_traffic():
    """HBM bytes per scan launch from the committed FETCH_SIZE/WRITE_SIZE summary, scaled by
    the copy calibration; None once the scan's sources differ from those the counters saw."""
    path = os.path.join(ROOT, "profiles", "scan_kernel_128k_hbm_traffic.md")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and line.split(":")[0] in ("traffic_bytes_per_launch", "source_sha256"):
            k, v = line.split(":", 1)
            fields[k] = v.strip()
    src = b"".join(open(os.path.join(ROOT, "certified_sparse_attention_amd", "csrc", f), "rb").read()
                   for f in ("scan.hip", "common.h"))
    if fields.get("source_sha256") != hashlib.sha256(src).hexdigest():
        return None
    return float(fields["traffic_bytes_per_launch"])


def pct(xs):
    a = np.asarray(xs, dtype=np.float64)
    return {"median": float(np.median(a)), "p10": float(np.percentile(a, 10)), "p90": float(np.percentile(a, 90)),
            "n": int(a.size)}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def host_cores():
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


# ---------------------------------------------------------------- GPU timing helpers
class Timer:
    """Per-call times from torch events around each call on the current stream (the
    library launches on it), and the scan kernel's own dispatch times from library events."""

    def __init__(self, csa, torch, iters):
        self.torch = torch
        self.ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(iters)]
        self.sev = [(csa.Event(), csa.Event()) for _ in range(iters)]

    def calls(self, fn, iters):
        for i in range(iters):
            self.ev[i][0].record()
            fn(i, None)
            self.ev[i][1].record()
        self.torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in self.ev[:iters]]

    def scans(self, fn, iters):
        for i in range(iters):
            fn(i, (self.sev[i][0].handle, self.sev[i][1].handle))
        self.torch.cuda.synchronize()
        return [a.elapsed_ms(b) for a, b in self.sev[:iters]]


def gen_layers(nlayers, chunk=8):
    """Synthetic layers in order, generated on host threads a chunk at a time."""
    import synth
    with ThreadPoolExecutor(max_workers=chunk) as ex:
        for c0 in range(0, nlayers, chunk):
            for w in ex.map(synth.config3_layer, range(c0, min(nlayers, c0 + chunk))):
                yield w


def dense_ws(csa, K, G, n, torch):
    need = int(csa.api._lib.load().csa_dense_workspace_bytes(csa.api._shape(K, G), int(n)))
    return torch.empty(max(need, 1), dtype=torch.uint8, device=K.device)


def certified_leg(csa, torch, timer, items, iters, warm, dense=True):
    """items: list of dicts (q, K, V, packed, n, kw, ws, out, dws, dout) visited round robin.
    Returns the per-call, per-scan and per-dense statistics and the last outputs."""
    def call(i, events):
        it = items[i % len(items)]
        return csa.certified_decode_attention(it["q"], it["K"], it["V"], it["packed"], it["n"], workspace=it["ws"],
                                              out=it["out"], scan_events=events, step=i, **it["kw"])

    def dcall(i, _):
        it = items[i % len(items)]
        csa.dense_decode_attention(it["q"], it["K"], it["V"], it["n"], workspace=it["dws"], out=it["dout"])

    for i in range(warm):
        call(i, None)
    torch.cuda.synchronize()
    res = {"call_ms": pct(timer.calls(call, iters)), "scan_kernel_ms": pct(timer.scans(call, iters))}
    keys = torch.stack([it["out"][3] for it in items]).cpu().numpy().ravel()
    stops = torch.stack([it["out"][2] for it in items]).cpu().numpy().ravel()
    J = items[0]["kw"]["J"]
    res["keys_read"] = {"median": float(np.median(keys)), "p90": float(np.percentile(keys, 90))}
    res["stop_level"] = {"median": float(np.median(stops)), "p90": float(np.percentile(stops, 90)),
                         "fallbacks": int((stops > J).sum()), "heads": int(stops.size)}
    if dense:
        for i in range(warm):
            dcall(i, None)
        torch.cuda.synchronize()
        res["dense_ms"] = pct(timer.calls(dcall, iters))
    return res


def prepare_item(csa, torch, w, dev, K=None, V=None, packed=None, share=None):
    """One call's inputs and outputs on the GPU; ``share`` (an earlier item) lends its
    workspaces, which calls ordered on one stream may reuse."""
    q = torch.from_numpy(w.q).to(dev)
    if K is None:
        K = torch.from_numpy(w.K).to(dev)
        V = torch.from_numpy(w.V).to(dev)
    if packed is None:
        packed = csa.pack_kv_4bit(K, V)
    kw = dict(eps=w.eps, delta=w.delta, r=w.r, J=w.J, window=w.window, seed=w.seed, layer=w.layer)
    H_q = w.H_q
    out = (torch.empty((H_q, D), dtype=torch.float32, device=dev), torch.empty(H_q, dtype=torch.float64, device=dev),
           torch.empty(H_q, dtype=torch.int32, device=dev), torch.empty(H_q, dtype=torch.int64, device=dev))
    if share is not None:
        ws, dws = share["ws"], share["dws"]
    else:
        ws, dws = csa.allocate_workspace(K, w.G, w.n, w.J, w.window), dense_ws(csa, K, w.G, w.n, torch)
    return {"q": q, "K": K, "V": V, "packed": packed, "n": w.n, "kw": kw, "out": out, "ws": ws, "dws": dws,
            "dout": torch.empty((H_q, D), dtype=torch.float32, device=dev)}


def leg_32k(csa, torch, timer, dev, iters, warm):
    """The 32768-token layer; its 21 MiB of packed keys fit in the Infinity Cache, so the
    calls rotate over 32 copies of the cache in separate buffers (about 4.3 GB)."""
    import synth
    w = synth.config2()
    K0 = torch.from_numpy(w.K).to(dev)
    V0 = torch.from_numpy(w.V).to(dev)
    items = []
    for c in range(32):
        K, V = (K0, V0) if c == 0 else (K0.clone(), V0.clone())
        items.append(prepare_item(csa, torch, w, dev, K, V, share=items[0] if items else None))
    torch.cuda.synchronize()
    res = certified_leg(csa, torch, timer, items, iters, warm)
    res["workload"] = "8 KV heads x GQA 4, d=128, n=32768, sink 3.5 nats + 1% power-law heavy hitters, " \
                      "eps=0.05, delta=0.01, r=2, J=40, rotating 32 buffer copies"
    res["steps_per_s"] = 1e3 / res["call_ms"]["median"]
    res["scan_bytes"] = SCAN_BYTES_PER_TOKEN * (w.n - WINDOW) * w.H_kv
    res["scan_gbs_median"] = res["scan_bytes"] / (res["scan_kernel_ms"]["median"] * 1e-3) / 1e9
    return res


def leg_ragged(csa, torch, timer, dev, iters, warm):
    """The 16-request ragged batch (n from 16K to 128K, eps per request, odd requests
    near-flat), its caches in one [16][H_kv][131072][128] tensor (request b = slot b): a
    step as one batched call, and as 16 single calls issued back to back."""
    import synth
    with ThreadPoolExecutor(max_workers=8) as ex:
        ws_ = list(ex.map(synth.config4_request, range(16)))
    B = 16
    K_all = torch.zeros((B, H_KV, N_CTX, D), dtype=torch.float16, device=dev)
    V_all = torch.zeros_like(K_all)
    packed_all = csa.PackedKV.allocate(B * H_KV, N_CTX, dev)
    by_b = {}
    order = sorted(range(B), key=lambda b: -ws_[b].n)         # the longest first lends its workspaces
    for b in order:
        w = ws_[b]
        K_all[b, :, :w.n_cap].copy_(torch.from_numpy(w.K))
        V_all[b, :, :w.n_cap].copy_(torch.from_numpy(w.V))
        pk = csa.pack_kv_4bit(K_all[b], V_all[b], packed_all.slot(B, b))
        by_b[b] = prepare_item(csa, torch, w, dev, K_all[b], V_all[b], pk,
                               share=by_b[order[0]] if by_b else None)
    items = [by_b[b] for b in range(B)]
    torch.cuda.synchronize()
    per_req = certified_leg(csa, torch, timer, items, 16 * max(1, iters // 16) * 1, warm)

    def batch(i, events):
        for it in items:
            csa.certified_decode_attention(it["q"], it["K"], it["V"], it["packed"], it["n"], workspace=it["ws"],
                                           out=it["out"], step=i, **it["kw"])

    def dbatch(i, _):
        for it in items:
            csa.dense_decode_attention(it["q"], it["K"], it["V"], it["n"], workspace=it["dws"], out=it["dout"])

    bt = timer.calls(batch, iters)
    dbt = timer.calls(dbatch, iters)
    flat = [bool(w.extra["flat"]) for w in ws_]
    stops = [items[b]["out"][2].cpu().numpy() for b in range(B)]
    keys = [items[b]["out"][3].cpu().numpy() for b in range(B)]
    # the same step as one batched call
    qb = torch.stack([it["q"] for it in items])
    bitems = [dict(n=w.n, slot=b, eps=w.eps, seed=w.seed, step=0, layer=w.layer) for b, w in enumerate(ws_)]
    nbytes = csa.workspace_bytes_batch(K_all, GQA, B, N_CTX, 48, WINDOW)
    bws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    bout = (torch.empty((B, H_KV * GQA, D), dtype=torch.float32, device=dev),
            torch.empty((B, H_KV * GQA), dtype=torch.float64, device=dev),
            torch.empty((B, H_KV * GQA), dtype=torch.int32, device=dev),
            torch.empty((B, H_KV * GQA), dtype=torch.int64, device=dev))

    def one_call(i, _):
        for it in bitems:
            it["step"] = i
        csa.certified_decode_attention_batch(qb, K_all, V_all, packed_all, bitems, delta=0.01, r=2, J=48,
                                             window=WINDOW, workspace=bws, out=bout)
    for i in range(warm):
        one_call(i, None)
    torch.cuda.synchronize()
    ot = timer.calls(one_call, iters)
    bstops = bout[2].cpu().numpy()
    return {"workload": "16 requests x (8 KV heads x GQA 4), n ~ U{16384..131072}, eps in {0.02, 0.05, 0.1}, "
                        "odd requests near-flat (query x 0.1), delta=0.01, r=2, J=48",
            "batched_call_ms": pct(ot), "batched_call_steps_per_s": 1e3 / float(np.median(ot)),
            "single_calls_ms": pct(bt), "single_calls_steps_per_s": 1e3 / float(np.median(bt)),
            "dense_batch_ms": pct(dbt),
            "n": [int(w.n) for w in ws_], "eps": [float(w.eps) for w in ws_],
            "keys_read_median": {"peaked": float(np.median(np.concatenate([k for k, f in zip(keys, flat) if not f]))),
                                 "near_flat": float(np.median(np.concatenate([k for k, f in zip(keys, flat) if f])))},
            "stop_level_median": {"peaked": float(np.median(np.concatenate([s for s, f in zip(stops, flat) if not f]))),
                                  "near_flat": float(np.median(np.concatenate([s for s, f in zip(stops, flat) if f])))},
            "fallback_heads": int(sum(int((s > 48).sum()) for s in stops)),
            "batched_fallback_heads": int((bstops > 48).sum()),
            "per_request_call_ms": per_req["call_ms"], "per_request_scan_kernel_ms": per_req["scan_kernel_ms"]}


def leg_full_step_batched(csa, torch, dev, layers, K_all, V_all, packed_all, w0, iters, warm):
    """All L layers' attention calls of one decode step in one batched call (item l = layer
    l, cache slot l, fresh perturbations per layer and step).  In a model the layers run
    one after the other; the batched call is the form for independent work (requests of a
    batch, or a layer's calls gathered by a scheduler)."""
    L = len(layers)
    q = torch.stack([ly["q"] for ly in layers])
    items = [dict(n=N_CTX, slot=l, eps=w0.eps, seed=w0.seed, step=0, layer=ly["layer"]) for l, ly in enumerate(layers)]
    nbytes = csa.workspace_bytes_batch(K_all, GQA, L, N_CTX, w0.J, WINDOW)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    H_q = H_KV * GQA
    out = (torch.empty((L, H_q, D), dtype=torch.float32, device=dev), torch.empty((L, H_q), dtype=torch.float64, device=dev),
           torch.empty((L, H_q), dtype=torch.int32, device=dev), torch.empty((L, H_q), dtype=torch.int64, device=dev))

    def call(i, _=None):
        for it in items:
            it["step"] = i
        csa.certified_decode_attention_batch(q, K_all, V_all, packed_all, items, delta=w0.delta, r=w0.r, J=w0.J,
                                             window=WINDOW, workspace=ws, out=out)
    for i in range(warm):
        call(i)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
    for i in range(iters):
        evs[i][0].record()
        call(warm + i)
        evs[i][1].record()
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in evs]
    stops = out[2].cpu().numpy()
    keys = out[3].cpu().numpy()
    med = float(np.median(ms))
    return {"workload": f"{L} layers x ({H_KV} KV heads x GQA {GQA}), n={N_CTX}, one batched call per step",
            "call_ms": pct(ms), "full_steps_per_s": 1e3 / med, "layer_calls_per_s": L * 1e3 / med,
            "scan_gbs_whole_call": SCAN_BYTES_PER_TOKEN * (N_CTX - WINDOW) * H_KV * L / (med * 1e-3) / 1e9,
            "workspace_bytes": nbytes,
            "keys_read_median": float(np.median(keys)), "stop_level_median": float(np.median(stops)),
            "fallback_heads": int((stops > w0.J).sum())}


def leg_appending(csa, torch, dev, steps=256):
    """The Qwen-shaped layer (4 KV heads x GQA 7) over 256 decode steps: n = 131072 + t, query
    AR(1), fresh perturbations each step, a block packed whenever an append completes it.
    Returns the timing and the per-step outputs (for the failure rate)."""
    import synth
    w = synth.config5_base(steps=steps)
    n0 = w.n
    K = torch.from_numpy(w.K).to(dev)
    V = torch.from_numpy(w.V).to(dev)
    packed = csa.pack_kv_4bit(K, V, block_end=n0 // 32)
    nb = n0 // 32
    qs = torch.from_numpy(np.ascontiguousarray(w.extra["q_seq"])).to(dev)
    H_q = w.H_q
    ws = csa.allocate_workspace(K, w.G, n0 + steps, w.J, w.window)
    dws = dense_ws(csa, K, w.G, n0 + steps, torch)
    o_all = torch.empty((steps, H_q, D), dtype=torch.float32, device=dev)
    st_all = torch.empty((steps, H_q), dtype=torch.int32, device=dev)
    kr_all = torch.empty((steps, H_q), dtype=torch.int64, device=dev)
    beta = torch.empty(H_q, dtype=torch.float64, device=dev)
    kw = dict(eps=w.eps, delta=w.delta, r=w.r, J=w.J, window=w.window, seed=w.seed)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for t in range(steps):
        n = n0 + t
        while n // 32 > nb:
            csa.pack_kv_4bit(K, V, packed, block_begin=nb, block_end=nb + 1)
            nb += 1
        csa.certified_decode_attention(qs[t], K, V, packed, n, workspace=ws, step=t,
                                       out=(o_all[t], beta, st_all[t], kr_all[t]), **kw)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    dout = torch.empty((H_q, D), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    d0 = time.perf_counter()
    for t in range(steps):
        csa.dense_decode_attention(qs[t], K, V, n0 + t, workspace=dws, out=dout)
    torch.cuda.synchronize()
    del_ = time.perf_counter() - d0
    stops = st_all.cpu().numpy()
    res = {"workload": "4 KV heads x GQA 7, d=128, n = 131072 + t for t = 0..255, query AR(1) rho=0.95, "
                       "fresh perturbations per step, eps=0.05, delta=0.01, r=2, J=48",
           "steps": steps, "ms_per_step": el * 1e3 / steps, "steps_per_s": steps / el,
           "dense_ms_per_step": del_ * 1e3 / steps,
           "certified_heads": int((stops <= w.J).sum()), "heads": int(stops.size),
           "keys_read_median": float(np.median(kr_all.cpu().numpy()))}
    return res, {"w": w, "o": o_all.cpu().numpy().astype(np.float64), "stop": stops}


# ---------------------------------------------------------------- CPU legs (the only place
# bench.py touches the oracle)
def _oracle_head_job(args):
    """Worker: the oracle's certified decode of one KV head of layer 0 (timed)."""
    h, = args
    import oracle
    from threadpoolctl import threadpool_limits
    st = _WORKER
    with threadpool_limits(1):
        t0 = time.perf_counter()
        oracle.certified_decode(st["q"][h * GQA:(h + 1) * GQA], st["K"][h], st["V"][h], st["pk"], h, st["n"],
                                eps=st["eps"], delta=st["delta"], r=st["r"], J=st["J"], window=WINDOW,
                                seed=st["seed"], layer=0, with_dense=False)
        return time.perf_counter() - t0


_WORKER = {}


def _oracle_worker_init():
    import oracle
    import synth
    from threadpoolctl import threadpool_limits
    with threadpool_limits(1):
        w = synth.config3_layer(0)
        _WORKER.update(q=w.q, K=w.K, V=w.V, n=w.n, eps=w.eps, delta=w.delta, r=w.r, J=w.J, seed=w.seed,
                       pk=oracle.pack_kv_4bit(w.K, w.V, w.n // 32))


def cpu_legs(w0, appending):
    """The oracle as it stands on one layer step of the 128K layer: on one core, and with
    a process per KV head; a CPU fp64 dense attention of the same step; and the appending
    layer's empirical failure rate against the oracle's exact attention."""
    import multiprocessing as mp
    from concurrent.futures import ProcessPoolExecutor
    from threadpoolctl import threadpool_limits
    import oracle
    out = {}
    with threadpool_limits(1):
        t0 = time.perf_counter()
        pk = oracle.pack_kv_4bit(w0.K, w0.V, w0.n // 32)
        t1 = time.perf_counter()
        oracle.certified_decode_layer(w0.q, w0.K, w0.V, pk, w0.n, GQA, eps=w0.eps, delta=w0.delta, r=w0.r,
                                      J=w0.J, window=w0.window, seed=w0.seed, layer=0, with_dense=False)
        t2 = time.perf_counter()
        for h in range(H_KV):
            oracle.dense_attention_heads(w0.q[h * GQA:(h + 1) * GQA], w0.K[h], w0.V[h], w0.n)
        t3 = time.perf_counter()
    out["one_core_s"] = t2 - t1
    out["pack_s"] = t1 - t0
    out["dense_fp64_one_core_s"] = t3 - t2
    workers = max(1, min(H_KV, host_cores(), 16))
    log(f"oracle with {workers} worker processes (each generates and packs the layer first)")
    with ProcessPoolExecutor(max_workers=workers, mp_context=mp.get_context("spawn"),
                             initializer=_oracle_worker_init) as ex:
        list(ex.map(_oracle_head_job, [(h,) for h in range(workers)]))        # warm: data ready in each
        t4 = time.perf_counter()
        per = list(ex.map(_oracle_head_job, [(h,) for h in range(H_KV)]))
        t5 = time.perf_counter()
    out["all_cores_s"] = t5 - t4
    out["workers"] = workers
    out["per_head_s_median"] = float(np.median(per))
    if appending is not None:
        w, o_all, stops = appending["w"], appending["o"], appending["stop"]
        n0 = w.extra["n0"]
        steps = o_all.shape[0]
        K64 = [w.K[h, :n0 + steps].astype(np.float64) for h in range(w.H_kv)]
        V64 = [w.V[h, :n0 + steps].astype(np.float64) for h in range(w.H_kv)]
        fails = cert = 0
        for t in range(steps):
            q16 = w.extra["q_seq"][t]
            for h in range(w.H_kv):
                d = oracle.dense_attention_heads(q16[h * w.G:(h + 1) * w.G], w.K[h], w.V[h], n0 + t, K64[h], V64[h])
                for g in range(w.G):
                    hq = h * w.G + g
                    if stops[t, hq] <= w.J:
                        cert += 1
                        fails += float(np.linalg.norm(o_all[t, hq] - d["o"][g])) > w.eps * d["M"][g]
        out["appending_failure"] = {"fails": fails, "certified": cert, "trials": int(stops.size),
                                    "rate": fails / stops.size}
    return out


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the certified decode "
              "path has no multi-GPU form", file=sys.stderr)
        sys.exit(2)
    import torch
    import certified_sparse_attention_amd as csa
    dev = torch.device("cuda:0")
    L = args.layers
    t_gen = time.perf_counter()
    layers = []
    w0 = None
    # the step's caches in one tensor [L][H_kv][n][128] (layer l = cache slot l), packed as
    # L * H_kv heads; single calls take a layer's views
    K_all = torch.empty((L, H_KV, N_CTX, D), dtype=torch.float16, device=dev)
    V_all = torch.empty_like(K_all)
    packed_all = csa.PackedKV.allocate(L * H_KV, N_CTX, dev)
    for w in gen_layers(L):
        if w0 is None:
            w0 = w
        l = w.layer
        K_all[l].copy_(torch.from_numpy(w.K))
        V_all[l].copy_(torch.from_numpy(w.V))
        K, V = K_all[l], V_all[l]
        q = torch.from_numpy(w.q).to(dev)
        packed = csa.pack_kv_4bit(K, V, packed_all.slot(L, l))
        layers.append({"q": q, "K": K, "V": V, "packed": packed, "layer": w.layer})
        if w is not w0:
            del w
        if len(layers) % 8 == 0 or len(layers) == L:
            log(f"{len(layers)}/{L} layers generated and packed ({time.perf_counter() - t_gen:.0f} s)")
    torch.cuda.synchronize()
    t_gen = time.perf_counter() - t_gen
    kw = dict(eps=w0.eps, delta=w0.delta, r=w0.r, J=w0.J, window=w0.window, seed=w0.seed)
    ws = csa.allocate_workspace(layers[0]["K"], GQA, N_CTX, w0.J, WINDOW)
    H_Q = H_KV * GQA
    outs = (torch.empty((H_Q, D), dtype=torch.float32, device=dev),
            torch.empty(H_Q, dtype=torch.float64, device=dev),
            torch.empty(H_Q, dtype=torch.int32, device=dev),
            torch.empty(H_Q, dtype=torch.int64, device=dev))

    def step(i, events=None):
        ly = layers[i % L]
        return csa.certified_decode_attention(ly["q"], ly["K"], ly["V"], ly["packed"], N_CTX, workspace=ws,
                                              layer=ly["layer"], step=i, out=outs, scan_events=events, **kw)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # the headline: exactly --steps steps between two synchronizations; the scan's own
    # start/end times are taken on every EVENT_EVERY-th of them
    ev_steps = list(range(0, args.steps, EVENT_EVERY))
    evs = {i: (csa.Event(), csa.Event()) for i in ev_steps}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, (evs[i][0].handle, evs[i][1].handle) if i in evs else None)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    scan_ms = [a.elapsed_ms(b) for a, b in evs.values()]
    scan_avg_ms = float(np.mean(scan_ms))
    stop_levels = outs[2].cpu().numpy().tolist()
    keys = outs[3].cpu().numpy().tolist()

    # distributions over STATS_ITERS calls: the certified call, its scan kernel, dense
    iters = args.stats_iters
    timer = Timer(csa, torch, max(iters, 16))
    stats_keys, stats_stops = [], []

    def stat_step(i, events):
        r = step(args.warmup + args.steps + i, events)
        stats_keys.append(r[3].clone())
        stats_stops.append(r[2].clone())
    call_ms = timer.calls(stat_step, iters)
    scan_ms_all = timer.scans(stat_step, iters)
    kr = torch.stack(stats_keys).cpu().numpy()
    sl = torch.stack(stats_stops).cpu().numpy()

    dws = dense_ws(csa, layers[0]["K"], GQA, N_CTX, torch)
    dout = torch.empty((H_Q, D), dtype=torch.float32, device=dev)

    def dstep(i, _=None):
        ly = layers[i % L]
        csa.dense_decode_attention(ly["q"], ly["K"], ly["V"], N_CTX, workspace=dws, out=dout)
    for i in range(args.warmup):
        dstep(i)
    torch.cuda.synchronize()
    d0 = time.perf_counter()
    for i in range(args.steps):
        dstep(i)
    torch.cuda.synchronize()
    dense_ms = (time.perf_counter() - d0) * 1e3 / args.steps
    dense_dist = timer.calls(dstep, iters)

    npool = N_CTX - WINDOW
    scan_bytes = SCAN_BYTES_PER_TOKEN * npool * H_KV
    # context for the roofline: a plain read (16-byte loads, no arithmetic) of the scan's
    # byte count, rotating over L separate buffers so each read is as cold as the scan's
    nb = int(scan_bytes)
    rbufs = torch.empty((L, nb), dtype=torch.uint8, device=dev)
    sink = torch.empty(4096, dtype=torch.int32, device=dev)
    for i in range(args.warmup):
        csa.stream_read(rbufs[i % L], sink=sink)
    rev = [(csa.Event(), csa.Event()) for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        csa.stream_read(rbufs[(args.warmup + i) % L], sink=sink, events=(rev[i][0].handle, rev[i][1].handle))
    torch.cuda.synchronize()
    read_ms = float(np.mean([a.elapsed_ms(b) for a, b in rev]))
    del rbufs
    # the scan kernel's average launch duration: its own dispatch start and end events on
    # every one of the STATS_ITERS distribution calls (the timed steps' every-EVENT_EVERY-th
    # launches are reported beside it)
    scan_mean_ms = float(np.mean(scan_ms_all))
    achieved = scan_bytes / (scan_mean_ms * 1e-3) / 1e9
    dense_bytes = DENSE_BYTES_PER_TOKEN * N_CTX * H_KV
    result = {
        "metric": "certified decode-attn steps/s + HBM GB/s (% peak), 8 KV heads d=128 @128K",
        "value": 1e3 / ms_per_step,
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f64",
        "data": "synthetic",
        "config": {"workload": f"one layer of a {L}-layer decode step, rotating layers: {H_KV} KV heads x GQA "
                               f"{GQA}, d={D}, n={N_CTX}, fp16 K/V, sink U(1,6) + 1% power-law heavy "
                               "hitters, eps=0.05, delta=0.01, r=2, J=48, window 64",
                   "n": N_CTX, "kv_heads": H_KV, "group": GQA, "layers_rotated": L},
        "roofline": {"bound": "hbm", "kernel": "scan_kernel", "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": scan_traffic(),
                     "algorithmic_bytes_per_launch": scan_bytes, "avg_launch_ms": scan_mean_ms,
                     "launches": len(scan_ms_all), "timed_steps_avg_launch_ms": scan_avg_ms,
                     "timed_steps_launches": len(scan_ms), "timed_every": EVENT_EVERY},
        "read_ceiling": {"kernel": "stream_read_kernel (16-byte loads only, 4096 workgroups)",
                         "bytes": nb, "avg_launch_ms": read_ms, "GB/s": nb / (read_ms * 1e-3) / 1e9,
                         "frac": nb / (read_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                         "scan_over_read": scan_mean_ms / read_ms},
        "hbm_gbs_whole_step": scan_bytes / (ms_per_step * 1e-3) / 1e9,
        "distributions_128k": {"iters": iters, "call_ms": pct(call_ms), "scan_kernel_ms": pct(scan_ms_all),
                               "dense_ms": pct(dense_dist),
                               "scan_gbs_median": scan_bytes / (float(np.median(scan_ms_all)) * 1e-3) / 1e9,
                               "keys_read": {"median": float(np.median(kr)), "p90": float(np.percentile(kr, 90))},
                               "stop_level": {"median": float(np.median(sl)), "p90": float(np.percentile(sl, 90)),
                                              "fallbacks": int((sl > w0.J).sum()), "heads": int(sl.size)}},
        "dense_hip": {"ms_per_step": dense_ms, "steps_per_s": 1e3 / dense_ms,
                      "gbs": dense_bytes / (dense_ms * 1e-3) / 1e9, "frac": dense_bytes / (dense_ms * 1e-3) / 1e9 /
                      HBM_PEAK_GBS, "note": "the library's own dense decode (split kernel about 0.7 of HBM "
                                            "peak), the comparison the speedup is taken against"},
        "speedup_vs_dense_hip": dense_ms / ms_per_step,
        "stop_levels_last_step": stop_levels,
        "keys_read_last_step_median": float(np.median(keys)),
        "setup_s": t_gen,
        "host": {"cpu": cpu_model(), "cores": host_cores(), "gpu": torch.cuda.get_device_name(0),
                 "torch": torch.__version__},
    }
    appending = None
    if not args.headline_only:
        log("full step of all layers in one batched call")
        result["full_step_batched"] = leg_full_step_batched(csa, torch, dev, layers, K_all, V_all, packed_all, w0,
                                                            max(10, iters // 5), 3)
        torch.cuda.empty_cache()
        for name, fn in (("config_32k_layer", lambda: leg_32k(csa, torch, timer, dev, iters, args.warmup)),
                         ("config_ragged_batch", lambda: leg_ragged(csa, torch, timer, dev, iters, args.warmup))):
            log(f"{name} leg")
            result[name] = fn()
            torch.cuda.empty_cache()
        log("config_appending_gqa7 leg (256 steps)")
        result["config_appending_gqa7"], appending = leg_appending(csa, torch, dev)
    if not args.no_cpu_baseline:
        log("CPU legs: the oracle on layer 0 (1 core, then a process per KV head), CPU fp64 dense")
        c = cpu_legs(w0, appending)
        result["cpu_baseline"] = {
            "value": 1.0 / c["one_core_s"], "unit": "steps/s", "cores": 1, "kind": "oracle",
            "sample": f"one certified decode step of layer 0 (all {H_KV} KV heads x {GQA} query heads, n={N_CTX}) "
                      f"by the fp64 oracle on 1 thread: {c['one_core_s']:.2f} s (packing the layer, a prefill step, "
                      f"took a further {c['pack_s']:.2f} s and is not timed)",
            "all_cores": {"value": 1.0 / c["all_cores_s"], "unit": "steps/s", "cores": c["workers"],
                          "sample": f"the same step with one worker process per KV head ({c['workers']} processes, "
                                    f"1 thread each): {c['all_cores_s']:.2f} s"},
            "dense_fp64": {"value": 1.0 / c["dense_fp64_one_core_s"], "unit": "steps/s", "cores": 1,
                           "sample": "exact fp64 attention of the same step (all heads) on 1 thread: "
                                     f"{c['dense_fp64_one_core_s']:.2f} s"},
            "cpu_model": cpu_model(),
        }
        if "appending_failure" in c:
            result["config_appending_gqa7"]["failure_vs_oracle_exact"] = c["appending_failure"]
    print(json.dumps(result, default=lambda o: o.item() if hasattr(o, "item") else str(o)))


if __name__ == "__main__":
    main()
