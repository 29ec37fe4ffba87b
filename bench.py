"""Benchmark: certified decode-attention steps/s at 128K context, 8 KV heads, d = 128.

One step is one certified decode step of one layer: all 8 KV heads x GQA 4 query
heads at n = 131072 over a 16-bit cache (window and exact reads, the 4-bit scan,
the exact maximum, buckets, exact rescoring, level sums, certificates, the stop).
The timed loop rotates over the 32 layers of a Llama-3.1-8B-shaped decode step
(synthetic sink + power-law heavy-hitter caches, 16 GiB of K/V resident in HBM) so
that no layer's data is still in the 256 MB Infinity Cache when it is read again.

Prints one JSON line (rank 0 only).  Only one GPU is used: --gpus above 1 exits.
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


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=64)
    p.add_argument("--warmup", type=int, default=8)
    p.add_argument("--layers", type=int, default=32)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain 1 GiB device-to-device copy 4 times (reference for "
                        "scaling the FETCH_SIZE / WRITE_SIZE counters)")
    return p.parse_args()


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


def gen_layers(nlayers, chunk=8):
    """Synthetic layers in order, generated on host threads a chunk at a time."""
    import synth
    with ThreadPoolExecutor(max_workers=chunk) as ex:
        for c0 in range(0, nlayers, chunk):
            for w in ex.map(synth.config3_layer, range(c0, min(nlayers, c0 + chunk))):
                yield w


def cpu_baseline(w0):
    """The oracle as it stands on one whole layer step (all 8 KV heads) of layer 0."""
    from threadpoolctl import threadpool_limits
    import oracle
    with threadpool_limits(1):
        t0 = time.perf_counter()
        pk = oracle.pack_kv_4bit(w0.K, w0.V, w0.n // 32)
        t1 = time.perf_counter()
        oracle.certified_decode_layer(w0.q, w0.K, w0.V, pk, w0.n, GQA, eps=w0.eps, delta=w0.delta, r=w0.r,
                                      J=w0.J, window=w0.window, seed=w0.seed, layer=0, with_dense=False)
        t2 = time.perf_counter()
    return {"value": 1.0 / (t2 - t1), "unit": "steps/s", "cores": 1, "kind": "oracle",
            "sample": f"one certified decode step of layer 0 (all {H_KV} KV heads x {GQA} query heads, "
                      f"n={N_CTX}) by the fp64 oracle on 1 thread: {t2 - t1:.2f} s; packing the layer "
                      f"took a further {t1 - t0:.2f} s (prefill, not timed)"}


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
    for w in gen_layers(L):
        if w0 is None:
            w0 = w
        K = torch.from_numpy(w.K).to(dev)
        V = torch.from_numpy(w.V).to(dev)
        q = torch.from_numpy(w.q).to(dev)
        packed = csa.pack_kv_4bit(K, V)
        layers.append({"q": q, "K": K, "V": V, "packed": packed, "layer": w.layer})
        if w is not w0:
            del w
        if len(layers) % 8 == 0 or len(layers) == L:
            print(f"[bench] {len(layers)}/{L} layers generated and packed "
                  f"({time.perf_counter() - t_gen:.0f} s)", file=sys.stderr, flush=True)
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
    # the scan's own start/end times are taken on every EVENT_EVERY-th timed step (each
    # timed pair costs a few microseconds of the step it is in)
    ev_steps = list(range(0, args.steps, EVENT_EVERY))
    evs = {i: (csa.Event(), csa.Event()) for i in ev_steps}
    stop_levels, keys = [], []
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

    # dense HIP decode at the same shape, same rotation
    dws = torch.empty(int(csa.api._lib.load().csa_dense_workspace_bytes(
        csa.api._shape(layers[0]["K"], GQA), N_CTX)), dtype=torch.uint8, device=dev)
    dout = torch.empty((H_Q, D), dtype=torch.float32, device=dev)
    for i in range(args.warmup):
        ly = layers[i % L]
        csa.dense_decode_attention(ly["q"], ly["K"], ly["V"], N_CTX, workspace=dws, out=dout)
    torch.cuda.synchronize()
    d0 = time.perf_counter()
    for i in range(args.steps):
        ly = layers[i % L]
        csa.dense_decode_attention(ly["q"], ly["K"], ly["V"], N_CTX, workspace=dws, out=dout)
    torch.cuda.synchronize()
    dense_ms = (time.perf_counter() - d0) * 1e3 / args.steps

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
    achieved = scan_bytes / (scan_avg_ms * 1e-3) / 1e9
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
                     "algorithmic_bytes_per_launch": scan_bytes, "avg_launch_ms": scan_avg_ms,
                     "timed_launches": len(scan_ms), "timed_every": EVENT_EVERY},
        "read_ceiling": {"kernel": "stream_read_kernel (16-byte loads only, 4096 workgroups)",
                         "bytes": nb, "avg_launch_ms": read_ms, "GB/s": nb / (read_ms * 1e-3) / 1e9,
                         "frac": nb / (read_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                         "scan_over_read": scan_avg_ms / read_ms},
        "hbm_gbs_whole_step": scan_bytes / (ms_per_step * 1e-3) / 1e9,
        "dense_hip": {"ms_per_step": dense_ms, "steps_per_s": 1e3 / dense_ms,
                      "gbs": dense_bytes / (dense_ms * 1e-3) / 1e9},
        "speedup_vs_dense_hip": dense_ms / ms_per_step,
        "stop_levels_last_step": stop_levels,
        "keys_read_last_step_median": float(np.median(keys)),
        "setup_s": t_gen,
        "host": {"cpu": platform.processor() or platform.machine(), "cores": os.cpu_count(),
                 "gpu": torch.cuda.get_device_name(0), "torch": torch.__version__},
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on layer 0", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(w0)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
