"""Seeded synthetic KV caches and queries.

The pages measure on real KV caches of three LLMs (Llama-3.1-8B among them) that
are not available here, so every input is drawn from numpy's PCG64 with a fixed
seed, with the shapes and score structure of the five workloads the method is
exercised on:

* ``config1``: one KV head, a group of 4 queries, n = 4096, keys and values
  N(0, 1), 8 planted heavy keys (x4), each query = 0.15 x a random cached key +
  N(0, 1) noise.
* ``config2``: a Llama-3.1-8B-shaped layer (8 KV heads x GQA 4, d = 128) at
  n = 32768 with an attention sink on tokens 0-3 and 1 % power-law heavy hitters
  aligned with the group's mean query.
* ``config3_layer``: the same recipe at n = 131072 per layer of a 32-layer model,
  sink strength drawn U(1, 6) per layer.
* ``config4_request``: ragged requests n ~ U{16384..131072}, per-request epsilon,
  odd requests with near-flat scores (query x 0.1).
* ``config5_*``: a Qwen2.5-7B-shaped layer (4 KV heads x GQA 7) that appends one
  token per decode step while the query drifts as AR(1) with rho = 0.95.

Layout conventions (the same as the C ABI): ``q`` is fp16 ``[H_q][128]`` with query
head ``hq`` served by KV head ``hq // G``; ``K`` and ``V`` are fp16
``[H_kv][n_cap][128]``, token-major.  Offsets "in nats" along the unit mean query
direction qbar add ``a * sqrt(d) * qbar / |qbar|^2`` to a key, which raises
``qbar . k / sqrt(d)`` by exactly ``a``.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

D = 128
HASH_SEED = 0x5EED


@dataclass
class Workload:
    name: str
    q: np.ndarray          # fp16 [H_q][128]
    K: np.ndarray          # fp16 [H_kv][n_cap][128]
    V: np.ndarray          # fp16 [H_kv][n_cap][128]
    n: int                 # cached tokens in use
    G: int                 # query heads per KV head
    window: int = 64
    r: int = 2
    J: int = 30
    eps: float = 0.05
    delta: float = 0.01
    seed: int = HASH_SEED
    step: int = 0
    layer: int = 0
    extra: dict = field(default_factory=dict)

    @property
    def H_kv(self) -> int:
        return int(self.K.shape[0])

    @property
    def H_q(self) -> int:
        return int(self.q.shape[0])

    @property
    def n_cap(self) -> int:
        return int(self.K.shape[1])


def _normal(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(size=shape, dtype=np.float32)


def recipe_layer(rng: np.random.Generator, H_kv: int, G: int, n: int, *, n_cap: int | None = None,
                 sink: float = 3.5, heavy_frac: float = 0.01, pareto_alpha: float = 1.5,
                 heavy_cap: float = 40.0, window: int = 64, q_scale: float = 1.0):
    """One layer of the sink + power-law heavy-hitter recipe.

    Keys, values and queries are N(0, 1).  Tokens 0-3 get ``+sink`` nats, and
    floor(heavy_frac * n_pool) pool positions (outside the sink) get ``+a`` nats
    with a = U^(-1/alpha) (Pareto, x_m = 1) capped at ``heavy_cap``, both along the
    group's mean query direction.  ``q_scale`` multiplies the queries after the keys
    are built (0.1 gives near-flat scores).  Returns float32 q (unscaled), and fp16
    q, K, V.
    """
    n_cap = n if n_cap is None else n_cap
    q32 = _normal(rng, (H_kv * G, D))
    K = _normal(rng, (H_kv, n_cap, D))
    V = _normal(rng, (H_kv, n_cap, D))
    q16 = q32.astype(np.float16)
    n_pool = max(n - window, 0)
    m = int(np.floor(heavy_frac * n_pool))
    for h in range(H_kv):
        qbar = q16[h * G:(h + 1) * G].astype(np.float64).mean(axis=0)
        dirv = (np.sqrt(D) * qbar / float(qbar @ qbar)).astype(np.float32)
        K[h, :min(4, n)] += np.float32(sink) * dirv
        if m > 0 and n_pool > 4:
            pos = 4 + rng.choice(n_pool - 4, size=min(m, n_pool - 4), replace=False)
            u = 1.0 - rng.random(pos.shape[0])            # (0, 1]
            a = np.minimum(u ** (-1.0 / pareto_alpha), heavy_cap).astype(np.float32)
            K[h, pos] += a[:, None] * dirv[None, :]
    q_out = (q32 * np.float32(q_scale)).astype(np.float16)
    return q32, q_out, K.astype(np.float16), V.astype(np.float16)


def config1() -> Workload:
    """Parity case: 1 KV head, GQA 4, n = 4096, r = 2, J = 30."""
    rng = np.random.default_rng(1)
    n, G, W = 4096, 4, 64
    K = _normal(rng, (1, n, D))
    V = _normal(rng, (1, n, D))
    heavy = rng.choice(n - W, size=8, replace=False)
    K[0, heavy] *= np.float32(4.0)
    picks = rng.integers(0, n, size=G)
    xi = _normal(rng, (G, D))
    q = (np.float32(0.15) * K[0, picks] + xi).astype(np.float16)
    return Workload("config1", q, K.astype(np.float16), V.astype(np.float16), n, G,
                    window=W, r=2, J=30, eps=0.05, delta=0.01,
                    extra={"heavy": heavy, "picks": picks})


def peaked_head(n: int, seed: int, G: int = 4, heavy: int = 8, q_mix: float = 0.15,
                window: int = 64, J: int = 30, eps: float = 0.05, q_scale: float = 1.0) -> Workload:
    """The config1 recipe at any size: one KV head, query = q_mix x a cached key + noise.

    ``q_scale`` multiplies the query (a wider score spread for values above 1).
    """
    rng = np.random.default_rng(seed)
    K = _normal(rng, (1, n, D))
    V = _normal(rng, (1, n, D))
    if heavy and n > window:
        pos = rng.choice(n - window, size=min(heavy, n - window), replace=False)
        K[0, pos] *= np.float32(4.0)
    picks = rng.integers(0, n, size=G)
    q = ((np.float32(q_mix) * K[0, picks] + _normal(rng, (G, D))) * np.float32(q_scale)).astype(np.float16)
    return Workload(f"peaked{n}", q, K.astype(np.float16), V.astype(np.float16), n, G,
                    window=window, r=2, J=J, eps=eps, delta=0.01)


def config2() -> Workload:
    """One Llama-3.1-8B-shaped layer at n = 32768, r = 2, J = 40."""
    rng = np.random.default_rng(2)
    _, q, K, V = recipe_layer(rng, 8, 4, 32768, sink=3.5)
    return Workload("config2", q, K, V, 32768, 4, window=64, r=2, J=40, eps=0.05, delta=0.01)


def config3_layer(layer: int, n: int = 131072) -> Workload:
    """Layer ``layer`` of the 32-layer, n = 131072 full decode step (J = 48)."""
    rng = np.random.default_rng(3 + layer)
    sink = float(rng.uniform(1.0, 6.0))
    _, q, K, V = recipe_layer(rng, 8, 4, n, sink=sink)
    return Workload(f"config3.layer{layer}", q, K, V, n, 4, window=64, r=2, J=48,
                    eps=0.05, delta=0.01, layer=layer, extra={"sink": sink})


def config4_request(b: int) -> Workload:
    """Request ``b`` (0..15) of the ragged batch; odd requests are near-flat."""
    rng = np.random.default_rng(400 + b)
    n = int(rng.integers(16384, 131072, endpoint=True))
    eps = float(rng.choice(np.array([0.02, 0.05, 0.1])))
    _, q, K, V = recipe_layer(rng, 8, 4, n, sink=3.5, q_scale=(0.1 if b % 2 else 1.0))
    return Workload(f"config4.req{b}", q, K, V, n, 4, window=64, r=2, J=48, eps=eps,
                    delta=0.01, seed=HASH_SEED + b, extra={"flat": bool(b % 2)})


def config5_base(n0: int = 131072, steps: int = 256) -> Workload:
    """Qwen2.5-7B-shaped layer (4 KV heads x GQA 7) with room for ``steps`` appends.

    ``extra['q_seq']`` holds the fp16 query of every step: q_0 from the recipe and
    q_t = 0.95 q_(t-1) + sqrt(1 - 0.95^2) xi_t.  Tokens n0.. are plain N(0, 1).
    """
    rng = np.random.default_rng(5)
    q32, _, K, V = recipe_layer(rng, 4, 7, n0, n_cap=n0 + steps, sink=3.5)
    rho = np.float32(0.95)
    c = np.float32(np.sqrt(1.0 - 0.95 ** 2))
    seq = np.empty((steps,) + q32.shape, dtype=np.float16)
    cur = q32.copy()
    for t in range(steps):
        if t > 0:
            cur = rho * cur + c * _normal(rng, q32.shape)
        seq[t] = cur.astype(np.float16)
    return Workload("config5", seq[0], K, V, n0, 7, window=64, r=2, J=48, eps=0.05,
                    delta=0.01, extra={"q_seq": seq, "n0": n0, "steps": steps})


def config5_step_query(w: Workload, t: int) -> np.ndarray:
    return w.extra["q_seq"][t]
