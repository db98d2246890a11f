"""Seeded synthetic Q/K/V for one attention layer, stored as bf16 bit patterns.

The pages evaluate the method on prefill activations of Llama-3.1-8B and
Qwen2.5-7B over long-context benchmarks; neither the weights nor the data
exist here, so these inputs stand in for them with the same shapes (heads,
grouped KV heads, head dimension, token counts) and a planted attention
structure of the two kinds the pages route between:

* "VS-planted" query heads attend to a few fixed key columns (an attention
  sink at keys 0-3 plus a set of random "vertical" keys) and to their own
  position (a slash/diagonal), the vertical-slash head type of the digest
  page "CRISP: Cliff-awaRe Input-adaptive Sparse Prefilling with
  Structural-Mass-Motivated Routing", section on the VS/PE dichotomy.
* "PE-diffuse" query heads are small random queries whose attention spreads
  over all keys, the pooled-estimation head type of the same section.

Recipe (all draws float32, then rounded to bf16 with round-to-nearest-even):

1. Base values.  VS query heads: Q ~ N(0, 1).  PE query heads: Q ~ N(0, 0.1^2)
   (0.1 read as a standard deviation).  K, V ~ N(0, 1) per KV head, except
   that a KV head used only by PE heads in a multi-head (non-grouped) layout
   draws K, V ~ N(0, 0.1^2) too (the tiny workload's diffuse head).
2. Planting, per KV group g that serves at least one VS head: a random unit
   vector u_g; sink keys 0..3; n_vert distinct random keys in [128, n-128).
   Each planted *set* of size k gets a logit bonus
   Delta = s + ln(n / k) for the stated scale s, so that against n
   background keys the set holds mass of order e^s / (e^s + 1); this reads the
   "scale" of the planted vector as a logit gap in the background-mass model
   epsilon = e^-Delta / (k + (n-k) e^-Delta) of the digest's method section.
   Concretely every VS query of group g gains a*u_g and every key of a set
   gains c*u_g, with a = sqrt(Delta_sink*sqrt(d)) and c = Delta_set*sqrt(d)/a,
   so that (a*u).(c*u)/sqrt(d) = Delta_set.
3. Slash: every VS query row i gains 0.5*k_i (its own position's planted key).

Nothing here computes attention, routing or block selection.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "Shape",
    "Workload",
    "WORKLOADS",
    "workload",
    "head_roles",
    "make_inputs",
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
]


@dataclass(frozen=True)
class Shape:
    batch: int
    n: int
    h_q: int
    h_kv: int
    d: int

    @property
    def group(self) -> int:
        return self.h_q // self.h_kv

    @property
    def n_blocks(self) -> int:
        return self.n // 128


@dataclass(frozen=True)
class Workload:
    """One attention layer's synthetic input recipe plus its method settings."""

    name: str
    shape: Shape
    vs_fraction: float          # share of query heads that are VS-planted
    sink_scale: float           # logit scale s of the planted sets
    n_vert: int                 # planted vertical keys per KV group
    slash: float = 0.5          # q_i += slash * k_i on VS heads
    pe_std: float = 0.1         # std of PE-diffuse queries
    alphas: tuple = (1.0,)      # noise-floor multipliers this workload is run at
    seed: int = 0
    tau: float = 0.2
    gamma: float = 0.95
    k_min_tokens: int = 1024
    tags: dict = field(default_factory=dict, compare=False, hash=False)


def _wl(idx, name, shape, vs, s, nv, alphas):
    return Workload(name=name, shape=shape, vs_fraction=vs, sink_scale=s,
                    n_vert=nv, alphas=alphas, seed=1000 * idx)


# The five single-layer workloads.  Index 1 is small enough for the fp64
# oracle to finish everything in seconds; 3 and 5 are the 128k / 512k layers.
WORKLOADS = {
    1: _wl(1, "tiny_n4096_h2_d64", Shape(1, 4096, 2, 2, 64), 0.5, 3.0, 4, (1.0,)),
    2: _wl(2, "llama3_8b_layer_n32768", Shape(1, 32768, 32, 8, 128), 0.5, 3.0, 16, (1.0,)),
    3: _wl(3, "llama3_8b_layer_n131072", Shape(1, 131072, 32, 8, 128), 0.75, 3.0, 64, (1.0, 1.25)),
    4: _wl(4, "qwen2_7b_layer_n262144", Shape(1, 262144, 28, 4, 128), 0.9, 4.0, 128, (1.0,)),
    5: _wl(5, "llama3_8b_layer_n524288", Shape(1, 524288, 32, 8, 128), 0.75, 3.0, 64, (1.0, 1.25)),
}


def workload(idx: int) -> Workload:
    return WORKLOADS[idx]


def head_roles(h_q: int, h_kv: int, vs_fraction: float) -> np.ndarray:
    """Boolean per query head: True = VS-planted, False = PE-diffuse.

    n_pe = h_q - round(vs_fraction * h_q) heads are PE.  With grouped KV heads
    they are taken in the order (position inside the group, descending; group,
    ascending), so every group keeps its first heads VS; without grouping the
    last heads are PE.
    """
    if h_q % h_kv:
        raise ValueError("h_q must be a multiple of h_kv")
    g = h_q // h_kv
    n_vs = int(round(vs_fraction * h_q))
    n_pe = h_q - n_vs
    if g == 1:
        order = list(range(h_q - 1, -1, -1))
    else:
        order = sorted(range(h_q), key=lambda h: (-(h % g), h // g))
    is_vs = np.ones(h_q, dtype=bool)
    is_vs[order[:n_pe]] = False
    return is_vs


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest, ties to even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u >> np.uint32(16)) & np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u
    r >>= np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _plant_group(rng, n, d, n_vert, sink_scale):
    u = rng.standard_normal(d)
    u = u / np.linalg.norm(u)
    n_vert = max(0, min(n_vert, n - 256))
    vert = np.sort(rng.choice(np.arange(128, n - 128), size=n_vert, replace=False)) if n_vert else np.zeros(0, np.int64)
    sink = np.arange(min(4, n))
    d_sink = sink_scale + math.log(n / len(sink))
    a = math.sqrt(d_sink * math.sqrt(d))
    c_sink = d_sink * math.sqrt(d) / a
    c_vert = (sink_scale + math.log(n / n_vert)) * math.sqrt(d) / a if n_vert else 0.0
    return dict(u=u.astype(np.float32), sink=sink, vert=vert, a=np.float32(a),
                c_sink=np.float32(c_sink), c_vert=np.float32(c_vert))


def make_inputs(shape: Shape, *, vs_fraction: float = 0.5, sink_scale: float = 3.0,
                n_vert: int = 4, slash: float = 0.5, pe_std: float = 0.1,
                seed: int = 0, is_vs: np.ndarray | None = None, workers: int | None = None):
    """Generate one layer's inputs.

    Returns a dict with ``q`` [batch][h_q][n][d], ``k`` and ``v``
    [batch][h_kv][n][d] as uint16 bf16 bit patterns, ``is_vs`` (bool per query
    head) and ``planted`` (per batch, per group: sink and vertical key indices).
    Deterministic in (shape, parameters, seed); the thread count does not
    change the result.
    """
    B, n, H, Hk, d = shape.batch, shape.n, shape.h_q, shape.h_kv, shape.d
    if H % Hk:
        raise ValueError("h_q must be a multiple of h_kv")
    G = H // Hk
    if is_vs is None:
        is_vs = head_roles(H, Hk, vs_fraction)
    is_vs = np.asarray(is_vs, dtype=bool)
    q = np.empty((B, H, n, d), np.uint16)
    k = np.empty((B, Hk, n, d), np.uint16)
    v = np.empty((B, Hk, n, d), np.uint16)
    planted = [[None] * Hk for _ in range(B)]

    def task(bg):
        b, g = bg
        # One seed stream per (batch, group): planting, K, V, then each query head.
        ss = np.random.SeedSequence([seed, b, g])
        kids = ss.spawn(3 + G)
        heads = list(range(g * G, (g + 1) * G))
        any_vs = bool(is_vs[heads].any())
        kv_std = 1.0 if (any_vs or G > 1) else pe_std
        kg = np.random.Generator(np.random.PCG64(kids[1])).standard_normal((n, d), dtype=np.float32)
        vg = np.random.Generator(np.random.PCG64(kids[2])).standard_normal((n, d), dtype=np.float32)
        if kv_std != 1.0:
            kg *= np.float32(kv_std)
            vg *= np.float32(kv_std)
        info = None
        if any_vs:
            info = _plant_group(np.random.Generator(np.random.PCG64(kids[0])), n, d, n_vert, sink_scale)
            kg[info["sink"]] += info["c_sink"] * info["u"]
            if len(info["vert"]):
                kg[info["vert"]] += info["c_vert"] * info["u"]
        for j, h in enumerate(heads):
            qh = np.random.Generator(np.random.PCG64(kids[3 + j])).standard_normal((n, d), dtype=np.float32)
            if is_vs[h]:
                qh += info["a"] * info["u"]
                qh += np.float32(slash) * kg
            else:
                qh *= np.float32(pe_std)
            q[b, h] = f32_to_bf16_bits(qh)
            del qh
        k[b, g] = f32_to_bf16_bits(kg)
        v[b, g] = f32_to_bf16_bits(vg)
        planted[b][g] = None if info is None else dict(sink=info["sink"], vert=info["vert"])

    tasks = [(b, g) for b in range(B) for g in range(Hk)]
    if workers is None:
        workers = min(16, os.cpu_count() or 1, len(tasks))
    if workers <= 1:
        for t in tasks:
            task(t)
    else:
        with ThreadPoolExecutor(workers) as ex:
            list(ex.map(task, tasks))
    return dict(q=q, k=k, v=v, is_vs=is_vs, planted=planted)


def workload_inputs(wl: Workload, workers: int | None = None):
    return make_inputs(wl.shape, vs_fraction=wl.vs_fraction, sink_scale=wl.sink_scale,
                       n_vert=wl.n_vert, slash=wl.slash, pe_std=wl.pe_std, seed=wl.seed,
                       workers=workers)
