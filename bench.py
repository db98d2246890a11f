"""Benchmark of the CRISP sparse-attention prefill on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload llama512k]

A step is one pass of the whole method over one synthetic attention layer
already resident in HBM: crisp_route (PatSearch proxy + structural mass),
crisp_select (VS noise floor / PE gamma-cumsum, block CSR) and
crisp_sparse_attn (exact attention over the selected blocks).  Prints one JSON
line with the per-layer time, the attention kernel against the bf16 MFMA
roofline, the in-house dense kernel on the same layer, and the fp64 oracle
timed on the host cores on a bounded sample.  Progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse prefill attn ms/layer at 128k & 512k; MFMA util; x vs dense"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
ALIASES = {"tiny": 1, "llama32k": 2, "llama128k": 3, "qwen256k": 4, "llama512k": 5}
TILE_FLOP_PER_D = 4.0 * 128 * 128   # QK^T + PV of one 128x128 tile, per unit of head dim


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="llama512k", help="|".join(ALIASES))
    ap.add_argument("--alpha", type=float, default=None, help="default: the workload's first setting")
    ap.add_argument("--also", default="llama512k@1.25,llama512k@1.5,llama128k,llama128k@1.25",
                    help="extra workload[@alpha] list reported under 'also' ('' = none)")
    ap.add_argument("--dense-steps", type=int, default=1)
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-flex", action="store_true", help="skip the FlexPrefill baseline path")
    ap.add_argument("--no-probe", action="store_true", help="skip the measured MFMA-rate probe")
    ap.add_argument("--no-variants", action="store_true", help="skip the selection variants (median floor, slash band, per-row PE)")
    ap.add_argument("--tau-jsd", type=float, default=0.1, help="JSD threshold of the FlexPrefill router")
    ap.add_argument("--traffic", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="measured HBM bytes per attention launch (JSON), if current")
    ap.add_argument("--copy-calibration", type=int, default=0,
                    help="only run a device copy of this many MiB (HBM counter calibration) and exit")
    ap.add_argument("--model-sweep", type=int, default=0, metavar="LAYERS",
                    help="only sum CRISP, FlexPrefill and dense attention over this many Llama-3.1-8B-shaped "
                         "layers (distinct seeds) at 64k, 128k, 256k and 512k tokens")
    ap.add_argument("--sweep-lengths", default="65536,131072,262144,524288")
    ap.add_argument("--sweep-n-vert", type=int, default=64, help="planted vertical keys per KV group in the sweep")
    ap.add_argument("--crossover", action="store_true",
                    help="only sweep the sequence length (Llama-shaped layers, 4k-128k) and report where the "
                         "sparse path overtakes dense attention")
    return ap.parse_args()


def source_sha256(name="attn.hip"):
    """Digest of a kernel source file: HBM counters taken on another version are not reported."""
    import hashlib
    path = os.path.join(ROOT, "long_context_sparse_patsearch_amd", "csrc", name)
    with open(path, "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()


def attn_source_sha256():
    return source_sha256("attn.hip")


STAGE_SOURCES = {"route": "route.hip", "select": "select.hip", "attn": "attn.hip"}


def _stored_traffic(path, workload, alpha, tiles):
    if not path or not os.path.exists(path):
        return None
    with open(path) as fh:
        tr = json.load(fh)
    if tr.get("workload") == workload and tr.get("alpha") == alpha and tr.get("tiles") == tiles:
        return tr
    return None


def measured_traffic(path, workload, alpha, tiles):
    """HBM bytes per attention launch from the stored counter run, or None when that run
    measured another workload, setting, tile count or attention source."""
    tr = _stored_traffic(path, workload, alpha, tiles)
    if tr and tr.get("attn_source_sha256") == attn_source_sha256():
        return tr.get("bytes_per_launch")
    return None


def measured_stage_bytes(path, workload, alpha, tiles):
    """HBM bytes per call of each stage (route, select, the whole attention call) from the
    stored FETCH_SIZE / WRITE_SIZE runs, for the stages whose source is unchanged since."""
    tr = _stored_traffic(path, workload, alpha, tiles)
    if not tr:
        return {}
    srcs = tr.get("sources", {})
    return {st: b for st, b in tr.get("stages", {}).items()
            if st in STAGE_SOURCES and srcs.get(STAGE_SOURCES[st]) == source_sha256(STAGE_SOURCES[st])}


def _event():
    import torch
    return torch.cuda.Event(enable_timing=True)


class Layer:
    """One workload resident on the GPU with every buffer preallocated."""

    def __init__(self, idx):
        import numpy as np
        import torch

        import long_context_sparse_patsearch_amd as crisp
        from prefill_inputs import WORKLOADS, workload_inputs

        self.crisp = crisp
        self.wl = WORKLOADS[idx] if isinstance(idx, int) else idx
        sh = self.wl.shape
        t0 = time.perf_counter()
        self.inp = workload_inputs(self.wl)
        log(f"[bench] {self.wl.name}: inputs generated in {time.perf_counter() - t0:.1f}s")
        dev = torch.device("cuda:0")
        self.q, self.k, self.v = (torch.from_numpy(self.inp[t].view(np.int16)).to(dev).view(torch.bfloat16)
                                  for t in ("q", "k", "v"))
        self.shape = crisp.shape_of(self.q, self.k)
        bh, nb = sh.batch * sh.h_q, sh.n_blocks
        self.bh, self.nb = bh, nb
        cfg0 = crisp.config()
        self.r_out = dict(c_struct=torch.empty(bh, dtype=torch.float32, device=dev),
                          pattern=torch.empty(bh, dtype=torch.int8, device=dev),
                          p_vert=torch.empty(bh, nb, dtype=torch.float32, device=dev),
                          p_slash=torch.empty(bh, nb, dtype=torch.float32, device=dev))
        self.s_out = dict(row_ptr=torch.empty(bh * nb + 1, dtype=torch.int64, device=dev),
                          col_idx=torch.empty(crisp.max_blocks(self.shape), dtype=torch.int32, device=dev))
        self.o = torch.empty(self.q.shape, dtype=torch.float32, device=dev)
        self.ws_r = torch.empty(max(1, crisp.workspace_bytes(self.shape, cfg0, 0)), dtype=torch.uint8, device=dev)
        self.ws_s = torch.empty(max(1, crisp.workspace_bytes(self.shape, cfg0, 1)), dtype=torch.uint8, device=dev)

    def cfg(self, alpha):
        wl = self.wl
        return self.crisp.config(tau=wl.tau, alpha=alpha, gamma=wl.gamma, k_min_tokens=wl.k_min_tokens)

    def step(self, cfg, evs=None, variant=0):
        c = self.crisp
        if evs:
            evs[0].record()
        c.route(self.q, self.k, cfg, out=self.r_out, ws=self.ws_r)
        if evs:
            evs[1].record()
        c.select(self.q, self.k, self.r_out, cfg, out=self.s_out, ws=self.ws_s, variant=variant)
        if evs:
            evs[2].record()
        c.sparse_attn(self.q, self.k, self.v, self.s_out, cfg, out=self.o)
        if evs:
            evs[3].record()

    def measure(self, alpha, steps, warmup, variant=0):
        import numpy as np
        import torch
        cfg = self.cfg(alpha)
        for _ in range(warmup):
            self.step(cfg, variant=variant)
        torch.cuda.synchronize()
        evs = [[_event() for _ in range(4)] for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            self.step(cfg, evs[i], variant=variant)
        torch.cuda.synchronize()
        wall_ms = (time.perf_counter() - t0) * 1e3 / steps
        per = {"route": [e[0].elapsed_time(e[1]) for e in evs], "select": [e[1].elapsed_time(e[2]) for e in evs],
               "attn": [e[2].elapsed_time(e[3]) for e in evs]}
        st = {k_: sum(v_) / steps for k_, v_ in per.items()}
        med = {k_: float(np.median(v_)) for k_, v_ in per.items()}
        layer_med = float(np.median([sum(x) for x in zip(*per.values())]))
        tiles = int(self.s_out["row_ptr"][-1].item())
        pattern = self.r_out["pattern"].cpu().numpy()
        sh = self.wl.shape
        flop = tiles * TILE_FLOP_PER_D * sh.d
        dense_tiles = self.bh * self.nb * (self.nb + 1) // 2
        return dict(workload=self.wl.name, alpha=alpha, ms_per_layer=wall_ms,
                    stage_ms={k_: round(v_, 4) for k_, v_ in st.items()},
                    stage_ms_median={k_: round(v_, 4) for k_, v_ in med.items()},
                    layer_ms_median=round(layer_med, 4), tiles=tiles,
                    tile_fraction=tiles / dense_tiles, vs_heads=int(pattern.sum()),
                    pe_heads=int(len(pattern) - pattern.sum()), attn_flop=flop,
                    attn_tflops=flop / (st["attn"] * 1e-3) / 1e12, _pattern=pattern)

    def flex_step(self, cfg, tau_jsd, evs=None):
        c = self.crisp
        if evs:
            evs[0].record()
        c.route(self.q, self.k, cfg, out=self.r_out, ws=self.ws_r)
        if evs:
            evs[1].record()
        f = c.flex_route(self.q, self.k, self.r_out, tau_jsd, cfg, out=self.f_out, ws=self.ws_f)
        if evs:
            evs[2].record()
        c.flex_select(self.q, self.k, f, cfg, out=self.s_out, ws=self.ws_s)
        if evs:
            evs[3].record()
        c.sparse_attn(self.q, self.k, self.v, self.s_out, cfg, out=self.o)
        if evs:
            evs[4].record()

    def measure_flex(self, alpha, tau_jsd, steps, warmup):
        """The FlexPrefill baseline path on the same layer (JSD routing, gamma-cumsum VS budget)."""
        import torch
        cfg = self.cfg(alpha)
        dev = self.q.device
        self.f_out = dict(jsd=torch.empty(self.bh, dtype=torch.float32, device=dev),
                          pattern=torch.empty(self.bh, dtype=torch.int8, device=dev))
        self.ws_f = torch.empty(max(1, self.crisp.workspace_bytes(self.shape, cfg, self.crisp.CALL_FLEX_ROUTE)),
                                dtype=torch.uint8, device=dev)
        for _ in range(warmup):
            self.flex_step(cfg, tau_jsd)
        torch.cuda.synchronize()
        evs = [[_event() for _ in range(5)] for _ in range(steps)]
        t0 = time.perf_counter()
        for i in range(steps):
            self.flex_step(cfg, tau_jsd, evs[i])
        torch.cuda.synchronize()
        wall_ms = (time.perf_counter() - t0) * 1e3 / steps
        names = ("route", "flex_route", "select", "attn")
        st = {nm: sum(e[j].elapsed_time(e[j + 1]) for e in evs) / steps for j, nm in enumerate(names)}
        tiles = int(self.s_out["row_ptr"][-1].item())
        pattern = self.f_out["pattern"].cpu().numpy()
        self.f_out = self.ws_f = None
        return dict(workload=self.wl.name, tau_jsd=tau_jsd, gamma=self.wl.gamma, ms_per_layer=round(wall_ms, 3),
                    stage_ms={k_: round(v_, 4) for k_, v_ in st.items()}, tiles=tiles,
                    vs_heads=int(pattern.sum()), pe_heads=int(len(pattern) - pattern.sum()))

    def dense(self, steps):
        import torch
        c = self.crisp
        c.dense_attn(self.q, self.k, self.v, out=self.o)
        torch.cuda.synchronize()
        e0, e1 = _event(), _event()
        e0.record()
        for _ in range(steps):
            c.dense_attn(self.q, self.k, self.v, out=self.o)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        flop = self.bh * self.nb * (self.nb + 1) / 2 * TILE_FLOP_PER_D * self.wl.shape.d
        return ms, flop / (ms * 1e-3) / 1e12

    def host_csr(self):
        rp = self.s_out["row_ptr"].cpu().numpy()
        col = self.s_out["col_idx"][: int(rp[-1])].cpu().numpy()
        return rp, col

    def free(self):
        import torch
        for name in ("q", "k", "v", "o", "ws_r", "ws_s", "s_out", "r_out", "f_out", "ws_f"):
            setattr(self, name, None)
        torch.cuda.empty_cache()


def mfma_rate():
    """The bf16 MFMA rate this GPU sustains (crisp_mfma_probe, two waves per SIMD on every CU),
    with random bf16 operands in [-2, 2) and with zeros; HIP events on the current stream."""
    import torch
    import long_context_sparse_patsearch_amd as crisp
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(1234)
    out = {}
    for name, ops in (("random_operands", torch.empty(crisp.PROBE_OPERAND_BYTES // 2, dtype=torch.bfloat16,
                                                      device=dev).uniform_(-2.0, 2.0, generator=g)),
                      ("zero_operands", torch.zeros(crisp.PROBE_OPERAND_BYTES // 2, dtype=torch.bfloat16, device=dev))):
        crisp.mfma_probe(ops, iters=2000)
        torch.cuda.synchronize()
        e0, e1 = _event(), _event()
        e0.record()
        flop = crisp.mfma_probe(ops, iters=20000)
        e1.record()
        torch.cuda.synchronize()
        out[name + "_tflops"] = round(flop / (e0.elapsed_time(e1) * 1e-3) / 1e12, 1)
    out["published_tflops"] = PEAK_BF16_TFLOPS
    return out


def cpu_baseline(layer, res, rp, col):
    """The fp64 oracle as it stands, on a bounded sample of the same layer.

    Routing + selection run in full (every head of the layer, heads in
    parallel over the workers); exact attention runs on forty-eight random query
    blocks per worker, of random heads, on the GPU's own block lists, and is
    extrapolated linearly (by selected tiles) to the whole layer."""
    import numpy as np

    from oracle.driver import default_workers, layer_attention, layer_selection

    wl = layer.wl
    H, nb = wl.shape.h_q, wl.shape.n_blocks
    pattern = res["_pattern"]
    cfg = layer.cfg(res["alpha"])
    ckw = dict(tau=float(np.float32(cfg.tau)), alpha=float(np.float32(cfg.alpha)),
               gamma=float(np.float32(cfg.gamma)), k_min_tokens=cfg.k_min_tokens)
    workers = default_workers()
    rng = np.random.default_rng(0)
    heads = list(range(H))
    n_pe = int(np.count_nonzero(pattern == 0))
    t0 = time.perf_counter()
    layer_selection(layer.inp["q"], layer.inp["k"], heads=[(0, h) for h in heads], workers=workers, **ckw)
    t_sel = time.perf_counter() - t0
    t_sel_layer = t_sel
    # attention sample
    blocks = {}
    rows_of = {}
    for _ in range(48 * workers):
        h = int(rng.integers(0, H))
        qb = int(rng.integers(0, nb))
        blocks.setdefault((0, h), []).append(qb)
    sampled_tiles = 0
    for (b, h), qbs in blocks.items():
        rows_of[(b, h)] = {qb: col[rp[h * nb + qb]: rp[h * nb + qb + 1]].astype(np.int64) for qb in qbs}
        sampled_tiles += sum(len(rows_of[(b, h)][qb]) for qb in qbs)
    t0 = time.perf_counter()
    layer_attention(layer.inp["q"], layer.inp["k"], layer.inp["v"], rows_of, blocks, workers=workers)
    t_attn = time.perf_counter() - t0
    t_attn_layer = t_attn * res["tiles"] / max(1, sampled_tiles)
    return {"value": round((t_sel_layer + t_attn_layer) * 1e3, 1), "unit": "ms/layer", "cores": workers,
            "kind": "oracle",
            "sample": (f"routing+selection of all {H} heads ({n_pe} PE) in full and exact attention on "
                       f"{sum(len(v) for v in blocks.values())} random query blocks ({sampled_tiles} of "
                       f"{res['tiles']} selected tiles) of {wl.name}, the attention extrapolated linearly to "
                       f"one layer; measured {t_sel:.1f}s + {t_attn:.1f}s"),
            "stage_ms": {"route_select": round(t_sel_layer * 1e3, 1), "attn": round(t_attn_layer * 1e3, 1)}}


def stage_rates(sh, res, counted=None):
    """Algorithmic bytes / time of the routing and selection stages (GB/s), and, where a
    current counter run exists, the HBM bytes the counters measured / time.

    route: one pass reads every KV head's K once, plus the 128 proxy query rows
    of every head.  select: PEIndex reads the Q of its PE heads and the K of
    every KV group holding one, then passes over each PE head's triangular map
    of N_b(N_b+1)/2 fp32 scores six times (logits written; softmax read and
    written; three radix passes read)."""
    kv = sh.batch * sh.h_kv * sh.n * sh.d * 2
    route_b = kv + sh.batch * sh.h_q * 128 * sh.d * 2
    pe = res["pe_heads"]
    pe_groups = min(sh.batch * sh.h_kv, pe)   # at most one group per PE head
    tri = sh.n_blocks * (sh.n_blocks + 1) // 2
    sel_b = pe * sh.n * sh.d * 2 + pe_groups * sh.n * sh.d * 2 + 6 * 4 * tri * pe
    out = {"route": round(route_b / (res["stage_ms"]["route"] * 1e-3) / 1e9, 1), "route_bytes": route_b,
           "select": round(sel_b / (res["stage_ms"]["select"] * 1e-3) / 1e9, 1), "select_bytes": sel_b,
           "peak_hbm_gbs": 8000.0}
    for st, b in (counted or {}).items():
        if st in ("route", "select"):
            out[f"{st}_counter_bytes"] = b
            out[f"{st}_counter_gbs"] = round(b / (res["stage_ms"][st] * 1e-3) / 1e9, 1)
    return out


def crossover_workload(n):
    """A Llama-shaped layer of n tokens from the 128k layer's recipe (75% VS heads,
    sink scale 3), with the planted vertical keys scaled with n."""
    from prefill_inputs import Shape, Workload
    return Workload(name=f"llama3_8b_layer_n{n}", shape=Shape(1, n, 32, 8, 128), vs_fraction=0.75,
                    sink_scale=3.0, n_vert=max(4, round(64 * n / 131072)), alphas=(1.0,),
                    seed=9000 + n.bit_length())


def sweep_workload(n, layer, n_vert=64):
    """Layer `layer` of a Llama-3.1-8B-shaped model at n tokens: the recipe of the 128k and
    512k layers (75% VS heads, sink scale 3, 64 planted vertical keys per KV group)."""
    from prefill_inputs import Shape, Workload
    return Workload(name=f"llama3_8b_model_n{n}_layer{layer}", shape=Shape(1, n, 32, 8, 128), vs_fraction=0.75,
                    sink_scale=3.0, n_vert=n_vert, alphas=(1.0,), seed=20000 + 100 * n.bit_length() + layer)


def model_sweep(args):
    """Attention-only whole-model totals: sum over the layers of one prefill."""
    rows = []
    for n in [int(x) for x in args.sweep_lengths.split(",") if x]:
        tot = dict(crisp=0.0, flex=0.0, tiles=0, flex_tiles=0)
        dense_ms = None
        for L in range(args.model_sweep):
            layer = Layer(sweep_workload(n, L, args.sweep_n_vert))
            r = layer.measure(1.0, 2, 1)
            f = layer.measure_flex(1.0, args.tau_jsd, 2, 1)
            if dense_ms is None:
                dense_ms, _ = layer.dense(max(1, args.dense_steps))
            tot["crisp"] += r["ms_per_layer"]
            tot["flex"] += f["ms_per_layer"]
            tot["tiles"] += r["tiles"]
            tot["flex_tiles"] += f["tiles"]
            log(f"[sweep] n={n} layer {L}: CRISP {r['ms_per_layer']:.2f} ms, FlexPrefill {f['ms_per_layer']:.2f} ms")
            layer.free()
        L = args.model_sweep
        rows.append(dict(n=n, layers=L, crisp_ms=round(tot["crisp"], 1), flex_ms=round(tot["flex"], 1),
                         dense_ms=round(dense_ms * L, 1), crisp_vs_dense=round(dense_ms * L / tot["crisp"], 3),
                         flex_vs_dense=round(dense_ms * L / tot["flex"], 3),
                         crisp_vs_flex=round(tot["flex"] / tot["crisp"], 3), tiles=tot["tiles"],
                         flex_tiles=tot["flex_tiles"]))
        log(f"[sweep] n={n}: {rows[-1]}")
    print(json.dumps({"model_sweep": rows, "model": "Llama-3.1-8B-shaped, 32/8 heads, d=128, attention only",
                      "n_vert": args.sweep_n_vert,
                      "dense": "one layer's dense time x layers (dense time depends only on the shape)"}))


def crossover(args):
    """Sparse layer (route + select + attention) vs dense attention over n."""
    rows = []
    for n in (4096, 5120, 6144, 7168, 8192, 10240, 12288, 16384, 32768, 65536, 131072):
        layer = Layer(crossover_workload(n))
        res = layer.measure(1.0, max(args.steps, 5), max(args.warmup, 2))
        dense_ms, _ = layer.dense(max(args.dense_steps, 5))
        rows.append(dict(n=n, sparse_ms=round(res["ms_per_layer"], 3), stage_ms=res["stage_ms"],
                         dense_ms=round(dense_ms, 3), tile_fraction=round(res["tile_fraction"], 4),
                         speedup=round(dense_ms / res["ms_per_layer"], 3)))
        log(f"[crossover] n={n}: sparse {res['ms_per_layer']:.3f} ms (route {res['stage_ms']['route']:.3f}, "
            f"select {res['stage_ms']['select']:.3f}), dense {dense_ms:.3f} ms, x{dense_ms / res['ms_per_layer']:.2f}")
        layer.free()
    first = next((r["n"] for r in rows if r["speedup"] > 1.0), None)
    print(json.dumps({"crossover": rows, "sparse_faster_from_n": first}))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported: the method is per attention "
              "head and this library runs one GPU's share of heads (sharding across GPUs is not implemented).",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if args.copy_calibration:
        nbytes = args.copy_calibration << 20
        # an elementwise kernel that reads nbytes and writes nbytes (dst = src + 1)
        src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.add(src, 1, out=dst)
        torch.cuda.synchronize()
        print(json.dumps({"copy_kernel": "torch.add(uint8, 1)", "read_bytes_per_launch": nbytes,
                          "write_bytes_per_launch": nbytes, "launches": 3}))
        return

    if args.crossover:
        crossover(args)
        return
    if args.model_sweep:
        model_sweep(args)
        return

    idx = ALIASES.get(args.workload) or int(args.workload)
    specs = [(idx, args.alpha)]
    for spec in [x for x in args.also.split(",") if x]:
        name, _, a = spec.partition("@")
        specs.append((ALIASES.get(name) or int(name), float(a) if a else None))
    order = []
    for j, _ in specs:
        if j not in order:
            order.append(j)
    results, dense, keep, flex, variants = [], {}, None, [], []
    for j in order:
        layer = Layer(j)
        for jj, a in specs:
            if jj != j:
                continue
            a = layer.wl.alphas[0] if a is None else a
            if any(r["workload"] == layer.wl.name and r["alpha"] == a for r in results):
                continue
            primary = j == idx and not results
            # the primary line times exactly --steps; the shorter layers of the 'also' list take the
            # median of at least 10 steps (their stages are a few ms, so more steps cost little)
            steps = args.steps if primary or layer.wl.shape.n > 131072 else max(args.steps, 10)
            r = layer.measure(a, steps, args.warmup)
            r["steps"] = steps
            log(f"[bench] {r['workload']} alpha={a}: {r['ms_per_layer']:.2f} ms/layer {r['stage_ms']} "
                f"tiles={r['tiles']} attn {r['attn_tflops']:.1f} TFLOP/s")
            r["_primary"] = primary
            results.append(r)
            if r["_primary"]:
                rp, col = layer.host_csr()
                keep = (layer, rp, col, r)
                if not args.no_variants:
                    c = layer.crisp
                    for nm, bits in (("median_floor", c.VARIANT_MEDIAN_FLOOR), ("slash_band", c.VARIANT_SLASH_BAND),
                                     ("pe_per_row", c.VARIANT_PE_PER_ROW)):
                        vr = layer.measure(a, 2, 1, variant=bits)
                        variants.append(dict(variant=nm, workload=vr["workload"], alpha=a,
                                             ms_per_layer=round(vr["ms_per_layer"], 3), stage_ms=vr["stage_ms"],
                                             tiles=vr["tiles"]))
                        log(f"[bench] {vr['workload']} variant {nm}: {vr['ms_per_layer']:.2f} ms/layer "
                            f"tiles={vr['tiles']}")
        if not args.no_flex:
            a0 = next(a for jj, a in specs if jj == j)
            a0 = layer.wl.alphas[0] if a0 is None else a0
            fr = layer.measure_flex(a0, args.tau_jsd, args.steps, args.warmup)
            crisp_r = next(r for r in results if r["workload"] == layer.wl.name and r["alpha"] == a0)
            fr["crisp_ms"] = round(crisp_r["ms_per_layer"], 3)
            fr["crisp_tiles"] = crisp_r["tiles"]
            fr["crisp_speedup_over_flex"] = round(fr["ms_per_layer"] / crisp_r["ms_per_layer"], 3)
            flex.append(fr)
            log(f"[bench] {layer.wl.name} FlexPrefill (tau_jsd={args.tau_jsd}, gamma={layer.wl.gamma}): "
                f"{fr['ms_per_layer']:.2f} ms/layer {fr['stage_ms']} tiles={fr['tiles']}; CRISP is "
                f"x{fr['crisp_speedup_over_flex']:.3f} faster")
        if not args.no_dense:
            dense[layer.wl.name] = layer.dense(args.dense_steps)
            log(f"[bench] {layer.wl.name} dense: {dense[layer.wl.name][0]:.1f} ms "
                f"({dense[layer.wl.name][1]:.0f} TFLOP/s)")
        layer.free()
    for r in results:
        if r["workload"] in dense:
            r["dense_ms"], r["dense_tflops"] = dense[r["workload"]]
            r["speedup_vs_dense"] = r["dense_ms"] / r["ms_per_layer"]
    layer, rp, col, res = keep
    alpha = res["alpha"]
    dense_ms, dense_tf = dense.get(res["workload"], (None, None))
    also = [r for r in results if not r["_primary"]]

    traffic = measured_traffic(args.traffic, res["workload"], alpha, res["tiles"])
    tflops = res["attn_tflops"]
    out = {
        "metric": METRIC,
        "value": round(res["ms_per_layer"], 3),
        "unit": "ms/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["ms_per_layer"], 3),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded Gaussian Q/K/V with planted VS and diffuse PE heads)",
        "config": {"workload": res["workload"], "alpha": alpha, "batch": layer.wl.shape.batch,
                   "n": layer.wl.shape.n, "h_q": layer.wl.shape.h_q, "h_kv": layer.wl.shape.h_kv,
                   "d": layer.wl.shape.d, "vs_heads": res["vs_heads"], "pe_heads": res["pe_heads"],
                   "parallelism": "single GPU"},
        "stage_ms": res["stage_ms"],
        "stage_ms_median": res["stage_ms_median"],
        "layer_ms_median": res["layer_ms_median"],
        "tiles": res["tiles"],
        "tile_fraction": round(res["tile_fraction"], 4),
        "mfma_util": round(tflops / PEAK_BF16_TFLOPS, 4),
        "dense_ms": None if dense_ms is None else round(dense_ms, 2),
        "speedup_vs_dense": None if dense_ms is None else round(dense_ms / res["ms_per_layer"], 3),
        "dense_mfma_util": None if dense_tf is None else round(dense_tf / PEAK_BF16_TFLOPS, 4),
        "roofline": {"bound": "mfma", "kernel": "attn_q64_kernel (crisp_sparse_attn)",
                     "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                     "flop_per_launch": res["attn_flop"], "avg_launch_ms": res["stage_ms"]["attn"]},
        "also": [{k_: (round(v_, 4) if isinstance(v_, float) else v_) for k_, v_ in x.items() if not k_.startswith("_")}
                 for x in also],
    }
    # effective rate over the unmasked causal (query, key) pairs of the selected tiles (every row keeps
    # its diagonal tile, of which 128*129/2 pairs are unmasked), and the routing / selection byte rates
    sh = layer.wl.shape
    rows = sh.batch * sh.h_q * sh.n_blocks
    pairs = res["tiles"] * 128 * 128 - rows * (128 * 128 - 128 * 129 // 2)
    out["attn_tflops_causal_pairs"] = round(4 * sh.d * pairs / (res["stage_ms"]["attn"] * 1e-3) / 1e12, 2)
    out["selection_gbs"] = stage_rates(sh, res, measured_stage_bytes(args.traffic, res["workload"], alpha,
                                                                     res["tiles"]))
    if flex:
        out["flexprefill"] = flex
    if variants:
        out["variants"] = variants
    if not args.no_probe:
        mr = mfma_rate()
        mr["attn_frac_of_random_operand_rate"] = round(tflops / mr["random_operands_tflops"], 4)
        out["mfma_rate_measured"] = mr
        log(f"[bench] measured MFMA rate: {mr}")
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle) ...")
        out["cpu_baseline"] = cpu_baseline(layer, res, rp, col)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
