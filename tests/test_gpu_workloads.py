"""GPU parity on the five single-layer workloads at full size.

Routing and selection are compared in full on every head.  Outputs are
compared in full on the 4k and 32k layers.  From 128k tokens on, every head
has 64 query blocks compared with all 128 rows (always the first and the last
block, the middle one and 61 seeded others; PE heads 16 at the layer's later
alphas, since PE selection does not depend on alpha) and one VS head every
block; at the first alpha one PE head has every block compared, with all rows
at 128k and 8 rows per block at 256k (a whole PE head there is about 1.9
million tiles).  Always against the oracle's attention on the GPU's own CSR.
The dense kernel is compared in full on the 4k layer, on every block of 8
heads at 32k and on 64-block samples of 8 heads from 128k on.  The launch configuration is the one the
benchmark times.
"""
import gc
import os

import numpy as np
import pytest
import torch

import long_context_sparse_patsearch_amd as crisp
from oracle import crisp_oracle as co
from parity import (cfg_kwargs, check_csr_structure, check_outputs, check_selection, device_inputs, gpu_layer,
                    oracle_layer, rows_of, sample_blocks)
from prefill_inputs import WORKLOADS, workload_inputs

pytestmark = pytest.mark.gpu

CASES = [(i, a) for i in sorted(WORKLOADS) for a in WORKLOADS[i].alphas]
SAMPLE_BLOCKS = 64      # query blocks per head compared (all rows) from 128k tokens on
_cache = {}


def _state(idx):
    if _cache.get("idx") != idx:
        _cache.clear()
        gc.collect()
        torch.cuda.empty_cache()
        wl = WORKLOADS[idx]
        inp = workload_inputs(wl)
        _cache.update(idx=idx, wl=wl, inp=inp, dev=device_inputs(inp), ora={})
    return _cache


def _log(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("idx,alpha", CASES, ids=[f"{WORKLOADS[i].name}-alpha{a}" for i, a in CASES])
def test_layer_parity(idx, alpha):
    st = _state(idx)
    wl, inp = st["wl"], st["inp"]
    sh = wl.shape
    nb = sh.n_blocks
    cfg = crisp.config(tau=wl.tau, alpha=alpha, gamma=wl.gamma, k_min_tokens=wl.k_min_tokens)
    ckw = cfg_kwargs(cfg)
    q, k, v = st["dev"]
    _log(f"[{wl.name} alpha={alpha}] gpu layer")
    g = gpu_layer(q, k, v, cfg)
    check_csr_structure(g, sh.batch * sh.h_q, nb, crisp.max_blocks(crisp.shape_of(q, k)))
    # every (head, query block) item of the attention's work queues is run, and runs alike every time:
    # a second launch into a NaN-filled buffer must write every element, with the first launch's bits
    again = torch.full_like(g["out"], float("nan"))
    crisp.sparse_attn(q, k, v, g["sel"], cfg, out=again)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(again).all()), "an output row was not written"
    assert torch.equal(again, g["out"]), "a second launch gave other bits"
    again = None
    _log(f"[{wl.name} alpha={alpha}] oracle selection")
    ora = oracle_layer(inp, ckw)
    ora, stats = check_selection(g, inp, ora, ckw, sh.h_q, nb)
    tiles = int(g["row_ptr"][-1])
    _log(f"[{wl.name} alpha={alpha}] selection ok: tiles={tiles} exempt diffs={stats}")
    rng = np.random.default_rng(idx * 10 + int(alpha * 100))
    rows = {bh: rows_of(g, bh[0] * sh.h_q + bh[1], nb) for bh in ora}
    first = alpha == wl.alphas[0]
    if idx in (1, 2):
        blocks = {bh: range(nb) for bh in ora}
    else:
        # 64 blocks per head; PE heads select the same blocks at every alpha, so
        # at later alphas 16 of theirs suffice
        blocks = {bh: sample_blocks(nb, rng, extra=(SAMPLE_BLOCKS if first or ora[bh]["is_vs"] else 16) - 3)
                  for bh in ora}
        blocks[next(x for x in sorted(ora) if ora[x]["is_vs"])] = range(nb)   # one whole VS head
        pe = [x for x in sorted(ora) if not ora[x]["is_vs"]]
        if first and pe and idx == 3:
            blocks[pe[0]] = range(nb)                                          # one whole PE head
        elif first and pe and idx == 4:
            # one whole PE head, 8 rows of each block: its full oracle run costs
            # about 1,500 core-seconds (about 0.9 of all causal tiles selected)
            pe_rows = np.unique(np.concatenate([[0, 1, 63, 64, 126, 127], rng.integers(0, 128, 2)]))
            _log(f"[{wl.name} alpha={alpha}] oracle attention on every block of PE head {pe[0]}, rows {pe_rows}")
            worst, mean = check_outputs(g["out"], inp, {pe[0]: rows[pe[0]]}, {pe[0]: range(nb)}, q_rows=pe_rows)
            _log(f"[{wl.name} alpha={alpha}] whole PE head ok: max-abs {worst:.2e} mean-abs {mean:.2e}")
    _log(f"[{wl.name} alpha={alpha}] oracle attention on {sum(len(b_) for b_ in blocks.values())} query blocks")
    worst, mean = check_outputs(g["out"], inp, rows, blocks)
    _log(f"[{wl.name} alpha={alpha}] outputs ok: max-abs {worst:.2e} mean-abs {mean:.2e}")
    if alpha == wl.alphas[0]:
        dense = crisp.dense_attn(q, k, v, out=torch.full(q.shape, float("nan"), dtype=torch.float32, device=q.device))
        torch.cuda.synchronize()
        assert bool(torch.isfinite(dense).all()), "a dense output row was not written"
        drows = {bh: co.dense_rows(nb) for bh in ora}
        dheads = list(ora)[::max(1, sh.h_q // 8)]
        dblocks = {bh: (range(nb) if idx == 1 else
                        (blocks[bh] if idx == 2 else sample_blocks(nb, rng, extra=SAMPLE_BLOCKS - 3)))
                   for bh in dheads}
        _log(f"[{wl.name}] dense: oracle attention on {sum(len(b_) for b_ in dblocks.values())} query blocks")
        worst, mean = check_outputs(dense, inp, drows, dblocks)
        _log(f"[{wl.name}] dense ok: max-abs {worst:.2e} mean-abs {mean:.2e}")
        del dense
    del g


# The pages' variant settings on the same kernels: alpha = 1.5 (their fastest
# setting at 512k, checked on the 128k and the 512k layer) and the routing
# thresholds tau = 0.15 and 0.25 of their sensitivity study.  Routing and
# selection in full; outputs on sampled blocks (64 per head with all rows and
# one whole VS head at 512k).
VARIANTS = [(5, 1.5, None), (3, 1.5, None), (4, 1.25, None), (2, 1.0, 0.15), (2, 1.0, 0.25)]


@pytest.mark.parametrize("idx,alpha,tau", VARIANTS,
                         ids=[f"{WORKLOADS[i].name}-alpha{a}-tau{t}" for i, a, t in VARIANTS])
def test_variant_settings(idx, alpha, tau):
    st = _state(idx)
    wl, inp = st["wl"], st["inp"]
    sh = wl.shape
    nb = sh.n_blocks
    cfg = crisp.config(tau=wl.tau if tau is None else tau, alpha=alpha, gamma=wl.gamma,
                       k_min_tokens=wl.k_min_tokens)
    ckw = cfg_kwargs(cfg)
    q, k, v = st["dev"]
    g = gpu_layer(q, k, v, cfg)
    check_csr_structure(g, sh.batch * sh.h_q, nb, crisp.max_blocks(crisp.shape_of(q, k)))
    ora = oracle_layer(inp, ckw)
    ora, stats = check_selection(g, inp, ora, ckw, sh.h_q, nb)
    _log(f"[{wl.name} alpha={alpha} tau={ckw['tau']}] selection ok: tiles={int(g['row_ptr'][-1])} "
         f"vs={int(g['pattern'].sum())} diffs={stats}")
    rng = np.random.default_rng(idx * 7 + int(alpha * 10))
    if idx == 5:
        blocks = {bh: sample_blocks(nb, rng, extra=SAMPLE_BLOCKS - 3) for bh in ora}
        blocks[next(x for x in sorted(ora) if ora[x]["is_vs"])] = range(nb)
    else:
        blocks = {bh: sample_blocks(nb, rng) for bh in ora}
    rows = {bh: rows_of(g, bh[0] * sh.h_q + bh[1], nb) for bh in ora}
    worst, mean = check_outputs(g["out"], inp, rows, blocks)
    _log(f"[{wl.name} alpha={alpha} tau={ckw['tau']}] outputs ok: max-abs {worst:.2e} mean-abs {mean:.2e}")
    del g
