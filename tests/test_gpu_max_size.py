"""GPU parity at the longest supported input: n = 1,048,576 tokens (N_b = 8192,
the size of the selection kernels' LDS arrays), 4 query heads on one KV head
(two VS, two PE).  Routing and selection are compared in full against the
oracle; outputs on 8 sampled rows of the first, middle, last and one random
query block of every head, plus the dense kernel on two heads.  A second case
runs the d = 64 kernels at 128k tokens with batch 2 and GQA 4: selection in
full, six query blocks of every head with all rows, dense on two heads."""
import numpy as np
import pytest
import torch

import long_context_sparse_patsearch_amd as crisp
from oracle import crisp_oracle as co
from parity import (cfg_kwargs, check_csr_structure, check_outputs, check_selection, device_inputs, gpu_layer,
                    oracle_layer, rows_of, sample_blocks)
from prefill_inputs import Shape, make_inputs

pytestmark = pytest.mark.gpu

SHAPE = Shape(1, 1 << 20, 4, 1, 128)


def test_longest_supported_layer():
    sh = SHAPE
    nb = sh.n_blocks
    assert nb == 8192
    inp = make_inputs(sh, vs_fraction=0.5, sink_scale=3.0, n_vert=64, seed=4242)
    q, k, v = device_inputs(inp)
    cfg = crisp.config()
    ckw = cfg_kwargs(cfg)
    print("[1M] gpu layer", flush=True)
    g = gpu_layer(q, k, v, cfg)
    check_csr_structure(g, sh.batch * sh.h_q, nb, crisp.max_blocks(crisp.shape_of(q, k)))
    print("[1M] oracle selection", flush=True)
    ora = oracle_layer(inp, ckw)
    ora, stats = check_selection(g, inp, ora, ckw, sh.h_q, nb)
    assert {r["is_vs"] for r in ora.values()} == {True, False}
    print(f"[1M] selection ok: tiles={int(g['row_ptr'][-1])} diffs={stats}", flush=True)
    rng = np.random.default_rng(77)
    blocks = {bh: sample_blocks(nb, rng) for bh in ora}
    q_rows = np.unique(np.concatenate([[0, 1, 63, 64, 126, 127], rng.integers(0, 128, 2)]))
    rows = {bh: rows_of(g, bh[0] * sh.h_q + bh[1], nb) for bh in ora}
    worst, mean = check_outputs(g["out"], inp, rows, blocks, q_rows=q_rows)
    print(f"[1M] outputs ok: max-abs {worst:.2e} mean-abs {mean:.2e}", flush=True)
    del g
    dense = crisp.dense_attn(q, k, v)
    torch.cuda.synchronize()
    heads = [(0, 0), (0, 3)]
    drows = {bh: co.dense_rows(nb) for bh in heads}
    dblocks = {bh: [0, nb // 3, nb - 1] for bh in heads}
    worst, mean = check_outputs(dense, inp, drows, dblocks, q_rows=q_rows)
    print(f"[1M] dense ok: max-abs {worst:.2e} mean-abs {mean:.2e}", flush=True)


D64_SHAPE = Shape(2, 131072, 8, 2, 64)


def test_long_d64_layer():
    """The d = 64 kernels (four-wave attention workgroups, 64-dim proxy tiles) at 128k tokens, batch 2,
    GQA 4: selection in full, sampled outputs of the sparse and dense kernels."""
    sh = D64_SHAPE
    nb = sh.n_blocks
    inp = make_inputs(sh, vs_fraction=0.5, sink_scale=3.0, n_vert=32, seed=6464)
    q, k, v = device_inputs(inp)
    cfg = crisp.config()
    ckw = cfg_kwargs(cfg)
    print("[d64 128k] gpu layer", flush=True)
    g = gpu_layer(q, k, v, cfg)
    check_csr_structure(g, sh.batch * sh.h_q, nb, crisp.max_blocks(crisp.shape_of(q, k)))
    ora = oracle_layer(inp, ckw)
    ora, stats = check_selection(g, inp, ora, ckw, sh.h_q, nb)
    assert {r["is_vs"] for r in ora.values()} == {True, False}
    print(f"[d64 128k] selection ok: tiles={int(g['row_ptr'][-1])} diffs={stats}", flush=True)
    rng = np.random.default_rng(64)
    blocks = {bh: sample_blocks(nb, rng, extra=3) for bh in ora}
    rows = {bh: rows_of(g, bh[0] * sh.h_q + bh[1], nb) for bh in ora}
    worst, mean = check_outputs(g["out"], inp, rows, blocks)
    print(f"[d64 128k] outputs ok: max-abs {worst:.2e} mean-abs {mean:.2e}", flush=True)
    del g
    dense = crisp.dense_attn(q, k, v)
    torch.cuda.synchronize()
    heads = [(0, 0), (1, 7)]
    drows = {bh: co.dense_rows(nb) for bh in heads}
    dblocks = {bh: [0, nb // 2, nb - 1] for bh in heads}
    worst, mean = check_outputs(dense, inp, drows, dblocks)
    print(f"[d64 128k] dense ok: max-abs {worst:.2e} mean-abs {mean:.2e}", flush=True)
