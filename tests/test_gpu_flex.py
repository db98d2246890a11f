"""GPU parity of the FlexPrefill baseline path (JSD routing, gamma-cumsum VS
budget, the shared PEIndex and attention) against the fp64 oracle's flex_head,
on the 4k, 32k, 128k, 256k (Qwen-shaped, GQA 7) and 512k layers (128k and
512k are the ones the bench times), under the rules of parity.py: routing and
selection in full, outputs
in full at 4k and on sampled blocks (and, at 512k, sampled rows) above; plus two
sequences with GQA 4 at 32k, outputs in full."""
import gc

import numpy as np
import pytest
import torch

import long_context_sparse_patsearch_amd as crisp
from oracle.driver import layer_selection_flex
from parity import (cfg_kwargs, check_csr_structure, check_flex_selection, check_outputs, device_inputs,
                    gpu_flex_layer, rows_of, sample_blocks)
from prefill_inputs import WORKLOADS, workload_inputs

pytestmark = pytest.mark.gpu

TAU_JSD = 0.1


def _log(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("idx", [1, 2, 3, 4, 5], ids=lambda i: WORKLOADS[i].name)
def test_flex_layer_parity(idx):
    wl = WORKLOADS[idx]
    sh = wl.shape
    nb = sh.n_blocks
    inp = workload_inputs(wl)
    q, k, v = device_inputs(inp)
    cfg = crisp.config(tau=wl.tau, alpha=1.0, gamma=wl.gamma, k_min_tokens=wl.k_min_tokens)
    ckw = cfg_kwargs(cfg)
    kw = dict(tau_jsd=TAU_JSD, gamma=ckw["gamma"], k_min_tokens=ckw["k_min_tokens"])
    _log(f"[{wl.name}] flex gpu layer")
    g = gpu_flex_layer(q, k, v, cfg, TAU_JSD)
    check_csr_structure(g, sh.batch * sh.h_q, nb, crisp.max_blocks(crisp.shape_of(q, k)))
    _log(f"[{wl.name}] flex oracle selection")
    ora = layer_selection_flex(inp["q"], inp["k"], **kw)
    ora, stats = check_flex_selection(g, inp, ora, kw, sh.h_q, nb)
    _log(f"[{wl.name}] flex selection ok: tiles={int(g['row_ptr'][-1])} exempt diffs={stats}")
    # the JSD router agrees with the planted roles on these inputs
    assert np.array_equal(g["pattern"].astype(bool), inp["is_vs"].reshape(-1)), (g["pattern"], inp["is_vs"])
    rng = np.random.default_rng(100 + idx)
    blocks = {bh: (range(nb) if idx == 1 else sample_blocks(nb, rng)) for bh in ora}
    q_rows = None if sh.n <= 131072 else np.unique(np.concatenate([[0, 1, 63, 64, 126, 127],
                                                                   rng.integers(0, 128, 2)]))
    rows = {bh: rows_of(g, bh[0] * sh.h_q + bh[1], nb) for bh in ora}
    worst, mean = check_outputs(g["out"], inp, rows, blocks, q_rows=q_rows)
    _log(f"[{wl.name}] flex outputs ok: max-abs {worst:.2e} mean-abs {mean:.2e}")
    del g, q, k, v
    gc.collect()
    torch.cuda.empty_cache()


def test_flex_batch2_gqa():
    """The FlexPrefill path with two sequences and GQA 4 (32k tokens): routing and selection in full,
    outputs on every block of every head."""
    from prefill_inputs import Shape, make_inputs
    sh = Shape(2, 32768, 8, 2, 128)
    nb = sh.n_blocks
    inp = make_inputs(sh, vs_fraction=0.5, sink_scale=3.0, n_vert=16, seed=777)
    q, k, v = device_inputs(inp)
    cfg = crisp.config()
    ckw = cfg_kwargs(cfg)
    kw = dict(tau_jsd=TAU_JSD, gamma=ckw["gamma"], k_min_tokens=ckw["k_min_tokens"])
    g = gpu_flex_layer(q, k, v, cfg, TAU_JSD)
    check_csr_structure(g, sh.batch * sh.h_q, nb, crisp.max_blocks(crisp.shape_of(q, k)))
    ora = layer_selection_flex(inp["q"], inp["k"], **kw)
    ora, stats = check_flex_selection(g, inp, ora, kw, sh.h_q, nb)
    _log(f"[flex batch2] selection ok: tiles={int(g['row_ptr'][-1])} exempt diffs={stats}")
    rows = {bh: rows_of(g, bh[0] * sh.h_q + bh[1], nb) for bh in ora}
    worst, mean = check_outputs(g["out"], inp, rows, {bh: range(nb) for bh in ora})
    _log(f"[flex batch2] outputs ok: max-abs {worst:.2e} mean-abs {mean:.2e}")
