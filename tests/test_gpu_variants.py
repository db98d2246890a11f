"""GPU parity of the selection variants (median noise floor, slash band,
per-row PE gamma-cumsum) against the oracle's crisp_head(floor=..., band=...,
pe_per_row=...): routing and selection in full; outputs in full on the 4k
layer and on sampled blocks at 32k and 128k; all three together on the
Qwen-shaped 256k layer (GQA 7); at 512k (where the bench times each variant)
every variant alone; sampled rows of sampled blocks from 256k on."""
import numpy as np
import pytest

import long_context_sparse_patsearch_amd as crisp
from parity import (cfg_kwargs, check_csr_structure, check_outputs, check_selection, device_inputs, gpu_layer,
                    oracle_layer, rows_of, sample_blocks)
from prefill_inputs import WORKLOADS, workload_inputs

pytestmark = pytest.mark.gpu

VARIANTS = {"median": (crisp.VARIANT_MEDIAN_FLOOR, "median", False, False),
            "band": (crisp.VARIANT_SLASH_BAND, "mean", True, False),
            "median+band": (crisp.VARIANT_MEDIAN_FLOOR | crisp.VARIANT_SLASH_BAND, "median", True, False),
            "pe_row": (crisp.VARIANT_PE_PER_ROW, "mean", False, True),
            "all": (crisp.VARIANT_MEDIAN_FLOOR | crisp.VARIANT_SLASH_BAND | crisp.VARIANT_PE_PER_ROW, "median", True,
                    True)}
CASES = ([(i, v) for i in (1, 2, 3) for v in VARIANTS] + [(4, "all")]
         + [(5, v) for v in ("median", "band", "pe_row")])


@pytest.mark.parametrize("idx,name", CASES, ids=[f"{WORKLOADS[i].name}-{v}" for i, v in CASES])
def test_variant_parity(idx, name):
    variant, floor, band, pe_rows = VARIANTS[name]
    wl = WORKLOADS[idx]
    sh = wl.shape
    nb = sh.n_blocks
    inp = workload_inputs(wl)
    q, k, v = device_inputs(inp)
    cfg = crisp.config(tau=wl.tau, alpha=1.0, gamma=wl.gamma, k_min_tokens=wl.k_min_tokens)
    ckw = cfg_kwargs(cfg)
    g = gpu_layer(q, k, v, cfg, variant=variant)
    check_csr_structure(g, sh.batch * sh.h_q, nb, crisp.max_blocks(crisp.shape_of(q, k)))
    ora = oracle_layer(inp, ckw, floor=floor, band=band, pe_per_row=pe_rows)
    ora, stats = check_selection(g, inp, ora, ckw, sh.h_q, nb, floor=floor, band=band, pe_per_row=pe_rows)
    print(f"[{wl.name} {name}] selection ok: tiles={int(g['row_ptr'][-1])} diffs={stats}", flush=True)
    rng = np.random.default_rng(200 + idx)
    blocks = {bh: (range(nb) if idx == 1 else sample_blocks(nb, rng)) for bh in ora}
    q_rows = None if sh.n <= 131072 else np.unique(np.concatenate([[0, 1, 63, 64, 126, 127],
                                                                   rng.integers(0, 128, 2)]))
    rows = {bh: rows_of(g, bh[0] * sh.h_q + bh[1], nb) for bh in ora}
    worst, mean = check_outputs(g["out"], inp, rows, blocks, q_rows=q_rows)
    print(f"[{wl.name} {name}] outputs ok: max-abs {worst:.2e} mean-abs {mean:.2e}", flush=True)
