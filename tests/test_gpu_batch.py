"""GPU parity with more than one sequence at scale: a batch of two 256k-token
Llama-shaped sequences (32 query / 8 KV heads, d = 128, 75% VS heads).  Q holds
2^31 elements, so the second sequence's element offsets pass 2^31.  Routing
and selection are compared in full against the oracle on all 64 heads;
outputs on 8 rows of the first, middle, last and one random query block of
every head.  Then each sequence alone (batch 1), attended over its own rows of
the batch's CSR, must give the batch run's output bits for that sequence: the
work items of one sequence do not depend on the other's."""
import numpy as np
import pytest
import torch

import long_context_sparse_patsearch_amd as crisp
from parity import (cfg_kwargs, check_csr_structure, check_outputs, check_selection, device_inputs, gpu_layer,
                    oracle_layer, rows_of, sample_blocks)
from prefill_inputs import Shape, make_inputs

pytestmark = pytest.mark.gpu

SHAPE = Shape(2, 262144, 32, 8, 128)


def test_batch_of_two_long_sequences():
    sh = SHAPE
    nb, H = sh.n_blocks, sh.h_q
    assert sh.batch * H * sh.n * sh.d == 1 << 31
    inp = make_inputs(sh, vs_fraction=0.75, sink_scale=3.0, n_vert=64, seed=2626)
    q, k, v = device_inputs(inp)
    cfg = crisp.config()
    ckw = cfg_kwargs(cfg)
    print("[batch2 256k] gpu layer", flush=True)
    g = gpu_layer(q, k, v, cfg)
    check_csr_structure(g, sh.batch * H, nb, crisp.max_blocks(crisp.shape_of(q, k)))
    print("[batch2 256k] oracle selection", flush=True)
    ora = oracle_layer(inp, ckw)
    ora, stats = check_selection(g, inp, ora, ckw, H, nb)
    assert {r["is_vs"] for r in ora.values()} == {True, False}
    print(f"[batch2 256k] selection ok: tiles={int(g['row_ptr'][-1])} diffs={stats}", flush=True)
    rng = np.random.default_rng(2626)
    blocks = {bh: sample_blocks(nb, rng) for bh in ora}
    q_rows = np.unique(np.concatenate([[0, 1, 63, 64, 126, 127], rng.integers(0, 128, 2)]))
    rows = {bh: rows_of(g, bh[0] * H + bh[1], nb) for bh in ora}
    worst, mean = check_outputs(g["out"], inp, rows, blocks, q_rows=q_rows)
    print(f"[batch2 256k] outputs ok: max-abs {worst:.2e} mean-abs {mean:.2e}", flush=True)

    # each sequence alone over its rows of the same CSR: the same bits
    rp = g["sel"]["row_ptr"]
    for b in range(sh.batch):
        r0, r1 = b * H * nb, (b + 1) * H * nb
        base = int(rp[r0])
        sel = dict(row_ptr=(rp[r0:r1 + 1] - base).contiguous(),
                   col_idx=g["sel"]["col_idx"][base:int(rp[r1])].contiguous())
        qb_, kb_, vb_ = (t[b:b + 1].contiguous() for t in (q, k, v))
        one = crisp.sparse_attn(qb_, kb_, vb_, sel, cfg)
        torch.cuda.synchronize()
        assert torch.equal(one[0], g["out"][b]), f"sequence {b} alone gave other bits"
        del one, qb_, kb_, vb_, sel
        print(f"[batch2 256k] sequence {b} alone: same bits", flush=True)
