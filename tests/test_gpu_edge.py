"""GPU parity on small and degenerate shapes, with full-output comparison.

Every case goes through the C-ABI library and is compared with the fp64 oracle
on the same seeded inputs (prefill_inputs), under the rules of parity.py.
"""
import os
import re

import numpy as np
import pytest
import torch

import long_context_sparse_patsearch_amd as crisp
from oracle import crisp_oracle as co
from oracle.driver import layer_attention
from parity import (MAX_ABS, MEAN_ABS, cfg_kwargs, check_csr_structure, check_outputs, check_selection,
                    device_inputs, gpu_layer, oracle_layer, rows_of, to_dev)
from prefill_inputs import Shape, make_inputs

pytestmark = pytest.mark.gpu

SHAPES = {
    "minimal_nb3_d64": Shape(1, 384, 1, 1, 64),
    "minimal_nb3_d128": Shape(1, 384, 2, 1, 128),
    "ragged_nb9_b2_g2": Shape(2, 1152, 4, 2, 128),
    "gqa7_nb16": Shape(1, 2048, 7, 1, 128),
    "mha_nb32_d64": Shape(1, 4096, 2, 2, 64),
}


def _inputs(sh, seed=11, vs_fraction=0.5, **kw):
    return make_inputs(sh, vs_fraction=vs_fraction, sink_scale=3.0, n_vert=4, seed=seed, **kw)


def _full_blocks(sh):
    return {(b, h): range(sh.n_blocks) for b in range(sh.batch) for h in range(sh.h_q)}


@pytest.mark.parametrize("name", list(SHAPES))
def test_dense_attention_full(name):
    sh = SHAPES[name]
    inp = _inputs(sh, seed=21)
    q, k, v = device_inputs(inp)
    for dt in (torch.float32, torch.bfloat16):
        out = crisp.dense_attn(q, k, v, out_dtype=dt)
        torch.cuda.synchronize()
        rows = {bh: co.dense_rows(sh.n_blocks) for bh in _full_blocks(sh)}
        tol = 1 if dt == torch.float32 else 2
        ref = layer_attention(inp["q"], inp["k"], inp["v"], rows, _full_blocks(sh))
        errs = []
        for (b, h, qb), o in ref.items():
            e = np.abs(out[b, h, qb * 128:(qb + 1) * 128].float().cpu().numpy() - o)
            assert e.max() <= MAX_ABS * tol, (name, dt, b, h, qb, e.max())
            errs.append(e.mean())
        assert np.mean(errs) <= MEAN_ABS * tol


@pytest.mark.parametrize("name", list(SHAPES))
def test_sparse_attention_on_given_csr(name):
    """Random CSR rows (some without the diagonal, some empty, some holding
    blocks after the query block or past the end, some opening with 70 such
    entries, more than one 64-entry read) against the oracle."""
    sh = SHAPES[name]
    nb = sh.n_blocks
    inp = _inputs(sh, seed=31)
    q, k, v = device_inputs(inp)
    rng = np.random.default_rng(5)
    rows_all, rows_oracle = [], {}
    for b in range(sh.batch):
        for h in range(sh.h_q):
            per = []
            for qb in range(nb):
                kind = rng.integers(0, 7)
                if kind == 0:
                    row = []
                elif kind == 1:
                    row = sorted(rng.choice(qb + 1, size=min(qb + 1, 2), replace=False).tolist())
                else:
                    row = sorted(set(rng.choice(qb + 1, size=rng.integers(1, qb + 2), replace=False).tolist()) | {qb})
                if kind == 5 and qb + 1 < nb:
                    row = row + [qb + 1]          # a future block: fully masked
                if kind == 4:
                    row = row + [nb]              # past the end: skipped
                if kind == 6:
                    row = [nb if i % 2 else min(qb + 1, nb) for i in range(70)] + row   # skipped, then valid
                per.append(row)
            rows_all.extend(per)
            rows_oracle[(b, h)] = [np.array([c for c in r if c < nb], dtype=np.int64) for r in per]
    counts = np.array([len(r) for r in rows_all])
    row_ptr = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    col = np.array([c for r in rows_all for c in r] or [0], dtype=np.int32)
    sel = dict(row_ptr=torch.from_numpy(row_ptr).cuda(), col_idx=torch.from_numpy(col).cuda())
    out = crisp.sparse_attn(q, k, v, sel, crisp.config())
    torch.cuda.synchronize()
    check_outputs(out, inp, rows_oracle, _full_blocks(sh))


CASES = [
    ("minimal_nb3_d64", {}),
    ("minimal_nb3_d128", {}),
    ("ragged_nb9_b2_g2", {}),
    ("gqa7_nb16", {}),
    ("mha_nb32_d64", {}),
    ("ragged_nb9_b2_g2", dict(alpha=0.0)),
    ("gqa7_nb16", dict(alpha=1.25, k_min_tokens=0)),
    ("gqa7_nb16", dict(k_min_tokens=2048)),
    ("mha_nb32_d64", dict(gamma=1.0)),
    ("mha_nb32_d64", dict(gamma=0.5, tau=0.05)),
    ("mha_nb32_d64", dict(alpha=3.0, k_min_tokens=1536)),
    ("ragged_nb9_b2_g2", dict(alpha=3.0, k_min_tokens=768)),
]


@pytest.mark.parametrize("name,kw", CASES, ids=[f"{n}-{'-'.join(f'{a}{b}' for a, b in kw.items()) or 'default'}" for n, kw in CASES])
def test_pipeline_small_full(name, kw):
    sh = SHAPES[name]
    inp = _inputs(sh, seed=41)
    cfg = crisp.config(**kw)
    ckw = cfg_kwargs(cfg)
    q, k, v = device_inputs(inp)
    g = gpu_layer(q, k, v, cfg)
    check_csr_structure(g, sh.batch * sh.h_q, sh.n_blocks, crisp.max_blocks(crisp.shape_of(q, k)))
    ora = oracle_layer(inp, ckw)
    ora, _ = check_selection(g, inp, ora, ckw, sh.h_q, sh.n_blocks)
    rows = {bh: rows_of(g, bh[0] * sh.h_q + bh[1], sh.n_blocks) for bh in ora}
    check_outputs(g["out"], inp, rows, _full_blocks(sh))


@pytest.mark.parametrize("vs_fraction", [0.0, 1.0])
def test_pipeline_all_one_kind(vs_fraction):
    sh = Shape(1, 2048, 8, 2, 128)
    inp = _inputs(sh, seed=51, vs_fraction=vs_fraction)
    cfg = crisp.config()
    ckw = cfg_kwargs(cfg)
    g = gpu_layer(*device_inputs(inp), cfg)
    ora = oracle_layer(inp, ckw)
    assert all(r["is_vs"] == bool(vs_fraction) for r in ora.values())
    ora, _ = check_selection(g, inp, ora, ckw, sh.h_q, sh.n_blocks)
    rows = {bh: rows_of(g, bh[1], sh.n_blocks) for bh in ora}
    check_outputs(g["out"], inp, rows, _full_blocks(sh))


def test_pe_ties_uniform_map():
    """Zero queries on the PE heads make every pooled row uniform: equal scores,
    so the gamma cut falls inside a run of ties that must go to the lowest flat
    indices.  With 32 blocks the oracle keeps rows 0-29, 13 cells of row 30 and
    the diagonal of row 31; the GPU must match cell for cell."""
    sh = Shape(1, 4096, 2, 2, 128)
    inp = _inputs(sh, seed=61)
    inp["q"][0, 1] = 0
    cfg = crisp.config()
    ckw = cfg_kwargs(cfg)
    g = gpu_layer(*device_inputs(inp), cfg)
    ora = oracle_layer(inp, ckw)
    assert not ora[(0, 1)]["is_vs"]
    got = rows_of(g, 1, sh.n_blocks)
    for qb in range(sh.n_blocks):
        assert got[qb].tolist() == ora[(0, 1)]["rows"][qb].tolist(), qb
    assert got[30].tolist() == list(range(13)) + [30]
    check_outputs(g["out"], inp, {(0, 1): got}, {(0, 1): range(sh.n_blocks)})


def test_deterministic_and_bf16_output():
    sh = SHAPES["ragged_nb9_b2_g2"]
    inp = _inputs(sh, seed=71)
    q, k, v = device_inputs(inp)
    cfg = crisp.config()
    a = gpu_layer(q, k, v, cfg)
    b = gpu_layer(q, k, v, cfg)
    for key in ("c", "pattern", "p_vert", "p_slash", "row_ptr", "col", "mask"):
        assert np.array_equal(a[key], b[key]), key
    assert torch.equal(a["out"], b["out"])
    o16 = crisp.sparse_attn(q, k, v, a["sel"], cfg, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ref = a["out"].to(torch.bfloat16)
    assert torch.equal(o16, ref)
    d1 = crisp.dense_attn(q, k, v)
    d2 = crisp.dense_attn(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(d1, d2)


def test_empty_batch_is_a_no_op():
    q = torch.empty((0, 2, 4096, 64), dtype=torch.bfloat16, device="cuda")
    k = torch.empty((0, 2, 4096, 64), dtype=torch.bfloat16, device="cuda")
    r = crisp.route(q, k)
    s = crisp.select(q, k, r)
    o = crisp.sparse_attn(q, k, k, s)
    d = crisp.dense_attn(q, k, k)
    torch.cuda.synchronize()
    assert r["pattern"].numel() == 0 and o.numel() == 0 and d.numel() == 0 and s["row_ptr"].numel() == 1


_HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "crisp.h")
_GATE = int(re.search(r"#define\s+CRISP_DENSE_BELOW_TOKENS\s+(\d+)", open(_HEADER).read()).group(1))


@pytest.mark.parametrize("n", [4096, _GATE - 128, _GATE])
def test_prefill_length_gate(n):
    """prefill() runs dense attention below the library's crossover length and
    the sparse path from it on; either way the output is exactly what the
    chosen path's own calls give (those are checked against the oracle above)."""
    sh = Shape(1, n, 4, 2, 64)
    q, k, v = device_inputs(_inputs(sh, seed=61))
    cfg = crisp.config()
    res = crisp.prefill(q, k, v, cfg)
    want_dense = n < _GATE
    assert crisp.use_dense(crisp.shape_of(q, k)) is want_dense
    assert res["path"] == ("dense" if want_dense else "sparse")
    if want_dense:
        ref = crisp.dense_attn(q, k, v)
    else:
        r = crisp.route(q, k, cfg)
        ref = crisp.sparse_attn(q, k, v, crisp.select(q, k, r, cfg), cfg)
    torch.cuda.synchronize()
    assert torch.equal(res["out"], ref)
    ungated = crisp.prefill(q, k, v, cfg, gate=False)
    assert ungated["path"] == "sparse" and ungated["route"] is not None
