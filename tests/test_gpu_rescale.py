"""GPU parity on inputs whose row maxima keep growing along the keys.

The attention kernels keep a reference maximum per query row.  At d = 128 a
wave whose rows' Cauchy-Schwarz logit bound (c2 |q| max|k|) lies at most 64
log2 units above the first stage's maximum keeps that maximum for the whole
row; otherwise it tracks the maximum and raises it (rescaling the row's output
and row sum) when a stage's maximum exceeds it by more than 2^8.  At d = 64
every row tracks.  On the workload recipe every wave keeps its first maximum.
Here the keys are scaled up block by block, with an extra jump four blocks
before the end, so rows raise their reference several times, by small and by
large steps, at both head dims, through dense_attn and sparse_attn; a third
shape mixes one KV head of such keys with one of plain keys, so that one launch
runs waves of both kinds.
"""
import numpy as np
import pytest
import torch

import long_context_sparse_patsearch_amd as crisp
from oracle import crisp_oracle as co
from parity import check_outputs, device_inputs
from prefill_inputs import Shape, make_inputs
from prefill_inputs.gen import bf16_bits_to_f32, f32_to_bf16_bits

pytestmark = pytest.mark.gpu

SHAPES = {
    "d128_gqa2": Shape(1, 2048, 2, 1, 128),
    "d64_mha": Shape(1, 2048, 2, 2, 64),
    "d128_mixed": Shape(1, 2048, 4, 2, 128),
}
STAGE = 64
RAISE_LOG2 = 8.0
FIXED_SPAN = 64.0


def _growing_inputs(sh, seed):
    """Keys scaled up block by block; in the mixed shape only KV head 1's."""
    inp = make_inputs(sh, vs_fraction=0.5, sink_scale=3.0, n_vert=4, seed=seed)
    nb = sh.n_blocks
    kb = np.arange(sh.n) // 128
    g = 1.0 + 0.4 * kb
    g[kb == nb - 4] *= 3.0
    gk = np.ones((sh.h_kv, sh.n), dtype=np.float32)
    gk[1 if sh is SHAPES["d128_mixed"] else 0:] = g
    k = bf16_bits_to_f32(inp["k"]) * gk[None, :, :, None]
    inp["k"] = f32_to_bf16_bits(k)
    return inp


def _tracking_waves(inp, sh, rows_by_head):
    """(waves that track their maxima, waves that keep the first one) at d = 128,
    from the rule the kernel applies (64 query rows per wave)."""
    c2 = np.log2(np.e) / np.sqrt(sh.d)
    G = sh.h_q // sh.h_kv
    track = keep = 0
    for (b, h), rows in rows_by_head.items():
        q = bf16_bits_to_f32(inp["q"][b, h]).astype(np.float64)
        k = bf16_bits_to_f32(inp["k"][b, h // G]).astype(np.float64)
        kn = np.sqrt((k * k).sum(axis=1).max())
        for qb, cols in enumerate(rows):
            c = int(sorted(cols)[0])
            for w in range(2):
                rr = qb * 128 + 64 * w + np.arange(64)
                s = (q[rr] @ k[c * 128:c * 128 + STAGE].T) * c2
                if c == qb:
                    s = np.where(c * 128 + np.arange(STAGE)[None, :] > rr[:, None], -np.inf, s)
                bound = c2 * np.sqrt((q[rr] * q[rr]).sum(axis=1)) * kn
                if np.any(bound - s.max(axis=1) > FIXED_SPAN):
                    track += 1
                else:
                    keep += 1
    return track, keep


def _raises(inp, sh, rows_by_head):
    """Stages (64 keys, in row order) in which some 32-row tile raises its
    reference maximum after its first stage, counted over all heads."""
    c2 = np.log2(np.e) / np.sqrt(sh.d)
    G = sh.h_q // sh.h_kv
    total = 0
    for (b, h), rows in rows_by_head.items():
        q = bf16_bits_to_f32(inp["q"][b, h]).astype(np.float64)
        k = bf16_bits_to_f32(inp["k"][b, h // G]).astype(np.float64)
        for qb, cols in enumerate(rows):
            qq = q[qb * 128:(qb + 1) * 128]
            m = np.full(128, -np.inf)
            first = True
            for c in sorted(int(x) for x in cols):
                for half in range(2):
                    j0 = c * 128 + half * STAGE
                    s = (qq @ k[j0:j0 + STAGE].T) * c2
                    if c == qb:
                        s = np.where(j0 + np.arange(STAGE)[None, :] > qb * 128 + np.arange(128)[:, None], -np.inf, s)
                    t = s.max(axis=1)
                    up = t > m + RAISE_LOG2
                    if not first and up.reshape(4, 32).any(axis=1).any():
                        total += 1
                    m = np.where(up, t, m)
                    first = False
    return total


@pytest.mark.parametrize("name", list(SHAPES))
def test_dense_with_growing_maxima(name):
    sh = SHAPES[name]
    inp = _growing_inputs(sh, seed=81)
    rows = {(0, h): co.dense_rows(sh.n_blocks) for h in range(sh.h_q)}
    assert _raises(inp, sh, rows) > 4 * sh.h_q
    if sh.d == 128:
        track, keep = _tracking_waves(inp, sh, rows)
        assert track > 0 and keep > 0, (track, keep)
    q, k, v = device_inputs(inp)
    out = crisp.dense_attn(q, k, v)
    torch.cuda.synchronize()
    worst, mean = check_outputs(out, inp, rows, {bh: range(sh.n_blocks) for bh in rows})
    print(f"[{name} dense, growing maxima] max-abs {worst:.2e} mean-abs {mean:.2e}", flush=True)


@pytest.mark.parametrize("name", list(SHAPES))
def test_sparse_with_growing_maxima(name):
    sh = SHAPES[name]
    nb = sh.n_blocks
    inp = _growing_inputs(sh, seed=91)
    rng = np.random.default_rng(17)
    rows_all, rows = [], {}
    for h in range(sh.h_q):
        per = []
        for qb in range(nb):
            pick = rng.choice(qb + 1, size=rng.integers(1, qb + 2), replace=False).tolist()
            per.append(sorted(set(pick) | {0, qb}))
        rows_all.extend(per)
        rows[(0, h)] = [np.array(r, dtype=np.int64) for r in per]
    assert _raises(inp, sh, rows) > 2 * sh.h_q
    if sh.d == 128:
        track, keep = _tracking_waves(inp, sh, rows)
        assert track > 0 and keep > 0, (track, keep)
    row_ptr = np.concatenate([[0], np.cumsum([len(r) for r in rows_all])]).astype(np.int64)
    col = np.array([c for r in rows_all for c in r], dtype=np.int32)
    sel = dict(row_ptr=torch.from_numpy(row_ptr).cuda(), col_idx=torch.from_numpy(col).cuda())
    q, k, v = device_inputs(inp)
    out = crisp.sparse_attn(q, k, v, sel, crisp.config())
    torch.cuda.synchronize()
    worst, mean = check_outputs(out, inp, rows, {bh: range(nb) for bh in rows})
    print(f"[{name} sparse, growing maxima] max-abs {worst:.2e} mean-abs {mean:.2e}", flush=True)
