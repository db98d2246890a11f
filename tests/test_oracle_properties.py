"""Property tests of the fp64 oracle on random tiny layers (CPU, hypothesis).

Each property is a fact of the mathematics that any correct implementation
satisfies whatever the inputs, checked on random shapes (3 to 6 blocks of 128
tokens, d in {64, 128}), random logit sharpness and random settings:

* proxy rows are causal probability distributions;
* the vertical and slash block scores each sum to 1, and the structural mass
  equals the vertical score of the two anchor blocks;
* every selected row is sorted, causal and holds its diagonal block; a VS row
  holds the sink block;
* the noise-floor selection keeps every block above the floor and the anchors,
  at least k_min blocks, and a top-k set otherwise;
* the gamma-cumsum keeps a descending prefix whose mass reaches gamma and
  whose last element is needed;
* attention over every causal block equals dense attention; adding a vector to
  every value row adds it to every output; scaling the values scales the
  outputs; values and keys after a query block do not change its outputs.
"""
import numpy as np
import pytest

hyp = pytest.importorskip("hypothesis")
from hypothesis import given, settings, strategies as st  # noqa: E402

from oracle import crisp_oracle as co  # noqa: E402

B = co.BLOCK
SET = settings(max_examples=20, deadline=None, derandomize=True)


def layer(seed, nb, d, sharp):
    rng = np.random.default_rng(seed)
    n = nb * B
    q = rng.standard_normal((n, d)) * sharp
    k = rng.standard_normal((n, d))
    v = rng.standard_normal((n, d))
    return q, k, v


shapes = st.tuples(st.integers(0, 2 ** 31 - 1), st.integers(3, 6), st.sampled_from([64, 128]),
                   st.sampled_from([0.05, 0.5, 1.0, 2.0]))


@SET
@given(shapes)
def test_proxy_rows_are_causal_distributions(shape):
    q, k, _ = layer(*shape)
    a = co.proxy_attention(q, k)
    n = k.shape[0]
    assert a.shape == (B, n)
    assert np.all(a >= 0)
    assert np.allclose(a.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    pos = n - B + np.arange(B)
    assert np.all(a[np.arange(n)[None, :] > pos[:, None]] == 0)


@SET
@given(shapes)
def test_block_scores_sum_to_one_and_anchor_mass(shape):
    q, k, _ = layer(*shape)
    a = co.proxy_attention(q, k)
    p_v, p_s = co.vs_scores(a)
    assert np.all(p_v >= 0) and np.all(p_s >= 0)
    assert abs(p_v.sum() - 1) < 1e-12 and abs(p_s.sum() - 1) < 1e-12
    c = co.structural_mass(a)
    assert abs(c - (p_v[0] + p_v[-1])) < 1e-12


@SET
@given(shapes, st.sampled_from([0.0, 0.2, 0.5, 1.1]), st.sampled_from([0.5, 1.0, 1.5]),
       st.sampled_from([0.5, 0.95]), st.sampled_from([128, 256, 1024]))
def test_head_rows_are_causal_with_diagonal(shape, tau, alpha, gamma, kmin):
    q, k, _ = layer(*shape)
    nb = shape[1]
    r = co.crisp_head(q, k, tau=tau, alpha=alpha, gamma=gamma, k_min_tokens=kmin)
    assert len(r["rows"]) == nb
    for qb, row in enumerate(r["rows"]):
        assert np.all(np.diff(row) > 0) and row[0] >= 0 and row[-1] == qb
        if r["is_vs"]:
            assert row[0] == 0
    assert r["is_vs"] == (r["c_struct"] >= tau)


@SET
@given(st.integers(0, 2 ** 31 - 1), st.integers(3, 40), st.sampled_from([0.0, 0.5, 1.0, 2.0]),
       st.integers(0, 50), st.booleans())
def test_noise_floor_selection(seed, nb, alpha, kmin, ties):
    rng = np.random.default_rng(seed)
    p = rng.dirichlet(np.ones(nb) * 0.5)
    if ties:
        p = np.round(p * 8) / 8 + 1e-3
        p /= p.sum()
    sel, mu, above = co.noise_floor_select(p, alpha, kmin)
    s = set(sel.tolist())
    assert {0, nb - 1} <= s
    assert {j for j in range(nb) if p[j] > alpha * mu} <= s
    need = min(max(above, kmin), nb)
    assert len(s) >= need
    # without the anchors it adds, the kept set is a top set: nothing left out scores above a kept block
    core = sorted(s - ({0, nb - 1} - set(np.lexsort((np.arange(nb), -p))[:need].tolist())))
    out = [j for j in range(nb) if j not in s]
    if out and core:
        assert max(p[out]) <= min(p[core])


@SET
@given(st.integers(0, 2 ** 31 - 1), st.integers(1, 60), st.floats(0.05, 1.0))
def test_gamma_cumsum_minimal_prefix(seed, m, gamma):
    rng = np.random.default_rng(seed)
    x = rng.dirichlet(np.ones(m)) * rng.uniform(0.5, 1.2)
    kept, order, cs = co.gamma_cumsum(x, gamma)
    assert np.array_equal(kept, order[: len(kept)])
    assert np.all(np.diff(x[order]) <= 0)
    if x.sum() >= gamma:
        assert x[kept].sum() >= gamma * (1 - 1e-12)
        assert x[kept[:-1]].sum() < gamma
    else:
        assert len(kept) == m


@SET
@given(shapes, st.sampled_from([0.3, 0.8, 0.95]))
def test_pe_selection_reaches_gamma(shape, gamma):
    q, k, _ = layer(*shape)
    nb = shape[1]
    a_bar = co.pooled_map(q, k)
    assert np.allclose(a_bar.sum(axis=1), 1.0, atol=1e-12) and np.all(np.triu(a_bar, 1) == 0)
    pe = co.pe_select(a_bar, gamma)
    mass = sum(a_bar[qb, row].sum() for qb, row in enumerate(pe["rows"])) / nb
    assert mass >= gamma * (1 - 1e-12)
    for qb, row in enumerate(pe["rows"]):
        assert row[-1] == qb and np.all(np.diff(row) > 0)


@SET
@given(shapes)
def test_attention_invariants(shape):
    q, k, v = layer(*shape)
    nb, d = shape[1], shape[2]
    rng = np.random.default_rng(shape[0] ^ 0x5EED)
    full = co.block_sparse_attention(q, k, v, co.dense_rows(nb))
    dense = co.dense_attention(q, k, v)
    for qb in range(nb):
        assert np.allclose(full[qb], dense[qb], rtol=0, atol=1e-12)
    # a random selection containing every diagonal
    rows = [np.union1d(np.nonzero(rng.random(qb + 1) < 0.5)[0], [qb]).astype(np.int64) for qb in range(nb)]
    base = co.block_sparse_attention(q, k, v, rows)
    c = rng.standard_normal(d)
    shifted = co.block_sparse_attention(q, k, v + c, rows)
    scaled = co.block_sparse_attention(q, k, 3.0 * v, rows)
    for qb in range(nb):
        assert np.allclose(shifted[qb], base[qb] + c, rtol=0, atol=1e-10)
        assert np.allclose(scaled[qb], 3.0 * base[qb], rtol=0, atol=1e-10)
    # causality: keys and values after query block 1 do not reach it
    k2, v2 = k.copy(), v.copy()
    k2[2 * B:] = rng.standard_normal(k2[2 * B:].shape)
    v2[2 * B:] = rng.standard_normal(v2[2 * B:].shape)
    late = co.block_sparse_attention(q, k2, v2, rows, q_blocks=[0, 1])
    for qb in (0, 1):
        assert np.array_equal(late[qb], base[qb])
