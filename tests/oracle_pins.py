"""Pin checks for the fp64 oracle.

Each ``check_*`` takes the oracle module (or a stand-in with the same
functions) and raises AssertionError when the oracle disagrees with something
fixed independently of it: a closed form from the pages, an invariant, a
textbook/library routine, brute force on a tiny input, or a worked example of
the pages.  ``test_oracle_pins.py`` runs them on the real oracle and
``test_oracle_mutants.py`` runs them on deliberately broken copies to show each
plausible mistake is caught.
"""
import json
import math
import os

import numpy as np

B = 128
HERE = os.path.dirname(os.path.abspath(__file__))


def _rand(rng, n, d, scale=1.0):
    return rng.standard_normal((n, d)) * scale


# --- proxy softmax ------------------------------------------------------------
def check_proxy_rows_sum_and_causal(co, seed=0):
    rng = np.random.default_rng(seed)
    n, d = 640, 64
    q, k = _rand(rng, n, d), _rand(rng, n, d)
    a = co.proxy_attention(q, k, B)
    assert a.shape == (B, n)
    assert np.allclose(a.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    for i in range(B):
        assert np.all(a[i, n - B + i + 1:] == 0.0), "proxy row sees future keys"
        assert np.all(a[i, : n - B + i + 1] > 0.0)
    # one row against the softmax written out with scipy
    from scipy.special import softmax
    i = 37
    s = q[n - B + i] @ k[: n - B + i + 1].T / math.sqrt(d)
    assert np.allclose(a[i, : n - B + i + 1], softmax(s), rtol=1e-12, atol=0)


def check_background_mass_closed_form(co):
    """k keys at logit Delta over background 0: every background key holds
    eps = e^-Delta / (k + (n-k) e^-Delta) (digest, "Core method", the mass-cliff
    derivation); n = the keys a proxy row can see."""
    n, d = 1024, 64
    delta = 4.0
    c = math.sqrt(delta * math.sqrt(d))
    sig = [10, 100, 300, 500, 700]
    q = np.zeros((n, d))
    q[:, 0] = c
    k = np.zeros((n, d))
    k[:, 1] = 1.0
    k[sig, 1] = 0.0
    k[sig, 0] = c
    a = co.proxy_attention(q, k, B)
    ks = len(sig)
    for i in range(B):
        nv = n - B + i + 1
        eps = math.exp(-delta) / (ks + (nv - ks) * math.exp(-delta))
        bg = np.setdiff1d(np.arange(nv), sig)
        assert np.allclose(a[i, bg], eps, rtol=1e-12, atol=0)
        assert np.allclose(a[i, sig], 1.0 / (ks + (nv - ks) * math.exp(-delta)), rtol=1e-12)


# --- block scores and structural mass ------------------------------------------
def check_block_scores_brute_force(co, seed=1):
    rng = np.random.default_rng(seed)
    n, d = 640, 32
    q, k = _rand(rng, n, d, 1.5), _rand(rng, n, d)
    a = co.proxy_attention(q, k, B)
    pv, ps = co.vs_scores(a, B)
    nb = n // B
    assert np.isclose(pv.sum(), 1.0, atol=1e-12) and np.isclose(ps.sum(), 1.0, atol=1e-12)
    # brute force over every proxy entry: column index j, diagonal index t = j + b-1-i
    bv = np.zeros(nb)
    bs = np.zeros(nb)
    for i in range(B):
        for j in range(n - B + i + 1):
            bv[j // B] += a[i, j] / B
            bs[(j + B - 1 - i) // B] += a[i, j] / B
    assert np.allclose(pv, bv, rtol=1e-12, atol=1e-15)
    assert np.allclose(ps, bs, rtol=1e-12, atol=1e-15)


def check_block_scores_tile_identity(co, seed=2):
    """With b = B the slash block of entry (i, j in key block kb) is kb when the
    in-tile column jj <= i and kb+1 otherwise, so
    p_v[kb] = (L_kb + U_kb)/b and p_s[kb] = (L_kb + U_{kb-1})/b
    with L (U) the lower-with-diagonal (strict upper) sum of the proxy tile."""
    rng = np.random.default_rng(seed)
    n, d = 1024, 64
    q, k = _rand(rng, n, d, 1.2), _rand(rng, n, d)
    a = co.proxy_attention(q, k, B)
    pv, ps = co.vs_scores(a, B)
    nb = n // B
    low = np.tril(np.ones((B, B), dtype=bool))
    L = np.array([a[:, kb * B:(kb + 1) * B][low].sum() for kb in range(nb)])
    U = np.array([a[:, kb * B:(kb + 1) * B][~low].sum() for kb in range(nb)])
    assert U[-1] == 0.0
    assert np.allclose(pv, (L + U) / B, rtol=1e-12, atol=1e-16)
    assert np.allclose(ps, (L + np.concatenate([[0.0], U[:-1]])) / B, rtol=1e-12, atol=1e-16)


def check_scores_orientation(co, seed=10):
    """Semantic pins of reading R5 (which way the slash index runs).

    A head looking only at key 0 puts its vertical and slash mass in block 0
    (the sink side); a head looking only at its own position puts both in block
    N_b-1 (the local side); a head looking at the key 200 positions back puts
    its slash mass in block (n-1-200) // B."""
    rng = np.random.default_rng(seed)
    n, d = 1024, 64
    nb = n // B
    big = 40.0
    q = np.zeros((n, d))
    q[:, 0] = big
    k = np.zeros((n, d))
    k[0, 0] = big
    pv, ps = co.vs_scores(co.proxy_attention(q, k, B), B)
    assert pv[0] > 0.999 and ps[0] > 0.999
    k = rng.standard_normal((n, d))
    pv, ps = co.vs_scores(co.proxy_attention(3.0 * k, k, B), B)
    assert pv[nb - 1] > 0.99 and ps[nb - 1] > 0.99
    q = np.zeros((n, d))
    q[200:] = 3.0 * k[:-200]
    pv, ps = co.vs_scores(co.proxy_attention(q, k, B), B)
    assert ps[(n - 1 - 200) // B] > 0.99


def check_structural_mass_brute_force(co, seed=3):
    rng = np.random.default_rng(seed)
    n, d = 768, 64
    q, k = _rand(rng, n, d, 1.3), _rand(rng, n, d)
    a = co.proxy_attention(q, k, B)
    c = co.structural_mass(a, 128, 128)
    tot = 0.0
    for i in range(B):
        for j in list(range(128)) + list(range(n - 128, n)):
            tot += a[i, j]
    assert math.isclose(c, tot / B, rel_tol=1e-12)
    pv, _ = co.vs_scores(a, B)
    assert math.isclose(c, pv[0] + pv[-1], rel_tol=1e-12)
    assert co.route(0.2, 0.2) is True and co.route(0.2 - 1e-12, 0.2) is False


# --- noise floor ----------------------------------------------------------------
def _floor_expected(p, alpha, kmin):
    nb = len(p)
    mu = max(1.0 - p[0] - p[nb - 1], 0.0) / (nb - 2)
    cand = [j for j in range(nb) if p[j] > alpha * mu]
    if len(cand) >= kmin:
        keep = set(cand)
    else:
        ranked = sorted(range(nb), key=lambda j: (-p[j], j))
        keep = set(ranked[: min(kmin, nb)])
    return keep | {0, nb - 1}, mu, len(cand)


def check_noise_floor(co, seed=4):
    rng = np.random.default_rng(seed)
    for nb in (3, 7, 32, 200):
        for conc in (0.05, 0.3, 3.0):
            p = rng.dirichlet(np.full(nb, conc))
            for alpha in (0.0, 0.5, 1.0, 1.25, 4.0):
                sel, mu, above = co.noise_floor_select(p, alpha, 8)
                keep, mu_cf, cnt = _floor_expected(p, alpha, 8)
                assert math.isclose(mu, mu_cf, rel_tol=1e-14, abs_tol=0), (nb, alpha)
                assert above == cnt
                assert set(sel.tolist()) == keep, (nb, conc, alpha)
    # ties go to the lower block index in the padding
    p = np.array([0.5, 0.1, 0.1, 0.1, 0.1, 0.0, 0.0, 0.0, 0.0, 0.0, 0.1])
    sel, _, above = co.noise_floor_select(p, 10.0, 4)
    assert above == 1 and set(sel.tolist()) == {0, 1, 2, 3, 10}
    # rounding can push p[0] + p[-1] past 1; the max(., 0) guard makes mu = 0
    p = np.zeros(10)
    p[0], p[-1], p[4] = 0.6, 0.4 + 1e-12, 1e-13
    sel, mu, above = co.noise_floor_select(p, 1.0, 1)
    assert mu == 0.0 and above == 3 and set(sel.tolist()) == {0, 4, 9}


def check_vs_rows(co):
    nb = 10
    rows = co.vs_rows(np.array([0, 3, 9]), np.array([9, 7, 0]), nb)
    # slash block 9 -> diagonal 0, 7 -> diagonal 2, 0 -> diagonal 9
    assert rows[0].tolist() == [0]
    assert rows[2].tolist() == [0, 2]
    assert rows[5].tolist() == [0, 3, 5]
    assert rows[9].tolist() == [0, 3, 7, 9]


def check_block_mass_fixtures(co):
    with open(os.path.join(HERE, "golden", "block_mass_examples.json")) as fh:
        fixtures = json.load(fh)
    for f in fixtures:
        p = np.array(f["p"])
        sel, mu, above = co.noise_floor_select(p, f["alpha"], f["k_min_blocks"])
        assert sel.tolist() == f["expect_floor_set"], f["name"]
        kept, order, cs = co.gamma_cumsum(p, f["gamma"])
        assert len(kept) == f["expect_gamma_kept"], f["name"]
        sig = set(f["signal_blocks"])
        noise = [j for j in kept if j not in sig and j not in (0, len(p) - 1)]
        assert len(noise) == f["expect_gamma_noise_blocks"], f["name"]
        missed = len(sig - set(kept.tolist()))
        assert missed == f["expect_gamma_missed_signal"], f["name"]


# --- gamma-cumsum and the pooled map ---------------------------------------------
def check_gamma_garbage_closed_form(co):
    """One sink block of mass m plus N background blocks of mass eps: the
    cumulative rule keeps the sink and ceil((gamma - m)/eps) background blocks
    (N_garbage = gamma_residual / eps, digest "Core method")."""
    for m, N in ((0.5, 999), (0.8, 4095), (0.9, 333)):
        eps = (1.0 - m) / N
        x = np.concatenate([[m], np.full(N, eps)])
        kept, _, _ = co.gamma_cumsum(x, 0.95)
        assert len(kept) == 1 + math.ceil((0.95 - m) / eps)
        assert kept[0] == 0 and np.all(np.diff(kept[1:]) == 1)
    # the prefix may meet gamma exactly: ">=" stops there
    kept, _, _ = co.gamma_cumsum(np.array([0.25, 0.5, 0.25]), 0.75)
    assert kept.tolist() == [1, 0]


def check_pe_uniform_closed_form(co):
    """Zero queries make every pooled logit 0, so row r of A_bar is uniform
    1/(r+1) and x = 1/(N_b (r+1)).  Descending order visits whole rows top-down
    (ties toward the lower flat index), so gamma-cumsum keeps rows
    0..R-1 (R = floor(gamma N_b)) and ceil((gamma N_b - R)(R+1)) leading cells of
    row R; the diagonal is then forced in every row."""
    rng = np.random.default_rng(5)
    for nb in (24, 32):
        n, d = nb * B, 64
        q = np.zeros((n, d))
        k = _rand(rng, n, d)
        a_bar = co.pooled_map(q, k, B)
        for r in range(nb):
            assert np.allclose(a_bar[r, : r + 1], 1.0 / (r + 1), rtol=1e-13)
            assert np.all(a_bar[r, r + 1:] == 0.0)
        pe = co.pe_select(a_bar, 0.95)
        R = int(math.floor(0.95 * nb))
        m = int(math.ceil((0.95 * nb - R) * (R + 1)))
        for r in range(nb):
            got = pe["rows"][r].tolist()
            if r < R:
                assert got == list(range(r + 1))
            elif r == R:
                assert got == sorted(set(range(m)) | {r})
            else:
                assert got == [r]
    # nb = 32 is the example worked out for the tiny workload: 13 cells of row 30
    assert int(math.ceil((0.95 * 32 - 30) * 31)) == 13


def check_pooled_map_means(co, seed=6):
    rng = np.random.default_rng(seed)
    nb, d = 6, 16
    n = nb * B
    q, k = _rand(rng, n, d), _rand(rng, n, d)
    a_bar = co.pooled_map(q, k, B)
    for r in range(nb):
        qm = q[r * B:(r + 1) * B].mean(axis=0)
        logits = [qm @ k[c * B:(c + 1) * B].mean(axis=0) / math.sqrt(d) for c in range(r + 1)]
        w = np.exp(np.array(logits) - max(logits))
        assert np.allclose(a_bar[r, : r + 1], w / w.sum(), rtol=1e-12)


# --- exact attention ---------------------------------------------------------------
def check_dense_brute_force(co, seed=7):
    rng = np.random.default_rng(seed)
    n, d = 384, 32
    q, k, v = _rand(rng, n, d, 2.0), _rand(rng, n, d), _rand(rng, n, d)
    out = co.dense_attention(q, k, v)
    for p in range(0, n, 7):
        s = np.array([q[p] @ k[j] for j in range(p + 1)]) / math.sqrt(d)
        w = np.exp(s - s.max())
        ref = (w[:, None] * v[: p + 1]).sum(axis=0) / w.sum()
        assert np.allclose(out[p // B][p % B], ref, rtol=1e-11, atol=1e-12), p


def check_masked_attention_vs_sdpa(co, seed=8):
    """Block-sparse masked attention equals torch's scaled_dot_product_attention
    (float64, CPU) given the explicit token mask causal AND selected-block."""
    import torch
    rng = np.random.default_rng(seed)
    n, d = 768, 64
    nb = n // B
    q, k, v = _rand(rng, n, d, 1.5), _rand(rng, n, d), _rand(rng, n, d)
    rows = []
    for qb in range(nb):
        pick = sorted(set(rng.choice(qb + 1, size=rng.integers(1, qb + 2), replace=False).tolist()) | {qb})
        rows.append(np.array(pick))
    mask = np.zeros((n, n), dtype=bool)
    for qb in range(nb):
        for kb in rows[qb]:
            mask[qb * B:(qb + 1) * B, kb * B:(kb + 1) * B] = True
    mask &= np.tril(np.ones((n, n), dtype=bool))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None],
        attn_mask=torch.from_numpy(mask)[None]).numpy()[0]
    out = co.block_sparse_attention(q, k, v, rows)
    got = np.concatenate([out[qb] for qb in range(nb)])
    assert np.allclose(got, ref, rtol=1e-10, atol=1e-12)
    # one block, causal: the textbook case
    q1, k1, v1 = q[:B], k[:B], v[:B]
    ref1 = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q1)[None], torch.from_numpy(k1)[None], torch.from_numpy(v1)[None],
        is_causal=True).numpy()[0]
    got1 = co.block_sparse_attention(q1, k1, v1, [np.array([0])])[0]
    assert np.allclose(got1, ref1, rtol=1e-10, atol=1e-12)


def check_alpha_zero_is_dense(co, seed=9):
    """alpha = 0 keeps every block whose score is positive, i.e. all of them, so
    the VS path reproduces dense causal attention."""
    rng = np.random.default_rng(seed)
    n, d = 768, 32
    nb = n // B
    q, k, v = _rand(rng, n, d), _rand(rng, n, d), _rand(rng, n, d)
    res = co.crisp_head(q, k, alpha=0.0, force_vs=True)
    assert res["sel_v"].tolist() == list(range(nb)) and res["sel_s"].tolist() == list(range(nb))
    for qb in range(nb):
        assert res["rows"][qb].tolist() == list(range(qb + 1))
    o_s = co.block_sparse_attention(q, k, v, res["rows"])
    o_d = co.dense_attention(q, k, v)
    for qb in range(nb):
        assert np.array_equal(o_s[qb], o_d[qb])


# --- the FlexPrefill baseline path --------------------------------------------
def check_jsd_against_library(co, seed=20):
    """D_JS against scipy's Jensen-Shannon distance (natural log; scipy returns
    the square root), plus its fixed values: 0 for equal arguments, ln 2 for
    disjoint supports, symmetry."""
    from scipy.spatial.distance import jensenshannon
    rng = np.random.default_rng(seed)
    for n in (2, 7, 64):
        p, q = rng.random(n), rng.random(n)
        p[rng.random(n) < 0.3] = 0.0
        p, q = p / p.sum(), q / q.sum()
        want = float(jensenshannon(p, q)) ** 2
        assert math.isclose(co.jensen_shannon(p, q), want, rel_tol=1e-10, abs_tol=1e-14)
        assert math.isclose(co.jensen_shannon(p, q), co.jensen_shannon(q, p), rel_tol=1e-12)
        assert abs(co.jensen_shannon(p, p)) < 1e-15
    assert math.isclose(co.jensen_shannon(np.array([1.0, 0, 0]), np.array([0, 0.5, 0.5])), math.log(2), rel_tol=1e-12)


def check_pooled_estimate_brute_force(co, seed=21):
    """a_bar: mean of the last b queries against each block's mean key, scaled
    softmax over every block, written out with loops."""
    rng = np.random.default_rng(seed)
    nb, d = 5, 16
    n = nb * B
    q, k = _rand(rng, n, d), _rand(rng, n, d)
    got = co.pooled_proxy_estimate(q, k, B, B)
    qm = [sum(q[n - B + i, c] for i in range(B)) / B for c in range(d)]
    logits = []
    for blk in range(nb):
        km = [sum(k[blk * B + j, c] for j in range(B)) / B for c in range(d)]
        logits.append(sum(qm[c] * km[c] for c in range(d)) / math.sqrt(d))
    w = np.exp(np.array(logits) - max(logits))
    assert np.allclose(got, w / w.sum(), rtol=1e-12)


def check_gamma_direction_brute_force(co, seed=22):
    """The gamma-cumsum set of one direction is a smallest subset reaching gamma
    (brute force over every subset of 8 blocks), ties go to the lower index,
    the count is clipped to [k_min, N_b] and the anchors are added."""
    import itertools
    rng = np.random.default_rng(seed)
    nb = 8
    for trial in range(20):
        p = rng.random(nb) ** 3
        if trial % 4 == 0:
            p[2] = p[5]                      # a tie
        p /= p.sum()
        for gamma in (0.3, 0.7, 0.95, 1.0 - 1e-12):
            best = min(len(c) for r in range(1, nb + 1) for c in itertools.combinations(range(nb), r)
                       if sum(p[list(c)]) >= gamma)
            sel, cnt = co.gamma_direction_select(p, gamma, 0)
            assert cnt == best
            core = sorted(np.lexsort((np.arange(nb), -p))[:best].tolist())
            assert sorted(set(core) | {0, nb - 1}) == sel.tolist()
            for kmin in (3, 6, 20):
                sel_k, _ = co.gamma_direction_select(p, gamma, kmin)
                k = min(max(best, kmin), nb)
                top = np.lexsort((np.arange(nb), -p))[:k].tolist()
                assert sel_k.tolist() == sorted(set(top) | {0, nb - 1})
    # tie toward the lower index: two equal largest scores, gamma reached by one of them
    p = np.array([0.1, 0.4, 0.1, 0.4, 0.0, 0.0, 0.0, 0.0])
    sel, cnt = co.gamma_direction_select(p, 0.35, 0)
    assert cnt == 1 and sel.tolist() == [0, 1, 7]


def check_flex_routes_planted(co):
    """The JSD router sends the planted VS head of the 4k workload to VS and the
    diffuse head to PE (the pages: JSD reproduces C_struct's decisions on such
    heads), and its VS sets keep the sink block and the planted vertical blocks."""
    from prefill_inputs import WORKLOADS, workload_inputs
    inp = workload_inputs(WORKLOADS[1])
    q0, k0 = co.bf16_to_f64(inp["q"][0, 0]), co.bf16_to_f64(inp["k"][0, 0])
    q1, k1 = co.bf16_to_f64(inp["q"][0, 1]), co.bf16_to_f64(inp["k"][0, 1])
    r0 = co.flex_head(q0, k0, tau_jsd=0.1)
    r1 = co.flex_head(q1, k1, tau_jsd=0.1)
    assert r0["is_vs"] and r0["jsd"] > 0.2
    assert not r1["is_vs"] and r1["jsd"] < 0.02
    planted = set((np.asarray(inp["planted"][0][0]["vert"]) // B).tolist())
    assert len(planted) > 0
    assert 0 in r0["sel_v"].tolist() and planted <= set(r0["sel_v"].tolist())


# --- variants -----------------------------------------------------------------------
def check_median_floor(co, seed=30):
    """The median floor is the median of the non-anchor scores (statistics.median),
    equals the mean floor when those scores are all equal, and then keeps what
    the mean floor keeps."""
    import statistics
    rng = np.random.default_rng(seed)
    for nb in (7, 8, 33):
        p = rng.random(nb) ** 2
        p /= p.sum()
        _, mu, cnt = co.noise_floor_select(p, 1.0, 0, floor="median")
        med = statistics.median(p[1:nb - 1].tolist())
        assert math.isclose(mu, med, rel_tol=1e-12)
        assert cnt == sum(1 for x in p if x > med)
    nb = 10
    p = np.full(nb, 0.05)
    p[0], p[nb - 1] = 0.4 - 0.05, 0.6 - 0.4 + 0.05   # anchors hold the rest; non-anchors equal
    p /= p.sum()
    a = co.noise_floor_select(p, 0.9, 2, floor="median")
    b = co.noise_floor_select(p, 0.9, 2, floor="mean")
    assert math.isclose(a[1], b[1], rel_tol=1e-12) and a[0].tolist() == b[0].tolist()


def check_slash_band_tokens(co):
    """With the band, tile (qb, kb) of a VS row is selected by the slash part
    exactly when some causal token pair of the tile has its offset inside a
    selected slash block's 128-token range (brute force over tokens)."""
    nb = 6
    n = nb * B
    sel_s = np.array([nb - 1, nb - 3])            # deltas 0 and 2
    rows = co.vs_rows(np.array([], dtype=np.int64), sel_s, nb, band=True)
    deltas = nb - 1 - sel_s
    q = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    off = q - j
    covered = (off >= 0) & np.isin(off // B, deltas)
    tiles = covered.reshape(nb, B, nb, B).any(axis=(1, 3))
    for qb in range(nb):
        assert rows[qb].tolist() == np.nonzero(tiles[qb])[0].tolist(), qb
    plain = co.vs_rows(np.array([], dtype=np.int64), sel_s, nb)
    assert all(set(a.tolist()) <= set(b.tolist()) for a, b in zip(plain, rows))


def check_pe_per_row_uniform_closed_form(co):
    """Per-row PE (R22) on zero queries: row r of A_bar is uniform 1/(r+1), so the
    row keeps its first ceil(gamma (r+1)) blocks (ties to the lower block) and
    its diagonal."""
    rng = np.random.default_rng(6)
    for nb, gamma in ((24, 0.9437), (17, 0.5213)):
        # gamma (r + 1) stays clear of integers, so rounding in the prefix sums cannot move the cut
        assert min(abs(gamma * (r + 1) - round(gamma * (r + 1))) for r in range(nb)) > 1e-3
        n, d = nb * B, 64
        a_bar = co.pooled_map(np.zeros((n, d)), _rand(rng, n, d), B)
        pe = co.pe_select(a_bar, gamma, per_row=True)
        for r in range(nb):
            k = int(math.ceil(gamma * (r + 1)))
            assert pe["rows"][r].tolist() == sorted(set(range(k)) | {r}), (nb, r)


def check_pe_per_row_brute_force(co, seed=31):
    """Per-row PE (R22) against exhaustive search on short rows: the kept set of
    a row is a smallest subset whose mass reaches gamma, made of the largest
    scores (ties to the lower block), plus the diagonal."""
    import itertools
    rng = np.random.default_rng(seed)
    nb = 7
    for trial in range(6):
        logits = rng.normal(scale=1.5, size=(nb, nb))
        if trial == 5:
            logits = np.round(logits)                      # force ties
        logits[np.triu_indices(nb, 1)] = -np.inf
        a_bar = np.exp(logits - logits.max(axis=1, keepdims=True))
        a_bar /= a_bar.sum(axis=1, keepdims=True)
        gamma = 0.6 + 0.05 * trial
        pe = co.pe_select(a_bar, gamma, per_row=True)
        for r in range(nb):
            row = a_bar[r, : r + 1]
            best = None
            for size in range(1, r + 2):
                for sub in itertools.combinations(range(r + 1), size):
                    if row[list(sub)].sum() >= gamma:
                        best = size
                        break
                if best:
                    break
            order = sorted(range(r + 1), key=lambda j: (-row[j], j))
            want = set(order[:best]) | {r}
            assert set(pe["rows"][r].tolist()) == want, (trial, r)


# --- the layer driver: GQA head map, head subsets, forced routes, row subsets ------
# These take the driver module (``dcheck_*``): the layer driver produces every
# expected value of the GPU parity tests, so its query-head -> KV-head map and its
# query-row selection are pinned here against formulations that do not share it:
# K and V repeated per query head (torch's repeat_interleave / numpy's repeat).
def _gqa_bits(seed, batch=2, h_q=8, h_kv=2, n=384, d=32, q_scale=1.5):
    from prefill_inputs import f32_to_bf16_bits
    rng = np.random.default_rng(seed)
    q = f32_to_bf16_bits((rng.standard_normal((batch, h_q, n, d)) * q_scale).astype(np.float32))
    k = f32_to_bf16_bits(rng.standard_normal((batch, h_kv, n, d)).astype(np.float32))
    v = f32_to_bf16_bits(rng.standard_normal((batch, h_kv, n, d)).astype(np.float32))
    return q, k, v


def dcheck_layer_attention_gqa(drv, seed=40):
    """layer_attention on a GQA layer (batch 2, 8 query heads on 2 KV heads) equals
    torch's scaled_dot_product_attention (float64, CPU) with K and V repeated per
    query head and the explicit causal-and-selected token mask, on chosen query
    blocks and on chosen rows inside them."""
    import torch
    from prefill_inputs import bf16_bits_to_f32
    q, k, v = _gqa_bits(seed)
    nbat, H, n, d = q.shape
    G = H // k.shape[1]
    nb = n // B
    rng = np.random.default_rng(seed + 1)
    rows_of, blocks_of = {}, {}
    for b in range(nbat):
        for h in range(H):
            rows_of[(b, h)] = [np.array(sorted(set(rng.choice(qb + 1, size=int(rng.integers(1, qb + 2)),
                                                              replace=False).tolist()) | {qb}))
                               for qb in range(nb)]
            blocks_of[(b, h)] = [0, nb - 1] if (b + h) % 2 else [1]
    q_rows = [0, 5, 64, 127]
    got = drv.layer_attention(q, k, v, rows_of, blocks_of, workers=2, q_rows=q_rows)
    qt = torch.from_numpy(bf16_bits_to_f32(q).astype(np.float64))
    kt = torch.from_numpy(bf16_bits_to_f32(k).astype(np.float64)).repeat_interleave(G, dim=1)
    vt = torch.from_numpy(bf16_bits_to_f32(v).astype(np.float64)).repeat_interleave(G, dim=1)
    mask = np.zeros((nbat, H, n, n), dtype=bool)
    for (b, h), rows in rows_of.items():
        for qb, cols in enumerate(rows):
            for kb in cols:
                mask[b, h, qb * B:(qb + 1) * B, kb * B:(kb + 1) * B] = True
    mask &= np.tril(np.ones((n, n), dtype=bool))
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=torch.from_numpy(mask)).numpy()
    assert set(got) == {(b, h, qb) for (b, h), qbs in blocks_of.items() for qb in qbs}
    for (b, h, qb), o in got.items():
        want = ref[b, h, qb * B + np.asarray(q_rows)]
        assert o.shape == want.shape, (b, h, qb)
        assert np.allclose(o, want, rtol=1e-10, atol=1e-12), (b, h, qb)


def _selection_case(seed):
    q, k, _ = _gqa_bits(seed, n=768, q_scale=3.0)
    G = q.shape[1] // k.shape[1]
    return q, k, np.repeat(k, G, axis=1)   # kq[b, h]: the keys query head h reads


def dcheck_layer_selection_gqa(drv, seed=41):
    """layer_selection on a GQA layer matches crisp_head run head by head on the
    keys repeated per query head; a head subset and a forced route are honoured."""
    from oracle import crisp_oracle as co
    q, k, kq = _selection_case(seed)
    heads = [(0, 1), (0, 6), (1, 3), (1, 4)]
    got = drv.layer_selection(q, k, heads=heads, force_vs={(1, 3): False}, workers=2)
    assert sorted(got) == sorted(heads)
    for (b, h), r in got.items():
        ref = co.crisp_head(co.bf16_to_f64(q[b, h]), co.bf16_to_f64(kq[b, h]),
                            force_vs=False if (b, h) == (1, 3) else None)
        assert r["c_struct"] == ref["c_struct"] and r["is_vs"] == ref["is_vs"], (b, h)
        assert all(np.array_equal(x, y) for x, y in zip(r["rows"], ref["rows"])), (b, h)
    # on this short layer every head routes VS by itself (local window); the forced one is PE
    assert not got[(1, 3)]["is_vs"] and got[(0, 1)]["is_vs"]


def dcheck_layer_selection_flex_gqa(drv, seed=42):
    """layer_selection_flex on a GQA layer matches flex_head run head by head on
    the keys repeated per query head; a head subset and a forced route are honoured."""
    from oracle import crisp_oracle as co
    q, k, kq = _selection_case(seed)
    heads = [(0, 1), (0, 4), (1, 2), (1, 6)]
    got = drv.layer_selection_flex(q, k, heads=heads, force_vs={(0, 4): True}, workers=2)
    assert sorted(got) == sorted(heads)
    for (b, h), r in got.items():
        ref = co.flex_head(co.bf16_to_f64(q[b, h]), co.bf16_to_f64(kq[b, h]),
                           force_vs=True if (b, h) == (0, 4) else None)
        assert r["jsd"] == ref["jsd"] and r["is_vs"] == ref["is_vs"], (b, h)
        assert all(np.array_equal(x, y) for x, y in zip(r["rows"], ref["rows"])), (b, h)
    # Gaussian heads route PE under the JSD router; the forced one is VS
    assert got[(0, 4)]["is_vs"] and not got[(0, 1)]["is_vs"]
