"""Plain, slow fp64 CPU oracle of the CRISP sparse-attention prefill.

TEST INFRASTRUCTURE.  Only the test suite, the package's smoke check and the
benchmark's CPU-baseline leg may import or run this module.  It shares no code
with the GPU path: every step below is written from the pages' definitions in
numpy float64, computed from the exact bf16 input bits.

Citations name pages by title:

* [digest] -- the paper digest page "CRISP: Cliff-awaRe Input-adaptive Sparse
  Prefilling with Structural-Mass-Motivated Routing" (Chinese, with the
  prerequisite sections, the method, the method-steps section and the captions
  of Algorithms 1-4).
* [abstract] -- the English abstract carried by the other pages.

Readings taken where the pages are silent or ambiguous (each also recorded in
the design notes of the repository):

R1  The proxy softmax is causal: proxy row i is query position n-b+i and sees
    keys j <= n-b+i (autoregressive prefill).
R2  The final attention is causal and masked to the selected blocks.
R3  b = B = 128, so the proxy rows are exactly the last query block.
R4  "Column mean" / "diagonal mean" average over the b proxy rows; block
    pooling sums the per-token scores inside each 128-token block, so both
    block-score vectors sum to 1.
R5  Slash index t = j + (b-1-i): t = n-1 is the main diagonal, so slash block
    N_b-1 holds offsets 0..127 (local) and slash block 0 the farthest offsets.
R6  Slash block k selects the block diagonal delta = N_b-1-k, i.e. tiles
    (qb, qb-delta) for qb >= delta.
R7  The anchors {0, N_b-1} join both directions: every VS row keeps key block
    0 and its own diagonal block.
R8  Comparisons are exactly as printed: routing C >= tau, noise floor p > alpha*mu
    (strict), gamma-cumsum prefix >= gamma.
R9  The per-direction clip counts blocks (k_min tokens / B); if fewer blocks pass
    the floor, the next largest scores pad the set (top-k).  The floor is tested
    over every block including 0 and N_b-1; anchors are added after the clip.
R10 Every ordering breaks ties toward the smaller index (block j, or flat
    index qb*N_b + kb).
R11 The PE gamma-cumsum runs globally over the whole block-causal pooled map
    after dividing by N_b (so the flattened scores sum to 1).
R12 PE pooling is the mean of Q rows and of K rows inside each block, logits
    are scaled by 1/sqrt(d), and the pooled softmax is block-causal (kb <= qb).
R13 Every PE row keeps its diagonal block, so each query sees at least its own
    block and the masked softmax exists.
R14 Grouped KV heads: query head h uses KV head floor(h / (h_q / h_kv)); routing
    and selection are per query head.
R15 If the whole flattened PE map sums to less than gamma (rounding), every
    entry is kept.
R18 FlexPrefill's JSD router (the method CRISP replaces): a_hat is the proxy's
    "softmax, then average" key-block distribution, i.e. p_v of R4; a_bar is
    the "pool, then softmax" estimate: the b proxy queries mean-pooled into one
    query against the mean-pooled key of every block, logits / sqrt(d), softmax
    over all N_b blocks (the last query block sees every key block).  D_JS uses
    the natural log; the head routes VS iff D_JS >= tau_jsd.  The pages give
    no value for tau_jsd; it is a parameter.
R20 Median noise floor (the variant of the pages' Table 9): mu is the median
    of the N_b-2 non-anchor block scores instead of their mean; the rest of the
    rule is unchanged.
R21 Slash band (variant of R6): a selected slash block covers the token
    offsets 128 delta .. 128 delta + 127, which fall in the tiles of block
    diagonals delta and delta + 1, so both are selected.
R19 FlexPrefill's VS index is Algorithm 3 with the per-direction noise-floor
    rule replaced by the gamma-cumsum budget rule (same gamma as the PE path):
    the shortest descending prefix of p_d reaching gamma, its count clipped to
    [k_min, N_b] (top-k), then the anchors {0, N_b-1}.
R22 Per-row PE (variant of R11): the gamma-cumsum runs inside each row of the
    pooled map, which is a distribution over kb <= qb: a row keeps its own
    shortest descending prefix reaching gamma (ties to the lower block, R10;
    the whole row if it falls short, R15), and its diagonal as in R13.
"""
from __future__ import annotations

import math

import numpy as np

BLOCK = 128


# ----------------------------------------------------------------------------
# inputs
# ----------------------------------------------------------------------------
def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns as float64 (a bf16 is the top half of a float32)."""
    w = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return w.view(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------
# Algorithm 2 (PatSearch): proxy attention, structural mass, routing
# ----------------------------------------------------------------------------
def proxy_attention(q_h: np.ndarray, k_g: np.ndarray, b: int = BLOCK) -> np.ndarray:
    """A_hat = Softmax(Q_hat K^T / sqrt(d)) with Q_hat the last b queries.

    [digest] section "Core method" (PatSearch) and the Algorithm 2 caption;
    causal per reading R1.  Returns a (b, n) array whose rows sum to 1.
    """
    n, d = k_g.shape
    qhat = q_h[n - b:]
    s = (qhat @ k_g.T) / math.sqrt(d)
    pos = n - b + np.arange(b)
    future = np.arange(n)[None, :] > pos[:, None]
    s[future] = -np.inf
    s -= s.max(axis=1, keepdims=True)
    e = np.exp(s)
    return e / e.sum(axis=1, keepdims=True)


def structural_mass(a_hat: np.ndarray, w_sink: int = 128, w_local: int = 128) -> float:
    """C_struct = (1/|Q_hat|) sum_i sum_{j in S_anchor} A_hat[i, j].

    S_anchor = the first w_sink keys and the last w_local keys.  [digest]
    section "Core method", Algorithm 2 caption.
    """
    b, n = a_hat.shape
    anchor = np.zeros(n, dtype=bool)
    anchor[:w_sink] = True
    anchor[n - w_local:] = True
    return float(a_hat[:, anchor].sum() / b)


def route(c_struct: float, tau: float = 0.2) -> bool:
    """True = Vertical-Slash, False = Pooled-Estimation: VS iff C_struct >= tau (R8)."""
    return bool(c_struct >= tau)


# ----------------------------------------------------------------------------
# Algorithm 3 (VSIndex, sink-aware)
# ----------------------------------------------------------------------------
def vs_scores(a_hat: np.ndarray, block: int = BLOCK):
    """Vertical and slash scores, block-pooled (R4, R5).

    a_v[j] = mean over proxy rows of A_hat[i, j]; a_s[t] = mean over proxy rows
    of the entries on diagonal t = j + (b-1-i); p_d[k] = sum of a_d over block k.
    [digest] section "Method steps" step 2 and the Algorithm 3 caption.
    """
    b, n = a_hat.shape
    a_v = a_hat.sum(axis=0) / b
    a_s = np.zeros(n)
    for i in range(b):
        off = b - 1 - i
        a_s[off:] += a_hat[i, : n - off]
    a_s /= b
    nb = n // block
    p_v = a_v.reshape(nb, block).sum(axis=1)
    p_s = a_s.reshape(nb, block).sum(axis=1)
    return p_v, p_s


def noise_floor_select(p: np.ndarray, alpha: float, k_min_blocks: int, floor: str = "mean"):
    """Sink-aware noise-floor selection for one direction.

    r = max(1 - p[0] - p[N_b-1], 0), mu = r / (N_b - 2); keep every block with
    p[j] > alpha*mu, clip the count to [k_min, N_b] (top-k, ties to the lower
    index), then add the anchor blocks 0 and N_b-1.  [digest] sections "Core
    method" and "Method steps" step 2, Algorithm 3 caption; readings R8-R10.
    ``floor="median"`` takes mu as the median of the non-anchor scores (R20).
    Returns (sorted selected blocks, mu, number above the floor).
    """
    nb = len(p)
    r = max(1.0 - p[0] - p[nb - 1], 0.0)
    mu = r / (nb - 2)
    if floor == "median":
        mu = float(np.median(p[1:nb - 1]))
    above = int(np.count_nonzero(p > alpha * mu))
    k = min(max(above, k_min_blocks), nb)
    order = np.lexsort((np.arange(nb), -p))
    sel = set(order[:k].tolist()) | {0, nb - 1}
    return np.array(sorted(sel), dtype=np.int64), mu, above


def vs_rows(sel_v: np.ndarray, sel_s: np.ndarray, nb: int, band: bool = False):
    """Key blocks of every query block of a VS head (R6, R7).

    Row qb = {kb in S_v : kb <= qb} U {qb - delta : delta = N_b-1-k, k in S_s, delta <= qb};
    with ``band`` the diagonals delta + 1 join as well (R21).
    """
    deltas = nb - 1 - np.asarray(sel_s)
    if band:
        deltas = np.union1d(deltas, deltas + 1)
    rows = []
    for qb in range(nb):
        v = sel_v[sel_v <= qb]
        s = qb - deltas[deltas <= qb]
        rows.append(np.union1d(v, s).astype(np.int64))
    return rows


# ----------------------------------------------------------------------------
# Algorithm 4 (PEIndex, global adaptive) and the gamma-cumsum rule
# ----------------------------------------------------------------------------
def pooled_map(q_h: np.ndarray, k_g: np.ndarray, block: int = BLOCK) -> np.ndarray:
    """A_bar: block-causal softmax of mean-pooled queries against mean-pooled keys.

    Pools all queries (not only the proxy rows).  [digest] section "Method
    steps" step 3 and the Algorithm 4 caption; reading R12.  Returns an
    (N_b, N_b) array, zero above the diagonal, rows summing to 1.
    """
    n, d = q_h.shape
    nb = n // block
    qbar = q_h.reshape(nb, block, d).mean(axis=1)
    kbar = k_g.reshape(nb, block, d).mean(axis=1)
    s = (qbar @ kbar.T) / math.sqrt(d)
    future = np.arange(nb)[None, :] > np.arange(nb)[:, None]
    s[future] = -np.inf
    s -= s.max(axis=1, keepdims=True)
    e = np.exp(s)
    return e / e.sum(axis=1, keepdims=True)


def gamma_cumsum(x: np.ndarray, gamma: float):
    """Smallest prefix of x sorted descending whose sum reaches gamma.

    The budget rule "minimise |S| subject to sum_{j in S} a_j >= gamma",
    realised by sorting and accumulating until gamma is reached.  [digest]
    prerequisite section on the cumulative-coverage threshold; ties go to the
    lower index (R10); if the total falls short every entry is kept (R15).
    Returns (kept indices in sorted order, the descending order, the prefix
    sums along it).
    """
    order = np.lexsort((np.arange(len(x)), -x))
    cs = np.cumsum(x[order])
    hit = np.nonzero(cs >= gamma)[0]
    k = int(hit[0]) + 1 if len(hit) else len(x)
    return order[:k], order, cs


def pe_select(a_bar: np.ndarray, gamma: float, per_row: bool = False):
    """Global gamma-cumsum over the flattened block-causal map (R11, R13).

    Entries are the valid (qb, kb <= qb) cells in row-major order, scored
    x = A_bar / N_b.  Returns dict(rows, x, qb, kb, order, cs, kept) where
    ``kept`` are positions into x (the flattened valid cells).  With
    ``per_row`` each row runs its own gamma-cumsum over A_bar[qb, :qb+1]
    (R22); the dict then holds, per row, ``row_order`` and ``row_cs`` (the
    row's descending order and prefix sums) and ``row_kept``.
    """
    nb = a_bar.shape[0]
    qb, kb = np.tril_indices(nb)
    x = a_bar[qb, kb] / nb
    mask = np.zeros((nb, nb), dtype=bool)
    if per_row:
        row_kept, row_order, row_cs = [], [], []
        for r in range(nb):
            k_r, o_r, c_r = gamma_cumsum(a_bar[r, : r + 1], gamma)
            mask[r, k_r] = True
            row_kept.append(k_r)
            row_order.append(o_r)
            row_cs.append(c_r)
        mask[np.diag_indices(nb)] = True
        rows = [np.nonzero(mask[r, : r + 1])[0].astype(np.int64) for r in range(nb)]
        return dict(rows=rows, x=x, qb=qb, kb=kb, per_row=True, row_kept=row_kept, row_order=row_order,
                    row_cs=row_cs)
    kept, order, cs = gamma_cumsum(x, gamma)
    mask[qb[kept], kb[kept]] = True
    mask[np.arange(nb), np.arange(nb)] = True
    rows = [np.nonzero(mask[r, : r + 1])[0].astype(np.int64) for r in range(nb)]
    return dict(rows=rows, x=x, qb=qb, kb=kb, order=order, cs=cs, kept=kept)


# ----------------------------------------------------------------------------
# exact masked attention A(Q, K, V, S)
# ----------------------------------------------------------------------------
def block_sparse_attention(q_h, k_g, v_g, rows, q_blocks=None, block: int = BLOCK,
                           q_rows=None):
    """A(Q,K,V,S) = Softmax(QK^T/sqrt(d) + M_S) V, causal (R2).

    M_S leaves only the keys of the selected key blocks of each query block.
    [digest] prerequisite section on prefill and sparse attention, and
    "Method steps" step 4.  Computes the query blocks in ``q_blocks`` (default
    all); ``q_rows`` optionally restricts to given row offsets inside each
    block.  A query with no visible key gets a zero output.  Returns
    {qb: (rows, d) array}.
    """
    n, d = q_h.shape
    nb = n // block
    scale = 1.0 / math.sqrt(d)
    out = {}
    for qb in (range(nb) if q_blocks is None else q_blocks):
        cols = np.asarray(rows[qb], dtype=np.int64)
        r_off = np.arange(block) if q_rows is None else np.asarray(q_rows)
        qpos = qb * block + r_off
        if len(cols) == 0:
            out[qb] = np.zeros((len(qpos), d))
            continue
        keys = (cols[:, None] * block + np.arange(block)[None, :]).reshape(-1)
        s = (q_h[qpos] @ k_g[keys].T) * scale
        vis = keys[None, :] <= qpos[:, None]
        s = np.where(vis, s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        has = np.isfinite(m[:, 0])
        m[~has] = 0.0
        e = np.where(vis, np.exp(s - m), 0.0)
        den = e.sum(axis=1, keepdims=True)
        den[~has] = 1.0
        out[qb] = (e @ v_g[keys]) / den
    return out


def dense_rows(nb: int):
    """Every causal key block of every query block (the dense baseline's set)."""
    return [np.arange(qb + 1, dtype=np.int64) for qb in range(nb)]


def dense_attention(q_h, k_g, v_g, q_blocks=None, block: int = BLOCK, q_rows=None):
    """Exact causal softmax attention, the result FlashAttention computes.

    [digest] prerequisite section on FlashAttention (the dense reference).
    """
    return block_sparse_attention(q_h, k_g, v_g, dense_rows(q_h.shape[0] // block),
                                  q_blocks=q_blocks, block=block, q_rows=q_rows)


# ----------------------------------------------------------------------------
# Algorithm 1: one head end to end
# ----------------------------------------------------------------------------
def crisp_head(q_h, k_g, *, tau=0.2, alpha=1.0, gamma=0.95, k_min_tokens=1024,
               block=BLOCK, force_vs=None, floor="mean", band=False, pe_per_row=False):
    """Routing and selection of one query head, as Algorithm 1 assembles them.

    PatSearch, then VSIndex if the head routes VS, else PEIndex.  ``force_vs``
    overrides the routing decision (used to re-run a head whose structural mass
    sits on the threshold); ``floor``, ``band`` and ``pe_per_row`` select the
    variants R20, R21 and R22.  Returns a dict with the route, the scores and the per-query-block
    key-block rows.
    """
    n = q_h.shape[0]
    nb = n // block
    a_hat = proxy_attention(q_h, k_g, block)
    c = structural_mass(a_hat, block, block)
    p_v, p_s = vs_scores(a_hat, block)
    del a_hat
    is_vs = route(c, tau) if force_vs is None else bool(force_vs)
    res = dict(c_struct=c, is_vs=is_vs, p_v=p_v, p_s=p_s)
    if is_vs:
        kmin = k_min_tokens // block
        sv, mu_v, cnt_v = noise_floor_select(p_v, alpha, kmin, floor)
        ss, mu_s, cnt_s = noise_floor_select(p_s, alpha, kmin, floor)
        res.update(sel_v=sv, sel_s=ss, mu_v=mu_v, mu_s=mu_s, cnt_v=cnt_v, cnt_s=cnt_s,
                   rows=vs_rows(sv, ss, nb, band))
    else:
        pe = pe_select(pooled_map(q_h, k_g, block), gamma, per_row=pe_per_row)
        res.update(pe=pe, rows=pe["rows"])
    return res


# ----------------------------------------------------------------------------
# the FlexPrefill baseline path (the routing and VS budget rule CRISP replaces)
# ----------------------------------------------------------------------------
def pooled_proxy_estimate(q_h: np.ndarray, k_g: np.ndarray, b: int = BLOCK, block: int = BLOCK) -> np.ndarray:
    """a_bar: the "pool first, then softmax" estimate of the proxy's key-block distribution (R18).

    [digest] prerequisite section on Jensen-Shannon divergence.  Returns N_b
    probabilities summing to 1.
    """
    n, d = q_h.shape
    nb = n // block
    qbar = q_h[n - b:].mean(axis=0)
    kbar = k_g.reshape(nb, block, d).mean(axis=1)
    s = (kbar @ qbar) / math.sqrt(d)
    e = np.exp(s - s.max())
    return e / e.sum()


def jensen_shannon(p: np.ndarray, q: np.ndarray) -> float:
    """D_JS = 1/2 KL(p || m) + 1/2 KL(q || m) with m = (p + q) / 2, natural log.

    [digest] prerequisite section on Jensen-Shannon divergence.  Terms with a
    zero numerator contribute 0.
    """
    p = np.asarray(p, dtype=np.float64)
    q = np.asarray(q, dtype=np.float64)
    m = 0.5 * (p + q)
    def kl(a):
        nz = a > 0
        return float(np.sum(a[nz] * np.log(a[nz] / m[nz])))
    return 0.5 * kl(p) + 0.5 * kl(q)


def jsd_route(d_js: float, tau_jsd: float) -> bool:
    """FlexPrefill's router: Vertical-Slash iff D_JS >= tau_jsd (R18, R8)."""
    return bool(d_js >= tau_jsd)


def gamma_direction_select(p: np.ndarray, gamma: float, k_min_blocks: int):
    """FlexPrefill's budget rule for one VS direction (R19).

    The gamma-cumsum set of p (ties to the lower index), its count clipped to
    [k_min, N_b] by taking the top-k, then the anchors 0 and N_b-1.  [digest]
    prerequisite section on the cumulative-coverage threshold and the Algorithm
    3 caption.  Returns (sorted selected blocks, size of the gamma-cumsum set).
    """
    nb = len(p)
    kept, order, _ = gamma_cumsum(np.asarray(p, dtype=np.float64), gamma)
    k = min(max(len(kept), k_min_blocks), nb)
    sel = {0, nb - 1}.union(order[:k].tolist())
    return np.array(sorted(sel), dtype=np.int64), len(kept)


def flex_head(q_h, k_g, *, tau_jsd=0.1, gamma=0.95, k_min_tokens=1024, block=BLOCK, force_vs=None):
    """FlexPrefill's routing and selection of one query head, the baseline the pages compare with.

    The same proxy as PatSearch; JSD routing between a_hat = p_v and the pooled
    estimate a_bar (R18); VS heads take the gamma-cumsum budget rule in both
    directions (R19), PE heads the same PEIndex as CRISP.  ``force_vs``
    overrides the routing decision.
    """
    n = q_h.shape[0]
    nb = n // block
    a_hat = proxy_attention(q_h, k_g, block)
    p_v, p_s = vs_scores(a_hat, block)
    del a_hat
    a_bar = pooled_proxy_estimate(q_h, k_g, block, block)
    d_js = jensen_shannon(p_v, a_bar)
    is_vs = jsd_route(d_js, tau_jsd) if force_vs is None else bool(force_vs)
    res = dict(jsd=d_js, is_vs=is_vs, p_v=p_v, p_s=p_s, a_bar=a_bar)
    if is_vs:
        kmin = k_min_tokens // block
        sv, cnt_v = gamma_direction_select(p_v, gamma, kmin)
        ss, cnt_s = gamma_direction_select(p_s, gamma, kmin)
        res.update(sel_v=sv, sel_s=ss, cnt_v=cnt_v, cnt_s=cnt_s, rows=vs_rows(sv, ss, nb))
    else:
        pe = pe_select(pooled_map(q_h, k_g, block), gamma)
        res.update(pe=pe, rows=pe["rows"])
    return res

