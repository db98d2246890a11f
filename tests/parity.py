"""Helpers of the GPU parity tests: run the C-ABI path, check it against the oracle.

Rules (all decided with the oracle's values):
* routing: the pattern must match unless |C_struct - tau| <= 1e-5 * tau; such a
  head is re-run in the oracle with the GPU's pattern forced.
* VS selection: a block may differ only if its score is within 1e-5 relative of
  alpha*mu, or (when fewer than k_min blocks pass) of the k-th largest score.
* PE selection: a cell may differ only if its score is within 1e-5 relative of
  the cut score x_(K*-1), or the oracle's prefix mass before it is within
  1e-5 * gamma of gamma.
* CSR: VS rows must equal the rows the oracle builds from the GPU's own block
  sets; every row is ascending, distinct, <= qb, and holds its diagonal.
* outputs: against the oracle's exact attention on the GPU's own CSR,
  max-abs <= 1e-2 and mean-abs <= 1e-3 (bf16 inputs, fp32 accumulation).
"""
from __future__ import annotations

import math

import numpy as np
import torch

import long_context_sparse_patsearch_amd as crisp
from oracle import crisp_oracle as co
from oracle.driver import layer_attention, layer_selection

REL = 1e-5
MAX_ABS = 1e-2
MEAN_ABS = 1e-3


def f32(x):
    return float(np.float32(x))


def to_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda").view(torch.bfloat16)


def device_inputs(inp):
    return tuple(to_dev(inp[t]) for t in ("q", "k", "v"))


def gpu_layer(q, k, v, cfg, attn=True, out_dtype=torch.float32, variant=0):
    r = crisp.route(q, k, cfg)
    s = crisp.select(q, k, r, cfg, with_mask=True, variant=variant)
    o = crisp.sparse_attn(q, k, v, s, cfg, out_dtype=out_dtype) if attn else None
    torch.cuda.synchronize()
    row_ptr = s["row_ptr"].cpu().numpy()
    nnz = int(row_ptr[-1])
    return dict(c=r["c_struct"].cpu().numpy(), pattern=r["pattern"].cpu().numpy(),
                p_vert=r["p_vert"].cpu().numpy(), p_slash=r["p_slash"].cpu().numpy(),
                row_ptr=row_ptr, col=s["col_idx"][:nnz].cpu().numpy(), mask=s["sel_mask"].cpu().numpy(),
                sel=s, out=o)


def rows_of(g, bh, nb):
    rp, col = g["row_ptr"], g["col"]
    return [col[rp[bh * nb + qb]: rp[bh * nb + qb + 1]].astype(np.int64) for qb in range(nb)]


def check_csr_structure(g, bh_total, nb, cap):
    rp = g["row_ptr"]
    assert rp[0] == 0 and np.all(np.diff(rp) >= 0) and rp[-1] <= cap
    for bh in range(bh_total):
        for qb, row in enumerate(rows_of(g, bh, nb)):
            assert len(row) >= 1 and row[-1] == qb, (bh, qb)
            assert np.all(np.diff(row) > 0) and row[0] >= 0, (bh, qb)


def check_route(g, ora, H, tau):
    """Returns {(b,h): gpu pattern} for heads on the routing threshold (exempt)."""
    exempt = {}
    for (b, h), r in ora.items():
        i = b * H + h
        c_o = r["c_struct"]
        assert abs(g["c"][i] - c_o) <= 2e-5 * abs(c_o) + 1e-7, ((b, h), g["c"][i], c_o)
        gv = bool(g["pattern"][i])
        if abs(c_o - tau) <= REL * abs(tau):
            exempt[(b, h)] = gv
        else:
            assert gv == r["is_vs"], ((b, h), c_o)
        nb = len(r["p_v"])
        assert np.allclose(g["p_vert"][i], r["p_v"], rtol=1e-4, atol=1e-9), (b, h)
        assert np.allclose(g["p_slash"][i], r["p_s"], rtol=1e-4, atol=1e-9), (b, h)
        assert g["p_vert"][i].shape == (nb,)
    return exempt


def _vs_exempt(p, j, alpha, mu, cnt, kmin):
    thr = alpha * mu
    if abs(p[j] - thr) <= REL * thr:
        return True
    nb = len(p)
    k = min(max(cnt, kmin), nb)
    if cnt < kmin and k < nb:
        pk = np.sort(p)[::-1][k - 1]
        if abs(p[j] - pk) <= REL * pk:
            return True
    return False


def check_vs(g, bh, r, alpha, kmin, nb, band=False):
    mask = g["mask"][bh]
    sets = {}
    for dir_, key_sel, key_p, key_mu, key_cnt in ((0, "sel_v", "p_v", "mu_v", "cnt_v"), (1, "sel_s", "p_s", "mu_s", "cnt_s")):
        gs = set(np.nonzero(mask[dir_])[0].tolist())
        os_ = set(r[key_sel].tolist())
        for j in gs ^ os_:
            assert j not in (0, nb - 1)
            assert _vs_exempt(r[key_p], j, alpha, r[key_mu], r[key_cnt], kmin), \
                (bh, dir_, j, r[key_p][j], alpha * r[key_mu])
        sets[dir_] = np.array(sorted(gs), dtype=np.int64)
    want = co.vs_rows(sets[0], sets[1], nb, band)
    got = rows_of(g, bh, nb)
    for qb in range(nb):
        assert np.array_equal(got[qb], want[qb]), (bh, qb)
    return sum(len(x ^ y) for x, y in [(set(np.nonzero(mask[0])[0]), set(r["sel_v"])),
                                        (set(np.nonzero(mask[1])[0]), set(r["sel_s"]))])


def check_pe_rows(g, bh, r, gamma, nb):
    """Per-row PE (R22): every row's set equals the oracle's, except cells on
    that row's own cut (score or prefix within REL of the row's threshold)."""
    assert not g["mask"][bh].any()
    pe = r["pe"]
    x = pe["x"]
    got = rows_of(g, bh, nb)
    ndiff = 0
    for qb in range(nb):
        a, b_ = set(got[qb].tolist()), set(pe["rows"][qb].tolist())
        if a == b_:
            continue
        base = qb * (qb + 1) // 2
        order, cs, kept = pe["row_order"][qb], pe["row_cs"][qb], pe["row_kept"][qb]
        v = x[base: base + qb + 1] * nb
        v_cut = v[kept[-1]]
        rank = np.empty(qb + 1, dtype=np.int64)
        rank[order] = np.arange(qb + 1)
        for kb in a ^ b_:
            before = cs[rank[kb] - 1] if rank[kb] > 0 else 0.0
            ok = abs(v[kb] - v_cut) <= REL * v_cut or abs(before - gamma) <= REL * gamma
            assert ok, (bh, qb, kb, v[kb], v_cut, before)
            ndiff += 1
    return ndiff


def check_pe(g, bh, r, gamma, nb):
    if r["pe"].get("per_row"):
        return check_pe_rows(g, bh, r, gamma, nb)
    assert not g["mask"][bh].any()
    pe = r["pe"]
    x, order, cs = pe["x"], pe["order"], pe["cs"]
    kstar = len(pe["kept"])
    x_cut = x[order[kstar - 1]]
    rank = np.empty(len(x), dtype=np.int64)
    rank[order] = np.arange(len(x))
    got = rows_of(g, bh, nb)
    ndiff = 0
    for qb in range(nb):
        a, b_ = set(got[qb].tolist()), set(pe["rows"][qb].tolist())
        for kb in a ^ b_:
            pos = qb * (qb + 1) // 2 + kb
            before = cs[rank[pos] - 1] if rank[pos] > 0 else 0.0
            ok = abs(x[pos] - x_cut) <= REL * x_cut or abs(before - gamma) <= REL * gamma
            assert ok, (bh, qb, kb, x[pos], x_cut, before)
            ndiff += 1
    return ndiff


def oracle_layer(inp, cfg_kw, force_vs=None, workers=None, floor="mean", band=False, pe_per_row=False):
    return layer_selection(inp["q"], inp["k"], force_vs=force_vs, workers=workers, floor=floor, band=band,
                           pe_per_row=pe_per_row, **cfg_kw)


def check_selection(g, inp, ora, cfg_kw, H, nb, floor="mean", band=False, pe_per_row=False):
    """Route + select checks; returns the oracle dict actually compared (after re-runs)."""
    exempt = check_route(g, ora, H, cfg_kw["tau"])
    if exempt:
        redo = {bh: v for bh, v in exempt.items() if v != ora[bh]["is_vs"]}
        if redo:
            ora = dict(ora)
            ora.update(layer_selection(inp["q"], inp["k"], heads=list(redo), force_vs=redo, floor=floor,
                                        band=band, pe_per_row=pe_per_row, **cfg_kw))
    kmin = cfg_kw["k_min_tokens"] // 128
    stats = dict(vs_diff=0, pe_diff=0)
    for (b, h), r in ora.items():
        bh = b * H + h
        if r["is_vs"]:
            stats["vs_diff"] += check_vs(g, bh, r, cfg_kw["alpha"], kmin, nb, band)
        else:
            stats["pe_diff"] += check_pe(g, bh, r, cfg_kw["gamma"], nb)
    return ora, stats


def check_outputs(out_dev, inp, rows_by_head, blocks_by_head, q_rows=None, G=1):
    """Compare sampled output blocks of the GPU (tensor on device) with the oracle."""
    ref = layer_attention(inp["q"], inp["k"], inp["v"], rows_by_head, blocks_by_head, q_rows=q_rows)
    worst = 0.0
    errs = []
    for (b, h, qb), o in ref.items():
        r_off = np.arange(128) if q_rows is None else np.asarray(q_rows)
        got = out_dev[b, h, qb * 128 + torch.as_tensor(r_off, device=out_dev.device)].float().cpu().numpy()
        e = np.abs(got - o)
        worst = max(worst, float(e.max()))
        errs.append(e.mean())
        assert e.max() <= MAX_ABS, ((b, h, qb), float(e.max()))
    mean = float(np.mean(errs)) if errs else 0.0
    assert mean <= MEAN_ABS, mean
    return worst, mean


def sample_blocks(nb, rng, extra=1):
    pick = {0, nb - 1, nb // 2}
    while len(pick) < min(nb, 3 + extra):
        pick.add(int(rng.integers(0, nb)))
    return sorted(pick)


def cfg_kwargs(cfg):
    return dict(tau=f32(cfg.tau), alpha=f32(cfg.alpha), gamma=f32(cfg.gamma), k_min_tokens=cfg.k_min_tokens)


# --- the FlexPrefill baseline path --------------------------------------------------------------
JSD_RTOL = 1e-4


def gpu_flex_layer(q, k, v, cfg, tau_jsd, attn=True):
    r = crisp.route(q, k, cfg)
    f = crisp.flex_route(q, k, r, tau_jsd, cfg)
    s = crisp.flex_select(q, k, f, cfg, with_mask=True)
    o = crisp.sparse_attn(q, k, v, s, cfg) if attn else None
    torch.cuda.synchronize()
    row_ptr = s["row_ptr"].cpu().numpy()
    nnz = int(row_ptr[-1])
    return dict(jsd=f["jsd"].cpu().numpy(), pattern=f["pattern"].cpu().numpy(),
                p_vert=r["p_vert"].cpu().numpy(), p_slash=r["p_slash"].cpu().numpy(),
                row_ptr=row_ptr, col=s["col_idx"][:nnz].cpu().numpy(), mask=s["sel_mask"].cpu().numpy(),
                sel=s, out=o)


def check_flex_route(g, ora, H, tau_jsd):
    """D_JS to JSD_RTOL of the oracle's; the pattern exact unless the oracle's
    D_JS is within 1e-5 relative of tau_jsd (the routing rule of CRISP's router).
    Returns {(b,h): gpu pattern} for exempt heads."""
    exempt = {}
    for (b, h), r in ora.items():
        i = b * H + h
        j_o = r["jsd"]
        assert abs(g["jsd"][i] - j_o) <= JSD_RTOL * abs(j_o) + 1e-7, ((b, h), g["jsd"][i], j_o)
        gv = bool(g["pattern"][i])
        if abs(j_o - tau_jsd) <= REL * tau_jsd:
            exempt[(b, h)] = gv
        else:
            assert gv == r["is_vs"], ((b, h), j_o)
    return exempt


def _gamma_exempt(p, j, gamma, kmin):
    """Block j may differ between the GPU's and the oracle's gamma-cumsum set when
    the oracle's prefix mass before it (which decides whether it is kept) is
    within 1e-5 gamma of gamma, or its score ties the score at the cut (or at the
    k_min boundary) within 1e-5 relative."""
    nb = len(p)
    order = np.lexsort((np.arange(nb), -p))
    cs = np.cumsum(p[order])
    hit = np.nonzero(cs >= gamma)[0]
    cnt = int(hit[0]) + 1 if len(hit) else nb
    pos = int(np.nonzero(order == j)[0][0])
    before = cs[pos - 1] if pos > 0 else 0.0
    if abs(before - gamma) <= REL * gamma:
        return True
    k = min(max(cnt, kmin), nb)
    edge = p[order[k - 1]]
    return abs(p[j] - edge) <= REL * max(edge, 1e-30)


def check_flex_vs(g, bh, r, gamma, kmin, nb):
    mask = g["mask"][bh]
    sets = {}
    ndiff = 0
    for dir_, key_sel, key_p in ((0, "sel_v", "p_v"), (1, "sel_s", "p_s")):
        gs = set(np.nonzero(mask[dir_])[0].tolist())
        os_ = set(r[key_sel].tolist())
        for j in gs ^ os_:
            assert j not in (0, nb - 1)
            assert _gamma_exempt(r[key_p], j, gamma, kmin), (bh, dir_, j, r[key_p][j])
            ndiff += 1
        sets[dir_] = np.array(sorted(gs), dtype=np.int64)
    want = co.vs_rows(sets[0], sets[1], nb)
    got = rows_of(g, bh, nb)
    for qb in range(nb):
        assert np.array_equal(got[qb], want[qb]), (bh, qb)
    return ndiff


def check_flex_selection(g, inp, ora, kw, H, nb):
    """FlexPrefill route + select checks; returns the oracle dict compared (after re-runs)."""
    from oracle.driver import layer_selection_flex
    exempt = check_flex_route(g, ora, H, kw["tau_jsd"])
    if exempt:
        redo = {bh: v for bh, v in exempt.items() if v != ora[bh]["is_vs"]}
        if redo:
            ora = dict(ora)
            ora.update(layer_selection_flex(inp["q"], inp["k"], heads=list(redo), force_vs=redo, **kw))
    kmin = kw["k_min_tokens"] // 128
    stats = dict(vs_diff=0, pe_diff=0)
    for (b, h), r in ora.items():
        bh = b * H + h
        if r["is_vs"]:
            stats["vs_diff"] += check_flex_vs(g, bh, r, kw["gamma"], kmin, nb)
        else:
            stats["pe_diff"] += check_pe(g, bh, r, kw["gamma"], nb)
    return ora, stats
