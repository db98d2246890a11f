"""Each plausible mistake planted in a copy of the oracle fails at least one pin.

The mutation is a textual edit of the oracle's source, loaded as a separate
module on the CPU; the real oracle is untouched.
"""
import types

import pytest

import oracle_pins as pins
from oracle import crisp_oracle, driver

SRC = open(crisp_oracle.__file__).read()

MUTANTS = {
    "proxy_not_causal": ("    s[future] = -np.inf\n    s -= s.max(axis=1, keepdims=True)\n    e = np.exp(s)\n    return e / e.sum(axis=1, keepdims=True)\n\n\ndef structural",
                         "    s -= s.max(axis=1, keepdims=True)\n    e = np.exp(s)\n    return e / e.sum(axis=1, keepdims=True)\n\n\ndef structural"),
    "proxy_no_scale": ("    s = (qhat @ k_g.T) / math.sqrt(d)", "    s = (qhat @ k_g.T)"),
    "slash_flipped": ("        off = b - 1 - i\n", "        off = i\n"),
    "vertical_not_mean": ("    a_v = a_hat.sum(axis=0) / b", "    a_v = a_hat.sum(axis=0)"),
    "mu_over_nb": ("    mu = r / (nb - 2)", "    mu = r / nb"),
    "floor_non_strict": ("    above = int(np.count_nonzero(p > alpha * mu))", "    above = int(np.count_nonzero(p >= alpha * mu))"),
    "floor_no_clamp": ("    r = max(1.0 - p[0] - p[nb - 1], 0.0)", "    r = 1.0 - p[0] - p[nb - 1]"),
    "ties_to_higher": ("    order = np.lexsort((np.arange(nb), -p))", "    order = np.lexsort((-np.arange(nb), -p))"),
    "no_anchors": ("    sel = set(order[:k].tolist()) | {0, nb - 1}", "    sel = set(order[:k].tolist())"),
    "slash_delta_wrong": ("    deltas = nb - 1 - np.asarray(sel_s)", "    deltas = np.asarray(sel_s)"),
    "pool_sum_not_mean": ("    qbar = q_h.reshape(nb, block, d).mean(axis=1)", "    qbar = q_h.reshape(nb, block, d).sum(axis=1)"),
    "pooled_not_causal": ("    future = np.arange(nb)[None, :] > np.arange(nb)[:, None]\n    s[future] = -np.inf\n",
                          "    future = np.arange(nb)[None, :] > np.arange(nb)[:, None]\n"),
    "gamma_strict": ("    hit = np.nonzero(cs >= gamma)[0]", "    hit = np.nonzero(cs > gamma)[0]"),
    "gamma_off_by_one": ("    k = int(hit[0]) + 1 if len(hit) else len(x)", "    k = int(hit[0]) if len(hit) else len(x)"),
    "pe_not_normalised": ("    x = a_bar[qb, kb] / nb\n", "    x = a_bar[qb, kb]\n"),
    "pe_no_diagonal": ("    mask[np.arange(nb), np.arange(nb)] = True\n", ""),
    "attn_no_scale": ("    scale = 1.0 / math.sqrt(d)\n    out = {}", "    scale = 1.0\n    out = {}"),
    "attn_not_causal": ("        vis = keys[None, :] <= qpos[:, None]", "        vis = keys[None, :] >= 0"),
    "attn_v_misindexed": ("        out[qb] = (e @ v_g[keys]) / den", "        out[qb] = (e @ v_g[np.sort(keys)[::-1]]) / den"),
    "jsd_log2": ("        return float(np.sum(a[nz] * np.log(a[nz] / m[nz])))",
                 "        return float(np.sum(a[nz] * np.log2(a[nz] / m[nz])))"),
    "jsd_m_not_halved": ("    m = 0.5 * (p + q)\n", "    m = p + q\n"),
    "jsd_route_flipped": ("    return bool(d_js >= tau_jsd)", "    return bool(d_js < tau_jsd)"),
    "pooled_est_all_queries": ("    qbar = q_h[n - b:].mean(axis=0)", "    qbar = q_h.mean(axis=0)"),
    "pooled_est_no_scale": ("    s = (kbar @ qbar) / math.sqrt(d)", "    s = (kbar @ qbar)"),
    "flex_no_kmin": ("    k = min(max(len(kept), k_min_blocks), nb)", "    k = min(len(kept), nb)"),
    "flex_no_anchors": ("    sel = {0, nb - 1}.union(order[:k].tolist())", "    sel = set(order[:k].tolist())"),
    "median_with_anchors": ("        mu = float(np.median(p[1:nb - 1]))", "        mu = float(np.median(p))"),
    "band_wrong_side": ("        deltas = np.union1d(deltas, deltas + 1)", "        deltas = np.union1d(deltas, deltas - 1)"),
    "pe_row_scaled_by_nb": ("            k_r, o_r, c_r = gamma_cumsum(a_bar[r, : r + 1], gamma)",
                            "            k_r, o_r, c_r = gamma_cumsum(a_bar[r, : r + 1] / nb, gamma)"),
    "pe_row_no_diagonal": ("        mask[np.diag_indices(nb)] = True\n", ""),
    "pe_row_global_cut": ("            k_r, o_r, c_r = gamma_cumsum(a_bar[r, : r + 1], gamma)",
                          "            k_r, o_r, c_r = gamma_cumsum(a_bar[r, : r + 1], gamma * (r + 1) / nb)"),
    "bf16_decode_shift": ("    w = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)",
                          "    w = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(15)"),
}

CHECKS = [getattr(pins, n) for n in dir(pins) if n.startswith("check_")]

# Mistakes planted in copies of the layer driver, each to be caught by a driver pin.
DRIVER_SRC = open(driver.__file__).read()
DRIVER_MUTANTS = {
    "attn_k_head_mod": ("kv[(b, h // G)] = (co.bf16_to_f64(k_bits[b, h // G]),",
                        "kv[(b, h // G)] = (co.bf16_to_f64(k_bits[b, h % k_bits.shape[1]]),"),
    "attn_v_head_mod": ("co.bf16_to_f64(v_bits[b, h // G]))", "co.bf16_to_f64(v_bits[b, h % k_bits.shape[1]]))"),
    "attn_q_block_misread": ("q[qb * B:(qb + 1) * B] = co.bf16_to_f64(q_bits[b, h, qb * B:(qb + 1) * B])",
                             "q[qb * B:(qb + 1) * B] = co.bf16_to_f64(q_bits[b, h, 0:B])"),
    "attn_q_rows_ignored": ("q_blocks=[qb], q_rows=q_rows)[qb]", "q_blocks=[qb])[qb]"),
    "attn_q_rows_reversed": ("q_blocks=[qb], q_rows=q_rows)[qb]",
                             "q_blocks=[qb], q_rows=None if q_rows is None else list(q_rows)[::-1])[qb]"),
    "sel_head_mod": ("        k = co.bf16_to_f64(k_bits[b, h // G])\n        return bh, co.crisp_head(",
                     "        k = co.bf16_to_f64(k_bits[b, h % k_bits.shape[1]])\n        return bh, co.crisp_head("),
    "sel_force_ignored": ("force_vs=force_vs.get(bh), floor=floor", "force_vs=None, floor=floor"),
    "flex_head_mod": ("        k = co.bf16_to_f64(k_bits[b, h // G])\n        return bh, co.flex_head(",
                      "        k = co.bf16_to_f64(k_bits[b, h % k_bits.shape[1]])\n        return bh, co.flex_head("),
    "flex_force_ignored": ("                                force_vs=force_vs.get(bh))",
                           "                                force_vs=None)"),
}
DRIVER_CHECKS = [getattr(pins, n) for n in dir(pins) if n.startswith("dcheck_")]


def _load(name, old, new):
    assert SRC.count(old) == 1, f"mutation {name} does not match the oracle source exactly once"
    mod = types.ModuleType(f"oracle_mutant_{name}")
    exec(compile(SRC.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


def _bf16_pin(co):
    import numpy as np
    bits = np.array([0x3F80, 0xC000, 0x3E00], dtype=np.uint16)   # 1.0, -2.0, 0.125
    assert co.bf16_to_f64(bits).tolist() == [1.0, -2.0, 0.125]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    mod = _load(name, *MUTANTS[name])
    failed = []
    for chk in CHECKS + [_bf16_pin]:
        try:
            chk(mod)
        except AssertionError:
            failed.append(chk.__name__)
        except (ValueError, IndexError, FloatingPointError, ZeroDivisionError):
            failed.append(chk.__name__)
    assert failed, f"no pin catches mutant {name}"


def test_real_oracle_passes_bf16_pin():
    _bf16_pin(crisp_oracle)


def _load_driver(name, old, new):
    assert DRIVER_SRC.count(old) == 1, f"mutation {name} does not match the driver source exactly once"
    src = DRIVER_SRC.replace(old, new).replace("from . import crisp_oracle as co", "from oracle import crisp_oracle as co")
    mod = types.ModuleType(f"driver_mutant_{name}")
    exec(compile(src, f"<driver mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(DRIVER_MUTANTS))
def test_driver_mutant_is_caught(name):
    mod = _load_driver(name, *DRIVER_MUTANTS[name])
    failed = []
    for chk in DRIVER_CHECKS:
        try:
            chk(mod)
        except (AssertionError, ValueError, IndexError):
            failed.append(chk.__name__)
    assert failed, f"no driver pin catches mutant {name}"


def test_real_driver_passes_driver_pins():
    for chk in DRIVER_CHECKS:
        chk(driver)
