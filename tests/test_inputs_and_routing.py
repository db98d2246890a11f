"""The seeded input generator, and the oracle routing planted heads as designed (CPU)."""
import numpy as np
import pytest
import torch

from oracle import crisp_oracle as co
from oracle.driver import layer_selection
from prefill_inputs import (WORKLOADS, Shape, bf16_bits_to_f32, f32_to_bf16_bits,
                            head_roles, make_inputs, workload_inputs)


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        # exact halfway cases between two bf16 values
                        (np.arange(1, 2000, dtype=np.uint32) << 16 | 0x8000).view(np.float32)])
    ours = f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(bf16_bits_to_f32(ours), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_generator_deterministic_and_thread_independent():
    sh = Shape(2, 1024, 4, 2, 64)
    a = make_inputs(sh, seed=7, workers=1)
    b = make_inputs(sh, seed=7, workers=4)
    c = make_inputs(sh, seed=8, workers=4)
    for key in ("q", "k", "v"):
        assert a[key].dtype == np.uint16
        assert np.array_equal(a[key], b[key])
        assert not np.array_equal(a[key], c[key])
    assert a["q"].shape == (2, 4, 1024, 64) and a["k"].shape == (2, 2, 1024, 64)


@pytest.mark.parametrize("idx,n_pe,pe_heads", [
    (1, 1, [1]),
    (2, 16, [2, 3, 6, 7, 10, 11, 14, 15, 18, 19, 22, 23, 26, 27, 30, 31]),
    (3, 8, [3, 7, 11, 15, 19, 23, 27, 31]),
    (4, 3, [6, 13, 20]),
    (5, 8, [3, 7, 11, 15, 19, 23, 27, 31]),
])
def test_head_roles(idx, n_pe, pe_heads):
    wl = WORKLOADS[idx]
    roles = head_roles(wl.shape.h_q, wl.shape.h_kv, wl.vs_fraction)
    assert int((~roles).sum()) == n_pe
    assert np.nonzero(~roles)[0].tolist() == pe_heads


def test_tiny_workload_routes_as_planted():
    wl = WORKLOADS[1]
    inp = workload_inputs(wl)
    res = layer_selection(inp["q"], inp["k"], tau=wl.tau, alpha=1.0, gamma=wl.gamma)
    assert res[(0, 0)]["is_vs"] and res[(0, 0)]["c_struct"] >= wl.tau * (1 + 1e-3)
    assert not res[(0, 1)]["is_vs"] and res[(0, 1)]["c_struct"] < 0.1
    # the planted vertical keys' blocks are selected by the vertical direction
    vert_blocks = set((inp["planted"][0][0]["vert"] // 128).tolist())
    assert vert_blocks <= set(res[(0, 0)]["sel_v"].tolist())


@pytest.mark.parametrize("idx", [2, 3, 4, 5])
def test_reduced_length_workloads_route_as_planted(idx):
    """Each large workload's recipe at n = 8192: same heads and planting, with the
    number of planted vertical keys scaled to keep their density per token."""
    wl = WORKLOADS[idx]
    sh = Shape(1, 8192, wl.shape.h_q, wl.shape.h_kv, wl.shape.d)
    n_vert = max(1, round(wl.n_vert * sh.n / wl.shape.n))
    inp = make_inputs(sh, vs_fraction=wl.vs_fraction, sink_scale=wl.sink_scale,
                      n_vert=n_vert, slash=wl.slash, seed=wl.seed)
    res = layer_selection(inp["q"], inp["k"], tau=wl.tau, alpha=1.0, gamma=wl.gamma)
    G = sh.h_q // sh.h_kv
    for h in range(sh.h_q):
        r = res[(0, h)]
        assert r["is_vs"] == bool(inp["is_vs"][h]), (h, r["c_struct"])
        if r["is_vs"]:
            # most planted vertical keys' blocks are found (a planted key with a
            # strongly negative random logit offset can fall under the floor),
            # and the vertical set stays small
            vb = set((inp["planted"][0][h // G]["vert"] // 128).tolist())
            found = len(vb & set(r["sel_v"].tolist()))
            assert found >= 0.5 * len(vb), (h, found, len(vb))
            assert len(r["sel_v"]) <= len(vb) + 8
        else:
            tiles = sum(len(x) for x in r["rows"])
            assert tiles > 0.8 * sh.n_blocks * (sh.n_blocks + 1) / 2
