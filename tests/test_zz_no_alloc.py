"""crisp_route_noalloc (static device scratch, no allocation) against crisp_route.

Two calls in a row through the C-ABI, the second on a smaller layer, each
compared bit for bit with crisp_route on a caller workspace: the same kernels
run on the same inputs, so every output must be identical.
"""
import ctypes

import numpy as np
import pytest
import torch

import long_context_sparse_patsearch_amd as crisp
from parity import device_inputs
from prefill_inputs import Shape, make_inputs

pytestmark = pytest.mark.gpu


def _route_noalloc_abi(q, k, cfg):
    """crisp_route_noalloc called through ctypes with preallocated outputs."""
    sh = crisp.shape_of(q, k)
    bh, nb = sh.batch * sh.h_q, sh.n // 128
    out = dict(c_struct=torch.full((bh,), float("nan"), dtype=torch.float32, device=q.device),
               pattern=torch.full((bh,), -1, dtype=torch.int8, device=q.device),
               p_vert=torch.full((bh, nb), float("nan"), dtype=torch.float32, device=q.device),
               p_slash=torch.full((bh, nb), float("nan"), dtype=torch.float32, device=q.device))
    lib = crisp.load()
    st = lib.crisp_route_noalloc(ctypes.byref(sh), ctypes.byref(cfg), ctypes.c_void_p(q.data_ptr()),
                                 ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(out["c_struct"].data_ptr()),
                                 ctypes.c_void_p(out["pattern"].data_ptr()), ctypes.c_void_p(out["p_vert"].data_ptr()),
                                 ctypes.c_void_p(out["p_slash"].data_ptr()),
                                 ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, crisp.load().crisp_status_string(st)
    return out


def test_route_noalloc_matches_route_twice():
    cfg = crisp.config()
    for sh, seed in ((Shape(1, 65536, 8, 2, 128), 5), (Shape(2, 4096, 4, 2, 128), 6)):
        print(f"[noalloc] shape {sh}", flush=True)
        inp = make_inputs(sh, vs_fraction=0.5, sink_scale=3.0, n_vert=8, seed=seed)
        q, k, _ = device_inputs(inp)
        got = _route_noalloc_abi(q, k, cfg)
        torch.cuda.synchronize()
        ref = crisp.route(q, k, cfg)
        torch.cuda.synchronize()
        for key in ("c_struct", "pattern", "p_vert", "p_slash"):
            assert torch.equal(got[key], ref[key]), (sh, key)
        pattern = got["pattern"].cpu().numpy()
        assert 0 < int(pattern.sum()) < len(pattern), pattern   # both routes present
