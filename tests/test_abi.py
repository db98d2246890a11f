"""The C-ABI library on the CPU: it loads, exports every declared symbol, and
rejects bad arguments with the documented status before any HIP call."""
import ctypes
import os
import re

import pytest

import long_context_sparse_patsearch_amd as crisp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "crisp.h")

OK, NULL, SHAPE, PARAM, UNSUP, WS, CAP, HIP, ALIGN, SCRATCH = 0, -1, -2, -3, -4, -5, -6, -7, -8, -9
FAKE = 0x10000          # an aligned address that is never dereferenced: validation fails first


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", src, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(crisp.library_path()):
        from long_context_sparse_patsearch_amd.build import build
        build(verbose=False)
    return crisp.load()


def test_header_declares_the_method_calls():
    names = declared_functions()
    for f in ("crisp_route", "crisp_select", "crisp_sparse_attn", "dense_attn", "crisp_use_dense",
              "crisp_workspace_bytes", "crisp_max_blocks", "crisp_status_string", "crisp_last_error"):
        assert f in names


def test_library_exports_every_declared_symbol(lib):
    raw = ctypes.CDLL(crisp.library_path())
    for f in declared_functions():
        assert hasattr(raw, f), f"{f} declared in crisp.h but not exported"


def shape(batch=1, n=4096, h_q=2, h_kv=2, d=64):
    return crisp.Shape(batch, n, h_q, h_kv, d)


@pytest.mark.parametrize("sh,status", [
    (shape(), OK),
    (shape(n=4096 + 64), SHAPE), (shape(n=256), SHAPE), (shape(n=0), SHAPE), (shape(n=1 << 21), SHAPE),
    (shape(d=96), SHAPE), (shape(h_q=3, h_kv=2), SHAPE), (shape(h_kv=0), SHAPE), (shape(batch=-1), SHAPE),
    (shape(batch=0), OK), (shape(n=384), OK), (shape(n=1 << 20, h_q=8, h_kv=1, d=128), OK),
])
def test_shape_validation(lib, sh, status):
    n = ctypes.c_size_t(7)
    assert lib.crisp_workspace_bytes(ctypes.byref(sh), ctypes.byref(crisp.config()), 0, ctypes.byref(n)) == status


@pytest.mark.parametrize("kw,status", [
    (dict(), OK), (dict(block=64), UNSUP), (dict(k_min_tokens=100), PARAM), (dict(k_min_tokens=-128), PARAM),
    (dict(gamma=0.0), PARAM), (dict(gamma=1.5), PARAM), (dict(gamma=1.0), OK), (dict(alpha=-0.1), PARAM),
    (dict(alpha=0.0), OK), (dict(tau=float("nan")), PARAM), (dict(alpha=float("inf")), PARAM),
])
def test_cfg_validation(lib, kw, status):
    cfg = crisp.config(**kw)
    n = ctypes.c_size_t(0)
    assert lib.crisp_workspace_bytes(ctypes.byref(shape()), ctypes.byref(cfg), 1, ctypes.byref(n)) == status


def test_workspace_and_capacity_queries(lib):
    sh = shape(batch=2, n=4096, h_q=4, h_kv=2, d=128)
    cfg = crisp.config()
    sizes = [crisp.workspace_bytes(sh, cfg, c) for c in (0, 1, 2, 3)]
    assert all(x > 0 for x in sizes)
    nb = 4096 // 128
    # the selection workspace holds at least the pooled map of every head
    assert sizes[1] >= 2 * 4 * nb * (nb + 1) // 2 * 4
    assert crisp.max_blocks(sh) == 2 * 4 * nb * (nb + 1) // 2
    n = ctypes.c_size_t(0)
    assert lib.crisp_workspace_bytes(ctypes.byref(sh), ctypes.byref(cfg), 9, ctypes.byref(n)) == PARAM
    assert lib.crisp_workspace_bytes(ctypes.byref(sh), ctypes.byref(cfg), 0, None) == NULL
    assert crisp.workspace_bytes(shape(batch=0), cfg, 1) == 0


def test_dense_gate(lib):
    """Short inputs take the dense path: the threshold is the header's CRISP_DENSE_BELOW_TOKENS."""
    limit = int(re.search(r"#define\s+CRISP_DENSE_BELOW_TOKENS\s+(\d+)", open(HEADER).read()).group(1))
    # a whole number of blocks, and a length where both paths are plausible (the pages' own
    # GPU crossed over between 8K and 64K; the measured crossover here is lower)
    assert limit % 128 == 0 and 4096 < limit <= 65536
    for n, want in ((384, True), (4096, True), (limit - 128, True), (limit, False), (131072, False)):
        assert crisp.use_dense(shape(n=n)) is want, n
    flag = ctypes.c_int32(7)
    assert lib.crisp_use_dense(ctypes.byref(shape(n=4096 + 64)), ctypes.byref(flag)) == SHAPE
    assert lib.crisp_use_dense(ctypes.byref(shape()), None) == NULL
    assert lib.crisp_use_dense(None, ctypes.byref(flag)) == NULL


def _route(lib, sh, cfg, ptrs, ws_bytes):
    q, k, c, p, pv, ps, ws = ptrs
    return lib.crisp_route(ctypes.byref(sh), ctypes.byref(cfg), q, k, c, p, pv, ps, ws, ws_bytes, None)


def test_route_rejects_before_any_hip_call(lib):
    sh, cfg = shape(), crisp.config()
    need = crisp.workspace_bytes(sh, cfg, 0)
    good = [FAKE] * 7
    assert _route(lib, sh, cfg, [FAKE, None] + good[2:], need) == NULL
    assert _route(lib, sh, cfg, [FAKE + 8] + good[1:], need) == ALIGN
    assert _route(lib, sh, cfg, good, need - 1) == WS
    assert _route(lib, shape(n=100), cfg, good, need) == SHAPE
    assert _route(lib, sh, crisp.config(block=256), good, need) == UNSUP
    assert lib.crisp_route(None, ctypes.byref(cfg), *good, need, None) == NULL
    # an empty batch enqueues nothing, whatever the pointers
    assert _route(lib, shape(batch=0), cfg, [None] * 7, 0) == OK


def test_select_rejects_before_any_hip_call(lib):
    sh, cfg = shape(), crisp.config()
    need = crisp.workspace_bytes(sh, cfg, 1)
    cap = crisp.max_blocks(sh)

    def call(cap_, ws_bytes, mask=None, rp=FAKE):
        return lib.crisp_select(ctypes.byref(sh), ctypes.byref(cfg), FAKE, FAKE, FAKE, FAKE, FAKE, rp, FAKE,
                                cap_, mask, FAKE, ws_bytes, None)
    assert call(cap - 1, need) == CAP
    assert call(cap, need - 1) == WS
    assert call(cap, need, mask=FAKE + 4) == ALIGN
    assert call(cap, need, rp=None) == NULL


def test_flex_calls_reject_before_any_hip_call(lib):
    sh, cfg = shape(), crisp.config()
    need_r = crisp.workspace_bytes(sh, cfg, crisp.CALL_FLEX_ROUTE)
    need_s = crisp.workspace_bytes(sh, cfg, crisp.CALL_FLEX_SELECT)
    assert need_r == 1 * 2 * (4096 // 128) * 64 * 4          # pooled keys of every KV group, fp32
    assert need_s == crisp.workspace_bytes(sh, cfg, crisp.CALL_SELECT)

    def route(tau=0.1, ws_bytes=need_r, ptrs=None, sh_=sh):
        ptrs = ptrs or [FAKE] * 6
        return lib.flex_route(ctypes.byref(sh_), ctypes.byref(cfg), ctypes.c_float(tau), *ptrs, ws_bytes, None)
    for bad in (-0.1, float("nan"), float("inf")):
        assert route(tau=bad) == PARAM
    assert route(ws_bytes=need_r - 1) == WS
    assert route(ptrs=[FAKE, FAKE, None, FAKE, FAKE, FAKE]) == NULL
    assert route(ptrs=[FAKE, FAKE, FAKE + 4, FAKE, FAKE, FAKE]) == ALIGN
    assert route(sh_=shape(n=1000)) == SHAPE
    assert route(sh_=shape(batch=0), ptrs=[None] * 6, ws_bytes=0) == OK
    cap = crisp.max_blocks(sh)

    def select(cap_, ws_bytes, rp=FAKE):
        return lib.flex_select(ctypes.byref(sh), ctypes.byref(cfg), FAKE, FAKE, FAKE, FAKE, FAKE, rp, FAKE,
                               cap_, None, FAKE, ws_bytes, None)
    assert select(cap - 1, need_s) == CAP
    assert select(cap, need_s - 1) == WS
    assert select(cap, need_s, rp=None) == NULL


def test_select_variant_rejects_unknown_bits(lib):
    sh, cfg = shape(), crisp.config()
    need = crisp.workspace_bytes(sh, cfg, 1)
    cap = crisp.max_blocks(sh)

    def call(variant, cap_=cap):
        return lib.crisp_select_variant(ctypes.byref(sh), ctypes.byref(cfg), variant, FAKE, FAKE, FAKE, FAKE, FAKE,
                                        FAKE, FAKE, cap_, None, FAKE, need, None)
    assert call(8) == PARAM and call(-1) == PARAM
    assert call(crisp.VARIANT_MEDIAN_FLOOR | crisp.VARIANT_SLASH_BAND, cap_=cap - 1) == CAP
    assert call(crisp.VARIANT_PE_PER_ROW, cap_=cap - 1) == CAP


def test_attention_rejects_before_any_hip_call(lib):
    sh, cfg = shape(), crisp.config()
    need = crisp.workspace_bytes(sh, cfg, 2)
    dneed = crisp.workspace_bytes(sh, cfg, 3)
    assert need > 0 and dneed > 0

    def sp(ws, ws_bytes, dtype=0, col=FAKE, cap=10):
        return lib.crisp_sparse_attn(ctypes.byref(sh), ctypes.byref(cfg), FAKE, FAKE, FAKE, FAKE, col, cap, FAKE,
                                     dtype, ws, ws_bytes, None)
    assert sp(FAKE, need, dtype=2) == PARAM
    assert sp(FAKE, need, col=None) == NULL
    assert sp(FAKE, need, cap=-1) == PARAM
    assert sp(None, need) == NULL
    assert sp(FAKE, need - 1) == WS
    assert sp(FAKE + 4, need) == ALIGN

    def dn(q=FAKE, out=FAKE, ws=FAKE, ws_bytes=dneed, s=sh):
        return lib.dense_attn(ctypes.byref(s), q, FAKE, FAKE, out, 0, ws, ws_bytes, None)
    assert dn(out=FAKE + 2) == ALIGN
    assert dn(q=None) == NULL
    assert dn(ws=None) == NULL
    assert dn(ws_bytes=dneed - 1) == WS
    assert dn(s=shape(d=32)) == SHAPE


def test_status_strings(lib):
    for st in (OK, NULL, SHAPE, PARAM, UNSUP, WS, CAP, HIP, ALIGN, 123):
        assert lib.crisp_status_string(st)
    assert lib.crisp_last_error() == b""


def test_binding_raises_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(crisp, "_lib", None)
    monkeypatch.setattr(crisp, "_LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(crisp.CrispError):
        crisp.load()


def test_mfma_probe_rejects_before_any_hip_call(lib):
    flop = ctypes.c_double(0.0)
    assert lib.crisp_mfma_probe(None, FAKE, 10, ctypes.byref(flop), None) == NULL
    assert lib.crisp_mfma_probe(FAKE, None, 10, ctypes.byref(flop), None) == NULL
    assert lib.crisp_mfma_probe(FAKE, FAKE, 10, None, None) == NULL
    assert lib.crisp_mfma_probe(FAKE + 8, FAKE, 10, ctypes.byref(flop), None) == ALIGN
    assert lib.crisp_mfma_probe(FAKE, FAKE, 0, ctypes.byref(flop), None) == PARAM
    assert lib.crisp_mfma_probe(FAKE, FAKE, 10 ** 7 + 1, ctypes.byref(flop), None) == PARAM


def test_route_noalloc_validates_before_any_hip_call(lib):
    """crisp_route_noalloc: bad arguments and shapes whose routing workspace exceeds the
    static scratch are rejected on the host (these calls never reach the GPU)."""
    P = ctypes.c_void_p
    cfg = crisp.config()
    args = [P(FAKE)] * 6 + [P(0)]
    sh = shape(n=4096, h_q=2, h_kv=2, d=128)
    assert lib.crisp_route_noalloc(ctypes.byref(sh), ctypes.byref(cfg), P(0), *args[1:]) == NULL
    assert lib.crisp_route_noalloc(ctypes.byref(sh), ctypes.byref(cfg), P(FAKE + 4), *args[1:]) == ALIGN
    assert lib.crisp_route_noalloc(ctypes.byref(shape(n=4096 + 64)), ctypes.byref(cfg), *args) == SHAPE
    assert lib.crisp_route_noalloc(ctypes.byref(shape(batch=0)), ctypes.byref(cfg), *args) == OK
    need = ctypes.c_size_t(0)
    for big in (shape(n=524288, h_q=32, h_kv=8, d=128), shape(n=262144, h_q=28, h_kv=4, d=128),
                shape(batch=1, n=131072, h_q=64, h_kv=8, d=128)):
        assert lib.crisp_workspace_bytes(ctypes.byref(big), ctypes.byref(cfg), 0, ctypes.byref(need)) == OK
        assert need.value > 64 << 20
        assert lib.crisp_route_noalloc(ctypes.byref(big), ctypes.byref(cfg), *args) == SCRATCH
    # up to 32 heads at 131072 tokens fit
    for fits in (shape(n=131072, h_q=32, h_kv=8, d=128), shape(n=32768, h_q=32, h_kv=8, d=128),
                 shape(n=4096, h_q=2, h_kv=2, d=64)):
        assert lib.crisp_workspace_bytes(ctypes.byref(fits), ctypes.byref(cfg), 0, ctypes.byref(need)) == OK
        assert need.value <= 64 << 20, need.value
    assert lib.crisp_status_string(SCRATCH).decode().startswith("shape needs more scratch")
