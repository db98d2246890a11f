"""CRISP sparse-attention prefill on MI355X: Python binding of libcrisp.

Argument marshalling only.  Every step runs in the HIP kernels of
``libcrisp.so``; torch supplies device memory and the current stream.  There
is no fallback: if the library is missing, ``CrispError`` is raised.

    import long_context_sparse_patsearch_amd as crisp
    cfg = crisp.config(alpha=1.0)
    r = crisp.route(q, k, cfg)              # pattern, c_struct, p_vert, p_slash
    s = crisp.select(q, k, r, cfg)          # block CSR (row_ptr, col_idx)
    o = crisp.sparse_attn(q, k, v, s, cfg)  # A(Q, K, V, S)
    o = crisp.dense_attn(q, k, v)           # dense causal baseline

q: [batch, h_q, n, d] and k, v: [batch, h_kv, n, d] torch.bfloat16 CUDA
tensors, contiguous.
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["CrispError", "config", "shape_of", "workspace_bytes", "max_blocks", "use_dense", "route",
           "route_noalloc", "select",
           "sparse_attn", "dense_attn", "prefill", "flex_route", "flex_select", "flex_prefill", "library_path",
           "load"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libcrisp.so")
_lib = None

CALL_ROUTE, CALL_SELECT, CALL_ATTN, CALL_DENSE, CALL_FLEX_ROUTE, CALL_FLEX_SELECT = 0, 1, 2, 3, 4, 5
VARIANT_MEDIAN_FLOOR, VARIANT_SLASH_BAND, VARIANT_PE_PER_ROW = 1, 2, 4
OUT_F32, OUT_BF16 = 0, 1


class CrispError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"crisp status {status}: {msg}")
        self.status = status


class Shape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n", ctypes.c_int32), ("h_q", ctypes.c_int32),
                ("h_kv", ctypes.c_int32), ("d", ctypes.c_int32)]


class Cfg(ctypes.Structure):
    _fields_ = [("block", ctypes.c_int32), ("last_q", ctypes.c_int32), ("w_sink", ctypes.c_int32),
                ("w_local", ctypes.c_int32), ("k_min_tokens", ctypes.c_int32), ("tau", ctypes.c_float),
                ("alpha", ctypes.c_float), ("gamma", ctypes.c_float)]


def library_path() -> str:
    return _LIB_PATH


def load():
    """Load libcrisp.so (once).  Raises CrispError if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise CrispError(-100, f"{_LIB_PATH} is missing: build it with "
                               "`python -m long_context_sparse_patsearch_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    P, I, I64, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    ps, pc = ctypes.POINTER(Shape), ctypes.POINTER(Cfg)
    lib.crisp_workspace_bytes.argtypes = [ps, pc, I, ctypes.POINTER(SZ)]
    lib.crisp_max_blocks.argtypes = [ps, ctypes.POINTER(I64)]
    lib.crisp_use_dense.argtypes = [ps, ctypes.POINTER(ctypes.c_int32)]
    lib.crisp_route.argtypes = [ps, pc, P, P, P, P, P, P, P, SZ, P]
    lib.crisp_route_noalloc.argtypes = [ps, pc, P, P, P, P, P, P, P]
    lib.crisp_select.argtypes = [ps, pc, P, P, P, P, P, P, P, I64, P, P, SZ, P]
    lib.crisp_sparse_attn.argtypes = [ps, pc, P, P, P, P, P, I64, P, I, P, SZ, P]
    lib.dense_attn.argtypes = [ps, P, P, P, P, I, P, SZ, P]
    lib.flex_route.argtypes = [ps, pc, ctypes.c_float, P, P, P, P, P, P, SZ, P]
    lib.flex_select.argtypes = [ps, pc, P, P, P, P, P, P, P, I64, P, P, SZ, P]
    lib.crisp_select_variant.argtypes = [ps, pc, I, P, P, P, P, P, P, P, I64, P, P, SZ, P]
    lib.crisp_mfma_probe.argtypes = [P, P, I, ctypes.POINTER(ctypes.c_double), P]
    lib.crisp_status_string.argtypes = [I]
    lib.crisp_status_string.restype = ctypes.c_char_p
    lib.crisp_last_error.restype = ctypes.c_char_p
    for f in ("crisp_workspace_bytes", "crisp_max_blocks", "crisp_use_dense", "crisp_route", "crisp_route_noalloc",
              "crisp_select",
              "crisp_sparse_attn", "dense_attn", "flex_route", "flex_select", "crisp_select_variant",
              "crisp_mfma_probe"):
        getattr(lib, f).restype = I
    _lib = lib
    return lib


def _check(st: int):
    if st != 0:
        lib = load()
        msg = lib.crisp_status_string(st).decode()
        if st == -7:
            msg += ": " + lib.crisp_last_error().decode()
        raise CrispError(st, msg)


def config(tau: float = 0.2, alpha: float = 1.0, gamma: float = 0.95, k_min_tokens: int = 1024,
           block: int = 128) -> Cfg:
    """Method settings; defaults are the pages' tau, alpha (accuracy setting), gamma and k_min."""
    return Cfg(block, block, block, block, k_min_tokens, tau, alpha, gamma)


def shape_of(q, k) -> Shape:
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q, k must be [batch, heads, n, d]")
    b, h, n, d = q.shape
    return Shape(b, n, h, k.shape[1], d)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(stream=None):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _check_qkv(q, k, v=None):
    import torch
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t is None:
            continue
        if not t.is_cuda or t.dtype != torch.bfloat16 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous bfloat16 CUDA tensor")
    if k.shape[0] != q.shape[0] or k.shape[2:] != q.shape[2:] or (v is not None and v.shape != k.shape):
        raise ValueError("q [b,h_q,n,d], k and v [b,h_kv,n,d] disagree")


def workspace_bytes(shape: Shape, cfg: Cfg, call: int) -> int:
    out = ctypes.c_size_t(0)
    _check(load().crisp_workspace_bytes(ctypes.byref(shape), ctypes.byref(cfg), call, ctypes.byref(out)))
    return out.value


def max_blocks(shape: Shape) -> int:
    out = ctypes.c_int64(0)
    _check(load().crisp_max_blocks(ctypes.byref(shape), ctypes.byref(out)))
    return out.value


def use_dense(shape: Shape) -> bool:
    """True when a prefill of this shape should run dense attention (short inputs)."""
    out = ctypes.c_int32(0)
    _check(load().crisp_use_dense(ctypes.byref(shape), ctypes.byref(out)))
    return bool(out.value)


def _workspace(nbytes, device, ws=None):
    import torch
    if ws is not None and ws.numel() >= nbytes:
        return ws
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def route(q, k, cfg: Cfg | None = None, out: dict | None = None, ws=None, stream=None) -> dict:
    """PatSearch: structural mass, VS/PE pattern and the proxy's block scores."""
    import torch
    cfg = cfg or config()
    _check_qkv(q, k)
    sh = shape_of(q, k)
    bh, nb = sh.batch * sh.h_q, sh.n // 128
    dev = q.device
    out = out or dict(c_struct=torch.empty(bh, dtype=torch.float32, device=dev),
                      pattern=torch.empty(bh, dtype=torch.int8, device=dev),
                      p_vert=torch.empty(bh, nb, dtype=torch.float32, device=dev),
                      p_slash=torch.empty(bh, nb, dtype=torch.float32, device=dev))
    nws = workspace_bytes(sh, cfg, CALL_ROUTE)
    ws = _workspace(nws, dev, ws)
    _check(load().crisp_route(ctypes.byref(sh), ctypes.byref(cfg), _ptr(q), _ptr(k), _ptr(out["c_struct"]),
                              _ptr(out["pattern"]), _ptr(out["p_vert"]), _ptr(out["p_slash"]), _ptr(ws),
                              nws, _stream(stream)))
    return out


def route_noalloc(q, k, cfg: Cfg | None = None, out: dict | None = None, stream=None) -> dict:
    """route() on the library's static device scratch (crisp_route_noalloc): no
    workspace is allocated; pass ``out`` to allocate nothing at all."""
    import torch
    cfg = cfg or config()
    _check_qkv(q, k)
    sh = shape_of(q, k)
    bh, nb = sh.batch * sh.h_q, sh.n // 128
    dev = q.device
    out = out or dict(c_struct=torch.empty(bh, dtype=torch.float32, device=dev),
                      pattern=torch.empty(bh, dtype=torch.int8, device=dev),
                      p_vert=torch.empty(bh, nb, dtype=torch.float32, device=dev),
                      p_slash=torch.empty(bh, nb, dtype=torch.float32, device=dev))
    _check(load().crisp_route_noalloc(ctypes.byref(sh), ctypes.byref(cfg), _ptr(q), _ptr(k), _ptr(out["c_struct"]),
                                      _ptr(out["pattern"]), _ptr(out["p_vert"]), _ptr(out["p_slash"]),
                                      _stream(stream)))
    return out


def select(q, k, routed: dict, cfg: Cfg | None = None, out: dict | None = None, ws=None,
           with_mask: bool = False, stream=None, _flex: bool = False, variant: int = 0) -> dict:
    """VSIndex / PEIndex: the selected block set as a CSR over (batch, head, query block).

    ``variant``: bits VARIANT_MEDIAN_FLOOR / VARIANT_SLASH_BAND / VARIANT_PE_PER_ROW (crisp_select_variant)."""
    import torch
    cfg = cfg or config()
    _check_qkv(q, k)
    sh = shape_of(q, k)
    bh, nb = sh.batch * sh.h_q, sh.n // 128
    dev = q.device
    cap = max_blocks(sh)
    if out is None:
        out = dict(row_ptr=torch.empty(bh * nb + 1, dtype=torch.int64, device=dev),
                   col_idx=torch.empty(max(cap, 1), dtype=torch.int32, device=dev))
        if with_mask:
            out["sel_mask"] = torch.empty(bh, 2, nb, dtype=torch.uint8, device=dev)
    nws = workspace_bytes(sh, cfg, CALL_FLEX_SELECT if _flex else CALL_SELECT)
    ws = _workspace(nws, dev, ws)
    if variant:
        lib = load()
        fn = lambda *a: lib.crisp_select_variant(a[0], a[1], variant, *a[2:])   # noqa: E731
    else:
        fn = load().flex_select if _flex else load().crisp_select
    _check(fn(ctypes.byref(sh), ctypes.byref(cfg), _ptr(q), _ptr(k), _ptr(routed["pattern"]),
                               _ptr(routed["p_vert"]), _ptr(routed["p_slash"]), _ptr(out["row_ptr"]),
                               _ptr(out["col_idx"]), out["col_idx"].numel(), _ptr(out.get("sel_mask")),
                               _ptr(ws), nws, _stream(stream)))
    return out


def flex_route(q, k, routed: dict, tau_jsd: float = 0.1, cfg: Cfg | None = None, out: dict | None = None, ws=None,
               stream=None) -> dict:
    """FlexPrefill's router: D_JS between the proxy's block distribution (routed['p_vert'],
    from route()) and the pooled estimate; VS iff D_JS >= tau_jsd.  Returns jsd, pattern and
    the p_vert / p_slash it was given (the input of flex_select)."""
    import torch
    cfg = cfg or config()
    _check_qkv(q, k)
    sh = shape_of(q, k)
    bh = sh.batch * sh.h_q
    dev = q.device
    out = out or dict(jsd=torch.empty(bh, dtype=torch.float32, device=dev),
                      pattern=torch.empty(bh, dtype=torch.int8, device=dev))
    nws = workspace_bytes(sh, cfg, CALL_FLEX_ROUTE)
    ws = _workspace(nws, dev, ws)
    _check(load().flex_route(ctypes.byref(sh), ctypes.byref(cfg), ctypes.c_float(tau_jsd), _ptr(q), _ptr(k),
                             _ptr(routed["p_vert"]), _ptr(out["jsd"]), _ptr(out["pattern"]), _ptr(ws), nws,
                             _stream(stream)))
    return dict(out, p_vert=routed["p_vert"], p_slash=routed["p_slash"])


def flex_select(q, k, froute: dict, cfg: Cfg | None = None, out: dict | None = None, ws=None,
                with_mask: bool = False, stream=None) -> dict:
    """FlexPrefill's index selection (gamma-cumsum VS budget, the same PEIndex) as a block CSR."""
    return select(q, k, froute, cfg, out=out, ws=ws, with_mask=with_mask, stream=stream, _flex=True)


def sparse_attn(q, k, v, sel: dict, cfg: Cfg | None = None, out=None, out_dtype=None, ws=None,
                stream=None):
    """Exact causal attention over the selected blocks."""
    import torch
    cfg = cfg or config()
    _check_qkv(q, k, v)
    sh = shape_of(q, k)
    out_dtype = out_dtype or torch.float32
    code = OUT_BF16 if out_dtype == torch.bfloat16 else OUT_F32
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    nws = workspace_bytes(sh, cfg, CALL_ATTN)
    ws = _workspace(nws, q.device, ws)
    _check(load().crisp_sparse_attn(ctypes.byref(sh), ctypes.byref(cfg), _ptr(q), _ptr(k), _ptr(v),
                                    _ptr(sel["row_ptr"]), _ptr(sel["col_idx"]), sel["col_idx"].numel(),
                                    _ptr(out), code, _ptr(ws), nws, _stream(stream)))
    return out


def dense_attn(q, k, v, out=None, out_dtype=None, ws=None, stream=None):
    """Exact causal attention over every block (the dense baseline)."""
    import torch
    _check_qkv(q, k, v)
    sh = shape_of(q, k)
    out_dtype = out_dtype or torch.float32
    code = OUT_BF16 if out_dtype == torch.bfloat16 else OUT_F32
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    nws = workspace_bytes(sh, config(), CALL_DENSE)
    ws = _workspace(nws, q.device, ws)
    _check(load().dense_attn(ctypes.byref(sh), _ptr(q), _ptr(k), _ptr(v), _ptr(out), code, _ptr(ws), nws,
                             _stream(stream)))
    return out


PROBE_OPERAND_BYTES, PROBE_SINK_FLOATS = 65536, 4096


def mfma_probe(operands, iters: int = 20000, sink=None, stream=None) -> float:
    """Launch the sustained-MFMA-rate probe (crisp_mfma_probe) on ``operands``, a
    device tensor of PROBE_OPERAND_BYTES bytes of bf16 values; returns the
    launch's FLOP.  The caller times the launch on ``stream``."""
    import torch
    if operands.device.type != "cuda" or operands.numel() * operands.element_size() != PROBE_OPERAND_BYTES:
        raise CrispError(-3, "operands must be a device tensor of PROBE_OPERAND_BYTES bytes")
    if sink is None:
        sink = torch.empty(PROBE_SINK_FLOATS, dtype=torch.float32, device=operands.device)
    flop = ctypes.c_double(0.0)
    _check(load().crisp_mfma_probe(_ptr(operands), _ptr(sink), int(iters), ctypes.byref(flop), _stream(stream)))
    return flop.value


def prefill(q, k, v, cfg: Cfg | None = None, out_dtype=None, stream=None, gate: bool = True) -> dict:
    """The whole method on one layer: route, select, sparse attention.

    With gate=True, inputs shorter than the library's crossover length
    (crisp_use_dense) run dense attention instead; 'path' says which ran."""
    cfg = cfg or config()
    _check_qkv(q, k, v)
    if gate and use_dense(shape_of(q, k)):
        return dict(route=None, select=None, out=dense_attn(q, k, v, out_dtype=out_dtype, stream=stream),
                    path="dense")
    r = route(q, k, cfg, stream=stream)
    s = select(q, k, r, cfg, stream=stream)
    o = sparse_attn(q, k, v, s, cfg, out_dtype=out_dtype, stream=stream)
    return dict(route=r, select=s, out=o, path="sparse")


def flex_prefill(q, k, v, cfg: Cfg | None = None, tau_jsd: float = 0.1, out_dtype=None, stream=None) -> dict:
    """The FlexPrefill baseline on one layer: proxy, JSD routing, gamma-cumsum VS / PE selection,
    the same sparse attention."""
    cfg = cfg or config()
    r = route(q, k, cfg, stream=stream)
    f = flex_route(q, k, r, tau_jsd, cfg, stream=stream)
    s = flex_select(q, k, f, cfg, stream=stream)
    o = sparse_attn(q, k, v, s, cfg, out_dtype=out_dtype, stream=stream)
    return dict(route=r, flex_route=f, select=s, out=o)
