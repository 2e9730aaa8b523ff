"""Python binding of libmoe_rocm.so, the routed MoE expert layer for MI355X.

Argument marshalling only: every step runs in the library's HIP kernels.  The
binding allocates output tensors with torch on the current device, passes raw
pointers and torch's current HIP stream, and raises on any non-zero status.
There is no CPU fallback: if the library is missing, loading fails loudly.

bf16 tensors are torch.bfloat16 (the library reads them as 16-bit patterns);
MXFP8 data and scales are torch.uint8.  Expert weights are stored
output-major: w_gate/w_up [E, H, D], w_down [E, D, H], w_r [E, D].
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np
from dataclasses import dataclass
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_rocm.so")

MOE_OK = 0
MOE_BF16, MOE_MXFP8 = 0, 1
MOE_EPI_NONE, MOE_EPI_SWIGLU, MOE_EPI_SWIGLU_BWD = 0, 1, 2
MOE_OP_ROUTE, MOE_OP_GEMM, MOE_OP_LAYER_FWD, MOE_OP_LAYER_BWD, MOE_OP_ROUTER = 1, 2, 3, 4, 5
MOE_OP_LAYER_BWD_MXFP8 = 6
MOE_OP_LAYER_BWD_MXFP8_NATIVE = 7
MOE_SCHED_STAGED, MOE_SCHED_READY, MOE_SCHED_SINGLE = 0, 1, 2

_vp = C.c_void_p
_i64 = C.c_int64
_i32 = C.c_int32


class Dims(C.Structure):
    _fields_ = [("N", _i64), ("D", _i64), ("E", _i64), ("K", _i64), ("H", _i64),
                ("align", _i32), ("renorm", _i32), ("n_group", _i32), ("topk_group", _i32),
                ("n_shared", _i32), ("reserved", _i32)]


class GemmFwdArgs(C.Structure):
    _fields_ = [("dtype", _i32), ("epilogue", _i32), ("E", _i64), ("rows_cap", _i64),
                ("k_dim", _i64), ("n_dim", _i64), ("offsets", _vp), ("a", _vp), ("a_scales", _vp),
                ("b0", _vp), ("b0_scales", _vp), ("b1", _vp), ("b1_scales", _vp), ("c0", _vp),
                ("c1", _vp), ("act", _vp), ("act_q", _vp), ("act_scales", _vp)]


class GemmBwdArgs(C.Structure):
    _fields_ = [("dtype", _i32), ("epilogue", _i32), ("E", _i64), ("rows_cap", _i64),
                ("k_dim", _i64), ("n_dim", _i64), ("offsets", _vp), ("a", _vp), ("b0", _vp),
                ("b1", _vp), ("dc0", _vp), ("dc1", _vp), ("da", _vp), ("g", _vp), ("u", _vp),
                ("dg", _vp), ("du", _vp), ("db0", _vp), ("db1", _vp)]


class LayerArgs(C.Structure):
    _fields_ = [("dims", Dims), ("dtype", _i32), ("sched", _i32), ("x", _vp), ("w_r", _vp),
                ("bias", _vp), ("drop", _vp), ("w_gate", _vp), ("w_up", _vp), ("w_down", _vp),
                ("wg_q", _vp), ("wg_s", _vp), ("wu_q", _vp), ("wu_s", _vp), ("wd_q", _vp),
                ("wd_s", _vp), ("aux_alpha", C.c_float), ("wdt_q", _vp), ("wdt_s", _vp), ("wgut_q", _vp),
                ("wgut_s", _vp), ("ready_test_polls", _i32), ("mx_wgrad", _i32)]


class LayerSaved(C.Structure):
    _fields_ = [(n, _vp) for n in ("logits", "topk_idx", "topk_prob", "counts", "offsets",
                                   "dst_rows", "row_route", "xd", "xd_q", "xd_s", "g", "u", "h",
                                   "h_q", "h_s", "y", "aux", "status")]

# moe_layer_saved fields in order, with their element type and shape
# (rows_cap rc, Ex = E + n_shared experts) as moe_saved_carve lays them out
_SAVED_FIELDS = ("logits", "topk_idx", "topk_prob", "counts", "offsets", "dst_rows", "row_route", "xd",
                 "xd_q", "xd_s", "g", "u", "h", "h_q", "h_s", "y", "aux", "status")
MOE_STATUS_WAIT_EXPIRED, MOE_STATUS_NO_FINITE_LOGIT = 1, 2
MOE_NOALLOC_SCRATCH_BYTES = 64 << 20


class LayerGrads(C.Structure):
    _fields_ = [(n, _vp) for n in ("dx", "dprob", "dw_gate", "dw_up", "dw_down", "dw_r", "db_r", "dlogits")] + \
               [("d_aux", C.c_float)]


EXPORTS = {
    "moe_rows_cap": (_i64, [C.POINTER(Dims)]),
    "moe_workspace_size": (C.c_size_t, [C.c_int, C.POINTER(Dims)]),
    "moe_status_string": (C.c_char_p, [C.c_int]),
    "moe_last_hip_error": (C.c_int, []),
    "moe_router_logits": (C.c_int, [_vp, _vp, _vp, C.POINTER(Dims), _vp, _vp, C.c_size_t, _vp]),
    "moe_route": (C.c_int, [_vp, _vp, C.POINTER(Dims), _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                            C.c_size_t, _vp]),
    "moe_dispatch": (C.c_int, [_vp, _vp, _vp, _vp, _vp, C.POINTER(Dims), C.c_int, _vp, _vp, _vp]),
    "moe_combine": (C.c_int, [_vp, _vp, _vp, C.POINTER(Dims), _vp, _vp]),
    "moe_combine_bwd": (C.c_int, [_vp, _vp, _vp, _vp, C.POINTER(Dims), _vp, _vp, _vp]),
    "moe_quantize_mxfp8": (C.c_int, [_vp, _i64, _i64, _vp, _vp, _vp]),
    "moe_quantize_mxfp8_cols": (C.c_int, [_vp, _i64, _i64, _i64, _i64, _i64, _vp, _vp, _vp]),
    "moe_swiglu": (C.c_int, [_vp, _vp, _i64, _i64, C.c_int, _vp, _vp, _vp, _vp]),
    "moe_grouped_gemm_fwd": (C.c_int, [C.POINTER(GemmFwdArgs), _vp, C.c_size_t, _vp]),
    "moe_grouped_gemm_bwd": (C.c_int, [C.POINTER(GemmBwdArgs), _vp, C.c_size_t, _vp]),
    "moe_saved_size": (C.c_size_t, [C.POINTER(Dims), C.c_int]),
    "moe_saved_carve": (C.c_int, [C.POINTER(Dims), C.c_int, _vp, C.c_size_t, C.POINTER(LayerSaved)]),
    "moe_layer_fwd": (C.c_int, [C.POINTER(LayerArgs), C.POINTER(LayerSaved), _vp, _vp, C.c_size_t, _vp]),
    "moe_layer_fwd_noalloc": (C.c_int, [C.POINTER(LayerArgs), C.POINTER(LayerSaved), _vp, _vp]),
    "moe_layer_bwd": (C.c_int, [C.POINTER(LayerArgs), C.POINTER(LayerSaved), _vp,
                                C.POINTER(LayerGrads), _vp, C.c_size_t, _vp]),
}

_lib = None


def load(path: str = LIB_PATH) -> C.CDLL:
    """Load the library (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with "
                               "`python -m mixture_experts_expert_router_amd.build`")
        lib = C.CDLL(path)
        for name, (res, args) in EXPORTS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


class MoeError(RuntimeError):
    pass


def _check(status: int, what: str):
    if status != MOE_OK:
        lib = load()
        msg = lib.moe_status_string(status).decode()
        extra = f" (hipError {lib.moe_last_hip_error()})" if status == -7 else ""
        raise MoeError(f"{what}: {msg} [{status}]{extra}")


def _torch():
    import torch
    return torch


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream():
    return _torch().cuda.current_stream().cuda_stream


def dims(N, D, E, K, H=0, align=1, renorm=0, n_group=0, topk_group=0, n_shared=0) -> Dims:
    return Dims(int(N), int(D), int(E), int(K), int(H), int(align), int(renorm), int(n_group), int(topk_group),
                int(n_shared), 0)


def rows_cap(d: Dims) -> int:
    return load().moe_rows_cap(C.byref(d))


def workspace(op: int, d: Dims, device=None):
    torch = _torch()
    n = load().moe_workspace_size(op, C.byref(d))
    return torch.empty(max(int(n), 256), dtype=torch.uint8, device=device or "cuda")


# ---- single steps --------------------------------------------------------------


def router_logits(x, w_r, bias=None, out=None, ws=None):
    torch = _torch()
    N, D = x.shape
    E = w_r.shape[0]
    d = dims(N, D, E, 1)
    out = out if out is not None else torch.empty((N, E), dtype=torch.float32, device=x.device)
    ws = ws if ws is not None else workspace(MOE_OP_ROUTER, d, x.device)
    _check(load().moe_router_logits(_ptr(x), _ptr(w_r), _ptr(bias), C.byref(d), _ptr(out), _ptr(ws),
                                    ws.numel(), _stream()), "moe_router_logits")
    return out


def route(logits, K, drop=None, renorm=0, align=1, ws=None, n_group=0, topk_group=0):
    """Returns dict(topk_idx, topk_prob, counts, offsets, dst_rows, row_route).
    n_group > 1: group-limited top-K keeping topk_group groups."""
    torch = _torch()
    N, E = logits.shape
    d = dims(N, 8, E, K, align=align, renorm=renorm, n_group=n_group, topk_group=topk_group)
    dev = logits.device
    rc = rows_cap(d)
    o = dict(topk_idx=torch.empty((N, K), dtype=torch.int32, device=dev),
             topk_prob=torch.empty((N, K), dtype=torch.float32, device=dev),
             counts=torch.empty(E, dtype=torch.int32, device=dev),
             offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
             dst_rows=torch.empty((N, K), dtype=torch.int32, device=dev),
             row_route=torch.empty(rc, dtype=torch.int32, device=dev))
    ws = ws if ws is not None else workspace(MOE_OP_ROUTE, d, dev)
    _check(load().moe_route(_ptr(logits), _ptr(drop), C.byref(d), _ptr(o["topk_idx"]),
                            _ptr(o["topk_prob"]), _ptr(o["counts"]), _ptr(o["offsets"]),
                            _ptr(o["dst_rows"]), _ptr(o["row_route"]), _ptr(ws), ws.numel(),
                            _stream()), "moe_route")
    return o


def dispatch(x, dst_rows, E, weight=None, counts=None, offsets=None, align=1, mxfp8=False,
             out=None, out_scales=None):
    """bf16: returns xd [rows_cap, D]; MXFP8: returns (q [rows_cap, D] u8, s [rows_cap, D/32] u8)."""
    torch = _torch()
    N, D = x.shape
    K = dst_rows.shape[1]
    d = dims(N, D, E, K, align=align)
    rc = rows_cap(d)
    if mxfp8:
        q = out if out is not None else torch.empty((rc, D), dtype=torch.uint8, device=x.device)
        s = out_scales if out_scales is not None else torch.empty((rc, D // 32), dtype=torch.uint8, device=x.device)
        _check(load().moe_dispatch(_ptr(x), _ptr(dst_rows), _ptr(weight), _ptr(counts), _ptr(offsets),
                                   C.byref(d), MOE_MXFP8, _ptr(q), _ptr(s), _stream()), "moe_dispatch")
        return q, s
    xd = out if out is not None else torch.empty((rc, D), dtype=torch.bfloat16, device=x.device)
    _check(load().moe_dispatch(_ptr(x), _ptr(dst_rows), _ptr(weight), _ptr(counts), _ptr(offsets),
                               C.byref(d), MOE_BF16, _ptr(xd), None, _stream()), "moe_dispatch")
    return xd


def combine(y, dst_rows, weight=None, E=None, out=None):
    torch = _torch()
    N, K = dst_rows.shape
    D = y.shape[1]
    d = dims(N, D, E or max(K, 1), K)
    out = out if out is not None else torch.empty((N, D), dtype=torch.bfloat16, device=y.device)
    _check(load().moe_combine(_ptr(y), _ptr(dst_rows), _ptr(weight), C.byref(d), _ptr(out), _stream()),
           "moe_combine")
    return out


def combine_bwd(dout, dst_rows, weight, y, rows_cap_, E=None, with_dprob=True, dyd=None):
    torch = _torch()
    N, D = dout.shape
    K = dst_rows.shape[1]
    d = dims(N, D, E or max(K, 1), K)
    dyd = dyd if dyd is not None else torch.empty((rows_cap_, D), dtype=torch.bfloat16, device=dout.device)
    dprob = torch.empty((N, K), dtype=torch.float32, device=dout.device) if with_dprob else None
    _check(load().moe_combine_bwd(_ptr(dout), _ptr(dst_rows), _ptr(weight), _ptr(y), C.byref(d),
                                  _ptr(dyd), _ptr(dprob), _stream()), "moe_combine_bwd")
    return dyd, dprob


def quantize_mxfp8(src):
    torch = _torch()
    rows, cols = src.shape
    q = torch.empty((rows, cols), dtype=torch.uint8, device=src.device)
    s = torch.empty((rows, cols // 32), dtype=torch.uint8, device=src.device)
    _check(load().moe_quantize_mxfp8(_ptr(src), rows, cols, _ptr(q), _ptr(s), _stream()),
           "moe_quantize_mxfp8")
    return q, s


def swiglu(g, u, mxfp8=False):
    torch = _torch()
    rows, n = g.shape
    h = torch.empty((rows, n), dtype=torch.bfloat16, device=g.device)
    if mxfp8:
        q = torch.empty((rows, n), dtype=torch.uint8, device=g.device)
        s = torch.empty((rows, n // 32), dtype=torch.uint8, device=g.device)
        _check(load().moe_swiglu(_ptr(g), _ptr(u), rows, n, MOE_MXFP8, _ptr(h), _ptr(q), _ptr(s), _stream()),
               "moe_swiglu")
        return h, q, s
    _check(load().moe_swiglu(_ptr(g), _ptr(u), rows, n, MOE_BF16, _ptr(h), None, None, _stream()),
           "moe_swiglu")
    return h


def grouped_gemm_fwd(a, b0, offsets, b1=None, swiglu=False, a_scales=None, b0_scales=None,
                     b1_scales=None, quantize_act=False, ws=None, out=None):
    """c0 = a . b0[e]^T per expert segment (bf16, or MXFP8 when scales are given).
    swiglu: returns (G, U, H[, H_q, H_s]) with b1 the up weight."""
    torch = _torch()
    mx = a_scales is not None
    rc, k_dim = a.shape
    E, n_dim, _ = b0.shape
    dev = a.device
    mk = lambda: torch.empty((rc, n_dim), dtype=torch.bfloat16, device=dev)
    c0 = out if out is not None else mk()
    c1 = mk() if swiglu else None
    act = mk() if swiglu else None
    aq = torch.empty((rc, n_dim), dtype=torch.uint8, device=dev) if quantize_act else None
    asc = torch.empty((rc, n_dim // 32), dtype=torch.uint8, device=dev) if quantize_act else None
    g = GemmFwdArgs(MOE_MXFP8 if mx else MOE_BF16, MOE_EPI_SWIGLU if swiglu else MOE_EPI_NONE, E, rc,
                    k_dim, n_dim, _ptr(offsets), _ptr(a), _ptr(a_scales), _ptr(b0), _ptr(b0_scales),
                    _ptr(b1), _ptr(b1_scales), _ptr(c0), _ptr(c1), _ptr(act), _ptr(aq), _ptr(asc))
    d = dims(1, 8, E, 1)
    ws = ws if ws is not None else _gemm_ws(rc, E, dev)
    _check(load().moe_grouped_gemm_fwd(C.byref(g), _ptr(ws), ws.numel(), _stream()), "moe_grouped_gemm_fwd")
    if swiglu:
        return (c0, c1, act, aq, asc) if quantize_act else (c0, c1, act)
    return c0


def _gemm_ws(rc, E, dev):
    torch = _torch()
    d = Dims(int(rc), 8, int(E), 1, 8, 1, 0)        # rows_cap = N*K with K = 1
    n = load().moe_workspace_size(MOE_OP_GEMM, C.byref(d))
    return torch.empty(max(int(n), 256), dtype=torch.uint8, device=dev)


def grouped_gemm_bwd(offsets, dc0, b0=None, a=None, dc1=None, b1=None, swiglu_g=None, swiglu_u=None,
                     dgrad=True, wgrad=True, ws=None):
    """Gradients of c = a . b[e]^T.  Returns dict with da (or dg, du when the
    SwiGLU backward is fused) and db0 (db1)."""
    torch = _torch()
    rc, n_dim = dc0.shape
    dev = dc0.device
    if b0 is not None:
        E, _, k_dim = b0.shape
    else:
        E, k_dim = offsets.numel() - 1, a.shape[1]
    swb = swiglu_g is not None
    out = {}
    da = dg = du = db0 = db1 = None
    if dgrad:
        if swb:
            dg = torch.empty((rc, k_dim), dtype=torch.bfloat16, device=dev)
            du = torch.empty((rc, k_dim), dtype=torch.bfloat16, device=dev)
            out.update(dg=dg, du=du)
        else:
            da = torch.empty((rc, k_dim), dtype=torch.bfloat16, device=dev)
            out.update(da=da)
    if wgrad:
        db0 = torch.empty((E, n_dim, k_dim), dtype=torch.bfloat16, device=dev)
        out["db0"] = db0
        if dc1 is not None:
            db1 = torch.empty((E, n_dim, k_dim), dtype=torch.bfloat16, device=dev)
            out["db1"] = db1
    g = GemmBwdArgs(MOE_BF16, MOE_EPI_SWIGLU_BWD if swb else MOE_EPI_NONE, E, rc, k_dim, n_dim,
                    _ptr(offsets), _ptr(a), _ptr(b0), _ptr(b1), _ptr(dc0), _ptr(dc1), _ptr(da),
                    _ptr(swiglu_g), _ptr(swiglu_u), _ptr(dg), _ptr(du), _ptr(db0), _ptr(db1))
    ws = ws if ws is not None else _gemm_ws(rc, E, dev)
    _check(load().moe_grouped_gemm_bwd(C.byref(g), _ptr(ws), ws.numel(), _stream()), "moe_grouped_gemm_bwd")
    return out


# ---- whole layer ---------------------------------------------------------------


@dataclass
class LayerWeights:
    w_r: object
    w_gate: Optional[object] = None
    w_up: Optional[object] = None
    w_down: Optional[object] = None
    bias: Optional[object] = None
    wq: Optional[dict] = None        # MXFP8: wg_q, wg_s, wu_q, wu_s, wd_q, wd_s; for the backward
                                     # also wdt_q, wdt_s, wgut_q, wgut_s (quantize_weights_mxfp8_dgrad)


def quantize_weights_mxfp8(w_gate, w_up, w_down) -> dict:
    """Pre-quantize the expert weights along their contraction dimension."""
    out = {}
    for name, w in (("wg", w_gate), ("wu", w_up), ("wd", w_down)):
        E, n, k = w.shape
        q, s = quantize_mxfp8(w.reshape(E * n, k))
        out[name + "_q"] = q.reshape(E, n, k)
        out[name + "_s"] = s.reshape(E, n, k // 32)
    return out


def quantize_mxfp8_cols(src, q, scales, col0=0):
    """Column-wise MXFP8 copy of bf16 src [B, R, C] into q [B, C, ld] (columns
    col0 .. col0 + R - 1) and scales [B, C, ld // 32], blocks along R."""
    B, R, Cn = src.shape
    ld = q.shape[2]
    _check(load().moe_quantize_mxfp8_cols(_ptr(src), B, R, Cn, ld, col0, _ptr(q), _ptr(scales), _stream()),
           "moe_quantize_mxfp8_cols")


def quantize_weights_mxfp8_dgrad(w_gate, w_up, w_down) -> dict:
    """The weight copies of the MXFP8 data gradients, each quantized from the
    bf16 weights along its other dimension: wdt_q [E, H, D] (W_down^T along D)
    and wgut_q [E, D, 2H] ([W_gate^T | W_up^T] along H), with their scales."""
    torch = _torch()
    E, H, D = w_gate.shape
    dev = w_gate.device
    u8 = lambda *s: torch.empty(s, dtype=torch.uint8, device=dev)
    out = dict(wdt_q=u8(E, H, D), wdt_s=u8(E, H, D // 32), wgut_q=u8(E, D, 2 * H), wgut_s=u8(E, D, 2 * H // 32))
    quantize_mxfp8_cols(w_down, out["wdt_q"], out["wdt_s"])
    quantize_mxfp8_cols(w_gate, out["wgut_q"], out["wgut_s"], 0)
    quantize_mxfp8_cols(w_up, out["wgut_q"], out["wgut_s"], H)
    return out


def _layer_args(x, wts: LayerWeights, K, drop, renorm, mxfp8, sched=MOE_SCHED_STAGED, n_group=0, topk_group=0,
                aux_alpha=0.0):
    N, D = x.shape
    E = wts.w_r.shape[0]
    wg = wts.wq["wg_q"] if mxfp8 else wts.w_gate
    H = wg.shape[1]
    n_shared = wg.shape[0] - E          # expert weights beyond the routed ones: the shared expert
    if n_shared not in (0, 1):
        raise ValueError("expert weights must hold E or E + 1 experts")
    d = dims(N, D, E, K, H, align=32 if mxfp8 else 1, renorm=renorm, n_group=n_group, topk_group=topk_group,
             n_shared=n_shared)
    q = wts.wq or {}
    a = LayerArgs(d, MOE_MXFP8 if mxfp8 else MOE_BF16, sched, _ptr(x), _ptr(wts.w_r), _ptr(wts.bias),
                  _ptr(drop), _ptr(wts.w_gate), _ptr(wts.w_up), _ptr(wts.w_down),
                  _ptr(q.get("wg_q")), _ptr(q.get("wg_s")), _ptr(q.get("wu_q")), _ptr(q.get("wu_s")),
                  _ptr(q.get("wd_q")), _ptr(q.get("wd_s")), float(aux_alpha), _ptr(q.get("wdt_q")),
                  _ptr(q.get("wdt_s")), _ptr(q.get("wgut_q")), _ptr(q.get("wgut_s")))
    return a, d


def alloc_saved(d: Dims, mxfp8: bool, device):
    """One buffer of moe_saved_size bytes, carved by moe_saved_carve; returns
    the dict of torch views of every field the dtype uses (plus "_buf")."""
    torch = _torch()
    lib = load()
    dt = MOE_MXFP8 if mxfp8 else MOE_BF16
    n = lib.moe_saved_size(C.byref(d), dt)
    if n == 0:
        raise MoeError("moe_saved_size: invalid dims")
    buf = torch.empty(int(n) + 256, dtype=torch.uint8, device=device)
    base = (buf.data_ptr() + 255) // 256 * 256
    sv_c = LayerSaved()
    _check(lib.moe_saved_carve(C.byref(d), dt, base, int(n), C.byref(sv_c)), "moe_saved_carve")
    N, D, E, K, H = d.N, d.D, d.E, d.K, d.H
    rc, Ex = rows_cap(d), d.E + d.n_shared
    f32, i32, bf, u8 = torch.float32, torch.int32, torch.bfloat16, torch.uint8
    spec = dict(logits=(f32, (N, E)), topk_idx=(i32, (N, K)), topk_prob=(f32, (N, K)), counts=(i32, (Ex,)),
                offsets=(i32, (Ex + 1,)), dst_rows=(i32, (N, K)), row_route=(i32, (rc,)), xd=(bf, (rc, D)),
                xd_q=(u8, (rc, D)), xd_s=(u8, (rc, D // 32)), g=(bf, (rc, H)), u=(bf, (rc, H)), h=(bf, (rc, H)),
                h_q=(u8, (rc, H)), h_s=(u8, (rc, H // 32)), y=(bf, (rc, D)), aux=(f32, (1,)), status=(i32, (1,)))
    sv = {"_buf": buf}
    for name in _SAVED_FIELDS:
        p = getattr(sv_c, name)
        if p is None:
            continue
        dtype, shape = spec[name]
        off = p - buf.data_ptr()
        nbytes = int(np.prod(shape)) * torch.tensor([], dtype=dtype).element_size()
        sv[name] = buf[off:off + nbytes].view(dtype).view(shape)
    return sv


def _saved_struct(sv: dict) -> LayerSaved:
    return LayerSaved(*[_ptr(sv.get(n)) for n, _ in LayerSaved._fields_])


def saved_tensors(sv: dict) -> dict:
    """The saved tensors without the backing buffer."""
    return {k: v for k, v in sv.items() if not k.startswith("_")}


class MoeLayer:
    """Holds the weights, saved tensors and workspaces of one layer so that
    repeated forward/backward calls allocate nothing.  sched selects the
    launch scheme: MOE_SCHED_STAGED, MOE_SCHED_READY (forward; the backward
    then runs staged) or MOE_SCHED_SINGLE (one launch per direction)."""

    def __init__(self, wts: LayerWeights, N: int, K: int, mxfp8=False, renorm=0, drop=None,
                 device="cuda", with_bwd=False, sched=MOE_SCHED_STAGED, router_bwd=False, n_group=0,
                 topk_group=0, aux_alpha=0.0, mx_wgrad=False):
        """n_group/topk_group: group-limited top-K; aux_alpha != 0: the aux loss
        goes to saved["aux"] and its gradient into the router backward;
        mx_wgrad: the MXFP8 backward's weight gradients on block-scaled MFMA
        (column-wise copies) instead of bf16 products."""
        torch = _torch()
        self.wts, self.K, self.mxfp8, self.renorm, self.drop = wts, K, mxfp8, renorm, drop
        self.sched = sched
        self.mx_wgrad = bool(mx_wgrad and mxfp8)
        self._opts = dict(n_group=n_group, topk_group=topk_group, aux_alpha=aux_alpha)
        D = wts.w_r.shape[1]
        self._x_proto = torch.empty((N, D), dtype=torch.bfloat16, device=device)
        _, self.d = _layer_args(self._x_proto, wts, K, drop, renorm, mxfp8, **self._opts)
        self.saved = alloc_saved(self.d, mxfp8, device)
        self._sv = _saved_struct(self.saved)
        self.ready_test_polls = 0      # testing the status word of the READY / SINGLE schedules only
        self.out = torch.empty((N, D), dtype=torch.bfloat16, device=device)
        self.ws_f = workspace(MOE_OP_LAYER_FWD, self.d, device)
        self.grads = None
        if with_bwd:
            E, H = self.d.E + self.d.n_shared, self.d.H
            op = (MOE_OP_LAYER_BWD_MXFP8_NATIVE if self.mx_wgrad else MOE_OP_LAYER_BWD_MXFP8) if mxfp8 \
                else MOE_OP_LAYER_BWD
            self.ws_b = workspace(op, self.d, device)
            self.grads = dict(dx=torch.empty((N, D), dtype=torch.bfloat16, device=device),
                              dprob=torch.empty((N, K), dtype=torch.float32, device=device),
                              dw_gate=torch.empty((E, H, D), dtype=torch.bfloat16, device=device),
                              dw_up=torch.empty((E, H, D), dtype=torch.bfloat16, device=device),
                              dw_down=torch.empty((E, D, H), dtype=torch.bfloat16, device=device))
            if router_bwd:
                # router gradients too; dx then includes dlogits . W_r
                Er = self.d.E
                self.grads.update(dw_r=torch.empty((Er, D), dtype=torch.bfloat16, device=device),
                                  db_r=torch.empty((Er,), dtype=torch.float32, device=device),
                                  dlogits=torch.empty((N, Er), dtype=torch.float32, device=device))
            self._gr = LayerGrads(**{n: _ptr(self.grads.get(n)) for n, t in LayerGrads._fields_ if t is _vp})

    def forward(self, x):
        a, _ = _layer_args(x, self.wts, self.K, self.drop, self.renorm, self.mxfp8, self.sched, **self._opts)
        a.ready_test_polls = int(self.ready_test_polls)
        _check(load().moe_layer_fwd(C.byref(a), C.byref(self._sv), _ptr(self.out), _ptr(self.ws_f),
                                    self.ws_f.numel(), _stream()), "moe_layer_fwd")
        return self.out

    def forward_noalloc(self, x):
        """The forward through moe_layer_fwd_noalloc: the library's static
        scratch instead of this layer's workspace."""
        a, _ = _layer_args(x, self.wts, self.K, self.drop, self.renorm, self.mxfp8, self.sched, **self._opts)
        _check(load().moe_layer_fwd_noalloc(C.byref(a), C.byref(self._sv), _ptr(self.out), _stream()),
               "moe_layer_fwd_noalloc")
        return self.out

    def backward(self, x, dout, recompute_h=False, d_aux=0.0):
        """recompute_h: do not read the saved H (bf16) or H codes (MXFP8); the
        library recomputes H from the saved G and U (SwiGLU-recompute mode).
        d_aux: upstream gradient of the aux loss (used when aux_alpha != 0)."""
        a, _ = _layer_args(x, self.wts, self.K, self.drop, self.renorm, self.mxfp8, self.sched, **self._opts)
        a.ready_test_polls = int(self.ready_test_polls)
        a.mx_wgrad = int(self.mx_wgrad)
        self._gr.d_aux = float(d_aux)
        sv = self._sv
        if recompute_h:
            sv = LayerSaved(*[getattr(self._sv, n) for n, _ in LayerSaved._fields_])
            sv.h = None
            sv.h_q = None
            sv.h_s = None
        _check(load().moe_layer_bwd(C.byref(a), C.byref(sv), _ptr(dout), C.byref(self._gr),
                                    _ptr(self.ws_b), self.ws_b.numel(), _stream()), "moe_layer_bwd")
        return self.grads


def layer_fwd(x, wts: LayerWeights, K, drop=None, renorm=0, mxfp8=False):
    """One forward call; returns (out, saved dict)."""
    layer = MoeLayer(wts, x.shape[0], K, mxfp8=mxfp8, renorm=renorm, drop=drop, device=x.device)
    out = layer.forward(x)
    return out, layer.saved
