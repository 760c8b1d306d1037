"""ctypes wrapper around the fp64 CPU oracle (orc.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product package.  Inputs are numpy
arrays holding fp32 values or bf16 bit patterns (uint16); every result is
float64 (or int32 for routing).  See orc.c for the step-by-step definition and
its source: "LongCat-Flash Technical Report", section 2.1 Eq.(1) and section
2.1.1 Eq.(2).
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

F32, BF16 = 0, 1
_i64, _i32, _f64 = C.c_int64, C.c_int, C.c_double
_p = C.c_void_p


def lib():
    global _LIB
    if _LIB is None:
        path = os.path.join(HERE, "liborc.so")
        if not os.path.exists(path):
            from oracle import build as _b  # noqa: WPS433
            _b.build()
        L = C.CDLL(path)
        L.orc_exp.restype = C.c_double
        L.orc_exp.argtypes = [C.c_double]
        L.orc_logits.argtypes = [_i64, _i64, _i64, _i32, _p, _p, _p]
        L.orc_route.argtypes = [_i64, _i64, _i64, _i64, _i32, _p, _p, _p, _p, _p, _p, _p, _p, _p]
        L.orc_forward.argtypes = [_i64, _i64, _i64, _i64, _i64, _i32, _f64, _p, _p, _p, _p,
                                  _p, _p, _i64, _p, _p, _p]
        L.orc_ffn_act.argtypes = [_i64, _i64, _i64, _i64, _i32, _p, _p, _p, _i64, _p, _p, _p,
                                  _p, _p]
        L.orc_backward.argtypes = [_i64, _i64, _i64, _i64, _i64, _i64, _i32, _i32, _f64, _p, _p,
                                   _p, _p, _p, _p, _p, _p, _p, _i64, _p, _p, _p, _p, _p, _p,
                                   _p]
        L.orc_lb_loss.argtypes = [_i64, _i64, _i64, _i64, _i64, _f64, _f64, _p, _p, _p, _p]
        L.orc_route_stats.argtypes = [_i64, _i64, _i64, _p, _p, _p, _p]
        L.orc_e4m3_value.restype = C.c_double
        L.orc_e4m3_value.argtypes = [_i32]
        L.orc_e4m3_encode.restype = C.c_int
        L.orc_e4m3_encode.argtypes = [C.c_double]
        L.orc_mx_quantize.argtypes = [_i64, _i64, _i32, _p, _p, _p]
        L.orc_mx_dequantize.argtypes = [_i64, _i64, _p, _p, _p]
        L.orc_forward_mx.argtypes = [_i64, _i64, _i64, _i64, _i64, _i32, _f64, _p, _p, _p, _p,
                                     _p, _p, _p, _p, _p, _i64, _p, _p, _p]
        L.orc_mx_flip_bound.argtypes = [_i64, _i64, _i64, _i64, _i64, _i32, _f64, _p, _p, _p,
                                        _p, _p, _p, _p, _p, _p, _i64, _p, _f64, _p]
        L.orc_num_threads.restype = C.c_int
        L.orc_num_threads.argtypes = []
        L.orc_pid_update.argtypes = [_i64, _i64, _i64, _p, _i64, _f64, _f64, _p]
        for f in ("orc_logits", "orc_route", "orc_forward", "orc_ffn_act", "orc_backward",
                  "orc_pid_update",
                  "orc_lb_loss", "orc_route_stats", "orc_mx_quantize", "orc_mx_dequantize",
                  "orc_forward_mx", "orc_mx_flip_bound"):
            getattr(L, f).restype = C.c_int
        _LIB = L
    return _LIB


def _dt(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError(f"oracle inputs are fp32 or bf16 bits (uint16), got {a.dtype}")


def _ptr(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dtype=None):
    if a is None:
        return None
    a = np.ascontiguousarray(a if dtype is None else a.astype(dtype, copy=False))
    return a


def num_threads() -> int:
    return int(lib().orc_num_threads())


def exp(z: float) -> float:
    """Routing-key exponential (Cody-Waite + degree-13 Taylor, see orc.c)."""
    return lib().orc_exp(float(z))


def logits(x: np.ndarray, wr: np.ndarray) -> np.ndarray:
    """O1: l = x Wr^T in fp64.  x [T,d], wr [E,d]."""
    x, wr = _c(x), _c(wr)
    T, d = x.shape
    E = wr.shape[0]
    assert wr.shape[1] == d and _dt(x) == _dt(wr)
    out = np.empty((T, E), np.float64)
    rc = lib().orc_logits(T, d, E, _dt(x), _ptr(x), _ptr(wr), _ptr(out))
    assert rc == 0
    return out


class Route:
    """Result of O2..O5."""

    def __init__(self, T, E, N, K):
        self.keys = np.empty((T, E), np.float64)
        self.topk_idx = np.empty((T, K), np.int32)
        self.gates = np.empty((T, K), np.float64)
        self.counts = np.empty(E, np.int32)
        self.offsets = np.empty(N + 1, np.int32)
        self.perm = np.full(T * K, -1, np.int32)
        self.inv = np.empty(T * K, np.int32)

    @property
    def p_real(self) -> int:
        return int(self.offsets[-1])


def route(lg: np.ndarray, bias: np.ndarray, N: int, K: int, gate_norm: int = 1,
          want_keys: bool = True) -> Route:
    """O2..O5 from logits (any float array, widened exactly to fp64)."""
    lg = _c(lg, np.float64)
    bias = _c(bias, np.float32)
    T, E = lg.shape
    assert bias.shape == (E,)
    r = Route(T, E, N, K)
    if not want_keys:
        r.keys = None
    rc = lib().orc_route(T, E, N, K, int(gate_norm), _ptr(lg), _ptr(bias), _ptr(r.keys),
                         _ptr(r.topk_idx), _ptr(r.gates), _ptr(r.counts), _ptr(r.offsets),
                         _ptr(r.perm), _ptr(r.inv))
    assert rc == 0
    r.perm = r.perm[: r.p_real].copy()
    return r


def _table(ws, N):
    """Per-expert pointer table from a list/array/dict of expert weight blocks."""
    arr = (C.c_void_p * N)()
    keep = []
    for e in range(N):
        w = ws.get(e) if isinstance(ws, dict) else ws[e]
        if w is None:
            arr[e] = None
            continue
        w = np.ascontiguousarray(w)
        keep.append(w)
        arr[e] = w.ctypes.data
    return arr, keep


def forward(x, wg, wu, wd, topk_idx, gates, N, out_scale=1.0, toks=None, want_y=False):
    """O6+O7 for tokens `toks` (all when None).  wg/wu/wd: [N,...] arrays or
    per-expert dicts {e: block}; blocks must share x's storage dtype."""
    x = _c(x)
    T, d = x.shape
    K = topk_idx.shape[1]
    e0 = next(iter(wg.values())) if isinstance(wg, dict) else wg[0]
    I = e0.shape[0]
    tg, kg = _table(wg, N)
    tu, ku = _table(wu, N)
    td, kd = _table(wd, N)
    ti = _c(topk_idx, np.int32)
    gg = _c(gates, np.float64)
    tk = None if toks is None else _c(np.asarray(toks), np.int64)
    n = T if tk is None else len(tk)
    out = np.empty((n, d), np.float64)
    y = np.empty((n, K, d), np.float64) if want_y else None
    rc = lib().orc_forward(T, d, N, I, K, _dt(x), float(out_scale), _ptr(x), tg, tu, td,
                           _ptr(ti), _ptr(gg), n, _ptr(tk), _ptr(out), _ptr(y))
    assert rc == 0, "oracle forward failed (missing expert weights or bad token)"
    del kg, ku, kd
    return (out, y) if want_y else out


def ffn_activations(x, wg, wu, N, tok, ex):
    """O6's pre-activations and hidden row of the picks (tok[q], ex[q]):
    a = W_g[e] x_t, u = W_u[e] x_t, h = silu(a) u, each [n][I] in binary64.
    wg/wu: [N,...] arrays or per-expert dicts {e: block} sharing x's
    storage dtype."""
    x = _c(x)
    T, d = x.shape
    e0 = next(iter(wg.values())) if isinstance(wg, dict) else wg[0]
    I = e0.shape[0]
    tg, kg = _table(wg, N)
    tu, ku = _table(wu, N)
    tk = _c(np.asarray(tok), np.int64)
    te = _c(np.asarray(ex), np.int32)
    n = len(tk)
    a, u, h = (np.empty((n, I), np.float64) for _ in range(3))
    rc = lib().orc_ffn_act(T, d, N, I, _dt(x), _ptr(x), tg, tu, n, _ptr(tk), _ptr(te), _ptr(a),
                           _ptr(u), _ptr(h))
    assert rc == 0, "oracle activations failed (missing expert weights or bad pick)"
    del kg, ku
    return a, u, h


def backward(x, wr, wg, wu, wd, lg, topk_idx, gates, dY, N, Z, gate_norm=1, out_scale=1.0,
             toks=None, want_experts=None, want_dwr=True, dl_extra=None, want_dx=True):
    """O9.  Returns dict with dx [n,d] (None when not want_dx), dwr [E,d] (or
    None), dwg/dwu/dwd as {e: array} for experts in want_experts (all N when
    None).  dl_extra ([T,E], e.g. lb_loss's dlogits) is added to the
    router-score gradient.  want_dx = want_dwr = False differentiates only
    the picks of the wanted experts (their weight gradients need nothing
    else); wg/wu/wd then need blocks for those experts only."""
    x, wr, dY = _c(x), _c(wr), _c(dY)
    T, d = x.shape
    E = N + Z
    K = topk_idx.shape[1]
    e0 = next(iter(wg.values())) if isinstance(wg, dict) else wg[0]
    I = e0.shape[0]
    tg, kg = _table(wg, N)
    tu, ku = _table(wu, N)
    td, kd = _table(wd, N)
    lg = _c(lg, np.float64)
    ti = _c(topk_idx, np.int32)
    gg = _c(gates, np.float64)
    tk = None if toks is None else _c(np.asarray(toks), np.int64)
    ex = None if dl_extra is None else _c(dl_extra, np.float64)
    if ex is not None:
        assert ex.shape == (T, E)
    n = T if tk is None else len(tk)
    assert want_dx or not want_dwr, "the router gradient comes with dx"
    dx = np.empty((n, d), np.float64) if want_dx else None
    dwr = np.zeros((E, d), np.float64) if want_dwr else None
    wanted = range(N) if want_experts is None else want_experts
    dwg = {e: np.zeros((I, d), np.float64) for e in wanted}
    dwu = {e: np.zeros((I, d), np.float64) for e in wanted}
    dwd = {e: np.zeros((d, I), np.float64) for e in wanted}
    pg, qg = _table(dwg, N)
    pu, qu = _table(dwu, N)
    pd, qd = _table(dwd, N)
    rc = lib().orc_backward(T, d, N, Z, I, K, _dt(x), int(gate_norm), float(out_scale), _ptr(x),
                            _ptr(wr), tg, tu, td, _ptr(lg), _ptr(ti), _ptr(gg), _ptr(dY), n,
                            _ptr(tk), _ptr(ex), _ptr(dx), _ptr(dwr), pg, pu, pd)
    assert rc == 0, f"oracle backward failed rc={rc}"
    del kg, ku, kd, qg, qu, qd
    return {"dx": dx, "dwr": dwr, "dwg": dwg, "dwu": dwu, "dwd": dwd}


def pid_update(counts, T_all, bias, N, Z, K, mu, K_e) -> np.ndarray:
    """O8 (Eq.(2)); returns the updated fp32 bias (input left untouched)."""
    c = _c(counts, np.int32)
    b = np.array(bias, dtype=np.float32, copy=True)
    rc = lib().orc_pid_update(N, Z, K, _ptr(c), int(T_all), float(mu), float(K_e), _ptr(b))
    assert rc == 0
    return b


def lb_loss(lg, topk_idx, N, D, K_e, alpha, want_grad=True):
    """O10: device-level load-balance loss (section 2.1.2, Eq.(4)-(5)).
    Returns (L, f [D+1], P [D+1], dlogits [T,E] or None)."""
    lg = _c(lg, np.float64)
    ti = _c(topk_idx, np.int32)
    T, E = lg.shape
    K = ti.shape[1]
    out = np.zeros(1 + 2 * (D + 1), np.float64)
    dl = np.empty((T, E), np.float64) if want_grad else None
    rc = lib().orc_lb_loss(T, E, N, K, D, float(K_e), float(alpha), _ptr(lg), _ptr(ti),
                           _ptr(out), _ptr(dl))
    if rc != 0:
        raise ValueError(f"oracle lb_loss rejected its arguments (rc={rc})")
    return float(out[0]), out[1:D + 2].copy(), out[D + 2:].copy(), dl


def route_stats(topk_idx, N):
    """O11: FFN experts per token -> (hist [K+1] int32, mean, std)."""
    ti = _c(topk_idx, np.int32)
    T, K = ti.shape
    hist = np.zeros(K + 1, np.int32)
    m, s = C.c_double(), C.c_double()
    rc = lib().orc_route_stats(T, N, K, _ptr(ti), _ptr(hist), C.byref(m), C.byref(s))
    assert rc == 0, f"oracle route_stats failed rc={rc}"
    return hist, m.value, s.value


def e4m3_value(code: int) -> float:
    """O12: value of an OCP FP8 E4M3 code."""
    return lib().orc_e4m3_value(int(code))


def e4m3_encode(v: float) -> int:
    """O12: nearest E4M3 code (ties to even, saturating at 448)."""
    return int(lib().orc_e4m3_encode(float(v)))


def mx_quantize(a: np.ndarray):
    """O12: MXFP8 (E4M3 codes, E8M0 scale per 32 along the last axis) of a 2-D
    fp32 / bf16-bits / float64 array.  Returns (codes uint8, scales uint8)."""
    if a.dtype == np.float64:
        dt = 2
    else:
        dt = _dt(a)
    a = _c(a)
    rows, cols = a.shape
    codes = np.empty((rows, cols), np.uint8)
    scales = np.empty((rows, cols // 32), np.uint8)
    rc = lib().orc_mx_quantize(rows, cols, dt, _ptr(a), _ptr(codes), _ptr(scales))
    if rc != 0:
        raise ValueError("oracle mx_quantize rejected its arguments")
    return codes, scales


def mx_dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    codes, scales = _c(codes, np.uint8), _c(scales, np.uint8)
    rows, cols = codes.shape
    out = np.empty((rows, cols), np.float64)
    rc = lib().orc_mx_dequantize(rows, cols, _ptr(codes), _ptr(scales), _ptr(out))
    assert rc == 0
    return out


def mx_weights(w: np.ndarray):
    """MXFP8 image (codes, scales) of one expert weight [R][C], blocks of 32
    along C (the reduction dimension)."""
    return mx_quantize(w)


def _mx_tables(wgq, wuq, wdq, N):
    tabs, keep = [], []
    for src in (wgq, wuq, wdq):
        for part in (0, 1):
            arrs = {e: _c(v[part], np.uint8) for e, v in src.items()}
            t, k = _table(arrs, N)
            tabs.append(t)
            keep.append((arrs, k))
    return tabs, keep


def forward_mx(x, wgq, wuq, wdq, topk_idx, gates, N, out_scale=1.0, toks=None, want_y=False):
    """O13: the layer forward with MXFP8 expert operands (h quantized from its
    binary64 value).  wgq / wuq / wdq: {expert: (codes, scales)}
    (mx_weights) for every FFN expert the listed tokens pick."""
    x = _c(x)
    T, d = x.shape
    K = topk_idx.shape[1]
    I = next(iter(wgq.values()))[0].shape[0] if wgq else 32  # no FFN pick: any I
    tabs, keep = _mx_tables(wgq, wuq, wdq, N)
    ti = _c(topk_idx, np.int32)
    gg = _c(gates, np.float64)
    tk = None if toks is None else _c(np.asarray(toks), np.int64)
    n = T if tk is None else len(tk)
    out = np.empty((n, d), np.float64)
    y = np.empty((n * K, d), np.float64) if want_y else None
    rc = lib().orc_forward_mx(T, d, N, I, K, _dt(x), float(out_scale), _ptr(x), *tabs,
                              _ptr(ti), _ptr(gg), n, _ptr(tk), _ptr(out), _ptr(y))
    assert rc == 0, f"oracle forward_mx failed rc={rc}"
    del keep
    return (out, y) if want_y else out


def mx_flip_bound(x, wgq, wuq, wdq, topk_idx, gates, N, eps, out_scale=1.0, toks=None):
    """Tolerance helper for comparisons against forward_mx (not part of the
    layer): per output element, the largest change that h codes lying within
    the fp32 uncertainty of h (eps relative to the dot products' sums of
    absolute products) of a code or scale boundary can cause.  Same
    arguments as forward_mx; returns [n, d]."""
    x = _c(x)
    T, d = x.shape
    K = topk_idx.shape[1]
    I = next(iter(wgq.values()))[0].shape[0] if wgq else 32
    tabs, keep = _mx_tables(wgq, wuq, wdq, N)
    ti = _c(topk_idx, np.int32)
    gg = _c(gates, np.float64)
    tk = None if toks is None else _c(np.asarray(toks), np.int64)
    n = T if tk is None else len(tk)
    fl = np.empty((n, d), np.float64)
    rc = lib().orc_mx_flip_bound(T, d, N, I, K, _dt(x), float(out_scale), _ptr(x), *tabs,
                                 _ptr(ti), _ptr(gg), n, _ptr(tk), float(eps), _ptr(fl))
    assert rc == 0, f"oracle mx_flip_bound failed rc={rc}"
    del keep
    return fl
