"""Python binding of libzcmoe (include/zc_moe.h): argument marshalling only.

Every step of the layer runs in the HIP library; this module turns torch
tensors into the device pointers, sizes and the stream handle the C ABI
takes, checks dtypes, shapes and devices before the call, and raises
ZcError on any non-OK status.  PyTorch supplies device memory and streams.
There is no fallback: if the library is not built, loading it raises.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libzcmoe.so")

ZC_OK, ZC_ERR_INVALID, ZC_ERR_UNSUPPORTED, ZC_ERR_WORKSPACE, ZC_ERR_HIP = range(5)
ZC_F32, ZC_BF16 = 0, 1
ZC_OP_ROUTE, ZC_OP_FORWARD, ZC_OP_BACKWARD, ZC_OP_LB_LOSS, ZC_OP_ROUTE_STATS = 0, 1, 2, 3, 4
ZC_WEIGHTS_ROWMAJOR, ZC_WEIGHTS_PACKED, ZC_WEIGHTS_MXFP8 = 0, 1, 2
ZC_PACK_GATE_UP, ZC_PACK_DOWN = 0, 1

# Every symbol include/zc_moe.h declares.
EXPORTS = ("zc_moe_workspace_size", "zc_moe_saved_size", "zc_moe_route", "zc_moe_forward",
           "zc_moe_forward_noalloc", "zc_moe_backward", "zc_moe_lb_loss", "zc_moe_route_stats", "zc_moe_accumulate_counts",
           "zc_moe_pid_update", "zc_moe_pack_weights", "zc_moe_quantized_weight_bytes",
           "zc_moe_quantize_weights",
           "zc_moe_profile",
           "zc_moe_profile_read",
           "zc_moe_phase_name", "zc_status_string", "zc_last_error")
ZC_NUM_PHASES = 22


class ZcError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: status {status}: {detail}")
        self.status = status


class zc_moe_desc(C.Structure):
    _fields_ = [("T", C.c_int64), ("d", C.c_int64), ("N", C.c_int64), ("Z", C.c_int64),
                ("I", C.c_int64), ("K", C.c_int64), ("dtype", C.c_int32),
                ("gate_norm", C.c_int32), ("out_scale", C.c_float),
                ("weight_layout", C.c_int32), ("cu_limit", C.c_int32)]


class zc_lb_cfg(C.Structure):
    _fields_ = [("D", C.c_int64), ("K_e", C.c_double), ("alpha", C.c_double)]


class zc_route_buf(C.Structure):
    _fields_ = [("logits", C.c_void_p), ("topk_idx", C.c_void_p), ("topk_gate", C.c_void_p),
                ("counts", C.c_void_p), ("offsets", C.c_void_p), ("perm", C.c_void_p),
                ("inv", C.c_void_p)]


_LIB = None


def lib() -> C.CDLL:
    """Load libzcmoe.so; raises if it has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m moe_layer_zero_amd.build` (no fallback path exists)")
        L = C.CDLL(LIB_PATH)
        P, D = C.POINTER(zc_moe_desc), C.POINTER(zc_route_buf)
        v, i64, sz = C.c_void_p, C.c_int64, C.c_size_t
        L.zc_moe_workspace_size.argtypes = [P, C.c_int]
        L.zc_moe_workspace_size.restype = sz
        L.zc_moe_saved_size.argtypes = [P]
        L.zc_moe_saved_size.restype = sz
        L.zc_moe_route.argtypes = [P, v, v, v, D, v, sz, v]
        L.zc_moe_forward.argtypes = [P, v, v, v, v, v, v, v, D, v, v, sz, v]
        L.zc_moe_forward_noalloc.argtypes = [P, v, v, v, v, v, v, v, D, v]
        LB = C.POINTER(zc_lb_cfg)
        L.zc_moe_backward.argtypes = [P, v, v, v, v, v, D, v, v, v, v, v, v, v, LB, v, sz, v]
        L.zc_moe_lb_loss.argtypes = [P, LB, D, v, v, sz, v]
        L.zc_moe_route_stats.argtypes = [P, D, v, v, v, sz, v]
        L.zc_moe_accumulate_counts.argtypes = [i64, v, v, v]
        L.zc_moe_pid_update.argtypes = [i64, i64, i64, v, i64, C.c_double, C.c_double, v, v]
        L.zc_moe_pack_weights.argtypes = [P, C.c_int, v, v, v]
        L.zc_moe_quantized_weight_bytes.argtypes = [P]
        L.zc_moe_quantized_weight_bytes.restype = sz
        L.zc_moe_quantize_weights.argtypes = [P, C.c_int, v, v, v]
        for f in ("zc_moe_route", "zc_moe_forward", "zc_moe_forward_noalloc",
                  "zc_moe_backward", "zc_moe_lb_loss",
                  "zc_moe_route_stats", "zc_moe_accumulate_counts", "zc_moe_pid_update",
                  "zc_moe_pack_weights", "zc_moe_quantize_weights"):
            getattr(L, f).restype = C.c_int
        L.zc_moe_profile.argtypes = [C.c_int]
        L.zc_moe_profile.restype = C.c_int
        L.zc_moe_profile_read.argtypes = [C.POINTER(C.c_double), C.POINTER(C.c_int32)]
        L.zc_moe_profile_read.restype = C.c_int
        L.zc_moe_phase_name.argtypes = [C.c_int]
        L.zc_moe_phase_name.restype = C.c_char_p
        L.zc_status_string.argtypes = [C.c_int]
        L.zc_status_string.restype = C.c_char_p
        L.zc_last_error.argtypes = []
        L.zc_last_error.restype = C.c_char_p
        _LIB = L
    return _LIB


def _check(status: int, where: str) -> None:
    if status != ZC_OK:
        raise ZcError(status, where, lib().zc_last_error().decode())


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError("tensors passed to the HIP library must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors passed to the HIP library must be contiguous")
    return C.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


@dataclass
class LayerDesc:
    T: int
    d: int
    N: int
    Z: int
    I: int
    K: int
    dtype: torch.dtype = torch.bfloat16
    gate_norm: int = 1
    out_scale: float = 1.0
    weight_layout: int = ZC_WEIGHTS_ROWMAJOR
    cu_limit: int = 0

    @property
    def E(self) -> int:
        return self.N + self.Z

    def c(self) -> zc_moe_desc:
        if self.dtype not in (torch.float32, torch.bfloat16):
            raise ValueError("layer dtype must be float32 or bfloat16")
        return zc_moe_desc(self.T, self.d, self.N, self.Z, self.I, self.K,
                           ZC_F32 if self.dtype == torch.float32 else ZC_BF16,
                           self.gate_norm, self.out_scale, self.weight_layout,
                           self.cu_limit)


class RouteBuffers:
    """Device buffers of zc_route_buf, allocated with torch."""

    def __init__(self, desc: LayerDesc, device="cuda"):
        T, E, N, K = desc.T, desc.E, desc.N, desc.K
        i32 = torch.int32
        self.logits = torch.empty((T, E), dtype=torch.float32, device=device)
        self.topk_idx = torch.empty((T, K), dtype=i32, device=device)
        self.topk_gate = torch.empty((T, K), dtype=torch.float32, device=device)
        self.counts = torch.empty(E, dtype=i32, device=device)
        self.offsets = torch.empty(N + 1, dtype=i32, device=device)
        self.perm = torch.empty(max(T * K, 1), dtype=i32, device=device)
        self.inv = torch.empty(max(T * K, 1), dtype=i32, device=device)

    def c(self) -> zc_route_buf:
        return zc_route_buf(*(_ptr(getattr(self, f)) for f, _ in zc_route_buf._fields_))


def zc_moe_workspace_size(desc: LayerDesc, op: int) -> int:
    d = desc.c()
    return int(lib().zc_moe_workspace_size(C.byref(d), op))


def zc_moe_saved_size(desc: LayerDesc) -> int:
    d = desc.c()
    return int(lib().zc_moe_saved_size(C.byref(d)))


def workspace(desc: LayerDesc, op: int, device="cuda") -> torch.Tensor:
    n = zc_moe_workspace_size(desc, op)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def saved_buffer(desc: LayerDesc, device="cuda") -> torch.Tensor:
    return torch.empty(max(zc_moe_saved_size(desc), 256), dtype=torch.uint8, device=device)


def saved_views(desc: LayerDesc, saved: torch.Tensor) -> dict:
    """Views of a filled saved buffer (its layout is the one zc_moe_saved_size
    documents): a, u, h fp32 [T*K][I] and y [T*K][d] in the layer dtype,
    rows in dispatch order."""
    rows, I, d = desc.T * desc.K, desc.I, desc.d
    a256 = lambda n: (n + 255) // 256 * 256  # noqa: E731
    piece = a256(rows * I * 4)
    out = {}
    for i, k in enumerate(("a", "u", "h")):
        out[k] = saved[i * piece:i * piece + rows * I * 4].view(torch.float32).view(rows, I)
    es = 4 if desc.dtype == torch.float32 else 2
    out["y"] = saved[3 * piece:3 * piece + rows * d * es].view(desc.dtype).view(rows, d)
    return out


def _check_layer_tensor(t, shape, dtype, name):
    if t is None:
        return
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"{name}: expected {tuple(shape)} {dtype}, got {tuple(t.shape)} {t.dtype}")


def _check_weights(desc, w_router, w_gate, w_up, w_down):
    dt = desc.dtype
    _check_layer_tensor(w_router, (desc.E, desc.d), dt, "w_router")
    if desc.weight_layout == ZC_WEIGHTS_MXFP8:
        d = desc.c()
        n = int(lib().zc_moe_quantized_weight_bytes(C.byref(d)))
        for t, name in ((w_gate, "w_gate"), (w_up, "w_up"), (w_down, "w_down")):
            if t is not None and (t.dtype != torch.uint8 or t.numel() < n):
                raise ValueError(f"{name}: expected a quantized weight set of {n} uint8")
        return
    _check_layer_tensor(w_gate, (desc.N, desc.I, desc.d), dt, "w_gate")
    _check_layer_tensor(w_up, (desc.N, desc.I, desc.d), dt, "w_up")
    _check_layer_tensor(w_down, (desc.N, desc.d, desc.I), dt, "w_down")


def zc_moe_route(desc: LayerDesc, x, w_router, bias, route: RouteBuffers, ws=None, stream=None):
    """Router + dispatch.  x = w_router = None routes the scores already in
    route.logits."""
    if x is not None:
        _check_layer_tensor(x, (desc.T, desc.d), desc.dtype, "x")
        _check_weights(desc, w_router, None, None, None)
    _check_layer_tensor(bias, (desc.E,), torch.float32, "bias")
    if ws is None:
        ws = workspace(desc, ZC_OP_ROUTE, bias.device)
    d, r = desc.c(), route.c()
    _check(lib().zc_moe_route(C.byref(d), _ptr(x), _ptr(w_router), _ptr(bias), C.byref(r),
                              _ptr(ws), ws.numel(), _stream(stream)), "zc_moe_route")


def zc_moe_forward(desc: LayerDesc, x, w_router, bias, w_gate, w_up, w_down, out,
                   route: RouteBuffers, saved=None, ws=None, stream=None):
    _check_layer_tensor(x, (desc.T, desc.d), desc.dtype, "x")
    _check_layer_tensor(out, (desc.T, desc.d), desc.dtype, "out")
    _check_layer_tensor(bias, (desc.E,), torch.float32, "bias")
    _check_weights(desc, w_router, w_gate, w_up, w_down)
    if ws is None:
        ws = workspace(desc, ZC_OP_FORWARD, x.device)
    d, r = desc.c(), route.c()
    _check(lib().zc_moe_forward(C.byref(d), _ptr(x), _ptr(w_router), _ptr(bias), _ptr(w_gate),
                                _ptr(w_up), _ptr(w_down), _ptr(out), C.byref(r), _ptr(saved),
                                _ptr(ws), ws.numel(), _stream(stream)), "zc_moe_forward")


NOALLOC_SCRATCH_BYTES = 64 << 20  # ZC_NOALLOC_SCRATCH_BYTES


def zc_moe_forward_noalloc(desc: LayerDesc, x, w_router, bias, w_gate, w_up, w_down, out,
                           route: RouteBuffers, stream=None):
    """The inference forward on the library's own per-device scratch (no
    workspace argument, nothing allocated); rejects layers whose forward
    workspace exceeds NOALLOC_SCRATCH_BYTES."""
    _check_layer_tensor(x, (desc.T, desc.d), desc.dtype, "x")
    _check_layer_tensor(out, (desc.T, desc.d), desc.dtype, "out")
    _check_layer_tensor(bias, (desc.E,), torch.float32, "bias")
    _check_weights(desc, w_router, w_gate, w_up, w_down)
    d, r = desc.c(), route.c()
    _check(lib().zc_moe_forward_noalloc(C.byref(d), _ptr(x), _ptr(w_router), _ptr(bias),
                                        _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(out),
                                        C.byref(r), _stream(stream)), "zc_moe_forward_noalloc")


@dataclass
class LoadBalance:
    """Device-level load-balance loss settings: D groups of N/D consecutive
    FFN experts, expected FFN experts per token K_e, balance factor alpha."""
    D: int
    K_e: float
    alpha: float

    def c(self) -> zc_lb_cfg:
        return zc_lb_cfg(int(self.D), float(self.K_e), float(self.alpha))


def zc_moe_backward(desc: LayerDesc, x, w_router, w_gate, w_up, w_down, route: RouteBuffers,
                    saved, dout, dx, dw_router, dw_gate, dw_up, dw_down, ws=None, stream=None,
                    lb: "LoadBalance | None" = None):
    for t, n in ((x, "x"), (dout, "dout"), (dx, "dx")):
        _check_layer_tensor(t, (desc.T, desc.d), desc.dtype, n)
    _check_weights(desc, w_router, w_gate, w_up, w_down)
    _check_weights(desc, dw_router, dw_gate, dw_up, dw_down)
    if ws is None:
        ws = workspace(desc, ZC_OP_BACKWARD, x.device)
    d, r = desc.c(), route.c()
    lbc = None if lb is None else C.byref(lb.c())
    _check(lib().zc_moe_backward(C.byref(d), _ptr(x), _ptr(w_router), _ptr(w_gate), _ptr(w_up),
                                 _ptr(w_down), C.byref(r), _ptr(saved), _ptr(dout), _ptr(dx),
                                 _ptr(dw_router), _ptr(dw_gate), _ptr(dw_up), _ptr(dw_down),
                                 lbc, _ptr(ws), ws.numel(), _stream(stream)), "zc_moe_backward")


def zc_moe_lb_loss(desc: LayerDesc, lb: LoadBalance, route: RouteBuffers, out=None, ws=None,
                   stream=None):
    """Queues the device-level load-balance loss of the routed batch; returns
    out, a float64 GPU tensor [1 + 2(D+1)]: L, f_1..f_{D+1}, P_1..P_{D+1}."""
    if out is None:
        out = torch.empty(1 + 2 * (lb.D + 1), dtype=torch.float64, device=route.counts.device)
    _check_layer_tensor(out, (1 + 2 * (lb.D + 1),), torch.float64, "out")
    if ws is None:
        ws = workspace(desc, ZC_OP_LB_LOSS, route.counts.device)
    d, r, c = desc.c(), route.c(), lb.c()
    _check(lib().zc_moe_lb_loss(C.byref(d), C.byref(c), C.byref(r), _ptr(out), _ptr(ws),
                                ws.numel(), _stream(stream)), "zc_moe_lb_loss")
    return out


def zc_moe_route_stats(desc: LayerDesc, route: RouteBuffers, hist=None, moments=None, ws=None,
                       stream=None):
    """Queues the FFN-experts-per-token statistics of a routed batch; returns
    (hist [K+1] int32, moments [2] float64 = mean, std), both on the GPU."""
    dev = route.counts.device
    if hist is None:
        hist = torch.empty(desc.K + 1, dtype=torch.int32, device=dev)
    if moments is None:
        moments = torch.empty(2, dtype=torch.float64, device=dev)
    _check_layer_tensor(hist, (desc.K + 1,), torch.int32, "hist")
    _check_layer_tensor(moments, (2,), torch.float64, "moments")
    if ws is None:
        ws = workspace(desc, ZC_OP_ROUTE_STATS, dev)
    d, r = desc.c(), route.c()
    _check(lib().zc_moe_route_stats(C.byref(d), C.byref(r), _ptr(hist), _ptr(moments), _ptr(ws),
                                    ws.numel(), _stream(stream)), "zc_moe_route_stats")
    return hist, moments


def zc_moe_accumulate_counts(counts, acc, stream=None):
    """acc += counts (int32 [E] GPU tensors): per-expert token counts over
    several micro-batches, for one Eq.(2) update with T_all = their tokens."""
    E = counts.numel()
    _check_layer_tensor(counts, (E,), torch.int32, "counts")
    _check_layer_tensor(acc, (E,), torch.int32, "acc")
    _check(lib().zc_moe_accumulate_counts(E, _ptr(counts), _ptr(acc), _stream(stream)),
           "zc_moe_accumulate_counts")


def zc_moe_pid_update(N: int, Z: int, K: int, counts, T_all: int, mu: float, K_e: float, bias,
                      stream=None):
    _check_layer_tensor(counts, (N + Z,), torch.int32, "counts")
    _check_layer_tensor(bias, (N + Z,), torch.float32, "bias")
    _check(lib().zc_moe_pid_update(N, Z, K, _ptr(counts), T_all, float(mu), float(K_e),
                                   _ptr(bias), _stream(stream)), "zc_moe_pid_update")


def zc_moe_pack_weights(desc: LayerDesc, which: int, src, dst, stream=None):
    """Packs w_gate or w_up (which = ZC_PACK_GATE_UP, [N][I][d]) or w_down
    (ZC_PACK_DOWN, [N][d][I]) into dst, a tensor of the same shape and dtype
    whose bytes then hold the packed layout."""
    shape = (desc.N, desc.I, desc.d) if which == ZC_PACK_GATE_UP else (desc.N, desc.d, desc.I)
    _check_layer_tensor(src, shape, desc.dtype, "src")
    _check_layer_tensor(dst, shape, desc.dtype, "dst")
    d = desc.c()
    _check(lib().zc_moe_pack_weights(C.byref(d), which, _ptr(src), _ptr(dst), _stream(stream)),
           "zc_moe_pack_weights")


def pack_expert_weights(desc: LayerDesc, w_gate, w_up, w_down, stream=None):
    """Packed copies (new tensors) of the three expert weight tensors."""
    out = []
    for w, which in ((w_gate, ZC_PACK_GATE_UP), (w_up, ZC_PACK_GATE_UP), (w_down, ZC_PACK_DOWN)):
        p = torch.empty_like(w)
        zc_moe_pack_weights(desc, which, w, p, stream)
        out.append(p)
    return tuple(out)


def zc_moe_profile(on: bool) -> None:
    _check(lib().zc_moe_profile(1 if on else 0), "zc_moe_profile")


def zc_moe_profile_read() -> dict:
    """{phase name: (total ms, launches)} of the events recorded since the
    last read (waits for them)."""
    tot = (C.c_double * ZC_NUM_PHASES)()
    cnt = (C.c_int32 * ZC_NUM_PHASES)()
    _check(lib().zc_moe_profile_read(tot, cnt), "zc_moe_profile_read")
    return {lib().zc_moe_phase_name(i).decode(): (tot[i], cnt[i])
            for i in range(ZC_NUM_PHASES) if cnt[i]}


def zc_moe_quantize_weights(desc: LayerDesc, which: int, src, dst=None, stream=None):
    """FP8 blockwise (MXFP8) quantization of w_gate or w_up (which =
    ZC_PACK_GATE_UP, [N][I][d]) or w_down (ZC_PACK_DOWN, [N][d][I]) into dst,
    a uint8 GPU tensor of zc_moe_quantized_weight_bytes(desc) bytes (allocated
    when None).  Returns dst."""
    shape = (desc.N, desc.I, desc.d) if which == ZC_PACK_GATE_UP else (desc.N, desc.d, desc.I)
    _check_layer_tensor(src, shape, desc.dtype, "src")
    d = desc.c()
    n = int(lib().zc_moe_quantized_weight_bytes(C.byref(d)))
    if dst is None:
        dst = torch.empty(max(n, 16), dtype=torch.uint8, device=src.device)
    if dst.dtype != torch.uint8 or dst.numel() < n:
        raise ValueError(f"dst: expected at least {n} uint8, got {dst.numel()} {dst.dtype}")
    _check(lib().zc_moe_quantize_weights(C.byref(d), which, _ptr(src), _ptr(dst), _stream(stream)),
           "zc_moe_quantize_weights")
    return dst


def quantize_expert_weights(desc: LayerDesc, w_gate, w_up, w_down, stream=None):
    """The three MXFP8 weight sets a ZC_WEIGHTS_MXFP8 forward takes."""
    return (zc_moe_quantize_weights(desc, ZC_PACK_GATE_UP, w_gate, stream=stream),
            zc_moe_quantize_weights(desc, ZC_PACK_GATE_UP, w_up, stream=stream),
            zc_moe_quantize_weights(desc, ZC_PACK_DOWN, w_down, stream=stream))
