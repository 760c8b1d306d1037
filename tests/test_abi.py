"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, sizes its buffers, and rejects bad arguments with the
documented status codes before queuing any work."""
import ctypes as C
import os
import re

import pytest
import torch

from moe_layer_zero_amd import zcmoe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    for f in os.listdir(os.path.join(ROOT, "include")):
        if f.endswith(".h"):
            src = open(os.path.join(ROOT, "include", f)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names |= set(re.findall(r"\b(zc_[a-z_0-9]+)\s*\(", src))
    return names


@pytest.fixture(scope="module")
def L():
    return zcmoe.lib()


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert names == set(zcmoe.EXPORTS), names
    for n in names:
        assert hasattr(L, n), n


def desc(**kw):
    base = dict(T=64, d=128, N=8, Z=4, I=64, K=2, dtype=torch.float32)
    base.update(kw)
    return zcmoe.LayerDesc(**base)


def test_sizes_are_positive_and_grow_with_T():
    for dt in (torch.float32, torch.bfloat16):
        a = desc(dtype=dt)
        b = desc(dtype=dt, T=4096)
        for op in (zcmoe.ZC_OP_ROUTE, zcmoe.ZC_OP_FORWARD, zcmoe.ZC_OP_BACKWARD,
                   zcmoe.ZC_OP_LB_LOSS):
            assert 0 < zcmoe.zc_moe_workspace_size(a, op) < zcmoe.zc_moe_workspace_size(b, op)
        # the statistics' scratch is one small histogram per block of 256 tokens
        op = zcmoe.ZC_OP_ROUTE_STATS
        assert 0 < zcmoe.zc_moe_workspace_size(a, op) <= zcmoe.zc_moe_workspace_size(b, op)
        assert 0 < zcmoe.zc_moe_saved_size(a) < zcmoe.zc_moe_saved_size(b)
    # an invalid description sizes to 0
    assert zcmoe.zc_moe_workspace_size(desc(K=0), zcmoe.ZC_OP_FORWARD) == 0
    assert zcmoe.zc_moe_workspace_size(desc(), 7) == 0


# Fake, 256-byte aligned, never dereferenced device addresses: every call
# below fails its host-side checks before any work is queued.
FAKE = C.c_void_p(1 << 20)


def route_buf():
    return zcmoe.zc_route_buf(*([FAKE] * 7))


def call_route(L, d, ws_bytes=1 << 30, **over):
    args = dict(x=FAKE, wr=FAKE, bias=FAKE, r=route_buf(), ws=FAKE)
    args.update(over)
    dd = d.c() if d is not None else None
    return L.zc_moe_route(C.byref(dd) if dd is not None else None, args["x"], args["wr"],
                          args["bias"], C.byref(args["r"]), args["ws"], ws_bytes, None)


@pytest.mark.parametrize("bad,code", [
    (dict(K=0), zcmoe.ZC_ERR_INVALID),
    (dict(K=13), zcmoe.ZC_ERR_INVALID),        # K > N+Z
    (dict(N=0, Z=0), zcmoe.ZC_ERR_INVALID),
    (dict(N=1000, Z=100), zcmoe.ZC_ERR_INVALID),  # N+Z > 1024
    (dict(T=-1), zcmoe.ZC_ERR_INVALID),
    (dict(d=100), zcmoe.ZC_ERR_UNSUPPORTED),
    (dict(dtype=torch.bfloat16, d=96), zcmoe.ZC_ERR_UNSUPPORTED),
    (dict(dtype=torch.bfloat16, I=32), zcmoe.ZC_ERR_UNSUPPORTED),
    (dict(gate_norm=2), zcmoe.ZC_ERR_INVALID),
    (dict(out_scale=float("nan")), zcmoe.ZC_ERR_INVALID),
    (dict(cu_limit=-8), zcmoe.ZC_ERR_INVALID),
    (dict(cu_limit=12), zcmoe.ZC_ERR_INVALID),     # not a multiple of 8
])
def test_bad_descriptions(L, bad, code):
    assert call_route(L, desc(**bad)) == code
    assert L.zc_last_error().decode() != ""


def test_bad_pointers_and_workspace(L):
    d = desc()
    assert call_route(L, None) == zcmoe.ZC_ERR_INVALID
    assert call_route(L, d, bias=None) == zcmoe.ZC_ERR_INVALID
    assert call_route(L, d, x=None) == zcmoe.ZC_ERR_INVALID       # x without w_router
    assert call_route(L, d, x=C.c_void_p((1 << 20) + 4)) == zcmoe.ZC_ERR_INVALID  # misaligned
    r = route_buf()
    r.perm = None
    assert call_route(L, d, r=r) == zcmoe.ZC_ERR_INVALID
    need = zcmoe.zc_moe_workspace_size(d, zcmoe.ZC_OP_ROUTE)
    assert call_route(L, d, ws_bytes=need - 1) == zcmoe.ZC_ERR_WORKSPACE
    assert "needed" in L.zc_last_error().decode()
    assert call_route(L, d, ws=None) == zcmoe.ZC_ERR_WORKSPACE


def test_forward_backward_argument_checks(L):
    d = desc()
    dd = d.c()
    r = route_buf()
    big = 1 << 40
    # N > 0 needs the expert weights
    st = L.zc_moe_forward(C.byref(dd), FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, C.byref(r), None,
                          FAKE, big, None)
    assert st == zcmoe.ZC_ERR_INVALID and "w_gate" in L.zc_last_error().decode()
    st = L.zc_moe_forward(C.byref(dd), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, C.byref(r), None,
                          FAKE, 16, None)
    assert st == zcmoe.ZC_ERR_WORKSPACE
    # backward needs the saved activations
    st = L.zc_moe_backward(C.byref(dd), FAKE, FAKE, FAKE, FAKE, FAKE, C.byref(r), None, FAKE, FAKE,
                           FAKE, FAKE, FAKE, FAKE, None, FAKE, big, None)
    assert st == zcmoe.ZC_ERR_INVALID and "saved" in L.zc_last_error().decode()
    # Eq.(2) update: T_all >= 1
    st = L.zc_moe_pid_update(8, 4, 2, FAKE, 0, 1.0, 1.5, FAKE, None)
    assert st == zcmoe.ZC_ERR_INVALID


def test_status_strings(L):
    for s in range(5):
        assert L.zc_status_string(s)
    assert L.zc_status_string(99) == b"unknown status"


def test_binding_rejects_host_tensors():
    d = desc()
    x = torch.zeros(64, 128)
    with pytest.raises((ValueError, zcmoe.ZcError)):
        zcmoe.zc_moe_route(d, x, torch.zeros(12, 128), torch.zeros(12),
                           zcmoe.RouteBuffers(d, device="cpu"), ws=x)


@pytest.mark.parametrize("bad,code", [
    (dict(weight_layout=3), zcmoe.ZC_ERR_INVALID),
    (dict(weight_layout=zcmoe.ZC_WEIGHTS_MXFP8), zcmoe.ZC_ERR_UNSUPPORTED),    # fp32 layer
    (dict(weight_layout=zcmoe.ZC_WEIGHTS_MXFP8, dtype=torch.bfloat16, d=256, I=512),
     zcmoe.ZC_ERR_UNSUPPORTED),                                              # d % 512
    (dict(weight_layout=zcmoe.ZC_WEIGHTS_MXFP8, dtype=torch.bfloat16, d=512, I=768),
     zcmoe.ZC_ERR_UNSUPPORTED),                                              # I % 512
    (dict(weight_layout=zcmoe.ZC_WEIGHTS_PACKED), zcmoe.ZC_ERR_UNSUPPORTED),   # fp32 layer
    (dict(weight_layout=zcmoe.ZC_WEIGHTS_PACKED, dtype=torch.bfloat16), zcmoe.ZC_ERR_UNSUPPORTED),
    (dict(weight_layout=zcmoe.ZC_WEIGHTS_PACKED, dtype=torch.bfloat16, d=256, I=128),
     zcmoe.ZC_ERR_UNSUPPORTED),
])
def test_bad_weight_layouts(L, bad, code):
    assert call_route(L, desc(**bad)) == code


def test_packed_weight_argument_checks(L):
    d = desc(dtype=torch.bfloat16, d=256, I=256, weight_layout=zcmoe.ZC_WEIGHTS_PACKED)
    dd = d.c()
    r = route_buf()
    big = 1 << 40
    # packed weights serve the inference forward only
    st = L.zc_moe_forward(C.byref(dd), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, C.byref(r), FAKE,
                          FAKE, big, None)
    assert st == zcmoe.ZC_ERR_UNSUPPORTED and "row-major" in L.zc_last_error().decode()
    st = L.zc_moe_backward(C.byref(dd), FAKE, FAKE, FAKE, FAKE, FAKE, C.byref(r), FAKE, FAKE, FAKE,
                           FAKE, FAKE, FAKE, FAKE, None, FAKE, big, None)
    assert st == zcmoe.ZC_ERR_UNSUPPORTED and "row-major" in L.zc_last_error().decode()
    # the packing call itself
    other = C.c_void_p(1 << 40)
    assert L.zc_moe_pack_weights(C.byref(dd), 5, FAKE, other, None) == zcmoe.ZC_ERR_INVALID
    assert L.zc_moe_pack_weights(C.byref(dd), 0, FAKE, FAKE, None) == zcmoe.ZC_ERR_INVALID
    assert "overlap" in L.zc_last_error().decode()
    f32 = desc(d=256, I=256).c()
    assert L.zc_moe_pack_weights(C.byref(f32), 0, FAKE, other, None) == zcmoe.ZC_ERR_UNSUPPORTED
    odd = desc(dtype=torch.bfloat16, d=256, I=192).c()
    assert L.zc_moe_pack_weights(C.byref(odd), 1, FAKE, other, None) == zcmoe.ZC_ERR_UNSUPPORTED


@pytest.mark.parametrize("cfg,kw", [
    (dict(D=3, K_e=1.5, alpha=0.1), {}),              # 3 does not divide N = 8
    (dict(D=0, K_e=1.5, alpha=0.1), {}),
    (dict(D=16, K_e=1.5, alpha=0.1), {}),             # more groups than experts
    (dict(D=2, K_e=2.0, alpha=0.1), {}),              # K_e = K with Z > 0
    (dict(D=2, K_e=0.0, alpha=0.1), {}),
    (dict(D=2, K_e=float("nan"), alpha=0.1), {}),
    (dict(D=2, K_e=1.5, alpha=float("inf")), {}),
    (dict(D=1, K_e=1.0, alpha=0.1), dict(N=0, Z=4)),  # no FFN experts
])
def test_lb_loss_argument_checks(L, cfg, kw):
    d = desc(**kw).c()
    c = zcmoe.zc_lb_cfg(cfg["D"], cfg["K_e"], cfg["alpha"])
    r = route_buf()
    st = L.zc_moe_lb_loss(C.byref(d), C.byref(c), C.byref(r), FAKE, FAKE, 1 << 40, None)
    assert st == zcmoe.ZC_ERR_INVALID, L.zc_last_error()
    # the backward checks the same settings before anything else is queued
    st = L.zc_moe_backward(C.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, C.byref(r), FAKE, FAKE, FAKE,
                           FAKE, FAKE, FAKE, FAKE, C.byref(c), FAKE, 1 << 40, None)
    assert st == zcmoe.ZC_ERR_INVALID


def test_lb_loss_accepts_k_e_equal_k_without_zero_experts(L):
    d = desc(Z=0).c()
    c = zcmoe.zc_lb_cfg(4, 2.0, 0.1)
    r = route_buf()
    # valid settings: fails only on the workspace
    st = L.zc_moe_lb_loss(C.byref(d), C.byref(c), C.byref(r), FAKE, FAKE, 8, None)
    assert st == zcmoe.ZC_ERR_WORKSPACE
    st = L.zc_moe_lb_loss(C.byref(d), C.byref(c), C.byref(r), None, FAKE, 1 << 40, None)
    assert st == zcmoe.ZC_ERR_INVALID and "out" in L.zc_last_error().decode()


def test_route_stats_and_accumulate_argument_checks(L):
    d = desc().c()
    r = route_buf()
    big = 1 << 40
    assert L.zc_moe_route_stats(C.byref(d), None, FAKE, FAKE, FAKE, big, None) == \
        zcmoe.ZC_ERR_INVALID
    assert L.zc_moe_route_stats(C.byref(d), C.byref(r), None, FAKE, FAKE, big, None) == \
        zcmoe.ZC_ERR_INVALID
    assert L.zc_moe_route_stats(C.byref(d), C.byref(r), FAKE, FAKE, FAKE, 4, None) == \
        zcmoe.ZC_ERR_WORKSPACE
    other = C.c_void_p(1 << 40)
    assert L.zc_moe_accumulate_counts(0, FAKE, other, None) == zcmoe.ZC_ERR_INVALID
    assert L.zc_moe_accumulate_counts(1025, FAKE, other, None) == zcmoe.ZC_ERR_INVALID
    assert L.zc_moe_accumulate_counts(12, FAKE, FAKE, None) == zcmoe.ZC_ERR_INVALID
    assert L.zc_moe_accumulate_counts(12, None, other, None) == zcmoe.ZC_ERR_INVALID


def test_quantized_weight_argument_checks(L):
    d = desc(dtype=torch.bfloat16, d=512, I=512)
    dd = d.c()
    n = L.zc_moe_quantized_weight_bytes(C.byref(dd))
    assert n == 8 * 512 * 512 * 33 // 32
    assert L.zc_moe_quantized_weight_bytes(C.byref(desc(K=0).c())) == 0
    other = C.c_void_p(1 << 40)
    assert L.zc_moe_quantize_weights(C.byref(dd), 2, FAKE, other, None) == zcmoe.ZC_ERR_INVALID
    assert L.zc_moe_quantize_weights(C.byref(dd), 0, FAKE, FAKE, None) == zcmoe.ZC_ERR_INVALID
    assert "overlap" in L.zc_last_error().decode()
    f32 = desc(d=512, I=512).c()
    assert L.zc_moe_quantize_weights(C.byref(f32), 0, FAKE, other, None) == \
        zcmoe.ZC_ERR_UNSUPPORTED
    # the MXFP8 forward serves inference only: no saved activations, no backward
    mx = desc(dtype=torch.bfloat16, d=512, I=512, weight_layout=zcmoe.ZC_WEIGHTS_MXFP8).c()
    r = route_buf()
    st = L.zc_moe_forward(C.byref(mx), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, C.byref(r), FAKE,
                          FAKE, 1 << 40, None)
    assert st == zcmoe.ZC_ERR_UNSUPPORTED
    st = L.zc_moe_backward(C.byref(mx), FAKE, FAKE, FAKE, FAKE, FAKE, C.byref(r), FAKE, FAKE, FAKE,
                           FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 40, None)
    assert st == zcmoe.ZC_ERR_UNSUPPORTED
    # its workspace holds the quantized activations on top of the bf16 forward's
    bf = desc(dtype=torch.bfloat16, d=512, I=512).c()
    assert L.zc_moe_workspace_size(C.byref(mx), zcmoe.ZC_OP_FORWARD) > \
        L.zc_moe_workspace_size(C.byref(bf), zcmoe.ZC_OP_FORWARD)


def test_noalloc_forward_rejects_oversized_layers_before_any_work(L):
    # a layer whose forward workspace exceeds the library's scratch: refused
    # on the host (fake, never dereferenced pointers)
    d = desc(dtype=torch.bfloat16, T=4096, d=1024, N=64, Z=32, I=512, K=6)
    assert zcmoe.zc_moe_workspace_size(d, zcmoe.ZC_OP_FORWARD) > zcmoe.NOALLOC_SCRATCH_BYTES
    dd, r = d.c(), route_buf()
    st = L.zc_moe_forward_noalloc(C.byref(dd), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                  C.byref(r), None)
    assert st == zcmoe.ZC_ERR_WORKSPACE
    assert "scratch" in L.zc_last_error().decode()
    # and the LongCat-Flash decode batch fits
    dec = desc(dtype=torch.bfloat16, T=256, d=6144, N=512, Z=256, I=2048, K=12)
    for lay in (zcmoe.ZC_WEIGHTS_ROWMAJOR, zcmoe.ZC_WEIGHTS_PACKED, zcmoe.ZC_WEIGHTS_MXFP8):
        dec.weight_layout = lay
        assert zcmoe.zc_moe_workspace_size(dec, zcmoe.ZC_OP_FORWARD) <= zcmoe.NOALLOC_SCRATCH_BYTES


@pytest.mark.parametrize("dims", [(64, 128, 8, 4, 64, 2, "fp32"), (300, 1024, 64, 32, 512, 6, "bf16"),
                                  (8192, 2048, 128, 64, 1024, 8, "bf16")])
def test_saved_buffer_layout_matches_the_library_size(dims):
    """The saved buffer is a, u, h in fp32 ([T*K][I] each) then y ([T*K][d] in
    the layer dtype), each piece 256-byte aligned: the library's size and the
    binding's views agree with that layout."""
    T, d, N, Z, I, K, dt = dims
    desc = zcmoe.LayerDesc(T=T, d=d, N=N, Z=Z, I=I, K=K,
                           dtype=torch.float32 if dt == "fp32" else torch.bfloat16)
    rows, es = T * K, 4 if dt == "fp32" else 2
    a256 = lambda n: (n + 255) // 256 * 256  # noqa: E731
    size = zcmoe.zc_moe_saved_size(desc)
    assert size == 3 * a256(rows * I * 4) + a256(rows * d * es)
    buf = torch.zeros(size, dtype=torch.uint8)
    v = zcmoe.saved_views(desc, buf)
    base = buf.data_ptr()
    for i, k in enumerate(("a", "u", "h")):
        assert v[k].shape == (rows, I) and v[k].dtype == torch.float32
        assert v[k].data_ptr() - base == i * a256(rows * I * 4)
    assert v["y"].shape == (rows, d) and v["y"].dtype == desc.dtype
    assert v["y"].data_ptr() - base == 3 * a256(rows * I * 4)
