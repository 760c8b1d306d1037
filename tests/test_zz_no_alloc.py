"""GPU test of zc_moe_forward_noalloc, the inference forward that allocates
nothing (its scratch is a device array inside the library, for callers
that cannot allocate: graph capture, serving loops).  Called through the C
ABI, it must give exactly what zc_moe_forward gives with a workspace of its
own -- the same kernels in the same order -- on consecutive calls of
different sizes (the scratch keeps the previous call's contents), for
row-major, packed and MXFP8 weights, and it must reject a layer whose
workspace exceeds the scratch before queuing anything."""
import dataclasses

import pytest
import torch

from moe_layer_zero_amd import synth, zcmoe
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu


def weights_for(desc, Lg, layout):
    if layout == zcmoe.ZC_WEIGHTS_PACKED:
        return zcmoe.pack_expert_weights(desc, Lg["wg"], Lg["wu"], Lg["wd"])
    if layout == zcmoe.ZC_WEIGHTS_MXFP8:
        return zcmoe.quantize_expert_weights(desc, Lg["wg"], Lg["wu"], Lg["wd"])
    return Lg["wg"], Lg["wu"], Lg["wd"]


def both(sh, layout, Lg):
    desc = dataclasses.replace(H.desc_of(sh), weight_layout=layout)
    assert zcmoe.zc_moe_workspace_size(desc, zcmoe.ZC_OP_FORWARD) <= zcmoe.NOALLOC_SCRATCH_BYTES
    wg, wu, wd = weights_for(desc, Lg, layout)
    res = []
    for fn in ("noalloc", "ws"):
        route = zcmoe.RouteBuffers(desc)
        out = torch.full((sh.T, sh.d), float("nan"), dtype=sh.torch_dtype, device="cuda")
        if fn == "noalloc":
            zcmoe.zc_moe_forward_noalloc(desc, Lg["x"], Lg["wr"], Lg["bias"], wg, wu, wd, out,
                                         route)
        else:
            zcmoe.zc_moe_forward(desc, Lg["x"], Lg["wr"], Lg["bias"], wg, wu, wd, out, route)
        torch.cuda.synchronize()
        P = int(route.offsets[-1].item())
        res.append([out, route.logits, route.topk_idx, route.topk_gate, route.counts,
                    route.offsets, route.perm[:P], route.inv])
    for a, b in zip(*res):
        assert torch.equal(a, b)
    return res[0][0]


def test_noalloc_forward_matches_the_workspace_forward():
    base = synth.CONFIGS["small_bf16"]
    L = synth.make_layer(base.with_T(1024), "cpu")
    Lg = H.to_dev(L)
    # two calls in a row, the second smaller, for each weight layout
    for layout in (zcmoe.ZC_WEIGHTS_ROWMAJOR, zcmoe.ZC_WEIGHTS_PACKED, zcmoe.ZC_WEIGHTS_MXFP8):
        for T in (1024, 300):
            print(f"[noalloc] layout={layout} T={T}", flush=True)
            sh = base.with_T(T)
            Ls = dict(Lg, x=Lg["x"][:T].contiguous())
            out = both(sh, layout, Ls)
            assert torch.isfinite(out.float()).all()
    # the tiny fp32 layer, then an empty batch
    tf = synth.CONFIGS["tiny_fp32"]
    Lt = H.to_dev(synth.make_layer(tf, "cpu"))
    print("[noalloc] tiny fp32", flush=True)
    both(tf, zcmoe.ZC_WEIGHTS_ROWMAJOR, Lt)
    e0 = tf.with_T(0)
    d0 = H.desc_of(e0)
    r0 = zcmoe.RouteBuffers(d0)
    zcmoe.zc_moe_forward_noalloc(d0, Lt["x"][:0], Lt["wr"], Lt["bias"], Lt["wg"], Lt["wu"],
                                 Lt["wd"], Lt["x"][:0], r0)
    torch.cuda.synchronize()
    assert r0.counts.abs().sum().item() == 0


def test_noalloc_forward_rejects_a_layer_beyond_its_scratch():
    sh = synth.CONFIGS["small_bf16"]   # T = 4096: a 75 MB forward workspace
    desc = H.desc_of(sh)
    assert zcmoe.zc_moe_workspace_size(desc, zcmoe.ZC_OP_FORWARD) > zcmoe.NOALLOC_SCRATCH_BYTES
    Lg = H.to_dev(synth.make_layer(sh, "cpu"))
    route = zcmoe.RouteBuffers(desc)
    out = torch.full((sh.T, sh.d), 7.0, dtype=sh.torch_dtype, device="cuda")
    with pytest.raises(zcmoe.ZcError) as ei:
        zcmoe.zc_moe_forward_noalloc(desc, Lg["x"], Lg["wr"], Lg["bias"], Lg["wg"], Lg["wu"],
                                     Lg["wd"], out, route)
    assert ei.value.status == zcmoe.ZC_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert (out.float() == 7.0).all()
