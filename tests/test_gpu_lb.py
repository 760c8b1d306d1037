"""GPU parity of the device-level load-balance loss ("LongCat-Flash Technical
Report", section 2.1.2, Eq.(4)-(5)) and of the backward that adds its
score gradient, against the fp64 oracle.

The loss reads the router scores and the per-expert pick counts of a routed
batch.  Both sides route the same fp32 scores (the picks agree bit for bit,
asserted below), so f is an exact count on both sides and agrees bitwise;
P and L are binary64 sums in different orders and agree to 1e-12 relative.
The backward's extra router-score term is checked through dW_r and dx with
the layer tolerances of gpu_harness, once alone (dout = 0) and once beside
the gate gradients.
"""
import numpy as np
import pytest
import torch

from moe_layer_zero_amd import synth, zcmoe
from oracle import oracle
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu

LB_RTOL = 1e-12

LB_CASES = [
    # (name, T, N, Z, K, D, K_e, alpha, score std)
    ("small", 4096, 64, 32, 6, 8, 4.5, 0.01, 0.64),
    ("prefill", 16384, 512, 256, 12, 32, 8.0, 1e-3, 0.47),
    ("train", 8192, 128, 64, 8, 8, 6.0, 1e-3, 0.9),
    ("ragged", 65, 64, 32, 6, 4, 3.0, 1.0, 0.64),
    ("one_token", 1, 512, 256, 12, 8, 8.0, 1.0, 0.47),
    ("per_expert_groups", 500, 96, 0, 6, 96, 6.0, 1.0, 0.5),
    ("one_group_e1024", 300, 1024, 0, 32, 1, 32.0, 1.0, 0.5),
    ("e1024_mixed", 777, 768, 256, 16, 12, 12.0, 0.5, 0.5),
    ("k1", 333, 40, 24, 1, 5, 0.5, 2.0, 1.0),
]


def route_given(T, N, Z, K, std, seed):
    E = N + Z
    lg = synth.make_logits(T, E, std, seed)
    desc = zcmoe.LayerDesc(T, 64, N, Z, 64, K, torch.bfloat16)
    route = zcmoe.RouteBuffers(desc)
    route.logits.copy_(lg)
    bias = torch.zeros(E, device="cuda")
    zcmoe.zc_moe_route(desc, None, None, bias, route)
    torch.cuda.synchronize()
    o = oracle.route(lg.numpy(), np.zeros(E, np.float32), N, K, want_keys=False)
    np.testing.assert_array_equal(route.topk_idx.cpu().numpy(), o.topk_idx)
    np.testing.assert_array_equal(route.counts.cpu().numpy(), o.counts)
    return desc, route, lg.numpy(), o


@pytest.mark.parametrize("case", LB_CASES, ids=[c[0] for c in LB_CASES])
def test_lb_loss_matches_oracle(case):
    name, T, N, Z, K, D, K_e, alpha, std = case
    print(f"[lb] {name} T={T} N={N} Z={Z} K={K} D={D}", flush=True)
    desc, route, lg, o = route_given(T, N, Z, K, std, 31_000 + T)
    lb = zcmoe.LoadBalance(D, K_e, alpha)
    out = zcmoe.zc_moe_lb_loss(desc, lb, route).cpu().numpy()
    L, f, P, _ = oracle.lb_loss(lg, o.topk_idx, N, D, K_e, alpha, want_grad=False)
    np.testing.assert_array_equal(out[1:D + 2], f)
    np.testing.assert_allclose(out[D + 2:], P, rtol=LB_RTOL, atol=1e-300)
    assert abs(out[0] - L) <= LB_RTOL * abs(L), (out[0], L)


def test_lb_loss_is_deterministic_and_t0_gives_zeros():
    desc, route, _, _ = route_given(4096, 64, 32, 6, 0.64, 4242)
    lb = zcmoe.LoadBalance(4, 4.0, 0.1)
    a = zcmoe.zc_moe_lb_loss(desc, lb, route).cpu()
    b = zcmoe.zc_moe_lb_loss(desc, lb, route).cpu()
    assert torch.equal(a, b)
    d0 = zcmoe.LayerDesc(0, 64, 64, 32, 64, 6, torch.bfloat16)
    r0 = zcmoe.RouteBuffers(d0)
    z = zcmoe.zc_moe_lb_loss(d0, lb, r0, out=torch.full((11,), 7.0, dtype=torch.float64,
                                                           device="cuda")).cpu()
    assert torch.equal(z, torch.zeros(11, dtype=torch.float64))


def lb_backward_case(sh, lb, zero_dout=False, experts_checked=None):
    L = synth.make_layer(sh, "cpu")
    dY = synth.make_dy(sh)
    if zero_dout:
        dY = torch.zeros_like(dY)
    Lg = H.to_dev(L)
    desc = H.desc_of(sh)
    print(f"[lb backward] {sh.name} T={sh.T} D={lb.D} alpha={lb.alpha} zero_dout={zero_dout}",
          flush=True)
    route, _, saved = H.run_forward(desc, Lg, saved=True)
    g = {k: torch.empty_like(Lg[w]) for k, w in
         (("dx", "x"), ("dwr", "wr"), ("dwg", "wg"), ("dwu", "wu"), ("dwd", "wd"))}
    zcmoe.zc_moe_backward(desc, Lg["x"], Lg["wr"], Lg["wg"], Lg["wu"], Lg["wd"], route, saved,
                          dY.cuda(), g["dx"], g["dwr"], g["dwg"], g["dwu"], g["dwd"], lb=lb)
    torch.cuda.synchronize()
    xh, wrh = H.host(L["x"]), H.host(L["wr"])
    lg = oracle.logits(xh, wrh)
    o = oracle.route(lg, L["bias"].numpy(), sh.N, sh.K)
    _, namb = H.routing_agreement(route.topk_idx.cpu().numpy(), o.keys, o.topk_idx, lg, sh.K)
    assert namb == 0, "backward parity needs identical routing; pick another seed"
    _, _, _, dl = oracle.lb_loss(lg, o.topk_idx, sh.N, lb.D, lb.K_e, lb.alpha)
    ref = oracle.backward(xh, wrh, H.host(L["wg"]), H.host(L["wu"]), H.host(L["wd"]), lg,
                          o.topk_idx, o.gates, H.host(dY), sh.N, sh.Z, dl_extra=dl,
                          want_experts=experts_checked)
    dt = sh.torch_dtype
    errs = {"dx": H.assert_close(g["dx"], ref["dx"], dt, "dx"),
            "dwr": H.assert_close(g["dwr"], ref["dwr"], dt, "dW_r")}
    if not zero_dout:
        es = list(ref["dwg"].keys())
        got = g["dwg"][torch.tensor(es).cuda()]
        errs["dwg"] = H.assert_close(got, np.stack([ref["dwg"][e] for e in es]), dt, "dW_g")
    print("  errors " + ", ".join(f"{k} {v:.3e}" for k, v in errs.items()), flush=True)
    return ref


def test_backward_lb_term_alone_fp32():
    # dout = 0: every router and input gradient comes from the loss alone
    ref = lb_backward_case(synth.CONFIGS["tiny_fp32"], zcmoe.LoadBalance(4, 1.5, 5.0),
                           zero_dout=True)
    assert np.abs(ref["dwr"]).max() > 0


def test_backward_lb_fp32():
    lb_backward_case(synth.CONFIGS["tiny_fp32"], zcmoe.LoadBalance(2, 1.5, 2.0))


def test_backward_lb_train_shape_bf16():
    sh = synth.CONFIGS["train_bf16"].with_T(256)
    lb_backward_case(sh, zcmoe.LoadBalance(synth.TRAIN_LB_D, synth.TRAIN_K_E, 0.5),
                     experts_checked=[0, 77])


def test_backward_lb_alone_train_shape_bf16():
    sh = synth.CONFIGS["train_bf16"].with_T(256)
    lb_backward_case(sh, zcmoe.LoadBalance(synth.TRAIN_LB_D, synth.TRAIN_K_E, 50.0),
                     zero_dout=True)
