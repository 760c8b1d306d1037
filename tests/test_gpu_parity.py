"""GPU parity: the HIP layer, called through the C ABI, against the fp64
oracle on the same seeded inputs (tolerances in gpu_harness).

Layer: "LongCat-Flash Technical Report", section 2.1, Eq.(1) (router,
biased top-K, unbiased gates, zero-computation experts returning x) and
section 2.1.1, Eq.(2) (bias update).  Shapes are the five workloads of
moe_layer_zero_amd.synth plus edge cases (one token, ragged token counts,
K = 1, K = E, E = 1024, no FFN experts, no zero-computation experts).
"""
import numpy as np
import pytest
import torch

from moe_layer_zero_amd import synth, zcmoe
from oracle import oracle
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu

CF = synth.CONFIGS


def logit_std(sh):
    return sh.w_std * sh.d ** 0.5


# ------------------------------------------------------------ routing from given scores
ROUTE_CASES = [
    # (name, T, N, Z, K, bias kind, std, gate_norm)
    ("tiny", 64, 8, 4, 2, "zero", 0.23, 1),
    ("tiny_literal", 64, 8, 4, 2, "uniform", 0.23, 0),
    ("small", 4096, 64, 32, 6, "uniform", 0.64, 1),
    ("decode", 256, 512, 256, 12, "zero", 0.47, 1),
    ("prefill", 16384, 512, 256, 12, "zipf", 0.47, 1),
    ("train", 8192, 128, 64, 8, "zero", 0.9, 1),
    ("one_token", 1, 512, 256, 12, "zipf", 0.47, 1),
    ("ragged", 65, 64, 32, 6, "uniform", 0.64, 1),
    ("k1", 333, 40, 24, 1, "uniform", 1.0, 1),
    ("k_eq_e", 100, 9, 3, 12, "uniform", 1.0, 1),
    ("e1024", 300, 1024, 0, 32, "uniform", 0.5, 1),
    ("no_ffn", 200, 0, 16, 4, "uniform", 0.5, 1),
    ("no_identity", 500, 96, 0, 6, "uniform", 0.5, 0),
    ("ties", 128, 24, 8, 5, "ties", 0.5, 1),
    # eight slots per lane with a partial last one, ties in bias and scores
    ("e400_ties", 700, 300, 100, 10, "ties", 0.5, 1),
    # every expert picked: the last rounds find one free slot in the wave
    ("k_eq_e32", 64, 20, 12, 32, "ties", 1.0, 0),
]


def make_bias(kind, N, Z, seed):
    E = N + Z
    g = torch.Generator().manual_seed(seed)
    if kind == "zero":
        return torch.zeros(E)
    if kind == "uniform":
        return torch.rand(E, generator=g) * 0.2 - 0.1
    if kind == "zipf":
        b = torch.zeros(E, dtype=torch.float64)
        b[:N] = synth.ZIPF_B0 * (torch.randperm(N, generator=g) + 1).double() ** -synth.ZIPF_S
        return b.float()
    if kind == "ties":  # groups of experts with identical bias
        return (torch.randint(0, 3, (E,), generator=g) * 0.01).float()
    raise ValueError(kind)


@pytest.mark.parametrize("case", ROUTE_CASES, ids=[c[0] for c in ROUTE_CASES])
def test_route_given_scores_is_bit_exact(case):
    name, T, N, Z, K, kind, std, gate_norm = case
    E = N + Z
    print(f"[route] {name} T={T} N={N} Z={Z} K={K}", flush=True)
    lg = synth.make_logits(T, E, std, 7_000 + T)
    if kind == "ties":  # duplicate score columns as well
        lg[:, 1::4] = lg[:, 0::4][:, : lg[:, 1::4].shape[1]]
    bias = make_bias(kind, N, Z, 11 + T)
    desc = zcmoe.LayerDesc(T, 64, N, Z, 64, K, torch.bfloat16, gate_norm)
    route = zcmoe.RouteBuffers(desc)
    route.logits.copy_(lg)
    zcmoe.zc_moe_route(desc, None, None, bias.cuda(), route)
    torch.cuda.synchronize()
    o = oracle.route(lg.numpy(), bias.numpy(), N, K, gate_norm=gate_norm, want_keys=False)
    np.testing.assert_array_equal(route.topk_idx.cpu().numpy(), o.topk_idx)
    np.testing.assert_array_equal(route.topk_gate.cpu().numpy(), o.gates.astype(np.float32))
    np.testing.assert_array_equal(route.counts.cpu().numpy(), o.counts)
    np.testing.assert_array_equal(route.offsets.cpu().numpy(), o.offsets)
    P = o.p_real
    np.testing.assert_array_equal(route.perm.cpu().numpy()[:P], o.perm)
    np.testing.assert_array_equal(route.inv.cpu().numpy()[: T * K], o.inv)


def test_route_is_deterministic_and_t0_is_a_no_op():
    T, N, Z, K = 4096, 64, 32, 6
    desc = zcmoe.LayerDesc(T, 64, N, Z, 64, K, torch.bfloat16)
    lg = synth.make_logits(T, N + Z, 0.6, 99).cuda()
    bias = make_bias("uniform", N, Z, 5).cuda()
    outs = []
    for _ in range(2):
        r = zcmoe.RouteBuffers(desc)
        r.logits.copy_(lg)
        zcmoe.zc_moe_route(desc, None, None, bias, r)
        torch.cuda.synchronize()
        P = int(r.offsets[-1].item())
        outs.append([r.topk_idx.cpu(), r.topk_gate.cpu(), r.perm[:P].cpu(), r.inv.cpu()])
    for a, b in zip(*outs):
        assert torch.equal(a, b)
    d0 = zcmoe.LayerDesc(0, 64, N, Z, 64, K, torch.bfloat16)
    r0 = zcmoe.RouteBuffers(d0)
    zcmoe.zc_moe_route(d0, None, None, bias, r0)
    torch.cuda.synchronize()
    assert r0.counts.sum().item() == 0 and r0.offsets.abs().sum().item() == 0


# ------------------------------------------------------------ Eq.(2)
@pytest.mark.parametrize("N,Z,K,T,mu,Ke", [(128, 64, 8, 8192, 1.0, 6.0), (512, 256, 12, 256, 0.3, 8.0),
                                          (7, 0, 3, 5, 2.5, 1.5)])
def test_pid_update_is_bit_exact(N, Z, K, T, mu, Ke):
    g = torch.Generator().manual_seed(N + T)
    counts = torch.randint(0, 2 * T * K // max(N + Z, 1) + 2, (N + Z,), generator=g, dtype=torch.int32)
    bias = torch.randn(N + Z, generator=g) * 0.01
    b = bias.cuda()
    zcmoe.zc_moe_pid_update(N, Z, K, counts.cuda(), T, mu, Ke, b)
    torch.cuda.synchronize()
    want = oracle.pid_update(counts.numpy(), T, bias.numpy(), N, Z, K, mu, Ke)
    np.testing.assert_array_equal(b.cpu().numpy(), want)


# ------------------------------------------------------------ forward, small layers
def forward_case(sh, gate_norm=1, out_scale=1.0, bias=None, toks=None, packed=False):
    L = synth.make_layer(sh, "cpu")
    if bias is not None:
        L["bias"] = bias
    Lg = H.to_dev(L)
    desc = H.desc_of(sh, gate_norm, out_scale)
    print(f"[forward] {sh.name} T={sh.T} gate_norm={gate_norm} packed={packed}", flush=True)
    route, out, _ = H.run_forward(desc, Lg, packed=packed)
    xh, wrh = H.host(L["x"]), H.host(L["wr"])
    lg = oracle.logits(xh, wrh)
    H.assert_logits(route.logits, lg)
    o = oracle.route(lg, L["bias"].numpy(), sh.N, sh.K, gate_norm=gate_norm)
    same, namb = H.routing_agreement(route.topk_idx.cpu().numpy(), o.keys, o.topk_idx, lg, sh.K)
    sel = np.flatnonzero(same) if toks is None else np.array([t for t in toks if same[t]])
    ref, ys = oracle.forward(xh, H.host(L["wg"]), H.host(L["wu"]), H.host(L["wd"]), o.topk_idx,
                             o.gates, sh.N, out_scale=out_scale, toks=sel, want_y=True)
    got = out[torch.from_numpy(sel).cuda()]
    err = H.assert_close(got, ref, sh.torch_dtype, "layer output")
    ferr = H.assert_ffn_part(got, ref, o.topk_idx[sel], o.gates[sel], sh.N, xh[sel],
                             "layer output", ys, out_scale, dtype=sh.torch_dtype)
    print(f"  ambiguous tokens {namb}, checked {len(sel)}, err {err:.3e}, FFN part {ferr:.3e}",
          flush=True)
    return L, Lg, desc, route, out, o


def test_forward_tiny_fp32():
    forward_case(CF["tiny_fp32"])


def test_forward_tiny_fp32_literal_gates_and_scale():
    forward_case(CF["tiny_fp32"], gate_norm=0, out_scale=1.7)


def test_forward_small_bf16():
    forward_case(CF["small_bf16"])


def test_forward_ragged_bf16():
    # several row tiles per expert plus ragged tails
    sh = CF["small_bf16"].with_T(1000)
    forward_case(sh, bias=torch.zeros(sh.E))


def test_forward_all_zero_computation_picks():
    sh = CF["small_bf16"].with_T(300)
    b = torch.zeros(sh.E)
    b[sh.N:] = 1.0
    L, Lg, desc, route, out, o = forward_case(sh, bias=b)
    assert route.offsets[-1].item() == 0
    # out = (sum of gates = 1) * x, up to the fp32 gate sum and bf16 rounding
    torch.testing.assert_close(out.float(), Lg["x"].float(), rtol=1e-2, atol=0)


def test_forward_single_expert_mlp():
    sh = synth.LayerShape("mlp", 9, 200, 256, 1, 0, 128, 1, "bf16", 0.05, "zero")
    forward_case(sh)


def test_forward_more_than_sixteen_picks():
    # K = 20: the combine issues its picks' row loads in a group of 16, then
    # a group with 4 picks and 12 empty slots (bf16 row-major and packed, fp32)
    sh = synth.LayerShape("k20", 13, 300, 256, 24, 8, 256, 20, "bf16", 0.02, "uniform")
    forward_case(sh)
    forward_case(sh, packed=True)
    forward_case(synth.LayerShape("k20_f32", 14, 200, 128, 24, 8, 64, 20, "f32", 0.05, "uniform"))


def test_forward_dense_mixture_k_equals_e():
    sh = synth.LayerShape("dense", 9, 130, 128, 6, 2, 64, 8, "f32", 0.05, "uniform")
    forward_case(sh)


def test_forward_is_deterministic():
    sh = CF["small_bf16"]
    Lg = H.to_dev(synth.make_layer(sh, "cpu"))
    desc = H.desc_of(sh)
    _, a, _ = H.run_forward(desc, Lg)
    _, b, _ = H.run_forward(desc, Lg)
    assert torch.equal(a, b)


# ------------------------------------------------------------ forward, LongCat-Flash shapes
def big_case(sh, layouts=("rowmajor", "packed"), seed=123):
    """The LongCat-Flash layer ("LongCat-Flash Technical Report", section 2.4:
    d = 6144, 512 FFN experts of inner size 2048, 256 zero-computation
    experts, top-12) on both bf16 inference paths (row-major weights and the
    packed layout), checked on a token sample with a row in every 128-row
    stretch of every touched expert's dispatch segment -- every row tile of
    the grouped GEMMs holds a checked row -- or on every token of a batch of
    at most 256.  The output and, apart, its FFN part (out - c_t x_t: the
    identity term dominates RMS(out) at these shapes)."""
    print(f"[forward-big] {sh.name} T={sh.T} layouts={layouts}", flush=True)
    Lg = synth.make_layer(sh, "cuda")
    desc = H.desc_of(sh)
    runs = {}
    for lay in layouts:
        route, out, _ = H.run_forward(desc, Lg, packed=lay == "packed")
        runs[lay] = (route, out)
    route0 = runs[layouts[0]][0]
    for lay, (r, _) in runs.items():  # the same router and dispatch kernels
        assert torch.equal(r.topk_idx, route0.topk_idx) and torch.equal(r.offsets, route0.offsets)
    gidx = route0.topk_idx.cpu().numpy()
    toks = np.arange(sh.T) if sh.T <= 256 else H.covering_tokens(gidx, sh.N, 128, seed)
    tk = torch.from_numpy(toks).cuda()
    xh = H.host(Lg["x"][tk])
    lg = oracle.logits(xh, H.host(Lg["wr"]))
    H.assert_logits(route0.logits[tk], lg)
    o = oracle.route(lg, Lg["bias"].cpu().numpy(), sh.N, sh.K)
    same, namb = H.routing_agreement(gidx[toks], o.keys, o.topk_idx, lg, sh.K)
    pick = np.flatnonzero(same)
    experts = sorted({int(e) for e in o.topk_idx[pick].ravel() if e < sh.N})
    wg = {e: H.host(Lg["wg"][e]) for e in experts}
    wu = {e: H.host(Lg["wu"][e]) for e in experts}
    wd = {e: H.host(Lg["wd"][e]) for e in experts}
    ref, ys = oracle.forward(xh, wg, wu, wd, o.topk_idx, o.gates, sh.N, toks=pick, want_y=True)
    rows = tk[torch.from_numpy(pick).cuda()]
    for lay, (r, out) in runs.items():
        got = out[rows]
        err = H.assert_close(got, ref, sh.torch_dtype, f"layer output [{lay}]")
        ferr = H.assert_ffn_part(got, ref, o.topk_idx[pick], o.gates[pick], sh.N, xh[pick],
                                 f"layer output [{lay}]", ys)
        print(f"  {lay}: err {err:.3e} of RMS(out), FFN part {ferr:.3e} of its RMS", flush=True)
    touched = int((route0.counts[: sh.N] > 0).sum().item())
    print(f"  ambiguous {namb}/{len(toks)}, P_real {route0.offsets[-1].item()}, checked "
          f"{len(pick)} tokens over {len(experts)} of {touched} touched experts", flush=True)
    assert len(experts) == touched or namb > 0
    del Lg, runs
    torch.cuda.empty_cache()


def test_forward_decode_full_size():
    big_case(CF["decode_bf16"])


def test_forward_prefill_full_size():
    big_case(CF["prefill_bf16"])


# ------------------------------------------------------------ packed expert weights
def test_pack_weights_is_the_documented_permutation():
    g = torch.Generator(device="cuda").manual_seed(5)
    for which, shape in ((zcmoe.ZC_PACK_GATE_UP, (3, 512, 256)), (zcmoe.ZC_PACK_DOWN, (3, 256, 512))):
        desc = zcmoe.LayerDesc(64, 256, 3, 1, 512, 2, torch.bfloat16)
        w = torch.randn(shape, generator=g, device="cuda").to(torch.bfloat16)
        p = torch.empty_like(w)
        zcmoe.zc_moe_pack_weights(desc, which, w, p)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(H.host(p), H.pack_ref(H.host(w)))


def test_forward_packed_small_bf16():
    forward_case(CF["small_bf16"], packed=True)


def test_forward_packed_ragged_and_literal_gates():
    sh = CF["small_bf16"].with_T(1000)
    forward_case(sh, gate_norm=0, out_scale=0.7, bias=torch.zeros(sh.E), packed=True)


def test_forward_packed_few_rows_per_expert():
    # decode-like: most experts get a handful of rows, most of every row tile
    # reads outside the activation buffer
    forward_case(CF["small_bf16"].with_T(40), packed=True)


def test_forward_packed_single_expert_mlp():
    sh = synth.LayerShape("mlp256", 9, 600, 256, 1, 0, 256, 1, "bf16", 0.05, "zero")
    forward_case(sh, packed=True)


@pytest.mark.parametrize("T", [300, 4096])
def test_forward_packed_all_zero_computation_picks(T):
    # 4096 tokens: the 256-row kernels, launched on an empty tile list
    sh = CF["small_bf16"].with_T(T)
    b = torch.zeros(sh.E)
    b[sh.N:] = 1.0
    L, Lg, desc, route, out, o = forward_case(sh, bias=b, packed=True)
    assert route.offsets[-1].item() == 0


def test_forward_packed_four_slab_down_tiles_on_any_grid():
    # I = 256: the 256-row down projection has four 64-step slabs per tile,
    # so the next tile's first three slabs load under the last three and the
    # epilogue; grids of 8 and 64 workgroups make each workgroup run many
    # such tiles back to back.  Every token against the oracle, then the
    # same bits on the smaller grids.
    import dataclasses
    sh = synth.LayerShape("down_k256", 10, 4096, 2048, 8, 4, 256, 4, "bf16", 0.02, "zero")
    L, Lg, desc, route, out, o = forward_case(sh, packed=True)
    for lim in (64, 8):
        print(f"[forward] {sh.name} packed, cu_limit={lim}", flush=True)
        _, b, _ = H.run_forward(dataclasses.replace(desc, cu_limit=lim), Lg, packed=True)
        assert torch.equal(out, b)


def test_forward_packed_twelve_slab_gate_up_tiles_on_any_grid():
    # d = 768: the 256-row gate/up tiles have twelve 64-step slabs (a short
    # reduction next to the prefill's 96); grids of 8 and 64 workgroups make
    # each workgroup claim many tiles back to back, across the XCDs' counters.
    # Every token against the oracle, then the same bits on the smaller grids.
    import dataclasses
    sh = synth.LayerShape("gateup_k768", 11, 4096, 768, 8, 4, 256, 4, "bf16", 0.02, "zero")
    L, Lg, desc, route, out, o = forward_case(sh, packed=True)
    for lim in (64, 8):
        print(f"[forward] {sh.name} packed, cu_limit={lim}", flush=True)
        _, b, _ = H.run_forward(dataclasses.replace(desc, cu_limit=lim), Lg, packed=True)
        assert torch.equal(out, b)


def test_forward_packed_is_deterministic():
    sh = CF["small_bf16"]
    Lg = H.to_dev(synth.make_layer(sh, "cpu"))
    desc = H.desc_of(sh)
    _, a, _ = H.run_forward(desc, Lg, packed=True)
    _, b, _ = H.run_forward(desc, Lg, packed=True)
    assert torch.equal(a, b)


# ------------------------------------------------------------ backward
def backward_case(sh, gate_norm=1, out_scale=1.0, experts_checked=None, bias=None,
                  dwr_rows=None):
    L = synth.make_layer(sh, "cpu")
    if bias is not None:
        L["bias"] = bias
    nrep = H.replace_near_ties(L, sh.N, sh.K, gate_norm)
    dY = synth.make_dy(sh)
    Lg = H.to_dev(L)
    desc = H.desc_of(sh, gate_norm, out_scale)
    print(f"[backward] {sh.name} T={sh.T} gate_norm={gate_norm} (near-tie rows replaced: "
          f"{nrep})", flush=True)
    route, out, saved = H.run_forward(desc, Lg, saved=True)
    g = H.run_backward(desc, Lg, route, saved, dY.cuda())
    xh, wrh = H.host(L["x"]), H.host(L["wr"])
    lg = oracle.logits(xh, wrh)
    o = oracle.route(lg, L["bias"].numpy(), sh.N, sh.K, gate_norm=gate_norm)
    same, namb = H.routing_agreement(route.topk_idx.cpu().numpy(), o.keys, o.topk_idx, lg, sh.K)
    assert namb == 0, "backward parity needs identical routing; pick another seed"
    ref = oracle.backward(xh, wrh, H.host(L["wg"]), H.host(L["wu"]), H.host(L["wd"]), lg,
                          o.topk_idx, o.gates, H.host(dY), sh.N, sh.Z, gate_norm=gate_norm,
                          out_scale=out_scale, want_experts=experts_checked)
    dt = sh.torch_dtype
    errs = {"dx": H.assert_close(g["dx"], ref["dx"], dt, "dx")}
    if dwr_rows is None:
        errs["dwr"] = H.assert_close(g["dwr"], ref["dwr"], dt, "dW_r")
    else:
        # only these router rows receive gradient (renormalised gates give
        # the other experts' scores none): the bound on them, exact zeros
        # elsewhere, as for a subset of expert gradients
        rows = torch.tensor(dwr_rows)
        errs["dwr"] = H.assert_close(g["dwr"][rows.cuda()], ref["dwr"][dwr_rows], dt, "dW_r")
        rest = torch.ones(sh.E, dtype=torch.bool)
        rest[rows] = False
        assert not np.any(ref["dwr"][rest.numpy()])
        assert torch.count_nonzero(g["dwr"][rest.cuda()]).item() == 0
    es = list(ref["dwg"].keys())
    for name, key in (("dwg", "dW_g"), ("dwu", "dW_u"), ("dwd", "dW_d")):
        got = g[name][torch.tensor(es).cuda()]
        want = np.stack([ref[name][e] for e in es])
        errs[name] = H.assert_close(got, want, dt, key)
    print("  errors " + ", ".join(f"{k} {v:.3e}" for k, v in errs.items()), flush=True)
    return route, g


def test_backward_tiny_fp32():
    backward_case(CF["tiny_fp32"])


def test_backward_tiny_fp32_literal_gates():
    backward_case(CF["tiny_fp32"], gate_norm=0, out_scale=0.5)


def test_backward_fp32_long_batch_splits_router_gradient():
    # T = 1024 tokens: the router weight gradient is computed in 4 token chunks
    # whose fp32 partials are added in chunk order
    backward_case(CF["tiny_fp32"].with_T(1024))


# ------------------------------------------------------------ router scores, large batches
@pytest.mark.parametrize("T", [8192, 8292])
def test_router_scores_of_a_large_batch(T):
    """Large bf16 batches with E a multiple of 256 compute the router scores
    (section 2.1's logits = x W_r^T, fp32 accumulation) on the 256 x 256-tile
    kernel: against the oracle's binary64 scores within the logits bound, on
    an exact number of row tiles and on a ragged last one; and the routing
    of those scores is the oracle's bit for bit."""
    sh = synth.LayerShape("router_big", 41, T, 320, 768, 256, 64, 8, "bf16", 0.05, "uniform")
    assert sh.T * sh.E >= 1 << 23  # the size the tiled router takes
    L = synth.make_layer(sh, "cuda", want_experts=False)
    desc = H.desc_of(sh)
    route = zcmoe.RouteBuffers(desc)
    print(f"[router-big] T={T} E={sh.E} d={sh.d}", flush=True)
    zcmoe.zc_moe_route(desc, L["x"], L["wr"], L["bias"], route)
    torch.cuda.synchronize()
    lg = oracle.logits(H.host(L["x"]), H.host(L["wr"]))
    H.assert_logits(route.logits, lg)
    lg_gpu = route.logits.cpu().numpy()
    o = oracle.route(lg_gpu, L["bias"].cpu().numpy(), sh.N, sh.K, want_keys=False)
    np.testing.assert_array_equal(route.topk_idx.cpu().numpy(), o.topk_idx)
    np.testing.assert_array_equal(route.counts.cpu().numpy(), o.counts)


# ------------------------------------------------------------ training forward
def training_forward_case(sh, stride=7):
    """The forward that keeps its activations for the backward (bf16 layers
    with row-major weights run the training kernels): the layer output and
    its FFN part against the oracle on a token sample with a row in every
    128-row stretch of every expert's dispatch segment, and the saved fp32
    a = x W_g^T, u = x W_u^T, h = silu(a) u of every `stride`-th FFN pick in
    dispatch order (so every 32-row block of every row tile) and of the last
    row of every expert segment, against the oracle's binary64 values.
    Bounds: an fp32 sum of d exact bf16 products in any order is within
    gamma_d * sum |w x| (gamma_d = d u / (1 - d u), u = 2^-24); h carries
    that through silu (slope at most 1.1) plus 2^-20 |h| for its
    exponential, reciprocal and products."""
    L = synth.make_layer(sh, "cpu")
    Lg = H.to_dev(L)
    desc = H.desc_of(sh)
    print(f"[training-forward] {sh.name} T={sh.T}", flush=True)
    route, out, saved = H.run_forward(desc, Lg, saved=True)
    xh, wrh = H.host(L["x"]), H.host(L["wr"])
    wg, wu, wd = H.host(L["wg"]), H.host(L["wu"]), H.host(L["wd"])
    lg = oracle.logits(xh, wrh)
    H.assert_logits(route.logits, lg)
    o = oracle.route(lg, L["bias"].numpy(), sh.N, sh.K)
    gidx = route.topk_idx.cpu().numpy()
    same, namb = H.routing_agreement(gidx, o.keys, o.topk_idx, lg, sh.K)
    toks = np.array([t for t in H.covering_tokens(gidx, sh.N, 128, seed=5) if same[t]])
    ref, ys = oracle.forward(xh, wg, wu, wd, o.topk_idx, o.gates, sh.N, toks=toks, want_y=True)
    got = out[torch.from_numpy(toks).cuda()]
    H.assert_close(got, ref, torch.bfloat16, "layer output (training forward)")
    H.assert_ffn_part(got, ref, o.topk_idx[toks], o.gates[toks], sh.N, xh[toks],
                      "layer output (training forward)", ys)
    # saved activations of sampled picks: they depend only on x_t and W_e,
    # so the GPU's own routing names the picks
    offs = route.offsets.cpu().numpy()
    perm = route.perm.cpu().numpy()
    P = int(offs[sh.N])
    ends = offs[1:][offs[1:] > offs[:-1]] - 1
    rows = np.union1d(np.arange(0, P, stride), ends)
    tok = perm[rows] // sh.K
    ex = gidx[tok, perm[rows] % sh.K]
    assert (ex < sh.N).all()
    a, u, h = oracle.ffn_activations(xh, wg, wu, sh.N, tok, ex)
    sv = zcmoe.saved_views(desc, saved)
    ridx = torch.from_numpy(rows).cuda()
    ga, gu, gh = (sv[k][ridx].double().cpu().numpy() for k in ("a", "u", "h"))
    x64 = H.bf16_to_f64(xh)
    gamma = sh.d * 2.0 ** -24 / (1 - sh.d * 2.0 ** -24)
    worst = {"a": 0.0, "u": 0.0, "h": 0.0}
    for e in np.unique(ex):
        qs = np.flatnonzero(ex == e)
        xa = np.abs(x64[tok[qs]])                                   # [n][d]
        tol_a = gamma * (xa @ np.abs(H.bf16_to_f64(wg[e])).T) + 1e-30  # [n][I]
        tol_u = gamma * (xa @ np.abs(H.bf16_to_f64(wu[e])).T) + 1e-30
        tol_h = (1.1 * tol_a * (np.abs(u[qs]) + tol_u) + (np.abs(a[qs]) + tol_a) * tol_u
                 + 2.0 ** -20 * np.abs(h[qs]) + 1e-30)
        for k, g_, r_, t_ in (("a", ga, a, tol_a), ("u", gu, u, tol_u), ("h", gh, h, tol_h)):
            ratio = np.abs(g_[qs] - r_[qs]) / t_
            worst[k] = max(worst[k], float(ratio.max()))
            bad = np.argwhere(ratio > 1.0)
            assert len(bad) == 0, (f"saved {k} of dispatch row {rows[qs[bad[0][0]]]} (expert "
                                   f"{e}, column {bad[0][1]}): {float(ratio.max()):.3f} of its "
                                   f"bound")
    print(f"  {len(toks)} tokens, {len(rows)} saved rows; worst error / bound: "
          + ", ".join(f"{k} {v:.3f}" for k, v in worst.items()), flush=True)


@pytest.mark.parametrize("shape", ["small_bf16", "small_bf16_T300", "train_bf16_T1024"])
def test_training_forward_output_and_saved_activations(shape):
    sh = {"small_bf16": CF["small_bf16"], "small_bf16_T300": CF["small_bf16"].with_T(300),
          "train_bf16_T1024": CF["train_bf16"].with_T(1024)}[shape]
    training_forward_case(sh)


def test_backward_train_shape_bf16():
    # the training layer's shapes with fewer tokens, so the fp64 oracle
    # finishes in seconds; all 128 experts' gradients compared
    backward_case(CF["train_bf16"].with_T(256))


def test_backward_bf16_several_slabs_per_expert():
    # about 85 rows per FFN expert: the weight gradients reduce over several
    # 32-row slabs with a ragged last one; experts of every size checked
    sh = CF["train_bf16"].with_T(2048)
    backward_case(sh, experts_checked=[0, 1, 17, 64, 100, 127])


def test_backward_bf16_literal_gates_and_scale():
    backward_case(CF["small_bf16"].with_T(300), gate_norm=0, out_scale=0.5)


def test_backward_bf16_expert_without_rows():
    # expert 3 is never picked: its weight gradients are exactly zero
    sh = CF["train_bf16"].with_T(256)
    b = torch.zeros(sh.E)
    b[3] = -100.0
    route, g = backward_case(sh, experts_checked=[2, 3, 4], bias=b)
    cnt = route.offsets[4].item() - route.offsets[3].item()
    assert cnt == 0
    for k in ("dwg", "dwu", "dwd"):
        assert torch.count_nonzero(g[k][3]).item() == 0


def test_backward_bf16_64_row_tiles():
    # about 64 rows per FFN expert: the backward GEMMs run 64-row tiles
    sh = CF["train_bf16"].with_T(1024)
    backward_case(sh, experts_checked=[0, 5, 64, 127])


def test_backward_bf16_few_experts_take_every_token():
    # experts 0..K-1 are picked by every token (their bias exceeds any score
    # gap): 257 rows each, eight full 32-row slabs and a one-row tail in the
    # weight gradients; every other FFN expert gets no rows
    sh = CF["train_bf16"].with_T(257)
    b = torch.zeros(sh.E)
    b[: sh.K] = 1.0
    route, g = backward_case(sh, experts_checked=[0, sh.K - 1, sh.K], bias=b,
                             dwr_rows=list(range(sh.K)))
    off = route.offsets.cpu().numpy()
    assert all(off[e + 1] - off[e] == sh.T for e in range(sh.K))
    assert off[-1] == sh.T * sh.K
    for k in ("dwg", "dwu", "dwd"):
        assert torch.count_nonzero(g[k][sh.K:]).item() == 0


@pytest.mark.parametrize("shape", ["small_bf16", "tiny_fp32"])
def test_backward_with_no_tokens_gives_zero_weight_gradients(shape):
    # an empty batch: every weight gradient is exactly zero (written, not
    # left as it was), on the packed-weight path (bf16) and the generic one
    sh = CF[shape]
    Lg = H.to_dev(synth.make_layer(sh.with_T(0), "cpu"))
    desc = H.desc_of(sh.with_T(0))
    route, out, saved = H.run_forward(desc, Lg, saved=True)
    assert out.numel() == 0 and route.offsets.abs().sum().item() == 0
    dx = torch.empty_like(Lg["x"])
    g = {k: torch.full_like(Lg[w], float("nan")) for k, w in
         (("dwr", "wr"), ("dwg", "wg"), ("dwu", "wu"), ("dwd", "wd"))}
    zcmoe.zc_moe_backward(desc, Lg["x"], Lg["wr"], Lg["wg"], Lg["wu"], Lg["wd"], route, saved,
                          torch.empty_like(Lg["x"]), dx, g["dwr"], g["dwg"], g["dwu"], g["dwd"])
    torch.cuda.synchronize()
    for k, t in g.items():
        assert torch.count_nonzero(t).item() == 0, k


# d and I multiples of 64 but not of 256: the bf16 layer takes the generic
# grouped-GEMM backward (and the 256 x 256 row-major forward with partial
# column tiles)
BF16_ODD = synth.LayerShape("bf16_odd", 12, 300, 384, 16, 8, 192, 4, "bf16", 0.02, "uniform")


def test_forward_bf16_dims_not_multiple_of_256():
    forward_case(BF16_ODD)


def test_backward_bf16_dims_not_multiple_of_256():
    backward_case(BF16_ODD)


# ------------------------------------------------------------ non-finite inputs
def test_route_non_finite_scores_is_bit_exact_and_in_range():
    # NaN and infinite scores make every key of their token NaN; NaN keys rank
    # below every number on both sides, so such tokens pick 0..K-1
    T, N, Z, K = 96, 24, 8, 5
    E = N + Z
    lg = synth.make_logits(T, E, 0.5, 4242)
    lg[3, 7] = float("nan")
    lg[10, 2] = float("inf")
    lg[20, :] = float("-inf")
    lg[30, 5] = float("-inf")
    lg[40, :] = float("nan")
    bias = make_bias("uniform", N, Z, 9)
    bias[11] = float("nan")
    for gate_norm in (1, 0):
        print(f"[route non-finite] gate_norm={gate_norm}", flush=True)
        desc = zcmoe.LayerDesc(T, 64, N, Z, 64, K, torch.bfloat16, gate_norm)
        route = zcmoe.RouteBuffers(desc)
        route.logits.copy_(lg)
        zcmoe.zc_moe_route(desc, None, None, bias.cuda(), route)
        torch.cuda.synchronize()
        o = oracle.route(lg.numpy(), bias.numpy(), N, K, gate_norm=gate_norm, want_keys=False)
        idx = route.topk_idx.cpu().numpy()
        assert ((idx >= 0) & (idx < E)).all()
        for t in (10, 20, 40):
            assert list(idx[t]) == list(range(K))
        np.testing.assert_array_equal(idx, o.topk_idx)
        np.testing.assert_array_equal(route.topk_gate.cpu().numpy(), o.gates.astype(np.float32))
        np.testing.assert_array_equal(route.counts.cpu().numpy(), o.counts)
        np.testing.assert_array_equal(route.offsets.cpu().numpy(), o.offsets)
        np.testing.assert_array_equal(route.perm.cpu().numpy()[: o.p_real], o.perm)
        np.testing.assert_array_equal(route.inv.cpu().numpy(), o.inv)


@pytest.mark.parametrize("packed", [False, True])
def test_a_nan_input_row_stays_in_its_token(packed):
    # a NaN row of x: its scores are NaN, it picks experts 0..K-1, its output
    # (and, through the backward, its dx) is NaN; every other token is finite
    sh = CF["small_bf16"].with_T(300)
    L = synth.make_layer(sh, "cpu")
    L["x"][17] = float("nan")
    Lg = H.to_dev(L)
    desc = H.desc_of(sh)
    print(f"[nan row] packed={packed}", flush=True)
    route, out, saved = H.run_forward(desc, Lg, saved=not packed, packed=packed)
    idx = route.topk_idx.cpu()
    assert ((idx >= 0) & (idx < sh.E)).all()
    assert idx[17].tolist() == list(range(sh.K))
    rest = torch.ones(sh.T, dtype=torch.bool)
    rest[17] = False
    o = out.float().cpu()
    assert torch.isnan(o[17]).all()
    assert torch.isfinite(o[rest]).all()
    if not packed:
        g = H.run_backward(desc, Lg, route, saved, synth.make_dy(sh).cuda())
        dx = g["dx"].float().cpu()
        assert torch.isnan(dx[17]).all()
        assert torch.isfinite(dx[rest]).all()


# ------------------------------------------------------------ grid-size independence
def test_results_do_not_depend_on_the_grid_size():
    # every sum has a fixed order whichever workgroup computes it: the same
    # bits from persistent grids sized for 256, 64 and 136 compute units
    import dataclasses
    sh = CF["train_bf16"].with_T(2048)
    L = synth.make_layer(sh, "cpu")
    Lg = H.to_dev(L)
    dY = synth.make_dy(sh).cuda()
    ref = None
    for lim in (0, 64, 136):
        print(f"[grid] training shape, cu_limit={lim}", flush=True)
        desc = dataclasses.replace(H.desc_of(sh), cu_limit=lim)
        route, out, saved = H.run_forward(desc, Lg, saved=True)
        g = H.run_backward(desc, Lg, route, saved, dY)
        P = int(route.offsets[-1].item())
        got = [out, route.logits, route.topk_idx, route.topk_gate, route.counts, route.perm[:P],
               route.inv] + [g[k] for k in sorted(g)]
        if ref is None:
            ref = got
        else:
            for a, b in zip(ref, got):
                assert torch.equal(a, b)
    sq = CF["small_bf16"]
    Lq = H.to_dev(synth.make_layer(sq, "cpu"))
    ref = None
    for lim in (0, 64, 136):
        print(f"[grid] packed and FP8 inference, cu_limit={lim}", flush=True)
        desc = dataclasses.replace(H.desc_of(sq), cu_limit=lim)
        _, out_p, _ = H.run_forward(desc, Lq, packed=True)
        qg, qu, qd = zcmoe.quantize_expert_weights(desc, Lq["wg"], Lq["wu"], Lq["wd"])
        dq = dataclasses.replace(desc, weight_layout=zcmoe.ZC_WEIGHTS_MXFP8)
        rq = zcmoe.RouteBuffers(dq)
        out_q = torch.empty_like(out_p)
        zcmoe.zc_moe_forward(dq, Lq["x"], Lq["wr"], Lq["bias"], qg, qu, qd, out_q, rq)
        torch.cuda.synchronize()
        if ref is None:
            ref = (out_p, out_q)
        else:
            assert torch.equal(ref[0], out_p) and torch.equal(ref[1], out_q)
