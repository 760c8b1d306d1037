"""GPU parity of the FP8 (MXFP8) inference forward against the fp64 oracle.

Blockwise FP8 follows the LongCat deployment notes (expert GEMMs in FP8,
sensitive parts kept in higher precision), in the OCP Microscaling format
the gfx950 matrix cores scale natively: E4M3 codes, one E8M0 scale per 32
reduction steps.

Checks:
  - weight quantization: the packed codes and scales, unpacked with the
    layout documented in gemm_fwdq.hip, equal the oracle's MX quantization
    of the same bf16 weights bit for bit (+0 and -0 codes are the same value);
  - the layer forward against the oracle's FP8 forward (orc_forward_mx: x
    and h quantized the same way, the identity term on unquantized x), on
    tokens both sides route identically; the output with the bf16 tolerance
    of gpu_harness, and the FFN part (out minus the identity term) with the
    same bound relative to its own RMS;
  - edge cases: ragged and few rows per expert (32-row tiles), a single
    expert, all picks on identity experts, determinism;
  - the quantization's own distance to the bf16 oracle forward is reported.
"""
import dataclasses

import numpy as np
import pytest
import torch

from moe_layer_zero_amd import synth, zcmoe
from oracle import oracle
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu

CF = synth.CONFIGS


def flip_eps(d: int) -> float:
    """h' codes are decided on fp32 values whose last bits depend on the
    summation order of the gate/up dot products (d products each).  The
    oracle treats a and u as known to within this factor times the sum of
    their absolute products -- four standard deviations of a random walk of
    fp32 roundings -- and bounds the effect of every h code that could
    legitimately come out one code apart within that margin."""
    return 4.0 * d ** 0.5 * 2.0 ** -24


def unpack_codes(buf: np.ndarray, N: int, R: int, C: int):
    """Codes [N][R][C] and scales [N][R][C/32] from a quantized weight set."""
    n = N * R * C
    q = buf[:n].reshape(N, R // 32, C // 128, 2, 2, 2, 32, 16)   # g t step half h lane16 byte
    # element (r, c): r = 32 g + l, c = 128 t + 64 step + 32 half + 16 h + byte
    codes = q.transpose(0, 1, 6, 2, 3, 4, 5, 7).reshape(N, R, C)
    s = buf[n:n + n // 32].reshape(N, R // 32, C // 128, 2, 32, 2)  # g t hh l byte
    # word (lane l + 32 hh) = (block 4t + hh, block 4t + 2 + hh)
    sc = np.empty((N, R // 32, 32, C // 128, 4), np.uint8)
    for hh in range(2):
        for byte in range(2):
            sc[:, :, :, :, hh + 2 * byte] = s[:, :, :, hh, :, byte].transpose(0, 1, 3, 2)
    return codes, sc.reshape(N, R, C // 32)


def same_codes(a: np.ndarray, b: np.ndarray) -> bool:
    z = lambda c: np.where((c & 0x7f) == 0, 0, c)   # noqa: E731  (+0 == -0)
    return np.array_equal(z(a), z(b))


@pytest.mark.parametrize("which", [zcmoe.ZC_PACK_GATE_UP, zcmoe.ZC_PACK_DOWN])
def test_quantize_weights_matches_oracle(which):
    sh = CF["small_bf16"]
    desc = H.desc_of(sh)
    L = synth.make_layer(sh, "cpu")
    w = L["wg"] if which == zcmoe.ZC_PACK_GATE_UP else L["wd"]
    N, R, C = w.shape
    buf = zcmoe.zc_moe_quantize_weights(desc, which, w.cuda())
    torch.cuda.synchronize()
    codes, scales = unpack_codes(buf.cpu().numpy(), N, R, C)
    for e in (0, 1, N // 2, N - 1):
        oc, os_ = oracle.mx_quantize(H.host(w[e]))
        assert same_codes(codes[e], oc), f"expert {e}: codes differ"
        np.testing.assert_array_equal(scales[e], os_)
    # a spread of magnitudes per block, down to bf16 subnormal-range values
    g = torch.Generator().manual_seed(5)
    w2 = (torch.randn((2, 512, 512), generator=g) *
          torch.exp(torch.empty(2, 512, 1).uniform_(-30, 10, generator=g))).to(torch.bfloat16)
    d2 = zcmoe.LayerDesc(8, 512, 2, 0, 512, 1, torch.bfloat16)
    buf2 = zcmoe.zc_moe_quantize_weights(d2, which, w2.cuda())
    torch.cuda.synchronize()
    c2, s2 = unpack_codes(buf2.cpu().numpy(), 2, 512, 512)
    for e in range(2):
        oc, os_ = oracle.mx_quantize(H.host(w2[e]))
        assert same_codes(c2[e], oc)
        np.testing.assert_array_equal(s2[e], os_)


def run_mx(desc, Lg):
    qg, qu, qd = zcmoe.quantize_expert_weights(desc, Lg["wg"], Lg["wu"], Lg["wd"])
    dq = dataclasses.replace(desc, weight_layout=zcmoe.ZC_WEIGHTS_MXFP8)
    route = zcmoe.RouteBuffers(dq)
    out = torch.empty((desc.T, desc.d), dtype=desc.dtype, device="cuda")
    zcmoe.zc_moe_forward(dq, Lg["x"], Lg["wr"], Lg["bias"], qg, qu, qd, out, route)
    torch.cuda.synchronize()
    return route, out


def check_case(sh, Lg, route, out, toks, n_out=None, bias=None):
    """Oracle FP8 forward on the listed tokens that route identically."""
    xh = H.host(Lg["x"][torch.from_numpy(toks).cuda()])
    lg = oracle.logits(xh, H.host(Lg["wr"]))
    H.assert_logits(route.logits[torch.from_numpy(toks).cuda()], lg)
    b = (Lg["bias"] if bias is None else bias).cpu().numpy()
    o = oracle.route(lg, b, sh.N, sh.K)
    same, namb = H.routing_agreement(route.topk_idx.cpu().numpy()[toks], o.keys, o.topk_idx, lg,
                                     sh.K)
    pick = [i for i in range(len(toks)) if same[i]][:n_out]
    experts = sorted({int(e) for i in pick for e in o.topk_idx[i] if e < sh.N})
    wq = {k: {e: oracle.mx_weights(H.host(Lg[k][e])) for e in experts} for k in ("wg", "wu", "wd")}
    ref, ys = oracle.forward_mx(xh, wq["wg"], wq["wu"], wq["wd"], o.topk_idx, o.gates, sh.N,
                                toks=pick, want_y=True)
    # the tolerance helper: output change that h codes decided within the
    # fp32 uncertainty of h may cause (the oracle decides on binary64 h)
    flip = oracle.mx_flip_bound(xh, wq["wg"], wq["wu"], wq["wd"], o.topk_idx, o.gates, sh.N,
                                flip_eps(sh.d), toks=pick)
    got = out[torch.from_numpy(toks[pick]).cuda()]
    g64 = H.f64(got)
    # the output: the bf16 bound of gpu_harness plus the near-tie allowance
    rms_out = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
    err = H._bounded(np.abs(g64 - ref), rms_out, 0.5 * H.bf16_ulp(ref), "FP8 layer output",
                     flip) if ref.size else 0.0
    # the FFN part alone: the identity term (same x, same gates) removed
    ffn_err = H.assert_ffn_part(got, ref, o.topk_idx[pick], o.gates[pick], sh.N, xh[pick],
                                "FP8 layer output", ys.reshape(len(pick), sh.K, sh.d),
                                flip=flip) if ref.size else 0.0
    if ref.size:
        print(f"  flip allowance max {float(flip.max()):.3e} (absolute)", flush=True)
    print(f"  ambiguous {namb}/{len(toks)}, checked {len(pick)} tokens over {len(experts)} "
          f"experts: err {err:.3e}, FFN-part err {ffn_err:.3e} of its RMS", flush=True)
    return o, pick, experts, ref


def small_case(sh, n_out=None, bias=None):
    L = synth.make_layer(sh, "cpu")
    if bias is not None:
        L["bias"] = bias
    Lg = H.to_dev(L)
    desc = H.desc_of(sh)
    print(f"[fp8 forward] {sh.name} T={sh.T}", flush=True)
    route, out = run_mx(desc, Lg)
    toks = np.arange(sh.T)
    return (Lg, route, out) + check_case(sh, Lg, route, out, toks, n_out)


def test_fp8_forward_small():
    small_case(CF["small_bf16"].with_T(700))


def test_fp8_forward_ragged_few_rows_per_expert():
    # about 9 rows per expert: 32-row tiles, ragged tails everywhere
    small_case(CF["small_bf16"].with_T(97), bias=torch.zeros(CF["small_bf16"].E))


def test_fp8_forward_single_expert():
    sh = synth.LayerShape("mlp512", 9, 300, 512, 1, 0, 512, 1, "bf16", 0.05, "zero")
    small_case(sh)


def test_fp8_forward_all_zero_computation_picks():
    sh = CF["small_bf16"].with_T(200)
    b = torch.zeros(sh.E)
    b[sh.N:] = 1.0
    Lg, route, out, *_ = small_case(sh, bias=b)
    assert route.offsets[-1].item() == 0
    torch.testing.assert_close(out.float(), Lg["x"].float(), rtol=1e-2, atol=0)


def test_fp8_forward_is_deterministic():
    sh = CF["small_bf16"].with_T(1024)
    Lg = H.to_dev(synth.make_layer(sh, "cpu"))
    desc = H.desc_of(sh)
    _, a = run_mx(desc, Lg)
    _, b = run_mx(desc, Lg)
    assert torch.equal(a, b)


@pytest.mark.parametrize("d,I", [(512, 1024), (512, 2048), (1536, 512), (2048, 1024)])
def test_fp8_forward_256_row_tiles_on_any_grid(d, I):
    # about 1000 rows per expert: 256-row tiles.  The down projection
    # (reduction I, at least 8 slabs of 128) loads the next tile's first
    # slabs under the current one's last slabs and epilogue: the smallest
    # reduction it takes and 16 slabs (the prefill layer's I = 2048); the
    # gate/up projection with reductions of 4, 12 and 16 slabs.  A token in
    # every 32-row stretch of every expert against the oracle, then the
    # same bits on grids of 64 and 8 workgroups, where each workgroup runs
    # many tiles back to back.
    sh = synth.LayerShape(f"fp8_pipe_d{d}_i{I}", 11, 3000, d, 8, 4, I, 4, "bf16", 0.05, "zero")
    Lg = H.to_dev(synth.make_layer(sh, "cpu"))
    desc = H.desc_of(sh)
    print(f"[fp8 forward] {sh.name} T={sh.T}", flush=True)
    route, out = run_mx(desc, Lg)
    toks = H.covering_tokens(route.topk_idx.cpu().numpy(), sh.N, 32, seed=5)
    check_case(sh, Lg, route, out, toks)
    for lim in (64, 8):
        print(f"[fp8 forward] {sh.name} cu_limit={lim}", flush=True)
        _, b = run_mx(dataclasses.replace(desc, cu_limit=lim), Lg)
        assert torch.equal(out, b)


def big_case(sh, n_logit_tok=128, n_out_tok=16):
    print(f"[fp8 forward-big] {sh.name} T={sh.T}", flush=True)
    Lg = synth.make_layer(sh, "cuda")
    desc = H.desc_of(sh)
    route, out = run_mx(desc, Lg)
    g = torch.Generator().manual_seed(321)
    toks = torch.randperm(sh.T, generator=g)[: min(n_logit_tok, sh.T)].sort().values.numpy()
    o, pick, experts, ref = check_case(sh, Lg, route, out, toks, n_out_tok)
    # distance of the FP8 layer to the bf16 oracle forward on the same tokens
    wb = {k: {e: H.host(Lg[k][e]) for e in experts} for k in ("wg", "wu", "wd")}
    xh = H.host(Lg["x"][torch.from_numpy(toks).cuda()])
    ref16 = oracle.forward(xh, wb["wg"], wb["wu"], wb["wd"], o.topk_idx, o.gates, sh.N, toks=pick)
    rel = float(np.sqrt(np.mean((ref - ref16) ** 2) / np.mean(ref16 ** 2)))
    print(f"  FP8 vs bf16 forward (oracle, same tokens): relative RMS {rel:.3e}", flush=True)
    assert rel < 0.05
    del Lg
    torch.cuda.empty_cache()


@pytest.mark.timeout(600)
def test_fp8_forward_decode_full_size():
    big_case(CF["decode_bf16"])


@pytest.mark.timeout(600)
def test_fp8_forward_prefill_full_size():
    big_case(CF["prefill_bf16"])
