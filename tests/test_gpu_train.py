"""GPU parity of the training loop at the training workload's full size:
T=8192 tokens, d=2048, 128 SwiGLU experts (inner size 1024) + 64
zero-computation experts, top-8, bf16.  Each of 50 steps runs the layer's
forward and backward on fresh seeded inputs, then the Eq.(2) bias update
("LongCat-Flash Technical Report", section 2.1.1) toward K_e = 6 FFN experts
per token with mu = 1 (weights stay fixed: the bias is the only state).

Checks:
  - every step, bit for bit: the oracle's routing of the GPU's own fp32
    router scores under the GPU's bias b_s reproduces the GPU's picks,
    gates, counts, offsets, dispatch order and inverse map, and the
    oracle's Eq.(2) on the GPU's counts and b_s reproduces the GPU's
    b_{s+1};
  - the closed loop: the oracle's own trajectory (its fp64 router scores,
    its routing, its Eq.(2)) stays within 3 mu / (K T) of the GPU's bias at
    every step -- three tokens' worth of counts -- and the number of tokens
    routed differently is reported;
  - both loops converge: the mean number of FFN experts per token over
    steps 40..49 is within 1% of K_e (the page reports under 1% fluctuation);
  - forward and backward parity at steps 0, 1 and 49, on the routing the
    oracle takes from the GPU's scores: the output and its FFN part and dx
    on a token sample with a row in every 128-row stretch of every expert's
    dispatch segment; dW_g, dW_u, dW_d of 16 experts over all their tokens
    (the hottest, the coldest, one from each load-balance group of 16, and
    the rest spread over the load ranks); dW_r rows of three experts.
"""
import numpy as np
import pytest
import torch

from moe_layer_zero_amd import synth, zcmoe
from oracle import oracle
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu


@pytest.mark.timeout(900)
def test_training_loop_bias_trajectory_and_parity():
    sh = synth.CONFIGS["train_bf16"]
    T, N, Z, K, E = sh.T, sh.N, sh.Z, sh.K, sh.E
    mu, Ke = synth.TRAIN_MU, synth.TRAIN_K_E
    L = synth.make_layer(sh, "cuda")
    desc = H.desc_of(sh)
    route = zcmoe.RouteBuffers(desc)
    out = torch.empty((T, sh.d), dtype=torch.bfloat16, device="cuda")
    saved = zcmoe.saved_buffer(desc)
    grads = {k: torch.empty_like(L[w]) for k, w in (("dx", "x"), ("dwr", "wr"), ("dwg", "wg"),
                                                    ("dwu", "wu"), ("dwd", "wd"))}
    bias = torch.zeros(E, device="cuda")
    wr = H.host(L["wr"])
    w_host = {k: H.host(L[k]) for k in ("wg", "wu", "wd")}
    b_orc = np.zeros(E, np.float32)
    tol = 3.0 * mu / (K * T)
    m_gpu, m_orc, worst = [], [], 0.0
    for s in range(synth.TRAIN_STEPS):
        print(f"[train] step {s}", flush=True)
        x = synth.step_x(sh, s, "cuda")
        dY = synth.step_dy(sh, s, "cuda")
        b_before = bias.cpu().numpy().copy()
        zcmoe.zc_moe_forward(desc, x, L["wr"], bias, L["wg"], L["wu"], L["wd"], out, route, saved)
        zcmoe.zc_moe_backward(desc, x, L["wr"], L["wg"], L["wu"], L["wd"], route, saved, dY,
                              grads["dx"], grads["dwr"], grads["dwg"], grads["dwu"], grads["dwd"])
        zcmoe.zc_moe_pid_update(N, Z, K, route.counts, T, mu, Ke, bias)
        torch.cuda.synchronize()
        m_gpu.append(route.offsets[-1].item() / T)

        # bit-exact step: routing of the GPU's scores under b_s, then Eq.(2)
        lg_gpu = route.logits.cpu().numpy()
        og = oracle.route(lg_gpu, b_before, N, K, want_keys=False)
        gidx = route.topk_idx.cpu().numpy()
        np.testing.assert_array_equal(gidx, og.topk_idx)
        np.testing.assert_array_equal(route.topk_gate.cpu().numpy(), og.gates.astype(np.float32))
        counts = route.counts.cpu().numpy()
        np.testing.assert_array_equal(counts, og.counts)
        np.testing.assert_array_equal(route.offsets.cpu().numpy(), og.offsets)
        np.testing.assert_array_equal(route.perm.cpu().numpy()[: og.p_real], og.perm)
        np.testing.assert_array_equal(route.inv.cpu().numpy(), og.inv)
        np.testing.assert_array_equal(bias.cpu().numpy(),
                                      oracle.pid_update(counts, T, b_before, N, Z, K, mu, Ke))

        # closed loop on the oracle's own scores
        xh = H.host(x)
        lg = oracle.logits(xh, wr)
        o = oracle.route(lg, b_orc, N, K, want_keys=False)
        m_orc.append(o.p_real / T)
        flips = int((gidx != o.topk_idx).any(1).sum())
        if s in (0, 1, 49):
            H.assert_logits(route.logits, lg)
            step_parity(sh, L, w_host, dY, xh, wr, lg_gpu, og, route, out, grads)
        b_orc = oracle.pid_update(o.counts, T, b_orc, N, Z, K, mu, Ke)
        diff = float(np.abs(bias.cpu().numpy() - b_orc).max())
        worst = max(worst, diff)
        print(f"  bit-exact ok; mean FFN experts gpu {m_gpu[-1]:.4f} oracle {m_orc[-1]:.4f}, "
              f"tokens routed differently {flips}, max|db| {diff:.3e} (tol {tol:.3e})",
              flush=True)
        assert diff <= tol, f"step {s}: bias trajectories apart by {diff:.3e} > {tol:.3e}"
    for m in (m_gpu, m_orc):
        late = float(np.mean(m[40:]))
        assert abs(late - Ke) < 0.01 * Ke, f"mean FFN experts over steps 40..49 = {late:.4f}"
    print(f"  worst bias gap {worst:.3e}; late means gpu {np.mean(m_gpu[40:]):.4f} "
          f"oracle {np.mean(m_orc[40:]):.4f}", flush=True)


def pick_experts(counts: np.ndarray, N: int, groups: int, n: int = 16):
    """The hottest and the coldest expert, the median-load member of each
    load-balance group, then experts at evenly spaced load ranks until n
    are chosen."""
    order = [int(e) for e in np.argsort(-counts[:N], kind="stable")]
    chosen = {order[0], order[-1]}
    G = N // groups
    for g in range(groups):
        members = sorted(range(g * G, (g + 1) * G), key=lambda e: (-counts[e], e))
        chosen.add(members[len(members) // 2])
    for k in range(4 * n):
        if len(chosen) >= n:
            break
        chosen.add(order[round(k * (N - 1) / (4 * n - 1))])
    return sorted(chosen)


def step_parity(sh, L, w_host, dY, xh, wr, lg_gpu, og, route, out, grads):
    """Forward/backward parity of one training step on the routing the oracle
    takes from the GPU's scores (identical to the GPU's, checked above)."""
    N, Z, K, T = sh.N, sh.Z, sh.K, sh.T
    dYh = H.host(dY)
    gidx = route.topk_idx.cpu().numpy()
    toks = H.covering_tokens(gidx, N, 128, seed=77)
    tk = torch.from_numpy(toks).cuda()
    wg, wu, wd = w_host["wg"], w_host["wu"], w_host["wd"]
    ref_out, ys = oracle.forward(xh, wg, wu, wd, og.topk_idx, og.gates, N, toks=toks,
                                 want_y=True)
    got = out[tk]
    H.assert_close(got, ref_out, torch.bfloat16, "layer output")
    H.assert_ffn_part(got, ref_out, og.topk_idx[toks], og.gates[toks], N, xh[toks],
                      "layer output", ys)
    rb = oracle.backward(xh, wr, wg, wu, wd, lg_gpu, og.topk_idx, og.gates, dYh, N, Z, toks=toks,
                         want_experts=[], want_dwr=False)
    H.assert_close(grads["dx"][tk], rb["dx"], torch.bfloat16, "dx")
    counts = og.counts
    experts = pick_experts(counts, N, synth.TRAIN_LB_D)
    assert len(experts) >= 16
    re = oracle.backward(xh, wr, {e: wg[e] for e in experts}, {e: wu[e] for e in experts},
                         {e: wd[e] for e in experts}, lg_gpu, og.topk_idx, og.gates, dYh, N, Z,
                         want_experts=experts, want_dwr=False, want_dx=False)
    for name, key in (("dwg", "dW_g"), ("dwu", "dW_u"), ("dwd", "dW_d")):
        for e in experts:
            H.assert_close(grads[name][e], re[name][e], torch.bfloat16, f"{key}[{e}]")
    # dW_r rows of three experts sum over exactly the tokens that picked them
    order = np.argsort(-counts[:N], kind="stable")
    rows = [int(order[0]), int(order[N // 2]), int(order[-1])]
    etoks = np.flatnonzero(np.isin(og.topk_idx, rows).any(1))
    need = sorted({int(e) for e in og.topk_idx[etoks].ravel() if e < N})
    rr = oracle.backward(xh, wr, {e: wg[e] for e in need}, {e: wu[e] for e in need},
                         {e: wd[e] for e in need}, lg_gpu, og.topk_idx, og.gates, dYh, N, Z,
                         toks=etoks, want_experts=[], want_dwr=True)
    for e in rows:
        H.assert_close(grads["dwr"][e], rr["dwr"][e], torch.bfloat16, f"dW_r[{e}]")
    print(f"  step parity ok: {len(toks)} tokens (every 128-row stretch), dW of experts "
          f"{experts} ({[int(counts[e]) for e in experts]} tokens), dW_r rows {rows}",
          flush=True)
