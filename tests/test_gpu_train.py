"""GPU parity of the training loop at the training workload's full size:
T=8192 tokens, d=2048, 128 SwiGLU experts (inner size 1024) + 64
zero-computation experts, top-8, bf16.  Each of 50 steps runs the layer's
forward and backward on fresh seeded inputs, then the Eq.(2) bias update
("LongCat-Flash Technical Report", section 2.1.1) toward K_e = 6 FFN experts
per token with mu = 1 (weights stay fixed: the bias is the only state).

Checks:
  - the GPU bias trajectory follows the oracle's closed loop (its own fp64
    router scores, its own routing and Eq.(2)): max |b_gpu - b_oracle| stays
    within a few tokens' worth of counts, mu * 4 / (K * T), at every step;
    the number of tokens routed differently is reported;
  - both loops converge: the mean number of FFN experts per token over
    steps 40..49 is within 1% of K_e (the page reports under 1% fluctuation);
  - forward and backward parity at steps 0, 1 and 49 on sampled tokens and
    experts (outputs, dx rows, dW of sampled experts over all their tokens,
    dW_r rows of sampled experts).
"""
import numpy as np
import pytest
import torch

from moe_layer_zero_amd import synth, zcmoe
from oracle import oracle
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu


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
    b_orc = np.zeros(E, np.float32)
    tol = 4.0 * mu / (K * T)
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

        xh = H.host(x)
        lg = oracle.logits(xh, wr)
        o = oracle.route(lg, b_orc, N, K, want_keys=s in (0, 1, 49))
        m_orc.append(o.p_real / T)
        flips = int((route.topk_idx.cpu().numpy() != o.topk_idx).any(1).sum())
        if s in (0, 1, 49):
            step_parity(sh, L, x, dY, xh, wr, lg, o, route, out, grads, b_before, b_orc)
        b_orc = oracle.pid_update(o.counts, T, b_orc, N, Z, K, mu, Ke)
        diff = float(np.abs(bias.cpu().numpy() - b_orc).max())
        worst = max(worst, diff)
        print(f"  mean FFN experts gpu {m_gpu[-1]:.4f} oracle {m_orc[-1]:.4f}, tokens routed "
              f"differently {flips}, max|db| {diff:.3e} (tol {tol:.3e})", flush=True)
        assert diff <= tol, f"step {s}: bias trajectories apart by {diff:.3e} > {tol:.3e}"
    for m in (m_gpu, m_orc):
        late = float(np.mean(m[40:]))
        assert abs(late - Ke) < 0.01 * Ke, f"mean FFN experts over steps 40..49 = {late:.4f}"
    print(f"  worst bias gap {worst:.3e}; late means gpu {np.mean(m_gpu[40:]):.4f} "
          f"oracle {np.mean(m_orc[40:]):.4f}", flush=True)


def step_parity(sh, L, x, dY, xh, wr, lg, o, route, out, grads, b_gpu, b_orc):
    """Forward/backward parity of one training step on samples the oracle can
    afford: 16 tokens (outputs and dx), 3 experts (dW over all their tokens),
    and the router rows of those experts."""
    N, Z, K = sh.N, sh.Z, sh.K
    # the two loops' biases differ by at most the trajectory tolerance; that
    # gap widens the near-tie margin of the routing comparison
    db = float(np.abs(b_gpu - b_orc).max())
    H.assert_logits(route.logits, lg)
    same, namb = H.routing_agreement(route.topk_idx.cpu().numpy(), o.keys, o.topk_idx, lg, K,
                                     extra_margin=2.0 * db)
    g = torch.Generator().manual_seed(77)
    toks = [int(t) for t in torch.randperm(sh.T, generator=g)[:64] if same[int(t)]][:16]
    counts = o.counts[:N]
    # experts whose gradients both sides must agree on: none of their tokens
    # may be one of the (validated) near-tie tokens routed differently
    gidx = route.topk_idx.cpu().numpy()
    touched = {int(e) for t in np.flatnonzero(~same) for e in (*o.topk_idx[t], *gidx[t])}
    order = np.argsort(-counts, kind="stable")
    clean = [int(e) for e in order if int(e) not in touched]
    experts = [clean[0], clean[len(clean) // 2], clean[-1]]
    # tokens of the sampled experts (for their full weight gradients)
    etoks = sorted({t for t in range(sh.T) for r in range(K) if o.topk_idx[t, r] in experts})
    assert all(same[t] for t in etoks)
    need = sorted({int(e) for t in set(toks) | set(etoks) for e in o.topk_idx[t] if e < N})
    wg = {e: H.host(L["wg"][e]) for e in need}
    wu = {e: H.host(L["wu"][e]) for e in need}
    wd = {e: H.host(L["wd"][e]) for e in need}
    dYh = H.host(dY)
    ref_out = oracle.forward(xh, wg, wu, wd, o.topk_idx, o.gates, N, toks=toks)
    H.assert_close(out[torch.tensor(toks).cuda()], ref_out, torch.bfloat16, "layer output")
    rb = oracle.backward(xh, wr, wg, wu, wd, lg, o.topk_idx, o.gates, dYh, N, Z, toks=toks,
                         want_experts=[], want_dwr=False)
    H.assert_close(grads["dx"][torch.tensor(toks).cuda()], rb["dx"], torch.bfloat16, "dx")
    re = oracle.backward(xh, wr, wg, wu, wd, lg, o.topk_idx, o.gates, dYh, N, Z, toks=etoks,
                         want_experts=experts, want_dwr=True)
    for name, key in (("dwg", "dW_g"), ("dwu", "dW_u"), ("dwd", "dW_d")):
        for e in experts:
            H.assert_close(grads[name][e], re[name][e], torch.bfloat16, f"{key}[{e}]")
    # dW_r rows of the sampled experts sum over exactly the tokens that picked them
    for e in experts:
        H.assert_close(grads["dwr"][e], re["dwr"][e], torch.bfloat16, f"dW_r[{e}]")
    print(f"  step parity ok: {len(toks)} tokens, experts {experts} "
          f"({[int(counts[e]) for e in experts]} tokens), ambiguous {namb}", flush=True)
