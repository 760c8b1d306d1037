"""GPU parity of the budget-control variants ("LongCat-Flash Technical
Report", section 2.1.1): the per-token FFN-expert statistics the report
tracks (Fig.3b/3c) and the Eq.(2) update over counts accumulated across
micro-batches (a global batch, or a lower update frequency) with a decaying
mu, against the fp64 oracle.

Statistics: the histogram and the mean are integer work plus one division
and agree bit for bit; the standard deviation is summed in a different order
on each side and agrees to 1e-13 relative.  Closed loop: both sides route
the same seeded fp32 scores with their own (identical) biases, so the picks,
the accumulated counts and every bias after every update agree bit for bit.
"""
import numpy as np
import pytest
import torch

from moe_layer_zero_amd import synth, zcmoe
from oracle import oracle

pytestmark = pytest.mark.gpu

STATS_CASES = [
    # (name, T, N, Z, K, score std)
    ("prefill", 16384, 512, 256, 12, 0.47),
    ("decode", 256, 512, 256, 12, 0.47),
    ("train", 8192, 128, 64, 8, 0.9),
    ("one_token", 1, 512, 256, 12, 0.47),
    ("ragged", 1001, 64, 32, 6, 0.64),
    ("k1", 333, 40, 24, 1, 1.0),
    ("k32", 300, 768, 256, 32, 0.5),
    ("no_identity", 500, 96, 0, 6, 0.5),
    ("no_ffn", 200, 0, 16, 4, 0.5),
]


def route_given(desc, lg, bias):
    route = zcmoe.RouteBuffers(desc)
    route.logits.copy_(lg)
    zcmoe.zc_moe_route(desc, None, None, bias, route)
    return route


@pytest.mark.parametrize("case", STATS_CASES, ids=[c[0] for c in STATS_CASES])
def test_route_stats_match_oracle(case):
    name, T, N, Z, K, std = case
    print(f"[stats] {name} T={T} N={N} Z={Z} K={K}", flush=True)
    E = N + Z
    lg = synth.make_logits(T, E, std, 61_000 + T)
    bias = (torch.rand(E, generator=torch.Generator().manual_seed(T)) * 0.1 - 0.05)
    desc = zcmoe.LayerDesc(T, 64, N, Z, 64, K, torch.bfloat16)
    route = route_given(desc, lg, bias.cuda())
    hist, mom = zcmoe.zc_moe_route_stats(desc, route)
    torch.cuda.synchronize()
    o = oracle.route(lg.numpy(), bias.numpy(), N, K, want_keys=False)
    np.testing.assert_array_equal(route.topk_idx.cpu().numpy(), o.topk_idx)
    h, m, s = oracle.route_stats(o.topk_idx, N)
    mom = mom.cpu().numpy()
    np.testing.assert_array_equal(hist.cpu().numpy(), h)
    assert mom[0] == m, (mom[0], m)
    assert abs(mom[1] - s) <= 1e-13 * max(s, 1e-300), (mom[1], s)


def test_route_stats_empty_batch():
    desc = zcmoe.LayerDesc(0, 64, 64, 32, 64, 6, torch.bfloat16)
    r = zcmoe.RouteBuffers(desc)
    hist = torch.full((7,), 5, dtype=torch.int32, device="cuda")
    mom = torch.full((2,), 1.0, dtype=torch.float64, device="cuda")
    zcmoe.zc_moe_route_stats(desc, r, hist, mom)
    torch.cuda.synchronize()
    assert not hist.any() and not mom.any()


def test_micro_batch_accumulation_with_decaying_mu_is_bit_exact():
    """Eq.(2) applied once per 3 micro-batches over their summed counts
    (T_all = 3 T), mu decaying as mu_0 / (1 + s/10): 30 updates, the GPU and
    the oracle bias equal bit for bit after every update, and the mean
    number of FFN experts per token settles within 1% of K_e."""
    N, Z, K, T, Ke, n_micro = 128, 64, 8, 2048, 6.0, 3
    E = N + Z
    desc = zcmoe.LayerDesc(T, 64, N, Z, 64, K, torch.bfloat16)
    bias = torch.zeros(E, device="cuda")
    acc = torch.empty(E, dtype=torch.int32, device="cuda")
    b_orc = np.zeros(E, np.float32)
    means = []
    for s in range(30):
        mu = 1.0 / (1 + s / 10)
        acc.zero_()
        acc_orc = np.zeros(E, np.int64)
        for m in range(n_micro):
            lg = synth.make_logits(T, E, 0.9, 500_000 + 10 * s + m)
            route = route_given(desc, lg, bias)
            zcmoe.zc_moe_accumulate_counts(route.counts, acc)
            _, mom = zcmoe.zc_moe_route_stats(desc, route)
            o = oracle.route(lg.numpy(), b_orc, N, K, want_keys=False)
            acc_orc += o.counts
            _, m_orc, _ = oracle.route_stats(o.topk_idx, N)
            assert float(mom[0].item()) == m_orc
            means.append(m_orc)
        np.testing.assert_array_equal(acc.cpu().numpy(), acc_orc)
        zcmoe.zc_moe_pid_update(N, Z, K, acc, n_micro * T, mu, Ke, bias)
        b_orc = oracle.pid_update(acc_orc.astype(np.int32), n_micro * T, b_orc, N, Z, K, mu, Ke)
        np.testing.assert_array_equal(bias.cpu().numpy(), b_orc)
        if s % 10 == 9:
            print(f"  update {s}: mu {mu:.3f}, mean FFN experts {np.mean(means[-3:]):.4f}",
                  flush=True)
    late = float(np.mean(means[-30:]))
    assert abs(late - Ke) < 0.01 * Ke, late


def test_training_bias_resumes_bit_exactly_from_a_checkpoint(tmp_path):
    """The training workload's router and Eq.(2) loop on the GPU (T = 8192,
    128 + 64 experts, top-8, mu = 1, K_e = 6): stopped after 10 steps, the
    fp32 bias saved to disk, every buffer dropped, the bias read back into
    fresh buffers -- the next 10 steps give the same counts and biases bit
    for bit as the run that never stopped (the bias is the only state)."""
    sh = synth.CONFIGS["train_bf16"]
    L = synth.make_layer(sh, "cuda", want_experts=False)
    desc = zcmoe.LayerDesc(sh.T, sh.d, sh.N, sh.Z, sh.I, sh.K, torch.bfloat16)

    def steps(bias, s0, s1):
        route = zcmoe.RouteBuffers(desc)
        out = []
        for s in range(s0, s1):
            zcmoe.zc_moe_route(desc, synth.step_x(sh, s, "cuda"), L["wr"], bias, route)
            zcmoe.zc_moe_pid_update(sh.N, sh.Z, sh.K, route.counts, sh.T, synth.TRAIN_MU,
                                    synth.TRAIN_K_E, bias)
            torch.cuda.synchronize()
            out.append((route.counts.cpu().numpy().copy(), bias.cpu().numpy().copy()))
        return out

    whole = steps(torch.zeros(sh.E, device="cuda"), 0, 20)
    b = torch.zeros(sh.E, device="cuda")
    first = steps(b, 0, 10)
    np.save(tmp_path / "bias.npy", b.cpu().numpy())
    del b
    torch.cuda.synchronize()
    resumed = torch.from_numpy(np.load(tmp_path / "bias.npy")).cuda()
    second = steps(resumed, 10, 20)
    for (c1, b1), (c2, b2) in zip(whole, first + second):
        np.testing.assert_array_equal(c1, c2)
        np.testing.assert_array_equal(b1, b2)
    # and the loop converges toward K_e = 6 FFN experts per token
    late = np.mean([c[: sh.N].sum() / sh.T for c, _ in whole[15:]])
    assert abs(late - synth.TRAIN_K_E) < 0.05 * synth.TRAIN_K_E, late


def test_per_step_telemetry_lines(tmp_path):
    """bench.py --telemetry: one JSON line per training step with the
    budget-control statistics; checked against the oracle's statistics of
    the same routing for the first step and for consistency on all."""
    import importlib.util
    import json
    import os
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    spec = importlib.util.spec_from_file_location("bench_telemetry", os.path.join(root, "bench.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    path = str(tmp_path / "telemetry.jsonl")
    lines = b.train_telemetry(path, steps=6, T=1024)
    recs = [json.loads(l) for l in open(path)]
    assert recs == json.loads(json.dumps(lines)) and len(recs) == 6
    sh = synth.CONFIGS["train_bf16"]
    for r in recs:
        h = np.array(r["hist"])
        assert h.sum() == 1024 and len(h) == sh.K + 1
        assert abs((h * np.arange(sh.K + 1)).sum() / 1024 - r["mean_ffn_experts"]) < 1e-12
        assert abs(r["zero_pick_fraction"] - (1 - r["mean_ffn_experts"] / sh.K)) < 1e-12
        assert r["lb_loss"] > 0 and r["ffn_count_cv"] >= 0
    # first step (zero bias): the oracle's statistics of the oracle's routing
    # the same (GPU-drawn) inputs bench.py routed
    L = synth.make_layer(sh.with_T(1024), "cuda", want_experts=False)
    x = synth.to_np(synth.step_x(sh.with_T(1024), 0, "cuda"))
    o = oracle.route(oracle.logits(x, synth.to_np(L["wr"])), np.zeros(sh.E, np.float32), sh.N,
                     sh.K, want_keys=False)
    hist, m, s = oracle.route_stats(o.topk_idx, sh.N)
    # scores differ in their last bits (fp32 vs fp64): near-ties may flip
    # a pick or two
    assert abs(m - recs[0]["mean_ffn_experts"]) < 4.0 / 1024
    assert abs(s - recs[0]["std_ffn_experts"]) < 0.01
