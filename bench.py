"""Benchmark of the MoE layer with zero-computation experts on one MI355X.

Headline: the LongCat-Flash-shaped prefill layer (T=16384 tokens, d=6144,
512 SwiGLU experts with inner size 2048 + 256 zero-computation experts,
top-12, Zipf-skewed expert bias), forward pass; value = layer tokens/s with
every input already in HBM.  The same JSON line also carries the decode-size
layer (T=256, same shapes, memory-bound) and the training step (T=8192,
d=2048, 128+64 experts, top-8: forward, backward, bias update), each timed
the same way, and the fp64 CPU oracle timed on a bounded sample of the
headline workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--only prefill]
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from moe_layer_zero_amd import synth, zcmoe  # noqa: E402

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, vendor figure
BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, vendor figure
FP8_PEAK_TFLOPS = 5000.0    # MI355X dense fp8 MFMA, vendor figure

# HBM bytes of one prefill launch of each expert GEMM, read from rocprofv3
# counters (FETCH_SIZE x 2.0 and WRITE_SIZE x 1.0, the factors a plain copy
# of known size gives; profiles/fwdp_gemm_prefill_decode.md), valid for the
# kernel source they were measured on: reported as traffic only while that
# source is unchanged.
TRAFFIC_SOURCE = {"source": "moe_layer_zero_amd/csrc/gemm_fwdp.hip",
                  "sha256": "6da607ee05ec0056bf593fcbaf1611681979463641bf2b92d9fb59e70c18880c"}
TRAFFIC = {"gate_up_gemm": {"fetch_bytes": 32638338645, "write_bytes": 588773376},
           "down_gemm": {"fetch_bytes": 14785799637, "write_bytes": 1765676032}}


def measured_traffic(kernel: str = "gate_up_gemm"):
    path = os.path.join(ROOT, TRAFFIC_SOURCE["source"])
    if TRAFFIC_SOURCE["sha256"] is None or not os.path.exists(path):
        return None
    sha = hashlib.sha256(open(path, "rb").read()).hexdigest()
    if sha != TRAFFIC_SOURCE["sha256"] or kernel not in TRAFFIC:
        return None
    return TRAFFIC[kernel]["fetch_bytes"] + TRAFFIC[kernel]["write_bytes"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def desc_of(sh, gate_norm=1):
    return zcmoe.LayerDesc(sh.T, sh.d, sh.N, sh.Z, sh.I, sh.K, sh.torch_dtype, gate_norm)


def timed(fn, steps, warmup):
    """Run fn() warmup times, then time exactly `steps` calls with events on
    the current stream; kernel phases are read from the library's events over
    the timed region.  Returns (ms per step, {phase: (ms per launch, launches per step)})."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    zcmoe.zc_moe_profile(True)
    zcmoe.zc_moe_profile_read()  # discard warm-up records
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(steps):
        fn()
    b.record()
    torch.cuda.synchronize()
    prof = zcmoe.zc_moe_profile_read()
    zcmoe.zc_moe_profile(False)
    phases = {k: (tot / n, n / steps) for k, (tot, n) in prof.items()}
    return a.elapsed_time(b) / steps, phases


def layer_forward_bench(sh, steps, warmup, packed=True, fp8=False):
    """Inference forward of one layer.  packed: the expert weights are
    rearranged once (untimed, like loading a model) into the packed layout
    the bf16 inference kernels stream; the row-major copies are dropped.
    fp8: the expert weights are quantized once (untimed) to MXFP8 instead."""
    log(f"[bench] generating {sh.name} layer on the GPU")
    Lg = synth.make_layer(sh, "cuda")
    desc = desc_of(sh)
    if fp8:
        Lg["wg"], Lg["wu"], Lg["wd"] = zcmoe.quantize_expert_weights(desc, Lg["wg"], Lg["wu"],
                                                                     Lg["wd"])
        desc = dataclasses.replace(desc, weight_layout=zcmoe.ZC_WEIGHTS_MXFP8)
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    elif packed:
        Lg["wg"], Lg["wu"], Lg["wd"] = zcmoe.pack_expert_weights(desc, Lg["wg"], Lg["wu"],
                                                                 Lg["wd"])
        desc = dataclasses.replace(desc, weight_layout=zcmoe.ZC_WEIGHTS_PACKED)
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    route = zcmoe.RouteBuffers(desc)
    out = torch.empty((sh.T, sh.d), dtype=sh.torch_dtype, device="cuda")
    ws = zcmoe.workspace(desc, zcmoe.ZC_OP_FORWARD)

    def step():
        zcmoe.zc_moe_forward(desc, Lg["x"], Lg["wr"], Lg["bias"], Lg["wg"], Lg["wu"], Lg["wd"],
                             out, route, None, ws)

    ms, phases = timed(step, steps, warmup)
    counts = route.counts.cpu().numpy()
    p_real = int(route.offsets[-1].item())
    touched = int((counts[: sh.N] > 0).sum())
    return Lg, ms, phases, p_real, touched, counts


def gemm_roofline(kernel, flops, nbytes, ms):
    """Roofline of one expert-GEMM launch from its algorithmic flop and bytes
    and its measured duration, against the vendor peaks; the binding
    roofline is the one with the higher floor, and the other fraction rides
    along (mfma_frac / hbm_frac) so the matrix-core share is always shown."""
    t = ms * 1e-3
    tflops, gbs = flops / t / 1e12, nbytes / t / 1e9
    hbm_floor = nbytes / (HBM_PEAK_GBS * 1e9)
    mfma_floor = flops / (BF16_PEAK_TFLOPS * 1e12)
    mfma = {"bound": "mfma", "achieved": round(tflops, 2), "peak": BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": round(tflops / BF16_PEAK_TFLOPS, 4)}
    hbm = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
           "frac": round(gbs / HBM_PEAK_GBS, 4)}
    roof = dict(hbm if hbm_floor > mfma_floor else mfma)
    roof.update(kernel=kernel, traffic=measured_traffic(kernel),
                mfma_frac=mfma["frac"], hbm_frac=hbm["frac"],
                algorithmic={"flop": flops, "bytes": nbytes, "hbm_floor_ms": hbm_floor * 1e3,
                             "mfma_floor_ms": mfma_floor * 1e3})
    return roof, mfma, hbm


def gate_up_roofline(sh, p_real, touched, gu_ms):
    """Gate/up GEMM: 4 d I flop per FFN pick; bytes: gate and up weights of
    every touched expert once, the gathered x row and the h row of every
    pick."""
    d, I = sh.d, sh.I
    return gemm_roofline("gate_up_gemm", 4.0 * d * I * p_real,
                         2.0 * 2 * d * I * touched + 2.0 * d * p_real + 2.0 * I * p_real, gu_ms)


def down_roofline(sh, p_real, touched, dn_ms):
    """Down GEMM: 2 d I flop per FFN pick; bytes: down weights of every
    touched expert once, the h row read and the y row written per pick."""
    d, I = sh.d, sh.I
    return gemm_roofline("down_gemm", 2.0 * d * I * p_real,
                         2.0 * d * I * touched + 2.0 * I * p_real + 2.0 * d * p_real, dn_ms)


def prefill(steps, warmup, packed=True):
    sh = synth.CONFIGS["prefill_bf16"]
    Lg, ms, ph, p_real, touched, counts = layer_forward_bench(sh, steps, warmup, packed)
    d, I = sh.d, sh.I
    flops_gu = 4.0 * d * I * p_real          # gate and up projections of every FFN pick
    flops_dn = 2.0 * d * I * p_real
    gu_ms = ph["gate_up_gemm"][0]
    dn_ms = ph["down_gemm"][0]
    roof, mfma, hbm = gate_up_roofline(sh, p_real, touched, gu_ms)
    droof, dmfma, dhbm = down_roofline(sh, p_real, touched, dn_ms)
    res = {
        "ms_per_step": ms,
        "tokens_per_s": sh.T / (ms / 1e3),
        "p_real": p_real,
        "touched_experts": touched,
        "zero_pick_fraction": 1.0 - p_real / (sh.T * sh.K),
        "tokens_per_ffn_expert_max_over_mean": float(counts[: sh.N].max() / counts[: sh.N].mean()),
        "kernels_ms": {k: round(v[0], 4) for k, v in ph.items()},
        "gate_up_mfma_frac": mfma["frac"],
        "gate_up_hbm_frac": hbm["frac"],
        "gate_up_tflops": flops_gu / (gu_ms * 1e-3) / 1e12,
        "down_tflops": flops_dn / (dn_ms * 1e-3) / 1e12,
        "down_mfma_frac": dmfma["frac"],
        "down_hbm_frac": dhbm["frac"],
        "down_roofline": droof,
        "expert_gemms_tflops": (flops_gu + flops_dn) / ((gu_ms + dn_ms) * 1e-3) / 1e12,
        "expert_gemms_mfma_frac": (flops_gu + flops_dn) / ((gu_ms + dn_ms) * 1e-3) / 1e12
        / BF16_PEAK_TFLOPS,
    }
    del Lg
    torch.cuda.empty_cache()
    return sh, res, roof


def decode(steps, warmup, packed=True):
    sh = synth.CONFIGS["decode_bf16"]
    Lg, ms, ph, p_real, touched, counts = layer_forward_bench(sh, steps, warmup, packed)
    d, I, E = sh.d, sh.I, sh.E
    w_bytes = 2.0 * 3 * d * I * touched       # every touched expert's weights once (bf16)
    layer_bytes = w_bytes + 2.0 * d * E + 2 * 2.0 * sh.T * d + 4.0 * E + 8.0 * sh.T * sh.K
    gu_ms = ph["gate_up_gemm"][0]
    res = {
        "ms_per_step": ms,
        "tokens_per_s": sh.T / (ms / 1e3),
        "p_real": p_real,
        "touched_experts": touched,
        "layer_gbs": layer_bytes / (ms * 1e-3) / 1e9,
        "layer_hbm_frac": layer_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "gate_up_gbs": (2.0 * 2 * d * I * touched) / (gu_ms * 1e-3) / 1e9,
        "kernels_ms": {k: round(v[0], 4) for k, v in ph.items()},
    }
    del Lg
    torch.cuda.empty_cache()
    return res


def train(steps, warmup):
    sh = synth.CONFIGS["train_bf16"]
    log("[bench] generating training layer on the GPU")
    L = synth.make_layer(sh, "cuda")
    desc = desc_of(sh)
    route = zcmoe.RouteBuffers(desc)
    out = torch.empty((sh.T, sh.d), dtype=sh.torch_dtype, device="cuda")
    saved = zcmoe.saved_buffer(desc)
    wsf = zcmoe.workspace(desc, zcmoe.ZC_OP_FORWARD)
    wsb = zcmoe.workspace(desc, zcmoe.ZC_OP_BACKWARD)
    grads = {k: torch.empty_like(L[w]) for k, w in (("dx", "x"), ("dwr", "wr"), ("dwg", "wg"),
                                                    ("dwu", "wu"), ("dwd", "wd"))}
    n = warmup + steps
    xs = [synth.step_x(sh, s, "cuda") for s in range(n)]
    dys = [synth.step_dy(sh, s, "cuda") for s in range(n)]
    bias = torch.zeros(sh.E, device="cuda")
    lb = zcmoe.LoadBalance(synth.TRAIN_LB_D, synth.TRAIN_K_E, synth.TRAIN_LB_ALPHA)
    wsl = zcmoe.workspace(desc, zcmoe.ZC_OP_LB_LOSS)
    lb_out = torch.empty(1 + 2 * (lb.D + 1), dtype=torch.float64, device="cuda")
    it = [0]

    def step():
        s = it[0] % n
        it[0] += 1
        x = xs[s]
        zcmoe.zc_moe_forward(desc, x, L["wr"], bias, L["wg"], L["wu"], L["wd"], out, route, saved,
                             wsf)
        zcmoe.zc_moe_lb_loss(desc, lb, route, lb_out, wsl)
        zcmoe.zc_moe_backward(desc, x, L["wr"], L["wg"], L["wu"], L["wd"], route, saved, dys[s],
                              grads["dx"], grads["dwr"], grads["dwg"], grads["dwu"], grads["dwd"],
                              wsb, lb=lb)
        zcmoe.zc_moe_pid_update(sh.N, sh.Z, sh.K, route.counts, sh.T, synth.TRAIN_MU,
                                synth.TRAIN_K_E, bias)

    ms, ph = timed(step, steps, warmup)
    p_real = int(route.offsets[-1].item())
    flops = 18.0 * sh.d * sh.I * p_real + 6.0 * sh.T * sh.d * sh.E
    res = {"ms_per_step": ms, "tokens_per_s": sh.T / (ms / 1e3), "p_real_last": p_real,
           "mean_real_experts_last": p_real / sh.T, "tflops": flops / (ms * 1e-3) / 1e12,
           "lb_loss_last": float(lb_out[0].item()),
           "kernels_ms": {k: round(v[0], 4) for k, v in ph.items()}}
    del L, xs, dys, saved
    torch.cuda.empty_cache()
    return res


def train_telemetry(path, steps=None, T=None):
    """Budget-control telemetry of the training workload ("LongCat-Flash
    Technical Report", section 2.1.1 tracks how many FFN experts each token
    activates, Fig.3b/3c): the router + Eq.(2) loop from zero bias on the
    step inputs of the training run (weights are fixed, so the bias
    trajectory depends on the routing alone), one JSON line per step to
    `path`: mean and population std of the FFN experts per token and their
    histogram (zc_moe_route_stats), the zero-computation share of the picks,
    the coefficient of variation and max/mean of the per-FFN-expert token
    counts, the device-level load-balance loss, and the FFN bias range after
    the step's update.  Outside any timed region."""
    sh = synth.CONFIGS["train_bf16"]
    if T is not None:
        sh = sh.with_T(T)
    steps = synth.TRAIN_STEPS if steps is None else steps
    L = synth.make_layer(sh, "cuda", want_experts=False)
    desc = desc_of(sh)
    route = zcmoe.RouteBuffers(desc)
    bias = torch.zeros(sh.E, device="cuda")
    lb = zcmoe.LoadBalance(synth.TRAIN_LB_D, synth.TRAIN_K_E, synth.TRAIN_LB_ALPHA)
    lines = []
    with open(path, "w") as f:
        for s in range(steps):
            zcmoe.zc_moe_route(desc, synth.step_x(sh, s, "cuda"), L["wr"], bias, route)
            hist, mom = zcmoe.zc_moe_route_stats(desc, route)
            lbo = zcmoe.zc_moe_lb_loss(desc, lb, route)
            zcmoe.zc_moe_pid_update(sh.N, sh.Z, sh.K, route.counts, sh.T, synth.TRAIN_MU,
                                    synth.TRAIN_K_E, bias)
            c = route.counts.cpu().numpy()[: sh.N].astype(np.float64)
            m = mom.cpu().numpy()
            b = bias.cpu().numpy()[: sh.N]
            rec = {"step": s, "tokens": sh.T, "mean_ffn_experts": float(m[0]),
                   "std_ffn_experts": float(m[1]), "hist": hist.cpu().numpy().tolist(),
                   "zero_pick_fraction": 1.0 - float(c.sum()) / (sh.T * sh.K),
                   "ffn_count_cv": float(c.std() / c.mean()) if c.mean() > 0 else 0.0,
                   "ffn_count_max_over_mean": float(c.max() / c.mean()) if c.mean() > 0 else 0.0,
                   "lb_loss": float(lbo[0].item()), "bias_ffn_min": float(b.min()),
                   "bias_ffn_max": float(b.max()), "mu": synth.TRAIN_MU, "K_e": synth.TRAIN_K_E}
            f.write(json.dumps(rec) + "\n")
            lines.append(rec)
    del L
    torch.cuda.empty_cache()
    return lines


def fp8_forward(name, steps, warmup):
    """The MXFP8 inference forward (E4M3 codes, one E8M0 scale per 32
    reduction steps) of the prefill or decode layer.  Algorithmic bytes of
    the gate/up GEMM: W_g and W_u of every touched expert once at 33/32 bytes
    per weight, the quantized x row and scales of every pick, and the
    quantized h row and scales it writes; of the whole layer at decode: all
    expert weights touched at 33/32 bytes, the router weights, x, out, and
    the routing arrays."""
    sh = synth.CONFIGS[name]
    Lg, ms, ph, p_real, touched, counts = layer_forward_bench(sh, steps, warmup, fp8=True)
    d, I, E = sh.d, sh.I, sh.E
    q = 33.0 / 32.0
    gu_ms, dn_ms = ph["gate_up_gemm"][0], ph["down_gemm"][0]
    flops_gu = 4.0 * d * I * p_real
    flops_dn = 2.0 * d * I * p_real
    gu_bytes = q * 2 * d * I * touched + q * d * p_real + q * I * p_real
    res = {
        "ms_per_step": ms,
        "tokens_per_s": sh.T / (ms / 1e3),
        "p_real": p_real,
        "touched_experts": touched,
        "kernels_ms": {k: round(v[0], 4) for k, v in ph.items()},
        "gate_up_tflops": flops_gu / (gu_ms * 1e-3) / 1e12,
        "gate_up_fp8_mfma_frac": flops_gu / (gu_ms * 1e-3) / 1e12 / FP8_PEAK_TFLOPS,
        "gate_up_gbs": gu_bytes / (gu_ms * 1e-3) / 1e9,
        "gate_up_hbm_frac": gu_bytes / (gu_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "down_tflops": flops_dn / (dn_ms * 1e-3) / 1e12,
    }
    if name == "decode_bf16":
        layer_bytes = (q * 3 * d * I * touched + 2.0 * d * E + 2 * 2.0 * sh.T * d + 4.0 * E +
                       8.0 * sh.T * sh.K)
        res["layer_gbs"] = layer_bytes / (ms * 1e-3) / 1e9
        res["layer_hbm_frac"] = res["layer_gbs"] / HBM_PEAK_GBS
    del Lg
    torch.cuda.empty_cache()
    return res


def cpu_baseline(target_s=15.0, max_tokens=4096):
    """The fp64 oracle on a bounded sample of the prefill workload: router
    scores, routing and layer output for the first n tokens of a seeded
    random order, n sized so that the timed work takes about target_s
    seconds.  Returns tokens/s of that sample."""
    from oracle import oracle

    sh = synth.CONFIGS["prefill_bf16"]
    log("[bench] cpu baseline: regenerating the prefill layer, copying it to the host")
    Lg = synth.make_layer(sh, "cuda")
    g = torch.Generator().manual_seed(2024)
    order = torch.randperm(sh.T, generator=g)[:max_tokens].numpy()
    xs = synth.to_np(Lg["x"][torch.from_numpy(order).cuda()])
    wr = synth.to_np(Lg["wr"])
    bias = Lg["bias"].cpu().numpy()
    wg, wu, wd = (synth.to_np(Lg[k]) for k in ("wg", "wu", "wd"))
    del Lg
    torch.cuda.empty_cache()

    def run(n):
        x = np.ascontiguousarray(xs[:n])
        t0 = time.perf_counter()
        lg = oracle.logits(x, wr)
        r = oracle.route(lg, bias, sh.N, sh.K, want_keys=False)
        oracle.forward(x, wg, wu, wd, r.topk_idx, r.gates, sh.N)
        return time.perf_counter() - t0

    t_probe = run(16)
    n = int(min(max_tokens, max(16, 16 * target_s / max(t_probe, 1e-3))))
    log(f"[bench] cpu baseline: 16 tokens in {t_probe:.2f} s, timing {n} tokens")
    dt = run(n)
    return {"value": n / dt, "unit": "tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{n} tokens of the prefill workload (seeded random subset): router "
                      f"scores, routing, SwiGLU experts and combine in fp64, {dt:.1f} s"}


def copy_probe(nbytes: int):
    """A plain device copy of known size, for scaling HBM byte counters."""
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": nbytes, "launches": 3}), flush=True)


def bmm_reference(steps: int):
    """The vendor library on the prefill gate/up GEMM's volume, for scale:
    hipBLASLt (torch.bmm, bf16) on 512 experts of 288 rows each (the prefill
    workload's 143644 FFN picks spread evenly, rounded up to 32) times
    [6144 x 4096] weights -- the same weight bytes and about the same flop
    as the grouped kernel, without its ragged segments, row gather or
    SwiGLU.  Prints one JSON line."""
    sh = synth.CONFIGS["prefill_bf16"]
    E, M, K, N = sh.N, 288, sh.d, 2 * sh.I
    g = torch.Generator(device="cuda").manual_seed(0)
    a = torch.randn(E, M, K, device="cuda", dtype=torch.bfloat16, generator=g)
    b = (torch.randn(E, K, N, device="cuda", dtype=torch.bfloat16, generator=g) * 0.01).contiguous()
    out = torch.empty(E, M, N, device="cuda", dtype=torch.bfloat16)
    for _ in range(3):
        torch.bmm(a, b, out=out)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(steps):
        torch.bmm(a, b, out=out)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / steps
    flop = 2.0 * E * M * K * N
    print(json.dumps({"reference": "hipBLASLt bmm (torch.bmm, bf16)", "shape": [E, M, K, N],
                      "ms": round(ms, 4), "tflops": round(flop / ms / 1e9, 1),
                      "weight_GBps": round(E * K * N * 2 / ms / 1e6, 1), "steps": steps}),
          flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--only", choices=["prefill", "decode", "train", "fp8-prefill", "fp8-decode"],
                    default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--rowmajor", action="store_true",
                    help="inference on row-major expert weights instead of the packed layout")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES (counter calibration)")
    ap.add_argument("--bmm-reference", action="store_true",
                    help="only time hipBLASLt's batched GEMM on the prefill gate/up volume")
    ap.add_argument("--telemetry", default=None, metavar="PATH",
                    help="also write the training loop's per-step routing telemetry "
                         "(JSON lines) to PATH, outside the timed region")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this layer's benchmark has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    if args.bmm_reference:
        bmm_reference(max(args.steps, 20))
        return
    zcmoe.lib()
    extra = {}
    sh = synth.CONFIGS["prefill_bf16"]
    res = roof = None
    if args.only in (None, "prefill"):
        sh, res, roof = prefill(args.steps, args.warmup, not args.rowmajor)
        log(f"[bench] prefill {res['ms_per_step']:.3f} ms/step")
    if args.only in (None, "decode"):
        extra["decode"] = decode(args.steps, args.warmup, not args.rowmajor)
        log(f"[bench] decode {extra['decode']['ms_per_step']:.3f} ms/step")
    if args.only in (None, "train"):
        extra["train"] = train(args.steps, args.warmup)
        log(f"[bench] train {extra['train']['ms_per_step']:.3f} ms/step")
    for key, name in (("fp8-prefill", "prefill_bf16"), ("fp8-decode", "decode_bf16")):
        if args.only in (None, key):
            extra[key.replace("-", "_")] = fp8_forward(name, args.steps, args.warmup)
            log(f"[bench] {key} {extra[key.replace('-', '_')]['ms_per_step']:.3f} ms/step")
    if args.telemetry:
        tl = train_telemetry(args.telemetry)
        log(f"[bench] telemetry: {len(tl)} steps to {args.telemetry}, last mean FFN experts "
            f"{tl[-1]['mean_ffn_experts']:.4f}")
    cpu = None if args.no_cpu_baseline or args.only not in (None, "prefill") else cpu_baseline()
    if res is None:  # a secondary workload alone: report it as the line
        k = args.only
        res = extra.pop(k.replace("-", "_"))
        sh = synth.CONFIGS["train_bf16" if k == "train" else
                           "prefill_bf16" if k == "fp8-prefill" else "decode_bf16"]
        roof = None
    line = {
        "metric": "MoE-layer tokens/s at 1 GPU (prefill forward; % bf16 MFMA peak of the "
                  "grouped GEMM; decode % HBM BW in 'decode')",
        "value": round(res["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) inputs, N(0,std) weights, random init)",
        "config": {"workload": sh.name, "T": sh.T, "d": sh.d, "N": sh.N, "Z": sh.Z, "I": sh.I,
                   "K": sh.K, "bias": sh.bias,
                   "expert_weights": "mxfp8" if (args.only or "").startswith("fp8") else
                   "row-major" if args.rowmajor or sh.name == "train_bf16" else "packed"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "detail": res,
        **extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
