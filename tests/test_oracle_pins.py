"""Pins of the fp64 CPU oracle against facts that do not come from the oracle.

Source of the method: "LongCat-Flash Technical Report", section 2.1
(Eq.(1): biased TopK over N FFN + Z zero-computation experts, gates from the
unbiased softmax; E_i(x) = x for the zero-computation experts) and section
2.1.1 (Eq.(2): bias increment).  Each test checks the oracle against brute
force, a closed form, an invariant, or a special case that reduces to a
library routine (numpy / torch), so that a dropped term, a wrong sign or index
or a transposed operand in the oracle fails at least one of them.
"""
import itertools
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from moe_layer_zero_amd import synth

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")


def rng(seed):
    return np.random.default_rng(seed)


def ulp_diff(a: float, b: float) -> int:
    ia = np.array([a], np.float64).view(np.int64)[0]
    ib = np.array([b], np.float64).view(np.int64)[0]
    return abs(int(ia) - int(ib))


# ---------------------------------------------------------------- exp spec
def test_exp_matches_libm_within_2ulp(orc):
    zs = np.concatenate([-np.logspace(-12, math.log10(700.0), 4000),
                         np.linspace(-700.0, 0.0, 4001),
                         rng(1).uniform(-40.0, 0.0, 4000)])
    zs = zs[zs >= -700.0]  # below -700 the spec returns 0 on purpose
    worst = 0
    for z in zs:
        worst = max(worst, ulp_diff(orc.exp(float(z)), math.exp(float(z))))
    assert worst <= 2, worst


def test_exp_special_points(orc):
    assert orc.exp(0.0) == 1.0
    assert orc.exp(-0.0) == 1.0
    assert orc.exp(-700.5) == 0.0
    assert orc.exp(-1e300) == 0.0
    # e^(-k ln 2) = 2^-k up to the rounding of k*ln2 in the argument
    for k in (1, 2, 10, 100, 1000):
        assert abs(orc.exp(-k * math.log(2.0)) / 2.0 ** -k - 1.0) < 1e-12


# ---------------------------------------------------------------- logits
def test_logits_against_numpy_and_unit_vectors(orc):
    r = rng(2)
    x = r.standard_normal((7, 33)).astype(np.float32)
    wr = (0.02 * r.standard_normal((5, 33))).astype(np.float32)
    lg = orc.logits(x, wr)
    ref = x.astype(np.float64) @ wr.astype(np.float64).T
    np.testing.assert_allclose(lg, ref, rtol=1e-13, atol=1e-15)
    # x = unit vector e_k selects column k of Wr exactly (no transposition)
    eye = np.eye(33, dtype=np.float32)[:5]
    np.testing.assert_array_equal(orc.logits(eye, wr), wr[:, :5].T.astype(np.float64))


def test_logits_bf16_storage(orc):
    t = torch.randn(6, 64, generator=torch.Generator().manual_seed(3)).to(torch.bfloat16)
    w = (0.02 * torch.randn(9, 64, generator=torch.Generator().manual_seed(4))).to(torch.bfloat16)
    lg = orc.logits(synth.to_np(t), synth.to_np(w))
    ref = t.double() @ w.double().T
    np.testing.assert_allclose(lg, ref.numpy(), rtol=1e-13, atol=1e-15)


# ---------------------------------------------------------------- routing
def _brute_topk(keys, K):
    """All C(E,K) subsets: the picked set is the one whose every member beats
    every non-member under (larger key, then smaller index)."""
    E = len(keys)
    better = lambda i, j: keys[i] > keys[j] or (keys[i] == keys[j] and i < j)  # noqa: E731
    winners = [S for S in itertools.combinations(range(E), K)
               if all(better(i, j) for i in S for j in range(E) if j not in S)]
    assert len(winners) == 1
    S = winners[0]
    # slot order: repeatedly the best remaining member
    order = []
    rem = list(S)
    while rem:
        b = rem[0]
        for i in rem[1:]:
            if better(i, b):
                b = i
        order.append(b)
        rem.remove(b)
    return order


@pytest.mark.parametrize("seed", range(6))
def test_topk_brute_force(orc, seed):
    r = rng(10 + seed)
    E = int(r.integers(4, 13))
    K = int(r.integers(1, min(3, E) + 1))
    N = int(r.integers(0, E + 1))
    T = 40
    lg = r.standard_normal((T, E)).astype(np.float32) * 0.5
    # exact ties: duplicate logit columns and bias values
    lg[:, E - 1] = lg[:, 0]
    bias = (r.uniform(-0.05, 0.05, E)).astype(np.float32)
    bias[E - 1] = bias[0]
    if E > 3:
        bias[2] = bias[1]
        lg[::3, 2] = lg[::3, 1]
    out = orc.route(lg, bias, N, K)
    for t in range(T):
        assert list(out.topk_idx[t]) == _brute_topk(out.keys[t], K)


def test_topk_stays_total_on_non_finite_scores(orc):
    """A NaN score, an infinite one (inf - inf inside the softmax) or a row of
    -inf scores makes every key of the token NaN; NaN keys order as -inf,
    so the selection still returns K distinct valid indices -- 0..K-1 for
    such a token, by the lower-index tie rule.  Eq.(1) gates (p = e/S) are
    then NaN; renormalised gates are the softmax of the picked scores,
    NaN as soon as a picked exponential is.  A NaN bias sends only its own
    expert behind every finite key."""
    E, N, K = 10, 6, 3
    r = rng(30)
    lg = r.standard_normal((5, E)) * 0.5
    lg[0, 4] = np.nan
    lg[1, 7] = np.inf
    lg[2, :] = -np.inf
    bias = r.uniform(-0.05, 0.05, E).astype(np.float32)
    out = orc.route(lg, bias, N, K)
    lit = orc.route(lg, bias, N, K, gate_norm=0)
    for t in (0, 1, 2):
        assert list(out.topk_idx[t]) == list(range(K)), t
        assert list(lit.topk_idx[t]) == list(range(K)), t
        assert np.isnan(lit.gates[t]).all()
    # token 0: its NaN score is not among the picks
    want = torch.softmax(torch.from_numpy(lg[0, :K]), dim=0).numpy()
    np.testing.assert_allclose(out.gates[0], want, rtol=1e-14)
    # token 1: e = 0 for every finite score next to the infinite one
    assert np.isnan(out.gates[1]).all() and np.isnan(out.gates[2]).all()
    assert ((out.topk_idx >= 0) & (out.topk_idx < E)).all()
    assert out.counts.sum() == 5 * K
    # finite scores, NaN bias on the expert each token would pick first
    p = torch.softmax(torch.from_numpy(lg[3:]), dim=1).numpy()
    for t in range(2):
        b = bias.copy()
        b[int(np.argmax(p[t] + bias))] = np.nan
        o = orc.route(lg[3 + t:4 + t], b, N, K)
        keys = p[t] + b.astype(np.float64)
        keys[np.isnan(keys)] = -np.inf
        assert list(o.topk_idx[0]) == _brute_topk(keys, K)
        assert np.isfinite(o.gates).all()


def test_keys_are_softmax_plus_bias(orc):
    r = rng(20)
    lg = (r.standard_normal((50, 96)) * 2.0).astype(np.float32)
    bias = r.uniform(-0.1, 0.1, 96).astype(np.float32)
    out = orc.route(lg, bias, 64, 6)
    p = torch.softmax(torch.from_numpy(lg).double(), dim=1).numpy()
    np.testing.assert_allclose(out.keys, p + bias.astype(np.float64), rtol=0, atol=1e-16 * 8)
    # slot order is a stable descending sort of the keys
    ref = np.argsort(-out.keys, axis=1, kind="stable")[:, :6]
    np.testing.assert_array_equal(out.topk_idx, ref)


@pytest.mark.parametrize("gate_norm", [1, 0])
def test_gates(orc, gate_norm):
    r = rng(21)
    lg = (r.standard_normal((64, 12)) * 1.5).astype(np.float32)
    bias = r.uniform(-0.2, 0.2, 12).astype(np.float32)
    out = orc.route(lg, bias, 8, 3, gate_norm=gate_norm)
    L = torch.from_numpy(lg).double()
    idx = torch.from_numpy(out.topk_idx).long()
    if gate_norm:
        ref = torch.softmax(torch.gather(L, 1, idx), dim=1)
        np.testing.assert_allclose(out.gates.sum(1), 1.0, rtol=0, atol=4e-16)
    else:
        ref = torch.gather(torch.softmax(L, dim=1), 1, idx)
    np.testing.assert_allclose(out.gates, ref.numpy(), rtol=1e-14, atol=0)


def test_gates_use_unbiased_softmax(orc):
    """A huge bias changes which experts are picked but not the gate values
    of a given pick (Eq.(1): gate = R_i, bias only in the TopK argument)."""
    r = rng(22)
    lg = r.standard_normal((30, 10)).astype(np.float32)
    b0 = np.zeros(10, np.float32)
    b1 = np.zeros(10, np.float32)
    b1[[3, 7]] = 5.0  # forces experts 3 and 7 (K=2) regardless of R
    o1 = orc.route(lg, b1, 6, 2, gate_norm=0)
    assert (np.sort(o1.topk_idx, 1) == [3, 7]).all()
    p = torch.softmax(torch.from_numpy(lg).double(), 1).numpy()
    np.testing.assert_allclose(o1.gates, np.take_along_axis(p, o1.topk_idx.astype(np.int64), 1),
                               rtol=1e-14)
    o0 = orc.route(lg, b0, 6, 2, gate_norm=0)
    # with zero bias the keys are the softmax itself: picks = the 2 largest logits
    np.testing.assert_array_equal(o0.topk_idx, np.argsort(-lg, 1, kind="stable")[:, :2])


def test_dispatch_invariants(orc):
    r = rng(23)
    T, E, N, K = 333, 40, 25, 5
    lg = r.standard_normal((T, E)).astype(np.float32)
    bias = r.uniform(-0.05, 0.05, E).astype(np.float32)
    o = orc.route(lg, bias, N, K)
    idx = o.topk_idx
    assert o.counts.sum() == T * K
    np.testing.assert_array_equal(o.counts, np.bincount(idx.ravel(), minlength=E))
    assert o.offsets[0] == 0
    np.testing.assert_array_equal(np.diff(o.offsets), o.counts[:N])
    real = np.flatnonzero(idx.ravel() < N)
    assert o.p_real == len(real)
    # perm: real slots sorted by (expert, token)
    slots = o.perm
    e_of = idx.ravel()[slots]
    t_of = slots // K
    key = e_of.astype(np.int64) * T + t_of
    assert (np.diff(key) > 0).all()
    assert sorted(slots.tolist()) == sorted(real.tolist())
    # inv o perm = identity; identity picks get -1
    np.testing.assert_array_equal(o.inv[slots], np.arange(o.p_real))
    assert (o.inv[idx.ravel() >= N] == -1).all()


# ---------------------------------------------------------------- forward
def _layer(T, d, N, Z, I, K, seed, w_std=0.1, bias=None, dtype=np.float32):
    r = rng(seed)
    E = N + Z
    L = {
        "x": r.standard_normal((T, d)).astype(dtype),
        "wr": (w_std * r.standard_normal((E, d))).astype(dtype),
        "wg": (w_std * r.standard_normal((N, I, d))).astype(dtype),
        "wu": (w_std * r.standard_normal((N, I, d))).astype(dtype),
        "wd": (w_std * r.standard_normal((N, d, I))).astype(dtype),
        "bias": np.zeros(E, np.float32) if bias is None else bias,
    }
    return L


def _torch_swiglu(x, wg, wu, wd):
    return F.linear(F.silu(F.linear(x, wg)) * F.linear(x, wu), wd)


def _run(orc, L, N, K, gate_norm=1, out_scale=1.0):
    lg = orc.logits(L["x"], L["wr"])
    ro = orc.route(lg, L["bias"], N, K, gate_norm=gate_norm)
    out = orc.forward(L["x"], L["wg"], L["wu"], L["wd"], ro.topk_idx, ro.gates, N,
                      out_scale=out_scale)
    return lg, ro, out


def test_forward_z0_b0_is_standard_topk_moe(orc):
    """Z = 0, b = 0: plain softmax top-K MoE with renormalised gates, written
    with torch library ops (topk, softmax, linear, silu)."""
    T, d, N, I, K = 48, 32, 6, 16, 2
    L = _layer(T, d, N, 0, I, K, seed=30)
    _, ro, out = _run(orc, L, N, K)
    x = torch.from_numpy(L["x"]).double()
    logits = x @ torch.from_numpy(L["wr"]).double().T
    probs = torch.softmax(logits, dim=1)
    topv, topi = torch.topk(probs, K, dim=1)
    gates = topv / topv.sum(1, keepdim=True)
    ref = torch.zeros_like(x)
    for e in range(N):
        ye = _torch_swiglu(x, *(torch.from_numpy(L[k][e]).double() for k in ("wg", "wu", "wd")))
        w = (gates * (topi == e)).sum(1, keepdim=True)
        ref += w * ye
    np.testing.assert_array_equal(ro.topk_idx, topi.numpy())
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("gate_norm", [1, 0])
def test_forward_all_identity_picks(orc, gate_norm):
    """Force every pick onto a zero-computation expert: output = x (renormalised
    gates) or (sum of the picked R_i) * x (Eq.(1) literal)."""
    T, d, N, Z, I, K = 40, 24, 5, 4, 8, 3
    bias = np.zeros(N + Z, np.float32)
    bias[N:] = 1.0
    L = _layer(T, d, N, Z, I, K, seed=31, bias=bias)
    lg, ro, out = _run(orc, L, N, K, gate_norm=gate_norm)
    assert (ro.topk_idx >= N).all()
    x = L["x"].astype(np.float64)
    if gate_norm:
        np.testing.assert_allclose(out, x, rtol=1e-15, atol=1e-15)
    else:
        p = torch.softmax(torch.from_numpy(lg), 1).numpy()
        s = np.take_along_axis(p, ro.topk_idx.astype(np.int64), 1).sum(1, keepdims=True)
        np.testing.assert_allclose(out, s * x, rtol=1e-13)


def test_forward_k_equals_e_is_dense_mixture(orc):
    """K = E: every expert is picked whatever the bias; output is the dense
    softmax mixture sum_j R_j E_j(x)."""
    T, d, N, Z, I = 20, 16, 3, 2, 8
    E = N + Z
    bias = rng(32).uniform(-1, 1, E).astype(np.float32)
    L = _layer(T, d, N, Z, I, E, seed=33, bias=bias)
    lg, ro, out = _run(orc, L, N, E)
    x = torch.from_numpy(L["x"]).double()
    R = torch.softmax(torch.from_numpy(lg), 1)
    ref = R[:, N:].sum(1, keepdim=True) * x
    for e in range(N):
        ref += R[:, e:e + 1] * _torch_swiglu(
            x, *(torch.from_numpy(L[k][e]).double() for k in ("wg", "wu", "wd")))
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-12, atol=1e-14)


def test_forward_single_expert_is_swiglu_mlp(orc):
    T, d, I = 10, 16, 12
    L = _layer(T, d, 1, 0, I, 1, seed=34)
    _, ro, out = _run(orc, L, 1, 1)
    x = torch.from_numpy(L["x"]).double()
    ref = _torch_swiglu(x, *(torch.from_numpy(L[k][0]).double() for k in ("wg", "wu", "wd")))
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-12, atol=1e-14)
    np.testing.assert_array_equal(ro.gates, 1.0)


def test_ffn_activations_on_permutation_weights(orc):
    """a = W_g[e] x_t, u = W_u[e] x_t, h = silu(a) u of a pick, in closed
    form: with W_g[e] = alpha_e P_e and W_u[e] = beta_e Q_e for permutation
    matrices (row i holds one entry, in column pi_e(i) or sigma_e(i)),
    a_i = alpha_e x[t, pi_e(i)] and u_i = beta_e x[t, sigma_e(i)].  Distinct
    non-involutive permutations per expert make a transposed weight, a swapped
    gate/up pair, a wrong expert or token row fail; silu comes from torch."""
    r = rng(91)
    T, d, N, I = 7, 12, 3, 9
    x = r.standard_normal((T, d)).astype(np.float32)
    wg = np.zeros((N, I, d), np.float32)
    wu = np.zeros((N, I, d), np.float32)
    alpha = np.array([0.5, -1.25, 2.0])
    beta = np.array([1.5, 0.75, -0.5])
    pis, sigmas = [], []
    for e in range(N):
        pi = r.permutation(d)[:I]
        sg = r.permutation(d)[:I]
        pis.append(pi)
        sigmas.append(sg)
        wg[e, np.arange(I), pi] = alpha[e]
        wu[e, np.arange(I), sg] = beta[e]
    tok = np.array([0, 3, 6, 3, 1])
    ex = np.array([2, 0, 1, 1, 2])
    a, u, h = orc.ffn_activations(x, wg, wu, N, tok, ex)
    for q, (t, e) in enumerate(zip(tok, ex)):
        a_ref = alpha[e] * x[t, pis[e]].astype(np.float64)
        u_ref = beta[e] * x[t, sigmas[e]].astype(np.float64)
        np.testing.assert_array_equal(a[q], a_ref)
        np.testing.assert_array_equal(u[q], u_ref)
        h_ref = F.silu(torch.from_numpy(a_ref)).numpy() * u_ref
        np.testing.assert_allclose(h[q], h_ref, rtol=1e-14, atol=0)


def test_ffn_activations_match_torch_swiglu_hidden_row(orc):
    """On random bf16 weights the hidden row of each pick equals torch's
    silu(x W_g^T) * (x W_u^T) in float64 (a special case reducing to
    library linear layers), for the picks' experts and tokens."""
    r = rng(92)
    T, d, N, I = 6, 32, 4, 16
    L = _layer(T, d, N, 0, I, 1, seed=93)
    bits = {k: synth.to_np(torch.from_numpy(L[k]).to(torch.bfloat16)) for k in ("x", "wg", "wu")}
    tok = r.integers(0, T, 10)
    ex = r.integers(0, N, 10)
    a, u, h = orc.ffn_activations(bits["x"], bits["wg"], bits["wu"], N, tok, ex)
    xv = torch.from_numpy(bits["x"].astype(np.int32) << 16).view(torch.float32).double()
    for q, (t, e) in enumerate(zip(tok, ex)):
        wgv = torch.from_numpy(bits["wg"][e].astype(np.int32) << 16).view(torch.float32).double()
        wuv = torch.from_numpy(bits["wu"][e].astype(np.int32) << 16).view(torch.float32).double()
        a_ref = F.linear(xv[t], wgv)
        u_ref = F.linear(xv[t], wuv)
        np.testing.assert_allclose(a[q], a_ref.numpy(), rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(u[q], u_ref.numpy(), rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(h[q], (F.silu(a_ref) * u_ref).numpy(), rtol=1e-12, atol=1e-14)


def test_forward_token_subset_and_out_scale(orc):
    T, d, N, Z, I, K = 30, 16, 4, 2, 8, 2
    L = _layer(T, d, N, Z, I, K, seed=35)
    lg, ro, out = _run(orc, L, N, K)
    toks = [29, 3, 3, 0]
    sub = orc.forward(L["x"], L["wg"], L["wu"], L["wd"], ro.topk_idx, ro.gates, N,
                      out_scale=2.5, toks=toks)
    np.testing.assert_allclose(sub, 2.5 * out[toks], rtol=1e-15)


# ---------------------------------------------------------------- backward
def _torch_fixed_route_loss(x, wr, wg, wu, wd, idx, N, gate_norm, dY, out_scale=1.0):
    """Forward with the routing held fixed, as torch ops, for autograd."""
    logits = x @ wr.T
    if gate_norm:
        gates = torch.softmax(torch.gather(logits, 1, idx), 1)
    else:
        gates = torch.gather(torch.softmax(logits, 1), 1, idx)
    out = torch.zeros_like(x)
    for r in range(idx.shape[1]):
        e_r = idx[:, r]
        g = gates[:, r:r + 1]
        ident = (e_r >= N).double().unsqueeze(1)
        out = out + g * ident * x
        for e in range(N):
            m = (e_r == e).double().unsqueeze(1)
            if m.sum() == 0:
                continue
            out = out + g * m * _torch_swiglu(x, wg[e], wu[e], wd[e])
    return (out_scale * out * dY).sum()


@pytest.mark.parametrize("gate_norm", [1, 0])
def test_backward_against_autograd(orc, gate_norm):
    T, d, N, Z, I, K = 24, 16, 4, 3, 8, 3
    bias = rng(40).uniform(-0.05, 0.05, N + Z).astype(np.float32)
    L = _layer(T, d, N, Z, I, K, seed=41, bias=bias, w_std=0.3)
    dY = rng(42).standard_normal((T, d)).astype(np.float32)
    lg, ro, _ = _run(orc, L, N, K, gate_norm=gate_norm)
    g = orc.backward(L["x"], L["wr"], L["wg"], L["wu"], L["wd"], lg, ro.topk_idx, ro.gates,
                     dY, N, Z, gate_norm=gate_norm, out_scale=1.5)
    ts = {k: torch.from_numpy(L[k]).double().requires_grad_(True)
          for k in ("x", "wr", "wg", "wu", "wd")}
    loss = _torch_fixed_route_loss(ts["x"], ts["wr"], ts["wg"], ts["wu"], ts["wd"],
                                   torch.from_numpy(ro.topk_idx).long(), N, gate_norm,
                                   torch.from_numpy(dY).double(), out_scale=1.5)
    loss.backward()
    np.testing.assert_allclose(g["dx"], ts["x"].grad.numpy(), rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(g["dwr"], ts["wr"].grad.numpy(), rtol=1e-11, atol=1e-13)
    for e in range(N):
        np.testing.assert_allclose(g["dwg"][e], ts["wg"].grad[e].numpy(), rtol=1e-11, atol=1e-13)
        np.testing.assert_allclose(g["dwu"][e], ts["wu"].grad[e].numpy(), rtol=1e-11, atol=1e-13)
        np.testing.assert_allclose(g["dwd"][e], ts["wd"].grad[e].numpy(), rtol=1e-11, atol=1e-13)


def test_backward_expert_gradients_alone_against_autograd(orc):
    """Asked for the weight gradients of some experts only (no dx, no router
    gradient), the backward needs and reads those experts' weights alone and
    still matches autograd on them."""
    T, d, N, Z, I, K = 24, 16, 5, 3, 8, 3
    L = _layer(T, d, N, Z, I, K, seed=43, w_std=0.3)
    dY = rng(44).standard_normal((T, d)).astype(np.float32)
    lg, ro, _ = _run(orc, L, N, K)
    want = [1, 3]
    only = {k: {e: L[k][e] for e in want} for k in ("wg", "wu", "wd")}
    g = orc.backward(L["x"], L["wr"], only["wg"], only["wu"], only["wd"], lg, ro.topk_idx,
                     ro.gates, dY, N, Z, out_scale=0.75, want_experts=want, want_dwr=False,
                     want_dx=False)
    assert g["dx"] is None and g["dwr"] is None
    ts = {k: torch.from_numpy(L[k]).double().requires_grad_(True)
          for k in ("x", "wr", "wg", "wu", "wd")}
    loss = _torch_fixed_route_loss(ts["x"], ts["wr"], ts["wg"], ts["wu"], ts["wd"],
                                   torch.from_numpy(ro.topk_idx).long(), N, 1,
                                   torch.from_numpy(dY).double(), out_scale=0.75)
    loss.backward()
    assert any((ro.topk_idx == e).any() for e in want)
    for e in want:
        np.testing.assert_allclose(g["dwg"][e], ts["wg"].grad[e].numpy(), rtol=1e-11, atol=1e-13)
        np.testing.assert_allclose(g["dwu"][e], ts["wu"].grad[e].numpy(), rtol=1e-11, atol=1e-13)
        np.testing.assert_allclose(g["dwd"][e], ts["wd"].grad[e].numpy(), rtol=1e-11, atol=1e-13)


def test_backward_finite_differences(orc):
    """Central differences of <dY, out> through the whole oracle (route +
    forward), at coordinates where the routing does not flip."""
    T, d, N, Z, I, K = 16, 12, 3, 2, 6, 2
    L = _layer(T, d, N, Z, I, K, seed=43, w_std=0.3)
    dY = rng(44).standard_normal((T, d)).astype(np.float32)
    lg, ro, _ = _run(orc, L, N, K)
    g = orc.backward(L["x"], L["wr"], L["wg"], L["wu"], L["wd"], lg, ro.topk_idx, ro.gates,
                     dY, N, Z)

    def loss(LL):
        _, r2, out = _run(orc, LL, N, K)
        return float((out * dY.astype(np.float64)).sum()), r2.topk_idx

    picks = [("x", (3, 5)), ("x", (11, 0)), ("wr", (1, 7)), ("wr", (4, 2)),
             ("wg", (0, 2, 3)), ("wu", (2, 5, 11)), ("wd", (1, 4, 0)), ("wd", (0, 11, 5))]
    grads = {"x": g["dx"], "wr": g["dwr"]}
    for name, ix in picks:
        h = 2.0 ** -12
        Lp = {k: v.copy() for k, v in L.items()}
        Lm = {k: v.copy() for k, v in L.items()}
        Lp[name][ix] += h
        Lm[name][ix] -= h
        fp, ip = loss(Lp)
        fm, im = loss(Lm)
        assert (ip == ro.topk_idx).all() and (im == ro.topk_idx).all()
        fd = (fp - fm) / (float(Lp[name][ix]) - float(Lm[name][ix]))
        if name in grads:
            an = grads[name][ix]
        else:
            key = {"wg": "dwg", "wu": "dwu", "wd": "dwd"}[name]
            an = g[key][ix[0]][ix[1:]]
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, ix, fd, an)


def test_backward_all_identity(orc):
    """All picks on zero-computation experts with renormalised gates: out = x,
    so dx = dY and every weight gradient is zero."""
    T, d, N, Z, I, K = 20, 16, 4, 4, 8, 3
    bias = np.zeros(N + Z, np.float32)
    bias[N:] = 1.0
    L = _layer(T, d, N, Z, I, K, seed=45, bias=bias)
    dY = rng(46).standard_normal((T, d)).astype(np.float32)
    lg, ro, _ = _run(orc, L, N, K)
    g = orc.backward(L["x"], L["wr"], L["wg"], L["wu"], L["wd"], lg, ro.topk_idx, ro.gates,
                     dY, N, Z)
    np.testing.assert_allclose(g["dx"], dY.astype(np.float64), rtol=1e-14, atol=1e-15)
    # dl = g dg (1 - sum g): zero up to the rounding of sum g = 1
    assert np.abs(g["dwr"]).max() < 1e-13
    for e in range(N):
        assert not g["dwg"][e].any() and not g["dwu"][e].any() and not g["dwd"][e].any()


# ---------------------------------------------------------------- Eq.(2)
def test_pid_closed_forms(orc):
    N, Z, K, T, mu, Ke = 16, 8, 4, 100, 0.7, 3.0
    r = rng(50)
    idx = np.stack([r.choice(N + Z, K, replace=False) for _ in range(T)])
    counts = np.bincount(idx.ravel(), minlength=N + Z).astype(np.int32)
    b0 = r.uniform(-0.01, 0.01, N + Z).astype(np.float32)
    b1 = orc.pid_update(counts, T, b0, N, Z, K, mu, Ke)
    # identity entries untouched, bit for bit
    np.testing.assert_array_equal(b1[N:], b0[N:])
    # per expert: mu*(Ke/(K N) - T_i/(K T)) up to one fp32 rounding of b
    want = b0[:N].astype(np.float64) + mu * (Ke / (K * N) - counts[:N] / (K * T))
    np.testing.assert_allclose(b1[:N], want, rtol=0, atol=np.spacing(np.float32(0.05)))
    # sum of increments = mu (Ke - P_real/T) / K
    p_real = counts[:N].sum()
    dsum = (want - b0[:N]).sum()
    assert abs(dsum - mu * (Ke - p_real / T) / K) < 1e-12
    # sign: fewer FFN picks than Ke per token on average -> FFN biases rise on average
    assert (p_real / T < Ke) == (dsum > 0)


def test_pid_fixed_point_is_exact(orc):
    N, Z, K, T, Ke = 8, 4, 2, 64, 6.0 / 4.0 * 2.0 / 2.0
    # T_i = Ke*T/N for every FFN expert -> no change at all
    Ke = 1.5
    counts = np.full(N + Z, 0, np.int32)
    counts[:N] = int(Ke * T / N)
    b0 = np.linspace(-0.01, 0.01, N + Z).astype(np.float32)
    b1 = orc.pid_update(counts, T, b0, N, Z, K, 1.0, Ke)
    np.testing.assert_array_equal(b1, b0)


# ---------------------------------------------------------------- workloads
def test_zero_bias_identity_share_is_z_over_e(orc):
    """With zero bias and iid router columns, each pick lands on a
    zero-computation expert with probability Z/E (symmetry)."""
    sh = synth.CONFIGS["decode_bf16"]
    T, E, N, K = 2048, 96, 64, 6
    lg = synth.make_logits(T, E, 0.5, 7).numpy()
    o = orc.route(lg, np.zeros(E, np.float32), N, K, want_keys=False)
    frac = 1.0 - o.p_real / (T * K)
    se = math.sqrt((32 / 96) * (64 / 96) / (T * K))
    assert abs(frac - 32 / 96) < 5 * se
    assert sh.Z / sh.E == pytest.approx(1 / 3)


def test_shapes_match_activated_parameter_range():
    """Section 2.4: 512 FFN experts with inner size 2048 at hidden 6144, 12
    picks of which 0..12 are FFN experts, 28 layers: 12 FFN picks more than
    none adds 12*28*3*d*I parameters = the printed 31.3B - 18.6B spread."""
    sh = synth.CONFIGS["prefill_bf16"]
    per_expert = 3 * sh.d * sh.I
    assert per_expert == 37_748_736
    spread = sh.K * 28 * per_expert
    assert abs(spread / 1e9 - (31.3 - 18.6)) < 0.05
