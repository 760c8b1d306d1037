"""Pins of the oracle's device-level load-balance loss and its gradient.

Source: "LongCat-Flash Technical Report", section 2.1.2 ("Load balance
control"): L_LB = alpha * sum_j f_j P_j over D groups of G = N/D FFN experts
plus one extra group holding every zero-computation expert, with P_j of
Eq.(4) (mean router probability mass of the group) and f_j of Eq.(5) (pick
frequency scaled by D/(K_e T), or 1/((K-K_e) T) for the extra group).  The
checks are closed forms (balanced picks give L = alpha; uniform scores give
P_j = |Group_j| / E), a case that tells contiguous from strided grouping,
central finite differences of the loss for the gradient, the softmax
Jacobian's row-sum invariant, and autograd through the full layer for the
extra router-score gradient that the backward accepts.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")


def rng(seed):
    return np.random.default_rng(seed)


def _random_picks(r, T, E, K):
    return np.stack([r.permutation(E)[:K] for _ in range(T)]).astype(np.int32)


def test_balanced_picks_give_alpha(orc):
    """Every group receives exactly K_e T / D FFN picks and the extra group
    (K - K_e) T picks: all f_j = 1, and sum_j P_j = 1 because each token's
    softmax sums to one, so L = alpha for any scores."""
    N, Z, D, K, K_e, T = 8, 4, 4, 3, 2.0, 8
    E = N + Z
    picks = np.array([[(2 * t) % N, (2 * t + 1) % N, N + t % Z] for t in range(T)], np.int32)
    lg = rng(1).standard_normal((T, E)) * 3.0
    L, f, P, _ = orc.lb_loss(lg, picks, N, D, K_e, alpha=0.37)
    np.testing.assert_allclose(f, np.ones(D + 1), rtol=0, atol=1e-15)
    assert abs(P.sum() - 1.0) < 1e-14
    assert abs(L - 0.37) < 1e-14


def test_uniform_scores_closed_form(orc):
    """Equal scores: R = 1/E, so P_j = G/E for FFN groups and Z/E for the
    extra group; with n_ffn / n_zero the FFN / zero-computation pick counts,
    L = alpha/(E T) * (N n_ffn / K_e + Z n_zero / (K - K_e))."""
    N, Z, D, K, K_e, T, alpha = 12, 6, 3, 4, 2.5, 20, 0.01
    E = N + Z
    r = rng(2)
    picks = _random_picks(r, T, E, K)
    lg = np.full((T, E), 0.75)
    L, f, P, _ = orc.lb_loss(lg, picks, N, D, K_e, alpha)
    G = N // D
    np.testing.assert_allclose(P, [G / E] * D + [Z / E], rtol=1e-15)
    n_ffn = int((picks < N).sum())
    n_zero = T * K - n_ffn
    want = alpha / (E * T) * (N * n_ffn / K_e + Z * n_zero / (K - K_e))
    assert abs(L - want) <= 1e-15 * abs(want)
    # the pick frequencies themselves: group of expert e is e // G
    for j in range(D):
        cnt = int(((picks < N) & (picks // G == j)).sum())
        assert abs(f[j] - D / (K_e * T) * cnt) <= 1e-15 * max(1.0, f[j])
    assert abs(f[D] - n_zero / ((K - K_e) * T)) <= 1e-15 * max(1.0, f[D])


def test_groups_are_contiguous_index_ranges(orc):
    """Half the tokens put all router mass and their FFN pick on expert 0,
    the other half on expert 1.  With G = 2 both experts are in group 1, so
    f_1 = D, P_1 = 1 and L = alpha D; a strided grouping (expert e in group
    e mod D) would give alpha D / 2."""
    N, Z, D, K, K_e, T = 8, 2, 4, 2, 1.0, 10
    E = N + Z
    lg = np.zeros((T, E))
    picks = np.zeros((T, K), np.int32)
    for t in range(T):
        hot = t % 2
        lg[t, hot] = 60.0  # other probabilities ~ e^-60
        picks[t] = [hot, N + (t % Z)]
    L, f, P, _ = orc.lb_loss(lg, picks, N, D, K_e, alpha=1.0)
    assert abs(f[0] - D) < 1e-14 and np.all(f[1:D] == 0.0) and abs(f[D] - 1.0) < 1e-14
    assert abs(P[0] - 1.0) < 1e-15
    assert abs(L - D) < 1e-12


def test_no_zero_experts_single_group_gives_alpha(orc):
    """Z = 0, D = 1, K_e = K: every pick is an FFN pick, so f_1 = 1, all
    router mass is on the one group, P_1 = 1 and L = alpha; the extra group's
    slots stay 0."""
    N, K, T = 10, 3, 15
    r = rng(3)
    lg = r.standard_normal((T, N)) * 2
    picks = _random_picks(r, T, N, K)
    L, f, P, dl = orc.lb_loss(lg, picks, N, 1, float(K), alpha=2.0)
    assert abs(f[0] - 1.0) < 1e-15 and f[1] == 0.0 and P[1] == 0.0
    assert abs(P[0] - 1.0) < 1e-14 and abs(L - 2.0) < 1e-14
    # a constant c over all experts: the gradient vanishes
    assert np.abs(dl).max() < 1e-16


def _fd_case(seed):
    N, Z, D, K, K_e, T = 6, 3, 3, 3, 2.0, 7
    E = N + Z
    r = rng(seed)
    lg = r.standard_normal((T, E))
    picks = _random_picks(r, T, E, K)
    return N, Z, D, K, K_e, T, E, lg, picks


def test_gradient_central_differences(orc):
    N, Z, D, K, K_e, T, E, lg, picks = _fd_case(4)
    alpha = 0.8
    _, _, _, dl = orc.lb_loss(lg, picks, N, D, K_e, alpha)
    h = 2.0 ** -14
    for t, i in [(0, 0), (1, 5), (3, N), (6, E - 1), (2, 2), (5, 4)]:
        lp, lm = lg.copy(), lg.copy()
        lp[t, i] += h
        lm[t, i] -= h
        fp = orc.lb_loss(lp, picks, N, D, K_e, alpha, want_grad=False)[0]
        fm = orc.lb_loss(lm, picks, N, D, K_e, alpha, want_grad=False)[0]
        fd = (fp - fm) / (2 * h)
        assert abs(fd - dl[t, i]) <= 1e-9 * max(1.0, abs(dl[t, i])), (t, i, fd, dl[t, i])


def test_gradient_rows_sum_to_zero(orc):
    """Adding a constant to one token's scores leaves its softmax, hence L,
    unchanged: every row of dL/dl sums to 0."""
    N, Z, D, K, K_e, T, E, lg, picks = _fd_case(5)
    _, _, _, dl = orc.lb_loss(lg, picks, N, D, K_e, 1.3)
    assert np.abs(dl.sum(axis=1)).max() < 1e-16
    assert np.abs(dl).max() > 1e-3


def test_argument_checks(orc):
    lg = np.zeros((4, 6))
    picks = np.array([[0, 5]] * 4, np.int32)
    with pytest.raises(ValueError):
        orc.lb_loss(lg, picks, 4, 3, 1.0, 1.0)   # D does not divide N
    with pytest.raises(ValueError):
        orc.lb_loss(lg, picks, 4, 2, 2.0, 1.0)   # K_e = K with zero experts
    with pytest.raises(ValueError):
        orc.lb_loss(lg, picks, 4, 2, 0.0, 1.0)   # K_e must be positive
    L, f, P, dl = orc.lb_loss(np.zeros((0, 6)), np.zeros((0, 2), np.int32), 4, 2, 1.0, 1.0)
    assert L == 0.0 and not f.any() and not P.any() and dl.shape == (0, 6)


# ------------------------------------------------- backward with the loss
def _torch_layer_plus_lb(x, wr, wg, wu, wd, idx, N, D, K_e, alpha, dY):
    """<dY, out> + L_LB with the routing held fixed, in torch ops."""
    logits = x @ wr.T
    gates = torch.softmax(torch.gather(logits, 1, idx), 1)
    out = torch.zeros_like(x)
    for r in range(idx.shape[1]):
        e_r = idx[:, r]
        g = gates[:, r:r + 1]
        out = out + g * (e_r >= N).double().unsqueeze(1) * x
        for e in range(N):
            m = (e_r == e).double().unsqueeze(1)
            if m.sum() > 0:
                y = F.linear(F.silu(F.linear(x, wg[e])) * F.linear(x, wu[e]), wd[e])
                out = out + g * m * y
    T, E = logits.shape
    K = idx.shape[1]
    G = N // D
    R = torch.softmax(logits, 1)
    grp = torch.tensor([e // G if e < N else D for e in range(E)])
    onehot = F.one_hot(grp, D + 1).double()            # [E, D+1]
    P = (R @ onehot).sum(0) / T
    cnt = F.one_hot(grp[idx.reshape(-1)], D + 1).double().sum(0)
    scale = torch.tensor([D / (K_e * T)] * D + [1.0 / ((K - K_e) * T)], dtype=torch.float64)
    lb = alpha * (scale * cnt * P).sum()
    return (out * dY).sum() + lb


def test_backward_with_lb_gradient_against_autograd(orc):
    from test_oracle_pins import _layer, _run
    T, d, N, Z, I, K, D, K_e, alpha = 20, 16, 4, 3, 8, 3, 2, 2.0, 0.5
    L = _layer(T, d, N, Z, I, K, seed=50, w_std=0.3)
    dY = rng(51).standard_normal((T, d)).astype(np.float32)
    lg, ro, _ = _run(orc, L, N, K)
    _, _, _, dl = orc.lb_loss(lg, ro.topk_idx, N, D, K_e, alpha)
    g = orc.backward(L["x"], L["wr"], L["wg"], L["wu"], L["wd"], lg, ro.topk_idx, ro.gates,
                     dY, N, Z, dl_extra=dl)
    ts = {k: torch.from_numpy(L[k]).double().requires_grad_(True)
          for k in ("x", "wr", "wg", "wu", "wd")}
    obj = _torch_layer_plus_lb(ts["x"], ts["wr"], ts["wg"], ts["wu"], ts["wd"],
                               torch.from_numpy(ro.topk_idx).long(), N, D, K_e, alpha,
                               torch.from_numpy(dY).double())
    obj.backward()
    np.testing.assert_allclose(g["dx"], ts["x"].grad.numpy(), rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(g["dwr"], ts["wr"].grad.numpy(), rtol=1e-11, atol=1e-13)
    # the loss term really moved the router gradient
    g0 = orc.backward(L["x"], L["wr"], L["wg"], L["wu"], L["wd"], lg, ro.topk_idx, ro.gates,
                      dY, N, Z)
    assert np.abs(g["dwr"] - g0["dwr"]).max() > 1e-4


# ------------------------------------------------- budget-control telemetry
def test_route_stats_closed_forms(orc):
    """All picks FFN: every token activates K, mean K, std 0.  Tokens whose
    FFN-pick count cycles through 0..K: the discrete uniform law, mean K/2,
    variance ((K+1)^2 - 1)/12."""
    N, Z, K, T = 6, 6, 4, 5 * 7
    idx = np.tile(np.arange(K, dtype=np.int32), (T, 1))
    hist, m, s = orc.route_stats(idx, N)
    assert hist.tolist() == [0] * K + [T] and m == K and s == 0.0
    rows = []
    for t in range(T):
        k = t % (K + 1)
        rows.append(list(range(k)) + list(range(N, N + K - k)))
    hist, m, s = orc.route_stats(np.array(rows, np.int32), N)
    assert hist.tolist() == [T // (K + 1)] * (K + 1)
    assert abs(m - K / 2) < 1e-15
    assert abs(s - np.sqrt(((K + 1) ** 2 - 1) / 12)) < 1e-15


def test_route_stats_against_numpy_and_counts(orc):
    """Random routing: numpy's bincount / mean / std (population) of the
    per-token FFN-pick counts, and sum_k k hist[k] = sum of the FFN experts'
    token counts from the routing."""
    r = rng(9)
    N, Z, K, T = 24, 12, 6, 500
    lg = r.standard_normal((T, N + Z))
    ro = orc.route(lg, np.zeros(N + Z, np.float32), N, K)
    hist, m, s = orc.route_stats(ro.topk_idx, N)
    n_t = (ro.topk_idx < N).sum(1)
    np.testing.assert_array_equal(hist, np.bincount(n_t, minlength=K + 1))
    assert abs(m - n_t.mean()) < 1e-14 and abs(s - n_t.std()) < 1e-14
    assert int((np.arange(K + 1) * hist).sum()) == int(ro.counts[:N].sum())
    h0, m0, s0 = orc.route_stats(np.zeros((0, K), np.int32), N)
    assert not h0.any() and m0 == 0.0 and s0 == 0.0


def test_global_batch_counts_are_micro_batch_sums(orc):
    """Routing is per token, so the T_i of Eq.(2) over a global batch equal
    the sums of the micro-batches' counts, and one bias update on the summed
    counts with T_all = sum of T equals the update on the whole batch."""
    r = rng(10)
    N, Z, K = 16, 8, 4
    bias = r.uniform(-0.05, 0.05, N + Z).astype(np.float32)
    parts = [r.standard_normal((T, N + Z)) for T in (37, 64, 5)]
    whole = orc.route(np.concatenate(parts), bias, N, K)
    acc = sum(orc.route(p, bias, N, K).counts.astype(np.int64) for p in parts)
    np.testing.assert_array_equal(acc, whole.counts)
    T_all = sum(p.shape[0] for p in parts)
    b1 = orc.pid_update(acc.astype(np.int32), T_all, bias, N, Z, K, 0.7, 2.5)
    b2 = orc.pid_update(whole.counts, T_all, bias, N, Z, K, 0.7, 2.5)
    np.testing.assert_array_equal(b1, b2)
