"""Pins of the oracle's FP8 blockwise (MXFP8) quantizer and FP8 layer forward.

Format: OCP Microscaling MXFP8 with E4M3 elements: 32 consecutive values
along the reduction dimension share a power-of-two scale 2^(S-127) (E8M0);
elements are E4M3 (bias 7, 3 mantissa bits, subnormals m/8 * 2^-6, largest
finite 448, code 0x7f / 0xff NaN).  Checked against the format's closed
forms (decoded values of named codes), a brute-force nearest-value search
over all 256 codes, exact round trips of representable blocks, the error
bound of the rounding, and for the layer forward: identity experts return
the unquantized x, dense layers reduce to a plain composition of library
matmuls on the quantized operands, and the result stays within the
quantization's expected distance of the bf16 forward.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")


def rng(seed):
    return np.random.default_rng(seed)


def test_e4m3_named_codes(orc):
    v = orc.e4m3_value
    assert v(0x38) == 1.0 and v(0xb8) == -1.0
    assert v(0x7e) == 448.0 and v(0xfe) == -448.0          # largest finite
    assert v(0x08) == 2.0 ** -6                              # smallest normal
    assert v(0x01) == 2.0 ** -9 and v(0x07) == 7 * 2.0 ** -9  # subnormals
    assert v(0x00) == 0.0 and np.signbit(v(0x80))
    assert np.isnan(v(0x7f)) and np.isnan(v(0xff))
    assert v(0x40) == 2.0 and v(0x3c) == 1.5 and v(0x77) == 240.0


def _brute(x, table):
    finite = [c for c in range(256) if not np.isnan(table[c])]
    ax = min(abs(x), 448.0)
    x = np.copysign(ax, x)
    dmin = min(abs(table[c] - x) for c in finite)
    near = [c for c in finite if abs(table[c] - x) == dmin]
    even = [c for c in near if c % 2 == 0] or near
    if len(even) > 1:  # +0 / -0: the sign of x
        even = [c for c in even if (c >= 128) == bool(np.signbit(x))]
    return even[0]


def test_e4m3_encode_is_nearest_ties_to_even(orc):
    table = [orc.e4m3_value(c) for c in range(256)]
    finite = sorted({table[c] for c in range(256) if not np.isnan(table[c])})
    xs = list(finite)
    xs += [(a + b) / 2 for a, b in zip(finite[:-1], finite[1:])]          # every tie
    xs += [a + (b - a) * f for a, b in zip(finite[:-1], finite[1:]) for f in (0.25, 0.75)]
    xs += [460.0, 464.0, 500.0, 1e6, -470.0, 2.0 ** -11, -2.0 ** -10, 3 * 2.0 ** -11]
    xs += list(rng(1).uniform(-500, 500, 2000))
    for x in xs:
        got = orc.e4m3_encode(x)
        want = _brute(x, table)
        assert table[got] == table[want] and (got == want or table[got] == 0.0), (x, got, want)


def test_e4m3_round_trip_of_every_code(orc):
    for c in range(256):
        v = orc.e4m3_value(c)
        if np.isnan(v):
            continue
        assert orc.e4m3_encode(v) == c or v == 0.0


def test_mx_scale_closed_forms(orc):
    # one block per row: amax 1.0 -> S = 0 - 8 + 127; amax in [2^k, 2^(k+1))
    # -> S = k - 8 + 127; the block maximum lands in [256, 448] after scaling
    rows = []
    for amax in (1.0, 1.9, 2.0, 0.3, 448.0, 1e-3, 5e4):
        r = np.zeros(32)
        r[7] = -amax
        r[3] = amax / 3
        rows.append(r)
    rows.append(np.zeros(32))
    codes, scales = orc.mx_quantize(np.array(rows))
    for i, amax in enumerate((1.0, 1.9, 2.0, 0.3, 448.0, 1e-3, 5e4)):
        k = int(np.floor(np.log2(amax)))
        assert scales[i, 0] == k - 8 + 127
        top = -orc.e4m3_value(codes[i, 7])
        assert 256.0 <= top <= 448.0
    assert scales[-1, 0] == 0 and not (codes[-1] & 0x7f).any()


def test_mx_round_trip_of_representable_blocks(orc):
    r = rng(2)
    finite = [c for c in range(256) if not np.isnan(orc.e4m3_value(c))]
    big = [c for c in finite if 256 <= abs(orc.e4m3_value(c)) <= 448]
    rows, want_codes, want_s = [], [], []
    for i in range(50):
        S = int(r.integers(100, 150))
        cs = r.choice(finite, 32)
        cs[int(r.integers(32))] = r.choice(big)
        rows.append([orc.e4m3_value(c) * 2.0 ** (S - 127) for c in cs])
        want_codes.append(cs)
        want_s.append(S)
    codes, scales = orc.mx_quantize(np.array(rows))
    np.testing.assert_array_equal(scales[:, 0], want_s)
    deq = orc.mx_dequantize(codes, scales)
    np.testing.assert_array_equal(deq, np.array(rows))


def test_mx_error_bound_and_storage_types(orc):
    """Each element is within half an E4M3 step of its value at its own
    binade (2^(floor(log2|v|) - 4) X-relative), or 2^-10 X in the subnormal
    range, or saturated at 448 X; fp32 and bf16 inputs quantize like their
    binary64 values."""
    r = rng(3)
    a = (r.standard_normal((64, 256)) * np.exp(r.uniform(-6, 6, (64, 1)))).astype(np.float32)
    codes, scales = orc.mx_quantize(a)
    deq = orc.mx_dequantize(codes, scales)
    X = np.repeat(2.0 ** (scales.astype(np.float64) - 127), 32, axis=1)
    v = a.astype(np.float64) / X
    err = np.abs(deq / X - np.clip(v, -448, 448))
    bound = np.where(np.abs(v) >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(np.abs(v), 1e-300))) - 4),
                     2.0 ** -10)
    assert (err <= bound * (1 + 1e-12)).all()
    c64, s64 = orc.mx_quantize(a.astype(np.float64))
    np.testing.assert_array_equal(codes, c64)
    np.testing.assert_array_equal(scales, s64)
    bits = (a.view(np.uint32) >> 16).astype(np.uint16)   # bf16 truncation of a
    as_f = (bits.astype(np.uint32) << 16).view(np.float32)
    cb, sb = orc.mx_quantize(bits)
    cf, sf = orc.mx_quantize(as_f)
    np.testing.assert_array_equal(cb, cf)
    np.testing.assert_array_equal(sb, sf)


# ------------------------------------------------- the FP8 layer forward
def _layer(T, d, N, Z, I, K, seed, std=0.1):
    r = rng(seed)
    x = r.standard_normal((T, d)).astype(np.float32)
    wg = (std * r.standard_normal((N, I, d))).astype(np.float32)
    wu = (std * r.standard_normal((N, I, d))).astype(np.float32)
    wd = (std * r.standard_normal((N, d, I))).astype(np.float32)
    lg = r.standard_normal((T, N + Z))
    return x, wg, wu, wd, lg


def _mxq(orc, w):
    return {e: orc.mx_weights(w[e]) for e in range(w.shape[0])}


def test_forward_mx_is_a_composition_of_quantized_matmuls(orc):
    """Dense top-K = N + Z layer: the FP8 forward equals quantize(x) ->
    numpy matmuls -> SwiGLU in binary64 -> quantize(h) -> matmul -> gated
    sum, built from the pinned quantizer and library routines."""
    T, d, N, Z, I, K = 12, 64, 3, 2, 64, 5
    x, wg, wu, wd, lg = _layer(T, d, N, Z, I, K, seed=4)
    ro = orc.route(lg, np.zeros(N + Z, np.float32), N, K)
    Gq, Uq, Dq = _mxq(orc, wg), _mxq(orc, wu), _mxq(orc, wd)
    out = orc.forward_mx(x, Gq, Uq, Dq, ro.topk_idx, ro.gates, N, out_scale=0.5)
    G = {e: orc.mx_dequantize(*v) for e, v in Gq.items()}
    U = {e: orc.mx_dequantize(*v) for e, v in Uq.items()}
    D = {e: orc.mx_dequantize(*v) for e, v in Dq.items()}
    xq = orc.mx_dequantize(*orc.mx_quantize(x))
    want = np.zeros((T, d))
    for t in range(T):
        for r in range(K):
            e, g = ro.topk_idx[t, r], ro.gates[t, r]
            if e >= N:
                want[t] += g * x[t].astype(np.float64)
                continue
            a = G[e] @ xq[t]
            u = U[e] @ xq[t]
            h = a / (1 + np.exp(-a)) * u
            hq = orc.mx_dequantize(*orc.mx_quantize(h[None, :]))[0]
            want[t] += g * (D[e] @ hq)
    np.testing.assert_allclose(out, 0.5 * want, rtol=1e-12, atol=1e-12)


def test_forward_mx_identity_experts_use_unquantized_x(orc):
    T, d, N, Z, I, K = 8, 64, 2, 4, 32, 2
    x, wg, wu, wd, lg = _layer(T, d, N, Z, I, K, seed=5)
    idx = np.array([[N + t % Z, N + (t + 1) % Z] for t in range(T)], np.int32)
    gates = np.full((T, K), 0.5)
    out = orc.forward_mx(x, _mxq(orc, wg), _mxq(orc, wu), _mxq(orc, wd), idx, gates, N)
    np.testing.assert_array_equal(out, x.astype(np.float64))


def test_forward_mx_is_close_to_the_unquantized_forward(orc):
    """E4M3 keeps 4 significant bits: each operand is off by at most 2^-4
    relative, about 1.8% RMS for uniformly spread mantissas, so the layer
    output lands within a few percent (RMS) of the bf16-free fp64 forward,
    and clearly not on it."""
    T, d, N, Z, I, K = 32, 128, 4, 2, 64, 3
    x, wg, wu, wd, lg = _layer(T, d, N, Z, I, K, seed=6)
    ro = orc.route(lg, np.zeros(N + Z, np.float32), N, K)
    ref = orc.forward(x, wg, wu, wd, ro.topk_idx, ro.gates, N)
    out = orc.forward_mx(x, _mxq(orc, wg), _mxq(orc, wu), _mxq(orc, wd), ro.topk_idx, ro.gates, N)
    rel = np.sqrt(np.mean((out - ref) ** 2)) / np.sqrt(np.mean(ref ** 2))
    assert 1e-3 < rel < 0.06, rel


def test_forward_mx_flip_bound_covers_perturbed_h(orc):
    """The flip bound (largest output change from h codes within relative
    eps of a boundary, plus the fp32 rounding of h) is 0 for eps = 0 apart
    from that rounding, and covers the actual change when every h_i is
    moved by a random factor within 1 +- eps or is rounded to fp32 (numpy
    composition of the pinned quantizer), and is not vacuous."""
    T, d, N, Z, I, K = 10, 64, 3, 2, 64, 4
    x, wg, wu, wd, lg = _layer(T, d, N, Z, I, K, seed=7)
    ro = orc.route(lg, np.zeros(N + Z, np.float32), N, K)
    Gq, Uq, Dq = _mxq(orc, wg), _mxq(orc, wu), _mxq(orc, wd)
    eps = 2.0 ** -7
    out = orc.forward_mx(x, Gq, Uq, Dq, ro.topk_idx, ro.gates, N)
    fl = orc.mx_flip_bound(x, Gq, Uq, Dq, ro.topk_idx, ro.gates, N, eps)
    fl0 = orc.mx_flip_bound(x, Gq, Uq, Dq, ro.topk_idx, ro.gates, N, 0.0)
    assert fl.max() > 0 and (fl0 <= fl).all()
    G = {e: orc.mx_dequantize(*v) for e, v in Gq.items()}
    U = {e: orc.mx_dequantize(*v) for e, v in Uq.items()}
    D = {e: orc.mx_dequantize(*v) for e, v in Dq.items()}
    xq = orc.mx_dequantize(*orc.mx_quantize(x))
    r = rng(8)
    moved = 0.0
    for trial in range(7):
        want = np.zeros((T, d))
        for t in range(T):
            for k in range(K):
                e, g = ro.topk_idx[t, k], ro.gates[t, k]
                if e >= N:
                    want[t] += g * x[t].astype(np.float64)
                    continue
                a, u = G[e] @ xq[t], U[e] @ xq[t]
                h = a / (1 + np.exp(-a)) * u
                if trial == 0:  # the h an fp32 evaluation holds
                    h = h.astype(np.float32).astype(np.float64)
                else:
                    h = h * (1 + r.uniform(-eps, eps, I))
                hq = orc.mx_dequantize(*orc.mx_quantize(h[None, :]))[0]
                want[t] += g * (D[e] @ hq)
        diff = np.abs(want - out)
        moved = max(moved, diff.max())
        assert (diff <= (fl0 if trial == 0 else fl) * (1 + 1e-9) + 1e-13).all()
    assert moved > 0  # the perturbations did flip codes
