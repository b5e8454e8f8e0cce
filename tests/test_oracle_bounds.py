"""Pins of the oracle's device-deviation bounds (reading R10) against
simulations of the device's arithmetic (CPU only).

Each bound is derived on paper; these tests compute the same quantity the
way an fp32 device would (sequential fp32 sums in several orders and
groupings, the exponential and reciprocal perturbed by one unit in the last
place in every combination) and check that the bound contains every
simulated result, and that the bound's zero cases (exactly representable
partial sums) really are exact.  Dropping a term of a bound (the |g| factor
of the exponential's argument, the input-error propagation of SiLU, the two
roundings of the reciprocal multiply) makes one of them fail."""

import math

import numpy as np
import pytest

from oracle import formats as F
from oracle import moe_oracle as O

f32 = np.float32


def _fp32_seq_sum(terms: np.ndarray, order: np.ndarray) -> np.float32:
    acc = f32(0.0)
    for t in terms[order]:
        acc = f32(acc + f32(t))
    return acc


def _device_like_dot(xq, sx, wq, sw, rng, order_kind):
    """One output element the way the FP8 expert GEMM forms it: per 128-wide
    K block an fp32 sum of the exact code products (in some order), then
    acc = fl32(acc + p * fl32(sx * sw)) block by block."""
    K = xq.size
    acc = f32(0.0)
    for b in range(K // 128):
        prods = (xq[b * 128:(b + 1) * 128] * wq[b * 128:(b + 1) * 128]).astype(np.float64)
        if order_kind == "forward":
            order = np.arange(128)
        elif order_kind == "reverse":
            order = np.arange(128)[::-1]
        else:
            order = rng.permutation(128)
        p = _fp32_seq_sum(prods, order)
        sc = f32(f32(sx[b]) * f32(sw[b]))
        acc = f32(np.float64(acc) + np.float64(p) * np.float64(sc))
    return float(acc)


@pytest.mark.parametrize("order_kind", ["forward", "reverse", "random"])
def test_accumulation_bound_contains_fp32_sums(order_kind):
    rng = np.random.default_rng(11)
    m, N, K = 3, 5, 1024
    spec = O.Spec(m, K, 1, 1, 128)
    xq = F.E4M3_TABLE[rng.integers(0, 0x7F, size=(m, K)) | (rng.integers(0, 2, size=(m, K)) << 7)]
    wq = F.E4M3_TABLE[rng.integers(0, 0x7F, size=(N, K)) | (rng.integers(0, 2, size=(N, K)) << 7)]
    sx = F.f32_round(rng.uniform(0.001, 0.01, size=(m, K // 128)))
    sw = F.f32_round(rng.uniform(1e-4, 1e-3, size=(N, K // 128)))
    xh = xq * np.repeat(sx, 128, axis=1)
    wh = wq * np.repeat(sw, 128, axis=1)
    exact = xh @ wh.T
    bound = O.accumulation_bound(spec, xh, wh, scales_pow2=False)
    assert np.all(bound > 0)
    for r in range(m):
        for c in range(N):
            dev = _device_like_dot(xq[r], sx[r], wq[c], sw[c], rng, order_kind)
            assert abs(dev - exact[r, c]) <= bound[r, c], (r, c, abs(dev - exact[r, c]), bound[r, c])


def test_exact_sums_detected_and_exact():
    # x on multiples of 0.5 within [-4, 4], weights n * 2**-6 (|n| <= 15), all
    # scales powers of two: every partial sum is exact in fp32.
    rng = np.random.default_rng(12)
    m, N, K = 4, 6, 1024
    x = rng.integers(-8, 9, size=(m, K)) * 0.5 * 0.25
    w = rng.integers(-15, 16, size=(N, K)) * 2.0 ** -6 * 2.0
    assert np.all(O.fp32_sums_exact(x, w, scales_pow2=True))
    spec = O.Spec(m, K, 1, 1, 128)
    assert np.all(O.accumulation_bound(spec, x, w, True) == 0)
    exact = x @ w.T
    for r in range(m):
        for c in range(N):
            for order in (np.arange(K), rng.permutation(K)):
                assert float(_fp32_seq_sum(x[r] * w[c], order)) == exact[r, c]
    # one off-grid weight, or non-power-of-two scales, and the claim is withdrawn
    w2 = w.copy()
    w2[0, 0] = 1.0 / 3.0
    assert not O.fp32_sums_exact(x, w2, True).all()
    assert not O.fp32_sums_exact(x, w, False).any()
    # magnitude: sums past 2**24 grid units are not claimed exact
    big = np.full((1, K), 4096.5)                  # 2**24.6 units of 2**-7
    assert not O.fp32_sums_exact(big, np.full((1, K), 2.0 ** -6 * 3), True).any()
    assert O.fp32_sums_exact(big[:, :512], np.full((1, 512), 2.0 ** -6 * 3), True).all()


def _ulp32(v):
    v = np.float32(v)
    return float(np.nextafter(np.abs(v), np.float32(np.inf)) - np.abs(v))


def _device_silu_mul(g, u, exp_bump, rcp_bump):
    """a = g * rcp(1 + exp2(fl32(g * fl32(-log2 e)))) * u in fp32, with the
    exponential and the reciprocal off by exp_bump / rcp_bump units in the
    last place (the instructions' stated accuracy is one unit)."""
    g, u = f32(g), f32(u)
    t = f32(g * f32(-1.4426950408889634))
    e = f32(2.0 ** float(t))
    e = f32(float(e) + exp_bump * _ulp32(e))
    d = f32(f32(1.0) + e)
    r = f32(1.0 / float(d))
    r = f32(float(r) + rcp_bump * _ulp32(r))
    return float(f32(f32(g * r) * u))


def test_swiglu_bound_contains_device_evaluation():
    rng = np.random.default_rng(13)
    gs = np.concatenate([rng.standard_normal(300) * 3, rng.uniform(-79, 60, 300), [0.0, -1e-30, 1e-3]])
    us = rng.standard_normal(gs.size) * rng.choice([1e-3, 1.0, 40.0], gs.size)
    gs = F.f32_round(gs)
    us = F.f32_round(us)
    exact = O.swiglu(gs, us)
    b = O.swiglu_bound(gs, us, 0.0, 0.0)
    worst = 0.0
    for i in range(gs.size):
        for eb in (-1, 0, 1):
            for rb in (-1, 0, 1):
                d = abs(_device_silu_mul(gs[i], us[i], eb, rb) - exact[i])
                assert d <= b[i], (gs[i], us[i], eb, rb, d, b[i])
                if b[i] > 0:
                    worst = max(worst, d / b[i])
    # the bound is not vacuous: the simulated errors reach a fair part of it
    assert worst > 0.05


def test_swiglu_bound_propagates_input_error():
    rng = np.random.default_rng(14)
    g = rng.standard_normal(500) * 4
    u = rng.standard_normal(500) * 2
    eg = np.abs(rng.standard_normal(500)) * 1e-3
    eu = np.abs(rng.standard_normal(500)) * 1e-3
    b = O.swiglu_bound(g, u, eg, eu)
    for sgn_g in (-1, 1):
        for sgn_u in (-1, 1):
            dev = O.swiglu(g + sgn_g * eg, u + sgn_u * eu)
            assert np.all(np.abs(dev - O.swiglu(g, u)) <= b)


def test_requant_window_two_roundings_and_scale_window():
    # a / s at exactly 336 (the midpoint of 320 and 352) scaled so that s = 1:
    # a relative offset well inside the reciprocal-multiply rounding (U1) is a
    # near-tie, one well outside is not.
    a = np.zeros((1, 128))
    a[0, 0] = 448.0
    a[0, 1] = 336.0 * (1 + 1e-9)
    a[0, 2] = 336.0 * (1 + 1e-5)
    a[0, 3] = -2.375 * (1 - 1e-9)
    ea = np.zeros_like(a)
    codes, s, deq = O.requant_fp8(a)
    assert s[0, 0] == 1.0
    v, lo, hi = O.requant_window(a, ea, s)
    assert (lo[0, 0, 1], hi[0, 0, 1]) == (320.0, 352.0)
    assert lo[0, 0, 2] == hi[0, 0, 2] == 352.0
    assert (lo[0, 0, 3], hi[0, 0, 3]) == (-2.5, -2.25)
    other = codes.copy()
    other[0, 1] = F.e4m3_encode(np.array([320.0]))[0]
    other[0, 3] = F.e4m3_encode(np.array([-2.5]))[0]
    c2, _, d2 = O.requant_fp8(a, ea, resolve=other)
    assert d2[0, 1] == 320.0 and d2[0, 3] == -2.5
    bad = codes.copy()
    bad[0, 2] = F.e4m3_encode(np.array([320.0]))[0]          # away from a near-tie
    with pytest.raises(ValueError):
        O.requant_fp8(a, ea, resolve=bad)
    # +0 and -0 are the same value
    z = codes.copy()
    z[0, 100] = 0x80
    O.requant_fp8(a, ea, resolve=z)
    # scale window: amax 448 exactly gives only s = 1; an amax error moves it
    s_lo, s_hi, _, _ = O.scale_window(a, ea)
    assert s_lo[0, 0] == s_hi[0, 0] == 1.0
    with pytest.raises(ValueError):
        O.requant_fp8(a, ea, resolve=codes, resolve_scales=np.array([[float(np.nextafter(f32(1), f32(2)))]]))
    ea2 = np.zeros_like(a)
    ea2[0, 0] = 448.0 * 2.0 ** -20
    s_lo2, s_hi2, _, _ = O.scale_window(a, ea2)
    up = float(np.nextafter(f32(1), f32(2)))
    assert s_lo2[0, 0] < 1.0 < s_hi2[0, 0] and s_hi2[0, 0] >= up
    O.requant_fp8(a, ea2, resolve=codes, resolve_scales=np.array([[up]]))
    # a zero block may come out of the device as scale 1 only
    zero = np.zeros((1, 128))
    O.requant_fp8(zero, np.zeros_like(zero), resolve=np.zeros((1, 128), np.uint8),
                  resolve_scales=np.array([[1.0]]))
    with pytest.raises(ValueError):
        O.requant_fp8(zero, np.zeros_like(zero), resolve=np.zeros((1, 128), np.uint8),
                      resolve_scales=np.array([[0.5]]))


def test_bf16_intermediate_window():
    a = np.array([[1.0 + 2.0 ** -8 * (1 + 1e-9), 1.0 + 2.0 ** -8 * 1.5, 3.0]])
    ea = np.full_like(a, 1e-6)
    spec = O.Spec(1, 128, 1, 1, 3, "bf16", "bf16")
    r = F.bf16_round(a)
    # first element: at a BF16 midpoint within ea -> both neighbours accepted
    alt = r.copy()
    alt[0, 0] = 1.0
    bits = np.asarray(alt, dtype=np.float32).view(np.uint32) >> 16
    got = O.quantise_intermediate(spec, a, ea, bits.astype(np.uint16))
    assert got[0, 0] == 1.0
    alt2 = r.copy()
    alt2[0, 1] = 1.0                                             # not a near-tie
    bits2 = (np.asarray(alt2, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)
    with pytest.raises(ValueError):
        O.quantise_intermediate(spec, a, ea, bits2)


def test_logit_bound_zero_on_exact_inputs_and_contains_fp32():
    rng = np.random.default_rng(15)
    T, H, E = 3, 512, 4
    spec = O.Spec(T, H, E, 1, 128)
    x = rng.integers(-8, 9, size=(T, H)) * 0.5
    wr = rng.integers(-64, 65, size=(E, H)) * 2.0 ** -6
    wr_bits = (wr.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    bias = (rng.integers(-64, 65, size=E) * 2.0 ** -6).astype(np.float32)
    xcodes = F.e4m3_encode(x)
    ones = np.ones((T, H // 128), np.float32)
    inp = dict(x=xcodes, x_scales=ones, router_w=wr_bits, router_bias=bias)
    assert np.all(O.logit_bound(spec, inp) == 0)
    # Gaussian activations with fp32 scales: the bound contains fp32 sums
    gcodes = F.e4m3_encode(rng.standard_normal((T, H)) * 50)
    sx = np.full((T, H // 128), 0.0073, dtype=np.float32)
    xg = O.decode_activations(spec, gcodes, sx)
    b = O.logit_bound(spec, dict(x=gcodes, x_scales=sx, router_w=wr_bits, router_bias=bias))
    assert np.all(b > 0)
    ex = xg @ F.bf16_decode(wr_bits).T + bias
    for t in range(T):
        for e in range(E):
            dev = f32(_fp32_seq_sum(xg[t] * F.bf16_decode(wr_bits)[e], rng.permutation(H)) + f32(bias[e]))
            assert abs(float(dev) - ex[t, e]) <= b[t, e]


def test_gamma_closed_form():
    assert O.gamma(1) == pytest.approx(2.0 ** -23, rel=1e-6)
    assert O.gamma(186) == pytest.approx(186 * 2.0 ** -23 / (1 - 186 * 2.0 ** -23), rel=1e-12)
    # the lowest-set-bit helper: 3 * 2**-7 and 5 * 2**-3 -> -7
    assert O._lowest_bit_exponent(np.array([3 * 2.0 ** -7, 5 * 2.0 ** -3, 0.0])) == -7
    assert O._lowest_bit_exponent(np.array([6.0])) == 1
    assert O.powers_of_two([1.0, 0.5, 2.0 ** -30]) and not O.powers_of_two([1.0, 3.0])


def test_pow2_requant_scale_codes_and_windows():
    rng = np.random.default_rng(16)
    a = rng.standard_normal((4, 256)) * np.array([0.01, 3.0, 700.0, 1e-30]).repeat(64)[None, :]
    codes, s, deq = O.requant_fp8(a, pow2=True)
    blocks = np.abs(a).reshape(4, 2, 128)
    amax = blocks.max(axis=2)
    assert O.powers_of_two(s)
    assert np.all((224.0 * s < amax) & (amax <= 448.0 * s))
    # the scaling is exact: the codes are the E4M3 rounding of a / s itself
    assert np.array_equal(codes, F.e4m3_encode((a.reshape(4, 2, 128) / s[:, :, None]).reshape(4, 256)))
    # idempotent on its own output
    c2, s2, d2 = O.requant_fp8(deq, pow2=True)
    assert np.array_equal(d2, deq) and np.array_equal(s2, s)
    # windows: with no device error only exact midpoints are ambiguous (no
    # reciprocal-multiply term for power-of-two scales)
    ea = np.zeros_like(a)
    _, lo, hi = O.requant_window(a, ea, s, pow2=True)
    assert np.all(lo == hi)
    # a device maximum a hair above a power-of-two boundary may double the scale
    b = np.zeros((1, 128))
    b[0, 0] = 448.0
    s_lo, s_hi, _, _ = O.scale_window(b, np.full_like(b, 1e-3), pow2=True)
    assert s_lo[0, 0] == 1.0 and s_hi[0, 0] == 2.0
    O.requant_fp8(b, np.full_like(b, 1e-3), resolve=F.e4m3_encode(b / 2), resolve_scales=np.array([[2.0]]), pow2=True)
    with pytest.raises(ValueError):
        O.requant_fp8(b, np.zeros_like(b), resolve=F.e4m3_encode(b / 2), resolve_scales=np.array([[2.0]]), pow2=True)
