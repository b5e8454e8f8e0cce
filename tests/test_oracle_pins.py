"""Pins that tie the oracle to the mathematics rather than to itself (CPU only).

The pages print no worked example, so each step of the oracle is pinned by a
closed form, an invariant, a brute force on tiny inputs, or a second
independent formulation; the comment on each test names the mistake it would
catch."""

import math

import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle import moe_oracle as O
from workloads import gen as G


def _bf16_bits(a):
    return torch.tensor(np.asarray(a, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _fp8_bytes(a):
    return torch.tensor(np.asarray(a, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


# ------------------------------------------------------------------ decoding
def test_fp8_weight_block_orientation():
    # scales differ per (n-block, k-block); N != K so a transposed index fails
    N, K = 256, 384
    q = np.full((N, K), 0x38, dtype=np.uint8)                   # every value 1.0
    S = (np.arange(6, dtype=np.float32).reshape(2, 3) + 1) * 0.5
    w = O.decode_weight(O.Spec(1, K, 1, 1, N // 2, "fp8", "fp8"), q, S)
    for n in (0, 127, 128, 255):
        for k in (0, 127, 128, 300, 383):
            assert w[n, k] == S[n // 128, k // 128]


def test_fp4_weight_scale_groups_and_nibbles():
    N, K = 2, 64
    packed = np.zeros((N, K // 2), dtype=np.uint8)
    packed[0, 0] = 0x21            # k=0 -> 0.5, k=1 -> 1.0
    packed[1, 16] = 0x0F           # k=32 -> -6.0
    sc = np.array([[127, 130], [120, 128]], dtype=np.uint8)   # 1, 8 ; 2**-7, 2
    w = O.decode_weight(O.Spec(1, K, 1, 1, 1, "fp8", "fp4"), packed, sc)
    assert w[0, 0] == 0.5 and w[0, 1] == 1.0
    assert w[1, 32] == -6.0 * 2.0
    assert np.count_nonzero(w) == 3


def test_activation_scales_per_token_per_128():
    T, H = 2, 256
    x = np.full((T, H), 0x38, dtype=np.uint8)
    sx = np.array([[1.0, 2.0], [3.0, 4.0]], dtype=np.float32)
    v = O.decode_activations(O.Spec(T, H, 1, 1, 128), x, sx)
    assert v[0, 127] == 1.0 and v[0, 128] == 2.0 and v[1, 0] == 3.0 and v[1, 255] == 4.0


# ------------------------------------------------------------------- routing
def test_router_logits_exact_integer_arithmetic():
    # On the exact-arithmetic grid the logits equal an integer dot product:
    # x = a/2, Wr = b/64  =>  l * 128 = sum(a * b).  Catches a transposed
    # router matrix, a dropped scale or a dropped bias.
    inp = G.make_exact_router_inputs(16, 256, 8, seed=3, with_bias=True)
    ov = G.oracle_view(inp)
    spec = O.Spec(16, 256, 8, 2, 128)
    xh = O.decode_activations(spec, ov["x"], ov["x_scales"])
    l = O.router_logits(xh, ov["router_w"], ov["router_bias"])
    a = (F.E4M3_TABLE[ov["x"]] * 2).astype(np.int64)
    b = (F.bf16_decode(ov["router_w"]) * 64).astype(np.int64)
    bias = (ov["router_bias"].astype(np.float64) * 64).astype(np.int64)
    want = [[sum(int(a[t, h]) * int(b[e, h]) for h in range(256)) + 2 * int(bias[e])
             for e in range(8)] for t in range(16)]
    assert np.array_equal(l * 128, np.array(want, dtype=np.float64))


def test_topk_brute_force_with_ties():
    rng = np.random.default_rng(0)
    logits = rng.integers(-3, 4, size=(200, 9)).astype(np.float64)   # many exact ties
    for k in (1, 3, 9):
        ids = O.topk_select(logits, k)
        for t in range(logits.shape[0]):
            want = sorted(range(9), key=lambda e: (-logits[t, e], e))[:k]
            assert ids[t].tolist() == want


def test_zero_router_selects_first_k_with_uniform_weights():
    logits = np.zeros((5, 16))
    ids = O.topk_select(logits, 4)
    assert (ids == np.arange(4)).all()
    w = O.topk_weights(logits, ids)
    assert np.array_equal(w, np.full((5, 4), 0.25))


def test_weights_equal_full_softmax_renormalised():
    rng = np.random.default_rng(1)
    logits = rng.standard_normal((64, 32)) * 3
    ids = O.topk_select(logits, 6)
    w = O.topk_weights(logits, ids)
    full = np.exp(logits) / np.exp(logits).sum(axis=1, keepdims=True)
    sel = np.take_along_axis(full, ids, axis=1)
    assert np.allclose(w, sel / sel.sum(axis=1, keepdims=True), rtol=1e-13, atol=0)
    assert np.allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    assert np.all(np.diff(w, axis=1) <= 0)     # emitted in descending order
    assert np.array_equal(O.topk_weights(logits, O.topk_select(logits, 1)), np.ones((64, 1)))


def test_weights_closed_form_two_experts():
    # two selected logits a > b: w = (1/(1+e^(b-a)), e^(b-a)/(1+e^(b-a)))
    logits = np.array([[0.3, 2.0, -1.0, 1.5]])
    ids = O.topk_select(logits, 2)
    assert ids.tolist() == [[1, 3]]
    w = O.topk_weights(logits, ids)
    d = math.exp(-0.5)
    assert abs(w[0, 0] - 1 / (1 + d)) < 1e-15 and abs(w[0, 1] - d / (1 + d)) < 1e-15


# --------------------------------------------------------------- permutation
def test_permutation_two_formulations_agree():
    rng = np.random.default_rng(2)
    T, k, E = 300, 4, 13
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)])
    counts, offsets, perm, row_of = O.permutation(ids, E)
    flat = ids.reshape(-1)
    perm2 = np.argsort(flat, kind="stable")
    assert np.array_equal(perm, perm2)
    assert np.array_equal(counts, np.bincount(flat, minlength=E))
    assert offsets[0] == 0 and offsets[-1] == T * k
    # unpermute(permute(v)) == v
    v = rng.standard_normal(T * k)
    assert np.array_equal(v[perm][row_of], v)
    for e in range(E):
        seg = perm[offsets[e]:offsets[e + 1]]
        assert (flat[seg] == e).all()
        assert np.all(np.diff(seg // k) > 0)   # ascending, distinct tokens


def test_permutation_empty_and_single_expert():
    ids = np.zeros((7, 1), dtype=np.int64) + 2
    counts, offsets, perm, _ = O.permutation(ids, 4)
    assert counts.tolist() == [0, 0, 7, 0] and offsets.tolist() == [0, 0, 0, 7, 7]
    assert perm.tolist() == list(range(7))


# ------------------------------------------------------------ expert compute
def test_silu_closed_forms():
    z = np.array([0.0, math.log(3.0), -math.log(3.0), 40.0])
    s = O.silu(z)
    assert s[0] == 0.0
    assert abs(s[1] - 0.75 * math.log(3.0)) < 1e-15        # sigma(ln 3) = 3/4
    assert abs(s[2] - (-0.25 * math.log(3.0))) < 1e-15     # sigma(-ln 3) = 1/4
    assert abs(s[3] - 40.0) < 1e-12
    r = np.random.default_rng(3).standard_normal(100)
    assert np.allclose(O.silu(-r), O.silu(r) - r, rtol=0, atol=1e-14)
    assert np.array_equal(O.swiglu(r, np.zeros(100)), np.zeros(100))


def test_requant_properties():
    rng = np.random.default_rng(4)
    a = rng.standard_normal((6, 384)) * np.array([1e-3, 1.0, 50.0])[None, :].repeat(128, axis=1)
    a[5, 128:256] = 0.0
    codes, s, deq = O.requant_fp8(a)
    blocks = a.reshape(6, 3, 128)
    amax = np.abs(blocks).max(axis=2)
    # the largest element of every non-zero block maps to +-448
    arg = np.abs(blocks).argmax(axis=2)
    cb = codes.reshape(6, 3, 128)
    for r in range(6):
        for b in range(3):
            if amax[r, b] > 0:
                assert cb[r, b, arg[r, b]] & 0x7F == 0x7E
    # a zero block gets scale 1 and zero codes
    assert s[5, 1] == 1.0 and np.all(cb[5, 1] & 0x7F == 0)
    # scale is the fp32 rounding of amax / 448
    nz = amax > 0
    assert np.array_equal(s[nz], np.float32(amax[nz] / 448.0).astype(np.float64))
    # error bound: half an E4M3 ulp, relative 2**-4 for normals, s * 2**-10 below
    ratio = np.abs(blocks) / s[:, :, None]
    err = np.abs(blocks - deq.reshape(6, 3, 128))
    normal = ratio >= 2.0 ** -6
    assert np.all(err[normal] <= 2.0 ** -4 * np.abs(blocks[normal]) * (1 + 1e-12))
    assert np.all(err[~normal] <= (s[:, :, None] * 2.0 ** -10 * np.ones_like(blocks))[~normal] * (1 + 1e-12))
    # idempotent on already-quantised values
    codes2, s2, deq2 = O.requant_fp8(deq)
    assert np.array_equal(deq2, deq)


def _onehot_layer(alpha, beta, gamma, spec_act="fp8"):
    """T=1 token, x = e_h; gate row c has alpha at h, up row c has beta at h,
    down column c has gamma at row h2; all other weights zero, one expert."""
    H, I, h, c, h2 = 128, 128, 5, 17, 99
    spec = O.Spec(1, H, 1, 1, I, spec_act, "bf16")
    x = np.zeros((1, H), dtype=np.float32)
    x[0, h] = 1.0
    wgu = np.zeros((2 * I, H), dtype=np.float32)
    wgu[c, h] = alpha
    wgu[I + c, h] = beta
    wd = np.zeros((H, I), dtype=np.float32)
    wd[h2, c] = gamma
    inputs = dict(router_w=_bf16_bits(np.zeros((1, H))), router_bias=None,
                  w_gate_up=_bf16_bits(wgu)[None], w_gate_up_scales=None,
                  w_down=_bf16_bits(wd)[None], w_down_scales=None)
    if spec_act == "fp8":
        inputs["x"] = _fp8_bytes(x)
        inputs["x_scales"] = np.ones((1, 1), dtype=np.float32)
    else:
        inputs["x"] = _bf16_bits(x)
        inputs["x_scales"] = None
    return spec, inputs, h2


def test_onehot_closed_form_fixes_gate_up_order_and_orientation():
    # y[h2] = silu(alpha) * beta * gamma, up to the FP8 re-quantisation of a
    # single-element block (which is exact to fp32 rounding of the scale).
    # Swapping gate/up, or transposing either weight, changes the answer.
    alpha, beta, gamma = 1.5, -2.0, 0.75
    spec, inputs, h2 = _onehot_layer(alpha, beta, gamma)
    r = O.layer(spec, inputs)
    want = alpha / (1 + math.exp(-alpha)) * beta * gamma
    assert abs(r["y"][0, h2] - want) <= 1e-6 * abs(want)
    assert np.count_nonzero(r["y"]) == 1
    # BF16 intermediate for all-BF16 layers: a is rounded to BF16
    spec_b, inputs_b, _ = _onehot_layer(alpha, beta, gamma, "bf16")
    rb = O.layer(spec_b, inputs_b)
    a = alpha / (1 + math.exp(-alpha)) * beta
    assert rb["y"][0, h2] == F.bf16_round(np.array([a]))[0] * gamma


def _random_layer(T, H, E, k, I, act, weight, seed, identical=False, zero_router=False):
    cfg = G.LayerConfig("pin", T, H, E, k, I, act, weight)
    inp = G.make_inputs(cfg, seed=seed)
    if identical:
        for key in ("w_gate_up", "w_gate_up_scales", "w_down", "w_down_scales"):
            if inp[key] is not None:
                inp[key] = inp[key][:1].expand_as(inp[key]).contiguous()
    if zero_router:
        inp["router_w"] = torch.zeros_like(inp["router_w"])
    return O.Spec(T, H, E, k, I, act, weight), G.oracle_view(inp)


def _dense_bruteforce(spec, inp):
    """Every expert on every token, masked by the routing: no permutation,
    no gather, no scatter."""
    xh, logits, ids, w = O.route(spec, inp)
    y = np.zeros((spec.T, spec.H))
    for e in range(spec.E):
        mask = np.zeros(spec.T)
        for j in range(spec.k):
            mask += np.where(ids[:, j] == e, w[:, j], 0.0)
        s1 = None if inp["w_gate_up_scales"] is None else inp["w_gate_up_scales"][e]
        s2 = None if inp["w_down_scales"] is None else inp["w_down_scales"][e]
        wgu = O.decode_weight(spec, inp["w_gate_up"][e], s1)
        wd = O.decode_weight(spec, inp["w_down"][e], s2)
        y += mask[:, None] * O.expert_ffn(spec, xh, wgu, wd)
    return y


@pytest.mark.parametrize("act,weight,scales", [("bf16", "bf16", "f32"), ("fp8", "fp8", "f32"), ("fp8", "fp4", "f32"),
                                               ("fp8", "fp4", "pow2"), ("fp8", "fp8", "pow2")])
def test_layer_equals_dense_bruteforce(act, weight, scales):
    spec, inp = _random_layer(37, 256, 6, 3, 256, act, weight, seed=5)
    spec = O.Spec(spec.T, spec.H, spec.E, spec.k, spec.I, spec.act, spec.weight, scales)
    r = O.layer(spec, inp)
    ref = _dense_bruteforce(spec, inp)
    assert np.allclose(r["y"], ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_topk_all_experts_with_zero_router_is_dense_mixture():
    spec, inp = _random_layer(9, 128, 4, 4, 128, "fp8", "fp8", seed=6, zero_router=True)
    r = O.layer(spec, inp)
    xh = O.decode_activations(spec, inp["x"], inp["x_scales"])
    mix = np.zeros_like(r["y"])
    for e in range(4):
        wgu = O.decode_weight(spec, inp["w_gate_up"][e], inp["w_gate_up_scales"][e])
        wd = O.decode_weight(spec, inp["w_down"][e], inp["w_down_scales"][e])
        mix += O.expert_ffn(spec, xh, wgu, wd) / 4
    assert np.allclose(r["y"], mix, rtol=1e-12, atol=1e-13)
    assert np.array_equal(r["weights"], np.full((9, 4), 0.25))


def test_identical_experts_make_output_routing_independent():
    spec, inp = _random_layer(21, 256, 8, 3, 128, "fp8", "fp4", seed=7, identical=True)
    r1 = O.layer(spec, inp)
    inp2 = dict(inp)
    inp2["router_w"] = _bf16_bits(np.random.default_rng(8).standard_normal((8, 256)) * 0.3)
    r2 = O.layer(spec, inp2)
    assert not np.array_equal(r1["ids"], r2["ids"])
    assert np.allclose(r1["y"], r2["y"], rtol=1e-12, atol=1e-13)
    xh = O.decode_activations(spec, inp["x"], inp["x_scales"])
    wgu = O.decode_weight(spec, inp["w_gate_up"][0], inp["w_gate_up_scales"][0])
    wd = O.decode_weight(spec, inp["w_down"][0], inp["w_down_scales"][0])
    assert np.allclose(r1["y"], O.expert_ffn(spec, xh, wgu, wd), rtol=1e-12, atol=1e-13)


def test_doubling_down_weights_doubles_output_exactly():
    spec, inp = _random_layer(11, 128, 4, 2, 128, "fp8", "fp8", seed=9)
    r1 = O.layer(spec, inp)
    inp2 = dict(inp)
    inp2["w_down_scales"] = inp["w_down_scales"] * np.float32(2.0)
    r2 = O.layer(spec, inp2)
    assert np.array_equal(r2["y"], 2 * r1["y"])


def test_token_subset_equals_full_rows():
    spec, inp = _random_layer(40, 128, 5, 2, 128, "fp8", "fp8", seed=10)
    full = O.layer(spec, inp)
    toks = np.array([0, 7, 39])
    part = O.layer(spec, inp, tokens=toks)
    # equal up to BLAS blocking, which depends on the number of rows
    assert np.allclose(part["y"], full["y"][toks], rtol=1e-13, atol=1e-14)


def test_given_ids_are_used():
    spec, inp = _random_layer(10, 128, 4, 2, 128, "fp8", "fp8", seed=11)
    ids = np.tile(np.array([[3, 0]]), (10, 1))
    r = O.layer(spec, inp, ids=ids)
    assert np.array_equal(r["ids"], ids)
    assert r["counts"].tolist() == [10, 0, 0, 10]


# ------------------------------------------------------- input quantisation
def test_input_quant_amax_maps_to_448_and_zero_block():
    rng = np.random.default_rng(20)
    x = F.bf16_decode(_bf16_bits(rng.standard_normal((5, 384)) * np.array([1e-3, 1.0, 300.0]).repeat(128)))
    x[4, 128:256] = 0.0
    for pow2 in (False, True):
        codes, s = O.quantise_tokens_fp8(x, pow2)
        b = np.abs(x).reshape(5, 3, 128)
        cb = codes.reshape(5, 3, 128)
        amax = b.max(axis=2)
        arg = b.argmax(axis=2)
        assert s[4, 1] == 1.0 and np.all(cb[4, 1] & 0x7F == 0)
        nz = amax > 0
        if pow2:
            assert O.powers_of_two(s[nz])
            assert np.all(448.0 * s[nz] >= amax[nz]) and np.all(224.0 * s[nz] < amax[nz])
        else:
            # the amax element maps to +-448 (the reciprocal multiply may land a
            # hair above 448, which saturates)
            for r in range(5):
                for blk in range(3):
                    if nz[r, blk]:
                        assert cb[r, blk, arg[r, blk]] & 0x7F == 0x7E
            assert np.array_equal(s[nz], np.float32(amax[nz].astype(np.float32) / np.float32(448)).astype(np.float64))


def test_input_quant_reciprocal_multiply_matches_exact_rational():
    # fl32(x * fl32(1/s)) recomputed with exact rationals and one rounding per
    # step: catches a division taken in fp64, a missing fp32 rounding of the
    # reciprocal, or the product not rounded to fp32 before the E4M3 rounding.
    from fractions import Fraction
    rng = np.random.default_rng(21)
    x = F.bf16_decode(_bf16_bits(rng.standard_normal((3, 256)) * 7.3))
    codes, s = O.quantise_tokens_fp8(x)

    def rnd32(q: Fraction) -> float:
        # round a rational to the nearest fp32 (ties to even) via fp64 bracketing
        f = float(q)                               # correctly rounded to fp64
        c = np.float32(f)
        cands = [np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))]
        best = min(cands, key=lambda y: (abs(Fraction(float(y)) - q),
                                         int(np.frombuffer(np.float32(y).tobytes(), np.uint32)[0]) & 1))
        return float(best)

    # blocks where the fp32 reciprocal multiply and an exact division round to
    # different codes (found by search): amax 880 with x = 0.013427734375,
    # amax 800 with x = 150 and with x = 1.171875
    special = np.zeros((3, 256))
    special[0, 0], special[0, 1] = 880.0, 0.013427734375
    special[1, 0], special[1, 1] = 800.0, 150.0
    special[2, 0], special[2, 1] = 800.0, 1.171875
    sc, ss = O.quantise_tokens_fp8(special)
    exact_div = F.e4m3_encode(special[:, 1] / ss[:, 0])
    assert np.all(sc[:, 1] != exact_div)                       # the cases do tell the two apart
    x = np.concatenate([x, special])
    codes, s = O.quantise_tokens_fp8(x)
    for t in range(6):
        for blk in range(2):
            seg = x[t, blk * 128:(blk + 1) * 128]
            amax = Fraction(float(np.abs(seg).max()))
            s32 = rnd32(amax / 448) if amax > 0 else 1.0
            inv = rnd32(1 / Fraction(s32))
            assert s[t, blk] == s32
            for i in (0, 1, 17, 64, 127):
                v = rnd32(Fraction(float(seg[i])) * Fraction(inv))
                assert codes[t, blk * 128 + i] == F.e4m3_encode(np.array([v]))[0]


def test_input_quant_midpoints_with_unit_scale():
    # with a 448 in each block the scale is exactly 1 and v = x: codes are the
    # E4M3 round-to-nearest-even of x itself, ties to the even code
    x = np.zeros((1, 256))
    x[0, 0] = 448.0
    x[0, 1:6] = [336.0, -2.375, 15.5, 0.013671875, 1000.0 / 1024]   # ties: 320|352, -2.25|-2.5, 15|16
    x[0, 128] = -448.0
    x[0, 129] = 0.001953125 * 1.5                                     # between subnormals 2^-9 and 2^-8
    codes, s = O.quantise_tokens_fp8(x)
    assert s[0, 0] == 1.0 and s[0, 1] == 1.0
    vals = F.E4M3_TABLE[codes[0]]
    assert vals[1] == 320.0 and vals[2] == -2.5 and vals[3] == 16.0       # the even mantissa each time
    assert vals[129] == 0.00390625                                    # tie 1.5 * 2^-9 -> 2 * 2^-9 (even)
    assert np.array_equal(codes[0], F.e4m3_encode(x[0]))


def test_input_quant_pow2_exponent_exact():
    amax = np.array([448.0, 448.0000001, 224.0, 224.0 * (1 + 2 ** -20), 1e-45, 3.0e38, 0.0])
    e = O.pow2_scale_exponent(amax)
    assert e.tolist()[:4] == [0, 1, -1, 0]
    assert e[4] == -127 and e[5] == 120 and e[6] == 0          # 448 * 2**119 < 3e38 <= 448 * 2**120
    # dequantised values are within half an E4M3 step of x, in the normal range
    rng = np.random.default_rng(22)
    x = F.bf16_decode(_bf16_bits(rng.standard_normal((4, 128)) * 50))
    codes, s = O.quantise_tokens_fp8(x, pow2=True)
    deq = F.E4M3_TABLE[codes] * np.repeat(s, 128, axis=1)
    normal = np.abs(x) / np.repeat(s, 128, axis=1) >= 2.0 ** -6
    assert np.all(np.abs(deq - x)[normal] <= 2.0 ** -4 * np.abs(x)[normal])


def test_layer_quantising_its_input_equals_prequantised_layer():
    # A BF16-input layer that quantises its input (R12) computes exactly the
    # pre-quantised FP8 layer on the codes and scales of quantise_tokens_fp8,
    # except that its router reads the BF16 input.
    cfg = G.LayerConfig("pin_q", 29, 256, 6, 2, 128, "bf16", "fp8")
    inp = G.make_inputs(cfg, seed=23)
    wcfg = G.LayerConfig("pin_q", 29, 256, 6, 2, 128, "fp8", "fp8")
    winp = G.make_inputs(wcfg, seed=23)           # FP8 weights of the same shapes
    ov = G.oracle_view(inp)
    ov_w = G.oracle_view(winp)
    for key in ("w_gate_up", "w_gate_up_scales", "w_down", "w_down_scales"):
        ov[key] = ov_w[key]
    spec_q = O.Spec(29, 256, 6, 2, 128, "bf16_fp8", "fp8")
    xb = F.bf16_decode(ov["x"])
    codes, s = O.quantise_tokens_fp8(xb)
    ov_p = dict(ov, x=codes, x_scales=s.astype(np.float32))
    spec_p = O.Spec(29, 256, 6, 2, 128, "fp8", "fp8")
    rq = O.layer(spec_q, ov)
    # the router reads the BF16 input
    assert np.array_equal(rq["logits"], xb @ F.bf16_decode(ov["router_w"]).T)
    rp = O.layer(spec_p, ov_p, ids=rq["ids"])
    # the experts read exactly the quantised input
    assert np.array_equal(rq["xhat"], rp["xhat"])
    assert np.array_equal(rq["xhat"], F.E4M3_TABLE[codes] * np.repeat(s, 128, axis=1))
    # and the whole layer equals the mask-weighted dense brute force over it
    bf = _dense_bruteforce(spec_q, ov)
    assert np.allclose(rq["y"], bf, rtol=1e-12, atol=1e-12 * np.abs(bf).max())


# --------------------------------------------- per-channel FP8 weight scales
def test_fp8_weight_channel_scale_orientation():
    # R13: one scale per output row n over all of K.  N != K and every code
    # 1.0, so a scale applied per K column (or per 128-row block) fails.
    N, K = 256, 384
    q = np.full((N, K), 0x38, dtype=np.uint8)
    s = (np.arange(N, dtype=np.float32) + 1) * 0.25
    w = O.decode_weight(O.Spec(1, K, 1, 1, N // 2, "fp8", "fp8", wscale="channel"), q, s)
    for n in (0, 1, 127, 128, 255):
        assert np.all(w[n] == s[n])
    with pytest.raises(ValueError):
        O.decode_weight(O.Spec(1, K, 1, 1, N // 2, "fp8", "fp8", wscale="channel"), q, s[:K // 128])


def test_channel_scales_equal_block_scales_constant_along_k():
    # a block-scaled matrix whose scales do not change along K is the same
    # matrix with one scale per row (each 128-row block's scale repeated)
    rng = np.random.default_rng(3)
    N, K = 256, 512
    q = rng.integers(0, 256, (N, K), dtype=np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x38                                # no NaN codes
    sb = np.repeat(rng.uniform(0.5, 2.0, (N // 128, 1)).astype(np.float32), K // 128, axis=1)
    sc = np.repeat(sb[:, 0], 128)
    wb = O.decode_weight(O.Spec(1, K, 1, 1, N // 2, "fp8", "fp8"), q, sb)
    wc = O.decode_weight(O.Spec(1, K, 1, 1, N // 2, "fp8", "fp8", wscale="channel"), q, sc)
    assert np.array_equal(wb, wc)


def test_onehot_layer_with_channel_scales():
    # one token, one expert, one nonzero weight per matrix, each with its own
    # channel scale: y[h2] = silu(a * sg) * (b * su) * (c * sd), up to the
    # exact-to-fp32 re-quantisation of a one-element block.  A scale taken
    # from the wrong row (or the gate's scale applied to up) changes it.
    H, I = 256, 128
    h1, i1, h2 = 5, 7, 200
    q_gu = np.zeros((1, 2 * I, H), dtype=np.uint8)
    q_gu[0, i1, h1] = _fp8_bytes([1.5])[0]
    q_gu[0, I + i1, h1] = _fp8_bytes([-2.0])[0]
    q_d = np.zeros((1, H, I), dtype=np.uint8)
    q_d[0, h2, i1] = _fp8_bytes([0.75])[0]
    s_gu = np.ones((1, 2 * I), dtype=np.float32)
    s_gu[0, i1], s_gu[0, I + i1] = 0.5, 4.0
    s_d = np.ones((1, H), dtype=np.float32)
    s_d[0, h2] = 0.125
    x = np.zeros((1, H), dtype=np.uint8)
    x[0, h1] = 0x38
    inputs = dict(x=x, x_scales=np.ones((1, H // 128), dtype=np.float32),
                  router_w=_bf16_bits(np.zeros((1, H))), router_bias=None,
                  w_gate_up=q_gu, w_gate_up_scales=s_gu, w_down=q_d, w_down_scales=s_d)
    spec = O.Spec(1, H, 1, 1, I, "fp8", "fp8", wscale="channel")
    r = O.layer(spec, inputs)
    g, u = 1.5 * 0.5, -2.0 * 4.0
    want = g / (1 + math.exp(-g)) * u * (0.75 * 0.125)
    assert abs(r["y"][0, h2] - want) <= 1e-6 * abs(want)
    assert np.count_nonzero(r["y"]) == 1


def test_layer_with_channel_scales_equals_dense_bruteforce():
    cfg = G.LayerConfig("pin_chan", 37, 256, 6, 3, 256, "fp8", "fp8", wscale="channel")
    inp = G.oracle_view(G.make_inputs(cfg, seed=5))
    spec = G.spec_of(cfg)
    assert inp["w_gate_up_scales"][0].shape == (2 * cfg.I,) and inp["w_down_scales"][0].shape == (cfg.H,)
    r = O.layer(spec, inp)
    ref = _dense_bruteforce(spec, inp)
    assert np.allclose(r["y"], ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


# ------------------------------------------------ E5M6 quantisation (R15)
def test_e5m6_quantisation_block_max_and_error_bound():
    rng = np.random.default_rng(21)
    x = (rng.standard_normal((6, 384)) * np.exp2(rng.integers(-10, 10, (6, 1)))).astype(np.float32).astype(np.float64)
    x[2, 128:256] = 0.0                                          # a zero block
    for pow2 in (False, True):
        codes, s = O.quantise_tokens_e5m6(x, pow2=pow2)
        b = x.reshape(6, 3, 128)
        amax = np.abs(b).max(axis=2)
        assert s[2, 1] == 1.0 and np.all(codes[2, 128:256] == 0)
        if pow2:
            assert O.powers_of_two(s)
            nz = amax > 0
            assert np.all(F.E5M6_MAX * s[nz] >= amax[nz]) and np.all(F.E5M6_MAX * s[nz] / 2 < amax[nz])
            assert np.array_equal(codes.reshape(6, 3, 128), F.e5m6_encode(b / s[:, :, None]))
        else:
            # the block maximum lands on the largest code
            arg = np.abs(b).argmax(axis=2)
            top = np.take_along_axis(codes.reshape(6, 3, 128), arg[:, :, None], 2)[:, :, 0] & 0x7FF
            assert np.all(top[amax > 0] == 0x7BF)
        deq = O.dequantise_e5m6(codes, s)
        # half a unit in the 6th fraction bit, the subnormal step, and the fp32 roundings
        bound = np.abs(x) * (2.0 ** -7 + 2.0 ** -22) + np.repeat(s, 128, axis=1) * 2.0 ** -21
        assert np.all(np.abs(deq - x) <= bound)


def test_e5m6_quantisation_uses_the_e5m6_maximum():
    # a block whose maximum is 448 would keep its values unscaled under the
    # E4M3 rule; under the E5M6 rule the maximum maps to 65024
    x = np.zeros((1, 128))
    x[0, 0] = 448.0
    x[0, 1] = 3.0
    codes, s = O.quantise_tokens_e5m6(x)
    assert F.e5m6_decode(codes[0, 0]) == F.E5M6_MAX
    assert np.float32(s[0, 0]) == np.float32(448.0) / np.float32(F.E5M6_MAX)
    _, s2 = O.quantise_tokens_e5m6(x, pow2=True)
    assert s2[0, 0] == 2.0 ** -7                                # 65024 / 128 = 508 >= 448 > 254
