"""Pins of the oracle's backward pass (reading R14) against the forward
function it differentiates (CPU only): central finite differences along
random directions for every parameter, which a dropped term, a wrong sign
or a transposed operand in the analytic gradients would fail; and the
unrounded forward function against the oracle's layer."""

import numpy as np
import pytest

from oracle import moe_oracle as O
from workloads import gen as G


def _params(seed, T=7, H=24, E=5, k=2, I=8):
    rng = np.random.default_rng(seed)
    xh = rng.normal(size=(T, H))
    wr = rng.normal(size=(E, H)) / np.sqrt(H)
    b = rng.normal(size=E) * 0.3
    w_gu = rng.normal(size=(E, 2 * I, H)) / np.sqrt(H)
    w_d = rng.normal(size=(E, H, I)) / np.sqrt(I)
    logits = xh @ wr.T + b
    ids = O.topk_select(logits, k)
    # no near-ties, so a small perturbation keeps the selection
    srt = np.sort(logits, axis=1)[:, ::-1]
    assert np.min(srt[:, k - 1] - srt[:, k]) > 1e-4
    dy = rng.normal(size=(T, H))
    return dict(xh=xh, wr=wr, b=b, w_gu=w_gu, w_d=w_d), ids, dy, I


def _f(p, ids, dy, I):
    return float(np.sum(dy * O.forward_exact(p["xh"], p["xh"], p["wr"], p["b"], p["w_gu"], p["w_d"], ids, I)))


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("name,grad", [("xh", "dx"), ("w_gu", "dw_gate_up"), ("w_d", "dw_down"),
                                       ("wr", "dw_router"), ("b", "dbias")])
def test_backward_matches_finite_differences(seed, name, grad):
    p, ids, dy, I = _params(seed)
    g = O.backward_exact(p["xh"], p["xh"], p["wr"], p["b"], p["w_gu"], p["w_d"], ids, dy, I)[grad]
    rng = np.random.default_rng(100 + seed)
    eps = 1e-6
    for _ in range(3):
        v = rng.normal(size=p[name].shape)
        hi = dict(p, **{name: p[name] + eps * v})
        lo = dict(p, **{name: p[name] - eps * v})
        fd = (_f(hi, ids, dy, I) - _f(lo, ids, dy, I)) / (2 * eps)
        an = float(np.sum(g * v))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)


def test_router_gradient_vanishes_with_one_expert_per_token():
    # k = 1: the single weight is 1 whatever the logits, so the router and
    # bias get no gradient, and dx is the experts' part alone
    p, _, dy, I = _params(3)
    ids = O.topk_select(p["xh"] @ p["wr"].T + p["b"], 1)
    r = O.backward_exact(p["xh"], p["xh"], p["wr"], p["b"], p["w_gu"], p["w_d"], ids, dy, I)
    assert np.all(r["dw_router"] == 0) and np.all(r["dbias"] == 0)
    assert np.array_equal(r["dx"], r["dx_experts"])


def test_unused_experts_get_zero_gradients():
    p, ids, dy, I = _params(4, E=9, k=2)
    r = O.backward_exact(p["xh"], p["xh"], p["wr"], p["b"], p["w_gu"], p["w_d"], ids, dy, I)
    unused = sorted(set(range(9)) - set(ids.ravel().tolist()))
    assert unused, "the draw should leave some expert unused"
    for e in unused:
        assert np.all(r["dw_gate_up"][e] == 0) and np.all(r["dw_down"][e] == 0)
        assert np.all(r["dw_router"][e] == 0) and r["dbias"][e] == 0


def test_forward_exact_is_the_layer_up_to_the_intermediate_rounding():
    # BF16 layer: the oracle's layer rounds the intermediate to BF16; the
    # unrounded function differs from it by at most that rounding's effect
    cfg = G.LayerConfig("bwd_pin", 11, 256, 6, 2, 128, "bf16", "bf16")
    inp = G.oracle_view(G.make_inputs(cfg, seed=2))
    spec = G.spec_of(cfg)
    r = O.layer(spec, inp)
    from oracle import formats as F
    xh = F.bf16_decode(inp["x"])
    w_gu = np.stack([F.bf16_decode(inp["w_gate_up"][e]) for e in range(cfg.E)])
    w_d = np.stack([F.bf16_decode(inp["w_down"][e]) for e in range(cfg.E)])
    wr = F.bf16_decode(inp["router_w"])
    y = O.forward_exact(xh, xh, wr, np.zeros(cfg.E), w_gu, w_d, r["ids"], cfg.I)
    rms = np.sqrt((r["y"] ** 2).mean(axis=1, keepdims=True))
    assert np.max(np.abs(y - r["y"]) / rms) < 2 ** -7
    assert not np.array_equal(y, r["y"])


def test_layer_backward_decodes_the_inputs():
    cfg = G.LayerConfig("bwd_dec", 9, 256, 4, 2, 128, "bf16", "bf16")
    raw = G.make_inputs(cfg, seed=1)
    inp = G.oracle_view(raw)
    spec = G.spec_of(cfg)
    ids = O.route(spec, inp)[2]
    dy = np.random.default_rng(0).normal(size=(cfg.T, cfg.H))
    r = O.layer_backward(spec, inp, ids, dy)
    from oracle import formats as F
    xh = F.bf16_decode(inp["x"])
    w_gu = np.stack([F.bf16_decode(inp["w_gate_up"][e]) for e in range(cfg.E)])
    w_d = np.stack([F.bf16_decode(inp["w_down"][e]) for e in range(cfg.E)])
    ref = O.backward_exact(xh, xh, F.bf16_decode(inp["router_w"]), np.zeros(cfg.E), w_gu, w_d, ids, dy, cfg.I)
    for key in ("dx", "dw_gate_up", "dw_down", "dw_router", "dbias"):
        assert np.array_equal(r[key], ref[key]), key


def test_weight_grad_elements_match_backward_exact():
    # the per-element definition used for full-size sampling against the
    # whole-layer backward on a small problem, for a busy and a sparse expert
    rng = np.random.default_rng(77)
    T, H, E, k, I = 40, 24, 6, 3, 8
    xh = rng.standard_normal((T, H))
    wr = rng.standard_normal((E, H)) / 5
    b = rng.standard_normal(E) / 10
    w_gu = rng.standard_normal((E, 2 * I, H)) / 5
    w_d = rng.standard_normal((E, H, I)) / 3
    dy = rng.standard_normal((T, H))
    ids = O.topk_select(xh @ wr.T + b, k)
    ref = O.backward_exact(xh, xh, wr, b, w_gu, w_d, ids, dy, I)
    counts = np.bincount(ids.ravel(), minlength=E)
    chans = np.array([0, 3, I - 1])
    cols = np.array([1, 5, H - 1, 7])
    for e in (int(counts.argmax()), int(counts.argmin())):
        got = O.weight_grad_elements(xh, xh, wr, b, w_gu[e], w_d[e], e, ids, dy, I, chans, cols)
        np.testing.assert_allclose(got["dw_gate"], ref["dw_gate_up"][e][np.ix_(chans, cols)], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(got["dw_up"], ref["dw_gate_up"][e][np.ix_(I + chans, cols)], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(got["dw_down"], ref["dw_down"][e][np.ix_(cols, chans)], rtol=1e-12, atol=1e-12)


def test_router_and_bias_gradients_sum_to_zero_over_experts():
    # the routing weights of a token sum to one, so the logit gradients of a
    # token sum to zero: sum_e dbias[e] = 0 and sum_e dW_r[e] = 0 exactly
    rng = np.random.default_rng(78)
    T, H, E, k, I = 30, 16, 8, 4, 8
    xh = rng.standard_normal((T, H))
    wr = rng.standard_normal((E, H)) / 4
    b = rng.standard_normal(E) / 10
    w_gu = rng.standard_normal((E, 2 * I, H)) / 4
    w_d = rng.standard_normal((E, H, I)) / 3
    dy = rng.standard_normal((T, H))
    ids = O.topk_select(xh @ wr.T + b, k)
    ref = O.backward_exact(xh, xh, wr, b, w_gu, w_d, ids, dy, I)
    assert abs(ref["dbias"].sum()) < 1e-12 * np.abs(ref["dbias"]).sum()
    assert np.all(np.abs(ref["dw_router"].sum(axis=0)) < 1e-12 * np.abs(ref["dw_router"]).sum(axis=0))
