"""The backward pass (moe_backward) against the oracle's gradients (reading
R14), through the C ABI: BF16 layers, the routing a forward call returned,
every gradient element-wise within BWD_TOL of the reference scale, and exact
zeros where the reference is zero (experts no token chose).

BWD_TOL: the device's operands are exact (BF16 inputs and weights) or within
2^-17 of fp32 intermediates (split into two BF16 parts), and its sums are
fp32, so each gradient element is within a few fp32 roundings per term of
the exact sum: relative to the largest terms, below 1e-4 for the sums here.
1e-3 leaves a wide margin above that and lies well below what a single BF16
rounding of the intermediate gradients gives (1e-2 to 4e-2 on these cases)."""

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from oracle import formats as F
from workloads import gen

from tests._helpers import to_dev

pytestmark = pytest.mark.gpu

BWD_TOL = 1e-3

CASES = [
    gen.LayerConfig("b_small", 70, 256, 6, 2, 128, "bf16", "bf16"),
    gen.LayerConfig("b_multi", 300, 384, 16, 4, 256, "bf16", "bf16"),       # H % 128 == 0, H % 256 != 0
    gen.LayerConfig("b_one_token", 1, 256, 4, 2, 128, "bf16", "bf16"),
    gen.LayerConfig("b_k_eq_e", 90, 256, 4, 4, 128, "bf16", "bf16"),        # every expert for every token
    gen.LayerConfig("b_zipf", 260, 512, 24, 4, 384, "bf16", "bf16", zipf=1.1),  # skewed loads, unused experts
]


def _check(name, got, ref, rms_axes):
    """|got - ref| / max(|ref|, rms of ref over rms_axes) <= BWD_TOL, and
    exact zeros where the whole reference block is zero."""
    rms = np.sqrt((ref ** 2).mean(axis=rms_axes, keepdims=True))
    zero = rms == 0
    if np.any(zero):
        assert np.all(got[np.broadcast_to(zero, got.shape)] == 0), f"{name}: nonzero gradient of an unused block"
    floor = np.where(zero, 1.0, rms)
    err = np.abs(got - ref) / np.maximum(np.abs(ref), floor)
    assert np.all(np.isfinite(got)), f"{name}: non-finite"
    assert err.max() <= BWD_TOL, f"{name}: max relative error {err.max():.3e} at {np.unravel_index(err.argmax(), err.shape)}"
    return float(err.max())


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_backward_matches_oracle(gpu_lib, cfg):
    from moe_layer_router_amd import layer as L
    raw = gen.make_inputs(cfg, seed=11)
    dev = to_dev(raw)
    fwd = L.forward(L.pack_weights(dev), cfg.k, mode="mega")
    g = torch.Generator(device="cpu").manual_seed(12)
    dy = torch.randn(cfg.T, cfg.H, generator=g).to(torch.bfloat16).cuda()
    out = L.backward(dev, fwd["topk_ids"], fwd["topk_weights"], dy)
    torch.cuda.synchronize()
    spec = gen.spec_of(cfg)
    ov = gen.oracle_view(raw)
    ids = fwd["topk_ids"].cpu().numpy().astype(np.int64)
    w_dev = fwd["topk_weights"].cpu().numpy().astype(np.float64)
    ref = O.layer_backward(spec, ov, ids, F.bf16_decode(dy.cpu().view(torch.int16).numpy().view(np.uint16)))
    # the device's routing weights are the forward call's; the oracle's own
    # softmax of its fp64 logits differs from them by <= 1e-5, far inside the bar
    assert np.allclose(O.topk_weights(O.route(spec, ov)[1], ids), w_dev, atol=1e-5)
    errs = {}
    errs["dx"] = _check("dx", out["dx"].cpu().numpy(), ref["dx"], (1,))
    errs["dw_gate_up"] = _check("dw_gate_up", out["dw_gate_up"].cpu().numpy(), ref["dw_gate_up"], (1, 2))
    errs["dw_down"] = _check("dw_down", out["dw_down"].cpu().numpy(), ref["dw_down"], (1, 2))
    errs["dw_router"] = _check("dw_router", out["dw_router"].cpu().numpy(), ref["dw_router"], (0, 1))
    errs["dbias"] = _check("dbias", out["dbias"].cpu().numpy(), ref["dbias"], (0,))
    print(cfg.name, {k: f"{v:.2e}" for k, v in errs.items()})


def test_backward_is_deterministic(gpu_lib):
    from moe_layer_router_amd import layer as L
    cfg = CASES[1]
    dev = to_dev(gen.make_inputs(cfg, seed=3))
    fwd = L.forward(L.pack_weights(dev), cfg.k, mode="separate")
    dy = torch.randn(cfg.T, cfg.H, generator=torch.Generator(device="cpu").manual_seed(4)).to(torch.bfloat16).cuda()
    a = L.backward(dev, fwd["topk_ids"], fwd["topk_weights"], dy)
    b = L.backward(dev, fwd["topk_ids"], fwd["topk_weights"], dy)
    torch.cuda.synchronize()
    for key in a:
        assert torch.equal(a[key], b[key]), key
