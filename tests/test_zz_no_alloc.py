"""moe_forward_static (the allocation-free entry point) against moe_forward,
through the C ABI: the same outputs bit for bit, on two calls in a row of
which the second is smaller (the static workspace keeps the first call's
contents), in both launch modes; and the size limit."""

import pytest
import torch

from workloads import gen

pytestmark = pytest.mark.gpu

CASES = [
    gen.LayerConfig("na_big", 256, 2048, 64, 8, 512, "fp8", "fp8", zipf=1.1),
    gen.LayerConfig("na_small", 37, 512, 8, 2, 256, "fp8", "fp4"),
]


def _static_forward(L, lib, inp, k, mode):
    desc = L.desc_from_inputs(inp, k, mode)
    T, H = inp["x"].shape
    E = inp["w_gate_up"].shape[0]
    dev = inp["x"].device
    out = dict(y=torch.full((T, H), float("nan"), dtype=torch.bfloat16, device=dev),
               topk_ids=torch.full((T, k), -1, dtype=torch.int32, device=dev),
               topk_weights=torch.full((T, k), float("nan"), dtype=torch.float32, device=dev),
               expert_offsets=torch.full((E + 1,), -1, dtype=torch.int32, device=dev),
               perm=torch.full((T * k,), -1, dtype=torch.int32, device=dev))
    lib.moe_forward_static(desc, inp["x"], inp.get("x_scales"), inp["router_w"], inp.get("router_bias"),
                           inp["w_gate_up"], inp.get("w_gate_up_scales"), inp["w_down"], inp.get("w_down_scales"),
                           out["y"], out["topk_ids"], out["topk_weights"], out["expert_offsets"], out["perm"])
    return out


@pytest.mark.parametrize("mode", ["mega", "separate"])
def test_static_workspace_matches_forward(gpu_lib, mode):
    from moe_layer_router_amd import layer as L, lib
    for cfg in CASES:                                    # the second call is the smaller one
        print(f"[no_alloc] {cfg.name} {mode}", flush=True)
        inp = L.pack_weights(gen.make_inputs(cfg, seed=2, device="cuda"))
        assert lib.moe_workspace_size(L.desc_from_inputs(inp, cfg.k, mode)) <= lib.MOE_STATIC_WORKSPACE_BYTES
        got = _static_forward(L, lib, inp, cfg.k, mode)
        ref = L.forward(inp, cfg.k, mode=mode)
        torch.cuda.synchronize()
        for key in ("y", "topk_ids", "topk_weights", "expert_offsets", "perm"):
            assert torch.equal(got[key], ref[key]), f"{cfg.name}/{mode}: {key} differs from moe_forward"


def test_static_workspace_rejects_large_layers(gpu_lib):
    from moe_layer_router_amd import layer as L, lib
    cfg = gen.LayerConfig("na_large", 4096, 2048, 16, 8, 512, "fp8", "fp8")
    desc = lib.make_desc(cfg.T, cfg.H, cfg.E, cfg.I, cfg.k)
    assert lib.moe_workspace_size(desc) > lib.MOE_STATIC_WORKSPACE_BYTES
    x = torch.zeros(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(lib.MoeError) as ei:
        lib.moe_forward_static(desc, x, x, x, None, x, x, x, x, x, x, x, None, None)
    assert ei.value.status == lib.MOE_ERR_WORKSPACE_TOO_SMALL
    assert "moe_forward_static" in lib.moe_last_error()
