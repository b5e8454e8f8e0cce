"""The opt-in phase trace of the persistent kernel (MOE_FLAG_TRACE): the
traced call gives the same outputs as an untraced one, and the stamps are
ordered phase by phase in every workgroup."""

import numpy as np
import pytest
import torch

from workloads import gen

pytestmark = pytest.mark.gpu


def test_trace_stamps_ordered_and_outputs_unchanged(gpu_lib):
    from moe_layer_router_amd import layer as L, lib
    cfg = gen.LayerConfig("trace", 600, 512, 16, 4, 256, "fp8", "fp8")
    inp = L.pack_weights(gen.make_inputs(cfg, seed=8, device="cuda"))
    a = L.forward(inp, cfg.k, mode="mega")
    b = L.forward(inp, cfg.k, mode="mega", trace=True)
    torch.cuda.synchronize()
    for key in ("y", "topk_ids", "topk_weights", "perm", "expert_offsets"):
        assert torch.equal(a[key], b[key]), key
    reg = lib.moe_get_workspace_regions(b["desc"])
    raw = b["workspace"][reg["trace"]: reg["trace"] + 1024 * 8 * 8].view(torch.int64).cpu().numpy().reshape(1024, 8)
    used = raw[:, 0] > 0
    assert used.sum() >= 1
    st = raw[used, :6]
    assert np.all(np.diff(st, axis=1) >= 0), "phase stamps out of order"
    ph = L.trace_phases(b)
    assert ph["exit"]["last"] >= ph["gateup_end"]["first"] >= 0
    n_gu = raw[used, 6].sum()
    assert n_gu == int(np.ceil(np.diff(b["expert_offsets"].cpu().numpy()) / 144).sum()) * (cfg.I // 128)
