"""Convenience wrapper: allocate outputs and workspace with PyTorch and call
moe_forward / moe_route / moe_permute.  No arithmetic happens here."""

import torch

from . import lib


def pack_weights(inputs: dict, top_k: int = 1, stream=None) -> dict:
    """Copy of `inputs` whose expert weights (and FP4 scales) are in the
    MFMA-tiled layout moe_forward reads (moe_pack_weights).  The input dict
    is not modified; the result carries "weights_packed": True."""
    if inputs.get("weights_packed"):
        return inputs
    desc = desc_from_inputs(inputs, top_k, layout="row_major")
    fp4 = desc.weight_dtype == lib.MOE_DTYPE_FP4_E2M1
    out = dict(inputs)
    for which, w, sc in ((lib.MOE_WEIGHTS_GATE_UP, "w_gate_up", "w_gate_up_scales"),
                         (lib.MOE_WEIGHTS_DOWN, "w_down", "w_down_scales")):
        dst = torch.empty_like(inputs[w])
        dst_sc = torch.empty_like(inputs[sc]) if fp4 else None
        lib.moe_pack_weights(desc, which, inputs[w].contiguous(), inputs[sc].contiguous() if fp4 else None,
                             dst, dst_sc, stream)
        out[w] = dst
        if fp4:
            out[sc] = dst_sc
    out["weights_packed"] = True
    return out


def desc_from_inputs(inputs: dict, top_k: int, mode: str = "mega", flags: int = 0, I=None, layout=None,
                     inter_scale: str = "f32") -> lib.MoeDesc:
    x = inputs["x"]
    T, H = x.shape
    E = inputs["w_gate_up"].shape[0]
    if I is None:
        I = inputs["w_gate_up"].shape[1] // 2
    act = "bf16" if x.dtype == torch.bfloat16 else "fp8"
    wgu = inputs["w_gate_up"]
    if wgu.dtype == torch.bfloat16:
        weight = "bf16"
    elif wgu.shape[2] == H:
        weight = "fp8"
    else:
        weight = "fp4"
    if layout is None:
        layout = "tiled" if inputs.get("weights_packed") else "row_major"
    # FP8 weight scales: [E][N/128][K/128] per block, [E][N] per output channel
    sc = inputs.get("w_gate_up_scales")
    wscale = "channel" if weight == "fp8" and sc is not None and sc.dim() == 2 else "block"
    return lib.make_desc(T, H, E, I, top_k, act, weight, mode, flags, layout, inter_scale, wscale)


class Workspace:
    """A cached device workspace, grown on demand."""

    def __init__(self, device="cuda"):
        self.device = device
        self.buf = None

    def get(self, nbytes: int) -> torch.Tensor:
        if self.buf is None or self.buf.numel() < nbytes:
            self.buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=self.device)
        return self.buf


def forward(inputs: dict, top_k: int, mode: str = "mega", workspace: Workspace = None,
            routing=None, want_perm: bool = True, stream=None, out=None, inter_scale: str = "f32",
            trace: bool = False) -> dict:
    """Run the layer on inputs whose weights went through pack_weights().
    routing=(topk_ids, topk_weights) feeds given routing
    (MOE_FLAG_ROUTING_GIVEN).  Returns dict(y, topk_ids, topk_weights,
    expert_offsets, perm)."""
    if not inputs.get("weights_packed"):
        raise ValueError("forward() needs MFMA-tiled weights: pass the inputs through pack_weights() first")
    flags = (lib.MOE_FLAG_ROUTING_GIVEN if routing is not None else 0) | (lib.MOE_FLAG_TRACE if trace else 0)
    desc = desc_from_inputs(inputs, top_k, mode, flags, inter_scale=inter_scale)
    dev = inputs["x"].device
    T, H, E, k = desc.T, desc.H, desc.E, desc.top_k
    if out is None:
        out = dict(y=torch.empty(T, H, dtype=torch.bfloat16, device=dev),
                   topk_ids=torch.empty(T, k, dtype=torch.int32, device=dev),
                   topk_weights=torch.empty(T, k, dtype=torch.float32, device=dev),
                   expert_offsets=torch.empty(E + 1, dtype=torch.int32, device=dev) if want_perm else None,
                   perm=torch.empty(T * k, dtype=torch.int32, device=dev) if want_perm else None)
    if routing is not None:
        out["topk_ids"].copy_(routing[0])
        out["topk_weights"].copy_(routing[1])
    ws = (workspace or Workspace(dev)).get(lib.moe_workspace_size(desc))
    if trace:      # rows of workgroups that do not run must read as unused
        reg = lib.moe_get_workspace_regions(desc)
        ws[reg["trace"]: reg["trace"] + lib.MOE_TRACE_GROUPS * lib.MOE_TRACE_FIELDS * 8].zero_()
    lib.moe_forward(desc, inputs["x"], inputs.get("x_scales"), inputs["router_w"], inputs.get("router_bias"),
                    inputs["w_gate_up"], inputs.get("w_gate_up_scales"), inputs["w_down"],
                    inputs.get("w_down_scales"), out["y"], out["topk_ids"], out["topk_weights"],
                    out["expert_offsets"], out["perm"], ws, stream)
    out["workspace"] = ws
    out["desc"] = desc
    return out


def intermediate(out: dict):
    """Views of the intermediate activations of a finished forward() call:
    (codes or BF16 values [T*k][I] in permuted row order, scales [T*k][I/128]
    or None)."""
    desc, ws = out["desc"], out["workspace"]
    reg = lib.moe_get_workspace_regions(desc)
    rows, I = desc.T * desc.top_k, desc.I
    if desc.weight_dtype != lib.MOE_DTYPE_BF16:     # FP8 / FP4 experts: E4M3 intermediate
        codes = ws[reg["inter"]: reg["inter"] + rows * I].view(rows, I)
        sc = ws[reg["inter_scales"]: reg["inter_scales"] + rows * (I // 128) * 4].view(torch.float32)
        return codes, sc.view(I // 128, rows).t()       # stored K block major
    vals = ws[reg["inter"]: reg["inter"] + rows * I * 2].view(torch.bfloat16).view(rows, I)
    return vals, None


def quantize_input(x: torch.Tensor, scale_mode: str = "f32", stream=None):
    """Per-token FP8 quantisation of [T, H] BF16 / fp32 activations
    (moe_quantize_input): returns (codes uint8 [T, H], scales float32 [T, H/128])."""
    T, H = x.shape
    xq = torch.empty(T, H, dtype=torch.uint8, device=x.device)
    xs = torch.empty(T, H // 128, dtype=torch.float32, device=x.device)
    lib.moe_quantize_input(x.contiguous(), xq, xs, scale_mode, stream)
    return xq, xs


def quantize_e5m6(x: torch.Tensor, scale_mode: str = "f32", stream=None):
    """Per-token, per-128-channel E5M6 quantisation (moe_quantize_e5m6) of a
    [T, H] bfloat16 / float32 tensor: (codes [T, 3H/2] uint8, scales
    [T, H/128] float32)."""
    T, H = x.shape
    xq = torch.empty(T, H // 2 * 3, dtype=torch.uint8, device=x.device)
    xs = torch.empty(T, H // 128, dtype=torch.float32, device=x.device)
    lib.moe_quantize_e5m6(x.contiguous(), xq, xs, scale_mode, stream)
    return xq, xs


def dequantize_e5m6(xq: torch.Tensor, xs: torch.Tensor, stream=None) -> torch.Tensor:
    """float32 [T, H] values of E5M6 codes and their scales (moe_dequantize_e5m6)."""
    T, H = xq.shape[0], xq.shape[1] // 3 * 2
    out = torch.empty(T, H, dtype=torch.float32, device=xq.device)
    lib.moe_dequantize_e5m6(xq.contiguous(), xs.contiguous(), out, stream)
    return out


def backward(inputs: dict, topk_ids: torch.Tensor, topk_weights: torch.Tensor, dy: torch.Tensor,
             workspace: Workspace = None, stream=None, want_dbias: bool = True, out: dict = None) -> dict:
    """Gradients of a BF16 layer (moe_backward) for the routing a forward
    call returned, from row-major weights (inputs as generated, not packed).
    Returns dict(dx, dw_gate_up, dw_down, dw_router, dbias), fp32 (`out`, a
    previous result, is reused)."""
    if inputs.get("weights_packed"):
        raise ValueError("backward() reads the row-major weights: pass the inputs before pack_weights()")
    x = inputs["x"]
    T, H = x.shape
    k = topk_ids.shape[1]
    desc = desc_from_inputs(inputs, k, layout="row_major")
    E, I = desc.E, desc.I
    dev = x.device
    f32 = dict(dtype=torch.float32, device=dev)
    if out is None:
        out = dict(dx=torch.empty(T, H, **f32), dw_gate_up=torch.empty(E, 2 * I, H, **f32),
                   dw_down=torch.empty(E, H, I, **f32), dw_router=torch.empty(E, H, **f32),
                   dbias=torch.empty(E, **f32) if want_dbias else None)
    ws = (workspace or Workspace(dev)).get(lib.moe_backward_workspace_size(desc))
    lib.moe_backward(desc, x, inputs["router_w"], inputs["w_gate_up"].contiguous(), inputs["w_down"].contiguous(),
                     topk_ids.contiguous(), topk_weights.contiguous(), dy.contiguous(), out["dx"], out["dw_gate_up"],
                     out["dw_down"], out["dw_router"], out["dbias"], ws, stream)
    return out


def trace_phases(out: dict) -> dict:
    """Phase timing of a finished forward(..., trace=True) call in the
    persistent kernel, from the per-workgroup stamps (100 MHz clock):
    microseconds from the first workgroup's entry to each phase boundary
    (first / median / last workgroup), and the items per workgroup."""
    import numpy as np
    desc, ws = out["desc"], out["workspace"]
    reg = lib.moe_get_workspace_regions(desc)
    n = lib.MOE_TRACE_GROUPS * lib.MOE_TRACE_FIELDS
    raw = ws[reg["trace"]: reg["trace"] + n * 8].view(torch.int64).cpu().numpy().reshape(lib.MOE_TRACE_GROUPS, -1)
    used = raw[:, 0] > 0
    t = raw[used, :6].astype(np.float64)
    t0 = t[:, 0].min()
    us = (t - t0) / 100.0
    names = ["entry", "routing_end", "gateup_start", "gateup_end", "down_end", "exit"]
    res = {nm: {"first": round(float(us[:, i].min()), 1), "median": round(float(np.median(us[:, i])), 1),
                "last": round(float(us[:, i].max()), 1)} for i, nm in enumerate(names)}
    res["gateup_items_per_wg"] = [int(raw[used, 6].min()), int(raw[used, 6].max())]
    res["down_items_per_wg"] = [int(raw[used, 7].min()), int(raw[used, 7].max())]
    res["workgroups"] = int(used.sum())
    return res


def route(inputs: dict, top_k: int, E: int, I: int = 128, workspace: Workspace = None, stream=None) -> dict:
    x = inputs["x"]
    T, H = x.shape
    act = "bf16" if x.dtype == torch.bfloat16 else "fp8"
    desc = lib.make_desc(T, H, E, I, top_k, act, "bf16" if act == "bf16" else "fp8")
    dev = x.device
    out = dict(logits=torch.empty(T, E, dtype=torch.float32, device=dev),
               topk_ids=torch.empty(T, top_k, dtype=torch.int32, device=dev),
               topk_weights=torch.empty(T, top_k, dtype=torch.float32, device=dev))
    ws = (workspace or Workspace(dev)).get(lib.moe_route_workspace_size(desc))
    lib.moe_route(desc, x, inputs.get("x_scales"), inputs["router_w"], inputs.get("router_bias"),
                  out["logits"], out["topk_ids"], out["topk_weights"], ws, stream)
    return out


def permute(topk_ids: torch.Tensor, E: int, H: int = 128, I: int = 128, workspace: Workspace = None,
            stream=None) -> dict:
    T, k = topk_ids.shape
    desc = lib.make_desc(T, H, E, I, k, "fp8", "fp8")
    dev = topk_ids.device
    out = dict(expert_offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
               perm=torch.empty(T * k, dtype=torch.int32, device=dev),
               row_of=torch.empty(T * k, dtype=torch.int32, device=dev))
    ws = (workspace or Workspace(dev)).get(lib.moe_permute_workspace_size(desc))
    lib.moe_permute(desc, topk_ids.to(torch.int32).contiguous(), out["expert_offsets"], out["perm"],
                    out["row_of"], ws, stream)
    return out
