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
    desc = desc_from_inputs(inputs, top_k)
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


def desc_from_inputs(inputs: dict, top_k: int, mode: str = "mega", flags: int = 0, I=None) -> lib.MoeDesc:
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
    return lib.make_desc(T, H, E, I, top_k, act, weight, mode, flags)


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
            routing=None, want_perm: bool = True, stream=None, out=None) -> dict:
    """Run the layer on inputs whose weights went through pack_weights().
    routing=(topk_ids, topk_weights) feeds given routing
    (MOE_FLAG_ROUTING_GIVEN).  Returns dict(y, topk_ids, topk_weights,
    expert_offsets, perm)."""
    if not inputs.get("weights_packed"):
        raise ValueError("forward() needs MFMA-tiled weights: pass the inputs through pack_weights() first")
    flags = lib.MOE_FLAG_ROUTING_GIVEN if routing is not None else 0
    desc = desc_from_inputs(inputs, top_k, mode, flags)
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
    if desc.act_dtype == lib.MOE_DTYPE_FP8_E4M3:
        codes = ws[reg["inter"]: reg["inter"] + rows * I].view(rows, I)
        sc = ws[reg["inter_scales"]: reg["inter_scales"] + rows * (I // 128) * 4].view(torch.float32)
        return codes, sc.view(I // 128, rows).t()       # stored K block major
    vals = ws[reg["inter"]: reg["inter"] + rows * I * 2].view(torch.bfloat16).view(rows, I)
    return vals, None


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
