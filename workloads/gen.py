"""Seeded synthetic inputs for the MoE layer.

The pages benchmark the layer on a DeepSeek-V3-shaped workload (8K tokens,
hidden 7168, top-8, FP8 dispatch, BF16: youleyou, "DeepSeek 模型更新解读 Tile
Kernels 与 DeepEP V2 新特性", section "性能表现") but publish no data; every
tensor here is synthetic and stands in for real activations and trained
weights.

Recipe (per tensor, from a torch generator seeded by (seed, workload, tensor,
expert), so any one expert's weights can be regenerated alone):

* x ~ N(0, 1) [T, H].  BF16 workloads round it to BF16; FP8 workloads quantise
  it per token per 128 channels with an fp32 scale amax / 448.
* router weights Wr ~ N(0, 1/H) [E, H], BF16.
* gate|up weights ~ N(0, 1/H) stored [E, 2I, H]; down weights ~ N(0, 1/I)
  stored [E, H, I] (K-contiguous).  FP8: one fp32 scale amax / 448 per
  128 x 128 block (or, for per-channel workloads, per output row).  FP4: one E8M0 scale 2**(floor(log2 amax) - 2) per 32
  consecutive K, E2M1 values rounded to nearest, two per byte (even K in the
  low nibble).
* Skewed workloads add a popularity bias b_e = ln p_e to the router logits,
  p_e proportional to rank_e**(-s) with rank a seeded permutation of 1..E.

Quantisation here is input preparation, not part of the layer: whatever bytes
it produces are what both the device path and the oracle decode.  FP8 encoding
uses PyTorch's own float8_e4m3fn cast.
"""

import hashlib
from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch


@dataclass(frozen=True)
class LayerConfig:
    name: str
    T: int
    H: int
    E: int
    k: int
    I: int
    act: str            # "bf16" | "fp8"
    weight: str         # "bf16" | "fp8" | "fp4"
    zipf: Optional[float] = None
    note: str = ""
    scales: str = "f32"  # the layer's own FP8 quantisation scales: "f32" or "pow2"
    wscale: str = "block"  # FP8 weight scales: "block" (128 x 128) or "channel" (one per output row)


CONFIGS = {
    "tiny_bf16": LayerConfig("tiny_bf16", 64, 256, 8, 2, 128, "bf16", "bf16",
                             note="tiny all-BF16 layer, top-2"),
    "dsv3_fp8": LayerConfig("dsv3_fp8", 8192, 7168, 256, 8, 2048, "fp8", "fp8",
                            note="DeepSeek-V3-shaped layer, FP8 x FP8 (128x128 block scales)"),
    "dsv3_fp8xfp4": LayerConfig("dsv3_fp8xfp4", 8192, 7168, 256, 8, 2048, "fp8", "fp4",
                                note="DeepSeek-V3-shaped layer, FP8 x FP4 (E8M0 per 32)"),
    "decode_fp8_zipf": LayerConfig("decode_fp8_zipf", 256, 7168, 256, 8, 2048, "fp8", "fp8",
                                   zipf=1.1, note="decode-shaped, Zipf(1.1) expert popularity"),
    "dsv3_bf16": LayerConfig("dsv3_bf16", 8192, 7168, 256, 8, 2048, "bf16", "bf16",
                             note="DeepSeek-V3-shaped layer in BF16 (the backward pass's workload)"),
    "mega_e1024_fp4_zipf": LayerConfig("mega_e1024_fp4_zipf", 16384, 7168, 1024, 16, 1024, "fp8",
                                       "fp4", zipf=1.0,
                                       note="1024 experts, top-16, FP8 x FP4, Zipf(1.0)"),
}


def spec_of(cfg: LayerConfig):
    """The oracle's Spec for a config (a plain tuple of shapes and dtypes)."""
    from oracle.moe_oracle import Spec  # imported lazily: tests only
    # BF16 activations with FP8 / FP4 weights: the layer quantises its input
    act = "bf16_fp8" if cfg.act == "bf16" and cfg.weight != "bf16" else cfg.act
    return Spec(cfg.T, cfg.H, cfg.E, cfg.k, cfg.I, act, cfg.weight, cfg.scales, cfg.wscale)


_TENSOR_IDS = {"x": 1, "router_w": 2, "w_gate_up": 3, "w_down": 4, "zipf_rank": 5,
               "exact_x": 6, "exact_wr": 7, "exact_bias": 8}


def _seed(seed: int, cfg_name: str, tensor: str, expert: int = -1) -> int:
    h = hashlib.sha256(f"{seed}|{cfg_name}|{_TENSOR_IDS[tensor]}|{expert}".encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _randn(shape, std, device, seed):
    return torch.randn(shape, generator=_gen(device, seed), device=device,
                       dtype=torch.float32) * std


# ---------------------------------------------------------- input encoders
def _fp8_bytes(v: torch.Tensor) -> torch.Tensor:
    v = v.clamp(-448.0, 448.0)
    return v.to(torch.float8_e4m3fn).view(torch.uint8)


def quantise_rows_fp8(x: torch.Tensor):
    """[T, H] fp32 -> (uint8 [T, H], fp32 scales [T, H/128])."""
    T, H = x.shape
    b = x.reshape(T, H // 128, 128)
    amax = b.abs().amax(dim=2)
    s = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    q = _fp8_bytes(b / s[:, :, None])
    return q.reshape(T, H), s.contiguous()


def quantise_blocks_fp8(w: torch.Tensor):
    """[N, K] fp32 -> (uint8 [N, K], fp32 scales [N/128, K/128])."""
    N, K = w.shape
    b = w.reshape(N // 128, 128, K // 128, 128)
    amax = b.abs().amax(dim=(1, 3))
    s = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    q = _fp8_bytes(b / s[:, None, :, None])
    return q.reshape(N, K), s.contiguous()


def quantise_channels_fp8(w: torch.Tensor):
    """[N, K] fp32 -> (uint8 [N, K], fp32 scales [N]): one scale amax / 448
    per output row."""
    amax = w.abs().amax(dim=1)
    s = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    return _fp8_bytes(w / s[:, None]), s.contiguous()


_E2M1_MAGS = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def quantise_fp4(w: torch.Tensor):
    """[N, K] fp32 -> (uint8 [N, K/2] packed E2M1, uint8 [N, K/32] E8M0)."""
    N, K = w.shape
    b = w.reshape(N, K // 32, 32)
    amax = b.abs().amax(dim=2)
    _, ex = torch.frexp(amax)                   # amax = m * 2**ex, 0.5 <= m < 1
    e = torch.where(amax > 0, ex - 1 - 2, torch.full_like(ex, -127))
    e = e.clamp(-127, 127)
    scale = torch.ldexp(torch.ones_like(amax), e)
    v = (b / scale[:, :, None]).clamp(-6.0, 6.0)
    mags = torch.tensor(_E2M1_MAGS, device=w.device)
    mids = (mags[1:] + mags[:-1]) / 2
    code = torch.bucketize(v.abs(), mids)       # nearest magnitude
    code = code | ((v < 0).to(code.dtype) << 3)
    code = code.reshape(N, K).to(torch.uint8)
    packed = code[:, 0::2] | (code[:, 1::2] << 4)
    return packed.contiguous(), (e + 127).to(torch.uint8).contiguous()


def _quantise_weight(w: torch.Tensor, kind: str, wscale: str = "block"):
    if kind == "bf16":
        return w.to(torch.bfloat16), None
    if kind == "fp8":
        return quantise_channels_fp8(w) if wscale == "channel" else quantise_blocks_fp8(w)
    if kind == "fp4":
        return quantise_fp4(w)
    raise ValueError(kind)


def zipf_bias(E: int, s: float, seed: int, name: str) -> torch.Tensor:
    """b_e = ln p_e with p_e proportional to rank_e**-s over a seeded
    permutation of ranks 1..E (fp32, on the CPU)."""
    rank = torch.randperm(E, generator=_gen("cpu", _seed(seed, name, "zipf_rank"))) + 1
    p = rank.to(torch.float64) ** (-s)
    p = p / p.sum()
    return torch.log(p).to(torch.float32)


def make_inputs(cfg: LayerConfig, seed: int = 0, device="cpu") -> dict:
    """All layer inputs for `cfg` as torch tensors on `device`.

    Keys: x, x_scales, router_w, router_bias, w_gate_up, w_gate_up_scales,
    w_down, w_down_scales (scales / bias are None where the format has none).
    BF16 tensors have dtype bfloat16, FP8 / FP4 / E8M0 tensors uint8."""
    T, H, E, I = cfg.T, cfg.H, cfg.E, cfg.I
    name = cfg.name
    x = _randn((T, H), 1.0, device, _seed(seed, name, "x"))
    if cfg.act == "bf16":
        xq, sx = x.to(torch.bfloat16), None
    else:
        xq, sx = quantise_rows_fp8(x)
    del x
    wr = _randn((E, H), H ** -0.5, device, _seed(seed, name, "router_w")).to(torch.bfloat16)
    bias = None
    if cfg.zipf is not None:
        bias = zipf_bias(E, cfg.zipf, seed, name).to(device)

    gu_q, gu_s, d_q, d_s = [], [], [], []
    for e in range(E):
        wgu = _randn((2 * I, H), H ** -0.5, device, _seed(seed, name, "w_gate_up", e))
        q, s = _quantise_weight(wgu, cfg.weight, cfg.wscale)
        gu_q.append(q)
        gu_s.append(s)
        del wgu
        wd = _randn((H, I), I ** -0.5, device, _seed(seed, name, "w_down", e))
        q, s = _quantise_weight(wd, cfg.weight, cfg.wscale)
        d_q.append(q)
        d_s.append(s)
        del wd
    out = dict(x=xq.contiguous(), x_scales=sx, router_w=wr.contiguous(), router_bias=bias,
               w_gate_up=torch.stack(gu_q), w_down=torch.stack(d_q),
               w_gate_up_scales=None if gu_s[0] is None else torch.stack(gu_s),
               w_down_scales=None if d_s[0] is None else torch.stack(d_s))
    return out


def make_exact_router_inputs(T: int, H: int, E: int, seed: int = 0, dup_pairs=(),
                             with_bias: bool = False, device="cpu") -> dict:
    """Router inputs on which fp32 accumulation in any order is exact.

    x holds FP8 codes of multiples of 0.5 in [-4, 4] with all scales 1;
    Wr = n * 2**-6 with |n| <= 64 (BF16-exact); the optional bias lies on the
    same grid.  Every product is a multiple of 2**-7 of magnitude <= 4, so
    partial sums stay below 2**24 units of 2**-7 for H <= 16384.
    dup_pairs: (a, b) pairs of experts whose router rows are made identical,
    which forces exact ties."""
    assert H <= 16384
    gx = _gen("cpu", _seed(seed, "exact", "exact_x"))
    xv = torch.randint(-8, 9, (T, H), generator=gx).to(torch.float32) * 0.5
    xq = _fp8_bytes(xv)
    sx = torch.ones(T, H // 128, dtype=torch.float32)
    gw = _gen("cpu", _seed(seed, "exact", "exact_wr"))
    wr = torch.randint(-64, 65, (E, H), generator=gw).to(torch.float32) * 2.0 ** -6
    for a, b in dup_pairs:
        wr[b] = wr[a]
    bias = None
    if with_bias:
        gb = _gen("cpu", _seed(seed, "exact", "exact_bias"))
        bias = torch.randint(-64, 65, (E,), generator=gb).to(torch.float32) * 2.0 ** -6
        for a, b in dup_pairs:
            bias[b] = bias[a]
    out = dict(x=xq, x_scales=sx, router_w=wr.to(torch.bfloat16), router_bias=bias)
    return {k: (None if v is None else v.to(device)) for k, v in out.items()}


def make_exact_layer_inputs(cfg: LayerConfig, seed: int = 0, device="cpu") -> dict:
    """Layer inputs on which the gate|up GEMM is exact in fp32 whatever the
    order and grouping of its additions: every product lies on a common grid
    and the sums stay below 2**24 grid units, with power-of-two scales.

    x: FP8 codes of multiples of 0.5 in [-4, 4], scales drawn from
    {1/4, 1/2, 1} (BF16 layers: the same values in BF16).  Router: as
    make_exact_router_inputs.  Weights: FP8 codes of n * 2**-6 (|n| <= 15)
    with block (or per-channel) scales from {1/8 .. 1}; FP4 random E2M1 codes with E8M0 scales
    2**-6 .. 2**-3; BF16 n * 2**-6.  For H <= 2048 every product is a
    multiple of 2**-12 (FP4: 2**-10) of magnitude below 4, so partial sums stay
    below 2**23 grid units.  The down GEMM is not exact (its intermediate
    scales are amax / 448)."""
    T, H, E, I = cfg.T, cfg.H, cfg.E, cfg.I
    assert H <= 2048
    r = make_exact_router_inputs(T, H, E, seed=seed)
    gx = _gen("cpu", _seed(seed, cfg.name, "exact_x"))
    if cfg.act == "bf16":
        xv = torch.randint(-8, 9, (T, H), generator=gx).to(torch.float32) * 0.5
        x, sx = xv.to(torch.bfloat16), None
    else:
        x = r["x"]
        sx = 2.0 ** (-torch.randint(0, 3, (T, H // 128), generator=gx).to(torch.float32))

    def weights(N, K, tensor, e):
        g = _gen("cpu", _seed(seed, cfg.name, tensor, e))
        if cfg.weight == "fp4":
            codes = torch.randint(0, 16, (N, K), generator=g, dtype=torch.int32).to(torch.uint8)
            packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).contiguous()
            sc = (121 + torch.randint(0, 4, (N, K // 32), generator=g, dtype=torch.int32)).to(torch.uint8)
            return packed, sc
        v = torch.randint(-15, 16, (N, K), generator=g).to(torch.float32) * 2.0 ** -6
        if cfg.weight == "bf16":
            return v.to(torch.bfloat16), None
        shape = (N,) if cfg.wscale == "channel" else (N // 128, K // 128)
        sc = 2.0 ** (-torch.randint(0, 4, shape, generator=g).to(torch.float32))
        return _fp8_bytes(v), sc.contiguous()

    gu, gus, d, ds = [], [], [], []
    for e in range(E):
        q, s = weights(2 * I, H, "w_gate_up", e)
        gu.append(q)
        gus.append(s)
        q, s = weights(H, I, "w_down", e)
        d.append(q)
        ds.append(s)
    out = dict(x=x.contiguous(), x_scales=sx, router_w=r["router_w"], router_bias=None,
               w_gate_up=torch.stack(gu), w_down=torch.stack(d),
               w_gate_up_scales=None if gus[0] is None else torch.stack(gus),
               w_down_scales=None if ds[0] is None else torch.stack(ds))
    return {k: (None if v is None else v.to(device)) for k, v in out.items()}


# ------------------------------------------------------- host-side views
def _np(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


class _PerExpert:
    """Indexable view that copies one expert's slice to host on demand."""

    def __init__(self, t: torch.Tensor):
        self.t = t

    def __getitem__(self, e):
        return _np(self.t[e])

    def __len__(self):
        return self.t.shape[0]


def oracle_view(inputs: dict, lazy_weights: bool = False) -> dict:
    """Numpy view of `inputs` in the form the oracle takes (BF16 as uint16
    bit patterns).  With lazy_weights the expert tensors stay where they are
    and each expert is copied to host only when indexed."""
    out = {}
    for k, v in inputs.items():
        if v is None:
            out[k] = None
        elif lazy_weights and k.startswith("w_"):
            out[k] = _PerExpert(v)
        else:
            out[k] = _np(v)
    return out
