"""The per-token FP8 input quantisation kernel (moe_quantize_input) against
the oracle, bit for bit, and a sweep of the device's E4M3 encoder (the one the
GEMM epilogue's re-quantisation also uses) over every rounding midpoint and
its fp32 neighbours, saturation and the subnormal range."""

import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle import moe_oracle as O

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L(gpu_lib):
    from moe_layer_router_amd import layer
    return layer


def _check(L, x: torch.Tensor, mode: str):
    xq, xs = L.quantize_input(x.cuda(), mode)
    torch.cuda.synchronize()
    xv = x.float().double().numpy()
    codes, s = O.quantise_tokens_fp8(xv, mode == "pow2")
    got = xq.cpu().numpy()
    gs = xs.cpu().numpy().astype(np.float64)
    assert np.array_equal(gs, s), f"scales differ at {np.argwhere(gs != s)[:5].tolist()}"
    bad = np.argwhere(got != codes)
    assert bad.size == 0, (f"{bad.shape[0]} codes differ, e.g. x={xv[tuple(bad[0])]!r} "
                           f"device {got[tuple(bad[0])]:#04x} oracle {codes[tuple(bad[0])]:#04x}")


@pytest.mark.parametrize("mode", ["f32", "pow2"])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_quantize_input_bit_exact(L, mode, dtype):
    g = torch.Generator().manual_seed(31)
    T, H = 203, 1536                                  # ragged T, 12 blocks per token
    mag = torch.tensor([1e-6, 1e-2, 1.0, 7.0, 300.0, 5e4], dtype=torch.float32)
    x = torch.randn(T, H, generator=g) * mag[torch.randint(0, 6, (T, H // 128), generator=g)].repeat_interleave(128, 1)
    x[5, 128:256] = 0.0                               # zero block
    x[7, :128] = -0.0
    x = x.to(dtype)
    _check(L, x, mode)


def test_e4m3_encoder_sweep(L):
    """fp32 inputs with a 448 in every block, so the scale is exactly 1 and
    the device encodes x itself: every midpoint between adjacent E4M3 values
    (both signs), one fp32 ulp either side of it, the values themselves,
    the subnormal range and zero; plus blocks whose maximum is just above 448
    (the saturating clamp) and far above it."""
    pos = F.E4M3_TABLE[: 0x7F]                         # 0 .. 448
    mids = (pos[1:] + pos[:-1]) / 2
    m32 = mids.astype(np.float32)
    vals = np.concatenate([pos, mids, np.nextafter(m32, np.float32(0)), np.nextafter(m32, np.float32(1e9)),
                           np.float32(2.0 ** -10) * np.arange(1, 40, dtype=np.float32)]).astype(np.float32)
    vals = np.concatenate([vals, -vals])
    per = 127
    nblk = (vals.size + per - 1) // per
    x = np.zeros((nblk, 128), dtype=np.float32)
    flat = np.zeros(nblk * per, dtype=np.float32)
    flat[: vals.size] = vals
    x[:, 0] = 448.0
    x[:, 1:] = flat.reshape(nblk, per)
    sat = np.zeros((4, 128), dtype=np.float32)
    sat[0, :4] = [np.nextafter(np.float32(448), np.float32(1e9)), 448.0, 464.0, -447.9]
    sat[1, :3] = [449.0, -448.5, 300.0]
    sat[2, :3] = [1e30, -3e29, 7.0]
    sat[3, :2] = [np.float32(2.0 ** -100), np.float32(-2.0 ** -101)]
    x = np.concatenate([x, sat])
    if x.shape[0] % 2:                                 # two blocks per token row
        pad = np.zeros((1, 128), dtype=np.float32)
        pad[0, 0] = 448.0
        x = np.concatenate([x, pad])
    x = x.reshape(-1, 256)
    for mode in ("f32", "pow2"):
        _check(L, torch.from_numpy(x), mode)
