"""E5M6 quantisation and dequantisation (moe_quantize_e5m6 /
moe_dequantize_e5m6, reading R15) against the oracle, bit for bit: random
activations of mixed magnitudes (with zero blocks and subnormal codes), a
sweep of the device's E5M6 encoder over every rounding midpoint and its
fp32 neighbours, and the decoder over all 4096 codes."""

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
    xq, xs = L.quantize_e5m6(x.cuda(), mode)
    torch.cuda.synchronize()
    xv = x.float().double().numpy()
    codes, s = O.quantise_tokens_e5m6(xv, mode == "pow2")
    gs = xs.cpu().numpy().astype(np.float64)
    assert np.array_equal(gs, s), f"scales differ at {np.argwhere(gs != s)[:5].tolist()}"
    got = F.e5m6_unpack(xq.cpu().numpy())
    bad = np.argwhere(got != codes)
    assert bad.size == 0, (f"{bad.shape[0]} codes differ, e.g. x={xv[tuple(bad[0])]!r} "
                           f"device {got[tuple(bad[0])]:#05x} oracle {codes[tuple(bad[0])]:#05x}")
    assert np.array_equal(xq.cpu().numpy(), F.e5m6_pack(codes))
    return xq, xs, codes, s


@pytest.mark.parametrize("mode", ["f32", "pow2"])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_quantize_e5m6_bit_exact(L, mode, dtype):
    g = torch.Generator().manual_seed(41)
    T, H = 203, 1536                                  # ragged T, 12 blocks per token
    mag = torch.tensor([1e-6, 1e-2, 1.0, 7.0, 300.0, 5e4], dtype=torch.float32)
    x = torch.randn(T, H, generator=g) * mag[torch.randint(0, 6, (T, H // 128), generator=g)].repeat_interleave(128, 1)
    x[5, 128:256] = 0.0                               # zero block
    x[7, :128] = -0.0
    x[9, :128] = torch.logspace(-12, 4, 128)          # subnormal codes below max * 2^-30
    x = x.to(dtype)
    xq, xs, codes, s = _check(L, x, mode)
    # dequantisation of the device's own codes
    out = L.dequantize_e5m6(xq, xs)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().astype(np.float64), O.dequantise_e5m6(codes, s))


def test_e5m6_encoder_sweep(L):
    """fp32 inputs with a 65024 in every block, so the scale is exactly 1 and
    the device encodes x itself: every midpoint between adjacent E5M6 values
    (both signs), one fp32 ulp either side of it, the values themselves and
    the subnormal range; plus blocks whose maximum is above 65024 (the
    saturating clamp on x * (1/s) near the top)."""
    pos = F.E5M6_TABLE[: 0x7C0]                        # 0 .. 65024
    mids = (pos[1:] + pos[:-1]) / 2
    m32 = mids.astype(np.float32)
    assert np.array_equal(m32.astype(np.float64), mids)   # midpoints are fp32 numbers
    vals = np.concatenate([pos, mids, np.nextafter(m32, np.float32(0)), np.nextafter(m32, np.float32(1e9)),
                           np.float32(2.0 ** -24) * np.arange(1, 60, dtype=np.float32)]).astype(np.float32)
    vals = np.concatenate([vals, -vals])
    per = 127
    nblk = (vals.size + per - 1) // per
    x = np.zeros((nblk, 128), dtype=np.float32)
    flat = np.zeros(nblk * per, dtype=np.float32)
    flat[: vals.size] = vals
    x[:, 0] = 65024.0
    x[:, 1:] = flat.reshape(nblk, per)
    sat = np.zeros((4, 128), dtype=np.float32)
    sat[0, :4] = [np.nextafter(np.float32(65024), np.float32(1e9)), 65024.0, 65300.0, -65000.0]
    sat[1, :3] = [65536.0, -65400.0, 300.0]
    sat[2, :3] = [1e30, -3e29, 7.0]
    sat[3, :2] = [np.float32(2.0 ** -100), np.float32(-2.0 ** -101)]
    x = np.concatenate([x, sat])
    if x.shape[0] % 2:                                 # two blocks per token row
        pad = np.zeros((1, 128), dtype=np.float32)
        pad[0, 0] = 65024.0
        x = np.concatenate([x, pad])
    x = x.reshape(-1, 256)
    for mode in ("f32", "pow2"):
        _check(L, torch.from_numpy(x), mode)


def test_e5m6_decoder_all_codes(L):
    codes = np.tile(np.arange(4096, dtype=np.uint16), 2).reshape(2, 4096)
    s = np.array([[1.0] * 16 + [0.5] * 16, [3.7] * 16 + [2.0 ** -20] * 16], dtype=np.float32)
    xq = torch.from_numpy(F.e5m6_pack(codes)).cuda()
    xs = torch.from_numpy(s).cuda()
    out = L.dequantize_e5m6(xq, xs)
    torch.cuda.synchronize()
    ref = O.dequantise_e5m6(codes, s.astype(np.float64))
    got = out.cpu().numpy().astype(np.float64)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok]) and np.array_equal(np.signbit(got[ok]), np.signbit(ref[ok]))
