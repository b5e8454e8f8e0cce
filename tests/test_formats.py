"""Pins for the oracle's number-format tables and encoders (CPU only).

The tables are built from the OCP FP8 / MX bit-field definitions; here they
are checked exhaustively against PyTorch's independent float8 casts and
against closed-form values of the formats."""

import numpy as np
import pytest
import torch

from oracle import formats as F


def test_e4m3_table_matches_torch_cast_exhaustively():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = F.E4M3_TABLE
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(ours))
    assert np.array_equal(ref[~nan], ours[~nan])
    assert sorted(np.flatnonzero(nan).tolist()) == [0x7F, 0xFF]


def test_e4m3_closed_form_landmarks():
    assert F.E4M3_TABLE[0x7E] == 448.0            # largest finite
    assert F.E4M3_TABLE[0x01] == 2.0 ** -9        # smallest subnormal
    assert F.E4M3_TABLE[0x08] == 2.0 ** -6        # smallest normal
    assert F.E4M3_TABLE[0x38] == 1.0
    assert F.E4M3_TABLE[0xB8] == -1.0
    assert F.E4M3_TABLE[0x80] == 0.0 and np.signbit(F.E4M3_TABLE[0x80])
    pos = F.E4M3_TABLE[:0x7F]
    assert np.all(np.diff(pos) > 0)               # strictly increasing in code order


def test_e2m1_table_matches_mx_element_list():
    # OCP MX v1.0 lists the E2M1 magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6.
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert F.E2M1_TABLE[:8].tolist() == mags
    assert F.E2M1_TABLE[8:].tolist() == [-m for m in mags]


def test_e8m0_matches_torch_cast_exhaustively():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    ours = F.e8m0_decode(np.arange(256))
    assert np.isnan(ours[255]) and np.isnan(ref[255])
    assert np.array_equal(ref[:255], ours[:255])
    assert ours[127] == 1.0 and ours[0] == 2.0 ** -127


def test_e2m1_nibble_order():
    # byte 0x21: low nibble 1 (0.5) is element 0, high nibble 2 (1.0) element 1
    out = F.e2m1_unpack(np.array([[0x21, 0xF9]], dtype=np.uint8))
    assert out.tolist() == [[0.5, 1.0, -0.5, -6.0]]


def test_bf16_decode_matches_torch():
    rng = np.random.default_rng(0)
    v = torch.tensor(rng.standard_normal(4096) * 100, dtype=torch.float32).to(torch.bfloat16)
    bits = v.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(F.bf16_decode(bits), v.to(torch.float64).numpy())


def test_e4m3_encode_roundtrips_every_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = F.E4M3_TABLE[codes]
    back = F.e4m3_encode(vals)
    assert np.array_equal(back, codes)


def test_e4m3_encode_midpoints_go_to_even_code():
    pos = F.E4M3_TABLE[:0x7F]
    mids = (pos[1:] + pos[:-1]) / 2          # between code c and c+1
    got = F.e4m3_encode(mids)
    lower = np.arange(0x7E)
    want = np.where(lower % 2 == 0, lower, lower + 1)
    assert np.array_equal(got, want.astype(np.uint8))
    # just off the midpoint goes to the nearer code
    eps = 1e-9
    assert np.array_equal(F.e4m3_encode(mids - eps * pos[1:]), lower.astype(np.uint8))
    assert np.array_equal(F.e4m3_encode(mids + eps * pos[1:]), (lower + 1).astype(np.uint8))


def test_e4m3_encode_saturates():
    got = F.e4m3_encode(np.array([448.0, 463.9, 464.0, 500.0, 1e30, -449.0, -1e9]))
    assert got.tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE]
    with pytest.raises(ValueError):
        F.e4m3_encode(np.array([np.nan]))


def test_e4m3_encode_agrees_with_torch_cast():
    rng = np.random.default_rng(1)
    v = np.concatenate([rng.standard_normal(20000) * 50,
                        rng.standard_normal(20000) * 2.0 ** -7]).astype(np.float32)
    ref = torch.tensor(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = F.e4m3_encode(v.astype(np.float64))
    # torch keeps the sign of values that round to zero as well
    assert np.array_equal(ours, ref)


def test_bf16_round_matches_torch_rne():
    rng = np.random.default_rng(2)
    v = (rng.standard_normal(50000) * 10).astype(np.float32)
    ref = torch.tensor(v).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(F.bf16_round(v.astype(np.float64)), ref)
    # an exact tie between two BF16 values rounds to the even mantissa
    one = 1.0
    ulp = 2.0 ** -7
    assert F.bf16_round(np.array([one + ulp / 2]))[0] == one
    assert F.bf16_round(np.array([one + 1.5 * ulp]))[0] == one + 2 * ulp


def test_f32_round():
    assert F.f32_round(np.array([1.0 + 2.0 ** -30]))[0] == 1.0
    assert F.f32_round(np.array([1.0 + 2.0 ** -23]))[0] == 1.0 + 2.0 ** -23


# ------------------------------------------------------------- E5M6 (R15)
def _fp16_from_e5m6_fields(code: int) -> float:
    # E5M6 has binary16's sign and exponent fields and the top 6 of its 10
    # fraction bits: the same value as the binary16 number with the low four
    # fraction bits zero (numpy's float16 decodes it independently)
    bits = ((code >> 11) & 1) << 15 | ((code >> 6) & 0x1F) << 10 | (code & 0x3F) << 4
    return float(np.array([bits], dtype=np.uint16).view(np.float16)[0])


def test_e5m6_table_matches_binary16_subset_exhaustively():
    ref = np.array([_fp16_from_e5m6_fields(c) for c in range(4096)])
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(F.E5M6_TABLE))
    assert np.array_equal(ref[~nan], F.E5M6_TABLE[~nan])
    assert nan.sum() == 2 * 63                                   # exponent 31, fraction != 0


def test_e5m6_closed_form_landmarks():
    assert F.E5M6_TABLE[0x7BF] == F.E5M6_MAX == (2 - 2.0 ** -6) * 2.0 ** 15
    assert F.E5M6_TABLE[0x001] == 2.0 ** -20                    # smallest subnormal
    assert F.E5M6_TABLE[0x040] == 2.0 ** -14                    # smallest normal
    assert F.E5M6_TABLE[0x3C0] == 1.0 and F.E5M6_TABLE[0xBC0] == -1.0
    assert np.isinf(F.E5M6_TABLE[0x7C0]) and np.signbit(F.E5M6_TABLE[0x800])
    assert np.all(np.diff(F.E5M6_TABLE[:0x7C0]) > 0)


def test_e5m6_encode_ties_even_and_saturates():
    pos = F.E5M6_TABLE[:0x7C0]
    mids = (pos[:-1] + pos[1:]) / 2
    lo = np.arange(0x7BF)
    even = np.where(lo % 2 == 0, lo, lo + 1)
    assert np.array_equal(F.e5m6_encode(mids), even)
    assert np.array_equal(F.e5m6_encode(np.nextafter(mids, 0)), lo)
    assert np.array_equal(F.e5m6_encode(np.nextafter(mids, np.inf)), lo + 1)
    assert np.array_equal(F.e5m6_encode(pos), np.arange(0x7C0))
    assert np.array_equal(F.e5m6_encode(-pos[1:]), np.arange(1, 0x7C0) | 0x800)
    assert F.e5m6_encode([65024.0 + 300, 1e30, -1e30]).tolist() == [0x7BF, 0x7BF, 0xFBF]
    assert F.e5m6_encode([-0.0])[0] == 0x800


def test_e5m6_encode_matches_arithmetic_rounding():
    # the same rounding written as arithmetic: the value's unit in the last
    # of 6 fraction bits (2**-20 below the normal range), np.rint (ties to
    # even) of the quotient, then saturation
    rng = np.random.default_rng(5)
    v = rng.standard_normal(200000) * np.exp2(rng.uniform(-24, 18, 200000))
    a = np.abs(v)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    ulp = np.exp2(np.maximum(e, -14) - 6)
    ref = np.minimum(np.rint(a / ulp) * ulp, F.E5M6_MAX) * np.sign(v)
    got = F.e5m6_decode(F.e5m6_encode(v))
    assert np.array_equal(got, ref)


def test_e5m6_pack_layout_and_round_trip():
    assert F.e5m6_pack([0x123, 0xABC]).tolist() == [0x23, 0xC1, 0xAB]
    rng = np.random.default_rng(6)
    c = rng.integers(0, 4096, size=(3, 256)).astype(np.uint16)
    p = F.e5m6_pack(c)
    assert p.shape == (3, 384)
    assert np.array_equal(F.e5m6_unpack(p), c)
