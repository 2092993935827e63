"""Pins of the oracle's decoders and encoders against things other than itself:
torch's dtype conversions (library routines), the pages' printed tables and
exact rational brute force."""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import codecs
from tests import exact


def test_e4m3_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = codecs.decode_e4m3(codes)
    lib = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    nan = np.isnan(lib)
    assert np.array_equal(np.isnan(ours), nan)
    assert set(np.flatnonzero(nan)) == {0x7F, 0xFF}
    assert np.array_equal(ours[~nan], lib[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(lib[~nan]))


def test_e4m3_max_and_order(golden):
    ours = codecs.decode_e4m3(np.arange(0x7F, dtype=np.uint8))
    assert ours[-1] == golden["fp8_max"]["value"] == 448.0
    assert np.all(np.diff(ours) > 0)                      # codes 0..0x7E increase with value
    assert ours[1] == 2.0 ** -9 and ours[8] == 2.0 ** -6   # smallest subnormal, smallest normal


def test_e2m1_decode_matches_page_table(golden):
    lut = np.array(golden["e2m1_lut"]["value"])
    ours = codecs.decode_e2m1(np.arange(16, dtype=np.uint8))
    assert np.array_equal(ours, lut)
    assert np.array_equal(np.signbit(ours), np.signbit(lut))


def test_e8m0_decode_matches_torch(golden):
    e = np.arange(256, dtype=np.uint8)
    ours = codecs.decode_e8m0(e)
    lib = torch.from_numpy(e).view(torch.float8_e8m0fnu).double().numpy()
    assert np.isnan(ours[255]) and np.isnan(lib[255])
    assert np.array_equal(ours[:255], lib[:255])
    assert ours[golden["e8m0_bias"]["value"]] == 1.0


def test_bf16_decode_matches_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = codecs.decode_bf16(bits)
    lib = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    nan = np.isnan(lib)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], lib[~nan])


def test_unpack_fp4_nibble_order(golden):
    assert golden["fp4_nibble_order"]["value"] == ["low", "high"]
    packed = np.array([[0x21, 0xF0]], dtype=np.uint8)
    assert codecs.unpack_fp4(packed).tolist() == [[1, 2, 0, 15]]


# ------------------------------------------------------------------ bf16 RNE
def test_bf16_round_matches_torch_on_fp32_values():
    g = np.random.default_rng(1)
    x = np.concatenate([
        g.standard_normal(200000).astype(np.float32),
        (g.standard_normal(20000) * 1e-39).astype(np.float32),      # fp32 subnormal range
        (g.standard_normal(20000) * 3e38).astype(np.float32),       # near overflow
        np.array([0.0, -0.0, 2.0 ** -133, 2.0 ** -134, 3 * 2.0 ** -135], np.float32),
    ])
    with np.errstate(over="ignore", invalid="ignore"):
        ours = codecs.round_to_bf16(x.astype(np.float64))
    lib = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, lib)


def test_bf16_round_is_single_rounding():
    # 1 + 2**-8 + 2**-30: above the bf16 midpoint, but fp32 rounds it onto the midpoint first
    v = 1.0 + 2.0 ** -8 + 2.0 ** -30
    assert codecs.decode_bf16(codecs.round_to_bf16(np.array([v])))[0] == 1.0 + 2.0 ** -7
    assert codecs.decode_bf16(codecs.round_to_bf16(np.array([1.0 + 2.0 ** -8])))[0] == 1.0   # tie -> even


def test_bf16_round_matches_fraction_brute_force():
    g = np.random.default_rng(2)
    x = g.standard_normal(3000) * np.exp2(g.integers(-140, 120, 3000))
    ours = codecs.decode_bf16(codecs.round_to_bf16(x))
    for xi, oi in zip(x, ours):
        assert Fraction(float(oi)) == exact.bf16_round(Fraction(float(xi))), xi


def test_bf16_ulp_matches_lattice():
    bits = np.arange(0x0001, 0x7F7F, 97, dtype=np.uint16)
    vals = codecs.decode_bf16(bits)
    nxt = codecs.decode_bf16(bits + 1)
    # ulp at a lattice point equals the gap to the next point
    assert np.array_equal(codecs.bf16_ulp(vals), nxt - vals)


# ------------------------------------------------------------------ e4m3 RNE
def test_e4m3_encode_roundtrip_every_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = codecs.decode_e4m3(codes)
    assert np.array_equal(codecs.round_to_e4m3(vals), codes)


def test_e4m3_encode_midpoints_go_to_even_code():
    codes = np.arange(0, 0x7E, dtype=np.uint8)
    lo = codecs.decode_e4m3(codes)
    hi = codecs.decode_e4m3(codes + 1)
    mid = (lo + hi) / 2
    got = codecs.round_to_e4m3(mid)
    expect = np.where(codes % 2 == 0, codes, codes + 1)
    assert np.array_equal(got, expect)
    assert np.array_equal(codecs.round_to_e4m3(-mid), expect | 0x80)


def test_e4m3_encode_matches_torch_conversion():
    g = np.random.default_rng(3)
    x = np.concatenate([
        (g.standard_normal(300000) * 60).astype(np.float32),
        (g.standard_normal(100000) * 0.01).astype(np.float32),
        g.uniform(-448, 448, 100000).astype(np.float32),
    ])
    x = np.clip(x, -448, 448)
    ours = codecs.round_to_e4m3(x.astype(np.float64))
    lib = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, lib)


def test_e4m3_encode_fraction_brute_force():
    g = np.random.default_rng(4)
    x = g.uniform(-448, 448, 400) * np.exp2(-g.integers(0, 16, 400))
    got = codecs.decode_e4m3(codecs.round_to_e4m3(x))
    for xi, gi in zip(x, got):
        assert Fraction(float(gi)) == exact.e4m3_round(Fraction(float(xi)))


def test_e4m3_encode_rejects_unclamped():
    with pytest.raises(ValueError):
        codecs.round_to_e4m3(np.array([449.0]))


def test_step_index_identifies_signed_zero():
    idx = codecs.e4m3_step_index(np.array([0x00, 0x80, 0x01, 0x81, 0x7E, 0xFE], np.uint8))
    assert idx.tolist() == [0, 0, 1, -1, 126, -126]
