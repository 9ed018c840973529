"""Pins for the oracle's number formats (bf16 widening, OCP e4m3fn codec).

The e4m3fn format is fixed by its definition (sign, 4-bit exponent with bias
7, 3-bit mantissa, no infinities, S.1111.111 = NaN, max 448); torch's
float8_e4m3fn dtype is an independent library implementation of it.
"""
import numpy as np
import pytest
import torch

from oracle import decode_bf16, decode_e4m3, encode_e4m3
from oracle.layer import act_quant_e4m3


def test_bf16_widening_matches_library():
    bits = np.arange(0, 65536, 7, dtype=np.uint16)
    ref = torch.from_numpy(bits.astype(np.int32).astype(np.int16)).view(torch.bfloat16).double().numpy()
    got = decode_bf16(bits)
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()


def test_bf16_known_values():
    assert decode_bf16(np.array([0x3F80], np.uint16))[0] == 1.0
    assert decode_bf16(np.array([0xC000], np.uint16))[0] == -2.0
    assert decode_bf16(np.array([0x3F81], np.uint16))[0] == 1.0 + 2.0 ** -7


def test_e4m3_table_matches_library_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    got = decode_e4m3(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(got[fin], ref[fin])
    # signed zero of 0x80
    assert np.signbit(got[0x80])


def test_e4m3_known_values():
    d = decode_e4m3(np.array([0x7E, 0x01, 0x07, 0x08, 0x38, 0xB8, 0x7F, 0xFF], np.uint8))
    assert d[0] == 448.0
    assert d[1] == 2.0 ** -9            # smallest subnormal
    assert d[2] == 7 * 2.0 ** -9        # largest subnormal
    assert d[3] == 2.0 ** -6            # smallest normal
    assert d[4] == 1.0 and d[5] == -1.0
    assert np.isnan(d[6]) and np.isnan(d[7])
    assert np.isfinite(decode_e4m3(np.arange(256, dtype=np.uint8))).sum() == 254


def test_e4m3_encode_roundtrip_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    assert np.array_equal(encode_e4m3(decode_e4m3(codes)), codes)


def test_e4m3_encode_midpoints_go_to_even_code():
    vals = decode_e4m3(np.arange(0x7F, dtype=np.uint8))   # 0 .. 448 increasing
    assert np.all(np.diff(vals) > 0)
    mids = (vals[:-1] + vals[1:]) / 2
    got = encode_e4m3(mids).astype(int)
    lo = np.arange(0x7E)
    want = np.where(lo % 2 == 0, lo, lo + 1)
    assert np.array_equal(got, want)
    # and just off the midpoint it goes to the nearer one
    assert np.array_equal(encode_e4m3(np.nextafter(mids, -np.inf)).astype(int), lo)
    assert np.array_equal(encode_e4m3(np.nextafter(mids, np.inf)).astype(int), lo + 1)


def test_e4m3_saturates():
    got = encode_e4m3(np.array([448.0, 449.0, 464.0, 1e9, -500.0, -1e30]))
    assert list(got) == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE]


def test_e4m3_encode_matches_library_on_random_values():
    g = np.random.default_rng(7)
    v = np.concatenate([g.standard_normal(20000) * 50, g.standard_normal(20000) * 1e-2,
                        g.uniform(-448, 448, 20000)]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = encode_e4m3(v)
    assert np.array_equal(got, ref)


def test_act_quant_properties():
    g = np.random.default_rng(3)
    x = g.standard_normal((9, 300)).astype(np.float32)
    x[4] = 0.0
    codes, s = act_quant_e4m3(x)
    # the amax element of every non-zero row maps to +-448
    for i in range(9):
        if i == 4:
            assert s[i] == 1.0 and np.all(decode_e4m3(codes[i]) == 0)
            continue
        j = int(np.argmax(np.abs(x[i])))
        assert abs(decode_e4m3(codes[i, j:j + 1])[0]) == 448.0
        assert s[i] == np.float32(np.abs(x[i]).max() / np.float32(448.0))
    # relative reconstruction error within half an e4m3 ulp (2^-4) for normals
    rec = decode_e4m3(codes) * s[:, None].astype(np.float64)
    big = np.abs(x) > 2.0 ** -6 * s[:, None]
    assert np.all(np.abs(rec[big] - x[big]) <= 2.0 ** -4 * np.abs(x[big]) + 1e-30)
