"""Pins for the oracle's number formats: exhaustive tables from the format definitions and
cross-checks against independent library casts (torch, NumPy)."""

import json
import os

import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle.quantize import pack_codes, unpack_codes

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def test_e4m3_anchor_values():
    g = _gold("fp_formats.json")
    for code, val in g["e4m3_anchors"]:
        got = F.e4m3_decode(np.array([code]))[0]
        assert got == val and np.signbit(got) == np.signbit(val), (code, got, val)


def test_e4m3_decode_matches_bitfield_definition_all_codes():
    # independent restatement: sign * 2^(e-7) * (1 + m/8), subnormal 2^-6 * m/8, NaN at S.1111.111
    for c in range(256):
        s, e, m = c >> 7, (c >> 3) & 15, c & 7
        if e == 15 and m == 7:
            assert np.isnan(F.e4m3_decode(np.array([c]))[0])
            continue
        v = (m / 8) * 2.0 ** -6 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
        v = -v if s else v
        assert F.e4m3_decode(np.array([c]))[0] == v


def test_e4m3_encode_roundtrip_all_codes():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F])
    vals = F.e4m3_decode(codes).astype(np.float32)
    assert np.array_equal(F.e4m3_encode(vals), codes.astype(np.uint8))


def test_e4m3_encode_matches_torch_cast():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32) * np.float32(30),
        rng.uniform(-464, 464, 100000).astype(np.float32),
        (rng.standard_normal(50000) * 1e-3).astype(np.float32),
    ])
    # every tie point between consecutive finite codes
    pos = np.sort(F.e4m3_decode(np.arange(0, 127)))
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    x = np.concatenate([x, mids, -mids]).astype(np.float32)
    x = x[np.abs(x) <= 464]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = F.e4m3_encode(x)
    assert np.array_equal(got, ref)


def test_e4m3_saturates_and_error_bounds():
    assert F.e4m3_encode(np.array([1e6, -500.0, 464.0, 449.0], dtype=np.float32)).tolist() == [
        0x7E, 0xFE, 0x7E, 0x7E]
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(100000) * 50).astype(np.float32)
    x = x[np.abs(x) < 448]
    back = F.e4m3_decode(F.e4m3_encode(x))
    err = np.abs(back - x)
    normal = np.abs(x) >= 2.0 ** -6
    assert np.all(err[normal] <= np.abs(x[normal]) * 2.0 ** -4)
    assert np.all(err[~normal] <= 2.0 ** -10)


def test_e2m1_table_and_ties():
    g = _gold("fp_formats.json")
    table = F.e2m1_decode(np.arange(16))
    for c, v in enumerate(g["e2m1_table"]):
        assert table[c] == v and np.signbit(table[c]) == np.signbit(v)
    # independent restatement of E2M1: bias 1, subnormal when e == 0
    for c in range(16):
        s, e, m = c >> 3, (c >> 1) & 3, c & 1
        v = 0.5 * m if e == 0 else 2.0 ** (e - 1) * (1 + m / 2)
        assert table[c] == (-v if s else v)
    for y, code in g["e2m1_ties"]:
        assert F.e2m1_encode(np.array([y], dtype=np.float32))[0] == code, y


def test_e2m1_encode_is_nearest():
    rng = np.random.default_rng(2)
    y = rng.uniform(-8, 8, 100000).astype(np.float32)
    c = F.e2m1_encode(y)
    v = F.e2m1_decode(c)
    mags = F.E2M1_VALUES
    best = np.min(np.abs(np.abs(y)[:, None].astype(np.float64) - mags[None, :]), axis=1)
    assert np.allclose(np.abs(np.abs(y) - np.abs(v)), best)
    assert np.all(np.signbit(v) == np.signbit(y))


def test_fp16_round_matches_torch():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(100000) * 1e3, rng.standard_normal(100000) * 1e-5,
                        rng.standard_normal(1000) * 1e5]).astype(np.float32)
    x = x[np.abs(x) < 65504]
    ref = torch.from_numpy(x).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(F.fp16_bits(x), ref)


def test_bf16_decode_matches_torch():
    bits = np.arange(0, 65536, 7, dtype=np.uint32).astype(np.uint16)
    t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = F.bf16_to_f64(bits)
    finite = np.isfinite(t)
    assert np.array_equal(got[finite], t[finite])


def test_packing_known_vectors_and_roundtrip():
    g = _gold("packing.json")
    for case in g["cases"]:
        codes = np.array([case["codes"]], dtype=np.uint8)
        got = pack_codes(codes, case["bits"])[0].tolist()
        assert got == case["bytes"], case
        back = unpack_codes(np.array([case["bytes"]], dtype=np.uint8), case["bits"], codes.shape[1])
        assert back[0].tolist() == case["codes"], case
    rng = np.random.default_rng(4)
    for bits in (2, 4, 8):
        c = rng.integers(0, 1 << bits, size=(7, 128)).astype(np.uint8)
        assert np.array_equal(unpack_codes(pack_codes(c, bits), bits, 128), c)
