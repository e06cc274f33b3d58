"""Pins for the oracle's E4M3 / E8M0 codecs against closed forms, brute force and
torch's CPU float8 cast (a library routine independent of the oracle)."""
import numpy as np
import pytest
import torch

from oracle import (bf16_bits_to_f64, e4m3_decode, e4m3_encode, e4m3_encode_bruteforce,
                    e8m0_decode)


def test_e4m3_closed_forms():
    v = e4m3_decode(np.array([0x38, 0x7E, 0x01, 0x08, 0x07, 0x00, 0x80, 0xB8, 0xFE, 0x40]))
    assert v[0] == 1.0
    assert v[1] == 448.0
    assert v[2] == 2.0 ** -9
    assert v[3] == 2.0 ** -6
    assert v[4] == 7 * 2.0 ** -9
    assert v[5] == 0.0 and not np.signbit(v[5])
    assert v[6] == 0.0 and np.signbit(v[6])
    assert v[7] == -1.0
    assert v[8] == -448.0
    assert v[9] == 2.0
    assert np.isnan(e4m3_decode(np.array([0x7F, 0xFF]))).all()


def test_e8m0_closed_forms():
    v = e8m0_decode(np.array([127, 0, 254, 128, 100, 255]))
    assert v[0] == 1.0 and v[1] == 2.0 ** -127 and v[2] == 2.0 ** 127
    assert v[3] == 2.0 and v[4] == 2.0 ** -27 and np.isnan(v[5])


def test_e4m3_value_table_monotone_and_count():
    vals = e4m3_decode(np.arange(0x7F))
    assert np.all(np.diff(vals) > 0)
    assert len(np.unique(np.abs(e4m3_decode(np.arange(256))[~np.isnan(e4m3_decode(np.arange(256)))]))) == 127


def test_e4m3_roundtrip_all_finite_codes():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F])
    assert np.array_equal(e4m3_encode(e4m3_decode(codes)), codes.astype(np.uint8))


def test_e4m3_ties_and_saturation():
    cases = {
        1.5 * 2.0 ** -9: 0x02,     # tie between 1 and 2 quanta -> even (2)
        0.5 * 2.0 ** -9: 0x00,     # tie between 0 and 1 quantum -> even (0)
        -0.25 * 2.0 ** -9: 0x80,   # rounds to -0
        2.5 * 2.0 ** -9: 0x02,
        3.5 * 2.0 ** -9: 0x04,
        464.0: 0x7E,               # tie between 448 and 480 -> even mantissa (448)
        463.999: 0x7E,
        464.001: 0x7E,             # would round to 480: saturates
        1e30: 0x7E,
        -500.0: 0xFE,
        1.0625: 0x38,              # tie between 1 and 1.125 -> 1
        1.1875: 0x3A,              # tie between 1.125 and 1.25 -> 1.25 (even)
        -0.0: 0x80,
    }
    got = e4m3_encode(np.array(list(cases.keys())))
    assert list(got) == list(cases.values())


def test_e4m3_matches_bruteforce():
    rng = np.random.default_rng(0)
    mags = np.ldexp(rng.random(4000) + 0.5, rng.integers(-14, 11, size=4000))
    mids = (e4m3_decode(np.arange(1, 0x7F)) + e4m3_decode(np.arange(0, 0x7E))) / 2  # every tie
    y = np.concatenate([mags * rng.choice([-1, 1], size=mags.size), mids, -mids, [0.0, 448.0, 470.0, 1e5]])
    assert np.array_equal(e4m3_encode(y), e4m3_encode_bruteforce(y))


def test_e4m3_matches_torch_cast_in_range():
    # every bf16 value with |v| < 464 (torch does not saturate above that)
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = bf16_bits_to_f64(bits)
    ok = np.isfinite(v) & (np.abs(v) < 464)
    t = torch.from_numpy(v[ok].astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(e4m3_encode(v[ok]), t)
    # random float32 values across the whole E4M3 range
    rng = np.random.default_rng(1)
    r = (np.ldexp(rng.random(200000) + 0.5, rng.integers(-16, 9, size=200000)) *
         rng.choice([-1, 1], size=200000)).astype(np.float32)
    r = r[np.abs(r) < 464]
    t = torch.from_numpy(r).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(e4m3_encode(r.astype(np.float64)), t)


def test_e4m3_rejects_non_finite():
    with pytest.raises(ValueError):
        e4m3_encode(np.array([np.inf]))
