"""Pins of the oracle's OCP E4M3 encoder/decoder (no GPU).

Pinned against: the OCP OFP8 specification's E4M3 values (fixture
tests/golden/ofp8_e4m3_spec.txt), an exhaustive round trip over every code,
and a brute-force nearest-value search (ties to the even mantissa) built from
the decoded value table, independent of the oracle's frexp/rint encoder.
"""
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "ofp8_e4m3_spec.txt")


def _spec_rows():
    rows = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        code, val = line.split()
        rows.append((int(code, 16), val))
    return rows


@pytest.mark.parametrize("code,val", _spec_rows())
def test_spec_values_decode(code, val):
    got = float(oracle.e4m3_decode(np.array([code], np.uint8))[0])
    if val == "nan":
        assert math.isnan(got)
    elif val == "-0":
        assert got == 0.0 and math.copysign(1.0, got) < 0
    else:
        assert got == float(val)


@pytest.mark.parametrize("code,val", [r for r in _spec_rows() if r[1] != "nan"])
def test_spec_values_encode(code, val):
    v = -0.0 if val == "-0" else float(val)
    assert int(oracle.e4m3_encode(np.array([v], np.float32))[0]) == code


def test_exhaustive_round_trip():
    codes = np.arange(256, dtype=np.uint8)
    vals = oracle.e4m3_decode(codes)
    finite = ~np.isnan(vals)
    assert finite.sum() == 254                       # only S.1111.111 is NaN
    back = oracle.e4m3_encode(vals[finite].astype(np.float32))
    assert np.array_equal(back, codes[finite])


def _brute_force_encode(v):
    """Nearest finite E4M3 value; ties go to the code with an even mantissa;
    magnitudes above 448 saturate.  Uses only the decode table."""
    codes = np.arange(256, dtype=np.uint8)
    table = oracle.e4m3_decode(codes)
    pos = np.where(~np.isnan(table) & (codes < 0x80))[0]        # 0x00..0x7E
    tv = table[pos]
    v = np.asarray(v, np.float64)
    a = np.minimum(np.abs(v), 448.0)
    out = np.empty(v.shape, np.uint8)
    for s in range(0, v.size, 4096):
        blk = a[s:s + 4096, None]
        dist = np.abs(blk - tv[None, :])
        best = dist.min(axis=1, keepdims=True)
        cand = dist == best
        # among equal-distance candidates prefer the even mantissa (code bit 0 clear)
        even = cand & ((pos[None, :] & 1) == 0)
        pick = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
        out[s:s + 4096] = pos[pick]
    sign = np.signbit(v)
    return np.where(sign, out | 0x80, out).astype(np.uint8)


def test_brute_force_nearest():
    rng = np.random.default_rng(7)
    codes = np.arange(0x7F, dtype=np.uint8)
    tv = np.sort(oracle.e4m3_decode(codes))
    mids = (tv[1:] + tv[:-1]) / 2                     # exact ties
    mids32 = mids.astype(np.float32)
    assert np.array_equal(mids32.astype(np.float64), mids)
    up = np.nextafter(mids32, np.float32(np.inf))
    dn = np.nextafter(mids32, np.float32(-np.inf))
    samples = [tv.astype(np.float32), mids32, up, dn,
               rng.uniform(-480, 480, 100000).astype(np.float32),
               (np.exp(rng.uniform(np.log(1e-5), np.log(480), 100000))
                * rng.choice([-1, 1], 100000)).astype(np.float32),
               np.array([448.0, 449.0, 463.99, 464.0, 500.0, 1e30, -1e30, 0.0, -0.0], np.float32)]
    v = np.concatenate([s.ravel() for s in samples] + [-mids32, -up, -dn])
    got = oracle.e4m3_encode(v)
    want = _brute_force_encode(v)
    assert np.array_equal(got, want), v[got != want][:10]


def test_rne_ties_examples():
    # 1.0625 lies halfway between 1.0 (mantissa 0, even) and 1.125 (mantissa 1)
    # 1.1875 lies halfway between 1.125 (mantissa 1) and 1.25 (mantissa 2, even)
    got = oracle.e4m3_encode(np.array([1.0625, 1.1875, 0.0009765625, 0.0029296875], np.float32))
    # 2^-10 is halfway between 0 and 2^-9 -> 0 (even); 1.5 * 2^-9 -> 2 * 2^-9
    assert list(got) == [0x38, 0x3A, 0x00, 0x02]
