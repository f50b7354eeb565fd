"""Pins for the oracle's e4m3 codec (CPU only).

The encoder is checked three independent ways: hand-derived encodings from
the format definition (tests/golden/e4m3_codes.txt), an exhaustive
comparison over all 2^32 fp32 bit patterns against a nearest-value search
(inside the C library, different code path), and a NumPy nearest-value
encoder written separately in tests/dense_ref.py.
"""
import os

import numpy as np
import pytest

import oracle
import dense_ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_codes.txt")


def _golden():
    rows = []
    for line in open(GOLDEN):
        line = line.split("#")[0].strip()
        if not line:
            continue
        v, c = line.split()[:2]
        rows.append((np.float32(float(v)), int(c, 16)))
    return rows


def test_golden_encodings():
    rows = _golden()
    assert len(rows) >= 15
    vals = np.array([v for v, _ in rows], dtype=np.float32)
    got = oracle.encode(vals)
    want = np.array([c for _, c in rows], dtype=np.uint8)
    np.testing.assert_array_equal(got, want)


def test_decode_matches_closed_form():
    # decode table vs (-1)^s 2^(e-7) (1 + m/8), subnormal (m/8) 2^-6, written separately
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.decode(codes).astype(np.float64)
    want = dense_ref.e4m3_values()
    nan = np.isnan(want)
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    assert np.all(np.isnan(got[nan]))
    np.testing.assert_array_equal(got[~nan], want[~nan])
    assert oracle.decode(np.uint8(0x7E)) == 448.0
    assert oracle.decode(np.uint8(0x01)) == 2.0 ** -9


def test_roundtrip_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    np.testing.assert_array_equal(oracle.encode(oracle.decode(codes)), codes)


def test_exhaustive_against_nearest_search():
    # every fp32 bit pattern: bit-level encoder == nearest finite value search
    bad, first = oracle.codec_selfcheck(0, 1 << 32)
    assert bad == 0, f"{bad} mismatches, first pattern {first:#010x}"


def test_against_independent_numpy_encoder():
    rng = np.random.default_rng(0)
    parts = [
        rng.standard_normal(200000).astype(np.float32) * np.float32(100),
        rng.standard_normal(200000).astype(np.float32) * np.float32(0.01),
        (rng.random(100000) * 1000 - 500).astype(np.float32),
    ]
    # every midpoint between neighbouring codes, and one fp32 ulp either side
    vals = dense_ref.e4m3_values()[:127]
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    parts += [mids, np.nextafter(mids, np.float32(np.inf)), np.nextafter(mids, np.float32(0)),
              -mids, vals.astype(np.float32), np.array([np.inf, -np.inf, 464.0, 463.99], np.float32)]
    v = np.concatenate(parts).astype(np.float32)
    np.testing.assert_array_equal(oracle.encode(v), dense_ref.encode_nearest(v))


def test_nan_maps_to_nan_code():
    v = np.array([np.nan, -np.nan], dtype=np.float32)
    got = oracle.encode(v)
    assert (got[0] & 0x7F) == 0x7F and (got[1] & 0x7F) == 0x7F
