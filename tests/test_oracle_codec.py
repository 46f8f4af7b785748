"""Pins for the oracle's 8-bit codecs (CPU only).

E4M3FN: the OCP 8-bit floating-point format, E4M3 variant without
infinities (the format the FP8_Dynamic and Block_FP8 paths use).  Pinned
against (a) fixed values of the format, (b) PyTorch's float8_e4m3fn dtype,
an independent library implementation, and (c) brute-force nearest-value
search with exact rationals.  int8: pinned against numpy's rint/clip.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from tests import exact


def test_e4m3_decode_fixed_points(oracle_mod):
    d = oracle_mod.e4m3_decode(np.arange(256))
    assert d[0x00] == 0.0 and not np.signbit(d[0x00])
    assert d[0x80] == 0.0 and np.signbit(d[0x80])
    assert d[0x7E] == 448.0 and d[0xFE] == -448.0          # largest finite
    assert d[0x38] == 1.0                                   # exponent field = bias
    assert d[0x08] == 2.0 ** -6                             # smallest normal
    assert d[0x01] == 2.0 ** -9                             # smallest subnormal
    assert d[0x07] == 7 * 2.0 ** -9                         # largest subnormal
    assert np.isnan(d[0x7F]) and np.isnan(d[0xFF])          # the only NaNs
    assert np.isnan(d).sum() == 2


def test_e4m3_decode_matches_torch_all_codes(oracle_mod):
    ours = oracle_mod.e4m3_decode(np.arange(256))
    ref = exact.torch_e4m3_table()
    same = (ours == ref) | (np.isnan(ours) & np.isnan(ref))
    assert same.all(), np.nonzero(~same)
    assert (np.signbit(ours) == np.signbit(ref))[~np.isnan(ref)].all()


def test_e4m3_decode_monotone(oracle_mod):
    d = oracle_mod.e4m3_decode(np.arange(0x7F))
    assert (np.diff(d) > 0).all()
    # 126 positive finite values plus zero; each has at most 4 significant bits
    for v in d[1:]:
        f = Fraction(float(v))
        num = f.numerator
        while num % 2 == 0:
            num //= 2
        assert num < 16


def _encode_sample():
    """Dense sample: every midpoint between neighbouring E4M3FN values and the
    fp32 neighbours of each, the values themselves, random log-uniform
    magnitudes, and the special cases around zero and saturation."""
    vals = exact.torch_e4m3_table()[:0x7F].astype(np.float32)
    mids = ((vals[:-1].astype(np.float64) + vals[1:].astype(np.float64)) / 2).astype(np.float32)
    pts = np.concatenate([vals, mids])
    up = np.nextafter(pts, np.float32(np.inf))
    down = np.nextafter(pts, np.float32(-np.inf))
    rng = np.random.default_rng(1234)
    rnd = (2.0 ** rng.uniform(-14, 9.5, 20000)).astype(np.float32)
    special = np.array([0.0, 2 ** -10, 2 ** -10 * 1.0000001, 447.99, 448, 449, 464, 465, 480,
                        1e4, 3e38, 1e-30, 1.4e-45, 2 ** -6, 2 ** -7 * 3], dtype=np.float32)
    pos = np.concatenate([pts, up, down, rnd, special])
    pos = pos[pos >= 0]
    return np.concatenate([pos, -pos, np.array([-0.0], dtype=np.float32)])


def test_e4m3_encode_matches_torch_on_clamped(oracle_mod):
    v = _encode_sample()
    ours = oracle_mod.e4m3_encode(v)
    clamped = np.clip(v, -448, 448)
    ref = torch.from_numpy(clamped).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    bad = np.nonzero(ours != ref)[0]
    assert bad.size == 0, [(float(v[i]), int(ours[i]), int(ref[i])) for i in bad[:10]]


def test_e4m3_encode_brute_force(oracle_mod):
    v = _encode_sample()
    rng = np.random.default_rng(7)
    idx = rng.choice(v.size, 3000, replace=False)
    sample = np.concatenate([v[idx], np.array([0.0, -0.0, 448, -448, 1000, -1000, 2 ** -10,
                                               -(2 ** -10), 2 ** -11], dtype=np.float32)])
    ours = oracle_mod.e4m3_encode(sample)
    for x, c in zip(sample, ours):
        f = Fraction(float(x))
        want = exact.e4m3_nearest_code(f, bool(np.signbit(x)))
        assert c == want, (float(x), hex(c), hex(want))


def test_e4m3_encode_roundtrip_every_code(oracle_mod):
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    d = oracle_mod.e4m3_decode(codes).astype(np.float32)
    assert (oracle_mod.e4m3_encode(d) == codes).all()


def test_e4m3_encode_ties_to_even(oracle_mod):
    # 1.0625 lies halfway between 1.0 (0x38, even) and 1.125 (0x39): goes to 1.0.
    # 1.1875 lies halfway between 1.125 (0x39) and 1.25 (0x3A, even): goes to 1.25.
    # 2^-10 lies halfway between 0 and 2^-9: goes to +0 / -0.
    # 15.5 lies halfway between 15 (0x57, odd) and 16 (0x58): carries into the next binade.
    got = oracle_mod.e4m3_encode(np.array([1.0625, 1.1875, 2 ** -10, -(2 ** -10), 15.5],
                                          dtype=np.float32))
    assert list(got) == [0x38, 0x3A, 0x00, 0x80, 0x58]


def test_int8_encode_matches_numpy(oracle_mod):
    rng = np.random.default_rng(3)
    v = np.concatenate([rng.uniform(-140, 140, 50000),
                        np.arange(-130, 130.5, 0.5),
                        [126.5, 127.49, 127.5, 128, -127.5, -128, -1e9, 1e9, -0.0]]).astype(np.float32)
    ours = oracle_mod.int8_encode(v)
    ref = np.clip(np.rint(v), -127, 127).astype(np.int8)
    assert (ours == ref).all()
    assert ours.min() >= -127     # -128 is never produced
