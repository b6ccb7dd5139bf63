"""Pins for the oracle's OCP e5m2 codec (CPU only).

Decode is checked against torch's float8_e5m2 for every byte and against the
format's named values (bias 15, 2 mantissa bits, infinities and NaN in
exponent 31, largest finite 57344).  The encoder (round to nearest even,
saturating at 57344) is checked against a brute-force nearest search over all
finite e5m2 values, exhaustively over every binary16 input, on ties and their
neighbours, on random fp32 values, and against torch's conversion where torch
does not overflow.
"""
import numpy as np
import pytest
import torch

import oracle as O


def _torch_values():
    b = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return b.view(torch.float8_e5m2).to(torch.float32).double().numpy()


def test_e5m2_decode_matches_torch_for_all_bytes():
    ours = O.e5m2_values(np.arange(256, dtype=np.uint8))
    ref = _torch_values()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_e5m2_named_values():
    v = O.e5m2_values(np.arange(256, dtype=np.uint8))
    assert v[0x7B] == 57344.0 and v[0xFB] == -57344.0       # largest finite
    assert v[0x7C] == np.inf and v[0xFC] == -np.inf          # S.11111.00
    assert v[0x01] == 2.0 ** -16                             # smallest subnormal
    assert v[0x03] == 3 * 2.0 ** -16                         # largest subnormal
    assert v[0x04] == 2.0 ** -14                             # smallest normal
    assert v[0x3C] == 1.0 and v[0xBC] == -1.0
    assert np.isnan(v[[0x7D, 0x7E, 0x7F, 0xFD, 0xFE, 0xFF]]).all()
    assert np.isnan(v).sum() == 6 and np.isinf(v).sum() == 2
    # every e5m2 value is the binary16 value of the byte followed by 8 zero bits
    as_f16 = (np.arange(256, dtype=np.uint16) << 8).view(np.float16).astype(np.float64)
    fin = ~np.isnan(v)
    assert np.array_equal(v[fin], as_f16[fin])


def _finite_table():
    codes = np.arange(0x7C, dtype=np.uint8)                  # 0x00..0x7B, non-negative
    return codes, O.e5m2_values(codes)


def _brute_force_encode(x: np.ndarray) -> np.ndarray:
    """Nearest finite e5m2 value by exhaustive search; ties to the even code;
    magnitudes beyond the finite range (infinities too) take the largest."""
    codes, vals = _finite_table()
    with np.errstate(invalid="ignore"):
        a = np.minimum(np.abs(x.astype(np.float64)), 1e12)
    out = np.empty(x.shape, np.uint8)
    for lo in range(0, a.size, 8192):
        aa = a[lo:lo + 8192, None]
        dist = np.abs(aa - vals[None, :])
        best = dist.min(axis=1, keepdims=True)
        cand = dist == best
        even = cand & (codes[None, :] % 2 == 0)
        pick = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
        out[lo:lo + 8192] = codes[pick]
    sign = np.signbit(x).astype(np.uint8) << 7
    out = out | sign
    out[np.isnan(x)] = (sign[np.isnan(x)] | 0x7F)
    return out


def test_e5m2_encode_exhaustive_over_binary16():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = bits.view(np.float16).astype(np.float32)
    assert np.array_equal(O.e5m2_encode(x), _brute_force_encode(x))


def test_e5m2_encode_ties_and_neighbours():
    codes, vals = _finite_table()
    mids = (vals[:-1] + vals[1:]) / 2
    xs = [mids, np.nextafter(mids.astype(np.float32), np.float32(np.inf)),
          np.nextafter(mids.astype(np.float32), np.float32(-np.inf)), vals]
    x = np.concatenate([a.astype(np.float32) for a in xs])
    x = np.concatenate([x, -x, np.float32([61440.0, 61439.0, 65504.0, 1e30, np.inf, -np.inf,
                                            2.0 ** -17, 2.0 ** -18, 1e-30, 0.0, -0.0])])
    assert np.array_equal(O.e5m2_encode(x), _brute_force_encode(x))
    # 1.125 lies halfway between 1.0 (0x3C) and 1.25 (0x3D): the even code wins
    assert O.e5m2_encode(np.float32([1.125]))[0] == 0x3C
    assert O.e5m2_encode(np.float32([1.375]))[0] == 0x3E


def test_e5m2_encode_random_fp32():
    rng = np.random.default_rng(4321)
    x = np.concatenate([rng.standard_normal(200000).astype(np.float32) * s
                        for s in (1e-5, 0.05, 1.0, 300.0, 20000.0)])
    assert np.array_equal(O.e5m2_encode(x), _brute_force_encode(x))


def test_e5m2_encode_matches_torch_below_overflow():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = bits.view(np.float16).astype(np.float32)
    x = x[np.isfinite(x) & (np.abs(x) < 57344.0)]
    ref = torch.from_numpy(x).to(torch.float8_e5m2).view(torch.uint8).numpy()
    assert np.array_equal(O.e5m2_encode(x), ref)


@pytest.mark.parametrize("x,code", [(57344.0, 0x7B), (60000.0, 0x7B), (61440.0, 0x7B),
                                    (1e9, 0x7B), (float("inf"), 0x7B), (-1e9, 0xFB),
                                    (float("nan"), 0x7F)])
def test_e5m2_encode_saturates(x, code):
    assert O.e5m2_encode(np.float32([x]))[0] == code
