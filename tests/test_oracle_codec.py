"""Pins for the oracle's number codecs (CPU only).

binary16 decode is checked against numpy's own float16 conversion for every
bit pattern.  OCP e4m3fn decode is checked against torch's float8_e4m3fn for
every byte and against the format's named values.  The encoder (round to
nearest even, saturating at 448) is checked against a brute-force nearest
search over all finite e4m3fn values, exhaustively over every binary16 input,
and against torch's conversion where torch does not saturate.
"""
import numpy as np
import pytest
import torch

import oracle as O


def test_f16_decode_matches_numpy_for_all_bit_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = O.f16_values(bits)
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def _torch_e4m3_values():
    b = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return b.view(torch.float8_e4m3fn).to(torch.float32).double().numpy()


def test_e4m3_decode_matches_torch_for_all_bytes():
    ours = O.e4m3fn_values(np.arange(256, dtype=np.uint8))
    ref = _torch_e4m3_values()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_e4m3_named_values():
    v = O.e4m3fn_values(np.arange(256, dtype=np.uint8))
    assert v[0x7E] == 448.0 and v[0xFE] == -448.0          # largest finite
    assert v[0x01] == 2.0 ** -9                              # smallest subnormal
    assert v[0x07] == 7 * 2.0 ** -9                          # largest subnormal
    assert v[0x08] == 2.0 ** -6                              # smallest normal
    assert v[0x38] == 1.0 and v[0xB8] == -1.0
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])          # S.1111.111
    assert np.isnan(v).sum() == 2                            # no other NaN, no inf
    assert not np.isinf(v).any()


def _finite_table():
    codes = np.arange(0x7F, dtype=np.uint8)                  # 0x00..0x7E, non-negative
    vals = O.e4m3fn_values(codes)
    return codes, vals


def _brute_force_encode(x: np.ndarray) -> np.ndarray:
    """Nearest finite e4m3fn value by exhaustive search; ties to the even code."""
    codes, vals = _finite_table()
    with np.errstate(invalid="ignore"):
        a = np.abs(x.astype(np.float64))
    # beyond 1e6 float64 differences to the table lose resolution; every such
    # magnitude (and infinity) is nearest to the largest finite value anyway
    a = np.minimum(a, 1e6)
    out = np.empty(x.shape, np.uint8)
    for lo in range(0, a.size, 8192):
        aa = a[lo:lo + 8192, None]
        dist = np.abs(aa - vals[None, :])
        best = dist.min(axis=1, keepdims=True)
        cand = dist == best
        # among the nearest, prefer an even mantissa (even code)
        even = cand & (codes[None, :] % 2 == 0)
        pick = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
        out[lo:lo + 8192] = codes[pick]
    sign = np.signbit(x).astype(np.uint8) << 7
    out = out | sign
    out[np.isnan(x)] = (sign[np.isnan(x)] | 0x7F)
    return out


def test_e4m3_encode_exhaustive_over_binary16():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = bits.view(np.float16).astype(np.float32)
    ours = O.e4m3fn_encode(x)
    ref = _brute_force_encode(x)
    assert np.array_equal(ours, ref)


def test_e4m3_encode_ties_and_neighbours():
    codes, vals = _finite_table()
    v = vals.astype(np.float64)
    mids = (v[:-1] + v[1:]) / 2                    # exact ties (representable in fp32)
    xs = [mids, np.nextafter(mids.astype(np.float32), np.float32(np.inf)),
          np.nextafter(mids.astype(np.float32), np.float32(-np.inf)), v]
    x = np.concatenate([a.astype(np.float32) for a in xs])
    x = np.concatenate([x, -x, np.float32([464.0, 463.99, 500.0, 1e30, np.inf, -np.inf,
                                            2.0 ** -10, 2.0 ** -11, 1e-30, 0.0, -0.0])])
    assert np.array_equal(O.e4m3fn_encode(x), _brute_force_encode(x))
    # ties go to the even mantissa: 1.0625 lies between 1.0 (0x38) and 1.125 (0x39)
    assert O.e4m3fn_encode(np.float32([1.0625, 1.1875]))[0] == 0x38
    assert O.e4m3fn_encode(np.float32([1.1875]))[0] == 0x3A


def test_e4m3_encode_random_fp32():
    rng = np.random.default_rng(1234)
    x = np.concatenate([rng.standard_normal(200000).astype(np.float32) * s
                        for s in (1e-3, 0.05, 1.0, 30.0, 300.0)])
    assert np.array_equal(O.e4m3fn_encode(x), _brute_force_encode(x))


def test_e4m3_encode_matches_torch_below_saturation():
    # torch rounds to nearest even too but maps out-of-range values to NaN, so
    # compare where no saturation happens.
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = bits.view(np.float16).astype(np.float32)
    keep = np.isfinite(x) & (np.abs(x) < 448.0)
    x = x[keep]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(O.e4m3fn_encode(x), ref)


@pytest.mark.parametrize("x,code", [(448.0, 0x7E), (460.0, 0x7E), (464.0, 0x7E), (1e9, 0x7E),
                                    (float("inf"), 0x7E), (-1e9, 0xFE), (float("nan"), 0x7F)])
def test_e4m3_encode_saturates(x, code):
    assert O.e4m3fn_encode(np.float32([x]))[0] == code
