"""Pins for the oracle's FP8 E4M3FN codec.

* decode: all 256 codes against the closed form of the format and against
  PyTorch's float8_e4m3fn -> float32 conversion (an independent library);
* encode: every bfloat16 bit pattern and a dense float32 sweep against
  PyTorch's float32 -> float8_e4m3fn conversion wherever that conversion is
  finite (|y| below the rounding midpoint 464 above 448), and against the
  saturation reading (+-448) above it;
* brute force on a sample: the chosen code is a nearest finite value, ties
  to the even code.
"""
import numpy as np
import pytest
import torch


def _torch_encode(y: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(y, np.float32)).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy()


def test_decode_all_codes(orc):
    codes = np.arange(256, dtype=np.uint8)
    got = orc.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy().astype(np.float64)
    nan = np.isnan(ref)
    assert nan.sum() == 2 and np.isnan(got[nan]).all()
    assert (got[~nan] == ref[~nan]).all()
    # closed form
    for c in range(256):
        s, e, m = c >> 7, (c >> 3) & 15, c & 7
        if e == 15 and m == 7:
            continue
        v = (m / 8) * 2.0 ** -6 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
        assert got[c] == (-v if s else v)
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6


def _check_against_torch(orc, y):
    got = orc.e4m3_encode(y)
    a = np.abs(y.astype(np.float64))
    finite = np.isfinite(a) & (a < 464.0)
    ref = _torch_encode(y)
    assert (got[finite] == ref[finite]).all(), np.argwhere(got[finite] != ref[finite])[:5]
    big = np.isfinite(a) & (a >= 464.0) | np.isinf(a)
    assert (got[big] == np.where(np.signbit(y[big]), 0xFE, 0x7E)).all()
    assert (got[np.isnan(y)] == 0x7F).all()


def test_encode_every_bf16(orc):
    bits = np.arange(1 << 16, dtype=np.uint32) << 16
    y = bits.view(np.float32)
    _check_against_torch(orc, y)


def test_encode_float32_sweep(orc):
    rng = np.random.default_rng(0)
    # all fp32 with exponent near the e4m3 range, random mantissas, plus every
    # exact midpoint between consecutive finite codes (the tie cases)
    u = rng.integers(0, 1 << 32, size=1 << 22, dtype=np.uint64).astype(np.uint32)
    exp = rng.integers(100, 140, size=u.size).astype(np.uint32)
    u = (u & np.uint32(0x807FFFFF)) | (exp << np.uint32(23))
    vals = orc.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    assert (mids.astype(np.float64) == (vals[:-1] + vals[1:]) / 2).all()
    y = np.concatenate([u.view(np.float32), mids, -mids, vals.astype(np.float32),
                        np.float32([0.0, -0.0, 448.0, 449.0, 463.99, 464.0, 1e30, np.inf, -np.inf, np.nan])])
    _check_against_torch(orc, y)


def test_encode_ties_to_even_and_nearest(orc):
    vals = orc.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = (vals[:-1] + vals[1:]) / 2
    got = orc.e4m3_encode(mids.astype(np.float32))
    lo = np.arange(0x7E)
    want = np.where(lo % 2 == 0, lo, lo + 1)
    assert (got == want).all()
    # smallest subnormal / 2 rounds to +0 (tie, even code 0); just above goes to code 1
    assert orc.e4m3_encode(np.float32([2.0 ** -10]))[0] == 0
    assert orc.e4m3_encode(np.float32([np.nextafter(np.float32(2.0 ** -10), np.float32(1))]))[0] == 1
    assert orc.e4m3_encode(np.float32([-2.0 ** -12]))[0] == 0x80


@pytest.mark.parametrize("seed", range(3))
def test_encode_brute_force_nearest(orc, seed):
    rng = np.random.default_rng(seed)
    y = (rng.standard_normal(20000) * 10.0 ** rng.uniform(-4, 2.7, 20000)).astype(np.float32)
    got = orc.e4m3_encode(y)
    table = orc.e4m3_decode(np.arange(256, dtype=np.uint8))
    fin = np.isfinite(table)
    for yi, ci in zip(y[:4000], got[:4000]):
        a = float(yi)
        if abs(a) > 448:
            assert table[ci] == np.sign(a) * 448
            continue
        d = np.abs(table[fin] - a)
        best = d.min()
        assert abs(table[ci] - a) == best
        cands = np.arange(256)[fin][d == best]
        if len(cands) > 1 and not (a == 0):
            assert ci % 2 == 0 or all(c % 2 == 1 for c in cands)
