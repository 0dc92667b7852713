"""Pins for the oracle's codecs (bf16 RNE, OCP E4M3 encode / decode).

Each oracle codec is checked against something other than itself:
  * torch's float8_e4m3fn and bfloat16 casts (library special cases), where
    they are defined the same way (torch's E4M3 cast does not saturate above
    464, so it is used only for |v| <= 464);
  * a brute-force nearest-code search over the 127 finite magnitudes with ties
    to the even code, a different algorithm from the oracle's exponent /
    mantissa rounding;
  * the two values the method fixes: 448 is the largest finite code (0x7E),
    which is why scales are amax/448 (the headline workload's FP8 recipe), and
    2^-9 is the smallest subnormal (0x01).
"""
import numpy as np
import pytest
import torch

import oracle


def torch_e4m3(v: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy()


def torch_e4m3_decode_table() -> np.ndarray:
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float32).numpy()


def test_decode_table_matches_torch_and_fixed_points():
    table = oracle.e4m3_decode(np.arange(256, dtype=np.uint8))
    ref = torch_e4m3_decode_table()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(table), nan)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.array_equal(table[~nan].view(np.uint32), ref[~nan].view(np.uint32))  # incl. -0
    assert table[0x7E] == 448.0 and table[0xFE] == -448.0
    assert table[0x01] == 2.0 ** -9 and table[0x08] == 2.0 ** -6
    assert table[0x38] == 1.0
    assert np.signbit(table[0x80]) and table[0x80] == 0.0


def _brute_force_encode(v: np.ndarray) -> np.ndarray:
    """Nearest finite E4M3 magnitude by search; ties to the even code;
    magnitudes >= 448 saturate to 0x7E; sign copied."""
    mags = torch_e4m3_decode_table()[:0x7F].astype(np.float64)  # codes 0x00..0x7E, ascending
    assert np.all(np.diff(mags) > 0)
    a = np.abs(v.astype(np.float64))
    hi = np.searchsorted(mags, a, side="left").clip(0, 0x7E)
    lo = (hi - 1).clip(0, 0x7E)
    dlo = np.abs(a - mags[lo])
    dhi = np.abs(mags[hi] - a)
    code = np.where(dlo < dhi, lo, hi)
    tie = dlo == dhi
    code = np.where(tie, np.where(lo % 2 == 0, lo, hi), code)
    code = np.where(a >= 448.0, 0x7E, code)
    sign = np.signbit(v).astype(np.uint8) << 7
    return (code.astype(np.uint8) | sign).astype(np.uint8)


def _probe_values() -> np.ndarray:
    mags = torch_e4m3_decode_table()[:0x7F].astype(np.float32)
    mids = ((mags[:-1].astype(np.float64) + mags[1:]) / 2).astype(np.float32)
    pts = np.concatenate([mags, mids, [464.0, 463.99997, 448.0, 447.99997, 0.0]]).astype(np.float32)
    # each point and its two fp32 neighbours
    near = np.concatenate([pts, np.nextafter(pts, np.float32(np.inf)), np.nextafter(pts, np.float32(0))])
    # every positive bf16 pattern up to 464, widened exactly
    bf = (np.arange(0, 0x43E9, dtype=np.uint32) << 16).view(np.float32)
    rng = np.random.default_rng(1)
    rnd = (2.0 ** rng.uniform(-160, 9, 400_000)).astype(np.float32)
    rnd = rnd[rnd <= 464]
    # fp32 subnormals (the quotient x/s can be one)
    sub = (rng.integers(1, 1 << 23, 50_000, dtype=np.uint32)).view(np.float32)
    allv = np.concatenate([near, bf, rnd, sub]).astype(np.float32)
    return np.concatenate([allv, -allv])


def test_encode_matches_brute_force_nearest():
    v = _probe_values()
    assert np.array_equal(oracle.e4m3_encode(v), _brute_force_encode(v))


def test_encode_matches_torch_cast_up_to_464():
    v = _probe_values()
    v = v[np.abs(v) <= 464]
    assert np.array_equal(oracle.e4m3_encode(v), torch_e4m3(v))


def test_encode_matches_torch_on_fp32_lattice():
    # fp32 patterns (i << 8) | low for all i with |v| <= 464 and four low-bit
    # patterns: covers every E4M3 rounding boundary in every binade, subnormal
    # fp32 inputs included.
    top = 0x43E80000 >> 8
    base = np.arange(0, top + 1, dtype=np.uint32) << 8
    for low in (0x00, 0x7F, 0x80, 0xFF):
        v = (base | np.uint32(low)).view(np.float32)
        v = v[np.abs(v) <= 464]
        assert np.array_equal(oracle.e4m3_encode(v), torch_e4m3(v)), hex(low)
        assert np.array_equal(oracle.e4m3_encode(-v), torch_e4m3(-v)), hex(low)


def test_encode_saturates_and_special_values():
    v = np.array([448.0, 464.0, 464.00003, 480.0, 1e30, np.inf, -np.inf, -500.0,
                  0.0, -0.0, -1e-30, 2.0 ** -10, 3 * 2.0 ** -11, np.nan], np.float32)
    got = oracle.e4m3_encode(v)
    assert list(got[:8]) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE]
    assert list(got[8:13]) == [0x00, 0x80, 0x80, 0x00, 0x01]
    assert got[13] & 0x7F == 0x7F


def test_bf16_rne_matches_torch():
    rng = np.random.default_rng(2)
    bits = rng.integers(0, 1 << 32, 2_000_000, dtype=np.uint64).astype(np.uint32)
    edge = np.array([0x3F808000, 0x3F818000, 0x3F80FFFF, 0x3F807FFF, 0x7F7FFFFF, 0x7F7F8000,
                     0x7F7F7FFF, 0x00008000, 0x00018000, 0x80008000, 0x7F800000, 0xFF800000,
                     0x00000001, 0x80000000, 0x00000000], np.uint32)
    v = np.concatenate([bits, edge]).view(np.float32)
    got = oracle.bf16_rne(v)
    ref = torch.from_numpy(v.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    isnan = np.isnan(v)
    assert np.array_equal(got[~isnan], ref[~isnan])
    # NaN stays NaN (exponent all ones, nonzero mantissa), sign kept
    g = got[isnan]
    assert np.all((g & 0x7F80) == 0x7F80) and np.all((g & 0x007F) != 0)
    assert np.array_equal(g >> 15, (v[isnan].view(np.uint32) >> 31).astype(np.uint16))


def test_bf16_widening_is_exact():
    b = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    f = oracle.bf16_to_f32(b)
    ref = torch.from_numpy(b.view(np.int16).copy()).view(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(f.view(np.uint32), ref.view(np.uint32))
    back = oracle.bf16_rne(f)
    ok = ~np.isnan(f)
    assert np.array_equal(back[ok], b[ok])
