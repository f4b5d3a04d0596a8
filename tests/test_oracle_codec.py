"""Pins for the oracle's number formats: e4m3 decode/round, bf16 round, the pow2 quantiser.

Pinned against the worked values the paper prints (tests/golden/e4m3_worked_values.txt),
exact-rational brute force, and library conversions (torch CPU float8_e4m3fn / bfloat16)."""
from fractions import Fraction

import numpy as np
import pytest
import torch

from conftest import load_golden


def test_e4m3_worked_values(orc):
    for val, code, _src in load_golden("e4m3_worked_values.txt"):
        assert int(orc.e4m3_rne(float(val))[0]) == int(code), (val, code)
        if float(val) >= 2.0 ** -9:
            assert orc.e4m3_value(int(code)) == float(val)


def test_e4m3_structure(orc):
    t = orc.e4m3_table()
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    pos = t[:127]
    assert np.all(np.diff(pos) > 0)                     # codes 0..126 increase
    assert np.array_equal(t[128:255], -pos)             # sign bit
    assert pos[126] == 448.0
    # subnormal spacing 2^-9 below 2^-6, 8 values per binade above (paper Sec. II-C, fn 5)
    assert np.allclose(np.diff(pos[:9]), 2.0 ** -9)
    for e in range(-6, 8):
        codes = [c for c in range(127) if 2.0 ** e <= pos[c] < 2.0 ** (e + 1)]
        assert len(codes) == 8
        # adding 8 to a code doubles the value (paper Sec. IV-B1, fn 10)
        for c in codes:
            if c + 8 <= 126:
                assert pos[c + 8] == 2 * pos[c]


def test_e4m3_rne_matches_exact_rationals(orc):
    t = orc.e4m3_table()
    xs, want = [], []
    for c in range(0, 126):
        lo, hi = Fraction(t[c]), Fraction(t[c + 1])
        mid = (lo + hi) / 2
        eps = (hi - lo) / 1024
        even = c if c % 2 == 0 else c + 1
        for x, w in ((mid, even), (mid - eps, c), (mid + eps, c + 1), (lo, c), (hi, c + 1)):
            xs.append(float(x)); want.append(w)
            xs.append(-float(x)); want.append(w | 0x80)
    got = orc.e4m3_rne(np.array(xs))
    assert np.array_equal(got, np.array(want, dtype=np.uint8))
    # saturation beyond 448 (reading: satfinite)
    assert list(orc.e4m3_rne(np.array([449.0, 1e6, -1e6]))) == [126, 126, 254]


def test_e4m3_rne_matches_torch(orc):
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(200000) * 60, np.exp2(rng.uniform(-12, 8.8, 100000))])
    x = x[np.abs(x) <= 448].astype(np.float32).astype(np.float64)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = orc.e4m3_rne(x)
    # torch keeps the sign of values that round to zero; so do we
    assert np.array_equal(got, ref)


def test_bf16_rne_matches_torch(orc):
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(300000) * np.exp2(rng.uniform(-30, 30, 300000))).astype(np.float32)
    # exact ties: low 16 bits = 0x8000
    bits = x.view(np.uint32)
    ties = ((bits[:1000] & 0xFFFF0000) | 0x8000).view(np.float32)
    x = np.concatenate([x, ties])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(orc.bf16_rne(x), ref)


def test_quantiser_scale_and_snr(orc, golden_bounds):
    rng = np.random.default_rng(2)
    x = rng.standard_normal((1 << 20,)).astype(np.float32)
    codes, ds = orc.quantize_e4m3(x)
    amax = float(np.abs(x).max())
    k = -int(np.log2(ds))
    assert ds == 2.0 ** -k                                  # power-of-two descale
    assert amax * 2.0 ** k <= 448.0 < amax * 2.0 ** (k + 1)  # largest pow2 with no saturation
    deq = orc.e4m3_table()[codes] * ds
    snr = 10 * np.log10(np.sum(x.astype(np.float64) ** 2) / np.sum((deq - x) ** 2))
    assert golden_bounds["e4m3_snr_db_lo"] - 0.5 <= snr <= golden_bounds["e4m3_snr_db_hi"] + 0.5, snr
    # codes equal torch's rounding of the scaled values
    ref = torch.from_numpy(x.astype(np.float64) * 2.0 ** k).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, ref)


@pytest.mark.parametrize("amax", [0.0, 1e-42, 3e38, 448.0, 448.00003, 1.0])
def test_quantiser_edges(orc, amax):
    x = np.array([amax, -amax / 3, 0.0], dtype=np.float32)
    codes, ds = orc.quantize_e4m3(x)
    if amax == 0.0:
        assert ds == 1.0 and not (codes & 0x7F).any()
        return
    assert np.isfinite(ds) and ds > 0
    val = orc.e4m3_table()[codes] * ds
    assert abs(val[0]) <= abs(float(x[0])) * 1.07 + 1e-300
    assert orc.e4m3_table()[codes[0]] <= 448.0
