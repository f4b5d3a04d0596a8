"""Pins for the probability codes: lean P (paper Sec. IV-B1, Eq. 2) and exact P.

Each bound below is a number the paper states (tests/golden/lean_p_bounds.txt); the
oracle's code functions must reproduce it from their own arithmetic."""
import numpy as np
import pytest


def _decode(orc, codes):
    return orc.e4m3_table()[np.asarray(codes, dtype=np.int64)]


def _lean(orc, xs, sigma=6, beta=0.35):
    return np.array([orc.leanp_code(float(x), sigma, beta) for x in xs])


def test_block_max_gets_code_of_one(orc, golden_bounds):
    # x = 0 (the block maximum after per-block scaling) gets the code of 2^sigma
    s = int(golden_bounds["sigma"])
    assert orc.leanp_code(0.0) == int(golden_bounds["block_max_code"])
    assert orc.exactp_code(0.0) == int(golden_bounds["block_max_code"])
    assert orc.e4m3_value(int(golden_bounds["block_max_code"])) == 2.0 ** s


def test_lean_p_exact_at_integers(orc):
    # at whole binades the straight line meets 2^x, so lean P is exact there
    for n in range(0, 13):
        c = orc.leanp_code(-float(n))
        assert orc.e4m3_value(c) == 2.0 ** (6 - n)


def test_interpolation_error(orc, golden_bounds):
    # value of the continuous code y on the piecewise-linear e4m3 curve vs 2^(x+sigma)
    x = np.linspace(-1.0, 0.0, 200001)
    sigma = golden_bounds["sigma"]

    def err(beta):
        y = 8 * (x + sigma + 7) - beta
        e, f = np.floor(y / 8), y / 8 - np.floor(y / 8)
        val = 2.0 ** (e - 7) * (1 + f)
        return np.max(np.abs(val / 2.0 ** (x + sigma) - 1))

    with_b, without_b = err(golden_bounds["beta"]), err(0.0)
    assert with_b <= golden_bounds["interp_err_with_bias"]
    assert with_b > 0.8 * golden_bounds["interp_err_with_bias"]
    assert abs(without_b - golden_bounds["interp_err_without_bias"]) < 0.003


def test_rounded_error_bounds(orc, golden_bounds):
    # over the normal range of the scaled probability the error depends only on frac(x)
    x = np.linspace(-6.0, 0.0, 60001)
    p = 2.0 ** (x + golden_bounds["sigma"])
    lean = _decode(orc, _lean(orc, x))
    exact = _decode(orc, [orc.exactp_code(float(v)) for v in x])
    el = np.max(np.abs(lean / p - 1))
    ee = np.max(np.abs(exact / p - 1))
    assert el <= golden_bounds["leanp_rounded_err"] and el > 0.9 * golden_bounds["leanp_rounded_err"]
    assert ee <= golden_bounds["exactp_rounded_err"] and ee > 0.95 * golden_bounds["exactp_rounded_err"]
    assert abs(ee - 1 / 17) < 1e-4  # half a mantissa step at the bottom of a binade


def test_subnormal_underestimate(orc, golden_bounds):
    # codes 1..7 are subnormal; lean P under-reads them (largest at the top of code 1)
    x = np.linspace(-12.85, -12.0, 20001)
    codes = _lean(orc, x)
    sub = (codes >= 1) & (codes <= 7)
    p = 2.0 ** (x + 6)
    under = np.max(1 - _decode(orc, codes[sub]) / p[sub])
    assert abs(under - golden_bounds["leanp_subnormal_underestimate"]) < 0.02, under


def test_underflow_depth(orc, golden_bounds):
    nl = golden_bounds["leanp_underflow_binades"]
    ne = golden_bounds["exactp_underflow_binades"]
    # lean P: code 0 once y < 0.5, i.e. x < -(sigma + 7) + (0.5 + beta)/8 = -12.894
    assert orc.leanp_code(-12.90) == 0 and orc.leanp_code(-12.89) >= 1
    assert nl - 0.2 < 12.894 < nl + 0.2
    # exact P: 2^(x+6) below 2^-10 (half the smallest subnormal) rounds to zero
    assert orc.exactp_code(-ne) == 0 and orc.exactp_code(-ne + 0.01) == 1


def test_codes_stay_below_nan(orc, golden_bounds):
    # with a stale maximum x can exceed 0 by less than tau; codes stay < 127 (no NaN / sign)
    tau = golden_bounds["tau_fp8"]
    for x in np.linspace(0, tau - 1e-9, 101):
        c = orc.leanp_code(float(x))
        assert c <= 105
        assert orc.exactp_code(float(x)) <= 105
    assert _decode(orc, [orc.leanp_code(tau - 1e-9)])[0] <= 64 * 2 ** tau * 1.075


@pytest.mark.parametrize("sigma", [0, 6])
def test_sigma_shifts_codes_by_8_per_binade(orc, sigma):
    xs = np.linspace(-5, 0, 501)
    a = _lean(orc, xs, sigma=sigma)
    b = _lean(orc, xs - 1, sigma=sigma)
    ok = (b > 8)
    assert np.array_equal(a[ok] - b[ok], np.full(ok.sum(), 8))
