"""Pins of the oracle's rotation and K smoothing (paper Sec. V-E, "Rotation and K
smoothing"; Table XIII): the matrices against library routines, orthogonality, the score
invariance (QR)(KR)^T = QK^T, the softmax invariance of subtracting one mean key, the
fp64 quantiser against the pinned fp32 one, and the error reduction on inputs whose large
channels coincide in q and k (the situation the paper's rotation addresses)."""
import math

import numpy as np
import pytest
import scipy.fft
import scipy.linalg

import synth


def _signs(D, seed=0):
    return np.where(np.random.default_rng(seed).integers(0, 2, D) == 1, 1.0, -1.0)


@pytest.mark.parametrize("n", [1, 2, 4, 8, 64, 128])
def test_hadamard_matches_library(orc, n):
    assert np.array_equal(orc.hadamard(n), scipy.linalg.hadamard(n) / math.sqrt(n))


@pytest.mark.parametrize("m", [1, 2, 3, 4])
def test_dct2_matches_library(orc, m):
    ref = scipy.fft.dct(np.eye(m), type=2, norm="ortho", axis=0)
    assert np.allclose(orc.dct2(m), ref, atol=1e-15)


@pytest.mark.parametrize("D", [128, 192])
def test_rotation_orthogonal_and_structured(orc, D):
    s = _signs(D)
    R = orc.rotation(s)
    assert np.abs(R @ R.T - np.eye(D)).max() < 1e-13
    assert np.abs(R.T @ R - np.eye(D)).max() < 1e-13
    # every row of the transform spreads one channel evenly: |R_ij| = 1/sqrt(D) at D = 128
    if D == 128:
        assert np.allclose(np.abs(R), 1 / math.sqrt(D))
    # flipping a sign flips exactly one row of R
    s2 = s.copy()
    s2[5] = -s2[5]
    R2 = orc.rotation(s2)
    assert np.array_equal(R2[5], -R[5]) and np.array_equal(np.delete(R2, 5, 0), np.delete(R, 5, 0))


@pytest.mark.parametrize("D", [128, 192])
def test_scores_invariant(orc, D):
    rng = np.random.default_rng(D)
    q = rng.standard_normal((1, 64, 2, D))
    k = rng.standard_normal((1, 64, 2, D))
    s = _signs(D, 1)
    qr, kr = orc.rotate(q, s), orc.rotate(k, s)
    for h in range(2):
        a = q[0, :, h] @ k[0, :, h].T
        b = qr[0, :, h] @ kr[0, :, h].T
        assert np.abs(a - b).max() < 1e-11 * np.abs(a).max()


def test_key_mean_and_smoothing_shift(orc):
    rng = np.random.default_rng(3)
    k = rng.standard_normal((2, 96, 3, 128)) + rng.standard_normal((2, 1, 3, 128))
    mu = orc.key_mean(k)
    assert mu.shape == (2, 3, 128)
    assert np.allclose(mu, k.sum(axis=1) / 96, atol=1e-14)
    ks = orc.rotate(k, np.ones(128) , mu) @ orc.rotation(np.ones(128)).T  # rotate back
    assert np.allclose(ks.mean(axis=1), 0.0, atol=1e-13)


def test_smoothing_cancels_in_attention(orc):
    """Subtracting one mean key per head lowers every score of a row by the same value, so
    fp64 attention (oracle) is unchanged; checked on bf16-exact inputs whose shifted keys
    stay exact."""
    rng = np.random.default_rng(9)
    B, S, H, D = 1, 256, 2, 128
    q = np.round(rng.standard_normal((B, S, H, D)) * 8) / 8
    k = np.round(rng.standard_normal((B, S, H, D)) * 8) / 8
    v = np.round(rng.standard_normal((B, S, H, D)) * 8) / 8
    mu = np.round(rng.standard_normal((B, H, D)) * 4) / 4          # any per-head vector
    ks = k - mu[:, None]
    qb, kb, kbs, vb = (orc.bf16_rne(x.astype(np.float32)) for x in (q, k, ks, v))
    rows = orc.group_rows(np.array([[0, h, r] for h in range(H) for r in range(0, S, 32)]), 32)
    o1, l1 = orc.attn_exact(qb, kb, vb, dtype="bf16", c=1 / math.sqrt(D), rows=rows)
    o2, l2 = orc.attn_exact(qb, kbs, vb, dtype="bf16", c=1 / math.sqrt(D), rows=rows)
    assert np.abs(o1 - o2).max() < 1e-12
    # the LSE moves by exactly c q.mu per row
    shift = np.einsum("rd,rd->r", q[0, rows[:, 2], rows[:, 1]], mu[0, rows[:, 1]]) / math.sqrt(D)
    assert np.abs((l1 - l2) - shift).max() < 1e-9


def test_quantize_f64_matches_f32_quantiser(orc):
    rng = np.random.default_rng(4)
    x = (rng.standard_normal(4096) * 3).astype(np.float32)
    c32, d32 = orc.quantize_e4m3(x)
    c64, d64 = orc.quantize_e4m3_f64(x.astype(np.float64))
    assert d32 == d64 and np.array_equal(c32, c64)


@pytest.mark.parametrize("D", [128, 192])
def test_rotation_lowers_input_error_with_outlier_channels(orc, D):
    """Large channels shared by q and k make the score rounding error large; the rotation
    spreads them over all channels (the paper reports about half the input error)."""
    B, S, H = 1, 512, 2
    q, k, _ = synth.activation_like(B, S, H, D, 128, 5)
    s = _signs(D)
    mu = orc.key_mean(k)

    def score_err(qq, kk, rot):
        if rot:
            qc, dq = orc.rotate_quantize_e4m3(qq, s)
            kc, dk = orc.rotate_quantize_e4m3(kk, s, mu)
        else:
            (qc, dq), (kc, dk) = orc.quantize_e4m3(qq), orc.quantize_e4m3(kk)
        t = orc.e4m3_table()
        qh, kh = t[qc] * dq, t[kc] * dk
        err = []
        for h in range(H):
            exact = qq[0, :, h].astype(np.float64) @ kk[0, :, h].astype(np.float64).T
            approx = qh[0, :, h] @ kh[0, :, h].T
            exact = exact - (qq[0, :, h].astype(np.float64) @ mu[0, h])[:, None] if rot else exact
            err.append(np.linalg.norm(approx - exact) / np.linalg.norm(exact))
        return float(np.mean(err))

    e0, e1 = score_err(q, k, False), score_err(q, k, True)
    assert e1 < 0.75 * e0, (e0, e1)


def test_static_quantiser_equals_per_call_at_its_descale(orc):
    """With the descale the per-call rule picks, the static quantiser gives the same codes
    (fp32 and fp64 inputs, plain and rotated)."""
    rng = np.random.default_rng(12)
    x = (rng.standard_normal((1, 64, 2, 128)) * 5).astype(np.float32)
    c, d = orc.quantize_e4m3(x)
    assert np.array_equal(orc.quantize_e4m3_static(x, d), c)
    s = _signs(128, 2)
    c2, d2 = orc.rotate_quantize_e4m3(x, s, orc.key_mean(x))
    assert np.array_equal(orc.rotate_quantize_e4m3_static(x, s, d2, orc.key_mean(x)), c2)
    # a larger descale (coarser codes) halves every value before rounding: codes of x/2
    assert np.array_equal(orc.quantize_e4m3_static(x, 2 * d), c_half := orc.quantize_e4m3_static(x / 2, d))
    assert c_half.shape == x.shape


def test_static_quantiser_saturates(orc):
    t = orc.e4m3_table()
    x = np.array([1000.0, -1000.0, 448.0, 449.0, 463.9, 464.0, 480.0, -3e38, 0.5, -0.0])
    got = t[orc.quantize_e4m3_static(x, 1.0)]
    assert np.array_equal(got[:8], [448, -448, 448, 448, 448, 448, 448, -448])
    assert got[8] == 0.5 and got[9] == 0.0
    # descale 2^-3: x / descale = 8 x, so |x| > 56 saturates
    y = np.array([56.0, 57.0, -200.0, 0.125])
    assert np.array_equal(t[orc.quantize_e4m3_static(y, 0.125)] * 0.125, [56.0, 56.0, -56.0, 0.125])


@pytest.mark.parametrize("bad", [0.0, 3.0, 0.75, -0.5, 2.0 ** 127, 2.0 ** -127, float("inf"), float("nan")])
def test_static_descale_must_be_power_of_two(orc, bad):
    with pytest.raises(ValueError):
        orc.quantize_e4m3_static(np.ones(4), bad)
