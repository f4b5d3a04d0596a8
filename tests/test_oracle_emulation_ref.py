"""Independent pin of the oracle's FP8-scheme emulation (``oracle.emulate_fp8``).

A second implementation of the scheme, written separately and deliberately naive: plain
Python, one query row at a time, its own e4m3 codec taken from the format definition,
exact integer dot products, ``np.float32`` scalars wherever the mirrored kernel takes an
fp32 decision, and exact rationals (``fractions.Fraction``) for the fused multiply-add.
It shares no code with ``oracle/oracle.c`` and does not call it.

What it follows ("ZYFA: Speed and Accuracy of FP8 FlashAttention on AMD CDNA4"):
  * Sec. II-C and its footnote on the format: e4m3 (bias 7, subnormals f/8 2^-6, 448 max);
  * Sec. II-B and Sec. IV-A: base-2 scores t = s c', keys visited from key 0 upward in
    128-key tiles; the running maximum of a 32-row wave is kept unless some row of the
    wave grows by at least tau (the lazy rescale, with the footnote that a stale maximum
    lets probabilities exceed 1 by at most 2^tau); on a rescale acc and l are multiplied
    by 2^(m_old - m_new);
  * Sec. IV-B1, Eq. 2: lean P y = 8 (x + sigma + 7) - beta rounded to an integer code,
    or exact P, 2^(x + sigma) rounded to e4m3;
  * Sec. IV-B2: per (row, 64-key block) o = number of whole binades between the block
    maximum and the running maximum, added to x, removed again by 2^-o;
  * Sec. IV-B3: l is the sum of the same rounded probabilities that multiply V;
    O = dv acc / l and LSE = ln 2 (m + log2 l - sigma).

Both implementations must agree bit for bit on o and on every code, and within 1e-12 on
O and the LSE, on small inputs chosen to exercise each decision: stepped block maxima
(o > 0), rows of one wave that disagree on the lazy decision, a sink over a flat tail,
rising logits (many rescales), lean and exact P, mirror and ideal modes.  Two mutated
copies of the naive walk (a per-row lazy decision; tiles not anchored at key 0) must
disagree with the oracle on the inputs built for them, which shows that these cases can
see such mistakes.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import synth

SIGMA = 6
BETA32 = np.float32(0.35)
TAU = np.float32(0.125)
TILE = 128
BLOCK = 64
GROUP = 32
LOG2E = 1.4426950408889634  # nearest double to log2(e)
F32 = np.float32


# ----------------------------------------------------------------------------- e4m3 from its definition
def e4m3_decode(code: int) -> float:
    """Value of an e4m3 (OCP fn) code: sign, 4-bit exponent with bias 7, 3-bit fraction;
    exponent field 0 holds the subnormals f/8 * 2^-6; S.1111.111 is NaN."""
    code = int(code)
    sign = -1.0 if code & 0x80 else 1.0
    e, f = (code >> 3) & 0xF, code & 0x7
    if e == 0xF and f == 0x7:
        return math.nan
    if e == 0:
        return sign * f * 2.0 ** -9
    return sign * (8 + f) * 2.0 ** (e - 10)


_E4M3_CODE_OF = {e4m3_decode(c): c for c in range(0x7F)}  # non-negative codes 0..126


def e4m3_round_positive(p: float) -> int:
    """Code of the e4m3 value nearest to p >= 0 (ties to the even fraction), p below 464.
    Each binade [2^(e-1), 2^e) holds 8 values spaced 2^(e-4) apart; below 2^-6 the
    spacing is 2^-9 (subnormals)."""
    if p == 0.0:
        return 0
    _, e = math.frexp(p)  # p in [2^(e-1), 2^e)
    quantum = 2.0 ** max(e - 4, -9)
    n = round(p / quantum)  # exact quotient; Python rounds halves to even
    return _E4M3_CODE_OF[n * quantum]


def int_values(codes: np.ndarray) -> np.ndarray:
    """e4m3 values times 2^9, as exact integers (448 * 2^9 = 229376)."""
    table = np.array([int(round(e4m3_decode(c) * 512)) if c & 0x7F != 0x7F else 0 for c in range(256)],
                     dtype=np.int64)
    return table[codes]


# ----------------------------------------------------------------------------- fp32 helpers
def f32_nearest(r: Fraction) -> np.float32:
    """The fp32 value nearest to the exact rational r, ties to an even significand."""
    g = F32(float(r))
    cands = [np.nextafter(g, F32(-np.inf)), g, np.nextafter(g, F32(np.inf))]
    return min(cands, key=lambda c: (abs(Fraction(float(c)) - r), int(np.array(c).view(np.uint32)) & 1))


def fmaf(a, b, c) -> np.float32:
    """fp32 fused multiply-add: a b + c computed exactly, rounded once."""
    return f32_nearest(Fraction(float(a)) * Fraction(float(b)) + Fraction(float(c)))


def rne_int(y: float) -> int:
    """Round to the nearest integer, halves to even (Python's round)."""
    return int(round(y))


# ----------------------------------------------------------------------------- the naive walk
def naive_emulate(qc, kc, vc, dq, dk, dv, c, *, exact_p, ideal, mutant=None):
    """Per-row emulation of the FP8 scheme for every row of every (b, h).

    Returns (out [B*H*S, dv] fp64, lse [B*H*S], o [B*H*S, S/64] with 255 for blocks a row
    does not see, codes [B*H*S, S] with 0 for masked keys, rescales)."""
    B, S, H, dqk = qc.shape
    dvd = vc.shape[3]
    nblk = S // BLOCK
    c32 = F32(c)  # the softmax scale crosses the C ABI as an fp32 value
    cp = F32(float(c32) * dq * dk * LOG2E)  # c' = c dq dk log2 e, rounded to fp32
    cp8 = F32(8) * cp
    cp_d = float(c32) * dq * dk * LOG2E     # ideal mode: fp64
    out = np.zeros((B * H * S, dvd))
    lse = np.zeros(B * H * S)
    o_all = np.full((B * H * S, nblk), 255, dtype=np.uint8)
    codes_all = np.zeros((B * H * S, S), dtype=np.uint8)
    rescales = 0
    for b in range(B):
        for h in range(H):
            qi = int_values(qc[b, :, h])
            ki = int_values(kc[b, :, h])
            dots = qi @ ki.T                                  # exact integers, scale 2^18
            vval = np.array([[e4m3_decode(x) for x in row] for row in vc[b, :, h]])
            base = (b * H + h) * S

            def raw(i, j):
                return dots[i, j] / 2.0 ** 18                 # exact double of the exact dot product

            first_tile_key = TILE // 2 if mutant == "tile_offset" else 0
            for r0 in range(0, S, GROUP):
                rows = list(range(r0, min(r0 + GROUP, S)))
                m = {i: None for i in rows}
                l = {i: 0.0 for i in rows}
                acc = {i: np.zeros(dvd) for i in rows}
                if ideal:  # the exact final row maximum, fp64
                    for i in rows:
                        m[i] = max(raw(i, j) * cp_d for j in range(i + 1))
                # tiles of keys [k0, k1), from key 0 (the mutant shifts the tile edges)
                edges = [0] + list(range(first_tile_key or TILE, S, TILE)) + [S]
                for ti in range(len(edges) - 1):
                    k0, k1 = edges[ti], edges[ti + 1]
                    if k0 > rows[-1]:
                        break
                    if not ideal:
                        new_m = {}
                        for i in rows:
                            ts = [F32(raw(i, j)) * cp for j in range(k0, min(k1, i + 1))]
                            cand = ts + ([m[i]] if m[i] is not None else [])
                            new_m[i] = max(cand)
                        if ti == 0:
                            for i in rows:
                                m[i] = new_m[i]
                        else:
                            grows = {i: (new_m[i] - m[i]) >= TAU for i in rows}
                            for i in rows:
                                decide = grows[i] if mutant == "per_row_lazy" else any(grows.values())
                                if decide:
                                    f = 2.0 ** float(m[i] - new_m[i])
                                    acc[i] = acc[i] * f
                                    l[i] = l[i] * f
                                    m[i] = new_m[i]
                            rescales += any(grows.values())
                    # 64-key scale blocks of the tile
                    for kb in range(k0, k1, BLOCK):
                        blk_keys = range(kb, min(kb + BLOCK, k1))
                        for i in rows:
                            vis = [j for j in blk_keys if j <= i]
                            if not vis:
                                continue
                            if ideal:
                                bmax = max(raw(i, j) * cp_d for j in vis)
                                o = min(max(math.floor(m[i] - bmax), 0), 127)
                            else:
                                bmax = max(F32(raw(i, j)) * cp for j in vis)
                                o = int(min(max(np.floor(m[i] - bmax), F32(0)), F32(127)))
                            o_all[base + i, kb // BLOCK] = o
                            block_sum = 0.0
                            block_pv = np.zeros(dvd)
                            for j in vis:
                                if ideal:
                                    x = raw(i, j) * cp_d - m[i] + o
                                    if exact_p:
                                        code = e4m3_round_positive(2.0 ** (x + SIGMA))
                                    else:
                                        y = 8.0 * (x + SIGMA + 7.0) - float(BETA32)
                                        code = min(max(rne_int(y), 0), 255)
                                else:
                                    s32 = F32(raw(i, j))
                                    if exact_p:
                                        x = fmaf(s32, cp, F32(SIGMA + o) - m[i])
                                        code = e4m3_round_positive(2.0 ** float(x))
                                    else:
                                        cst = F32(8) * (F32(SIGMA + 7 + o) - m[i]) - BETA32
                                        y = fmaf(s32, cp8, cst)
                                        code = min(max(rne_int(float(y)), 0), 255)
                                assert code <= 126
                                codes_all[base + i, j] = code
                                p = e4m3_decode(code)
                                block_sum += p
                                block_pv += p * vval[j]
                            l[i] += 2.0 ** -o * block_sum
                            acc[i] += 2.0 ** -o * block_pv
                for i in rows:
                    out[base + i] = dv * acc[i] / l[i]
                    lse[base + i] = math.log(2) * (float(m[i]) + math.log2(l[i]) - SIGMA)
    return out, lse, o_all, codes_all, rescales


def _oracle_all(orc, qc, kc, vc, dq, dk, dv, c, exact_p, ideal):
    B, S, H, _ = qc.shape
    emu = orc.emulate_fp8(qc, kc, vc, dq=dq, dk=dk, dv=dv, c=c,
                          scheme=orc.Fp8Scheme(exact_p=exact_p, ideal=ideal), debug=True)
    # the oracle's groups run (b, h, r0) in that order, the same row order as above
    return emu


CASES = [
    # (generator, d_qk, S, exact_p, ideal)
    ("stepped_max", 128, 512, False, False),
    ("alternating_rows", 128, 512, False, False),
    ("sink_flat_tail", 128, 256, False, False),
    ("rising_logits", 128, 512, False, False),
    ("stepped_max", 128, 256, True, False),
    ("logit_sd_4", 192, 256, True, False),
    ("stepped_max", 128, 256, False, True),
    ("sink_flat_tail", 192, 256, True, True),
]


@pytest.mark.parametrize("gen,dqk,S,exact_p,ideal", CASES)
def test_emulation_matches_naive_reimplementation(orc, gen, dqk, S, exact_p, ideal):
    B, H = 1, 1
    q, k, v = synth.STRESS[gen](B, S, H, dqk, 128, 71)
    (qc, dq), (kc, dk), (vc, dv) = (orc.quantize_e4m3(x) for x in (q, k, v))
    c = 1.0 / math.sqrt(dqk)
    out, lse, o, codes, rescales = naive_emulate(qc, kc, vc, dq, dk, dv, c, exact_p=exact_p, ideal=ideal)
    emu = _oracle_all(orc, qc, kc, vc, dq, dk, dv, c, exact_p, ideal)
    assert np.array_equal(emu["o"], o)
    assert np.array_equal(emu["codes"], codes)
    assert np.max(np.abs(emu["out"] - out)) <= 1e-12
    assert np.max(np.abs(emu["lse"] - lse)) <= 1e-12
    # each case exercises what it was chosen for
    seen = o != 255
    if gen in ("stepped_max", "sink_flat_tail"):
        assert np.any(o[seen] > 0)
    if gen in ("rising_logits", "alternating_rows") and not ideal:
        assert rescales > 0


def test_naive_codec_against_format_definition():
    """The naive codec's own sanity: the worked values of Sec. IV-B1's footnote (codes
    56, 64, 72 for 1, 2, 4; code 60 stands for 1.5), 448 at 0x7E, the smallest subnormal,
    and round-to-nearest-even at a midpoint."""
    assert [e4m3_decode(c) for c in (56, 64, 72, 60)] == [1.0, 2.0, 4.0, 1.5]
    assert e4m3_decode(0x7E) == 448.0 and e4m3_decode(1) == 2.0 ** -9
    assert e4m3_round_positive(1.0625) == 56  # midpoint of 1 and 1.125: even fraction
    assert e4m3_round_positive(1.1875) == 58  # midpoint of 1.125 and 1.25: even fraction
    assert e4m3_round_positive(2.0 ** -10) == 0 and e4m3_round_positive(1.5 * 2.0 ** -10) == 1
    assert fmaf(F32(1 + 2 ** -12), F32(1 + 2 ** -12), F32(-1)) == F32(2 ** -11 + 2 ** -24)


@pytest.mark.parametrize("mutant,gen", [("per_row_lazy", "alternating_rows"), ("tile_offset", "stepped_max")])
def test_mutants_are_seen(orc, mutant, gen):
    """A per-row lazy decision, or 128-key tiles not anchored at key 0, gives other codes
    than the oracle on these inputs: the comparison above would catch either mistake in
    the oracle."""
    B, H, S, dqk = 1, 1, 512, 128
    q, k, v = synth.STRESS[gen](B, S, H, dqk, 128, 71)
    (qc, dq), (kc, dk), (vc, dv) = (orc.quantize_e4m3(x) for x in (q, k, v))
    c = 1.0 / math.sqrt(dqk)
    _, _, o, codes, _ = naive_emulate(qc, kc, vc, dq, dk, dv, c, exact_p=False, ideal=False, mutant=mutant)
    emu = _oracle_all(orc, qc, kc, vc, dq, dk, dv, c, False, False)
    assert not (np.array_equal(emu["codes"], codes) and np.array_equal(emu["o"], o))


@pytest.mark.parametrize("gen,dqk,exact_p", [("stepped_max", 128, False), ("logit_sd_4", 192, True)])
def test_emulation_from_given_scores(orc, gen, dqk, exact_p):
    """The oracle's run from given fp32 scores equals its own run when handed the exact dot
    products rounded once to fp32, which is what its mirror mode does with them (step 1)."""
    B, H, S = 2, 2, 256
    q, k, v = synth.STRESS[gen](B, S, H, dqk, 128, 72)
    (qc, dq), (kc, dk), (vc, dv) = (orc.quantize_e4m3(x) for x in (q, k, v))
    t = orc.e4m3_table()
    sc = np.einsum("bihd,bjhd->bhij", t[qc], t[kc])  # exact: products and sums fit in fp64
    scores = sc.reshape(B * H * S, S).astype(np.float32)
    c = 1.0 / math.sqrt(dqk)
    scheme = orc.Fp8Scheme(exact_p=exact_p)
    a = orc.emulate_fp8(qc, kc, vc, dq=dq, dk=dk, dv=dv, c=c, scheme=scheme, debug=True)
    b = orc.emulate_fp8_from_scores(scores, vc, dq=dq, dk=dk, dv=dv, c=c, scheme=scheme, debug=True)
    for key in ("o", "codes", "out", "lse"):
        assert np.array_equal(a[key], b[key]), key
