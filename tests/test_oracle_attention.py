"""Pins for the exact fp64 attention oracle and the FP8-scheme emulation.

Exact attention (paper Sec. II-B) is pinned against mpmath brute force, torch's CPU
float64 scaled_dot_product_attention, and closed forms.  The emulation (paper
Sec. IV-A, IV-B) is pinned against closed forms (identical keys -> causal prefix
mean; one dominant key -> its value row), invariants (rounded weights sum to one,
convex hull) and the paper's bounds (LSE within 0.04 nats; stale max bound)."""
import math

import mpmath
import numpy as np
import pytest
import torch

import synth


def _quant(orc, q, k, v):
    qc, dq = orc.quantize_e4m3(q)
    kc, dk = orc.quantize_e4m3(k)
    vc, dv = orc.quantize_e4m3(v)
    return qc, kc, vc, dq, dk, dv


def _bf16(orc, *xs):
    return [orc.bf16_rne(x) for x in xs]


# ----------------------------------------------------------------------------- exact
@pytest.mark.parametrize("dtype", ["fp8", "bf16"])
def test_exact_vs_mpmath(orc, dtype):
    B, S, H, d = 1, 10, 2, 8
    q, k, v = synth.gaussian(B, S, H, d, d, seed=3)
    c = 1 / math.sqrt(d)
    if dtype == "fp8":
        qc, kc, vc, dq, dk, dvs = _quant(orc, q, k, v)
        t = orc.e4m3_table()
        Q, K, V = t[qc] * dq, t[kc] * dk, t[vc] * dvs
        out, lse = orc.attn_exact(qc, kc, vc, dtype="fp8", c=c, dq=dq, dk=dk, dv=dvs)
    else:
        qb, kb, vb = _bf16(orc, q, k, v)
        Q, K, V = orc.bf16_value(qb), orc.bf16_value(kb), orc.bf16_value(vb)
        out, lse = orc.attn_exact(qb, kb, vb, dtype="bf16", c=c)
    mpmath.mp.dps = 40
    n = 0
    for h in range(H):
        for i in range(S):
            sc = [mpmath.mpf(c) * mpmath.fsum(mpmath.mpf(Q[0, i, h, e]) * mpmath.mpf(K[0, j, h, e]) for e in range(d))
                  for j in range(i + 1)]
            w = [mpmath.exp(s) for s in sc]
            den = mpmath.fsum(w)
            for e in range(d):
                num = mpmath.fsum(w[j] * mpmath.mpf(V[0, j, h, e]) for j in range(i + 1))
                assert abs(float(num / den) - out[n, e]) < 1e-12
            assert abs(float(mpmath.log(den)) - lse[n]) < 1e-12
            n += 1


def test_exact_vs_torch_sdpa(orc):
    B, S, H, d = 2, 96, 3, 128
    q, k, v = synth.gaussian(B, S, H, d, d, seed=4)
    qb, kb, vb = _bf16(orc, q, k, v)
    c = 1 / math.sqrt(d)
    out, lse = orc.attn_exact(qb, kb, vb, dtype="bf16", c=c)
    tq, tk, tv = (torch.from_numpy(orc.bf16_value(x)).permute(0, 2, 1, 3) for x in (qb, kb, vb))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=c)
    ref = ref.permute(0, 2, 1, 3).reshape(-1, d)  # (b, s, h) order
    # oracle rows are ordered (b, h, i)
    o = out.reshape(B, H, S, d).transpose(0, 2, 1, 3).reshape(-1, d)
    assert np.max(np.abs(o - ref.numpy())) < 1e-12
    sc = (tq @ tk.transpose(-1, -2)) * c
    sc = sc.masked_fill(torch.triu(torch.ones(S, S, dtype=torch.bool), 1), float("-inf"))
    assert np.max(np.abs(lse - torch.logsumexp(sc, -1).reshape(-1).numpy())) < 1e-12


def test_exact_closed_forms(orc):
    B, S, H, d = 1, 64, 2, 16
    q, k, v = synth.identical_keys(B, S, H, d, d, seed=5)
    qb, kb, vb = _bf16(orc, q, k, v)
    out, lse = orc.attn_exact(qb, kb, vb, dtype="bf16", c=0.25)
    V = orc.bf16_value(vb)
    pref = np.cumsum(V, axis=1) / np.arange(1, S + 1)[None, :, None, None]
    o = out.reshape(B, H, S, d).transpose(0, 2, 1, 3)
    assert np.max(np.abs(o - pref)) < 1e-13
    # row 0 sees only key 0
    Q, K = orc.bf16_value(qb), orc.bf16_value(kb)
    for h in range(H):
        assert np.allclose(o[0, 0, h], V[0, 0, h], atol=0)
        assert abs(lse[h * S] - 0.25 * float(Q[0, 0, h] @ K[0, 0, h])) < 1e-12


def test_exact_rejects_bad_rows(orc):
    q = np.zeros((1, 4, 1, 8), dtype=np.uint16)
    with pytest.raises(ValueError):
        orc.attn_exact(q, q, q, dtype="bf16", c=1.0, rows=np.array([[0, 0, 4]]))


# ----------------------------------------------------------------------------- emulation
def _emu(orc, q, k, v, exact_p=False, **kw):
    qc, kc, vc, dq, dk, dv = _quant(orc, q, k, v)
    d = q.shape[3]
    scheme = orc.Fp8Scheme(exact_p=exact_p, **kw)
    r = orc.emulate_fp8(qc, kc, vc, dq=dq, dk=dk, dv=dv, c=1 / math.sqrt(d), scheme=scheme, debug=True)
    return r, (qc, kc, vc, dq, dk, dv)


def _rows_bhi(res, group):
    import oracle
    return oracle.group_rows(res["groups"], group)


@pytest.mark.parametrize("exact_p", [False, True])
@pytest.mark.parametrize("ideal", [False, True])
def test_emulation_identical_keys_prefix_mean(orc, exact_p, ideal):
    B, S, H, d = 1, 320, 1, 128
    q, k, v = synth.identical_keys(B, S, H, d, d, seed=6)
    r, (qc, kc, vc, dq, dk, dv) = _emu(orc, q, k, v, exact_p=exact_p, ideal=ideal)
    codes = r["codes"]
    mask = np.tril(np.ones((S, S), dtype=bool))
    assert np.all(codes[mask] == 104) and np.all(codes[~mask] == 0)
    V = orc.e4m3_table()[vc][0, :, 0] * dv
    pref = np.cumsum(V, axis=0) / np.arange(1, S + 1)[:, None]
    assert np.max(np.abs(r["out"] - pref)) < 1e-12
    # an off-by-one mask would move row i by (v_{i+1} - mean)/(i+2): far above this bound
    shifted = (np.cumsum(V, axis=0)[1:] / np.arange(2, S + 1)[:, None])
    assert np.min(np.max(np.abs(shifted[:8] - pref[:8]), axis=1)) > 1e-3


@pytest.mark.parametrize("exact_p", [False, True])
def test_emulation_one_hot(orc, exact_p):
    B, S, H, d = 1, 256, 2, 128
    q, k, v = synth.one_hot_key(B, S, H, d, d, seed=7, key=0, lift=60.0)
    r, (qc, kc, vc, dq, dk, dv) = _emu(orc, q, k, v, exact_p=exact_p)
    V0 = orc.e4m3_table()[vc][0, 0] * dv  # [H, d]
    rows = _rows_bhi(r, 32)
    want = V0[rows[:, 1]]
    assert np.array_equal(r["out"], want)


@pytest.mark.parametrize("name", ["logit_sd_1", "logit_sd_4", "four_key_sink", "sink_flat_tail", "full_range"])
def test_emulation_weights_sum_to_one(orc, name):
    B, S, H, d = 1, 512, 1, 128
    q, k, v = synth.STRESS[name](B, S, H, d, d, 8)
    v[:] = 1.0
    r, _ = _emu(orc, q, k, v)
    assert np.max(np.abs(r["out"] - 1.0)) < 1e-12
    # the unrounded row sum (as in a kernel that divides by the unrounded sum) shrinks rows
    r2, _ = _emu(orc, q, k, v, rounded_sum=False)
    assert np.max(np.abs(r2["out"] - 1.0)) > 1e-4


def test_emulation_convex_hull(orc):
    B, S, H, d = 1, 384, 2, 128
    q, k, v = synth.logit_sd(B, S, H, d, d, 9, sd=16)
    r, (qc, kc, vc, dq, dk, dv) = _emu(orc, q, k, v)
    V = orc.e4m3_table()[vc] * dv
    rows = _rows_bhi(r, 32)
    for n, (b, h, i) in enumerate(rows):
        vis = V[b, : i + 1, h]
        assert np.all(r["out"][n] >= vis.min(0) - 1e-12) and np.all(r["out"][n] <= vis.max(0) + 1e-12)


@pytest.mark.parametrize("exact_p", [False, True])
@pytest.mark.parametrize("name", ["logit_sd_1", "logit_sd_4", "stepped_max", "rising_logits", "sink_flat_tail"])
def test_emulation_close_to_fp64(orc, golden_bounds, exact_p, name):
    B, S, H, d = 1, 1024, 1, 128
    q, k, v = synth.STRESS[name](B, S, H, d, d, 10)
    r, (qc, kc, vc, dq, dk, dv) = _emu(orc, q, k, v, exact_p=exact_p)
    rows = _rows_bhi(r, 32)
    ex, lse = orc.attn_exact(qc, kc, vc, dtype="fp8", c=1 / math.sqrt(d), dq=dq, dk=dk, dv=dv, rows=rows)
    rel = np.linalg.norm(r["out"] - ex) / np.linalg.norm(ex)
    assert rel < 6e-2, rel
    assert np.max(np.abs(r["lse"] - lse)) <= golden_bounds["leanp_lse_worst_nats"]


def test_stale_max_codes_bounded(orc, golden_bounds):
    # footnote 9: a stale maximum lets p exceed 1 (here 2^sigma) by less than 2^tau
    B, S, H, d = 1, 1024, 1, 128
    q, k, v = synth.stepped_max(B, S, H, d, d, 11, step=0.06)
    r, _ = _emu(orc, q, k, v)
    assert r["codes"].max() <= 105
    r2, _ = _emu(orc, q, k, v, tau=0.0)
    assert r2["codes"].max() <= 104


def test_block_scaling_reduces_error(orc):
    # Fig. 5: without per-block scaling most of a long flat tail underflows, and dividing by
    # the unrounded sum turns the lost mass into shrinkage; scaling + rounded sum avoids both
    B, S, H, d = 1, 2048, 1, 128
    q, k, v = synth.sink_flat_tail(B, S, H, d, d, 12)
    v += np.float32(2.0)  # dropped keys then carry value mass that shrinkage loses
    res = {}
    for tag, kw in {"zyfa": {}, "noscale": {"scale_blocks": False},
                    "noscale_unrounded": {"scale_blocks": False, "rounded_sum": False}}.items():
        r, (qc, kc, vc, dq, dk, dv) = _emu(orc, q, k, v, ideal=True, **kw)
        rows = _rows_bhi(r, 32)
        ex, _ = orc.attn_exact(qc, kc, vc, dtype="fp8", c=1 / math.sqrt(d), dq=dq, dk=dk, dv=dv, rows=rows)
        res[tag] = np.linalg.norm(r["out"] - ex) / np.linalg.norm(ex)
    assert res["noscale"] > 2 * res["zyfa"], res
    assert res["noscale_unrounded"] > 2 * res["zyfa"], res


def test_mirror_and_ideal_agree_roughly(orc):
    B, S, H, d = 1, 1024, 1, 128
    q, k, v = synth.gaussian(B, S, H, d, d, 13)
    r1, _ = _emu(orc, q, k, v)
    r2, _ = _emu(orc, q, k, v, ideal=True)
    rel = np.linalg.norm(r1["out"] - r2["out"]) / np.linalg.norm(r2["out"])
    assert 0 < rel < 3e-2
