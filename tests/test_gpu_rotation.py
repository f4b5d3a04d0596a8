"""GPU parity of the quantisation pre-pass with rotation and K smoothing ("ZYFA: Speed and
Accuracy of FP8 FlashAttention on AMD CDNA4", Sec. V-E, "Rotation and K smoothing").

  * key mean: the library's fp64-accumulated mean against the oracle's fp64 mean, to the
    fp32 rounding of the result (identical keys: exactly);
  * rotate + quantise: the per-tensor descale equal to the oracle's; every code equal to
    the oracle's fp64 rounding except where the fp64 value lies within the fp32
    transform's error of a rounding midpoint (there either neighbour is correct);
  * end to end: attention on the rotated codes against the oracle's emulation on the
    oracle's own rotated codes (the usual element-wise gates), and against exact fp64
    attention of the BF16-rounded original inputs, where the rotated path must have well
    under the error of plain quantisation on inputs with outlier channels shared by q
    and k, a per-head key offset, and a logit spread of a few nats.
Each test prints its case before touching the GPU."""
import math

import numpy as np
import pytest
import torch

import bf16_causal_flashattention_amd as cfa
import oracle
import synth
from gpu_util import (DEV, LSE_EMU_NATS, LSE_FP64_NATS, TOL_EMU_MAXABS, TOL_EMU_RMS, TOL_FP64_RMS_FP8, all_groups,
                      gpu_rows, lse_rows, rms_rel)

pytestmark = pytest.mark.gpu


def _case(*a):
    print("CASE", *a, flush=True)


def _signs(D, seed):
    return np.where(np.random.default_rng(seed).integers(0, 2, D) == 1, 1.0, -1.0)


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV)


def _inputs(B, S, H, D, seed):
    return synth.activation_like(B, S, H, D, 128, seed, outlier_gain=20.0, sink_sigmas=2.0, key_bias=8.0)


@pytest.mark.parametrize("B,S,H,D", [(2, 300, 3, 128), (1, 1, 2, 192), (1, 4096, 4, 128), (2, 1000, 2, 192)])
def test_key_mean(B, S, H, D):
    _case("key_mean", B, S, H, D)
    _, k, _ = _inputs(B, S, H, D, 3 * S + D)
    g = cfa.key_mean(_dev(k)).cpu().numpy().astype(np.float64)
    torch.cuda.synchronize()
    m = oracle.key_mean(k)
    # fp32 rounding of the fp64 mean (half an ulp) plus the fp64 summation error
    tol = np.abs(m) * 2.0 ** -24 + S * 2.0 ** -52 * np.abs(k).mean(axis=1)
    assert np.all(np.abs(g - m) <= tol), float(np.max(np.abs(g - m) - tol))


def test_key_mean_identical_keys_exact():
    B, S, H, D = 1, 777, 2, 128
    _case("key_mean identical", B, S, H, D)
    _, k, _ = synth.identical_keys(B, S, H, D, 128, 8)
    g = cfa.key_mean(_dev(k)).cpu().numpy()
    assert np.array_equal(g, k[:, 0])


def _check_codes(codes_g, ds_g, x, signs, mean64, static=False):
    """GPU codes against the oracle's fp64 rotation + quantiser (per-call scale, or the
    static descale ds_g)."""
    y = oracle.rotate(x, signs, mean64)
    if static:
        oc, od = oracle.quantize_e4m3_static(y, ds_g), ds_g
    else:
        oc, od = oracle.quantize_e4m3_f64(y)
    assert ds_g == od, (ds_g, od)
    g = codes_g.view(torch.uint8).cpu().numpy()
    diff = g != oc
    n_diff = int(diff.sum())
    if n_diff:
        t = oracle.e4m3_table()
        ys = (y / od)[diff]                      # the value being rounded, in code units
        a, b = t[g[diff]], t[oc[diff]]
        lo, hi = np.minimum(a, b), np.maximum(a, b)
        assert np.all((lo <= ys) & (ys <= hi)), "a code is not a neighbour of the exact value"
        # the fp32 transform is good to a few ulps of the row's 2-norm
        xc = np.asarray(x, np.float64) - (mean64[:, None] if mean64 is not None else 0.0)
        row = np.linalg.norm(xc, axis=3, keepdims=True) * np.ones_like(xc)
        tol = 2.0 ** -18 * row[diff] / od
        assert np.all(np.abs(ys - (a + b) / 2) <= tol), "a code differs away from a rounding midpoint"
    print("RESULT", {"n": g.size, "codes_off_by_one": n_diff}, flush=True)
    assert n_diff <= max(2, g.size // 1000)
    return g


@pytest.mark.parametrize("B,S,H,D,smooth", [(2, 301, 3, 128, True), (2, 303, 3, 192, True),
                                            (1, 512, 2, 128, False), (1, 777, 2, 192, False),
                                            (1, 4096, 8, 128, True), (1, 2048, 4, 192, True),
                                            (1, 42, 2050, 128, True)])
def test_rotate_quantize(B, S, H, D, smooth):
    """S not a multiple of the 4 positions a wave takes at a time; more than 2048 heads
    (waves move from head to head and reload the mean)."""
    _case("rotate_quantize", B, S, H, D, smooth)
    q, k, _ = _inputs(B, S, H, D, 5 * S + D + smooth)
    s = _signs(D, S + D)
    sg = _dev(s)
    for name, x in (("q", q), ("k", k)):
        xg = _dev(x)
        mg = cfa.key_mean(xg) if smooth else None
        codes, ds = cfa.rotate_quantize_e4m3(xg, sg, mg)
        torch.cuda.synchronize()
        print("tensor", name, flush=True)
        _check_codes(codes, float(ds.item()), x, s, oracle.key_mean(x) if smooth else None)


@pytest.mark.parametrize("B,S,H,D,smooth", [(2, 300, 3, 128, True), (1, 777, 2, 192, False),
                                            (1, 2048, 4, 192, True)])
def test_rotate_quantize_static(B, S, H, D, smooth):
    """The one-pass static-scale form: at the per-call descale it must give the per-call
    codes bit for bit (same transform, same rounding); at a quarter of it the largest
    values saturate, checked against the oracle's static quantiser."""
    _case("rotate_quantize_static", B, S, H, D, smooth)
    _, k, _ = _inputs(B, S, H, D, 9 * S + D)
    s = _signs(D, 2 * S + D)
    sg, kg = _dev(s), _dev(k)
    mg = cfa.key_mean(kg) if smooth else None
    c_call, d_call = cfa.rotate_quantize_e4m3(kg, sg, mg)
    d_call = float(d_call.item())
    c_static = cfa.rotate_quantize_e4m3_static(kg, sg, d_call, mg)
    c_sat = cfa.rotate_quantize_e4m3_static(kg, sg, d_call / 4, mg)
    torch.cuda.synchronize()
    assert torch.equal(c_call.view(torch.uint8), c_static.view(torch.uint8))
    g = _check_codes(c_sat, d_call / 4, k, s, oracle.key_mean(k) if smooth else None, static=True)
    n_sat = int(np.sum((g & 0x7F) == 0x7E))
    print("RESULT", {"saturated": n_sat}, flush=True)
    assert n_sat > 0


@pytest.mark.parametrize("n", [4096 * 33, 1001])
def test_quantize_static(n):
    """Plain static-scale quantiser: bit-exact against the oracle (the scaling by a power of
    two is exact, the rounding is RNE), with and without saturation, ragged n."""
    _case("quantize_static", n)
    x = (np.random.default_rng(n).standard_normal(n) * 3).astype(np.float32)
    _, d = oracle.quantize_e4m3(x)
    xg = _dev(x)
    for ds in (d, d / 8, d * 2):
        got = cfa.quantize_e4m3_static(xg, ds).view(torch.uint8).cpu().numpy()
        assert np.array_equal(got, oracle.quantize_e4m3_static(x, ds)), ds


def test_rotate_quantize_degenerate():
    D = 192
    sg = _dev(_signs(D, 1))
    _case("rotate_quantize empty", D)
    codes, ds = cfa.rotate_quantize_e4m3(torch.empty((1, 0, 2, D), dtype=torch.float32, device=DEV), sg)
    torch.cuda.synchronize()
    assert codes.numel() == 0 and float(ds.item()) == 1.0
    _case("rotate_quantize no batch", D)
    codes, ds = cfa.rotate_quantize_e4m3(torch.empty((0, 256, 2, D), dtype=torch.float32, device=DEV), sg)
    torch.cuda.synchronize()
    assert codes.numel() == 0 and float(ds.item()) == 1.0
    _case("rotate_quantize zeros", D)
    codes, ds = cfa.rotate_quantize_e4m3(torch.zeros((1, 64, 2, D), dtype=torch.float32, device=DEV), sg)
    torch.cuda.synchronize()
    assert float(ds.item()) == 1.0 and not codes.view(torch.uint8).any()
    _case("rotate_quantize identical keys smoothed", D)
    _, k, _ = synth.identical_keys(1, 300, 2, D, 128, 4)
    kg = _dev(k)
    codes, ds = cfa.rotate_quantize_e4m3(kg, sg, cfa.key_mean(kg))
    torch.cuda.synchronize()
    assert float(ds.item()) == 1.0 and not codes.view(torch.uint8).any()


@pytest.mark.parametrize("D", [128, 192])
def test_rotated_attention_end_to_end(D):
    B, S, H = 1, 1024, 2
    _case("rotated attention", B, S, H, D)
    q, k, v = _inputs(B, S, H, D, 41)
    c = 2.5 / synth.activation_sigma_raw(D)  # raw logits with a spread of a few nats
    s = _signs(D, D)
    entry = cfa.attn_fwd_causal_fp8 if D == 128 else cfa.attn_fwd_causal_mla
    exact_p = D == 192
    qg, kg, vg, sg = _dev(q), _dev(k), _dev(v), _dev(s)
    qr, dq = cfa.rotate_quantize_e4m3(qg, sg)
    kr, dk = cfa.rotate_quantize_e4m3(kg, sg, cfa.key_mean(kg))
    vc_g, dv = cfa.quantize_e4m3(vg)
    dq, dk, dv = float(dq.item()), float(dk.item()), float(dv.item())
    out, lse = entry(qr, kr, vc_g, dq, dk, dv, softmax_scale=c)
    (qp, dqp), (kp, dkp) = cfa.quantize_e4m3(qg), cfa.quantize_e4m3(kg)
    out_p, lse_p = entry(qp, kp, vc_g, float(dqp.item()), float(dkp.item()), dv, softmax_scale=c)
    torch.cuda.synchronize()

    mu = oracle.key_mean(k)
    qc, dq_o = oracle.rotate_quantize_e4m3(q, s)
    kc, dk_o = oracle.rotate_quantize_e4m3(k, s, mu)
    vc, dv_o = oracle.quantize_e4m3(v)
    assert (dq, dk, dv) == (dq_o, dk_o, dv_o)
    scheme = oracle.Fp8Scheme(exact_p=exact_p)
    groups = all_groups(B, H, S)
    rows = oracle.group_rows(groups, scheme.group)
    emu = oracle.emulate_fp8(qc, kc, vc, dq=dq, dk=dk, dv=dv, c=c, scheme=scheme, groups=groups)
    ex, ex_lse = oracle.attn_exact(qc, kc, vc, dtype="fp8", c=c, dq=dq, dk=dk, dv=dv, rows=rows)
    ref, ref_lse = oracle.attn_exact(oracle.bf16_rne(q), oracle.bf16_rne(k), oracle.bf16_rne(v), dtype="bf16", c=c,
                                     rows=rows)
    got, glse = gpu_rows(out, rows), lse_rows(lse, rows)
    got_p, glse_p = gpu_rows(out_p, rows), lse_rows(lse_p, rows)
    # K smoothing lowers every score of row i by c q_i.mu, and the LSE with them
    shift = c * np.einsum("rd,rd->r", q[rows[:, 0], rows[:, 2], rows[:, 1]].astype(np.float64),
                          mu[rows[:, 0], rows[:, 1]])
    e_lse, e_lse_p = glse + shift - ref_lse, glse_p - ref_lse
    res = {"emu_maxabs": float(np.max(np.abs(got - emu["out"]))), "emu_rms": rms_rel(got, emu["out"]),
           "fp64_rms": rms_rel(got, ex), "lse_emu": float(np.max(np.abs(glse - emu["lse"]))),
           "lse_fp64": float(np.max(np.abs(glse - ex_lse))),
           "orig_rms_rotated": rms_rel(got, ref), "orig_rms_plain": rms_rel(got_p, ref),
           "orig_lse_rms_rotated": float(np.sqrt(np.mean(e_lse ** 2))),
           "orig_lse_rms_plain": float(np.sqrt(np.mean(e_lse_p ** 2))),
           "orig_lse_max_rotated": float(np.max(np.abs(e_lse)))}
    print("RESULT", res, flush=True)
    # the attention kernel on rotated codes: the usual gates against the oracle
    assert res["emu_maxabs"] <= TOL_EMU_MAXABS and res["emu_rms"] <= TOL_EMU_RMS, res
    assert res["fp64_rms"] <= TOL_FP64_RMS_FP8, res
    assert res["lse_emu"] <= LSE_EMU_NATS and res["lse_fp64"] <= LSE_FP64_NATS, res
    # the pre-pass: output and LSE error against the original inputs (the oracle's own
    # emulation gives 0.037 vs 0.095-0.115 for the output, 0.03 vs 0.13 nats for the LSE)
    assert res["orig_rms_rotated"] <= 0.5 * res["orig_rms_plain"], res
    assert res["orig_lse_rms_rotated"] <= 0.5 * res["orig_lse_rms_plain"], res
    assert res["orig_lse_max_rotated"] <= 0.3, res
