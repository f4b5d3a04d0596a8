"""GPU parity at the full benchmark sizes, in the launch configuration bench.py times.

Inputs are generated and quantised exactly as for the benchmark; the GPU quantiser's
codes are compared with the oracle's bit for bit over the whole tensors, and the
attention output is compared on sampled 32-row groups (first rows, last rows and seeded
positions) with the oracle's step-by-step FP8 emulation and with exact fp64 attention,
which it computes row by row.  Each test prints its case before touching the GPU."""
import math

import numpy as np
import pytest
import torch

import bf16_causal_flashattention_amd as cfa
import oracle
import synth
from gpu_util import (DEV, LSE_EMU_NATS, LSE_FP64_NATS, TOL_EMU_MAXABS, TOL_EMU_RMS, TOL_FP64_RMS_BF16,
                      TOL_FP64_RMS_FP8, gpu_rows, lse_rows, rms_rel, sample_groups, snr_db)

pytestmark = pytest.mark.gpu


def _case(*a):
    print("CASE", *a, flush=True)


def _fp8_full(gen, B, H, S, dqk, exact_p, seed, n_groups):
    q, k, v = gen(B, S, H, dqk, 128, seed)
    gpu = []
    for x in (q, k, v):
        c, d = cfa.quantize_e4m3(torch.from_numpy(x).to(DEV))
        gpu.append((c, float(d.item())))
    torch.cuda.synchronize()
    host = [oracle.quantize_e4m3(x) for x in (q, k, v)]
    del q, k, v
    for (gc, gd), (hc, hd) in zip(gpu, host):
        assert gd == hd
        assert np.array_equal(gc.view(torch.uint8).cpu().numpy(), hc)  # a0 bit-exact at full size
    (qg, dq), (kg, dk), (vg, dv) = gpu
    c = 1.0 / math.sqrt(dqk)
    out = torch.full((B, S, H, 128), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((B, H, S), float("nan"), dtype=torch.float32, device=DEV)
    entry = cfa.attn_fwd_causal_fp8 if dqk == 128 else cfa.attn_fwd_causal_mla
    entry(qg, kg, vg, dq, dk, dv, softmax_scale=c, out=out, lse=lse)
    torch.cuda.synchronize()
    assert not torch.isnan(out.float()).any() and not torch.isnan(lse).any()  # every tile written
    groups = sample_groups(B, H, S, n_groups, seed)
    qc, kc, vc = (h[0] for h in host)
    emu = oracle.emulate_fp8(qc, kc, vc, dq=dq, dk=dk, dv=dv, c=c, scheme=oracle.Fp8Scheme(exact_p=exact_p),
                             groups=groups)
    rows = oracle.group_rows(groups, 32)
    ex, ex_lse = oracle.attn_exact(qc, kc, vc, dtype="fp8", c=c, dq=dq, dk=dk, dv=dv, rows=rows)
    got, glse = gpu_rows(out, rows), lse_rows(lse, rows)
    res = {"emu_maxabs": float(np.max(np.abs(got - emu["out"]))), "emu_rms": rms_rel(got, emu["out"]),
           "fp64_rms": rms_rel(got, ex), "fp64_maxabs": float(np.max(np.abs(got - ex))),
           "fp64_snr_db": snr_db(got, ex), "lse_emu": float(np.max(np.abs(glse - emu["lse"]))),
           "lse_fp64": float(np.max(np.abs(glse - ex_lse)))}
    print("RESULT", res, flush=True)
    del out, lse, gpu
    torch.cuda.empty_cache()
    return res


def test_c2_fp8_b1_h32_s32768():
    _case("C2 FP8 B1 H32 S32768 d128 lean P")
    r = _fp8_full(synth.gaussian, 1, 32, 32768, 128, False, 0, 12)
    assert r["emu_maxabs"] <= TOL_EMU_MAXABS and r["emu_rms"] <= TOL_EMU_RMS
    assert r["fp64_rms"] <= TOL_FP64_RMS_FP8
    assert r["lse_emu"] <= LSE_EMU_NATS and r["lse_fp64"] <= LSE_FP64_NATS


def test_c4_mla_b1_h16_s32768():
    _case("C4 MLA FP8 B1 H16 S32768 192/128 exact P")
    r = _fp8_full(synth.gaussian, 1, 16, 32768, 192, True, 1, 12)
    assert r["emu_maxabs"] <= TOL_EMU_MAXABS and r["emu_rms"] <= TOL_EMU_RMS
    assert r["fp64_rms"] <= TOL_FP64_RMS_FP8
    assert r["lse_emu"] <= LSE_EMU_NATS and r["lse_fp64"] <= LSE_FP64_NATS


def test_c5_activation_like_b1_h32_s16384():
    _case("C5 FP8 activation-like B1 H32 S16384 d128")
    r = _fp8_full(synth.activation_like, 1, 32, 16384, 128, False, 2, 12)
    assert r["emu_maxabs"] <= TOL_EMU_MAXABS and r["emu_rms"] <= TOL_EMU_RMS
    assert r["fp64_rms"] <= TOL_FP64_RMS_FP8
    assert r["lse_emu"] <= LSE_EMU_NATS and r["lse_fp64"] <= LSE_FP64_NATS


@pytest.mark.parametrize("S", [4096, 8192, 16384, 32768])
def test_c3_bf16_b1_h32_sweep(S):
    _case("C3 BF16 B1 H32", S)
    B, H = 1, 32
    q, k, v = synth.gaussian(B, S, H, 128, 128, 3)
    gq, gk, gv = (cfa.round_bf16(torch.from_numpy(x).to(DEV)) for x in (q, k, v))
    hq, hk, hv = (oracle.bf16_rne(x) for x in (q, k, v))
    del q, k, v
    for g_, h_ in ((gq, hq), (gk, hk), (gv, hv)):
        assert np.array_equal(g_.view(torch.int16).cpu().numpy().view(np.uint16), h_)
    out = torch.full((B, S, H, 128), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((B, H, S), float("nan"), dtype=torch.float32, device=DEV)
    cfa.attn_fwd_causal_bf16(gq, gk, gv, softmax_scale=1 / math.sqrt(128), out=out, lse=lse)
    torch.cuda.synchronize()
    assert not torch.isnan(out.float()).any() and not torch.isnan(lse).any()
    rows = oracle.group_rows(sample_groups(B, H, S, 8, S), 32)
    ex, ex_lse = oracle.attn_exact(hq, hk, hv, dtype="bf16", c=1 / math.sqrt(128), rows=rows)
    got, glse = gpu_rows(out, rows), lse_rows(lse, rows)
    res = {"fp64_rms": rms_rel(got, ex), "fp64_maxabs": float(np.max(np.abs(got - ex))),
           "fp64_snr_db": snr_db(got, ex), "lse_fp64": float(np.max(np.abs(glse - ex_lse)))}
    print("RESULT", res, flush=True)
    assert res["fp64_rms"] <= TOL_FP64_RMS_BF16 and res["lse_fp64"] <= 1e-3
    del out, lse, gq, gk, gv
    torch.cuda.empty_cache()


def _fp8_ex_full(B, H, Hkv, S, dqk, p_mode, exact_p, seed, n_groups):
    """The general entry point at a bench.py size: q with H heads, k/v with Hkv heads (inputs
    as bench.py makes them); the oracle sees k/v expanded to H heads."""
    q = synth.gaussian(B, S, H, dqk, 128, seed)[0]
    _, k, v = synth.gaussian(B, S, Hkv, dqk, 128, seed + 1)
    gpu = []
    for x in (q, k, v):
        c, d = cfa.quantize_e4m3(torch.from_numpy(x).to(DEV))
        gpu.append((c, float(d.item())))
    torch.cuda.synchronize()
    host = [oracle.quantize_e4m3(x) for x in (q, k, v)]
    del q, k, v
    for (gc, gd), (hc, hd) in zip(gpu, host):
        assert gd == hd
        assert np.array_equal(gc.view(torch.uint8).cpu().numpy(), hc)
    (qg, dq), (kg, dk), (vg, dv) = gpu
    c = 1.0 / math.sqrt(dqk)
    out = torch.full((B, S, H, 128), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((B, H, S), float("nan"), dtype=torch.float32, device=DEV)
    cfa.attn_fwd_causal_fp8_ex(qg, kg, vg, dq, dk, dv, softmax_scale=c, p_mode=p_mode, out=out, lse=lse)
    torch.cuda.synchronize()
    assert not torch.isnan(out.float()).any() and not torch.isnan(lse).any()
    G = H // Hkv
    qc = host[0][0]
    kc, vc = (np.repeat(h[0], G, axis=2) for h in host[1:])
    groups = sample_groups(B, H, S, n_groups, seed)
    emu = oracle.emulate_fp8(qc, kc, vc, dq=dq, dk=dk, dv=dv, c=c, scheme=oracle.Fp8Scheme(exact_p=exact_p),
                             groups=groups)
    rows = oracle.group_rows(groups, 32)
    ex, ex_lse = oracle.attn_exact(qc, kc, vc, dtype="fp8", c=c, dq=dq, dk=dk, dv=dv, rows=rows)
    got, glse = gpu_rows(out, rows), lse_rows(lse, rows)
    res = {"emu_maxabs": float(np.max(np.abs(got - emu["out"]))), "emu_rms": rms_rel(got, emu["out"]),
           "fp64_rms": rms_rel(got, ex), "fp64_maxabs": float(np.max(np.abs(got - ex))),
           "fp64_snr_db": snr_db(got, ex), "lse_emu": float(np.max(np.abs(glse - emu["lse"]))),
           "lse_fp64": float(np.max(np.abs(glse - ex_lse)))}
    print("RESULT", res, flush=True)
    del out, lse, gpu
    torch.cuda.empty_cache()
    assert res["emu_maxabs"] <= TOL_EMU_MAXABS and res["emu_rms"] <= TOL_EMU_RMS, res
    assert res["fp64_rms"] <= TOL_FP64_RMS_FP8, res
    assert res["lse_emu"] <= LSE_EMU_NATS and res["lse_fp64"] <= LSE_FP64_NATS, res


def test_fp8_gqa_b1_h32_hkv8_s32768():
    _case("FP8 GQA B1 H32 Hkv8 S32768 d128 lean P (general entry point)")
    _fp8_ex_full(1, 32, 8, 32768, 128, cfa.P_LEAN, False, 0, 12)


def test_mla_lean_p_b1_h16_s32768():
    _case("FP8 MLA B1 H16 S32768 192/128 lean P (general entry point)")
    _fp8_ex_full(1, 16, 16, 32768, 192, cfa.P_LEAN, False, 0, 12)


def test_bf16_mla_b1_h16_s32768():
    _case("BF16 MLA B1 H16 S32768 192/128 (general entry point)")
    B, H, S = 1, 16, 32768
    q, k, v = synth.gaussian(B, S, H, 192, 128, 4)
    gq, gk, gv = (cfa.round_bf16(torch.from_numpy(np.ascontiguousarray(x)).to(DEV)) for x in (q, k, v))
    hq, hk, hv = (oracle.bf16_rne(x) for x in (q, k, v))
    del q, k, v
    c = 1 / math.sqrt(192)
    out, lse = cfa.attn_fwd_causal_bf16_ex(gq, gk, gv, softmax_scale=c)
    torch.cuda.synchronize()
    assert not torch.isnan(out.float()).any() and not torch.isnan(lse).any()
    rows = oracle.group_rows(sample_groups(B, H, S, 12, 4), 32)
    ex, ex_lse = oracle.attn_exact(hq, hk, hv, dtype="bf16", c=c, rows=rows)
    got, glse = gpu_rows(out, rows), lse_rows(lse, rows)
    res = {"fp64_rms": rms_rel(got, ex), "fp64_maxabs": float(np.max(np.abs(got - ex))),
           "fp64_snr_db": snr_db(got, ex), "lse_fp64": float(np.max(np.abs(glse - ex_lse)))}
    print("RESULT", res, flush=True)
    assert res["fp64_rms"] <= TOL_FP64_RMS_BF16, res
    assert res["lse_fp64"] <= 1e-3 + 1e-6 * np.max(np.abs(ex_lse)), res
