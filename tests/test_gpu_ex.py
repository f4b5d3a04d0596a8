"""GPU parity of the general entry points: grouped-query attention (H query heads over
H_kv key/value heads, paper Table VI), strided layouts (BHSD, BSHD with padded heads),
and the FP8 probability mode at both head dimensions (lean P at d_qk = 192 and exact P
at 128, paper Sec. IV-B1 and the MLA ablation of Sec. VI-A).

Two kinds of check per case:
  * against the oracle, with k/v expanded to H heads on the host (query head h reads
    key/value head h // (H / H_kv)) and the tensors brought back to dense BSHD;
  * bit for bit against the basic BSHD entry point run on dense copies with the key/value
    heads expanded: only the addressing differs, so the outputs must be identical.
Each test prints its case before touching the GPU."""
import math

import numpy as np
import pytest
import torch

import bf16_causal_flashattention_amd as cfa
import oracle
import synth
from gpu_util import (DEV, LSE_EMU_NATS, LSE_FP64_NATS, TOL_EMU_MAXABS, TOL_EMU_RMS, TOL_FP64_RMS_BF16,
                      TOL_FP64_RMS_FP8, all_groups, check_fp8_on_gpu_scores, gpu_rows, lse_rows, rms_rel)

pytestmark = pytest.mark.gpu


def _case(*a):
    print("CASE", *a, flush=True)


def _relayout(x, layout):
    """A BSHD-shaped view of a copy of x (dense BSHD GPU tensor) stored in `layout`."""
    if layout == "bshd":
        return x.clone()
    if layout == "bhsd":
        return x.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    if layout == "padded":  # BSHD with two spare heads per row
        B, S, H, d = x.shape
        buf = torch.zeros((B, S, H + 2, d), dtype=x.dtype, device=x.device)
        buf[:, :, 1:H + 1] = x
        return buf[:, :, 1:H + 1]
    raise ValueError(layout)


def _out_like(B, S, H, layout):
    o = torch.full((B, S, H, 128), float("nan"), dtype=torch.bfloat16, device=DEV)
    return _relayout(o, layout)


def _assert_spare_heads_untouched(out, layout):
    """With the padded layout, the kernel must not write the spare heads around the view."""
    if layout == "padded":
        base = out._base
        assert base is not None and base.shape[2] == out.shape[2] + 2
        assert not base[:, :, 0].view(torch.int16).any() and not base[:, :, -1].view(torch.int16).any()


def _inputs(B, H, Hkv, S, dqk, seed):
    q = synth.gaussian(B, S, H, dqk, 128, seed)[0]
    _, k, v = synth.gaussian(B, S, Hkv, dqk, 128, seed + 1)
    return q, k, v


def _expand_heads_gpu(t, G):
    return t.repeat_interleave(G, dim=2).contiguous()


@pytest.mark.parametrize("B,H,Hkv,S,dqk,p_mode,layout", [
    (2, 4, 2, 768, 128, None, "bshd"),      # GQA G=2, odd tile count
    (1, 8, 1, 512, 128, None, "bhsd"),      # MQA G=8, BHSD
    (1, 4, 4, 1024, 128, None, "padded"),   # MHA, padded head stride
    (2, 4, 2, 512, 192, None, "bhsd"),      # MLA shape, exact P, GQA
    (1, 2, 2, 1024, 128, cfa.P_EXACT, "bshd"),
    (1, 2, 1, 768, 192, cfa.P_LEAN, "bhsd"),
])
def test_fp8_ex(B, H, Hkv, S, dqk, p_mode, layout):
    _case("fp8_ex", B, H, Hkv, S, dqk, p_mode, layout)
    G = H // Hkv
    q, k, v = _inputs(B, H, Hkv, S, dqk, seed=7 * S + H + dqk)
    gq = [cfa.quantize_e4m3(torch.from_numpy(x).to(DEV)) for x in (q, k, v)]
    # codes handled as uint8 (the binding accepts them; float8 tensors lack some copy kernels)
    (qg, dq), (kg, dk), (vg, dv) = [(c.view(torch.uint8), float(d.item())) for c, d in gq]
    (qc, dq_o), (kc, dk_o), (vc, dv_o) = [oracle.quantize_e4m3(x) for x in (q, k, v)]
    assert (dq, dk, dv) == (dq_o, dk_o, dv_o)
    c = 1.0 / math.sqrt(dqk)
    qL, kL, vL = (_relayout(t, layout) for t in (qg, kg, vg))
    out = _out_like(B, S, H, layout)
    lse = torch.full((B, H, S), float("nan"), dtype=torch.float32, device=DEV)
    cfa.attn_fwd_causal_fp8_ex(qL, kL, vL, dq, dk, dv, softmax_scale=c, p_mode=p_mode, out=out, lse=lse)
    torch.cuda.synchronize()
    assert not torch.isnan(out.float()).any() and not torch.isnan(lse).any()
    _assert_spare_heads_untouched(out, layout)

    # bit-exact against the dense MHA path on expanded heads (same P mode)
    exact_p = (p_mode == cfa.P_EXACT) or (p_mode is None and dqk == 192)
    ref_out = torch.empty((B, S, H, 128), dtype=torch.bfloat16, device=DEV)
    ref_lse = torch.empty((B, H, S), dtype=torch.float32, device=DEV)
    kE, vE = _expand_heads_gpu(kg, G), _expand_heads_gpu(vg, G)
    cfa.attn_fwd_causal_fp8_ex(qg.contiguous(), kE, vE, dq, dk, dv, softmax_scale=c,
                               p_mode=cfa.P_EXACT if exact_p else cfa.P_LEAN, out=ref_out, lse=ref_lse)
    torch.cuda.synchronize()
    assert torch.equal(out.contiguous().view(torch.int16), ref_out.view(torch.int16))
    assert torch.equal(lse, ref_lse)

    _check_fp8_oracle(out.contiguous(), lse, qc, kc, vc, G, dq, dk, dv, c, exact_p, B, H, S)


def _check_fp8_oracle(out, lse, qc, kc, vc, G, dq, dk, dv, c, exact_p, B, H, S, strict=True):
    """out (BSHD) and lse against the oracle, with k/v codes expanded to H heads.  strict adds
    the element-wise max-abs gate against the emulation (see test_fp8_vt for when it is not a
    bound)."""
    kcE, vcE = np.repeat(kc, G, axis=2), np.repeat(vc, G, axis=2)
    scheme = oracle.Fp8Scheme(exact_p=exact_p)
    groups = all_groups(B, H, S)
    emu = oracle.emulate_fp8(qc, kcE, vcE, dq=dq, dk=dk, dv=dv, c=c, scheme=scheme, groups=groups)
    rows = oracle.group_rows(groups, scheme.group)
    ex, ex_lse = oracle.attn_exact(qc, kcE, vcE, dtype="fp8", c=c, dq=dq, dk=dk, dv=dv, rows=rows)
    got, glse = gpu_rows(out.contiguous(), rows), lse_rows(lse, rows)
    res = {"emu_maxabs": float(np.max(np.abs(got - emu["out"]))), "emu_rms": rms_rel(got, emu["out"]),
           "fp64_rms": rms_rel(got, ex), "lse_emu": float(np.max(np.abs(glse - emu["lse"]))),
           "lse_fp64": float(np.max(np.abs(glse - ex_lse)))}
    print("RESULT", res, flush=True)
    assert res["emu_maxabs"] <= TOL_EMU_MAXABS or not strict, res
    assert res["emu_rms"] <= TOL_EMU_RMS, res
    assert res["fp64_rms"] <= TOL_FP64_RMS_FP8, res
    assert res["lse_emu"] <= LSE_EMU_NATS and res["lse_fp64"] <= LSE_FP64_NATS, res


def _channel_major(vg, padded):
    """[B, H_kv, 128, S] view of the key-major codes vg [B, S, H_kv, 128] (uint8); with
    padded, each channel row sits in a row of S + 256 bytes, 128 bytes in."""
    vt = vg.permute(0, 2, 3, 1).contiguous()
    if not padded:
        return vt
    B, Hkv, d, S = vt.shape
    buf = torch.zeros((B, Hkv, d, S + 256), dtype=torch.uint8, device=DEV)
    buf[..., 128:128 + S] = vt
    return buf[..., 128:128 + S]


@pytest.mark.parametrize("B,H,Hkv,S,dqk,p_mode,padded", [
    (2, 4, 2, 768, 128, None, False),      # GQA G=2, odd tile count
    (1, 4, 4, 1024, 128, None, True),      # MHA, padded channel rows
    (2, 4, 2, 512, 192, None, True),       # MLA shape, exact P
    (1, 2, 2, 1024, 128, cfa.P_EXACT, False),
    (1, 2, 1, 768, 192, cfa.P_LEAN, False),
    (1, 1, 1, 256, 128, None, False),      # a single tile
])
def test_fp8_vt(B, H, Hkv, S, dqk, p_mode, padded):
    """Channel-major V: identical bit for bit to the key-major entry point, within the
    oracle's RMS bounds, and element-wise (max-abs, LSE) within the gates of the emulation
    run on the kernel's own scores.  The element-wise gate is not taken against the
    exact-score emulation here: a probability code whose exact value lies within the FP8
    MFMA's score-error band of a rounding boundary may round either way, and in a row of few
    keys one such code moves O by more than that gate (0.026 in the 24-key row 23 of the
    512-key MLA case, test_mla_short_row_regression)."""
    _case("fp8_vt", B, H, Hkv, S, dqk, p_mode, padded)
    G = H // Hkv
    q, k, v = _inputs(B, H, Hkv, S, dqk, seed=5 * S + H + dqk)
    gq = [cfa.quantize_e4m3(torch.from_numpy(x).to(DEV)) for x in (q, k, v)]
    (qg, dq), (kg, dk), (vg, dv) = [(c_.view(torch.uint8), float(d_.item())) for c_, d_ in gq]
    c = 1.0 / math.sqrt(dqk)
    vt = _channel_major(vg, padded)
    out, lse = cfa.attn_fwd_causal_fp8_vt(qg, kg, vt, dq, dk, dv, softmax_scale=c, p_mode=p_mode)
    ref_out, ref_lse = cfa.attn_fwd_causal_fp8_ex(qg, kg, vg, dq, dk, dv, softmax_scale=c, p_mode=p_mode)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)) and torch.equal(lse, ref_lse)
    (qc, _), (kc, _), (vc, _) = [oracle.quantize_e4m3(x) for x in (q, k, v)]
    exact_p = (p_mode == cfa.P_EXACT) or (p_mode is None and dqk == 192)
    _check_fp8_oracle(out, lse, qc, kc, vc, G, dq, dk, dv, c, exact_p, B, H, S, strict=False)
    check_fp8_on_gpu_scores(qg, kg, vg, dq, dk, dv, c, p_mode, ref=(out, lse))


def test_mla_short_row_regression():
    """B2 H4 over 2 KV heads, S512 at the MLA shape with exact P, seed 2756: row 23 of one head
    has 24 keys, and one of its codes sits inside the MFMA's score-error band of a rounding
    boundary and rounds the other way than in the exact-score emulation, which moves O by
    0.026 there.  Checked element-wise against the emulation on the kernel's own scores."""
    B, H, Hkv, S, dqk = 2, 4, 2, 512, 192
    _case("mla short-row regression", B, H, Hkv, S, dqk)
    q, k, v = _inputs(B, H, Hkv, S, dqk, seed=5 * S + H + dqk)
    gq = [cfa.quantize_e4m3(torch.from_numpy(x).to(DEV)) for x in (q, k, v)]
    (qg, dq), (kg, dk), (vg, dv) = [(c_.view(torch.uint8), float(d_.item())) for c_, d_ in gq]
    c = 1.0 / math.sqrt(dqk)
    out, lse = cfa.attn_fwd_causal_fp8_ex(qg, kg, vg, dq, dk, dv, softmax_scale=c)
    torch.cuda.synchronize()
    check_fp8_on_gpu_scores(qg, kg, vg, dq, dk, dv, c, None, ref=(out, lse))


@pytest.mark.parametrize("H,Hkv,dqk", [(32, 32, 128), (32, 8, 128), (16, 16, 192)])
def test_fp8_vt_full_size_bitwise(H, Hkv, dqk):
    """At S = 32768 (the paper's long-sequence shapes): channel-major V equals key-major V bit
    for bit, over every output."""
    B, S = 1, 32768
    _case("fp8_vt full size", B, H, Hkv, S, dqk)
    g = torch.Generator(device=DEV)
    g.manual_seed(1000 + H + Hkv + dqk)
    q, k, v = (torch.randn((B, S, h, d), generator=g, device=DEV).mul_(16).to(torch.float8_e4m3fn)
               .view(torch.uint8) for h, d in ((H, dqk), (Hkv, dqk), (Hkv, 128)))
    vt = v.permute(0, 2, 3, 1).contiguous()
    o1, l1 = cfa.attn_fwd_causal_fp8_ex(q, k, v, 1 / 16, 1 / 16, 1 / 16)
    o2, l2 = cfa.attn_fwd_causal_fp8_vt(q, k, vt, 1 / 16, 1 / 16, 1 / 16)
    torch.cuda.synchronize()
    assert not torch.isnan(o1.float()).any()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


def test_fp8_ex_matches_basic_entry_points():
    """Dense BSHD, H_kv = H and the default P mode: identical to attn_fwd_causal_fp8 / _mla."""
    for dqk, basic in ((128, cfa.attn_fwd_causal_fp8), (192, cfa.attn_fwd_causal_mla)):
        B, H, S = 1, 3, 512
        _case("fp8_ex vs basic", dqk, B, H, S)
        q, k, v = synth.gaussian(B, S, H, dqk, 128, 11)
        (qg, dq), (kg, dk), (vg, dv) = [(c_, float(d_.item())) for c_, d_ in
                                        (cfa.quantize_e4m3(torch.from_numpy(x).to(DEV)) for x in (q, k, v))]
        o1, l1 = basic(qg, kg, vg, dq, dk, dv)
        o2, l2 = cfa.attn_fwd_causal_fp8_ex(qg, kg, vg, dq, dk, dv)
        torch.cuda.synchronize()
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


@pytest.mark.parametrize("B,H,Hkv,S,dqk,layout", [(2, 4, 2, 768, 128, "bhsd"), (1, 8, 2, 1024, 128, "padded"),
                                                  (1, 4, 1, 512, 128, "bshd"), (1, 2, 2, 1024, 192, "bshd"),
                                                  (2, 4, 2, 768, 192, "bhsd"), (1, 4, 1, 512, 192, "padded")])
def test_bf16_ex(B, H, Hkv, S, dqk, layout):
    _case("bf16_ex", B, H, Hkv, S, dqk, layout)
    q, k, v = _inputs(B, H, Hkv, S, dqk, seed=5 * S + H + dqk)
    _bf16_ex_check(q, k, v, layout)


@pytest.mark.parametrize("name", ["rising_logits", "sink_flat_tail", "stepped_max", "logit_sd_16"])
def test_bf16_mla_stress(name):
    """BF16 at the MLA shape (lazy threshold 8 binades) on the stress inputs: the rescale
    path and far-below-maximum blocks against exact fp64."""
    B, H, S = 1, 2, 1024
    _case("bf16 mla stress", name, B, H, S)
    q, k, v = synth.STRESS[name](B, S, H, 192, 128, 33)
    _bf16_ex_check(q, k, v, "bshd")


def _bf16_ex_check(q, k, v, layout):
    B, S, H, dqk = q.shape
    Hkv = k.shape[2]
    G = H // Hkv
    qg, kg, vg = (cfa.round_bf16(torch.from_numpy(np.ascontiguousarray(x)).to(DEV)) for x in (q, k, v))
    qb, kb, vb = (oracle.bf16_rne(x) for x in (q, k, v))
    c = 1.0 / math.sqrt(dqk)
    qL, kL, vL = (_relayout(t, layout) for t in (qg, kg, vg))
    out = _out_like(B, S, H, layout)
    lse = torch.full((B, H, S), float("nan"), dtype=torch.float32, device=DEV)
    cfa.attn_fwd_causal_bf16_ex(qL, kL, vL, softmax_scale=c, out=out, lse=lse)
    ref_out, ref_lse = cfa.attn_fwd_causal_bf16_ex(qg, _expand_heads_gpu(kg, G), _expand_heads_gpu(vg, G),
                                                   softmax_scale=c)
    torch.cuda.synchronize()
    assert not torch.isnan(out.float()).any() and not torch.isnan(lse).any()
    _assert_spare_heads_untouched(out, layout)
    assert torch.equal(out.contiguous().view(torch.int16), ref_out.view(torch.int16))
    assert torch.equal(lse, ref_lse)
    if dqk == 128 and G == 1:
        o2, l2 = cfa.attn_fwd_causal_bf16(qg, kg, vg, softmax_scale=c)
        torch.cuda.synchronize()
        assert torch.equal(o2.view(torch.int16), ref_out.view(torch.int16)) and torch.equal(l2, ref_lse)
    rows = oracle.group_rows(all_groups(B, H, S), 32)
    ex, ex_lse = oracle.attn_exact(qb, np.repeat(kb, G, axis=2), np.repeat(vb, G, axis=2), dtype="bf16", c=c,
                                   rows=rows)
    got, glse = gpu_rows(out.contiguous(), rows), lse_rows(lse, rows)
    res = {"fp64_rms": rms_rel(got, ex), "lse_fp64": float(np.max(np.abs(glse - ex_lse)))}
    print("RESULT", res, flush=True)
    assert res["fp64_rms"] <= TOL_FP64_RMS_BF16, res
    assert res["lse_fp64"] <= 1e-3 + 1e-6 * np.max(np.abs(ex_lse)), res


@pytest.mark.parametrize("kind,dqk", [("fp8", 128), ("fp8", 192), ("bf16", 128), ("bf16", 192)])
@pytest.mark.parametrize("B,H,Hkv,S", [(3, 96, 48, 512), (2, 10, 5, 8192), (2, 9, 3, 1024), (1, 8, 2, 2048)])
def test_many_items_per_workgroup(kind, dqk, B, H, Hkv, S):
    """More tile pairs than workgroups (288 and 320 items for at most 256 workgroups), over
    several batches and grouped key/value heads: a workgroup then steps through several work
    items, from one pair of a head to the next (S = 8192, 16 pairs per head) and across heads
    and batches (S = 512, one pair per head).  A causal row does not depend on which workgroup
    runs it, so every (b, h) of the launch must equal a launch on that head alone, bit for bit.
    With an even group (G = 2, 4) the launch runs the head-pair mode (two heads, 128-row tiles)
    and the single-head launches do not; G = 3 runs 256-row tiles of one head."""
    _case("many items per workgroup", kind, dqk, B, H, Hkv, S)
    G = H // Hkv
    q, k, v = _inputs(B, H, Hkv, S, dqk, seed=B * H + S + dqk)
    if kind == "fp8":
        (qg, dq), (kg, dk), (vg, dv) = [(c_, float(d_.item())) for c_, d_ in
                                        (cfa.quantize_e4m3(torch.from_numpy(x).to(DEV)) for x in (q, k, v))]
        run = lambda a, b_, c: cfa.attn_fwd_causal_fp8_ex(a, b_, c, dq, dk, dv)
    else:
        qg, kg, vg = (cfa.round_bf16(torch.from_numpy(x).to(DEV)) for x in (q, k, v))
        run = lambda a, b_, c: cfa.attn_fwd_causal_bf16_ex(a, b_, c)
    out, lse = run(qg, kg, vg)
    torch.cuda.synchronize()
    assert not torch.isnan(out.float()).any() and not torch.isnan(lse).any()
    for b in range(B):
        for h in range(H):
            o1, l1 = run(qg[b:b + 1, :, h:h + 1].contiguous(), kg[b:b + 1, :, h // G:h // G + 1].contiguous(),
                         vg[b:b + 1, :, h // G:h // G + 1].contiguous())
            assert torch.equal(out[b:b + 1, :, h:h + 1].contiguous().view(torch.int16), o1.view(torch.int16)), (b, h)
            assert torch.equal(lse[b, h], l1[0, 0]), (b, h)
    torch.cuda.synchronize()
