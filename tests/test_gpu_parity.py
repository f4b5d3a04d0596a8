"""GPU parity of the HIP path against the CPU oracle at sizes the oracle finishes in
seconds (several 256-row tiles, batches and heads, the paper's stress inputs).

Every test prints the case it runs before touching the GPU."""
import math

import numpy as np
import pytest
import torch

import bf16_causal_flashattention_amd as cfa
import oracle
import synth
from gpu_util import (DEV, all_groups, check_bf16_against_oracle, check_fp8_against_oracle,
                      check_fp8_on_gpu_scores, fp8_entry, prep_fp8_gpu)

# stress inputs whose logit ranges make the element-wise result depend on the FP8 MFMA's
# score precision: gated element-wise against the emulation on the kernel's own scores
# (after checking those against the exact ones); the rest against the exact-score emulation
WIDE = {"logit_sd_4", "logit_sd_16", "stepped_max", "full_range", "rising_logits", "alternating_rows"}

pytestmark = pytest.mark.gpu


def _case(*a):
    print("CASE", *a, flush=True)


# ----------------------------------------------------------------------------- input prep (a0)
@pytest.mark.parametrize("n", [1, 3, 4, 1000, 4097, 1 << 20])
@pytest.mark.parametrize("dist", ["normal", "tiny", "huge", "zero", "full_range"])
def test_quantize_bitexact(n, dist):
    _case("quantize", n, dist)
    rng = np.random.default_rng(n)
    x = rng.standard_normal(n).astype(np.float32)
    if dist == "tiny":
        x *= np.float32(1e-30)
    elif dist == "huge":
        x *= np.float32(1e30)
    elif dist == "zero":
        x[:] = 0
    elif dist == "full_range":
        x = (np.exp2(rng.uniform(-20, 20, n)) * np.sign(x)).astype(np.float32)
    codes, ds = cfa.quantize_e4m3(torch.from_numpy(x).to(DEV))
    oc, ods = oracle.quantize_e4m3(x)
    assert float(ds.item()) == ods
    assert np.array_equal(codes.view(torch.uint8).cpu().numpy(), oc)


def test_round_bf16_bitexact():
    _case("round_bf16")
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(1 << 20) * np.exp2(rng.uniform(-40, 40, 1 << 20))).astype(np.float32)
    got = cfa.round_bf16(torch.from_numpy(x).to(DEV)).view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, oracle.bf16_rne(x))


# ----------------------------------------------------------------------------- FP8 d=128, lean P
@pytest.mark.parametrize("B,H,S", [(1, 1, 256), (1, 1, 512), (2, 3, 1024), (1, 2, 1280)])
def test_fp8_gaussian(B, H, S):
    _case("fp8 gaussian", B, H, S)
    qkv = synth.gaussian(B, S, H, 128, 128, seed=B * 100 + S)
    check_fp8_against_oracle(qkv, 128, all_groups(B, H, S), False, fp8_entry(128))


@pytest.mark.parametrize("name", sorted(synth.STRESS))
def test_fp8_stress(name):
    B, H, S = 1, 2, 1024
    _case("fp8 stress", name, B, H, S)
    qkv = synth.STRESS[name](B, S, H, 128, 128, 21)
    check_fp8_against_oracle(qkv, 128, all_groups(B, H, S), False, fp8_entry(128), strict=name not in WIDE,
                             check_lse=name != "full_range")


def test_fp8_activation_like_small():
    B, H, S = 1, 2, 1024
    _case("fp8 activation-like", B, H, S)
    qkv = synth.activation_like(B, S, H, 128, 128, 22)
    check_fp8_against_oracle(qkv, 128, all_groups(B, H, S), False, fp8_entry(128))


# ----------------------------------------------------------------------------- FP8 MLA 192/128, exact P
@pytest.mark.parametrize("B,H,S", [(1, 1, 256), (2, 2, 768), (1, 3, 1024)])
def test_mla_gaussian(B, H, S):
    _case("mla gaussian", B, H, S)
    qkv = synth.gaussian(B, S, H, 192, 128, seed=B * 7 + S)
    check_fp8_against_oracle(qkv, 192, all_groups(B, H, S), True, fp8_entry(192))


@pytest.mark.parametrize("name", ["logit_sd_16", "sink_flat_tail", "stepped_max", "full_range"])
def test_mla_stress(name):
    B, H, S = 1, 2, 1024
    _case("mla stress", name)
    qkv = synth.STRESS[name](B, S, H, 192, 128, 23)
    check_fp8_against_oracle(qkv, 192, all_groups(B, H, S), True, fp8_entry(192), strict=name not in WIDE,
                             check_lse=name != "full_range")


# ----------------------------------------------------------------------------- BF16 d=128
@pytest.mark.parametrize("B,H,S", [(1, 1, 256), (2, 3, 1024), (1, 2, 1280)])
def test_bf16_gaussian(B, H, S):
    _case("bf16 gaussian", B, H, S)
    qkv = synth.gaussian(B, S, H, 128, 128, seed=S + 3)
    rows = oracle.group_rows(all_groups(B, H, S), 32)
    check_bf16_against_oracle(qkv, rows)


@pytest.mark.parametrize("name", ["logit_sd_16", "sink_flat_tail", "stepped_max", "full_range", "alternating_rows"])
def test_bf16_stress(name):
    B, H, S = 1, 2, 1024
    _case("bf16 stress", name)
    qkv = synth.STRESS[name](B, S, H, 128, 128, 24)
    rows = oracle.group_rows(all_groups(B, H, S), 32)
    check_bf16_against_oracle(qkv, rows)


# ----------------------------------------------------------------------------- the kernel's own scores
@pytest.mark.parametrize("dqk,S,name,p_mode", [
    (128, 256, "gaussian", None), (128, 512, "stepped_max", None), (192, 512, "gaussian", None),
    (128, 512, "sink_flat_tail", None), (128, 512, "logit_sd_16", None), (128, 512, "full_range", None),
    (128, 512, "alternating_rows", None), (128, 512, "rising_logits", None),
    (192, 512, "stepped_max", cfa.P_LEAN), (128, 512, "logit_sd_4", cfa.P_EXACT), (192, 512, "full_range", None)])
def test_decisions_on_gpu_scores(dqk, S, name, p_mode):
    """Every raw score within the MFMA bound of the exact dot product; on those scores the
    emulation's block exponents and codes are the kernel's, bit for bit (exact P: up to
    v_exp_f32's rounding band); O and the LSE within the gates of that emulation."""
    _case("gpu scores", dqk, S, name, p_mode)
    B, H = 1, 2
    gen = synth.gaussian if name == "gaussian" else synth.STRESS[name]
    q, k, v = gen(B, S, H, dqk, 128, 31)
    (qg, dq), (kg, dk), (vg, dv) = prep_fp8_gpu(q, k, v)
    qg, kg, vg = (t.view(torch.uint8) for t in (qg, kg, vg))
    c = 1 / math.sqrt(dqk)
    ref = cfa.attn_fwd_causal_fp8_ex(qg, kg, vg, dq, dk, dv, softmax_scale=c, p_mode=p_mode)
    check_fp8_on_gpu_scores(qg, kg, vg, dq, dk, dv, c, p_mode, ref=ref)


# ----------------------------------------------------------------------------- closed forms on the GPU
@pytest.mark.parametrize("dqk", [128, 192])
def test_identical_keys_prefix_mean(dqk):
    _case("identical keys", dqk)
    B, H, S = 1, 2, 512
    q, k, v = synth.identical_keys(B, S, H, dqk, 128, 41)
    (qg, dq), (kg, dk), (vg, dv) = prep_fp8_gpu(q, k, v)
    out, _ = fp8_entry(dqk)(qg, kg, vg, dq, dk, dv)
    V = oracle.e4m3_table()[vg.view(torch.uint8).cpu().numpy()] * dv
    pref = np.cumsum(V, axis=1) / np.arange(1, S + 1)[None, :, None, None]
    want = oracle.bf16_value(oracle.bf16_rne(pref.astype(np.float32)))
    got = out.float().cpu().numpy()
    assert np.max(np.abs(got - want) / (np.abs(want) + 1e-3)) < 2 ** -7


@pytest.mark.parametrize("dqk", [128, 192])
def test_one_hot_returns_value_row(dqk):
    _case("one hot", dqk)
    B, H, S = 1, 2, 512
    q, k, v = synth.one_hot_key(B, S, H, dqk, 128, 42, key=0, lift=60.0)
    (qg, dq), (kg, dk), (vg, dv) = prep_fp8_gpu(q, k, v)
    out, _ = fp8_entry(dqk)(qg, kg, vg, dq, dk, dv)
    V0 = oracle.e4m3_table()[vg.view(torch.uint8).cpu().numpy()[:, 0]] * dv  # [B, H, d]
    want = oracle.bf16_value(oracle.bf16_rne(V0.astype(np.float32)))
    got = out.float().cpu().numpy()
    assert np.array_equal(got, np.broadcast_to(want[:, None], got.shape))


# ----------------------------------------------------------------------------- determinism and coverage
@pytest.mark.parametrize("kind", ["fp8", "mla", "bf16"])
def test_bitwise_reproducible_with_interferer(kind):
    """200 launches, bit for bit equal to the first, with an interferer before each: a BF16
    GEMM and a BF16 attention call in turn (paper Table XII), the latter on a second stream
    so that it overlaps the checked launch."""
    _case("determinism", kind)
    B, H, S = 1, 8, 2048
    dqk = 192 if kind == "mla" else 128
    q, k, v = synth.gaussian(B, S, H, dqk, 128, 51)
    if kind == "bf16":
        qg, kg, vg = (cfa.round_bf16(torch.from_numpy(x).to(DEV)) for x in (q, k, v))
        run = lambda: cfa.attn_fwd_causal_bf16(qg, kg, vg)
    else:
        (qg, dq), (kg, dk), (vg, dv) = prep_fp8_gpu(q, k, v)
        run = lambda: fp8_entry(dqk)(qg, kg, vg, dq, dk, dv)
    a = torch.randn(2048, 2048, device=DEV, dtype=torch.bfloat16)
    b = torch.randn(2048, 2048, device=DEV, dtype=torch.bfloat16)
    xi = [cfa.round_bf16(torch.from_numpy(x).to(DEV)) for x in synth.gaussian(1, 4096, 4, 128, 128, 52)]
    side = torch.cuda.Stream(device=DEV)
    ref_o, ref_l = run()
    ref_o, ref_l = ref_o.clone(), ref_l.clone()
    torch.cuda.synchronize()
    for i in range(200):
        if i % 2:
            (a @ b).sum()  # a BF16 GEMM between launches
        else:
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):  # BF16 attention overlapping the next launch
                cfa.attn_fwd_causal_bf16(*xi)
        o, l = run()
        assert torch.equal(o.view(torch.int16), ref_o.view(torch.int16)), i
        assert torch.equal(l.view(torch.int32), ref_l.view(torch.int32)), i
    torch.cuda.synchronize()


def test_every_tile_written():
    _case("coverage", "nan sentinel")
    B, H, S = 3, 5, 1280  # odd tile count: the middle tile runs alone
    q, k, v = synth.gaussian(B, S, H, 128, 128, 61)
    (qg, dq), (kg, dk), (vg, dv) = prep_fp8_gpu(q, k, v)
    out = torch.full((B, S, H, 128), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((B, H, S), float("nan"), dtype=torch.float32, device=DEV)
    cfa.attn_fwd_causal_fp8(qg, kg, vg, dq, dk, dv, out=out, lse=lse)
    torch.cuda.synchronize()
    assert not torch.isnan(out.float()).any() and not torch.isnan(lse).any()


def test_empty_problem():
    _case("empty")
    x = torch.empty((0, 256, 1, 128), dtype=torch.uint8, device=DEV)
    out, lse = cfa.attn_fwd_causal_fp8(x, x, torch.empty((0, 256, 1, 128), dtype=torch.uint8, device=DEV),
                                       1.0, 1.0, 1.0)
    assert out.numel() == 0 and lse.numel() == 0
