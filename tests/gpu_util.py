"""Helpers shared by the GPU tests: run the library's own input preparation on the
GPU, run the oracle's independently on the CPU, and compare outputs row by row."""
import math

import numpy as np
import torch

import bf16_causal_flashattention_amd as cfa
import oracle

DEV = torch.device("cuda:0")

# tolerances stated for this path: GPU vs the FP8 emulation (max-abs, RMS-rel),
# GPU vs exact fp64 (RMS-rel) for FP8 and BF16
TOL_EMU_MAXABS = 2e-2
TOL_EMU_RMS = 1e-2
TOL_FP64_RMS_FP8 = 6e-2
TOL_FP64_RMS_BF16 = 1e-2
LSE_FP64_NATS = 0.04  # worst-row LSE bound for lean P (paper Sec. IV-B3)
# LSE vs the emulation: one code that rounds the other way at a rounding boundary moves
# l by up to one e4m3 step (1/8) of that probability's share of the row
LSE_EMU_NATS = 0.02
# FP8 MFMA score error bound (measured on gfx950): |s_gpu - s_exact| <= 2^-10 per 64-wide
# chunk of the largest |q_d k_d| product
MFMA_ERR_PER_CHUNK = 2.0 ** -10


def rms_rel(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def snr_db(got, ref):
    """Signal-to-noise ratio of got against ref in dB: 10 log10(sum ref^2 / sum (got - ref)^2)."""
    ref = np.asarray(ref, np.float64)
    err = np.asarray(got, np.float64) - ref
    e2 = float(np.sum(err * err))
    return float("inf") if e2 == 0.0 else float(10 * np.log10(np.sum(ref * ref) / e2))


def prep_fp8_gpu(q, k, v):
    """Quantise fp32 host arrays with the library's GPU quantiser."""
    outs = []
    for x in (q, k, v):
        tx = torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
        codes, ds = cfa.quantize_e4m3(tx)
        outs.append((codes, float(ds.item())))
        del tx
    return outs


def prep_fp8_cpu(q, k, v):
    return [oracle.quantize_e4m3(x) for x in (q, k, v)]


def prep_bf16_gpu(q, k, v):
    return [cfa.round_bf16(torch.from_numpy(np.ascontiguousarray(x)).to(DEV)) for x in (q, k, v)]


def gpu_rows(out, rows):
    """Gather rows (b, h, i) of a [B, S, H, d] GPU output as float64 numpy."""
    o = out.float().cpu().numpy()
    return o[rows[:, 0], rows[:, 2], rows[:, 1]].astype(np.float64)


def lse_rows(lse, rows):
    x = lse.cpu().numpy()
    return x[rows[:, 0], rows[:, 1], rows[:, 2]].astype(np.float64)


def all_groups(B, H, S, group=32):
    bb, hh, rr = np.meshgrid(np.arange(B), np.arange(H), np.arange(0, S, group), indexing="ij")
    return np.stack([bb.ravel(), hh.ravel(), rr.ravel()], axis=1).astype(np.int64)


def sample_groups(B, H, S, n, seed, group=32):
    """Row groups (b, h, r0) spread over the sequence: first, last, and seeded ones."""
    rng = np.random.default_rng(seed)
    g = [(0, 0, 0), (B - 1, H - 1, S - group)]
    while len(g) < n:
        g.append((int(rng.integers(B)), int(rng.integers(H)), int(rng.integers(S // group)) * group))
    return np.array(sorted(set(g)), dtype=np.int64)


def check_fp8_against_oracle(qkv32, dqk, groups, exact_p, entry, report=None, strict=True, check_lse=True):
    """Run the GPU path (GPU quantiser + attention) and compare with the oracle
    (CPU quantiser + emulation + exact fp64) on the given row groups.

    strict: the element-wise gates (max-abs vs the emulation) apply.  For inputs with
    wide logit ranges the element-wise result is not unique at the FP8 MFMA's
    accumulation precision (scores carry errors up to ~2^-11 of the largest product),
    so those cases are gated on the RMS errors and the LSE bound only."""
    q, k, v = qkv32
    B, S, H, _ = q.shape
    (qg, dq), (kg, dk), (vg, dv) = prep_fp8_gpu(q, k, v)
    (qc, dq_o), (kc, dk_o), (vc, dv_o) = prep_fp8_cpu(q, k, v)
    # input preparation is bit-exact
    assert (dq, dk, dv) == (dq_o, dk_o, dv_o)
    for g_, c_ in ((qg, qc), (kg, kc), (vg, vc)):
        assert np.array_equal(g_.view(torch.uint8).cpu().numpy(), c_)
    c = 1.0 / math.sqrt(dqk)
    out = torch.full((B, S, H, 128), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((B, H, S), float("nan"), dtype=torch.float32, device=DEV)
    entry(qg, kg, vg, dq, dk, dv, softmax_scale=c, out=out, lse=lse)
    torch.cuda.synchronize()
    scheme = oracle.Fp8Scheme(exact_p=exact_p)
    emu = oracle.emulate_fp8(qc, kc, vc, dq=dq, dk=dk, dv=dv, c=c, scheme=scheme, groups=groups)
    rows = oracle.group_rows(groups, scheme.group)
    keep = rows[:, 2] < S
    rows = rows[keep]
    ex, ex_lse = oracle.attn_exact(qc, kc, vc, dtype="fp8", c=c, dq=dq, dk=dk, dv=dv, rows=rows)
    got = gpu_rows(out, rows)
    glse = lse_rows(lse, rows)
    emu_out, emu_lse = emu["out"][keep], emu["lse"][keep]
    assert np.all(np.isfinite(got)) and np.all(np.isfinite(glse))
    res = {
        "emu_maxabs": float(np.max(np.abs(got - emu_out))),
        "emu_rms": rms_rel(got, emu_out),
        "fp64_rms": rms_rel(got, ex),
        "lse_emu": float(np.max(np.abs(glse - emu_lse))),
        "lse_fp64": float(np.max(np.abs(glse - ex_lse))),
    }
    if report is not None:
        report.update(res)
    if strict:
        assert res["emu_maxabs"] <= TOL_EMU_MAXABS, res
        assert res["lse_emu"] <= LSE_EMU_NATS, res
    assert res["emu_rms"] <= TOL_EMU_RMS, res
    assert res["fp64_rms"] <= TOL_FP64_RMS_FP8, res
    if check_lse:
        assert res["lse_fp64"] <= LSE_FP64_NATS, res
    return res


def check_bf16_against_oracle(qkv32, rows, report=None):
    q, k, v = qkv32
    B, S, H, d = q.shape
    qg, kg, vg = prep_bf16_gpu(q, k, v)
    qb, kb, vb = (oracle.bf16_rne(x) for x in (q, k, v))
    for g_, c_ in ((qg, qb), (kg, kb), (vg, vb)):
        assert np.array_equal(g_.view(torch.int16).cpu().numpy().view(np.uint16), c_)
    c = 1.0 / math.sqrt(d)
    out = torch.full((B, S, H, 128), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((B, H, S), float("nan"), dtype=torch.float32, device=DEV)
    cfa.attn_fwd_causal_bf16(qg, kg, vg, softmax_scale=c, out=out, lse=lse)
    torch.cuda.synchronize()
    ex, ex_lse = oracle.attn_exact(qb, kb, vb, dtype="bf16", c=c, rows=rows)
    got = gpu_rows(out, rows)
    glse = lse_rows(lse, rows)
    assert np.all(np.isfinite(got))
    res = {"fp64_rms": rms_rel(got, ex), "fp64_maxabs": float(np.max(np.abs(got - ex))),
           "lse_fp64": float(np.max(np.abs(glse - ex_lse)))}
    if report is not None:
        report.update(res)
    assert res["fp64_rms"] <= TOL_FP64_RMS_BF16, res
    # fp32 m and l: LSE good to ~1e-6 relative of the row's largest logit
    lse_tol = 1e-3 + 1e-6 * np.max(np.abs(ex_lse))
    assert res["lse_fp64"] <= lse_tol, res
    return res


def fp8_entry(dqk):
    if dqk == 128:
        return lambda qg, kg, vg, dq, dk, dv, **kw: cfa.attn_fwd_causal_fp8(qg, kg, vg, dq, dk, dv, **kw)
    return lambda qg, kg, vg, dq, dk, dv, **kw: cfa.attn_fwd_causal_mla(qg, kg, vg, dq, dk, dv, **kw)


def score_error_bound(qc, kc, dqk, b=0, h=0):
    """Per (query, key) bound on the FP8 MFMA score error for head (b, h), in raw
    (descaled-free) units: MFMA_ERR_PER_CHUNK * chunks * max_d |q_d k_d|."""
    t = oracle.e4m3_table()
    Q = np.abs(t[qc[b, :, h]])
    K = np.abs(t[kc[b, :, h]])
    mp = np.zeros((Q.shape[0], K.shape[0]))
    for d in range(Q.shape[1]):
        np.maximum(mp, np.outer(Q[:, d], K[:, d]), out=mp)
    return MFMA_ERR_PER_CHUNK * (dqk // 64) * mp
