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
# FP8 MFMA score error bound on gfx950: |s_gpu - s_exact| <= 2^-10 times the largest
# |q_d k_d| product of each 64-wide chunk, summed over the chunks, plus two fp32 roundings
# of the sum.  The MFMA does not round its 64-term sums correctly (about 2^-11 of the
# largest product is measured).  check_fp8_on_gpu_scores checks the bound on every score the
# kernel forms (test_gpu_parity.py::test_decisions_on_gpu_scores, including full-range e4m3
# inputs, and the prefix check of the activation-like full-size test) and reports the largest
# error over bound, 0.5-0.6 in the runs so far.
MFMA_ERR_PER_CHUNK = 2.0 ** -10
# exact P: the GPU's 2^x (v_exp_f32) is within about an fp32 ulp; a code may round the
# other way when 2^x lies this close (relative) to an e4m3 rounding boundary
EXP2_REL_BAND = 2.0 ** -20
# O and LSE against the emulation run on the kernel's own scores: same codes, so what is
# left is the fp32 MFMA accumulation of PV, the hardware exp2 of the rare rescale and the
# bf16 rounding of O (half an ulp, 2^-9 relative)
LSE_SCORES_NATS = 1e-3


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

    strict: the element-wise gates (max-abs and LSE) apply against the emulation on exact
    scores.  For inputs with wide logit ranges the element-wise result is not unique at the
    FP8 MFMA's accumulation precision (scores carry errors up to ~2^-11 of the largest
    product, and a code near a rounding boundary may go either way), so there the
    element-wise gates apply against the emulation run on the kernel's own scores instead
    (check_fp8_on_gpu_scores), after those scores are checked against the exact ones; the
    RMS gates against both references apply in every case."""
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
    else:
        check_fp8_on_gpu_scores(qg.view(torch.uint8), kg.view(torch.uint8), vg.view(torch.uint8), dq, dk, dv, c,
                                cfa.P_EXACT if exact_p else cfa.P_LEAN, ref=(out, lse), report=res)
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


def exact_scores(qc, kc):
    """Exact raw dot products of the decoded codes, [B*H*S, S] (row (b*H + h)*S + i).  qc, kc:
    [B, S, H, d] codes with the same H.  Every product is a multiple of 2^-18 below 2^18 in
    magnitude, so all partial sums are exact in fp64 whatever the summation order."""
    t = oracle.e4m3_table()
    Q, K = t[qc], t[kc]
    B, S, H, _ = qc.shape
    out = np.empty((B, H, S, S))
    for b in range(B):
        for h in range(H):
            out[b, h] = Q[b, :, h] @ K[b, :, h].T
    return out.reshape(B * H * S, S)


def chunk_error_bound(qc, kc):
    """Per (query, key) MFMA score-error bound in raw units, [B*H*S, S]: MFMA_ERR_PER_CHUNK times
    the sum over 64-wide chunks of the largest |q_d k_d| in the chunk."""
    t = np.abs(oracle.e4m3_table())
    Q, K = t[qc], t[kc]
    B, S, H, d = qc.shape
    out = np.zeros((B, H, S, S))
    for b in range(B):
        for h in range(H):
            for c0 in range(0, d, 64):
                mp = np.zeros((S, S))
                for e in range(c0, c0 + 64):
                    np.maximum(mp, np.outer(Q[b, :, h, e], K[b, :, h, e]), out=mp)
                out[b, h] += mp
    return MFMA_ERR_PER_CHUNK * out.reshape(B * H * S, S)


def _max_ratio(err, bound):
    """Largest err/bound; an element with a zero bound counts 0 if its error is 0, else inf."""
    r = np.divide(err, bound, out=np.where(err > 0, np.inf, 0.0), where=bound > 0)
    return float(np.max(r))


def check_fp8_on_gpu_scores(qg, kg, vg, dq, dk, dv, c, p_mode, ref=None, report=None):
    """Complete check of one FP8 call at a size the debug hook allows (B*H*S^2 <= 2^28):

    1. every raw score the kernel formed lies within the MFMA bound of the exact dot product;
    2. the oracle's emulation, run on those scores, takes the kernel's decisions: the same
       block exponents o everywhere and the same code for every key (exact P: a code may
       differ by one step only where 2^x lies within EXP2_REL_BAND of a rounding boundary);
    3. O within the stated max-abs and RMS gates, and the LSE within LSE_SCORES_NATS, of that
       emulation.
    qg, kg, vg: GPU uint8 codes [B, S, H, d_qk], [B, S, H_kv, d_qk], [B, S, H_kv, 128].
    ref: optional (out, lse) of the production call on the same inputs; the debug call must
    equal it bit for bit.  Returns a dict of the measured quantities."""
    out, lse, go, gc, gs = cfa.attn_fwd_causal_fp8_debug_ex(qg, kg, vg, dq, dk, dv, softmax_scale=c, p_mode=p_mode)
    torch.cuda.synchronize()
    if ref is not None:
        assert torch.equal(out.view(torch.int16), ref[0].contiguous().view(torch.int16))
        assert torch.equal(lse, ref[1])
    B, S, H, dqk = qg.shape
    G = H // kg.shape[2]
    exact_p = (p_mode == cfa.P_EXACT) or (p_mode is None and dqk == 192)
    qc = qg.cpu().numpy()
    kc = np.repeat(kg.cpu().numpy(), G, axis=2)
    vc = np.repeat(vg.cpu().numpy(), G, axis=2)
    go, gc, gs = go.cpu().numpy(), gc.cpu().numpy(), gs.cpu().numpy()
    vis = np.tile(np.tril(np.ones((S, S), dtype=bool)), (B * H, 1))
    # 1. scores
    ex = exact_scores(qc, kc)
    bound = chunk_error_bound(qc, kc) + 2.0 ** -23 * np.abs(ex)
    assert not np.any(np.isnan(gs[vis])), "a visible score was not written"
    err = np.abs(gs.astype(np.float64) - ex)
    ratio = float(np.max((err / np.where(bound > 0, bound, 1.0))[vis]))
    assert np.all(err[vis] <= bound[vis]), ("score outside the MFMA bound", ratio)
    # 2. decisions on the kernel's scores
    scheme = oracle.Fp8Scheme(exact_p=exact_p)
    emu = oracle.emulate_fp8_from_scores(np.where(vis, gs, 0.0).astype(np.float32), vc, dq=dq, dk=dk, dv=dv, c=c,
                                         scheme=scheme, debug=True)
    seen = emu["o"] != 255
    assert np.array_equal(go[seen], emu["o"][seen]), int(np.sum(go[seen] != emu["o"][seen]))
    mism = gc != emu["codes"]
    if exact_p:
        allowed = emu["ymargin"] < EXP2_REL_BAND
        assert not np.any(mism & ~allowed), int(np.sum(mism & ~allowed))
        assert np.all(np.abs(gc[mism].astype(int) - emu["codes"][mism].astype(int)) == 1)
    else:
        assert not np.any(mism), int(np.sum(mism))
    # 3. outputs against the emulation on the same scores
    rows = oracle.group_rows(emu["groups"], scheme.group)
    got, glse = gpu_rows(out, rows), lse_rows(lse, rows)
    err, lerr = np.abs(got - emu["out"]), np.abs(glse - emu["lse"])
    o_bound, l_bound = output_error_bound(emu["codes"], emu["o"], vc, dv, emu["out"])
    l_bound = l_bound + 2.0 ** -21 * np.abs(emu["lse"])  # the kernel forms the LSE in fp32
    res = {"score_err_over_bound": ratio, "code_mismatch_in_band": int(mism.sum()),
           "maxabs": float(np.max(err)), "rms": rms_rel(got, emu["out"]), "lse": float(np.max(lerr)),
           "maxabs_over_bound": _max_ratio(err, o_bound), "lse_over_bound": _max_ratio(lerr, l_bound)}
    print("GPU-SCORES", res, flush=True)
    if report is not None:
        report.update(res)
    # every element within the stated max-abs gate, or within the MFMA bound where V's range
    # makes that bound the larger one
    assert np.all(err <= np.maximum(TOL_EMU_MAXABS, o_bound)), res
    assert np.all(lerr <= np.maximum(LSE_SCORES_NATS, l_bound)), res
    assert res["rms"] <= TOL_EMU_RMS, res
    return res


def output_error_bound(codes, o, vc, dv, o_ref):
    """Per-element bound on |O_gpu - O_emu| and |LSE_gpu - LSE_emu| when the kernel and the
    emulation use the same codes and exponents: the PV and row-sum MFMAs carry
    MFMA_ERR_PER_CHUNK of the largest product of each 64-key block (times its 2^-o), O is
    rounded to bf16 (2^-9 relative, 2^-8 taken), plus 2^-20 relative for the fp32 rescales.
    codes [n, S] and o [n, S/64] in the emulation's row order (all rows of each (b, h));
    vc: e4m3 codes [B, S, H, d_v] with H query heads; o_ref: the emulation's O [n, d_v]."""
    t = oracle.e4m3_table()
    B, S, H, dvd = vc.shape
    P = t[codes].reshape(B, H, S, S)
    scale = np.where(o == 255, 0.0, np.exp2(-o.astype(np.float64))).reshape(B, H, S, S // 64)
    pv_err = np.zeros((B, H, S, dvd))
    l_err = np.zeros((B, H, S))
    l = np.zeros((B, H, S))
    for b in range(B):
        for h in range(H):
            V = np.abs(t[vc[b, :, h]])
            for n in range(S // 64):
                blk = P[b, h][:, 64 * n:64 * n + 64]
                sc = scale[b, h, :, n][:, None]
                pv_err[b, h] += sc * (blk[:, :, None] * V[None, 64 * n:64 * n + 64]).max(axis=1)
                l_err[b, h] += sc[:, 0] * blk.max(axis=1)
                l[b, h] += sc[:, 0] * blk.sum(axis=1)
    pv_err = (MFMA_ERR_PER_CHUNK * pv_err).reshape(B * H * S, dvd)
    l_rel = (MFMA_ERR_PER_CHUNK * l_err / l).reshape(B * H * S)
    l = l.reshape(B * H * S)
    o_bound = dv * pv_err / l[:, None] + np.abs(o_ref) * (l_rel[:, None] + 2.0 ** -8 + 2.0 ** -20)
    l_bound = l_rel + 1e-5
    return o_bound, l_bound


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
