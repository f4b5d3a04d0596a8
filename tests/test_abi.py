"""CPU tests of the C ABI: the library loads, exports every declared symbol, rejects
bad arguments on the host before any device call, and its persistent-grid schedule
covers every query tile exactly once with balanced work (paper Sec. IV-A, causal
pairing).  Only invalid arguments are passed here, so nothing is ever launched."""
import ctypes
import math
import os
import re

import numpy as np
import pytest

import bf16_causal_flashattention_amd as cfa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    names = []
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            txt = open(os.path.join(ROOT, "include", fn)).read()
            names += re.findall(r"^\s*(?:int|int64_t|const char\s*\*)\s+(attn_\w+)\s*\(", txt, re.M)
    return names


def test_exports_every_declared_symbol():
    names = _declared()
    assert len(names) >= 9
    L = ctypes.CDLL(cfa.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n


FAKE = ctypes.c_void_p(1 << 20)       # never dereferenced: validation fails first
MISALIGNED = ctypes.c_void_p((1 << 20) + 8)


def _fp8(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, lse=None, qd=1.0, kd=1.0, vd=1.0, sm=0.1, B=1, H=1, S=256,
             dqk=128, dv=128)
    a.update(kw)
    return cfa.lib().attn_fwd_causal_fp8(a["q"], a["k"], a["v"], a["out"], a["lse"], a["qd"], a["kd"], a["vd"],
                                         a["sm"], a["B"], a["H"], a["S"], a["dqk"], a["dv"], None)


def _bf16(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, lse=None, sm=0.1, B=1, H=1, S=256, dqk=128, dv=128)
    a.update(kw)
    return cfa.lib().attn_fwd_causal_bf16(a["q"], a["k"], a["v"], a["out"], a["lse"], a["sm"], a["B"], a["H"],
                                          a["S"], a["dqk"], a["dv"], None)


def _mla(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, lse=None, qd=1.0, kd=1.0, vd=1.0, sm=0.1, B=1, H=1, S=256,
             dqk=192, dv=128)
    a.update(kw)
    return cfa.lib().attn_fwd_causal_mla(a["q"], a["k"], a["v"], a["out"], a["lse"], a["qd"], a["kd"], a["vd"],
                                         a["sm"], a["B"], a["H"], a["S"], a["dqk"], a["dv"], None)


@pytest.mark.parametrize("call", [_fp8, _bf16, _mla])
def test_validation_errors(call):
    assert call(q=None) == -1
    assert call(out=None) == -1
    assert call(S=300) == -2
    assert call(S=128) == -2
    assert call(S=-256) == -2
    assert call(B=-1) == -2
    assert call(dv=64) == -2
    assert call(q=MISALIGNED) == -3
    assert call(out=MISALIGNED) == -3
    assert call(lse=ctypes.c_void_p((1 << 20) + 2)) == -3
    assert call(B=1, H=1 << 14, S=1 << 20) == -4
    assert call(sm=float("nan")) == -5
    assert call(sm=0.0) == -5
    assert call(sm=float("inf")) == -5


@pytest.mark.parametrize("call", [_fp8, _mla])
def test_validation_errors_descales(call):
    assert call(qd=0.0) == -5
    assert call(kd=-1.0) == -5
    assert call(vd=float("nan")) == -5


def _st(b, h, s):
    return ctypes.byref(cfa.Strides(b, h, s))


def _fp8_ex(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, lse=None, qd=1.0, kd=1.0, vd=1.0, sm=0.1, B=1, H=4, Hkv=2, S=256,
             dqk=128, dv=128, sq=None, sk=None, sv=None, so=None, pm=-1)
    a.update(kw)
    return cfa.lib().attn_fwd_causal_fp8_ex(a["q"], a["k"], a["v"], a["out"], a["lse"], a["qd"], a["kd"], a["vd"],
                                            a["sm"], a["B"], a["H"], a["Hkv"], a["S"], a["dqk"], a["dv"], a["sq"],
                                            a["sk"], a["sv"], a["so"], a["pm"], None)


def _fp8_vt(**kw):
    # channel-major V: the v strides are (batch, head, channel row), keys contiguous
    a = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, lse=None, qd=1.0, kd=1.0, vd=1.0, sm=0.1, B=1, H=4, Hkv=2, S=256,
             dqk=128, dv=128, sq=None, sk=None, sv=None, so=None, pm=-1)
    a.update(kw)
    return cfa.lib().attn_fwd_causal_fp8_vt(a["q"], a["k"], a["v"], a["out"], a["lse"], a["qd"], a["kd"], a["vd"],
                                            a["sm"], a["B"], a["H"], a["Hkv"], a["S"], a["dqk"], a["dv"], a["sq"],
                                            a["sk"], a["sv"], a["so"], a["pm"], None)


def _bf16_ex(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, lse=None, sm=0.1, B=1, H=4, Hkv=2, S=256, dqk=128, dv=128,
             sq=None, sk=None, sv=None, so=None)
    a.update(kw)
    return cfa.lib().attn_fwd_causal_bf16_ex(a["q"], a["k"], a["v"], a["out"], a["lse"], a["sm"], a["B"], a["H"],
                                             a["Hkv"], a["S"], a["dqk"], a["dv"], a["sq"], a["sk"], a["sv"],
                                             a["so"], None)


@pytest.mark.parametrize("call", [_fp8_ex, _fp8_vt, _bf16_ex])
def test_ex_validation_errors(call):
    assert call(q=None) == -1
    assert call(Hkv=3) == -2             # H_kv must divide H
    assert call(Hkv=0) == -2
    assert call(Hkv=-1) == -2
    assert call(S=384) == -2
    assert call(dv=64) == -2
    assert call(sq=_st(-1, 128, 512)) == -5                  # negative stride
    assert call(sk=_st(65536, 130, 256)) == -3               # head stride not 16-byte aligned
    assert call(so=_st(1 << 31, 128, 512)) == -4             # batch stride beyond 2^31
    assert call(sv=_st(1 << 20, 1 << 27, 1 << 24)) == -4     # 128 rows of the seq stride beyond 2^31 bytes
    assert call(B=0, q=None, k=None, v=None, out=None) == 0  # empty problem
    assert call(sm=0.0) == -5


@pytest.mark.parametrize("call", [_fp8_ex, _fp8_vt, _bf16_ex])
def test_out_rows_must_not_overlap(call):
    # the rows of out must be disjoint: expanded (zero-stride) and interleaved views are refused
    B, H, S = 2, 4, 256
    assert call(B=B, H=H, so=_st(S * H * 128, 0, H * 128)) == -5     # every head writes the same row
    assert call(B=B, H=H, so=_st(S * H * 128, 128, 0)) == -5         # every position writes the same row
    assert call(B=B, H=H, so=_st(0, 128, H * 128)) == -5             # both batches write the same rows
    assert call(B=B, H=H, so=_st(S * H * 128, 128, 64)) == -5        # a row overlaps the next position's
    assert call(B=B, H=H, so=_st(S * H * 128, 128, 128)) == -5       # heads and positions interleaved
    assert call(B=B, H=H, so=_st(S * H * 128 - 128, 128, H * 128)) == -5  # batches overlap by one row


def test_vt_strides_checked_channel_major():
    # the channel-major V tensor is [B][H_kv][128][S]: its third stride steps between channel rows
    assert _fp8_vt(sv=_st(2 * 128 * 256, 128 * 256, 40)) == -3        # channel stride not 16-byte aligned
    assert _fp8_vt(sv=_st(0, 3 << 29, 1 << 23)) == -4                 # last channel row beyond 2^31
    assert _fp8_vt(S=1 << 17, H=2, Hkv=2, sv=_st(0, 1 << 30, 1 << 24)) == -4  # 128 channel rows beyond 2^31
    assert _fp8_vt(pm=2) == -5
    assert _fp8_vt(dqk=64) == -2


def test_ex_p_mode_and_head_dims():
    assert _fp8_ex(pm=2) == -5
    assert _fp8_ex(pm=-2) == -5
    assert _fp8_ex(dqk=192, pm=5) == -5
    assert _fp8_ex(dqk=64) == -2
    assert _bf16_ex(dqk=64) == -2
    assert _bf16_ex(dqk=192, dv=64) == -2


def test_ex_bhsd_extent_checked():
    # BHSD strides whose last element offset reaches 2^31 are rejected before any launch
    B, H, S, D = 2, 64, 1 << 17, 128   # 2^31 elements in total
    bhsd = _st(H * S * D, S * D, D)
    assert _fp8_ex(B=B, H=H, Hkv=H, S=S, sq=bhsd) == -4


def test_head_dims_per_entry_point():
    assert _fp8(dqk=192) == -2
    assert _mla(dqk=128) == -2
    assert _bf16(dqk=192) == -2


@pytest.mark.parametrize("call", [_fp8, _bf16, _mla])
def test_empty_problem_is_noop(call):
    # zero-sized problems return ok without touching the device, even with null pointers
    assert call(B=0, q=None, k=None, v=None, out=None) == 0
    assert call(H=0, q=None, k=None, v=None, out=None) == 0
    assert call(S=0, q=None, k=None, v=None, out=None) == 0


def test_prep_validation():
    L = cfa.lib()
    assert L.attn_quantize_e4m3(FAKE, -1, FAKE, FAKE, FAKE, None) == -5
    assert L.attn_quantize_e4m3(None, 16, FAKE, FAKE, FAKE, None) == -1
    assert L.attn_quantize_e4m3(FAKE, 16, FAKE, None, FAKE, None) == -1
    assert L.attn_quantize_e4m3(MISALIGNED, 16, FAKE, FAKE, FAKE, None) == -3
    assert L.attn_round_bf16(FAKE, -3, FAKE, None) == -5
    assert L.attn_round_bf16(None, 3, FAKE, None) == -1
    assert L.attn_round_bf16(FAKE, 0, None, None) == 0


def test_key_mean_noalloc_validation():
    L = cfa.lib()
    assert L.attn_key_mean_noalloc(FAKE, 1, 1 << 17, 64, 128, FAKE, None) == -8   # 8 MiB of partials > 4 MiB
    assert L.attn_key_mean_noalloc(FAKE, 2, 1 << 16, 33, 128, FAKE, None) == -8   # 4.1 MiB
    assert L.attn_key_mean_noalloc(FAKE, 1, 256, 1, 96, FAKE, None) == -2
    assert L.attn_key_mean_noalloc(FAKE, 1, 0, 1, 128, FAKE, None) == -2
    assert L.attn_key_mean_noalloc(None, 0, 256, 1, 128, None, None) == 0
    assert L.attn_key_mean_noalloc(None, 1, 256, 1, 128, FAKE, None) == -1
    assert L.attn_key_mean_noalloc(FAKE, 1, 256, 1, 128, ctypes.c_void_p((1 << 20) + 2), None) == -3
    assert cfa.lib().attn_status_string(-8).decode().startswith("problem needs more scratch")


def test_rotation_prepass_validation():
    L = cfa.lib()
    odd = ctypes.c_void_p((1 << 20) + 2)  # not 4-byte aligned
    assert L.attn_key_mean_workspace(2, 1500, 3, 128) == 2 * 3 * 2 * 128 * 8  # two chunks of 1024 keys, fp64
    assert L.attn_key_mean_workspace(1, 256, 1, 64) == -2
    assert L.attn_key_mean(FAKE, 1, 256, 1, 96, FAKE, FAKE, None) == -2
    assert L.attn_key_mean(FAKE, 1, 0, 1, 128, FAKE, FAKE, None) == -2
    assert L.attn_key_mean(None, 0, 256, 1, 128, None, None, None) == 0
    assert L.attn_key_mean(None, 1, 256, 1, 128, FAKE, FAKE, None) == -1
    assert L.attn_key_mean(odd, 1, 256, 1, 128, FAKE, FAKE, None) == -3
    assert L.attn_key_mean(FAKE, 1, 256, 1, 128, FAKE, ctypes.c_void_p((1 << 20) + 4), None) == -3
    assert L.attn_key_mean(FAKE, 1 << 14, 256, 8, 128, FAKE, FAKE, None) == -4
    rq = L.attn_rotate_quantize_e4m3
    assert rq(FAKE, None, FAKE, 1, 256, 1, 64, FAKE, FAKE, FAKE, None) == -2
    assert rq(FAKE, None, FAKE, -1, 256, 1, 128, FAKE, FAKE, FAKE, None) == -2
    assert rq(FAKE, None, None, 1, 256, 1, 128, FAKE, FAKE, FAKE, None) == -1
    assert rq(None, None, FAKE, 1, 256, 1, 128, FAKE, FAKE, FAKE, None) == -1
    assert rq(FAKE, odd, FAKE, 1, 256, 1, 192, FAKE, FAKE, FAKE, None) == -3
    assert rq(FAKE, None, FAKE, 1 << 10, 1 << 12, 8, 128, FAKE, FAKE, FAKE, None) == -4
    # empty tensors with no heads: nothing to rotate, and no host division by B*H
    assert rq(None, None, FAKE, 0, 256, 0, 128, None, FAKE, FAKE, None) in (0, -6, -7)
    assert rq(None, None, FAKE, 2, 256, 0, 192, None, FAKE, FAKE, None) in (0, -6, -7)
    rs = L.attn_rotate_quantize_e4m3_static
    for bad in (0.0, 3.0, -0.5, 2.0 ** 127, 2.0 ** -127, float("inf"), float("nan")):
        assert rs(FAKE, None, FAKE, 1, 256, 1, 128, bad, FAKE, None) == -5, bad
        assert L.attn_quantize_e4m3_static(FAKE, 16, bad, FAKE, None) == -5, bad
    assert rs(FAKE, None, FAKE, 1, 256, 1, 96, 1.0, FAKE, None) == -2
    assert rs(FAKE, None, None, 1, 256, 1, 128, 1.0, FAKE, None) == -1
    assert rs(FAKE, None, FAKE, 1, 256, 1, 128, 1.0, None, None) == -1
    assert rs(None, None, FAKE, 0, 256, 1, 128, 2.0 ** -126, None, None) == 0
    assert L.attn_quantize_e4m3_static(MISALIGNED, 16, 1.0, FAKE, None) == -3
    assert L.attn_quantize_e4m3_static(FAKE, -1, 1.0, FAKE, None) == -5
    assert L.attn_quantize_e4m3_static(None, 0, 2.0 ** 126, None, None) == 0


def test_status_strings():
    L = cfa.lib()
    for c in range(-7, 1):
        assert L.attn_status_string(c)
    assert b"unknown" in L.attn_status_string(-99)


@pytest.mark.parametrize("B,H,Hkv,S,grid", [(1, 1, 1, 256, 1), (1, 32, 32, 32768, 256), (2, 3, 3, 1280, 7),
                                            (1, 16, 16, 32768, 256), (4, 5, 5, 2048, 13), (1, 1, 1, 768, 256),
                                            (3, 2, 2, 2560, 256), (1, 32, 8, 32768, 256), (2, 6, 3, 1280, 7),
                                            (1, 2, 1, 256, 1), (3, 8, 2, 2560, 256), (1, 6, 2, 768, 5),
                                            (2, 4, 4, 512, 3)])
def test_schedule_covers_every_tile_once(B, H, Hkv, S, grid):
    """Every 128-row strip of every (b, h) is processed exactly once; workgroups get balanced
    work; each item is a causal pair (j, T-1-j) of one head, or of the two heads 2u, 2u+1 of a
    head pair with 128-row tiles when H / Hkv is even (ZYFA paper, Sec. IV-A)."""
    pair = (H // Hkv) % 2 == 0
    R = 128 if pair else 256
    T = S // R
    g = min(grid, cfa.default_grid(B, H, S, grid, Hkv=Hkv))
    rec = cfa.schedule(B, H, S, g, Hkv=Hkv)
    assert rec.shape[0] == B * H * T
    assert np.all(rec[:, 4] == R) and np.all(rec[:, 3] % R == 0)
    seen = np.zeros((B, H, S // 128), dtype=np.int64)
    for r in range(R // 128):
        np.add.at(seen, (rec[:, 1], rec[:, 2], rec[:, 3] // 128 + r), 1)
    assert np.all(seen == 1)
    # a tile of R rows at tile index t takes (t+1) R / 128 steps of 128 keys; in the head-pair
    # mode its two records (one per head) share those steps
    steps = (rec[:, 3] // R + 1) * (R // 128)
    share = 0.5 if pair else 1.0
    work = np.zeros(g, dtype=np.float64)
    np.add.at(work, rec[:, 0], steps * share)
    hs = H // 2 if pair else H
    items = B * hs * ((T + 1) // 2)
    per = math.ceil(items / g)
    assert work.max() <= per * (T + 1) * (R // 128)
    # consecutive tiles of a workgroup: (j, T-1-j), for one head or for the heads 2u, 2u+1
    n = 2 if pair else 1
    for wg in range(min(g, 4)):
        r = rec[rec[:, 0] == wg]
        assert len(r) % n == 0
        tiles = r[::n]
        for e in range(1, n):  # the second head of each pair tile
            assert np.all(r[e::n, 2] == tiles[:, 2] + e) and np.all(r[e::n, 3] == tiles[:, 3])
            assert np.all(tiles[:, 2] % 2 == 0)
        i = 0
        while i < len(tiles):
            t = tiles[i, 3] // R
            if t == T - 1 - t:  # middle tile of an odd T runs alone
                i += 1
                continue
            nxt = tiles[i + 1]
            assert nxt[3] // R == T - 1 - t and nxt[1] == tiles[i, 1] and nxt[2] == tiles[i, 2]
            i += 2


@pytest.mark.parametrize("Hkv", [32, 8])
def test_xcd_remap_is_contiguous_per_chiplet(Hkv):
    # workgroup i runs on chiplet i % 8; its first item should be a contiguous run per chiplet
    B, H, S, g = 1, 32, 32768, 256
    rec = cfa.schedule(B, H, S, g, Hkv=Hkv)
    first = {}
    for wg, b, h, r0, rows in rec:
        if wg not in first:
            first[wg] = h
    for x in range(8):
        heads = {first[wg] for wg in range(x, g, 8)}
        assert len(heads) == 1  # 32 workgroups of one chiplet start on one head (head pair)


def test_default_grid():
    assert cfa.default_grid(1, 32, 32768, 256) == 256
    assert cfa.default_grid(1, 1, 256, 256) == 1
    assert cfa.default_grid(1, 1, 300, 256) == -2
    assert cfa.default_grid(1, 2, 256, 256, Hkv=1) == 1  # one head pair, one 128-row tile pair
    assert cfa.default_grid(1, 4, 512, 256, Hkv=3) == -2  # H not a multiple of H_kv


def test_binding_rejects_host_tensors_before_any_call():
    """The Python binding refuses tensors that are not on the GPU (here: all on the host),
    so no host pointer ever reaches a kernel."""
    import torch
    q = torch.zeros((1, 256, 1, 128), dtype=torch.uint8)
    with pytest.raises((ValueError, TypeError)):
        cfa.attn_fwd_causal_fp8_ex(q, q, q, 1.0, 1.0, 1.0)
    with pytest.raises((ValueError, TypeError)):
        cfa.attn_fwd_causal_fp8(q, q, q, 1.0, 1.0, 1.0)
    with pytest.raises((ValueError, TypeError)):
        cfa.attn_fwd_causal_fp8_vt(q, q, q.view(1, 1, 128, 256), 1.0, 1.0, 1.0)
    b = torch.zeros((1, 256, 1, 128), dtype=torch.bfloat16)
    with pytest.raises((ValueError, TypeError)):
        cfa.attn_fwd_causal_bf16_ex(b, b, b)
    x = torch.zeros((1, 256, 1, 128), dtype=torch.float32)
    for fn in (lambda: cfa.quantize_e4m3(x), lambda: cfa.round_bf16(x), lambda: cfa.key_mean(x),
               lambda: cfa.quantize_e4m3_static(x, 1.0), lambda: cfa.rotate_quantize_e4m3(x, torch.ones(128))):
        with pytest.raises((ValueError, TypeError)):
            fn()
