"""CPU oracle for causal attention forward with FP8 e4m3 / BF16 operands.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product library
(``bf16_causal_flashattention_amd``) never imports it and shares no code with it.

The arithmetic lives in ``oracle.c`` (plain C, fp64 unless it mirrors the fp32
decisions of a kernel); this module only marshals numpy arrays through ctypes.
Every function names the passage of "ZYFA: Speed and Accuracy of FP8
FlashAttention on AMD CDNA4" (arXiv:2611.07496) that it follows.

Pins (what ties each function to something other than itself) live in
``tests/test_oracle_*.py``.  Functions without an external pin: none.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

# Paper values (Sec. IV-A, IV-B1, IV-B2): shift sigma = 6, bias beta = 0.35,
# scale blocks of 64 keys, lazy threshold tau = 0.125 in FP8.
SIGMA = 6
BETA = 0.35
SCALE_BLOCK = 64
TAU_FP8 = 0.125


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (IEEE semantics, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
               "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        L = ctypes.CDLL(_LIB)
        L.orc_e4m3_value.restype = ctypes.c_double
        L.orc_e4m3_value.argtypes = [ctypes.c_int]
        L.orc_e4m3_rne.restype = ctypes.c_int
        L.orc_e4m3_rne.argtypes = [ctypes.c_double]
        L.orc_bf16_rne.restype = ctypes.c_uint16
        L.orc_bf16_rne.argtypes = [ctypes.c_float]
        L.orc_quantize_e4m3.restype = ctypes.c_float
        L.orc_quantize_e4m3.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
        L.orc_quantize_e4m3_f64.restype = ctypes.c_float
        L.orc_quantize_e4m3_f64.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
        L.orc_leanp_code.restype = ctypes.c_int
        L.orc_leanp_code.argtypes = [ctypes.c_double, ctypes.c_int, ctypes.c_double]
        L.orc_exactp_code.restype = ctypes.c_int
        L.orc_exactp_code.argtypes = [ctypes.c_double, ctypes.c_int]
        L.orc_attn_exact.restype = ctypes.c_int
        L.orc_attn_exact.argtypes = [ctypes.c_int] + [ctypes.c_void_p] * 3 + [ctypes.c_double] * 4 + \
            [ctypes.c_int] * 5 + [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
        L.orc_emulate_fp8.restype = ctypes.c_int
        L.orc_emulate_fp8.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_float] * 4 + [ctypes.c_int] * 5 + \
            [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64] + [ctypes.c_void_p] * 8
        L.orc_emulate_fp8_scores.restype = ctypes.c_int
        L.orc_emulate_fp8_scores.argtypes = [ctypes.c_void_p] * 2 + [ctypes.c_float] * 4 + [ctypes.c_int] * 4 + \
            [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64] + [ctypes.c_void_p] * 8
        L.orc_e4m3_rne_array.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
        L.orc_bf16_rne_array.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


# --------------------------------------------------------------------------- codecs
def e4m3_value(code: int) -> float:
    """Value of one e4m3 code (paper Sec. II-C and footnote 5; OCP e4m3fn, bias 7)."""
    return lib().orc_e4m3_value(int(code))


def e4m3_table() -> np.ndarray:
    """Values of all 256 codes (NaN for 0x7F and 0xFF)."""
    return np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def e4m3_rne(x) -> np.ndarray:
    """Round reals to e4m3 codes, nearest-even, saturating at 448."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float64).reshape(-1))
    out = np.empty(x.size, dtype=np.uint8)
    lib().orc_e4m3_rne_array(_ptr(x), x.size, _ptr(out))
    return out


def bf16_rne(x) -> np.ndarray:
    """Round fp32 values to bf16 bit patterns (uint16), nearest-even."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    out = np.empty(x.shape, dtype=np.uint16)
    lib().orc_bf16_rne_array(_ptr(x), x.size, _ptr(out))
    return out


def bf16_value(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def quantize_e4m3(x: np.ndarray):
    """Per-tensor power-of-two quantiser (paper Sec. V-E, footnote 17).

    Returns (codes uint8 with x's shape, descale float)."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    codes = np.empty(x.shape, dtype=np.uint8)
    ds = lib().orc_quantize_e4m3(_ptr(x), x.size, _ptr(codes))
    return codes, float(ds)


def quantize_e4m3_f64(x: np.ndarray):
    """The per-tensor quantiser on fp64 values (no fp32 rounding before the e4m3 rounding)."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    codes = np.empty(x.shape, dtype=np.uint8)
    ds = lib().orc_quantize_e4m3_f64(_ptr(x), x.size, _ptr(codes))
    return codes, float(ds)


def static_exponent(descale: float) -> int:
    """k with descale = 2^-k, for a power-of-two descale in [2^-126, 2^126]."""
    m, e = math.frexp(float(descale))
    if m != 0.5 or not -126 <= 1 - e <= 126:
        raise ValueError(f"descale {descale!r} is not a power of two in [2^-126, 2^126]")
    return 1 - e


def quantize_e4m3_static(x: np.ndarray, descale: float) -> np.ndarray:
    """The quantiser with a given (static) power-of-two descale instead of one from the
    tensor's maximum (paper Sec. V-E: the fused quantisation pass uses a static scale
    set from calibration, footnote 17 on power-of-two descales): codes are
    e4m3_rne(x / descale), so scaled values beyond 448 saturate to +-448."""
    k = static_exponent(descale)
    x = np.asarray(x, dtype=np.float64)
    return e4m3_rne(np.ldexp(x, k)).reshape(x.shape)


# ----------------------------------------------------------------------------- rotation
# Paper Sec. V-E, "Rotation and K smoothing": after RoPE, Q and K are multiplied by the
# same orthogonal R = diag(s) (C_m kron H_{D/m}), s random signs, H the normalised
# Sylvester-Hadamard matrix, C_m the orthonormal DCT-II; m = 1 for D = 128 and m = 3 for
# D = 192.  K smoothing subtracts the mean key of each head over the sequence before the
# rotation.  FP8 scales are taken after the rotation; V and O are not rotated.
# Reading of the Kronecker indices: element (a, b) -> (a', b') of C kron H is
# C[a, a'] H[b, b'] with a row/column index a*(D/m) + b, and C[k, n] is the DCT-II
# coefficient of frequency k at sample n (the matrix used as the left factor of kron).

def hadamard(n: int) -> np.ndarray:
    """Normalised Sylvester-Hadamard matrix of size n (a power of two), fp64."""
    assert n >= 1 and n & (n - 1) == 0
    h = np.ones((1, 1))
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h / np.sqrt(n)


def dct2(m: int) -> np.ndarray:
    """Orthonormal DCT-II matrix C[k, n] = a_k cos(pi (2n + 1) k / (2m)), a_0 = sqrt(1/m),
    a_k = sqrt(2/m) otherwise."""
    k = np.arange(m)[:, None]
    n = np.arange(m)[None, :]
    a = np.where(k == 0, np.sqrt(1.0 / m), np.sqrt(2.0 / m))
    return a * np.cos(np.pi * (2 * n + 1) * k / (2 * m))


def rotation(signs) -> np.ndarray:
    """R = diag(signs) (C_m kron H_{D/m}) with m = 1 when D is a power of two, else 3."""
    s = np.asarray(signs, dtype=np.float64)
    D = s.size
    m = 1 if D & (D - 1) == 0 else 3
    assert D % m == 0 and (D // m) & (D // m - 1) == 0
    return np.diag(s) @ np.kron(dct2(m), hadamard(D // m))


def key_mean(k: np.ndarray) -> np.ndarray:
    """Mean key of each head over the sequence: k [B][S][H][D] -> [B][H][D], fp64."""
    return np.asarray(k, dtype=np.float64).mean(axis=1)


def rotate(x: np.ndarray, signs, mean: np.ndarray = None) -> np.ndarray:
    """(x - mean) R for x [B][S][H][D] (mean [B][H][D] or None), fp64."""
    y = np.asarray(x, dtype=np.float64)
    if mean is not None:
        y = y - np.asarray(mean, dtype=np.float64)[:, None, :, :]
    return y @ rotation(signs)


def rotate_quantize_e4m3(x: np.ndarray, signs, mean: np.ndarray = None):
    """Rotation (and optional K smoothing) in fp64, then the per-tensor quantiser."""
    return quantize_e4m3_f64(rotate(x, signs, mean))


def rotate_quantize_e4m3_static(x: np.ndarray, signs, descale: float, mean: np.ndarray = None) -> np.ndarray:
    """Rotation (and optional K smoothing) in fp64, then the static-scale quantiser."""
    return quantize_e4m3_static(rotate(x, signs, mean), descale)


def leanp_code(x: float, sigma: int = SIGMA, beta: float = BETA) -> int:
    """Lean-P code for x = log2 p (paper Sec. IV-B1, Eq. 2), fp64 arithmetic."""
    return lib().orc_leanp_code(float(x), int(sigma), float(beta))


def exactp_code(x: float, sigma: int = SIGMA) -> int:
    """Exact-P code: e4m3 rounding of 2^(x + sigma) (paper Sec. IV-B1)."""
    return lib().orc_exactp_code(float(x), int(sigma))


# --------------------------------------------------------------------------- attention
def attn_exact(q, k, v, *, dtype: str, c: float, dq: float = 1.0, dk: float = 1.0, dv: float = 1.0,
               rows=None):
    """Exact causal softmax attention in fp64 (paper Sec. II-B, Eq. for O and the LSE).

    q, k: [B, S, H, d_qk], v: [B, S, H, d_v] as e4m3 codes (uint8, dtype="fp8", values
    are code * descale) or bf16 bit patterns (uint16, dtype="bf16").  rows: int64
    array of (b, h, i) triples (default: every row).  Returns (out [n, d_v] fp64,
    lse [n] fp64, natural-log units)."""
    q = np.ascontiguousarray(q); k = np.ascontiguousarray(k); v = np.ascontiguousarray(v)
    B, S, H, dqk = q.shape
    dvd = v.shape[3]
    assert k.shape == (B, S, H, dqk) and v.shape[:3] == (B, S, H)
    if dtype == "fp8":
        assert q.dtype == np.uint8 and k.dtype == np.uint8 and v.dtype == np.uint8
        dt = 0
    elif dtype == "bf16":
        assert q.dtype == np.uint16 and k.dtype == np.uint16 and v.dtype == np.uint16
        dt = 1
    else:
        raise ValueError(dtype)
    if rows is None:
        bb, hh, ii = np.meshgrid(np.arange(B), np.arange(H), np.arange(S), indexing="ij")
        rows = np.stack([bb.ravel(), hh.ravel(), ii.ravel()], axis=1)
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1, 3))
    n = rows.shape[0]
    out = np.empty((n, dvd), dtype=np.float64)
    lse = np.empty(n, dtype=np.float64)
    rc = lib().orc_attn_exact(dt, _ptr(q), _ptr(k), _ptr(v), dq, dk, dv, c, B, H, S, dqk, dvd,
                              _ptr(rows), n, _ptr(out), _ptr(lse))
    if rc != 0:
        raise ValueError("orc_attn_exact: bad row index")
    return out, lse


class _Params(ctypes.Structure):
    _fields_ = [("n_tile", ctypes.c_int), ("group", ctypes.c_int), ("tau", ctypes.c_float),
                ("sigma", ctypes.c_int), ("beta", ctypes.c_float), ("block", ctypes.c_int),
                ("exact_p", ctypes.c_int), ("ideal", ctypes.c_int), ("scale_blocks", ctypes.c_int),
                ("rounded_sum", ctypes.c_int)]


@dataclass
class Fp8Scheme:
    """Parameters of the FP8 scheme (paper Sec. IV-A, IV-B).

    n_tile: keys per running-max update; group: rows sharing one lazy decision
    (the rows of one wave); tau: lazy threshold in base-2 units; exact_p: exact P
    instead of lean P; ideal: exact final row max in fp64 instead of the mirrored
    fp32 trajectory; scale_blocks / rounded_sum: switch off per-block scaling or the
    rounded-sum normaliser to model the variants the paper contrasts."""
    n_tile: int = 128
    group: int = 32
    tau: float = TAU_FP8
    sigma: int = SIGMA
    beta: float = BETA
    block: int = SCALE_BLOCK
    exact_p: bool = False
    ideal: bool = False
    scale_blocks: bool = True
    rounded_sum: bool = True

    def c(self):
        return _Params(self.n_tile, self.group, self.tau, self.sigma, self.beta, self.block,
                       int(self.exact_p), int(self.ideal), int(self.scale_blocks), int(self.rounded_sum))


def emulate_fp8(q, k, v, *, dq: float, dk: float, dv: float, c: float, scheme: Fp8Scheme = None,
                groups=None, debug: bool = False):
    """Step-by-step emulation of the FP8 scheme (paper Sec. IV-A, IV-B1-B3).

    q, k, v: e4m3 codes [B, S, H, d].  groups: int64 (b, h, r0) triples, each a group
    of ``scheme.group`` consecutive rows (default: all groups).  Returns a dict with
    ``out`` [n_groups*group, d_v] fp64 (O before bf16 rounding), ``out_bf16`` (uint16),
    ``lse``; with debug=True also ``o`` (per row and 64-key block, 255 = unseen),
    ``codes`` (per row and key), ``ymargin``, ``omargin`` and ``lazy_margin``."""
    scheme = scheme or Fp8Scheme()
    q = np.ascontiguousarray(q, dtype=np.uint8)
    k = np.ascontiguousarray(k, dtype=np.uint8)
    v = np.ascontiguousarray(v, dtype=np.uint8)
    B, S, H, dqk = q.shape
    dvd = v.shape[3]
    G = scheme.group
    if groups is None:
        bb, hh, rr = np.meshgrid(np.arange(B), np.arange(H), np.arange(0, S, G), indexing="ij")
        groups = np.stack([bb.ravel(), hh.ravel(), rr.ravel()], axis=1)
    groups = np.ascontiguousarray(np.asarray(groups, dtype=np.int64).reshape(-1, 3))
    ng = groups.shape[0]
    nrow = ng * G
    nblk = (S + scheme.block - 1) // scheme.block
    ntile = (S + scheme.n_tile - 1) // scheme.n_tile
    res = {
        "out": np.empty((nrow, dvd), dtype=np.float64),
        "out_bf16": np.empty((nrow, dvd), dtype=np.uint16),
        "lse": np.empty(nrow, dtype=np.float64),
    }
    if debug:
        res["o"] = np.full((nrow, nblk), 255, dtype=np.uint8)  # 255: block never visited
        res["codes"] = np.zeros((nrow, S), dtype=np.uint8)
        res["ymargin"] = np.full((nrow, S), np.inf, dtype=np.float32)
        res["omargin"] = np.full((nrow, nblk), np.inf, dtype=np.float32)
        res["lazy_margin"] = np.full((ng, ntile), np.inf, dtype=np.float32)
    prm = scheme.c()
    rc = lib().orc_emulate_fp8(
        _ptr(q), _ptr(k), _ptr(v), dq, dk, dv, c, B, H, S, dqk, dvd, ctypes.byref(prm), _ptr(groups), ng,
        _ptr(res["out"]), _ptr(res["out_bf16"]), _ptr(res["lse"]),
        _ptr(res.get("o")), _ptr(res.get("codes")), _ptr(res.get("ymargin")), _ptr(res.get("omargin")),
        _ptr(res.get("lazy_margin")))
    if rc != 0:
        raise RuntimeError(f"orc_emulate_fp8 failed: {rc}")
    res["groups"] = groups
    return res


def emulate_fp8_from_scores(scores, v, *, dq: float, dk: float, dv: float, c: float, scheme: Fp8Scheme = None,
                            groups=None, debug: bool = False):
    """The FP8 scheme of ``emulate_fp8`` (paper Sec. IV-A, IV-B1-B3) run on given raw fp32
    scores instead of the exact dot products of q and k.

    scores: float32 [B*H*S, S], row (b*H + h)*S + i holding the raw scores of query i of
    head (b, h) (entries j > i are not read); v: e4m3 codes [B, S, H, d_v].  For checking the
    decisions of a kernel given the scores it computed; the parity gates use ``emulate_fp8``.
    Returns the dict of ``emulate_fp8``."""
    scheme = scheme or Fp8Scheme()
    v = np.ascontiguousarray(v, dtype=np.uint8)
    B, S, H, dvd = v.shape
    scores = np.ascontiguousarray(scores, dtype=np.float32)
    assert scores.shape == (B * H * S, S)
    G = scheme.group
    if groups is None:
        bb, hh, rr = np.meshgrid(np.arange(B), np.arange(H), np.arange(0, S, G), indexing="ij")
        groups = np.stack([bb.ravel(), hh.ravel(), rr.ravel()], axis=1)
    groups = np.ascontiguousarray(np.asarray(groups, dtype=np.int64).reshape(-1, 3))
    ng = groups.shape[0]
    nrow = ng * G
    nblk = (S + scheme.block - 1) // scheme.block
    ntile = (S + scheme.n_tile - 1) // scheme.n_tile
    res = {
        "out": np.empty((nrow, dvd), dtype=np.float64),
        "out_bf16": np.empty((nrow, dvd), dtype=np.uint16),
        "lse": np.empty(nrow, dtype=np.float64),
    }
    if debug:
        res["o"] = np.full((nrow, nblk), 255, dtype=np.uint8)
        res["codes"] = np.zeros((nrow, S), dtype=np.uint8)
        res["ymargin"] = np.full((nrow, S), np.inf, dtype=np.float32)
        res["omargin"] = np.full((nrow, nblk), np.inf, dtype=np.float32)
        res["lazy_margin"] = np.full((ng, ntile), np.inf, dtype=np.float32)
    prm = scheme.c()
    rc = lib().orc_emulate_fp8_scores(
        _ptr(scores), _ptr(v), dq, dk, dv, c, B, H, S, dvd, ctypes.byref(prm), _ptr(groups), ng,
        _ptr(res["out"]), _ptr(res["out_bf16"]), _ptr(res["lse"]),
        _ptr(res.get("o")), _ptr(res.get("codes")), _ptr(res.get("ymargin")), _ptr(res.get("omargin")),
        _ptr(res.get("lazy_margin")))
    if rc != 0:
        raise RuntimeError(f"orc_emulate_fp8_scores failed: {rc}")
    res["groups"] = groups
    return res


def group_rows(groups: np.ndarray, group: int) -> np.ndarray:
    """(b, h, i) triples of every row covered by the given groups (in output order)."""
    g = np.asarray(groups, dtype=np.int64).reshape(-1, 3)
    r = np.repeat(g, group, axis=0)
    r[:, 2] += np.tile(np.arange(group), g.shape[0])
    return r
