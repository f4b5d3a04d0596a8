"""Causal attention forward (prefill) for AMD Instinct MI355X (gfx950).

Thin ctypes binding over ``libattn_fwd_causal.so`` (C ABI: ``include/attn_fwd_causal.h``).
Every step of the computation runs in the library's HIP kernels; this module only
checks tensor metadata and passes device pointers, sizes and the current HIP stream.
PyTorch serves as the device allocator and stream provider.

Functions mirror the C entry points:
    attn_fwd_causal_fp8(q, k, v, q_descale, k_descale, v_descale, softmax_scale=None)
    attn_fwd_causal_bf16(q, k, v, softmax_scale=None)
    attn_fwd_causal_mla(q, k, v, q_descale, k_descale, v_descale, softmax_scale=None)
    attn_fwd_causal_fp8_ex(q, k, v, q_descale, k_descale, v_descale, softmax_scale=None, p_mode=None)
    attn_fwd_causal_fp8_vt(q, k, vt, q_descale, k_descale, v_descale, softmax_scale=None, p_mode=None)
    attn_fwd_causal_bf16_ex(q, k, v, softmax_scale=None)
    quantize_e4m3(x) -> (codes, descale)      round_bf16(x) -> bf16 tensor
    key_mean(k) -> mean [B, H, D]             rotate_quantize_e4m3(x, signs, mean=None) -> (codes, descale)
    quantize_e4m3_static(x, descale) -> codes rotate_quantize_e4m3_static(x, signs, descale, mean=None) -> codes
Tensors are BSHD: q, k [B, S, H, d_qk], v [B, S, H, d_v]; outputs out [B, S, H, d_v]
(bfloat16) and lse [B, H, S] (float32).  The *_ex functions take BSHD-shaped views of any
strided layout (e.g. a BHSD tensor x passed as x.permute(0, 2, 1, 3)) with the head
dimension contiguous, and grouped-query k/v with H_kv heads (H a multiple of H_kv).
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libattn_fwd_causal.so")

_STATUS = {0: "ok", -1: "null pointer", -2: "unsupported shape", -3: "misaligned pointer",
           -4: "tensor too large", -5: "invalid argument", -6: "kernel launch failed", -7: "no usable HIP device"}


class AttnError(RuntimeError):
    def __init__(self, fn, code):
        super().__init__(f"{fn}: {code} ({_STATUS.get(code, 'unknown')})")
        self.code = code


P_DEFAULT, P_LEAN, P_EXACT = -1, 0, 1


class Strides(ctypes.Structure):
    """attn_strides: element strides (batch, head, seq) of one tensor."""
    _fields_ = [("batch", ctypes.c_int64), ("head", ctypes.c_int64), ("seq", ctypes.c_int64)]


_lib = None


def lib():
    """Load the HIP library; raises if it has not been built (no fallback path exists)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with python -m bf16_causal_flashattention_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        P, F, I, I64 = ctypes.c_void_p, ctypes.c_float, ctypes.c_int, ctypes.c_int64
        L.attn_fwd_causal_fp8.argtypes = [P, P, P, P, P, F, F, F, F, I, I, I, I, I, P]
        L.attn_fwd_causal_mla.argtypes = [P, P, P, P, P, F, F, F, F, I, I, I, I, I, P]
        L.attn_fwd_causal_fp8_debug.argtypes = [P, P, P, P, P, F, F, F, F, I, I, I, I, I, P, P, P]
        L.attn_fwd_causal_bf16.argtypes = [P, P, P, P, P, F, I, I, I, I, I, P]
        SP = ctypes.POINTER(Strides)
        L.attn_fwd_causal_fp8_debug_ex.argtypes = [P, P, P, P, P, F, F, F, F, I, I, I, I, I, I, SP, SP, SP, SP, I,
                                                   P, P, P, P]
        L.attn_fwd_causal_fp8_ex.argtypes = [P, P, P, P, P, F, F, F, F, I, I, I, I, I, I, SP, SP, SP, SP, I, P]
        L.attn_fwd_causal_fp8_vt.argtypes = [P, P, P, P, P, F, F, F, F, I, I, I, I, I, I, SP, SP, SP, SP, I, P]
        L.attn_fwd_causal_bf16_ex.argtypes = [P, P, P, P, P, F, I, I, I, I, I, I, SP, SP, SP, SP, P]
        L.attn_quantize_e4m3.argtypes = [P, I64, P, P, P, P]
        L.attn_round_bf16.argtypes = [P, I64, P, P]
        L.attn_key_mean_workspace.argtypes = [I, I, I, I]
        L.attn_key_mean_workspace.restype = I64
        L.attn_key_mean.argtypes = [P, I, I, I, I, P, P, P]
        L.attn_key_mean_noalloc.argtypes = [P, I, I, I, I, P, P]
        L.attn_rotate_quantize_e4m3.argtypes = [P, P, P, I, I, I, I, P, P, P, P]
        L.attn_quantize_e4m3_static.argtypes = [P, I64, F, P, P]
        L.attn_rotate_quantize_e4m3_static.argtypes = [P, P, P, I, I, I, I, F, P, P]
        L.attn_default_grid.argtypes = [I, I, I, I, I]
        L.attn_schedule.argtypes = [I, I, I, I, I, P, I64]
        L.attn_schedule.restype = I64
        L.attn_status_string.argtypes = [I]
        L.attn_status_string.restype = ctypes.c_char_p
        for name in ("attn_fwd_causal_fp8", "attn_fwd_causal_mla", "attn_fwd_causal_fp8_debug",
                     "attn_fwd_causal_fp8_debug_ex",
                     "attn_fwd_causal_bf16", "attn_fwd_causal_fp8_ex", "attn_fwd_causal_fp8_vt", "attn_fwd_causal_bf16_ex",
                     "attn_quantize_e4m3", "attn_round_bf16", "attn_default_grid", "attn_key_mean",
                     "attn_key_mean_noalloc",
                     "attn_rotate_quantize_e4m3", "attn_quantize_e4m3_static", "attn_rotate_quantize_e4m3_static"):
            getattr(L, name).restype = I
        _lib = L
    return _lib


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t):
    """The current HIP stream of the current device, which must be the device of tensor t
    (the library launches on the current device)."""
    if t.device.index != torch.cuda.current_device():
        raise ValueError(f"tensors are on {t.device} but the current device is cuda:{torch.cuda.current_device()}; "
                         f"call under torch.cuda.device({t.device.index})")
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(fn, rc):
    if rc != 0:
        raise AttnError(fn, rc)


def _fp8_view(t):
    if t.dtype == torch.float8_e4m3fn:
        return t
    if t.dtype == torch.uint8:
        return t.view(torch.float8_e4m3fn)
    raise TypeError(f"expected float8_e4m3fn (OCP e4m3, not fnuz) or uint8 codes, got {t.dtype}")


def _outputs(q, v, out, lse):
    B, S, H, _ = q.shape
    dv = v.shape[3]
    if out is None:
        out = torch.empty((B, S, H, dv), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    return out, lse


def _same_device(*ts):
    dev = ts[0].device
    for t in ts:
        if not t.is_cuda or t.device != dev:
            raise ValueError("all tensors must be on the same GPU")


def _meta(q, k, v, out, lse):
    for t in (q, k, v, out, lse):
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("tensors must be contiguous and on the GPU")
    _same_device(q, k, v, out, lse)
    if out.dtype != torch.bfloat16 or lse.dtype != torch.float32:
        raise TypeError("out must be bfloat16 and lse float32")
    B, S, H, dqk = q.shape
    if tuple(k.shape) != (B, S, H, dqk) or tuple(v.shape[:3]) != (B, S, H):
        raise ValueError("q, k, v shapes disagree")
    dv = v.shape[3]
    if tuple(out.shape) != (B, S, H, dv) or tuple(lse.shape) != (B, H, S):
        raise ValueError("out / lse shapes disagree")
    return B, S, H, dqk, dv


def _fp8_call(fn_name, q, k, v, q_descale, k_descale, v_descale, softmax_scale, out, lse, debug=None):
    q, k, v = _fp8_view(q), _fp8_view(k), _fp8_view(v)
    out, lse = _outputs(q, v, out, lse)
    B, S, H, dqk, dv = _meta(q, k, v, out, lse)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(dqk)
    args = [_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), float(q_descale), float(k_descale),
            float(v_descale), float(softmax_scale), B, H, S, dqk, dv]
    if debug is not None:
        args += [_ptr(debug[0]), _ptr(debug[1])]
    _check(fn_name, getattr(lib(), fn_name)(*args, _stream(q)))
    return out, lse


def attn_fwd_causal_fp8(q, k, v, q_descale, k_descale, v_descale, softmax_scale=None, out=None, lse=None):
    """FP8 e4m3 causal attention, d_qk = d_v = 128, lean P.  Returns (out bf16, lse fp32)."""
    return _fp8_call("attn_fwd_causal_fp8", q, k, v, q_descale, k_descale, v_descale, softmax_scale, out, lse)


def attn_fwd_causal_mla(q, k, v, q_descale, k_descale, v_descale, softmax_scale=None, out=None, lse=None):
    """FP8 e4m3 causal attention at the MLA shape d_qk = 192, d_v = 128, exact P."""
    return _fp8_call("attn_fwd_causal_mla", q, k, v, q_descale, k_descale, v_descale, softmax_scale, out, lse)


def attn_fwd_causal_fp8_debug(q, k, v, q_descale, k_descale, v_descale, softmax_scale=None):
    """Test hook: FP8 attention (d_qk 128 or 192) that also returns the per-(row, 64-key block)
    scale exponents and the probability codes the kernel formed (255 / 0 where untouched)."""
    B, S, H, _ = q.shape
    dbg_o = torch.full((B * H * S, S // 64), 255, dtype=torch.uint8, device=q.device)
    dbg_c = torch.zeros((B * H * S, S), dtype=torch.uint8, device=q.device)
    out, lse = _fp8_call("attn_fwd_causal_fp8_debug", q, k, v, q_descale, k_descale, v_descale, softmax_scale,
                         None, None, debug=(dbg_o, dbg_c))
    return out, lse, dbg_o, dbg_c


def attn_fwd_causal_fp8_debug_ex(q, k, v, q_descale, k_descale, v_descale, softmax_scale=None, p_mode=None):
    """Test hook: attn_fwd_causal_fp8_ex (key-major V) that also returns the per-(row, 64-key block)
    scale exponents (255 where untouched), the probability codes (0 where untouched) and the raw
    fp32 scores the score MFMA produced, before the causal mask (NaN where untouched); the last
    three are [B*H*S, S/64] and [B*H*S, S] with row (b*H + h)*S + i."""
    q, k, v = _fp8_view(q), _fp8_view(k), _fp8_view(v)
    B, S, H, Hkv, dqk, dv, out, lse, st = _ex_meta(q, k, v, None, None)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(dqk)
    pm = P_DEFAULT if p_mode is None else int(p_mode)
    dbg_o = torch.full((B * H * S, S // 64), 255, dtype=torch.uint8, device=q.device)
    dbg_c = torch.zeros((B * H * S, S), dtype=torch.uint8, device=q.device)
    dbg_s = torch.full((B * H * S, S), float("nan"), dtype=torch.float32, device=q.device)
    rc = lib().attn_fwd_causal_fp8_debug_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), float(q_descale),
                                            float(k_descale), float(v_descale), float(softmax_scale), B, H, Hkv, S,
                                            dqk, dv, *[ctypes.byref(x) for x in st], pm, _ptr(dbg_o), _ptr(dbg_c),
                                            _ptr(dbg_s), _stream(q))
    _check("attn_fwd_causal_fp8_debug_ex", rc)
    return out, lse, dbg_o, dbg_c, dbg_s


def attn_fwd_causal_bf16(q, k, v, softmax_scale=None, out=None, lse=None):
    """BF16 causal attention, d_qk = d_v = 128.  Returns (out bf16, lse fp32)."""
    for t in (q, k, v):
        if t.dtype != torch.bfloat16:
            raise TypeError("q, k, v must be bfloat16")
    out, lse = _outputs(q, v, out, lse)
    B, S, H, dqk, dv = _meta(q, k, v, out, lse)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(dqk)
    rc = lib().attn_fwd_causal_bf16(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), float(softmax_scale),
                                    B, H, S, dqk, dv, _stream(q))
    _check("attn_fwd_causal_bf16", rc)
    return out, lse


def _strides(t):
    """attn_strides of a BSHD-shaped view whose head dimension is contiguous."""
    if not t.is_cuda:
        raise ValueError("tensors must be on the GPU")
    if t.dim() != 4 or t.stride(3) != 1:
        raise ValueError("expected a 4-D (B, S, H, d) view with a contiguous last dimension")
    return Strides(t.stride(0), t.stride(2), t.stride(1))


def _ex_meta(q, k, v, out, lse, v_channel_major=False):
    B, S, H, dqk = q.shape
    Bk, Sk, Hkv, dk = k.shape
    if v.dim() != 4:
        raise ValueError("v must be 4-D")
    # v is [B, S, H_kv, d_v], or [B, H_kv, d_v, S] when channel-major
    vB, vS, vH, dv = (v.shape[0], v.shape[3], v.shape[1], v.shape[2]) if v_channel_major else tuple(v.shape)
    if (Bk, Sk, dk) != (B, S, dqk) or (vB, vS, vH) != (B, S, Hkv) or Hkv == 0 or H % Hkv:
        raise ValueError("q, k, v shapes disagree (k, v need H_kv heads with H a multiple of H_kv)")
    if out is None:
        out = torch.empty((B, S, H, dv), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    if out.dtype != torch.bfloat16 or lse.dtype != torch.float32:
        raise TypeError("out must be bfloat16 and lse float32")
    if tuple(out.shape) != (B, S, H, dv) or tuple(lse.shape) != (B, H, S) or not lse.is_contiguous():
        raise ValueError("out / lse shapes disagree (lse must be a dense [B, H, S] tensor)")
    _same_device(q, k, v, out, lse)
    if v_channel_major:
        if not v.is_cuda or v.stride(3) != 1:
            raise ValueError("vt must be a [B, H_kv, d_v, S] GPU view with contiguous keys")
        st = [_strides(q), _strides(k), Strides(v.stride(0), v.stride(1), v.stride(2)), _strides(out)]
    else:
        st = [_strides(t) for t in (q, k, v, out)]
    return B, S, H, Hkv, dqk, dv, out, lse, st


def attn_fwd_causal_fp8_ex(q, k, v, q_descale, k_descale, v_descale, softmax_scale=None, p_mode=None,
                           out=None, lse=None):
    """FP8 causal attention with strided BSHD-shaped views, grouped-query k/v and a P mode
    (P_LEAN, P_EXACT or None for the default of the head dimension).  Returns (out, lse)."""
    q, k, v = _fp8_view(q), _fp8_view(k), _fp8_view(v)
    B, S, H, Hkv, dqk, dv, out, lse, st = _ex_meta(q, k, v, out, lse)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(dqk)
    pm = P_DEFAULT if p_mode is None else int(p_mode)
    rc = lib().attn_fwd_causal_fp8_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), float(q_descale),
                                      float(k_descale), float(v_descale), float(softmax_scale), B, H, Hkv, S, dqk,
                                      dv, *[ctypes.byref(x) for x in st], pm, _stream(q))
    _check("attn_fwd_causal_fp8_ex", rc)
    return out, lse


def attn_fwd_causal_fp8_vt(q, k, vt, q_descale, k_descale, v_descale, softmax_scale=None, p_mode=None,
                           out=None, lse=None):
    """attn_fwd_causal_fp8_ex with V channel-major: vt is a [B, H_kv, d_v, S] view with contiguous
    keys (vt[b, g, d, s] = v[b, s, g, d]).  Results equal attn_fwd_causal_fp8_ex bit for bit."""
    q, k, vt = _fp8_view(q), _fp8_view(k), _fp8_view(vt)
    B, S, H, Hkv, dqk, dv, out, lse, st = _ex_meta(q, k, vt, out, lse, v_channel_major=True)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(dqk)
    pm = P_DEFAULT if p_mode is None else int(p_mode)
    rc = lib().attn_fwd_causal_fp8_vt(_ptr(q), _ptr(k), _ptr(vt), _ptr(out), _ptr(lse), float(q_descale),
                                      float(k_descale), float(v_descale), float(softmax_scale), B, H, Hkv, S, dqk,
                                      dv, *[ctypes.byref(x) for x in st], pm, _stream(q))
    _check("attn_fwd_causal_fp8_vt", rc)
    return out, lse


def attn_fwd_causal_bf16_ex(q, k, v, softmax_scale=None, out=None, lse=None):
    """BF16 causal attention with strided BSHD-shaped views and grouped-query k/v."""
    for t in (q, k, v):
        if t.dtype != torch.bfloat16:
            raise TypeError("q, k, v must be bfloat16")
    B, S, H, Hkv, dqk, dv, out, lse, st = _ex_meta(q, k, v, out, lse)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(dqk)
    rc = lib().attn_fwd_causal_bf16_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), float(softmax_scale),
                                       B, H, Hkv, S, dqk, dv, *[ctypes.byref(x) for x in st], _stream(q))
    _check("attn_fwd_causal_bf16_ex", rc)
    return out, lse


def quantize_e4m3(x, workspace=None):
    """Per-tensor power-of-two e4m3 quantisation of a float32 GPU tensor.

    Returns (codes as float8_e4m3fn with x's shape, descale as a 1-element float32 tensor)."""
    if x.dtype != torch.float32 or not x.is_cuda or not x.is_contiguous():
        raise TypeError("x must be a contiguous float32 GPU tensor")
    codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    descale = torch.empty(1, dtype=torch.float32, device=x.device)
    if workspace is None:
        workspace = torch.empty(1, dtype=torch.int32, device=x.device)
    rc = lib().attn_quantize_e4m3(_ptr(x), x.numel(), _ptr(codes), _ptr(descale), _ptr(workspace), _stream(x))
    _check("attn_quantize_e4m3", rc)
    return codes.view(torch.float8_e4m3fn), descale


def _bshd_f32(x, name):
    if x.dtype != torch.float32 or not x.is_cuda or not x.is_contiguous() or x.dim() != 4:
        raise TypeError(f"{name} must be a contiguous float32 GPU tensor [B, S, H, D]")
    return x.shape


def key_mean(k):
    """Mean key of each head over the sequence (K smoothing), float32 [B, H, D]."""
    B, S, H, D = _bshd_f32(k, "k")
    L = lib()
    n_ws = L.attn_key_mean_workspace(B, S, H, D)
    if n_ws < 0:
        raise AttnError("attn_key_mean_workspace", int(n_ws))
    mean = torch.empty((B, H, D), dtype=torch.float32, device=k.device)
    ws = torch.empty(max((int(n_ws) + 7) // 8, 1), dtype=torch.float64, device=k.device)
    _check("attn_key_mean", L.attn_key_mean(_ptr(k), B, S, H, D, _ptr(mean), _ptr(ws), _stream(k)))
    return mean


def key_mean_noalloc(k, out):
    """attn_key_mean_noalloc: the mean key of each head of k [B, S, H, D] written into out, a
    contiguous float32 [B, H, D] GPU tensor, with no device allocation (the partial sums use the
    library's static scratch array; calls on one GPU must not overlap).  Returns out."""
    B, S, H, D = _bshd_f32(k, "k")
    if out.dtype != torch.float32 or not out.is_contiguous() or tuple(out.shape) != (B, H, D):
        raise ValueError("out must be a contiguous float32 [B, H, D] tensor")
    _same_device(k, out)
    _check("attn_key_mean_noalloc", lib().attn_key_mean_noalloc(_ptr(k), B, S, H, D, _ptr(out), _stream(k)))
    return out


def _rot_checks(x, signs, mean):
    B, S, H, D = _bshd_f32(x, "x")
    if signs.dtype != torch.float32 or not signs.is_cuda or signs.shape != (D,) or not signs.is_contiguous():
        raise TypeError("signs must be a contiguous float32 GPU tensor of D values")
    if mean is not None and (mean.dtype != torch.float32 or not mean.is_cuda or mean.shape != (B, H, D)
                             or not mean.is_contiguous()):
        raise TypeError("mean must be a contiguous float32 GPU tensor [B, H, D]")
    return B, S, H, D


def quantize_e4m3_static(x, descale):
    """e4m3 codes of x / descale for a given power-of-two descale (static scale); scaled
    values beyond 448 saturate.  Returns codes as float8_e4m3fn with x's shape."""
    if x.dtype != torch.float32 or not x.is_cuda or not x.is_contiguous():
        raise TypeError("x must be a contiguous float32 GPU tensor")
    codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    rc = lib().attn_quantize_e4m3_static(_ptr(x), x.numel(), float(descale), _ptr(codes), _stream(x))
    _check("attn_quantize_e4m3_static", rc)
    return codes.view(torch.float8_e4m3fn)


def rotate_quantize_e4m3_static(x, signs, descale, mean=None):
    """The rotation of rotate_quantize_e4m3 followed by the static-scale quantiser (one
    pass over x).  Returns codes as float8_e4m3fn with x's shape."""
    B, S, H, D = _rot_checks(x, signs, mean)
    codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    rc = lib().attn_rotate_quantize_e4m3_static(_ptr(x), _ptr(mean), _ptr(signs), B, S, H, D, float(descale),
                                                _ptr(codes), _stream(x))
    _check("attn_rotate_quantize_e4m3_static", rc)
    return codes.view(torch.float8_e4m3fn)


def rotate_quantize_e4m3(x, signs, mean=None, workspace=None):
    """Rotate rows of x [B, S, H, D] by diag(signs) (C_m kron H_{D/m}) after subtracting
    mean [B, H, D] (if given), then quantise to e4m3 with one power-of-two scale.

    Returns (codes as float8_e4m3fn with x's shape, descale as a 1-element float32 tensor)."""
    B, S, H, D = _rot_checks(x, signs, mean)
    codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    descale = torch.empty(1, dtype=torch.float32, device=x.device)
    if workspace is None:
        workspace = torch.empty(1, dtype=torch.int32, device=x.device)
    rc = lib().attn_rotate_quantize_e4m3(_ptr(x), _ptr(mean), _ptr(signs), B, S, H, D, _ptr(codes), _ptr(descale),
                                         _ptr(workspace), _stream(x))
    _check("attn_rotate_quantize_e4m3", rc)
    return codes.view(torch.float8_e4m3fn), descale


def round_bf16(x):
    """fp32 -> bf16, round to nearest even, on the GPU."""
    if x.dtype != torch.float32 or not x.is_cuda or not x.is_contiguous():
        raise TypeError("x must be a contiguous float32 GPU tensor")
    out = torch.empty(x.shape, dtype=torch.int16, device=x.device)
    _check("attn_round_bf16", lib().attn_round_bf16(_ptr(x), x.numel(), _ptr(out), _stream(x)))
    return out.view(torch.bfloat16)


def default_grid(B, H, S, num_cu, Hkv=None):
    return lib().attn_default_grid(B, H, H if Hkv is None else Hkv, S, num_cu)


def schedule(B, H, S, grid, Hkv=None):
    """Execution-order (workgroup, b, h, first row, rows) records of the persistent grid
    (host only); with H / Hkv even a tile is 128 rows of two heads (two records)."""
    import numpy as np
    rec = np.zeros((B * H * (S // 128), 5), dtype=np.int32)
    n = lib().attn_schedule(B, H, H if Hkv is None else Hkv, S, grid, ctypes.c_void_p(rec.ctypes.data),
                            rec.shape[0])
    if n < 0:
        raise AttnError("attn_schedule", int(n))
    return rec[:n]


def flops(B, H, S, dqk, dv):
    """Causal forward FLOP count F = B H S^2 (d_qk + d_v) (paper Sec. II-B, Eq. 1)."""
    return float(B) * H * S * S * (dqk + dv)
