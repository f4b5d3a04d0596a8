"""Seeded synthetic inputs for causal attention (fp32 q, k, v in BSHD layout).

Shared by the tests, the benchmark and the oracle's pins.  Holds no arithmetic of the
attention method itself (no quantisation, no softmax): it only draws numbers.

Every generator takes (B, S, H, d_qk, d_v, seed) and returns three float32 arrays
q, k: [B, S, H, d_qk], v: [B, S, H, d_v].  Streams: numpy PCG64 seeded through
``SeedSequence(seed).spawn(4)`` (q, k, v, and one stream for structural choices).

The distributions follow "ZYFA: Speed and Accuracy of FP8 FlashAttention on AMD
CDNA4": kernel-benchmark Gaussians (Sec. V-B), the synthetic error distributions of
Fig. 15, and an activation-like input with outlier channels and a sink key standing
in for captured activations (Sec. V-C), which are not available here.
"""
from __future__ import annotations

import numpy as np


def _streams(seed: int):
    ss = np.random.SeedSequence(int(seed))
    return [np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(4)]


def _normal(rng, shape, std=1.0):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def gaussian(B, S, H, dqk, dv, seed, std=1.0):
    """q, k, v ~ N(0, std^2) (std 1 for the benchmark configs, 0.1 in the paper's timing runs)."""
    rq, rk, rv, _ = _streams(seed)
    return (_normal(rq, (B, S, H, dqk), std), _normal(rk, (B, S, H, dqk), std),
            _normal(rv, (B, S, H, dv), std))


def _add_key_offsets(q, k, offsets, rows_mask=None):
    """Shift the logits c q.k of key j by offsets[j] nats (c = 1/sqrt(d_qk)) through
    channel 0: q[..., 0] = 4 (or 0 on rows outside rows_mask), k[..., j, 0] = offsets[j] sqrt(d) / 4."""
    d = q.shape[3]
    q[..., 0] = 4.0
    if rows_mask is not None:
        q[:, ~rows_mask, :, 0] = 0.0
    k[..., 0] = (np.asarray(offsets, dtype=np.float64)[None, :, None] * np.sqrt(d) / 4.0).astype(np.float32)


def logit_sd(B, S, H, dqk, dv, seed, sd=1):
    """Fig. 15 'Logit SD 1/4/16': standard normal q, k scaled by 1, 2 or 4."""
    s = {1: 1.0, 4: 2.0, 16: 4.0}[sd]
    q, k, v = gaussian(B, S, H, dqk, dv, seed)
    return q * np.float32(s), k * np.float32(s), v


def stepped_max(B, S, H, dqk, dv, seed, step=1.0):
    """Fig. 15 'Stepped Max': each successive 64-key block's logits rise by `step` nats."""
    q, k, v = gaussian(B, S, H, dqk, dv, seed)
    _add_key_offsets(q, k, step * (np.arange(S) // 64))
    return q, k, v


def four_key_sink(B, S, H, dqk, dv, seed):
    """Fig. 15 '4-Key Sink': the first four keys scaled by 8."""
    q, k, v = gaussian(B, S, H, dqk, dv, seed)
    k[:, :4] *= np.float32(8.0)
    return q, k, v


def rising_logits(B, S, H, dqk, dv, seed, total=8.0):
    """Fig. 15 'Rising Logits': a linear ramp of `total` nats along the keys, every row."""
    q, k, v = gaussian(B, S, H, dqk, dv, seed)
    _add_key_offsets(q, k, total * np.arange(S) / max(S - 1, 1))
    return q, k, v


def alternating_rows(B, S, H, dqk, dv, seed, total=8.0):
    """Fig. 15 'Alternating Rows': the same ramp on every other query row only."""
    q, k, v = gaussian(B, S, H, dqk, dv, seed)
    _add_key_offsets(q, k, total * np.arange(S) / max(S - 1, 1), rows_mask=(np.arange(S) % 2 == 0))
    return q, k, v


def sink_flat_tail(B, S, H, dqk, dv, seed, lift=12.0):
    """Fig. 15 'Sink + Flat Tail': key 0 sits `lift` nats above a nearly uniform rest
    (q, k scaled by 0.1, so the other logits have SD about 0.01)."""
    q, k, v = gaussian(B, S, H, dqk, dv, seed)
    q *= np.float32(0.1)
    k *= np.float32(0.1)
    off = np.zeros(S)
    off[0] = lift
    _add_key_offsets(q, k, off)
    return q, k, v


def full_range(B, S, H, dqk, dv, seed):
    """Fig. 15 'Full Range': magnitudes log-uniform in [2^-6, 2^8], random signs."""
    rq, rk, rv, _ = _streams(seed)

    def draw(rng, shape):
        mag = np.exp2(rng.uniform(-6.0, 8.0, size=shape)).astype(np.float32)
        sgn = np.where(rng.random(size=shape) < 0.5, -1.0, 1.0).astype(np.float32)
        return mag * sgn

    return draw(rq, (B, S, H, dqk)), draw(rk, (B, S, H, dqk)), draw(rv, (B, S, H, dv))


def identical_keys(B, S, H, dqk, dv, seed):
    """Every key equal (one row broadcast), so every visible score of a row is equal."""
    q, k, v = gaussian(B, S, H, dqk, dv, seed)
    k[:] = k[:, :1]
    return q, k, v


def one_hot_key(B, S, H, dqk, dv, seed, key=0, lift=40.0):
    """Key `key` leads every other visible key of every row by about `lift` nats."""
    q, k, v = gaussian(B, S, H, dqk, dv, seed)
    q *= np.float32(0.05)
    k *= np.float32(0.05)
    off = np.zeros(S)
    off[key] = lift
    _add_key_offsets(q, k, off)
    return q, k, v


def activation_sigma_raw(dqk, n_outlier=4, outlier_gain=20.0):
    """Standard deviation of the raw non-sink dot products q.k of activation_like."""
    return float(np.sqrt((dqk - n_outlier) + n_outlier * outlier_gain ** 4))


def activation_like(B, S, H, dqk, dv, seed, n_outlier=4, outlier_gain=20.0, sink_sigmas=12.0, key_bias=0.0):
    """Activation-like input: q, k ~ N(0,1) with `n_outlier` seeded channels scaled by
    `outlier_gain` in both q and k, plus a sink key at position 0 whose dot product with
    every query equals `sink_sigmas` times the standard deviation of the raw non-sink
    dot products.  Construction: one further seeded channel c_s (not an outlier) is set
    to `outlier_gain` in every query; key 0 is zero except k[0, c_s] =
    sink_sigmas * sigma_raw / outlier_gain, with sigma_raw^2 = sum over channels of
    E[q_ch^2] E[k_ch^2].  v ~ N(0, 1).  key_bias > 0 adds one offset vector per (b, h),
    ~ N(0, key_bias^2) per channel, to every key (a component shared by all keys of a
    head, the part that K smoothing removes)."""
    rq, rk, rv, rs = _streams(seed)
    q = _normal(rq, (B, S, H, dqk))
    k = _normal(rk, (B, S, H, dqk))
    v = _normal(rv, (B, S, H, dv))
    ch = rs.choice(dqk, size=n_outlier + 1, replace=False)
    outl, cs = ch[:n_outlier], int(ch[n_outlier])
    q[..., outl] *= np.float32(outlier_gain)
    k[..., outl] *= np.float32(outlier_gain)
    var = np.ones(dqk)
    var[outl] = outlier_gain ** 4          # E[q^2] E[k^2] on an outlier channel
    sigma_raw = float(np.sqrt(var.sum()))  # the sink channel of q meets k ~ N(0,1) on other keys
    q[..., cs] = np.float32(outlier_gain)
    k[:, 0] = 0.0
    k[:, 0, :, cs] = np.float32(sink_sigmas * sigma_raw / outlier_gain)
    if key_bias:
        k += _normal(rs, (B, 1, H, dqk), key_bias)
    return q, k, v


STRESS = {
    "gaussian_0.1": lambda *a: gaussian(*a, std=0.1),
    "logit_sd_1": lambda *a: logit_sd(*a, sd=1),
    "logit_sd_4": lambda *a: logit_sd(*a, sd=4),
    "logit_sd_16": lambda *a: logit_sd(*a, sd=16),
    "stepped_max": stepped_max,
    "four_key_sink": four_key_sink,
    "rising_logits": rising_logits,
    "alternating_rows": alternating_rows,
    "sink_flat_tail": sink_flat_tail,
    "full_range": full_range,
}
