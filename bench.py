"""Benchmark: causal attention forward (prefill) on one MI355X.

Headline: FP8 e4m3 causal prefill, B=1, H=32, S=32768, d_qk=d_v=128 (lean P), reported
as TFLOP/s with F = B H S^2 (d_qk + d_v) and as a fraction of the dense FP8 MFMA peak.
Timing is kernel-only as in "ZYFA: Speed and Accuracy of FP8 FlashAttention on AMD
CDNA4", Sec. V-B: warm-up launches, then the mean over K launches measured with HIP
events recorded on the launch stream; the per-tensor quantisation of the inputs runs
before the timed region (Sec. V-E) and is timed on its own.  The line also carries
the BF16 kernel at the same shape, the MLA-shaped FP8 kernel (B=1, H=16, S=32768,
192/128), the activation-like FP8 input (B=1, H=32, S=16384) and the oracle timed on
host cores over a bounded sample of the headline workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--only-headline] [--no-cpu-baseline]
       python bench.py --line {act,bf16,bf16_mla,fp8_4k,gqa,mla,mla_lean} [--steps K] [--warmup W]
Prints one JSON line (with --line: that configuration's time alone, for profiler runs).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import subprocess
import sys
import threading
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "causal prefill TFLOPS and % of FP8/BF16 MFMA peak, S=32K, d=128 and MLA 192/128"
PEAK_TFLOPS = {"fp8": 5000.0, "bf16": 2500.0}  # MI355X dense MFMA peaks at 2.4 GHz
HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fp8_attn_B1_H32_S32768_d128_traffic.json")
KERNEL_SRC = os.path.join(ROOT, "bf16_causal_flashattention_amd", "csrc", "attn_fp8.hip")


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def flops(B, H, S, dqk, dv):
    return float(B) * H * S * S * (dqk + dv)


def fp8_hbm_bytes(B, H, S, dqk, dv, elem=1):
    """Algorithmic HBM bytes of one call: read Q, K, V once, write O (bf16) and LSE (fp32)."""
    return B * S * H * (2 * dqk + dv) * elem + B * S * H * dv * 2 + B * H * S * 4


def src_hash(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


class ClockSampler:
    """Samples the shader clock (slowest XCD) and the socket power with amd-smi while the timed
    window runs (best effort)."""

    def __init__(self):
        self.samples = []
        self.power = []
        self._stop = threading.Event()
        self._t = None

    def _one(self):
        try:
            r = subprocess.run(["amd-smi", "metric", "-g", "0", "-c", "-p", "--json"], capture_output=True,
                               text=True, timeout=5)
            data = json.loads(r.stdout)
            if isinstance(data, dict) and "gpu_data" in data:
                data = data["gpu_data"]
            if isinstance(data, list):
                data = data[0]
            clk = data.get("clock", data)
            vals = []
            for key, val in clk.items():
                if key.startswith("gfx") and isinstance(val, dict):
                    cur = val.get("clk", val.get("cur_clk"))
                    if isinstance(cur, dict):
                        cur = cur.get("value")
                    if cur not in (None, "N/A"):
                        vals.append(float(cur))
            if vals:
                self.samples.append(min(vals))
            pw = data.get("power", {}).get("socket_power")
            if isinstance(pw, dict):
                pw = pw.get("value")
            if pw not in (None, "N/A"):
                self.power.append(float(pw))
        except Exception:
            pass

    def _run(self):
        while not self._stop.is_set():
            self._one()
            self._stop.wait(0.25)

    def __enter__(self):
        self._t = threading.Thread(target=self._run, daemon=True)
        self._t.start()
        return self

    def __exit__(self, *a):
        self._stop.set()
        self._t.join(timeout=10)

    def median(self):
        return float(np.median(self.samples)) if self.samples else None

    def median_power(self):
        return float(np.median(self.power)) if self.power else None


def time_launches(torch, fn, warmup, steps):
    """Mean device time per launch (ms) over `steps` launches, HIP events on the launch stream."""
    for _ in range(warmup):
        fn()
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        fn()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def prep_fp8(torch, cfa, synth_fn, B, S, H, dqk, dv, seed):
    import synth
    q, k, v = synth_fn(B, S, H, dqk, dv, seed)
    dev = torch.device("cuda:0")
    tens = [torch.from_numpy(x).to(dev) for x in (q, k, v)]
    del q, k, v
    out = [cfa.quantize_e4m3(t) for t in tens]
    torch.cuda.synchronize()
    prep = lambda: [cfa.quantize_e4m3(t) for t in tens]
    return tens, [o[0] for o in out], [float(o[1].item()) for o in out], prep


def sustained(torch, fn, F, reps=1):
    """Sustained-clock timing as in the paper (Sec. V-B): `reps` runs, each after 2 s of idle,
    of sustained_window; reports the median run (by time) with the range over the runs."""
    runs = []
    for _ in range(reps):
        torch.cuda.synchronize()
        time.sleep(2.0)
        runs.append(sustained_window(torch, fn, F))
    runs.sort(key=lambda r: r["ms"])
    med = dict(runs[len(runs) // 2])
    med["repetitions"] = len(runs)
    med["tflops_range"] = [runs[-1]["tflops"], runs[0]["tflops"]]
    med["sclk_mhz_range"] = [min((r["sclk_mhz_median_slowest_xcd"] or 0) for r in runs),
                             max((r["sclk_mhz_median_slowest_xcd"] or 0) for r in runs)]
    return med


def sustained_window(torch, fn, F, chunk_s=0.5, window_s=4.0, max_warm_s=6.0):
    """One sustained-clock run: back-to-back launches in 0.5 s chunks until two consecutive
    chunks agree within 0.3% (at least 1 s), then a timed window of about window_s seconds
    while amd-smi samples the shader clock (slowest XCD per sample) and the socket power."""
    def chunk(seconds):
        # launches per chunk from a short probe
        stream = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        torch.cuda.synchronize()
        n = max(1, int(seconds * 1e3 / max(e0.elapsed_time(e1), 1e-3)))
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n, n
    t0 = time.time()
    prev, _ = chunk(chunk_s)
    while True:
        cur, _ = chunk(chunk_s)
        if (time.time() - t0 >= 1.0 and abs(cur - prev) <= 0.003 * prev) or time.time() - t0 > max_warm_s:
            break
        prev = cur
    with ClockSampler() as clk:
        ms, n = chunk(window_s)
    tflops = F / (ms * 1e-3) / 1e12
    watts = clk.median_power()
    return {"ms": round(ms, 4), "tflops": round(tflops, 2), "launches": n,
            "warm_in_s": round(time.time() - t0 - window_s, 2), "sclk_mhz_median_slowest_xcd": clk.median(),
            "clock_samples": len(clk.samples), "socket_power_w_median": watts,
            "tflop_per_joule": round(tflops / watts, 3) if watts else None}


def run_fp8(torch, cfa, kind, synth_fn, B, H, S, dqk, warmup, steps, seed=0, sustained_reps=0,
            v_channel_major=False, softmax_scale=None):
    """FP8 attention through the basic entry point, or with v_channel_major through the entry
    point that takes V as [B, H, 128, S] (the transposed copy is made before the timing).
    softmax_scale None means 1/sqrt(d_qk)."""
    log(f"{kind} B={B} H={H} S={S} d_qk={dqk}: generating inputs")
    tens, codes, ds, prep = prep_fp8(torch, cfa, synth_fn, B, S, H, dqk, 128, seed)
    qg, kg, vg = codes
    out = torch.empty((B, S, H, 128), dtype=torch.bfloat16, device="cuda:0")
    lse = torch.empty((B, H, S), dtype=torch.float32, device="cuda:0")
    entry = cfa.attn_fwd_causal_fp8 if dqk == 128 else cfa.attn_fwd_causal_mla
    fn = lambda: entry(qg, kg, vg, ds[0], ds[1], ds[2], softmax_scale=softmax_scale, out=out, lse=lse)
    if v_channel_major:
        vt = vg.view(torch.uint8).permute(0, 2, 3, 1).contiguous()
        fn = lambda: cfa.attn_fwd_causal_fp8_vt(qg, kg, vt, ds[0], ds[1], ds[2], softmax_scale=softmax_scale,
                                                out=out, lse=lse)
    ms = time_launches(torch, fn, warmup, steps)
    prep_ms = time_launches(torch, prep, 2, 5)
    log(f"{kind} B={B} H={H} S={S} d_qk={dqk}: {ms:.4f} ms/launch")
    F = flops(B, H, S, dqk, 128)
    res = {"ms": ms, "tflops": F / (ms * 1e-3) / 1e12, "prep_ms": prep_ms,
           "bytes": fp8_hbm_bytes(B, H, S, dqk, 128, 1)}
    if sustained_reps:
        res["sustained"] = sustained(torch, fn, F, sustained_reps)
    del tens
    return res


def run_fp8_ex(torch, cfa, B, H, Hkv, S, dqk, p_mode, warmup, steps, seed=0):
    """FP8 through the general entry point: grouped-query k/v (Hkv heads) and a P mode."""
    import synth
    log(f"fp8_ex B={B} H={H} Hkv={Hkv} S={S} d_qk={dqk} p_mode={p_mode}: generating inputs")
    dev = torch.device("cuda:0")
    q = synth.gaussian(B, S, H, dqk, 128, seed)[0]
    _, k, v = synth.gaussian(B, S, Hkv, dqk, 128, seed + 1)
    codes, ds = [], []
    for x in (q, k, v):
        c, d = cfa.quantize_e4m3(torch.from_numpy(x).to(dev))
        codes.append(c)
        ds.append(float(d.item()))
    del q, k, v
    out = torch.empty((B, S, H, 128), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, H, S), dtype=torch.float32, device=dev)
    fn = lambda: cfa.attn_fwd_causal_fp8_ex(codes[0], codes[1], codes[2], ds[0], ds[1], ds[2], p_mode=p_mode,
                                            out=out, lse=lse)
    ms = time_launches(torch, fn, warmup, steps)
    F = flops(B, H, S, dqk, 128)
    log(f"fp8_ex B={B} H={H} Hkv={Hkv} S={S} d_qk={dqk}: {ms:.4f} ms/launch")
    return {"ms": ms, "tflops": F / (ms * 1e-3) / 1e12}


def run_bf16(torch, cfa, B, H, S, warmup, steps, seed=0, sustained_reps=0, dqk=128, std=1.0):
    import synth
    log(f"bf16 B={B} H={H} S={S} d_qk={dqk} std={std}: generating inputs")
    q, k, v = synth.gaussian(B, S, H, dqk, 128, seed, std=std)
    dev = torch.device("cuda:0")
    tens = [torch.from_numpy(x).to(dev) for x in (q, k, v)]
    del q, k, v
    qg, kg, vg = (cfa.round_bf16(t) for t in tens)
    out = torch.empty((B, S, H, 128), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, H, S), dtype=torch.float32, device=dev)
    if dqk == 128:
        fn = lambda: cfa.attn_fwd_causal_bf16(qg, kg, vg, out=out, lse=lse)
    else:
        fn = lambda: cfa.attn_fwd_causal_bf16_ex(qg, kg, vg, out=out, lse=lse)
    ms = time_launches(torch, fn, warmup, steps)
    F = flops(B, H, S, dqk, 128)
    log(f"bf16 B={B} H={H} S={S} d_qk={dqk}: {ms:.4f} ms/launch")
    res = {"ms": ms, "tflops": F / (ms * 1e-3) / 1e12}
    if sustained_reps:
        res["sustained"] = sustained(torch, fn, F, sustained_reps)
    return res


def run_rotate_prepass(torch, cfa, B, H, S, D, warmup, steps, seed=0):
    """Input preparation of q, k, v from fp32 in HBM, four ways: per-call scales (each
    quantiser reads its tensor twice, since the scale needs max |y| before the first
    code) or static power-of-two scales (one pass, the paper's fused quantisation pass),
    each plain or with the rotation of q and k and K smoothing (the key mean reads k once
    more).  Algorithmic bytes per element of each tensor: 9 per-call, 5 static, +4 for the
    key mean."""
    import synth
    q, k, v = synth.gaussian(B, S, H, D, D, seed)
    dev = torch.device("cuda:0")
    qg, kg, vg = (torch.from_numpy(x).to(dev) for x in (q, k, v))
    del q, k, v
    sg = torch.from_numpy(np.where(np.random.default_rng(seed).integers(0, 2, D) == 1, 1.0, -1.0)
                          .astype(np.float32)).to(dev)
    mean = cfa.key_mean(kg)
    ds = [float(cfa.rotate_quantize_e4m3(qg, sg)[1].item()), float(cfa.rotate_quantize_e4m3(kg, sg, mean)[1].item()),
          float(cfa.quantize_e4m3(vg)[1].item())]
    dp = [float(cfa.quantize_e4m3(t)[1].item()) for t in (qg, kg)]

    def call_rot():
        cfa.rotate_quantize_e4m3(qg, sg)
        cfa.rotate_quantize_e4m3(kg, sg, cfa.key_mean(kg))
        cfa.quantize_e4m3(vg)

    def call_plain():
        for t in (qg, kg, vg):
            cfa.quantize_e4m3(t)

    def static_rot():
        cfa.rotate_quantize_e4m3_static(qg, sg, ds[0])
        cfa.rotate_quantize_e4m3_static(kg, sg, ds[1], cfa.key_mean(kg))
        cfa.quantize_e4m3_static(vg, ds[2])

    def static_rot_nosmooth():
        cfa.rotate_quantize_e4m3_static(qg, sg, ds[0])
        cfa.rotate_quantize_e4m3_static(kg, sg, ds[1])
        cfa.quantize_e4m3_static(vg, ds[2])

    def static_plain():
        for t, d in zip((qg, kg, vg), dp + [ds[2]]):
            cfa.quantize_e4m3_static(t, d)

    n = B * S * H * D
    out = {}
    for name, fn, nbytes in (("per_call_rotated_smoothed", call_rot, 31 * n), ("per_call_plain", call_plain, 27 * n),
                             ("static_rotated_smoothed", static_rot, 19 * n),
                             ("static_rotated", static_rot_nosmooth, 15 * n), ("static_plain", static_plain, 15 * n)):
        ms = time_launches(torch, fn, warmup, steps)
        out[name] = {"ms": round(ms, 4), "hbm_gbs_at_algorithmic_bytes": round(nbytes / (ms * 1e-3) / 1e9, 1)}
    del qg, kg, vg
    return out


def cpu_baseline(B, H, S, dqk, stride=8, seed=0):
    """The oracle timed on the host cores (a reported baseline, not a target): exact fp64
    attention (orc_attn_exact) and the FP8 scheme emulation (orc_emulate_fp8, mirror mode)
    on the same rows of the headline workload, heads {0, H/2, H-1}, every `stride`-th
    32-row group of each head from a seeded offset (so the causal row lengths, and with them
    the cost, are sampled evenly); and the tiny configuration B=1 H=1 S=256 in full.
    Throughput counts the causal half of each row: 2 (i + 1) (d_qk + d_v) FLOP for row i."""
    import oracle
    import synth
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    c = 1.0 / math.sqrt(dqk)

    def legs(qc, kc, vc, dq, dk, dv, groups):
        rows = oracle.group_rows(groups, 32)
        f = float(np.sum(2.0 * (rows[:, 2] + 1) * (dqk + 128)))
        t1 = time.perf_counter()
        oracle.attn_exact(qc, kc, vc, dtype="fp8", c=c, dq=dq, dk=dk, dv=dv, rows=rows)
        t_ex = time.perf_counter() - t1
        t1 = time.perf_counter()
        oracle.emulate_fp8(qc, kc, vc, dq=dq, dk=dk, dv=dv, c=c, groups=groups)
        t_em = time.perf_counter() - t1
        return f, t_ex, t_em, len(rows)

    # tiny configuration, every row
    q, k, v = synth.gaussian(1, 256, 1, dqk, 128, seed)
    (qc, dq), (kc, dk), (vc, dv) = (oracle.quantize_e4m3(x) for x in (q, k, v))
    tg = np.array([(0, 0, r) for r in range(0, 256, 32)], dtype=np.int64)
    f1, t1_ex, t1_em, _ = legs(qc, kc, vc, dq, dk, dv, tg)
    # headline workload, head subset
    q, k, v = synth.gaussian(B, S, H, dqk, 128, seed)
    t0 = time.time()
    (qc, dq), (kc, dk), (vc, dv) = (oracle.quantize_e4m3(x) for x in (q, k, v))
    t_quant = time.time() - t0
    del q, k, v
    heads = sorted({0, H // 2, H - 1})
    off = int(np.random.default_rng(seed + 1).integers(stride))
    groups = np.array([(0, h, 32 * g) for h in heads for g in range(off, S // 32, stride)], dtype=np.int64)
    log(f"cpu baseline: oracle quantised inputs in {t_quant:.1f} s; {len(groups)} row groups of heads {heads}")
    f, t_ex, t_em, nrows = legs(qc, kc, vc, dq, dk, dv, groups)
    sample = (f"heads {heads} of the B={B} H={H} S={S} d={dqk} workload, every {stride}th 32-row group from "
              f"offset {off} ({nrows} rows, {f:.3e} FLOP of causal work); host quantisation ({t_quant:.1f} s) "
              f"excluded")
    return {"value": round(f / t_em / 1e12, 5), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": "FP8 scheme emulation (mirror mode) on " + sample,
            "fp64_exact": {"value": round(f / t_ex / 1e12, 5), "unit": "TFLOP/s", "seconds": round(t_ex, 2),
                           "sample": "exact fp64 attention on the same rows"},
            "emulation_seconds": round(t_em, 2),
            "tiny_B1_H1_S256_full": {"fp64_exact_ms": round(1e3 * t1_ex, 2), "emulation_ms": round(1e3 * t1_em, 2),
                                     "flop": f1}}


def traffic_entry():
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
        if t.get("kernel_src_sha256_16") != src_hash(KERNEL_SRC):
            return None  # kernel changed since the counters were taken
        return t.get("bytes_per_launch")
    except Exception:
        return None


def act_2sigma(B, S, H, dqk, dv, seed):
    """The activation-like input with its sink at 2 sigma instead of 12: with the softmax scale
    ACT_2SIGMA_SCALE the non-sink logits have standard deviation 2.5 and the sink's logit is 5,
    so the probabilities spread over many keys instead of sitting on the sink."""
    import synth
    return synth.activation_like(B, S, H, dqk, dv, seed, sink_sigmas=2.0)


def _act_2sigma_scale():
    import synth
    return 2.5 / synth.activation_sigma_raw(128)


ACT_2SIGMA_SCALE = _act_2sigma_scale()


# single configurations for --line: (torch, cfa, synth, warmup, steps) -> result of the run_* helper
LINES = {
    "bf16": lambda t, c, sy, w, n: run_bf16(t, c, 1, 32, 32768, w, n),
    "mla": lambda t, c, sy, w, n: run_fp8(t, c, "mla", sy.gaussian, 1, 16, 32768, 192, w, n),
    "mla_lean": lambda t, c, sy, w, n: run_fp8_ex(t, c, 1, 16, 16, 32768, 192, c.P_LEAN, w, n),
    "bf16_mla": lambda t, c, sy, w, n: run_bf16(t, c, 1, 16, 32768, w, n, dqk=192),
    "gqa": lambda t, c, sy, w, n: run_fp8_ex(t, c, 1, 32, 8, 32768, 128, c.P_LEAN, w, n),
    "act": lambda t, c, sy, w, n: run_fp8(t, c, "fp8", sy.activation_like, 1, 32, 16384, 128, w, n),
    "act_2sigma": lambda t, c, sy, w, n: run_fp8(t, c, "fp8", act_2sigma, 1, 32, 16384, 128, w, n,
                                                 softmax_scale=ACT_2SIGMA_SCALE),
    "fp8_vt": lambda t, c, sy, w, n: run_fp8(t, c, "fp8", sy.gaussian, 1, 32, 32768, 128, w, n, v_channel_major=True),
    "fp8_4k": lambda t, c, sy, w, n: run_fp8(t, c, "fp8", sy.gaussian, 1, 32, 4096, 128, w, n),
}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--only-headline", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sustained", action="store_true", help="skip the sustained-clock window")
    ap.add_argument("--cpu-stride", type=int, default=8,
                    help="the CPU baseline samples every n-th 32-row group of three heads")
    ap.add_argument("--line", choices=sorted(LINES),
                    help="time one other configuration alone with --warmup/--steps and print its result "
                         "(for profiler and counter runs)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(heads shard across GPUs with no communication)", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    import bf16_causal_flashattention_amd as cfa
    cfa.lib()  # fail loudly when the HIP library is missing

    if args.copy_calibration:
        # a plain copy of known size: FETCH_SIZE / WRITE_SIZE of this kernel, divided by
        # 2^30 bytes, give the scale factor of the byte counters
        x = torch.empty(1 << 30, dtype=torch.uint8, device="cuda:0").fill_(1)
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
        log("copy calibration: 3 copies of 2^30 bytes")
        del x, y
    if args.line:
        r = LINES[args.line](torch, cfa, synth, args.warmup, args.steps)
        print(json.dumps({"line": args.line, "ms": round(r["ms"], 4), "tflops": round(r["tflops"], 2),
                          "warmup": args.warmup, "steps": args.steps}), flush=True)
        return
    B, H, S, D = 1, 32, 32768, 128
    head = run_fp8(torch, cfa, "fp8", synth.gaussian, B, H, S, D, args.warmup, args.steps,
                   sustained_reps=0 if args.no_sustained else 3)
    F = flops(B, H, S, D, D)
    achieved = F / (head["ms"] * 1e-3) / 1e12
    result = {
        "metric": METRIC,
        "value": round(head["tflops"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3 (fp32 accumulate, bf16 out)",
        "data": "synthetic: q, k, v ~ N(0,1) fp32 from seed 0, quantised per tensor to e4m3 on the GPU",
        "config": {"workload": "FP8 causal prefill B=1 H=32 S=32768 d_qk=d_v=128, lean P", "B": B, "H": H,
                   "S": S, "d_qk": D, "d_v": D, "parallelism": "single GPU"},
        "pct_fp8_peak": round(100 * head["tflops"] / PEAK_TFLOPS["fp8"], 2),
        "sustained": head.get("sustained"),
        "prep_ms_qkv_quantise": round(head["prep_ms"], 4),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_TFLOPS["fp8"],
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_TFLOPS["fp8"], 4),
                     "traffic": traffic_entry(),
                     "algorithmic_hbm_bytes": head["bytes"],
                     "hbm_gbs_at_algorithmic_bytes": round(head["bytes"] / (head["ms"] * 1e-3) / 1e9, 1)},
    }
    if not args.only_headline:
        also = {}
        # the paper's kernel-only burst protocol (Sec. V-B): 500 warm-up launches, then the
        # mean of 100 (a short launch of S = 4K takes under 0.1 ms, so few launches would
        # time a GPU still ramping its clock)
        wb, sb = 500, 100
        r = run_bf16(torch, cfa, 1, 32, 32768, wb, sb, sustained_reps=0 if args.no_sustained else 1)
        also["bf16_B1_H32_S32768_d128"] = {"tflops": round(r["tflops"], 2), "ms": round(r["ms"], 4),
                                           "pct_bf16_peak": round(100 * r["tflops"] / PEAK_TFLOPS["bf16"], 2),
                                           "sustained": r.get("sustained")}
        for s in (4096, 8192, 16384):
            r = run_bf16(torch, cfa, 1, 32, s, wb, sb)
            also[f"bf16_B1_H32_S{s}_d128"] = {"tflops": round(r["tflops"], 2), "ms": round(r["ms"], 4)}
            r = run_fp8(torch, cfa, "fp8", synth.gaussian, 1, 32, s, 128, wb, sb)
            also[f"fp8_B1_H32_S{s}_d128"] = {"tflops": round(r["tflops"], 2), "ms": round(r["ms"], 4)}
        # V channel-major ([B, H, 128, S]): the same computation, operands read without transposes
        r = run_fp8(torch, cfa, "fp8", synth.gaussian, 1, 32, 32768, 128, wb, sb, v_channel_major=True)
        also["fp8_B1_H32_S32768_d128_v_channel_major"] = {
            "tflops": round(r["tflops"], 2), "ms": round(r["ms"], 4),
            "pct_fp8_peak": round(100 * r["tflops"] / PEAK_TFLOPS["fp8"], 2)}
        r = run_fp8(torch, cfa, "mla", synth.gaussian, 1, 16, 32768, 192, wb, sb,
                    sustained_reps=0 if args.no_sustained else 1)
        also["mla_fp8_B1_H16_S32768_192_128"] = {"tflops": round(r["tflops"], 2), "ms": round(r["ms"], 4),
                                                  "pct_fp8_peak": round(100 * r["tflops"] / PEAK_TFLOPS["fp8"], 2),
                                                  "sustained": r.get("sustained")}
        r = run_bf16(torch, cfa, 1, 16, 32768, wb, sb, dqk=192)
        also["mla_bf16_B1_H16_S32768_192_128"] = {"tflops": round(r["tflops"], 2), "ms": round(r["ms"], 4),
                                                   "pct_bf16_peak": round(100 * r["tflops"] / PEAK_TFLOPS["bf16"], 2)}
        r = run_fp8_ex(torch, cfa, 1, 16, 16, 32768, 192, cfa.P_LEAN, wb, sb)
        also["mla_fp8_leanP_B1_H16_S32768_192_128"] = {"tflops": round(r["tflops"], 2), "ms": round(r["ms"], 4),
                                                        "pct_fp8_peak": round(100 * r["tflops"] / PEAK_TFLOPS["fp8"], 2)}
        r = run_fp8_ex(torch, cfa, 1, 32, 8, 32768, 128, cfa.P_LEAN, wb, sb)
        also["fp8_gqa_B1_H32_Hkv8_S32768_d128"] = {"tflops": round(r["tflops"], 2), "ms": round(r["ms"], 4),
                                                    "pct_fp8_peak": round(100 * r["tflops"] / PEAK_TFLOPS["fp8"], 2)}
        r = run_fp8(torch, cfa, "fp8", synth.activation_like, 1, 32, 16384, 128, wb, sb)
        also["fp8_activation_like_B1_H32_S16384_d128"] = {"tflops": round(r["tflops"], 2), "ms": round(r["ms"], 4),
                                                           "note": "12-sigma sink: every row's softmax is one-hot"}
        r = run_fp8(torch, cfa, "fp8", act_2sigma, 1, 32, 16384, 128, wb, sb, softmax_scale=ACT_2SIGMA_SCALE)
        also["fp8_activation_like_2sigma_B1_H32_S16384_d128"] = {
            "tflops": round(r["tflops"], 2), "ms": round(r["ms"], 4),
            "note": "2-sigma sink, softmax scale 2.5/sigma_raw: logit sd 2.5, rows not one-hot"}
        # the paper's own timing inputs, N(0, 0.1^2): nearly uniform probabilities, so other
        # operand bits switch and the clock differs (Sec. III-C)
        gauss01 = lambda B_, S_, H_, dqk_, dv_, seed_: synth.gaussian(B_, S_, H_, dqk_, dv_, seed_, std=0.1)
        r = run_fp8(torch, cfa, "fp8", gauss01, 1, 32, 32768, 128, wb, sb)
        also["fp8_B1_H32_S32768_d128_gaussian_sd0.1"] = {"tflops": round(r["tflops"], 2), "ms": round(r["ms"], 4),
                                                         "pct_fp8_peak": round(100 * r["tflops"] / PEAK_TFLOPS["fp8"], 2)}
        r = run_bf16(torch, cfa, 1, 32, 32768, wb, sb, std=0.1)
        also["bf16_B1_H32_S32768_d128_gaussian_sd0.1"] = {"tflops": round(r["tflops"], 2), "ms": round(r["ms"], 4),
                                                          "pct_bf16_peak": round(100 * r["tflops"] / PEAK_TFLOPS["bf16"], 2)}
        also["prepass_rotate_smooth_B1_H32_S32768_d128"] = run_rotate_prepass(torch, cfa, 1, 32, 32768, 128, wb, sb)
        also["prepass_rotate_smooth_B1_H16_S32768_d192"] = run_rotate_prepass(torch, cfa, 1, 16, 32768, 192, wb, sb)
        result["also"] = also
        result["fp8_over_bf16_speedup_S32768"] = round(head["tflops"] / also["bf16_B1_H32_S32768_d128"]["tflops"], 3)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(B, H, S, D, stride=args.cpu_stride)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
