#!/usr/bin/env python3
"""Attention throughput on one MI355X: TFLOP/s and fraction of the bf16 MFMA peak.

One step = one pass of the hot path over the long-context causal workload
(B=1, H=32, N=16384, d=128, bf16): the fused forward (O and LSE) followed by
the recompute-based backward (dQ, dK, dV). Inputs are seeded synthetic
N(0, 1) tensors already resident in device memory.

FLOP convention: forward 4*B*H*N^2*d, backward 2.5x forward (five matrix
products), halved for the causal mask.

Prints one JSON line. ``--gpus N`` with N > 1 is refused: the library runs
the whole workload on one GPU.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA, published
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense fp8 MFMA, published
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E, published
PEAK_FP32_MFMA_TFLOPS = 157.3 # MI355X dense fp32 matrix, published
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "exact_tiled_attention_12_amd", "csrc")


def attention_flops(B, H, N, d, causal, backward=False):
    f = 4.0 * B * H * N * N * d
    if causal:
        f *= 0.5
    return f * (2.5 if backward else 1.0)


def kernel_source_sha(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(kernel_key, files, per_launch_units):
    """HBM bytes per launch from committed rocprofv3 counter summaries, if current."""
    path = os.path.join(PROFILES, "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    ent = data.get(kernel_key)
    if not ent or ent.get("src_sha") != kernel_source_sha(files):
        return None
    return ent.get("hbm_bytes_per_launch")


def load_counters(kernel_key, files):
    """Clock and MFMA-busy figures from committed rocprofv3 counter summaries, if current.

    The clock is GRBM_GUI_ACTIVE over the eight XCDs divided by the launch's
    duration in the counter run; the fraction at that clock prices the
    achieved rate against 1024 FLOP per SIMD per cycle (bf16) at that clock.
    """
    path = os.path.join(PROFILES, "counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    ent = data.get(kernel_key)
    if not ent or ent.get("src_sha") != kernel_source_sha(files):
        return None
    return ent


def at_clock(achieved, peak, kernel_key, files):
    """measured_clock_ghz, mfma_busy and frac_at_measured_clock for a roofline entry (None if stale)."""
    c = load_counters(kernel_key, files)
    if not c or "clock_ghz" not in c or "peak_tflops_at_measured_clock" not in c:
        return {"measured_clock_ghz": None, "mfma_busy": None, "frac_at_measured_clock": None}
    p = peak * c["clock_ghz"] / 2.4
    return {"measured_clock_ghz": c["clock_ghz"], "mfma_busy": c.get("mfma_busy"),
            "frac_at_measured_clock": round(achieved / p, 4)}


def host_info():
    """Host cores and the BLAS library numpy runs the oracle's products on."""
    info = {"host_cpus": os.cpu_count()}
    try:
        from threadpoolctl import threadpool_info
        pools = threadpool_info()
        blas = [p for p in pools if p.get("user_api") == "blas"]
        info["blas"] = "; ".join(f"{p.get('internal_api')} {p.get('version')}"
                                 + (f" ({p['threading_layer']})" if p.get("threading_layer") else "")
                                 for p in blas) or "unknown"
        info["blas_threads"] = max([p.get("num_threads", 1) for p in blas] or [1])
    except Exception:  # pragma: no cover
        info["blas"] = "unknown"
        info["blas_threads"] = os.cpu_count() or 1
    return info


def cpu_baseline(heads: int):
    """The float64 oracle, timed on this host on a bounded sample of the workload."""
    import numpy as np
    import seeded_inputs as si
    from oracle import attention as A
    hi = host_info()
    w = si.workload(4)
    rng = np.random.default_rng(w.seed)
    shape = (w.N, w.d)
    x = {n: si.bf16_round(rng.standard_normal(size=shape, dtype=np.float32))[1] for n in ("q", "k", "v", "do")}
    t0 = time.perf_counter()
    for _ in range(heads):
        A.forward(x["q"], x["k"], x["v"], w.scale, True)
        A.backward(x["q"], x["k"], x["v"], x["do"], w.scale, True)
    dt = time.perf_counter() - t0
    flops = heads * (attention_flops(1, 1, w.N, w.d, True) + attention_flops(1, 1, w.N, w.d, True, True))
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(hi["blas_threads"]), "kind": "oracle",
            "sample": f"{heads} head(s) of the N=16384 d=128 causal workload, forward + backward, "
                      f"float64 numpy, {dt:.1f} s",
            "host_cpus": hi["host_cpus"], "blas": hi["blas"]}


def oracle_configs():
    """The float64 oracle timed once per workload on this host (a baseline, not a target).

    Heads are independent, so where a whole workload would take long a seeded
    subset of its heads is timed and the time scaled by heads / subset.
    FLOPs follow the same convention as the GPU figures (the oracle also
    computes the masked half of a causal score matrix). The fp8 workload's
    leg is its full oracle path: quantisation (rotated Q, K), the tiled fp8
    emulation, the per-tensor fp8 baseline emulation and the exact forward.
    """
    import numpy as np
    import seeded_inputs as si
    from oracle import attention as A
    from oracle import fp8 as F
    res = {"host": host_info()}
    subset = {1: 1, 2: 96, 3: 8, 4: 2, 5: 1}   # heads timed
    for k in (1, 2, 3, 4, 5):
        w = si.workload(k)
        nh = subset[k]
        # a sample of nh heads (B = 1, H = nh) drawn with the workload's seed
        # and recipe; workload 2 is timed whole
        ws = w.resized(B=1, H=nh) if w.B * w.H > nh else w
        x = si.make_inputs(ws)
        t0 = time.perf_counter()
        if k == 5:
            q8, sq, _ = F.quantize(x["q"], 64, x["rot"])
            k8, sk, _ = F.quantize(x["k"], 64, x["rot"])
            v8, sv, _ = F.quantize(x["v"], 64, pow2=True)
            F.fp8_attention_tiled(q8, sq, k8, sk, v8, sv, w.scale, w.causal)
            q8, sq, _ = F.quantize(x["q"], 0)
            k8, sk, _ = F.quantize(x["k"], 0)
            v8, sv, _ = F.quantize(x["v"], 0, pow2=True)
            F.fp8_attention_tiled(q8, sq, k8, sk, v8, sv, w.scale, w.causal)
            A.forward(x["q"], x["k"], x["v"], w.scale, w.causal)
        else:
            A.forward(x["q"], x["k"], x["v"], w.scale, w.causal)
            if w.backward:
                A.backward(x["q"], x["k"], x["v"], x["do"], w.scale, w.causal)
        dt = time.perf_counter() - t0
        heads_done = ws.B * ws.H
        total_heads = w.B * w.H
        full_s = dt * total_heads / heads_done
        flops = attention_flops(w.B, w.H, w.N, w.d, w.causal, False)
        if w.backward:
            flops += attention_flops(w.B, w.H, w.N, w.d, w.causal, True)
        res[f"workload_{k}"] = {"shape": [w.B, w.H, w.N, w.d], "dtype": w.dtype, "causal": w.causal,
                                "legs": "fp8 path (quantise, block + per-tensor emulation, exact forward)"
                                if k == 5 else ("forward + backward" if w.backward else "forward"),
                                "heads_timed": heads_done, "seconds_timed": round(dt, 3),
                                "seconds_full": round(full_s, 4), "extrapolated": heads_done < total_heads,
                                "useful_gflops": round(flops / full_s / 1e9, 2)}
        print(json.dumps({f"workload_{k}": res[f"workload_{k}"]}), flush=True)
    return res


def configs_section(fa, which=(1, 2, 3)):
    """Forward-only workloads 1-3 on their seeded inputs: median of timed reps.

    5 warm-up calls, then 100 timed calls (workloads 1 and 2) or 20
    (workload 3), each between two events on the launch stream.
    """
    import numpy as np
    import torch
    import seeded_inputs as si
    res = {}
    for k in which:
        w = si.workload(k)
        x = si.make_inputs(w, names=("q", "k", "v"))
        if w.dtype == "f32":
            t = {n: torch.from_numpy(x[n]).cuda() for n in "qkv"}
        else:
            t = {n: torch.from_numpy(x[n + "_bits"].view(np.int16)).view(torch.bfloat16).cuda() for n in "qkv"}
        del x
        o = torch.empty_like(t["q"])
        lse = torch.empty((w.B, w.H, w.N), device="cuda", dtype=torch.float32)
        reps = 100 if k in (1, 2) else 20
        for _ in range(5):
            fa.fwd(t["q"], t["k"], t["v"], causal=w.causal, scale=w.scale, out=o, lse=lse)
        torch.cuda.synchronize()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
        for e in ev:
            e[0].record()
            fa.fwd(t["q"], t["k"], t["v"], causal=w.causal, scale=w.scale, out=o, lse=lse)
            e[1].record()
        torch.cuda.synchronize()
        ms = float(np.median([e[0].elapsed_time(e[1]) for e in ev]))
        tf = attention_flops(w.B, w.H, w.N, w.d, w.causal) / (ms * 1e-3) / 1e12
        peak = PEAK_FP32_MFMA_TFLOPS if w.dtype == "f32" else PEAK_BF16_TFLOPS
        res[f"workload_{k}"] = {"shape": [w.B, w.H, w.N, w.d], "dtype": w.dtype, "causal": w.causal,
                                "fwd_ms": round(ms, 4), "fwd_tflops": round(tf, 2),
                                "frac_of_peak": round(tf / peak, 4), "peak_tflops": peak}
        ck = {2: "attn_fwd_bf16_d64_N1024_B8_H12", 3: "attn_fwd_bf16_d128_causal_N4096_B2_H32"}.get(k)
        if ck:
            res[f"workload_{k}"].update(at_clock(tf, peak, ck, ["fa_fwd_bf16.hip", "fa_device.h"]))
        del t, o, lse
    return res


def fp8_section(fa, steps: int, warmup: int):
    """Times the fp8 workload (B=4, H=32, N=8192, d=128, non-causal): quantisation and attention.

    Inputs: seeded N(0, 1) bf16 tensors drawn on the device, with the
    workload's four shared outlier channels scaled by 30 in Q, K and V and a
    seeded Haar rotation applied to Q and K by the quantiser.
    """
    import numpy as np
    import torch
    import seeded_inputs as si
    w = si.workload(5)
    B, H, N, d = w.B, w.H, w.N, w.d
    rng = np.random.default_rng(w.seed)
    ch = si.outlier_channels(rng, H, d, w.outlier_frac)
    rot = torch.from_numpy(si.haar_orthogonal(rng, d).astype(np.float32)).cuda()
    gen = torch.Generator(device="cuda").manual_seed(w.seed)
    x = {}
    for n in "qkv":
        t = torch.randn((B, H, N, d), device="cuda", generator=gen, dtype=torch.float32)
        for hh, dd in ch:
            t[:, int(hh), :, int(dd)] *= w.outlier_gain
        x[n] = t.to(torch.bfloat16)
        del t
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]

    def run(e=None):
        if e:
            e[0].record()
        q8, sq = fa.quant_fp8(x["q"], rot=rot)
        k8, sk = fa.quant_fp8(x["k"], rot=rot)
        v8, sv = fa.quant_fp8(x["v"], pow2=True)
        if e:
            e[1].record()
        fa.fwd_fp8(q8, k8, v8, sq, sk, sv, causal=False, scale=w.scale)
        if e:
            e[2].record()

    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    for i in range(steps):
        run(ev[i])
    torch.cuda.synchronize()
    q_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    f_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    tf = attention_flops(B, H, N, d, False) / (f_ms * 1e-3) / 1e12

    # The backward of the fp8 forward (fa_bwd_fp8: Q, K, V decoded exactly
    # into bf16, then the bf16 backward), on all-power-of-two quantisation as
    # it requires; dO seeded N(0, 1).
    q8, sq = fa.quant_fp8(x["q"], rot=rot, pow2=True)
    k8, sk = fa.quant_fp8(x["k"], rot=rot, pow2=True)
    v8, sv = fa.quant_fp8(x["v"], pow2=True)
    del x
    o, lse = fa.fwd_fp8(q8, k8, v8, sq, sk, sv, causal=False, scale=w.scale)
    do = torch.randn((B, H, N, d), device="cuda", generator=gen, dtype=torch.float32).to(torch.bfloat16)
    ws = torch.empty(fa.bwd_fp8_workspace_bytes(B, H, N, d), device="cuda", dtype=torch.uint8)
    grads = [torch.empty_like(o) for _ in range(3)]

    def run_bwd():
        fa.bwd_fp8(q8, k8, v8, sq, sk, sv, o, lse, do, causal=False, scale=w.scale, workspace=ws,
                   dq=grads[0], dk=grads[1], dv=grads[2])

    for _ in range(warmup):
        run_bwd()
    torch.cuda.synchronize()
    evb = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for e in evb:
        e[0].record()
        run_bwd()
        e[1].record()
    torch.cuda.synchronize()
    b_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evb]))
    b_tf = attention_flops(B, H, N, d, False, True) / (b_ms * 1e-3) / 1e12
    del ws, grads, do, o, lse
    # Quantiser: algorithmic HBM bytes of the three launches (2 B read and 1 B
    # written per element, plus the block scales).
    q_bytes = 3 * (B * H * N * d * 3 + B * H * (-(-N // 64)) * 4)
    q_gbs = q_bytes / (q_ms * 1e-3) / 1e9
    return {"workload": "fp8 e4m3 attention, B=4 H=32 N=8192 d=128, non-causal, block scales + rotation",
            "quant_ms": round(q_ms, 4), "quant_gbps": round(q_gbs, 1),
            "quant_frac_of_hbm_peak": round(q_gbs / PEAK_HBM_GBS, 4),
            "fwd_ms": round(f_ms, 4), "fwd_tflops": round(tf, 2),
            "fwd_frac_of_fp8_peak": round(tf / PEAK_FP8_TFLOPS, 4),
            "fwd_at_clock": at_clock(tf, PEAK_FP8_TFLOPS, "attn_fwd_fp8_d128_N8192_B4_H32", ["fa_fp8.hip", "fa_device.h"]),
            "bwd_ms": round(b_ms, 4), "bwd_tflops": round(b_tf, 2),
            "bwd_frac_of_bf16_peak": round(b_tf / PEAK_BF16_TFLOPS, 4),
            "bwd_note": "fa_bwd_fp8 (exact bf16 decoding of Q, K, V + the bf16 backward), power-of-two scales"}


def det_section(fa, q, k, v, o, lse, do, causal: bool, steps: int, warmup: int, bwd_ms: float):
    """Times the fixed-order (deterministic) backward, fa_bwd_det, on the same
    tensors as the main step: all three launches of one call per step."""
    import numpy as np
    import torch
    B, H, N, d = q.shape
    ws = torch.empty(fa.bwd_det_workspace_bytes(B, H, N, d, causal), device=q.device, dtype=torch.uint8)
    out = [torch.empty_like(q) for _ in range(3)]

    def run():
        fa.bwd(q, k, v, o, lse, do, causal=causal, workspace=ws, dq=out[0], dk=out[1], dv=out[2],
               deterministic=True)

    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for e in ev:
        e[0].record()
        run()
        e[1].record()
    torch.cuda.synchronize()
    ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    tf = attention_flops(B, H, N, d, causal, True) / (ms * 1e-3) / 1e12
    res = {"workload": f"fixed-order backward, B={B} H={H} N={N} d={d}, causal={causal}",
           "bwd_ms": round(ms, 4), "bwd_tflops": round(tf, 2),
           "workspace_gb": round(ws.numel() / 1e9, 3),
           "time_vs_atomic_bwd": round(ms / bwd_ms, 4) if bwd_ms > 0 else None}
    del ws
    return res


def gqa_section(fa, steps: int, warmup: int, H_kv_list=(8, 1)):
    """Times grouped-query (and multi-query) forward + backward at the main
    workload's shape (B=1, H=32 query heads, N=16384, d=128, causal) with
    H_kv K/V heads. Inputs: seeded N(0, 1) bf16 tensors drawn on the device."""
    import numpy as np
    import torch
    B, H, N, d = 1, 32, 16384, 128
    gen = torch.Generator(device="cuda").manual_seed(2024)
    mk = lambda h: torch.randn((B, h, N, d), device="cuda", generator=gen, dtype=torch.float32).to(torch.bfloat16)
    q, do = mk(H), mk(H)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), device="cuda", dtype=torch.float32)
    dq = torch.empty_like(q)
    res = {}
    for H_kv in H_kv_list:
        k, v = mk(H_kv), mk(H_kv)
        ws = torch.empty(fa.bwd_gqa_workspace_bytes(B, H, H_kv, N, d), device="cuda", dtype=torch.uint8)
        dk, dv = torch.empty_like(k), torch.empty_like(v)
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]

        def run(e=None):
            if e:
                e[0].record()
            fa.fwd(q, k, v, causal=True, out=o, lse=lse)
            if e:
                e[1].record()
            fa.bwd(q, k, v, o, lse, do, causal=True, workspace=ws, dq=dq, dk=dk, dv=dv)
            if e:
                e[2].record()

        for _ in range(warmup):
            run()
        torch.cuda.synchronize()
        for e in ev:
            run(e)
        torch.cuda.synchronize()
        f_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
        b_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
        ff, fb = attention_flops(B, H, N, d, True), attention_flops(B, H, N, d, True, True)
        res[f"H_kv={H_kv}"] = {"fwd_ms": round(f_ms, 4), "bwd_ms": round(b_ms, 4),
                               "fwd_tflops": round(ff / (f_ms * 1e-3) / 1e12, 2),
                               "bwd_tflops": round(fb / (b_ms * 1e-3) / 1e12, 2),
                               "tflops": round((ff + fb) / ((f_ms + b_ms) * 1e-3) / 1e12, 2)}
        del k, v, dk, dv, ws
    return {"workload": f"grouped-query causal bf16 attention, B={B} H={H} N={N} d={d}, fwd + bwd", **res}


def varlen_section(fa, steps: int, warmup: int):
    """Times a packed variable-length batch: 16 causal sequences with seeded
    lengths uniform in [256, 16384] (H=32, d=128, bf16), forward + backward.
    FLOPs are counted per sequence (4 H n^2 d / 2 forward, x2.5 backward)."""
    import numpy as np
    import torch
    H, d = 32, 128
    lens = [int(x) for x in np.random.default_rng(2400).integers(256, 16385, size=16)]
    T = sum(lens)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)).cuda()
    gen = torch.Generator(device="cuda").manual_seed(2401)
    mk = lambda: torch.randn((H, T, d), device="cuda", generator=gen, dtype=torch.float32).to(torch.bfloat16)
    q, k, v, do = mk(), mk(), mk(), mk()
    o = torch.empty_like(q)
    lse = torch.empty((H, T), device="cuda", dtype=torch.float32)
    g = [torch.empty_like(q) for _ in range(3)]
    ws = torch.empty(int(fa.load().fa_bwd_varlen_workspace_bytes(T, H, H, d)), device="cuda", dtype=torch.uint8)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]

    def run(e=None):
        if e:
            e[0].record()
        fa.fwd_varlen(q, k, v, cu, max(lens), causal=True, out=o, lse=lse)
        if e:
            e[1].record()
        fa.bwd_varlen(q, k, v, o, lse, do, cu, max(lens), causal=True, workspace=ws, dq=g[0], dk=g[1], dv=g[2])
        if e:
            e[2].record()

    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    for e in ev:
        run(e)
    torch.cuda.synchronize()
    f_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    b_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    ff = sum(attention_flops(1, H, n, d, True) for n in lens)
    return {"workload": f"packed variable-length causal bf16 attention, 16 sequences (lengths uniform in "
                        f"[256, 16384], seeded), total {T} rows, H={H} d={d}, fwd + bwd",
            "fwd_ms": round(f_ms, 4), "bwd_ms": round(b_ms, 4),
            "fwd_tflops": round(ff / (f_ms * 1e-3) / 1e12, 2), "bwd_tflops": round(2.5 * ff / (b_ms * 1e-3) / 1e12, 2),
            "tflops": round(3.5 * ff / ((f_ms + b_ms) * 1e-3) / 1e12, 2)}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--fwd-only", action="store_true", help="time the forward only")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-fp8", action="store_true", help="skip the fp8 workload timing")
    ap.add_argument("--no-det", action="store_true", help="skip the fixed-order backward timing")
    ap.add_argument("--no-gqa", action="store_true", help="skip the grouped-query timing")
    ap.add_argument("--no-varlen", action="store_true", help="skip the variable-length batch timing")
    ap.add_argument("--fp8-only", action="store_true",
                    help="time only the fp8 workload and print its figures as one JSON line")
    ap.add_argument("--cpu-heads", type=int, default=1)
    ap.add_argument("--no-configs", action="store_true", help="skip the forward timing of workloads 1-3")
    ap.add_argument("--config-only", type=int, default=0, metavar="K",
                    help="time only the forward of workload K (1, 2 or 3) and print its figures")
    ap.add_argument("--oracle-configs", action="store_true",
                    help="time the float64 oracle once per workload on this host (no GPU needed)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="before the warm-up, copy MIB MiB device-to-device once (a transfer of known "
                         "size for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the attention of each (batch, head) is independent, so heads would shard across GPUs)",
              file=sys.stderr)
        sys.exit(2)

    if args.oracle_configs:
        print(json.dumps({"oracle_configs": oracle_configs()}), flush=True)
        return

    import numpy as np
    import torch
    import exact_tiled_attention_12_amd as fa
    import seeded_inputs as si

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    fa.load()
    if args.calibrate_copy > 0:
        n = args.calibrate_copy << 20
        src = torch.ones(n, device="cuda", dtype=torch.uint8)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.fp8_only:
        print(json.dumps({"fp8": fp8_section(fa, args.steps, args.warmup)}), flush=True)
        return
    if args.config_only:
        print(json.dumps({"configs": configs_section(fa, (args.config_only,))}), flush=True)
        return
    w = si.workload(4)
    B, H, N, d = w.B, w.H, w.N, w.d
    x = si.make_inputs(w)
    dev = torch.device("cuda:0")

    def t(n):
        return torch.from_numpy(x[n + "_bits"].view(np.int16)).view(torch.bfloat16).to(dev)

    q, k, v, do = (t(n) for n in ("q", "k", "v", "do"))
    del x
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), device=dev, dtype=torch.float32)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    ws = torch.empty(fa.bwd_workspace_bytes(B, H, N, d), device=dev, dtype=torch.uint8)
    do_bwd = not args.fwd_only

    def step(ev=None):
        # Events on torch's current stream, which is the stream the library launches on.
        if ev:
            ev[0].record()
        fa.fwd(q, k, v, causal=True, out=o, lse=lse)
        if ev:
            ev[1].record()
        if do_bwd:
            for i, stage in enumerate((1, 2, 4)):
                fa.bwd_stages(q, k, v, o, lse, do, ws, dq, dk, dv, stage_mask=stage, causal=True)
                if ev:
                    ev[2 + i].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    fwd_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    bwd_ms = float(np.mean([e[1].elapsed_time(e[4]) for e in evs])) if do_bwd else 0.0
    bwd_main_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in evs])) if do_bwd else 0.0
    bwd_pre_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs])) if do_bwd else 0.0
    bwd_fin_ms = float(np.mean([e[3].elapsed_time(e[4]) for e in evs])) if do_bwd else 0.0
    ms_per_step = wall * 1e3 / args.steps

    f_fwd = attention_flops(B, H, N, d, True)
    f_bwd = attention_flops(B, H, N, d, True, True) if do_bwd else 0.0
    value = (f_fwd + f_bwd) / (ms_per_step * 1e-3) / 1e12

    # Roofline of the dominant kernel: algorithmic FLOPs per launch / its event-timed duration.
    # All five products of the backward run in its main kernel (the other two
    # launches are O(N d) streaming passes).
    if do_bwd and bwd_main_ms > fwd_ms:
        dom, dom_ms, dom_flops, files = "attn_bwd_main", bwd_main_ms, f_bwd, ["fa_bwd_bf16.hip", "fa_device.h"]
    else:
        dom, dom_ms, dom_flops, files = "attn_fwd", fwd_ms, f_fwd, ["fa_fwd_bf16.hip", "fa_device.h"]
    achieved = dom_flops / (dom_ms * 1e-3) / 1e12
    roofline = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": load_traffic(f"{dom}_bf16_d128_causal_N16384_B1_H32", files, 1)}
    roofline.update(at_clock(achieved, PEAK_BF16_TFLOPS, f"{dom}_bf16_d128_causal_N16384_B1_H32", files))

    out = {
        "metric": "attention fwd/bwd TFLOP/s at d=128 causal bf16, % of MFMA peak (1 GPU)",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "causal bf16 attention, B=1 H=32 N=16384 d=128, "
                               + ("forward only" if args.fwd_only else "forward + backward"),
                   "B": B, "H": H, "N": N, "d": d, "causal": True},
        "frac_of_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "breakdown": {"fwd_ms": round(fwd_ms, 4), "bwd_ms": round(bwd_ms, 4),
                      "bwd_pre_ms": round(bwd_pre_ms, 4), "bwd_main_ms": round(bwd_main_ms, 4),
                      "bwd_finish_ms": round(bwd_fin_ms, 4),
                      "fwd_tflops": round(f_fwd / (fwd_ms * 1e-3) / 1e12, 2),
                      "bwd_tflops": round(f_bwd / (bwd_ms * 1e-3) / 1e12, 2) if do_bwd else None,
                      "fwd_at_clock": at_clock(f_fwd / (fwd_ms * 1e-3) / 1e12, PEAK_BF16_TFLOPS,
                                               "attn_fwd_bf16_d128_causal_N16384_B1_H32",
                                               ["fa_fwd_bf16.hip", "fa_device.h"])},
        "roofline": roofline,
    }
    if do_bwd and not args.no_det:
        del ws
        torch.cuda.empty_cache()
        out["bwd_det"] = det_section(fa, q, k, v, o, lse, do, True, args.steps, args.warmup, bwd_ms)
    if not args.no_fp8 or (do_bwd and not (args.no_gqa and args.no_varlen)):
        del q, k, v, do, o, lse, dq, dk, dv
        torch.cuda.empty_cache()
    if do_bwd and not args.no_gqa:
        out["gqa"] = gqa_section(fa, args.steps, args.warmup)
        torch.cuda.empty_cache()
    if do_bwd and not args.no_varlen:
        out["varlen"] = varlen_section(fa, args.steps, args.warmup)
        torch.cuda.empty_cache()
    if not args.no_fp8:
        torch.cuda.empty_cache()
        out["fp8"] = fp8_section(fa, args.steps, args.warmup)
    if not args.no_configs:
        torch.cuda.empty_cache()
        out["configs"] = configs_section(fa)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.cpu_heads)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
