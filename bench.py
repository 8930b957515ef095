"""Benchmark of the ternary linear layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Workload (the headline): decode GEMV, W 4096x4096 ternary from N(0, 0.02)
fp32 (per-tensor absmean scale, packed 4 MiB), one bf16 token ~N(0, 1)
quantised per token to int8, fp32 output.  One step = per-token int8
quantisation of the token + the packed-weight GEMV with its fused scale
epilogue.  Steps rotate over 128 distinct packed-weight buffers (512 MiB,
more than twice the 256 MB Infinity Cache) so that the weight stream comes
from HBM, as it does when a decode pass walks through a model's layers.
Inputs are resident in HBM before timing starts.  Launches are captured in a
HIP graph (torch.cuda.CUDAGraph) so that the host never paces the GPU.

Prints one JSON line.  ``value`` is algorithmic bytes of the step over its
time (GB/s).  ``roofline`` describes the GEMV kernel: its algorithmic bytes
per launch over its average launch time, against 8 TB/s.  ``cpu_baseline``
times the CPU oracle on a bounded sample of the same workload.  ``extra``
carries the prefill GEMM (int8 MFMA TOPS), a 4096^3 GEMM (one full round of
wide tiles) with the vendor int8 GEMM beside it, the BitLinear prologue, the FFN
decode shapes, the pack kernels (absmean, threshold, code-format
conversion), the steady-state GEMV rate (stacked projections in one launch),
1-bit binary weights, the SwiGLU decode FFN and the backward of the prefill
layer.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
PROFILE = os.path.join(ROOT, "profiles", "k_gemv_dot_decode_4096x4096_b1.md")
KERNEL_SOURCES = [os.path.join(ROOT, "ternary_quantized_linear_absmean_amd", "csrc", f)
                  for f in ("k_gemv.hip", "tq_device.hpp")]
INT8_PEAK_TOPS = 5000.0        # MI355X dense int8 MFMA, 5.0 POP/s
POOL = 128                     # distinct packed weights in the rotation


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=2048)
    p.add_argument("--warmup", type=int, default=256)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-extra", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--only", default="",
                   help="comma list of extra workloads to run: "
                        "prefill,square,bitlinear,pack,ffn,steady,binary1,ffn_decode,backward,"
                        "context")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run a plain 256 MiB device copy (for counter scaling)")
    return p.parse_args()


def gemv_bytes(M, N, K, per_row):
    # packed W + scale(s) + int8 tokens + sx + fp32 output
    return N * K // 4 + (4 * N if per_row else 4) + M * K + 4 * M + 4 * M * N


def quant_bytes(M, K, xbytes):
    return M * K * xbytes + M * K + 4 * M


def fused_bytes(M, N, K, xbytes, per_row):
    # tokens in + packed W + scale(s) + int8 tokens and sx out + fp32 output
    # (the int8 tokens are not read back: the kernel keeps them on chip)
    return M * K * xbytes + N * K // 4 + (4 * N if per_row else 4) + M * K + 4 * M + 4 * M * N


def source_digest():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def counter_traffic():
    """HBM bytes per launch of the fused decode kernel, from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary, or None when that summary is
    missing or was taken on a different version of the kernel source."""
    if not os.path.exists(PROFILE):
        return None
    fields = {}
    with open(PROFILE) as f:
        for line in f:
            if ":" in line and line.startswith("- "):
                k, v = line[2:].split(":", 1)
                fields[k.strip()] = v.strip().strip("`")
    if fields.get("kernel_source_sha256_16") != source_digest():
        return None
    try:
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def timed_graph(torch, graph, reps):
    """Replay `graph` reps times between synchronisations; seconds per replay."""
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s.record()
    for _ in range(reps):
        graph.replay()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / 1e3 / reps


def warm(torch, graph, seconds=0.05):
    """Replay `graph` for about `seconds` untimed: the GPU leaves its idle
    clocks only after some milliseconds of sustained matrix-core work, and a
    compute-bound kernel timed straight after latency-bound work reads 10-15%
    slow otherwise."""
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        graph.replay()
        torch.cuda.synchronize()


def capture(torch, fn):
    g = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        fn()                                   # warm the path once outside capture
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); this build has no "
              "multi-GPU path.", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import tq_inputs as ti
    from ternary_quantized_linear_absmean_amd import tq

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    # ------------------------------------------------------------ decode
    N, K = ti.WORKLOADS["decode"]["mats"][0]
    W = torch.from_numpy(ti.workload_weights("decode")).to(dev)
    X = torch.from_numpy(ti.workload_activations("decode")).to(dev).to(torch.bfloat16)
    packed0, scale = tq.tq_pack_ternary(W, "tensor")
    pool = [packed0.clone() for _ in range(POOL)]
    del W
    qbuf = torch.empty((1, K), dtype=torch.int8, device=dev)
    sxbuf = torch.empty((1,), dtype=torch.float32, device=dev)
    ybuf = torch.empty((1, N), dtype=torch.float32, device=dev)

    def decode_pass():
        # one decode step = per-token int8 quantisation + GEMV + scale epilogue
        for p in pool:
            tq.tq_quant_ternary_gemv(X, p, scale, N, K, "tensor", "f32", q=qbuf, sx=sxbuf,
                                     Y=ybuf)

    def decode_pass_two_calls():
        for p in pool:
            tq.tq_quant_act_int8(X, q=qbuf, sx=sxbuf)
            tq.tq_ternary_gemv(qbuf, sxbuf, p, scale, N, K, "tensor", "f32", Y=ybuf)

    def gemv_pass():
        for p in pool:
            tq.tq_ternary_gemv(qbuf, sxbuf, p, scale, N, K, "tensor", "f32", Y=ybuf)

    g_step = capture(torch, decode_pass)
    g_gemv = capture(torch, gemv_pass)
    g_two = capture(torch, decode_pass_two_calls)
    reps_w = max(1, args.warmup // POOL)
    reps = max(1, args.steps // POOL)
    steps = reps * POOL
    timed_graph(torch, g_step, reps_w)
    timed_graph(torch, g_gemv, reps_w)

    # timed region: exactly `steps` steps between synchronisations
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    sec_per_pass = timed_graph(torch, g_step, reps)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_s = sec_per_pass / POOL
    b_gemv = gemv_bytes(1, N, K, False)
    b_step = fused_bytes(1, N, K, 2, False)
    value = b_step / step_s / 1e9

    gemv_s = timed_graph(torch, g_gemv, reps) / POOL
    gemv_gbs = b_gemv / gemv_s / 1e9
    two_s = timed_graph(torch, g_two, reps) / POOL
    traffic = counter_traffic()

    result = {
        "metric": "ternary GEMV GB/s (% HBM peak) at K=N=4096 b=1; GEMM TOPS (% int8 MFMA peak)",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": reps_w * POOL,
        "ms_per_step": round(step_s * 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8 x ternary -> int32 acc, fp32 epilogue",
        "data": "synthetic (seeded N(0,0.02) weights, N(0,1) bf16 token)",
        "config": {"workload": "decode GEMV: bf16 token 1x4096 -> per-token int8, "
                               "packed ternary W 4096x4096 (per-tensor absmean), fp32 out; "
                               f"{POOL} distinct weight buffers in rotation",
                   "M": 1, "N": N, "K": K, "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
                   "entry_point": "tq_quant_ternary_gemv (quantise + GEMV, one launch)",
                   "two_call_step_us": round(two_s * 1e6, 3),
                   "kernel_source_sha256_16": source_digest(),
                   "timed_wall_s": round(wall, 4)},
        # the step is one launch of the fused quantise + GEMV kernel, so its
        # average launch time is the step time measured above
        "roofline": {"bound": "hbm", "kernel": "k_gemv_dot<bf16 X, K<=4096> (tq_quant_ternary_gemv)",
                     "achieved": round(value, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(value / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "bytes_per_launch": b_step, "avg_launch_us": round(step_s * 1e6, 3)},
        "gemv_int8_input": {"kernel": "k_gemv_dot<int8 q, K<=4096> (tq_ternary_gemv)",
                            "bytes_per_launch": b_gemv, "avg_launch_us": round(gemv_s * 1e6, 3),
                            "GBs": round(gemv_gbs, 2)},
    }

    if not args.no_extra:
        only = set(x for x in args.only.split(",") if x)
        result["extra"] = extras(torch, np, ti, tq, dev, only)
    if args.copy_calibration:
        result["copy_calibration"] = copy_calibration(torch, dev)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(np, ti, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def extras(torch, np, ti, tq, dev, only=frozenset()):
    out = {}
    want = (lambda name: not only or name in only)
    if want("prefill") or want("pack"):
        out.update(extra_prefill(torch, ti, tq, dev, want))
    if want("square"):
        out.update(extra_square(torch, tq, dev))
    if want("bitlinear"):
        out.update(extra_bitlinear(torch, ti, tq, dev))
    if want("ffn"):
        out.update(extra_ffn(torch, ti, tq, dev))
    if want("steady"):
        out.update(extra_steady(torch, ti, tq, dev))
    if want("binary1"):
        out.update(extra_binary1(torch, ti, tq, dev))
    if want("ffn_decode"):
        out.update(extra_ffn_decode(torch, ti, tq, dev))
    if want("backward"):
        out.update(extra_backward(torch, ti, tq, dev))
    if want("context"):
        out.update(extra_context(torch, dev))
    torch.cuda.synchronize()
    return out


def extra_prefill(torch, ti, tq, dev, want):
    out = {}
    # prefill GEMM 2048 x 11008 x 4096 -> bf16, int8 MFMA
    M = 2048
    N, K = ti.WORKLOADS["prefill"]["mats"][0]
    W = torch.from_numpy(ti.workload_weights("prefill")).to(dev)
    packed, scale = tq.tq_pack_ternary(W, "tensor")
    X = torch.from_numpy(ti.workload_activations("prefill")).to(dev).to(torch.bfloat16)
    q, sx = tq.tq_quant_act_int8(X)
    Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    reps = 8
    if want("prefill"):
        g = capture(torch, lambda: [tq.tq_ternary_gemm(q, sx, packed, scale, N, K, "tensor",
                                                       "bf16", Y=Y) for _ in range(reps)])
        warm(torch, g)
        t = timed_graph(torch, g, 5) / reps
        tops = 2.0 * M * N * K / t / 1e12
        out["prefill_gemm"] = {"shape": [M, N, K], "out": "bf16", "us": round(t * 1e6, 2),
                               "TOPS": round(tops, 1),
                               "pct_int8_peak": round(100 * tops / INT8_PEAK_TOPS, 2)}
        qx = torch.empty_like(q)
        sxx = torch.empty_like(sx)
        g = capture(torch, lambda: [tq.tq_quant_act_int8(X, q=qx, sx=sxx) for _ in range(reps)])
        t = timed_graph(torch, g, 5) / reps
        out["prefill_quant"] = {"shape": [M, K], "us": round(t * 1e6, 2),
                                "GBs": round(quant_bytes(M, K, 2) / t / 1e9, 1)}
    if want("pack"):
        # pack of the prefill weight (per-tensor: reduce + pack passes)
        pk = torch.empty_like(packed)
        sc = torch.empty_like(scale)
        ws = torch.empty((tq.tq_pack_workspace_bytes(N, K, "tensor"),), dtype=torch.uint8,
                         device=dev)
        g = capture(torch, lambda: tq.tq_pack_ternary(W, "tensor", packed=pk, scale=sc,
                                                      workspace=ws))
        t = timed_graph(torch, g, 10)
        out["pack_tensor"] = {"shape": [N, K], "us": round(t * 1e6, 2),
                              "GBs": round((4 * N * K + N * K // 4) / t / 1e9, 1)}
        # BitRASP's 0.55 threshold per row, and conversion of the packed
        # weight to Hetman-2b's Format 0 (11 MB read + 11 MB written)
        pr = torch.empty_like(packed)
        sr = torch.empty((N,), dtype=torch.float32, device=dev)
        g = capture(torch, lambda: tq.tq_pack_ternary_threshold(W, "row", "relative", 0.55,
                                                                packed=pr, scale=sr))
        t = timed_graph(torch, g, 10)
        out["pack_threshold_row_0.55"] = {"shape": [N, K], "us": round(t * 1e6, 2),
                                          "GBs": round((4 * N * K + N * K // 4) / t / 1e9, 1)}
        f0 = torch.empty_like(packed)
        g = capture(torch, lambda: [tq.tq_convert_codes(packed, "native", "f0", dst=f0)
                                    for _ in range(reps)])
        timed_graph(torch, g, 2)
        t = timed_graph(torch, g, 10) / reps
        out["convert_codes_to_f0"] = {"bytes": 2 * packed.numel(), "us": round(t * 1e6, 2),
                                      "GBs": round(2 * packed.numel() / t / 1e9, 1)}
    return out


def extra_square(torch, tq, dev):
    """GEMM 4096 x 4096 x 4096 -> bf16: 256 tiles of 256 x 256, one full
    round of the wide-tile kernel (one workgroup per CU), next to the vendor
    int8 GEMM on the same shape."""
    M = N = K = 4096
    gen = torch.Generator(device=dev)
    gen.manual_seed(4096)
    W = torch.randn((N, K), generator=gen, device=dev) * 0.02
    packed, scale = tq.tq_pack_ternary(W, "tensor")
    X = torch.randn((M, K), generator=gen, device=dev).to(torch.bfloat16)
    q, sx = tq.tq_quant_act_int8(X)
    Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    reps = 8
    g = capture(torch, lambda: [tq.tq_ternary_gemm(q, sx, packed, scale, N, K, "tensor", "bf16",
                                                   Y=Y) for _ in range(reps)])
    warm(torch, g)
    t = timed_graph(torch, g, 5) / reps
    tops = 2.0 * M * N * K / t / 1e12
    out = {"gemm_4096x4096x4096": {"shape": [M, N, K], "out": "bf16", "kernel": "k_gemm_wide",
                                   "us": round(t * 1e6, 2), "TOPS": round(tops, 1),
                                   "pct_int8_peak": round(100 * tops / INT8_PEAK_TOPS, 2)}}
    try:
        B = (torch.randint(-1, 2, (N, K), generator=gen, device=dev)).to(torch.int8)
        g = capture(torch, lambda: [torch._int_mm(q, B.t()) for _ in range(reps)])
        warm(torch, g)
        t = timed_graph(torch, g, 5) / reps
        out["vendor_int8_gemm_4096x4096x4096"] = {
            "api": "torch._int_mm (int8 x int8 -> int32)", "us": round(t * 1e6, 2),
            "TOPS": round(2.0 * M * N * K / t / 1e12, 1)}
    except Exception as e:  # the reference is optional context
        out["vendor_int8_gemm_4096x4096x4096"] = {"error": str(e)[:200]}
    return out


def extra_bitlinear(torch, ti, tq, dev):
    out = {}
    reps = 8
    # BitLinear: prologue (RMSNorm + FWHT-512 + int8) and GEMM 512 x 4096 x 4096, fp32 out
    Wb = torch.from_numpy(ti.workload_weights("bitlinear")).to(dev)
    Xb = torch.from_numpy(ti.workload_activations("bitlinear")).to(dev).to(torch.bfloat16)
    pb, sb = tq.tq_pack_ternary(Wb, "row")
    qb = torch.empty((512, 4096), dtype=torch.int8, device=dev)
    sxb = torch.empty((512,), dtype=torch.float32, device=dev)
    Yb = torch.empty((512, 4096), dtype=torch.float32, device=dev)
    g = capture(torch, lambda: [tq.tq_quant_act_int8(Xb, clamp=(0.05, 40.0), rmsnorm=True,
                                                     fwht_block=512, q=qb, sx=sxb)
                                for _ in range(reps)])
    t = timed_graph(torch, g, 5) / reps
    out["bitlinear_prologue"] = {"shape": [512, 4096], "us": round(t * 1e6, 2),
                                 "GBs": round(quant_bytes(512, 4096, 2) / t / 1e9, 1)}
    g = capture(torch, lambda: [tq.tq_ternary_gemm(qb, sxb, pb, sb, 4096, 4096, "row", "f32",
                                                   Y=Yb) for _ in range(reps)])
    warm(torch, g)
    t = timed_graph(torch, g, 5) / reps
    tops = 2.0 * 512 * 4096 * 4096 / t / 1e12
    out["bitlinear_gemm"] = {"shape": [512, 4096, 4096], "us": round(t * 1e6, 2),
                             "TOPS": round(tops, 1),
                             "pct_int8_peak": round(100 * tops / INT8_PEAK_TOPS, 2)}
    return out


def extra_ffn(torch, ti, tq, dev):
    out = {}
    # FFN decode shapes (per-row scales), GEMV rotation over 64 buffers each
    ffn = {}
    for j, (N, K) in enumerate(ti.WORKLOADS["ffn"]["mats"]):
        W = torch.from_numpy(ti.workload_weights("ffn", j)).to(dev)
        p0, s0 = tq.tq_pack_ternary(W, "row")
        del W
        pool = [p0.clone() for _ in range(64)]
        for b in ti.WORKLOADS["ffn"]["batches"]:
            Xf = torch.from_numpy(ti.workload_activations("ffn", j, b)).to(dev).to(torch.bfloat16)
            qf, sf = tq.tq_quant_act_int8(Xf)
            Yf = torch.empty((b, N), dtype=torch.float32, device=dev)
            g = capture(torch, lambda: [tq.tq_ternary_gemv(qf, sf, p, s0, N, K, "row", "f32",
                                                           Y=Yf) for p in pool])
            timed_graph(torch, g, 2)
            t = timed_graph(torch, g, 10) / len(pool)
            gb = gemv_bytes(b, N, K, True) / t / 1e9
            ffn[f"{'up' if j == 0 else 'down'}_{N}x{K}_b{b}"] = {
                "us": round(t * 1e6, 3), "GBs": round(gb, 1),
                "pct_hbm_peak": round(100 * gb / HBM_PEAK_GBS, 1)}
        del pool
    out["ffn_gemv"] = ffn
    return out


def extra_steady(torch, ti, tq, dev):
    """Steady-state decode GEMV throughput, labelled as such: G stacked 4096x4096
    projections that share one token (N = 4096*G rows), one launch each, the
    stacked weights rotating over at least 512 MiB.  One 4 MiB launch is bound
    by latency; this shows the rate once more bytes are in flight."""
    K = 4096
    W = torch.from_numpy(ti.workload_weights("decode", 0)).to(dev)
    p0, s0 = tq.tq_pack_ternary(W, "tensor")
    del W
    X = torch.from_numpy(ti.workload_activations("decode", 0, 1)).to(dev).to(torch.bfloat16)
    q, sx = tq.tq_quant_act_int8(X)
    out = {}
    for G in (8, 32):
        N = 4096 * G
        stacked = torch.cat([p0] * G, dim=0)
        pool = [stacked.clone() for _ in range(max(2, 128 // G))]
        del stacked
        Y = torch.empty((1, N), dtype=torch.float32, device=dev)
        g = capture(torch, lambda: [tq.tq_ternary_gemv(q, sx, p, s0, N, K, "tensor", "f32", Y=Y)
                                    for p in pool])
        timed_graph(torch, g, 2)
        t = timed_graph(torch, g, 8) / len(pool)
        gb = gemv_bytes(1, N, K, False) / t / 1e9
        out[f"stacked_{G}x4096x4096_b1"] = {"us": round(t * 1e6, 3), "GBs": round(gb, 1),
                                             "pct_hbm_peak": round(100 * gb / HBM_PEAK_GBS, 1)}
        del pool
    return {"gemv_steady_state": out}


def extra_binary1(torch, ti, tq, dev):
    """1-bit sign-packed binary weights (R*C/8 bytes) against the same binary
    weights in the 2-bit code format, decode GEMV 4096x4096 per-row scales,
    1 and 16 tokens, the packed weights rotating over 512 MiB per form."""
    N = K = 4096
    W = torch.from_numpy(ti.workload_weights("bitlinear", 0)).to(dev)
    p1, s1 = tq.tq_pack_binary1(W, "row")
    p2, s2 = tq.tq_pack_ternary(W, "row", "binary")
    del W
    out = {}
    for b in (1, 16):
        X = torch.from_numpy(ti.workload_activations("bitlinear", 0, b)[:b]).to(dev)
        q, sx = tq.tq_quant_act_int8(X)
        Y = torch.empty((b, N), dtype=torch.float32, device=dev)
        for name, fn, p0, s0, wbytes in (
                ("1bit", tq.tq_binary1_gemv, p1, s1, N * K // 8),
                ("2bit", tq.tq_ternary_gemv, p2, s2, N * K // 4)):
            pool = [p0.clone() for _ in range(max(2, (512 << 20) // wbytes))]
            g = capture(torch, lambda: [fn(q, sx, p, s0, N, K, "row", "f32", Y=Y) for p in pool])
            timed_graph(torch, g, 2)
            t = timed_graph(torch, g, 8) / len(pool)
            nbytes = wbytes + 4 * N + b * K + 4 * b + 4 * b * N
            gb = nbytes / t / 1e9
            out[f"{name}_4096x4096_b{b}"] = {"us": round(t * 1e6, 3), "bytes": nbytes,
                                             "GBs": round(gb, 1),
                                             "pct_hbm_peak": round(100 * gb / HBM_PEAK_GBS, 1)}
            del pool
    return {"binary_gemv": out}


def extra_ffn_decode(torch, ti, tq, dev):
    """Decode FFN with the SwiGLU clamp (gate/up 6912x2560, down 2560x6912,
    per-row scales): tq_ffn_swiglu_decode, two launches per step, the three
    packed matrices rotating over 40 sets (about 530 MB)."""
    d_model, d_ffn = 2560, 6912
    mats = []
    for W in (ti.normal_weights(ti.weight_seed(ti.WORKLOADS["ffn"]["cfg"], 2), d_ffn, d_model),
              ti.workload_weights("ffn", 0), ti.workload_weights("ffn", 1)):
        p0, s0 = tq.tq_pack_ternary(torch.from_numpy(W).to(dev), "row")
        mats.append((p0, s0))
    sets = [[(p.clone(), s) for (p, s) in mats] for _ in range(40)]
    wbytes = 3 * d_ffn * d_model // 4 + 4 * (2 * d_ffn + d_model)
    out = {}
    for b in (1, 4, 16):
        X = torch.from_numpy(ti.workload_activations("ffn", 0, b)).to(dev).to(torch.bfloat16)
        Y, buf = tq.tq_ffn_swiglu_decode(X, *mats, d_model, d_ffn)
        g = capture(torch, lambda: [tq.tq_ffn_swiglu_decode(X, *st, d_model, d_ffn, buffers=buf,
                                                            Y=Y) for st in sets])
        timed_graph(torch, g, 2)
        t = timed_graph(torch, g, 8) / len(sets)
        # weights + X in, q_x/sx_x out, H out and back in, q_h/sx_h out, Y out
        nbytes = (wbytes + 2 * b * d_model + (b * d_model + 4 * b) + 2 * 4 * b * d_ffn +
                  (b * d_ffn + 4 * b) + 4 * b * d_model)
        gb = nbytes / t / 1e9
        out[f"b{b}"] = {"us": round(t * 1e6, 3), "bytes": nbytes, "GBs": round(gb, 1),
                        "pct_hbm_peak": round(100 * gb / HBM_PEAK_GBS, 1), "launches": 2}
    del sets
    return {"ffn_swiglu_decode": out}


BF16_MFMA_PEAK_TFLOPS = 2500.0


def extra_backward(torch, ti, tq, dev):
    """Backward through the prefill layer (2048 tokens, W 11008 x 4096,
    per-tensor scale): the input gradient through the packed codes and the
    weight gradient X^T dY, seeded gradients ~N(0, 1).  TFLOP/s counts the
    2 M N K of the product; mfma_frac counts the bf16 matrix-core passes the
    kernel issues (three per fp32 operand split) against the dense bf16 peak.
    torch's dense fp32 and bf16 products of the same shape are context."""
    M, N, K = 2048, 11008, 4096
    W = torch.from_numpy(ti.workload_weights("prefill")).to(dev)
    packed, scale = tq.tq_pack_ternary(W, "tensor")
    del W
    dY32 = torch.from_numpy(ti.workload_output_grads("prefill")).to(dev)
    X16 = torch.from_numpy(ti.workload_activations("prefill")).to(dev).to(torch.bfloat16)
    X32 = X16.float()
    flops = 2.0 * M * N * K
    out = {}
    R = 5

    def timed(fn):
        g = capture(torch, lambda: [fn() for _ in range(R)])
        warm(torch, g)
        return timed_graph(torch, g, 3) / R

    dX = torch.empty((M, K), dtype=torch.float32, device=dev)
    for name, dY, passes in (("f32", dY32, 3), ("bf16", dY32.bfloat16(), 1)):
        t = timed(lambda: tq.tq_ternary_backward_input(dY, packed, scale, K, dX=dX))
        out[f"input_grad_dY_{name}"] = {
            "us": round(t * 1e6, 1), "TFLOPs": round(flops / t / 1e12, 1),
            "mfma_frac": round(passes * flops / t / 1e12 / BF16_MFMA_PEAK_TFLOPS, 3)}
    dW = torch.empty((N, K), dtype=torch.float32, device=dev)
    for name, X, dY, passes in (("X_f32_dY_f32", X32, dY32, 6), ("X_bf16_dY_f32", X16, dY32, 3),
                                ("X_bf16_dY_bf16", X16, dY32.bfloat16(), 1)):
        t = timed(lambda: tq.tq_ternary_backward_weight(X, dY, dW=dW))
        out[f"weight_grad_{name}"] = {
            "us": round(t * 1e6, 1), "TFLOPs": round(flops / t / 1e12, 1),
            "mfma_frac": round(passes * flops / t / 1e12 / BF16_MFMA_PEAK_TFLOPS, 3)}
    Wd = torch.randn((N, K), device=dev)
    for name, dt in (("f32", torch.float32), ("bf16", torch.bfloat16)):
        a, b = dY32.to(dt), Wd.to(dt)
        t = timed(lambda: torch.mm(a, b))
        out[f"context_torch_dense_mm_{name}"] = {"us": round(t * 1e6, 1),
                                                "TFLOPs": round(flops / t / 1e12, 1)}
    return {"backward_prefill_2048x11008x4096": out}


def extra_context(torch, dev):
    """Reference points, not this library's work: what a plain torch kernel
    needs to stream 4 MiB per launch under the same 128-buffer rotation and
    graph replay (the floor a 4 MiB decode GEMV sits on), and the vendor
    int8 GEMM (hipBLASLt through torch._int_mm, int8 weights) on the prefill
    shape."""
    out = {}
    pool = [torch.ones(1 << 20, dtype=torch.int32, device=dev) for _ in range(POOL)]
    dst = torch.empty(1 << 20, dtype=torch.int32, device=dev)
    res = torch.empty((), dtype=torch.int32, device=dev)
    g = capture(torch, lambda: [dst.copy_(p) for p in pool])
    timed_graph(torch, g, 2)
    t = timed_graph(torch, g, 16) / POOL
    out["torch_copy_4MiB_rotating"] = {"us": round(t * 1e6, 3),
                                       "GBs_read_plus_write": round(8 * 2**20 / t / 1e9, 1)}
    g = capture(torch, lambda: [torch.amax(p, dim=0, out=res) for p in pool])
    timed_graph(torch, g, 2)
    t = timed_graph(torch, g, 16) / POOL
    out["torch_amax_4MiB_rotating"] = {"us": round(t * 1e6, 3),
                                       "GBs_read": round(4 * 2**20 / t / 1e9, 1)}
    del pool
    try:
        M, N, K = 2048, 11008, 4096
        A = torch.randint(-127, 128, (M, K), dtype=torch.int8, device=dev)
        B = torch.randint(-1, 2, (N, K), dtype=torch.int8, device=dev)
        g = capture(torch, lambda: [torch._int_mm(A, B.t()) for _ in range(8)])
        warm(torch, g)
        t = timed_graph(torch, g, 5) / 8
        out["vendor_int8_gemm_prefill"] = {"api": "torch._int_mm (int8 x int8 -> int32)",
                                           "shape": [M, N, K], "us": round(t * 1e6, 2),
                                           "TOPS": round(2.0 * M * N * K / t / 1e12, 1)}
    except Exception as e:  # the reference is optional context
        out["vendor_int8_gemm_prefill"] = {"error": str(e)[:200]}
    return out


def copy_calibration(torch, dev):
    """A plain elementwise kernel of known traffic (reads 256 MiB, writes
    256 MiB, beyond the Infinity Cache): its FETCH_SIZE / WRITE_SIZE
    readings scale the counters of the kernels above to bytes."""
    n = 64 << 20                                   # fp32 elements = 256 MiB
    a = torch.ones(n, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        torch.neg(a, out=b)
    torch.cuda.synchronize()
    return {"kernel": "torch.neg fp32", "bytes_read": 4 * n, "bytes_written": 4 * n,
            "launches": 3}


def cpu_baseline(np, ti, seconds):
    """The oracle on the host: per-token quantisation + integer contraction
    + fp64 epilogue for the decode workload, repeated for ~`seconds`."""
    import oracle
    N, K = ti.WORKLOADS["decode"]["mats"][0]
    W = ti.workload_weights("decode")
    X = ti.workload_activations("decode")
    packed, scale = oracle.pack_ternary(W, "tensor")
    n = 0
    t0 = time.perf_counter()
    while True:
        q, sx = oracle.quant_act_int8(X)
        acc = oracle.contract(q, packed, K)
        oracle.epilogue(acc, scale, sx)
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    per = el / n
    b = gemv_bytes(1, N, K, False) + quant_bytes(1, K, 2)
    return {"value": round(b / per / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{n} decode steps (quant + contraction + epilogue, 1x4096x4096) in "
                      f"{el:.1f} s, numpy int64 on one host thread",
            "ms_per_step": round(per * 1e3, 3)}


if __name__ == "__main__":
    main()
