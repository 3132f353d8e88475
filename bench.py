#!/usr/bin/env python3
"""Benchmark of the SVDQuant W4A4 + low-rank linear and the INT8 KV-cache quantizer on one GPU.

One step is one pass of the whole hot path over one batch of synthetic input:
  svdq_quantize_act_e3m2 + svdq_w4a4_gemm_e3m2
                                       on the FFN up-projection shape
                                       (X [4608, 3072] bf16, W [3072, 12288], r = 32, group 64;
                                       INT4 codes carried as BF6 on the FP6 matrix units)
  kv_int8_quant + kv_int8_dequant      on K and V bf16 [10240 tokens, 32 heads, 128 dim]
Weight preparation (smoothing, SVD, residual packing) is offline and untimed.  The INT8-unit
route (svdq_quantize_act + svdq_w4a4_gemm, same codes and result) and the W4A8 variant
(svdq_quantize_act_a8 + svdq_w4a8_gemm: 8-bit activation codes, same INT4 weights) are timed
after the timed region and reported beside it, and so is kv_int8_attention (decode attention
of one query per head reading the INT8 K and V codes of one batch).

Timing: W warm-up steps, then K timed steps bracketed by torch.cuda.synchronize(); every call
is bracketed by HIP events on the stream it is launched on, so each kernel's mean duration is
measured live.  Inputs rotate over 3 batches (about 590 MB, more than twice the 256 MB
last-level cache) so the HBM-bound kernels read from HBM.

Prints one JSON line.  `value` is the fused W4A4 + low-rank GEMM throughput in TOPS
(2 M N K integer ops per launch / mean launch time); the KV quantizer's GB/s and each kernel's
time are reported beside it.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "fused W4A4+low-rank GEMM TOPS and % of INT8 MFMA peak; KV-quant GB/s"
INT8_PEAK_TOPS = 5000.0      # MI355X dense INT8 MFMA, 5.0 POP/s
FP6_PEAK_TOPS = 10100.0      # MI355X dense FP6 MFMA, 10.1 PFLOP/s (the GEMM's matrix dtype)
HBM_PEAK_GBPS = 8000.0       # MI355X HBM3E, 8 TB/s
M, K, N, RANK = 4608, 3072, 12288, 32
LORA_RANK = 16   # adapter rank of the LoRA line (reported beside the product path)
KV_T, KV_H, KV_D = 10240, 32, 128
ROTATE = 3


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=M,
                    help="token rows of the oracle's CPU baseline sample")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MB",
                    help="first copy MB megabytes device to device once (a plain copy of known "
                         "size, the reference for the HBM byte counters of a profiler run)")
    return ap.parse_args()


# HBM traffic of the GEMM kernel per launch, measured with rocprofv3 counters (FETCH_SIZE and
# WRITE_SIZE, each scaled by what the same counter reads for a plain copy of known size).  The
# measurement is recorded with the SHA-256 of the kernel source it was taken on; a different
# source reports no traffic.
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "w4a4_gemm_e3m2_ffn_up_4608x3072x12288_traffic.md")
GEMM_SOURCE = os.path.join(ROOT, "bit_post_quantized_amd", "csrc", "w4a4_gemm_e3m2.hip")


def recorded_traffic():
    import hashlib
    try:
        rec = dict(line.split(":", 1) for line in open(TRAFFIC_RECORD).read().splitlines()
                   if line.startswith(("source_sha256:", "traffic_bytes_per_launch:")))
        src = hashlib.sha256(open(GEMM_SOURCE, "rb").read()).hexdigest()
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256", "").strip() != src:
        return None
    return int(rec["traffic_bytes_per_launch"].strip())


def algorithmic_bytes():
    G = K // 64
    act = M * K * 2 + K * 4 + K * RANK * 2 + M * K * 3 // 4 + G * M * 2 + M * RANK * 4
    C = KV_H * KV_D
    kvq = KV_T * C * (2 + 1) + C * (4 + 1)        # per tensor: read x, write q, scale, zero
    kvd = KV_T * C * (1 + 2) + C * (4 + 1)        # per tensor: read q, scale, zero, write x'
    gemm = (M * K + N * K) * 3 // 4 + G * M * 2 + G * N * 2 + M * RANK * 4 + N * RANK * 2 + M * N * 2
    return dict(act=act, kv_quant=kvq, kv_dequant=kvd, gemm=gemm)


def clock_reader():
    """A function returning (graphics MHz, memory MHz) of the first GPU now, or None when the
    ROCm SMI library is not usable here (the clocks are then reported as null)."""
    try:
        import amdsmi
        amdsmi.amdsmi_init()
        h = amdsmi.amdsmi_get_processor_handles()[0]

        def read():
            return (amdsmi.amdsmi_get_clock_info(h, amdsmi.AmdSmiClkType.SYS)["clk"],
                    amdsmi.amdsmi_get_clock_info(h, amdsmi.AmdSmiClkType.MEM)["clk"])
        read()
        return read
    except Exception:  # no SMI library, no permission, no device: clocks are context only
        return None


def clock_summary(samples):
    if not samples:
        return None
    g = [a for a, _ in samples if isinstance(a, (int, float))]
    m = [b for _, b in samples if isinstance(b, (int, float))]
    if not g or not m:
        return None
    return {"sclk_mhz": {"mean": round(float(np.mean(g))), "min": min(g), "max": max(g)},
            "mclk_mhz": {"mean": round(float(np.mean(m))), "min": min(m), "max": max(m)},
            "samples": len(samples)}


def cpu_baseline(rows: int):
    """The oracle (as it stands) on a bounded sample: `rows` tokens of the same workload."""
    from oracle import svdquant as osq
    from synthetic import make_linear

    d = make_linear(3, M=rows)
    cfg_rank = RANK
    # weights: the oracle's own preparation of the same W (untimed offline step, as on the GPU)
    pw = osq.prepare_weights(d["X"], d["W"], 0.5, cfg_rank)
    packed = osq.pack_weights(pw["R32"])
    # repeat the oracle pass until about 10 s of CPU work have been timed (at least once)
    reps, dt = 0, 0.0
    while reps == 0 or (dt < 10.0 and reps < 4):
        t0 = time.perf_counter()
        act = osq.quantize_act(d["X"], pw["inv_lambda"], pw["L1b"])
        osq.linear_output(act["codes"], act["s_x"], packed["codes"], packed["s_w"], act["T"],
                          pw["L2b"])
        dt += time.perf_counter() - t0
        reps += 1
    cores = len(os.sched_getaffinity(0))
    return {"value": 2.0 * rows * N * K * reps / dt / 1e12, "unit": "TOPS", "cores": cores,
            "kind": "oracle",
            "sample": f"{rows} of {M} tokens of the {M}x{K}x{N} r={RANK} linear: activation "
                      f"quantization + low-rank down-projection + integer group GEMM + output "
                      f"(fp64 NumPy/OpenBLAS), {reps} pass(es) in {dt:.1f} s"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the linear layer and the "
              "KV quantizer run on one device; sharding them across GPUs is not implemented.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from bit_post_quantized_amd import binding as B
    from bit_post_quantized_amd import layer
    from synthetic import make_kv, make_linear

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    B.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    # ---- inputs (seeded, synthetic) and offline weight preparation
    t_setup = time.perf_counter()
    d = make_linear(3)
    pw = layer.convert_weights(bf16(d["W"]).cpu(), bf16(d["X"]).cpu(), 0.5, RANK, device=dev,
                               e3m2=True, keep_residual=True)
    wq4 = torch.empty(N, K // 2, dtype=torch.uint8, device=dev)   # INT8-route weights
    ws4 = torch.empty(K // 64, N, dtype=torch.float16, device=dev)
    X = [bf16(d["X"])] + [bf16(make_linear(3, seed=s)["X"]) for s in range(1, ROTATE)]
    kvs = []
    for s in range(ROTATE):
        kv = make_kv(seed=s)
        kvs.append((bf16(kv["K"]).view(KV_T, -1), bf16(kv["V"]).view(KV_T, -1)))
    C = KV_H * KV_D
    acts = [layer.alloc_act(M, K, RANK, dev, e3m2=True) for _ in range(ROTATE)]
    Y = [torch.empty(M, N, dtype=torch.bfloat16, device=dev) for _ in range(ROTATE)]
    q = [[torch.empty(KV_T, C, dtype=torch.uint8, device=dev) for _ in range(2)] for _ in range(ROTATE)]
    sc = [[torch.empty(C, dtype=torch.float32, device=dev) for _ in range(2)] for _ in range(ROTATE)]
    zp = [[torch.empty(C, dtype=torch.uint8, device=dev) for _ in range(2)] for _ in range(ROTATE)]
    xo = [[torch.empty(KV_T, C, dtype=torch.bfloat16, device=dev) for _ in range(2)] for _ in range(ROTATE)]
    wsp = torch.empty(B.kv_int8_workspace_bytes(KV_T, C), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t_setup

    stream = torch.cuda.current_stream()
    names = ["act", "gemm", "kv_quant", "kv_dequant"]
    if args.copy_probe > 0:
        n = args.copy_probe * 1024 * 1024 // 4   # fp32 elements: read MB, write MB (a negation)
        src_b = torch.ones(n, dtype=torch.float32, device=dev)
        dst_b = torch.empty(n, dtype=torch.float32, device=dev)
        torch.neg(src_b, out=dst_b)
        torch.cuda.synchronize()
        del src_b, dst_b

    def step(i, ev=None):
        b = i % ROTATE
        a = acts[b]
        calls = [
            ("act", lambda: B.svdq_quantize_act_e3m2(X[b], pw.inv_lambda, pw.L1p, RANK, a.xq,
                                                     a.x_scales, a.T, stream)),
            ("gemm", lambda: B.svdq_w4a4_gemm_e3m2(a.xq, a.x_scales, a.T, pw.wq, pw.w_scales,
                                                   pw.L2, None, RANK, Y[b], stream)),
        ]
        for t in range(2):
            calls.append(("kv_quant", lambda t=t: B.kv_int8_quant(kvs[b][t], q[b][t], sc[b][t],
                                                                  zp[b][t], wsp, stream)))
        for t in range(2):
            calls.append(("kv_dequant", lambda t=t: B.kv_int8_dequant(q[b][t], sc[b][t], zp[b][t],
                                                                      xo[b][t], stream)))
        for name, fn in calls:
            if ev is not None:
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                fn()
                e1.record(stream)
                ev[name].append((e0, e1))
            else:
                fn()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    read_clock = clock_reader()
    ev = {n: [] for n in names}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, ev)
    # clocks while the queued steps run (a few ms of host time, well inside the GPU's backlog)
    clk = []
    if read_clock is not None:
        for _ in range(8):
            try:
                clk.append(read_clock())
            except Exception:
                break
            time.sleep(0.001)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    samples = {n: np.array([a.elapsed_time(b) for a, b in ev[n]]) * 1e3 for n in names}  # us
    ms = {n: float(samples[n].mean()) * 1e-3 for n in names}
    stats_us = {n: {"median": round(float(np.median(v)), 2), "p10": round(float(np.percentile(v, 10)), 2),
                    "p90": round(float(np.percentile(v, 90)), 2), "calls": int(v.size)}
                for n, v in samples.items()}

    # ---- the INT8-unit route on the same batch, outside the timed region
    B.svdq_pack_weights(pw.R32, wq4, ws4)
    xq4 = torch.empty(M, K // 2, dtype=torch.uint8, device=dev)
    xs4 = torch.empty(M, K // 64, dtype=torch.float16, device=dev)
    T4 = torch.empty(M, RANK, dtype=torch.float32, device=dev)
    xq8 = torch.empty(M, K, dtype=torch.int8, device=dev)   # W4A8 variant: 8-bit activations

    def time10(fn):
        fn()
        torch.cuda.synchronize()
        evs = []
        for _ in range(10):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            evs.append((e0, e1))
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in evs]))

    int8_ms = {
        "act": time10(lambda: B.svdq_quantize_act(X[0], pw.inv_lambda, pw.L1p, RANK, xq4, xs4,
                                                  T4, stream)),
        "gemm": time10(lambda: B.svdq_w4a4_gemm(xq4, xs4, T4, wq4, ws4, pw.L2, None, RANK, Y[0],
                                                stream)),
    }
    w4a8_ms = {
        "act": time10(lambda: B.svdq_quantize_act_a8(X[0], pw.inv_lambda, pw.L1p, RANK, xq8, xs4,
                                                     T4, stream)),
        "gemm": time10(lambda: B.svdq_w4a8_gemm(xq8, xs4, T4, wq4, ws4, pw.L2, None, RANK, Y[0],
                                                stream)),
    }
    # LoRA: a seeded rank-16 adapter joined to the 16-bit branch (rank 32 + 16 = 48), FP6 route,
    # the residual's codes and scales shared with the base layer
    gl = torch.Generator().manual_seed(7)
    pwl = layer.attach_lora(pw, torch.randn(K, LORA_RANK, generator=gl, dtype=torch.float64) * 0.02,
                            torch.randn(LORA_RANK, N, generator=gl, dtype=torch.float64) * 0.02)
    al = layer.alloc_act(M, K, pwl.rank, dev, e3m2=True)
    lora_ms = {
        "act": time10(lambda: B.svdq_quantize_act_e3m2(X[0], pwl.inv_lambda, pwl.L1p, pwl.rank,
                                                       al.xq, al.x_scales, al.T, stream)),
        "gemm": time10(lambda: B.svdq_w4a4_gemm_e3m2(al.xq, al.x_scales, al.T, pwl.wq,
                                                     pwl.w_scales, pwl.L2, None, pwl.rank, Y[0],
                                                     stream)),
    }
    # decode attention over the INT8 cache of batch 0 (one query per head): reads the codes
    q_att = torch.randn(1, KV_H, KV_D, device=dev).to(torch.bfloat16)
    o_att = torch.empty(1, KV_H, KV_D, dtype=torch.bfloat16, device=dev)
    ws_att = torch.empty(B.kv_int8_attention_workspace_bytes(1, KV_T, KV_H, KV_D),
                         dtype=torch.uint8, device=dev)
    attn_ms = time10(lambda: B.kv_int8_attention(q_att, q[0][0], sc[0][0], zp[0][0], q[0][1],
                                                 sc[0][1], zp[0][1], KV_D ** -0.5, o_att, ws_att,
                                                 stream))
    attn_bytes = 2 * KV_T * C + 2 * C * 5 + 2 * 1 * C * 2
    gemm_ops = 2.0 * M * N * K
    gemm_tops = gemm_ops / (ms["gemm"] * 1e-3) / 1e12
    ab = algorithmic_bytes()
    gbps = {n: ab[n] / (ms[n] * 1e-3) / 1e9 for n in ("act", "kv_quant", "kv_dequant")}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args.cpu_rows)

    out = {
        "metric": METRIC,
        "value": round(gemm_tops, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp6-e3m2 codes, fp32 accumulate",
        "data": "synthetic",
        "config": {"workload": f"svdquant_linear M{M} K{K} N{N} r{RANK} g64 bf16-out + "
                               f"kv_int8 K,V [{KV_T},{KV_H},{KV_D}] bf16",
                   "M": M, "K": K, "N": N, "rank": RANK, "group": 64,
                   "kv_tokens": KV_T, "kv_heads": KV_H, "kv_dim": KV_D},
        "roofline": {"bound": "mfma", "kernel": "w4a4_gemm_e3m2", "achieved": round(gemm_tops, 2),
                     "peak": FP6_PEAK_TOPS, "unit": "TFLOP/s",
                     "frac": round(gemm_tops / FP6_PEAK_TOPS, 4), "traffic": recorded_traffic(),
                     "algorithmic_bytes": ab["gemm"]},
        "cpu_baseline": cpu,
        "pct_int8_peak": round(100.0 * gemm_tops / INT8_PEAK_TOPS, 2),
        "kv_quant_GBps": round(gbps["kv_quant"], 1),
        "kv_quant_pct_hbm_peak": round(100.0 * gbps["kv_quant"] / HBM_PEAK_GBPS, 2),
        "kv_dequant_GBps": round(gbps["kv_dequant"], 1),
        "act_quant_GBps": round(gbps["act"], 1),
        "linear_TOPS": round(gemm_ops / ((ms["act"] + ms["gemm"]) * 1e-3) / 1e12, 2),
        "kernel_ms": {n: round(v, 5) for n, v in ms.items()},
        "kernel_us_stats": stats_us,
        "smi_clocks_during_timed_steps": clock_summary(clk),
        "int8_route": {"gemm_ms": round(int8_ms["gemm"], 5), "act_ms": round(int8_ms["act"], 5),
                       "gemm_TOPS": round(gemm_ops / (int8_ms["gemm"] * 1e-3) / 1e12, 2),
                       "pct_int8_peak": round(100.0 * gemm_ops / (int8_ms["gemm"] * 1e-3) / 1e12
                                              / INT8_PEAK_TOPS, 2)},
        "w4a8_route": {"gemm_ms": round(w4a8_ms["gemm"], 5), "act_ms": round(w4a8_ms["act"], 5),
                       "gemm_TOPS": round(gemm_ops / (w4a8_ms["gemm"] * 1e-3) / 1e12, 2),
                       "pct_int8_peak": round(100.0 * gemm_ops / (w4a8_ms["gemm"] * 1e-3) / 1e12
                                              / INT8_PEAK_TOPS, 2)},
        "lora_route": {"rank": RANK + LORA_RANK, "adapter_rank": LORA_RANK,
                       "gemm_ms": round(lora_ms["gemm"], 5), "act_ms": round(lora_ms["act"], 5),
                       "gemm_TOPS": round(gemm_ops / (lora_ms["gemm"] * 1e-3) / 1e12, 2),
                       "pct_int8_peak": round(100.0 * gemm_ops / (lora_ms["gemm"] * 1e-3) / 1e12
                                              / INT8_PEAK_TOPS, 2)},
        "kv_attention": {"ms": round(attn_ms, 5), "queries": 1,
                         "GBps": round(attn_bytes / (attn_ms * 1e-3) / 1e9, 1),
                         "pct_hbm_peak": round(100.0 * attn_bytes / (attn_ms * 1e-3) / 1e9
                                               / HBM_PEAK_GBPS, 2)},
        "setup_s": round(setup_s, 1),
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
