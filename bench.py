#!/usr/bin/env python3
"""Benchmark of the SVDQuant W4A4 + low-rank linear and the INT8 KV-cache quantizer on one GPU.

One step is one pass of the whole hot path over one batch of synthetic input:
  svdq_quantize_act + svdq_w4a4_gemm   on the FFN up-projection shape
                                       (X [4608, 3072] bf16, W [3072, 12288], r = 32, group 64)
  kv_int8_quant + kv_int8_dequant      on K and V bf16 [10240 tokens, 32 heads, 128 dim]
Weight preparation (smoothing, SVD, residual packing) is offline and untimed.

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
HBM_PEAK_GBPS = 8000.0       # MI355X HBM3E, 8 TB/s
M, K, N, RANK = 4608, 3072, 12288, 32
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
    return ap.parse_args()


def algorithmic_bytes():
    G = K // 64
    act = M * K * 2 + K * 4 + K * RANK * 2 + M * K // 2 + G * M * 2 + M * RANK * 4
    C = KV_H * KV_D
    kvq = KV_T * C * (2 + 1) + C * (4 + 1)        # per tensor: read x, write q, scale, zero
    kvd = KV_T * C * (1 + 2) + C * (4 + 1)        # per tensor: read q, scale, zero, write x'
    gemm = M * K // 2 + N * K // 2 + G * M * 2 + G * N * 2 + M * RANK * 4 + N * RANK * 2 + M * N * 2
    return dict(act=act, kv_quant=kvq, kv_dequant=kvd, gemm=gemm)


def cpu_baseline(rows: int):
    """The oracle (as it stands) on a bounded sample: `rows` tokens of the same workload."""
    from oracle import svdquant as osq
    from synthetic import make_linear

    d = make_linear(3, M=rows)
    cfg_rank = RANK
    # weights: the oracle's own preparation of the same W (untimed offline step, as on the GPU)
    pw = osq.prepare_weights(d["X"], d["W"], 0.5, cfg_rank)
    packed = osq.pack_weights(pw["R32"])
    t0 = time.perf_counter()
    act = osq.quantize_act(d["X"], pw["inv_lambda"], pw["L1b"])
    osq.linear_output(act["codes"], act["s_x"], packed["codes"], packed["s_w"], act["T"],
                      pw["L2b"])
    dt = time.perf_counter() - t0
    cores = len(os.sched_getaffinity(0))
    return {"value": 2.0 * rows * N * K / dt / 1e12, "unit": "TOPS", "cores": cores,
            "kind": "oracle",
            "sample": f"{rows} of {M} tokens of the {M}x{K}x{N} r={RANK} linear: activation "
                      f"quantization + low-rank down-projection + integer group GEMM + output "
                      f"(fp64 NumPy/OpenBLAS), {dt:.1f} s"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the path is not "
              "sharded across GPUs in this build.", file=sys.stderr)
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
    pw = layer.convert_weights(bf16(d["W"]).cpu(), bf16(d["X"]).cpu(), 0.5, RANK, device=dev)
    X = [bf16(d["X"])] + [bf16(make_linear(3, seed=s)["X"]) for s in range(1, ROTATE)]
    kvs = []
    for s in range(ROTATE):
        kv = make_kv(seed=s)
        kvs.append((bf16(kv["K"]).view(KV_T, -1), bf16(kv["V"]).view(KV_T, -1)))
    C = KV_H * KV_D
    acts = [layer.alloc_act(M, K, RANK, dev) for _ in range(ROTATE)]
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

    def step(i, ev=None):
        b = i % ROTATE
        a = acts[b]
        calls = [
            ("act", lambda: B.svdq_quantize_act(X[b], pw.inv_lambda, pw.L1t, RANK, a.xq,
                                                a.x_scales, a.T, stream)),
            ("gemm", lambda: B.svdq_w4a4_gemm(a.xq, a.x_scales, a.T, pw.wq, pw.w_scales, pw.L2t,
                                              None, RANK, Y[b], stream)),
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

    ev = {n: [] for n in names}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, ev)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    ms = {n: float(np.mean([a.elapsed_time(b) for a, b in ev[n]])) for n in names}
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
        "dtype": "i8",
        "data": "synthetic",
        "config": {"workload": f"svdquant_linear M{M} K{K} N{N} r{RANK} g64 bf16-out + "
                               f"kv_int8 K,V [{KV_T},{KV_H},{KV_D}] bf16",
                   "M": M, "K": K, "N": N, "rank": RANK, "group": 64,
                   "kv_tokens": KV_T, "kv_heads": KV_H, "kv_dim": KV_D},
        "roofline": {"bound": "mfma", "kernel": "w4a4_gemm", "achieved": round(gemm_tops, 2),
                     "peak": INT8_PEAK_TOPS, "unit": "TOP/s",
                     "frac": round(gemm_tops / INT8_PEAK_TOPS, 4), "traffic": None},
        "cpu_baseline": cpu,
        "pct_int8_peak": round(100.0 * gemm_tops / INT8_PEAK_TOPS, 2),
        "kv_quant_GBps": round(gbps["kv_quant"], 1),
        "kv_quant_pct_hbm_peak": round(100.0 * gbps["kv_quant"] / HBM_PEAK_GBPS, 2),
        "kv_dequant_GBps": round(gbps["kv_dequant"], 1),
        "act_quant_GBps": round(gbps["act"], 1),
        "linear_TOPS": round(gemm_ops / ((ms["act"] + ms["gemm"]) * 1e-3) / 1e12, 2),
        "kernel_ms": {n: round(v, 5) for n, v in ms.items()},
        "setup_s": round(setup_s, 1),
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
