#!/usr/bin/env python3
"""Benchmark of the SVDQuant W4A4 + low-rank linear and the INT8 KV-cache quantizer on one GPU.

One step is one pass of the whole hot path over one batch of synthetic input:
  svdq_quantize_act_e3m2 + svdq_w4a4_gemm_e3m2
                                       on the FFN up-projection shape
                                       (X [4608, 3072] bf16, W [3072, 12288], r = 32, group 64;
                                       INT4 codes carried as BF6 on the FP6 matrix units)
  kv_int8_quant_pair                   K and V bf16 [10240 tokens, 32 heads, 128 dim] in one
                                       launch (per-channel range, scale, zero, codes)
  kv_int8_dequant (K, then V)          the inverse map of both caches
Weight preparation (smoothing, SVD, residual packing) is offline and untimed.

Timing: W warm-up steps, then K timed steps bracketed by torch.cuda.synchronize(); every call
is bracketed by a pair of HIP events (all created before the timed region) on the stream it is
launched on, so each kernel's duration is measured live.  Inputs rotate over 3 batches (about
590 MB, more than twice the 256 MB last-level cache) so the HBM-bound kernels read from HBM.

Before the step's warm-up, on the same process and device (outside the step), unless
--no-extras:
  * the INT8-unit route (svdq_quantize_act + svdq_w4a4_gemm, same codes and result), the W4A8
    variant, the LoRA-extended branch, the single-tensor kv_int8_quant, and decode attention
    over the INT8 cache;
  * the attention (3072 x 3072) and FFN down-projection (12288 -> 3072) shapes' activation pass
    and GEMM (random residual weights: the kernels' work does not depend on the values);
  * the step's GEMM alone, 100 launches back to back (last, just before the warm-up);
  * measured peaks of this device (FP6 / INT8 / bf16 MFMA issue loops and an HBM copy stream,
    libsvdq_peaks.so), against which each kernel's rate is also reported.
These seconds of load also let the device settle before the step is timed: from idle, the
GEMM's first ~80 launches run 10-25 % slower than its steady state.
After the timed region: the oracle's stages on the host cores (cpu_baseline), unless
--no-cpu-baseline.

Prints one JSON line.  `value` is the fused W4A4 + low-rank GEMM throughput in TOPS
(2 M N K integer ops per launch / mean launch time).
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "fused W4A4+low-rank GEMM TOPS and % of INT8 MFMA peak; KV-quant GB/s"
INT8_PEAK_TOPS = 5000.0      # MI355X dense INT8 MFMA, 5.0 POP/s
FP6_PEAK_TOPS = 10100.0      # MI355X dense FP6 MFMA, 10.1 PFLOP/s (the GEMM's matrix dtype)
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, 2.5 PFLOP/s
HBM_PEAK_GBPS = 8000.0       # MI355X HBM3E, 8 TB/s
M, K, N, RANK = 4608, 3072, 12288, 32
LORA_RANK = 16   # adapter rank of the LoRA line (reported beside the product path)
KV_T, KV_H, KV_D = 10240, 32, 128
ROTATE = 3
# the other two linear shapes of the workload: (config id, M, K, N)
OTHER_LINEARS = {"attn_proj": (2, 4608, 3072, 3072), "ffn_down": (4, 4608, 12288, 3072)}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    # 100 warm-up steps (≈ 37 ms of load): from idle the GEMM needs about 80 steps to reach its
    # steady rate (a warm-up transient of the device); the timed steps then measure that rate
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="time only the step (no routes, shapes, peaks after it)")
    ap.add_argument("--cpu-rows", type=int, default=M,
                    help="token rows of the oracle's CPU baseline sample")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MB",
                    help="first copy MB megabytes device to device once (a plain copy of known "
                         "size, the reference for the HBM byte counters of a profiler run)")
    return ap.parse_args()


# HBM traffic of the GEMM kernel per launch, measured with rocprofv3 counters (FETCH_SIZE and
# WRITE_SIZE, each scaled by what the same counter reads for a plain copy of known size).  The
# measurement is recorded with the SHA-256 of the kernel's sources (the kernel file, then the
# device header it includes) it was taken on; different sources report no traffic.
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "w4a4_gemm_e3m2_ffn_up_4608x3072x12288_traffic.md")
GEMM_SOURCES = [os.path.join(ROOT, "bit_post_quantized_amd", "csrc", f)
                for f in ("w4a4_gemm_e3m2.hip", "svdq_device.hpp")]


def gemm_source_sha256():
    import hashlib
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()


def recorded_traffic():
    try:
        rec = dict(line.split(":", 1) for line in open(TRAFFIC_RECORD).read().splitlines()
                   if line.startswith(("source_sha256:", "traffic_bytes_per_launch:")))
        src = gemm_source_sha256()
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256", "").strip() != src:
        return None
    return int(rec["traffic_bytes_per_launch"].strip())


def act_bytes(M_, K_, r):
    """Activation pass: read X, inv_lambda, L1; write the INT4 codes (0.5 B each), s_x, T."""
    return M_ * K_ * 2 + K_ * 4 + K_ * r * 2 + M_ * K_ // 2 + (K_ // 64) * M_ * 2 + M_ * r * 4


def gemm_bytes(M_, K_, N_, r, code_bytes=0.5):
    """GEMM: read both code matrices, both scale matrices, T and L2; write Y (bf16)."""
    G = K_ // 64
    return int((M_ * K_ + N_ * K_) * code_bytes) + G * M_ * 2 + G * N_ * 2 + M_ * r * 4 + \
        N_ * r * 2 + M_ * N_ * 2


def algorithmic_bytes():
    C = KV_H * KV_D
    kvq = KV_T * C * (2 + 1) + C * (4 + 1)        # per tensor: read x, write q, scale, zero
    kvd = KV_T * C * (1 + 2) + C * (4 + 1)        # per tensor: read q, scale, zero, write x'
    return dict(act=act_bytes(M, K, RANK), kv_pair=2 * kvq, kv_quant=kvq, kv_dequant=kvd,
                gemm=gemm_bytes(M, K, N, RANK), gemm_container=gemm_bytes(M, K, N, RANK, 0.75))


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


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or None


def blas_name():
    try:
        cfg = np.__config__.CONFIG["Build Dependencies"]["blas"]
        return f"{cfg.get('name')} {cfg.get('version')}"
    except Exception:
        return None


def cpu_baseline(rows: int):
    """The oracle (as it stands) on bounded samples of the same workload, stage by stage."""
    from oracle import kv_int8 as okv
    from oracle import svdquant as osq
    from synthetic import make_kv, make_linear

    d = make_linear(3, M=rows)
    stages = {}
    # weight preparation of the full FFN up-projection weight: smoothing, SVD, residual
    t0 = time.perf_counter()
    pw = osq.prepare_weights(d["X"], d["W"], 0.5, RANK)
    stages["prepare_weights_s"] = round(time.perf_counter() - t0, 3)
    t0 = time.perf_counter()
    packed = osq.pack_weights(pw["R32"])
    stages["pack_weights_s"] = round(time.perf_counter() - t0, 3)
    # activation pass + integer group GEMM + output, repeated until about 10 s were timed
    reps, dt_act, dt_gemm = 0, 0.0, 0.0
    while reps == 0 or (dt_act + dt_gemm < 10.0 and reps < 4):
        t0 = time.perf_counter()
        act = osq.quantize_act(d["X"], pw["inv_lambda"], pw["L1b"])
        t1 = time.perf_counter()
        osq.linear_output(act["codes"], act["s_x"], packed["codes"], packed["s_w"], act["T"],
                          pw["L2b"])
        dt_act += t1 - t0
        dt_gemm += time.perf_counter() - t1
        reps += 1
    stages["act_quant_lowrank_s_per_pass"] = round(dt_act / reps, 3)
    stages["group_gemm_output_s_per_pass"] = round(dt_gemm / reps, 3)
    # KV quantize and dequantize of K and V on a 2048-token sample of the cache shape
    kv_t = 2048
    kv = make_kv(tokens=kv_t)
    C = KV_H * KV_D
    t0 = time.perf_counter()
    refs = [okv.kv_int8_quant(kv[n].reshape(kv_t, -1)) for n in ("K", "V")]
    t1 = time.perf_counter()
    for r in refs:
        okv.dequantize(r["q"], r["scale"], r["zero"])
    t2 = time.perf_counter()
    kv_bytes = 2 * (kv_t * C * 3 + C * 5)
    stages["kv_quant_K_V_GBps"] = round(kv_bytes / (t1 - t0) / 1e9, 3)
    stages["kv_dequant_K_V_GBps"] = round(kv_bytes / (t2 - t1) / 1e9, 3)
    stages["kv_sample"] = f"K and V [{kv_t}, {KV_H}, {KV_D}]"
    cores = len(os.sched_getaffinity(0))
    dt = dt_act + dt_gemm
    return {"value": 2.0 * rows * N * K * reps / dt / 1e12, "unit": "TOPS", "cores": cores,
            "kind": "oracle",
            "sample": f"{rows} of {M} tokens of the {M}x{K}x{N} r={RANK} linear: activation "
                      f"quantization + low-rank down-projection + integer group GEMM + output "
                      f"(fp64 NumPy), {reps} pass(es) in {dt:.1f} s",
            "cpu_model": cpu_model(), "blas": blas_name(),
            "blas_threads": os.environ.get("OPENBLAS_NUM_THREADS") or os.environ.get(
                "OMP_NUM_THREADS") or f"default ({cores} cores)",
            "stages": stages}


class Peaks:
    """The device's measured peaks through libsvdq_peaks.so (MFMA issue loops, HBM copy)."""

    def __init__(self, torch, stream):
        from bit_post_quantized_amd import build
        path = build.PEAKS_LIB
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built (run python -m bit_post_quantized_amd.build)")
        lib = ctypes.CDLL(path)
        lib.peaks_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                   ctypes.c_void_p]
        lib.peaks_mfma_flops.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
        lib.peaks_mfma_flops.restype = ctypes.c_double
        lib.peaks_mfma_out_floats.argtypes = [ctypes.c_int]
        lib.peaks_mfma_out_floats.restype = ctypes.c_size_t
        lib.peaks_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                   ctypes.c_int, ctypes.c_void_p]
        self.lib, self.torch, self.stream = lib, torch, stream

    def _time(self, fn, reps=5):
        torch = self.torch
        fn()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(reps)]
        torch.cuda.synchronize()
        for e0, e1 in evs:
            e0.record(self.stream)
            fn()
            e1.record(self.stream)
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in evs]))  # ms

    def mfma(self, kind, blocks=4096, iters=256):
        torch = self.torch
        out = torch.empty(self.lib.peaks_mfma_out_floats(blocks), dtype=torch.float32,
                          device="cuda")
        s = ctypes.c_void_p(self.stream.cuda_stream)

        def run():
            if self.lib.peaks_mfma(kind, blocks, iters, ctypes.c_void_p(out.data_ptr()), s) != 0:
                raise RuntimeError("peaks_mfma failed")
        ms = self._time(run)
        return self.lib.peaks_mfma_flops(kind, blocks, iters) / (ms * 1e-3) / 1e12  # T/s

    def copy(self, mode, blocks=0, mb=1024):
        torch = self.torch
        n = mb * 1024 * 1024
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        s = ctypes.c_void_p(self.stream.cuda_stream)

        def run():
            if self.lib.peaks_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()),
                                   n, mode, blocks, s) != 0:
                raise RuntimeError("peaks_copy failed")
        ms = self._time(run)
        ok = bool(torch.equal(src[:: 1 << 16], dst[:: 1 << 16]))
        del src, dst
        return 2.0 * n / (ms * 1e-3) / 1e9, ok  # GB/s read + write


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
    if args.copy_probe > 0:
        n = args.copy_probe * 1024 * 1024 // 4   # fp32 elements: read MB, write MB (a negation)
        src_b = torch.ones(n, dtype=torch.float32, device=dev)
        dst_b = torch.empty(n, dtype=torch.float32, device=dev)
        torch.neg(src_b, out=dst_b)
        torch.cuda.synchronize()
        del src_b, dst_b

    def step_calls(i):
        b = i % ROTATE
        a = acts[b]
        return [
            ("act", lambda: B.svdq_quantize_act_e3m2(X[b], pw.inv_lambda, pw.L1p, RANK, a.xq,
                                                     a.x_scales, a.T, stream)),
            ("gemm", lambda: B.svdq_w4a4_gemm_e3m2(a.xq, a.x_scales, a.T, pw.wq, pw.w_scales,
                                                   pw.L2p, None, RANK, Y[b], stream)),
            ("kv_pair", lambda: B.kv_int8_quant_pair(kvs[b][0], kvs[b][1], q[b][0], sc[b][0],
                                                     zp[b][0], q[b][1], sc[b][1], zp[b][1], wsp,
                                                     stream)),
            ("kv_dequant", lambda: B.kv_int8_dequant(q[b][0], sc[b][0], zp[b][0], xo[b][0],
                                                     stream)),
            ("kv_dequant", lambda: B.kv_int8_dequant(q[b][1], sc[b][1], zp[b][1], xo[b][1],
                                                     stream)),
        ]

    ab = algorithmic_bytes()

    # The extra measurements run before the step is warmed up and timed: on a device fresh
    # from idle the GEMM's first ~80 launches (~30 ms of load) ran 216 -> 248 -> 194 us before
    # holding at 194 us (a transient whose shape is that of power management), and these
    # measurements are several seconds of load.  Their percentages of the measured peaks are
    # computed once the step is timed.
    def time10(fn, reps=10):
        fn()
        torch.cuda.synchronize()
        ev10 = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                for _ in range(reps)]
        for e0, e1 in ev10:
            e0.record(stream)
            fn()
            e1.record(stream)
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in ev10]))

    def tops(ms_, ops=2.0 * M * N * K):
        return ops / (ms_ * 1e-3) / 1e12

    def route(gemm_ms, act_ms, **extra):
        return {**extra, "gemm_ms": round(gemm_ms, 5), "act_ms": round(act_ms, 5),
                "gemm_TOPS": round(tops(gemm_ms), 2),
                "pct_int8_peak": round(100.0 * tops(gemm_ms) / INT8_PEAK_TOPS, 2)}

    extras = {}
    if not args.no_extras:
        # ---- this device's measured peaks (first: the issue loops run at full power, and the
        #      GEMM-like measurements after them let the power management settle again)
        pk = Peaks(torch, stream)
        fp6 = pk.mfma(0)
        int8 = pk.mfma(1)
        bf = pk.mfma(2)
        shapes = {"runs_16KiB": (1, 0), "runs_64KiB": (2, 0), "stride_8192": (0, 8192)}
        copies = {k: pk.copy(*v) for k, v in shapes.items()}
        copy_gbps = max(c[0] for c in copies.values())
        copy_ok = all(c[1] for c in copies.values())
        extras["measured_peaks"] = {
            "fp6_TFLOPs": round(fp6, 1), "int8_TOPS": round(int8, 1), "bf16_TFLOPs": round(bf, 1),
            "hbm_copy_GBps": round(copy_gbps, 1), "copy_verified": copy_ok,
            "hbm_copy_GBps_by_launch": {k: round(c[0], 1) for k, c in copies.items()},
            "note": "MFMA issue loops (8 independent 32x32 MFMAs per wave, 4096 workgroups of "
                    "256) and a 1 GiB device copy (best of three launch shapes); "
                    "libsvdq_peaks.so"}
        # ---- the INT8-unit route and the W4A8 variant on the same batch
        wq4 = torch.empty(N, K // 2, dtype=torch.uint8, device=dev)
        ws4 = torch.empty(K // 64, N, dtype=torch.float16, device=dev)
        B.svdq_pack_weights(pw.R32, wq4, ws4)
        xq4 = torch.empty(M, K // 2, dtype=torch.uint8, device=dev)
        xs4 = torch.empty(M, K // 64, dtype=torch.float16, device=dev)
        T4 = torch.empty(M, RANK, dtype=torch.float32, device=dev)
        xq8 = torch.empty(M, K, dtype=torch.int8, device=dev)
        extras["int8_route"] = route(
            time10(lambda: B.svdq_w4a4_gemm(xq4, xs4, T4, wq4, ws4, pw.L2p, None, RANK, Y[0], stream)),
            time10(lambda: B.svdq_quantize_act(X[0], pw.inv_lambda, pw.L1p, RANK, xq4, xs4, T4,
                                               stream)))
        extras["w4a8_route"] = route(
            time10(lambda: B.svdq_w4a8_gemm(xq8, xs4, T4, wq4, ws4, pw.L2p, None, RANK, Y[0], stream)),
            time10(lambda: B.svdq_quantize_act_a8(X[0], pw.inv_lambda, pw.L1p, RANK, xq8, xs4, T4,
                                                  stream)))
        del wq4, ws4, xq4, xs4, T4, xq8
        # LoRA: a seeded rank-16 adapter joined to the 16-bit branch (rank 32 + 16 = 48)
        gl = torch.Generator().manual_seed(7)
        pwl = layer.attach_lora(pw, torch.randn(K, LORA_RANK, generator=gl, dtype=torch.float64) * 0.02,
                                torch.randn(LORA_RANK, N, generator=gl, dtype=torch.float64) * 0.02)
        al = layer.alloc_act(M, K, pwl.rank, dev, e3m2=True)
        extras["lora_route"] = route(
            time10(lambda: B.svdq_w4a4_gemm_e3m2(al.xq, al.x_scales, al.T, pwl.wq, pwl.w_scales,
                                                 pwl.L2p, None, pwl.rank, Y[0], stream)),
            time10(lambda: B.svdq_quantize_act_e3m2(X[0], pwl.inv_lambda, pwl.L1p, pwl.rank,
                                                    al.xq, al.x_scales, al.T, stream)),
            rank=RANK + LORA_RANK, adapter_rank=LORA_RANK)
        del pwl, al
        # the single-tensor quantizer, K then V (two launches), on batches 0 and 1 in turn
        kv_single = [time10(lambda t=t, b=b: B.kv_int8_quant(kvs[b][t], q[b][t], sc[b][t],
                                                                zp[b][t], wsp, stream), reps=10)
                     for b in range(2) for t in range(2)]
        kv_single_ms = float(np.mean(kv_single))
        extras["kv_quant_single"] = {
            "ms_per_tensor": round(kv_single_ms, 5),
            "GBps": round(ab["kv_quant"] / (kv_single_ms * 1e-3) / 1e9, 1),
            "note": "kv_int8_quant on one tensor; K + V as two launches take twice this"}
        # decode attention over the INT8 cache of batch 0 (one query per head)
        q_att = torch.randn(1, KV_H, KV_D, device=dev).to(torch.bfloat16)
        o_att = torch.empty(1, KV_H, KV_D, dtype=torch.bfloat16, device=dev)
        ws_att = torch.empty(B.kv_int8_attention_workspace_bytes(1, KV_T, KV_H, KV_D),
                             dtype=torch.uint8, device=dev)
        attn_ms = time10(lambda: B.kv_int8_attention(q_att, q[0][0], sc[0][0], zp[0][0], q[0][1],
                                                     sc[0][1], zp[0][1], KV_D ** -0.5, o_att,
                                                     ws_att, stream))
        attn_bytes = 2 * KV_T * C + 2 * C * 5 + 2 * 1 * C * 2
        extras["kv_attention"] = {"ms": round(attn_ms, 5), "queries": 1,
                                  "GBps": round(attn_bytes / (attn_ms * 1e-3) / 1e9, 1),
                                  "pct_hbm_peak": round(100.0 * attn_bytes / (attn_ms * 1e-3) / 1e9
                                                        / HBM_PEAK_GBPS, 2)}
        del q_att, o_att, ws_att
        # ---- the attention and FFN down-projection shapes (FP6 route)
        shapes = {}
        for tag, (cid, M_, K_, N_) in OTHER_LINEARS.items():
            g = torch.Generator(device=dev).manual_seed(cid)
            # three input batches in rotation, as in the step: one 113 MB batch read over and
            # over stays partly in the 256 MB last-level cache and flatters the pass
            Xs = [bf16(make_linear(cid, seed=s_)["X"]) for s_ in range(ROTATE)]
            R = torch.randn(K_, N_, generator=g, device=dev) * K_ ** -0.5
            wq6 = torch.empty(B.svdq_e3m2_bytes(N_, K_), dtype=torch.uint8, device=dev)
            ws6 = torch.empty(K_ // 64, N_, dtype=torch.float16, device=dev)
            B.svdq_pack_weights_e3m2(R, wq6, ws6)
            del R
            L1p = (torch.randn(RANK, K_, generator=g, device=dev) * 0.05).to(torch.bfloat16)
            L2s = layer.pack_lowrank_up(
                (torch.randn(RANK, N_, generator=g, device=dev) * 0.05).to(torch.bfloat16))
            inv = torch.ones(K_, dtype=torch.float32, device=dev)
            a_s = layer.alloc_act(M_, K_, RANK, dev, e3m2=True)
            Ys = torch.empty(M_, N_, dtype=torch.bfloat16, device=dev)
            rot = iter(range(1 << 30))
            act_ms = time10(lambda: B.svdq_quantize_act_e3m2(Xs[next(rot) % ROTATE], inv, L1p, RANK,
                                                             a_s.xq, a_s.x_scales, a_s.T, stream))
            # 100 launches (≈ 30 ms at the FFN-down shape): the last load before the step's
            # warm-up, so the device enters it settled (see the note at the top of these
            # measurements)
            g_ms = time10(lambda: B.svdq_w4a4_gemm_e3m2(a_s.xq, a_s.x_scales, a_s.T, wq6, ws6,
                                                        L2s, None, RANK, Ys, stream), reps=100)
            ops = 2.0 * M_ * N_ * K_
            shapes[tag] = {"M": M_, "K": K_, "N": N_, "rank": RANK,
                           "gemm_ms": round(g_ms, 5), "gemm_TOPS": round(tops(g_ms, ops), 2),
                           "pct_int8_peak": round(100.0 * tops(g_ms, ops) / INT8_PEAK_TOPS, 2),
                           "act_ms": round(act_ms, 5),
                           "act_GBps": round(act_bytes(M_, K_, RANK) / (act_ms * 1e-3) / 1e9, 1),
                           "act_pct_hbm_peak": round(100.0 * act_bytes(M_, K_, RANK) /
                                                     (act_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2),
                           "weights": "random residual codes and factors (timing only)"}
            del Xs, wq6, ws6, L1p, L2s, inv, a_s, Ys
        extras["other_shapes"] = shapes
        # ---- the step's GEMM alone (100 launches on one batch's codes), against its time inside
        #      the step; measured last, so the device enters the step's warm-up settled on this
        #      very load
        a0 = acts[0]
        B.svdq_quantize_act_e3m2(X[0], pw.inv_lambda, pw.L1p, RANK, a0.xq, a0.x_scales, a0.T, stream)
        alone_ms = time10(lambda: B.svdq_w4a4_gemm_e3m2(a0.xq, a0.x_scales, a0.T, pw.wq, pw.w_scales,
                                                        pw.L2p, None, RANK, Y[0], stream), reps=100)
        extras["gemm_alone"] = {"ms": round(alone_ms, 5), "TOPS": round(tops(alone_ms), 2),
                                "note": "svdq_w4a4_gemm_e3m2 at the step's shape, 100 launches "
                                        "back to back on one batch (outside the step)"}

    names = ["act", "gemm", "kv_pair", "kv_dequant"]
    per_step = len(step_calls(0))
    read_clock = clock_reader()
    for i in range(args.warmup):
        for _, fn in step_calls(i):
            fn()
    # the clocks are sampled while the warm-up steps run (the device state the timed steps
    # start in), so no host work but the launches falls inside the timed region
    clk = []
    if read_clock is not None:
        done = torch.cuda.Event()
        done.record(stream)
        for _ in range(8):
            if done.query():
                break
            try:
                clk.append(read_clock())
            except Exception:
                break
            time.sleep(0.0005)
    torch.cuda.synchronize()

    # every event of the timed region exists before it starts
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps * per_step)]
    plan = [step_calls(args.warmup + i) for i in range(args.steps)]
    clk_before = read_clock() if read_clock else None
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    j = 0
    for calls in plan:
        for _, fn in calls:
            e0, e1 = evs[j]
            e0.record(stream)
            fn()
            e1.record(stream)
            j += 1
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    clk_after = read_clock() if read_clock else None

    samples = {n: [] for n in names}
    j = 0
    for calls in plan:
        for name, _ in calls:
            e0, e1 = evs[j]
            samples[name].append(e0.elapsed_time(e1) * 1e3)  # us
            j += 1
    samples = {n: np.array(v) for n, v in samples.items()}
    ms = {n: float(samples[n].mean()) * 1e-3 for n in names}
    stats_us = {n: {"median": round(float(np.median(v)), 2), "p10": round(float(np.percentile(v, 10)), 2),
                    "p90": round(float(np.percentile(v, 90)), 2), "calls": int(v.size)}
                for n, v in samples.items()}

    gemm_ops = 2.0 * M * N * K
    gemm_tops = gemm_ops / (ms["gemm"] * 1e-3) / 1e12
    gbps = {n: ab[n] / (ms[n] * 1e-3) / 1e9 for n in ("act", "kv_pair", "kv_dequant")}

    if "measured_peaks" in extras:  # fp6, int8, copy_gbps: the peaks measured above
        extras["pct_measured_peak"] = {
            "gemm_vs_fp6_loop": round(100.0 * gemm_tops / fp6, 2),
            "gemm_vs_int8_loop": round(100.0 * gemm_tops / int8, 2),
            "act_vs_copy": round(100.0 * gbps["act"] / copy_gbps, 2),
            "kv_pair_vs_copy": round(100.0 * gbps["kv_pair"] / copy_gbps, 2),
            "kv_dequant_vs_copy": round(100.0 * gbps["kv_dequant"] / copy_gbps, 2)}

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
                     "algorithmic_bytes": ab["gemm"], "container_bytes": ab["gemm_container"]},
        "cpu_baseline": cpu,
        "pct_int8_peak": round(100.0 * gemm_tops / INT8_PEAK_TOPS, 2),
        "kv_quant_K_V_us": round(ms["kv_pair"] * 1e3, 2),
        "kv_quant_GBps": round(gbps["kv_pair"], 1),
        "kv_quant_pct_hbm_peak": round(100.0 * gbps["kv_pair"] / HBM_PEAK_GBPS, 2),
        "kv_dequant_GBps": round(gbps["kv_dequant"], 1),
        "kv_dequant_pct_hbm_peak": round(100.0 * gbps["kv_dequant"] / HBM_PEAK_GBPS, 2),
        "act_quant_GBps": round(gbps["act"], 1),
        "act_quant_pct_hbm_peak": round(100.0 * gbps["act"] / HBM_PEAK_GBPS, 2),
        "linear_TOPS": round(gemm_ops / ((ms["act"] + ms["gemm"]) * 1e-3) / 1e12, 2),
        "kernel_ms": {n: round(v, 5) for n, v in ms.items()},
        "kernel_us_stats": stats_us,
        "sum_of_kernel_means_ms": round(ms["act"] + ms["gemm"] + ms["kv_pair"] +
                                        2 * ms["kv_dequant"], 4),
        "smi_clocks": {"during_warmup": clock_summary(clk), "before_timed": clk_before,
                       "after_timed": clk_after},
        **extras,
        "setup_s": round(setup_s, 1),
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
