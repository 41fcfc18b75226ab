#!/usr/bin/env python3
"""Benchmark of the fused SVDQuant W4A4 + rank-r linear on one MI355X.

A step is one pass of the forward hot path over one batch: kernel 1 (smooth +
INT4 activation quantizer + down projection) then kernel 2 (W4A4 GEMM +
dequant + up projection + bias), on the FLUX MLP up-projection layer
(M = 4096 tokens, K = 3072, N = 12288, rank 32, group 64) unless --workload
says otherwise.  Weight preparation (smoothing, SVD, 4-bit residual) is a
one-time offline transform and runs before the timed region.

The INT4 layer runs on one of two engines: "fp6" (default; the INT4 codes in
E3M2 containers on the 6-bit float MFMA) or "int8" (nibble codes on the int8
MFMA); both compute the same layer.  Prints one JSON line.  value = effective
TOPS = 2*M*N*K / (time per step); the low-rank flops are not credited.  The
line also carries, each timed here: the int8 engine on the same layer, the
tiny layer (µs), the attention-output projection, the MLP down projection
with tanh-GELU fused into kernel 1, the batched rank sweep (ranks 0..128:
overhead per rank and error against fp64 X W), the MXFP4 variant, the fused
QKV epilogue, the AWQ modulation GEMV, the measured peaks and the CPU oracle
baseline (skip groups with the --no-* flags).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "effective TOPS of fused W4A4+rank-32 linear (FLUX shapes); % INT8 MFMA peak"
INT8_PEAK_TOPS = 5000.0      # MI355X dense INT8 MFMA, published
FP4_PEAK_TFLOPS = 10100.0    # MI355X dense FP4 / FP6 MFMA, published
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
COLD_EVICT_BYTES = 1 << 30     # written before each cold step (Infinity Cache is 256 MB)
COLD_ITERS = 20
# Untimed continuous load before the warmup steps of every measurement: on
# MI355X the step time falls from ~305 to ~260 us over the first ~30 ms of
# sustained work (and rises again after about a second idle), so a fixed
# number of warmup steps alone can leave the timed steps in that ramp.
SETTLE_S = 0.1


def settle(step, seconds=SETTLE_S):
    """Run `step` back to back for at least `seconds` of wall time."""
    import torch
    t0 = time.perf_counter()
    while True:
        for _ in range(8):
            step()
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            return

def graph_time(fn, n: int) -> float:
    """Average GPU time in ms of one fn() over n back-to-back calls: the n
    calls are captured once into a HIP graph (the library launches on the
    current stream, which is the capture stream there) and the graph is
    replayed between two HIP events.  For kernels shorter than the host's
    time to enqueue one (the AWQ GEMV, ~11 µs): events around each eager
    launch would time the GPU waiting for the host."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(n):
            fn()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    del g
    return e0.elapsed_time(e1) / n


# name -> (generator workload, layer index, act, description)
BENCH_WORKLOADS = {
    "mlp_up": ("mlp_pair", 0, "none", "FLUX MLP up-projection 4096x3072x12288"),
    "mlp_down": ("mlp_pair", 1, "gelu_tanh", "FLUX MLP down-projection 4096x12288x3072 (tanh-GELU in kernel 1)"),
    "attn_out": ("attn_out", 0, "none", "FLUX attention-output projection 4096x3072x3072"),
    "joint_qkv": ("joint_qkv", 0, "none", "FLUX joint-stream fused QKV 4608x3072x9216 (+bias)"),
    "rank_sweep": ("rank_sweep", 0, "none", "4 images x 4096 tokens, 16384x3072x12288"),
    "tiny": ("tiny", 0, "none", "single linear 256x512x512"),
}

# kernel-2 sources per engine: the stored traffic figures of an engine stay
# valid while these are unchanged
ENGINE_SOURCES = {
    "fp6": ("svdq_fp6_kernels.hip", "svdq_device.h"),
    "int8": ("svdq_kernels.hip", "svdq_device.h"),
    "mxfp4": ("svdq_mx_kernels.hip", "svdq_device.h"),
}
K2_KERNEL = {"fp6": "k_gemm_w4a4_fp6", "int8": "k_gemm_w4a4_lora_up", "mxfp4": "k_gemm_mxfp4_lora_up"}


def code_tokens(src: str) -> str:
    """C/C++ source with comments removed and whitespace runs collapsed."""
    import re
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return " ".join(src.split())


def kernel_source_hash(engine: str = "fp6") -> str:
    """Hash of an engine's kernel-2 sources with comments and whitespace
    removed, so that the stored counter figures stay valid across
    comment-only edits."""
    h = hashlib.sha256()
    for f in ENGINE_SOURCES[engine]:
        src = open(os.path.join(ROOT, "w4a4_rank_corrected_svdq_amd", "csrc", f)).read()
        h.update(code_tokens(src).encode())
    return h.hexdigest()[:16]


def scale_bytes(K, precision):
    """Scale bytes per row: fp16 per 64 (INT4) or one E8M0 byte per 32 (MXFP4)."""
    return 2 * (K // 64) if precision == "int4" else K // 32


def k1_bytes(M, K, r, precision="int4"):
    """Compulsory HBM bytes of kernel 1: read X (bf16), smooth_inv, L1; write
    codes (4 bits each), scales and lora_act."""
    return 2 * M * K + 4 * K + 2 * r * K + M * K // 2 + scale_bytes(K, precision) * M + 4 * M * r


def k2_bytes(M, N, K, r, bias, precision="int4"):
    """Compulsory HBM bytes of kernel 2: codes (4 bits), scales, lora_act,
    lora_up, bias; write Y (bf16)."""
    sb = scale_bytes(K, precision)
    return (M * K // 2 + sb * M + N * K // 2 + sb * N + 4 * M * r
            + 2 * N * r + (2 * N if bias else 0) + 2 * M * N)


def fp6_container_bytes(M, N, K):
    """Bytes of the 6-bit route's code containers (6 bits per code, rows
    padded to 32 activations / 128 weights) and padded activation scales."""
    G = K // 64
    RBa, RBb = (M + 31) // 32, 4 * ((N + 127) // 128)
    return {"x_codes": G * RBa * 1536, "x_scales": G * 32 * RBa * 2, "w_codes": G * RBb * 1536}


def load_traffic(workload: str, rank: int, engine: str = "fp6"):
    """HBM traffic of kernel 2 measured by rocprofv3 PMC counters (committed
    under profiles/), used only while the engine's kernel source is
    unchanged."""
    p = os.path.join(ROOT, "profiles", f"traffic_{workload}_r{rank}_{engine}.json")
    if not os.path.exists(p):
        return None
    d = json.load(open(p))
    if d.get("kernel_source_sha") != kernel_source_hash(engine):
        return None
    return d.get("k2_hbm_bytes")


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def blas_info():
    try:
        from threadpoolctl import threadpool_info
        return [{k: d.get(k) for k in ("internal_api", "version", "num_threads", "threading_layer")}
                | {"library": os.path.basename(d.get("filepath", ""))}
                for d in threadpool_info() if d.get("user_api") == "blas"]
    except Exception:  # pragma: no cover
        return []


def cpu_baseline(wl, layer, rank, target_s, precision="int4"):
    """The oracle (as it stands) on a bounded sample of rows of the same
    workload, timed on this host's cores: once with the BLAS thread pool as
    configured, once limited to one thread."""
    import oracle as O
    from threadpoolctl import threadpool_limits
    blas = blas_info()
    threads = max([b.get("num_threads") or 1 for b in blas] + [1])
    Lr = wl.layers[layer]
    K, N = Lr.K, Lr.N
    a = wl.act_absmax()
    t0 = time.perf_counter()
    po = O.prepare(Lr.weight, a, rank=rank) if precision == "int4" else O.mx.prepare_mx(Lr.weight, a, rank=rank)
    fwd = O.forward if precision == "int4" else O.mx.forward_mx
    t_prep = time.perf_counter() - t0

    def timed_rows(budget_s, max_passes):
        # chunks of 128 rows, in order, wrapping round the workload's rows
        rows_per_chunk, done, t_fwd = 128, 0, 0.0
        while t_fwd < budget_s and done < max_passes * wl.M:
            start = done % wl.M
            xr = wl.x[start:start + rows_per_chunk]
            t1 = time.perf_counter()
            fwd(xr, po, bias=Lr.bias)
            t_fwd += time.perf_counter() - t1
            done += xr.shape[0]
        return done, t_fwd

    rows, t_fwd = timed_rows(target_s, 4)
    with threadpool_limits(limits=1, user_api="blas"):
        rows1, t_fwd1 = timed_rows(target_s / 3, 1)
    tops = 2.0 * rows * N * K / t_fwd / 1e12
    return {"value": tops, "unit": "TOPS", "cores": int(threads), "kind": "oracle",
            "sample": f"oracle forward ({precision}, fp64 numpy emulation) on {rows} rows (128-row chunks "
                      f"taken in order from the workload's {wl.M}, wrapping round), {t_fwd:.1f} s",
            "single_thread": {"value": 2.0 * rows1 * N * K / t_fwd1 / 1e12, "unit": "TOPS",
                              "rows": rows1, "seconds": round(t_fwd1, 2)},
            "prepare_s": round(t_prep, 2),
            "prepare": "oracle prepare of the layer (LAPACK SVD), not counted in value",
            "cpu_model": cpu_model(), "blas": blas, "host_cpu_count": os.cpu_count()}


def bench_qkv(S, L, workloads, r, steps, warmup):
    """The joint-stream QKV projection (4608 x 3072 -> 9216, bias) with the
    fused per-head Q/K RMSNorm + rotary epilogue, against the same step with
    the plain epilogue, on both INT4 engines (the 6-bit one first)."""
    import torch
    wl = workloads.make_workload("joint_qkv")
    Lr = wl.layers[0]
    M, K, N = wl.M, Lr.K, Lr.N
    G, RBa = K // 64, (M + 31) // 32
    prep = S.prepare_weights(Lr.weight_bits, wl.act_absmax(), rank=r)
    bias = torch.from_numpy(Lr.bias_bits.view(np.int16).copy()).view(torch.bfloat16)
    (qb, _), (kb, _) = workloads.norm_weights()
    cos, sin = workloads.rope_tables(512, 64)
    gq = torch.from_numpy(qb.view(np.int16).copy()).view(torch.bfloat16).cuda()
    gk = torch.from_numpy(kb.view(np.int16).copy()).view(torch.bfloat16).cuda()
    cos_d, sin_d = torch.from_numpy(cos).cuda(), torch.from_numpy(sin).cuda()
    x = torch.from_numpy(wl.x_bits.view(np.int16).copy()).view(torch.bfloat16).cuda()
    la = torch.empty((M, r), dtype=torch.float32, device="cuda") if r else None
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    res = {"workload": "FLUX joint-stream QKV 4608x3072x9216 (+bias), rank 32, 24 heads of 128"}
    ops = 2.0 * M * N * K

    for engine in ("fp6", "int8"):
        lin = S.SVDQW4A4Linear(prep, bias, "cuda", engine=engine)
        if engine == "fp6":
            xc = torch.empty((G, RBa, 1536), dtype=torch.uint8, device="cuda")
            xs = torch.empty((G, 32 * RBa), dtype=torch.float16, device="cuda")
        else:
            xc = torch.empty((M, K // 2), dtype=torch.uint8, device="cuda")
            xs = torch.empty((G, M), dtype=torch.float16, device="cuda")

        def step_of(fused, lin=lin, engine=engine, xc=xc, xs=xs):
            if engine == "fp6":
                def step():
                    S.quant_act_lora_down_fp6(x, lin.smooth_inv, lin.lora_down, r, out=(xc, xs, la))
                    if fused:
                        S.gemm_w4a4_fp6_lora_up_qkv(xc, xs, lin.w_fp6, lin.w_scales, la, lin.lora_up, lin.bias,
                                                    gq, gk, cos_d, sin_d, M, N, K, r, out=y)
                    else:
                        S.gemm_w4a4_fp6_lora_up(xc, xs, lin.w_fp6, lin.w_scales, la, lin.lora_up, lin.bias,
                                                M, N, K, r, out=y)
            else:
                def step():
                    S.quant_act_lora_down(x, lin.smooth_inv, lin.lora_down, r, out=(xc, xs, la))
                    if fused:
                        S.gemm_w4a4_lora_up_qkv(xc, xs, lin.w_codes, lin.w_scales, la, lin.lora_up, lin.bias,
                                                gq, gk, cos_d, sin_d, M, N, K, r, out=y)
                    else:
                        S.gemm_w4a4_lora_up(xc, xs, lin.w_codes, lin.w_scales, la, lin.lora_up, lin.bias,
                                            M, N, K, r, out=y)
            return step

        def timed(step):
            settle(step)
            for _ in range(warmup):
                step()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(steps):
                step()
            torch.cuda.synchronize()
            return (time.perf_counter() - t0) * 1e3 / steps

        plain_ms, fused_ms = timed(step_of(False)), timed(step_of(True))
        pre = "" if engine == "fp6" else "int8_"
        res.update({pre + "plain_ms_per_step": round(plain_ms, 5), pre + "fused_ms_per_step": round(fused_ms, 5),
                    pre + "fused_effective_tops": round(ops / (fused_ms * 1e-3) / 1e12, 2),
                    pre + "epilogue_overhead_frac": round(fused_ms / plain_ms - 1.0, 4)})
        del lin, xc, xs
    res["engine"] = "fp6 (int8_* keys: the int8 engine)"
    return res


def bench_awq(S, workloads, steps, warmup, M=1):
    """AWQ W4A16 on the FLUX double-block modulation projection (3072 ->
    18432, bias), M conditioning rows: HBM-bound on the weight read.  One
    row runs the single-launch form (svdq_awq_linear_row: activation scaling
    fused into the GEMV); the two-launch path (svdq_awq_quant_act +
    svdq_awq_gemv) is timed beside it."""
    import torch
    wl = workloads.awq_workload(M, K=3072, N=18432, Mc=16, seed=7)
    K, N = wl["K"], wl["N"]
    G = K // 64
    prep = S.awq_prepare(wl["weight_bits"], wl["x_cal_bits"])
    lin = S.AWQW4A16Linear(prep, torch.from_numpy(wl["bias_bits"].view(np.int16).copy()).view(torch.bfloat16), "cuda")
    x = torch.from_numpy(wl["x_bits"].view(np.int16).copy()).view(torch.bfloat16).cuda()
    xh = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    xs = torch.empty((G, 16), dtype=torch.float32, device="cuda")
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

    def gemv():
        S.awq_gemv(xh, xs, lin.w_codes, lin.w_scales, lin.w_zeros, lin.bias, M, N, K, out=y)

    def two_launch():
        S.awq_quant_act(x, lin.inv_scale, out=(xh, xs))
        gemv()

    def one_launch():
        S.awq_linear_row(x, lin.inv_scale, lin.w_codes, lin.w_scales, lin.w_zeros, lin.bias, N, K, out=y)

    def timed(step, kernel):
        settle(step)
        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            step()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / steps
        # the kernel's average launch time: `steps` back-to-back launches
        # from a HIP graph between two events on its stream
        return ms, graph_time(kernel, steps)

    weights = N * K // 2 + 2 * N * G + N * G + 2 * N
    fused = M == 1
    ms2, gemv_ms = timed(two_launch, gemv)
    if fused:
        ms, k_ms = timed(one_launch, one_launch)
        nbytes = weights + 2 * K + 4 * K + 2 * N            # x and inv_scale in, y out
        kernel = "k_awq_gemv_row1 (activation scaling fused)"
    else:
        ms, k_ms = ms2, gemv_ms
        nbytes = weights + 2 * M * K + 4 * G * 16 + 2 * M * N
        kernel = "k_awq_gemv_stream"
    gbs = nbytes / (k_ms * 1e-3) / 1e9
    out = {"workload": f"FLUX modulation projection 3072 -> 18432 (+bias), M = {M}, AWQ INT4 group 64",
           "alpha": prep["alpha"], "ms_per_step": round(ms, 5),
           "roofline": {"bound": "hbm", "kernel": kernel, "achieved": round(gbs, 1),
                        "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                        "avg_launch_us": round(k_ms * 1e3, 2), "algorithmic_bytes_per_launch": nbytes}}
    if fused:
        out["two_launch_ms_per_step"] = round(ms2, 5)
        out["two_launch_gemv_us"] = round(gemv_ms * 1e3, 2)
    return out


def measure_peaks():
    """Dense int8 and FP4 MFMA rates (the library's register-only probe
    kernels, include/svdq_probe.h) and the device-to-device copy rate of
    1 GiB (read + write bytes), each after the same settle phase, averaged
    over 10 launches between HIP events."""
    import torch
    from w4a4_rank_corrected_svdq_amd import _lib as L
    st = torch.cuda.current_stream()
    res = {}

    def timed(fn, n=10):
        settle(fn)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    blocks, iters = 2048, 4096
    sink = torch.empty(blocks * 256 * 64, dtype=torch.uint8, device="cuda")
    for kind, key in ((L.SVDQ_PROBE_MFMA_I8, "int8_mfma_tops"), (L.SVDQ_PROBE_MFMA_FP4, "fp4_mfma_tflops")):
        def probe(kind=kind):
            L.check(L.lib().svdq_probe_mfma(kind, blocks, iters, sink.data_ptr(), st.cuda_stream), "peak probe")
        ms = timed(probe)
        res[key] = round(L.lib().svdq_probe_mfma_ops(kind, blocks, iters) / (ms * 1e-3) / 1e12, 1)
    del sink
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    ms = timed(lambda: dst.copy_(src))
    res["hbm_copy_gbs"] = round(2.0 * n / (ms * 1e-3) / 1e9, 1)
    del src, dst
    res["how"] = ("register-only MFMA loops (v_mfma_i32_32x32x32_i8, one chain per wave; FP4 "
                  "v_mfma_scale_f32_32x32x64_f8f6f4, four chains) over 2048 blocks of 4 waves, and a 1 GiB "
                  "device copy counted as read + write, after the settle phase")
    return res


def mix_probe(iters=2000):
    """The 6-bit route's inner loop on registers (include/svdq_probe.h kinds
    2-4): FP6 MFMAs only, the fp32 dequantization only, and both interleaved
    as kernel 2 issues them, at one and two waves per SIMD (1 x and 2 x CUs
    blocks of four waves).  Per kind: time per 32 x 32 tile on one SIMD."""
    import torch
    from w4a4_rank_corrected_svdq_amd import _lib as L
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    st = torch.cuda.current_stream()
    out = {"iters": iters, "tiles_per_wave_iteration": 8, "cus": cus, "runs": []}
    names = {L.SVDQ_PROBE_MFMA_FP6: "fp6_mfma_only", L.SVDQ_PROBE_DEQUANT: "dequant_valu_only",
             L.SVDQ_PROBE_FP6_DEQUANT: "fp6_mfma_plus_dequant"}
    for wps in (1, 2):
        blocks = cus * wps
        sink = torch.empty(blocks * 256 * 64, dtype=torch.uint8, device="cuda")
        for kind, name in names.items():
            def launch(kind=kind):
                L.check(L.lib().svdq_probe_mfma(kind, blocks, iters, sink.data_ptr(), st.cuda_stream), "mix probe")
            settle(launch)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(5):
                launch()
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / 5
            ns_tile = ms * 1e6 / (wps * iters * 8)
            run = {"kind": name, "waves_per_simd": wps, "ms": round(ms, 4),
                   "ns_per_tile_per_simd": round(ns_tile, 3), "cycles_per_tile_at_2.4GHz": round(ns_tile * 2.4, 1)}
            if kind != L.SVDQ_PROBE_DEQUANT:
                run["fp6_mfma_tflops"] = round(L.lib().svdq_probe_mfma_ops(kind, blocks, iters) / (ms * 1e-3) / 1e12, 1)
            else:
                run["valu_fp32_instr_per_simd_cycle_at_2.4GHz"] = round(32.0 / (ns_tile * 2.4), 3)
            out["runs"].append(run)
        del sink
    return out


SWEEP_RANKS = (0, 16, 32, 64, 128)
SWEEP_ROWS = 64


class Runner:
    """One layer's forward step on one engine with preallocated buffers:
    "fp6", "int8" and "mxfp4" run kernel 1 then kernel 2; "unfused" runs
    the int8 engine at rank 0, then the separate down projection (re-reads x)
    and up projection (reads and rewrites y)."""

    def __init__(self, S, lin, x, act_id, engine):
        import torch
        self.S, self.lin, self.x, self.act = S, lin, x, act_id
        M, K = x.shape
        # a 6-bit layer's step runs the kernels its forward() would (the
        # int8 engine's for few rows: SVDQW4A4Linear.route)
        self.engine = engine = lin.route(M) if engine == "fp6" else engine
        N, r = lin.N, lin.rank
        self.M, self.N, self.K = M, N, K
        dev = "cuda"
        self.la = torch.empty((M, r), dtype=torch.float32, device=dev) if r else None
        self.y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        if engine == "fp6":
            G, RB = K // 64, (M + 31) // 32
            self.xc = torch.empty((G, RB, 1536), dtype=torch.uint8, device=dev)
            self.xs = torch.empty((G, 32 * RB), dtype=torch.float16, device=dev)
            if lin.w_fp6 is None:
                raise ValueError("the layer holds no 6-bit weight container")
        elif engine == "mxfp4":
            self.xc = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
            self.xs = torch.empty((M, K // 32), dtype=torch.uint8, device=dev)
        else:
            self.xc = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
            self.xs = torch.empty((K // 64, M), dtype=torch.float16, device=dev)

    def k1(self):
        S, lin, x, r = self.S, self.lin, self.x, self.lin.rank
        if self.engine == "fp6":
            S.quant_act_lora_down_fp6(x, lin.smooth_inv, lin.lora_down, r, act=self.act, out=(self.xc, self.xs, self.la))
        elif self.engine == "mxfp4":
            S.quant_act_lora_down_mxfp4(x, lin.smooth_inv, lin.lora_down, r, act=self.act, out=(self.xc, self.xs, self.la))
        else:
            S.quant_act_lora_down(x, lin.smooth_inv, lin.lora_down, r, act=self.act, out=(self.xc, self.xs, self.la))

    def k2(self):
        S, lin, M, N, K, r = self.S, self.lin, self.M, self.N, self.K, self.lin.rank
        if self.engine == "fp6":
            lin.kernel2_fp6(self.xc, self.xs, self.la, M, out=self.y)
        elif self.engine == "mxfp4":
            S.gemm_mxfp4_lora_up(self.xc, self.xs, lin.w_codes, lin.w_scales, self.la, lin.lora_up, lin.bias,
                                 M, N, K, r, out=self.y)
        else:
            S.gemm_w4a4_lora_up(self.xc, self.xs, lin.w_codes, lin.w_scales, self.la, lin.lora_up, lin.bias,
                                M, N, K, r, out=self.y)

    def step(self, mid=None):
        S, lin, x, M, N, K, r = self.S, self.lin, self.x, self.M, self.N, self.K, self.lin.rank
        if self.engine == "unfused":
            S.quant_act_lora_down(x, lin.smooth_inv, None, 0, act=self.act, out=(self.xc, self.xs, None))
            S.gemm_w4a4_lora_up(self.xc, self.xs, lin.w_codes, lin.w_scales, None, None, lin.bias, M, N, K, 0,
                                out=self.y)
            S.lora_down(x, lin.smooth_inv, lin.lora_down, r, act=self.act, out=self.la)
            S.lora_up_add(self.la, lin.lora_up, self.y)
            return
        self.k1()
        if mid is not None:
            mid.record()
        self.k2()

    def time(self, steps, warmup, events=True, cold_iters=0):
        """Wall time of `steps` back-to-back steps after the settle phase and
        `warmup` steps; then (events) a second pass of the same length with
        HIP events before kernel 1, between the kernels and after kernel 2 of
        every step, for the kernels' average launch times (the GPU runs about
        a step behind the host there, so no host gap enters them; each event
        keeps the kernel after it from overlapping the one before, as a
        profiler's kernel trace does); then (cold_iters) single steps each
        after evicting the Infinity Cache."""
        import torch
        settle(self.step)
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            self.step()
        torch.cuda.synchronize()
        res = {"wall_s": time.perf_counter() - t0, "ms": (time.perf_counter() - t0) * 1e3 / steps}
        if events and self.engine != "unfused":
            ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
            for i in range(steps):
                ev[i][0].record()
                self.step(ev[i][1])
                ev[i][2].record()
            torch.cuda.synchronize()
            res["k1_ms"] = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
            res["k2_ms"] = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
            # kernel 1 (~13 us) is short enough that the events around it add
            # their own time: its launches back to back from a HIP graph
            res["k1_graph_ms"] = graph_time(self.k1, max(steps, 20))
        if cold_iters:
            # writing 1 GiB first evicts the 256 MB Infinity Cache, so codes,
            # scales and X come from HBM; the write is outside each step's
            # events
            scratch = torch.empty(COLD_EVICT_BYTES, dtype=torch.uint8, device="cuda")
            cev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(cold_iters)]
            for i in range(cold_iters):
                scratch.fill_(i & 0xFF)
                cev[i][0].record()
                self.step()
                cev[i][1].record()
            torch.cuda.synchronize()
            res["cold_ms"] = float(np.median([e[0].elapsed_time(e[1]) for e in cev]))
            del scratch
        return res


def k2_kernel_name(S, lin, engine, M):
    """The kernel-2 kernel a step of this layer launches (the 6-bit engine
    takes the 256 x 192 tile form, or the int8 engine's kernels for few
    rows, where the module's dispatch does)."""
    if engine == "fp6" and lin.route(M) == "int8":
        return K2_KERNEL["int8"]
    if engine == "fp6" and getattr(lin, "w_fp6_rows", None) is not None and S.fp6_n192_preferred(M, lin.N):
        return "k_gemm_w4a4_fp6_n192"
    return K2_KERNEL[engine]


def figures(res, M, N, K, r, bias, engine, workload=None, kname=None):
    """Step rate, kernel-2 roofline (MFMA) and kernel-1 roofline (HBM) of a
    timed step."""
    kname = kname or K2_KERNEL[engine]
    ops = 2.0 * M * N * K
    precision = "mxfp4" if engine == "mxfp4" else "int4"
    out = {"ms_per_step": round(res["ms"], 5), "value": round(ops / (res["ms"] * 1e-3) / 1e12, 2)}
    if "k2_ms" in res:
        k2_rate = ops / (res["k2_ms"] * 1e-3) / 1e12
        k1_ms = res.get("k1_graph_ms", res["k1_ms"])
        k1_gbs = k1_bytes(M, K, r, precision) / (k1_ms * 1e-3) / 1e9
        peak, unit = (FP4_PEAK_TFLOPS, "TFLOP/s") if engine == "mxfp4" else (INT8_PEAK_TOPS, "TOPS")
        out["roofline"] = {"bound": "mfma", "kernel": kname, "achieved": round(k2_rate, 2),
                           "peak": peak, "unit": unit, "frac": round(k2_rate / peak, 4),
                           "traffic": load_traffic(workload, r, engine) if workload and kname == K2_KERNEL[engine]
                           else None,
                           "avg_launch_us": round(res["k2_ms"] * 1e3, 2), "algorithmic_ops_per_launch": ops,
                           "algorithmic_hbm_bytes_per_launch": k2_bytes(M, N, K, r, bias, precision),
                           "how": "mean over the timed steps of the HIP-event interval around kernel 2"}
        if engine == "fp6":
            # the INT4 contraction runs on the 6-bit float MFMA: its own
            # instruction peak beside the INT8 peak the metric is quoted on
            out["roofline"]["fp6_mfma_peak"] = FP4_PEAK_TFLOPS
            out["roofline"]["frac_of_fp6_mfma_peak"] = round(k2_rate / FP4_PEAK_TFLOPS, 4)
        k1 = {"bound": "hbm", "kernel": "k_quant_act_lora_down" + (" (6-bit container output)" if engine == "fp6" else ""),
              "achieved": round(k1_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
              "frac": round(k1_gbs / HBM_PEAK_GBS, 4), "avg_launch_us": round(k1_ms * 1e3, 2),
              "event_launch_us": round(res["k1_ms"] * 1e3, 2),
              "algorithmic_bytes_per_launch": k1_bytes(M, K, r, precision),
              "how": ("mean of back-to-back launches replayed from a HIP graph between two HIP events "
                      "(event_launch_us: the mean HIP-event interval around kernel 1 within the timed steps)"
                      if "k1_graph_ms" in res else
                      "mean over the timed steps of the HIP-event interval around kernel 1")}
        if engine == "fp6":
            cb = fp6_container_bytes(M, N, K)
            k1["container_bytes_per_launch"] = (k1_bytes(M, K, r) - M * K // 2 - scale_bytes(K, "int4") * M
                                                + cb["x_codes"] + cb["x_scales"])
        out["roofline_k1"] = k1
    if "cold_ms" in res:
        out["cold"] = {"ms_per_step": round(res["cold_ms"], 5), "value": round(ops / (res["cold_ms"] * 1e-3) / 1e12, 2),
                       "steps": COLD_ITERS, "evict_bytes": COLD_EVICT_BYTES,
                       "how": "median of single steps, each after writing a 1 GiB buffer that evicts the "
                              "256 MB Infinity Cache (step time between HIP events, the write excluded)"}
    return out


def make_layer(S, weight_bits, act_absmax, rank, bias_bits=None, precision="int4", factors=None, engine="fp6"):
    import torch
    if precision == "mxfp4":
        prep = S.prepare_weights_mxfp4(weight_bits, act_absmax, rank=rank)
    else:
        prep = S.prepare_weights(weight_bits, act_absmax, rank=rank, factors=factors)
    bias = None
    if bias_bits is not None:
        bias = torch.from_numpy(bias_bits.view(np.int16).copy()).view(torch.bfloat16)
    return S.SVDQW4A4Linear(prep, bias, "cuda", engine=engine), prep


def dev_bf16(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def bench_mlp_chain(S, L, workloads, r, steps, warmup):
    """The FLUX MLP pair (4096 x 3072 -> 12288 -> GELU -> 3072, rank r on
    both layers, 6-bit engine) as one chain step -- kernel 1 of the up layer,
    the up layer's kernel 2 with the down layer's kernel 1 in its epilogue
    (and the partials' reduction), the down layer's kernel 2 -- against the
    two-layer step that stores the up output and reads it back in the down
    layer's kernel 1."""
    import torch
    wl = workloads.make_workload("mlp_pair")
    up_l, dn_l = wl.layers
    M, K, N, N2 = wl.M, up_l.K, up_l.N, dn_l.N
    up, _ = make_layer(S, up_l.weight_bits, wl.act_absmax(), r)
    x = dev_bf16(wl.x_bits)
    y_up = up(x)
    a_dn = torch.nn.functional.gelu(y_up.float(), approximate="tanh").abs().amax(0).cpu().numpy()
    dn, _ = make_layer(S, dn_l.weight_bits, a_dn.astype(np.float32), r)
    chain = S.SVDQMLPChain(up, dn)
    G, RB = K // 64, (M + 31) // 32
    xf = torch.empty((G, RB, 1536), dtype=torch.uint8, device="cuda")
    xs = torch.empty((G, 32 * RB), dtype=torch.float16, device="cuda")
    la = torch.empty((M, r), dtype=torch.float32, device="cuda") if r else None
    xf2 = torch.empty((N // 64, RB, 1536), dtype=torch.uint8, device="cuda")
    xs2 = torch.empty((N // 64, 32 * RB), dtype=torch.float16, device="cuda")
    la2 = torch.empty((M, r), dtype=torch.float32, device="cuda") if r else None
    ws = torch.empty(max(S.mlp_chain_workspace_bytes(M, N, r), 16), dtype=torch.uint8, device="cuda")
    y1 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    y2 = torch.empty((M, N2), dtype=torch.bfloat16, device="cuda")

    def k1_up():
        S.quant_act_lora_down_fp6(x, up.smooth_inv, up.lora_down, r, out=(xf, xs, la))

    def k2_dn():
        dn.kernel2_fp6(xf2, xs2, la2, M, out=y2)

    def chain_step():
        k1_up()
        S.gemm_w4a4_fp6_mlp_chain(xf, xs, up.w_fp6, up.w_scales, la, up.lora_up, up.bias, M, N, K, r,
                                  dn.smooth_inv, dn.lora_down, r, out=(xf2, xs2, la2), workspace=ws)
        k2_dn()

    def two_layer_step():
        k1_up()
        up.kernel2_fp6(xf, xs, la, M, out=y1)
        S.quant_act_lora_down_fp6(y1, dn.smooth_inv, dn.lora_down, r, act=L.SVDQ_ACT_GELU_TANH, out=(xf2, xs2, la2))
        k2_dn()

    def timed(step):
        settle(step)
        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            step()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / steps

    two_ms, chain_ms = timed(two_layer_step), timed(chain_step)
    ops = 2.0 * M * (K * N + N * N2)
    return {"workload": f"FLUX MLP pair {M}x{K} -> {N} -> tanh-GELU -> {N2}, rank {r} on both layers, 6-bit engine",
            "two_layer_ms_per_step": round(two_ms, 5), "chain_ms_per_step": round(chain_ms, 5),
            "chain_effective_tops": round(ops / (chain_ms * 1e-3) / 1e12, 2),
            "two_layer_effective_tops": round(ops / (two_ms * 1e-3) / 1e12, 2),
            "chain_saving_frac": round(1.0 - chain_ms / two_ms, 4),
            "how": "two-layer: up kernel 2 stores Y (bf16) and the down layer's kernel 1 reads it with GELU; "
                   "chain: the up kernel 2's epilogue writes the down layer's codes, scales and partial down "
                   "projections (reduced by a second kernel); both end with the down layer's kernel 2"}


def layer_input(S, wl, layer, act, rank):
    """The layer's bf16 input on the device and its calibration statistic
    max |input| per channel (after tanh-GELU when kernel 1 applies it).
    The MLP down projection's input is the up projection's output on the
    6-bit engine."""
    import torch
    if layer == 0:
        x = dev_bf16(wl.x_bits)
        a = wl.act_absmax()
    else:
        up, _ = make_layer(S, wl.layers[0].weight_bits, wl.act_absmax(), rank)
        x = up(dev_bf16(wl.x_bits))
        torch.cuda.synchronize()
        del up
        a = x.float().abs().amax(0).cpu().numpy()
    if act == "gelu_tanh":
        a = torch.nn.functional.gelu(x.float(), approximate="tanh").abs().amax(0).cpu().numpy()
    return x, np.asarray(a, np.float32)


def rank_sweep(S, workloads, steps, warmup):
    """The batched layer (4 x 4096 tokens, 3072 -> 12288) on the 6-bit
    engine at ranks 0, 16, 32, 64, 128: step time, overhead against rank 0,
    and the relative Frobenius error of the bf16 output against fp64 X W^T on
    SWEEP_ROWS seeded rows.  One rank-128 split of the smoothed weight is
    truncated per rank (the residual is recomputed per rank)."""
    import torch
    wl = workloads.make_workload("rank_sweep")
    Lr = wl.layers[0]
    M, K, N = wl.M, Lr.K, Lr.N
    a = wl.act_absmax()
    x = dev_bf16(wl.x_bits)
    rows = np.sort(np.random.default_rng(2024).choice(M, SWEEP_ROWS, replace=False))
    ref = workloads.bf16_bits_to_f64(wl.x_bits[rows]) @ Lr.weight.T
    t0 = time.perf_counter()
    full = S.prepare_weights(Lr.weight_bits, a, rank=max(SWEEP_RANKS))
    t_svd = time.perf_counter() - t0
    out = []
    for rr in SWEEP_RANKS:
        fac = (full["lora_down"][:rr], full["lora_up"][:, :rr]) if rr else None
        lin, _ = make_layer(S, Lr.weight_bits, a, rr, factors=fac)
        res = Runner(S, lin, x, 0, "fp6").time(steps, warmup)
        y = lin(x)
        torch.cuda.synchronize()
        yr = y[torch.from_numpy(rows).cuda()].float().cpu().numpy().astype(np.float64)
        err = float(np.linalg.norm(yr - ref) / np.linalg.norm(ref))
        f = figures(res, M, N, K, rr, False, "fp6")
        out.append({"rank": rr, "ms_per_step": f["ms_per_step"], "effective_tops": f["value"],
                    "k1_us": f["roofline_k1"]["avg_launch_us"], "k2_us": f["roofline"]["avg_launch_us"],
                    "rel_fro_err_vs_fp64": round(err, 6)})
        del lin, y
    ms0 = out[0]["ms_per_step"]
    for o in out:
        o["overhead_vs_rank0"] = round(o["ms_per_step"] / ms0 - 1.0, 4)
    return {"workload": "4 images x 4096 tokens, 16384x3072x12288, 6-bit engine", "M": M, "K": K, "N": N,
            "steps": steps, "warmup": warmup, "sampled_rows": SWEEP_ROWS, "svd_rank128_prepare_s": round(t_svd, 2),
            "ranks": out,
            "context": "pages: an unfused rank-32 branch costs +57% latency (NVIDIA, model card)"}


def _pmc_per_dispatch(d, counter):
    """{kernel name: [per-dispatch value]} of one counter from a rocprofv3
    --pmc csv directory (values of one dispatch summed)."""
    import csv
    import collections
    per = collections.defaultdict(float)
    names = {}
    with open(os.path.join(d, "pmc_counter_collection.csv")) as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] != counter:
                continue
            per[row["Dispatch_Id"]] += float(row["Counter_Value"])
            names[row["Dispatch_Id"]] = row["Kernel_Name"]
    out = collections.defaultdict(list)
    for did, v in per.items():
        out[names[did]].append(v)
    return out


def traffic_summary(engine, workload, rank, pmc_dir, copy_mib):
    """Kernel 2's HBM bytes per launch from rocprofv3 counter runs of this
    script under pmc_dir: fetch/ and write/ (FETCH_SIZE, WRITE_SIZE of a
    single-layer run of `engine`), copy_fetch/ and copy_write/ (the same
    counters of --copy-probe copy_mib).  Each counter is scaled by what it
    reads for the plain copy of known size.  Writes
    profiles/traffic_<workload>_r<rank>_<engine>.json."""
    kname = K2_KERNEL[engine]

    def mean_of(d, counter, key):
        vals = [v for k, lst in _pmc_per_dispatch(os.path.join(pmc_dir, d), counter).items() if key(k) for v in lst]
        return float(np.mean(vals)), len(vals)

    # demangled ("k_gemm_mxfp4_lora_up<0, 1, 256>") or mangled names
    # (the 256 x 192 form's name extends the 6-bit kernel's: not counted here)
    fetch, n = mean_of("fetch", "FETCH_SIZE", lambda k: kname in k and "_n192" not in k)
    write, _ = mean_of("write", "WRITE_SIZE", lambda k: kname in k and "_n192" not in k)
    if not n:
        raise SystemExit(f"no {kname} dispatches under {pmc_dir}")
    cdir = pmc_dir if os.path.isdir(os.path.join(pmc_dir, "copy_fetch")) else os.path.dirname(pmc_dir.rstrip("/"))
    copy_f = max(np.mean(v) for v in _pmc_per_dispatch(os.path.join(cdir, "copy_fetch"), "FETCH_SIZE").values())
    copy_w = max(np.mean(v) for v in _pmc_per_dispatch(os.path.join(cdir, "copy_write"), "WRITE_SIZE").values())
    copy_bytes = copy_mib * (1 << 20)
    rf, wf = copy_bytes / 1024.0 / copy_f, copy_bytes / 1024.0 / copy_w
    gen, layer, _, desc = BENCH_WORKLOADS[workload]
    import workloads
    wl = workloads.make_workload(gen)
    Lr = wl.layers[layer]
    M, K, N = wl.M, Lr.K, Lr.N
    precision = "mxfp4" if engine == "mxfp4" else "int4"
    alg_w = 2 * M * N
    d = {"kernel": kname, "engine": engine, "workload": f"{desc}, rank {rank}",
         "kernel_source_sha": kernel_source_hash(engine), "dispatches_averaged": n,
         "fetch_size_kib_per_dispatch": fetch, "write_size_kib_per_dispatch": write,
         "calibration": {"copy_bytes": copy_bytes, "fetch_size_kib": copy_f, "write_size_kib": copy_w,
                         "read_factor": round(rf, 4), "write_factor": round(wf, 4)},
         "k2_hbm_read_bytes": fetch * 1024 * rf, "k2_hbm_write_bytes": write * 1024 * wf,
         "k2_hbm_bytes": fetch * 1024 * rf + write * 1024 * wf,
         "algorithmic_read_bytes": k2_bytes(M, N, K, rank, Lr.bias_bits is not None, precision) - alg_w,
         "algorithmic_write_bytes": alg_w}
    p = os.path.join(ROOT, "profiles", f"traffic_{workload}_r{rank}_{engine}.json")
    with open(p, "w") as f:
        json.dump(d, f, indent=1)
    print(json.dumps({"wrote": p, **{k: d[k] for k in ("k2_hbm_bytes", "dispatches_averaged")}}))


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="mlp_up", choices=sorted(BENCH_WORKLOADS))
    ap.add_argument("--rank", type=int, default=32)
    ap.add_argument("--precision", default="int4", choices=["int4", "mxfp4"],
                    help="int4: INT4 group 64 with fp16 scales (the headline layer); "
                         "mxfp4: E2M1 codes with E8M0 scales per 32 on the block-scaled FP4 MFMA")
    ap.add_argument("--engine", default="fp6", choices=["fp6", "int8"],
                    help="engine of the INT4 layer: the 6-bit float MFMA (default) or the int8 MFMA")
    ap.add_argument("--no-overhead", action="store_true", help="skip the rank-0 and unfused comparison runs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-peaks", action="store_true", help="skip measuring the MFMA and copy peaks")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the int8 engine, MXFP4, QKV-epilogue and AWQ runs")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the tiny, attention-output, MLP-down and rank-sweep entries")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--rank-sweep", action="store_true",
                    help="only the batched rank sweep (16384x3072x12288, ranks 0/16/32/64/128), as one JSON line")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (HBM counter calibration)")
    ap.add_argument("--mix-probe", action="store_true",
                    help="only the register-only probe of the 6-bit route's inner loop (FP6 MFMA, fp32 "
                         "dequantization, both), as one JSON line")
    ap.add_argument("--qkv-only", action="store_true",
                    help="only the joint-stream QKV step with and without the fused epilogue, both INT4 "
                         "engines, as one JSON line")
    ap.add_argument("--traffic-summary", metavar="PMC_DIR",
                    help="no GPU work: write profiles/traffic_<workload>_r<rank>_<engine>.json from the "
                         "rocprofv3 counter runs under PMC_DIR (fetch/, write/; copy_fetch/, copy_write/ "
                         "there or one level up: the copy runs of --copy-probe 256)")
    args = ap.parse_args()
    if args.traffic_summary:
        traffic_summary("mxfp4" if args.precision == "mxfp4" else args.engine, args.workload, args.rank,
                        args.traffic_summary, 256)
        return

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); this layer's "
              "data-parallel path has no cross-GPU exchange, so per-GPU throughput is the "
              "one-GPU figure.", file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads
    import w4a4_rank_corrected_svdq_amd as S
    from w4a4_rank_corrected_svdq_amd import _lib as L

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.copy_probe:
        # a plain copy of known size: FETCH_SIZE / WRITE_SIZE of this kernel
        # calibrate the counters read for the layer's kernels
        n = args.copy_probe * (1 << 20)
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(max(args.steps, 1)):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "launches": max(args.steps, 1)}))
        return
    L.check(S.device_check(0), "device check")

    if args.rank_sweep:
        print(json.dumps({"rank_sweep": rank_sweep(S, workloads, args.steps, args.warmup)}))
        return
    if args.mix_probe:
        print(json.dumps({"mix_probe": mix_probe()}))
        return
    if args.qkv_only:
        print(json.dumps({"qkv_fused_epilogue": bench_qkv(S, L, workloads, args.rank, args.steps, args.warmup)}))
        return

    gen_name, layer, act, desc = BENCH_WORKLOADS[args.workload]
    wl = workloads.make_workload(gen_name)
    Lr = wl.layers[layer]
    M, K, N, r = wl.M, Lr.K, Lr.N, args.rank
    act_id = L.SVDQ_ACT_GELU_TANH if act == "gelu_tanh" else L.SVDQ_ACT_NONE
    engine = "mxfp4" if args.precision == "mxfp4" else args.engine
    x, a = layer_input(S, wl, layer, act, r)
    M = x.shape[0]
    has_bias = Lr.bias_bits is not None
    lin, _ = make_layer(S, Lr.weight_bits, a, r, Lr.bias_bits, args.precision,
                        engine="int8" if engine == "int8" else "fp6")
    run = Runner(S, lin, x, act_id, engine)
    res = run.time(args.steps, args.warmup, cold_iters=COLD_ITERS)
    main_m = figures(res, M, N, K, r, has_bias, run.engine, args.workload, k2_kernel_name(S, lin, engine, M))
    value = main_m["value"]
    out = {
        "metric": METRIC,
        "value": value,
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_s": SETTLE_S,
        "ms_per_step": main_m["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4 codes on fp6 (e3m2) MFMA" if engine == "fp6" else ("int4" if engine == "int8" else "fp4 (mxfp4)"),
        "data": "synthetic",
        "config": {"workload": f"{desc}, rank {r}, " + ("INT4 group 64" if args.precision == "int4" else "MXFP4 block 32"),
                   "M": M, "K": K, "N": N, "rank": r, "precision": args.precision, "engine": engine,
                   "group": 64 if args.precision == "int4" else 32, "act": act,
                   "bias": has_bias, "parallelism": "single GPU"},
        "pct_int8_peak": round(100.0 * value / INT8_PEAK_TOPS, 2),
        "roofline": main_m["roofline"],
        "roofline_k1": main_m["roofline_k1"],
        "cold": main_m["cold"],
    }
    if not args.no_overhead and r > 0 and args.precision == "int4":
        lin0, _ = make_layer(S, Lr.weight_bits, a, 0, Lr.bias_bits, engine="fp6")
        ms0 = Runner(S, lin0, x, act_id, engine).time(args.steps, args.warmup, events=False)["ms"]
        ms0_int8 = Runner(S, lin0, x, act_id, "int8").time(args.steps, args.warmup, events=False)["ms"]
        msu = Runner(S, lin, x, act_id, "unfused").time(args.steps, args.warmup, events=False)["ms"]
        out["low_rank_overhead"] = {
            "rank0_ms_per_step": round(ms0, 5), "overhead_frac": round(main_m["ms_per_step"] / ms0 - 1.0, 4),
            "unfused_ms_per_step": round(msu, 5), "int8_rank0_ms_per_step": round(ms0_int8, 5),
            "unfused_overhead_frac": round(msu / ms0_int8 - 1.0, 4),
            "how": "overhead_frac: this engine at rank r against rank 0; unfused_overhead_frac: the int8 "
                   "engine at rank 0 plus a separate down projection and a separate up projection "
                   "(read-modify-write of y), against the int8 engine at rank 0",
            "context": "pages: an unfused rank-32 branch costs +57% latency (NVIDIA, model card)"}
        del lin0
    if args.precision == "int4" and not args.no_variants:
        res8 = Runner(S, lin, x, act_id, "int8").time(args.steps, args.warmup)
        f8 = figures(res8, M, N, K, r, has_bias, "int8", args.workload)
        out["int8_engine"] = {"value": f8["value"], "ms_per_step": f8["ms_per_step"], "roofline": f8["roofline"],
                              "roofline_k1": f8["roofline_k1"]}
    configs = {}
    if args.precision == "int4" and not args.no_configs:
        for name in ("tiny", "attn_out", "mlp_down"):
            gname, li, cact, cdesc = BENCH_WORKLOADS[name]
            cw = workloads.make_workload(gname)
            cL = cw.layers[li]
            cact_id = L.SVDQ_ACT_GELU_TANH if cact == "gelu_tanh" else L.SVDQ_ACT_NONE
            cx, ca = layer_input(S, cw, li, cact, r)
            clin, _ = make_layer(S, cL.weight_bits, ca, r, cL.bias_bits)
            crun = Runner(S, clin, cx, cact_id, "fp6")
            cres = crun.time(args.steps, args.warmup)
            cM, cK, cN = cx.shape[0], cL.K, cL.N
            f = figures(cres, cM, cN, cK, r, cL.bias_bits is not None, crun.engine, name,
                        k2_kernel_name(S, clin, "fp6", cM))
            routed = " (few rows: the int8 engine's kernels)" if crun.engine == "int8" else ""
            entry = {"workload": cdesc + f", rank {r}, 6-bit engine{routed}", "M": cM, "K": cK, "N": cN,
                     "ms_per_step": f["ms_per_step"], "value": f["value"], "unit": "TOPS",
                     "pct_int8_peak": round(100.0 * f["value"] / INT8_PEAK_TOPS, 2),
                     "k1_us": f["roofline_k1"]["avg_launch_us"], "k2_us": f["roofline"]["avg_launch_us"],
                     "roofline": f["roofline"]}
            if name == "tiny":
                entry["us_per_step"] = round(f["ms_per_step"] * 1e3, 2)
            configs[name] = entry
            del clin, cx
        configs["mlp_chain"] = bench_mlp_chain(S, L, workloads, r, args.steps, args.warmup)
        configs["rank_sweep"] = rank_sweep(S, workloads, args.steps, args.warmup)
        out["configs"] = configs
    if args.precision == "int4" and not args.no_variants:
        lin_mx, _ = make_layer(S, Lr.weight_bits, a, r, Lr.bias_bits, "mxfp4")
        resm = Runner(S, lin_mx, x, act_id, "mxfp4").time(args.steps, args.warmup, cold_iters=COLD_ITERS)
        mx_m = figures(resm, M, N, K, r, has_bias, "mxfp4", args.workload)
        out["mxfp4_variant"] = {"value": mx_m["value"], "unit": "TFLOP/s (effective, 2MNK)",
                                "ms_per_step": mx_m["ms_per_step"], "cold": mx_m["cold"], "roofline": mx_m["roofline"],
                                "roofline_k1": mx_m["roofline_k1"]}
        del lin_mx
        out["qkv_fused_epilogue"] = bench_qkv(S, L, workloads, r, args.steps, args.warmup)
        out["awq_w4a16"] = bench_awq(S, workloads, max(args.steps, 20), args.warmup)
    if not args.no_peaks:
        # the same rooflines against the peaks measured on this device
        pk = measure_peaks()
        out["measured_peaks"] = pk
        mfma_pk = pk["fp4_mfma_tflops"] if engine == "mxfp4" else pk["int8_mfma_tops"]
        out["roofline"]["frac_of_measured_peak"] = round(out["roofline"]["achieved"] / mfma_pk, 4)
        out["roofline_k1"]["frac_of_measured_peak"] = round(out["roofline_k1"]["achieved"] / pk["hbm_copy_gbs"], 4)
        if "mxfp4_variant" in out:
            mv = out["mxfp4_variant"]
            mv["roofline"]["frac_of_measured_peak"] = round(mv["roofline"]["achieved"] / pk["fp4_mfma_tflops"], 4)
            mv["roofline_k1"]["frac_of_measured_peak"] = round(mv["roofline_k1"]["achieved"] / pk["hbm_copy_gbs"], 4)
        if "awq_w4a16" in out:
            aw = out["awq_w4a16"]["roofline"]
            aw["frac_of_measured_peak"] = round(aw["achieved"] / pk["hbm_copy_gbs"], 4)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, layer, r, args.cpu_seconds, args.precision)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
