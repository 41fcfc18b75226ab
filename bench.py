#!/usr/bin/env python3
"""Benchmark of the fused SVDQuant W4A4 + rank-r linear on one MI355X.

A step is one pass of the forward hot path over one batch: kernel 1 (smooth +
INT4 activation quantizer + down projection) then kernel 2 (W4A4 GEMM +
dequant + up projection + bias), on the FLUX MLP up-projection layer
(M = 4096 tokens, K = 3072, N = 12288, rank 32, group 64) unless --workload
says otherwise.  Weight preparation (smoothing, SVD, 4-bit residual) is a
one-time offline transform and runs before the timed region.

Prints one JSON line.  value = effective TOPS = 2*M*N*K / (time per step);
the low-rank flops are not credited.  --precision int4 (default) measures
the INT4 layer (group 64, fp16 scales); the same line carries the MXFP4
variant (E2M1 codes, E8M0 scale per 32, block-scaled FP4 MFMA) measured on
the same workload, unless --no-variants.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
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

# name -> (generator workload, layer index, act, description)
BENCH_WORKLOADS = {
    "mlp_up": ("mlp_pair", 0, "none", "FLUX MLP up-projection 4096x3072x12288"),
    "attn_out": ("attn_out", 0, "none", "FLUX attention-output projection 4096x3072x3072"),
    "joint_qkv": ("joint_qkv", 0, "none", "FLUX joint-stream fused QKV 4608x3072x9216 (+bias)"),
    "rank_sweep": ("rank_sweep", 0, "none", "4 images x 4096 tokens, 16384x3072x12288"),
}


def code_tokens(src: str) -> str:
    """C/C++ source with comments removed and whitespace runs collapsed."""
    import re
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return " ".join(src.split())


def kernel_source_hash() -> str:
    """Hash of the kernel sources with comments and whitespace removed, so
    that the stored counter figures stay valid across comment-only edits."""
    h = hashlib.sha256()
    for f in ("svdq_kernels.hip", "svdq_mx_kernels.hip", "svdq_device.h"):
        src = open(os.path.join(ROOT, "w4a4_rank_corrected_svdq_amd", "csrc", f)).read()
        h.update(code_tokens(src).encode())
    return h.hexdigest()[:16]


def scale_bytes(K, precision):
    """Scale bytes per row: fp16 per 64 (INT4) or one E8M0 byte per 32 (MXFP4)."""
    return 2 * (K // 64) if precision == "int4" else K // 32


def k1_bytes(M, K, r, precision="int4"):
    """Compulsory HBM bytes of kernel 1: read X (bf16), smooth_inv, L1; write
    codes, scales and lora_act."""
    return 2 * M * K + 4 * K + 2 * r * K + M * K // 2 + scale_bytes(K, precision) * M + 4 * M * r


def k2_bytes(M, N, K, r, bias, precision="int4"):
    sb = scale_bytes(K, precision)
    return (M * K // 2 + sb * M + N * K // 2 + sb * N + 4 * M * r
            + 2 * N * r + (2 * N if bias else 0) + 2 * M * N)


def load_traffic(workload: str, rank: int, precision: str = "int4"):
    """HBM traffic of kernel 2 measured by rocprofv3 PMC counters (committed
    under profiles/), used only while the kernel source is unchanged."""
    tag = "" if precision == "int4" else f"_{precision}"
    p = os.path.join(ROOT, "profiles", f"traffic_{workload}_r{rank}{tag}.json")
    if not os.path.exists(p):
        return None
    d = json.load(open(p))
    if d.get("kernel_source_sha") != kernel_source_hash():
        return None
    return d.get("k2_hbm_bytes")


def cpu_baseline(wl, layer, rank, target_s, precision="int4"):
    """The oracle (as it stands) on a bounded sample of rows of the same
    workload, timed on this host's cores."""
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([d.get("num_threads", 1) for d in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    Lr = wl.layers[layer]
    K, N = Lr.K, Lr.N
    a = wl.act_absmax()
    # preparation needs the SVD; rank-r factors from the oracle's own split
    t0 = time.perf_counter()
    po = O.prepare(Lr.weight, a, rank=rank) if precision == "int4" else O.mx.prepare_mx(Lr.weight, a, rank=rank)
    fwd = O.forward if precision == "int4" else O.mx.forward_mx
    t_prep = time.perf_counter() - t0
    # chunks of 128 rows, in order, wrapping round the workload's rows until
    # about target_s of forward time (at most four passes)
    rows_per_chunk = 128
    done_rows = 0
    t_fwd = 0.0
    x = wl.x
    while t_fwd < target_s and done_rows < 4 * wl.M:
        start = done_rows % wl.M
        xr = x[start:start + rows_per_chunk]
        t0 = time.perf_counter()
        fwd(xr, po, bias=Lr.bias)
        t_fwd += time.perf_counter() - t0
        done_rows += xr.shape[0]
    tops = 2.0 * done_rows * N * K / t_fwd / 1e12
    return {"value": tops, "unit": "TOPS", "cores": int(threads), "kind": "oracle",
            "sample": f"oracle forward ({precision}, fp64 numpy emulation) on {done_rows} rows (128-row chunks "
                      f"taken in order from the workload's {wl.M}, wrapping round), {t_fwd:.1f} s; oracle "
                      f"prepare (LAPACK SVD) took {t_prep:.1f} s and is not counted",
            "host_cpu_count": os.cpu_count()}


def bench_qkv(S, L, workloads, r, steps, warmup):
    """The joint-stream QKV projection (4608 x 3072 -> 9216, bias) with the
    fused per-head Q/K RMSNorm + rotary epilogue, against the same step with
    the plain epilogue."""
    import torch
    wl = workloads.make_workload("joint_qkv")
    Lr = wl.layers[0]
    M, K, N = wl.M, Lr.K, Lr.N
    prep = S.prepare_weights(Lr.weight_bits, wl.act_absmax(), rank=r)
    lin = S.SVDQW4A4Linear(prep, torch.from_numpy(Lr.bias_bits.view(np.int16).copy()).view(torch.bfloat16), "cuda")
    (qb, _), (kb, _) = workloads.norm_weights()
    cos, sin = workloads.rope_tables(512, 64)
    gq = torch.from_numpy(qb.view(np.int16).copy()).view(torch.bfloat16).cuda()
    gk = torch.from_numpy(kb.view(np.int16).copy()).view(torch.bfloat16).cuda()
    cos_d, sin_d = torch.from_numpy(cos).cuda(), torch.from_numpy(sin).cuda()
    x = torch.from_numpy(wl.x_bits.view(np.int16).copy()).view(torch.bfloat16).cuda()
    xc = torch.empty((M, K // 2), dtype=torch.uint8, device="cuda")
    xs = torch.empty((K // 64, M), dtype=torch.float16, device="cuda")
    la = torch.empty((M, r), dtype=torch.float32, device="cuda") if r else None
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

    def timed(fused):
        def step():
            S.quant_act_lora_down(x, lin.smooth_inv, lin.lora_down, r, out=(xc, xs, la))
            if fused:
                S.gemm_w4a4_lora_up_qkv(xc, xs, lin.w_codes, lin.w_scales, la, lin.lora_up, lin.bias, gq, gk,
                                        cos_d, sin_d, M, N, K, r, out=y)
            else:
                S.gemm_w4a4_lora_up(xc, xs, lin.w_codes, lin.w_scales, la, lin.lora_up, lin.bias, M, N, K, r, out=y)
        settle(step)
        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            step()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / steps

    plain_ms, fused_ms = timed(False), timed(True)
    ops = 2.0 * M * N * K
    return {"workload": "FLUX joint-stream QKV 4608x3072x9216 (+bias), rank 32, 24 heads of 128",
            "plain_ms_per_step": round(plain_ms, 5), "fused_ms_per_step": round(fused_ms, 5),
            "fused_effective_tops": round(ops / (fused_ms * 1e-3) / 1e12, 2),
            "epilogue_overhead_frac": round(fused_ms / plain_ms - 1.0, 4)}


def bench_awq(S, workloads, steps, warmup, M=1):
    """AWQ W4A16 on the FLUX double-block modulation projection (3072 ->
    18432, bias), M conditioning rows: HBM-bound on the weight read."""
    import torch
    wl = workloads.awq_workload(M, K=3072, N=18432, Mc=16, seed=7)
    K, N = wl["K"], wl["N"]
    prep = S.awq_prepare(wl["weight_bits"], wl["x_cal_bits"])
    lin = S.AWQW4A16Linear(prep, torch.from_numpy(wl["bias_bits"].view(np.int16).copy()).view(torch.bfloat16), "cuda")
    x = torch.from_numpy(wl["x_bits"].view(np.int16).copy()).view(torch.bfloat16).cuda()
    xh = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    xs = torch.empty((K // 64, 16), dtype=torch.float32, device="cuda")
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    st = torch.cuda.current_stream()

    def step(ev=None):
        S.awq_quant_act(x, lin.inv_scale, out=(xh, xs))
        if ev is not None:
            ev[0].record(st)
        S.awq_gemv(xh, xs, lin.w_codes, lin.w_scales, lin.w_zeros, lin.bias, M, N, K, out=y)
        if ev is not None:
            ev[1].record(st)

    settle(step)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    # kernel time from a second, event-instrumented pass
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    gemv_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    nbytes = N * K // 2 + 2 * N * (K // 64) + N * (K // 64) + 2 * M * K + 4 * (K // 64) * 16 + 2 * N + 2 * M * N
    gbs = nbytes / (gemv_ms * 1e-3) / 1e9
    return {"workload": f"FLUX modulation projection 3072 -> 18432 (+bias), M = {M}, AWQ INT4 group 64",
            "alpha": prep["alpha"], "ms_per_step": round(ms, 5),
            "roofline": {"bound": "hbm", "kernel": "k_awq_gemv_stream", "achieved": round(gbs, 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "avg_launch_us": round(gemv_ms * 1e3, 2), "algorithmic_bytes_per_launch": nbytes}}


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


SWEEP_RANKS = (0, 16, 32, 64, 128)
SWEEP_ROWS = 64


def rank_sweep(wl, Lr, desc, build_layer, run, x, M, K, N, args):
    """Step time per rank and the relative Frobenius error of the layer's
    bf16 output against fp64 X W^T on SWEEP_ROWS seeded rows (rank 0 is
    plain smoothed W4A4)."""
    import torch
    import workloads
    rows = np.sort(np.random.default_rng(2024).choice(M, SWEEP_ROWS, replace=False))
    ref = workloads.bf16_bits_to_f64(wl.x_bits[rows]) @ Lr.weight.T
    if Lr.bias is not None:
        ref = ref + Lr.bias
    out = []
    for rr in SWEEP_RANKS:
        lin = build_layer(rr)
        res = run(lin, args.steps, args.warmup, events=True)
        ms = res["wall_s"] * 1e3 / args.steps
        y = lin(x)
        torch.cuda.synchronize()
        yr = y[torch.from_numpy(rows).cuda()].float().cpu().numpy().astype(np.float64)
        err = float(np.linalg.norm(yr - ref) / np.linalg.norm(ref))
        out.append({"rank": rr, "ms_per_step": round(ms, 5),
                    "effective_tops": round(2.0 * M * N * K / (ms * 1e-3) / 1e12, 2),
                    "k1_us": round(res["k1_ms"] * 1e3, 1), "k2_us": round(res["k2_ms"] * 1e3, 1),
                    "rel_fro_err_vs_fp64": round(err, 6)})
        del lin, y
    ms0 = out[0]["ms_per_step"]
    for o in out:
        o["overhead_vs_rank0"] = round(o["ms_per_step"] / ms0 - 1.0, 4)
    return {"rank_sweep": {"workload": desc + f" ({args.precision})", "M": M, "K": K, "N": N,
                           "steps": args.steps, "warmup": args.warmup, "settle_s": SETTLE_S,
                           "sampled_rows": SWEEP_ROWS, "ranks": out,
                           "context": "pages: an unfused rank-32 branch costs +57% latency (NVIDIA, model card)"}}


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
    ap.add_argument("--no-overhead", action="store_true", help="skip the rank-0 comparison run")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-peaks", action="store_true", help="skip measuring the MFMA and copy peaks")
    ap.add_argument("--no-variants", action="store_true", help="skip the MXFP4 variant run")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--rank-sweep", action="store_true",
                    help="instead of the bench line: the batched rank sweep (16384x3072x12288, ranks "
                         "0/16/32/64/128) with step time, overhead against rank 0 and error against "
                         "fp64 X W on sampled rows, as one JSON line")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (HBM counter calibration)")
    args = ap.parse_args()

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
        args.workload = "rank_sweep"
    gen_name, layer, act, desc = BENCH_WORKLOADS[args.workload]
    wl = workloads.make_workload(gen_name)
    Lr = wl.layers[layer]
    M, K, N, r = wl.M, Lr.K, Lr.N, args.rank
    act_id = L.SVDQ_ACT_GELU_TANH if act == "gelu_tanh" else L.SVDQ_ACT_NONE

    prec = args.precision

    def build_layer(rank):
        if prec == "mxfp4":
            prep = S.prepare_weights_mxfp4(Lr.weight_bits, wl.act_absmax(), rank=rank)
        else:
            prep = S.prepare_weights(Lr.weight_bits, wl.act_absmax(), rank=rank)
        bias = None
        if Lr.bias_bits is not None:
            bias = torch.from_numpy(Lr.bias_bits.view(np.int16).copy()).view(torch.bfloat16)
        return S.SVDQW4A4Linear(prep, bias, "cuda")

    x = torch.from_numpy(wl.x_bits.view(np.int16).copy()).view(torch.bfloat16).cuda()

    def run(lin, steps, warmup, events=False, unfused=False, cold_iters=0):
        xc = torch.empty((M, K // 2), dtype=torch.uint8, device="cuda")
        if lin.precision == "mxfp4":
            xs = torch.empty((M, K // 32), dtype=torch.uint8, device="cuda")
        else:
            xs = torch.empty((K // 64, M), dtype=torch.float16, device="cuda")
        la = torch.empty((M, lin.rank), dtype=torch.float32, device="cuda") if lin.rank else None
        y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

        def step(mid=None):
            if unfused:
                # the low-rank branch as two extra passes: 4-bit path at
                # rank 0, then down projection (re-reads x) and up
                # projection (reads and rewrites y)
                S.quant_act_lora_down(x, lin.smooth_inv, None, 0, act=act_id, out=(xc, xs, None))
                S.gemm_w4a4_lora_up(xc, xs, lin.w_codes, lin.w_scales, None, None, lin.bias,
                                    M, N, K, 0, out=y)
                S.lora_down(x, lin.smooth_inv, lin.lora_down, lin.rank, act=act_id, out=la)
                S.lora_up_add(la, lin.lora_up, y)
                return
            if lin.precision == "mxfp4":
                S.quant_act_lora_down_mxfp4(x, lin.smooth_inv, lin.lora_down, lin.rank, act=act_id,
                                            out=(xc, xs, la))
                if mid is not None:
                    mid.record()
                S.gemm_mxfp4_lora_up(xc, xs, lin.w_codes, lin.w_scales, la, lin.lora_up, lin.bias,
                                     M, N, K, lin.rank, out=y)
                return
            S.quant_act_lora_down(x, lin.smooth_inv, lin.lora_down, lin.rank, act=act_id, out=(xc, xs, la))
            if mid is not None:
                mid.record()
            S.gemm_w4a4_lora_up(xc, xs, lin.w_codes, lin.w_scales, la, lin.lora_up, lin.bias,
                                M, N, K, lin.rank, out=y)

        settle(step)
        for _ in range(warmup):
            step()
        # the timed steps carry no instrumentation; a second pass of the same
        # length records HIP events around each kernel for the breakdown
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            step()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        res = {"wall_s": wall}
        if events:
            ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
            for i in range(steps):
                ev[i][0].record()
                step(ev[i][1])
                ev[i][2].record()
            torch.cuda.synchronize()
            res["k1_ms"] = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
            res["k2_ms"] = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
        if cold_iters:
            # cold steps: writing 1 GiB first evicts the 256 MB Infinity
            # Cache, so codes, scales and X come from HBM; the write is
            # outside each step's events
            scratch = torch.empty(COLD_EVICT_BYTES, dtype=torch.uint8, device="cuda")
            cev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(cold_iters)]
            for i in range(cold_iters):
                scratch.fill_(i & 0xFF)
                cev[i][0].record()
                step()
                cev[i][1].record()
            torch.cuda.synchronize()
            res["cold_ms"] = float(np.median([e[0].elapsed_time(e[1]) for e in cev]))
            del scratch
        return res

    def measure(precision):
        nonlocal prec
        prec = precision
        lin = build_layer(r)
        res = run(lin, args.steps, args.warmup, events=True, cold_iters=COLD_ITERS)
        ms = res["wall_s"] * 1e3 / args.steps
        ops = 2.0 * M * N * K
        k2_rate = ops / (res["k2_ms"] * 1e-3) / 1e12
        k1_gbs = k1_bytes(M, K, r, precision) / (res["k1_ms"] * 1e-3) / 1e9
        peak, unit = (INT8_PEAK_TOPS, "TOPS") if precision == "int4" else (FP4_PEAK_TFLOPS, "TFLOP/s")
        kname = "k_gemm_w4a4_lora_up" if precision == "int4" else "k_gemm_mxfp4_lora_up"
        return lin, ms, {
            "value": ops / (ms * 1e-3) / 1e12,
            "cold": {"ms_per_step": round(res["cold_ms"], 5), "value": round(ops / (res["cold_ms"] * 1e-3) / 1e12, 2),
                     "steps": COLD_ITERS, "evict_bytes": COLD_EVICT_BYTES,
                     "how": "median of single steps, each after writing a 1 GiB buffer that evicts the "
                            "256 MB Infinity Cache (step time between HIP events, the write excluded)"},
            "roofline": {"bound": "mfma", "kernel": kname,
                         "achieved": round(k2_rate, 2), "peak": peak, "unit": unit,
                         "frac": round(k2_rate / peak, 4), "traffic": load_traffic(args.workload, r, precision),
                         "avg_launch_us": round(res["k2_ms"] * 1e3, 2),
                         "algorithmic_ops_per_launch": ops,
                         "algorithmic_hbm_bytes_per_launch": k2_bytes(M, N, K, r, Lr.bias_bits is not None,
                                                                      precision)},
            "roofline_k1": {"bound": "hbm", "kernel": "k_quant_act_lora_down",
                            "achieved": round(k1_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                            "frac": round(k1_gbs / HBM_PEAK_GBS, 4),
                            "avg_launch_us": round(res["k1_ms"] * 1e3, 2),
                            "algorithmic_bytes_per_launch": k1_bytes(M, K, r, precision)},
        }

    if args.rank_sweep:
        print(json.dumps(rank_sweep(wl, Lr, desc, build_layer, run, x, M, K, N, args)))
        return

    lin, ms_per_step, main_m = measure(args.precision)
    value = main_m["value"]
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_s": SETTLE_S,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4" if args.precision == "int4" else "fp4 (mxfp4)",
        "data": "synthetic",
        "config": {"workload": f"{desc}, rank {r}, " + ("INT4 group 64" if args.precision == "int4"
                                                        else "MXFP4 block 32"),
                   "M": M, "K": K, "N": N, "rank": r, "precision": args.precision,
                   "group": 64 if args.precision == "int4" else 32,
                   "bias": Lr.bias_bits is not None, "parallelism": "single GPU"},
        "pct_int8_peak": round(100.0 * value / INT8_PEAK_TOPS, 2),
        "roofline": main_m["roofline"],
        "roofline_k1": main_m["roofline_k1"],
        "cold": main_m["cold"],
    }
    if not args.no_overhead and r > 0:
        lin0 = build_layer(0)
        res0 = run(lin0, args.steps, args.warmup, events=True)
        ms0 = res0["wall_s"] * 1e3 / args.steps
        ov = {"rank0_ms_per_step": round(ms0, 5), "overhead_frac": round(ms_per_step / ms0 - 1.0, 4)}
        if args.precision == "int4":
            resu = run(lin, args.steps, args.warmup, unfused=True)
            msu = resu["wall_s"] * 1e3 / args.steps
            ov.update(unfused_ms_per_step=round(msu, 5), unfused_overhead_frac=round(msu / ms0 - 1.0, 4))
        ov["context"] = "pages: an unfused rank-32 branch costs +57% latency (NVIDIA, model card)"
        out["low_rank_overhead"] = ov
    if args.precision == "int4" and not args.no_variants:
        _, ms_mx, mx_m = measure("mxfp4")
        out["mxfp4_variant"] = {"value": round(mx_m["value"], 2), "unit": "TFLOP/s (effective, 2MNK)",
                                "ms_per_step": round(ms_mx, 5), "cold": mx_m["cold"], "roofline": mx_m["roofline"],
                                "roofline_k1": mx_m["roofline_k1"]}
    if args.precision == "int4" and not args.no_variants:
        out["qkv_fused_epilogue"] = bench_qkv(S, L, workloads, r, args.steps, args.warmup)
        out["awq_w4a16"] = bench_awq(S, workloads, max(args.steps, 20), args.warmup)
    if not args.no_peaks:
        # the same rooflines against the peaks measured on this device
        pk = measure_peaks()
        out["measured_peaks"] = pk
        mfma_pk = pk["int8_mfma_tops"] if args.precision == "int4" else pk["fp4_mfma_tflops"]
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
