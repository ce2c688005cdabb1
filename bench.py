"""Throughput of exact attention forward and forward+backward on one MI355X.

A step is one pass of the whole path on one batch: fa_fwd (tiling + online
softmax) followed by fa_bwd (preprocess, dK/dV with recomputation, dQ).  The
workload is B=1, H=16, N=8192, d=128, bf16, seeded N(0,1) inputs already
resident in device memory.  Counted work: 4*B*H*N^2*d FLOP forward and 2.5x
that backward.

Prints one JSON line with the metric, the roofline of the dominant kernel
(its algorithmic FLOPs per launch over its average launch time, timed with
HIP events on the stream it runs on) and the CPU oracle timed on a bounded
sample of the same workload.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

Two further measurements print one JSON line per case instead:
    python bench.py --sweep     forward and fwd+bwd over N = 2048 .. 131072
                                 (d = 128, H = 16), with peak device memory
    python bench.py --splitkv   split-KV forward + merge against the plain
                                 forward when B*H is small
    python bench.py --fp32      the fp32 path (fa_fwd_f32, fa_bwd_f32) at several
                                 sizes, against the fp32 peak
    python bench.py --contrast  standard attention through device memory
                                 (S, then P, then O, with torch's own GEMM and
                                 softmax) beside fa_fwd, for contrast only
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 matrix-core peak (published)
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E (published)
METRIC = "attention TFLOP/s fwd & fwd+bwd, % of bf16 MFMA peak, N=8192 d=128"
WORKLOAD = "attn_bf16_b1h16_n8192_d128_fwdbwd"
COPY_BYTES = 512 << 20          # calibration copy: 512 MiB read + 512 MiB written
# HBM bytes per launch measured with rocprofv3 FETCH_SIZE / WRITE_SIZE passes
# (scaled by the same counters on the calibration copy), with the SHA-256 of
# the sources and build script the kernels were built from; reported only
# while those files are unchanged.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_bf16_b1h16_n8192_d128_hbm_traffic.json")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--settle", type=float, default=0.5,
                    help="seconds of untimed steps before the warm-up steps, so that the "
                         "shader clock has left its idle state (0 to skip)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=16,
                    help="heads of the workload the CPU oracle runs (forward+backward)")
    ap.add_argument("--sweep", action="store_true",
                    help="sequence-length sweep instead of the headline measurement")
    ap.add_argument("--splitkv", action="store_true",
                    help="split-KV forward + merge measurement instead of the headline one")
    ap.add_argument("--fp32", action="store_true",
                    help="fp32 path measurement instead of the headline one")
    ap.add_argument("--contrast", action="store_true",
                    help="materialised standard attention beside fa_fwd instead of the headline")
    ap.add_argument("--cpu-configs", action="store_true",
                    help="the fp64 oracle timed on a bounded sample of every named workload "
                         "(host cores only) instead of the headline")
    ap.add_argument("--configs", action="store_true",
                    help="forward and fwd+bwd throughput on every named workload instead of "
                         "the headline")
    ap.add_argument("--api-window", action="store_true",
                    help="run --steps whole steps (fa_fwd, fa_bwd) with every buffer allocated "
                         "beforehand, inside a roctx range named fa_steps, for a HIP API trace")
    return ap.parse_args()


def time_launches(fn, n, stream):
    """Average duration (ms) of n launches of fn, HIP events on `stream`."""
    import torch
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(n):
        fn()
    end.record(stream)
    end.synchronize()
    return start.elapsed_time(end) / n


def median_time(fn, inner, stream, outer=5):
    """Median over `outer` runs of the average duration (ms) of `inner`
    back-to-back launches of fn (so launch gaps do not count)."""
    return sorted(time_launches(fn, inner, stream) for _ in range(outer))[outer // 2]


def measured_traffic(kernel):
    """Calibrated HBM bytes per launch of `kernel`, or None if not measured
    for the current sources (digests of their code, comments excluded)."""
    from io_aware_softmax_02_amd.profile_summary import code_digest
    try:
        rec = json.load(open(TRAFFIC_FILE))["kernels"][kernel]
    except (OSError, KeyError, ValueError):
        return None
    for rel, digest in rec["source_sha256"].items():
        try:
            cur = code_digest(os.path.join(ROOT, rel))
        except OSError:
            return None
        if cur != digest:
            return None
    return int(rec["read_bytes"] + rec["write_bytes"])


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        return os.cpu_count() or 1


CPU_SAMPLE_HEADS = 4   # heads per workload the oracle runs in full for --cpu-configs


def cpu_configs(args):
    """The fp64 oracle (the CPU baseline, not tuned) timed on a bounded
    sample of each named workload: up to CPU_SAMPLE_HEADS heads in full (forward, and
    backward where the workload has one), and for the very long workload its
    sampled query rows against all keys.  Each line states the sample; the
    per-row time scaled to all rows and heads is labelled as an
    extrapolation."""
    import oracle
    import synth
    f64 = synth.to_f64
    threads = blas_threads()
    for name, w in synth.WORKLOADS.items():
        q, k, v, dO = synth.make_inputs(w)
        BH = w.B * w.H
        qf, kf, vf = (f64(x).reshape(BH, w.N, w.d) for x in (q, k, v))
        line = {"cpu_oracle": name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "cores": threads}
        if w.sample_rows is not None:
            rows = synth.sampled_rows(w)
            t0 = time.perf_counter()
            for bh in range(BH):
                oracle.sdpa_rows(qf[bh][rows[bh]], kf[bh], vf[bh], w.scale)
            dt = time.perf_counter() - t0
            nrows = BH * w.sample_rows
            flops = 4.0 * nrows * w.N * w.d
            line.update({"sample": f"{w.sample_rows} sampled query rows x {BH} heads against all "
                                   f"{w.N} keys, forward",
                         "seconds": round(dt, 2), "tflops": flops / dt / 1e12,
                         "extrapolated_full_forward_seconds": round(dt * (BH * w.N) / nrows, 1)})
        else:
            nh = min(BH, CPU_SAMPLE_HEADS)
            t0 = time.perf_counter()
            oracle.sdpa_forward(qf[:nh], kf[:nh], vf[:nh], w.scale)
            dtf = time.perf_counter() - t0
            flops = w.fwd_flops() * nh / BH
            dt = dtf
            what = "forward"
            if w.backward:
                gf = f64(dO).reshape(BH, w.N, w.d)
                t0 = time.perf_counter()
                oracle.sdpa_backward(qf[:nh], kf[:nh], vf[:nh], gf[:nh], w.scale)
                dt += time.perf_counter() - t0
                flops += w.bwd_flops() * nh / BH
                what = "forward + backward"
            line.update({"sample": f"{nh} of {BH} heads, {what}", "seconds": round(dt, 2),
                         "tflops": flops / dt / 1e12,
                         "extrapolated_all_heads_seconds": round(dt * BH / nh, 1)})
        print(json.dumps(line), flush=True)
        del q, k, v, dO, qf, kf, vf


def host_cores():
    """Host cores this process may run on (its CPU affinity)."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _limit_blas(threads):
    """Pool initializer: this worker's BLAS uses `threads` threads."""
    global _BLAS_LIMIT
    from threadpoolctl import threadpool_limits
    _BLAS_LIMIT = threadpool_limits(limits=threads)


def _oracle_head(args):
    """One head of the oracle, forward then backward (a pool task)."""
    import oracle
    q, k, v, g, scale = args
    oracle.sdpa_forward_head(q, k, v, scale)
    oracle.sdpa_backward_head(q, k, v, g, scale)
    return True


# Host memory one worker needs for a head of B=1, H=16, N=8192, d=128
# (S, P, dP and dS are 537 MB each in float64, plus temporaries).
CPU_BYTES_PER_WORKER = 3.5e9


def cpu_baseline(w, heads):
    """The fp64 oracle (forward + backward, materialising S and P) on `heads`
    of the workload's heads, spread over a process pool (one head per task,
    the BLAS threads of each worker = cores / workers, since the oracle's
    elementwise exp runs on one thread); returns a dict in the metric's
    unit.  The workers are started and warmed before the clock starts."""
    import concurrent.futures as cf
    import multiprocessing as mp
    import synth
    cores = host_cores()
    try:
        avail = os.sysconf("SC_AVPHYS_PAGES") * os.sysconf("SC_PAGE_SIZE")
    except (ValueError, OSError):  # pragma: no cover
        avail = 16e9
    workers = max(1, min(cores, heads, int(avail * 0.6 // CPU_BYTES_PER_WORKER)))
    per = max(1, cores // workers)
    q, k, v, dO = synth.make_inputs(w)
    f64 = synth.to_f64
    qf, kf, vf, gf = (f64(x).reshape(w.B * w.H, w.N, w.d)[:heads] for x in (q, k, v, dO))
    tasks = [(qf[h], kf[h], vf[h], gf[h], w.scale) for h in range(heads)]
    ctx = mp.get_context("spawn")
    with cf.ProcessPoolExecutor(max_workers=workers, mp_context=ctx, initializer=_limit_blas,
                                initargs=(per,)) as ex:
        tiny = [(x[:64], y[:64], z[:64], g[:64], w.scale) for x, y, z, g, _ in tasks[:workers]]
        list(ex.map(_oracle_head, tiny))          # workers started, modules imported
        t0 = time.perf_counter()
        list(ex.map(_oracle_head, tasks))
        dt = time.perf_counter() - t0
    flops = (w.fwd_flops() + w.bwd_flops()) * heads / (w.B * w.H)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(workers * per),
            "kind": "oracle",
            "sample": f"{heads} of {w.B * w.H} heads of B={w.B},H={w.H},N={w.N},d={w.d}, "
                      f"forward+backward, float64 numpy, process pool of {workers} workers x "
                      f"{per} BLAS threads ({cores} cores in the affinity set), {dt:.1f} s"}


def settle(seconds, dev):
    """Untimed bf16 products for `seconds`, so that the shader clock has left
    its idle state before a measurement mode's first timing."""
    import torch
    if seconds <= 0:
        return
    a = torch.randn(4096, 4096, device=dev).to(torch.bfloat16)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(10):
            torch.matmul(a, a)
        torch.cuda.synchronize()
    del a


def sweep(args):
    """Forward and fwd+bwd throughput and peak device memory over N at d=128,
    H=16, B=1 (the pages' long-context sizes, 2k .. 128k).  Alongside each
    line: the bytes one fp32 score matrix per head would take (the quantity
    the tiled method never stores)."""
    import torch
    import io_aware_softmax_02_amd as fa
    import synth
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    settle(args.settle, dev)
    stream = torch.cuda.current_stream(dev)
    B, H, d = 1, 16, 128
    for N in (2048, 4096, 8192, 16384, 32768, 65536, 131072):
        # the same inputs the long-sequence parity tests check
        q, k, v, dO = (x.to(dev) for x in synth.sweep_inputs(N))
        s = synth.default_scale(d)
        o = torch.empty_like(q)
        lse = torch.empty(B, H, N, dtype=torch.float32, device=dev)
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        torch.cuda.reset_peak_memory_stats()
        base = torch.cuda.memory_allocated()
        fa.fa_fwd(q, k, v, s, o=o, lse=lse)
        torch.cuda.synchronize()
        peak_fwd = torch.cuda.max_memory_allocated() - base
        dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
        ws = torch.empty(fa.fa_bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8, device=dev)
        inner = max(1, min(20, int(2e4 / (N / 1024) ** 2)))
        outer = 5 if N <= 32768 else 3
        fwd = lambda: fa.fa_fwd(q, k, v, s, o=o, lse=lse)
        bwd = lambda: fa.fa_bwd(q, k, v, o, lse, dO, s, dq=dq, dk=dk, dv=dv, workspace=ws)
        fwd(); bwd()
        torch.cuda.synchronize()
        med_f = median_time(fwd, inner, stream, outer)
        med_b = median_time(bwd, inner, stream, outer)
        fl_f = 4.0 * B * H * N * N * d
        print(json.dumps({
            "sweep": "N", "B": B, "H": H, "N": N, "d": d, "launches": inner, "runs": outer,
            "ms_fwd": round(med_f, 4), "ms_bwd": round(med_b, 4),
            "fwd_tflops": round(fl_f / (med_f * 1e-3) / 1e12, 1),
            "fwdbwd_tflops": round(3.5 * fl_f / ((med_f + med_b) * 1e-3) / 1e12, 1),
            "fwd_peak_extra_bytes": int(peak_fwd),
            "inputs_outputs_bytes_fwd": int(4 * q.numel() * 2 + lse.numel() * 4),
            "fp32_scores_per_head_bytes": int(N * N * 4),
        }), flush=True)
        del q, k, v, dO, o, lse, dq, dk, dv, ws


def configs(args):
    """Forward and forward+backward throughput on each named workload (the
    test and parity shapes, synth.WORKLOADS), one JSON line each.  The fp32
    workload runs the fp32 entry points; the others the bf16 ones."""
    import torch
    import io_aware_softmax_02_amd as fa
    import synth
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    settle(args.settle, dev)
    stream = torch.cuda.current_stream(dev)
    for name, w in synth.WORKLOADS.items():
        q, k, v, dO = (x.to(dev) for x in synth.make_inputs(w, backward=True))
        f32 = w.dtype == "f32"
        fwd_fn, bwd_fn = (fa.fa_fwd_f32, fa.fa_bwd_f32) if f32 else (fa.fa_fwd, fa.fa_bwd)
        ws_bytes = (fa.fa_bwd_f32_workspace_bytes if f32 else fa.fa_bwd_workspace_bytes)(
            w.B, w.H, w.N, w.d)
        o = torch.empty_like(q)
        lse = torch.empty(w.B, w.H, w.N, dtype=torch.float32, device=dev)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
        ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
        fwd = lambda: fwd_fn(q, k, v, w.scale, o=o, lse=lse)
        bwd = lambda: bwd_fn(q, k, v, o, lse, dO, w.scale, dq=dq, dk=dk, dv=dv, workspace=ws)
        fwd(); bwd()
        torch.cuda.synchronize()
        # about 50 ms of work per timed run, at least one launch
        est = median_time(lambda: (fwd(), bwd()), 1, stream, 1)
        inner = max(1, min(200, int(50.0 / max(est, 1e-3))))
        med_f = median_time(fwd, inner, stream)
        med_b = median_time(bwd, inner, stream)
        fl_f, fl_b = w.fwd_flops(), w.bwd_flops()
        print(json.dumps({
            "workload": name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "dtype": w.dtype,
            "launches": inner, "ms_fwd": round(med_f, 4), "ms_bwd": round(med_b, 4),
            "fwd_tflops": round(fl_f / (med_f * 1e-3) / 1e12, 2),
            "fwdbwd_tflops": round((fl_f + fl_b) / ((med_f + med_b) * 1e-3) / 1e12, 2),
            "peak_tflops": PEAK_FP32_TFLOPS if f32 else PEAK_BF16_TFLOPS,
        }), flush=True)
        del q, k, v, dO, o, lse, dq, dk, dv, ws
        torch.cuda.empty_cache()


def splitkv(args):
    """Split-KV forward + merge against the plain forward at small B*H,
    where the plain forward has fewer workgroups than the chip has CUs.
    The merge kernel's roofline is HBM bandwidth: per row it reads
    n_split * (4d + 4) bytes and writes 2d + 4."""
    import torch
    import io_aware_softmax_02_amd as fa
    import synth
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    settle(args.settle, dev)
    stream = torch.cuda.current_stream(dev)
    d = 128
    for B, H, N in ((1, 1, 8192), (1, 2, 16384), (1, 1, 65536), (1, 16, 8192)):
        q, k, v, _ = (x.to(dev) if x is not None else None
                      for x in synth.make_qkv(B, H, N, d, torch.bfloat16, seed=7))
        s = synth.default_scale(d)
        fl = 4.0 * B * H * N * N * d
        o0 = torch.empty_like(q)
        l0 = torch.empty(B, H, N, dtype=torch.float32, device=dev)
        fwd = lambda: fa.fa_fwd(q, k, v, s, o=o0, lse=l0)
        fwd()
        torch.cuda.synchronize()
        ms_plain = median_time(fwd, 10, stream)
        res = {"splitkv": True, "B": B, "H": H, "N": N, "d": d,
               "plain_ms": round(ms_plain, 4), "plain_tflops": round(fl / (ms_plain * 1e-3) / 1e12, 1),
               "splits": []}
        for P in (2, 4, 8, 16, 32):
            if P > fa.fa_fwd_split_max(B, H, N, d):
                continue
            op, lp = fa.fa_fwd_split(q, k, v, P, s)
            o, lse = fa.fa_merge(op, lp)
            split = lambda: fa.fa_fwd_split(q, k, v, P, s, o_part=op, lse_part=lp)
            merge = lambda: fa.fa_merge(op, lp, o=o, lse=lse)
            torch.cuda.synchronize()
            ms_s = median_time(split, 10, stream)
            ms_m = median_time(merge, 10, stream)
            rows = B * H * N
            mbytes = P * rows * (4 * d + 4) + rows * (2 * d + 4)
            res["splits"].append({
                "n_split": P, "split_ms": round(ms_s, 4), "merge_ms": round(ms_m, 4),
                "total_tflops": round(fl / ((ms_s + ms_m) * 1e-3) / 1e12, 1),
                "merge_GBps": round(mbytes / (ms_m * 1e-3) / 1e9, 1),
                "merge_frac_of_hbm": round(mbytes / (ms_m * 1e-3) / 1e9 / PEAK_HBM_GBS, 3)})
            del op, lp, o, lse
        print(json.dumps(res), flush=True)


PEAK_FP32_TFLOPS = 157.3      # MI355X fp32 (matrix and packed vector), published


def api_window(args):
    """The bench workload's step (fa_fwd, then fa_bwd) `args.steps` times,
    with outputs and workspace allocated and one step run beforehand, inside
    a roctx range named fa_steps.  Under `rocprofv3 --hip-trace
    --marker-trace` the HIP calls made inside the range are the library's own
    (plus the binding's device queries): no allocation, no copy, no memset."""
    import ctypes
    import torch
    import io_aware_softmax_02_amd as fa
    import synth
    w = synth.WORKLOADS[WORKLOAD]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q, k, v, dO = (x.to(dev) for x in synth.make_inputs(w))
    B, H, N, d = w.B, w.H, w.N, w.d
    o = torch.empty_like(q)
    lse = torch.empty(B, H, N, dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    ws = torch.empty(fa.fa_bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8, device=dev)

    def step():
        fa.fa_fwd(q, k, v, w.scale, o=o, lse=lse)
        fa.fa_bwd(q, k, v, o, lse, dO, w.scale, dq=dq, dk=dk, dv=dv, workspace=ws)

    step()
    torch.cuda.synchronize()
    roctx = ctypes.CDLL("librocprofiler-sdk-roctx.so")
    roctx.roctxRangePushA.argtypes = [ctypes.c_char_p]
    roctx.roctxRangePushA(b"fa_steps")
    for _ in range(args.steps):
        step()
    roctx.roctxRangePop()
    torch.cuda.synchronize()
    print(json.dumps({"api_window": True, "steps": args.steps, "workload": WORKLOAD}), flush=True)


def fp32(args):
    """Throughput of the fp32 path (fa_fwd_f32 / fa_bwd_f32) on seeded
    N(0,1) inputs, against the published fp32 peak."""
    import torch
    import io_aware_softmax_02_amd as fa
    import synth
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    settle(args.settle, dev)
    stream = torch.cuda.current_stream(dev)
    for B, H, N, d in ((1, 1, 64, 64), (1, 16, 2048, 64), (1, 16, 4096, 128), (1, 16, 8192, 128)):
        q, k, v, dO = (x.to(dev) for x in synth.make_qkv(B, H, N, d, torch.float32, seed=9,
                                                        backward=True))
        s = synth.default_scale(d)
        o = torch.empty_like(q)
        lse = torch.empty(B, H, N, dtype=torch.float32, device=dev)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
        ws = torch.empty(max(fa.fa_bwd_f32_workspace_bytes(B, H, N, d), 16), dtype=torch.uint8,
                         device=dev)
        fwd = lambda: fa.fa_fwd_f32(q, k, v, s, o=o, lse=lse)
        bwd = lambda: fa.fa_bwd_f32(q, k, v, o, lse, dO, s, dq=dq, dk=dk, dv=dv, workspace=ws)
        fwd(); bwd()
        torch.cuda.synchronize()
        inner = 20 if N <= 2048 else 3
        mf = median_time(fwd, inner, stream, 3)
        mb = median_time(bwd, inner, stream, 3)
        fl = 4.0 * B * H * N * N * d
        print(json.dumps({"fp32": True, "B": B, "H": H, "N": N, "d": d,
                          "ms_fwd": round(mf, 4), "ms_bwd": round(mb, 4),
                          "fwd_tflops": round(fl / (mf * 1e-3) / 1e12, 2),
                          "fwdbwd_tflops": round(3.5 * fl / ((mf + mb) * 1e-3) / 1e12, 2),
                          "fwd_frac_of_fp32_peak": round(fl / (mf * 1e-3) / 1e12 / PEAK_FP32_TFLOPS, 4)}),
              flush=True)
        del q, k, v, dO, o, lse, dq, dk, dv, ws


def standard_attention(q, k, v, scale, S=None, P=None, O=None):
    """Standard attention in three steps through device memory (the
    three-line form of 账房先生的奔命, section 五), for contrast with the
    tiled kernel only; no part of the library.  S = (scale Q) K^T is written
    as an N x N bf16 matrix per head, P = softmax(S) is read and written again,
    O = P V.  torch's own GEMM and softmax kernels do the work.  Returns
    (S, P, O); preallocated S, P, O are filled in place."""
    import torch
    B, H, N, d = q.shape
    # The right operand of a batched bf16 product is made contiguous first.
    kt = k.transpose(-1, -2).contiguous()
    qs = q * scale
    if S is None:
        S = torch.empty(B, H, N, N, dtype=q.dtype, device=q.device)
    if P is None:
        P = torch.empty_like(S)
    if O is None:
        O = torch.empty_like(q)
    torch.matmul(qs, kt, out=S)
    torch.softmax(S, dim=-1, out=P)
    torch.matmul(P, v, out=O)
    return S, P, O


def contrast(args):
    """Standard attention as three steps through device memory, for contrast
    with the tiled kernel (no part of the library): S = (s Q) K^T written as an
    N x N bf16 matrix per head, P = softmax(S) read and written again, O = P V.
    torch's GEMM and softmax kernels do the work.  Reported per step: time
    (median of back-to-back launches), the bytes of the N x N tensors it
    moves, and the peak device memory of the whole sequence, beside fa_fwd on
    the same inputs."""
    import torch
    import io_aware_softmax_02_amd as fa
    import synth
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    settle(args.settle, dev)
    stream = torch.cuda.current_stream(dev)
    # calibration copy for counter-based traffic (see the headline run)
    cal_src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
    cal_dst = torch.empty_like(cal_src)
    cal_dst.copy_(cal_src)
    torch.cuda.synchronize()
    del cal_src, cal_dst
    for name in ("fwd_bf16_b4h16_n2048_d64", "long_bf16_b1h16_n8192_d128"):
        w = synth.WORKLOADS[name]
        q, k, v, _ = (x.to(dev) if x is not None else None for x in synth.make_inputs(w))
        B, H, N, d, sc = w.B, w.H, w.N, w.d, w.scale
        # The right operand of a batched bf16 product is made contiguous first.
        kt = k.transpose(-1, -2).contiguous()
        qs = q * sc
        S, P, O = standard_attention(q, k, v, sc)
        step_s = lambda: torch.matmul(qs, kt, out=S)
        step_p = lambda: torch.softmax(S, dim=-1, out=P)
        step_o = lambda: torch.matmul(P, v, out=O)
        for f in (step_s, step_p, step_o):
            f()
        torch.cuda.synchronize()
        inner = 10
        ms = [median_time(f, inner, stream) for f in (step_s, step_p, step_o)]
        # peak memory of one pass, from nothing but the inputs
        del S, P
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        torch.cuda.reset_peak_memory_stats()
        base = torch.cuda.memory_allocated()
        S2, P2, O2 = standard_attention(q, k, v, sc)
        torch.cuda.synchronize()
        peak_std = torch.cuda.max_memory_allocated() - base
        del S2, P2
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        torch.cuda.reset_peak_memory_stats()
        base = torch.cuda.memory_allocated()
        o_fa, l_fa = fa.fa_fwd(q, k, v, sc)
        torch.cuda.synchronize()
        peak_fa = torch.cuda.max_memory_allocated() - base
        ms_fa = median_time(lambda: fa.fa_fwd(q, k, v, sc, o=o_fa, lse=l_fa), inner, stream)
        diff = float((O2.float() - o_fa.float()).abs().max())
        nn = B * H * N * N * 2
        gemm_flop = 2.0 * B * H * N * N * d
        print(json.dumps({
            "contrast": name, "B": B, "H": H, "N": N, "d": d,
            "ms_S_gemm": round(ms[0], 4), "ms_softmax": round(ms[1], 4), "ms_PV_gemm": round(ms[2], 4),
            "ms_standard_total": round(sum(ms), 4), "ms_fa_fwd": round(ms_fa, 4),
            "gemm_time_fraction": round((ms[0] + ms[2]) / sum(ms), 3),
            "S_gemm_tflops": round(gemm_flop / (ms[0] * 1e-3) / 1e12, 1),
            "PV_gemm_tflops": round(gemm_flop / (ms[2] * 1e-3) / 1e12, 1),
            "softmax_GBps_of_NxN_traffic": round(2 * nn / (ms[1] * 1e-3) / 1e9, 1),
            "nxn_bytes_per_tensor": nn,
            "peak_extra_bytes_standard": int(peak_std), "peak_extra_bytes_fa_fwd": int(peak_fa),
            "max_abs_diff_O_standard_vs_fa_fwd": round(diff, 5),
        }), flush=True)
        del q, k, v, kt, qs, O, O2, o_fa, l_fa


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the attention path is built and measured on a "
              "single MI355X (heads shard across GPUs with no communication, which is not "
              "built here). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.sweep:
        return sweep(args)
    if args.splitkv:
        return splitkv(args)
    if args.contrast:
        return contrast(args)
    if args.configs:
        return configs(args)
    if args.cpu_configs:
        return cpu_configs(args)
    if args.fp32:
        return fp32(args)
    if args.api_window:
        return api_window(args)

    import torch
    import io_aware_softmax_02_amd as fa
    import synth

    w = synth.WORKLOADS[WORKLOAD]
    # The CPU baseline runs first, while this process has not yet touched the
    # GPU, so that its worker processes start from a process without a GPU
    # context; the pool is shut down before the GPU work begins.
    cpu = None if args.no_cpu_baseline else cpu_baseline(w, args.cpu_heads)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q, k, v, dO = (x.to(dev) for x in synth.make_inputs(w))
    B, H, N, d = w.B, w.H, w.N, w.d
    s = w.scale
    o = torch.empty_like(q)
    lse = torch.empty(B, H, N, dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    ws = torch.empty(fa.fa_bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8, device=dev)
    delta = ws.view(torch.float32)[: B * H * N].view(B, H, N)
    stream = torch.cuda.current_stream(dev)
    # A plain device copy of known size, outside the timed region: its
    # FETCH_SIZE / WRITE_SIZE counters calibrate the traffic of the kernels.
    cal_src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
    cal_dst = torch.empty_like(cal_src)
    cal_dst.copy_(cal_src)
    ms_copy = time_launches(lambda: cal_dst.copy_(cal_src), 3, stream)
    del cal_src, cal_dst

    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    torch.cuda.reset_peak_memory_stats()
    mem_base = torch.cuda.memory_allocated()

    # One step is the whole path: the forward, then the backward's three
    # launches (fa_bwd runs exactly fa_bwd_preprocess, fa_bwd_dkdv and
    # fa_bwd_dq in this order; they are called one by one here so that an
    # event can be recorded between them).
    stages = (
        ("fwd_bf16", lambda: fa.fa_fwd(q, k, v, s, o=o, lse=lse)),
        ("bwd_pre_bf16", lambda: fa.fa_bwd_preprocess(o, dO, delta)),
        ("bwd_dkdv_bf16", lambda: fa.fa_bwd_dkdv(q, k, v, lse, dO, delta, s, dk=dk, dv=dv)),
        ("bwd_dq_bf16", lambda: fa.fa_bwd_dq(q, k, v, lse, dO, delta, s, dq=dq)),
    )

    def step():
        for _, fn in stages:
            fn()

    # fa_bwd itself gives the same gradients as its three stages (checked
    # before the clock is brought up: the host waits here).
    step()
    ref = (dq.clone(), dk.clone(), dv.clone())
    fa.fa_bwd(q, k, v, o, lse, dO, s, dq=dq, dk=dk, dv=dv, workspace=ws)
    torch.cuda.synchronize()
    assert all(torch.equal(x, y) for x, y in zip(ref, (dq, dk, dv)))
    del ref
    # Events of the timed region, chained on the launch stream, one after
    # every launch: the interval before launch i of step t ends where the
    # next begins, so the per-kernel averages add up to the time per step.
    ns = len(stages)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(ns * args.steps + 1)]

    # The shader clock ramps up over the first ~30 ms of work after idle
    # (per-launch durations fall by 20% over the first 15 launches); untimed
    # steps for `settle` seconds bring it to its working level, and the
    # warm-up steps run straight into the timed ones.
    t_settle = time.perf_counter()
    settle_steps = 0
    while time.perf_counter() - t_settle < args.settle:
        step()
        torch.cuda.synchronize()
        settle_steps += 1
    for _ in range(args.warmup):
        step()

    # Timed region: exactly K steps, synchronised on both sides.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev[0].record(stream)
    for t in range(args.steps):
        for i, (_, fn) in enumerate(stages):
            fn()
            ev[t * ns + i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_total = ev[0].elapsed_time(ev[-1])
    ms_step = ms_total / args.steps
    per_kernel = {name: sum(ev[t * ns + i].elapsed_time(ev[t * ns + i + 1])
                            for t in range(args.steps)) / args.steps
                  for i, (name, _) in enumerate(stages)}
    step_times = sorted(ev[t * ns].elapsed_time(ev[(t + 1) * ns]) for t in range(args.steps))
    peak_mem = torch.cuda.max_memory_allocated()
    ms_fwd = per_kernel["fwd_bf16"]
    ms_pre, ms_dkdv, ms_dq = (per_kernel[x] for x in ("bwd_pre_bf16", "bwd_dkdv_bf16",
                                                      "bwd_dq_bf16"))
    ms_bwd = ms_pre + ms_dkdv + ms_dq

    # Same-box reference for the matrix-core rate attainable on this kind of
    # data (outside the timed region): one 8192^3 bf16 GEMM through torch
    # (the vendor BLAS) on seeded N(0,1) operands.
    gen = torch.Generator(device=dev).manual_seed(7)
    ga = torch.randn(8192, 8192, generator=gen, device=dev).to(torch.bfloat16)
    gb = torch.randn(8192, 8192, generator=gen, device=dev).to(torch.bfloat16)
    gc = torch.empty(8192, 8192, dtype=torch.bfloat16, device=dev)
    torch.matmul(ga, gb, out=gc)
    ms_gemm = median_time(lambda: torch.matmul(ga, gb, out=gc), 5, stream, 3)
    gemm_tf = 2.0 * 8192 ** 3 / (ms_gemm * 1e-3) / 1e12
    del ga, gb, gc, gen

    pairs = B * H * N * N
    f_fwd = w.fwd_flops()
    f_bwd = w.bwd_flops()
    # algorithmic FLOPs per launch: forward 4d per (query, key) pair; the
    # dK/dV kernel does four of the backward's five counted contractions
    # (S, dP, dV, dK: 8d per pair); the dQ kernel does the fifth (2d per pair)
    # and recomputes S and dP, which are not counted again.
    kernels = {
        "fwd_bf16": {"ms": ms_fwd, "flop": 4.0 * d * pairs},
        "bwd_dkdv_bf16": {"ms": ms_dkdv, "flop": 8.0 * d * pairs},
        "bwd_dq_bf16": {"ms": ms_dq, "flop": 2.0 * d * pairs},
        "bwd_pre_bf16": {"ms": ms_pre, "flop": 0.0},
    }
    for kk in kernels.values():
        kk["tflops"] = kk["flop"] / (kk["ms"] * 1e-3) / 1e12
    dom = max(("fwd_bf16", "bwd_dkdv_bf16", "bwd_dq_bf16"), key=lambda x: kernels[x]["ms"])
    ach = kernels[dom]["tflops"]

    tf_step = (f_fwd + f_bwd) / (ms_step * 1e-3) / 1e12
    tf_fwd = f_fwd / (ms_fwd * 1e-3) / 1e12
    out = {
        "metric": METRIC,
        "value": round(tf_step, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_steps": settle_steps,
        "ms_per_step": round(ms_step, 4),
        "ms_per_step_median": round(step_times[len(step_times) // 2], 4),
        "ms_per_step_min": round(step_times[0], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded iid N(0,1) Q, K, V, dO rounded to bf16",
        "config": {"workload": WORKLOAD, "B": B, "H": H, "N": N, "d": d, "causal": False,
                   "scale": s, "counted_flop_fwd": f_fwd, "counted_flop_fwdbwd": f_fwd + f_bwd},
        "fwdbwd_tflops": round(tf_step, 2),
        "fwdbwd_frac_of_peak": round(tf_step / PEAK_BF16_TFLOPS, 4),
        "fwd_tflops": round(tf_fwd, 2),
        "fwd_frac_of_peak": round(tf_fwd / PEAK_BF16_TFLOPS, 4),
        "ms_fwd": round(ms_fwd, 4),
        "ms_bwd": round(ms_bwd, 4),
        "wall_s_timed_region": round(wall, 4),
        "kernels": {kname: {"ms": round(kv["ms"], 4), "tflops": round(kv["tflops"], 2)}
                    for kname, kv in kernels.items()},
        "kernels_timing": "average per launch over the timed steps (events between launches)",
        "hbm_copy_GBps": round(2 * COPY_BYTES / (ms_copy * 1e-3) / 1e9, 1),
        "reference_gemm": {"what": "torch.matmul bf16 8192x8192x8192, N(0,1) operands",
                           "tflops": round(gemm_tf, 1),
                           "frac_of_peak": round(gemm_tf / PEAK_BF16_TFLOPS, 4),
                           "cu_count": torch.cuda.get_device_properties(dev).multi_processor_count},
        "peak_mem_bytes": int(peak_mem),
        "mem_inputs_outputs_bytes": int(mem_base),
        "roofline": {"kernel": dom, "bound": "mfma", "achieved": round(ach, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(dom), "traffic_unit": "HBM bytes per launch"},
    }
    if cpu is not None:
        out["cpu_baseline"] = cpu
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
