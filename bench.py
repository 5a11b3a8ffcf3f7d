"""Benchmark of the sparse MoE block forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c4b] [--format block128|mx|mxfp4]
                    [--flush-mib 512]
    python bench.py --workload attn_prefill | attn_decode

A step is one whole forward (router + top-k + softmax + x quantisation,
routing scan and placement, gate/up grouped FP8 GEMM with SwiGLU and h
quantisation, down grouped FP8 GEMM, weighted combine) over one batch of
seeded synthetic input already resident in HBM.  The default workload is the
largest configuration that fits one GPU: the skewed gpt-oss-120b-like layer
at prefill size (T=16384 tokens, d=2944, f=2944, E=128, k=4, Zipf(1.1)
expert popularity) with 128x128 block-scaled FP8 weights (``--format mx``:
the MXFP8 variant, E8M0 scales per 32; ``--format mxfp4``: E2M1 weights with
those scales).  ``--workload c1`` is the decode-shaped layer (T=64).

Prints one JSON line: whole-job tokens/s; the roofline of the gate/up GEMM
(its duration measured with HIP events inside the timed region, on the
stream it runs on); ``layer_frac``, the whole step's algorithmic work over
the step time against the binding peak (FP8 MFMA flops for prefill shapes,
HBM bytes for decode shapes); and the CPU oracle timed on a bounded sample
of the same workload.

``--flush-mib N`` reads N MiB (more than the 4 MB L2 of each XCD and the
256 MB memory-side cache) between timed calls, outside the calls' own
events, so every call reads its weights from HBM; the step time is then the
mean of the per-call event times.  The flush reads rather than writes: a
written buffer would leave dirty lines whose write-back lands inside the
next timed call.

``--workload attn_prefill`` / ``attn_decode`` time the attention with per-head
sinks instead (gpt-oss shape: 64 query heads, 8 key/value heads, head dim
64): causal prefill of one 8192-token sequence, and one decode step of 64
sequences over KV caches of up to 4096 tokens (seeded ragged lengths).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import sparse_moe_layer_fp32_amd as moe  # noqa: E402
from sparse_moe_layer_fp32_amd import inputs as gen  # noqa: E402

METRIC = "MoE-layer tokens/s + % of FP8 MFMA peak (prefill) / % HBM BW (decode)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense FP8 MFMA, TFLOP/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
ATTN_METRIC = "attention tokens/s + % of bf16 MFMA peak (prefill) / % HBM BW (decode)"
GEMM_SRC = os.path.join(ROOT, "sparse_moe_layer_fp32_amd", "csrc", "gemm.hip")
ATTN_SRC = os.path.join(ROOT, "sparse_moe_layer_fp32_amd", "csrc", "attention.hip")

# HBM traffic of one gate/up GEMM launch from rocprofv3 --pmc runs (one run for
# FETCH_SIZE, one for WRITE_SIZE, KiB per dispatch) of
#   bench.py --workload W --steps 3 --warmup 1 --no-cpu-baseline --copy-calibration-mib 1024
# Each counter is scaled by what it reads for that run's 1 GiB device copy:
# FETCH_SIZE counts the 128-byte fabric reads of gfx950 as 64 bytes (the copy
# reads as 524312 KiB), WRITE_SIZE reads the copy exactly.  Keyed by the
# SHA-256 of the GEMM source the counters were taken on: any change to the
# kernels reports null until they are measured again.  Keys: workload, or
# workload-mx for the MXFP8 format.
TRAFFIC = {
    "c4b": {"gemm_sha256": "376c0a3adadda0ea029a814fc7ac8d4b51cf7e183117f09f550855471b4b7dc7",
        "fetch_kib": 2348308.521, "write_kib": 210638.406,
        "copy_fetch_kib": 524315.3125, "copy_write_kib": 1048576.0},
    "c1": {"gemm_sha256": "376c0a3adadda0ea029a814fc7ac8d4b51cf7e183117f09f550855471b4b7dc7",
        "fetch_kib": 271558.396, "write_kib": 759.208,
        "copy_fetch_kib": 524307.5, "copy_write_kib": 1048576.0},
    "c2": {"gemm_sha256": "376c0a3adadda0ea029a814fc7ac8d4b51cf7e183117f09f550855471b4b7dc7",
        "fetch_kib": 905262.146, "write_kib": 104102.63,
        "copy_fetch_kib": 524307.0, "copy_write_kib": 1048576.0},
    "c1-mx": {"gemm_sha256": "376c0a3adadda0ea029a814fc7ac8d4b51cf7e183117f09f550855471b4b7dc7",
        "fetch_kib": 279948.531, "write_kib": 761.156,
        "copy_fetch_kib": 524307.6875, "copy_write_kib": 1048576.0},
    "c2-mx": {"gemm_sha256": "376c0a3adadda0ea029a814fc7ac8d4b51cf7e183117f09f550855471b4b7dc7",
        "fetch_kib": 909948.875, "write_kib": 104154.87,
        "copy_fetch_kib": 524307.625, "copy_write_kib": 1048576.0},
    "c1-mxfp4": {"gemm_sha256": "376c0a3adadda0ea029a814fc7ac8d4b51cf7e183117f09f550855471b4b7dc7",
        "fetch_kib": 144511.323, "write_kib": 759.156,
        "copy_fetch_kib": 524313.125, "copy_write_kib": 1048576.0},
    "c2-mxfp4": {"gemm_sha256": "376c0a3adadda0ea029a814fc7ac8d4b51cf7e183117f09f550855471b4b7dc7",
        "fetch_kib": 552645.885, "write_kib": 104099.526,
        "copy_fetch_kib": 524305.375, "copy_write_kib": 1048576.0},
}


# The same for one attention call (decode: the decode and combine kernels of a
# call added; prefill: its one kernel), keyed by the SHA-256 of the attention
# source.
ATTN_TRAFFIC = {
    "attn_decode": {"attn_sha256": "6d6c0ca7148f64c1d2ebc260ac251caef4f263eb474b80f45f15010cd2236884",
        "fetch_kib": 197909.969, "write_kib": 3759.625,
        "copy_fetch_kib": 524316.4375, "copy_write_kib": 1048576.0},
    "attn_prefill": {"attn_sha256": "6d6c0ca7148f64c1d2ebc260ac251caef4f263eb474b80f45f15010cd2236884",
        "fetch_kib": 51132.094, "write_kib": 65536.000,
        "copy_fetch_kib": 524313.6875, "copy_write_kib": 1048576.0},
}


def src_sha(path):
    import hashlib
    with open(path, "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()


def gemm_src_sha():
    return src_sha(GEMM_SRC)


def _scaled_bytes(t):
    fetch = t["fetch_kib"] * (1 << 20) / t["copy_fetch_kib"]
    write = t["write_kib"] * (1 << 20) / t["copy_write_kib"]
    return int(round((fetch + write) * 1024))


def measured_traffic(workload):
    t = TRAFFIC.get(workload)
    if t is None or t["gemm_sha256"] != gemm_src_sha():
        return None
    return _scaled_bytes(t)


def measured_attn_traffic(workload):
    t = ATTN_TRAFFIC.get(workload)
    if t is None or t["attn_sha256"] != src_sha(ATTN_SRC):
        return None
    return _scaled_bytes(t)


def calibration_copy(mib, dev):
    """A device copy of known size in the profiled process: the counter runs
    scale FETCH_SIZE and WRITE_SIZE by what they read for it."""
    if mib <= 0:
        return
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    log(f"[bench] calibration copy of {n} bytes")
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def sampled_steps(steps, every):
    """Steps of the instrumented pass that carry the per-kernel events: one per
    ``every`` timed steps (at least one).  A timing event costs a few
    microseconds of device time, so the events run in an untimed pass of their
    own and the timed region holds plain calls only."""
    every = max(1, every)
    picked = [i for i in range(steps) if i % every == every - 1]
    return picked or [steps - 1]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def _scale_bytes(K, N, fmt):
    """Bytes of the scales of one K x N weight matrix: fp32 per 128x128 block,
    or one E8M0 byte per 32 K rows per column (MX)."""
    return (K // 32) * N if fmt in ("mx", "mxfp4") else 4 * (K // 128) * (N // 128)


def _weight_bytes(K, N, fmt):
    """Bytes of one K x N weight matrix's elements: e4m3, or two E2M1 per byte."""
    return K * N // 2 if fmt == "mxfp4" else K * N


def _act_scale_bytes(rows, K):
    """Scales of rows x K quantised activations: fp32 per 128 or E8M0 per 32:
    the same byte count."""
    return rows * (K // 32)


def gateup_algorithmic(inp, counts):
    """Algorithmic HBM bytes and FP8 flops of one gate/up GEMM launch.

    Bytes: every touched expert's gate/up weights (e4m3 codes, scales, bf16
    bias) once, the quantised activations of every token once (codes +
    scales), and the h codes + scales of every routed row once.
    Flops: 2 * rows * d * 2f."""
    T, d, f, k = inp["T"], inp["d"], inp["f"], inp["k"]
    fmt = inp.get("format", "block128")
    R = T * k
    touched = int(np.count_nonzero(counts))
    w = touched * (_weight_bytes(d, 2 * f, fmt) + _scale_bytes(d, 2 * f, fmt) + 2 * 2 * f)
    a = T * d + _act_scale_bytes(T, d)
    h = R * f + _act_scale_bytes(R, f)
    return dict(bytes=w + a + h, flops=2.0 * R * d * 2 * f, touched=touched)


def down_algorithmic(inp, counts):
    T, d, f, k = inp["T"], inp["d"], inp["f"], inp["k"]
    fmt = inp.get("format", "block128")
    R = T * k
    touched = int(np.count_nonzero(counts))
    w = touched * (_weight_bytes(f, d, fmt) + _scale_bytes(f, d, fmt) + 2 * d)
    return dict(bytes=w + R * f + _act_scale_bytes(R, f) + 4 * R * d, flops=2.0 * R * f * d)


def host_facts():
    """CPU model and the BLAS library NumPy runs the oracle's matmuls on."""
    from threadpoolctl import threadpool_info
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = [f"{i.get('internal_api')} {i.get('version')} ({i.get('threading_layer', 'n/a')} threads)"
            for i in threadpool_info() if i.get("user_api") == "blas"]
    return model, "; ".join(blas) or "unknown", f"numpy {np.__version__}"


def layer_algorithmic(inp, counts):
    """Algorithmic work of one whole forward: FP8 flops 2*T*k*(d*2f + f*d),
    and HBM bytes = every touched expert's weights, scales and biases once +
    the router weights and bias + x in + out (bf16)."""
    T, d, f, E, k = inp["T"], inp["d"], inp["f"], inp["E"], inp["k"]
    fmt = inp.get("format", "block128")
    touched = int(np.count_nonzero(counts))
    per_expert = (_weight_bytes(d, 2 * f, fmt) + _scale_bytes(d, 2 * f, fmt) + 2 * 2 * f +
                  _weight_bytes(f, d, fmt) + _scale_bytes(f, d, fmt) + 2 * d)
    byts = touched * per_expert + 4 * d * E + 4 * E + 2 * T * d + 2 * T * d
    return dict(bytes=byts, flops=2.0 * T * k * (d * 2 * f + f * d), touched=touched)


def cpu_baseline(inp, budget_s=12.0):
    """The CPU oracle (as it stands) on a bounded sample of the workload's tokens."""
    from threadpoolctl import threadpool_info

    from oracle import oracle as orc
    T = inp["T"]
    n = min(T, 64)
    toks = np.arange(n)
    t0 = time.perf_counter()
    reps = 0
    while True:
        orc.forward(inp, tokens=toks)
        reps += 1
        if time.perf_counter() - t0 >= budget_s or reps >= 50:
            break
    dt = time.perf_counter() - t0
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    model, blas, npv = host_facts()
    return {"value": round(reps * n / dt, 3), "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle", "cpu": model, "blas": blas, "numpy": npv,
            "sample": f"{reps} x oracle.forward on the first {n} of {T} tokens (routing of all "
                      f"{T} tokens, expert math of the sample, fp64 NumPy; {dt:.1f} s)"}


def attn_bench(args):
    """Sink attention: one call per step, HIP events around the timed steps."""
    from oracle import attention as att
    shape = gen.GPT_OSS_ATTN
    dev = torch.device("cuda:0")
    prefill = args.workload == "attn_prefill"
    if prefill:
        S = 8192
        inp = gen.make_attn_prefill(shape, S, seed=0)
        p = moe.attn_device_inputs(inp, dev)
        out = torch.empty((S, shape.Hq, shape.D), dtype=torch.bfloat16, device=dev)
        run = lambda: moe.attn_prefill(p["q"], p["k"], p["v"], p["sinks"], p["sm_scale"], out=out)
        tokens = S
        flops = 4.0 * shape.D * shape.Hq * S * (S + 1) / 2       # QK^T and PV over the causal triangle
        work = dict(flops=flops)
    else:
        B, L = 64, 4096
        inp = gen.make_attn_decode(shape, B, L, seed=0)
        p = moe.attn_device_inputs(inp, dev)
        out = torch.empty((B, shape.Hq, shape.D), dtype=torch.bfloat16, device=dev)
        ws = torch.empty(moe.attn_decode_workspace_bytes(B, shape.Hq, L), dtype=torch.uint8, device=dev)
        run = lambda: moe.attn_decode(p["q"], p["k"], p["v"], p["kv_len"], p["sinks"], p["sm_scale"],
                                      out=out, workspace=ws)
        tokens = B
        kv_bytes = int(inp["kv_len"].astype(np.int64).sum()) * shape.Hkv * shape.D * 2 * 2
        work = dict(bytes=kv_bytes + 2 * B * shape.Hq * shape.D * 2)  # K, V of the visible keys + q + out
    calibration_copy(args.copy_calibration_mib, dev)
    log(f"[bench] {args.workload}: warmup {args.warmup}")
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    sampled = sampled_steps(args.steps, args.event_every)
    evs = {i: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for i in sampled}
    for i in sampled:  # per-call times from an untimed instrumented pass
        evs[i][0].record()
        run()
        evs[i][1].record()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        run()
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps
    call_ms = float(np.mean([a.elapsed_time(b) for a, b in evs.values()]))
    if prefill:
        ach = work["flops"] / (call_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach / BF16_PEAK_TFLOPS, 4), "traffic": measured_attn_traffic(args.workload),
                "kernel": "attn_prefill_kernel<8, 2>", "avg_ms": round(call_ms, 5), "algorithmic_flops": work["flops"]}
    else:
        ach = work["bytes"] / (call_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": measured_attn_traffic(args.workload),
                "kernel": "attn_decode_kernel + attn_combine_kernel (the whole call)",
                "avg_ms": round(call_ms, 5), "algorithmic_bytes": work["bytes"]}
    roof["event_launches"] = len(sampled)
    cfg = ({"workload": f"attn_prefill: causal GQA attention with sinks, S=8192, Hq=64, Hkv=8, D=64",
            "S": 8192} if prefill else
           {"workload": f"attn_decode: one query per sequence, B=64, KV up to 4096 (ragged, mean "
                        f"{float(inp['kv_len'].mean()):.0f}), Hq=64, Hkv=8, D=64", "B": 64, "Lmax": 4096})
    cfg.update(Hq=shape.Hq, Hkv=shape.Hkv, D=shape.D)
    res = {"metric": ATTN_METRIC, "value": round(tokens / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic", "config": cfg,
           "roofline": roof}
    if not args.no_cpu_baseline:
        log("[bench] CPU oracle baseline")
        rng = np.random.default_rng(7)
        t0 = time.perf_counter()
        reps = 0
        while True:
            if prefill:
                rows = np.sort(rng.choice(S, size=8, replace=False))   # uniform rows: mean causal length
                att.prefill(inp["q"], inp["k"], inp["v"], inp["sinks"], inp["sm_scale"], rows=rows)
                n = len(rows)
            else:
                sl = slice(4 * (reps % (B // 4)), 4 * (reps % (B // 4)) + 4)
                att.decode(inp["q"][sl], inp["k"][sl], inp["v"][sl], inp["kv_len"][sl], inp["sinks"], inp["sm_scale"])
                n = 4
            reps += 1
            if time.perf_counter() - t0 >= 12.0 or reps >= 400:
                break
        dt = time.perf_counter() - t0
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
        res["cpu_baseline"] = {"value": round(reps * n / dt, 3), "unit": "tokens/s", "cores": int(threads),
                               "kind": "oracle",
                               "sample": f"{reps} x oracle on {n} " + ("seeded uniform query rows of 8192" if prefill
                                                                       else "consecutive sequences") + f"; {dt:.1f} s"}
    print(json.dumps(res), flush=True)


def peaks_bench(args):
    """Measured ceilings of this GPU (libmoe_peaks.so): FP8 MFMA issue rate and
    the shader clock it settles at, HBM streaming read and device copy rates,
    and the LDS read rates (bytes per clock per CU) of ds_read_b128 and the
    transposing ds_read_b64_tr_b8 the GEMMs read their fragments with."""
    import ctypes
    from sparse_moe_layer_fp32_amd import build as b
    if not os.path.exists(b.PEAKS_LIB):
        raise ImportError(f"{b.PEAKS_LIB} is missing: build the package first")
    L = ctypes.CDLL(b.PEAKS_LIB)
    P, I, LL = ctypes.c_void_p, ctypes.c_int, ctypes.c_longlong
    L.peak_mfma_fp8.argtypes = [I, I, P, P, P]
    L.peak_hbm_read.argtypes = [P, LL, I, P, P]
    L.peak_lds_read.argtypes = [I, I, I, I, P, P, P]
    dev = torch.device("cuda:0")
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        ms = []
        for _ in range(reps):
            a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            z.record()
            torch.cuda.synchronize()
            ms.append(a.elapsed_time(z))
        return ms

    res = {"metric": "peaks", "cus": cus, "device": torch.cuda.get_device_name(dev)}
    # FP8 MFMA: two waves per SIMD, 8 independent 16x16x128 chains each
    blocks, iters = 2 * cus, 20000
    sink = torch.empty(blocks * 4, dtype=torch.float32, device=dev)
    timing = torch.empty(blocks * 8, dtype=torch.int64, device=dev)
    log("[peaks] FP8 MFMA loop")
    for _ in range(20):                        # the clock settles under sustained load
        assert L.peak_mfma_fp8(blocks, iters, P(sink.data_ptr()), P(timing.data_ptr()), stream) == 0
    ms = timed(lambda: L.peak_mfma_fp8(blocks, iters, P(sink.data_ptr()), P(timing.data_ptr()), stream), 10)
    flops = blocks * 4 * iters * 8 * 2.0 * 16 * 16 * 128
    cyc = timing.view(-1, 2)[:, 0].double().mean().item()
    best = min(ms)
    res["fp8_mfma_tflops"] = round(flops / (best * 1e-3) / 1e12, 1)
    res["fp8_mfma_frac_of_spec"] = round(res["fp8_mfma_tflops"] / FP8_PEAK_TFLOPS, 4)
    res["clock_ghz_under_mfma_load"] = round(cyc / (best * 1e-3) / 1e9, 3)
    res["mfma_cycles_per_16x16x128"] = round(cyc / (iters * 8 * 2), 2)   # two waves share a SIMD
    # HBM streaming read of 4 GiB and a 2 GiB device copy
    n = 4 << 30
    buf = torch.empty(n, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    hsink = torch.empty(cus * 8, dtype=torch.int32, device=dev)
    log("[peaks] HBM read")
    ms = timed(lambda: L.peak_hbm_read(P(buf.data_ptr()), n, cus * 8, P(hsink.data_ptr()), stream), 10)
    res["hbm_read_GBs"] = round(n / (min(ms) * 1e-3) / 1e9, 1)
    res["hbm_read_frac_of_spec"] = round(res["hbm_read_GBs"] / HBM_PEAK_GBS, 4)
    del buf
    src = torch.ones(1 << 31, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    log("[peaks] device copy")
    ms = timed(lambda: dst.copy_(src), 10)
    res["copy_read_plus_write_GBs"] = round(2 * (1 << 31) / (min(ms) * 1e-3) / 1e9, 1)
    del src, dst
    # LDS read rates, one workgroup of 8 waves per CU
    iters = 4096
    lsink = torch.empty(cus * 8, dtype=torch.int32, device=dev)
    ltim = torch.empty(cus * 16, dtype=torch.int64, device=dev)
    for tr, name, lane_bytes in ((0, "ds_read_b128", 16), (1, "ds_read_b64_tr_b8", 8)):
        log(f"[peaks] LDS {name}")
        ms = timed(lambda: L.peak_lds_read(cus, 8, iters, tr, P(lsink.data_ptr()), P(ltim.data_ptr()), stream), 5)
        cyc = ltim.view(-1, 2)[:, 0].double().max().item()
        per_cu = 8 * iters * 8 * 64 * lane_bytes
        res[f"lds_{name}_bytes_per_clk_per_cu"] = round(per_cu / cyc, 1)
    # global -> LDS fill rate per CU: the GEMMs' DMA stage loads vs loads to
    # registers + LDS writes, from an L2-resident region and from HBM-sized ones
    L.peak_lds_fill.argtypes = [P, I, I, I, I, I, P, P, P]
    for region, name in ((256 << 10, "l2"), (8 << 20, "hbm")):
        fsrc = torch.ones(cus * region, dtype=torch.uint8, device=dev)
        fsink = torch.empty(cus * 8, dtype=torch.int32, device=dev)
        ftim = torch.empty(cus * 16, dtype=torch.int64, device=dev)
        iters = 256 if name == "l2" else 128
        for dma in (1, 0):
            log(f"[peaks] LDS fill {name} dma={dma}")
            fn = lambda: L.peak_lds_fill(P(fsrc.data_ptr()), cus, 8, region, iters, dma, P(fsink.data_ptr()),
                                         P(ftim.data_ptr()), stream)
            ms = timed(fn, 5)
            cyc = ftim.view(-1, 2)[:, 0].double().max().item()
            per_cu = 8 * iters * 8 * 1024
            res[f"lds_fill_{name}_{'dma' if dma else 'regs'}_bytes_per_clk_per_cu"] = round(per_cu / cyc, 1)
            res[f"lds_fill_{name}_{'dma' if dma else 'regs'}_GBs"] = round(cus * per_cu / (min(ms) * 1e-3) / 1e9, 1)
        del fsrc
    # the grouped GEMMs' MFMA sequence alone (fragments in registers)
    L.peak_mfma_sequence.argtypes = [I, I, I, I, P, P, P]
    for waves, mode, name in ((8, 0, "promote3_schedbarrier"), (8, 1, "promote3"), (8, 2, "accumulate"),
                              (4, 0, "promote3_schedbarrier_1wave"), (4, 2, "accumulate_1wave")):
        steps = 2000
        seq_sink = torch.empty(cus * waves, dtype=torch.float32, device=dev)
        seq_tim = torch.empty(cus * waves * 2, dtype=torch.int64, device=dev)
        log(f"[peaks] MFMA sequence {name}")
        fn = lambda: L.peak_mfma_sequence(cus, waves, steps, mode, P(seq_sink.data_ptr()), P(seq_tim.data_ptr()), stream)
        ms = timed(fn, 5)
        flops = cus * waves * steps * 24 * 2.0 * 16 * 16 * 128
        res[f"mfma_seq_{name}_tflops"] = round(flops / (min(ms) * 1e-3) / 1e12, 1)
    torch.cuda.synchronize()
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default: 50; 300 for decode-sized batches, whose steps take "
                         "~0.1-0.5 ms, so that the timed region is not dominated by its edges)")
    # compute-bound kernels reach their steady clock after about 20 launches
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default="c4b",
                    choices=sorted(gen.CONFIGS) + ["attn_decode", "attn_prefill", "peaks"])
    ap.add_argument("--tokens", type=int, default=0,
                    help="override the workload's token count T (same layer), e.g. 1 or 8 for small "
                         "decode batches of the c1 layer")
    ap.add_argument("--path", default="auto", choices=sorted(moe.PATHS))
    ap.add_argument("--format", default="block128", choices=sorted(moe.FORMATS),
                    help="weight format: 128x128 block-scaled FP8, MXFP8 (E8M0 per 32) or MXFP4")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--event-every", type=int, default=5,
                    help="one instrumented step (per-kernel timing events) per N timed steps, run in "
                         "an untimed pass before the timed region: each event costs a few "
                         "microseconds of device time, so the timed steps are plain calls")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of a HIP graph holding one forward (captured after the warm-up, "
                         "as a serving loop replays it) instead of eager calls")
    ap.add_argument("--flush-mib", type=int, default=0,
                    help="read this many MiB between timed calls (outside the calls' events) so "
                         "that every call reads its weights from HBM; 0: back-to-back steps")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="before the steps, one device-to-device copy of this many MiB "
                         "(a kernel of known traffic for scaling HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the MoE block here is "
              "built for a single MI355X (no sharding across GPUs is built).", file=sys.stderr)
        sys.exit(2)

    if args.workload.startswith("attn"):
        if args.steps is None:
            args.steps = 50
        attn_bench(args)
        return
    if args.workload == "peaks":
        peaks_bench(args)
        return

    cfg = gen.CONFIGS[args.workload]
    log(f"[bench] generating {cfg.name} (T={cfg.T}, d={cfg.layer.d}, f={cfg.layer.f}, "
        f"E={cfg.layer.E}, k={cfg.layer.k})")
    fmt = args.format
    inp = gen.make_inputs(cfg.name, fmt=fmt, T=args.tokens or None)
    dev = torch.device("cuda:0")
    p = moe.device_inputs(inp, dev)
    T, d, f, E, k = inp["T"], inp["d"], inp["f"], inp["E"], inp["k"]
    if args.steps is None:
        args.steps = 300 if T * k <= 32 * E else 50   # decode-sized (the library's auto path rule)
    w_args = (p["W_router"], p["b_router"], k, p["W_gateup"], p["S_gateup"], p["b_gateup"],
              p["W_down"], p["S_down"], p["b_down"])
    ws = torch.empty(moe.workspace_bytes(T, d, f, E, k), dtype=torch.uint8, device=dev)
    out = torch.empty((T, d), dtype=torch.bfloat16, device=dev)
    x = p["x"]

    calibration_copy(args.copy_calibration_mib, dev)

    dbg = moe.forward_debug(x, *w_args, path=args.path, fmt=fmt)
    torch.cuda.synchronize()
    counts = np.diff(dbg["offsets"].cpu().numpy())
    del dbg
    ga = gateup_algorithmic(inp, counts)
    da = down_algorithmic(inp, counts)

    def step(ev=None):
        if ev is None:  # one call of the block, as a user makes it
            moe.forward(x, *w_args, out=out, workspace=ws, path=args.path, fmt=fmt)
            return
        moe.forward_stages("router", "place", x, *w_args, out, ws, path=args.path, fmt=fmt)
        if ev is not None:
            ev[0].record()
        moe.forward_stages("gateup", "gateup", x, *w_args, out, ws, path=args.path, fmt=fmt)
        if ev is not None:
            ev[1].record()
        moe.forward_stages("down", "down", x, *w_args, out, ws, path=args.path, fmt=fmt)
        if ev is not None:
            ev[2].record()
        moe.forward_stages("combine", "combine", x, *w_args, out, ws, path=args.path, fmt=fmt)

    flush = None
    if args.flush_mib > 0:
        flush = torch.ones(args.flush_mib << 18, dtype=torch.float32, device=dev)
        flush_sink = torch.empty((), dtype=torch.float32, device=dev)

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    sampled = sampled_steps(args.steps, args.event_every)
    evs = {i: [torch.cuda.Event(enable_timing=True) for _ in range(3)] for i in sampled}
    # per-kernel times from an untimed pass of instrumented steps
    for i in sampled:
        step(evs[i])
    torch.cuda.synchronize()
    graph = None
    if args.graph:
        # one forward captured for the timed replays
        side = torch.cuda.Stream(dev)
        side.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream(dev).wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        for _ in range(3):
            graph.replay()
        torch.cuda.synchronize()
    calls = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(args.steps)] if flush is not None else None
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    log(f"[bench] timing {args.steps} steps (stage events from {len(sampled)} untimed steps"
        + (f", {args.flush_mib} MiB flush before each)" if flush is not None else ")"))
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        run = graph.replay if graph is not None else step
        if flush is not None:
            flush_sink.copy_(flush.sum())   # untimed read: evicts L2 and the memory-side cache
            calls[i][0].record()
            run()
            calls[i][1].record()
        else:
            run()
    stop.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    gate_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs.values()]))
    down_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs.values()]))
    if flush is not None:
        ms = float(np.mean([a.elapsed_time(b) for a, b in calls]))
    else:
        ms = total_ms / args.steps
    tok_s = T / (ms * 1e-3)

    decode = (args.path == "decode") or (args.path == "auto" and T * k <= 32 * E)
    tkey = args.workload + ("" if fmt == "block128" else "-" + fmt)
    if decode:
        ach = ga["bytes"] / (gate_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": measured_traffic(tkey)}
    else:
        ach = ga["flops"] / (gate_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": FP8_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / FP8_PEAK_TFLOPS, 4),
                "traffic": measured_traffic(tkey)}
    tf = {"block128": "false, false", "mx": "true, false", "mxfp4": "true, true"}[fmt]
    roof["kernel"] = (f"grouped_gemm_dma_kernel<true, 32, 256, {tf}>" if decode else
                      f"grouped_gemm_wide_kernel<true, {tf}>") + \
        " (gate/up + bias + SwiGLU + h quantisation)"
    roof["avg_ms"] = round(gate_ms, 5)
    roof["event_launches"] = len(sampled)
    roof["algorithmic_bytes"] = ga["bytes"]
    roof["algorithmic_flops"] = ga["flops"]

    la = layer_algorithmic(inp, counts)
    if decode:
        layer = {"bound": "hbm", "achieved": round(la["bytes"] / (ms * 1e-3) / 1e9, 1),
                 "peak": HBM_PEAK_GBS, "unit": "GB/s", "algorithmic_bytes": la["bytes"]}
    else:
        layer = {"bound": "mfma", "achieved": round(la["flops"] / (ms * 1e-3) / 1e12, 1),
                 "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s", "algorithmic_flops": la["flops"]}
    layer["frac"] = round(layer["achieved"] / layer["peak"], 4)

    res = {
        "metric": METRIC, "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp8",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: {cfg.layer.name} {cfg.role} T={T} d={d} "
                               f"(real {inp['d_real']}) f={f} E={E} k={k}"
                               + (f" (T overridden from {cfg.T})" if args.tokens else ""),
                   "T": T, "d": d, "f": f, "E": E, "k": k, "path": args.path, "format": fmt,
                   "experts_touched": ga["touched"]},
        "roofline": roof,
        "layer_frac": layer["frac"],
        "layer_roofline": layer,
        "flush_mib": args.flush_mib,
        "graph": bool(args.graph),
        "timed_region_ms": round(total_ms, 3),
        "stages_ms": {"gateup": round(gate_ms, 5), "down": round(down_ms, 5),
                      "rest": round(ms - gate_ms - down_ms, 5)},
        "down_gemm": {"achieved_GBs": round(da["bytes"] / (down_ms * 1e-3) / 1e9, 1),
                      "achieved_TFLOPs": round(da["flops"] / (down_ms * 1e-3) / 1e12, 1)},
        "step_tflops": round((ga["flops"] + da["flops"]) / (ms * 1e-3) / 1e12, 2),
    }
    if not args.no_cpu_baseline:
        log("[bench] CPU oracle baseline")
        res["cpu_baseline"] = cpu_baseline(inp)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
