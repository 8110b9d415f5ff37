"""Benchmark of the MI355X MoE-layer hot path (one GPU).

Default workload (the MegaMoE prefill-shaped layer, the largest single-GPU
layer of the pages' regimes): 8192 tokens, hidden 7168, intermediate 2048, 256
experts all local, topK 8, plus one shared expert over all tokens, MXFP8 E4M3
weights with E8M0 scales, bf16 activations N(0,1), fp32 softmax gate weights.
One step is one mega_moe call: routing -> gather + MX quantization -> GMM1 +
SwiGLU + MX requantization -> GMM2 -> shared expert -> weighted combine -> bf16
Y. Inputs and weights are resident in HBM before the timed region (weights are
generated on the GPU with a seeded generator and quantized by the library's own
MX quantizer, untimed).

Prints one JSON line: MoE layer tokens/s, the roofline of the dominant kernel
(its duration measured with HIP events that the library records on its stream
at every stage boundary during the timed steps) with both its MXFP8 MFMA and its
HBM fraction, and the CPU oracle timed on a bounded token sample of the same
workload on this host.

    python bench.py [--steps K] [--warmup W] [--config prefill|decode|skewed|tiny|routing]
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.txt")
COPY_BYTES = 1 << 30        # the plain copy measured for the counter calibration
MXFP8_PEAK_TFLOPS = 5000.0  # MI355X dense FP8 / MXFP8 MFMA
RIDGE = MXFP8_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def library_weights(torch, rp, moe_inputs, cfg, n_experts, shared, fp4=False):
    """Expert weights made on the GPU from the bf16 masters and MX-quantized by the library:
    FP8 of the layer's format, or MXFP4 (codes two a byte) with fp4."""
    t1, t2 = ("sw1", "sw2") if shared else ("w1", "w2")
    h, i = cfg.hidden, cfg.inter
    q = rp.QUANT_MXFP4 if fp4 else rp.QUANT_E4M3 if cfg.fmt == "e4m3" else rp.QUANT_E5M2
    cb = 2 if fp4 else 1   # elements per code byte
    w1q = torch.empty((n_experts, 2 * i, h // cb), dtype=torch.uint8, device="cuda")
    w1s = torch.empty((n_experts, 2 * i, h // 32), dtype=torch.uint8, device="cuda")
    w2q = torch.empty((n_experts, h, i // cb), dtype=torch.uint8, device="cuda")
    w2s = torch.empty((n_experts, h, i // 32), dtype=torch.uint8, device="cuda")
    for e in range(n_experts):
        c, s = rp.mx_quantize(moe_inputs.weight_master(cfg, t1, e, device="cuda"), q)
        w1q[e].copy_(c); w1s[e].copy_(s)
        c, s = rp.mx_quantize(moe_inputs.weight_master(cfg, t2, e, device="cuda"), q)
        w2q[e].copy_(c); w2s[e].copy_(s)
    return w1q, w1s, w2q, w2s


def layer_work(cfg, ids, fp4=False):
    """Algorithmic bytes and flops per launch of the two grouped GEMMs and the combine:
    GMM1 reads the touched experts' W1 (codes + 1/32 scales; half a byte a code for MXFP4
    weights) and the quantized rows, and writes the requantized rows; GMM2 reads W2 and
    those rows and writes O, bf16 rows (the default combine mode: each expert's output
    reaches the combine as BF16); the combine reads O (and the shared experts' O) and
    writes bf16 Y."""
    h, i, f = cfg.hidden, cfg.inter, cfg.flat
    touched = int(np.unique(ids).size)
    sc = 1.0 + 1.0 / 32.0
    wsc = (0.5 if fp4 else 1.0) + 1.0 / 32.0
    gmm1_bytes = touched * 2 * i * h * wsc + f * h * sc + f * i * sc
    gmm2_bytes = touched * h * i * wsc + f * i * sc + f * h * 2
    combine_bytes = f * h * 2 + cfg.shared * cfg.tokens * h * 2 + cfg.tokens * h * 2
    gmm1_flops = 2.0 * f * h * 2 * i
    gmm2_flops = 2.0 * f * i * h
    if cfg.shared:
        n = cfg.tokens
        gmm1_bytes_s = cfg.shared * (2 * i * h * wsc + n * h * sc + n * i * sc)
        gmm2_bytes_s = cfg.shared * (h * i * wsc + n * i * sc + n * h * 2)
        shared1 = dict(bytes=gmm1_bytes_s, flops=cfg.shared * 4.0 * n * h * i)
        shared2 = dict(bytes=gmm2_bytes_s, flops=cfg.shared * 2.0 * n * h * i)
    else:
        shared1 = shared2 = dict(bytes=0.0, flops=0.0)
    shared = dict(bytes=shared1["bytes"] + shared2["bytes"], flops=shared1["flops"] + shared2["flops"])
    return dict(touched=touched, gmm1=dict(bytes=gmm1_bytes, flops=gmm1_flops),
                gmm2=dict(bytes=gmm2_bytes, flops=gmm2_flops), combine=dict(bytes=combine_bytes, flops=0.0),
                shared=shared, shared1=shared1, shared2=shared2)


def shared_folded(cfg):
    """Whether the library runs the shared expert inside the routed experts' GEMM launches:
    one shared expert, and the LDS-streaming GEMMs for the routed experts (more than 128
    rows an expert on average, K steps of both GEMMs a multiple of 4) and for the shared
    expert (more than 128 tokens). The GMM stage times then include the shared expert."""
    h, i = cfg.hidden, cfg.inter
    steps4 = (h // 128) % 4 == 0 and (i // 128) % 4 == 0
    return cfg.shared == 1 and steps4 and cfg.flat / cfg.experts > 128 and cfg.tokens > 128


def kernel_source_hash():
    """sha256 over the library's kernel sources: a measured traffic figure is valid only
    for the sources it was measured on."""
    import hashlib
    h = hashlib.sha256()
    src = os.path.join(ROOT, "routing_permute_mxfp8_amd", "csrc")
    for name in sorted(os.listdir(src)):
        if name.endswith((".hip", ".h", ".cpp")):
            with open(os.path.join(src, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` on `workload` from the committed rocprofv3 counter
    summary: FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of the kernel, each scaled by
    the bytes a plain copy of COPY_BYTES moves per KiB that counter reports for it.
    None if there is no figure or the kernel sources changed since it was taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    vals, rows = {}, {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            parts = line.split()
            if not parts or parts[0].startswith("#"):
                continue
            if parts[0] == "kernel" and len(parts) >= 9:
                rows[(parts[1], parts[2])] = dict(zip(parts[3::2], parts[4::2]))
            elif len(parts) == 2:
                vals[parts[0]] = float(parts[1])
    row = rows.get((kernel, workload))
    if row is None or row.get("source") != kernel_source_hash():
        return None
    if not vals.get("copy_fetch_kib") or not vals.get("copy_write_kib"):
        return None
    fetch = float(row["fetch_kib"]) * vals["copy_bytes"] / vals["copy_fetch_kib"]
    write = float(row["write_kib"]) * vals["copy_bytes"] / vals["copy_write_kib"]
    return round(fetch + write)


def calibrate_copy(args, torch):
    """A plain device copy of COPY_BYTES (read COPY_BYTES, write COPY_BYTES), repeated, for
    the counter calibration of measured_traffic (run under rocprofv3 --pmc)."""
    x = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps):
        y.copy_(x)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / max(args.steps, 1)
    print(json.dumps(dict(calibration="copy", bytes_read=COPY_BYTES, bytes_written=COPY_BYTES, copies=args.steps,
                          ms_per_copy=round(ms, 4), copy_gbs=round(2 * COPY_BYTES / (ms * 1e-3) / 1e9, 1),
                          source=kernel_source_hash())), flush=True)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def percentiles(xs):
    a = np.sort(np.asarray(xs, dtype=np.float64))
    return dict(median=round(float(np.median(a)), 5), p10=round(float(np.percentile(a, 10)), 5),
                p90=round(float(np.percentile(a, 90)), 5))


def measure_peaks(torch, rp, nbytes=1 << 30, reps=5):
    """Measured peaks of this GPU with the library's probes: a streaming read and a copy
    of nbytes (16-byte lanes), and the FP8 block-scaled MFMA loop. Each median of reps."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        return float(np.median(ts))

    read_ms = timed(lambda: rp.probe_stream(src))
    copy_ms = timed(lambda: rp.probe_stream(src, dst, copy=True))
    out, flops = rp.probe_mfma(2000)
    mfma_ms = timed(lambda: rp.probe_mfma(2000, out))
    del src, dst
    torch.cuda.empty_cache()
    return dict(read_gbs=round(nbytes / (read_ms * 1e-3) / 1e9, 1),
                copy_gbs=round(2 * nbytes / (copy_ms * 1e-3) / 1e9, 1),
                mfma_fp8_tflops=round(flops / (mfma_ms * 1e-3) / 1e12, 1),
                note="library probes (peaks.hip): 1 GiB streaming read, 1 GiB copy, FP8 scaled-MFMA loop")


def roofline_entry(name, ms, work):
    """The kernel against the roofline that bounds it (MFMA above the ridge intensity,
    HBM below), with both fractions: mfma_frac = algorithmic MXFP8 flops / time / the
    MXFP8 peak, hbm_frac = algorithmic bytes / time / the HBM peak."""
    intensity = work["flops"] / max(work["bytes"], 1.0)
    tflops = work["flops"] / (ms * 1e-3) / 1e12
    gbs = work["bytes"] / (ms * 1e-3) / 1e9
    both = dict(mfma_tflops=round(tflops, 1), mfma_frac=round(tflops / MXFP8_PEAK_TFLOPS, 4),
                hbm_gbs=round(gbs, 1), hbm_frac=round(gbs / HBM_PEAK_GBS, 4),
                intensity_flop_per_byte=round(intensity, 1), flops_per_launch=work["flops"],
                bytes_per_launch=work["bytes"])
    if intensity >= RIDGE:
        return dict(kernel=name, bound="mfma", achieved=round(tflops, 2), peak=MXFP8_PEAK_TFLOPS,
                    unit="TFLOP/s", frac=round(tflops / MXFP8_PEAK_TFLOPS, 4), traffic=None,
                    algorithmic_per_launch=work["flops"], avg_launch_ms=round(ms, 5), **both)
    return dict(kernel=name, bound="hbm", achieved=round(gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                frac=round(gbs / HBM_PEAK_GBS, 4), traffic=None, algorithmic_per_launch=work["bytes"],
                avg_launch_ms=round(ms, 5), **both)


def cpu_baseline_mega(cfg, ids, x_cpu, w, sample_tokens, torch, moe_inputs, fp4=False):
    """The oracle (CPU, float64) on a bounded token sample: tokens/s of the per-token layer
    (MXFP4 weights with fp4)."""
    from concurrent.futures import ThreadPoolExecutor

    from oracle import moe, mxfp
    wfmt = "e2m1" if fp4 else cfg.fmt

    def q(m):
        c, sc = mxfp.quantize(m, wfmt)
        return (mxfp.pack_fp4(c) if fp4 else c), sc
    rng = np.random.default_rng(123)
    tokens = rng.choice(cfg.tokens, size=sample_tokens, replace=False)
    experts = sorted(set(int(e) for e in ids[tokens].reshape(-1)))
    # inputs of the oracle: the sampled experts' weights, quantized by the oracle (untimed,
    # in threads: it is input preparation, not the timed oracle)
    masters = {("w", e): (moe_inputs.weight_master(cfg, "w1", e, device="cuda").cpu(),
                          moe_inputs.weight_master(cfg, "w2", e, device="cuda").cpu()) for e in experts}
    for s in range(cfg.shared):
        masters[("s", s)] = (moe_inputs.weight_master(cfg, "sw1", s, device="cuda").cpu(),
                             moe_inputs.weight_master(cfg, "sw2", s, device="cuda").cpu())

    def prep(key):
        m1, m2 = masters[key]
        return key, (*q(m1.double().numpy()), *q(m2.double().numpy()))
    with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
        done = dict(ex.map(prep, list(masters)))
    cache = {e: done[("w", e)] for e in experts}
    shared = [done[("s", s)] for s in range(cfg.shared)]
    x = x_cpu.double().numpy()
    t0 = time.perf_counter()
    moe.per_token(x, ids, w, lambda e: cache[e], cfg.fmt, tokens, shared=shared, wfmt=wfmt)
    dt = time.perf_counter() - t0
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # threadpoolctl missing: numpy's elementwise work is single-threaded
        cores = 1
    return dict(value=round(sample_tokens / dt, 4), unit="tokens/s", cores=int(cores), kind="oracle",
                sample=f"{sample_tokens} tokens x topK {cfg.topk} experts ({len(experts)} distinct"
                       f"{', plus shared' if cfg.shared else ''}), per-token float64 oracle, {dt:.1f} s",
                seconds=round(dt, 2), host_cpus=os.cpu_count(), cpu_model=cpu_model())


def bench_mega(args, torch, rp, moe_inputs):
    cfg = moe_inputs.config(args.config)
    ids = moe_inputs.expert_ids(cfg)
    x_cpu = moe_inputs.activations(cfg)
    w = moe_inputs.gate_weights(cfg)
    log(f"[bench] {cfg.name}: generating weights on the GPU")
    fp4 = args.weight_dtype == "mxfp4"
    weights = library_weights(torch, rp, moe_inputs, cfg, cfg.experts, shared=False, fp4=fp4)
    shared = library_weights(torch, rp, moe_inputs, cfg, cfg.shared, shared=True, fp4=fp4) if cfg.shared else None
    wf = rp.WEIGHTS_PACKED if args.weights == "packed" else rp.WEIGHTS_ND
    if wf == rp.WEIGHTS_PACKED:   # one-time conversion to the MFMA-native layout, untimed
        weights = (*rp.pack_weights(weights[0], weights[1], fp4), *rp.pack_weights(weights[2], weights[3], fp4))
        if shared is not None:
            shared = (*rp.pack_weights(shared[0], shared[1], fp4), *rp.pack_weights(shared[2], shared[3], fp4))
    wd = rp.FP4_E2M1 if fp4 else 0
    x = x_cpu.cuda()
    ids_d = torch.from_numpy(ids).cuda()
    w_d = torch.from_numpy(w).cuda()
    fmt = rp.FP8_E4M3 if cfg.fmt == "e4m3" else rp.FP8_E5M2
    if fp4 and fmt != rp.FP8_E4M3:
        raise SystemExit("MXFP4 weights (A8W4-FP) take E4M3 activations")
    nbytes = rp.mega_moe_workspace_bytes(x, ids_d, w_d, *weights, shared=shared, quant_out_dtype=fmt, weight_format=wf,
                                         weight_dtype=wd)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        rp.mega_moe(x, ids_d, w_d, *weights, shared=shared, quant_out_dtype=fmt, workspace=ws, weight_format=wf,
                    weight_dtype=wd)
    torch.cuda.synchronize()
    # Stage events only where the stage times are read (GMM1, GMM2, shared experts +
    # combine): a timed event record costs a few microseconds of GPU time, inside the
    # timed region.
    timed = {0, 2, 3, 4, 6}
    evs = [[torch.cuda.Event(enable_timing=True) if j in timed else None for j in range(rp.MEGA_STAGE_EVENTS)]
           for _ in range(args.steps)]
    for st in evs:
        for ev in st:
            if ev is not None:
                ev.record()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} steps")
    t0 = time.perf_counter()
    start.record()
    for k in range(args.steps):
        rp.mega_moe(x, ids_d, w_d, *weights, shared=shared, quant_out_dtype=fmt, workspace=ws, stage_events=evs[k],
                    weight_format=wf, weight_dtype=wd)
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = start.elapsed_time(end) / args.steps
    def between(j0, j1):
        return float(np.mean([evs[k][j0].elapsed_time(evs[k][j1]) for k in range(args.steps)]))
    stage_ms = {"gmm1_swiglu_quant": between(2, 3), "gmm2": between(3, 4), "shared_experts_and_combine": between(4, 6)}
    stage_ms["routing_and_permute"] = between(0, 2)
    step_ms = [evs[k][0].elapsed_time(evs[k][6]) for k in range(args.steps)]
    work = layer_work(cfg, ids, fp4)
    folded = shared_folded(cfg)
    w1, w2 = work["gmm1"], work["gmm2"]
    if folded:   # the shared expert runs inside the GMM stages
        w1 = dict(bytes=w1["bytes"] + work["shared1"]["bytes"], flops=w1["flops"] + work["shared1"]["flops"])
        w2 = dict(bytes=w2["bytes"] + work["shared2"]["bytes"], flops=w2["flops"] + work["shared2"]["flops"])
    roof = {"gmm1_swiglu_quant": roofline_entry("gmm1_swiglu_kernel", stage_ms["gmm1_swiglu_quant"], w1),
            "gmm2": roofline_entry("gmm2_kernel", stage_ms["gmm2"], w2)}
    if folded:
        for r in roof.values():
            r["includes_shared_expert"] = True
    dominant = max(roof, key=lambda k: stage_ms[k])
    roofline = dict(roof[dominant])
    roofline["traffic"] = measured_traffic(roofline["kernel"], cfg.name + ("-mxfp4" if fp4 else ""))
    peaks = measure_peaks(torch, rp)
    ref = peaks["mfma_fp8_tflops"] if roofline["bound"] == "mfma" else peaks["read_gbs"]
    roofline["measured_peak"] = ref
    roofline["frac_of_measured"] = round(roofline["achieved"] / ref, 4)
    roofline["other"] = {k: v for k, v in roof.items() if k != dominant}
    for v in roofline["other"].values():
        v["traffic"] = measured_traffic(v["kernel"], cfg.name + ("-mxfp4" if fp4 else ""))
    total_bytes = work["gmm1"]["bytes"] + work["gmm2"]["bytes"] + work["combine"]["bytes"] + work["shared"]["bytes"]
    total_flops = work["gmm1"]["flops"] + work["gmm2"]["flops"] + work["shared"]["flops"]
    out = dict(metric="MoE layer tokens/s", value=round(cfg.tokens / (ms * 1e-3), 1), unit="tokens/s", n_gpus=1,
               steps=args.steps, warmup=args.warmup, ms_per_step=round(ms, 5), higher_is_better=True,
               scaling="weak", vs_baseline=None,
               dtype=("mxfp8 activations x mxfp4 e2m1 weights (e8m0 scales, fp32 accumulate)" if fp4 else
                      "mxfp8 (fp8 e4m3/e5m2 x e8m0 scales, fp32 accumulate)"),
               data=f"synthetic (seeded; weights N(0,1/sqrt(fan_in)) quantized to {'MXFP4' if fp4 else 'MXFP8'} "
                    "on the GPU)",
               config=dict(workload=f"{cfg.name}: {cfg.tokens} tokens, hidden {cfg.hidden}, inter {cfg.inter}, "
                                    f"{cfg.experts} experts, topK {cfg.topk}, shared {cfg.shared}, {cfg.fmt}"
                                    + (", A8W4-FP (MXFP4 weights)" if fp4 else ""),
                           weight_dtype=args.weight_dtype,
                           tokens=cfg.tokens, hidden=cfg.hidden, inter=cfg.inter, experts=cfg.experts,
                           topk=cfg.topk, shared=cfg.shared, fmt=cfg.fmt, touched_experts=work["touched"],
                           weight_layout=args.weights, combine_comm_mode=0),
               roofline=roofline,
               layer=dict(algorithmic_bytes=total_bytes, flops=total_flops,
                          hbm_frac=round(total_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                          mfma_frac=round(total_flops / (ms * 1e-3) / 1e12 / MXFP8_PEAK_TFLOPS, 4)),
               stages_ms={k: round(v, 5) for k, v in stage_ms.items()},
               measured_peaks=peaks,
               step_ms=percentiles(step_ms),
               wall_ms_per_step=round(wall * 1e3 / args.steps, 5))
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle)")
        out["cpu_baseline"] = cpu_baseline_mega(cfg, ids, x_cpu, w, args.cpu_sample or (1 if cfg.shared else 2),
                                                torch, moe_inputs, fp4)
    else:
        out["cpu_baseline"] = None
    return out


def bench_routing(args, torch, rp, moe_inputs):
    """moe_init_routing on the routing workload. Each timed call is bracketed by its own
    events, and a streaming read of a 512 MB scratch buffer between calls evicts x from
    the 256 MB MALL so that it is read from HBM (a read, not a write, leaves no dirty
    lines to drain during the call; the flush is outside the events)."""
    cfg = moe_inputs.config("routing")
    ids = moe_inputs.expert_ids(cfg)
    x_cpu = moe_inputs.activations(cfg)
    x = x_cpu.cuda()
    ids_d = torch.from_numpy(ids).cuda()
    s, e = cfg.active_range
    q = rp.QUANT_E4M3
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    for _ in range(args.warmup):
        rp.init_routing(x, ids_d, cfg.experts, (s, e), q, 1, 1)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    flush.fill_(0)
    for a, b in evs:
        rp.probe_stream(flush, fill_caches=True)
        a.record()
        rp.init_routing(x, ids_d, cfg.experts, (s, e), q, 1, 1)
        b.record()
    torch.cuda.synchronize()
    times = [a.elapsed_time(b) for a, b in evs]
    ms = float(np.mean(times))
    in_range = (ids >= s) & (ids < e)
    avail = int(in_range.sum())
    distinct = int(in_range.any(axis=1).sum())
    h = cfg.hidden
    alg = distinct * 2 * h + avail * (h + h // 32) + cfg.flat * 8 + (e - s) * 8
    achieved = alg / (ms * 1e-3) / 1e9
    peaks = measure_peaks(torch, rp)
    out = dict(metric="MoeInitRoutingV3 rows/s", value=round(avail / (ms * 1e-3), 1), unit="rows/s", n_gpus=1,
               steps=args.steps, warmup=args.warmup, ms_per_step=round(ms, 5), higher_is_better=True,
               scaling="weak", vs_baseline=None, dtype="u8 (fp8 e4m3 codes + e8m0)", data="synthetic",
               config=dict(workload=f"routing: {cfg.tokens} tokens x {h}, topK {cfg.topk}, {cfg.experts} experts, "
                                    f"active [{s},{e}), scatter index, count histogram, MXFP8 E4M3",
                           active_rows=avail, distinct_tokens=distinct),
               roofline=dict(kernel="moe_init_routing", bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS,
                             unit="GB/s", frac=round(achieved / HBM_PEAK_GBS, 4),
                             traffic=measured_traffic("moe_init_routing", "routing"), algorithmic_per_launch=alg,
                             avg_launch_ms=round(ms, 5),
                             kernels="route_count_block, route_scatter_block, permute_mx_kernel (one call)",
                             measured_peak=peaks["copy_gbs"],
                             frac_of_measured=round(achieved / peaks["copy_gbs"], 4)),
               step_ms=percentiles(times), measured_peaks=peaks, mall_flush="512 MB streaming read between calls")
    out["roofline"]["target_70pct_ms"] = round(alg / (0.7 * HBM_PEAK_GBS * 1e9) * 1e3, 5)
    out["roofline"]["measured_copy_ceiling_ms"] = round(alg / (peaks["copy_gbs"] * 1e9) * 1e3, 5)
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle)")
        out["cpu_baseline"] = cpu_baseline_routing(cfg, ids, x_cpu, avail, args.cpu_sample or 2048)
    else:
        out["cpu_baseline"] = None
    return out


def cpu_baseline_routing(cfg, ids, x_cpu, avail, sample_rows):
    """The oracle (CPU, float64) on the routing workload: the whole routing (stable sort,
    inverse, histogram, active range) on every id, and the quantized gather on a bounded
    sample of the active rows, scaled to all of them. Timed single-threaded (numpy's
    element-wise work is single-threaded; BLAS is not used), rows/s of the whole call."""
    from oracle import routing
    try:
        from threadpoolctl import threadpool_limits
    except Exception:  # threadpoolctl missing: nothing to limit
        threadpool_limits = None
    s, e = cfg.active_range
    x = x_cpu.double().numpy()
    ctx = threadpool_limits(limits=1) if threadpool_limits else None
    if ctx is not None:
        ctx.__enter__()
    try:
        t0 = time.perf_counter()
        r = routing.init_routing(ids, cfg.experts, (s, e), 1, 1)
        t_route = time.perf_counter() - t0
        n = min(sample_rows, r["avail"])
        t0 = time.perf_counter()
        routing.gather_rows(x, r["sorted_row_idx"], cfg.topk, 3, r["active_start"], n)
        t_gather = time.perf_counter() - t0
    finally:
        if ctx is not None:
            ctx.__exit__(None, None, None)
    total = t_route + t_gather * (avail / max(n, 1))
    out = dict(value=round(avail / total, 1), unit="rows/s", cores=1, kind="oracle",
               sample=f"routing of all {cfg.flat} ids ({t_route:.2f} s) + quantized gather of {n} of the "
                      f"{avail} active rows ({t_gather:.2f} s), scaled to all rows; float64, single thread",
               seconds=round(t_route + t_gather, 2), host_cpus=os.cpu_count(), cpu_model=cpu_model())
    # all cores: the gather's rows split over threads (numpy's array work releases the
    # GIL; each thread takes a contiguous slice of the sample), the routing pass as above
    # (one numpy sort)
    from concurrent.futures import ThreadPoolExecutor
    threads = max(1, min(16, os.cpu_count() or 1))
    m = min(n * threads, r["avail"])
    step = (m + threads - 1) // threads
    parts = [(r["active_start"] + i, min(step, m - i)) for i in range(0, m, step)]
    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(lambda q: routing.gather_rows(x, r["sorted_row_idx"], cfg.topk, 3, q[0], q[1]), parts))
    t_mt = time.perf_counter() - t0
    total_mt = t_route + t_mt * (avail / max(m, 1))
    out["all_cores"] = dict(value=round(avail / total_mt, 1), unit="rows/s", cores=threads,
                            sample=f"routing as above + quantized gather of {m} active rows in {threads} "
                                   f"threads ({t_mt:.2f} s), scaled to all rows",
                            seconds=round(t_mt, 2))
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="prefill", choices=["tiny", "decode", "prefill", "skewed", "routing"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=None, help="tokens in the CPU oracle sample")
    ap.add_argument("--weight-dtype", default="fp8", choices=["fp8", "mxfp4"],
                    help="expert weights: MXFP8 (A8W8-FP, the default) or MXFP4 (A8W4-FP)")
    ap.add_argument("--weights", default="packed", choices=["packed", "nd"],
                    help="weight layout: the library's MFMA-native packed layout or the pages' ND layout")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy --steps times (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}): the library has no multi-GPU "
              "path (the layer would shard by experts, one expert range per GPU)", file=sys.stderr)
        sys.exit(2)
    import torch
    if args.calibrate_copy:
        calibrate_copy(args, torch)
        return
    import moe_inputs
    import routing_permute_mxfp8_amd as rp
    rp.load()
    if args.config == "routing":
        out = bench_routing(args, torch, rp, moe_inputs)
    else:
        out = bench_mega(args, torch, rp, moe_inputs)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
