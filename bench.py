"""Benchmark of the deformable attention core on one MI355X.

One step = one pass of the whole hot path over one batch: msda_forward, then
msda_backward (binning + tile-owner grad_value kernels and the location/weight
gradient kernel),
on the 800x1333 encoder training workload (B=4, M=8, D=32, L=4 levels
(100,167),(50,84),(25,42),(13,21), K=4, Nq=Nv=22223, offsets N(0, 8 px),
fp32). Inputs are synthetic (seeded), resident in HBM before timing starts.

Prints ONE JSON line: points/s over the K timed steps (points =
B*Nq*M*L*K per step), the roofline of the dominant kernel measured live with HIP
events on the launch stream, the forward and the backward timed one call at a
time warm and cold (inputs evicted from the caches by a 512 MiB write before
each call; median, p10, p90), and the CPU oracle's rate on the host (a bounded
sample of the same workload).

With --frontend fused the step is msda_forward_fused + msda_backward_fused on
the same workload: the kernels take the raw reference points, pixel offsets
and attention logits and form the locations and softmax weights themselves,
and the backward returns the offset, reference-point and logit gradients.

With --frontend layer the step is the whole MSDeformAttn layer,
msda_layer_forward + msda_layer_backward: the value, offset, logit and output
projections on the matrix cores around the fused core, with every input and
parameter gradient. The GEMMs compute to fp32 accuracy as six bf16 products of
three-term operand splits, so the roofline is the matrix-core one of the
dominant GEMM against the bf16 dense peak over six (2500 / 6 TFLOP/s).

With --frontend dcn the step is the grouped single-level aggregation
(DCNv3), msda_dcn_forward + msda_dcn_backward, on a DCNv3 workload
(default dcnv3_stage2: the stride-8 stage of the 800x1333 input, 100x167
pixels, 8 groups of 16 channels, 3x3 grid).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                       [--workload NAME] [--frontend core|fused|layer|dcn]
                       [--no-directions]
       python bench.py --calibrate-copy MIB   (a plain copy-like kernel of known size,
                                               run under the counter profiler to scale
                                               its byte counters)
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0   # MI355X HBM3E, published
MFMA_F32_PEAK_TFLOPS = 157.3   # MI355X dense fp32 matrix, published
MFMA_BF16_PEAK_TFLOPS = 2500.0   # dense bf16 matrix peak
# the layer's GEMMs run each fp32 product as six bf16 products of three-term
# splits (fp32 accuracy): their ceiling is the bf16 peak over six
SPLIT_PRODUCTS = 6
METRIC = "sampled points/sec (B·Nq·M·L·K) fwd+bwd; achieved HBM GB/s vs peak"


def fused_locations(x):
    """The fused front-end's single-precision locations: reference point plus
    offset over the level's (W, H), the quotient and the sum each rounded."""
    ref, off = x["reference_points_levels"], x["sampling_offsets"]
    wh = np.array([[s_[1], s_[0]] for s_ in x["spatial_shapes"]], np.float32)   # [L, 2] (W, H)
    q = (off / wh[None, None, None, :, None, :]).astype(np.float32)
    return (ref[:, :, None, :, None, :] + q).astype(np.float32)


def touched_value_rows(w, x, loc=None):
    """(b, pixel, head) value rows that some sample's inside-the-level corner
    reads, counted from the inputs: the rows a gather must bring in at least
    once (all of them on the encoder workloads; about a third on the decoder,
    whose 300 queries sample a small part of the pyramid). The pixel
    coordinates are formed as the kernels form them (single-precision
    u * W - 0.5)."""
    loc = x["sampling_locations"] if loc is None else loc
    B, Nq, M, L, K, _ = loc.shape
    shapes, lsi = x["spatial_shapes"], x["level_start_index"]
    seen = np.zeros((B, w.Nv, M), bool)
    bi = np.arange(B)[:, None, None, None]
    mi = np.arange(M)[None, None, :, None]
    for l in range(L):
        H, W = int(shapes[l][0]), int(shapes[l][1])
        px = (loc[:, :, :, l, :, 0].astype(np.float32) * np.float32(W) - np.float32(0.5))
        py = (loc[:, :, :, l, :, 1].astype(np.float32) * np.float32(H) - np.float32(0.5))
        x0 = np.floor(px).astype(np.int64)
        y0 = np.floor(py).astype(np.int64)
        for dy in (0, 1):
            for dx in (0, 1):
                xc, yc = x0 + dx, y0 + dy
                ok = (xc >= 0) & (xc < W) & (yc >= 0) & (yc < H)
                row = int(lsi[l]) + np.where(ok, yc * W + xc, 0)
                bb, mm, rr = np.broadcast_arrays(bi, mi, row)
                seen[bb[ok], rr[ok], mm[ok]] = True
    return int(seen.sum())


def algorithmic_bytes(w, value_bytes_per_elem=4, fused=False, point_bytes=12, grad_value_bytes=4,
                      touched_rows=None):
    """Compulsory bytes of each launch (each input read once, each output
    written once). Per sampled point: location 8 B + weight 4 B (+ their
    gradients 8 B + 4 B in the backward); fused: offset 8 B + logit 4 B (+
    their gradients), the same count. Per (b,q,m): D*4 B of output (or
    upstream gradient). Per value row touched by some sample: D elements read
    once (touched_rows; every row if not given); per value element: grad_value
    written once in the backward (all of it: untouched rows are written as
    zeros). Fused also reads a reference point of 8 B per (b,q,l) (and writes
    its gradient in the backward)."""
    P = w.points
    T = w.B * w.num_queries * w.M
    V = w.B * w.Nv * w.M * w.D
    Vr = V if touched_rows is None else touched_rows * w.D
    R = w.B * w.num_queries * w.L * 8 if fused else 0
    pb, gb = point_bytes, grad_value_bytes
    fwd = Vr * value_bytes_per_elem + P * pb + T * w.D * 4 + R
    # location/weight gradients: value, locations, weights, upstream gradient
    # in; their gradients (12 B per point) out
    bwd_point = Vr * value_bytes_per_elem + P * pb + T * w.D * 4 + P * 12 + 2 * R
    # grad_value: locations, weights, upstream gradient in; grad_value out
    bwd_value = P * pb + T * w.D * 4 + V * gb + R
    # the whole backward reads each input once and writes each gradient once
    bwd = Vr * value_bytes_per_elem + P * pb + T * w.D * 4 + V * gb + P * 12 + 2 * R
    return {"forward": fwd, "bwd_point": bwd_point, "bwd_value": bwd_value, "backward": bwd,
            "step": fwd + bwd}


KERNEL_NAMES = {
    "core": ("msda_fwd_kernel", "msda_bwd_point_kernel", "msda_bin_kernel+msda_tile_kernel"),
    "dcn": ("msda_fwd_kernel<dcn>", "msda_bwd_point_kernel<dcn>",
            "msda_bin_kernel<dcn>+msda_tile_kernel"),
    "fused": ("msda_fwd_kernel<fused>",
              "msda_softmax_stats_kernel+msda_bwd_point_kernel<fused>+msda_ref_grad_kernel",
              "msda_softmax_stats_kernel+msda_bin_kernel<fused>+msda_tile_kernel"),
}

KERNEL_SOURCE = os.path.join(ROOT, "scale_deformable_attention_amd", "csrc", "msda.hip")

# The library's choice of forward kernel for the core and fused front-ends: the
# variant that reads the coarsest levels from LDS (msda_fwd_staged_kernel) for
# planes of at least 2048 queries and head rows of 64 or 128 bytes, when the
# coarsest level of a pyramid with Nv pixels over L levels, each halving both
# sides, 3 Nv / (4^L - 1) pixels, fits with one more row in 36 KB.
STAGE_BYTES, STAGED_MIN_QUERIES = 36 * 1024, 2048


def forward_kernel(w, value_bytes_per_elem, fused=False):
    head = w.D * value_bytes_per_elem
    coarsest = 3.0 * w.Nv / (4.0 ** w.L - 1.0)
    staged = (head in (64, 128) and w.num_queries >= STAGED_MIN_QUERIES and w.L * w.K > 0
              and (coarsest + 1.0) * head <= STAGE_BYTES)
    name = "msda_fwd_staged_kernel" if staged else "msda_fwd_kernel"
    return name + ("<fused>" if fused else "")


def source_digest():
    with open(KERNEL_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def read_traffic(workload):
    """Per-dispatch HBM-side byte counters of each kernel, from the committed
    counter summary for this workload (profiles/msda_kernels_<workload>_traffic.txt,
    with <workload> followed by _fused for the fused front-end).

    The summary holds FETCH_SIZE and WRITE_SIZE (KiB per dispatch, averaged over
    the dispatches of one run) for every kernel, the same two counters for the
    calibration copy kernel with its known byte counts, and the digest of the
    kernel source the counters were taken with. Returns {kernel: bytes per
    dispatch}, or None if the file is missing or the kernels have changed since."""
    path = os.path.join(ROOT, "profiles", f"msda_kernels_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    kern, calib, digest = {}, None, None
    with open(path) as f:
        for line in f:
            t = line.split()
            if not t or t[0].startswith("#"):
                continue
            if t[0] == "source_sha256":
                digest = t[1]
            elif t[0] == "copy":       # copy <read bytes> <written bytes> <FETCH KiB> <WRITE KiB>
                calib = tuple(float(v) for v in t[1:5])
            elif t[0] == "kernel":     # kernel <name> <FETCH KiB> <WRITE KiB> <dispatches>
                kern[t[1]] = (float(t[2]), float(t[3]))
    if digest != source_digest() or calib is None:
        return None
    f_read = calib[0] / (calib[2] * 1024.0)
    f_write = calib[1] / (calib[3] * 1024.0)
    return {k: fk * 1024.0 * f_read + wk * 1024.0 * f_write for k, (fk, wk) in kern.items()}


def calibrate_copy(mib):
    """Launch a plain elementwise kernel (dst = -src, fp32) over mib MiB five
    times: it reads and writes exactly mib MiB each, so its FETCH_SIZE and
    WRITE_SIZE readings give the counters' scale."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(5):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "neg fp32", "bytes_read": n * 4, "bytes_written": n * 4,
                      "launches": 5}), flush=True)


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(w, x, budget_s, fused=False):
    """The oracle as it stands (plain C, one thread per call, double
    accumulation) timed on a bounded sample of the same workload: whole batch
    entries, forward + backward, first on one thread, then on every host
    thread. For the second leg a batch entry's queries are split into one
    slice per thread, each thread runs the oracle's forward and backward on
    its slice (ctypes releases the interpreter lock during each call) and the
    slices' partial grad_value sums are added afterwards (inside the timing).
    Each leg runs batch entries until it has used half the budget."""
    import threading
    import oracle
    fwd, bwd = (oracle.forward_fused, oracle.backward_fused) if fused else \
        (oracle.forward, oracle.backward)
    keys = ("reference_points_levels", "sampling_offsets", "attention_logits") if fused else \
        ("sampling_locations", "attention_weights")
    per_batch = w.points // w.B
    Nq = w.num_queries

    def run_entry(b, nthreads):
        bounds = np.linspace(0, Nq, nthreads + 1).astype(int)
        parts = [None] * nthreads

        def work(i):
            qs = slice(bounds[i], bounds[i + 1])
            args = (x["value"][b:b + 1], x["spatial_shapes"], x["level_start_index"]) + \
                tuple(x[k][b:b + 1, qs] for k in keys)
            fwd(*args)
            parts[i] = bwd(*args, x["grad_output"][b:b + 1, qs])[0]
        if nthreads == 1:
            work(0)
        else:
            ts = [threading.Thread(target=work, args=(i,)) for i in range(nthreads)]
            for t in ts:
                t.start()
            for t in ts:
                t.join()
        gv = parts[0]
        for p_ in parts[1:]:
            gv = gv + p_
        return gv

    def leg(nthreads):
        done, t_total, entries = 0, 0.0, 0
        while t_total < budget_s / 2:
            b = entries % w.B
            t0 = time.perf_counter()
            run_entry(b, nthreads)
            t_total += time.perf_counter() - t0
            done += per_batch
            entries += 1
        return done / t_total, entries, done, t_total

    threads = os.cpu_count() or 1
    v1, e1, d1, t1 = leg(1)
    vn, en, dn, tn = leg(threads)
    model = cpu_model()
    return {"value": vn, "unit": "points/s", "cores": threads, "kind": "oracle",
            "sample": f"{en} batch entries of the same workload (each {per_batch} points, "
                      f"forward + backward) on {threads} threads, query slices per thread, "
                      f"{dn} points in {tn:.1f} s; double accumulation",
            "cpu_model": model,
            "single_thread": {"value": v1, "unit": "points/s", "cores": 1,
                              "sample": f"{e1} batch entries, {d1} points in {t1:.1f} s"}}


def layer_flops(w):
    """Multiply-add flops (2 per multiply-add) of the layer's GEMMs per step:
    forward value (Nv rows), offset + logit and output (Nq rows) projections;
    the backward does twice as many (input and weight gradients of each)."""
    C, A = w.M * w.D, w.M * w.L * w.K
    Rq, Rv = w.B * w.num_queries, w.B * w.Nv
    fwd = 2 * Rv * C * C + 2 * Rq * C * (3 * A) + 2 * Rq * C * C
    return fwd, 2 * fwd


def bench_layer(args, w, dev):
    import torch
    import scale_deformable_attention_amd as msda
    from scale_deformable_attention_amd import workloads as wl
    x = wl.generate_layer(w)
    t = {k: torch.from_numpy(np.ascontiguousarray(v)).to(dev) for k, v in x.items()}
    params = {k: t[k] for k in msda._binding.LAYER_PARAMS}
    largs = (t["query"], t["input_flatten"], t["reference_points"], t["spatial_shapes"],
             t["level_start_index"], params, w.M, w.K)
    nsaved, nws = msda.msda_layer_sizes(t["query"], t["input_flatten"], t["spatial_shapes"],
                                        w.M, w.K)
    saved = torch.empty(nsaved, dtype=torch.uint8, device=dev)
    ws = torch.empty(nws, dtype=torch.uint8, device=dev)
    out = torch.empty_like(t["query"])
    grads = {k: torch.empty_like(t[k]) for k in ("query", "input_flatten", "reference_points")}
    grads.update({k: torch.empty_like(v) for k, v in params.items()})
    stream = torch.cuda.current_stream(dev)

    def fwd():
        msda.msda_layer_forward(*largs, output=out, saved=saved)

    def bwd():
        msda.msda_layer_backward(*largs, saved, t["grad_output"], grads=grads, workspace=ws)

    def step():
        fwd()
        bwd()

    def timed(fn, n):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n)]
        for a, b in evs:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in evs]))

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(args.steps):
        step()
    stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = start.elapsed_time(stop) / args.steps

    # the pieces on their own, same stream: the layer's forward and backward;
    # the value projection's forward GEMM (Nv rows x C x C, one launch of
    # msda_gemm_kernel) and its weight-gradient GEMM (split over the rows,
    # plus the split reduction)
    C = w.M * w.D
    Rv = w.B * w.Nv
    X = t["input_flatten"].reshape(Rv, C)
    Wv = params["value_weight"]
    Y = torch.empty(Rv, C, device=dev)
    G = t["input_flatten"].reshape(Rv, C)
    lws = torch.empty(msda.msda_linear_backward_workspace_size(Rv, C, C), dtype=torch.uint8,
                      device=dev)
    kernels = {
        "layer_forward": timed(fwd, args.steps),
        "layer_backward": timed(bwd, args.steps),
        "msda_gemm_kernel (forward, value projection)": timed(
            lambda: msda.msda_linear_forward(X, Wv, params["value_bias"], output=Y), args.steps),
        "msda_gemm_kernel+msda_split_reduce_kernel (weight gradient, value projection)": timed(
            lambda: msda.msda_linear_backward(X, Wv, G, needs=(False, True, False),
                                              workspace=lws), args.steps),
    }
    step()
    torch.cuda.synchronize()
    f_fwd, f_bwd = layer_flops(w)
    gemm_flops = 2 * Rv * C * C
    gemm_name = "msda_gemm_kernel (forward, value projection)"
    g_ms = kernels[gemm_name]
    achieved = gemm_flops / (g_ms * 1e-3) / 1e12
    result = {
        "metric": METRIC,
        "value": w.points / (ms_per_step * 1e-3),
        "unit": "points/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32 (GEMMs as three-term bf16 splits on the bf16 matrix cores, fp32 "
                 "accumulation)",
        "data": "synthetic (dyadic-grid activations and weights)",
        "config": {"workload": f"{w.name}: MSDeformAttn layer (value, offset, logit and "
                               f"output projections around the fused core), fwd+bwd; B={w.B} "
                               f"M={w.M} D={w.D} C={C} L={w.L} K={w.K} Nq={w.num_queries} "
                               f"Nv={w.Nv} shapes={list(w.shapes)}",
                   "frontend": "layer", "points_per_step": w.points, "global_batch": w.B,
                   "parallelism": "none"},
        "roofline": {"bound": "mfma", "kernel": gemm_name, "achieved": achieved,
                     "peak": MFMA_BF16_PEAK_TFLOPS / SPLIT_PRODUCTS, "unit": "TFLOP/s",
                     "frac": achieved * SPLIT_PRODUCTS / MFMA_BF16_PEAK_TFLOPS, "traffic": None,
                     "algorithmic_flops": gemm_flops, "avg_ms": g_ms, "launches": 1,
                     "peak_note": "achieved = fp32-product flops / time; peak = the bf16 "
                                  "matrix peak (2500 TFLOP/s) over the six bf16 products "
                                  "each fp32 product takes; the fp32 matrix peak is "
                                  f"{MFMA_F32_PEAK_TFLOPS}",
                     "bf16_mfma_tflops": achieved * SPLIT_PRODUCTS},
        "step_gemm_tflops": (f_fwd + f_bwd) / (ms_per_step * 1e-3) / 1e12,
        "gemm_flops_per_step": f_fwd + f_bwd,
        "kernels_ms": kernels,
        "wall_s_timed": wall,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_layer(w, x, args.cpu_budget)
    print(json.dumps(result), flush=True)


def cpu_baseline_layer(w, x, budget_s):
    """The layer oracle (numpy double GEMMs + the C oracle's fused core) on
    whole batch entries until the budget is used."""
    from oracle import layer as olayer
    names = {"value_weight": "w_value", "value_bias": "b_value", "offset_weight": "w_offset",
             "offset_bias": "b_offset", "attn_weight": "w_attn", "attn_bias": "b_attn",
             "output_weight": "w_out", "output_bias": "b_out"}
    p = {names[k]: x[k] for k in names}
    done, t_total, batches = 0, 0.0, 0
    for b in range(w.B):
        sl = slice(b, b + 1)
        args = (p, x["query"][sl], x["input_flatten"][sl], x["reference_points"][sl],
                x["spatial_shapes"], x["level_start_index"], w.M, w.L, w.K)
        t0 = time.perf_counter()
        olayer.layer_forward(*args)
        olayer.layer_backward(*args, x["grad_output"][sl])
        t_total += time.perf_counter() - t0
        done += w.points // w.B
        batches += 1
        if t_total >= budget_s:
            break
    import os as _os
    return {"value": done / t_total, "unit": "points/s",
            "cores": len(_os.sched_getaffinity(0)), "kind": "oracle",
            "sample": f"{batches} of {w.B} batch entries, layer forward + backward, {done} "
                      f"points in {t_total:.1f} s (numpy double GEMMs on the host's BLAS "
                      f"threads, the C oracle's core on one thread)"}


class _DcnShape:
    """A DCNv3 workload seen as a core problem (one level, groups as heads,
    output pixels as queries), for the byte counts."""

    def __init__(self, w):
        Ho, Wo = w.out_size
        self.B, self.M, self.D, self.L, self.K = w.B, w.G, w.D, 1, w.K
        self.num_queries, self.Nv, self.points = Ho * Wo, w.H * w.W, w.points


def bench_dcn(args, w, dev):
    import torch
    import scale_deformable_attention_amd as msda
    from scale_deformable_attention_amd import workloads as wl
    x = wl.generate_dcn(w)
    if w.value_dtype == "bf16":
        inp = torch.from_numpy(x["input_bf16"].view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        inp = torch.from_numpy(x["input"]).to(dev)
    off = torch.from_numpy(x["offset"]).to(dev)
    mask = torch.from_numpy(x["mask"]).to(dev)
    gout = torch.from_numpy(x["grad_output"]).to(dev)
    geo = dict(kernel=w.kernel, stride=w.stride, pad=w.pad, dilation=w.dilation)
    Ho, Wo = w.out_size
    out = torch.empty(w.B, Ho, Wo, w.G * w.D, device=dev)
    gi = torch.empty(inp.shape, dtype=torch.float32, device=dev)
    go = torch.empty_like(off)
    gm = torch.empty_like(mask)
    ws = torch.empty(max(msda.msda_dcn_backward_workspace_size(inp, off, **geo), 1),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def fwd():
        msda.msda_dcn_forward(inp, off, mask, output=out, **geo)

    def bwd(needs=(True, True, True)):
        msda.msda_dcn_backward(inp, off, mask, gout, needs=needs, grad_input=gi, grad_offset=go,
                               grad_mask=gm, workspace=ws, **geo)

    def step():
        fwd()
        bwd()

    def timed(fn, n):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n)]
        for a, b in evs:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in evs]))

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(args.steps):
        step()
    stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = start.elapsed_time(stop) / args.steps
    names = KERNEL_NAMES["dcn"]
    kernels = {names[0]: timed(fwd, args.steps),
               names[1]: timed(lambda: bwd((False, True, True)), args.steps),
               names[2]: timed(lambda: bwd((True, False, False)), args.steps)}
    step()
    torch.cuda.synchronize()
    shape = _DcnShape(w)
    ab = algorithmic_bytes(shape, 2 if w.value_dtype == "bf16" else 4)
    kernel_bytes = dict(zip(names, (ab["forward"], ab["bwd_point"], ab["bwd_value"])))
    dom = max(kernels, key=kernels.get)
    achieved = kernel_bytes[dom] / (kernels[dom] * 1e-3) / 1e9
    measured = read_traffic(w.name)
    traffic = None
    if measured is not None and all(k in measured for k in dom.split("+")):
        traffic = sum(measured[k] for k in dom.split("+"))
    result = {
        "metric": METRIC,
        "value": w.points / (ms_per_step * 1e-3),
        "unit": "points/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if w.value_dtype == "f32" else "bf16 input, f32 math",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: DCNv3 aggregation, {w.note}; B={w.B} H={w.H} "
                               f"W={w.W} G={w.G} D={w.D} kernel={w.kernel} stride={w.stride} "
                               f"pad={w.pad} dilation={w.dilation} offsets N(0,{w.sigma_px} px)",
                   "frontend": "dcn", "points_per_step": w.points, "global_batch": w.B,
                   "parallelism": "none"},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic, "algorithmic_bytes": kernel_bytes[dom],
                     "avg_ms": kernels[dom], "launches": len(dom.split("+"))},
        "kernels_ms": kernels,
        "kernels_frac": {k: kernel_bytes[k] / (v * 1e-3) / 1e9 / HBM_PEAK_GBS
                         for k, v in kernels.items()},
        "wall_s_timed": wall,
    }
    if not args.no_cpu_baseline:
        import oracle
        t0 = time.perf_counter()
        oracle.dcn_forward(x["input"][:1], x["offset"][:1], x["mask"][:1], **geo)
        oracle.dcn_backward(x["input"][:1], x["offset"][:1], x["mask"][:1], x["grad_output"][:1],
                            **geo)
        dt = time.perf_counter() - t0
        result["cpu_baseline"] = {"value": (w.points // w.B) / dt, "unit": "points/s",
                                  "cores": 1, "kind": "oracle",
                                  "sample": f"1 of {w.B} batch entries, forward + backward, "
                                            f"{w.points // w.B} points in {dt:.1f} s, single "
                                            f"thread, double accumulation"}
    print(json.dumps(result), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="encoder_train")
    ap.add_argument("--frontend", choices=("core", "fused", "layer", "dcn"), default="core",
                    help="core: locations and weights given; fused: formed in the kernels "
                         "from reference points, offsets and logits; layer: the whole "
                         "MSDeformAttn layer with its four projections")
    ap.add_argument("--value-dtype", choices=("workload", "f32", "bf16", "f16"),
                    default="workload", help="storage of the value tensor (core front-end)")
    ap.add_argument("--loc-dtype", choices=("f32", "f16"), default="f32",
                    help="storage of the locations and weights (core front-end)")
    ap.add_argument("--grad-dtype", choices=("f32", "bf16"), default="f32",
                    help="storage of grad_value (core front-end)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-directions", action="store_true",
                    help="skip the one-call-at-a-time warm/cold timing (profiler runs)")
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of oracle work for the CPU baseline sample")
    ap.add_argument("--workspace-mib", type=float, default=0.0,
                    help="backward workspace in MiB (0: msda_backward_workspace_size, the "
                         "one-pass size; less runs the value gradient in passes)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the core runs on a single MI355X. A layer is "
              "sharded across GPUs by batch or by head, which needs no exchange, so the "
              "per-GPU figure is the one-GPU run at the per-GPU shape.", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return

    import torch
    import scale_deformable_attention_amd as msda
    from scale_deformable_attention_amd import workloads as wl

    dev = torch.device("cuda:0")
    msda.library()
    if args.frontend == "dcn":
        name = args.workload if args.workload in wl.DCN_WORKLOADS else "dcnv3_stage2"
        return bench_dcn(args, wl.DCN_WORKLOADS[name], dev)
    w = wl.WORKLOADS[args.workload]
    if args.frontend == "layer":
        return bench_layer(args, w, dev)
    narrow = args.value_dtype != "workload" or args.loc_dtype != "f32" or args.grad_dtype != "f32"
    if narrow and args.frontend != "core":
        print("--value-dtype/--loc-dtype/--grad-dtype apply to the core front-end",
              file=sys.stderr)
        sys.exit(2)
    if args.value_dtype != "workload":
        w = w.scaled(value_dtype=args.value_dtype)
    x = wl.generate(w)
    if w.value_dtype == "bf16":
        value = torch.from_numpy(x["value_bf16"].view(np.int16)).to(dev).view(torch.bfloat16)
    elif w.value_dtype == "f16":
        value = torch.from_numpy(x["value_f16"]).to(dev)
    else:
        value = torch.from_numpy(x["value"]).to(dev)
    shapes = torch.from_numpy(x["spatial_shapes"]).to(dev)
    lsi = torch.from_numpy(x["level_start_index"]).to(dev)
    loc_np, attn_np = x["sampling_locations"], x["attention_weights"]
    if args.loc_dtype == "f16":
        loc_np, attn_np = loc_np.astype(np.float16), attn_np.astype(np.float16)
    loc = torch.from_numpy(loc_np).to(dev)
    attn = torch.from_numpy(attn_np).to(dev)
    gout = torch.from_numpy(x["grad_output"]).to(dev)
    out = torch.empty(w.B, w.num_queries, w.M * w.D, device=dev)
    gdt = torch.bfloat16 if args.grad_dtype == "bf16" else torch.float32
    gv = torch.empty(w.B, w.Nv, w.M, w.D, dtype=gdt, device=dev)
    gl = torch.empty(loc.shape, dtype=torch.float32, device=dev)
    ga = torch.empty(attn.shape, dtype=torch.float32, device=dev)
    ws_bytes = msda.msda_backward_workspace_size(value, loc)
    if args.workspace_mib > 0:
        ws_bytes = int(args.workspace_mib * (1 << 20))
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    backward = w.backward
    fused = args.frontend == "fused"
    if fused:
        ref = torch.from_numpy(x["reference_points_levels"]).to(dev)
        off = torch.from_numpy(x["sampling_offsets"]).to(dev)
        logits = torch.from_numpy(x["attention_logits"]).to(dev)
        del loc, attn, gl, ga
        gref = torch.empty_like(ref)
        goff = torch.empty_like(off)
        glog = torch.empty_like(logits)
        ws_bytes = msda.msda_backward_fused_workspace_size(value, off)
        if args.workspace_mib > 0:
            ws_bytes = int(args.workspace_mib * (1 << 20))
        ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)

        def fwd():
            msda.msda_forward_fused(value, shapes, lsi, ref, off, logits, output=out)

        def bwd(needs=(True, True, True)):
            msda.msda_backward_fused(value, shapes, lsi, ref, off, logits, gout, grad_value=gv,
                                     grad_reference_points=gref, grad_sampling_offsets=goff,
                                     grad_attention_logits=glog,
                                     needs=(needs[0], needs[1], needs[1], needs[2]),
                                     workspace=ws)
    else:
        def fwd():
            msda.msda_forward(value, shapes, lsi, loc, attn, output=out)

        def bwd(needs=(True, True, True)):
            msda.msda_backward(value, shapes, lsi, loc, attn, gout, grad_value=gv,
                               grad_sampling_locations=gl, grad_attention_weights=ga,
                               needs=needs, workspace=ws, grad_value_dtype=gdt)

    def step():
        fwd()
        if backward:
            bwd()

    stream = torch.cuda.current_stream(dev)   # the library launches on this stream

    def timed(fn, n):
        """Average ms of fn over n calls, HIP events on the launch stream."""
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n)]
        for a, b in evs:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in evs]))

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # the timed region: exactly K steps
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(args.steps):
        step()
    stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = start.elapsed_time(stop)

    # each kernel on its own (same inputs, same stream): the forward kernel;
    # the backward with only the location/weight gradients (the point kernel);
    # the backward with only grad_value (bin + tile kernels)
    # (fused: the backward's softmax-statistics kernel runs in both halves, the
    # reference-point reduction after the point kernel)
    names = KERNEL_NAMES["fused" if fused else "core"]
    names = (forward_kernel(w, 4 if w.value_dtype == "f32" else 2, fused),) + names[1:]
    kernels = {names[0]: timed(fwd, args.steps)}
    if backward:
        kernels[names[1]] = timed(lambda: bwd((False, True, True)), args.steps)
        kernels[names[2]] = timed(lambda: bwd((True, False, False)), args.steps)
        step()   # leave a full set of gradients in place
        torch.cuda.synchronize()

    # forward and backward one call at a time, warm (back to back) and cold (a
    # 512 MiB buffer written before each call, more than the L2s and the
    # 256 MB MALL hold, so that the inputs start in HBM): median, p10, p90
    def spread(fn, n, scrub=None):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n)]
        for a, b in evs:
            if scrub is not None:
                scrub.fill_(1.0)
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        ms = np.array([a.elapsed_time(b) for a, b in evs])
        return {"median": float(np.median(ms)), "p10": float(np.percentile(ms, 10)),
                "p90": float(np.percentile(ms, 90))}

    directions = None
    if not args.no_directions:
        scrub = torch.empty(128 << 20, dtype=torch.float32, device=dev)
        directions = {"calls": args.steps,
                      "warm": {"forward_ms": spread(fwd, args.steps)},
                      "cold": {"forward_ms": spread(fwd, args.steps, scrub)}}
        if backward:
            directions["warm"]["backward_ms"] = spread(bwd, args.steps)
            directions["cold"]["backward_ms"] = spread(bwd, args.steps, scrub)
        del scrub
        torch.cuda.synchronize()

    ms_per_step = total_ms / args.steps
    pts_per_s = w.points / (ms_per_step * 1e-3)
    touched = touched_value_rows(w, x, fused_locations(x) if fused else
                                 (loc_np.astype(np.float32) if args.loc_dtype == "f16" else None))
    ab = algorithmic_bytes(w, 4 if w.value_dtype == "f32" else 2, fused,
                           6 if args.loc_dtype == "f16" else 12,
                           2 if args.grad_dtype == "bf16" else 4, touched)
    kernel_bytes = dict(zip(names, (ab["forward"], ab["bwd_point"], ab["bwd_value"])))
    dom_name = max(kernels, key=kernels.get)
    dom_ms, dom_bytes = kernels[dom_name], kernel_bytes[dom_name]
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9
    measured = None if narrow else read_traffic(w.name + ("_fused" if fused else ""))
    traffic = None
    if measured is not None and all(k in measured for k in dom_name.split("+")):
        traffic = sum(measured[k] for k in dom_name.split("+"))
    step_bytes = ab["step"] if backward else ab["forward"]
    step_gbs = step_bytes / (ms_per_step * 1e-3) / 1e9

    result = {
        "metric": METRIC,
        "value": pts_per_s,
        "unit": "points/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if not narrow and w.value_dtype == "f32" else
                 f"{w.value_dtype} value, {args.loc_dtype} locations and weights, "
                 f"{args.grad_dtype} grad_value; f32 math",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: {w.note}; B={w.B} M={w.M} D={w.D} L={w.L} K={w.K} "
                               f"Nq={w.num_queries} Nv={w.Nv} shapes={list(w.shapes)} "
                               f"offsets N(0,{w.sigma_px} px)"
                               + ("; fused front-end (reference points + offsets, softmax "
                                  "of logits, in the kernels)" if fused else ""),
                   "frontend": args.frontend,
                   "points_per_step": w.points, "global_batch": w.B, "parallelism": "none"},
        "roofline": {"bound": "hbm", "kernel": dom_name, "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic, "algorithmic_bytes": dom_bytes, "avg_ms": dom_ms,
                     "launches": len(dom_name.split("+"))},
        "step_roofline": {"algorithmic_bytes": step_bytes, "achieved": step_gbs,
                          "frac": step_gbs / HBM_PEAK_GBS},
        "kernels_ms": kernels,
        "kernels_frac": {k: kernel_bytes[k] / (v * 1e-3) / 1e9 / HBM_PEAK_GBS
                         for k, v in kernels.items()},
        "directions": directions,
        "wall_s_timed": wall,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, x, args.cpu_budget, fused)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
