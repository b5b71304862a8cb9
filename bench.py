"""Benchmark: FusedNormalization throughput on one MI355X.

One step = one fn_fused_normalize call over one batch of the headline
workload: 256 images of 224x224x3 uint8 NHWC -> fp16, flip p=0.5, erase
p=0.5, area fraction [0.02, 0.33], aspect ratio [0.3, 3.3] (the ImageNet
training shape of page "(11) FusedNormalization", section 1; synthetic
gradient images, no dataset).  Inputs are resident in HBM before timing;
the timed steps rotate over --sets distinct input/output buffer sets (over
1 GB in total) so the 256 MB Infinity Cache cannot hold the working set.

Prints ONE JSON line:
  value      images/s (whole job, one GPU)
  roofline   algorithmic bytes per launch (every input byte read once and
             every output element written once: N*H*W*C*(1+2)) divided by
             the launch's average duration from HIP events around the timed
             launches on the launch stream, against the 8 TB/s HBM peak;
             traffic = hardware bytes per launch from the committed
             rocprofv3 counter summary, if it was taken on the current
             build of libfn.so (else null)
  cpu_baseline  the oracle (plain C loops, fp32 output) timed on this
             host's cores over a bounded sample of the same workload;
             cpu_simd the page's own host method (SSE4.1 + F16C) beside it.

Timing: about --prewarm-seconds of untimed launches (the GPU clocks down
while the host builds inputs), --warmup untimed launches, then --steps timed
launches between two device synchronisations.

Extra legs: stream_ceiling times the library's streaming reference
(fn_test_stream: the same read:write mix and byte count with no arithmetic,
lane-contiguous 16-byte streaming stores), the practical roof for the fused
kernel; host_us is the host time per call while the timed launches are
enqueued; --all adds one line per workload on stderr; --sweep instead prints
per-batch-size lines for the headline shape (the fused call, the streaming
reference, and a minimal launch) and a fit of time = fixed + per-image cost.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, vendor figure
HEADLINE_METRIC = "images/s and % of HBM peak GB/s, 256×224²×3 u8→FP16 fused normalize"
PROFILE_COUNTERS = os.path.join(ROOT, "profiles", "fused_tiles_kernel_imagenet_train_counters.txt")
LIBRARY = os.path.join(ROOT, "augmentation_amd", "libfn.so")


def library_hash() -> str:
    """SHA-256 (first 16 hex digits) of the built library: the kernels and
    the host planning that launches them.  The build is deterministic, so
    source edits that change no code (comments) keep the hash."""
    h = hashlib.sha256()
    with open(LIBRARY, "rb") as f:
        h.update(f.read())
    return h.hexdigest()[:16]


def counter_traffic() -> dict | None:
    """Hardware bytes per launch from the committed counter summary, or None
    if it is missing or was taken on another build of the library."""
    if not os.path.exists(PROFILE_COUNTERS) or not os.path.exists(LIBRARY):
        return None
    kv = {}
    with open(PROFILE_COUNTERS) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("library_sha256") != library_hash():
        return None
    try:
        return {"bytes_per_launch": float(kv["hbm_bytes_per_launch"]),
                "fetch_bytes": float(kv["fetch_bytes_per_launch"]),
                "write_bytes": float(kv["write_bytes_per_launch"])}
    except (KeyError, ValueError):
        return None


OUT_NAMES = {0: "fp32", 1: "fp16", 2: "fp16, 4 channels per pixel"}
OUT_CODES = {"fp32": 0, "fp16": 1, "fp16_pad4": 2}


def describe(w) -> str:
    """The workload in words, e.g. "imagenet_train: 256x224x224x3 uint8 NHWC
    -> fp16 NHWC, flip 0.5, erase 0.5 [0.02,0.33]x[0.3,3.3], seed 123"."""
    src = ""
    if w.src_h:
        src = f" ({w.H}x{w.W} windows at ({w.y0},{w.x0}) of {w.src_h}x{w.src_w} sources)"
    erase = (f"erase {w.erase_p:g} [{w.scale[0]:g},{w.scale[1]:g}]x[{w.ratio[0]:g},{w.ratio[1]:g}]"
             if w.erase_p > 0 else "no erase")
    return (f"{w.name}: {w.N}x{w.H}x{w.W}x{w.C} uint8 NHWC{src} -> {OUT_NAMES[w.out_dtype]} NHWC, "
            f"flip {w.flip_p:g}, {erase}, seed {w.seeds[0]}")


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def host_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))  # a host's CPU share for one of its eight GPUs


def time_launches(launch, steps: int, warmup: int, sets: int, stream, prewarm_s: float,
                  host: list | None = None) -> float:
    """Average milliseconds per launch over `steps` launches (events on the
    launch stream), after `warmup` untimed ones.  Before those, launches run
    untimed for about `prewarm_s` seconds: the GPU clocks down while the host
    prepares inputs, and a few warmup launches (well under a millisecond)
    do not bring it back up.  `host`, if given, receives the host time per
    call (ms) spent enqueuing the timed launches."""
    import torch
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < prewarm_s:
        for k in range(50):
            launch(k % sets)
        torch.cuda.synchronize()
    for k in range(warmup):
        launch(k % sets)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    h0 = time.perf_counter()
    for k in range(steps):
        launch(k % sets)
    h1 = time.perf_counter()
    end.record(stream)
    torch.cuda.synchronize()
    if host is not None:
        host.append((h1 - h0) / steps * 1e3)
    return start.elapsed_time(end) / steps


def median_call_ms(launch, calls: int, sets: int, stream) -> float:
    """Median over `calls` individually timed launches (an event pair around
    each; untimed, after the main measurement)."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(calls)]
    for k, (e0, e1) in enumerate(evs):
        e0.record(stream)
        launch(k % sets)
        e1.record(stream)
    torch.cuda.synchronize()
    times = sorted(e0.elapsed_time(e1) for e0, e1 in evs)
    return times[len(times) // 2]


def bench_workload(b, w, steps: int, warmup: int, sets: int, prewarm_s: float,
                   out_offset: int = 0) -> dict:
    """Time workload w (rotating `sets` buffer sets).  out_offset > 0 puts
    each output that many bytes past a 16-byte boundary."""
    import torch
    stream = torch.cuda.current_stream()
    x = torch.from_numpy(w.make_input()).cuda()
    tdt = torch.float32 if w.out_dtype == 0 else torch.float16
    ins = [x] + [x.clone() for _ in range(sets - 1)]
    if out_offset:
        out_bytes = w.N * w.H * w.W * w.out_channels * w.out_bytes
        bufs = [torch.empty(out_bytes + 16, dtype=torch.uint8, device="cuda") for _ in range(sets)]
        outs = [t.data_ptr() + out_offset for t in bufs]
    else:
        bufs = None
        outs = [torch.empty(w.out_shape, dtype=tdt, device="cuda") for _ in range(sets)]
    torch.cuda.synchronize()
    seeds = w.seeds

    _, sh, sw, _ = w.source_shape
    row_stride, image_stride = sw * w.C, sh * sw * w.C
    first = (w.y0 * sw + w.x0) * w.C  # the window's first byte in each source image

    def launch(k):
        if (sh, sw) == (w.H, w.W):
            b.fn_fused_normalize(ins[k], w.N, w.H, w.W, w.C, w.mean, w.std, w.flip_p, w.erase_p,
                                 w.scale[0], w.scale[1], w.ratio[0], w.ratio[1],
                                 seeds[k % len(seeds)], w.out_dtype, outs[k], stream)
        else:
            b.fn_fused_normalize_ex(ins[k].data_ptr() + first, row_stride, image_stride, w.N,
                                    w.H, w.W, w.C, w.mean, w.std, w.flip_p, w.erase_p,
                                    w.scale[0], w.scale[1], w.ratio[0], w.ratio[1],
                                    seeds[k % len(seeds)], 0, w.out_dtype, outs[k], stream)

    host = []
    ms = time_launches(launch, steps, warmup, sets, stream, prewarm_s, host)
    med = median_call_ms(launch, min(steps, 200), sets, stream)
    del ins, outs, bufs
    torch.cuda.empty_cache()
    return {"ms": ms, "median_call_ms": med, "host_ms": host[0], "images_per_s": w.N / (ms * 1e-3),
            "gbs": w.nominal_bytes / (ms * 1e-3) / 1e9}


def bench_two_streams(b, w, steps: int, warmup: int, sets: int, prewarm_s: float) -> dict:
    """Independent batches of workload w issued alternately on two streams
    (each rotating buffer set bound to one of them): the whole job's time per
    batch, where one batch's ramp and tail overlap the other stream's work.
    A deployment pattern reported beside the metric, not the metric."""
    import torch
    main = torch.cuda.current_stream()
    other = torch.cuda.Stream()
    x = torch.from_numpy(w.make_input()).cuda()
    tdt = torch.float32 if w.out_dtype == 0 else torch.float16
    ins = [x] + [x.clone() for _ in range(sets - 1)]
    outs = [torch.empty(w.out_shape, dtype=tdt, device="cuda") for _ in range(sets)]
    torch.cuda.synchronize()
    seeds = w.seeds

    def launch(k):
        j = k % sets
        b.fn_fused_normalize(ins[j], w.N, w.H, w.W, w.C, w.mean, w.std, w.flip_p, w.erase_p,
                             w.scale[0], w.scale[1], w.ratio[0], w.ratio[1],
                             seeds[k % len(seeds)], w.out_dtype, outs[j], (main, other)[j % 2])

    t0 = time.perf_counter()
    while time.perf_counter() - t0 < prewarm_s:
        for k in range(50):
            launch(k)
        torch.cuda.synchronize()
    for k in range(warmup):
        launch(k)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(main)
    other.wait_event(start)
    for k in range(steps):
        launch(k)
    main.wait_stream(other)
    end.record(main)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    del ins, outs
    torch.cuda.empty_cache()
    return {"streams": 2, "ms_per_batch": round(ms, 5), "images_per_s": round(w.N / (ms * 1e-3), 1),
            "gbs": round(w.nominal_bytes / (ms * 1e-3) / 1e9, 1),
            "frac": round(w.nominal_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}


def stream_widen(w) -> int:
    """Bytes written per byte read by the streaming reference for workload
    w: 2 for fp16 outputs, 4 for fp32."""
    return 4 if w.out_dtype == 0 else 2


def bench_stream(b, nbytes: int, widen: int, steps: int, warmup: int, sets: int,
                 prewarm_s: float) -> dict:
    """The streaming reference moving about nbytes per launch: nbytes/(1+widen)
    read, widen times that written."""
    import torch
    stream = torch.cuda.current_stream()
    inb = (nbytes // (1 + widen)) // 16 * 16
    src = [torch.ones(inb, dtype=torch.uint8, device="cuda") for _ in range(sets)]
    dst = [torch.empty(inb * widen, dtype=torch.uint8, device="cuda") for _ in range(sets)]

    def launch(k):
        b.fn_test_stream(src[k], dst[k], inb, widen, stream)

    ms = time_launches(launch, steps, warmup, sets, stream, prewarm_s)
    del src, dst
    torch.cuda.empty_cache()
    moved = inb * (1 + widen)
    return {"ms": ms, "gbs": moved / (ms * 1e-3) / 1e9, "bytes": moved}


def sweep(b, steps: int, warmup: int, prewarm_s: float, sizes) -> None:
    """Per-launch time against batch size on the headline shape: the fused
    call, the streaming reference with the same bytes, and the streaming
    reference on 16 bytes (the cost of a launch itself).  Fits
    t(N) = fixed + N * per_image over the sizes; one JSON line each."""
    import numpy as np
    import torch
    from augmentation_amd import synth
    stream = torch.cuda.current_stream()
    w = synth.WORKLOADS[synth.HEADLINE]
    img = w.H * w.W * w.C
    tiny_src = torch.ones(16, dtype=torch.uint8, device="cuda")
    tiny_dst = torch.empty(32, dtype=torch.uint8, device="cuda")
    floor = time_launches(lambda k: b.fn_test_stream(tiny_src, tiny_dst, 16, 2, stream),
                          max(steps, 1000), warmup, 1, stream, prewarm_s)
    print(json.dumps({"sweep": "launch_floor", "us": round(floor * 1e3, 3),
                      "what": "fn_test_stream on 16 bytes, back to back"}), flush=True)
    base = torch.from_numpy(w.make_input()).cuda()
    pts = {"fused": [], "stream": []}
    for N in sizes:
        sets = max(2, -(-1_200_000_000 // (3 * N * img)))
        reps = -(-N // w.N)
        xs = base.repeat(reps, 1, 1, 1)[:N].contiguous()
        ins = [xs] + [xs.clone() for _ in range(sets - 1)]
        outs = [torch.empty((N, w.H, w.W, w.C), dtype=torch.float16, device="cuda")
                for _ in range(sets)]

        def fused(k):
            b.fn_fused_normalize(ins[k], N, w.H, w.W, w.C, w.mean, w.std, w.flip_p, w.erase_p,
                                 w.scale[0], w.scale[1], w.ratio[0], w.ratio[1], w.seeds[0],
                                 w.out_dtype, outs[k], stream)

        def ref(k):
            b.fn_test_stream(ins[k], outs[k], N * img, 2, stream)

        n_steps = steps if N <= 512 else max(20, steps // 5)
        for name, fn in (("fused", fused), ("stream", ref)):
            ms = time_launches(fn, n_steps, warmup, sets, stream, prewarm_s)
            pts[name].append((N, ms * 1e3))
            print(json.dumps({"sweep": name, "N": N, "us": round(ms * 1e3, 3),
                              "tbs": round(3 * N * img / (ms * 1e-3) / 1e12, 3)}), flush=True)
        del ins, outs, xs
        torch.cuda.empty_cache()
    for name, p in pts.items():
        n = np.array([q[0] for q in p], float)
        t = np.array([q[1] for q in p])
        per, fixed = np.polyfit(n, t, 1)
        print(json.dumps({"sweep": "fit", "kernel": name, "fixed_us": round(fixed, 3),
                          "per_image_ns": round(per * 1e3, 2),
                          "streaming_tbs": round(3 * img / (per * 1e-6) / 1e12, 3)}), flush=True)


def timeline(b, steps: int, warmup: int, prewarm_s: float, launches: int = 20) -> None:
    """Where the headline launch's microseconds go, from the instrumented
    build libfn_timeline.so: every tile's work-group records the 100 MHz
    real-time clock at its start, after staging (tile loaded, decisions
    drawn), when its stores are issued and when they are acknowledged
    (fn_test_timeline).  Each recorded launch is the last of 10 back-to-back
    ones over the rotating buffer sets.  Prints a text summary."""
    import numpy as np
    import torch
    from augmentation_amd import synth
    lib = b.timeline_library()
    st = torch.cuda.current_stream()
    w = synth.WORKLOADS[synth.HEADLINE]
    sets = 10
    x = torch.from_numpy(w.make_input()).cuda()
    ins = [x] + [x.clone() for _ in range(sets - 1)]
    outs = [torch.empty(w.out_shape, dtype=torch.float16, device="cuda") for _ in range(sets)]
    max_tiles = w.N * w.H  # a tile holds whole rows
    stamps = torch.zeros(max_tiles * 4, dtype=torch.int64, device="cuda")
    mean, std = b._host_floats(w.mean, w.C), b._host_floats(w.std, w.C)

    def launch(L, k):
        rc = L.fn_fused_normalize(ins[k].data_ptr(), w.N, w.H, w.W, w.C, mean, std, w.flip_p,
                                  w.erase_p, w.scale[0], w.scale[1], w.ratio[0], w.ratio[1],
                                  w.seeds[0], w.out_dtype, outs[k].data_ptr(), st.cuda_stream)
        if rc:
            raise b.FnError(rc, L.fn_last_error().decode())

    ms_prod = time_launches(lambda k: launch(b._lib, k), steps, warmup, sets, st, prewarm_s)
    if lib.fn_test_timeline(stamps.data_ptr(), max_tiles):
        raise b.FnError(-1, lib.fn_last_error().decode())
    ms_inst = time_launches(lambda k: launch(lib, k), steps, warmup, sets, st, prewarm_s)
    runs = []
    for _ in range(launches):
        stamps.zero_()
        for k in range(10):
            launch(lib, k % sets)
        torch.cuda.synchronize()
        d = stamps.view(-1, 4).cpu().numpy()
        runs.append(d[d[:, 0] != 0].astype(np.float64))
    lib.fn_test_timeline(None, 0)
    tiles = len(runs[0])
    in_tile = w.N * w.H * w.W * w.C / tiles  # bytes per tile, on average
    out_tile = in_tile * 2
    r = timeline_summary(runs, in_tile, out_tile)
    print(f"timeline: {describe(w)}; {tiles} tiles of {in_tile / 1e3:.2f} kB in, "
          f"{out_tile / 1e3:.2f} kB out")
    print(f"per-launch time, {steps} back-to-back launches: libfn.so {ms_prod * 1e3:.2f} us, "
          f"instrumented build {ms_inst * 1e3:.2f} us")
    print(f"recorded launches: {launches}, each the last of 10 back-to-back ones")
    sp = r["span"]
    print(f"span, first work-group start to last acknowledged store: median {sp[0]:.2f} us "
          f"(min {sp[1]:.2f}, max {sp[2]:.2f})")
    print("tile phases, us, median (10th-90th percentile) over all tiles of all recorded launches:")
    fmt = lambda v: "{:.2f} ({:.2f}-{:.2f})".format(*v)
    print(f"  start -> staged (loads landed, decisions drawn): {fmt(r['stage'])}")
    print(f"  staged -> stores issued (first wavefront):       {fmt(r['compute'])}")
    print(f"  issued -> stores acknowledged (all wavefronts):  {fmt(r['drain'])}")
    print(f"  whole life of a work-group:                       {fmt(r['life'])}")
    print("resident work-groups every 0.5 us (median launch): " +
          " ".join(str(int(v)) for v in r["occupancy"]))
    ret = r["first_generation_retire"]
    print(f"first generation: {r['first_generation']} work-groups start within 0.3 us of the first; "
          f"they retire at {ret[0]:.2f} / {ret[1]:.2f} / {ret[2]:.2f} us (10th / 50th / 90th "
          f"percentile)")
    print(f"last work-group start: {r['last_start']:.2f} us; below half the peak occupancy for the "
          f"last {r['tail_below_half']:.2f} us")
    print(f"modelled traffic (reads spread over each tile's staging, writes over the rest of its "
          f"life): {r['tbs_span']:.2f} TB/s over the span, {r['tbs_middle']:.2f} TB/s over its "
          f"middle half")


def timeline_summary(runs, in_tile: float, out_tile: float, tick_us: float = 0.01) -> dict:
    """Summary of recorded launches: runs holds one array per launch, a row
    of four clock stamps (start, staged, issued, acknowledged; tick_us per
    tick) per tile.  Medians over launches; phase figures are (50th, 10th,
    90th) percentiles over all tiles; times in microseconds from the first
    start of each launch; modelled traffic in TB/s."""
    import numpy as np
    spans, phase, occ_rows, first_gen, last_start, tail_half, rate_all, rate_mid = \
        [], {"stage": [], "compute": [], "drain": [], "life": []}, [], [], [], [], [], []
    for d in runs:
        d = np.asarray(d, dtype=np.float64)
        t0 = d[:, 0].min()
        S, G, I, A = [(d[:, k] - t0) * tick_us for k in range(4)]
        span = A.max()
        spans.append(span)
        for name, v in (("stage", G - S), ("compute", I - G), ("drain", A - I), ("life", A - S)):
            phase[name].append(v)
        grid = np.arange(0.0, span + 0.5, 0.5)
        active = np.array([np.sum((S <= t) & (A > t)) for t in grid])
        occ_rows.append(active)
        peak = active.max()
        gen = S <= 0.3
        first_gen.append((int(gen.sum()), np.percentile(A[gen], [10, 50, 90])))
        last_start.append(S.max())
        tail_half.append(span - grid[np.nonzero(active >= peak / 2)[0].max()])
        # modelled traffic: each tile's reads spread evenly over its staging,
        # its writes over the rest of its life
        step = 0.05
        fine = np.arange(0.0, span, step)
        rd = np.zeros_like(fine)
        wr = np.zeros_like(fine)
        for s_, g_, a_ in zip(S, G, A):
            i0, i1, i2 = (int(v / step) for v in (s_, g_, a_))
            rd[i0:max(i1, i0 + 1)] += in_tile / max(i1 - i0, 1)
            wr[i1:max(i2, i1 + 1)] += out_tile / max(i2 - i1, 1)
        total = rd + wr
        rate_all.append(total.sum() / span / 1e6)
        lo, hi = int(0.25 * len(fine)), int(0.75 * len(fine))
        rate_mid.append(total[lo:hi].sum() / ((hi - lo) * step) / 1e6)
    pct = lambda v: tuple(float(x) for x in np.percentile(np.concatenate(v), [50, 10, 90]))
    n = min(len(r) for r in occ_rows)
    return {
        "span": (float(np.median(spans)), float(min(spans)), float(max(spans))),
        "stage": pct(phase["stage"]), "compute": pct(phase["compute"]),
        "drain": pct(phase["drain"]), "life": pct(phase["life"]),
        "occupancy": np.median(np.stack([r[:n] for r in occ_rows]), axis=0),
        "first_generation": int(np.median([g[0] for g in first_gen])),
        "first_generation_retire": np.median(np.stack([g[1] for g in first_gen]), axis=0),
        "last_start": float(np.median(last_start)),
        "tail_below_half": float(np.median(tail_half)),
        "tbs_span": float(np.median(rate_all)), "tbs_middle": float(np.median(rate_mid)),
    }


def cpu_baseline(w, budget_s: float) -> dict:
    """The oracle as it stands, on this host's cores, over whole batches of
    the workload (fp32 output) until about budget_s seconds have passed;
    then on one thread over a few images for about a fifth of that."""
    import oracle
    threads = host_threads()
    x = w.window(w.make_input()) if w.src_h else w.make_input()
    reps, t0 = 0, time.perf_counter()
    while True:
        _, used = oracle.fused_normalize(x, w.mean, w.std, w.flip_p, w.erase_p, w.scale, w.ratio,
                                         seed=w.seeds[0], threads=threads)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    ips = reps * w.N / el
    one, t1 = 0, time.perf_counter()
    while True:
        n = one % w.N
        oracle.fused_normalize(x[n:n + 8], w.mean, w.std, w.flip_p, w.erase_p, w.scale, w.ratio,
                               seed=w.seeds[0], first_n=n, threads=1)
        one += 8
        el1 = time.perf_counter() - t1
        if el1 >= budget_s / 5:
            break
    return {"value": round(ips, 2), "unit": "images/s", "cores": used, "kind": "oracle",
            "sample": f"{reps} x the {w.N}-image {w.H}x{w.W}x{w.C} batch, fp32 output, "
                      f"{used} threads, {el:.1f} s wall; CPU: {cpu_model()}",
            "gbs_nominal": round(ips * w.H * w.W * w.C * (1 + 4) / 1e9, 3),
            "single_thread_images_per_s": round(one / el1, 2)}


def cpu_simd_rate(w, budget_s: float) -> dict:
    """The page's own method on the host (libfn_cpu.so: SSE4.1 + F16C, one
    image per worker call) on the same workload and output type, on this
    host's cores for about budget_s seconds, then on one thread for about a
    fifth of that."""
    import numpy as np
    from augmentation_amd import cpu_simd
    threads = host_threads()
    x = w.window(w.make_input()) if w.src_h else w.make_input()
    dt = np.float32 if w.out_dtype == 0 else np.float16
    out = np.empty(w.out_shape, dt)

    def run(batch, t):
        cpu_simd.fused_normalize(batch, w.mean, w.std, w.flip_p, w.erase_p, w.scale, w.ratio,
                                 seed=w.seeds[0], out_dtype=w.out_dtype, threads=t,
                                 out=out[:len(batch)])

    reps, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        run(x, threads)
        reps += 1
    el = time.perf_counter() - t0
    one, t1 = 0, time.perf_counter()
    while time.perf_counter() - t1 < budget_s / 5:
        run(x[:8], 1)
        one += 8
    el1 = time.perf_counter() - t1
    return {"value": round(reps * w.N / el, 2), "unit": "images/s", "cores": min(threads, w.N),
            "kind": "the page's host method (SSE4.1 + F16C, libfn_cpu.so)",
            "sample": f"{reps} x the {w.N}-image batch, {OUT_NAMES[w.out_dtype]} output, "
                      f"{el:.1f} s wall; CPU: {cpu_model()}",
            "single_thread_images_per_s": round(one / el1, 2)}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--sets", type=int, default=10, help="rotating buffer sets")
    ap.add_argument("--prewarm-seconds", type=float, default=0.3,
                    help="untimed launches before the warmup ones")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-stream", action="store_true", help="skip the streaming reference")
    ap.add_argument("--no-pipeline", action="store_true",
                    help="skip the two-stream pipeline (whose overlapping launches would "
                         "otherwise share a kernel trace with the one-stream ones)")
    ap.add_argument("--sweep", default=None, metavar="N,N,...",
                    help="time the headline shape at these batch sizes (and the streaming "
                         "reference and a minimal launch) instead of the JSON line")
    ap.add_argument("--timeline", action="store_true",
                    help="per-tile clock stamps of the headline launch from the instrumented "
                         "build libfn_timeline.so (a text summary instead of the JSON line)")
    ap.add_argument("--all", action="store_true", help="also time every workload (stderr)")
    ap.add_argument("--workload", default=None,
                    help="time this workload instead of the headline one (the JSON line then "
                         "describes it; the metric line of record is the default)")
    ap.add_argument("--shape", default=None, metavar="N,H,W,C",
                    help="time a synthetic batch of this shape instead (uniform bytes, flip and "
                         "erase 0.5, ImageNet constants for C = 3)")
    ap.add_argument("--out", default="fp16", choices=sorted(OUT_CODES),
                    help="output type for --shape")
    ap.add_argument("--out-offset", type=int, default=0, metavar="BYTES",
                    help="for --shape: put the output this many bytes past a 16-byte boundary "
                         "(a multiple of the element size)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the operation has no cross-GPU step and this "
              "build runs on a single MI355X (run with --gpus 1).", file=sys.stderr)
        return 2
    shape = None
    if args.shape:
        try:
            shape = tuple(int(v) for v in args.shape.split(","))
        except ValueError:
            shape = ()
        if len(shape) != 4 or min(shape) < 1:
            print("--shape takes N,H,W,C (positive integers)", file=sys.stderr)
            return 2
        esz = 4 if OUT_CODES[args.out] == 0 else 2
        if args.out_offset < 0 or args.out_offset % esz or args.out_offset >= 16:
            print("--out-offset must be a multiple of the element size below 16", file=sys.stderr)
            return 2

    import torch
    from augmentation_amd import binding as b
    from augmentation_amd import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    torch.cuda.set_device(0)
    if args.sweep:
        sweep(b, args.steps, args.warmup, args.prewarm_seconds,
              [int(v) for v in args.sweep.split(",")])
        return 0
    if args.timeline:
        timeline(b, args.steps, args.warmup, args.prewarm_seconds)
        return 0
    if shape:
        N, H, W, C = shape
        out_dtype = OUT_CODES[args.out]
        mean, std = ((synth.IMAGENET_MEAN, synth.IMAGENET_STD) if C == 3
                     else ((0.5,) * C, (0.25,) * C))
        name = f"shape {N}x{H}x{W}x{C} -> {args.out}" + (
            f", output {args.out_offset} bytes past 16-byte alignment" if args.out_offset else "")
        w = synth.Workload(name, N, H, W, C, mean, std, 0.5, 0.5, out_dtype, 1100)
        # inputs rotated beyond the 256 MB Infinity Cache (at least 600 MiB of
        # them), up to 64 sets; smaller shapes stay cache-resident
        sets = max(2, min(64, -(-(600 << 20) // w.elems)))
    else:
        name = args.workload or synth.HEADLINE
        if name not in synth.WORKLOADS:
            print(f"unknown workload {name!r}; known: {', '.join(synth.WORKLOADS)}",
                  file=sys.stderr)
            return 2
        w = synth.WORKLOADS[name]
        sets = args.sets
    r = bench_workload(b, w, args.steps, args.warmup, sets, args.prewarm_seconds,
                       args.out_offset if args.shape else 0)
    achieved = r["gbs"]
    traffic = counter_traffic() if name == synth.HEADLINE else None

    line = {
        "metric": (HEADLINE_METRIC if name == synth.HEADLINE
                   else f"images/s and % of HBM peak GB/s, {name}"),
        "value": round(r["images_per_s"], 1),
        "unit": "images/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": describe(w),
                   "N": w.N, "H": w.H, "W": w.W, "C": w.C, "out": OUT_NAMES[w.out_dtype],
                   "rotating_sets": sets},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": (round(traffic["bytes_per_launch"]) if traffic else None),
                     "traffic_gbs": (round(traffic["bytes_per_launch"] / (r["ms"] * 1e-3) / 1e9, 1)
                                     if traffic else None),
                     "bytes_per_launch": w.nominal_bytes},
        "median_call_ms": round(r["median_call_ms"], 5),
        "host_ms": round(r["host_ms"], 5),
    }
    if not args.no_stream:
        c = bench_stream(b, w.nominal_bytes, stream_widen(w), args.steps, args.warmup, args.sets,
                         args.prewarm_seconds)
        line["stream_ceiling"] = {"gbs": round(c["gbs"], 1), "bytes_per_launch": c["bytes"],
                                  "ms": round(c["ms"], 5),
                                  "fused_vs_stream": round(achieved / c["gbs"], 4)}
    if not args.no_stream and not args.no_pipeline and w.launches == 1:
        line["two_stream_pipeline"] = bench_two_streams(b, w, args.steps, args.warmup, sets,
                                                        args.prewarm_seconds)
    if args.all:
        for name, wl in synth.WORKLOADS.items():
            # the headline's method: as many warm-up launches (fewer timed
            # ones for the large batches, which take longer each)
            rr = bench_workload(b, wl, args.steps if wl.N < 1024 else max(10, args.steps // 4),
                                args.warmup, args.sets if wl.N < 1024 else 2, args.prewarm_seconds)
            print(json.dumps({"workload": name, "ms_per_launch": round(rr["ms"], 5),
                              "images_per_s": round(rr["images_per_s"], 1),
                              "gbs_nominal": round(rr["gbs"], 1),
                              "pct_of_peak": round(100 * rr["gbs"] / HBM_PEAK_GBS, 2)}),
                  file=sys.stderr, flush=True)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
        line["cpu_simd"] = cpu_simd_rate(w, args.cpu_seconds / 2)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
