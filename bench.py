"""Benchmark of the per-row MoE route on one MI355X.

One step = one route_fused_packed call (latent down projection 7168 -> 3584 in
BF16, FP32 router logits over 896 experts, standalone top-16) over one batch
of synthetic rows, inputs and weights resident in HBM. The weights are model
parameters: each weight copy is packed once by route_pack_weights (the decode
kernel's read order, same bytes) outside the timed region, as a server does
when it loads the weights. The headline workload is the 8-row decode round;
the weights rotate over 8 distinct copies (8 x 77 MB, more than the 256 MB
Infinity Cache) so every step streams its weights from HBM.

Timing protocol (the pages time graph replays and report medians of
repeated windows): the routes are replayed from HIP graphs, one holding 25
passes over the weight copies (200 calls, call i on copy i mod 8 with that
copy's input bank) and, when --steps is not a multiple of that, one holding
the remaining calls, so a window runs exactly --steps routes. Routes inside
one graph run back to back like the layers of one decode step; the headline
with one pass over the copies per graph (an extra graph boundary every 8
routes, about 5 us each) is reported beside it as `graph8_us`. --warmup routes run untimed first; then the headline
graph keeps replaying, untimed, for at least --clock-warmup-s seconds (the
shader clock leaves its idle level only after about 0.2 s of load; reported
on its own as `clock_warmup`). --windows windows of --steps routes are timed
with events on the launch stream between two device synchronisations, and
the median window gives the value. The shader clock read from the driver's
DPM table while each workload runs (outside the timed windows) is reported as
`sclk`.

Also reported: every decode width of the pages (1, 8, 9, 12, 16, 20 rows),
each also through route_fused on the [K][N] weights, the 3072-row prefill
chunk (packed weights, and the [K][N] path beside it), the decode kernel at
one tensor-parallel rank's share (448 x 112 at 8 ranks, 224 x 56 at 16 ranks;
1, 8 and 20 rows), the decode kernel's HBM roofline fraction, the prefill
MFMA fractions, and the CPU oracle timed on this host (a reported baseline
only).

Roofline: a decode route is one kernel launch. `achieved` divides the
algorithmic bytes of one launch (both weights once + the rows' inputs and
outputs) by the launch interval measured here (median window / steps: the
kernel's duration plus the ~1 us between back-to-back launches);
`kernel_trace` divides the same bytes by the kernel's average dispatch
duration in the committed rocprofv3 trace of this benchmark (no gaps), and
`traffic` is the HBM bytes per launch from the committed FETCH_SIZE /
WRITE_SIZE summary; both are read only while the kernel source is the one
they were taken on.

--profile-pass runs only what the counter runs need: 64 headline decode
launches (packed weights), a plain 512 MiB device copy (the counters'
calibration) and 8 packed prefill chunks.

Prints ONE JSON line on stdout.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "us per MoE-layer route (1-20 rows) + prefill rows/s; % HBM / MFMA peak"
HBM_PEAK_GBPS = 8000.0
# Decode graphs hold this many passes over the weight copies (200 routes for
# 8 copies): routes inside one graph run back to back like the layers of a
# decode step, while a graph boundary costs about 5 us of idle GPU (one graph
# per pass over the 8 copies measured 18.17 us per 8-row route, graphs of 40
# / 200 / 800 routes 17.57 / 17.49 / 17.47). The headline with one pass per
# graph is reported beside it as `graph8_us`.
GRAPH_CYCLES = 25
BF16_MFMA_PEAK_TFLOPS = 2500.0
K, N, E = 7168, 3584, 896
FIXED_BYTES = K * N * 2 + K * E * 4                       # 77,070,336
ROW_BYTES = K * 2 + N * 2 + E * 4 + 16 * 4 + 16 * 4       # 25,216
PREFILL_FLOPS_LATENT = 2.0 * 3072 * K * N                 # 157.84 GFLOP
PREFILL_FLOPS_ROUTER = 2.0 * 3072 * K * E                 # the method's router work, 39.46 GFLOP
PREFILL_FLOPS_ROUTER_MFMA = 3 * PREFILL_FLOPS_ROUTER      # bf16 x3 split, 118.4 GFLOP of MFMA work
PROFILE_COUNTERS = os.path.join(ROOT, "profiles", "decode_route_r8_counters.md")
PROFILE_TRACE = os.path.join(ROOT, "profiles", "decode_route_r8_kernel_trace.md")
DECODE_SOURCES = ["latent_projection_top_amd/csrc/decode_route.hip",
                  "latent_projection_top_amd/csrc/route_device.h"]


def decode_bytes(rows: int) -> int:
    return FIXED_BYTES + ROW_BYTES * rows


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def source_digest() -> str:
    h = hashlib.sha256()
    for p in DECODE_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def profile_fields(path: str) -> dict:
    """The `- name: `value`` fields of a committed profile summary, if it was
    taken on the current kernel source; else {}."""
    if not os.path.exists(path):
        return {}
    fields = {}
    for line in open(path):
        if ":" in line and line.strip().startswith("- "):
            k, v = line.strip()[2:].split(":", 1)
            fields[k.strip()] = v.strip().strip("`")
    return fields if fields.get("kernel_source_digest") == source_digest() else {}


def committed_float(path: str, name: str):
    try:
        return float(profile_fields(path)[name])
    except (KeyError, ValueError):
        return None


def committed_traffic():
    """HBM bytes per decode launch from the committed rocprofv3 counter summary,
    if it was taken on the current kernel source."""
    return committed_float(PROFILE_COUNTERS, "hbm_bytes_per_launch")


class DecodeSetup:
    def __init__(self, rows: int, copies, banks_dev, route, torch):
        self.rows = rows
        self.route = route
        self.torch = torch
        self.plan = route.Plan(route.MODE_DECODE, rows)
        n = len(copies)
        self.ws = [self.plan.new_workspace() for _ in range(n)]
        self.xs = [banks_dev[i][:rows].contiguous() for i in range(n)]
        dev = "cuda"
        self.lat = torch.empty((n, rows, N), dtype=torch.bfloat16, device=dev)
        self.lg = torch.empty((n, rows, E), dtype=torch.float32, device=dev)
        self.ids = torch.empty((n, rows, 16), dtype=torch.int32, device=dev)
        self.wt = torch.empty((n, rows, 16), dtype=torch.float32, device=dev)
        self.copies = copies

    def run_all(self, count: int | None = None):
        """`count` routes (default one per copy), call i on weight copy i mod
        copies with that copy's input bank, outputs and workspace."""
        r = self.route
        n = len(self.copies)
        for j in range(n if count is None else count):
            i = j % n
            w, wr = self.copies[i]
            r.fused(self.plan, self.xs[i], w, wr, self.lat[i], self.lg[i], self.ids[i], self.wt[i],
                    self.ws[i], rows=self.rows)

    def capture(self, count: int | None = None):
        return capture_graph(lambda: self.run_all(count), self.torch)

    def runner(self, counts, cycles: int = GRAPH_CYCLES):
        """A function that replays exactly n routes (n in `counts`): a graph of
        `cycles` passes over the weight copies, n // (cycles * copies) times,
        then a graph of the remaining routes. Every graph is captured here,
        before any timing."""
        g_routes = cycles * len(self.copies)
        full = self.capture(g_routes)
        part = {c % g_routes: self.capture(c % g_routes) for c in counts if c % g_routes}

        def run(n: int):
            for _ in range(n // g_routes):
                full.replay()
            if n % g_routes:
                part[n % g_routes].replay()
        run.full = full
        run.graph_routes = g_routes
        return run


class PackedDecodeSetup(DecodeSetup):
    """The same routes through route_fused_packed: each weight copy packed once
    (route_pack_weights, outside the timed region) into the decode kernel's
    consumption order."""

    def __init__(self, rows: int, copies, banks_dev, route, torch, packs):
        super().__init__(rows, copies, banks_dev, route, torch)
        self.packs = packs

    def run_all(self, count: int | None = None):
        r = self.route
        n = len(self.packs)
        for j in range(n if count is None else count):
            i = j % n
            r.fused_packed(self.plan, self.xs[i], self.packs[i], self.lat[i], self.lg[i], self.ids[i],
                           self.wt[i], self.ws[i], rows=self.rows)


def time_routes(run, n: int, torch):
    """ms of one window of exactly n routes (events on the current stream,
    which is the stream the graphs' kernels run on, between two device
    synchronisations)."""
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    run(n)
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end)


def time_graph(g, replays: int, torch):
    """Average ms per replay of `replays` back-to-back replays of one graph."""
    return time_routes(lambda n: [g.replay() for _ in range(n)], replays, torch) / replays


def read_sclk_mhz(path: str):
    """Current shader clock in MHz from the driver's DPM table (the line
    marked '*'), or None."""
    try:
        with open(path) as f:
            for line in f:
                if line.rstrip().endswith("*"):
                    return int(line.split(":")[1].strip().split("Mhz")[0].split("MHz")[0])
    except (OSError, ValueError, IndexError):
        return None
    return None


def sample_sclk(enqueue, torch, samples: int = 40):
    """Shader clock while the GPU runs a workload: `enqueue` queues a few ms
    of work without waiting for it; the clock is read from sysfs after each
    batch, while the GPU is still busy with it. Runs outside every timed
    window (reading the DPM table is a file read, no child process)."""
    paths = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
    if not paths:
        return None
    # the card of the current device, by PCI address, when the runtime gives it
    props = torch.cuda.get_device_properties(torch.cuda.current_device())
    bus = getattr(props, "pci_bus_id", None)
    if bus is not None:
        tag = f"{getattr(props, 'pci_domain_id', 0):04x}:{bus:02x}:{getattr(props, 'pci_device_id', 0):02x}."
        mine = [p for p in paths if tag in os.path.realpath(os.path.dirname(p))]
        if mine:
            paths = mine
    torch.cuda.synchronize()
    vals = []
    for _ in range(samples):
        enqueue()
        v = read_sclk_mhz(paths[0])
        if v is not None:
            vals.append(v)
    torch.cuda.synchronize()
    if not vals:
        return None
    vals.sort()
    return {"median_mhz": vals[len(vals) // 2], "min_mhz": vals[0], "max_mhz": vals[-1],
            "samples": len(vals), "source": paths[0]}


def capture_graph(fn, torch):
    """fn() run once on a side stream, then captured into a HIP graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def share_timings(copies, banks, route, torch, replays: int):
    """Decode kernel at one tensor-parallel rank's share (latent_router on the
    rank's contiguous column slices). Every rank's share of every weight copy
    is a distinct buffer (8 copies x all ranks = 616 MB, more than the
    Infinity Cache), and one graph replay runs each once."""
    out = {}
    for ranks, (lat, exp) in sorted(route.RANK_SHARES.items()):
        shares = [(w[:, r * lat:(r + 1) * lat].contiguous(), wr[:, r * exp:(r + 1) * exp].contiguous())
                  for w, wr in copies for r in range(ranks)]
        share_bytes = K * (lat * 2 + exp * 4)
        for rows in (1, 8, 20):
            plan = route.Plan(route.MODE_DECODE, rows, latent=lat, experts=exp)
            ws = plan.new_workspace()
            xs = [banks[i % len(banks)][:rows].contiguous() for i in range(len(shares))]
            lat_o = torch.empty((rows, lat), dtype=torch.bfloat16, device="cuda")
            lg_o = torch.empty((rows, exp), dtype=torch.float32, device="cuda")

            def run():
                for i, (w, wr) in enumerate(shares):
                    route.latent_router(plan, xs[i], w, wr, lat_o, lg_o, ws, rows=rows)

            g = capture_graph(run, torch)
            for _ in range(2):
                g.replay()
            us = time_graph(g, replays, torch) * 1000.0 / len(shares)
            nbytes = share_bytes + rows * (K * 2 + lat * 2 + exp * 4)
            out[f"{ranks}x{rows}"] = {"ranks": ranks, "latent": lat, "experts": exp, "rows": rows,
                                      "us": round(us, 3),
                                      "hbm_frac": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)}
            log(f"share {ranks} ranks ({lat}x{exp}) rows={rows}: {us:.2f} us per launch "
                f"({nbytes / us / 1e3:.0f} GB/s)")
            del g
        del shares
    return out


def pack_copies(copies, route, torch):
    """Each weight copy packed once into the decode format."""
    plan = route.Plan(route.MODE_DECODE, 20)
    packs = [route.pack_weights(plan, w, wr) for w, wr in copies]
    torch.cuda.synchronize()
    return packs


def prefill_inputs(route, torch, bf16, gen, w0, wr0):
    """The 3072-row prefill chunk (1 % outlier channels) with its plan,
    workspace, outputs and packed weights."""
    rows = 3072
    plan = route.Plan(route.MODE_PREFILL, rows)
    p = {"plan": plan, "ws": plan.new_workspace(), "rows": rows,
         "x": bf16(gen.hidden(rows, bank=4100, outliers=True)),
         "lat": torch.empty((rows, N), dtype=torch.bfloat16, device="cuda"),
         "lg": torch.empty((rows, E), dtype=torch.float32, device="cuda"),
         "ids": torch.empty((rows, 16), dtype=torch.int32, device="cuda"),
         "wt": torch.empty((rows, 16), dtype=torch.float32, device="cuda")}
    p["packed"] = route.pack_weights(plan, w0, wr0)
    torch.cuda.synchronize()
    return p


def profile_pass(rows: int, copies, banks, route, torch, bf16, gen):
    """Short run for the rocprofv3 counter passes: headline decode launches,
    one plain copy of known size, and packed prefill chunks."""
    d = PackedDecodeSetup(rows, copies, banks, route, torch, pack_copies(copies, route, torch))
    for _ in range(8):
        d.run_all()
    torch.cuda.synchronize()
    src = torch.empty(512 << 20, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    p = prefill_inputs(route, torch, bf16, gen, *copies[0])
    for _ in range(8):
        route.fused_packed(p["plan"], p["x"], p["packed"], p["lat"], p["lg"], p["ids"], p["wt"], p["ws"])
    torch.cuda.synchronize()
    log(f"profile pass: {8 * len(copies)} decode launches of {rows} rows, one 512 MiB copy, "
        f"8 packed 3072-row prefill chunks")


def cpu_baseline(rows: int, budget_s: float):
    """The oracle, as it is, on this host: route_ref_widened on 8-row batches
    with the weights widened to float64 once outside the timed region."""
    import numpy as np
    from oracle import route_oracle as orc
    from synth import generators as gen
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    w64, wr64 = orc.widen_weights(gen.latent_weight(0), gen.router_weight(0))
    banks = [gen.hidden(rows, bank=3000 + b) for b in range(16)]
    orc.route_ref_widened(banks[0], w64, wr64)      # warm-up
    n = 0
    t0 = time.perf_counter()
    while True:
        orc.route_ref_widened(banks[n % len(banks)], w64, wr64)
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s or n >= 5000:
            break
    return {"value": el / n * 1e6, "unit": "us", "cores": int(threads), "kind": "oracle",
            "sample": f"{n} decode routes of {rows} rows (float64 numpy oracle, weights widened "
                      f"once outside the timed region), {el:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1600,
                    help="routes per timed window (1600 = 200 replays of the 8-copy graph)")
    ap.add_argument("--warmup", type=int, default=80, help="untimed routes before the timing")
    ap.add_argument("--windows", type=int, default=5, help="timed windows; the median is reported")
    ap.add_argument("--clock-warmup-s", type=float, default=0.3,
                    help="after the warm-up routes, the headline graph replays untimed for at least "
                         "this long: the shader clock leaves its idle level only after about 0.2 s "
                         "of load")
    ap.add_argument("--rows", type=int, default=8)
    ap.add_argument("--copies", type=int, default=8)
    ap.add_argument("--widths", default="1,8,9,12,16,20")
    ap.add_argument("--prefill-reps", type=int, default=20)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="headline width only")
    ap.add_argument("--profile-pass", action="store_true",
                    help="only the launches the rocprofv3 counter passes need")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the route computes every row locally and has "
              "no multi-GPU path to time (run with --gpus 1).", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0 or args.windows < 1:
        print("--steps and --windows must be positive and --warmup non-negative", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from latent_projection_top_amd import route
    from synth import generators as gen

    torch.cuda.set_device(0)
    copies_n = args.copies
    steps, warm = args.steps, args.warmup

    log(f"generating {copies_n} weight copies ...")

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()

    copies = []
    for c in range(copies_n):
        copies.append((bf16(gen.latent_weight(c)), torch.from_numpy(gen.router_weight(c)).cuda()))
    banks = [bf16(gen.hidden(20, bank=4000 + b)) for b in range(copies_n)]
    if args.profile_pass:
        profile_pass(args.rows, copies, banks, route, torch, bf16, gen)
        return

    results = {}
    kn_results = {}
    widths = [args.rows] + ([int(w) for w in args.widths.split(",") if int(w) != args.rows]
                            if not args.no_extras else [])
    head = None
    clocks = {}
    clock_warm = None
    packs = pack_copies(copies, route, torch)
    for rows in widths:
        variants = [("packed", PackedDecodeSetup(rows, copies, banks, route, torch, packs))]
        if not args.no_extras:
            variants.append(("kn", DecodeSetup(rows, copies, banks, route, torch)))
        for name, d in variants:
            run = d.runner([steps, warm])
            if warm:
                run(warm)
            torch.cuda.synchronize()
            if clock_warm is None:
                # the first graph: keep replaying (untimed) until the clock is up
                t0 = time.perf_counter()
                reps = 0
                per = max(1, 400 // run.graph_routes)
                while time.perf_counter() - t0 < args.clock_warmup_s:
                    for _ in range(per):
                        run.full.replay()
                    reps += per
                    torch.cuda.synchronize()
                clock_warm = {"seconds": round(time.perf_counter() - t0, 3),
                              "routes": reps * run.graph_routes,
                              "note": "untimed replays of the headline graph after the warm-up routes"}
            windows = sorted(time_routes(run, steps, torch) for _ in range(args.windows))
            ms_win = windows[len(windows) // 2]
            us = ms_win * 1000.0 / steps
            (results if name == "packed" else kn_results)[rows] = us
            log(f"decode rows={rows} ({name} weights): {us:.2f} us per route "
                f"({decode_bytes(rows) / us / 1e3:.0f} GB/s; windows "
                f"{', '.join(f'{w * 1000.0 / steps:.2f}' for w in windows)})")
            if rows == args.rows and name == "packed":
                head = {"us": us, "ms_step": ms_win / steps, "graph_routes": run.graph_routes,
                        "windows_us": [round(w * 1000.0 / steps, 3) for w in windows]}
                clocks["decode"] = sample_sclk(
                    lambda: [run.full.replay() for _ in range(max(1, 200 // run.graph_routes))], torch)
                # the same windows with one pass over the weight copies per graph
                run1 = d.runner([steps], cycles=1)
                w1 = sorted(time_routes(run1, steps, torch) for _ in range(args.windows))
                head["graph8_us"] = round(w1[len(w1) // 2] * 1000.0 / steps, 3)
                del run1
            del run, d

    us8 = head["us"]
    nbytes = decode_bytes(args.rows)
    achieved = nbytes / (us8 * 1e-6) / 1e9
    trace_us = committed_float(PROFILE_TRACE, "kernel_avg_us")
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": committed_traffic(),
                "frac_basis": "algorithmic bytes per launch / launch interval (median window / steps, "
                              "kernel duration plus the gap between back-to-back launches)",
                "kernel": f"decode_route_kernel<{1 if args.rows <= 16 else 2}, DecodeShape<3584, 896, "
                          f"{'8, 8' if args.rows <= 4 else '4, 8'}>, true> (packed weights)",
                "launch_interval_us": round(us8, 3),
                "algorithmic_bytes_per_launch": nbytes,
                "kernel_trace": None if trace_us is None else {
                    "avg_dispatch_us": trace_us,
                    "achieved": round(nbytes / (trace_us * 1e-6) / 1e9, 1),
                    "frac": round(nbytes / (trace_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                    "source": "profiles/decode_route_r8_kernel_trace.md (rocprofv3 dispatch durations of "
                              "the timed launches, no inter-launch gaps)"}}

    prefill = None
    if not args.no_extras:
        p = prefill_inputs(route, torch, bf16, gen, *copies[0])
        plan, ws, x, lat, lg, ids, wt = (p[k] for k in ("plan", "ws", "x", "lat", "lg", "ids", "wt"))
        rows = p["rows"]
        w0, wr0 = copies[0]

        def t_call(fn, reps):
            # the first calls after the decode phase run slower (clocks rise
            # under the compute-bound GEMMs for about 25 ms of 3072-row
            # chunks): warm up for 120 calls, then take the median of five
            # timed windows
            for _ in range(120):
                fn()
            torch.cuda.synchronize()
            times = []
            for _ in range(5):
                s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                s.record()
                for _ in range(reps):
                    fn()
                e.record()
                torch.cuda.synchronize()
                times.append(s.elapsed_time(e) / reps * 1000.0)
            return sorted(times)[2]

        # packed weights (K-contiguous W, router parts split once) first: the
        # reported figure; then the [K][N] path, which splits the router
        # weight on every call
        packed = p["packed"]
        t_all = t_call(lambda: route.fused_packed(plan, x, packed, lat, lg, ids, wt, ws), args.prefill_reps)
        t_lr = t_call(lambda: route.latent_router_packed(plan, x, packed, lat, lg, ws), args.prefill_reps)
        # one top-16 call is shorter than its host-side launch, so eager calls
        # would time the host: time a graph of 20 calls instead
        g_tk = capture_graph(lambda: [route.topk16(plan, lg, ids, wt) for _ in range(20)], torch)
        t_tk = t_call(lambda: g_tk.replay(), args.prefill_reps) / 20
        del g_tk
        clocks["prefill_gemms"] = sample_sclk(
            lambda: [route.latent_router_packed(plan, x, packed, lat, lg, ws) for _ in range(10)], torch)
        t_all_kn = t_call(lambda: route.fused(plan, x, w0, wr0, lat, lg, ids, wt, ws), args.prefill_reps)
        t_lr_kn = t_call(lambda: route.latent_router(plan, x, w0, wr0, lat, lg, ws), args.prefill_reps)
        # the pages' other chunk size: 1024 rows (8 row tiles of 128 rows, K split in 2)
        t_1024 = t_call(lambda: route.fused_packed(plan, x[:1024], packed, lat[:1024], lg[:1024], ids[:1024],
                                                   wt[:1024], ws, rows=1024), args.prefill_reps)
        del packed, p
        method_flops = PREFILL_FLOPS_LATENT + PREFILL_FLOPS_ROUTER
        mfma_flops = PREFILL_FLOPS_LATENT + PREFILL_FLOPS_ROUTER_MFMA
        prefill = {
            "rows": rows, "weights": "packed (route_pack_weights, once per weight set)",
            "us_per_chunk": round(t_all, 2), "rows_per_s": round(rows / (t_all * 1e-6)),
            "latent_router_us": round(t_lr, 2), "topk16_us": round(t_tk, 2),
            "method_tflops": round(method_flops / (t_lr * 1e-6) / 1e12, 1),
            "method_frac": round(method_flops / (t_lr * 1e-6) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4),
            "mfma_work_tflops": round(mfma_flops / (t_lr * 1e-6) / 1e12, 1),
            "mfma_work_frac": round(mfma_flops / (t_lr * 1e-6) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4),
            "flops_note": "method: 2*M*K*(3584+896) = 197.3 GFLOP; MFMA work: the router runs on three "
                          "exact BF16 parts of its FP32 weight, 276.2 GFLOP; both over latent_router_us "
                          "(the two GEMMs; the router GEMM also recomputes any non-finite logit); per-kernel "
                          "times are in "
                          "profiles/prefill_gemm_3072_kernel_trace.md",
            "router_variant": "FP32 weight split into 3 exact BF16 parts, BF16 MFMA, FP32 chains "
                              "restarted every 256 K and folded into FP64",
            "kn_weights": {"us_per_chunk": round(t_all_kn, 2),
                           "rows_per_s": round(rows / (t_all_kn * 1e-6)),
                           "latent_router_us": round(t_lr_kn, 2),
                           "note": "[K][N] weights; includes the per-call router weight split"},
            "chunk_1024": {"rows": 1024, "us_per_chunk": round(t_1024, 2),
                           "rows_per_s": round(1024 / (t_1024 * 1e-6)),
                           "note": "packed weights, the same plan; chunks of 1..1728 rows split K over more "
                                   "workgroups (1024 rows: 2 splits, 128-row block tiles)"},
        }
        log(f"prefill 3072 (packed): {t_all:.1f} us ({prefill['rows_per_s']:.3g} rows/s), projection "
            f"{t_lr:.1f} us = {prefill['method_tflops']} TFLOP/s of the method's work "
            f"({prefill['mfma_work_tflops']} of MFMA work), top-16 {t_tk:.1f} us; [K][N] weights "
            f"{t_all_kn:.1f} us")

    shares = None
    if not args.no_extras:
        shares = share_timings(copies, banks, route, torch, replays=20)

    cpu = None
    if not args.no_cpu:
        log("timing the CPU oracle ...")
        cpu = cpu_baseline(args.rows, args.cpu_seconds)
        log(f"cpu oracle: {cpu['value']:.0f} us per route on {cpu['cores']} threads")

    out = {
        "metric": METRIC,
        "value": round(us8, 3),
        "unit": "us",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warm,
        "ms_per_step": round(head["ms_step"], 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16+fp32",
        "precision": {
            "latent": "BF16 x BF16 products, FP32 MFMA accumulation, K-split partials summed in FP64, "
                      "rounded once to BF16",
            "router": "FP32 weight x BF16 hidden value, accumulated in FP64 (decode; prefill: exact "
                      "three-part BF16 split on the BF16 MFMA, FP32 chains of 256 K folded into FP64), "
                      "rounded once to FP32",
            "top16": "32-bit integer keys of the FP32 logits; weights in FP64, rounded to FP32"},
        "data": "synthetic",
        "config": {
            "workload": f"decode route, {args.rows} rows: x[{args.rows},7168] BF16 -> latent "
                        f"[{args.rows},3584] BF16 + router logits [{args.rows},896] FP32 + "
                        f"top-16 ids/weights; {copies_n} rotating weight copies "
                        f"(W[7168,3584] BF16 + Wr[7168,896] FP32, {copies_n * FIXED_BYTES / 1e6:.0f} MB)",
            "rows": args.rows,
            "hidden": K, "latent": N, "experts": E, "topk": 16,
            "weight_copies": copies_n,
            "weights": "packed once per copy by route_pack_weights, outside the timed region",
            "timing": f"median of {args.windows} windows of exactly {steps} route_fused_packed calls "
                      f"replayed from HIP graphs of {head['graph_routes']} calls ({GRAPH_CYCLES} passes "
                      f"over the weight copies; fewer when the window is shorter), events on the launch "
                      f"stream",
            "graph_routes": head["graph_routes"],
        },
        "windows_us": head["windows_us"],
        "graph8_us": head["graph8_us"],
        "clock_warmup": clock_warm,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "decode_us_by_rows": {str(k): round(v, 3) for k, v in sorted(results.items())},
        "decode_hbm_frac_by_rows": {str(k): round(decode_bytes(k) / (v * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)
                                    for k, v in sorted(results.items())},
        "decode_kn_us_by_rows": {str(k): round(v, 3) for k, v in sorted(kn_results.items())},
        "prefill": prefill,
        "rank_share_decode": shares,
        "sclk": dict(clocks, note="shader clock (MHz) sampled from the driver's DPM table while "
                                  "the same workload ran, outside the timed windows; the peaks "
                                  "above assume 2400 MHz"),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
