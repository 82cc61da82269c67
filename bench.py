"""Throughput of the fused WTConv training step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload stage1]
                    [--backward fused|split]

A step is one pass of the whole hot path over one batch on synthetic inputs
already resident in device memory: wtconv_fwd, then the backward, by default
the fused wtconv_bwd (input and parameter gradients reading x and dy once),
with --backward split the two calls wtconv_bwd_input and wtconv_bwd_weight.
By default the step's kernels are replayed from a HIP graph (one graph of
one step per buffer set, in a row), as a training loop that captures its step
would run them; --launch eager times the calls as issued (also reported as
eager_ms_per_step).
W untimed steps, then exactly K timed steps bracketed by device
synchronisation; value = images per second over the K steps.  Each
step reads its own set of buffers, rotating over enough sets that no step
finds the previous step's tensors in the 256 MB last-level cache.

Also reported, on the same JSON line:
  roofline     the dominant call (longest average device time, timed with
               HIP events on the stream it is launched on) against the roof
               that bounds it by arithmetic intensity: algorithmic bytes over
               the 8 TB/s HBM peak when its FLOPs per byte fall below the ridge
               (157.3 TFLOP/s fp32 vector / 8 TB/s = 19.7 FLOP/B), else
               algorithmic FLOPs over 157.3 TFLOP/s; both fractions are
               reported.  Plain v_fmac_f32 issues at that vector rate on
               gfx950 (no packed-FP32 instruction is needed or used);
               traffic = HBM bytes per launch from the committed rocprofv3
               counter summary when it was taken on the current kernel source,
               else null
  cpu_baseline the fp64 oracle (test infrastructure, timed as it stands) on
               the host cores, on the same workload, about ten seconds of work,
               with the host CPU's model and a one-thread time on a few images
  step_ms      p10 / p50 / p90 of the per-step device times (a pass of K
               steps, each behind a short spin kernel so that HIP events see
               kernel time only; the per-call times come from the same
               events), the mean of the timed steps, and the mean with every
               step on the same buffer set (warm caches) beside the rotated,
               cache-cold one
  copy_probe   a plain device-to-device copy of 768 MiB timed on the same
               device: the HBM bandwidth reachable on this machine, and the step's
               effective bandwidth as a fraction of it
Before any of it the device runs the step, in the launch mode that is timed,
back to back for CLOCK_WARMUP_MS of wall time (untimed; reported as
clock_warmup_ms): the clocks and the launch path take some tens of
milliseconds of continuous work to settle, and a training loop runs in the
settled state.
  dw7x7_baseline  the plain 7x7 depthwise conv with bias (include/dwconv.h,
               the layer WTConv replaces) timed the same way on the same
               activations: forward + one-pass backward per step, and the
               WTConv/dw7x7 throughput ratios for training and inference
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP32_VALU_TFLOPS = 157.3  # MI355X fp32 vector peak (published); v_fmac_f32 issues at it
PEAK_HBM_GBS = 8000.0
RIDGE_FLOP_PER_BYTE = PEAK_FP32_VALU_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
KERNEL_SOURCES = os.path.join(ROOT, "aware_conv_amd", "csrc")
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "traffic_{workload}_{backward}.json")
COPY_PROBE_BYTES = 3 << 28  # 768 MiB: larger than any other copy of a bench run
CLOCK_WARMUP_MS = 500.0


def conv_flops_per_pixel(L, k):
    """Algorithmic FLOPs per input pixel of one pass: 2 k^2 for the base conv
    plus 4 subbands of 2 k^2 on a grid 4^l times smaller at each level l."""
    return 2.0 * k * k * (1.0 + sum(4.0 * 4.0 ** (-l) for l in range(1, L + 1)))


def io_model_reference(L):
    """Elements moved through device memory per input element by the unfused
    reference forward: 7 for the base path and the final add, 10.75 per level
    on a grid 4^(l-1) times smaller."""
    return 7.0 + 10.75 * sum(4.0 ** (-j) for j in range(L))


def source_hash():
    """Hash of the kernel sources' code: comments and blank lines are left
    out, so that a comment edit does not mark the counters stale."""
    import re
    h = hashlib.sha256()
    for name in sorted(os.listdir(KERNEL_SOURCES)):
        if name.endswith((".hip", ".h", ".cpp")):
            with open(os.path.join(KERNEL_SOURCES, name)) as f:
                text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
            code = [ln.split("//")[0].strip() for ln in text.splitlines()]
            h.update(name.encode() + b"\0" + "\n".join(c for c in code if c).encode())
    return h.hexdigest()[:16]


def template_args(kernel_name):
    """The template arguments of a demangled kernel name, as strings."""
    head = kernel_name.split("(")[0]
    if "<" not in head:
        return []
    inner = head[head.index("<") + 1:head.rindex(">")]
    return [a.strip() for a in inner.split(",")]


# Position of the FLIP argument (input gradient) of the apply kernels:
# k_plane_apply<K, L, H, W, P, NT, T, FLIP, RAG>, k_tile_apply<K, LT, TH, TW,
# NT, T, FLIP>, k_deep_apply<T, K, FLIP>; and of DX (input gradient computed)
# of k_plane_bwd1<K, L, H, W, P, NT, T, CROSS, DX, RAG>.
_FLIP_ARG = {"k_plane_apply": 7, "k_tile_apply": 6, "k_deep_apply": 2}
_BWD1_DX_ARG = 8


def _kernel(kernel_name):
    head = kernel_name.split("(")[0].split("<")[0]
    return head.split("::")[-1].split(" ")[-1]


def call_of(kernel_name, fused):
    """Entry point a profiled kernel belongs to, or None."""
    k = _kernel(kernel_name)
    args = template_args(kernel_name)
    c = None
    if k in _FLIP_ARG:
        flip = args[_FLIP_ARG[k]] == "true"
        c = "wtconv_bwd_input" if flip else "wtconv_fwd"
    elif k in ("k_plane_bww", "k_tile_bww", "k_deep_bww", "k_bww_final"):
        c = "wtconv_bwd_weight"
    elif k == "k_plane_bwd1":
        # DX false: the weight gradient alone
        c = "wtconv_bwd" if args[_BWD1_DX_ARG] == "true" else "wtconv_bwd_weight"
    elif k.startswith("k_plane_bwd") or k.startswith("k_tile_bwd"):
        c = "wtconv_bwd"
    if fused and c in ("wtconv_bwd_input", "wtconv_bwd_weight"):
        c = "wtconv_bwd"
    return c


def is_step_marker(kernel_name):
    """The forward's main kernel: launched exactly once per step."""
    k = _kernel(kernel_name)
    return k in ("k_plane_apply", "k_tile_apply") and \
        template_args(kernel_name)[_FLIP_ARG[k]] == "false"


def summarize_traffic(fetch_dir, write_dir, wl, act_bytes, fused):
    """HBM bytes per entry-point call from two rocprofv3 --pmc runs (FETCH_SIZE,
    WRITE_SIZE, KiB per dispatch), each scaled by what the same counter reads
    for the plain device copy of act_bytes that --copy-probe performs."""
    import csv
    import glob
    out = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        rows = [r for f in files for r in csv.DictReader(open(f)) if r["Counter_Name"] == counter]
        copies = [float(r["Counter_Value"]) for r in rows
                  if "copyBuffer" in r["Kernel_Name"] and int(r["Grid_Size"]) > 0]
        # the probe's three copies are the largest copies of the run
        copies = sorted(copies)[-3:]
        kib_copy = sum(copies) / len(copies)
        factor = COPY_PROBE_BYTES / (kib_copy * 1024.0)
        per_call = {}
        steps = sum(1 for r in rows if is_step_marker(r["Kernel_Name"]))
        for r in rows:
            c = call_of(r["Kernel_Name"], fused)
            if c is None:
                continue
            per_call[c] = per_call.get(c, 0.0) + float(r["Counter_Value"]) * 1024.0 * factor
        # every step calls each entry point once
        out[counter] = {"factor": factor, "copy_kib": kib_copy,
                        "bytes_per_call": {c: per_call[c] / max(1, steps) for c in per_call}}
    calls = sorted(set(out["FETCH_SIZE"]["bytes_per_call"]) | set(out["WRITE_SIZE"]["bytes_per_call"]))
    summary = {
        "workload": wl.name,
        "backward": "fused" if fused else "split",
        "source_sha256_16": source_hash(),
        "copy_probe_bytes": COPY_PROBE_BYTES,
        "fetch_factor": out["FETCH_SIZE"]["factor"],
        "write_factor": out["WRITE_SIZE"]["factor"],
        "bytes_per_launch": {c: out["FETCH_SIZE"]["bytes_per_call"].get(c, 0.0) +
                             out["WRITE_SIZE"]["bytes_per_call"].get(c, 0.0) for c in calls},
        "fetch_bytes_per_launch": out["FETCH_SIZE"]["bytes_per_call"],
        "write_bytes_per_launch": out["WRITE_SIZE"]["bytes_per_call"],
    }
    return summary


def roofline(call, flops, nbytes, dur_s, traffic, n_out):
    """The roofline record of one call: bound by arithmetic intensity
    (algorithmic FLOPs per algorithmic byte) against the ridge, achieved and
    peak in that roof's unit, and the other roof's fraction alongside."""
    gbs = nbytes / dur_s / 1e9
    tfs = flops / dur_s / 1e12
    ai = flops / nbytes
    hbm = ai < RIDGE_FLOP_PER_BYTE
    rec = {
        "kernel": call,
        "bound": "hbm" if hbm else "alu",
        "achieved": round(gbs if hbm else tfs, 2),
        "peak": PEAK_HBM_GBS if hbm else PEAK_FP32_VALU_TFLOPS,
        "unit": "GB/s" if hbm else "TFLOP/s",
        "frac": round(gbs / PEAK_HBM_GBS if hbm else tfs / PEAK_FP32_VALU_TFLOPS, 4),
        "traffic": traffic,
        "traffic_bytes_per_output_element": (round(traffic / n_out, 3)
                                              if traffic is not None else None),
        "flop_per_byte": round(ai, 2),
        "hbm_gbs": round(gbs, 1),
        "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
        "valu_tflops": round(tfs, 2),
        "valu_frac": round(tfs / PEAK_FP32_VALU_TFLOPS, 4),
        "flops_per_launch": flops,
        "algo_bytes_per_launch": nbytes,
    }
    return rec


def cpu_model():
    """The host CPU's model name, from /proc/cpuinfo (None if unreadable)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _oracle_rate(oracle, a, p, images, min_seconds):
    """Images per second of oracle fwd + bwd over the batch `a` (whole
    batches until min_seconds of work, at least one)."""
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.fwd(a["x"], *p)
        oracle.bwd(a["x"], a["dy"], *p)
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds:
            return reps, el, reps * images / el


def cpu_baseline(wl, min_seconds=10.0, one_thread_seconds=3.0):
    import oracle
    import wtconv_inputs as wi
    d = wi.workload_inputs(wl)
    a = {k: v.double().numpy() for k, v in d.items()}
    p = [a[n] for n in ("w_base", "b_base", "s_base", "w_wav", "s_wav")]
    cores = oracle.num_threads()
    reps, el, rate = _oracle_rate(oracle, a, p, wl.B, min_seconds)
    # one thread, on the first images of the batch (the same per-image work)
    nb = max(1, min(wl.B, 2))
    a1 = dict(a, x=a["x"][:nb].copy(), dy=a["dy"][:nb].copy())
    oracle.set_threads(1)
    try:
        reps1, el1, rate1 = _oracle_rate(oracle, a1, p, nb, one_thread_seconds)
    finally:
        oracle.set_threads(cores)
    return {"value": round(rate, 3), "unit": "images/s", "cores": cores,
            "kind": "oracle",
            "sample": "%d full %s batch(es) of %d images (fwd + bwd), fp64, %.1f s" % (
                reps, wl.name, wl.B, el),
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "one_thread": {"value": round(rate1, 3), "unit": "images/s",
                           "sample": "%d x %d image(s) of %s (fwd + bwd), fp64, %.1f s" % (
                               reps1, nb, wl.name, el1)}}


class GraphSteps:
    """Steps replayed from HIP graphs: one graph holds `len(sets)` steps in a
    row, one per buffer set (so that consecutive steps read different
    buffers), and graphs of the first r steps serve a remainder.  Replaying
    one graph over and over costs the runtime less than switching between
    graphs every step.  Nothing is allocated inside: every output is
    preallocated.  With same=True every step of the graphs uses sets[0]."""

    def __init__(self, torch, sets, step, same=False):
        self.torch, self.sets, self.step, self.same = torch, sets, step, same
        self.graphs = {}

    def graph(self, r):
        if r not in self.graphs:
            g = self.torch.cuda.CUDAGraph()
            with self.torch.cuda.graph(g):
                for i in range(r):
                    self.step(self.sets[0 if self.same else i])
            self.torch.cuda.synchronize()
            self.graphs[r] = g
        return self.graphs[r]

    def prepare(self, *counts):
        """Capture, ahead of any timing, every graph that run(n) needs for
        each n in counts."""
        for n in counts:
            full, r = divmod(n, len(self.sets))
            if full:
                self.graph(len(self.sets))
            if r:
                self.graph(r)
        return self

    def run(self, n):
        """Enqueue exactly n steps."""
        full, r = divmod(n, len(self.sets))
        if full:
            g = self.graph(len(self.sets))
            for _ in range(full):
                g.replay()
        if r:
            self.graph(r).replay()


def time_steps(torch, run, warmup, steps):
    """run(warmup) untimed, then run(steps) bracketed by device
    synchronisation; returns the elapsed seconds of the timed steps."""
    run(warmup)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run(steps)
    torch.cuda.synchronize()
    return time.perf_counter() - t0


def time_graphs(torch, sets, step, warmup, steps):
    """`steps` graph-replayed steps in rotation over the buffer sets after
    `warmup`; returns the elapsed seconds."""
    return time_steps(torch, GraphSteps(torch, sets, step).prepare(warmup, steps).run, warmup,
                      steps)


def gate_cycles(torch, us):
    """Argument of torch.cuda._sleep that keeps the stream busy for about
    `us` microseconds (calibrated here)."""
    n = 1 << 20
    for _ in range(2):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        torch.cuda._sleep(n)
        b.record()
        torch.cuda.synchronize()
        per_us = n / max(a.elapsed_time(b) * 1e3, 1e-3)
    return int(per_us * us)


def percentiles(v, qs=(10, 50, 90)):
    """Nearest-rank percentiles of the values v."""
    v = sorted(v)
    out = {}
    for q in qs:
        i = min(len(v) - 1, max(0, int(round(q / 100.0 * len(v) + 0.5)) - 1))
        out["p%d" % q] = round(v[i], 5)
    return out


def clock_warmup(torch, run, ms):
    """Keep the device busy with back-to-back steps (run(n) enqueues n) for
    about `ms` milliseconds (untimed), so that what follows sees settled
    clocks and a warm launch path: a few steps estimate the step time, then
    the rest are enqueued without a synchronisation between them (an idle
    gap lets the clocks drop again).  Returns (steps run, ms spent)."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run(8)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    run(8)
    torch.cuda.synchronize()
    est = max((time.perf_counter() - t1) * 1e3 / 8, 1e-3)
    n = int(max(0.0, ms - (time.perf_counter() - t0) * 1e3) / est)
    run(n)
    torch.cuda.synchronize()
    return 16 + n, (time.perf_counter() - t0) * 1e3


def copy_probe_gbs(torch, dev, nbytes=COPY_PROBE_BYTES, reps=5):
    """Read + write bandwidth (GB/s) of a plain device-to-device copy."""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    del src, dst
    return 2.0 * nbytes * reps / el / 1e9


def dw7_baseline(L, torch, sets, wl, warmup, steps, stream, launch):
    """Step time of the 7x7 depthwise conv (forward + fused backward) on the
    same rotated activations, or None when the shape has no kernel."""
    k = 7
    dev = sets[0]["x"].device
    g = torch.Generator().manual_seed(1)
    w = (0.02 * torch.randn(wl.C, 1, k, k, generator=g)).to(sets[0]["x"].dtype).to(dev)
    b = (0.02 * torch.randn(wl.C, generator=g)).to(sets[0]["x"].dtype).to(dev)
    try:
        need = L.dwconv_workspace_size(L.dw_shape_of(sets[0]["x"], w))
    except L.WTConvError:
        return None
    ws = torch.empty(max(16, need), dtype=torch.uint8, device=dev)
    dw, db = torch.empty_like(w), torch.empty_like(b)

    def step(t, ev=None):
        st = torch.cuda.current_stream(dev)
        if ev is not None:
            ev[0].record(st)
        L.dwconv_fwd(t["x"], w, b, y=t["y"], stream=st)
        if ev is not None:
            ev[1].record(st)
        L.dwconv_bwd(t["x"], t["dy"], w, dx=t["dx"], dw=dw, db=db, workspace=ws, stream=st)
        if ev is not None:
            ev[2].record(st)

    def eager(n):
        for i in range(n):
            step(sets[i % len(sets)])

    el = time_steps(torch, eager, warmup, steps)
    gate = gate_cycles(torch, 400.0)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for i in range(steps):
        torch.cuda._sleep(gate)
        step(sets[i % len(sets)], evs[i])
    torch.cuda.synchronize()
    fwd_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / steps
    bwd_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / steps
    if launch == "graph":
        el = time_graphs(torch, sets, step, warmup, steps)
    return {"k": k, "ms_per_step": round(el * 1e3 / steps, 4),
            "images_per_s": round(wl.B * steps / el, 1),
            "per_call_ms": {"dwconv_fwd": round(fwd_ms, 5), "dwconv_bwd": round(bwd_ms, 5)},
            "inference_images_per_s": round(wl.B / (fwd_ms * 1e-3), 1)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # the clocks settle after some 30 ms of back-to-back work: the default
    # warmup (~60 ms at stage 1) is past that, so the timed steps see the
    # steady state a training run sees
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--workload", default="stage1")
    ap.add_argument("--sets", type=int, default=0, help="buffer sets to rotate (0 = auto)")
    ap.add_argument("--backward", choices=("fused", "split"), default="fused",
                    help="fused: wtconv_bwd; split: wtconv_bwd_input + wtconv_bwd_weight")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dw-baseline", action="store_true",
                    help="skip the 7x7 depthwise conv baseline")
    ap.add_argument("--launch", choices=("graph", "eager"), default="graph",
                    help="graph: time replays of one HIP graph per buffer set (the "
                         "step's kernels without host launch gaps); eager: time the "
                         "calls as issued.  Per-call times always come from an eager "
                         "pass with events between the calls")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run three plain device copies of 768 MiB at the end "
                         "(calibrates rocprofv3 byte counters)")
    ap.add_argument("--clock-warmup-ms", type=float, default=CLOCK_WARMUP_MS,
                    help="untimed steps for this much wall time before anything is timed")
    ap.add_argument("--valu-probe", action="store_true",
                    help="run the vector-ALU issue-rate probe (built by build()) and print "
                         "its JSON line: the fp32 FMA rate the roofline's 157.3 TFLOP/s "
                         "stands for")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of "
                         "'bench.py --copy-probe' into profiles/traffic_<workload>.json")
    args = ap.parse_args()
    if args.summarize_traffic:
        import wtconv_inputs as wi
        wl = wi.WORKLOADS[args.workload]
        act = wl.N * (4 if wl.dtype == "f32" else 2)
        fused = args.backward == "fused"
        summ = summarize_traffic(args.summarize_traffic[0], args.summarize_traffic[1], wl, act,
                                 fused)
        path = TRAFFIC_SUMMARY.format(workload=wl.name, backward=args.backward)
        with open(path, "w") as f:
            json.dump(summ, f, indent=1, sort_keys=True)
        print(json.dumps(summ, indent=1, sort_keys=True))
        return
    if args.valu_probe:
        import subprocess
        probe = os.path.join(ROOT, "aware_conv_amd", "valu_probe")
        if not os.path.exists(probe):
            sys.exit("valu_probe is not built: run __graft_entry__.build() first")
        r = subprocess.run([probe], capture_output=True, text=True, timeout=120)
        sys.stdout.write(r.stdout)
        sys.stderr.write(r.stderr)
        sys.exit(r.returncode)
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch

    import wtconv_inputs as wi
    from aware_conv_amd import _lib as L

    wl = wi.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    esz = 4 if wl.dtype == "f32" else 2
    act_bytes = wl.N * esz
    nsets = args.sets or max(1, min(8, int((1.2e9 + 4 * act_bytes - 1) // (4 * act_bytes))))
    host = wi.workload_inputs(wl)
    sets = []
    for i in range(nsets):
        t = {k: v.to(dev) for k, v in host.items()}
        if i:
            t["x"] = t["x"].roll(i, dims=0).contiguous()
            t["dy"] = t["dy"].roll(i, dims=0).contiguous()
        t["y"] = torch.empty_like(t["x"])
        t["dx"] = torch.empty_like(t["x"])
        t["g"] = {n: torch.empty_like(t[s]) for n, s in
                  zip(L.GRAD_NAMES, ("w_base", "b_base", "s_base", "w_wav", "s_wav"))}
        sets.append(t)
    shape = L.shape_of(sets[0]["x"], sets[0]["w_wav"])
    ws = torch.empty(max(16, L.wtconv_workspace_size(shape)), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    fused = args.backward == "fused"
    calls = (["wtconv_fwd", "wtconv_bwd"] if fused else
             ["wtconv_fwd", "wtconv_bwd_input", "wtconv_bwd_weight"])

    def step(t, ev=None):
        st = torch.cuda.current_stream(dev)  # the capture stream while capturing
        p = (t["w_base"], t["b_base"], t["s_base"], t["w_wav"], t["s_wav"])
        run = {
            "wtconv_fwd": lambda: L.wtconv_fwd(t["x"], *p, y=t["y"], workspace=ws, stream=st),
            "wtconv_bwd": lambda: L.wtconv_bwd(t["x"], t["dy"], *p, dx=t["dx"], grads=t["g"],
                                               workspace=ws, stream=st),
            "wtconv_bwd_input": lambda: L.wtconv_bwd_input(t["dy"], p[0], p[2], p[3], p[4],
                                                           dx=t["dx"], workspace=ws,
                                                           stream=st),
            "wtconv_bwd_weight": lambda: L.wtconv_bwd_weight(t["x"], t["dy"], *p, grads=t["g"],
                                                             workspace=ws, stream=st),
        }
        for i, c in enumerate(calls):
            if ev is not None:
                ev[i].record(st)
            run[c]()
        if ev is not None:
            ev[len(calls)].record(st)

    def eager(n, same=False):
        for i in range(n):
            step(sets[0 if same else i % nsets])

    eager(2)  # first calls: library loading, launch set-up
    torch.cuda.synchronize()
    if args.launch == "graph":
        rot = GraphSteps(torch, sets, step).prepare(args.warmup, args.steps, 8)
        same = GraphSteps(torch, sets, step, same=True).prepare(args.warmup, args.steps)
        run = rot.run
    else:
        run = eager
    # the timed steps first, right after the warm-up, in the launch mode
    # they are timed in
    cw_steps, cw_ms = clock_warmup(torch, run, args.clock_warmup_ms)
    elapsed = time_steps(torch, run, args.warmup, args.steps)
    if args.launch == "graph":
        warm_el = time_steps(torch, same.run, args.warmup, args.steps)
        del rot, same
    else:
        warm_el = time_steps(torch, lambda n: eager(n, True), args.warmup, args.steps)
    eager_el = time_steps(torch, eager, args.warmup, args.steps)
    eager_ms_step = eager_el * 1e3 / args.steps
    # Per-call device time: every step waits behind a short spin kernel, so
    # that its calls are all enqueued before the device reaches them and the
    # events between them see kernel time only, not the host's launch work.
    gate = gate_cycles(torch, 400.0)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)]
           for _ in range(args.steps)]
    for i in range(args.steps):
        torch.cuda._sleep(gate)
        step(sets[i % nsets], evs[i])
    torch.cuda.synchronize()
    per = {c: [e[i].elapsed_time(e[i + 1]) for e in evs] for i, c in enumerate(calls)}
    avg_ms = {k: sum(v) / len(v) for k, v in per.items()}
    step_pct = percentiles([e[0].elapsed_time(e[len(calls)]) for e in evs])

    dw = None
    if not args.no_dw_baseline:
        dw = dw7_baseline(L, torch, sets, wl, args.warmup, args.steps, stream, args.launch)

    copy_gbs = copy_probe_gbs(torch, dev)

    if args.copy_probe:
        src = torch.ones(COPY_PROBE_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    ms_step = elapsed * 1e3 / args.steps
    value = wl.B * args.steps / elapsed
    flops_pass = wl.N * conv_flops_per_pixel(wl.L, wl.k)
    # algorithmic bytes and conv passes of each call: activations read and
    # written; the input gradient and the weight taps are one pass each
    algo_bytes = {"wtconv_fwd": 2 * act_bytes, "wtconv_bwd_input": 2 * act_bytes,
                  "wtconv_bwd_weight": 2 * act_bytes, "wtconv_bwd": 3 * act_bytes}
    passes = {"wtconv_fwd": 1, "wtconv_bwd_input": 1, "wtconv_bwd_weight": 1, "wtconv_bwd": 2}
    dom = max(avg_ms, key=avg_ms.get)
    dur_s = avg_ms[dom] * 1e-3
    traffic = None
    tpath = TRAFFIC_SUMMARY.format(workload=wl.name, backward=args.backward)
    if os.path.exists(tpath):
        with open(tpath) as f:
            tr = json.load(f)
        if tr.get("source_sha256_16") == source_hash() and dom in tr.get("bytes_per_launch", {}):
            traffic = tr["bytes_per_launch"][dom]
    step_bytes = sum(algo_bytes[c] for c in calls)
    rec = {
        "metric": "fused WTConv fwd+bwd images/s and effective HBM GB/s (% of peak), 1xMI355X",
        "value": round(value, 1),
        "unit": "images/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if wl.dtype == "f32" else "f16 storage, f32 accumulate",
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02^2) filters)",
        "config": {"workload": wl.name, "B": wl.B, "C": wl.C, "H": wl.H, "W": wl.W,
                   "levels": wl.L, "k": wl.k, "backward": args.backward,
                   "launch": args.launch, "buffer_sets": nsets},
        "eager_ms_per_step": round(eager_ms_step, 4),
        "clock_warmup_ms": round(cw_ms, 1),
        "clock_warmup_steps": cw_steps,
        "step_ms": dict(step_pct, mean=round(ms_step, 5),
                        warm_mean=round(warm_el * 1e3 / args.steps, 5)),
        "step_algo_bytes": step_bytes,
        "effective_hbm_gbs": round(step_bytes / (elapsed / args.steps) / 1e9, 1),
        "effective_hbm_frac": round(step_bytes / (elapsed / args.steps) / 1e9 / PEAK_HBM_GBS, 4),
        "copy_probe": {"gbs": round(copy_gbs, 1), "frac_of_peak": round(copy_gbs / PEAK_HBM_GBS, 4),
                       "effective_hbm_frac_of_copy": round(
                           step_bytes / (elapsed / args.steps) / 1e9 / copy_gbs, 4)},
        "valu_frac": round(sum(passes[c] for c in calls) * flops_pass / (elapsed / args.steps) /
                           1e12 / PEAK_FP32_VALU_TFLOPS, 4),
        "per_call_ms": {k: round(v, 5) for k, v in avg_ms.items()},
        # inference alone: the forward call of the same timed steps
        "inference_images_per_s": round(wl.B / (avg_ms["wtconv_fwd"] * 1e-3), 1),
        "roofline": roofline(dom, passes[dom] * flops_pass, algo_bytes[dom], dur_s, traffic, wl.N),
    }
    if dw is not None:
        dw["wtconv_over_dw_train"] = round(value / dw["images_per_s"], 3)
        dw["wtconv_over_dw_infer"] = round(rec["inference_images_per_s"] /
                                           dw["inference_images_per_s"], 3)
        rec["dw7x7_baseline"] = dw
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
