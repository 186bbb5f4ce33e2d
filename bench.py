"""Benchmark: DCNv4 forward GB/s, Gsamples/s and fraction of MI355X HBM peak.

    python bench.py [--gpus 1] [--steps 200] [--warmup 20] [--workload fiit_stage1] [--dtype f16]

One step = one launch of the whole operator (sampling, bilinear interpolation
and weighted aggregation fused in one kernel) over one batch of the workload.
Inputs are seeded and synthetic and already resident in HBM.  To keep each
launch reading HBM rather than the 256 MB Infinity Cache, the timed loop
rotates over several copies of the inputs (at least 1 GiB in all), so a copy
is reused only after >= 1 GiB of other traffic.

Before the W warmup launches, --spinup-s seconds (default 1) of the same
launches run untimed: the GPU leaves its idle clocks and every rotating copy
is touched, so that the K timed launches measure the steady state (measured
on the stage-1 f16 shape: 43-44 us per launch after 20 warmup launches
alone, 39 us after about a second of launches).  The JSON records the
spin-up.

Printed: one JSON line.  `value` = algorithmic bytes per step / wall-clock
time per step over the timed region.  `roofline.achieved` = the same bytes /
the kernel's mean launch duration, taken from two HIP events recorded on the
launch stream around the timed region (K back-to-back launches; the queue
stays full, so this is the kernel's duration plus the dispatch gap).
Algorithmic bytes per (pixel, group) unit = (2*Cg + 3*P)*s: x read once, out
written once, 2P offsets and P weights read once.  `roofline.traffic` = HBM
bytes per launch measured by rocprofv3 counters on the same kernel source
(profiles/<workload>_<dtype>_hbm_counters.json), else null; `l2_hit`
= the L2 hit rate from the same counter runs (TCC_HIT / (TCC_HIT + TCC_MISS)).
`configs` = every other measured configuration (the five workloads' I/O
types), event-timed in the same run the same way, with each one's fraction
of sampling points outside the image, and the stage-1 shape with spatially
smooth offsets (a sensitivity input, marked as such); then the backward, the DCNv3-style
variant and the module forward on the named workload (algorithmic bytes:
the backward's inputs read and binary32 gradients written; the module's
input read, output written and weights).  `cpu_baseline` = the CPU oracle on
one thread and on all the cores the process may use (one thread per slice of
images; the oracle itself stays single-threaded code).
"""
import argparse
import dataclasses
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0   # MI355X HBM3E, 8 TB/s
PROFILES = os.path.join(ROOT, "profiles")


def load_counters(workload, dtype):
    """The committed rocprofv3 counter record of a workload (HBM bytes per
    launch, L2 hits and misses), if it was taken on the current source of the
    forward operator's kernels; else None."""
    path = os.path.join(PROFILES, f"{workload}_{dtype}_hbm_counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    from deformable_convolution_vision_dcnv4_amd.build import source_hash
    if rec.get("kernel_source_hash") != source_hash("forward"):
        return None
    return rec


def _oracle_rate(wl, dtype, x, off, m, budget_s, threads):
    """Whole passes of the oracle over the first n images, n sized so that a
    pass takes about budget_s (repeated while under budget_s), the images
    split into `threads` contiguous slices run on as many threads (ctypes
    releases the GIL for the C call).  Returns (bytes/s, samples/s, n, reps, s)."""
    import concurrent.futures
    from oracle import ref
    kw = dict(K=wl.K, stride=wl.stride, pad=wl.pad, dil=wl.dil, offset_scale=wl.offset_scale,
              remove_center=wl.remove_center)
    t0 = time.perf_counter()
    ref.forward_f32(x[:1], off[:1], m[:1], dtype=dtype, **kw)
    per_img = max(time.perf_counter() - t0, 1e-6)
    n = int(max(threads, min(wl.N, budget_s * threads / per_img)))
    n = min(n, wl.N)
    bounds = [(i * n // threads, (i + 1) * n // threads) for i in range(threads)]
    bounds = [b for b in bounds if b[1] > b[0]]

    def part(b):
        ref.forward_f32(x[b[0]:b[1]], off[b[0]:b[1]], m[b[0]:b[1]], dtype=dtype, **kw)

    reps = 0
    with concurrent.futures.ThreadPoolExecutor(len(bounds)) as ex:
        t0 = time.perf_counter()
        while True:
            list(ex.map(part, bounds))
            reps += 1
            dt = time.perf_counter() - t0
            if dt >= budget_s or dt + dt / reps > 3 * budget_s:
                break
    frac = n / wl.N * reps
    return wl.algorithmic_bytes(dtype) * frac / dt, wl.samples() * frac / dt, n, reps, dt, len(bounds)


def cpu_baseline(wl, dtype, x, off, m, budget_s):
    """The CPU oracle (plain C, as it stands) on the same inputs: one thread,
    then one thread per slice of images on every core the process may use
    (at most 16, the host share of one GPU)."""
    cores = max(1, min(16, len(os.sched_getaffinity(0))))
    b1, s1, n1, r1, t1, _ = _oracle_rate(wl, dtype, x, off, m, budget_s, 1)
    bc, sc, nc, rc, tc, used = _oracle_rate(wl, dtype, x, off, m, budget_s, cores)
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as fh:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")), "")
    except OSError:
        pass
    return {"value": round(bc / 1e9, 4), "unit": "GB/s", "cores": used, "kind": "oracle",
            "sample": f"{rc} pass(es) over {nc} of the workload's {wl.N} images (same inputs) split over {used} "
                      f"threads, binary32-sequence oracle (plain C, single-threaded code), {tc:.1f} s; "
                      f"one thread: {r1} pass(es) over {n1} images, {t1:.1f} s",
            "gsamples_per_s": round(sc / 1e9, 6),
            "single_thread": {"value": round(b1 / 1e9, 4), "unit": "GB/s", "cores": 1,
                              "gsamples_per_s": round(s1 / 1e9, 6)},
            "cpu_model": cpu_model}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="fiit_stage1")
    ap.add_argument("--op", default="forward", choices=("forward", "backward", "softmax", "module"),
                    help="forward (the headline), the backward (gradients of x, offsets, weights), "
                         "softmax (the DCNv3-style aggregation, for comparison), or module (the module "
                         "forward around the operator: projection, group norm, predictor, operator, "
                         "centre gate, output projection, C in and out)")
    ap.add_argument("--dtype", default=None, help="f32 | f16 | bf16 (default: the workload's last)")
    ap.add_argument("--batch", type=int, default=None,
                    help="run the workload's shape at this batch size instead of its own")
    ap.add_argument("--rotate-bytes", type=float, default=1.0, help="GiB of rotating input copies")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true", help="time the named workload only")
    ap.add_argument("--config-steps", type=int, default=50, help="timed launches per other configuration")
    ap.add_argument("--spinup-s", type=float, default=1.0,
                    help="seconds of the workload's own launches before the warmup steps, so that the timed "
                         "launches run at the GPU's steady clocks with every rotating copy touched (0: none)")
    ap.add_argument("--quiet", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the operator is measured on one GPU's share "
              "(running it sharded over several GPUs is not implemented); use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from deformable_convolution_vision_dcnv4_amd import binding
    from deformable_convolution_vision_dcnv4_amd import inputs as gen
    from deformable_convolution_vision_dcnv4_amd.workloads import CONFIGS, SENSITIVITY, WORKLOADS, oob_fractions

    def log(*a):
        if not args.quiet:
            print("[bench]", *a, file=sys.stderr, flush=True)

    wl = WORKLOADS[args.workload] if args.workload in WORKLOADS else SENSITIVITY[args.workload]
    if args.batch is not None and args.batch != wl.N:
        if args.batch < 1:
            ap.error("--batch must be at least 1")
        wl = dataclasses.replace(wl, name=f"{wl.name}_n{args.batch}", N=args.batch)
    dtype = args.dtype or wl.dtypes[-1]
    assert dtype in ("f32", "f16", "bf16")
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    binding.lib()

    def spin_up(step, seconds):
        """Launch `step` back to back for about `seconds` (untimed): the GPU
        leaves its idle clocks and every rotating copy's pages are touched."""
        if seconds <= 0:
            return 0
        n, t0 = 0, time.perf_counter()
        while True:
            for _ in range(64):
                step(n)
                n += 1
            torch.cuda.synchronize()
            if time.perf_counter() - t0 >= seconds:
                return n

    def measure(wl, dtype, op, steps, warmup, rotate_gib, per_launch=True, spinup_s=0.0):
        """Time `steps` back-to-back launches of `op` on wl's synthetic inputs
        (resident in HBM, rotating over >= rotate_gib GiB of copies), after
        spinup_s seconds of untimed launches and `warmup` warmup launches."""
        tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]
        dcode = {"f32": binding.F32, "f16": binding.F16, "bf16": binding.BF16}[dtype]
        log(f"workload {wl.describe(dtype)}; generating inputs (seed {wl.seed})")
        x, off, m = gen.make_inputs(wl, dtype)

        def to_dev(a):
            if dtype == "bf16":
                return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
            return torch.from_numpy(a).to(dev)

        Ho, Wo = wl.out_hw()
        set_bytes = (x.nbytes + off.nbytes + m.nbytes + wl.N * Ho * Wo * wl.C * x.itemsize)
        copies = int(min(64, max(2, -(-rotate_gib * (1 << 30) // set_bytes))))
        xs0, os0, ms0 = to_dev(x), to_dev(off), to_dev(m)
        sets = []
        for i in range(copies):
            xi, oi, mi = (xs0, os0, ms0) if i == 0 else (xs0.clone(), os0.clone(), ms0.clone())
            outi = torch.empty((wl.N, Ho, Wo, wl.C), dtype=tdt, device=dev)
            sets.append((xi, oi, mi, outi))
        torch.cuda.synchronize()
        log(f"{copies} rotating input copies, {copies * set_bytes / 2**30:.2f} GiB")

        stream = torch.cuda.current_stream()
        sptr = stream.cuda_stream
        L = binding.lib()
        argv = [(st[0].data_ptr(), st[1].data_ptr(), st[2].data_ptr(), st[3].data_ptr(), wl.N, wl.H, wl.W,
                 wl.G, wl.Cg, wl.K, wl.stride, wl.pad, wl.dil, wl.offset_scale, dcode, sptr) for st in sets]
        fwd = L.dcnv4_forward
        if op == "backward":
            # grad_out: a copy of the output-shaped buffer filled with the forward's result;
            # gradients in binary32, one set shared by all steps (each step overwrites them)
            Pn = wl.P
            gx = torch.empty((wl.N, wl.H, wl.W, wl.C), dtype=torch.float32, device=dev)
            goff = torch.empty((wl.N, Ho, Wo, wl.G * 2 * Pn), dtype=torch.float32, device=dev)
            gm = torch.empty((wl.N, Ho, Wo, wl.G * Pn), dtype=torch.float32, device=dev)
            for a in argv:
                assert fwd(*a) == 0
            torch.cuda.synchronize()
            bargv = [(st[0].data_ptr(), st[1].data_ptr(), st[2].data_ptr(), st[3].data_ptr(), gx.data_ptr(),
                      goff.data_ptr(), gm.data_ptr(), wl.N, wl.H, wl.W, wl.G, wl.Cg, wl.K, wl.stride, wl.pad,
                      wl.dil, wl.offset_scale, int(wl.remove_center), 0, 0, dcode, sptr) for st in sets]
            bwd = L.dcnv4_backward
        if op == "softmax":
            sm = L.dcnv4_forward_softmax
            smargv = [a[:14] + (int(wl.remove_center), 0, 0) + a[14:] for a in argv]

        def step(i):
            if op == "backward":
                st = bwd(*bargv[i % copies])
            elif op == "softmax":
                st = sm(*smargv[i % copies])
            else:
                st = fwd(*argv[i % copies])
            if st != 0:
                raise RuntimeError(f"dcnv4 {op} failed: {binding.status_string(st)}: {binding.last_error()}")

        plan = binding.query_plan(sets[0][0], sets[0][1], sets[0][2], sets[0][3], kernel_size=wl.K,
                                  stride=wl.stride, pad=wl.pad, dilation=wl.dil, offset_scale=wl.offset_scale)
        log(f"plan {plan}")

        nspin = spin_up(step, spinup_s)
        if nspin:
            log(f"spin-up: {nspin} launches in about {spinup_s:.2f} s")
        for i in range(warmup):
            step(i)
        torch.cuda.synchronize()
        log(f"warmup {warmup} done")

        # timed region: K back-to-back launches between two events on the launch stream
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev0.record(stream)
        for i in range(steps):
            step(i)
        ev1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        region_ms = ev0.elapsed_time(ev1)
        kern_ms = region_ms / steps
        log(f"timed {steps} steps: wall {wall * 1e3:.3f} ms, events {region_ms:.3f} ms, "
            f"{kern_ms * 1e3:.2f} us per launch")
        r = {"wall_s": wall, "kern_ms": kern_ms, "copies": copies, "plan": plan, "inputs": (x, off, m),
             "spinup_launches": nspin}
        if per_launch:
            # secondary: one event pair per launch (adds the events' own cost; for a
            # short kernel it also shows host-side launch latency)
            starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
            ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
            for i in range(steps):
                starts[i].record(stream)
                step(i)
                ends[i].record(stream)
            torch.cuda.synchronize()
            durs = np.array([a.elapsed_time(b) for a, b in zip(starts, ends)])  # ms
            log(f"per-launch event pairs: median {np.median(durs) * 1e3:.2f} us, "
                f"p10 {np.percentile(durs, 10) * 1e3:.2f} us, p90 {np.percentile(durs, 90) * 1e3:.2f} us")
            r["median_ms"] = float(np.median(durs))
        del sets
        torch.cuda.empty_cache()
        return r

    if args.op == "module":
        return bench_module(args, wl, dtype, log)
    r = measure(wl, dtype, args.op, args.steps, args.warmup, args.rotate_bytes, spinup_s=args.spinup_s)
    x, off, m = r["inputs"]
    alg_bytes = wl.backward_bytes(dtype) if args.op == "backward" else wl.algorithmic_bytes(dtype)
    ms_per_step = r["wall_s"] * 1e3 / args.steps
    kern_ms = r["kern_ms"]
    value = alg_bytes / (ms_per_step * 1e-3) / 1e9
    achieved = alg_bytes / (kern_ms * 1e-3) / 1e9
    counters = load_counters(wl.name if args.op == "forward" else f"{wl.name}_{args.op}", dtype)

    # the other configurations, timed the same way (launch-to-launch events)
    configs = []
    if args.op == "forward" and not args.no_configs and args.batch is None:
        # then the sensitivity inputs (smooth offsets), marked as such
        sens = [(n, d) for n, swl in SENSITIVITY.items() for d in swl.dtypes]
        for name, cdt in list(CONFIGS) + sens:
            if (name, cdt) == (wl.name, dtype):
                continue
            cwl = WORKLOADS[name] if name in WORKLOADS else SENSITIVITY[name]
            cr = measure(cwl, cdt, "forward", args.config_steps, max(5, args.warmup // 4), args.rotate_bytes,
                         per_launch=False, spinup_s=min(args.spinup_s, 0.3))
            cbytes = cwl.algorithmic_bytes(cdt)
            ccnt = load_counters(name, cdt)
            oob, corner = oob_fractions(cwl, gen.as_f64(cr["inputs"][1], cdt))
            configs.append({
                "workload": cwl.describe(cdt), "dtype": cdt, "op": "forward",
                "kernel_us_mean": round(cr["kern_ms"] * 1e3, 3),
                "gbs": round(cbytes / (cr["kern_ms"] * 1e-3) / 1e9, 2),
                "hbm_fraction": round(cbytes / (cr["kern_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "gsamples_per_s": round(cwl.samples() / (cr["kern_ms"] * 1e-3) / 1e9, 3),
                "algorithmic_bytes": cbytes, "steps": args.config_steps,
                "plan": {k: cr["plan"][k] for k in ("kernel", "lanes_per_unit", "block", "grid", "tile_h", "tile_w",
                                                      "full_window")},
                "points_outside": round(oob, 4), "points_with_a_corner_outside": round(corner, 4),
                "l2_hit": ccnt.get("l2_hit") if ccnt else None,
                "hbm_traffic": ccnt.get("hbm_bytes_per_launch") if ccnt else None,
            })
            if name in SENSITIVITY:
                configs[-1]["sensitivity"] = (f"offsets box-filtered over {2 * cwl.offset_smooth + 1}x"
                                              f"{2 * cwl.offset_smooth + 1} output pixels, same standard "
                                              "deviation; reported beside the workloads, not instead of them")
        # the other operations on this workload: backward, the DCNv3-style
        # variant and the whole module forward, event-timed the same way
        from deformable_convolution_vision_dcnv4_amd.workloads import module_bytes
        for cop in ("backward", "softmax", "module"):
            if cop == "module":
                cr = time_module(wl, dtype, args.config_steps, max(5, args.warmup // 4), log,
                                 spinup_s=min(args.spinup_s, 0.3))
                cbytes = module_bytes(wl, dtype)
            else:
                cr = measure(wl, dtype, cop, args.config_steps, max(5, args.warmup // 4), args.rotate_bytes,
                             per_launch=False, spinup_s=min(args.spinup_s, 0.3))
                cbytes = wl.backward_bytes(dtype) if cop == "backward" else wl.algorithmic_bytes(dtype)
            configs.append({
                "workload": wl.describe(dtype), "dtype": dtype, "op": cop,
                "kernel_us_mean": round(cr["kern_ms"] * 1e3, 3),
                "gbs": round(cbytes / (cr["kern_ms"] * 1e-3) / 1e9, 2),
                "hbm_fraction": round(cbytes / (cr["kern_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "algorithmic_bytes": cbytes, "steps": args.config_steps,
            })

    cpu = None
    if not args.no_cpu_baseline and args.op == "forward":
        log("timing the CPU oracle baseline")
        cpu = cpu_baseline(wl, dtype, x, off, m, args.cpu_budget)

    oob, corner = oob_fractions(wl, gen.as_f64(off, dtype))
    rec = {
        "metric": {"forward": "DCNv4 fwd GB/s + Gsamples/s per MI355X; % of HBM roofline",
                   "backward": "DCNv4 bwd GB/s + Gsamples/s per MI355X; % of HBM roofline",
                   "softmax": "DCNv3-style (softmax weights) fwd GB/s + Gsamples/s per MI355X; % of HBM roofline"}[args.op],
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic (seeded counter-based generator; no dataset, no trained weights)",
        "config": {
            "workload": wl.describe(dtype),
            "op": args.op,
            "N": wl.N, "H": wl.H, "W": wl.W, "G": wl.G, "Cg": wl.Cg, "K": wl.K,
            "stride": wl.stride, "pad": wl.pad, "dilation": wl.dil, "offset_scale": wl.offset_scale,
            "inputs": {"x": list(wl.x_dist), "offset": list(wl.offset_dist), "mask": list(wl.mask_dist),
                       "seed": wl.seed, "offset_smooth_radius": wl.offset_smooth},
            "algorithmic_bytes_per_step": alg_bytes,
            "samples_per_step": wl.samples(),
            "rotating_copies": r["copies"],
            "spinup": {"seconds": args.spinup_s, "launches": r["spinup_launches"]},
            "plan": r["plan"],
            "points_outside": round(oob, 4),
            "points_with_a_corner_outside": round(corner, 4),
        },
        "gsamples_per_s": round(wl.samples() / (ms_per_step * 1e-3) / 1e9, 3),
        "hbm_fraction": round(value / HBM_PEAK_GBS, 4),
        "kernel_us_mean": round(kern_ms * 1e3, 3),
        "per_launch_event_us_median": round(r["median_ms"] * 1e3, 3),
        "l2_hit": counters.get("l2_hit") if counters else None,
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": counters.get("hbm_bytes_per_launch") if counters else None,
        },
        "configs": configs,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


def time_module(wl, dtype, steps, warmup, log, spinup_s=0.0):
    """Time the module forward (group norm over min(32, C) groups, centre gate,
    output projection; Cin = Cout = C) on seeded random weights: the wall
    time and the event time of `steps` back-to-back forwards."""
    import numpy as np
    import torch

    from deformable_convolution_vision_dcnv4_amd import binding
    from deformable_convolution_vision_dcnv4_amd import inputs as gen

    dev = torch.device("cuda:0")
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]
    C, G, P = wl.C, wl.G, wl.P
    R = 3 * G * P + G
    rng = np.random.default_rng(wl.seed)

    def mat(shape, std):
        h = gen.to_io(rng.standard_normal(shape) * std, dtype)
        if dtype == "bf16":
            return torch.from_numpy(h.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(h).to(dev)

    def vec(shape, std, mean=0.0):
        return torch.from_numpy((mean + rng.standard_normal(shape) * std).astype(np.float32)).to(dev)

    scale = np.concatenate([np.full(2 * G * P, 1.5), np.full(G * P, 0.5), np.full(G, 1.0)])[:, None]
    w_pred = gen.to_io(rng.standard_normal((R, C)) * scale / np.sqrt(C), dtype)
    weights = {"w_in": mat((C, C), 1 / np.sqrt(C)), "b_in": vec(C, 0.1), "gamma": vec(C, 0.1, 1.0),
               "beta": vec(C, 0.1), "w_dw": vec((C, 3, 3), 1 / 3), "b_dw": vec(C, 0.05),
               "w_pred": (torch.from_numpy(w_pred.view(np.int16)).view(torch.bfloat16) if dtype == "bf16"
                          else torch.from_numpy(w_pred)).to(dev),
               "b_pred": vec(R, 0.1), "w_out": mat((C, C), 1 / np.sqrt(C)), "b_out": vec(C, 0.1)}
    cfg = binding.module_config(Cin=C, G=G, Cg=wl.Cg, Cout=C, norm=binding.NORM_GROUP, norm_groups=min(32, C),
                                eps=1e-5, center_scale=True, out_proj=True)
    log(f"module on {wl.describe(dtype)}: generating inputs")
    x = gen.to_io(gen.draw(wl.seed, gen.STREAM_X, wl.N * wl.H * wl.W * C, wl.x_dist), dtype)
    xs = (torch.from_numpy(x.view(np.int16)).view(torch.bfloat16) if dtype == "bf16"
          else torch.from_numpy(x)).to(dev).reshape(wl.N, wl.H, wl.W, C)
    lay = binding.module_layout(wl.N, wl.H, wl.W, cfg, tdt)
    ws = torch.empty(lay["total"], dtype=torch.uint8, device=dev)
    out = torch.empty((wl.N, wl.H, wl.W, C), dtype=tdt, device=dev)
    t_spin = time.perf_counter()
    while spinup_s > 0 and time.perf_counter() - t_spin < spinup_s:
        for _ in range(16):
            binding.module_forward(xs, weights, cfg, out=out, workspace=ws)
        torch.cuda.synchronize()
    for _ in range(warmup):
        binding.module_forward(xs, weights, cfg, out=out, workspace=ws)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(steps):
        binding.module_forward(xs, weights, cfg, out=out, workspace=ws)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev0.elapsed_time(ev1) / steps
    log(f"timed {steps} module forwards: {ms * 1e3:.2f} us each (events), workspace {lay['total'] / 2**20:.1f} MiB")
    return {"wall_s": wall, "kern_ms": ms, "workspace_bytes": lay["total"], "norm_groups": min(32, C)}


def bench_module(args, wl, dtype, log):
    """The module forward's JSON line (--op module)."""
    from deformable_convolution_vision_dcnv4_amd.workloads import module_bytes

    r = time_module(wl, dtype, args.steps, args.warmup, log, spinup_s=args.spinup_s)
    ms = r["kern_ms"]
    alg = module_bytes(wl, dtype)
    ms_step = r["wall_s"] * 1e3 / args.steps
    C = wl.C
    rec = {
        "metric": "DCNv4 module fwd GB/s per MI355X (x in + out + weights); % of HBM roofline",
        "value": round(alg / (ms_step * 1e-3) / 1e9, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 6), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": dtype,
        "data": "synthetic (seeded inputs and random weights; no dataset, no trained weights)",
        "config": {"workload": wl.describe(dtype), "op": "module", "norm": "group", "norm_groups": r["norm_groups"],
                   "center_scale": True, "out_proj": True, "Cin": C, "Cout": C,
                   "algorithmic_bytes_per_step": alg, "workspace_bytes": r["workspace_bytes"]},
        "kernel_us_mean": round(ms * 1e3, 3),
        "roofline": {"bound": "hbm", "achieved": round(alg / (ms * 1e-3) / 1e9, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "traffic": None},
        "cpu_baseline": None,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
