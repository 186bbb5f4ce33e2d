"""Benchmark: DCNv4 forward GB/s, Gsamples/s and fraction of MI355X HBM peak.

    python bench.py [--gpus 1] [--steps 200] [--warmup 20] [--workload fiit_stage1] [--dtype f16]

One step = one launch of the whole operator (sampling, bilinear interpolation
and weighted aggregation fused in one kernel) over one batch of the workload.
Inputs are seeded and synthetic and already resident in HBM.  To keep each
launch reading HBM rather than the 256 MB Infinity Cache, the timed loop
rotates over several copies of the inputs (at least 1 GiB in all), so a copy
is reused only after >= 1 GiB of other traffic.

Printed: one JSON line.  `value` = algorithmic bytes per step / wall-clock
time per step over the timed region.  `roofline.achieved` = the same bytes /
the kernel's mean launch duration, taken from two HIP events recorded on the
launch stream around the timed region (K back-to-back launches; the queue
stays full, so this is the kernel's duration plus the dispatch gap).
Algorithmic bytes per (pixel, group) unit = (2*Cg + 3*P)*s: x read once, out
written once, 2P offsets and P weights read once.  `roofline.traffic` = HBM
bytes per launch measured by rocprofv3 counters on the same kernel source
(profiles/<workload>_<dtype>_hbm_counters.json), else null.
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


def load_traffic(workload, dtype, launches_bytes):
    """HBM traffic per launch from committed rocprofv3 counter runs, if they
    were taken on the current kernel source; else None."""
    path = os.path.join(PROFILES, f"{workload}_{dtype}_hbm_counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    from deformable_convolution_vision_dcnv4_amd.build import source_hash
    if rec.get("kernel_source_hash") != source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(wl, dtype, x, off, m, budget_s):
    """The CPU oracle (single-threaded C, as it stands) on the same inputs.

    A bounded sample: whole passes over the first n images, n sized so that
    one pass takes about budget_s; if the whole batch takes less, the batch is
    repeated until about budget_s of CPU time has been spent."""
    from oracle import ref
    kw = dict(K=wl.K, stride=wl.stride, pad=wl.pad, dil=wl.dil, offset_scale=wl.offset_scale,
              remove_center=wl.remove_center)
    t0 = time.perf_counter()
    ref.forward_f32(x[:1], off[:1], m[:1], dtype=dtype, **kw)
    per_img = max(time.perf_counter() - t0, 1e-6)
    n = int(max(1, min(wl.N, budget_s / per_img)))
    reps = 0
    t0 = time.perf_counter()
    while True:
        ref.forward_f32(x[:n], off[:n], m[:n], dtype=dtype, **kw)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= budget_s or dt + dt / reps > 3 * budget_s:
            break
    bytes_ = wl.algorithmic_bytes(dtype) * n / wl.N * reps
    return {"value": round(bytes_ / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{reps} pass(es) over {n} of the workload's {wl.N} images (same inputs), "
                      f"binary32-sequence oracle (plain C, one thread), {dt:.1f} s",
            "gsamples_per_s": round(wl.samples() * n / wl.N * reps / dt / 1e9, 6)}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="fiit_stage1")
    ap.add_argument("--op", default="forward", choices=("forward", "backward", "softmax"),
                    help="forward (the headline), the backward (gradients of x, offsets, weights), or "
                         "softmax (the DCNv3-style aggregation, for comparison)")
    ap.add_argument("--dtype", default=None, help="f32 | f16 | bf16 (default: the workload's last)")
    ap.add_argument("--batch", type=int, default=None,
                    help="run the workload's shape at this batch size instead of its own")
    ap.add_argument("--rotate-bytes", type=float, default=1.0, help="GiB of rotating input copies")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--quiet", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the operator is measured on one GPU's share "
              "(multi-GPU sharding is not part of this build); use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from deformable_convolution_vision_dcnv4_amd import binding
    from deformable_convolution_vision_dcnv4_amd import inputs as gen
    from deformable_convolution_vision_dcnv4_amd.workloads import WORKLOADS

    def log(*a):
        if not args.quiet:
            print("[bench]", *a, file=sys.stderr, flush=True)

    wl = WORKLOADS[args.workload]
    if args.batch is not None and args.batch != wl.N:
        if args.batch < 1:
            ap.error("--batch must be at least 1")
        wl = dataclasses.replace(wl, name=f"{wl.name}_n{args.batch}", N=args.batch)
    dtype = args.dtype or wl.dtypes[-1]
    assert dtype in ("f32", "f16", "bf16")
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]
    dcode = {"f32": binding.F32, "f16": binding.F16, "bf16": binding.BF16}[dtype]
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    binding.lib()

    log(f"workload {wl.describe(dtype)}; generating inputs (seed {wl.seed})")
    x, off, m = gen.make_inputs(wl, dtype)

    def to_dev(a):
        if dtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    Ho, Wo = wl.out_hw()
    set_bytes = (x.nbytes + off.nbytes + m.nbytes + wl.N * Ho * Wo * wl.C * x.itemsize)
    copies = int(min(64, max(2, -(-args.rotate_bytes * (1 << 30) // set_bytes))))
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
    argv = [(s[0].data_ptr(), s[1].data_ptr(), s[2].data_ptr(), s[3].data_ptr(), wl.N, wl.H, wl.W,
             wl.G, wl.Cg, wl.K, wl.stride, wl.pad, wl.dil, wl.offset_scale, dcode, sptr) for s in sets]
    fwd = L.dcnv4_forward
    if args.op == "backward":
        # grad_out: a copy of the output-shaped buffer filled with the forward's result;
        # gradients in binary32, one set shared by all steps (each step overwrites them)
        Pn = wl.P
        gx = torch.empty((wl.N, wl.H, wl.W, wl.C), dtype=torch.float32, device=dev)
        goff = torch.empty((wl.N, Ho, Wo, wl.G * 2 * Pn), dtype=torch.float32, device=dev)
        gm = torch.empty((wl.N, Ho, Wo, wl.G * Pn), dtype=torch.float32, device=dev)
        for a in argv:
            assert fwd(*a) == 0
        torch.cuda.synchronize()
        bargv = [(s[0].data_ptr(), s[1].data_ptr(), s[2].data_ptr(), s[3].data_ptr(), gx.data_ptr(),
                  goff.data_ptr(), gm.data_ptr(), wl.N, wl.H, wl.W, wl.G, wl.Cg, wl.K, wl.stride, wl.pad,
                  wl.dil, wl.offset_scale, int(wl.remove_center), 0, 0, dcode, sptr) for s in sets]
        bwd = L.dcnv4_backward

    if args.op == "softmax":
        sm = L.dcnv4_forward_softmax
        smargv = [a[:14] + (int(wl.remove_center), 0, 0) + a[14:] for a in argv]

    def step(i):
        if args.op == "backward":
            st = bwd(*bargv[i % copies])
        elif args.op == "softmax":
            st = sm(*smargv[i % copies])
        else:
            st = fwd(*argv[i % copies])
        if st != 0:
            raise RuntimeError(f"dcnv4 {args.op} failed: {binding.status_string(st)}: {binding.last_error()}")

    plan = binding.query_plan(sets[0][0], sets[0][1], sets[0][2], sets[0][3], kernel_size=wl.K,
                              stride=wl.stride, pad=wl.pad, dilation=wl.dil, offset_scale=wl.offset_scale)
    log(f"plan {plan}")

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} done")

    # timed region: K back-to-back launches between two events on the launch stream
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    region_ms = ev0.elapsed_time(ev1)
    kern_ms = region_ms / args.steps
    log(f"timed {args.steps} steps: wall {wall * 1e3:.3f} ms, events {region_ms:.3f} ms, "
        f"{kern_ms * 1e3:.2f} us per launch")

    # secondary: one event pair per launch (adds the events' own cost; for a
    # short kernel it also shows host-side launch latency)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    for i in range(args.steps):
        starts[i].record(stream)
        step(i)
        ends[i].record(stream)
    torch.cuda.synchronize()
    durs = np.array([s.elapsed_time(e) for s, e in zip(starts, ends)])  # ms
    log(f"per-launch event pairs: median {np.median(durs) * 1e3:.2f} us, "
        f"p10 {np.percentile(durs, 10) * 1e3:.2f} us, p90 {np.percentile(durs, 90) * 1e3:.2f} us")

    alg_bytes = wl.backward_bytes(dtype) if args.op == "backward" else wl.algorithmic_bytes(dtype)
    ms_per_step = wall * 1e3 / args.steps
    value = alg_bytes / (ms_per_step * 1e-3) / 1e9
    achieved = alg_bytes / (kern_ms * 1e-3) / 1e9
    traffic = load_traffic(wl.name if args.op == "forward" else f"{wl.name}_{args.op}", dtype, alg_bytes)

    cpu = None
    if not args.no_cpu_baseline and args.op == "forward":
        log("timing the CPU oracle baseline")
        cpu = cpu_baseline(wl, dtype, x, off, m, args.cpu_budget)

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
                       "seed": wl.seed},
            "algorithmic_bytes_per_step": alg_bytes,
            "samples_per_step": wl.samples(),
            "rotating_copies": copies,
            "plan": plan,
        },
        "gsamples_per_s": round(wl.samples() / (ms_per_step * 1e-3) / 1e9, 3),
        "hbm_fraction": round(value / HBM_PEAK_GBS, 4),
        "kernel_us_mean": round(kern_ms * 1e3, 3),
        "per_launch_event_us_median": round(float(np.median(durs)) * 1e3, 3),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
