"""Benchmark: emulated ring AllReduce on one MI355X.

Default workload: 8 virtual ranks x 256 MiB fp32 each (64Mi elements per
rank, uniform[-1, 1], seed 0 per rank), op Sum, ring, protocol and channel
count chosen by arTune (the library's cost model).  One step = one
arAllReduce over all ranks with inputs already resident in HBM.

Reported per step (S = bytes per rank, N = ranks, t = time per step):
  algbw = S / t;  busbw = algbw * 2(N-1)/N  (the pages' ring factor)
  deviceBytes = the device-memory bytes the plan's kernel must move: 2N * S
  when the ring's FIFO slots are in LDS (every input read once, every
  output written once), else modelBytes = 5(N-1) * S (a reduce-scatter step
  reads 2 chunks and writes 1, an all-gather step reads 1 and writes 1, N-1
  steps each over N ranks, every FIFO slot in device memory)
  roofline.achieved = deviceBytes / t, against the 8 TB/s HBM peak.
The CPU baseline is the oracle (single-threaded C) on the same inputs.
After the timed region, plain streaming kernels (a copy, two reads and a
write, a read, a write; csrc/probes/stream_ceiling.hip) measure the box's
practical HBM ceiling, reported beside the datasheet peak.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--nranks N]
       [--count ELEMS] [--dtype float32] [--proto auto|simple|ll|ll128]
       [--nchannels C] [--no-cpu-baseline] [--sweep] [--profile-steps K]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--nranks", type=int, default=8)
    ap.add_argument("--count", type=int, default=64 << 20, help="elements per rank")
    ap.add_argument("--dtype", default="float32")
    ap.add_argument("--proto", default="auto")
    ap.add_argument("--op", default="sum", choices=["sum", "max", "min"])
    ap.add_argument("--algo", default="ring", choices=["ring", "tree", "auto"],
                    help="AllReduce algorithm (the headline metric is the ring's)")
    ap.add_argument("--nchannels", type=int, default=64)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-stream-ceiling", action="store_true",
                    help="skip the streaming-kernel ceiling measured after the timed region")
    ap.add_argument("--device-inputs", action="store_true",
                    help="draw the inputs on the GPU (same distributions, torch's generator) instead of the host "
                         "generator; for timing large configurations (no CPU baseline then)")
    ap.add_argument("--sweep", action="store_true", help="8B..256MiB sweep, every protocol + auto")
    ap.add_argument("--sweep-max-log2", type=int, default=28)
    ap.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "traffic.json"))
    ap.add_argument("--lanes", type=int, default=0, help="force wavefronts per (rank, channel)")
    ap.add_argument("--no-lds-fifo", action="store_true",
                    help="keep every FIFO slot in device memory (arDebugLdsFifo 0), for comparison")
    ap.add_argument("--explore", default="", help="'nch1,nch2:lanes1,lanes2' grid of configurations")
    ap.add_argument("--coll", default="allreduce", choices=["allreduce", "reducescatter", "allgather"],
                    help="collective to time; for the two halves --count is the per-rank block "
                         "(default: 256 MiB per rank on the larger side)")
    ap.add_argument("--large-n-table", action="store_true",
                    help="time every algorithm x protocol at 24-72 ranks (rings of several workgroups)")
    ap.add_argument("--calibrate", action="store_true",
                    help="measure latency vs ranks and bandwidth vs channels per protocol and fit arTune's model")
    ap.add_argument("--calib-table", nargs="+", metavar="GRID_JSONL",
                    help="write the tuner's time table (the text format of AR_TUNE_FILE and of the library's "
                         "compiled table) from --calib-grid records; with --fit-models also fit the cost model")
    ap.add_argument("--fit-models", action="store_true",
                    help="with --calib-table: least-squares fit of the pages' cost model per algorithm and protocol "
                         "on the records of rings and trees inside one workgroup (at most 16 ranks)")
    ap.add_argument("--calib-grid", default="",
                    help="'N1,N2,..:log2size1,log2size2,..': time every algorithm x protocol at each rank count and "
                         "per-rank size (fp32 Sum, channels by the 32 KiB rule); one JSON line each")
    ap.add_argument("--group-sweep", default="",
                    help="'N:bytes:gs1,gs2,..': a ring (or --algo tree) of N ranks at this many bytes per rank "
                         "with at most gs members per workgroup, every protocol; one JSON line each, then a "
                         "per-protocol fit of time against the groups per ring (hops inside vs between groups)")
    ap.add_argument("--summarize-profiles", nargs=5, metavar=("TRACE", "FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="summarize rocprofv3 CSV output directories into markdown + profiles/traffic.json")
    ap.add_argument("--profile-label", default="", help="workload key for --summarize-profiles")
    ap.add_argument("--batch", type=int, default=0,
                    help="time T AllReduces of --count elements issued one by one, as one group, and "
                         "captured into a HIP graph and replayed")
    ap.add_argument("--copy-probe-bytes", type=int, default=0,
                    help="time a plain elementwise copy (torch.neg) of this many bytes instead")
    return ap.parse_args()


def main():
    args = parse()
    if args.summarize_profiles:
        return summarize_profiles(args)
    if args.calib_table:
        return calib_table(args)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this library emulates all ranks on one GPU; --gpus %d (WORLD_SIZE %d) is not "
              "supported -- run with --gpus 1" % (args.gpus, world), file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from ring_allreduce_reduction_amd import binding as B
    from ring_allreduce_reduction_amd import inputs as gen
    if not os.path.exists(B.LIB_PATH):
        from ring_allreduce_reduction_amd.build import build
        build()
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)

    if args.copy_probe_bytes:
        return copy_probe(args, torch)
    if args.sweep:
        return sweep(args, B, gen, torch, np)
    if args.calibrate:
        return calibrate(args, B, torch, np)
    if args.large_n_table:
        return large_n_table(args, B, torch, np)
    if args.group_sweep:
        return group_sweep(args, B, torch, np)
    if args.calib_grid:
        return calib_grid(args, B, torch, np)
    if args.batch:
        return bench_batch(args, B, gen, torch, np)

    if args.coll != "allreduce":
        return bench_halves(args, B, gen, torch, np)

    N, count, dtype = args.nranks, args.count, args.dtype
    esz = gen.ELEM_SIZE[dtype]
    S = count * esz
    tdt = {"float32": torch.float32, "int32": torch.int32, "float16": torch.float16,
           "bfloat16": torch.bfloat16}[dtype]
    sends, recvs = [], []
    if args.device_inputs:
        # the configurations' distributions: fp32 uniform[-1,1], 16-bit floats
        # normal(0,1) rounded to nearest-even, int32 uniform[-2^20, 2^20]
        log("drawing inputs on the GPU: %d ranks x %d %s (seed %d)" % (N, count, dtype, args.seed))
        xs = None
        for r in range(N):
            g = torch.Generator("cuda").manual_seed(args.seed * 1000 + r)
            if dtype == "float32":
                d = torch.rand(count, generator=g, device="cuda") * 2 - 1
            elif dtype == "int32":
                d = torch.randint(-(1 << 20), (1 << 20) + 1, (count,), generator=g, device="cuda", dtype=torch.int32)
            else:
                d = torch.randn(count, generator=g, device="cuda").to(tdt)
            sends.append(d)
            recvs.append(torch.empty_like(d))
    else:
        log("generating inputs: %d ranks x %d %s (seed %d)" % (N, count, dtype, args.seed))
        t0 = time.perf_counter()
        xs = gen.make_inputs(N, count, dtype, seed=args.seed)
        log("inputs ready in %.1fs; uploading" % (time.perf_counter() - t0))
        for x in xs:
            h = torch.from_numpy(x.view(np.int16) if x.dtype == np.uint16 else x)
            d = h.to("cuda")
            sends.append(d.view(tdt) if d.dtype != tdt else d)
            recvs.append(torch.empty_like(sends[-1]))
    torch.cuda.synchronize()

    comm = B.Comm(N, args.nchannels, args.proto, args.algo)
    if args.lanes:
        B.arSetDebug(comm.handle, B.arDebugLanes, args.lanes)
    if args.no_lds_fifo:
        B.arSetDebug(comm.handle, B.arDebugLdsFifo, 0)
    if args.explore:
        return explore(args, B, torch, comm, sends, recvs, count, dtype, N, S)
    plan = comm.plan(count, dtype)
    footprint = comm.footprint()
    log("plan: %s; comm device footprint %.1f MiB" % (json.dumps(plan), footprint / 2 ** 20))
    stream = torch.cuda.Stream()
    dt_code = B.DTYPE_BY_NAME[dtype]
    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            comm.allreduce(sends, recvs, B.OP_BY_NAME[args.op], stream=stream, count=count, dtype=dt_code)
        torch.cuda.synchronize()
        err = comm.async_error()
        if err != B.arSuccess:
            raise SystemExit("warmup failed: " + B.arGetErrorString(err))
        # per-launch durations: events on the launch stream around every call
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        for a, b in evs:
            a.record(stream)
            comm.allreduce(sends, recvs, B.OP_BY_NAME[args.op], stream=stream, count=count, dtype=dt_code)
            b.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - w0
    err = comm.async_error()
    if err != B.arSuccess:
        raise SystemExit("timed run failed: " + B.arGetErrorString(err))
    launch_ms = [a.elapsed_time(b) for a, b in evs]
    ms = sum(launch_ms) / len(launch_ms)
    t = ms / 1e3
    algbw = S / t / 1e9
    busbw = algbw * 2 * (N - 1) / N
    model_bytes = plan["modelBytes"]     # ring: 5(N-1)S; tree: (2N + 4(N-1))S
    device_bytes = plan["deviceBytes"]   # the kernel's own: 2NS with LDS FIFOs, else modelBytes
    achieved = device_bytes / t / 1e9
    log("per-launch ms: mean %.4f min %.4f max %.4f; wall per step %.4f ms"
        % (ms, min(launch_ms), max(launch_ms), wall / args.steps * 1e3))

    # Checks of the timed result: every rank holds identical bits (on the
    # device), rank 0 equals the oracle bit for bit (below, with the CPU
    # baseline), and a sample is within the stated bound of a float64 direct
    # reduction computed by torch.
    same = all(torch.equal(recvs[0].view(torch.uint8), r.view(torch.uint8)) for r in recvs[1:])
    idx = torch.randint(0, count, (100000,), device="cuda", generator=torch.Generator("cuda").manual_seed(1))
    vals = torch.stack([x[idx].double() for x in sends])
    ref = vals.sum(0) if args.op == "sum" else vals.max(0).values if args.op == "max" else vals.min(0).values
    err_max = (recvs[0][idx].double() - ref).abs().max().item()
    if args.op != "sum" or dtype == "int32":
        err_bound = 0.0                                    # order-free results are exact
    elif dtype == "float32":
        err_bound = 1e-6 * N * vals.abs().max().item()     # the stated fp32 bound
    else:                                                  # 16-bit: the dtype's own ring bound
        u = 2.0 ** -8 if dtype == "bfloat16" else 2.0 ** -11
        err_bound = (N - 1) * u / (1 - (N - 1) * u) * vals.abs().sum(0).max().item()
    log("all ranks identical: %s; sample max |err| vs float64 %s = %.3g (bound %.3g)"
        % (same, args.op, err_max, err_bound))
    rank0 = None if xs is None else recvs[0].view({4: torch.int32, 2: torch.int16}[esz]).cpu().numpy()

    traffic = None
    if os.path.exists(args.traffic_json):
        try:
            tj = json.load(open(args.traffic_json))
            key = workload_key(B.PROTO_NAMES[plan["proto"]], N, count, dtype)
            if plan["algo"] == B.arAlgoTree:
                key = "Tree" + key
            if key in tj and tj[key]["kernel_src_sha256"] == kernel_src_sha():
                traffic = tj[key]["bytes_per_launch"]
            elif key in tj:
                log("traffic counters predate the current kernel source: reporting null")
        except Exception as e:  # a stale or partial file must not break the bench
            log("traffic file unreadable: %s" % e)

    comm.close()
    del sends, recvs
    cpu, oracle_exact = None, None
    if xs is not None:
        cpu, want = cpu_baseline(xs, dtype, args.op, plan, N, S, B, timed=not args.no_cpu_baseline)
        raw = {4: np.uint32, 2: np.uint16}[esz]
        oracle_exact = bool(np.array_equal(rank0.view(raw), want.view(raw)))
        log("rank 0 bit-exact against the oracle on the plan it ran: %s" % oracle_exact)
        del rank0, want
    ceiling = None if args.no_stream_ceiling else stream_ceiling(torch)

    algo = B.ALGO_NAMES[plan["algo"]]
    out = {
        "metric": ("emulated ring AllReduce busbw GB/s + % HBM peak, 8 ranks x 256 MiB fp32"
                   if (algo, N, S, dtype, args.op) == ("ring", 8, 256 << 20, "float32", "sum")
                   else "emulated %s AllReduce busbw GB/s + %% HBM peak" % algo),
        "value": round(busbw, 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"float32": "f32", "bfloat16": "bf16", "float16": "f16", "int32": "i32"}[dtype],
        "data": "synthetic" + (" (drawn on the GPU)" if xs is None else ""),
        "config": {"workload": "%s AllReduce %s, %d virtual ranks x %d MiB %s per rank on one GPU"
                               % (algo, args.op.capitalize(), N, S >> 20, dtype), "algo": algo,
                   "nranks": N, "count_per_rank": count, "bytes_per_rank": S,
                   "proto": B.PROTO_NAMES[plan["proto"]], "nChannels": plan["nChannels"],
                   "chunkElems": plan["chunkElems"], "lanesPerChannel": plan["lanesPerChannel"],
                   "workgroups": plan["workgroups"], "threadsPerGroup": plan["threadsPerGroup"],
                   "slotBytes": plan["stepBytes"], "commDeviceBytes": footprint,
                   "selection": "arTune" if args.proto == "auto" else "forced"},
        "algbw_GBs": round(algbw, 3),
        "busbw_GBs": round(busbw, 3),
        "fifo_in_lds": plan["ldsFifoBytes"] > 0,
        "device_bytes_per_step": device_bytes,
        "hbm_frac": round(achieved / HBM_PEAK_GBS, 4),
        "model_bytes_per_step": model_bytes,
        "all_ranks_identical": bool(same),
        "oracle_exact": oracle_exact,
        "err_max": err_max,
        "err_bound": err_bound,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic},
        "cpu_baseline": cpu,
        "stream_ceiling": ceiling,
    }
    if ceiling:
        out["device_vs_copy_ceiling"] = round(achieved / ceiling["copy"], 4)
    print(json.dumps(out), flush=True)
    # a number is published only for a correct result
    if not same or oracle_exact is False or err_max > err_bound:
        log("RESULT CHECK FAILED: ranks identical %s, oracle exact %s, sample err %.3g (bound %.3g)"
            % (same, oracle_exact, err_max, err_bound))
        sys.exit(3)


def stream_ceiling(torch, nbytes=1 << 30, steps=10):
    """The box's practical HBM ceiling: plain streaming kernels (16-byte
    non-temporal vectors, csrc/probes/stream_ceiling.hip) over 1 GiB buffers,
    four times the Infinity Cache, timed with events on torch's stream.  A
    context figure beside the 8 TB/s peak, not the roofline's peak."""
    import ctypes
    from ring_allreduce_reduction_amd import build as lb
    if not os.path.exists(lb.PROBE_LIB):
        log("stream-ceiling probe not built: skipped")
        return None
    lib = ctypes.CDLL(lb.PROBE_LIB)
    lib.streamCeilingLaunch.restype = ctypes.c_int
    lib.streamCeilingLaunch.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p]
    a = torch.ones(nbytes // 4, device="cuda")
    c = torch.ones(nbytes // 4, device="cuda")
    b = torch.empty(nbytes // 4, device="cuda")
    stream = torch.cuda.current_stream()
    moved = {"copy": 2, "read2_write1": 3, "read": 1, "write": 1}
    out = {"unit": "GB/s", "buffer_bytes": nbytes}
    grid = torch.cuda.get_device_properties(0).multi_processor_count * 16
    for kind, name in enumerate(moved):
        launch = lambda: lib.streamCeilingLaunch(kind, a.data_ptr(), c.data_ptr(), b.data_ptr(), nbytes, grid,
                                                 ctypes.c_void_p(stream.cuda_stream))
        for _ in range(3):
            if launch() != 0:
                raise SystemExit("stream-ceiling probe launch failed")
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            launch()
        e1.record(stream)
        torch.cuda.synchronize()
        out[name] = round(moved[name] * nbytes / (e0.elapsed_time(e1) / steps / 1e3) / 1e9, 1)
    log("stream ceiling (GB/s): copy %.0f, 2 reads + 1 write %.0f, read %.0f, write %.0f"
        % (out["copy"], out["read2_write1"], out["read"], out["write"]))
    return out


def workload_key(proto, N, count, dtype):
    return "%s_n%d_count%d_%s" % (proto, N, count, dtype)


def kernel_src_sha():
    """Hash of the kernels' source: the device code and the translation units
    that instantiate and launch it."""
    import glob
    import hashlib
    csrc = os.path.join(ROOT, "ring_allreduce_reduction_amd", "csrc")
    h = hashlib.sha256()
    for f in [os.path.join(csrc, "ar_device.h")] + sorted(glob.glob(os.path.join(csrc, "ar_kernels*.hip"))):
        h.update(open(f, "rb").read())
    return h.hexdigest()


def summarize_profiles(args):
    """Read rocprofv3 CSV directories (kernel trace with --stats; FETCH_SIZE and
    WRITE_SIZE passes of the ring kernel and of the copy probe) and print a
    markdown summary; store the per-launch HBM traffic in profiles/traffic.json."""
    import csv
    import glob

    def rows(d, suffix):
        fs = glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True)
        if not fs:
            raise SystemExit("no *%s under %s" % (suffix, d))
        return list(csv.DictReader(open(fs[0])))

    def counter(d, name, match):
        vals = [float(r["Counter_Value"]) for r in rows(d, "counter_collection.csv")
                if match in r["Kernel_Name"] and r["Counter_Name"] == name]
        return sum(vals) / len(vals), len(vals)

    trace_dir, fetch_dir, write_dir, cf_dir, cw_dir = args.summarize_profiles
    stats = rows(trace_dir, "kernel_stats.csv")
    ring = [r for r in stats if "ringAllReduceKernel" in r["Name"]]
    fetch_kib, nf = counter(fetch_dir, "FETCH_SIZE", "ringAllReduceKernel")
    write_kib, nw = counter(write_dir, "WRITE_SIZE", "ringAllReduceKernel")
    cf_kib, _ = counter(cf_dir, "FETCH_SIZE", "vectorized_elementwise_kernel")
    cw_kib, _ = counter(cw_dir, "WRITE_SIZE", "vectorized_elementwise_kernel")
    copy_bytes = 1 << 30
    fscale = copy_bytes / (cf_kib * 1024.0)
    wscale = copy_bytes / (cw_kib * 1024.0)
    read_b = fetch_kib * 1024.0 * fscale
    write_b = write_kib * 1024.0 * wscale
    print("| kernel | calls | avg duration (us) | min | max |")
    print("|---|---|---|---|---|")
    for r in stats[:6]:
        print("| `%s` | %s | %.1f | %.1f | %.1f |" % (r["Name"][:90], r["Calls"], float(r["AverageNs"]) / 1e3,
                                                   float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3))
    print()
    print("Copy-probe calibration (torch.neg over 1 GiB: reads 1 GiB, writes 1 GiB):")
    print("FETCH_SIZE reads %.0f KiB per dispatch (scale x%.3f), WRITE_SIZE %.0f KiB (scale x%.3f).\n"
          % (cf_kib, fscale, cw_kib, wscale))
    print("Ring kernel, per launch (mean of %d / %d dispatches): FETCH_SIZE %.0f KiB -> %.3f GiB read; "
          "WRITE_SIZE %.0f KiB -> %.3f GiB written; total %.3f GiB (%.0f bytes)."
          % (nf, nw, fetch_kib, read_b / 2 ** 30, write_kib, write_b / 2 ** 30, (read_b + write_b) / 2 ** 30,
             read_b + write_b))
    if args.profile_label and ring:
        path = args.traffic_json
        tj = json.load(open(path)) if os.path.exists(path) else {}
        tj[args.profile_label] = {"bytes_per_launch": round(read_b + write_b), "read_bytes": round(read_b),
                                  "write_bytes": round(write_b), "fetch_scale": round(fscale, 4),
                                  "write_scale": round(wscale, 4),
                                  "kernel_avg_ns": float(ring[0]["AverageNs"]),
                                  "kernel_src_sha256": kernel_src_sha()}
        with open(path, "w") as f:
            json.dump(tj, f, indent=1, sort_keys=True)
        print("\nwrote %s[%s]" % (path, args.profile_label))


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(xs, dtype, op, plan, N, S, B, timed=True):
    """The oracle, as it stands, on the timed inputs and the plan that ran
    (single thread, pinned to one core of the process's set), repeated until
    about 10 s of CPU work; reported in the metric's unit.  Returns (the
    baseline record or None, the oracle's result of the first run)."""
    import oracle
    allowed = os.sched_getaffinity(0)
    core = min(allowed)
    os.sched_setaffinity(0, {core})
    try:
        reps, total, want = 0, 0.0, None
        while reps == 0 or (timed and total < 10.0 and reps < 50):
            t0 = time.perf_counter()
            if plan["algo"] == B.arAlgoTree:
                res = oracle.tree_allreduce(xs, dtype, op, plan["nChannels"])
            else:
                res = oracle.allreduce(xs, dtype, op, plan["nChannels"], plan["chunkElems"])
            total += time.perf_counter() - t0
            reps += 1
            if want is None:
                want = res
    finally:
        os.sched_setaffinity(0, allowed)
    if not timed:
        return None, want
    t = total / reps
    busbw = S / t / 1e9 * 2 * (N - 1) / N
    log("cpu oracle: %d runs, %.3f s per AllReduce on core %d of %d" % (reps, t, core, os.cpu_count()))
    return {"value": round(busbw, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "host_cores": os.cpu_count(), "cores_allowed": len(allowed), "cpu_model": cpu_model(),
            "pinned_core": core,
            "sample": "the full %d x %d MiB %s %s workload, %d run(s) of the single-threaded C oracle pinned to "
                      "one core (its one result array stands for every rank's output), %.2f s each"
                      % (N, S >> 20, dtype, op, reps, t)}, want


def bench_halves(args, B, gen, torch, np):
    """ReduceScatter or AllGather on their own (the two halves of the ring).
    B = block bytes; algbw = N*B/t, busbw = algbw*(N-1)/N; model bytes
    3N(N-1)B (reduce-scatter steps read 2 blocks, write 1) or 2N(N-1)B
    (all-gather steps read 1, write 1)."""
    N, dtype = args.nranks, args.dtype
    esz = gen.ELEM_SIZE[dtype]
    count = args.count // N if args.count == 64 << 20 else args.count   # block elements
    rs = args.coll == "reducescatter"
    Bb = count * esz
    tdt = {"float32": torch.float32, "int32": torch.int32, "float16": torch.float16,
           "bfloat16": torch.bfloat16}[dtype]
    in_count = N * count if rs else count
    log("generating inputs: %d ranks x %d %s (seed %d)" % (N, in_count, dtype, args.seed))
    xs = gen.make_inputs(N, in_count, dtype, seed=args.seed)

    def dev(x):
        d = torch.from_numpy(x.view(np.int16) if x.dtype == np.uint16 else x).to("cuda")
        return d.view(tdt) if d.dtype != tdt else d
    sends = [dev(x) for x in xs]
    recvs = [torch.empty(count if rs else N * count, dtype=tdt, device="cuda") for _ in range(N)]
    comm = B.Comm(N, args.nchannels, args.proto)
    plan = comm.plan(count, dtype, func=args.coll)
    log("plan: %s" % json.dumps(plan))
    stream = torch.cuda.Stream()
    dt_code = B.DTYPE_BY_NAME[dtype]

    def call():
        if rs:
            comm.reduce_scatter(sends, recvs, B.arSum, stream=stream, recvcount=count, dtype=dt_code)
        else:
            comm.all_gather(sends, recvs, stream=stream, sendcount=count, dtype=dt_code)
    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            call()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        torch.cuda.synchronize()
        for a, b in evs:
            a.record(stream)
            call()
            b.record(stream)
        torch.cuda.synchronize()
    if comm.async_error() != B.arSuccess:
        raise SystemExit("timed run failed")
    ms = sum(a.elapsed_time(b) for a, b in evs) / args.steps
    t = ms / 1e3
    algbw = N * Bb / t / 1e9
    busbw = algbw * (N - 1) / N
    model_bytes = plan["modelBytes"]
    achieved = plan["deviceBytes"] / t / 1e9
    if rs:   # sanity: a sample of rank 3's block against a float64 direct sum (torch, no oracle)
        idx = torch.randint(0, count, (100000,), device="cuda", generator=torch.Generator("cuda").manual_seed(1))
        s64 = sum(x[3 * count + idx].double() for x in sends)
        log("sample max |err| vs float64 = %.3g" % (recvs[3][idx].double() - s64).abs().max().item())
    else:
        log("every rank holds the concatenation: %s" % all(torch.equal(r, torch.cat(sends)) for r in recvs))
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        reps, total = 0, 0.0
        while total < 10.0 and reps < 50:
            t0 = time.perf_counter()
            if rs:
                oracle.reduce_scatter(xs, dtype, "sum")
            else:
                oracle.all_gather(xs, dtype)
            total += time.perf_counter() - t0
            reps += 1
        tc = total / reps
        cpu = {"value": round(N * Bb / tc / 1e9 * (N - 1) / N, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
               "sample": "the full workload, %d run(s) of the single-threaded C oracle, %.2f s each" % (reps, tc)}
    comm.close()
    name = "ReduceScatter" if rs else "AllGather"
    print(json.dumps({
        "metric": "emulated ring %s busbw GB/s + %% HBM peak" % name, "value": round(busbw, 3), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": {"float32": "f32", "bfloat16": "bf16", "float16": "f16", "int32": "i32"}[dtype],
        "data": "synthetic",
        "config": {"workload": "ring %s Sum, %d virtual ranks, %d MiB blocks (%d MiB per rank on the larger side)"
                               % (name, N, Bb >> 20, (N * Bb) >> 20), "nranks": N, "block_elems": count,
                   "proto": B.PROTO_NAMES[plan["proto"]], "nChannels": plan["nChannels"],
                   "lanesPerChannel": plan["lanesPerChannel"], "workgroups": plan["workgroups"]},
        "algbw_GBs": round(algbw, 3), "busbw_GBs": round(busbw, 3), "fifo_in_lds": plan["ldsFifoBytes"] > 0,
        "device_bytes_per_step": plan["deviceBytes"], "hbm_frac": round(achieved / HBM_PEAK_GBS, 4),
        "model_bytes_per_step": model_bytes,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None},
        "cpu_baseline": cpu}), flush=True)


def bench_batch(args, B, gen, torch, np):
    """T AllReduces of `count` fp32 elements per rank on N ranks, each with its
    own buffers: issued one by one, then between arGroupStart / arGroupEnd
    (aggregated into batched launches), then the T single calls captured once
    into a HIP graph and replayed.  Reports microseconds per AllReduce for
    each (events around the whole set, mean over --steps repetitions)."""
    N, T, count = args.nranks, args.batch, args.count
    xs = gen.make_inputs(N, count, "float32", seed=args.seed)
    sends = [[torch.from_numpy(x).cuda() for x in xs] for _ in range(T)]
    recvs = [[torch.empty_like(t) for t in row] for row in sends]
    comm = B.Comm(N, args.nchannels, args.proto, args.algo)
    stream = torch.cuda.Stream()
    # marshal once: the timed loop calls the C ABI directly, so the host side
    # costs about what a C caller's would
    import ctypes
    L = B.lib()
    sp = [B._ptrs(row) for row in sends]
    rp = [B._ptrs(row) for row in recvs]
    sh = ctypes.c_void_p(stream.cuda_stream)
    res = {}
    for mode in ("single", "group"):
        def one_set():
            if mode == "group":
                L.arGroupStart()
            for i in range(T):
                rc = L.arAllReduce(comm.handle, sp[i], rp[i], count, B.arFloat32, B.arSum, sh)
                if rc != B.arSuccess:
                    raise SystemExit("arAllReduce: " + B.arGetErrorString(rc))
            if mode == "group" and L.arGroupEnd() != B.arSuccess:
                raise SystemExit("arGroupEnd failed")
        with torch.cuda.stream(stream):
            for _ in range(args.warmup):
                one_set()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            a.record(stream)
            for _ in range(args.steps):
                one_set()
            b.record(stream)
            torch.cuda.synchronize()
        if comm.async_error() != B.arSuccess:
            raise SystemExit("batch run failed")
        res[mode] = a.elapsed_time(b) * 1e3 / (args.steps * T)
    # the T single calls recorded once (one kernel node each) and replayed
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=stream):
        for i in range(T):
            if L.arAllReduce(comm.handle, sp[i], rp[i], count, B.arFloat32, B.arSum, sh) != B.arSuccess:
                raise SystemExit("arAllReduce under capture failed")
    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            g.replay()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for _ in range(args.steps):
            g.replay()
        b.record(stream)
        torch.cuda.synchronize()
    if comm.async_error() != B.arSuccess:
        raise SystemExit("graph replay failed")
    res["graph"] = a.elapsed_time(b) * 1e3 / (args.steps * T)
    del g
    plan = comm.group_plan(0)
    single = comm.plan(count, "float32")
    comm.close()
    S = count * 4
    print(json.dumps({"batch": T, "nranks": N, "bytes_per_rank": S, "us_per_allreduce_single": round(res["single"], 3),
                      "us_per_allreduce_group": round(res["group"], 3),
                      "us_per_allreduce_graph": round(res["graph"], 3),
                      "speedup": round(res["single"] / res["group"], 3),
                      "single_plan": {"algo": B.ALGO_NAMES[single["algo"]], "proto": B.PROTO_NAMES[single["proto"]],
                                      "nch": single["nChannels"]},
                      "group_plan": {"algo": B.ALGO_NAMES[plan["algo"]], "proto": B.PROTO_NAMES[plan["proto"]],
                                     "nch": plan["nChannels"], "tasksInLaunch": plan["tasksInLaunch"]}}),
          flush=True)


def time_calls(B, torch, comm, sends, recvs, count, dt_code, warmup, steps):
    """Mean ms per AllReduce over `steps` calls on one stream (HIP events).
    The pointer arrays are built and checked once and the loop calls the C
    ABI directly: per-call marshalling in Python (tens of microseconds at 24
    ranks, a hundred at 72) would otherwise starve the GPU on short calls and
    time the host instead."""
    import ctypes
    L = B.lib()
    sp, rp = B._checked_ptrs(comm.handle, sends, recvs, dt_code, count, count)
    stream = torch.cuda.Stream()
    sh = ctypes.c_void_p(stream.cuda_stream)

    def call():
        rc = L.arAllReduce(comm.handle, sp, rp, count, dt_code, B.arSum, sh)
        if rc != B.arSuccess:
            raise B.ArError(rc, "arAllReduce")
    for _ in range(warmup):
        call()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(steps):
        call()
    b.record(stream)
    torch.cuda.synchronize()
    err = comm.async_error()
    if err != B.arSuccess:
        raise SystemExit("run failed: " + B.arGetErrorString(err))
    return a.elapsed_time(b) / steps


def explore(args, B, torch, comm, sends, recvs, count, dtype, N, S):
    """Time a grid of configurations in one process:
    --explore 'channels:lanes[:slotKiB[:direct[:depth[:sets[:lds]]]]]', each a comma list
    (lanes 0 = automatic, depth 0 = the protocol's default, sets 0 = one
    workgroup per (channel, lane), else at most that many workgroups; lds 1 =
    FIFO slots in LDS where they fit, the default, 0 = in device memory)."""
    parts = args.explore.split(":")
    parts += ["8", "1", "0", "0", "1"][len(parts) - 2:]
    chs, lanes, slots, directs, depths, setss, ldss = [[int(x) for x in p.split(",")] for p in parts[:7]]
    grid = [(a, b, c, e, f, h, q) for a in chs for b in lanes for c in slots for e in directs for f in depths
            for h in setss for q in ldss]
    proto = "simple" if args.proto == "auto" else args.proto
    comm.close()
    for nch, ln, sk, d, dp, st, lq in grid:
        # a fresh comm per configuration: knobs stay on a comm
        comm = B.Comm(N, nch, proto)
        if dp:
            B.arSetDebug(comm.handle, B.arDebugSlots, dp)
        B.arSetDebug(comm.handle, B.arDebugLanes, ln)
        if args.proto == "ll128":   # the slot field sets the LL128 slot (2 or 4 KiB)
            B.arSetDebug(comm.handle, B.arDebugLL128SlotKiB, sk)
        else:
            B.arSetDebug(comm.handle, B.arDebugSimpleSlotKiB, sk)
        B.arSetDebug(comm.handle, B.arDebugDirect, d)
        B.arSetDebug(comm.handle, B.arDebugLaneSets, st)
        B.arSetDebug(comm.handle, B.arDebugLdsFifo, lq)
        plan = comm.plan(count, dtype)
        ms = time_calls(B, torch, comm, sends, recvs, count, B.DTYPE_BY_NAME[dtype], 2, args.steps)
        frac = plan["deviceBytes"] / (ms / 1e3) / 1e9 / HBM_PEAK_GBS
        print(json.dumps({"nch": nch, "lanes": plan["lanesPerChannel"], "slotKiB": sk, "direct": d,
                          "depth": plan["nSlots"], "sets": st, "lds": plan["ldsFifoBytes"],
                          "grid": plan["workgroups"],
                          "block": plan["threadsPerGroup"], "groupSize": plan["ranksPerGroup"],
                          "nchRun": plan["nChannels"], "slotBytes": plan["stepBytes"],
                          "ms": round(ms, 4), "busbw": round(S / (ms / 1e3) / 1e9 * 2 * (N - 1) / N, 2),
                          "frac": round(frac, 4)}), flush=True)
        comm.close()


def copy_probe(args, torch):
    """A plain elementwise kernel that reads and writes a known number of bytes
    (the yardstick for the FETCH_SIZE / WRITE_SIZE counters)."""
    n = args.copy_probe_bytes // 4
    src = torch.rand(n, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(2):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(args.steps):
        torch.neg(src, out=dst)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / args.steps
    print(json.dumps({"copy_probe_bytes": n * 4, "ms": round(ms, 4),
                      "read_plus_write_GBs": round(2 * n * 4 / (ms / 1e3) / 1e9, 1)}), flush=True)


def _ring_model_us(params, factor, n, nch, S):
    """The ring cost model arTune evaluates (same form, any constants), with
    the cap scaled for N ranks sharing one HBM (8 / N)."""
    base, step, bw, cap = params
    bus = min(bw * nch * factor, cap * 8.0 / n)
    return base + 2 * (n - 1) * step + S / (1000.0 * bus * n / (2 * (n - 1)))


# the pages' tree efficiency by message size (rows LL, LL128, Simple), as arTune applies it
_TREE_CORR = [
    [1.0, 1.0, 1.0, 1.0, .9, .8, .7, .7, .7, .7, .6, .5, .4, .4, .5, .6, .7, .8, .9, 1.0, 1.0, 1.0, 1.0, 1.0],
    [1.0, 1.0, 1.0, 1.0, 1.0, .9, .8, .8, .8, .7, .6, .6, .6, .6, .6, .6, .8, .9, .9, .9, .9, 1.0, 1.0, 1.0],
    [.9, .9, .9, .9, .9, .9, .9, .8, .7, .6, .6, .5, .5, .5, .5, .6, .7, .8, .7, .7, .8, .9, .9, .9],
]


def _tree_model_us(params, proto, n, nch, S):
    """The tree cost model arTune evaluates (same form, any constants), with
    the cap scaled for N ranks sharing one HBM (44 / (6N - 4))."""
    base, step, bw, cap = params
    bus = min(bw * nch * 0.92 * {0: 1 / 3.8, 1: 120 / 128, 2: 1.0}[proto], cap * 44.0 / (6 * n - 4))
    q = S >> 6
    if q > 0 and q.bit_length() - 1 < 23:
        bus *= _TREE_CORR[proto][q.bit_length() - 1]
    return base + 2 * (n.bit_length() - 1) * step + S / (1000.0 * bus)


def _channels_for(S, maxch=64):
    """Channels where the model is capped: the most whose share is >= 32 KiB."""
    c = 1
    while c * 2 <= maxch and S // (c * 2) >= 32768:
        c *= 2
    return c


def calibrate(args, B, torch, np):
    """Fit the cost model's constants per protocol on this GPU, for the ring
    (default) or, with --algo tree, for the tree.

    Measured, fp32 Sum:
      latency:   4 KiB per rank, 1 channel, N = 2, 4, 8, 16 (one workgroup
                 holds a channel's members, as at the sweep's 8 ranks; past 16
                 the cross-workgroup edges add a cost neither model has);
      bandwidth: 128 MiB per rank, N = 8, 1..64 channels;
      mid sizes: 16 KiB .. 64 MiB per rank, N = 8, at the channel count the
                 32 KiB-per-channel rule allows (where arTune lands once the
                 bandwidth is capped).
    The four constants (base, step, bwPerCh, cap) are the least-squares fit of
    log(model time / measured time) over all of these points, the best of
    several starts (the closed-form estimates first).  Prints one JSON line per measurement, one per
    protocol with the fit's worst relative error, and one with the fitted
    models."""
    from scipy.optimize import least_squares
    tree = args.algo == "tree"
    factor = {B.arProtoLL: 0.5, B.arProtoLL128: 0.92, B.arProtoSimple: 1.0}
    ranks = (2, 4, 8, 16)
    fits = {}
    big = 32 << 20
    base = [torch.rand(big, device="cuda") for _ in range(16)]
    small = [torch.rand(1024, device="cuda") for _ in range(max(ranks))]
    small_out = [torch.empty_like(x) for x in small]
    outs = [torch.empty_like(x) for x in base]
    for proto in (B.arProtoLL, B.arProtoLL128, B.arProtoSimple):
        name = B.PROTO_NAMES[proto]
        pts = []   # (n, nch, bytes per rank, measured us)
        xs, ys = [], []
        for n in ranks:
            comm = B.Comm(n, 1, proto, args.algo)
            ms = time_calls(B, torch, comm, small[:n], small_out[:n], 1024, B.arFloat32, 20, 200)
            comm.close()
            xs.append(2 * (n.bit_length() - 1) if tree else 2 * (n - 1))
            ys.append(ms * 1e3)
            pts.append((n, 1, 4096, ms * 1e3))
            print(json.dumps({"calib": "latency", "algo": args.algo, "proto": name, "nranks": n,
                              "us": round(ms * 1e3, 3)}), flush=True)
        step, b0 = np.polyfit(np.array(xs, float), np.array(ys, float), 1)
        b0, step = max(float(b0), 0.0), max(float(step), 0.0)
        lat8 = b0 + (6 if tree else 14) * step
        comm = B.Comm(8, 64, proto, args.algo)
        bus = {}
        for nch in (1, 2, 4, 8, 16, 32, 64):
            comm.set_config(proto, nch)
            ms = time_calls(B, torch, comm, base[:8], outs[:8], big, B.arFloat32, 3, 10)
            S = big * 4
            pts.append((8, nch, S, ms * 1e3))
            bus[nch] = S / max(ms * 1e3 - lat8, 1e-3) / 1e3 * (1.0 if tree else 2 * 7 / 8)
            print(json.dumps({"calib": "bandwidth", "algo": args.algo, "proto": name, "nch": nch,
                              "us": round(ms * 1e3, 2), "busbw_GBs": round(bus[nch], 2)}), flush=True)
        for lg in range(14, 27, 2):
            S = 1 << lg
            nch = _channels_for(S)
            comm.set_config(proto, nch)
            ms = time_calls(B, torch, comm, base[:8], outs[:8], S // 4, B.arFloat32, 5, 100 if lg < 24 else 20)
            pts.append((8, nch, S, ms * 1e3))
            print(json.dumps({"calib": "mid", "algo": args.algo, "proto": name, "bytes": S, "nch": nch,
                              "us": round(ms * 1e3, 3)}), flush=True)
        comm.close()
        # the protocol's bandwidth factor in the model, to start bwPerCh from one channel's busBw
        f = 0.92 * {0: 1 / 3.8, 1: 120 / 128, 2: 1.0}[proto] if tree else factor[proto]

        def model(p, n, c, S):
            return _tree_model_us(p, proto, n, c, S) if tree else _ring_model_us(p, factor[proto], n, c, S)

        def resid(p):
            return [np.log(model(p, n, c, S) / t) for n, c, S, t in pts]

        starts = [[b0, step, max(bus[1] / f, 1e-2), max(max(bus.values()), 1e-2)],
                  [3.0, 2.0, 50.0, 100.0], [1.0, 1.0, 100.0, 100.0], [5.0, 3.0, 20.0, 60.0]]
        sol = None
        for x0 in starts:
            cand = least_squares(resid, np.array(x0, float), bounds=([0.0, 0.0, 1e-2, 1e-2], [np.inf] * 4))
            if sol is None or cand.cost < sol.cost:
                sol = cand
        worst = float(np.max(np.abs(np.expm1(sol.fun))))
        fits[name] = {"baseLatUs": round(float(sol.x[0]), 3), "stepLatUs": round(float(sol.x[1]), 4),
                      "bwPerChGBs": round(float(sol.x[2]), 2), "maxBwGBs": round(float(sol.x[3]), 2)}
        print(json.dumps({"calib": "fit_error", "algo": args.algo, "proto": name, "points": len(pts),
                          "worst_rel_err": round(worst, 3)}), flush=True)
    print(json.dumps({"calib": "fit", "algo": args.algo, "models": fits}), flush=True)


def large_n_table(args, B, torch, np):
    """Rings of more than one workgroup (24, 32, 48, 72 ranks): every
    algorithm x protocol at 4 KiB per rank on 1 channel, 256 KiB on 8, 4 and
    16 MiB on 64, fp32 Sum; one JSON line each, with arTune's choice for the
    size."""
    ranks = (24, 32, 48, 72)
    xs = [torch.rand(1 << 22, device="cuda") for _ in range(max(ranks))]
    ys = [torch.empty_like(x) for x in xs]
    for n in ranks:
        for count, nch in ((1024, 1), (1 << 16, 8), (1 << 20, 64), (1 << 22, 64)):
            with B.Comm(n, 64, "auto", "auto") as comm:
                a, p, ch, pred = B.arTuneAlgo(comm.handle, count * 4)
            for algo in ("ring", "tree"):
                for proto in (B.arProtoLL, B.arProtoLL128, B.arProtoSimple):
                    row = {"nranks": n, "bytes": count * 4, "nch": nch, "algo": algo,
                           "proto": B.PROTO_NAMES[proto], "arTune": "%s/%s/%d" % (B.ALGO_NAMES[a], B.PROTO_NAMES[p], ch)}
                    comm = B.Comm(n, nch, proto, algo)
                    try:
                        comm.plan(count, "float32")
                        row["us"] = round(time_calls(B, torch, comm, xs[:n], ys[:n], count, B.arFloat32, 3, 20) * 1e3, 2)
                    except B.ArError as e:
                        row["skipped"] = str(e)
                    comm.close()
                    print(json.dumps(row), flush=True)


TABLE_COLUMNS = [("ring", "ll"), ("ring", "ll128"), ("ring", "simple"), ("tree", "ll"), ("tree", "ll128"),
                 ("tree", "simple")]


def calib_table(args):
    """The tuner's time table from --calib-grid records: one line per (ranks,
    bytes per rank) with the median microseconds of ring LL, LL128, Simple and
    tree LL, LL128, Simple ("-" where a candidate could not run), the text
    format AR_TUNE_FILE reads and from which the build compiles the library's
    own table.  With --fit-models, "model" lines follow: the pages' cost model
    fitted per algorithm and protocol (least squares in log time) on the
    records of at most 16 ranks (rings and trees inside one workgroup, the
    regime that model describes)."""
    import collections
    T = collections.defaultdict(dict)
    for path in args.calib_table:
        for line in open(path):
            r = json.loads(line)
            if "us" in r and r["algo"] != "auto":
                T[(r["nranks"], r["bytes"])][(r["algo"], r["proto"])] = r["us"]
    print("# ranks bytes_per_rank  ring_LL ring_LL128 ring_Simple tree_LL tree_LL128 tree_Simple  (us, fp32 Sum,")
    print("# channels by the 32 KiB-per-channel rule; '-' = that candidate cannot run there)")
    for (n, S) in sorted(T):
        d = T[(n, S)]
        print("%d %d  %s" % (n, S, " ".join(("%.3f" % d[c]) if c in d else "-" for c in TABLE_COLUMNS)))
    if not args.fit_models:
        return
    import numpy as np
    from scipy.optimize import least_squares
    for algo in ("ring", "tree"):
        for proto in ("ll", "ll128", "simple"):
            pc = {"ll": 0, "ll128": 1, "simple": 2}[proto]
            pts = [(n, S, d[(algo, proto)]) for (n, S), d in T.items() if n <= 16 and (algo, proto) in d]

            def model(p, n, S):
                c = _channels_for(S)
                if algo == "tree":
                    return _tree_model_us(p, pc, n, c, S)
                return _ring_model_us(p, {0: 0.5, 1: 0.92, 2: 1.0}[pc], n, c, S)

            def resid(p):
                return [np.log(model(p, n, S) / t) for n, S, t in pts]
            sol = None
            for x0 in ([3.0, 1.0, 100.0, 200.0], [5.0, 2.0, 50.0, 100.0], [2.0, 0.5, 200.0, 300.0],
                       [10.0, 3.0, 20.0, 60.0]):
                cand = least_squares(resid, np.array(x0), bounds=([0.0, 0.0, 1e-2, 1e-2], [np.inf] * 4))
                if sol is None or cand.cost < sol.cost:
                    sol = cand
            worst = float(np.max(np.abs(np.expm1(sol.fun))))
            print("model %s %s %.3f %.4f %.2f %.2f   # %d points, worst %.0f%% off" % (
                algo, proto, sol.x[0], sol.x[1], sol.x[2], sol.x[3], len(pts), 100 * worst))


def calib_grid(args, B, torch, np):
    """The calibration record: every algorithm x protocol at every rank count
    and per-rank size of the grid, fp32 Sum, on device-drawn inputs, at the
    channel count the 32 KiB-per-channel rule gives the size (where the model
    lands in every regime: one channel below 64 KiB, the most allowed above).
    The six candidates of a size are timed round-robin, five rounds, each a
    run of back-to-back calls; the median round is reported, so a phase of
    the GPU (its clock moves under these loads) weighs on every candidate
    alike.  Sizes whose N buffers of send and receive would pass 24 GiB are
    skipped.  One JSON line per (N, size, algorithm, protocol) with the median
    and the spread of the rounds and the plan that ran."""
    rank_s, size_s = args.calib_grid.split(":")
    ranks = [int(x) for x in rank_s.split(",")]
    sizes = [1 << int(x) for x in size_s.split(",")]
    rounds = 5
    for n in ranks:
        fit = [S for S in sizes if 2 * n * S <= (24 << 30)]
        maxc = max(fit) // 4
        sends = [torch.rand(maxc, device="cuda") * 2 - 1 for _ in range(n)]
        recvs = [torch.empty_like(x) for x in sends]
        comm = B.Comm(n, 64, "simple", "ring")
        for S in fit:
            count = max(1, S // 4)
            nch = _channels_for(S)
            steps = 50 if S < (4 << 20) else 10 if S < (64 << 20) else 3
            rows, times = [], []
            cands = SWEEP_CANDIDATES + [("auto", "auto")]
            for algo, proto in cands:
                row = {"nranks": n, "bytes": S, "nch": nch, "algo": algo, "proto": proto}
                try:
                    comm.set_algo(algo)
                    comm.set_config(proto, 64 if algo == "auto" else nch)
                    plan = comm.plan(count, "float32")
                    row.update({"nchRun": plan["nChannels"], "lanes": plan["lanesPerChannel"],
                                "groupSize": plan["ranksPerGroup"], "grid": plan["workgroups"],
                                "slot": plan["stepBytes"], "ranAlgo": B.ALGO_NAMES[plan["algo"]],
                                "ranProto": B.PROTO_NAMES[plan["proto"]], "predUs": round(plan["predictedUs"], 2)})
                except B.ArError as e:
                    row["skipped"] = str(e)
                rows.append(row)
                times.append([])
            for _ in range(rounds):
                for i, (algo, proto) in enumerate(cands):
                    if "skipped" in rows[i]:
                        continue
                    comm.set_algo(algo)
                    comm.set_config(proto, 64 if algo == "auto" else nch)
                    times[i].append(time_calls(B, torch, comm, sends, recvs, count, B.arFloat32, 2, steps) * 1e3)
            for row, ts in zip(rows, times):
                if ts:
                    ts.sort()
                    row["us"] = round(ts[len(ts) // 2], 3)
                    row["us_min"] = round(ts[0], 3)
                    row["us_max"] = round(ts[-1], 3)
                print(json.dumps(row), flush=True)
        comm.close()
        del sends, recvs
        torch.cuda.empty_cache()


def group_sweep(args, B, torch, np):
    """Time a ring or tree of N ranks cut into groups of at most gs members
    (arDebugGroupSize), fp32 Sum on device-drawn inputs, for each protocol.
    The configurations of a protocol are timed round-robin, five rounds of
    back-to-back calls, and the median round is reported.  A ring cut into G
    groups (G > 1) has G edges between workgroups out of N, and a chunk's
    walk of 2(N-1) hops takes that share of them, so its time is about
    t(G) = c + 2(N-1) h + 2(N-1) (G/N) (H - h), with h a hop inside a
    workgroup and H one between workgroups; the last line per protocol is
    the least-squares line through the grouped points and the h and H - h it
    gives (c, the launch and fill, is folded into h)."""
    n_s, bytes_s, gs_s = args.group_sweep.split(":")
    N, S = int(n_s), int(bytes_s)
    sizes = [int(x) for x in gs_s.split(",")]
    count = max(1, S // 4)
    rounds = 5
    steps = 50 if S < (4 << 20) else 20
    sends = [torch.rand(count, device="cuda") * 2 - 1 for _ in range(N)]
    recvs = [torch.empty_like(x) for x in sends]
    comm = B.Comm(N, args.nchannels, "simple", args.algo if args.algo != "auto" else "ring")
    if args.no_lds_fifo:
        B.arSetDebug(comm.handle, B.arDebugLdsFifo, 0)
    for proto in ["simple", "ll", "ll128"]:
        comm.set_config(proto, args.nchannels)
        rows, times = [], []
        for gs in sizes:
            B.arSetDebug(comm.handle, B.arDebugGroupSize, gs)
            row = {"nranks": N, "bytes": S, "algo": args.algo, "proto": proto, "gsMax": gs,
                   "ldsFifo": not args.no_lds_fifo}
            try:
                plan = comm.plan(count, "float32")
                row.update({"nch": plan["nChannels"], "lanes": plan["lanesPerChannel"],
                            "groupSize": plan["ranksPerGroup"], "groups": -(-N // plan["ranksPerGroup"]),
                            "grid": plan["workgroups"], "block": plan["threadsPerGroup"],
                            "slot": plan["stepBytes"]})
            except B.ArError as e:
                row["skipped"] = str(e)
            rows.append(row)
            times.append([])
        for _ in range(rounds):
            for i, gs in enumerate(sizes):
                if "skipped" in rows[i]:
                    continue
                B.arSetDebug(comm.handle, B.arDebugGroupSize, gs)
                times[i].append(time_calls(B, torch, comm, sends, recvs, count, B.arFloat32, 2, steps) * 1e3)
        pts = []
        for row, ts in zip(rows, times):
            if ts:
                ts.sort()
                row["us"] = round(ts[len(ts) // 2], 2)
                row["us_min"] = round(ts[0], 2)
                row["us_max"] = round(ts[-1], 2)
                if row["groups"] > 1:
                    pts.append((row["groups"], row["us"]))
            print(json.dumps(row), flush=True)
        if len(pts) >= 2:
            g = np.array([p[0] for p in pts], dtype=np.float64)
            t = np.array([p[1] for p in pts], dtype=np.float64)
            slope, icpt = np.polyfit(g, t, 1)
            hops = 2 * (N - 1)
            print(json.dumps({"fit": proto, "nranks": N, "bytes": S, "points": len(pts),
                              "us_at_0_groups": round(float(icpt), 2), "us_per_group": round(float(slope), 3),
                              "hop_inside_us": round(float(icpt) / hops, 3),
                              "hop_between_extra_us": round(float(slope) * N / hops, 3)}), flush=True)
    B.arSetDebug(comm.handle, B.arDebugGroupSize, 0)
    comm.close()


SWEEP_CANDIDATES = [("ring", "ll"), ("ring", "ll128"), ("ring", "simple"),
                    ("tree", "ll"), ("tree", "ll128"), ("tree", "simple")]


def sweep(args, B, gen, torch, np):
    """N ranks (default 8) fp32 Sum, per-rank sizes 8 B .. 2^max bytes.  Each
    algorithm x protocol runs at the channel count arTune's model gives that
    pair for the size (the pages fix channels by size: at least 32 KiB per
    channel), then arTune's own choice over both algorithms; one JSON line per
    size with the regret t(chosen)/min t - 1."""
    N = args.nranks
    maxc = (1 << args.sweep_max_log2) // 4
    xs = gen.make_inputs(N, maxc, "float32", seed=args.seed)
    sends = [torch.from_numpy(x).cuda() for x in xs]
    recvs = [torch.empty_like(s) for s in sends]
    comm = B.Comm(N, args.nchannels, "auto", "auto")
    ring = [B.arTuneGetAlgoModel(comm.handle, B.arAlgoRing, p) for p in (0, 1, 2)]
    tree = [B.arTuneGetAlgoModel(comm.handle, B.arAlgoTree, p) for p in (0, 1, 2)]
    for lg in range(3, args.sweep_max_log2 + 1):
        count = (1 << lg) // 4
        S = count * 4
        iters = 200 if S < (64 << 20) else 20
        res = {}
        for algo, proto in SWEEP_CANDIDATES + [("auto", "auto")]:
            key = "auto" if algo == "auto" else (proto if algo == "ring" else "tree_" + proto)
            comm.set_algo(algo)
            if algo == "auto":
                comm.set_config("auto", args.nchannels)
            else:
                pcode = B.PROTO_BY_NAME[proto]
                _, _, nch, _ = B.arTuneEvalAlgo(0, N, args.nchannels, S, ring, tree,
                                                algoMask=1 << B.ALGO_BY_NAME[algo], protoMask=1 << pcode)
                comm.set_config(proto, max(1, nch))
            plan = comm.plan(count, "float32")
            ms = time_calls(B, torch, comm, sends, recvs, count, B.arFloat32, 5, iters)
            res[key] = {"us": round(ms * 1e3, 3), "algo": B.ALGO_NAMES[plan["algo"]],
                        "proto": B.PROTO_NAMES[plan["proto"]], "nch": plan["nChannels"],
                        "pred_us": round(plan["predictedUs"], 2)}
        best = min(v["us"] for k, v in res.items() if k != "auto")
        out = {"bytes": S, "nranks": N, "regret": round(res["auto"]["us"] / best - 1, 4),
               "busbw_auto_GBs": round(S / (res["auto"]["us"] / 1e6) / 1e9 * 2 * (N - 1) / N, 3)}
        out.update(res)
        print(json.dumps(out), flush=True)
    comm.close()

if __name__ == "__main__":
    main()
