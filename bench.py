#!/usr/bin/env python3
"""Benchmark: GEMM throughput (TFLOP/s) of the HIP library on one MI355X.

One step = one call of the library (argument checks, tile-config choice,
one kernel launch) over the resident inputs of the workload.  Default
workload: the 8192^3 bf16 NN product with bf16 output (A, B ~ N(0, 1),
seed 4).  The 4096^3 fp16 NN product, the ragged and batched products and
the 8192^3 E4M3 TN products (with and without block scales) are measured
alongside (their figures are reported under "also").  Inputs are generated on the host, copied to HBM
before timing, and stay there.

Prints ONE JSON line.  Timing of the headline workload:
  * W untimed warm-up steps, then more untimed steps until at least
    --settle seconds (default 0.3) of back-to-back launches have passed: the
    engine clock needs tens of milliseconds of load to settle after an idle
    spell (e.g. while the host generates inputs); the time spent is
    reported as ``timing.settle_s``;
  * exactly K timed steps between two device synchronisations (wall clock ->
    ``ms_per_step`` and ``value``), with a HIP event pair on the kernel's
    stream around them (-> ``timing.k_steps_kernel_ms``);
  * the roofline figure (``roofline.kernel_ms``, ``achieved``, ``frac``):
    the median over 5 blocks of back-to-back launches, each block at least
    50 ms long, one HIP event pair per block on the kernel's stream (the
    launches run back to back, so a block's span is their durations plus the
    small gaps between them).
The other workloads are timed the same way (settle, then the median of 5
blocks of at least 50 ms); the HBM-bound batched product is also timed with
the caches emptied before each launch.  "small" gives the per-call cost of
the two small workloads (host time of a C-ABI call and of the Python
wrapper, kernel time, wall time per call).  "mfma_ceiling" is the rate of the
bf16 kernel's MFMA stream with its operands in registers (libtdg_probe.so),
on the headline's operand distribution and on zeros: the engine clock is
power-limited and depends on the operand bits.  "gpu_state" is an amd-smi
sample taken while launches of the headline workload are still queued (the
line says whether the queue was still busy when the sample returned).
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GEMM TFLOP/s at 4096³ and 8192³ fp16 (fraction of MFMA peak), 1 MI355X"
PEAK_TFLOPS = {"f16": 2500.0, "bf16": 2500.0, "e4m3": 5000.0, "e5m2": 5000.0}   # MI355X dense MFMA, published
HBM_GBPS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def source_hash() -> str:
    """Hash of the kernel sources, to tell whether stored counters are stale."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "tiled_dense_gemm_03_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic(workload: str):
    """HBM bytes per launch from committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    runs, or None if absent or taken on different kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get(workload)
    if not e or e.get("source_hash") != source_hash():
        return None
    return e.get("hbm_bytes_per_launch")


def warm_up(torch, call, steps, min_seconds):
    """`steps` untimed calls, then more until `min_seconds` of wall time
    have passed (the engine clock needs tens of milliseconds of load to
    settle after an idle spell, e.g. while the host generates inputs).
    Returns the seconds spent."""
    t0 = time.perf_counter()
    for _ in range(steps):
        call()
    torch.cuda.synchronize()
    while time.perf_counter() - t0 < min_seconds:
        for _ in range(10):
            call()
        torch.cuda.synchronize()
    return time.perf_counter() - t0


def timed_runs(torch, call, stream, steps, repeats=1, min_total_s=0.0):
    """(wall ms, kernel ms) per call: `steps` back-to-back calls between two
    device synchronisations, with one HIP event pair on `stream` around them.
    With min_total_s, the call count is raised until a run takes at least
    that long (estimated from a first run); with repeats > 1 the run is
    repeated and the medians are returned."""
    import statistics

    def run(n):
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        start.record(stream)
        for _ in range(n):
            call()
        end.record(stream)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / n, start.elapsed_time(end) / n

    n = steps
    if min_total_s > 0:
        _, k_ms = run(steps)
        n = max(steps, int(min_total_s * 1e3 / max(k_ms, 1e-6)) + 1)
    res = [run(n) for _ in range(repeats)]
    return statistics.median(r[0] for r in res), statistics.median(r[1] for r in res)


def _resident(torch, w):
    """The workload's inputs in HBM and its output buffer."""
    from workloads import TORCH_DTYPE, workload_inputs
    a, b = workload_inputs(w)
    dev = torch.device("cuda:0")
    a, b = a.to(dev), b.to(dev)
    shape = (w.batch, w.M, w.N) if w.batch else (w.M, w.N)
    c = torch.empty(shape, dtype=TORCH_DTYPE[w.out_dtype], device=dev)
    return a, b, c, torch.cuda.current_stream(dev)


def time_workload(tdg, torch, w, steps, warmup, min_warm_s=0.0, repeats=1, min_total_s=0.0):
    from workloads import TORCH_DTYPE
    a, b, c, stream = _resident(torch, w)

    def call():
        tdg.gemm(a, b, layout=w.layout, out=c)
    warm_up(torch, call, warmup, min_warm_s)
    wall_ms, kernel_ms = timed_runs(torch, call, stream, steps, repeats, min_total_s)
    cfg = tdg.select_config(a, b, layout=w.layout, out_dtype=TORCH_DTYPE[w.out_dtype])
    return wall_ms, kernel_ms, tdg.tdg_config_name(cfg)


def time_headline(tdg, torch, w, steps, warmup, settle_s, blocks=5, block_s=0.05, config=-1):
    """The headline leg: warm-up and clock settling, exactly `steps` timed
    calls (wall clock between two synchronisations, and an event pair on the
    kernel's stream), then `blocks` blocks of at least `block_s` seconds of
    back-to-back calls for the roofline figure (median of the blocks).
    `config` >= 0 forces a tile configuration (for profiling the others)."""
    import statistics
    from workloads import TORCH_DTYPE
    a, b, c, stream = _resident(torch, w)

    def call():
        tdg.gemm(a, b, layout=w.layout, out=c, config=config)
    settled = warm_up(torch, call, warmup, settle_s)
    wall_ms, k_kernel_ms = timed_runs(torch, call, stream, steps)
    out = {"wall_ms": wall_ms, "k_steps_kernel_ms": k_kernel_ms, "settle_s": settled}
    if blocks > 0:
        n = max(1, int(block_s * 1e3 / max(k_kernel_ms, 1e-6)) + 1)
        per_block = [timed_runs(torch, call, stream, n)[1] for _ in range(blocks)]
        out["kernel_ms"] = statistics.median(per_block)
        out["block_kernel_ms"] = per_block
        out["block_calls"] = n
    else:
        out["kernel_ms"] = k_kernel_ms
    cfg = config if config >= 0 else tdg.select_config(a, b, layout=w.layout, out_dtype=TORCH_DTYPE[w.out_dtype])
    out["tile_config"] = tdg.tdg_config_name(cfg)
    return out


def time_small(tdg, torch, w, calls=3000):
    """Per-call cost of a small workload, where the fixed cost of a call
    dominates: the host time of one C-ABI call (argument checks, tile choice,
    enqueue; the GPU runs behind), the same through the Python wrapper, the
    kernel's duration from an event pair around back-to-back launches, and
    the wall time per call of the whole run (host and GPU)."""
    from workloads import TORCH_DTYPE, workload_inputs
    a, b = workload_inputs(w)
    dev = torch.device("cuda:0")
    a, b = a.to(dev), b.to(dev)
    c = torch.empty((w.M, w.N), dtype=TORCH_DTYPE[w.out_dtype], device=dev)
    stream = torch.cuda.current_stream(dev)
    code = {"f16": 0, "bf16": 1, "f32": 2}
    fn = tdg._binding.lib.tdg_gemm_tn if w.layout == "tn" else tdg._binding.lib.tdg_gemm_nn
    args = (w.M, w.N, w.K, a.data_ptr(), w.K, b.data_ptr(), w.K if w.layout == "tn" else w.N, c.data_ptr(), w.N,
            code[w.in_dtype], code[w.out_dtype], stream.cuda_stream)
    if fn(*args) != 0:
        raise RuntimeError("tdg_gemm_%s failed on %s" % (w.layout, w.name))

    def craw():
        fn(*args)

    def cpy():
        tdg.gemm(a, b, layout=w.layout, out=c)
    out = {"workload": w.name, "calls": calls}
    for name, call in (("c_abi", craw), ("python", cpy)):
        for _ in range(300):
            call()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(stream)
        for _ in range(calls):
            call()
        t1 = time.perf_counter()
        e1.record(stream)
        torch.cuda.synchronize()
        t2 = time.perf_counter()
        out[name] = {"host_us_per_call": round((t1 - t0) / calls * 1e6, 2),
                     "wall_us_per_call": round((t2 - t0) / calls * 1e6, 2),
                     "gpu_us_per_call": round(e0.elapsed_time(e1) / calls * 1e3, 2)}
    out["tflops_c_abi"] = round(w.flops / (out["c_abi"]["wall_us_per_call"] * 1e-6) / 1e12, 2)
    return out


def time_flushed(tdg, torch, w, reps=20):
    """Median kernel duration of `w` with the L2 caches and the Infinity
    Cache emptied of its operands before each launch: a 2 x 320 MiB device
    copy (more than the 256 MiB Infinity Cache) runs between launches, and
    an event pair on the stream brackets the launch alone."""
    import statistics
    from workloads import TORCH_DTYPE, workload_inputs
    a, b = workload_inputs(w)
    dev = torch.device("cuda:0")
    a, b = a.to(dev), b.to(dev)
    shape = (w.batch, w.M, w.N) if w.batch else (w.M, w.N)
    c = torch.empty(shape, dtype=TORCH_DTYPE[w.out_dtype], device=dev)
    src = torch.ones(320 << 20, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream(dev)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for i in range(reps + 3):
        dst.copy_(src)
        if i >= 3:
            ev[i - 3][0].record(stream)
        tdg.gemm(a, b, layout=w.layout, out=c)
        if i >= 3:
            ev[i - 3][1].record(stream)
    torch.cuda.synchronize()
    return statistics.median(s.elapsed_time(e) for s, e in ev)


def time_f8_workload(tdg, torch, w, steps, warmup, min_warm_s=0.0, repeats=1, min_total_s=0.0):
    """As time_workload, for an 8-bit workload (block-scale rows padded to a
    16-byte multiple, as the library asks)."""
    import numpy as np
    from workloads import TORCH_DTYPE, f8_workload_inputs
    a, b, xa, xb, sa, sb = f8_workload_inputs(w)
    dev = torch.device("cuda:0")

    def padded(x):
        if x is None:
            return None
        ld = -(-x.shape[1] // 16) * 16
        p = np.zeros((x.shape[0], ld), dtype=np.uint8)
        p[:, :x.shape[1]] = x
        return torch.from_numpy(p).to(dev)[:, :x.shape[1]]

    ad, bd = torch.from_numpy(a).to(dev), torch.from_numpy(b).to(dev)
    xad, xbd = padded(xa), padded(xb)
    sad = None if sa is None else torch.from_numpy(sa).to(dev)
    sbd = None if sb is None else torch.from_numpy(sb).to(dev)
    c = torch.empty((w.M, w.N), dtype=TORCH_DTYPE[w.out_dtype], device=dev)
    stream = torch.cuda.current_stream(dev)

    def call():
        tdg.gemm_f8(ad, bd, a_fmt=w.a_fmt, b_fmt=w.b_fmt, block_scale_a=xad, block_scale_b=xbd, scale_a=sad,
                    scale_b=sbd, out=c)
    warm_up(torch, call, warmup, min_warm_s)
    return timed_runs(torch, call, stream, steps, repeats, min_total_s)


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(w, seconds_min=10.0):
    """The oracle, unchanged, on a bounded row sample of the same workload:
    evenly spaced output rows (all columns, full K), doubling the row count
    until one run takes at least ``seconds_min`` (or covers every row)."""
    import numpy as np
    from oracle import oracle
    from workloads import bits, workload_inputs
    a, b = workload_inputs(w)
    ab, bb = bits(a), bits(b)
    nt = oracle.default_threads()
    omp = os.environ.get("OMP_NUM_THREADS")
    if omp and omp.isdigit():
        nt = min(nt, int(omp))
    nrows = 16
    while True:
        rows = np.linspace(0, w.M - 1, min(nrows, w.M)).astype(np.int64)
        t0 = time.perf_counter()
        oracle.gemm(ab, bb, w.in_dtype, w.layout, rows=rows, nthreads=nt)
        dt = time.perf_counter() - t0
        if dt >= seconds_min or nrows >= w.M:
            break
        nrows *= 2
    flops = 2.0 * len(rows) * w.N * w.K * max(1, w.batch)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": nt, "kind": "oracle",
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "sample": "%d of %d output rows%s (all %d columns, full K=%d), %.1f s; value = 2*rows*N*K%s / time"
                      % (len(rows), w.M, " of each of %d problems" % w.batch if w.batch else "", w.N, w.K, dt,
                         "*batch" if w.batch else "")}


def amd_smi_state():
    """GFX clock (mean over the XCDs), hotspot temperature and socket power of
    GPU 0 from amd-smi, or None when it cannot be read."""
    import subprocess
    try:
        out = subprocess.run(["amd-smi", "metric", "-g", "0", "-c", "-t", "-p", "--json"], capture_output=True,
                             text=True, timeout=20).stdout
        d = json.loads(out)
        g = d["gpu_data"][0] if isinstance(d, dict) else d[0]
        clks = [v["clk"]["value"] for k, v in g["clock"].items()
                if k.startswith("gfx_") and isinstance(v, dict) and isinstance(v.get("clk"), dict)]
        temp = g["temperature"].get("hotspot")
        power = g["power"].get("socket_power")
        return {"gfx_clock_mhz": round(sum(clks) / len(clks)) if clks else None,
                "hotspot_c": temp.get("value") if isinstance(temp, dict) else None,
                "socket_power_w": power.get("value") if isinstance(power, dict) else None}
    except Exception:   # no amd-smi, no permission, other output format
        return None


def mfma_ceiling(torch, seconds=0.25):
    """Rates of the kernels' per-wave MFMA streams with their operands held
    in registers (libtdg_probe.so, no memory traffic), one 8-wave workgroup
    per CU: the bf16 stream on N(0, 1) bf16 operands (the headline's inputs)
    and on zeros, the 8-bit stream on N(0, 1) E4M3 operands (the 8-bit legs'
    inputs) and on zeros.  The practical ceiling of the MFMA-bound products
    at the clock the board's power limit allows for those operand bits."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "tiled_dense_gemm_03_amd", "libtdg_probe.so"))
    argt = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    for f in ("tdgp_operand_elems", "tdgp_operand_bytes_f8"):
        getattr(lib, f).restype = ctypes.c_size_t
    for f in ("tdgp_flops", "tdgp_flops_f8"):
        getattr(lib, f).restype = ctypes.c_double
        getattr(lib, f).argtypes = [ctypes.c_int64, ctypes.c_int]
    lib.tdgp_mfma_stream.argtypes = argt
    lib.tdgp_mfma_stream_f8.argtypes = argt
    dev = torch.device("cuda")
    blocks = torch.cuda.get_device_properties(dev).multi_processor_count
    sink = torch.empty(blocks * 512, dtype=torch.float32, device=dev)
    clocks = torch.zeros(blocks * 2, dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream()
    gen = torch.Generator().manual_seed(4)

    def measure(launch, flops, ops):
        def run(iters):
            rc = launch(ops.data_ptr(), iters, blocks, sink.data_ptr(), clocks.data_ptr(),
                        ctypes.c_void_p(stream.cuda_stream))
            if rc != 0:
                raise RuntimeError("MFMA probe returned %d" % rc)

        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        iters = 2000
        t_end = time.perf_counter() + 0.2           # load the engine long enough for its clock to settle
        while time.perf_counter() < t_end:
            e0.record(stream)
            run(iters)
            e1.record(stream)
            torch.cuda.synchronize()
            iters = max(iters, int(iters * 0.05 / max(e0.elapsed_time(e1) * 1e-3, 1e-6)))
        iters = max(1, int(iters * seconds / 0.05))
        e0.record(stream)
        run(iters)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        ck = clocks.view(blocks, 2).double().cpu()
        ghz = float((ck[:, 0] / ck[:, 1]).mean()) * 0.1
        return {"tflops": round(flops(iters, blocks) / (ms * 1e-3) / 1e12, 1), "clock_ghz": round(ghz, 3),
                "ms": round(ms, 3)}

    n = lib.tdgp_operand_elems()
    out = {"kernel": "per-wave 16x16x32 bf16 MFMA stream of the 256x256 kernel (8x4 accumulator tiles, "
                     "2 K sub-steps per K tile), operands in registers, 8 waves per CU",
           "workgroups": blocks}
    for name, ops in (("random_normal", torch.randn(n, generator=gen).to(torch.bfloat16)),
                      ("zeros", torch.zeros(n, dtype=torch.bfloat16))):
        out[name] = measure(lib.tdgp_mfma_stream, lib.tdgp_flops, ops.to(dev))
    n8 = lib.tdgp_operand_bytes_f8()
    f8 = {"kernel": "per-wave scaled 32x32x64 E4M3 MFMA stream of the 8-bit 256x256 kernel (4x2 accumulator "
                    "tiles, 2 K sub-steps per K tile, unit scales), operands in registers, 8 waves per CU"}
    for name, ops in (("random_normal", torch.randn(n8, generator=gen).to(torch.float8_e4m3fn).view(torch.uint8)),
                      ("zeros", torch.zeros(n8, dtype=torch.uint8))):
        f8[name] = measure(lib.tdgp_mfma_stream_f8, lib.tdgp_flops_f8, ops.to(dev))
    out["e4m3"] = f8
    return out


def gpu_state_under_load(tdg, torch, w, kernel_ms, seconds=2.0):
    """amd-smi sampled while the GPU runs back-to-back launches of the
    workload: about `seconds` of launches are queued, the sample is taken in
    a second thread as soon as the first launches run, and an event recorded
    behind the last launch tells whether the queue was still busy when the
    sample returned (``under_load``)."""
    import threading
    a, b, c, stream = _resident(torch, w)
    tdg.gemm(a, b, layout=w.layout, out=c)
    torch.cuda.synchronize()
    n = max(10, int(seconds * 1e3 / max(kernel_ms, 1e-3)))
    done = torch.cuda.Event()
    box = {}
    sampler = threading.Thread(target=lambda: box.update(state=amd_smi_state()))
    t0 = time.perf_counter()
    for i in range(n):
        tdg.gemm(a, b, layout=w.layout, out=c)
        if i == 50:
            sampler.start()
    done.record(stream)
    if not sampler.is_alive() and "state" not in box:
        sampler.start()
    sampler.join()
    busy = not done.query()
    t_sample = time.perf_counter() - t0
    torch.cuda.synchronize()
    state = box.get("state")
    if state is not None:
        state["sampled"] = ("amd-smi started after 50 of %d queued back-to-back launches of %s (%.1f s of work); "
                            "returned after %.2f s" % (n, w.name, n * kernel_ms * 1e-3, t_sample))
        state["under_load"] = busy
    return state


def calibrate_copy(torch, nbytes=1 << 30, reps=3):
    """A plain copy kernel of known size, for scaling the HBM byte counters
    (FETCH_SIZE, WRITE_SIZE): each dispatch of the elementwise multiply-by-one
    reads nbytes and writes nbytes."""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(reps):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": nbytes, "dispatches": reps}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="nn_bf16_8192")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-also", action="store_true")
    ap.add_argument("--no-gpu-state", action="store_true", help="skip the amd-smi clock/temperature sample")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the MFMA-stream ceiling probe")
    ap.add_argument("--settle", type=float, default=0.3,
                    help="seconds of untimed back-to-back launches before timing (clock settling)")
    ap.add_argument("--blocks", type=int, default=5,
                    help="blocks of >= 50 ms whose median kernel time gives the roofline figure (0: the K steps)")
    ap.add_argument("--config", default=None,
                    help="force this tile configuration (by name) on the headline workload, for profiling")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a 1 GiB device copy (for scaling rocprofv3 byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py: this library runs on one GPU; --gpus %d is not offered (the product shards "
              "with no exchange over output tiles, see the design notes)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import tiled_dense_gemm_03_amd as tdg
    from workloads import WORKLOADS

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy:
        calibrate_copy(torch)
        return
    w = WORKLOADS[args.workload]
    forced = -1
    if args.config:
        names = [tdg.tdg_config_name(i) for i in range(tdg.tdg_num_configs())]
        if args.config not in names:
            print("bench.py: unknown configuration %r (one of %s)" % (args.config, ", ".join(names)), file=sys.stderr)
            sys.exit(2)
        forced = names.index(args.config)
    h = time_headline(tdg, torch, w, args.steps, args.warmup, args.settle, blocks=args.blocks, config=forced)
    ms, kernel_ms, cfg_name = h["wall_ms"], h["kernel_ms"], h["tile_config"]
    flops = w.flops
    value = flops / (ms * 1e-3) / 1e12
    achieved = flops / (kernel_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.in_dtype]
    traffic = stored_traffic(w.name)
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.in_dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "layout": w.layout, "M": w.M, "N": w.N, "K": w.K,
                   "batch": w.batch, "in_dtype": w.in_dtype, "out_dtype": w.out_dtype, "accumulate": "f32",
                   "inputs": "%s seed %d" % (w.dist, w.seed), "tile_config": cfg_name + (" (forced)" if forced >= 0 else ""),
                   "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4), "traffic": traffic,
                     "kernel_ms": round(kernel_ms, 5)},
        "timing": {"warmup_steps": args.warmup, "settle_s": round(h["settle_s"], 3),
                   "k_steps_wall_ms": round(ms, 5), "k_steps_kernel_ms": round(h["k_steps_kernel_ms"], 5),
                   "roofline_kernel_ms": ("median of %d blocks of %d back-to-back launches (>= 50 ms each), "
                                          "HIP event pair per block on the kernel's stream"
                                          % (args.blocks, h["block_calls"])) if args.blocks > 0
                   else "the K timed steps, HIP event pair on the kernel's stream",
                   "block_kernel_ms": [round(x, 5) for x in h.get("block_kernel_ms", [])]},
    }
    es = 4 if w.out_dtype == "f32" else 2
    alg_bytes = (2 * (w.M * w.K + w.K * w.N) + es * w.M * w.N) * max(1, w.batch)
    if flops / alg_bytes < peak / HBM_GBPS * 1e3:
        # below the ridge point: the kernel is bounded by HBM bytes, not FLOPs
        gbps = alg_bytes / (kernel_ms * 1e-3) / 1e9
        line["roofline"] = {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_GBPS, "unit": "GB/s",
                            "frac": round(gbps / HBM_GBPS, 4), "traffic": traffic, "kernel_ms": round(kernel_ms, 5),
                            "tflops": round(achieved, 2)}
    if not args.no_also:
        # the other measured workloads: the 4096^3 product of the metric, the
        # ragged single product and the HBM-bound batched TN product (whose
        # roofline is bytes, not FLOPs)
        also = []
        for name in ("nn_f16_4096", "nn_f16_ragged_4095x5000x3000", "tn_f16_batched_32x2048x2048x128"):
            if name == w.name:
                continue
            wa = WORKLOADS[name]
            ms_a, kms_a, cfg_a = time_workload(tdg, torch, wa, max(20, args.steps), args.warmup, 0.2,
                                               repeats=5, min_total_s=0.05)
            entry = {"workload": name, "value": round(wa.flops / (ms_a * 1e-3) / 1e12, 2),
                     "kernel_tflops": round(wa.flops / (kms_a * 1e-3) / 1e12, 2),
                     "frac": round(wa.flops / (kms_a * 1e-3) / 1e12 / PEAK_TFLOPS[wa.in_dtype], 4),
                     "ms_per_step": round(ms_a, 5), "kernel_ms": round(kms_a, 5), "tile_config": cfg_a}
            es = 4 if wa.out_dtype == "f32" else 2
            nbytes = (2 * (wa.M * wa.K + wa.K * wa.N) + es * wa.M * wa.N) * max(1, wa.batch)
            if wa.flops / nbytes < PEAK_TFLOPS[wa.in_dtype] / HBM_GBPS * 1e3:
                entry["hbm_gbps"] = round(nbytes / (kms_a * 1e-3) / 1e9, 1)
                entry["hbm_frac"] = round(nbytes / (kms_a * 1e-3) / 1e9 / HBM_GBPS, 4)
                # the inputs fit in the Infinity Cache: also with it emptied
                kms_f = time_flushed(tdg, torch, wa)
                entry["flushed"] = {"kernel_ms": round(kms_f, 5),
                                    "hbm_gbps": round(nbytes / (kms_f * 1e-3) / 1e9, 1),
                                    "hbm_frac": round(nbytes / (kms_f * 1e-3) / 1e9 / HBM_GBPS, 4),
                                    "method": "2 x 320 MiB device copy before each launch; event pair "
                                              "around the launch; median of 20"}
            if not args.no_cpu_baseline:
                # the oracle on the same workload (a bounded sample, as for the headline)
                entry["cpu_baseline"] = cpu_baseline(wa, seconds_min=2.0)
            also.append(entry)
        # the 8-bit TN products (roofline: the fp8 MFMA peak)
        from workloads import F8_WORKLOADS
        for name, wf in F8_WORKLOADS.items():
            ms_f, kms_f = time_f8_workload(tdg, torch, wf, max(20, args.steps), args.warmup, 0.2,
                                           repeats=5, min_total_s=0.05)
            also.append({"workload": name, "value": round(wf.flops / (ms_f * 1e-3) / 1e12, 2),
                         "kernel_tflops": round(wf.flops / (kms_f * 1e-3) / 1e12, 2),
                         "frac": round(wf.flops / (kms_f * 1e-3) / 1e12 / PEAK_TFLOPS[wf.a_fmt], 4),
                         "ms_per_step": round(ms_f, 5), "kernel_ms": round(kms_f, 5),
                         "dtype": wf.a_fmt, "out_dtype": wf.out_dtype,
                         "scales": ("E8M0 per 32-element K block" if wf.block_scales else "none") +
                                   (" + fp32 per row" if wf.row_scales else "")})
        # the two small workloads: the fixed cost of a call
        line["small"] = [time_small(tdg, torch, WORKLOADS[n]) for n in ("worked_128x256x192", "tn_exact_1024")]
        line["also"] = also
    if not args.no_ceiling and w.in_dtype in ("f16", "bf16"):
        ceil = mfma_ceiling(torch)
        ceil["headline_frac_of_random_ceiling"] = round(achieved / ceil["random_normal"]["tflops"], 4)
        ceil["random_ceiling_frac_of_peak"] = round(ceil["random_normal"]["tflops"] / peak, 4)
        c8 = ceil["e4m3"]["random_normal"]["tflops"]
        ceil["e4m3"]["random_ceiling_frac_of_peak"] = round(c8 / PEAK_TFLOPS["e4m3"], 4)
        for entry in line.get("also", []):
            if entry.get("dtype") == "e4m3":
                entry["frac_of_random_ceiling"] = round(entry["kernel_tflops"] / c8, 4)
        line["mfma_ceiling"] = ceil
    if not args.no_gpu_state:
        line["gpu_state"] = gpu_state_under_load(tdg, torch, w, kernel_ms)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
