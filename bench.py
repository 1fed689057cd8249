"""Throughput of the block-scaled FP4 hot path on one MI355X.

Default workload: the two-level-rotation activation tensor, 16384 x 8192 bf16
with per-32-channel-block variances exp(1.5 z) (synthetic, seeded). One step
is one fused call of the online path -- channel permutation, 32-point block
Hadamard, MXFP4 absmax / E8M0 scale / E2M1 rounding / nibble packing -- over
the whole tensor (one kernel launch). The permutation is calibrated once,
before timing, from the tensor's channel energies (offline step, reported).

value = input bytes (rows * cols * 2) / time per step, GB/s, with the input
resident in HBM: two input copies (2 x 268 MB, more than the 256 MB Infinity
Cache) are used alternately so no step reads the previous step's data from
cache. Timing uses HIP events on the stream the kernels run on.

The same run also reports the other rows of the path on their own workloads
(plain MXFP4, NVFP4 + RaZeR with and without the tensor-amax pass, the
dequantizers) and the CPU oracle timed on a bounded sample of the workload.

  python bench.py [--steps K] [--warmup W] [--workload c4|c2|c5] [--no-extras]
  python bench.py --pmc-summary FETCH_DIR WRITE_DIR [MFMA_DIR]

roofline.traffic is the HBM traffic per launch of the fused kernel taken from
rocprofv3 counters (FETCH_SIZE and WRITE_SIZE runs of this same program, each
scaled by the reading for torch's 1 GiB device copy in the same run). The
numbers live in profiles/traffic_perm_rotate_quantize_c4.md together with a
hash of the kernel's sources; when the sources have changed since, traffic is
reported as null. --pmc-summary writes that file's text from the rocprofv3
output directories.
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "quantize+pack GB/s (bf16 in) and % of HBM peak on 1 MI355X; SQNR dB"
HBM_PEAK_GBS = 8000.0
B_MX = 2 + 0.5 + 1 / 32   # algorithmic bytes per element, MXFP4 quantize
B_NV = 2 + 0.5 + 1 / 16   # NVFP4 quantize (without the tensor-amax read)


MFMA_PEAK_BF16_TFLOPS = 2500.0
ROT_KERNEL = "rotq_perm_kernel"  # fused permutation + Hadamard + FP4 quantize
ROT_INSTANCE = ROT_KERNEL + "<1, 0, true, false, false, 8>"  # the MXFP4 instance timed at 16384x8192
ROT_SOURCES = ["block_scaled_fp4_absmax_amd/csrc/rotate_kernels.hpp",
               "block_scaled_fp4_absmax_amd/csrc/rotate_mx.hip",
               "block_scaled_fp4_absmax_amd/csrc/rotation.hpp",
               "block_scaled_fp4_absmax_amd/csrc/fp4_device.hpp",
               "block_scaled_fp4_absmax_amd/csrc/launch.hpp"]
TRAFFIC_FILE = "profiles/traffic_perm_rotate_quantize_c4.md"
COPY_BYTES = 1 << 30  # torch device copy in device_copy(): 1 GiB read, 1 GiB written
# steps of the informational rows. On MI355X a kernel reaches its sustained
# speed only after some 25 ms of its own launches (the first launches of a
# new kernel, or on freshly allocated buffers, run up to 30% slower), so each
# row warms up for ROW_WARM_MS of its own calls before it is timed
ROW_STEPS, ROW_WARMUP, ROW_WARM_MS = 50, 30, 40.0


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def rot_source_hash():
    """sha256 (first 16 hex) of the fused kernel's sources with comments and
    blank lines removed: a change to the code invalidates the committed
    counters, a change to a comment does not."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in ROT_SOURCES:
        with open(os.path.join(ROOT, f)) as fh:
            text = re.sub(r"/\*.*?\*/", "", fh.read(), flags=re.S)
        for ln in text.splitlines():
            ln = re.sub(r"//.*", "", ln).rstrip()
            if ln:
                h.update(ln.encode() + b"\n")
    return h.hexdigest()[:16]


def committed_traffic():
    """(bytes per launch, source) from the counter summary, or (None, why)."""
    path = os.path.join(ROOT, TRAFFIC_FILE)
    if not os.path.exists(path):
        return None, "no counter summary"
    kv = {}
    with open(path) as fh:
        for ln in fh:
            if ln.startswith("- ") and ": " in ln:
                k, v = ln[2:].split(": ", 1)
                kv[k.strip()] = v.strip().strip("`")
    if kv.get("source_hash") != rot_source_hash():
        return None, "kernel sources changed since the counters were taken"
    return int(kv["traffic_bytes_per_launch"]), TRAFFIC_FILE


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=500)
    p.add_argument("--warmup", type=int, default=100)
    p.add_argument("--workload", default="c4", choices=["c4", "c1", "c2", "c3", "c5"])
    p.add_argument("--no-extras", action="store_true")
    p.add_argument("--no-cpu", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--trace-summary", nargs=2, metavar=("TRACE_DIR", "BENCH_LOG"),
                   help="write the kernel-time summary from a rocprofv3 --kernel-trace --stats "
                        "directory and the JSON line that the profiled run printed, and exit")
    p.add_argument("--kernel-op", choices=sorted(KERNEL_OPS),
                   help="time one kernel on its own (the run that rocprofv3 counter passes "
                        "profile) and print its JSON line")
    p.add_argument("--counter-summary", nargs="+", metavar=("OP_LOG", "DIR"),
                   help="write the counter summary of a --kernel-op run from its JSON line and "
                        "rocprofv3 --pmc output directories, and exit")
    p.add_argument("--pmc-summary", nargs="+", metavar="DIR",
                   help="write the traffic summary from rocprofv3 --pmc output directories "
                        "(FETCH_SIZE run, WRITE_SIZE run[, MFMA busy run]) and exit")
    return p.parse_args()


_SETTLE = {}
SETTLE_REST_S = float(os.environ.get("FP4_BENCH_REST_S", "0.5"))


def settle(torch, ms=30.0, rest_s=SETTLE_REST_S):
    """Let the GPU rest for rest_s seconds, then keep it busy for about ms
    milliseconds (device fills of a 256 MiB buffer, untimed) and wait. On
    MI355X the first ~10 ms of work after an idle second run up to 30% slower
    while the clocks come back up, and kernels timed right after long
    stretches of other full-bandwidth work run up to 15% slower than the same
    kernels on their own. The rest and the fills make every timed region start
    from the same state: the clocks of sustained operation, no backlog."""
    if "buf" not in _SETTLE:
        _SETTLE["buf"] = torch.empty(1 << 26, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    time.sleep(rest_s)
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(16):  # about 1 ms of back-to-back fills per wait
            _SETTLE["buf"].fill_(1.0)
        torch.cuda.synchronize()


def timed(torch, fn, steps, warmup, warm_ms=0.0):
    """ms per call of fn(i), measured with events on the current stream, after
    settle() and the warm-up calls: warmup calls, continued until the warm-up
    has run for at least warm_ms milliseconds."""
    settle(torch)
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < warm_ms:
        for _ in range(8):
            fn(warmup)
        torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(st)
    for i in range(steps):
        fn(warmup + i)
    b.record(st)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def graph_us(torch, fn, calls=20, replays=5):
    """us per call of fn(i) replayed from a HIP graph of calls i = 0..calls-1: the
    GPU-side time of launches too short for the Python binding to keep the
    queue ahead of them (the library records no allocation and no memset, so
    the calls capture as they run)."""
    settle(torch)
    cur = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    side.wait_stream(cur)
    with torch.cuda.stream(side):
        for i in range(calls):
            fn(i)  # warm-up on the capture stream
    cur.wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(calls):
            fn(i)
    g.replay()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(cur)
    for _ in range(replays):
        g.replay()
    b.record(cur)
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / (calls * replays)
    del g
    return us


def step_distribution(torch, fn, n):
    """p10 / p50 / p90 of single-step times (us): an event pair around each of n
    back-to-back steps; the queue stays ahead of the GPU, so each pair brackets
    that step's kernels only."""
    settle(torch)
    st = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n)]
    for i, (a, b) in enumerate(ev):
        a.record(st)
        fn(i)
        b.record(st)
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) * 1e3 for a, b in ev)
    return [round(t[n // 10], 2), round(t[n // 2], 2), round(t[(9 * n) // 10], 2)]


def dev_copies(torch, x_u16, n):
    import numpy as np
    t = torch.from_numpy(x_u16.view(np.int16)).cuda().view(torch.bfloat16)
    return [t] + [t.clone() for _ in range(n - 1)]


def copies_for(nbytes, floor=2):
    """Enough copies that their total exceeds twice the 256 MB Infinity Cache."""
    return max(floor, -(-512 * 2 ** 20 // nbytes))


def device_copy(torch):
    """Reference: torch's device-to-device copy of 1 GiB (read + write bytes / time)."""
    src = torch.empty(1 << 29, dtype=torch.int16, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    ms = timed(torch, lambda i: dst.copy_(src), 10, 2, ROW_WARM_MS)
    return {"bytes_moved": 2 << 30, "ms": round(ms, 4), "GBps": round(2 * (1 << 30) / ms / 1e6, 1)}


def sqnr_db(torch, x, xh):
    x = x.double()
    d = x - xh.double()
    return float(10 * torch.log10((x * x).sum() / (d * d).sum()))


def cpu_model():
    """The host CPU's model name with its family / model / stepping numbers
    (/proc/cpuinfo, first processor; a virtual machine may report a generic
    name), or None."""
    info = {}
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if not ln.strip():
                    break  # end of the first processor's entry
                k, _, v = ln.partition(":")
                info[k.strip()] = v.strip()
    except OSError:
        return None
    name = info.get("model name")
    if name is None:
        return None
    ids = [f"{k} {info[k]}" for k in ("cpu family", "model", "stepping") if k in info]
    return name + (f" ({', '.join(ids)})" if ids else "")


def cpu_threads():
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit():
        n = min(n, int(env))
    return max(1, n)


def cpu_baseline(workload, x, perm, target_s):
    """The oracle as it stands on a bounded row sample of the same tensor."""
    import numpy as np
    import oracle
    oracle.build(force=False)
    th = cpu_threads()
    oracle.set_threads(th)
    cols = x.shape[1]

    def run(rows):
        xs = np.ascontiguousarray(x[:rows])
        t0 = time.perf_counter()
        if workload == "c4":
            oracle.rotate_quantize(xs, perm, 32)
        else:
            oracle.nv_quantize(xs, True)
        return time.perf_counter() - t0

    probe = min(x.shape[0], 64)
    dt = run(probe)
    rows = int(min(x.shape[0], max(probe, probe * target_s / max(dt, 1e-6))))
    dt = run(rows)
    out = {"value": rows * cols * 2 / dt / 1e9, "unit": "GB/s", "cores": th, "kind": "oracle",
           "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
           "sample": f"first {rows} rows x {cols} cols of the same tensor "
                     f"({rows * cols} elements), {dt:.1f} s on {th} threads"}
    # the same on one thread, on a sample of about a quarter of that time
    oracle.set_threads(1)
    r1 = max(1, min(rows, int(probe * target_s / 4 / max(run(probe), 1e-6))))
    dt1 = run(r1)
    oracle.set_threads(th)
    out["one_thread"] = {"value": r1 * cols * 2 / dt1 / 1e9, "unit": "GB/s",
                         "sample": f"first {r1} rows, {dt1:.1f} s on 1 thread"}
    return out


def bench_c4(torch, fp4, inputs, args):
    import numpy as np
    rows, cols = inputs.FULL_SHAPES["c4"]
    log(f"[bench] generating c4 {rows}x{cols}")
    x = inputs.gen_c4()
    xs = dev_copies(torch, x, copies_for(x.nbytes))
    # the outputs cycle too: enough code (and scale) buffers that what the
    # steps write also exceeds twice the Infinity Cache, so that no step
    # overwrites codes still held in the cache (that would spare HBM the
    # writes); step i reads input copy i % len(xs) and writes buffer i % n
    nin = len(xs)
    n = copies_for(rows * cols // 2, nin)
    n += (-n) % nin
    xs = [xs[k % nin] for k in range(n)]
    codes = [torch.empty((rows, cols // 2), dtype=torch.uint8, device="cuda") for _ in range(n)]
    scales = [torch.empty((rows, cols // 32), dtype=torch.uint8, device="cuda") for _ in range(n)]

    log("[bench] calibrating the permutation (channel energy + host builder)")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    energy = fp4.channel_energy(xs[0])
    perm_cpu = fp4.build_permutation(energy)
    perm = perm_cpu.cuda()
    torch.cuda.synchronize()
    calib_ms = (time.perf_counter() - t0) * 1e3
    e_ms = timed(torch, lambda i: fp4.channel_energy(xs[i % n]), 5, 1)

    # one prepared library call per input copy: the arguments are checked once,
    # each step enqueues the fused kernel straight through the C ABI
    plans = [fp4.rotate_quantize(xs[k], perm, 32, codes=codes[k], scales=scales[k], prepare=True)
             for k in range(n)]

    def step(i):
        plans[i % n].run()

    log(f"[bench] timing {args.steps} steps after {args.warmup} warmup")
    ms = timed(torch, step, args.steps, args.warmup)
    dist = step_distribution(torch, step, 200)
    # the same step at its sustained speed: 500 steps timed after warm-up steps
    # have run for ROW_WARM_MS (informational; value keeps the protocol above)
    sustained_us = timed(torch, step, 500, args.warmup, ROW_WARM_MS) * 1e3
    elems = rows * cols
    value = elems * 2 / (ms * 1e-3) / 1e9
    achieved = elems * B_MX / (ms * 1e-3) / 1e9

    xh = fp4.dequantize(codes[0], scales[0], fp4.MXFP4, perm=perm, hadamard=32)
    q = sqnr_db(torch, xs[0].float(), xh.float())
    c_pl, s_pl, _ = fp4.quantize(xs[0], fp4.MXFP4)
    q_plain = sqnr_db(torch, xs[0].float(), fp4.dequantize(c_pl, s_pl, fp4.MXFP4).float())

    extras = {"step_us_p10_p50_p90": dist, "step_us_sustained": round(sustained_us, 2),
              "sustained_frac_hbm": round(elems * B_MX / sustained_us / 1e3 / HBM_PEAK_GBS, 4),
              "calibration_ms": round(calib_ms, 3), "channel_energy_ms": round(e_ms, 4),
              "sqnr_db_plain_mxfp4": round(q_plain, 3), "device_copy": device_copy(torch)}
    if not args.no_extras:
        extras.update(extra_rows(torch, fp4, inputs, xs, perm, codes, scales))
    res = {
        "ms": ms, "value": value, "elems": elems, "sqnr": q,
        "config": {"workload": "c4: 16384x8192 bf16 activations, per-32-channel-block "
                               "variance exp(1.5 z); channel permutation + block Hadamard-32 "
                               "+ MXFP4 (E8M0, block 32) quantize + pack",
                   "rows": rows, "cols": cols, "format": "mxfp4", "block": 32,
                   "rotation": "perm+hadamard32", "input_copies": nin, "output_copies": n},
        "roofline": roofline_c4(elems, ms),
        "extras": extras,
    }
    return res, x, perm_cpu.numpy()


def roofline_c4(elems, ms):
    achieved = elems * B_MX / (ms * 1e-3) / 1e9
    traffic, src = committed_traffic()
    r = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
         "frac": round(achieved / HBM_PEAK_GBS, 4),
         "traffic": None if traffic is None else round(traffic / (ms * 1e-3) / 1e9, 1),
         "kernel": ROT_KERNEL + "<1,0,true,false,false,8> (MXFP4; eight waves, one MFMA tile per wave per row)",
         "bytes_per_launch": int(elems * B_MX),
         "traffic_bytes_per_launch": traffic, "traffic_source": src,
         # the block Hadamard as a dense contraction: 2 x (32x32x16) MFMAs per 32 blocks
         "mfma_bf16_tflops_algorithmic": round(elems * 64 / (ms * 1e-3) / 1e12, 1),
         "mfma_bf16_frac_of_peak": round(elems * 64 / (ms * 1e-3) / 1e12 / MFMA_PEAK_BF16_TFLOPS,
                                         4)}
    return r


def extra_rows(torch, fp4, inputs, xs, perm, codes, scales):
    """The other rows of the path, each on its own workload, same protocol."""
    out = {}
    n = len(xs)
    rows, cols = xs[0].shape
    el = rows * cols

    def gbs(ms, elems, per_el):
        return {"ms": round(ms, 5), "input_GBps": round(elems * 2 / ms / 1e6, 1),
                "algorithmic_GBps": round(elems * per_el / ms / 1e6, 1)}

    def per_copy(make):
        """A step over the input copies from prepared calls (one per copy)."""
        ps = [make(k) for k in range(n)]
        return lambda i: ps[i % n].run()

    ms = timed(torch, per_copy(lambda k: fp4.quantize(xs[k], fp4.MXFP4, codes=codes[k],
                                                      scales=scales[k], prepare=True)), ROW_STEPS, ROW_WARMUP, ROW_WARM_MS)
    out["c4_mxfp4_plain_quantize"] = gbs(ms, el, B_MX)
    ms = timed(torch, per_copy(lambda k: fp4.rotate_quantize(xs[k], None, 32, codes=codes[k],
                                                             scales=scales[k], prepare=True)),
               ROW_STEPS, ROW_WARMUP, ROW_WARM_MS)
    out["c4_mxfp4_hadamard_only"] = gbs(ms, el, B_MX)
    # one output buffer per input copy: the outputs too cycle through more
    # memory than the 256 MB Infinity Cache holds
    outs = [torch.empty_like(xs[0]) for _ in range(n)]
    ms = timed(torch, per_copy(lambda k: fp4.dequantize(codes[k], scales[k], fp4.MXFP4, out=outs[k],
                                                        prepare=True)), ROW_STEPS, ROW_WARMUP, ROW_WARM_MS)
    out["c4_mxfp4_dequantize"] = gbs(ms, el, B_MX)
    ms = timed(torch, per_copy(lambda k: fp4.dequantize(codes[k], scales[k], fp4.MXFP4, perm=perm,
                                                        hadamard=32, out=outs[k], prepare=True)),
               ROW_STEPS, ROW_WARMUP, ROW_WARM_MS)
    out["c4_mxfp4_dequantize_unrotate"] = gbs(ms, el, B_MX)

    # NVFP4 + RaZeR after the two-level rotation on the same tensor (permutation
    # balanced over 16-channel blocks, 16-point Hadamard)
    perm16 = fp4.build_permutation(fp4.channel_energy(xs[0]), 16).cuda()
    s16 = [torch.empty((rows, cols // 16), dtype=torch.uint8, device="cuda") for _ in range(n)]
    t16 = [torch.empty(1, dtype=torch.float32, device="cuda") for _ in range(n)]

    def nv_rot(given):
        return per_copy(lambda k: fp4.rotate_quantize(
            xs[k], perm16, 16, codes=codes[k], scales=s16[k], fmt=fp4.NVFP4, mode=fp4.RAZER,
            tensor_scale=t16[k], scale_given=given, prepare=True))

    ms = timed(torch, nv_rot(False), ROW_STEPS, ROW_WARMUP, ROW_WARM_MS)
    out["c4_nvfp4_razer_perm_h16_with_amax"] = gbs(ms, el, B_NV + 2)
    ms = timed(torch, nv_rot(True), ROW_STEPS, ROW_WARMUP, ROW_WARM_MS)
    out["c4_nvfp4_razer_perm_h16_scale_given"] = gbs(ms, el, B_NV)
    ms = timed(torch, per_copy(lambda k: fp4.dequantize(codes[k], s16[k], fp4.NVFP4, fp4.RAZER,
                                                        t16[k], perm=perm16, hadamard=16,
                                                        out=outs[k], prepare=True)), ROW_STEPS, ROW_WARMUP, ROW_WARM_MS)
    out["c4_nvfp4_razer_dequantize_unrotate"] = gbs(ms, el, B_NV)
    xf = xs[0].float()
    for name, (pm, had) in {"perm_h16": (perm16, 16), "h16": (None, 16),
                            "plain": (None, 0)}.items():
        c, sc, _, ts = fp4.rotate_quantize(xs[0], pm, had, fmt=fp4.NVFP4, mode=fp4.RAZER)
        xh = fp4.dequantize(c, sc, fp4.NVFP4, fp4.RAZER, ts, perm=pm, hadamard=had)
        out[f"c4_sqnr_db_nvfp4_razer_{name}"] = round(sqnr_db(torch, xf, xh.float()), 3)
    del s16

    # MXINT4 (two's complement k/4 elements, E8M0 scale) on the same tensor
    ms = timed(torch, per_copy(lambda k: fp4.quantize(xs[k], fp4.MXINT4, codes=codes[k],
                                                      scales=scales[k], prepare=True)), ROW_STEPS, ROW_WARMUP, ROW_WARM_MS)
    out["c4_mxint4_plain_quantize"] = gbs(ms, el, B_MX)
    ms = timed(torch, per_copy(lambda k: fp4.rotate_quantize(xs[k], perm, 32, codes=codes[k],
                                                             scales=scales[k], fmt=fp4.MXINT4,
                                                             prepare=True)), ROW_STEPS, ROW_WARMUP, ROW_WARM_MS)
    out["c4_mxint4_perm_h32_quantize"] = gbs(ms, el, B_MX)
    ms = timed(torch, per_copy(lambda k: fp4.dequantize(codes[k], scales[k], fp4.MXINT4, perm=perm,
                                                        hadamard=32, out=outs[k], prepare=True)),
               ROW_STEPS, ROW_WARMUP, ROW_WARM_MS)
    out["c4_mxint4_dequantize_unrotate"] = gbs(ms, el, B_MX)
    for name, (pm, had) in {"perm_h32": (perm, 32), "h32": (None, 32),
                            "plain": (None, 0)}.items():
        c, sc, _ = fp4.rotate_quantize(xs[0], pm, had, fmt=fp4.MXINT4)
        xh = fp4.dequantize(c, sc, fp4.MXINT4, perm=pm, hadamard=had)
        out[f"c4_sqnr_db_mxint4_{name}"] = round(sqnr_db(torch, xf, xh.float()), 3)
    del xf

    # the full two-level rotation: the inter-block Givens layers (calibrated on
    # 256 rows after the permutation) applied on the GPU, then the learned block
    # matrix (calibrated on 256 rows of their output) fused with MXFP4
    log("[bench] two-level rotation rows (Givens layers, learned block matrix)")
    t0 = time.perf_counter()
    macro = fp4.calibrate_macro_rotation(xs[0][:256], perm.cpu())
    macro_ms = (time.perf_counter() - t0) * 1e3
    md = macro.to("cuda")
    zs = [torch.empty_like(xs[0]) for _ in range(n)]
    ms = timed(torch, per_copy(lambda k: fp4.apply_channel_rotation(xs[k], md, perm, out=zs[k],
                                                                    prepare=True)), ROW_STEPS, ROW_WARMUP, ROW_WARM_MS)
    out["c4_givens_layers_apply"] = gbs(ms, el, 4)
    ms = timed(torch, per_copy(lambda k: fp4.apply_channel_rotation(xs[k], md, None, out=zs[k],
                                                                    prepare=True)), ROW_STEPS, ROW_WARMUP, ROW_WARM_MS)
    out["c4_givens_layers_apply_no_perm"] = gbs(ms, el, 4)
    t0 = time.perf_counter()
    R, rloss = fp4.calibrate_block_rotation(zs[0][:256], None, iters=30, angles=32)
    block_ms = (time.perf_counter() - t0) * 1e3
    rt = R.cuda()
    ident = torch.arange(cols, dtype=torch.int32, device="cuda")
    ms = timed(torch, per_copy(lambda k: fp4.rotate_quantize_r(zs[k], ident, rt, codes=codes[k],
                                                               scales=scales[k], prepare=True)),
               ROW_STEPS, ROW_WARMUP, ROW_WARM_MS)
    out["c4_mxfp4_learned_r_quantize"] = gbs(ms, el, B_MX)
    ms = timed(torch, per_copy(lambda k: fp4.dequantize_r(codes[k], scales[k], ident, rt, out=outs[k],
                                                          prepare=True)), ROW_STEPS, ROW_WARMUP, ROW_WARM_MS)
    out["c4_mxfp4_learned_r_dequantize"] = gbs(ms, el, B_MX)
    xf, zf = xs[0].float(), zs[0].float()
    c, sc, _ = fp4.rotate_quantize_r(zs[0], ident, rt)
    q_gr = sqnr_db(torch, zf, fp4.dequantize_r(c, sc, ident, rt).float())
    c, sc, _ = fp4.rotate_quantize(zs[0], None, 32)
    q_gh = sqnr_db(torch, zf, fp4.dequantize(c, sc, fp4.MXFP4, hadamard=32).float())
    Rp, _ = fp4.calibrate_block_rotation(xs[0][:256], perm.cpu(), iters=30, angles=32)
    c, sc, _ = fp4.rotate_quantize_r(xs[0], perm, Rp.cuda())
    q_pr = sqnr_db(torch, xf, fp4.dequantize_r(c, sc, perm, Rp.cuda()).float())
    out["c4_two_level"] = {
        "givens_rotations": macro.n_rot, "givens_layers": macro.n_layers,
        "block_variance_spread_before_after": [round(v, 9) for v in macro.spread],
        "givens_calibration_ms": round(macro_ms, 1),
        "block_matrix_calibration_ms": round(block_ms, 1),
        "occupancy_loss_hadamard_learned": [round(v, 6) for v in rloss],
        # round trip in the rotated basis (the transforms are orthogonal)
        "sqnr_db_perm_learned_r": round(q_pr, 3),
        "sqnr_db_perm_givens_h32": round(q_gh, 3),
        "sqnr_db_perm_givens_learned_r": round(q_gr, 3)}
    del zs, xf, zf

    # the heavy-tailed 8192 x 8192 activations: the Hadamard alone, every format
    log("[bench] generating c3 for the rotation rows")
    x3h = inputs.gen_c3()
    x3s = dev_copies(torch, x3h, copies_for(x3h.nbytes))  # beyond the Infinity Cache
    del x3h
    x3 = x3s[0]
    r3, k3 = x3.shape
    p3 = [fp4.rotate_quantize(t, None, 32, prepare=True) for t in x3s]
    ms = timed(torch, lambda i: p3[i % len(p3)].run(), ROW_STEPS, ROW_WARMUP, ROW_WARM_MS)
    out["c3_mxfp4_h32_quantize"] = gbs(ms, r3 * k3, B_MX)
    # the inverse: dequantize + H32 back to bf16 (codes of each input copy)
    q3s = [fp4.rotate_quantize(t, None, 32)[:2] for t in x3s]
    o3 = [torch.empty_like(x3) for _ in q3s]
    d3 = [fp4.dequantize(c, sc, fp4.MXFP4, hadamard=32, out=o, prepare=True)
          for (c, sc), o in zip(q3s, o3)]
    ms = timed(torch, lambda i: d3[i % len(d3)].run(), ROW_STEPS, ROW_WARMUP, ROW_WARM_MS)
    out["c3_mxfp4_dequantize_h32"] = gbs(ms, r3 * k3, B_MX)
    del p3, x3s, q3s, d3, o3
    x3f = x3.float()
    q3 = {}
    for fmt, mode, had, name in ((fp4.MXFP4, fp4.PLAIN, 32, "mxfp4"),
                                 (fp4.MXINT4, fp4.PLAIN, 32, "mxint4"),
                                 (fp4.NVFP4, fp4.RAZER, 16, "nvfp4_razer")):
        for h in (0, had):
            r = fp4.rotate_quantize(x3, None, h, fmt=fmt, mode=mode)
            ts = r[3] if fmt == fp4.NVFP4 else None
            xh = fp4.dequantize(r[0], r[1], fmt, mode, ts, hadamard=h)
            q3[f"{name}_{'h%d' % h if h else 'plain'}"] = round(sqnr_db(torch, x3f, xh.float()), 3)
    out["c3_sqnr_db"] = q3
    del x3, x3f
    out["gemm_mxfp4"] = gemm_rows(torch, fp4, fp4.MXFP4)
    out["gemm_nvfp4_razer"] = gemm_rows(torch, fp4, fp4.NVFP4)

    # NVFP4 + RaZeR on the 4096x4096 weight recipe, enough copies to defeat the cache
    log("[bench] generating c2 for the NVFP4 rows")
    x2 = inputs.gen_c2()
    r2, c2 = x2.shape
    ys = dev_copies(torch, x2, copies_for(x2.nbytes))
    m = len(ys)
    cs = [torch.empty((r2, c2 // 2), dtype=torch.uint8, device="cuda") for _ in range(m)]
    ss = [torch.empty((r2, c2 // 16), dtype=torch.uint8, device="cuda") for _ in range(m)]
    tss = [torch.empty(1, dtype=torch.float32, device="cuda") for _ in range(m)]
    el2 = r2 * c2

    def graph_row(key, fn, per_el):
        # the same calls replayed from a HIP graph (host submission removed)
        us = graph_us(torch, fn, calls=2 * m)
        out[key]["graph_us_per_call"] = round(us, 2)
        out[key]["graph_algorithmic_GBps"] = round(el2 * per_el / us / 1e3, 1)
    def plan(fn, **kw):
        ps = [fn(k, **kw) for k in range(m)]
        return lambda i: ps[i % m].run()
    q_amax = plan(lambda k: fp4.quantize(ys[k], fp4.NVFP4, fp4.RAZER, tensor_scale=tss[k],
                                         scale_given=False, codes=cs[k], scales=ss[k],
                                         prepare=True))
    ms = timed(torch, q_amax, 2 * ROW_STEPS, ROW_WARMUP, ROW_WARM_MS)
    out["c2_nvfp4_razer_quantize_with_amax"] = gbs(ms, el2, B_NV + 2)
    xh = fp4.dequantize(cs[0], ss[0], fp4.NVFP4, fp4.RAZER, tss[0])
    out["c2_sqnr_db_razer"] = round(sqnr_db(torch, ys[0].float(), xh.float()), 3)
    q_razer = plan(lambda k: fp4.quantize(ys[k], fp4.NVFP4, fp4.RAZER, tensor_scale=tss[k],
                                          codes=cs[k], scales=ss[k], prepare=True))
    ms = timed(torch, q_razer, 2 * ROW_STEPS, ROW_WARMUP, ROW_WARM_MS)
    out["c2_nvfp4_razer_quantize_scale_given"] = gbs(ms, el2, B_NV)
    graph_row("c2_nvfp4_razer_quantize_scale_given", q_razer, B_NV)
    q_plain = plan(lambda k: fp4.quantize(ys[k], fp4.NVFP4, fp4.PLAIN, tensor_scale=tss[k],
                                          codes=cs[k], scales=ss[k], prepare=True))
    ms = timed(torch, q_plain, 2 * ROW_STEPS, ROW_WARMUP, ROW_WARM_MS)
    out["c2_nvfp4_plain_quantize_scale_given"] = gbs(ms, el2, B_NV)
    graph_row("c2_nvfp4_plain_quantize_scale_given", q_plain, B_NV)
    for k in range(m):
        fp4.quantize(ys[k], fp4.NVFP4, fp4.RAZER, tensor_scale=tss[k], codes=cs[k], scales=ss[k])
    obs = [torch.empty_like(ys[0]) for _ in range(m)]
    dq = plan(lambda k: fp4.dequantize(cs[k], ss[k], fp4.NVFP4, fp4.RAZER, tss[k], out=obs[k],
                                       prepare=True))
    ms = timed(torch, dq, 2 * ROW_STEPS, ROW_WARMUP, ROW_WARM_MS)
    out["c2_nvfp4_razer_dequantize"] = gbs(ms, el2, B_NV)
    graph_row("c2_nvfp4_razer_dequantize", dq, B_NV)
    ms = timed(torch, plan(lambda k: fp4.quantize(ys[k], fp4.NVFP4, fp4.RAZER_W,
                                                  tensor_scale=tss[k], codes=cs[k], scales=ss[k],
                                                  prepare=True)), 2 * ROW_STEPS, ROW_WARMUP, ROW_WARM_MS)
    out["c2_nvfp4_razer_w_quantize_scale_given"] = gbs(ms, el2, B_NV)
    cw, sw, tw = fp4.quantize(ys[0], fp4.NVFP4, fp4.RAZER_W)
    xw = fp4.dequantize(cw, sw, fp4.NVFP4, fp4.RAZER_W, tw)
    out["c2_sqnr_db_razer_w"] = round(sqnr_db(torch, ys[0].float(), xw.float()), 3)
    cp, sp, tp = fp4.quantize(ys[0], fp4.NVFP4, fp4.PLAIN)
    xp = fp4.dequantize(cp, sp, fp4.NVFP4, fp4.PLAIN, tp)
    out["c2_sqnr_db_plain_nvfp4"] = round(sqnr_db(torch, ys[0].float(), xp.float()), 3)
    del ys, cs, ss
    out["c1_mxfp4"] = c1_rows(torch, fp4, inputs)
    out["c5_layer_nvfp4_razer"] = c5_rows(torch, fp4, inputs)
    out["wide_rows_8192x28672"] = wide_rows(torch, fp4, inputs)
    return out


def wide_rows(torch, fp4, inputs):
    """The two-level rotation on rows as wide as the down projection's input
    (8192 x 28672, the c4 recipe at that width): the LDS-ring permuting kernel
    per format, beside plain MXFP4 quantization of the same tensor."""
    rows, cols = 8192, 28672
    log(f"[bench] generating {rows}x{cols} for the wide-row rotation rows")
    x = inputs.gen_c4(rows=rows, cols=cols)
    xs = dev_copies(torch, x, copies_for(x.nbytes))
    del x
    nin = len(xs)
    n = copies_for(rows * cols // 2, nin)  # code buffers beyond the cache as well
    n += (-n) % nin
    xs = [xs[k % nin] for k in range(n)]
    el = rows * cols
    perm = fp4.build_permutation(fp4.channel_energy(xs[0])).cuda()
    perm16 = fp4.build_permutation(fp4.channel_energy(xs[0]), 16).cuda()
    codes = [torch.empty((rows, cols // 2), dtype=torch.uint8, device="cuda") for _ in range(n)]
    s32 = [torch.empty((rows, cols // 32), dtype=torch.uint8, device="cuda") for _ in range(n)]
    s16 = [torch.empty((rows, cols // 16), dtype=torch.uint8, device="cuda") for _ in range(n)]
    t16 = [fp4.rotate_quantize(xs[k], perm16, 16, codes=codes[k], scales=s16[k], fmt=fp4.NVFP4,
                               mode=fp4.RAZER)[3] for k in range(n)]

    def row(make, per_el):
        ps = [make(k) for k in range(n)]
        ms = timed(torch, lambda i: ps[i % n].run(), ROW_STEPS, ROW_WARMUP, ROW_WARM_MS)
        return {"ms": round(ms, 5), "input_GBps": round(el * 2 / ms / 1e6, 1),
                "algorithmic_GBps": round(el * per_el / ms / 1e6, 1),
                "frac_hbm": round(el * per_el / ms / 1e6 / HBM_PEAK_GBS, 4)}

    out = {
        "mxfp4_plain_quantize": row(lambda k: fp4.quantize(xs[k], fp4.MXFP4, codes=codes[k],
                                                           scales=s32[k], prepare=True), B_MX),
        "mxfp4_perm_h32_quantize": row(lambda k: fp4.rotate_quantize(
            xs[k], perm, 32, codes=codes[k], scales=s32[k], prepare=True), B_MX),
        "mxint4_perm_h32_quantize": row(lambda k: fp4.rotate_quantize(
            xs[k], perm, 32, codes=codes[k], scales=s32[k], fmt=fp4.MXINT4, prepare=True), B_MX),
        "nvfp4_razer_perm_h16_scale_given": row(lambda k: fp4.rotate_quantize(
            xs[k], perm16, 16, codes=codes[k], scales=s16[k], fmt=fp4.NVFP4, mode=fp4.RAZER,
            tensor_scale=t16[k], scale_given=True, prepare=True), B_NV),
    }
    del xs, codes, s32, s16
    torch.cuda.empty_cache()
    return out


def c1_rows(torch, fp4, inputs):
    """C1: MXFP4 quantize and dequantize of the 256 x 4096 tensor (2 MB in,
    launch-bound: also timed from a HIP graph replay), bit-exactness aside
    (the tests cover it) and the round-trip SQNR."""
    log("[bench] c1 MXFP4 256x4096")
    x = inputs.gen_c1()
    xt = dev_copies(torch, x, 1)[0]
    r, c = x.shape
    el = r * c
    codes = torch.empty((r, c // 2), dtype=torch.uint8, device="cuda")
    scales = torch.empty((r, c // 32), dtype=torch.uint8, device="cuda")
    outb = torch.empty_like(xt)
    pq = fp4.quantize(xt, fp4.MXFP4, codes=codes, scales=scales, prepare=True)
    pd = fp4.dequantize(codes, scales, fp4.MXFP4, out=outb, prepare=True)
    q = lambda i: pq.run()
    d = lambda i: pd.run()
    res = {}
    for name, fn in (("quantize", q), ("dequantize", d)):
        ms = timed(torch, fn, 200, 20, ROW_WARM_MS)
        us = graph_us(torch, fn, calls=50)
        res[name] = {"us": round(ms * 1e3, 2), "graph_us_per_call": round(us, 2),
                     "graph_algorithmic_GBps": round(el * B_MX / us / 1e3, 1)}
    q(0)
    d(0)
    res["sqnr_db"] = round(sqnr_db(torch, xt.float(), outb.float()), 3)
    return res


def c5_rows(torch, fp4, inputs, steps=5, warmup=3, razer_w=False):
    """C5: the Llama-70B-shaped decoder layer's seven weights (855,638,016
    bf16), NVFP4 + RaZeR: quantize with the tensor amax pass, quantize with s_t
    given, dequantize to bf16, and the round trip (amax + quantize +
    dequantize); per-tensor and layer SQNR. One copy of each weight: the 1.7 GB
    layer is several times the 256 MB Infinity Cache, so every pass reads HBM."""
    xs, cs, ss, ts, outs, names = [], [], [], [], [], []
    el = 0
    for t, (name, r, c) in enumerate(inputs.C5_SHAPES):
        log(f"[bench] generating c5 {name} {r}x{c}")
        x = inputs.gen_c5(t)
        xs.append(dev_copies(torch, x, 1)[0])
        cs.append(torch.empty((r, c // 2), dtype=torch.uint8, device="cuda"))
        ss.append(torch.empty((r, c // 16), dtype=torch.uint8, device="cuda"))
        ts.append(torch.empty(1, dtype=torch.float32, device="cuda"))
        outs.append(torch.empty_like(xs[-1]))
        names.append(name)
        el += r * c
        del x
    n = len(xs)
    mode = fp4.RAZER_W if razer_w else fp4.RAZER

    def layer(make):
        """One pass over the seven tensors from prepared calls."""
        ps = [make(k) for k in range(n)]

        def run(i):
            for p in ps:
                p.run()
        return run

    def quant(m, given):
        return layer(lambda k: fp4.quantize(xs[k], fp4.NVFP4, m, tensor_scale=ts[k],
                                            scale_given=given, codes=cs[k], scales=ss[k],
                                            prepare=True))

    quant_amax, quant_given = quant(mode, False), quant(mode, True)
    dequant = layer(lambda k: fp4.dequantize(cs[k], ss[k], fp4.NVFP4, mode, ts[k], out=outs[k],
                                             prepare=True))

    def round_trip(i):
        quant_amax(i)
        dequant(i)

    res = {"elements": el}

    def row(name, fn, per):
        ms = timed(torch, fn, steps, warmup, ROW_WARM_MS)
        res[name] = {"ms": round(ms, 4), "input_GBps": round(el * 2 / ms / 1e6, 1),
                     "algorithmic_GBps": round(el * per / ms / 1e6, 1),
                     "frac_hbm": round(el * per / ms / 1e6 / HBM_PEAK_GBS, 4)}

    row("quantize_with_amax", quant_amax, B_NV + 2)
    row("quantize_scale_given", quant_given, B_NV)
    row("dequantize", dequant, B_NV)
    row("round_trip", round_trip, 2 * B_NV + 2)
    if not razer_w:
        # the same quantize passes in plain NVFP4: what RaZeR's choice costs
        row("plain_quantize_with_amax", quant(fp4.PLAIN, False), B_NV + 2)
        row("plain_quantize_scale_given", quant(fp4.PLAIN, True), B_NV)
    round_trip(0)
    torch.cuda.synchronize()
    num = den = 0.0
    per_t = {}
    for k in range(n):
        xd = xs[k].double()
        e = float(((xd - outs[k].double()) ** 2).sum())
        s2 = float((xd * xd).sum())
        per_t[names[k]] = round(10 * math.log10(s2 / e), 3)
        num += s2
        den += e
    res["sqnr_db_per_tensor"] = per_t
    res["sqnr_db_layer"] = round(10 * math.log10(num / den), 3)
    del xs, cs, ss, ts, outs
    return res


MFMA_PEAK_FP4_TFLOPS = 10100.0


def gemm_rows(torch, fp4, fmt):
    """The consumer: C = A B^T on quantized operands (activations [m, k],
    weights [n, k] of the Llama-70B-shaped layer), bf16 out. MXFP4 runs on the
    scaled FP4 matrix cores (peak 10.1 PFLOP/s), with both operands' scales in
    the GEMM order (the quantizers' FP4_FLAG_SCALES_GEMM output; the row-major
    time is given beside it); NVFP4 + RaZeR on both sides is decoded exactly
    to bf16 and runs on the bf16 ones (peak 2.5 PFLOP/s). Random codes and
    finite scale bytes: the time does not depend on values."""
    nv = fmt == fp4.NVFP4
    blk, lo, hi = (16, 40, 60) if nv else (32, 120, 131)
    peak = MFMA_PEAK_BF16_TFLOPS if nv else MFMA_PEAK_FP4_TFLOPS
    log(f"[bench] {'NVFP4+RaZeR' if nv else 'MXFP4'} GEMM rows")
    g = torch.Generator(device="cuda").manual_seed(5)
    ts = torch.ones(1, dtype=torch.float32, device="cuda")
    kw = dict(fmt=fp4.NVFP4, a_ts=ts, b_ts=ts, mode_a=fp4.RAZER, mode_b=fp4.RAZER) if nv else {}
    rows = {}
    for m, n, k in ((4096, 8192, 8192), (4096, 28672, 8192), (4096, 8192, 28672),
                    (16, 8192, 8192), (32, 28672, 8192)):
        # operand and output sets cycle over more than twice the Infinity Cache,
        # so no call finds its weights (or overwrites its output) still cached
        nset = copies_for((m + n) * (k // 2 + k // blk) + 2 * m * n)

        def rnd(shape, a_, b_):
            return torch.randint(a_, b_, shape, dtype=torch.uint8, device="cuda", generator=g)

        sets = [(rnd((m, k // 2), 0, 256), rnd((m, k // blk), lo, hi),
                 rnd((n, k // 2), 0, 256), rnd((n, k // blk), lo, hi),
                 torch.empty((m, n), dtype=torch.bfloat16, device="cuda")) for _ in range(nset)]
        row_major = None
        if not nv:
            p0 = [fp4.gemm(a, sa, b, sb, out=c, prepare=True) for a, sa, b, sb, c in sets]
            ms0 = timed(torch, lambda i: p0[i % nset].run(), 10, 2, ROW_WARM_MS)
            row_major = {"ms": round(ms0, 4), "frac_mfma_peak": round(
                2.0 * m * n * k / (ms0 * 1e-3) / 1e12 / peak, 4)}
            pl = [fp4.gemm(a, rnd(fp4.gemm_scale_shape(m, k), lo, hi), b,
                           rnd(fp4.gemm_scale_shape(n, k), lo, hi), out=c, prepare=True,
                           a_gemm_scales=True, b_gemm_scales=True)
                  for a, sa, b, sb, c in sets]
        else:
            pl = [fp4.gemm(a, sa, b, sb, out=c, prepare=True, **kw) for a, sa, b, sb, c in sets]
        ms = timed(torch, lambda i: pl[i % nset].run(), 10, 2, ROW_WARM_MS)
        tf = 2.0 * m * n * k / (ms * 1e-3) / 1e12
        by = (m + n) * (k / 2 + k / blk) + 2 * m * n
        rows[f"{m}x{n}x{k}"] = {"ms": round(ms, 4), "TFLOPs": round(tf, 1),
                                "frac_mfma_peak": round(tf / peak, 4),
                                "GBps": round(by / ms / 1e6, 1)}
        if row_major is not None:
            rows[f"{m}x{n}x{k}"]["scales"] = "GEMM order"
            rows[f"{m}x{n}x{k}"]["row_major_scales"] = row_major
        rows[f"{m}x{n}x{k}"]["operand_sets"] = nset
        if m <= 32:  # µs-scale launches: also their time replayed from a graph
            us = graph_us(torch, lambda i: pl[i % nset].run(), calls=max(20, nset))
            rows[f"{m}x{n}x{k}"]["graph_us_per_call"] = round(us, 2)
            rows[f"{m}x{n}x{k}"]["graph_frac_mfma_peak"] = round(
                2.0 * m * n * k / (us * 1e-6) / 1e12 / peak, 4)
        if not nv and m >= 256:
            rows[f"{m}x{n}x{k}"]["library"] = library_mx_gemm(torch, sets, peak)
        del sets, pl
    return rows


def library_mx_gemm(torch, sets, peak):
    """The same MXFP4 product through torch._scaled_mm (the ROCm math
    library's block-scaled FP4 GEMM), timed with the same protocol: a
    reference point for the hand-written kernel, not part of the path. Timing
    only (the operands are random bytes; the library's scale layout is not
    checked against ours)."""
    try:
        ops = [(a.view(torch.float4_e2m1fn_x2), b.view(torch.float4_e2m1fn_x2),
                sa.view(torch.float8_e8m0fnu), sb.view(torch.float8_e8m0fnu))
               for a, sa, b, sb, _ in sets]

        def fn(i):  # operands cycle as for the hand-written kernel (output allocated per call)
            A, B, SA, SB = ops[i % len(ops)]
            return torch._scaled_mm(A, B.t(), SA, SB, out_dtype=torch.bfloat16)

        fn(0)
        ms = timed(torch, fn, 10, 2, ROW_WARM_MS)
    except Exception as ex:  # not available in this torch build
        return {"error": f"{type(ex).__name__}: {str(ex)[:120]}"}
    a, b = sets[0][0], sets[0][2]
    m, k = a.shape[0], 2 * a.shape[1]
    n = b.shape[0]
    tf = 2.0 * m * n * k / (ms * 1e-3) / 1e12
    return {"call": "torch._scaled_mm", "ms": round(ms, 4), "TFLOPs": round(tf, 1),
            "frac_mfma_peak": round(tf / peak, 4)}


def bench_c1(torch, fp4, inputs, args):
    """C1: MXFP4 quantize + dequantize of the 256 x 4096 tensor, one step =
    both calls (launch-bound at this size)."""
    x = inputs.gen_c1()
    xt = dev_copies(torch, x, 1)[0]
    r, c = x.shape
    codes = torch.empty((r, c // 2), dtype=torch.uint8, device="cuda")
    scales = torch.empty((r, c // 32), dtype=torch.uint8, device="cuda")
    outb = torch.empty_like(xt)

    pq = fp4.quantize(xt, fp4.MXFP4, codes=codes, scales=scales, prepare=True)
    pd = fp4.dequantize(codes, scales, fp4.MXFP4, out=outb, prepare=True)

    def step(i):
        pq.run()
        pd.run()

    ms = timed(torch, step, args.steps, args.warmup)
    el = r * c
    return {"ms": ms, "value": el * 2 / ms / 1e6, "elems": el,
            "sqnr": sqnr_db(torch, xt.float(), outb.float()),
            "config": {"workload": "c1: 256x4096 bf16 N(0,0.02) + 0.1% outliers x20; MXFP4 "
                                   "(E8M0, block 32) quantize then dequantize", "rows": r,
                       "cols": c, "format": "mxfp4", "block": 32},
            "roofline": {"bound": "hbm", "achieved": el * 2 * B_MX / ms / 1e6,
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": el * 2 * B_MX / ms / 1e6 / HBM_PEAK_GBS, "traffic": None,
                         "kernel": "mx_quant_kernel + mx_dequant_kernel (launch-bound)",
                         "bytes_per_launch": int(el * B_MX)},
            "extras": {"graph": c1_rows(torch, fp4, inputs)}}, x, None


def bench_c3(torch, fp4, inputs, args):
    """C3: 32-point block Hadamard + MXFP4 on the 8192 x 8192 heavy-tailed
    activations (one fused launch per step, two input copies)."""
    x = inputs.gen_c3()
    xs = dev_copies(torch, x, copies_for(x.nbytes))
    n = len(xs)
    r, c = x.shape
    codes = [torch.empty((r, c // 2), dtype=torch.uint8, device="cuda") for _ in range(n)]
    scales = [torch.empty((r, c // 32), dtype=torch.uint8, device="cuda") for _ in range(n)]

    plans = [fp4.rotate_quantize(xs[k], None, 32, codes=codes[k], scales=scales[k], prepare=True)
             for k in range(n)]

    def step(i):
        plans[i % n].run()

    ms = timed(torch, step, args.steps, args.warmup)
    el = r * c
    xh = fp4.dequantize(codes[0], scales[0], fp4.MXFP4, hadamard=32)
    return {"ms": ms, "value": el * 2 / ms / 1e6, "elems": el,
            "sqnr": sqnr_db(torch, xs[0].float(), xh.float()),
            "config": {"workload": "c3: 8192x8192 bf16 activations 0.5 Student-t(3), 16 "
                                   "channels x50; block Hadamard-32 + MXFP4 quantize + pack",
                       "rows": r, "cols": c, "format": "mxfp4", "block": 32,
                       "rotation": "hadamard32", "input_copies": n},
            "roofline": {"bound": "hbm", "achieved": el * B_MX / ms / 1e6, "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": el * B_MX / ms / 1e6 / HBM_PEAK_GBS,
                         "traffic": None, "kernel": "mx_rotq_stream_mfma_kernel",
                         "bytes_per_launch": int(el * B_MX)},
            "extras": {"step_us_p10_p50_p90": step_distribution(torch, step, 200)}}, None, None


def bench_c2(torch, fp4, inputs, args):
    r, c = inputs.FULL_SHAPES["c2"]
    x = inputs.gen_c2()
    ys = dev_copies(torch, x, copies_for(x.nbytes))
    m = len(ys)
    cs = [torch.empty((r, c // 2), dtype=torch.uint8, device="cuda") for _ in range(m)]
    ss = [torch.empty((r, c // 16), dtype=torch.uint8, device="cuda") for _ in range(m)]
    tss = [torch.empty(1, dtype=torch.float32, device="cuda") for _ in range(m)]

    plans = [fp4.quantize(ys[k], fp4.NVFP4, fp4.RAZER, tensor_scale=tss[k], scale_given=False,
                          codes=cs[k], scales=ss[k], prepare=True) for k in range(m)]

    def step(i):
        plans[i % m].run()

    ms = timed(torch, step, args.steps, args.warmup)
    el = r * c
    xh = fp4.dequantize(cs[0], ss[0], fp4.NVFP4, fp4.RAZER, tss[0])
    res = {"ms": ms, "value": el * 2 / ms / 1e6, "elems": el,
           "sqnr": sqnr_db(torch, ys[0].float(), xh.float()),
           "config": {"workload": "c2: 4096x4096 bf16 weights N(0,0.02) + 0.5% Laplace(0,0.3); "
                                  "NVFP4 (E4M3 block 16 + fp32 tensor scale) + RaZeR, tensor "
                                  "amax computed each step", "rows": r, "cols": c,
                      "format": "nvfp4", "block": 16, "mode": "razer", "input_copies": m},
           "roofline": {"bound": "hbm", "achieved": el * (B_NV + 2) / ms / 1e6,
                        "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": el * (B_NV + 2) / ms / 1e6 / HBM_PEAK_GBS, "traffic": None,
                        "kernel": "nv_amax_kernel + nv_quant_kernel<true,true>",
                        "bytes_per_launch": int(el * (B_NV + 2))},
           "extras": {}}
    return res, x, None


def bench_c5(torch, fp4, inputs, args):
    """Llama-70B-shaped layer: NVFP4+RaZeR quantize then dequantize of all 7 weights."""
    xs, cs, ss, ts, outs = [], [], [], [], []
    el = 0
    for t, (name, r, c) in enumerate(inputs.C5_SHAPES):
        log(f"[bench] generating c5 {name} {r}x{c}")
        x = inputs.gen_c5(t)
        xs.append(dev_copies(torch, x, 1)[0])
        cs.append(torch.empty((r, c // 2), dtype=torch.uint8, device="cuda"))
        ss.append(torch.empty((r, c // 16), dtype=torch.uint8, device="cuda"))
        ts.append(torch.empty(1, dtype=torch.float32, device="cuda"))
        outs.append(torch.empty_like(xs[-1]))
        el += r * c
        del x

    plans = [p for k in range(len(xs)) for p in (
        fp4.quantize(xs[k], fp4.NVFP4, fp4.RAZER, tensor_scale=ts[k], scale_given=False,
                     codes=cs[k], scales=ss[k], prepare=True),
        fp4.dequantize(cs[k], ss[k], fp4.NVFP4, fp4.RAZER, ts[k], out=outs[k], prepare=True))]

    def step(i):
        for p in plans:
            p.run()

    ms = timed(torch, step, args.steps, args.warmup)
    import math

    def layer_sqnr():
        num = sum(float((xs[k].double() ** 2).sum()) for k in range(len(xs)))
        den = sum(float(((xs[k].double() - outs[k].double()) ** 2).sum())
                  for k in range(len(xs)))
        return 10 * math.log10(num / den)

    sqnr = layer_sqnr()

    # the same layer with RaZeR for weights (E3M3 scales, four special values)
    def step_w(i):
        for k in range(len(xs)):
            fp4.quantize(xs[k], fp4.NVFP4, fp4.RAZER_W, tensor_scale=ts[k], scale_given=False,
                         codes=cs[k], scales=ss[k])
            fp4.dequantize(cs[k], ss[k], fp4.NVFP4, fp4.RAZER_W, ts[k], out=outs[k])

    ms_w = timed(torch, step_w, max(3, args.steps // 2), 1)
    extras = {"razer_w_layer_round_trip": {"ms": round(ms_w, 4),
                                           "algorithmic_GBps": round(el * (2 * B_NV + 2) / ms_w
                                                                     / 1e6, 1),
                                           "sqnr_db": round(layer_sqnr(), 3)}}
    for k in range(len(xs)):
        fp4.quantize(xs[k], fp4.NVFP4, fp4.PLAIN, tensor_scale=ts[k], scale_given=False,
                     codes=cs[k], scales=ss[k])
        fp4.dequantize(cs[k], ss[k], fp4.NVFP4, fp4.PLAIN, ts[k], out=outs[k])
    extras["plain_nvfp4_sqnr_db"] = round(layer_sqnr(), 3)
    # the kernels of one timed step and their launches per step (for the
    # per-step sum of a kernel trace: other passes above launch some of them too)
    extras["step_kernel_calls"] = {"nv_amax_kernel<": len(xs), "nv_tensor_scale_kernel<": len(xs),
                                   "nv_quant_kernel<true, 1>": len(xs),
                                   "nv_dequant_kernel<true, 1>": len(xs)}
    per_el = (B_NV + 2) + B_NV
    res = {"ms": ms, "value": el * 2 / ms / 1e6, "elems": el, "sqnr": sqnr,
           "config": {"workload": "c5: Llama-70B-shaped decoder-layer weights q,k,v,o,gate,up,"
                                  "down (855,638,016 bf16), NVFP4+RaZeR quantize with tensor "
                                  "amax, then dequantize to bf16", "tensors": 7,
                      "format": "nvfp4", "block": 16, "mode": "razer"},
           "roofline": {"bound": "hbm", "achieved": el * per_el / ms / 1e6, "peak": HBM_PEAK_GBS,
                        "unit": "GB/s", "frac": el * per_el / ms / 1e6 / HBM_PEAK_GBS,
                        "traffic": None, "kernel": "nv_amax + nv_quant + nv_dequant (7 tensors)",
                        "bytes_per_launch": int(el * per_el)},
           "extras": extras}
    return res, None, None


KERNEL_OPS = {
    "c4_perm_mxfp4": "fused permutation + Hadamard-32 + MXFP4 quantize, 16384x8192 bf16 (c4)",
    "c4_perm_nvfp4_razer": "fused permutation + Hadamard-16 + NVFP4 + RaZeR quantize, tensor "
                           "scale given, 16384x8192 bf16 (c4)",
    "c4_unrot_mxfp4": "MXFP4 dequantize + inverse Hadamard-32 and permutation, 16384x8192 "
                      "(c4), bf16 out",
    "c4_unrot_mxint4": "MXINT4 dequantize + inverse Hadamard-32 and permutation, 16384x8192 "
                       "(c4), bf16 out",
    "c4_unrot_nvfp4_razer": "NVFP4 + RaZeR dequantize + inverse Hadamard-16 and permutation, "
                            "16384x8192 (c4), bf16 out",
    "c2_nvfp4_plain": "NVFP4 quantize, tensor scale given, 4096x4096 bf16 (c2)",
    "c2_nvfp4_razer": "NVFP4 + RaZeR quantize, tensor scale given, 4096x4096 bf16 (c2)",
    "gemm_mxfp4": "MXFP4 x MXFP4 GEMM, m=4096 n=8192 k=8192, bf16 out",
    "gemm_mxfp4_gemm_scales": "MXFP4 x MXFP4 GEMM, m=4096 n=8192 k=8192, bf16 out, both "
                              "operands' scales in the GEMM order",
}


def kernel_op(torch, fp4, inputs, args):
    """One kernel on its own: args.warmup untimed launches, then args.steps
    timed ones, over enough input copies to read from HBM. Prints one JSON line
    naming the kernel, the units one launch processes and the ms per launch,
    which --counter-summary reads beside the counter directories."""
    op = args.kernel_op
    if op.startswith("c4_"):
        rows, cols = inputs.FULL_SHAPES["c4"]
        x = inputs.gen_c4()
        xs = dev_copies(torch, x, copies_for(x.nbytes))
        del x
        nin = len(xs)
        n = copies_for(rows * cols // 2, nin)  # code buffers beyond the cache as well
        n += (-n) % nin
        xs = [xs[k % nin] for k in range(n)]
        nv = op in ("c4_perm_nvfp4_razer", "c4_unrot_nvfp4_razer")
        blk = 16 if nv else 32
        perm = fp4.build_permutation(fp4.channel_energy(xs[0]), blk).cuda()
        codes = [torch.empty((rows, cols // 2), dtype=torch.uint8, device="cuda") for _ in range(n)]
        scales = [torch.empty((rows, cols // blk), dtype=torch.uint8, device="cuda")
                  for _ in range(n)]
        kw = {}
        if nv:
            ts = [fp4.rotate_quantize(xs[k], perm, 16, fmt=fp4.NVFP4, mode=fp4.RAZER)[3]
                  for k in range(n)]
            kw = lambda k: dict(fmt=fp4.NVFP4, mode=fp4.RAZER, tensor_scale=ts[k])
        else:
            kw = lambda k: {}
        if op.startswith("c4_unrot_"):
            fmt = {"mxfp4": fp4.MXFP4, "mxint4": fp4.MXINT4, "nvfp4_razer": fp4.NVFP4}[op[9:]]
            mode = fp4.RAZER if nv else fp4.PLAIN
            outs = [torch.empty_like(xs[k]) for k in range(n)]
            ps = []
            for k in range(n):
                r = fp4.rotate_quantize(xs[k], perm, blk, codes=codes[k], scales=scales[k],
                                        fmt=fmt, mode=mode)
                ts_k = r[3] if nv else None
                ps.append(fp4.dequantize(codes[k], scales[k], fmt, mode, ts_k, perm=perm,
                                         hadamard=blk, out=outs[k], prepare=True))
            kernel = "dequant_unrotate_kernel<" + {fp4.MXFP4: "2, 0,", fp4.NVFP4: "1, 1,",
                                                    fp4.MXINT4: "1, 2,"}[fmt]
        else:
            ps = [fp4.rotate_quantize(xs[k], perm, blk, codes=codes[k], scales=scales[k],
                                      prepare=True, **kw(k)) for k in range(n)]
            kernel = ROT_KERNEL + ("<1, 1, true, true, false, 8>" if nv
                                   else "<1, 0, true, false, false, 8>")
        units, unit = rows * cols, "element"
    elif op.startswith("c2_"):
        x = inputs.gen_c2()
        r, c = x.shape
        xs = dev_copies(torch, x, copies_for(x.nbytes))
        del x
        n = len(xs)
        mode = fp4.RAZER if op == "c2_nvfp4_razer" else fp4.PLAIN
        ps = []
        for k in range(n):
            cq, sq, tq = fp4.quantize(xs[k], fp4.NVFP4, mode)  # tensor scale, untimed
            ps.append(fp4.quantize(xs[k], fp4.NVFP4, mode, tensor_scale=tq, codes=cq, scales=sq,
                                   prepare=True))
        kernel = f"nv_quant_kernel<true, {1 if mode == fp4.RAZER else 0}>"
        units, unit = r * c, "element"
    else:
        m, nn, k = 4096, 8192, 8192
        g = torch.Generator(device="cuda").manual_seed(5)
        a = torch.randint(0, 256, (m, k // 2), dtype=torch.uint8, device="cuda", generator=g)
        sa = torch.randint(120, 131, (m, k // 32), dtype=torch.uint8, device="cuda", generator=g)
        b = torch.randint(0, 256, (nn, k // 2), dtype=torch.uint8, device="cuda", generator=g)
        sb = torch.randint(120, 131, (nn, k // 32), dtype=torch.uint8, device="cuda", generator=g)
        cm = torch.empty((m, nn), dtype=torch.bfloat16, device="cuda")
        if op == "gemm_mxfp4_gemm_scales":  # random scale bytes, laid out in the GEMM order
            sa = torch.randint(120, 131, fp4.gemm_scale_shape(m, k), dtype=torch.uint8,
                               device="cuda", generator=g)
            sb = torch.randint(120, 131, fp4.gemm_scale_shape(nn, k), dtype=torch.uint8,
                               device="cuda", generator=g)
        gs = op == "gemm_mxfp4_gemm_scales"
        ps = [fp4.gemm(a, sa, b, sb, out=cm, prepare=True, a_gemm_scales=gs, b_gemm_scales=gs)]
        kernel = "mx_gemm_kernel<"
        units, unit = 2 * m * nn * k, "flop"
    ms = timed(torch, lambda i: ps[i % len(ps)].run(), args.steps, args.warmup)
    print(json.dumps({"kernel_op": op, "what": KERNEL_OPS[op], "kernel": kernel,
                      "units_per_launch": units, "unit": unit, "steps": args.steps,
                      "warmup": args.warmup, "ms_per_launch": round(ms, 5)}), flush=True)


# counters whose ratio the summary reports, when a pass holds both
def _pearson(a, b):
    n = len(a)
    ma, mb = sum(a) / n, sum(b) / n
    sab = sum((x - ma) * (y - mb) for x, y in zip(a, b))
    saa = sum((x - ma) ** 2 for x in a)
    sbb = sum((y - mb) ** 2 for y in b)
    return sab / math.sqrt(saa * sbb) if saa > 0 and sbb > 0 else float("nan")


COUNTER_RATIOS = [
    ("LDS bank-conflict cycles per indexed-LDS active cycle", "SQ_LDS_BANK_CONFLICT",
     "SQ_LDS_IDX_ACTIVE"),
    ("mean HBM read latency, cycles (outstanding reads per read request)",
     "TCC_EA0_RDREQ_LEVEL_sum", "TCC_EA0_RDREQ_sum"),
    ("mean HBM write latency, cycles", "TCC_EA0_WRREQ_LEVEL_sum", "TCC_EA0_WRREQ_sum"),
    ("waves waiting on any instruction per wave cycle", "SQ_WAIT_INST_ANY", "SQ_WAVE_CYCLES"),
    ("L2 hit rate", "TCC_HIT_sum", "TCC_REQ_sum"),
]


def counter_summary(op_log, dirs):
    """Markdown counter summary of a --kernel-op run: per counter, the median
    over the kernel's dispatches, the value per unit of work (wave instructions
    x 64 per element for SQ_INSTS_*), and the means over the fastest and the
    slowest third of the dispatches (durations from the counter runs' own
    timestamps), to show what separates slow launches from fast ones."""
    import csv
    import glob
    line = None
    with open(op_log) as fh:
        for ln in fh:
            if ln.startswith("{") and '"kernel_op"' in ln:
                line = json.loads(ln)
    if line is None:
        raise SystemExit(f"no --kernel-op line in {op_log}")
    pat, units, unit = line["kernel"], line["units_per_launch"], line["unit"]
    per, dur, passes, name = {}, {}, [], None
    for d in dirs:
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise SystemExit(f"no counter_collection.csv under {d}")
        ctrs = set()
        for f in files:
            for row in csv.DictReader(open(f)):
                if pat not in row["Kernel_Name"]:
                    continue
                name = name or row["Kernel_Name"]
                key = (d, row["Dispatch_Id"])
                c = row["Counter_Name"]
                ctrs.add(c)
                per.setdefault(key, {})
                per[key][c] = per[key].get(c, 0.0) + float(row["Counter_Value"])
                t = (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) / 1e3
                if t > 0:
                    dur[key] = t
        passes.append(sorted(ctrs))
    if not per:
        raise SystemExit(f"no dispatch of {pat!r} in the counter output")
    med = lambda v: sorted(v)[len(v) // 2]
    mean = lambda v: sum(v) / len(v) if v else float("nan")
    counters = sorted({c for v in per.values() for c in v})
    short = (name or pat).replace("(anonymous namespace)::", "").replace("void ", "").split("(")[0]
    out = [f"# Counters of `{short}`", "",
           f"Workload: {line['what']}; {units:,} {unit}s per launch; {line['ms_per_launch'] * 1e3:.2f} us "
           f"per launch by HIP events over the profiled run's timed launches ({line['steps']} after "
           f"{line['warmup']} warm-up; counter collection serialises launches, so this is not "
           f"the kernel's time). Durations below are the dispatches' own timestamps.", "",
           "| counter | dispatches | median per launch | per " + unit + " | mean, fastest third | "
           "mean, slowest third |", "|---|---|---|---|---|---|"]
    ratio_rows = []
    for c in counters:
        keys = [k for k, v in per.items() if c in v]
        vals = [per[k][c] for k in keys]
        timed_keys = sorted((k for k in keys if k in dur), key=lambda k: dur[k])
        third = max(1, len(timed_keys) // 3)
        fast = [per[k][c] for k in timed_keys[:third]]
        slow = [per[k][c] for k in timed_keys[-third:]]
        pu = med(vals) * (64 if c.startswith("SQ_INSTS_") else 1) / units
        out.append(f"| `{c}` | {len(vals)} | {med(vals):.6g} | {pu:.4g} | {mean(fast):.6g} | "
                   f"{mean(slow):.6g} |")
    out.append("")
    dur_rows = []
    for ps in passes:
        keys = sorted((k for k in dur if all(c in per[k] for c in ps)), key=lambda k: dur[k])
        if keys:
            third = max(1, len(keys) // 3)
            dur_rows.append((", ".join(f"`{c}`" for c in ps), len(keys), med([dur[k] for k in keys]),
                             mean([dur[k] for k in keys[:third]]),
                             mean([dur[k] for k in keys[-third:]])))
    out += ["Launch durations under each counter pass (us):", "",
            "| pass | dispatches | median | mean, fastest third | mean, slowest third |",
            "|---|---|---|---|---|"]
    out += [f"| {p} | {n} | {m:.2f} | {f:.2f} | {s_:.2f} |" for p, n, m, f, s_ in dur_rows]
    out.append("")
    for c in ("GRBM_COUNT", "GRBM_GUI_ACTIVE"):
        # counted cycles per us of launch: a falling rate in longer launches
        # means the clock, not the work, changed between them
        keys = sorted((k for k, v in per.items() if c in v and k in dur), key=lambda k: dur[k])
        if len(keys) < 3:
            continue
        third = len(keys) // 3
        rate = [per[k][c] / dur[k] for k in keys]
        ds = [dur[k] for k in keys]
        ratio_rows.append(f"| `{c}` per us of launch (rate of the counted clock; Pearson r "
                          f"with duration {_pearson(ds, rate):+.2f}, of the count itself "
                          f"{_pearson(ds, [per[k][c] for k in keys]):+.2f}) | `{c}` / duration | "
                          f"{med(rate):.5g} | {mean(rate[:third]):.5g} | {mean(rate[-third:]):.5g} |")
    if "SQ_VALU_MFMA_BUSY_CYCLES" in counters:
        # busy cycles are counted per SIMD: 1024 SIMDs, clocked at 2.4 GHz
        keys = sorted((k for k, v in per.items() if "SQ_VALU_MFMA_BUSY_CYCLES" in v and k in dur),
                      key=lambda k: dur[k])
        if keys:
            third = max(1, len(keys) // 3)
            fr = [per[k]["SQ_VALU_MFMA_BUSY_CYCLES"] / (1024 * dur[k] * 2400.0) for k in keys]
            ratio_rows.append(f"| MFMA busy per SIMD cycle (1024 SIMDs at 2.4 GHz over the "
                              f"launch) | `SQ_VALU_MFMA_BUSY_CYCLES` / (1024 x 2400 x us) | "
                              f"{med(fr):.4g} | {mean(fr[:third]):.4g} | {mean(fr[-third:]):.4g} |")
    if "SQ_VALU_MFMA_BUSY_CYCLES" in counters and "GRBM_COUNT" in counters:
        # against the counted clock instead (GRBM_COUNT sums the eight XCDs'
        # cycles); the two counters come from different passes, so only the
        # ratio of their medians is given
        busy = med([v["SQ_VALU_MFMA_BUSY_CYCLES"] for v in per.values()
                    if "SQ_VALU_MFMA_BUSY_CYCLES" in v])
        clk = med([v["GRBM_COUNT"] for v in per.values() if "GRBM_COUNT" in v])
        ratio_rows.append(f"| MFMA busy per SIMD cycle of the counted clock (medians) | "
                          f"(`SQ_VALU_MFMA_BUSY_CYCLES` / 1024) / (`GRBM_COUNT` / 8) | "
                          f"{busy / 1024 / (clk / 8):.4g} | - | - |")
    for label, a, b in COUNTER_RATIOS:
        keys = [k for k, v in per.items() if a in v and b in v and v[b] > 0]
        if not keys:
            continue
        r = [per[k][a] / per[k][b] for k in keys]
        tk = sorted((k for k in keys if k in dur), key=lambda k: dur[k])
        third = max(1, len(tk) // 3)
        ratio_rows.append(f"| {label} | `{a}` / `{b}` | {med(r):.4g} | "
                          f"{mean([per[k][a] / per[k][b] for k in tk[:third]]):.4g} | "
                          f"{mean([per[k][a] / per[k][b] for k in tk[-third:]]):.4g} |")
    if ratio_rows:
        out += ["| ratio | counters | median | mean, fastest third | mean, slowest third |",
                "|---|---|---|---|---|"] + ratio_rows + [""]
    op = line["kernel_op"]
    out += ["Commands (from the repository root, TMPDIR=/tmp; one rocprofv3 run per counter "
            "pass):", "", "```"]
    for i, ps in enumerate(passes):
        out.append(f"rocprofv3 --pmc {' '.join(ps)} --kernel-trace -d <dir{i + 1}> -o run "
                   f"--output-format csv -- python3 bench.py --kernel-op {op} --steps "
                   f"{line['steps']} --warmup {line['warmup']} > <op_log{i + 1}>")
    out += [f"python3 bench.py --counter-summary <op_log1> "
            + " ".join(f"<dir{i + 1}>" for i in range(len(passes))), "```"]
    print("\n".join(out))


def _pmc_rows(d, counter, per_us=False):
    """{kernel name: [per-dispatch counter value]} from a rocprofv3 --pmc CSV
    directory; with per_us, each value divided by its dispatch's duration (us)."""
    import csv
    import glob
    out = {}
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        per, dur = {}, {}
        with open(f) as fh:
            for row in csv.DictReader(fh):
                if row["Counter_Name"] != counter:
                    continue
                key = (row["Kernel_Name"], row["Dispatch_Id"])
                per[key] = per.get(key, 0.0) + float(row["Counter_Value"])
                dur[key] = (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) / 1e3
        for key, v in per.items():
            if per_us:
                if dur[key] <= 0:
                    continue
                v /= dur[key]
            out.setdefault(key[0], []).append(v)
    return out


def pmc_summary(dirs):
    """Markdown traffic summary for profiles/ from FETCH_SIZE / WRITE_SIZE runs."""
    def pick(rows, sub):
        ks = [k for k in rows if sub in k]
        if not ks:
            raise SystemExit(f"no kernel matching {sub!r} in the counter output")
        vals = [v for k in ks for v in rows[k]]
        return ks[0], vals

    fetch = _pmc_rows(dirs[0], "FETCH_SIZE")
    write = _pmc_rows(dirs[1], "WRITE_SIZE")
    copy_k, f_copy = pick(fetch, "copy")
    _, w_copy = pick(write, "copy")
    rot_k, f_rot = pick(fetch, ROT_INSTANCE)
    _, w_rot = pick(write, ROT_INSTANCE)
    med = lambda v: sorted(v)[len(v) // 2]
    f_fac = COPY_BYTES / (med(f_copy) * 1024)
    w_fac = COPY_BYTES / (med(w_copy) * 1024)
    rd = med(f_rot) * 1024 * f_fac
    wr = med(w_rot) * 1024 * w_fac
    rows, cols = 16384, 8192
    alg = rows * cols * B_MX
    lines = [
        "# HBM traffic of the fused permutation + Hadamard + MXFP4 kernel (16384x8192)",
        "",
        "Counters: rocprofv3 `FETCH_SIZE` and `WRITE_SIZE` (KiB per dispatch), one pass each,",
        "median over the dispatches of one run. Each is scaled by the same counter's reading",
        "for torch's 1 GiB device-to-device copy in the same run (1 GiB read, 1 GiB written).",
        "",
        "| | FETCH_SIZE KiB | WRITE_SIZE KiB |",
        "|---|---|---|",
        f"| copy 1 GiB (`{copy_k[:60]}`) | {med(f_copy):.0f} | {med(w_copy):.0f} |",
        f"| `{rot_k[:60]}` | {med(f_rot):.0f} | {med(w_rot):.0f} |",
        "",
        f"Scale factors: fetch {f_fac:.4f}, write {w_fac:.4f}.",
        "",
        f"Per launch: read {rd / 1e6:.1f} MB, written {wr / 1e6:.1f} MB, total "
        f"{(rd + wr) / 1e6:.1f} MB against {alg / 1e6:.1f} MB algorithmic "
        f"({(rd + wr) / alg:.3f}x).",
        "",
    ]
    if len(dirs) > 2:
        # busy cycles are counted per SIMD: 1024 SIMDs at 2.4 GHz over the launch
        _, b = pick(_pmc_rows(dirs[2], "SQ_VALU_MFMA_BUSY_CYCLES", per_us=True), ROT_INSTANCE)
        lines += [f"MFMA busy per SIMD cycle: SQ_VALU_MFMA_BUSY_CYCLES / (1024 x 2400 x launch "
                  f"us) = {med(b) / (1024 * 2400.0):.4f} (median dispatch).", ""]
        # instruction mix: wave instructions per 64 elements (one per lane
        # and element for a VALU op that every lane issues once per element)
        mix = []
        for ctr in ("SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_INSTS_SALU"):
            got = _pmc_rows(dirs[2], ctr)
            if any(ROT_INSTANCE in k for k in got):
                _, v = pick(got, ROT_INSTANCE)
                mix.append(f"{ctr} {med(v) / (rows * cols / 64):.3f}")
        if mix:
            lines += ["Instructions per element (wave instructions x 64 / elements, median "
                      "dispatch): " + ", ".join(mix) + ".", ""]
    lines += [
        "Commands (from the repository root, TMPDIR=/tmp):",
        "",
        "```",
        "rocprofv3 --pmc FETCH_SIZE --kernel-trace -d <fetch_dir> -o run --output-format csv "
        "-- python3 bench.py --steps 3 --warmup 1 --no-extras --no-cpu",
        "rocprofv3 --pmc WRITE_SIZE --kernel-trace -d <write_dir> -o run --output-format csv "
        "-- python3 bench.py --steps 3 --warmup 1 --no-extras --no-cpu",
        "rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU SQ_INSTS_MFMA "
        "SQ_INSTS_LDS SQ_INSTS_SALU --kernel-trace -d <mfma_dir> -o run --output-format csv "
        "-- python3 bench.py --steps 3 --warmup 1 --no-extras --no-cpu",
        "python3 bench.py --pmc-summary <fetch_dir> <write_dir> <mfma_dir>",
        "```",
        "",
        "Values read by bench.py (source_hash: sha256 of the kernel sources without comments, "
        "first 16 hex):",
        "",
        f"- source_hash: `{rot_source_hash()}`",
        f"- traffic_bytes_per_launch: {int(round(rd + wr))}",
        f"- read_bytes_per_launch: {int(round(rd))}",
        f"- write_bytes_per_launch: {int(round(wr))}",
        f"- algorithmic_bytes_per_launch: {int(alg)}",
    ]
    print("\n".join(lines))


def trace_summary(trace_dir, bench_log):
    """Markdown per-kernel time summary of a profiled bench.py run."""
    import csv
    import glob
    f = glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True)
    if not f:
        raise SystemExit(f"no kernel_stats.csv under {trace_dir}")
    rows = list(csv.DictReader(open(f[0])))
    line = None
    with open(bench_log) as fh:
        for ln in fh:
            if ln.startswith("{") and '"metric"' in ln:
                line = json.loads(ln)
    wl = line["config"]["workload"].split(":")[0] if line else "?"
    args = f"--workload {wl}" if wl != "c4" else ""
    out = [f"# Kernel times of one profiled bench.py run ({line['config']['workload'] if line else wl})",
           "", "| kernel | calls | avg us | min us | max us |", "|---|---|---|---|---|"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        name = r["Name"].replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "")
        if not name.startswith("fp4::") and "copyBuffer" not in name:
            continue
        out.append(f"| `{name[:80]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                   f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} |")
    out.append("")
    rot = [r for r in rows if ROT_INSTANCE in r["Name"]]
    if line and wl == "c4" and rot:
        avg = float(rot[0]["AverageNs"]) / 1e3
        ev = line["ms_per_step"] * 1e3
        out += [f"The fused kernel `{ROT_INSTANCE}` averages {avg:.2f} us per launch here (warm-up "
                f"launches included); the same run's HIP-event time per step is {ev:.2f} us "
                f"({ev / avg:.3f}x), one launch per step.", ""]
    elif line and line.get("extras", {}).get("step_kernel_calls"):
        calls = line["extras"]["step_kernel_calls"]
        ev = line["ms_per_step"] * 1e3
        per_step, parts = 0.0, []
        for pat, k in calls.items():
            hit = [r for r in rows if pat in r["Name"]]
            if not hit:
                continue
            avg = sum(float(r["TotalDurationNs"]) for r in hit) / sum(int(r["Calls"]) for r in hit)
            per_step += k * avg / 1e3
            parts.append(f"{k} x `{pat.rstrip('<')}` {avg / 1e3:.2f} us")
        out += [f"One timed step launches " + ", ".join(parts) + f": {per_step:.1f} us of kernel "
                f"time per step (average durations over every launch in the trace); the same "
                f"run's HIP-event time per step is {ev:.1f} us.", ""]
    out += ["Command (from the repository root, TMPDIR=/tmp):", "", "```",
            "rocprofv3 --kernel-trace --stats -d <trace_dir> -o run --output-format csv "
            f"-- python3 bench.py {args + ' ' if args else ''}"
            f"--steps {line['steps'] if line else 'K'} --warmup {line['warmup'] if line else 'W'} "
            "--no-cpu > <bench_log>",
            "python3 bench.py --trace-summary <trace_dir> <bench_log>", "```"]
    print("\n".join(out))


def main():
    args = parse()
    if args.trace_summary:
        trace_summary(*args.trace_summary)
        return
    if args.pmc_summary:
        pmc_summary(args.pmc_summary)
        return
    if args.counter_summary:
        counter_summary(args.counter_summary[0], args.counter_summary[1:])
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this path runs on one MI355X and has no "
              "multi-GPU mode (rows shard with no communication); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import block_scaled_fp4_absmax_amd as fp4
    from block_scaled_fp4_absmax_amd import inputs

    fp4.lib()  # fails loudly if the HIP library is not built
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.kernel_op:
        kernel_op(torch, fp4, inputs, args)
        return
    fn = {"c4": bench_c4, "c1": bench_c1, "c2": bench_c2, "c3": bench_c3,
          "c5": bench_c5}[args.workload]
    res, x_host, perm = fn(torch, fp4, inputs, args)

    cpu = None
    if not args.no_cpu and x_host is not None:
        log("[bench] timing the CPU oracle on a bounded sample")
        cpu = cpu_baseline(args.workload, x_host, perm, args.cpu_seconds)

    line = {
        "metric": METRIC,
        "value": round(res["value"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": res["config"],
        "hbm_frac_input": round(res["value"] / HBM_PEAK_GBS, 4),
        "sqnr_db": round(res["sqnr"], 3),
        "roofline": res["roofline"],
        "cpu_baseline": cpu,
        "extras": res["extras"],
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
