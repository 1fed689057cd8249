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
ROT_INSTANCE = ROT_KERNEL + "<2, 0, true, false, false>"  # the MXFP4 instance timed at 16384x8192
ROT_SOURCES = ["block_scaled_fp4_absmax_amd/csrc/rotate_kernels.hpp",
               "block_scaled_fp4_absmax_amd/csrc/rotate_mx.hip",
               "block_scaled_fp4_absmax_amd/csrc/rotation.hpp",
               "block_scaled_fp4_absmax_amd/csrc/fp4_device.hpp",
               "block_scaled_fp4_absmax_amd/csrc/launch.hpp"]
TRAFFIC_FILE = "profiles/traffic_perm_rotate_quantize_c4.md"
COPY_BYTES = 1 << 30  # torch device copy in device_copy(): 1 GiB read, 1 GiB written


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def rot_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in ROT_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
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
    p.add_argument("--workload", default="c4", choices=["c4", "c2", "c5"])
    p.add_argument("--no-extras", action="store_true")
    p.add_argument("--no-cpu", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--trace-summary", nargs=2, metavar=("TRACE_DIR", "BENCH_LOG"),
                   help="write the kernel-time summary from a rocprofv3 --kernel-trace --stats "
                        "directory and the JSON line that the profiled run printed, and exit")
    p.add_argument("--pmc-summary", nargs="+", metavar="DIR",
                   help="write the traffic summary from rocprofv3 --pmc output directories "
                        "(FETCH_SIZE run, WRITE_SIZE run[, MFMA busy run]) and exit")
    return p.parse_args()


def timed(torch, fn, steps, warmup):
    """ms per call of fn(i), measured with events on the current stream."""
    for i in range(warmup):
        fn(i)
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
    ms = timed(torch, lambda i: dst.copy_(src), 10, 2)
    return {"bytes_moved": 2 << 30, "ms": round(ms, 4), "GBps": round(2 * (1 << 30) / ms / 1e6, 1)}


def sqnr_db(torch, x, xh):
    x = x.double()
    d = x - xh.double()
    return float(10 * torch.log10((x * x).sum() / (d * d).sum()))


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
    n = len(xs)
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

    def step(i):
        k = i % n
        fp4.rotate_quantize(xs[k], perm, 32, codes=codes[k], scales=scales[k])

    log(f"[bench] timing {args.steps} steps after {args.warmup} warmup")
    ms = timed(torch, step, args.steps, args.warmup)
    dist = step_distribution(torch, step, 200)
    elems = rows * cols
    value = elems * 2 / (ms * 1e-3) / 1e9
    achieved = elems * B_MX / (ms * 1e-3) / 1e9

    xh = fp4.dequantize(codes[0], scales[0], fp4.MXFP4, perm=perm, hadamard=32)
    q = sqnr_db(torch, xs[0].float(), xh.float())
    c_pl, s_pl, _ = fp4.quantize(xs[0], fp4.MXFP4)
    q_plain = sqnr_db(torch, xs[0].float(), fp4.dequantize(c_pl, s_pl, fp4.MXFP4).float())

    extras = {"step_us_p10_p50_p90": dist,
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
                   "rotation": "perm+hadamard32", "input_copies": n},
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
         "kernel": ROT_KERNEL + "<2,0,true,false,false> (MXFP4; 2 MFMA tiles per wave per row)",
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

    ms = timed(torch, lambda i: fp4.quantize(xs[i % n], fp4.MXFP4, codes=codes[i % n],
                                             scales=scales[i % n]), 20, 3)
    out["c4_mxfp4_plain_quantize"] = gbs(ms, el, B_MX)
    ms = timed(torch, lambda i: fp4.rotate_quantize(xs[i % n], None, 32, codes=codes[i % n],
                                                    scales=scales[i % n]), 20, 3)
    out["c4_mxfp4_hadamard_only"] = gbs(ms, el, B_MX)
    outb = torch.empty_like(xs[0])
    ms = timed(torch, lambda i: fp4.dequantize(codes[i % n], scales[i % n], fp4.MXFP4, out=outb),
               20, 3)
    out["c4_mxfp4_dequantize"] = gbs(ms, el, B_MX)
    ms = timed(torch, lambda i: fp4.dequantize(codes[i % n], scales[i % n], fp4.MXFP4, perm=perm,
                                               hadamard=32, out=outb), 20, 3)
    out["c4_mxfp4_dequantize_unrotate"] = gbs(ms, el, B_MX)

    # NVFP4 + RaZeR after the two-level rotation on the same tensor (permutation
    # balanced over 16-channel blocks, 16-point Hadamard)
    perm16 = fp4.build_permutation(fp4.channel_energy(xs[0]), 16).cuda()
    s16 = [torch.empty((rows, cols // 16), dtype=torch.uint8, device="cuda") for _ in range(n)]
    t16 = [torch.empty(1, dtype=torch.float32, device="cuda") for _ in range(n)]

    def nv_rot(i, given):
        k = i % n
        fp4.rotate_quantize(xs[k], perm16, 16, codes=codes[k], scales=s16[k], fmt=fp4.NVFP4,
                            mode=fp4.RAZER, tensor_scale=t16[k], scale_given=given)

    ms = timed(torch, lambda i: nv_rot(i, False), 20, 3)
    out["c4_nvfp4_razer_perm_h16_with_amax"] = gbs(ms, el, B_NV + 2)
    ms = timed(torch, lambda i: nv_rot(i, True), 20, 3)
    out["c4_nvfp4_razer_perm_h16_scale_given"] = gbs(ms, el, B_NV)
    ms = timed(torch, lambda i: fp4.dequantize(codes[i % n], s16[i % n], fp4.NVFP4, fp4.RAZER,
                                               t16[i % n], perm=perm16, hadamard=16, out=outb),
               20, 3)
    out["c4_nvfp4_razer_dequantize_unrotate"] = gbs(ms, el, B_NV)
    xf = xs[0].float()
    for name, (pm, had) in {"perm_h16": (perm16, 16), "h16": (None, 16),
                            "plain": (None, 0)}.items():
        c, sc, _, ts = fp4.rotate_quantize(xs[0], pm, had, fmt=fp4.NVFP4, mode=fp4.RAZER)
        xh = fp4.dequantize(c, sc, fp4.NVFP4, fp4.RAZER, ts, perm=pm, hadamard=had)
        out[f"c4_sqnr_db_nvfp4_razer_{name}"] = round(sqnr_db(torch, xf, xh.float()), 3)
    del s16

    # MXINT4 (two's complement k/4 elements, E8M0 scale) on the same tensor
    ms = timed(torch, lambda i: fp4.quantize(xs[i % n], fp4.MXINT4, codes=codes[i % n],
                                             scales=scales[i % n]), 20, 3)
    out["c4_mxint4_plain_quantize"] = gbs(ms, el, B_MX)
    ms = timed(torch, lambda i: fp4.rotate_quantize(xs[i % n], perm, 32, codes=codes[i % n],
                                                    scales=scales[i % n], fmt=fp4.MXINT4), 20, 3)
    out["c4_mxint4_perm_h32_quantize"] = gbs(ms, el, B_MX)
    ms = timed(torch, lambda i: fp4.dequantize(codes[i % n], scales[i % n], fp4.MXINT4, perm=perm,
                                               hadamard=32, out=outb), 20, 3)
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
    ms = timed(torch, lambda i: fp4.apply_channel_rotation(xs[i % n], md, perm, out=zs[i % n]),
               20, 3)
    out["c4_givens_layers_apply"] = gbs(ms, el, 4)
    ms = timed(torch, lambda i: fp4.apply_channel_rotation(xs[i % n], md, None, out=zs[i % n]),
               20, 3)
    out["c4_givens_layers_apply_no_perm"] = gbs(ms, el, 4)
    t0 = time.perf_counter()
    R, rloss = fp4.calibrate_block_rotation(zs[0][:256], None, iters=30, angles=32)
    block_ms = (time.perf_counter() - t0) * 1e3
    rt = R.cuda()
    ident = torch.arange(cols, dtype=torch.int32, device="cuda")
    ms = timed(torch, lambda i: fp4.rotate_quantize_r(zs[i % n], ident, rt, codes=codes[i % n],
                                                      scales=scales[i % n]), 20, 3)
    out["c4_mxfp4_learned_r_quantize"] = gbs(ms, el, B_MX)
    ms = timed(torch, lambda i: fp4.dequantize_r(codes[i % n], scales[i % n], ident, rt,
                                                 out=outb), 20, 3)
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
    x3 = dev_copies(torch, inputs.gen_c3(), 1)[0]
    r3, k3 = x3.shape
    ms = timed(torch, lambda i: fp4.rotate_quantize(x3, None, 32), 20, 3)
    out["c3_mxfp4_h32_quantize"] = gbs(ms, r3 * k3, B_MX)
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
    ms = timed(torch, lambda i: fp4.quantize(ys[i % m], fp4.NVFP4, fp4.RAZER, tensor_scale=tss[i % m],
                                             scale_given=False, codes=cs[i % m],
                                             scales=ss[i % m]), 40, 5)
    out["c2_nvfp4_razer_quantize_with_amax"] = gbs(ms, el2, B_NV + 2)
    xh = fp4.dequantize(cs[0], ss[0], fp4.NVFP4, fp4.RAZER, tss[0])
    out["c2_sqnr_db_razer"] = round(sqnr_db(torch, ys[0].float(), xh.float()), 3)
    ms = timed(torch, lambda i: fp4.quantize(ys[i % m], fp4.NVFP4, fp4.RAZER, tensor_scale=tss[i % m],
                                             codes=cs[i % m], scales=ss[i % m]), 40, 5)
    out["c2_nvfp4_razer_quantize_scale_given"] = gbs(ms, el2, B_NV)
    graph_row("c2_nvfp4_razer_quantize_scale_given", lambda i: fp4.quantize(
        ys[i % m], fp4.NVFP4, fp4.RAZER, tensor_scale=tss[i % m], codes=cs[i % m],
        scales=ss[i % m]), B_NV)
    ms = timed(torch, lambda i: fp4.quantize(ys[i % m], fp4.NVFP4, fp4.PLAIN, tensor_scale=tss[i % m],
                                             codes=cs[i % m], scales=ss[i % m]), 40, 5)
    out["c2_nvfp4_plain_quantize_scale_given"] = gbs(ms, el2, B_NV)
    graph_row("c2_nvfp4_plain_quantize_scale_given", lambda i: fp4.quantize(
        ys[i % m], fp4.NVFP4, fp4.PLAIN, tensor_scale=tss[i % m], codes=cs[i % m],
        scales=ss[i % m]), B_NV)
    for k in range(m):
        fp4.quantize(ys[k], fp4.NVFP4, fp4.RAZER, tensor_scale=tss[k], codes=cs[k], scales=ss[k])
    ob = torch.empty_like(ys[0])
    ms = timed(torch, lambda i: fp4.dequantize(cs[i % m], ss[i % m], fp4.NVFP4, fp4.RAZER,
                                               tss[i % m], out=ob), 40, 5)
    out["c2_nvfp4_razer_dequantize"] = gbs(ms, el2, B_NV)
    graph_row("c2_nvfp4_razer_dequantize", lambda i: fp4.dequantize(
        cs[i % m], ss[i % m], fp4.NVFP4, fp4.RAZER, tss[i % m], out=ob), B_NV)
    ms = timed(torch, lambda i: fp4.quantize(ys[i % m], fp4.NVFP4, fp4.RAZER_W,
                                             tensor_scale=tss[i % m], codes=cs[i % m],
                                             scales=ss[i % m]), 40, 5)
    out["c2_nvfp4_razer_w_quantize_scale_given"] = gbs(ms, el2, B_NV)
    cw, sw, tw = fp4.quantize(ys[0], fp4.NVFP4, fp4.RAZER_W)
    xw = fp4.dequantize(cw, sw, fp4.NVFP4, fp4.RAZER_W, tw)
    out["c2_sqnr_db_razer_w"] = round(sqnr_db(torch, ys[0].float(), xw.float()), 3)
    cp, sp, tp = fp4.quantize(ys[0], fp4.NVFP4, fp4.PLAIN)
    xp = fp4.dequantize(cp, sp, fp4.NVFP4, fp4.PLAIN, tp)
    out["c2_sqnr_db_plain_nvfp4"] = round(sqnr_db(torch, ys[0].float(), xp.float()), 3)
    del ys, cs, ss
    return out


MFMA_PEAK_FP4_TFLOPS = 10100.0


def gemm_rows(torch, fp4, fmt):
    """The consumer: C = A B^T on quantized operands (activations [m, k],
    weights [n, k] of the Llama-70B-shaped layer), bf16 out. MXFP4 runs on the
    scaled FP4 matrix cores (peak 10.1 PFLOP/s); NVFP4 + RaZeR on both sides is
    decoded exactly to bf16 and runs on the bf16 ones (peak 2.5 PFLOP/s).
    Random codes and finite scale bytes: the time does not depend on values."""
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
        a = torch.randint(0, 256, (m, k // 2), dtype=torch.uint8, device="cuda", generator=g)
        sa = torch.randint(lo, hi, (m, k // blk), dtype=torch.uint8, device="cuda", generator=g)
        b = torch.randint(0, 256, (n, k // 2), dtype=torch.uint8, device="cuda", generator=g)
        sb = torch.randint(lo, hi, (n, k // blk), dtype=torch.uint8, device="cuda", generator=g)
        c = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
        ms = timed(torch, lambda i: fp4.gemm(a, sa, b, sb, out=c, **kw), 10, 2)
        tf = 2.0 * m * n * k / (ms * 1e-3) / 1e12
        by = (m + n) * (k / 2 + k / blk) + 2 * m * n
        rows[f"{m}x{n}x{k}"] = {"ms": round(ms, 4), "TFLOPs": round(tf, 1),
                                "frac_mfma_peak": round(tf / peak, 4),
                                "GBps": round(by / ms / 1e6, 1)}
        if m <= 32:  # µs-scale launches: also their time replayed from a graph
            us = graph_us(torch, lambda i: fp4.gemm(a, sa, b, sb, out=c, **kw))
            rows[f"{m}x{n}x{k}"]["graph_us_per_call"] = round(us, 2)
            rows[f"{m}x{n}x{k}"]["graph_frac_mfma_peak"] = round(
                2.0 * m * n * k / (us * 1e-6) / 1e12 / peak, 4)
        del a, sa, b, sb, c
    return rows


def bench_c2(torch, fp4, inputs, args):
    r, c = inputs.FULL_SHAPES["c2"]
    x = inputs.gen_c2()
    ys = dev_copies(torch, x, copies_for(x.nbytes))
    m = len(ys)
    cs = [torch.empty((r, c // 2), dtype=torch.uint8, device="cuda") for _ in range(m)]
    ss = [torch.empty((r, c // 16), dtype=torch.uint8, device="cuda") for _ in range(m)]
    tss = [torch.empty(1, dtype=torch.float32, device="cuda") for _ in range(m)]

    def step(i):
        k = i % m
        fp4.quantize(ys[k], fp4.NVFP4, fp4.RAZER, tensor_scale=tss[k], scale_given=False,
                     codes=cs[k], scales=ss[k])

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

    def step(i):
        for k in range(len(xs)):
            fp4.quantize(xs[k], fp4.NVFP4, fp4.RAZER, tensor_scale=ts[k], scale_given=False,
                         codes=cs[k], scales=ss[k])
            fp4.dequantize(cs[k], ss[k], fp4.NVFP4, fp4.RAZER, ts[k], out=outs[k])

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


def _pmc_rows(d, counter):
    """{kernel name: [per-dispatch counter value]} from a rocprofv3 --pmc CSV directory."""
    import csv
    import glob
    out = {}
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        per = {}
        with open(f) as fh:
            for row in csv.DictReader(fh):
                if row["Counter_Name"] != counter:
                    continue
                key = (row["Kernel_Name"], row["Dispatch_Id"])
                per[key] = per.get(key, 0.0) + float(row["Counter_Value"])
        for (k, _), v in per.items():
            out.setdefault(k, []).append(v)
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
        busy = _pmc_rows(dirs[2], "SQ_VALU_MFMA_BUSY_CYCLES")
        cu = _pmc_rows(dirs[2], "SQ_BUSY_CU_CYCLES")
        _, b = pick(busy, ROT_INSTANCE)
        _, c = pick(cu, ROT_INSTANCE)
        lines += [f"MFMA busy: SQ_VALU_MFMA_BUSY_CYCLES / SQ_BUSY_CU_CYCLES = "
                  f"{med(b) / max(med(c), 1):.4f} (median dispatch).", ""]
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
        "rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CU_CYCLES SQ_INSTS_VALU SQ_INSTS_MFMA "
        "SQ_INSTS_LDS SQ_INSTS_SALU --kernel-trace -d <mfma_dir> -o run --output-format csv "
        "-- python3 bench.py --steps 3 --warmup 1 --no-extras --no-cpu",
        "python3 bench.py --pmc-summary <fetch_dir> <write_dir> <mfma_dir>",
        "```",
        "",
        "Values read by bench.py (source_hash: sha256 of the kernel sources, first 16 hex):",
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
    fp4_total = 0.0
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        name = r["Name"].replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "")
        if not name.startswith("fp4::") and "copyBuffer" not in name:
            continue
        if name.startswith("fp4::"):
            fp4_total += float(r["TotalDurationNs"])
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
    elif line:
        n = line["steps"] + line["warmup"]
        ev = line["ms_per_step"] * 1e3
        out += [f"All fp4 kernels together take {fp4_total / 1e3 / n:.1f} us per step here "
                f"(total over the {n} warm-up and timed steps); the same run's HIP-event time per "
                f"step is {ev:.1f} us.", ""]
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
    fn = {"c4": bench_c4, "c2": bench_c2, "c5": bench_c5}[args.workload]
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
