#!/usr/bin/env python3
"""Benchmark of the fused dequant matrix products on one MI355X.

A step is one decode step of a Llama-3-8B-shaped Q4_K linear stack at batch 1:
32 layers x {q 4096x4096, k 1024x4096, v 1024x4096, o 4096x4096,
gate 14336x4096, up 14336x4096, down 4096x14336} = 224 fused-dequant
matrix-vector products (3,925,868,544 bytes of packed weights) computed by
one launch of the streaming multi-product kernel (gq_gemv_q4k_multi).  Every
matrix has its own weights (no reuse through the caches) and its own binary32
N(0,1) activation vector.  ``value`` is packed weight bytes per second over
the timed steps.  The same products as 224 separate launches replayed as one
HIP graph are reported beside it.

The same run also measures, outside the timed steps, the other forms of the
hot path (the stack at batch 4 and 16 in one launch each, single decode
matrices hot and rotated, the
prefill matrix products, the mixture-of-experts layer, the Q8_0 product) and
times the binary64 CPU oracle on a bounded sample of the stack.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Q4_K fused-dequant GEMV weight GB/s (decode); dequant-GEMM TFLOP/s (prefill)"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
FP16_PEAK_TFLOPS = 2500.0    # MI355X dense binary16 matrix cores
INT8_PEAK_TOPS = 5000.0      # MI355X dense int8 matrix cores
WARM_FLOOR_S = 0.5           # least sustained warm-up before the timed steps
LAYER = (("q", 4096, 4096), ("k", 1024, 4096), ("v", 1024, 4096), ("o", 4096, 4096),
         ("gate", 14336, 4096), ("up", 14336, 4096), ("down", 4096, 14336))
N_LAYERS = 32
STACK_WORKLOAD = 2           # generator stream ids shared with the parity tests
PREFILL_WORKLOAD = 3
MOE_WORKLOAD = 4


def q4k_bytes(M, K):
    return M * (K // 256) * 144


def gemv_bytes(M, K, B):
    """Algorithmic bytes of one matrix-vector product: packed weights, x, y."""
    return q4k_bytes(M, K) + 4 * B * K + 4 * B * M


class Stack:
    """The 224 weight matrices of the decode stack, resident in HBM."""

    def __init__(self, torch, synth):
        import hashlib
        self.mats = []
        h = hashlib.sha256()
        for layer in range(N_LAYERS):
            for i, (name, M, K) in enumerate(LAYER):
                t = layer * len(LAYER) + i
                wh = synth.q4k_blocks(STACK_WORKLOAD, t, M, K)
                h.update(wh.data)
                w = torch.from_numpy(wh).cuda()
                self.mats.append((name, M, K, t, w))
        self.sha256 = h.hexdigest()
        self.weight_bytes = sum(q4k_bytes(M, K) for _, M, K, _, _ in self.mats)


def stack_graph(torch, gq, synth, stack, B, stream):
    xs, ys = [], []
    for _, M, K, t, _ in stack.mats:
        xs.append(torch.from_numpy(synth.activations_f32(STACK_WORKLOAD, 100 * t + B, B, K)).cuda())
        ys.append(torch.empty((B, M), dtype=torch.float32, device="cuda"))

    def launch_all():
        for (_, M, K, _, w), x, y in zip(stack.mats, xs, ys):
            gq.gq_gemv_q4k(w, x, y, M, K, B, stream)

    with torch.cuda.stream(stream):
        launch_all()  # eager once: loads the library, checks every call
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        launch_all()
    torch.cuda.synchronize()
    return g, launch_all


def time_graph(torch, g, steps, warmup):
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        g.replay()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


def probe_ceilings(torch, stream, prefill, decode_gbs, stack_bytes):
    """Achievable ceilings from the measurement probes (libgq_probe.so, built
    beside libgq.so): a plain streaming read of the decode stack's byte count
    and a register-only binary16 matrix-instruction loop over every CU; and
    the decode and prefill results as fractions of them."""
    import ctypes
    from quantized_unpack_q4_amd import build as gqbuild
    if not os.path.exists(gqbuild.PROBE_LIB):
        return {"probes": "libgq_probe.so not built"}
    P = ctypes.CDLL(gqbuild.PROBE_LIB)
    vp = ctypes.c_void_p
    P.gqp_stream_read.argtypes = [vp, ctypes.c_longlong, vp, ctypes.c_int, ctypes.c_int, vp]
    P.gqp_mfma_f16.argtypes = [vp, ctypes.c_int, ctypes.c_int, vp]
    P.gqp_mfma_f16_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    P.gqp_mfma_f16_flops.restype = ctypes.c_longlong
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    out = {}
    nbytes = (stack_bytes + 15) // 16 * 16
    buf = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.empty(16 * cus * 4, dtype=torch.int32, device="cuda")
    sp = ctypes.c_void_p(stream.cuda_stream)
    # the best of four read forms (grid-stride; per-workgroup range with
    # cached or non-temporal loads, 256 or 512 threads) and several grids
    read_gbs, read_cfg = 0.0, None
    forms = ("grid-stride", "per-workgroup range", "per-workgroup range, non-temporal",
             "per-workgroup range, non-temporal, 512 threads")
    for kind in (0, 1, 2, 3):
        for mult in ((1, 2, 4) if kind == 3 else (2, 4, 8, 16)):
            grid = mult * cus

            def read():
                if P.gqp_stream_read(vp(buf.data_ptr()), nbytes, vp(sink.data_ptr()), grid,
                                     kind, sp) != 0:
                    raise RuntimeError("gqp_stream_read launch failed")
            s = event_time(torch, stream, read, reps=10, warm_s=0.02)
            if nbytes / s / 1e9 > read_gbs:
                read_gbs, read_cfg = nbytes / s / 1e9, "%s, %d workgroups" % (forms[kind], grid)
    out["stream_read_%dB_GB/s" % nbytes] = round(read_gbs, 1)
    out["stream_read_form"] = read_cfg
    out["decode_stack_frac_of_stream_read"] = round(decode_gbs / read_gbs, 4)
    del buf, sink
    iters = 4096
    msink = torch.empty(cus * 512, dtype=torch.float32, device="cuda")

    def mfma():
        if P.gqp_mfma_f16(vp(msink.data_ptr()), iters, cus, sp) != 0:
            raise RuntimeError("gqp_mfma_f16 launch failed")
    s = event_time(torch, stream, mfma, reps=10)
    mfma_tf = P.gqp_mfma_f16_flops(iters, cus) / s / 1e12
    out["mfma_f16_register_loop_TFLOP/s"] = round(mfma_tf, 1)
    for key, v in prefill.items():
        if "TFLOP/s" in v:
            out["prefill_%s_frac_of_mfma_loop" % key] = round(v["TFLOP/s"] / mfma_tf, 4)
    del msink
    return out


def event_time(torch, stream, fn, reps=20, warmup=3, warm_s=0.05):
    """Median per-call time (s) of fn() on `stream`, HIP events per rep, after
    at least `warmup` calls and `warm_s` seconds of untimed calls (steady clocks
    and caches for this workload)."""
    with torch.cuda.stream(stream):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < warm_s:
            for _ in range(8):
                fn()
            torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            b.synchronize()
            ts.append(a.elapsed_time(b) * 1e-3)
    ts.sort()
    return ts[len(ts) // 2]


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "gemv_q4k_stream_decode_stack.md")
TRAFFIC_SOURCES = ("quantized_unpack_q4_amd/csrc/gemv_stream.hip",
                   "quantized_unpack_q4_amd/csrc/gq_device.h",
                   "quantized_unpack_q4_amd/csrc/gq_internal.h")


def measured_traffic():
    """HBM bytes per launch of the streaming kernel on the decode stack, from the
    committed rocprofv3 FETCH_SIZE/WRITE_SIZE summary, or None when that
    summary is missing or was taken on other kernel sources."""
    import hashlib
    try:
        text = open(TRAFFIC_PROFILE).read()
        h = hashlib.sha256()
        for f in TRAFFIC_SOURCES:
            h.update(open(os.path.join(ROOT, f), "rb").read())
    except OSError:
        return None
    fields = dict(l.split(":", 1) for l in text.splitlines()
                  if l.startswith(("traffic_bytes_per_launch:", "source_sha256:")))
    if fields.get("source_sha256", "").strip() != h.hexdigest():
        return None
    return int(fields["traffic_bytes_per_launch"])


def cpu_threads():
    """Host threads for the all-cores oracle runs: the CPUs this process may
    use, at most 16 (one GPU's share of its host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _oracle_runs(fn, nrows, threads, reps=3):
    """Median, min and max seconds of fn(rows) over `reps` runs, the rows
    [0, nrows) cut into `threads` contiguous ranges, each range one call on
    its own host thread (the oracle's C code releases the interpreter lock);
    the oracle's arithmetic is unchanged."""
    import threading

    import numpy as np
    chunks = [c for c in np.array_split(np.arange(nrows), threads) if c.size]
    ts = []
    for _ in range(reps):
        ths = [threading.Thread(target=fn, args=(c,)) for c in chunks]
        a = time.perf_counter()
        for t in ths:
            t.start()
        for t in ths:
            t.join()
        ts.append(time.perf_counter() - a)
    ts.sort()
    return ts[len(ts) // 2], ts[0], ts[-1]


def cpu_baseline(synth):
    """The binary64 oracle, as it stands, on the host cores: every workload on
    one thread and on all cores (rows split over threads), median of 3 runs.
    Large workloads run a fixed sample and are extrapolated linearly (rows for
    products; tokens for the MoE layer; matrices for the decode stack), and
    say so.  Input generation is not timed."""
    import numpy as np

    import oracle
    oracle.lib()
    nthr = cpu_threads()
    out = {}

    def both(name, fn, nrows, scale, unit_work, unit, sample, extrapolated, nrows_all=None,
             scale_all=None):
        r1 = _oracle_runs(fn, nrows, 1)
        rn = _oracle_runs(fn, nrows_all or nrows, nthr)
        sa = scale_all or scale
        out[name] = {
            "sample": sample, "extrapolated": extrapolated,
            "single_thread_s": round(r1[0] * scale, 4),
            "single_thread_s_min_max": [round(r1[1] * scale, 4), round(r1[2] * scale, 4)],
            "all_cores_s": round(rn[0] * sa, 4),
            "all_cores_s_min_max": [round(rn[1] * sa, 4), round(rn[2] * sa, 4)],
            "unit": unit,
            "single_thread_rate": round(unit_work / (r1[0] * scale), 6),
            "all_cores_rate": round(unit_work / (rn[0] * sa), 6)}

    # C0: Q8_0 256 x 1024, batch 1, whole
    w = synth.q8_0_blocks(0, 0, 256, 1024)
    x = synth.activations_f32(0, 0, 1, 1024)
    both("q8_0_gemv_256x1024_b1", lambda r: oracle.gemv(oracle.Q8_0, w, x, 256, 1024, rows=r),
         256, 1.0, synth.q8_0_bytes(256, 1024) / 1e9, "GB/s of weights", "whole", False)
    # C1: Q4_K 4096 x 4096 (whole) and 14336 x 4096 (first quarter of the rows)
    for M, K, nr in ((4096, 4096, 4096), (14336, 4096, 3584)):
        w = synth.q4k_blocks(1, M, M, K)
        x = synth.activations_f32(1, M, 1, K)
        both("q4k_gemv_%dx%d_b1" % (M, K),
             lambda r, w=w, x=x, M=M, K=K: oracle.gemv(oracle.Q4_K, w, x, M, K, rows=r),
             nr, M / nr, q4k_bytes(M, K) / 1e9, "GB/s of weights",
             "whole" if nr == M else "first %d of %d rows, times %d" % (nr, M, M // nr),
             nr != M)
    # C2: the decode stack, batch 1: the first eighth of the rows of layer 0's
    # seven products, scaled to all rows and 32 layers
    layer0 = []
    for t, (name, M, K) in enumerate(LAYER):
        layer0.append((synth.q4k_blocks(STACK_WORKLOAD, t, M, K),
                       synth.activations_f32(STACK_WORKLOAD, 100 * t + 1, 1, K), M, K))
    offs = np.cumsum([0] + [m[2] // 8 for m in layer0])

    def stack_rows(rows):
        for i, (w, x, M, K) in enumerate(layer0):
            sel = rows[(rows >= offs[i]) & (rows < offs[i + 1])] - offs[i]
            if sel.size:
                oracle.gemv(oracle.Q4_K, w, x, M, K, rows=sel)
    both("decode_stack_b1", stack_rows, int(offs[-1]), 8.0 * N_LAYERS,
         stack_bytes_total() / 1e9, "GB/s of weights",
         "first eighth of the rows of layer 0's q, k, v, o, gate, up, down, times 8 x 32", True)
    del layer0
    # C3: prefill 14336 x 4096 at 512 and 4096 tokens: a row sample over all
    # tokens, scaled to all rows
    M, K = 14336, 4096
    w = synth.q4k_blocks(PREFILL_WORKLOAD, M, M, K)
    for N, nr in ((512, 8), (4096, 2)):
        x16 = synth.activations_f16(PREFILL_WORKLOAD, N, N, K)
        both("prefill_%dx%dxN%d" % (M, K, N),
             lambda r, x16=x16: oracle.gemm(oracle.Q4_K, w, x16, M, K, rows=r),
             nr, M / nr, 2.0 * M * K * N / 1e9, "GFLOP/s",
             "first %d rows (one thread) / first %d rows (one per thread) over all %d "
             "tokens, scaled to %d rows" % (nr, nthr, N, M), True,
             nrows_all=nthr, scale_all=M / nthr)
    del w
    # C4: the MoE layer (64 experts, top-8, 2048 / 1024) at 256 tokens: one
    # token on one thread, one token per thread on all cores, scaled to 256
    H, I, E, k, T = 2048, 1024, 64, 8, 256
    wg = synth.q4k_blocks(MOE_WORKLOAD, 0, E * I, H)
    wu = synth.q4k_blocks(MOE_WORKLOAD, 1, E * I, H)
    wd = synth.q4k_blocks(MOE_WORKLOAD, 2, E * H, I)
    x16 = synth.activations_f16(MOE_WORKLOAD, 0, T, H)
    ids, wts = oracle.moe_route(synth.router_logits(MOE_WORKLOAD, 0, T, E), k)
    wts = wts.astype(np.float32)

    def moe_tokens(r):
        oracle.moe_ffn(wg, wu, wd, x16[r], ids[r], wts[r], H, I, E)
    both("moe_olmoe_T256", moe_tokens, 1, float(T), 2.0 * T * k * 3 * H * I / 1e9, "GFLOP/s",
         "token 0 (one thread) / tokens 0..%d (one per thread), times 256 / %d"
         % (nthr - 1, nthr), True, nrows_all=nthr, scale_all=T / nthr)
    head = out["decode_stack_b1"]
    return {"value": head["all_cores_rate"], "unit": "GB/s", "cores": nthr, "kind": "oracle",
            "sample": "decode stack at batch 1: the first eighth of the rows of layer 0's "
                      "seven products, extrapolated to all rows of 32 layers; median of 3 "
                      "runs, rows split over %d threads" % nthr,
            "single_thread_value": head["single_thread_rate"],
            "cpu_model": cpu_model(), "nproc": os.cpu_count(), "threads": nthr,
            "configs": out}


def make_receipt(torch, stack_sha256):
    """Where and from what this line was measured."""
    import hashlib

    from quantized_unpack_q4_amd import build as gqbuild
    info = {}
    try:
        info = json.load(open(gqbuild.BUILD_INFO))
    except (OSError, ValueError):
        pass
    lib_h = hashlib.sha256()
    with open(gqbuild.LIB, "rb") as fh:
        lib_h.update(fh.read())
    props = torch.cuda.get_device_properties(0)
    return {"git_rev": info.get("git_rev"), "git_dirty": info.get("git_dirty"),
            "hipcc": info.get("hipcc"), "source_sha256": info.get("source_sha256"),
            "libgq_sha256": lib_h.hexdigest(),
            "gpu": torch.cuda.get_device_name(0),
            "gpu_arch": getattr(props, "gcnArchName", None),
            "gpu_cus": props.multi_processor_count,
            "hip_runtime": torch.version.hip, "torch": torch.__version__,
            "cpu_model": cpu_model(), "nproc": os.cpu_count(),
            "decode_stack_weights_sha256": stack_sha256}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # the GPU needs ~0.1 s of sustained load to reach steady clocks: 200
    # untimed steps of the decode stack are about 0.16 s
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--no-extra", action="store_true",
                    help="time the step only (skip the secondary measurements)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="also run a plain device-to-device copy of MIB MiB five times (the "
                         "reference kernel for scaling hardware byte counters)")
    ap.add_argument("--stack-batch", type=int, default=1, metavar="B",
                    help="activation rows of the timed decode-stack step (1 by default; 2-16 "
                         "time the batched one-launch form, for profiling it)")
    args = ap.parse_args()
    if not 1 <= args.stack_batch <= 16:
        print("--stack-batch must be in 1..16", file=sys.stderr)
        sys.exit(2)
    if args.gpus != 1:
        print("bench.py measures one GPU: the library runs the hot path on a single MI355X "
              "and has no multi-GPU path (--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from quantized_unpack_q4_amd import gq, synth

    torch.cuda.set_device(0)
    gq.lib()
    log = lambda *a: print(*a, file=sys.stderr, flush=True)  # noqa: E731

    log("generating the decode stack ...")
    stack = Stack(torch, synth)
    stack_sha256 = stack.sha256
    stream = torch.cuda.Stream()

    # the step: all 224 batch-1 products of the stack in one launch
    SB = args.stack_batch
    items = []
    for _, M, K, t, w in stack.mats:
        x = torch.from_numpy(synth.activations_f32(STACK_WORKLOAD, 100 * t + SB, SB, K)).cuda()
        y = torch.empty((SB, M), dtype=torch.float32, device="cuda")
        items.append((w, x, y, M, K))
    table = gq.GemvTable(items, batch=SB) if SB > 1 else gq.GemvTable(items)
    alg_bytes = sum(gemv_bytes(M, K, SB) for _, M, K, _, _ in stack.mats)

    # W warm-up steps, continued until at least WARM_FLOOR_S of sustained
    # load: the clocks of an idle GPU take ~0.1 s to come up, and a few
    # steps (5 are ~4 ms) would time the ramp, not the kernel
    log("timing %d steps after %d warm-up steps (and >= %.1f s of warm-up)"
        % (args.steps, args.warmup, WARM_FLOOR_S))
    warm_steps, tw = 0, time.perf_counter()
    with torch.cuda.stream(stream):
        while warm_steps < args.warmup or time.perf_counter() - tw < WARM_FLOOR_S:
            table.run(stream)
            warm_steps += 1
            if warm_steps % 32 == 0:
                torch.cuda.synchronize()
    torch.cuda.synchronize()
    warm_s = time.perf_counter() - tw
    # one event pair around each launch, on the stream the kernel runs on: the
    # kernel's average duration without the gaps between launches
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        for a, b in evs:
            a.record(stream)
            table.run(stream)
            b.record(stream)
    torch.cuda.synchronize()
    sec = (time.perf_counter() - t0) / args.steps
    value = stack.weight_bytes / sec / 1e9
    # the step is one launch of the streaming kernel: its average duration
    durs = sorted(a.elapsed_time(b) * 1e-3 for a, b in evs)
    avg_dur = sum(durs) / args.steps
    achieved = alg_bytes / avg_dur / 1e9

    extra = {"stack_b%d_one_launch" % SB: {
        "ms_per_step": round(sec * 1e3, 4), "kernel_ms_events": round(avg_dur * 1e3, 4),
        "kernel_ms_median": round(durs[len(durs) // 2] * 1e3, 4),
        "kernel_ms_min": round(durs[0] * 1e3, 4), "kernel_ms_max": round(durs[-1] * 1e3, 4),
        "warmup_steps_run": warm_steps, "warmup_s": round(warm_s, 3)}}
    if args.copy_probe > 0:
        n = args.copy_probe << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        with torch.cuda.stream(stream):
            for _ in range(5):
                dst.copy_(src)
        torch.cuda.synchronize()
        extra["copy_probe_bytes"] = n
        del src, dst

    if not args.no_extra:
        # the same 224 products as 224 launches, replayed as one HIP graph
        g1, _ = stack_graph(torch, gq, synth, stack, 1, stream)
        s224 = time_graph(torch, g1, max(3, args.steps // 2), 2)
        extra["stack_b1_224_launch_graph"] = {
            "ms_per_step": round(s224 * 1e3, 4),
            "weight_GB/s": round(stack.weight_bytes / s224 / 1e9, 1)}
        del g1

        # one GPU's share of the stack under 8-way tensor parallelism: q, k, v,
        # gate, up split by output rows (the first M/8 rows), o and down by K
        # at super-block boundaries (the first K/8 of each row), all 224
        # shards in one launch
        itS, shard_bytes = [], 0
        for name, M, K, t, w in stack.mats:
            if name in ("o", "down"):
                ks = K // 8
                ws = w.view(M, K // 256, 144)[:, :ks // 256, :].contiguous().view(-1)
                Ms, Ks = M, ks
            else:
                Ms, Ks = M // 8, K
                ws = w[:q4k_bytes(Ms, K)]
            x = torch.from_numpy(synth.activations_f32(STACK_WORKLOAD, 100 * t + 1, 1, Ks)).cuda()
            itS.append((ws, x, torch.empty((1, Ms), dtype=torch.float32, device="cuda"), Ms, Ks))
            shard_bytes += q4k_bytes(Ms, Ks)
        tabS = gq.GemvTable(itS)
        s = event_time(torch, stream, lambda: tabS.run(stream), reps=max(10, args.steps))
        extra["stack_b1_tp8_shard_one_launch"] = {
            "us_per_step": round(s * 1e6, 1), "weight_bytes": shard_bytes,
            "weight_GB/s": round(shard_bytes / s / 1e9, 1)}
        del tabS, itS

        for B in (4, 16):
            # the whole stack at batch B in one launch (gq_gemv_q4k_multi_batched)
            log("stack batch", B)
            itB = []
            for _, M, K, t, w in stack.mats:
                x = torch.from_numpy(synth.activations_f32(STACK_WORKLOAD, 100 * t + B, B, K)).cuda()
                itB.append((w, x, torch.empty((B, M), dtype=torch.float32, device="cuda"), M, K))
            tabB = gq.GemvTable(itB, batch=B)
            s = event_time(torch, stream, lambda: tabB.run(stream), reps=max(5, args.steps // 2))
            flops = sum(2 * M * K * B for _, M, K, _, _ in stack.mats)
            extra["stack_b%d_one_launch" % B] = {
                "ms_per_step": round(s * 1e3, 4),
                "weight_GB/s": round(stack.weight_bytes / s / 1e9, 1),
                "TFLOP/s": round(flops / s / 1e12, 2)}
            # the same with the activations staged once per product into a
            # workspace (gq_gemv_q4k_multi_batched_ws: three launches)
            tabP = gq.GemvTable(itB, batch=B, prestaged=True)
            s = event_time(torch, stream, lambda: tabP.run(stream), reps=max(5, args.steps // 2))
            extra["stack_b%d_prestaged" % B] = {
                "ms_per_step": round(s * 1e3, 4),
                "weight_GB/s": round(stack.weight_bytes / s / 1e9, 1),
                "workspace_bytes": int(tabP.ws.numel())}
            del itB, tabB, tabP
        # single decode matrices: hot (one matrix again and again) and rotated
        for name, M, K in (("q", 4096, 4096), ("gate", 14336, 4096)):
            mats = [m[4] for m in stack.mats if m[0] == name or (name == "q" and m[0] == "o")]
            # at least 1 GiB of distinct weights, past the 256 MB memory-side
            # cache (the stack's 64 q/o matrices are 604 MB: add copies)
            extra_copies = []
            while (len(mats) + len(extra_copies)) * q4k_bytes(M, K) < (1 << 30):
                extra_copies.append(mats[len(extra_copies) % len(mats)].clone())
            mats = mats + extra_copies
            x = torch.from_numpy(synth.activations_f32(1, M, 1, K)).cuda()
            y = torch.empty((1, M), dtype=torch.float32, device="cuda")
            w0 = mats[0]
            hot = event_time(torch, stream, lambda: gq.gq_gemv_q4k(w0, x, y, M, K, 1, stream))
            it = {"i": 0}

            def rot():
                w = mats[it["i"] % len(mats)]
                it["i"] += 1
                gq.gq_gemv_q4k(w, x, y, M, K, 1, stream)
            rotated = event_time(torch, stream, rot, reps=len(mats), warmup=len(mats))
            extra["gemv_%dx%d_b1" % (M, K)] = {
                "hot_us": round(hot * 1e6, 2), "hot_GB/s": round(q4k_bytes(M, K) / hot / 1e9, 1),
                "rotated_us": round(rotated * 1e6, 2),
                "rotated_GB/s": round(q4k_bytes(M, K) / rotated / 1e9, 1),
                "rotated_over_MB": round(len(mats) * q4k_bytes(M, K) / 1e6, 1)}
            del mats, extra_copies
        # a layer's gate and up products with the SwiGLU epilogue in one launch
        # (gq_gemv_q4k_swiglu), rotated over the 32 layers' pairs, beside the
        # same two products as two launches
        M, K = 14336, 4096
        gates = [m[4] for m in stack.mats if m[0] == "gate"]
        ups = [m[4] for m in stack.mats if m[0] == "up"]
        x = torch.from_numpy(synth.activations_f32(1, 2 * M, 1, K)).cuda()
        hbuf = torch.empty((M,), dtype=torch.float32, device="cuda")
        ybuf = torch.empty((2, M), dtype=torch.float32, device="cuda")
        it = {"i": 0}

        def fused():
            i = it["i"] % len(gates)
            it["i"] += 1
            gq.gq_gemv_q4k_swiglu(gates[i], ups[i], x, hbuf, M, K, stream)

        def separate():
            i = it["i"] % len(gates)
            it["i"] += 1
            gq.gq_gemv_q4k(gates[i], x, ybuf[0], M, K, 1, stream)
            gq.gq_gemv_q4k(ups[i], x, ybuf[1], M, K, 1, stream)
        sf = event_time(torch, stream, fused, reps=len(gates), warmup=len(gates))
        ss = event_time(torch, stream, separate, reps=len(gates), warmup=len(gates))
        extra["gemv_swiglu_%dx%d_b1" % (M, K)] = {
            "fused_us": round(sf * 1e6, 2), "fused_GB/s": round(2 * q4k_bytes(M, K) / sf / 1e9, 1),
            "two_launches_us": round(ss * 1e6, 2)}
        # the same at batch 4 and 16 on the matrix cores (gq_gemv_q4k_swiglu_batched)
        for B in (4, 16):
            xb = torch.from_numpy(synth.activations_f32(1, 2 * M + B, B, K)).cuda()
            hb = torch.empty((B, M), dtype=torch.float32, device="cuda")
            yb = torch.empty((2, B, M), dtype=torch.float32, device="cuda")
            it["i"] = 0

            def fused_b():
                i = it["i"] % len(gates)
                it["i"] += 1
                gq.gq_gemv_q4k_swiglu_batched(gates[i], ups[i], xb, hb, M, K, B, stream)

            def separate_b():
                i = it["i"] % len(gates)
                it["i"] += 1
                gq.gq_gemv_q4k(gates[i], xb, yb[0], M, K, B, stream)
                gq.gq_gemv_q4k(ups[i], xb, yb[1], M, K, B, stream)
            sf = event_time(torch, stream, fused_b, reps=len(gates), warmup=len(gates))
            ss = event_time(torch, stream, separate_b, reps=len(gates), warmup=len(gates))
            extra["gemv_swiglu_%dx%d_b%d" % (M, K, B)] = {
                "fused_us": round(sf * 1e6, 2),
                "fused_GB/s": round(2 * q4k_bytes(M, K) / sf / 1e9, 1),
                "two_launches_us": round(ss * 1e6, 2)}
            del xb, hb, yb
        # the opt-in integer-dot path (8-bit activation codes) on the same
        # rotated gate matrices at batch 1 and 16, beside the binary32 path
        q8k = {}
        for B in (1, 16):
            xb = torch.from_numpy(synth.activations_f32(1, 3 * M + B, B, K)).cuda()
            yb = torch.empty((B, M), dtype=torch.float32, device="cuda")
            xq, xd, xs = gq.quantize_q8k(xb)
            it["i"] = 0

            def intdot():
                i = it["i"] % len(gates)
                it["i"] += 1
                gq.gq_gemv_q4k_q8k(gates[i], xq, xd, xs, yb, M, K, B, stream)

            def fp32():
                i = it["i"] % len(gates)
                it["i"] += 1
                gq.gq_gemv_q4k(gates[i], xb, yb, M, K, B, stream)
            si = event_time(torch, stream, intdot, reps=len(gates), warmup=len(gates))
            sb = event_time(torch, stream, fp32, reps=len(gates), warmup=len(gates))
            sq = event_time(torch, stream, lambda: gq.gq_quantize_q8k(xb, xq, xd, xs, B, K, stream))
            q8k["b%d" % B] = {"int_dot_us": round(si * 1e6, 2),
                              "int_dot_GB/s": round(q4k_bytes(M, K) / si / 1e9, 1),
                              "binary32_us": round(sb * 1e6, 2), "quantize_us": round(sq * 1e6, 2)}
        extra["gemv_q4k_q8k_%dx%d" % (M, K)] = q8k
        # single Q4_K products at batch 2, 4 and 16 (gq_gemv_q4k: the K-split
        # binary32 form at these shapes), rotated over the 32 layers' matrices
        # of that shape; time per call, launch included
        single_b = {}
        for name, M, K in (("down", 4096, 14336), ("q", 4096, 4096)):
            ws = [m[4] for m in stack.mats if m[0] == name]
            for B in (2, 4, 16):
                xb = torch.from_numpy(synth.activations_f32(0, 40 + B, B, K)).cuda()
                yb = torch.empty((B, M), dtype=torch.float32, device="cuda")
                it = {"i": 0}

                def q4call():
                    gq.gq_gemv_q4k(ws[it["i"] % len(ws)], xb, yb, M, K, B, stream)
                    it["i"] += 1
                s = event_time(torch, stream, q4call, reps=2 * len(ws), warmup=len(ws))
                single_b["%s_%dx%d_b%d" % (name, M, K, B)] = {
                    "us_per_call": round(s * 1e6, 2),
                    "GB/s": round(q4k_bytes(M, K) / s / 1e9, 1)}
        extra["gemv_q4k_single_batched"] = single_b
        del stack
        torch.cuda.empty_cache()
        # prefill matrix products
        pre = {}
        for M, K in ((14336, 4096), (4096, 14336)):
            w = torch.from_numpy(synth.q4k_blocks(PREFILL_WORKLOAD, M, M, K)).cuda()
            for N in (512, 4096):
                x16 = torch.from_numpy(synth.activations_f16(PREFILL_WORKLOAD, N, N, K)).cuda()
                y16 = torch.empty((N, M), dtype=torch.float16, device="cuda")
                s = event_time(torch, stream, lambda: gq.gq_gemm_q4k(w, x16, y16, M, K, N, stream))
                tf = 2.0 * M * K * N / s / 1e12
                pre["%dx%dxN%d" % (M, K, N)] = {"us": round(s * 1e6, 1), "TFLOP/s": round(tf, 1),
                                                "frac_fp16_peak": round(tf / FP16_PEAK_TFLOPS, 4)}
                if N == 512:
                    # few tokens, long K: the split-K form with its own
                    # choice of split count and a caller workspace
                    need = gq.gq_gemm_q4k_splitk_workspace_bytes(M, K, N, 0)
                    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
                    s = event_time(torch, stream, lambda: gq.gq_gemm_q4k_splitk(
                        w, x16, y16, M, K, N, 0, ws, need, stream))
                    tf = 2.0 * M * K * N / s / 1e12
                    pre["%dx%dxN%d_splitk" % (M, K, N)] = {
                        "us": round(s * 1e6, 1), "TFLOP/s": round(tf, 1),
                        "frac_fp16_peak": round(tf / FP16_PEAK_TFLOPS, 4),
                        "splits": need // (4 * N * M)}
                    del ws
                # the opt-in integer-dot product over 8-bit activation codes
                # (gq_quantize_q8k, then gq_gemm_q4k_q8k; binary32 out)
                x32 = x16.float()
                xq, xd, xs = gq.quantize_q8k(x32)
                y32 = torch.empty((N, M), dtype=torch.float32, device="cuda")
                s = event_time(torch, stream, lambda: gq.gq_gemm_q4k_q8k(
                    w, xq, xd, y32, M, K, N, stream))
                sq = event_time(torch, stream, lambda: gq.gq_quantize_q8k(
                    x32, xq, xd, xs, N, K, stream))
                tf = 2.0 * M * K * N / s / 1e12
                pre["%dx%dxN%d_int_dot" % (M, K, N)] = {
                    "us": round(s * 1e6, 1), "TOP/s": round(tf, 1),
                    "frac_int8_peak": round(tf / INT8_PEAK_TOPS, 4),
                    "quantize_us": round(sq * 1e6, 1)}
                del x32, xq, xd, xs, y32
                del x16, y16
            del w
        # the same product over Q8_0 weights (the LDS-tile kernel)
        M, K, N = 14336, 4096, 4096
        wq8 = torch.from_numpy(synth.q8_0_blocks(PREFILL_WORKLOAD, M, M, K)).cuda()
        x16 = torch.from_numpy(synth.activations_f16(PREFILL_WORKLOAD, N, N, K)).cuda()
        y16 = torch.empty((N, M), dtype=torch.float16, device="cuda")
        s = event_time(torch, stream, lambda: gq.gq_gemm_q8_0(wq8, x16, y16, M, K, N, stream))
        tf = 2.0 * M * K * N / s / 1e12
        pre["q8_0_%dx%dxN%d" % (M, K, N)] = {"us": round(s * 1e6, 1), "TFLOP/s": round(tf, 1),
                                             "frac_fp16_peak": round(tf / FP16_PEAK_TFLOPS, 4)}
        del wq8, x16, y16
        extra["prefill_gemm"] = pre
        # achievable ceilings measured beside the kernels: a plain 1 GiB device
        # copy (read + write streaming) and the vendor library's binary16 product
        # on unquantized operands of the prefill shapes (torch -> hipBLASLt)
        ceil = {}
        src = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        s = event_time(torch, stream, lambda: dst.copy_(src), reps=10)
        ceil["d2d_copy_1GiB_read+write_GB/s"] = round(2 * (1 << 30) / s / 1e9, 1)
        del src, dst
        for M, K in ((14336, 4096), (4096, 14336)):
            a16 = torch.randn(4096, K, device="cuda").half()
            b16 = torch.randn(M, K, device="cuda").half()
            s = event_time(torch, stream, lambda: torch.matmul(a16, b16.t()), reps=10)
            ceil["fp16_library_matmul_%dx%dxN4096_TFLOP/s" % (M, K)] = round(
                2.0 * M * K * 4096 / s / 1e12, 1)
            del a16, b16
        ceil.update(probe_ceilings(torch, stream, pre, value, stack_bytes_total()))
        extra["measured_ceilings"] = ceil
        # mixture of experts, OLMoE-1B-7B shape; routing by the device router
        # (gq_moe_route), outside the timed layer
        H, I, E, k = 2048, 1024, 64, 8
        wg = torch.from_numpy(synth.q4k_blocks(MOE_WORKLOAD, 0, E * I, H)).cuda()
        wu = torch.from_numpy(synth.q4k_blocks(MOE_WORKLOAD, 1, E * I, H)).cuda()
        wd = torch.from_numpy(synth.q4k_blocks(MOE_WORKLOAD, 2, E * H, I)).cuda()
        # the 226 MB of expert weights fit the 256 MB memory-side cache: the
        # layer is timed rotating over 4 copies (906 MB), and on one copy
        # again and again (hot) beside it
        wcopies = [(wg, wu, wd)] + [(wg.clone(), wu.clone(), wd.clone()) for _ in range(3)]
        moe, moe_in = {}, {}
        wbytes = 3 * E * q4k_bytes(I, H)
        for T in (256, 2048):
            x16 = torch.from_numpy(synth.activations_f16(MOE_WORKLOAD, 0, T, H)).cuda()
            lg = torch.from_numpy(synth.router_logits(MOE_WORKLOAD, 0, T, E)).cuda()
            ids_d, wts_d = gq.moe_route(lg, k, stream=stream)
            torch.cuda.synchronize()
            need = gq.gq_moe_workspace_bytes(T, H, I, E, k)
            ws = torch.empty(need, dtype=torch.uint8, device="cuda")
            out = torch.empty((T, H), dtype=torch.float16, device="cuda")
            it = {"i": 0}

            def moe_rot():
                cg, cu, cd = wcopies[it["i"] % len(wcopies)]
                it["i"] += 1
                gq.gq_moe_gemm_q4k(cg, cu, cd, x16, ids_d, wts_d, out, T, H, I, E, k, ws, need,
                                   stream)
            s = event_time(torch, stream, moe_rot, reps=24, warmup=8)
            hot = event_time(torch, stream, lambda: gq.gq_moe_gemm_q4k(
                wg, wu, wd, x16, ids_d, wts_d, out, T, H, I, E, k, ws, need, stream))
            flops = 2.0 * T * k * 3 * H * I
            moe["T%d" % T] = {"us": round(s * 1e6, 1), "TFLOP/s": round(flops / s / 1e12, 1),
                              "weight_GB/s": round(wbytes / s / 1e9, 1),
                              "rotated_over_MB": round(len(wcopies) * wbytes / 1e6, 1),
                              "hot_us": round(hot * 1e6, 1)}
            # the routing step itself (gq_moe_route), timed apart
            rid = torch.empty((T, k), dtype=torch.int32, device="cuda")
            rwt = torch.empty((T, k), dtype=torch.float32, device="cuda")
            s = event_time(torch, stream, lambda: gq.gq_moe_route(lg, rid, rwt, T, E, k, 0, stream))
            moe["T%d" % T]["route_us"] = round(s * 1e6, 2)
            # the same layer with the weights on the experts' inputs (Llama 4 form)
            it["i"] = 0

            def moe_rot_iw():
                cg, cu, cd = wcopies[it["i"] % len(wcopies)]
                it["i"] += 1
                gq.gq_moe_gemm_q4k(cg, cu, cd, x16, ids_d, wts_d, out, T, H, I, E, k, ws, need,
                                   stream, input_weighted=True)
            s = event_time(torch, stream, moe_rot_iw, reps=24, warmup=8)
            moe["T%d" % T]["input_weighted_us"] = round(s * 1e6, 1)
            moe_in[T] = (x16, ids_d, wts_d, ws, need, out)
        extra["moe_olmoe"] = moe
        # one GPU's share under 8-way expert parallelism: experts 0..7 and the
        # rows an all-to-all dispatch would deliver, one row per (token, local
        # expert) assignment, routed top-1 to the local expert
        ep = {}
        for T in (256, 2048):
            lg = torch.from_numpy(synth.router_logits(MOE_WORKLOAD, 0, T, E)).cuda()
            ids_t, wts_t = gq.moe_route(lg, k, stream=stream)
            torch.cuda.synchronize()
            ids, wts = ids_t.cpu().numpy(), wts_t.cpu().numpy()
            tok, slot = np.nonzero(ids < E // 8)
            x16 = synth.activations_f16(MOE_WORKLOAD, 0, T, H)[tok]
            R = len(tok)
            xs_d = torch.from_numpy(np.ascontiguousarray(x16)).cuda()
            ids_d = torch.from_numpy(ids[tok, slot].astype(np.int32).reshape(R, 1)).cuda()
            wts_d = torch.from_numpy(wts[tok, slot].astype(np.float32).reshape(R, 1)).cuda()
            need = gq.gq_moe_workspace_bytes(R, H, I, E // 8, 1)
            ws = torch.empty(need, dtype=torch.uint8, device="cuda")
            out = torch.empty((R, H), dtype=torch.float16, device="cuda")
            s = event_time(torch, stream, lambda: gq.gq_moe_gemm_q4k(
                wg, wu, wd, xs_d, ids_d, wts_d, out, R, H, I, E // 8, 1, ws, need, stream))
            ep["T%d" % T] = {"rows": int(R), "us": round(s * 1e6, 1),
                             "TFLOP/s": round(2.0 * R * 3 * H * I / s / 1e12, 1),
                             "weight_GB/s": round(3 * (E // 8) * q4k_bytes(I, H) / s / 1e9, 1)}
        extra["moe_olmoe_ep8_shard"] = ep
        del wg, wu, wd, wcopies
        # the same layer over Q8_0 expert stacks
        wg = torch.from_numpy(synth.q8_0_blocks(MOE_WORKLOAD, 0, E * I, H)).cuda()
        wu = torch.from_numpy(synth.q8_0_blocks(MOE_WORKLOAD, 1, E * I, H)).cuda()
        wd = torch.from_numpy(synth.q8_0_blocks(MOE_WORKLOAD, 2, E * H, I)).cuda()
        moe8 = {}
        wbytes = 3 * E * I * (H // 32) * 34
        for T, (x16, ids_d, wts_d, ws, need, out) in moe_in.items():
            s = event_time(torch, stream, lambda: gq.gq_moe_gemm_q8_0(
                wg, wu, wd, x16, ids_d, wts_d, out, T, H, I, E, k, ws, need, stream))
            flops = 2.0 * T * k * 3 * H * I
            moe8["T%d" % T] = {"us": round(s * 1e6, 1), "TFLOP/s": round(flops / s / 1e12, 1),
                               "weight_GB/s": round(wbytes / s / 1e9, 1)}
        extra["moe_olmoe_q8_0"] = moe8
        del wg, wu, wd, moe_in
        # Q8_0 matrix-vector product, 256 x 1024
        wq = torch.from_numpy(synth.q8_0_blocks(0, 0, 256, 1024)).cuda()
        xq = torch.from_numpy(synth.activations_f32(0, 0, 1, 1024)).cuda()
        yq = torch.empty((1, 256), dtype=torch.float32, device="cuda")
        # a latency probe: timed right after the heavier work, without the
        # time-based warm-up (a stream of tiny launches lets the clocks drop)
        s = event_time(torch, stream, lambda: gq.gq_gemv_q8_0(wq, xq, yq, 256, 1024, 1, stream),
                       warm_s=0.0)
        extra["gemv_q8_0_256x1024_b1_us"] = round(s * 1e6, 2)
        # Q8_0 matrix-vector products at a decode shape, batch 1, 4 and 16,
        # rotated over 8 copies of the weights (272 MB, past the caches)
        M, K = 14336, 4096
        w8 = [torch.from_numpy(synth.q8_0_blocks(0, 1, M, K)).cuda()]
        w8 += [w8[0].clone() for _ in range(7)]
        q80 = {}
        for B in (1, 4, 16):
            xb = torch.from_numpy(synth.activations_f32(0, 2 + B, B, K)).cuda()
            yb = torch.empty((B, M), dtype=torch.float32, device="cuda")
            it = {"i": 0}

            def q8call():
                gq.gq_gemv_q8_0(w8[it["i"] % 8], xb, yb, M, K, B, stream)
                it["i"] += 1
            s = event_time(torch, stream, q8call, reps=48, warmup=16)
            q80["b%d" % B] = {"us": round(s * 1e6, 2),
                              "GB/s": round(w8[0].numel() / s / 1e9, 1)}
        extra["gemv_q8_0_%dx%d" % (M, K)] = q80
        del w8

    cpu = None if args.no_cpu else cpu_baseline(synth)
    receipt = make_receipt(torch, stack_sha256)

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(sec * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("q4_k weights x f32 activations (carried as a binary16 hi+lo pair, "
                  "~22 significant bits, into v_dot2_f32_f16), f32 accumulation"
                  if SB == 1 else
                  "q4_k weights x f32 activations (binary16 hi+lo pair into f16 MFMA), "
                  "f32 accumulation"),
        "data": "synthetic (seeded Q4_K blocks and N(0,1) activations)",
        "config": {"workload": "llama3-8b-shaped Q4_K decode stack, 32 layers x 7 GEMVs, "
                               "batch %d, one launch per step" % SB,
                   "weight_bytes_per_step": stack_bytes_total(),
                   "global_batch": SB, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic() if SB == 1 else None,
                     "kernel": ("gemv_q4k_stream_kernel" if SB == 1 else "gemv_q4k_mfma_kernel")
                     + " (224 products per launch)",
                     "avg_launch_us": round(avg_dur * 1e6, 3),
                     "alg_bytes_per_launch": int(alg_bytes)},
        "cpu_baseline": cpu,
        "receipt": receipt,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


def stack_bytes_total():
    return N_LAYERS * sum(q4k_bytes(M, K) for _, M, K in LAYER)


if __name__ == "__main__":
    main()
