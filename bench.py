"""Benchmark of the k-quant weight matmul hot path on one MI355X.

One step is one pass of the whole hot path over one batch of synthetic input:
  1. quantize the prefill activations  (M=3314, K=3584, f32 -> int8 plane)
  2. Q4_K prefill GEMM                 (M=3314, N=18944, K=3584; int8 MFMA)
  3. quantize the decode activation    (M=1, K=3584)
  4. Q4_K decode GEMV                  (M=1, N=18944, K=3584)
The inputs are the seeded 7B-class FFN up-projection workloads (prefill of a
3314-token prompt and one decode token), resident in HBM before timing. The
decode GEMV rotates through enough weight copies (>= 1 GiB) that the 256 MB
last-level cache cannot hold them, so its weight bytes come from HBM.

Prints one JSON line: value = int8 ops of the whole step (2*M*N*K of both
matmuls) per second, in TOPS, from the median of 21 windows of exactly K
steps, each between two events (p10 / p90 beside it), after a warm-up of at
least 0.5 s; "roofline" for the dominant kernel (the GEMM, MFMA-bound) and
"decode_roofline" for the GEMV (HBM-bound), both from a second,
instrumented pass over K steps: fence-free HIP events that the library
records at the kernels' own dispatch start and end (mq_time_next_kernel, the
quantity a kernel trace reports; the GEMM on even steps, the GEMV on odd
ones, the quantizers in a pass of their own); that pass is timed as a whole
too ("instrumented_vs_timed"). A third pass records events
around each call ("avg_us_call_bracket", which adds the launch gap).
"cpu_baseline" = the CPU oracle timed on the whole prefill GEMM (median of
3) and on one thread.

  python bench.py [--steps K] [--warmup W] [--no-cpu]
  python bench.py --all                  # per-matrix table of every workload
  python bench.py --copy-calibration     # plain copy kernel (counter scale)
  python bench.py --ceilings             # read-stream and MFMA/VALU ceiling probes
  python bench.py --case NAME --steps K  # one workload's matmul K times (profiling target)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
INT8_PEAK_TOPS = 5000.0      # MI355X dense int8 MFMA, published
ROTATE_BYTES = 1 << 30       # weight copies for HBM-bound kernels
WARMUP_S = 0.5               # warm-up of the contract run, at least
WINDOWS = 21                 # timed windows of K steps each
REWARM_S = 0.1               # plain steps queued right before each measured pass
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = {
    "gemm_q4k": "quant_gemm_amd/csrc/gemm_q4k.hip",
    "gemm_q6k": "quant_gemm_amd/csrc/gemm_q6k.hip",
    "gemv_q4k": "quant_gemm_amd/csrc/gemv.hip",
    "gemv_q6k": "quant_gemm_amd/csrc/gemv.hip",
    "quantize": "quant_gemm_amd/csrc/quantize.hip",
}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def source_hash(kernel: str) -> str:
    """Hash of what a kernel is built from: its source, the shared device
    header and the compiler flags of its source file."""
    from quant_gemm_amd import build as mq_build
    h = hashlib.sha256()
    for rel in sorted({KERNEL_SOURCES[kernel], "quant_gemm_amd/csrc/mq_device.h"}):
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    h.update(" ".join(mq_build.kernel_flags(KERNEL_SOURCES[kernel])).encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from committed counter runs, if the kernel source
    is unchanged since they were taken; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get(kernel, {}).get(workload)
    if not e or e.get("source_hash") != source_hash(kernel):
        return None
    return e.get("bytes_per_launch")


def q4k_gemv_bytes(M, N, K):
    return N * (K // 256) * 144 + M * (K + 2 * 4 * (K // 32)) + 4 * M * N


def q5k_gemv_bytes(M, N, K):
    return N * (K // 256) * 176 + M * (K + 2 * 4 * (K // 32)) + 4 * M * N


def q6k_gemv_bytes(M, N, K):
    return N * (K // 256) * 210 + M * (K + 4 * (K // 32)) + 4 * M * N


def cpu_baseline(W, x, case):
    """The oracle, as it is, on the whole prefill GEMM: one warm-up run and
    the median of three timed runs on all its OpenMP threads, plus the rate
    of one thread on the first 128 tokens."""
    import numpy as np
    import oracle
    oracle.lib()
    threads = oracle.max_threads()
    q, d, _ = oracle.quantize_act(x)

    def timed(tokens=None):
        t0 = time.perf_counter()
        oracle.matmul_q4k(W, q, d, case.N, case.K, tokens=tokens)
        return time.perf_counter() - t0

    warm = timed()
    runs = [timed() for _ in range(3 if warm < 20.0 else 1)]
    t = float(np.median(runs))
    macs = case.M * case.N * case.K
    ntok1 = min(128, case.M)
    oracle.set_threads(1)
    try:
        t1 = timed(np.arange(ntok1))
    finally:
        oracle.set_threads(threads)
    macs1 = ntok1 * case.N * case.K
    return {
        "value": round(2 * macs / t / 1e12, 4), "unit": "TOPS", "cores": threads, "kind": "oracle",
        "host_cpus": os.cpu_count(),
        "sample": (f"the whole Q4_K matmul of the M={case.M} prefill (N={case.N}, K={case.K}, "
                   f"{macs:.3g} MACs): median of {len(runs)} runs after one warm-up, "
                   f"{t:.2f} s each ({', '.join(f'{r:.2f}' for r in runs)} s) on {threads} OpenMP threads "
                   "(plain C, integer group dots, f64 combination)"),
        "one_thread": {"value": round(2 * macs1 / t1 / 1e12, 5), "unit": "TOPS", "cores": 1,
                       "sample": f"tokens 0..{ntok1 - 1} of the same matmul, {t1:.2f} s"},
    }


HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000


class KernelClock:
    """Raw hipEvent_t pairs that the library records at a kernel's own
    dispatch start and end (mq.time_next_kernel): the kernel's duration by
    HIP events, without the launch gap that events recorded around the call
    include. Created from the HIP runtime torch has loaded, without the
    system-scope fence (timing only: no cache write-back and invalidate
    around the kernels they time)."""

    def __init__(self, n, flags=HIP_EVENT_DISABLE_SYSTEM_FENCE):
        import ctypes
        import torch
        self.ct = ctypes
        lib = ctypes.CDLL(os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so"))
        lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.lib = lib
        self.ev = []
        for _ in range(n):
            pair = [ctypes.c_void_p(), ctypes.c_void_p()]
            for e in pair:
                if lib.hipEventCreateWithFlags(ctypes.byref(e), flags) != 0:
                    raise RuntimeError("hipEventCreateWithFlags failed")
            self.ev.append(pair)

    def arm(self, i):
        import quant_gemm_amd as mq
        mq.time_next_kernel(self.ev[i][0].value, self.ev[i][1].value)

    def us(self, i):
        ms = self.ct.c_float()
        if self.lib.hipEventElapsedTime(self.ct.byref(ms), self.ev[i][0], self.ev[i][1]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value * 1e3

    def close(self):
        for pair in self.ev:
            for e in pair:
                self.lib.hipEventDestroy(e)


def run_contract(args):
    import numpy as np
    import torch

    import quant_gemm_amd as mq
    from quant_gemm_amd import synth

    mq.load()
    dev = torch.device("cuda:0")
    pre = synth.case_by_name("q4k_prefill_ffn_up")
    dec = synth.case_by_name("q4k_decode_ffn_up")
    log(f"[bench] generating inputs: {pre.name} and {dec.name}")
    Wp_np = pre.make_weights()
    xp_np = pre.make_activations()
    Wd_np = dec.make_weights()
    xd_np = dec.make_activations()

    Wp = torch.from_numpy(Wp_np.reshape(-1)).to(dev)
    xp = torch.from_numpy(xp_np).to(dev)
    xd = torch.from_numpy(xd_np).to(dev)
    Wd0 = torch.from_numpy(Wd_np.reshape(-1)).to(dev)
    copies = max(1, -(-ROTATE_BYTES // Wd0.numel()))
    Wd = [Wd0] + [Wd0.clone() for _ in range(copies - 1)]
    qp = torch.empty((pre.M, pre.K), dtype=torch.int8, device=dev)
    dp = torch.empty((pre.M, pre.K // 32), dtype=torch.float32, device=dev)
    sp = torch.empty_like(dp)
    qd = torch.empty((dec.M, dec.K), dtype=torch.int8, device=dev)
    dd = torch.empty((dec.M, dec.K // 32), dtype=torch.float32, device=dev)
    sd = torch.empty_like(dd)
    outp = torch.empty((pre.M, pre.N), dtype=torch.float32, device=dev)
    outd = torch.empty((dec.M, dec.N), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    names = ["quantize_prefill", "gemm_q4k", "quantize_decode", "gemv_q4k"]

    def step(i, ev=None, kc=None):
        if ev: ev[0].record()
        if kc and kc[0]: kc[0].arm(i)
        mq.quantize_act(xp, qp, dp, sp)
        if ev: ev[1].record()
        if kc and kc[1]: kc[1].arm(i)
        mq.matmul_q4k(Wp, qp, dp, sp, pre.N, pre.K, out=outp)
        if ev: ev[2].record()
        if kc and kc[2]: kc[2].arm(i)
        mq.quantize_act(xd, qd, dd, sd)
        if ev: ev[3].record()
        if kc and kc[3]: kc[3].arm(i)
        mq.matmul_q4k(Wd[i % copies], qd, dd, sd, dec.N, dec.K, out=outd)
        if ev: ev[4].record()

    # Every event of the measured passes is created now: creating them
    # between passes would leave the GPU idle long enough for its clocks to
    # drop, and the first launches after that run slow.
    kclocks = [KernelClock(args.steps) for _ in names]
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]

    # Warm-up: the --warmup steps, continued until at least WARMUP_S seconds
    # of steps have run, so that clocks and caches have settled.
    log(f"[bench] warmup: {args.warmup} steps, at least {WARMUP_S} s")
    t0 = time.perf_counter()
    warm = 0
    while warm < args.warmup or time.perf_counter() - t0 < WARMUP_S:
        step(warm)
        warm += 1
        if warm % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    # The timed region: WINDOWS windows of exactly K steps each, every one
    # between a synchronize and two events with nothing else in it (no
    # per-call events, whose marker packets would add GPU time to each step).
    log(f"[bench] timing {WINDOWS} windows of {args.steps} steps")
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    win_ms = []
    for _ in range(WINDOWS):
        torch.cuda.synchronize()
        t_start.record()
        for i in range(args.steps):
            step(i)
        t_end.record()
        torch.cuda.synchronize()
        win_ms.append(t_start.elapsed_time(t_end))
    win_step = np.array(win_ms) / args.steps
    # Each measured pass below is queued right behind REWARM_S seconds of
    # plain steps, with no synchronization in between, so that it starts on
    # a busy GPU at the clocks of the timed windows.
    rewarm_steps = max(1, int(REWARM_S / (float(np.median(win_step)) * 1e-3)))

    def rewarm():
        for i in range(rewarm_steps):
            step(i)

    # A second pass over the same steps, instrumented: the GEMM (even steps)
    # and the GEMV (odd steps) record fence-free events at their own dispatch
    # start and end (the roofline figures). One timed kernel per step keeps
    # the instrumentation's own cost small; the pass is timed as a whole like
    # a window, so that its time per step shows that cost.
    log(f"[bench] per-kernel timing pass, {args.steps} steps")
    timed = {n: [] for n in names}

    def instrumented_pass(which):
        for i in range(args.steps):
            armed = [None] * 4
            for k in (which if args.steps < 2 else which[i % 2:i % 2 + 1]):
                armed[k] = kclocks[k]
                timed[names[k]].append(i)
            step(i, kc=armed)

    torch.cuda.synchronize()
    rewarm()
    t_start.record()
    instrumented_pass((1, 3))
    t_end.record()
    torch.cuda.synchronize()
    instr_ms_step = t_start.elapsed_time(t_end) / args.steps
    rewarm()
    instrumented_pass((0, 2))        # the two quantizers, in a pass of their own
    torch.cuda.synchronize()
    kernel_us = {n: np.array([kc.us(i) for i in timed[n]]) for n, kc in zip(names, kclocks)}
    for kc in kclocks:
        kc.close()
    # A third pass: events recorded around each call (kernel plus the launch
    # gap after the preceding one), kept apart from the kernel figures.
    rewarm()
    for i in range(args.steps):
        step(i, ev=evs[i])
    torch.cuda.synchronize()
    per = {n: np.array([evs[i][k].elapsed_time(evs[i][k + 1]) for i in range(args.steps)])
           for k, n in enumerate(names)}
    avg_us = {n: float(v.mean() * 1e3) for n, v in per.items()}
    kern_avg_us = {n: float(v.mean()) for n, v in kernel_us.items()}

    ops_pre = pre.ops
    ops_dec = dec.ops
    ms_step = float(np.median(win_step))
    value = (ops_pre + ops_dec) / (ms_step * 1e-3) / 1e12

    # roofline figures from the kernels' own durations (dispatch-boundary
    # events); the per-call event brackets are reported beside them
    gemm_us = float(kernel_us["gemm_q4k"].mean())
    gemv_us = float(kernel_us["gemv_q4k"].mean())
    gemm_tops = ops_pre / (gemm_us * 1e-6) / 1e12
    gemv_bytes = q4k_gemv_bytes(dec.M, dec.N, dec.K)
    gemv_gbs = gemv_bytes / (gemv_us * 1e-6) / 1e9
    qbytes = pre.M * pre.K * 4 + pre.M * pre.K + 2 * 4 * pre.M * (pre.K // 32)

    res = {
        "metric": "int8 TOPS + % MFMA peak (M=3314 GEMM); GB/s + % HBM peak (M=1 GEMV)",
        "value": round(value, 3),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "ms_per_step_p10": round(float(np.percentile(win_step, 10)), 4),
        "ms_per_step_p90": round(float(np.percentile(win_step, 90)), 4),
        "timing": (f"median over {WINDOWS} windows of {args.steps} steps (events around each window); "
                   f"warm-up {warm} steps, {WARMUP_S} s or more"),
        "instrumented_ms_per_step": round(instr_ms_step, 4),
        "instrumented_vs_timed": round(instr_ms_step / ms_step, 4),
        "kernels_sum_ms_per_step": round(sum(kern_avg_us.values()) * 1e-3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic (seeded Q4_K blocks and N(0,1) activations with 1% x20 outlier columns)",
        "config": {
            "workload": ("q4k ffn_up prefill M=3314 N=18944 K=3584 (quantize + GEMM) + "
                         "q4k ffn_up decode M=1 N=18944 K=3584 (quantize + GEMV)"),
            "prefill_tokens": pre.M, "decode_tokens": dec.M, "N": pre.N, "K": pre.K,
            "decode_weight_copies": copies, "parallelism": "none (1 GPU)",
        },
        "roofline": {
            "kernel": "gemm_q4k", "bound": "mfma", "achieved": round(gemm_tops, 2),
            "peak": INT8_PEAK_TOPS, "unit": "TOPS", "frac": round(gemm_tops / INT8_PEAK_TOPS, 4),
            "traffic": measured_traffic("gemm_q4k", "prefill_ffn_up"),
            "work_per_launch": f"{ops_pre:.4g} int8 ops (2*M*N*K)",
            "avg_us": round(gemm_us, 2), "timing": "kernel start/end events (hipExtLaunchKernel)",
            "avg_us_call_bracket": round(avg_us["gemm_q4k"], 2),
        },
        "decode_roofline": {
            "kernel": "gemv_q4k", "bound": "hbm", "achieved": round(gemv_gbs, 1),
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gemv_gbs / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic("gemv_q4k", "decode_ffn_up"),
            "work_per_launch": f"{gemv_bytes} bytes (weights + int8 plane + output)",
            "avg_us": round(gemv_us, 3), "median_us": round(float(np.median(kernel_us["gemv_q4k"])), 3),
            "timing": "kernel start/end events (hipExtLaunchKernel)",
            "avg_us_call_bracket": round(avg_us["gemv_q4k"], 3),
        },
        "kernels_avg_us": {n: round(v, 3) for n, v in kern_avg_us.items()},
        "kernels_avg_us_call_bracket": {n: round(v, 3) for n, v in avg_us.items()},
        "quantize_prefill_GBs": round(qbytes / (kern_avg_us["quantize_prefill"] * 1e-6) / 1e9, 1),
    }
    if not args.no_cpu:
        log("[bench] CPU oracle baseline")
        res["cpu_baseline"] = cpu_baseline(Wp_np, xp_np, pre)
    print(json.dumps(res), flush=True)


def run_all(args):
    """Per-matrix kernel times for every workload (a table, not the contract line)."""
    import numpy as np
    import torch

    import quant_gemm_amd as mq
    from quant_gemm_amd import synth

    mq.load()
    dev = torch.device("cuda:0")
    rows = []
    for grp, case in synth.all_cases():
        log(f"[bench --all] {case.name}")
        W_np = case.make_weights()
        x = torch.from_numpy(case.make_activations()).to(dev)
        W0 = torch.from_numpy(W_np.reshape(-1)).to(dev)
        hbm = case.M <= mq.gemv_max_m()
        copies = max(1, -(-ROTATE_BYTES // W0.numel())) if hbm else 1
        Ws = [W0] + [W0.clone() for _ in range(copies - 1)]
        q, d, s = mq.quantize_act(x)
        mm = {"q4k": mq.matmul_q4k, "q5k": mq.matmul_q5k, "q6k": mq.matmul_q6k}[case.fmt]
        out = torch.empty((case.M, case.N), dtype=torch.float32, device=dev)
        reps = max(copies, 20 if not hbm else 2 * copies)
        # warm-up of about the timed work, then the median of 3 rounds
        _time_rotating(lambda i: mm(Ws[i], q, d, s, case.N, case.K, out=out), copies, reps)
        us = float(np.median([_time_rotating(lambda i: mm(Ws[i], q, d, s, case.N, case.K, out=out), copies, reps)
                              for _ in range(3)]))
        row = {"group": grp, "case": case.name, "fmt": case.fmt, "M": case.M, "N": case.N,
               "K": case.K, "us": round(us, 2), "TOPS": round(case.ops / (us * 1e-6) / 1e12, 2)}
        if hbm:
            b = {"q4k": q4k_gemv_bytes, "q5k": q5k_gemv_bytes, "q6k": q6k_gemv_bytes}[case.fmt](case.M, case.N, case.K)
            row["GBs"] = round(b / (us * 1e-6) / 1e9, 1)
            row["frac_hbm"] = round(row["GBs"] / HBM_PEAK_GBS, 3)
        else:
            row["frac_int8_peak"] = round(row["TOPS"] / INT8_PEAK_TOPS, 4)
        rows.append(row)
        print(json.dumps(row), flush=True)
        del Ws, W0, out, q, d, s, x
        torch.cuda.empty_cache()
    run_producers(dev)
    run_ffn(dev)
    run_planes(dev)


_BUSY = []


def _time_rotating(fn, copies, reps):
    """GPU time per call (us) of reps calls over `copies` rotating inputs.

    The calls are queued behind ~15 ms of f32 matmul, so the events bracket
    GPU work only: back to back from Python, each call's host cost (~8.5 us
    of ctypes marshalling and checks) would bound the small decode kernels.
    """
    import time
    import torch
    if not _BUSY:
        _BUSY.append(torch.randn(8192, 8192, device="cuda"))
    a = _BUSY[0]
    for i in range(3):
        fn(i % copies)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    b0 = torch.cuda.Event(enable_timing=True)
    b0.record()
    torch.mm(a, a)
    torch.mm(a, a)
    e0.record()
    t0 = time.perf_counter()
    for i in range(reps):
        fn(i % copies)
    host_ms = (time.perf_counter() - t0) * 1e3
    e1.record()
    torch.cuda.synchronize()
    if host_ms > 0.8 * b0.elapsed_time(e0):
        log(f"[bench] warning: enqueueing {reps} calls took {host_ms:.1f} ms, about the busy "
            f"period ({b0.elapsed_time(e0):.1f} ms): the time may include host cost")
    return e0.elapsed_time(e1) * 1e3 / reps


def run_ffn(dev):
    """Fused FFN up half (gate and up matmuls + SwiGLU + plane in one call)
    against the separate calls (two matmuls, then mq_swiglu_quantize).
    Weights rotate through >= 1 GiB of copies at M = 1."""
    import numpy as np
    import torch

    import quant_gemm_amd as mq
    from quant_gemm_amd import synth

    for grp, M, N, K in (("ffn", 1, 18944, 3584), ("ffn", 4, 18944, 3584), ("ffn", 8, 18944, 3584),
                         ("ffn", 3314, 18944, 3584)):
        rng = np.random.default_rng(3000 + M)
        Wg0 = torch.from_numpy(synth.q4k_weights(rng, N, K).reshape(-1)).to(dev)
        Wu0 = torch.from_numpy(synth.q4k_weights(rng, N, K).reshape(-1)).to(dev)
        x = torch.from_numpy(synth.activations(rng, M, K, outliers=True)).to(dev)
        q, d, s = mq.quantize_act(x)
        copies = max(1, -(-ROTATE_BYTES // (2 * Wg0.numel()))) if M <= mq.gemv_max_m() else 1
        Wgs = [Wg0] + [Wg0.clone() for _ in range(copies - 1)]
        Wus = [Wu0] + [Wu0.clone() for _ in range(copies - 1)]
        qo = torch.empty((M, N), dtype=torch.int8, device=dev)
        do = torch.empty((M, N // 32), dtype=torch.float32, device=dev)
        so = torch.empty_like(do)
        reps = max(2 * copies, 10)
        fused_fn = lambda i: mq.ffn_q4k(Wgs[i], Wus[i], q, d, s, N, K, qo=qo, do=do, so=so)

        g_out = torch.empty((M, N), dtype=torch.float32, device=dev)
        u_out = torch.empty((M, N), dtype=torch.float32, device=dev)
        sep_fn = lambda i: (mq.matmul_q4k(Wgs[i], q, d, s, N, K, out=g_out),
                            mq.matmul_q4k(Wus[i], q, d, s, N, K, out=u_out),
                            mq.swiglu_quantize(g_out, u_out, q=qo, d=do, s=so))
        # alternate the two, 3 rounds each, and keep the medians (clocks drift)
        ft, st_ = [], []
        for _ in range(3):
            ft.append(_time_rotating(fused_fn, copies, reps))
            st_.append(_time_rotating(sep_fn, copies, reps))
        fused, sep = float(np.median(ft)), float(np.median(st_))
        ops = 2 * 2 * M * N * K
        row = {"group": grp, "case": f"ffn_q4k gate|up+SwiGLU+plane M={M} N={N} K={K}", "us": round(fused, 2),
               "TOPS": round(ops / (fused * 1e-6) / 1e12, 2), "separate_us": round(sep, 2)}
        if M <= mq.gemv_max_m():
            b = 2 * N * (K // 256) * 144 + M * (K + 8 * (K // 32)) + M * (N + 8 * (N // 32))
            row["GBs"] = round(b / (fused * 1e-6) / 1e9, 1)
            row["frac_hbm"] = round(row["GBs"] / HBM_PEAK_GBS, 3)
        else:
            row["frac_int8_peak"] = round(row["TOPS"] / INT8_PEAK_TOPS, 4)
        print(json.dumps(row), flush=True)
        del Wgs, Wus, Wg0, Wu0, g_out, u_out
        torch.cuda.empty_cache()


def run_planes(dev):
    """The GEMMs reading registration-time planes (Q6_K expansion, Q4_K
    decoded scales) against the same GEMMs on the raw blocks, on the
    prefill workloads; the planes' build time and size beside them."""
    import numpy as np
    import torch

    import quant_gemm_amd as mq
    from quant_gemm_amd import synth

    for name in ("layer_down", "q6k_ffn_down_m512", "q4k_prefill_ffn_up", "q4k_prefill_attn_o"):
        c = synth.case_by_name(name)
        W = torch.from_numpy(c.make_weights().reshape(-1)).to(dev)
        x = torch.from_numpy(c.make_activations()).to(dev)
        q, d, s = mq.quantize_act(x)
        out = torch.empty((c.M, c.N), dtype=torch.float32, device=dev)
        if c.fmt == "q6k":
            lo, hi, dw = mq.expand_q6k(W, c.N, c.K)
            build = lambda i: mq.expand_q6k(W, c.N, c.K, lo, hi, dw)
            # the raw-block GEMM: a workspace of the split-K part only (the
            # full one would expand W per call)
            ws = torch.empty(max(16, mq.matmul_split_workspace(mq.MQ_FMT_Q6K, c.M, c.N, c.K, mq.MQ_PATH_GEMM)),
                             dtype=torch.uint8, device=dev)
            raw = lambda i: mq.matmul_q6k(W, q, d, None, c.N, c.K, out=out, path=mq.MQ_PATH_GEMM, workspace=ws)
            planes = lambda i: mq.matmul_q6k_x(lo, hi, dw, q, d, c.N, c.K, out=out)
            kind, plane_bytes = "q6k expansion (lo, hi, d)", 2 * lo.numel() + 4 * dw.numel()
        else:
            fw, fm = mq.dsc_q4k(W, c.N, c.K)
            build = lambda i: mq.dsc_q4k(W, c.N, c.K, fw, fm)
            raw = lambda i: mq.matmul_q4k(W, q, d, s, c.N, c.K, out=out, path=mq.MQ_PATH_GEMM)
            planes = lambda i: mq.matmul_q4k_dsc(W, fw, fm, q, d, s, c.N, c.K, out=out)
            kind, plane_bytes = "q4k decoded scales (fw, fm)", 8 * fw.numel()
        rt, pt = [], []
        for _ in range(3):                        # alternate; medians (clocks drift)
            rt.append(_time_rotating(raw, 1, 20))
            pt.append(_time_rotating(planes, 1, 20))
        r, p_ = float(np.median(rt)), float(np.median(pt))
        row = {"group": "planes", "case": f"{name} {kind}", "M": c.M, "N": c.N, "K": c.K,
               "us": round(p_, 2), "TOPS": round(c.ops / (p_ * 1e-6) / 1e12, 2), "raw_us": round(r, 2),
               "speedup": round(r / p_, 3), "build_us": round(_time_rotating(build, 1, 3), 1),
               "plane_MB": round(plane_bytes / 1e6, 1), "raw_MB": round(W.numel() / 1e6, 1)}
        print(json.dumps(row), flush=True)
        del W, x, out
        torch.cuda.empty_cache()


def run_producers(dev):
    """Producer-fused quantizers (RMSNorm / SwiGLU -> int8 plane) against the
    unfused pair (producer writing f32, then the quantizer reading it). Inputs
    rotate through >= 1 GiB of copies so that they come from HBM."""
    import numpy as np
    import torch

    import quant_gemm_amd as mq
    from quant_gemm_amd import synth

    rng = np.random.default_rng(2024)
    for M, K in ((3314, 3584), (1, 3584)):
        x0 = torch.from_numpy(synth.activations(rng, M, K, outliers=True)).to(dev)
        w = torch.from_numpy((1.0 + 0.3 * rng.standard_normal(K)).astype(np.float32)).to(dev)
        copies = min(64, max(1, -(-ROTATE_BYTES // (x0.numel() * 4))))   # tiny inputs stay cached anyway
        xs = [x0] + [x0.clone() for _ in range(copies - 1)]
        q, d, s = mq.quantize_act(x0)
        y = torch.empty_like(x0)
        reps = max(2 * copies, 20)
        fused = _time_rotating(lambda i: mq.rmsnorm_quantize(xs[i], w, 1e-6, q=q, d=d, s=s), copies, reps)
        unfused = _time_rotating(lambda i: (mq.rmsnorm_quantize(xs[i], w, 1e-6, q=q, d=d, s=s, y=y),
                                            mq.quantize_act(y, q=q, d=d, s=s)), copies, reps)
        b = M * K * 4 + K * 4 + M * K + 8 * M * (K // 32)
        row = {"group": "producers", "case": f"rmsnorm_quantize M={M} K={K}", "us": round(fused, 2),
               "GBs": round(b / (fused * 1e-6) / 1e9, 1), "frac_hbm": round(b / (fused * 1e-6) / 1e9 / HBM_PEAK_GBS, 3),
               "unfused_us": round(unfused, 2)}
        print(json.dumps(row), flush=True)
        del xs, x0
        torch.cuda.empty_cache()
    for M, K in ((3314, 18944), (1, 18944)):
        gu0 = torch.from_numpy(np.concatenate([(rng.standard_normal((M, K)) * 2.5).astype(np.float32),
                                               synth.activations(rng, M, K, outliers=True)], axis=1)).to(dev)
        copies = min(64, max(1, -(-ROTATE_BYTES // (gu0.numel() * 4))))
        gus = [gu0] + [gu0.clone() for _ in range(copies - 1)]
        q = torch.empty((M, K), dtype=torch.int8, device=dev)
        d = torch.empty((M, K // 32), dtype=torch.float32, device=dev)
        s = torch.empty_like(d)
        y = torch.empty((M, K), dtype=torch.float32, device=dev)
        reps = max(4 * copies, 20)
        fused = _time_rotating(lambda i: mq.swiglu_quantize(gus[i][:, :K], gus[i][:, K:], q=q, d=d, s=s),
                               copies, reps)
        unfused = _time_rotating(lambda i: (mq.swiglu_quantize(gus[i][:, :K], gus[i][:, K:], q=q, d=d, s=s, y=y),
                                            mq.quantize_act(y, q=q, d=d, s=s)), copies, reps)
        b = 2 * M * K * 4 + M * K + 8 * M * (K // 32)
        row = {"group": "producers", "case": f"swiglu_quantize M={M} K={K}", "us": round(fused, 2),
               "GBs": round(b / (fused * 1e-6) / 1e9, 1), "frac_hbm": round(b / (fused * 1e-6) / 1e9 / HBM_PEAK_GBS, 3),
               "unfused_us": round(unfused, 2)}
        print(json.dumps(row), flush=True)
        del gus, gu0
        torch.cuda.empty_cache()


def run_case(args):
    """One named workload's matmul, K times through the library's default
    full plan (a workspace from the query), after one warm-up call: a
    profiling target (rocprofv3 -- python3 bench.py --case NAME). Prints
    the GPU time per call, queued behind busy work."""
    import numpy as np
    import torch

    import quant_gemm_amd as mq
    from quant_gemm_amd import synth

    mq.load()
    dev = torch.device("cuda:0")
    case = synth.case_by_name(args.case)
    W = torch.from_numpy(case.make_weights().reshape(-1)).to(dev)
    x = torch.from_numpy(case.make_activations()).to(dev)
    q, d, s = mq.quantize_act(x)
    mm = {"q4k": mq.matmul_q4k, "q5k": mq.matmul_q5k, "q6k": mq.matmul_q6k}[case.fmt]
    out = torch.empty((case.M, case.N), dtype=torch.float32, device=dev)
    fmt = {"q4k": mq.MQ_FMT_Q4K, "q5k": mq.MQ_FMT_Q5K, "q6k": mq.MQ_FMT_Q6K}[case.fmt]
    ws = torch.empty(max(1, mq.matmul_workspace(fmt, case.M, case.N, case.K)), dtype=torch.uint8, device=dev)
    fn = lambda i: mm(W, q, d, s, case.N, case.K, out=out, workspace=ws)
    fn(0)
    us = _time_rotating(fn, 1, args.steps)
    print(json.dumps({"case": case.name, "fmt": case.fmt, "M": case.M, "N": case.N, "K": case.K,
                      "calls": args.steps, "us": round(us, 2), "TOPS": round(case.ops / (us * 1e-6) / 1e12, 2)}),
          flush=True)


def run_copy_calibration(args):
    """A plain device copy of known size, to scale FETCH_SIZE / WRITE_SIZE."""
    import torch
    n = 256 << 20
    a = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(args.steps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": args.steps}))


def run_ceilings(args):
    """The hardware ceilings the kernels are judged against, from the probes
    in libmq_probes.so (GPU time per launch, queued behind busy work):
      * read stream: the best of grid-stride register loads (4, 8 or 16 in
        flight per lane) and an LDS-DMA ring (2, 4 or 8 slots per wavefront)
        over 1024-8192 workgroups, for byte counts of the decode matrices
        (Q4_K 18944 x 3584, Q6_K 3584 x 18944, the Q6_K output head) and
        1 GiB, each read from rotating copies in a 2 GiB pool;
      * int8 MFMA with k f32 VALU operations per int32 result (k = 0: the
        MFMAs alone; 3: convert, scale product, fma, as the GEMM epilogue);
      * the GEMM's sub-block step with operands from LDS on the f16 matrix
        cores (scale folded into the weights, one fma per result; with the
        weights and then the activations also converted in registers)
        against the same step on the int8 matrix cores;
      * the VALU issue rate per SIMD at 1, 2 and 4 wavefronts per SIMD, for
        f32 epilogue mixes alone and beside independent MFMAs, with the
        shader clock each wavefront ran at.
    --part read|mix|valu runs one of the three groups."""
    import ctypes
    import numpy as np
    import torch

    from quant_gemm_amd import build as mq_build
    if not os.path.exists(mq_build.PROBES_LIB):
        raise RuntimeError(f"{mq_build.PROBES_LIB} is not built (python -m quant_gemm_amd.build)")
    P = ctypes.CDLL(mq_build.PROBES_LIB)
    P.mqp_read.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                           ctypes.c_void_p, ctypes.c_void_p]
    P.mqp_read.restype = ctypes.c_int
    P.mqp_mix.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    P.mqp_mix.restype = ctypes.c_int
    P.mqp_valu.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    P.mqp_valu.restype = ctypes.c_int
    parts = ("read", "mix", "valu") if not args.part else (args.part,)
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    sink = torch.zeros(16, dtype=torch.int32, device="cuda")
    pool_bytes = 2 << 30
    pool = torch.empty(pool_bytes, dtype=torch.uint8, device="cuda")

    def check(rc):
        if rc != 0:
            raise RuntimeError(f"probe launch failed: hipError {rc}")

    sizes = [("Q4_K 18944 x 3584", 18944 * 14 * 144), ("Q6_K 3584 x 18944", 3584 * 74 * 210),
             ("Q6_K head 152064 x 3584", 152064 * 14 * 210), ("1 GiB", 1 << 30)]
    for name, nbytes in sizes if "read" in parts else ():
        copies = max(2, pool_bytes // nbytes)
        ptr = lambda i: ctypes.c_void_p(pool.data_ptr() + (i % copies) * nbytes)
        reps = max(20, 2 * copies)
        best = None
        for kind, depths in ((0, (4, 8, 16)), (1, (2, 4, 8))):
            for depth in depths:
                for grid in (1024, 2048, 4096, 8192):
                    fn = lambda i: check(P.mqp_read(kind, depth, ptr(i), nbytes, grid, ctypes.c_void_p(sink.data_ptr()), st))
                    us = _time_rotating(fn, copies, reps)
                    if best is None or us < best[0]:
                        best = (us, kind, depth, grid)
        _, kind, depth, grid = best
        fn = lambda i: check(P.mqp_read(kind, depth, ptr(i), nbytes, grid, ctypes.c_void_p(sink.data_ptr()), st))
        us = float(np.median([_time_rotating(fn, copies, reps) for _ in range(3)]))
        row = {"probe": "read", "case": name, "bytes": nbytes, "us": round(us, 2),
               "GBs": round(nbytes / (us * 1e-6) / 1e9, 1), "frac_hbm": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 3),
               "best": {"pattern": ["register loads", "LDS-DMA ring"][kind], "depth": depth, "workgroups": grid}}
        print(json.dumps(row), flush=True)
    del pool
    torch.cuda.empty_cache()

    # 2048 workgroups: many wavefronts per SIMD; 512: two per SIMD, the
    # occupancy of the GEMMs. The fp8 kinds count the same int8-equivalent
    # work per MFMA (one 32 x 32 x 32 sub-block product).
    iters = 1000
    names = {0: "int8 MFMA alone", 2: "int8 MFMA + cvt, fma", 3: "int8 MFMA + cvt, mul, fma",
             4: "int8 MFMA + cvt, mul, mul, fma", 10: "fp8 MFMA alone", 11: "fp8 MFMA + fma",
             12: "fp8 MFMA + mul, fma", 20: "LDS step: f16 MFMA pair alone", 21: "LDS step: f16 MFMA pair + fma",
             22: "LDS step: f16 + fma, weights converted", 23: "LDS step: f16 + fma, weights and activations converted",
             30: "LDS step: int8 MFMA + unpack, cvt, mul, fma"}
    for grid in (2048, 512) if "mix" in parts else ():
        out = torch.zeros(grid * 256, dtype=torch.float32, device="cuda")
        ops = grid * 4 * iters * 4 * 2 * 32 * 32 * 32
        for k in (0, 2, 3, 4, 10, 11, 12, 20, 21, 22, 23, 30):
            fn = lambda i: check(P.mqp_mix(k, iters, grid, ctypes.c_void_p(out.data_ptr()), st))
            us = float(np.median([_time_rotating(fn, 1, 5) for _ in range(3)]))
            tops = ops / (us * 1e-6) / 1e12
            row = {"probe": "MFMA + VALU ops per result", "kind": names[k], "k": k, "workgroups": grid,
                   "us": round(us, 1), "TOPS": round(tops, 1), "frac_int8_peak": round(tops / INT8_PEAK_TOPS, 3)}
            print(json.dumps(row), flush=True)

    # VALU issue rate. Per iteration and wavefront the probe loops issue
    # (counted in their gfx950 code): k = 0: 15 fma + 2 add; 1: 16 cvt,
    # 16 integer add, 16 fma, 1 add; 2: 14 mul, 16 fma, 1 add; 3 and 7-9:
    # 16 cvt, 15 mul, 16 fma, 16 integer add, 1 add, plus the MFMAs of 7-9.
    # 256 workgroups of 4 wavefronts put one wavefront on each of the 1024
    # SIMDs; 512 two, 1024 four.
    vnames = {0: "fma", 1: "cvt, fma", 2: "mul, fma", 3: "cvt, mul, fma (the GEMM epilogue)",
              7: "epilogue mix + 1 int8 MFMA", 8: "epilogue mix + 2 int8 MFMA", 9: "epilogue mix + 1 bf16 MFMA"}
    per_iter = {0: 17, 1: 49, 2: 31, 3: 64, 7: 64, 8: 64, 9: 64}
    viters = 20000
    for k in (0, 1, 2, 3, 7, 8, 9) if "valu" in parts else ():
        for wps in (1, 2, 4):
            grid = 256 * wps
            out = torch.zeros(grid * 256, dtype=torch.float32, device="cuda")
            cyc = torch.zeros(grid * 4, dtype=torch.int64, device="cuda")
            fn = lambda i: check(P.mqp_valu(k, viters, grid, ctypes.c_void_p(out.data_ptr()),
                                            ctypes.c_void_p(cyc.data_ptr()), st))
            us = float(np.median([_time_rotating(fn, 1, 3) for _ in range(3)]))
            wave_cycles = cyc.double().mean().item()
            n = per_iter[k] * viters            # VALU instructions per wavefront
            row = {"probe": "VALU issue", "kind": vnames[k], "k": k, "waves_per_simd": wps,
                   "us": round(us, 1), "clock_GHz": round(wave_cycles / (us * 1e3), 3),
                   "valu_per_ns_per_simd": round(n * wps / (us * 1e3), 3),
                   "cycles_per_valu_per_wave": round(wave_cycles / n, 2)}
            print(json.dumps(row), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--all", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--ceilings", action="store_true", help="read-stream and MFMA/VALU probes")
    ap.add_argument("--case", help="time one named workload's matmul (a profiling target)")
    ap.add_argument("--part", choices=("read", "mix", "valu"), help="with --ceilings: one probe group")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus}: this benchmark measures one GPU only; the multi-GPU "
              "path is a design (N-sharded weights), not an implementation", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        run_copy_calibration(args)
    elif args.ceilings:
        run_ceilings(args)
    elif args.case:
        run_case(args)
    elif args.all:
        run_all(args)
    else:
        run_contract(args)


if __name__ == "__main__":
    main()
