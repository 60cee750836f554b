"""Benchmark of the verification / logit-fusion pass on one MI355X.

One step = one ``asym_verify`` call over the large batched AsymSpec workload
(B=256 requests, K=4 drafts -> 1280 rows of a, b, t, V=151936, bf16), with
inputs resident in HBM.  Prints one JSON line: verified logit rows/s; the
dominant kernel's roofline (algorithmic HBM bytes per launch over its
event-timed duration, against 8 TB/s, with the measured traffic of the
committed counter summary while the kernel sources still match it, and its
VALU issue from the committed SQ summary); as secondary figures the B=64/K=2
workload, the RAPID pass, the AsymSpec ablation variants on the large
workload, the cross-family pass, the fused LM-head pass (against the bf16
matrix-core peak) and the E2-SCI adaptive acceptance on B=64 and B=1
windows; and the
fp64 CPU oracle timed on the host as a reported baseline.

Before each measurement's warmup the device's clocks are settled with
--settle seconds (default 0.3; 0 turns it off) of the read-only streaming
kernel, untimed, since host-side setup leaves the compute units idle long
enough for the clocks to drop; the line reports the figure used.

    python bench.py [--gpus 1] [--steps 200] [--warmup 20] [--no-cpu-baseline]
                    [--no-extra] [--calib-copy] [--settle S]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "verified logit rows/s (B·(K+1)·V) and achieved HBM GB/s vs peak, 1 GPU"
PEAK_HBM_GBS = 8000.0
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "asym_rows_kernel_bf16_B256_K4_V151936_traffic.txt")
VALU_SUMMARY = os.path.join(ROOT, "profiles", "asym_rows_kernel_bf16_B256_K4_V151936_valu.txt")


def _say(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def _device_inputs(vwl, x, copies=1):
    import torch
    sets = []
    base = [vwl.to_device_logits(getattr(x, n), x.dtype) for n in ("a", "b", "t")]
    draft = torch.from_numpy(x.draft).cuda()
    for c in range(copies):
        sets.append(([t.clone() for t in base] if c else base, draft))
    return sets


def _events(n):
    import torch
    return [torch.cuda.Event(enable_timing=True) for _ in range(n)]


SETTLE_S = 0.3  # default seconds of clock settling before each measurement's warmup
_settle_cfg = {"seconds": SETTLE_S}
_settle_state = {}


def settle_clocks(seconds=None):
    """Bring the device to its working clocks before a measurement: the
    read-only streaming kernel (libvwl_bench.so) over a 256 MiB buffer,
    relaunched for `seconds` of wall time, untimed.  Host-side setup before a
    measurement (input copies) leaves the compute units idle long enough for
    the clocks to drop, and a short timed burst would otherwise run partly
    at lower clocks.  Nothing of the measured call runs here."""
    import ctypes
    import time
    import torch
    import vocab_wide_logit_amd as vwl
    seconds = _settle_cfg["seconds"] if seconds is None else seconds
    if seconds <= 0:
        return
    st = _settle_state
    if not st:
        lib = ctypes.CDLL(os.path.join(os.path.dirname(vwl.LIB_PATH), "libvwl_bench.so"))
        lib.vwl_bench_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                              ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
        st["lib"] = lib
        st["buf"] = torch.zeros(64 << 20, dtype=torch.int32, device="cuda")
        st["sink"] = torch.zeros(1, dtype=torch.int32, device="cuda")
    lib, buf, sink = st["lib"], st["buf"], st["sink"]
    stream = torch.cuda.current_stream()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    threads, per_cu, unroll = STREAM_SHAPES[-1]
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(40):
            rc = lib.vwl_bench_stream_read(buf.data_ptr(), buf.numel() * 4, sink.data_ptr(), per_cu * cus, threads,
                                           unroll, stream.cuda_stream)
            if rc != 0:
                raise RuntimeError("stream reference launch failed: %d" % rc)
        torch.cuda.synchronize()


def time_asym(vwl, x, steps, warmup, copies=1, delta="a-b", gate="cda"):
    """asym_verify calls (asym_verify_variant for another fusion source or
    gate) on torch's current stream (the stream the library launches on),
    each bracketed by events, with the library recording a third event right
    after the row kernel.  Returns (wall seconds, per-call ms, per-call
    row-kernel ms)."""
    import torch
    sets = _device_inputs(vwl, x, copies)
    B, K = x.B, x.K
    out = vwl.asym_out(B, K, "cuda")
    stream = torch.cuda.current_stream()
    ws = vwl._workspace(0, B, K, x.V, vwl.VWL_BF16 if x.dtype == "bf16" else vwl.VWL_F32,
                        torch.device("cuda", torch.cuda.current_device()), stream.cuda_stream)
    def call(a, b, t, d):
        if delta == "a-b" and gate == "cda":
            vwl.asym_verify(a, b, t, d, x.beta, x.gamma, out=out, workspace=ws)
        else:
            vwl.asym_verify_variant(a, b, t, d, x.beta, x.gamma, delta, gate, out=out, workspace=ws)

    settle_clocks()
    for i in range(warmup):
        (a, b, t), d = sets[i % copies]
        call(a, b, t, d)
    start, mid, end = _events(steps), _events(steps), _events(steps)
    for e in mid:
        e.record(stream)  # creates the underlying HIP event
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        (a, b, t), d = sets[i % copies]
        start[i].record(stream)
        vwl.set_phase_event(mid[i])
        call(a, b, t, d)
        end[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    vwl.set_phase_event(None)
    per = [s.elapsed_time(e) for s, e in zip(start, end)]
    rows = [s.elapsed_time(m) for s, m in zip(start, mid)]
    if int(out.dev_err.cpu()[0]) != 0:
        raise RuntimeError("device error bits set: %d" % int(out.dev_err.cpu()[0]))
    return wall, per, rows


def time_rapid(vwl, x, steps, warmup, copies=4):
    """rapid_verify calls rotating `copies` input sets (four sets of the
    B=16 workload are 722 MB, past the 256 MB last-level cache, so each call
    reads its rows from HBM); per-call and row-kernel ms from events."""
    import torch
    base = (vwl.to_device_logits(x.z, x.dtype), vwl.to_device_logits(x.y, x.dtype))
    sets = [base] + [tuple(t.clone() for t in base) for _ in range(1, copies)]
    d = torch.from_numpy(x.draft).cuda()
    ua = torch.from_numpy(x.u_accept).cuda()
    us = torch.from_numpy(x.u_sample).cuda()
    out = vwl.rapid_out(x.B, x.G, x.V, "cuda")
    settle_clocks()
    for i in range(warmup):
        z, y = sets[i % copies]
        vwl.rapid_verify(z, y, d, ua, us, x.eta, x.T, out=out)
    stream = torch.cuda.current_stream()
    start, mid, end = _events(steps), _events(steps), _events(steps)
    for e in mid:
        e.record(stream)
    torch.cuda.synchronize()
    for i in range(steps):
        z, y = sets[i % copies]
        start[i].record(stream)
        vwl.set_phase_event(mid[i])
        vwl.rapid_verify(z, y, d, ua, us, x.eta, x.T, out=out)
        end[i].record(stream)
    torch.cuda.synchronize()
    vwl.set_phase_event(None)
    return ([s.elapsed_time(e) for s, e in zip(start, end)],
            [s.elapsed_time(m) for s, m in zip(start, mid)])


def time_e2sci(vwl, x, steps, warmup, copies=4):
    """e2sci_verify calls with the state carried on the device (thresholds
    updated in place), rotating `copies` input sets; per-call and row-kernel
    ms from events, as for the AsymSpec pass."""
    import torch
    sets = [(vwl.to_device_logits(x.y, x.dtype), vwl.to_device_logits(x.z, x.dtype))]
    for _ in range(1, copies):
        sets.append(tuple(t.clone() for t in sets[0]))
    T = torch.from_numpy(x.T.copy()).cuda()
    om = torch.from_numpy(x.omega.copy()).cuda()
    rh = torch.from_numpy(x.r_hat.copy()).cuda()
    prm = vwl.E2sciParams()
    out = vwl.e2sci_out(x.B, x.W, "cuda")
    settle_clocks()
    for i in range(warmup):
        y, z = sets[i % copies]
        vwl.e2sci_verify(y, z, T, om, rh, prm, T_out=T, out=out)
    stream = torch.cuda.current_stream()
    start, mid, end = _events(steps), _events(steps), _events(steps)
    for e in mid:
        e.record(stream)
    torch.cuda.synchronize()
    for i in range(steps):
        y, z = sets[i % copies]
        start[i].record(stream)
        vwl.set_phase_event(mid[i])
        vwl.e2sci_verify(y, z, T, om, rh, prm, T_out=T, out=out)
        end[i].record(stream)
    torch.cuda.synchronize()
    vwl.set_phase_event(None)
    return ([s.elapsed_time(e) for s, e in zip(start, end)],
            [s.elapsed_time(m) for s, m in zip(start, mid)])


def time_xfam(vwl, x, steps, warmup, copies=4):
    """asym_verify_xfam calls rotating `copies` input sets; per-call and
    row-pass ms (the event after the drafter and verifier passes)."""
    import torch
    base = [vwl.to_device_logits(getattr(x, n), x.dtype) for n in ("a", "b", "t")]
    sets = [base] + [[t.clone() for t in base] for _ in range(1, copies)]
    vm = torch.from_numpy(x.vmap).cuda()
    d = torch.from_numpy(x.draft).cuda()
    out = vwl.asym_out(x.B, x.K, "cuda")
    settle_clocks()
    for i in range(warmup):
        a, b, t = sets[i % copies]
        vwl.asym_verify_xfam(a, b, t, vm, d, x.beta, x.gamma, out=out)
    stream = torch.cuda.current_stream()
    start, mid, end = _events(steps), _events(steps), _events(steps)
    for e in mid:
        e.record(stream)
    torch.cuda.synchronize()
    for i in range(steps):
        a, b, t = sets[i % copies]
        start[i].record(stream)
        vwl.set_phase_event(mid[i])
        vwl.asym_verify_xfam(a, b, t, vm, d, x.beta, x.gamma, out=out)
        end[i].record(stream)
    torch.cuda.synchronize()
    vwl.set_phase_event(None)
    return ([s.elapsed_time(e) for s, e in zip(start, end)],
            [s.elapsed_time(m) for s, m in zip(start, mid)])


PEAK_BF16_TFLOPS = 2500.0  # dense bf16 matrix-core peak of one MI355X


def time_lmhead(vwl, x, steps, warmup, store_pairs=True):
    """asym_verify_lmhead calls on resident hidden states and heads; per-call
    ms and the ms up to the end of the last GEMM pass (the path that stores
    the (a, b) pairs, or with store_pairs=False the one that forms a and b
    twice)."""
    import numpy as np
    import torch
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).cuda()
    ha, hb, Wd, ht, Wt = bf(x.h_a), bf(x.h_b), bf(x.W_d), bf(x.h_t), bf(x.W_t)
    d = torch.from_numpy(x.draft).cuda()
    out = vwl.asym_out(x.B, x.K, "cuda")
    settle_clocks()
    for _ in range(warmup):
        vwl.asym_verify_lmhead(ha, hb, Wd, ht, Wt, d, x.beta, x.gamma, out=out, store_pairs=store_pairs)
    stream = torch.cuda.current_stream()
    start, mid, end = _events(steps), _events(steps), _events(steps)
    for e in mid:
        e.record(stream)
    torch.cuda.synchronize()
    for i in range(steps):
        start[i].record(stream)
        vwl.set_phase_event(mid[i])
        vwl.asym_verify_lmhead(ha, hb, Wd, ht, Wt, d, x.beta, x.gamma, out=out, store_pairs=store_pairs)
        end[i].record(stream)
    torch.cuda.synchronize()
    vwl.set_phase_event(None)
    return ([s.elapsed_time(e) for s, e in zip(start, end)],
            [s.elapsed_time(m) for s, m in zip(start, mid)])


def oracle_rows_per_s(fn, rows):
    """The oracle timed once on a bounded sample of a workload (rows/s)."""
    t0 = time.perf_counter()
    fn()
    return rows / (time.perf_counter() - t0)


# Launch shapes of the streaming reference (threads, workgroups per CU,
# 16-byte loads in flight per thread); the best of them is reported.
STREAM_SHAPES = ((256, 2, 4), (256, 32, 8), (512, 32, 8), (512, 32, 16))


def stream_read_gbs(nbytes, reps=20):
    """HBM read rate of the hand-written read-only streaming kernel
    (libvwl_bench.so, 16-byte loads) over nbytes of device memory: the best
    median over a few launch shapes.  Returns (GB/s, shape)."""
    import ctypes
    import torch
    import vocab_wide_logit_amd as vwl
    lib = ctypes.CDLL(os.path.join(os.path.dirname(vwl.LIB_PATH), "libvwl_bench.so"))
    lib.vwl_bench_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                          ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    buf = torch.empty(nbytes // 4, dtype=torch.int32, device="cuda").random_()
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    best = (0.0, None)
    for threads, per_cu, unroll in STREAM_SHAPES:
        def go():
            rc = lib.vwl_bench_stream_read(buf.data_ptr(), nbytes, sink.data_ptr(), per_cu * cus, threads, unroll,
                                           stream.cuda_stream)
            if rc != 0:
                raise RuntimeError("stream reference launch failed: %d" % rc)
        for _ in range(3):
            go()
        ev = _events(reps + 1)
        for i in range(reps):
            ev[i].record(stream)
            go()
        ev[reps].record(stream)
        torch.cuda.synchronize()
        ms = _median([ev[i].elapsed_time(ev[i + 1]) for i in range(reps)])
        gbs = nbytes / (ms * 1e-3) / 1e9
        if gbs > best[0]:
            best = (gbs, {"threads": threads, "workgroups": per_cu * cus, "loads_in_flight": unroll,
                          "bytes": nbytes, "median_ms": ms})
    del buf
    return best


def calib_copy():
    """The plain copy of known size that the counter runs scale by."""
    import torch
    from vocab_wide_logit_amd import profiling
    n = profiling.COPY_BYTES // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst


def _median(v):
    v = sorted(v)
    return v[len(v) // 2]


def _pct(v, q):
    v = sorted(v)
    return v[min(len(v) - 1, int(q * len(v)))]


def cpu_baseline(x, runs=3):
    """The fp64 oracle as it stands, on all host cores, over the same call."""
    import oracle
    oracle.build(force=False)
    times = []
    for _ in range(runs):
        t0 = time.perf_counter()
        oracle.asym(x.a, x.b, x.t, x.draft, x.beta, x.gamma, x.dtype)
        times.append(time.perf_counter() - t0)
    t = _median(times)
    rows = x.B * (x.K + 1)
    # one thread on a bounded sample (the first 8 requests)
    n = 8
    t0 = time.perf_counter()
    oracle.asym(x.a[:n], x.b[:n], x.t[:n], x.draft[:n], x.beta, x.gamma, x.dtype, nthreads=1)
    t1 = time.perf_counter() - t0
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    return {"value": rows / t, "unit": "rows/s", "cores": oracle.max_threads(), "kind": "oracle",
            "sample": "the full B=%d, K=%d, V=%d %s call (%d rows), median of %d runs (%.2f s each)" % (
                x.B, x.K, x.V, x.dtype, rows, runs, t),
            "one_thread_rows_per_s": n * (x.K + 1) / t1, "one_thread_sample": "the first %d requests" % n,
            "nproc": os.cpu_count(), "cpu_model": model}


def graph_call_ms(fn, steps, warmup):
    """Per-call device time of `fn` captured once in a HIP graph and replayed:
    each replay bracketed by events on the current stream, so the host's
    per-call cost (argument checks, launches) is outside the timed span.
    The call must allocate nothing (outputs and workspace given)."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(2):
            fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        fn()
    torch.cuda.synchronize()
    settle_clocks()
    for _ in range(warmup):
        g.replay()
    stream = torch.cuda.current_stream()
    start, end = _events(steps), _events(steps)
    for e in start:
        e.record(stream)
    torch.cuda.synchronize()
    for i in range(steps):
        start[i].record(stream)
        g.replay()
        end[i].record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in zip(start, end)]


def prepared_call_ms(call, steps, warmup):
    """Per-call time of a prepared call (arguments checked and marshalled
    once): each invocation bracketed by events on the current stream."""
    import torch
    settle_clocks()
    for _ in range(warmup):
        call()
    stream = torch.cuda.current_stream()
    start, end = _events(steps), _events(steps)
    for e in start:
        e.record(stream)
    torch.cuda.synchronize()
    for i in range(steps):
        start[i].record(stream)
        call()
        end[i].record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in zip(start, end)]


def latency(vwl, x, steps, warmup, copies=4):
    """Per-call latency of asym_verify on a small workload: median and p10/p90
    over `steps` calls after `warmup`, rotating `copies` input sets, and the
    same call replayed from a captured graph (device time without the host's
    per-call cost).  These calls are bound by launch and synchronisation
    latency, not by bytes (the inputs are a few MB at most and stay in the
    last-level cache)."""
    import torch
    _, per, rows = time_asym(vwl, x, steps, warmup, copies=copies)
    (a, b, t), d = _device_inputs(vwl, x)[0]
    ws = torch.zeros(vwl.workspace_bytes("asym", x.B, x.K, x.V, a.dtype), dtype=torch.uint8, device="cuda")
    out = vwl.asym_out(x.B, x.K, "cuda")
    gper = graph_call_ms(lambda: vwl.asym_verify(a, b, t, d, x.beta, x.gamma, out=out, workspace=ws),
                         steps, warmup)
    pper = prepared_call_ms(vwl.asym_verify(a, b, t, d, x.beta, x.gamma, out=out, workspace=ws, prepare=True),
                            steps, warmup)
    return {"B": x.B, "K": x.K, "V": x.V, "logits": x.dtype, "median_call_us": _median(per) * 1e3,
            "p10_call_us": _pct(per, 0.1) * 1e3, "p90_call_us": _pct(per, 0.9) * 1e3,
            "median_row_kernel_us": _median(rows) * 1e3,
            "median_graph_call_us": _median(gper) * 1e3,
            "median_prepared_call_us": _median(pper) * 1e3,
            "bound": "latency (launches and the per-row exchange), inputs cache-resident"}


def e2sci_graph_call_ms(vwl, x, steps, warmup):
    """e2sci_verify of one input set replayed from a captured graph and as a
    prepared call, the state carried on the device (see graph_call_ms and
    prepared_call_ms); returns both lists."""
    import torch
    y, z = vwl.to_device_logits(x.y, x.dtype), vwl.to_device_logits(x.z, x.dtype)
    T = torch.from_numpy(x.T.copy()).cuda()
    om = torch.from_numpy(x.omega.copy()).cuda()
    rh = torch.from_numpy(x.r_hat.copy()).cuda()
    prm = vwl.E2sciParams()
    ws = torch.zeros(int(vwl.load_library().vwl_e2sci_workspace_bytes(x.B, x.W, x.V, vwl._dt(y))),
                     dtype=torch.uint8, device="cuda")
    out = vwl.e2sci_out(x.B, x.W, "cuda")
    g = graph_call_ms(lambda: vwl.e2sci_verify(y, z, T, om, rh, prm, T_out=T, out=out, workspace=ws),
                      steps, warmup)
    p = prepared_call_ms(vwl.e2sci_verify(y, z, T, om, rh, prm, T_out=T, out=out, workspace=ws, prepare=True),
                         steps, warmup)
    return g, p


def secondary(args, vwl, W, x, bytes_per_call):
    """The secondary measurements: single-request and tiny latency, the
    B=64/K=2 workload and RAPID B=16 (each rotating four input sets, so they
    read from HBM), the streaming reference, the ablation variants on the
    large inputs, the cross-family pass, the fused LM-head pass and the E2-SCI
    windows."""
    import torch
    _say("secondary: latency (B=1 and B=4), B=64 K=2 bf16, RAPID B=16 G=10 fp32, stream reference, "
         "ablation variants, cross-family, LM-head, E2-SCI windows")
    out = {"latency": {}}
    for xs in (W.single_asym(), W.tiny_asym()):
        out["latency"][xs.name] = latency(vwl, xs, args.steps, args.warmup)
    x2 = W.batched_asym()
    _, per2, rows2 = time_asym(vwl, x2, args.steps, args.warmup, copies=4)
    ms2 = _median(per2)
    b2 = x2.algorithmic_bytes()
    r3 = W.rapid_c3()
    per3, rows3 = time_rapid(vwl, r3, args.steps, args.warmup, copies=4)
    ms3 = _median(per3)
    b3 = r3.algorithmic_bytes()
    out["stream_read_gbs"], out["stream_read_shape"] = stream_read_gbs(bytes_per_call)
    # the ablation variants on the large inputs (bytes actually read: the
    # fixed gate with delta = t - b skips a)
    variants = {}
    for delta, gate in (("a", "cda"), ("t-b", "cda"), ("a-b", "fixed"), ("a", "fixed"), ("t-b", "fixed")):
        _, pv, rv = time_asym(vwl, x, args.steps, args.warmup, delta=delta, gate=gate)
        nbytes = bytes_per_call * (2 if (delta, gate) == ("t-b", "fixed") else 3) // 3
        mr = _median(rv)
        variants["delta=%s,gate=%s" % (delta, gate)] = {
            "median_call_ms": _median(pv), "median_row_kernel_ms": mr,
            "row_kernel_gbs": nbytes / (mr * 1e-3) / 1e9,
            "plan": vwl.asym_plan_info(x.B, x.K, x.V, torch.bfloat16, delta, gate)}
    out["variants"] = variants
    sec = {
        x2.name: {"rows_per_s": x2.B * (x2.K + 1) / (ms2 * 1e-3), "median_call_ms": ms2,
                  "median_row_kernel_ms": _median(rows2), "input_sets": 4,
                  "gbs": b2 / (ms2 * 1e-3) / 1e9, "frac_of_peak": b2 / (ms2 * 1e-3) / 1e9 / PEAK_HBM_GBS},
        r3.name: {"rows_per_s": r3.B * (r3.G + 1) / (ms3 * 1e-3), "median_call_ms": ms3,
                  "median_row_kernel_ms": _median(rows3), "input_sets": 4,
                  "gbs": b3 / (ms3 * 1e-3) / 1e9, "frac_of_peak": b3 / (ms3 * 1e-3) / 1e9 / PEAK_HBM_GBS,
                  "row_kernel_gbs": b3 / (_median(rows3) * 1e-3) / 1e9, "eta": r3.eta},
    }
    xf = W.xfam_batched()
    pf, rf = time_xfam(vwl, xf, args.steps, args.warmup)
    mf, mrf = _median(pf), _median(rf)
    bf = xf.algorithmic_bytes()
    sec[xf.name] = {
        "rows_per_s": xf.B * (xf.K + 1) / (mf * 1e-3), "median_call_ms": mf, "median_row_passes_ms": mrf,
        "input_sets": 4, "gbs": bf / (mrf * 1e-3) / 1e9, "frac_of_peak": bf / (mrf * 1e-3) / 1e9 / PEAK_HBM_GBS}
    xl = W.lmhead_batched()
    pl, rl = time_lmhead(vwl, xl, min(args.steps, 50), min(args.warmup, 5))
    ml = _median(pl)
    Rl = xl.B * (xl.K + 1)
    # algorithmic work: the three products once, each head read once (the
    # launches form each product once); the stored (a, b) pairs add
    # 8 R V bytes written and read
    flops = 2.0 * Rl * xl.V * (2 * xl.Hd + xl.Ht)
    wbytes = float(xl.weight_bytes())
    bound_ms = max(flops / (PEAK_BF16_TFLOPS * 1e12), wbytes / (PEAK_HBM_GBS * 1e9)) * 1e3
    sec[xl.name] = {
        "rows_per_s": Rl / (ml * 1e-3), "median_call_ms": ml, "median_gemm_pass_ms": _median(rl),
        "tflops": flops / (ml * 1e-3) / 1e12, "frac_of_bf16_peak": flops / (ml * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "head_weight_gbs": wbytes / (ml * 1e-3) / 1e9,
        "roofline_bound_ms": bound_ms, "frac_of_roofline": bound_ms / ml,
        "flops_per_call": flops, "pair_bytes_per_call": 2.0 * 8 * Rl * xl.V}
    # the path with no pair storage (minimal workspace): a and b formed twice
    pn, rn = time_lmhead(vwl, xl, min(args.steps, 20), min(args.warmup, 3), store_pairs=False)
    mn = _median(pn)
    sec[xl.name]["no_pair_storage"] = {
        "median_call_ms": mn, "median_gemm_passes_ms": _median(rn), "tflops": flops / (mn * 1e-3) / 1e12,
        "executed_flops_per_call": flops + 2.0 * Rl * xl.V * 2 * xl.Hd, "frac_of_roofline": bound_ms / mn}
    for xe in (W.e2sci_batched(), W.e2sci_single()):
        pe, re_ = time_e2sci(vwl, xe, args.steps, args.warmup)
        me, mre = _median(pe), _median(re_)
        be = xe.algorithmic_bytes()
        sec[xe.name] = {
            "rows_per_s": xe.B * xe.W / (me * 1e-3), "median_call_ms": me, "median_row_kernel_ms": mre,
            "input_sets": 4, "row_kernel_gbs": be / (mre * 1e-3) / 1e9,
            "frac_of_peak": be / (mre * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "plan": vwl.e2sci_plan_info(xe.B, xe.W, xe.V, torch.bfloat16)}
        if xe.B == 1:
            g, pc = e2sci_graph_call_ms(vwl, xe, args.steps, args.warmup)
            sec[xe.name]["median_graph_call_ms"] = _median(g)
            sec[xe.name]["median_prepared_call_ms"] = _median(pc)
    out["secondary"] = sec
    out["inputs"] = (x2, r3, xf, xl)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the secondary workloads")
    ap.add_argument("--settle", type=float, default=SETTLE_S,
                    help="seconds of untimed streaming before each measurement's warmup (0: none)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run the 1 GiB copy that counter summaries are scaled by")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(requests are independent; sharding is by requests or by vocabulary "
              "slices, described in the design notes). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    _settle_cfg["seconds"] = max(0.0, args.settle)

    import numpy as np
    import torch
    import vocab_wide_logit_amd as vwl
    import workloads as W
    from vocab_wide_logit_amd import profiling

    torch.cuda.set_device(0)
    vwl.load_library()
    if args.calib_copy:
        _say("calibration copy of %d bytes" % profiling.COPY_BYTES)
        calib_copy()
    _say("generating B=256 K=4 V=151936 bf16 inputs")
    x = W.large_asym()
    rows = x.B * (x.K + 1)
    bytes_per_call = x.algorithmic_bytes()
    plan = vwl.plan_info("asym", x.B, x.K, x.V, torch.bfloat16)
    extra = None
    if not args.no_extra:
        # The secondary workloads run first: they are measurements of their
        # own, and the headline is then timed on a GPU at its working clocks.
        extra = secondary(args, vwl, W, x, bytes_per_call)
    _say("plan %s; timing %d steps after %d warmup" % (plan, args.steps, args.warmup))
    wall, per, rows_ms = time_asym(vwl, x, args.steps, args.warmup)
    ms_step = wall * 1e3 / args.steps
    ms_rows = sum(rows_ms) / len(rows_ms)
    ms_call = sum(per) / len(per)
    achieved = bytes_per_call / (ms_rows * 1e-3) / 1e9
    traffic = profiling.read_traffic(TRAFFIC_SUMMARY, "asym")
    result = {
        "metric": METRIC,
        "value": rows * args.steps / wall,
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "clock_settle_s": _settle_cfg["seconds"],
        "config": {"workload": x.name, "B": x.B, "K": x.K, "V": x.V, "logits": "bf16",
                   "beta": x.beta, "gamma": x.gamma, "rows_per_step": rows,
                   "identical_rows": 0.2, "tie_rows": 0.05, "plan": plan},
        "tokens_verified_per_s": x.B * x.K * args.steps / wall,
        "call_ms": {"mean": ms_call, "median": _median(per), "p10": _pct(per, 0.1), "p90": _pct(per, 0.9)},
        "hbm_gbs_per_call": bytes_per_call / (ms_call * 1e-3) / 1e9,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": traffic,
                     "kernel": "asym_rows_kernel<bf16,%d>" % plan["vec_per_thread"],
                     "bytes_per_launch": bytes_per_call, "avg_launch_ms": ms_rows,
                     "p10_ms": _pct(rows_ms, 0.1), "p90_ms": _pct(rows_ms, 0.9)},
    }
    valu = profiling.read_summary(VALU_SUMMARY, "asym")
    if valu is not None:
        # the kernel's co-bound: VALU issue, from the committed SQ counter run
        result["roofline"]["valu"] = {
            "busy": float(valu["valu_busy"]), "insts_per_launch": float(valu["SQ_INSTS_VALU"]),
            "floor_ms_at_full_issue": float(valu["valu_cycles_per_simd"]) / 2.4e9 * 1e3,
            "source": os.path.relpath(VALU_SUMMARY, ROOT)}
    if extra is not None:
        result["variants_" + x.name] = extra["variants"]
        result["stream_read_gbs"] = extra["stream_read_gbs"]
        result["stream_read_shape"] = extra["stream_read_shape"]
        result["roofline"]["frac_of_stream"] = achieved / extra["stream_read_gbs"]
        result["latency"] = extra["latency"]
        result["secondary"] = extra["secondary"]
        x2, r3, xf, xl = extra["inputs"]
    if not args.no_cpu_baseline:
        _say("timing the fp64 oracle on the host")
        result["cpu_baseline"] = cpu_baseline(x)
        if not args.no_extra:
            # the oracle beside each secondary pass, on a bounded sample
            # (the first 8 requests of each workload)
            import oracle
            n = 8
            sl = lambda v: np.ascontiguousarray(v[:n])
            sec = result["secondary"]
            sec[x2.name]["cpu_oracle_rows_per_s"] = oracle_rows_per_s(
                lambda: oracle.asym(sl(x2.a), sl(x2.b), sl(x2.t), sl(x2.draft), x2.beta, x2.gamma, x2.dtype),
                n * (x2.K + 1))
            sec[r3.name]["cpu_oracle_rows_per_s"] = oracle_rows_per_s(
                lambda: oracle.rapid(sl(r3.z), sl(r3.y), sl(r3.draft), sl(r3.u_accept), sl(r3.u_sample),
                                     r3.eta, r3.T, r3.dtype), n * (r3.G + 1))
            for key, v in result["variants_" + x.name].items():
                delta, gate = key.replace("delta=", "").replace("gate=", "").split(",")
                v["cpu_oracle_rows_per_s"] = oracle_rows_per_s(
                    lambda: oracle.asym(sl(x.a), sl(x.b), sl(x.t), sl(x.draft), x.beta, x.gamma, x.dtype,
                                        delta=delta, gate=gate), n * (x.K + 1))
            sec[xf.name]["cpu_oracle_rows_per_s"] = oracle_rows_per_s(
                lambda: oracle.asym_xfam(sl(xf.a), sl(xf.b), sl(xf.t), xf.vmap, sl(xf.draft), xf.beta, xf.gamma,
                                         xf.dtype), n * (xf.K + 1))
            m2 = 2
            sec[xl.name]["cpu_oracle_rows_per_s"] = oracle_rows_per_s(
                lambda: oracle.asym_lmhead(xl.h_a[:m2], xl.h_b[:m2], xl.W_d, xl.h_t[:m2], xl.W_t, xl.draft[:m2],
                                           xl.beta, xl.gamma), m2 * (xl.K + 1))
            for xe in (W.e2sci_batched(), W.e2sci_single()):
                m = min(n, xe.B)
                sec[xe.name]["cpu_oracle_rows_per_s"] = oracle_rows_per_s(
                    lambda: oracle.e2sci(xe.y[:m], xe.z[:m], xe.T[:m], xe.omega[:m], xe.r_hat[:m],
                                         dtype=xe.dtype), m * xe.W)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
