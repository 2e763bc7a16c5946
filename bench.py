#!/usr/bin/env python3
"""Benchmark of the planned GEMM on one MI355X.

One step is one dg_gemm call on the int8 4096^3 workload (plan from the
handle's cache, the tiled MFMA kernel, the fused epilogue): the workload the
headline throughput is quoted on.  The other workloads (fp16 4096^3, the bf16
M = 1 and M = 16 long-K GEMMs, the GELU GEMM, the e2m1 GEMMs, the small alpha/beta
GEMM, the MX fp8 x e2m1 GEMM through dg_gemm_mx and the MX quantiser through
dg_quant_mx) are timed after it, each after at least W warm-up steps and 50 ms
of untimed launches, and reported under "workloads".  Inputs are seeded
synthetic data drawn on the GPU and resident in HBM before any timing starts.

Timing: HIP events on the stream the kernels run on (torch's current stream),
bracketing K back-to-back steps after W warm-up steps; ms_per_step is the
average and `value` the whole-job rate.  `repeats` times five more runs of K
steps (each run's time, the median and the minimum) and the median of 100
launches each bracketed by its own event pair (an isolated launch with its
overhead).  A step is one launch of the kernel, so the roofline's `achieved`
divides the algorithmic work by the kernel's average duration over the K timed
launches (in a kernel trace of the same command, the mean of those launches).
After an idle start the power management settles over about 10 ms, during which
launches run slower; the default warm-up runs past it, and runs that start
inside it (short warm-ups) show it in `repeats`.  `telemetry` records the engine clock
and the package power over a 3 s loop of the headline kernel, `plan` the
headline plan's shape and compiled resources.  The roofline's `traffic` is the
HBM bytes per launch recorded from rocprofv3 counters in
profiles/hbm_traffic.txt, reported only while the kernel sources still hash to
the recorded value.  Small HBM-bound workloads rotate through copies of B
(>= 576 MB in all, twice the L2 + MALL) so that every step reads HBM, and are
also reported warm; workloads whose kernels are shorter than the host's launch
cost are replayed from a captured HIP graph (checked against an eager run).

The CPU baseline is the oracle (plain C, binary64 / int64) timed on a bounded
sample of the headline workload on this host's cores.
"""
import argparse
import ctypes as C
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("TFLOP/s (TOPS int8) at 4096³ + GB/s at M=1 long-K, each as % of MI355X peak")
PEAK = {"i8": 5033.2, "f16": 2516.6, "bf16": 2516.6, "e2m1": 2516.6,   # dense TOP/s / TFLOP/s
        "mx": 5033.2}                                                  # (fp8: the MX MFMA's rate)
HBM_PEAK = 8000.0                                                      # GB/s
CACHE_BYTES = 576 * 10 ** 6       # 2 x (256 MB MALL + 32 MB L2)

HEADLINE = "i8_4096x4096x4096"
# Untimed warm-up of each further workload: at least --warmup steps and at least
# this long.  Under sustained load the clocks take tens of milliseconds to
# settle (the long-K streaming GEMMs run about 5 % faster after the first
# 30 ms); the headline keeps exactly --warmup steps.
WORKLOAD_WARM_S = 0.05
SECONDARY = ["f16_4096x4096x4096", "bf16_1x4096x131072", "bf16_16x4096x131072",
             "f16_2048x2048x8192_bias_gelu", "e2m1_4096x4096x4096", "e2m1_1x4096x4096",
             "bf16_1x256x12800", "f16_256x256x256_alpha_beta_d", "mx_4096x4096x4096",
             "mxq_4096x4096"]


def algorithmic(w):
    """(ops, bytes): 2*M*N*K, and every operand read once plus C written once."""
    M, N, K = w.M, w.N, w.K
    if w.path == "mxq":   # quantiser: binary16 in, one code byte and 1/32 scale byte out
        return 0, M * K * 2 + M * K + M * (K // 32)
    ops = 2 * M * N * K
    if w.path == "mx":
        return ops, M * K + K * N // 2 + (M + N) * (K // 32) + M * N * 2
    ea = 1 if w.path == "i8" else 2
    eb = {"i8": 1, "e2m1": 0.5}.get(w.path, 2)
    eo = {"i32": 4, "f32": 4}.get(w.out, 2)
    b = M * K * ea + K * N * eb + M * N * eo
    if w.path == "e2m1":
        b += N * (K // 32) * 2
    if w.beta != 0:
        b += M * N * eo
    if "bias" in w.epilogue:
        b += N * 2
    return ops, int(b)


class Prepared:
    """Device operands of one workload and a pre-marshalled dg_gemm call."""

    def __init__(self, h, name, dev, rotate):
        import torch
        from tile_planned_generator_amd import dg, synth
        self.dg = dg
        self.w = w = synth.make(name, device=dev)
        t = w.tensors
        self.torch_out = {"f16": torch.float16, "bf16": torch.bfloat16, "i32": torch.int32}[w.out]
        self.A = t["A"].contiguous()
        if w.path == "e2m1":
            B0 = dg.pack_e2m1(t["codes"])
            S0 = dg.scales_gn(t["scale"])
            b_bytes = B0.numel() + S0.numel() * 2
        else:
            B0 = t["B"].contiguous()
            S0 = None
            b_bytes = B0.numel() * B0.element_size()
        R = 1
        if rotate and b_bytes < CACHE_BYTES:
            R = -(-CACHE_BYTES // b_bytes)
        self.R = R
        self.Bs = [B0] + [B0.clone() for _ in range(R - 1)]
        self.Ss = [S0] + [S0.clone() for _ in range(R - 1)] if S0 is not None else [None] * R
        self.D = t.get("D") if w.beta != 0 else None
        self.bias = t.get("bias")
        self.C = torch.empty(w.M, w.N, dtype=self.torch_out, device=dev)
        layout = dg.DG_COL_MAJOR if w.path == "e2m1" else dg.DG_ROW_MAJOR
        a = {"i8": "i8", "e2m1": "f16"}.get(w.path, w.path)
        b = w.path
        self.info = h.plan(w.M, w.N, w.K, a, b, w.out, layout, w.epilogue)
        self.ws = (torch.empty(self.info.workspace_bytes, dtype=torch.uint8, device=dev)
                   if self.info.workspace_bytes else None)
        self.dt, self.lay = dg.Handle.problem(a, b, w.out, layout)
        if w.path == "i8":
            self.al, self.be = C.c_int32(int(w.alpha)), C.c_int32(int(w.beta))
        else:
            self.al, self.be = C.c_float(w.alpha), C.c_float(w.beta)
        self.epi = dg.dg_epilogue(dg.EPI[w.epilogue], dg.DTYPE[w.path if w.path != "e2m1" else "f16"]
                                  if self.bias is not None else 0,
                                  self.bias.data_ptr() if self.bias is not None else None, 1.0)
        self.stream = torch.cuda.current_stream().cuda_stream
        self.lib = dg.load()
        self.h = h
        self.args = []
        for i in range(R):
            self.args.append((h.h, w.M, w.N, w.K, C.byref(self.dt), C.byref(self.lay),
                              self.A.data_ptr(), self.Bs[i].data_ptr(),
                              self.Ss[i].data_ptr() if self.Ss[i] is not None else None,
                              32 if w.path == "e2m1" else 0,
                              self.D.data_ptr() if self.D is not None else None,
                              self.C.data_ptr(), C.byref(self.al), C.byref(self.be),
                              C.byref(self.epi), None,
                              self.ws.data_ptr() if self.ws is not None else None,
                              self.ws.numel() if self.ws is not None else 0, self.stream))

    def launch(self, i=0):
        s = self.lib.dg_gemm(*self.args[i % self.R])
        if s != 0:
            self.dg.check(s)


class PreparedMx:
    """Device operands of the MX workloads and a pre-marshalled dg_gemm_mx or
    dg_quant_mx call (the same interface as Prepared)."""

    def __init__(self, h, name, dev, rotate):
        import torch
        from tile_planned_generator_amd import dg, synth
        self.dg = dg
        self.w = w = synth.make(name, device=dev)
        t = w.tensors
        self.lib = dg.load()
        self.h = h
        self.stream = torch.cuda.current_stream().cuda_stream
        M, N, K = w.M, w.N, w.K
        G = K // 32
        if w.path == "mxq":
            X0 = t["X"].contiguous()
            per = X0.numel() * 2
            self.R = -(-CACHE_BYTES // per) if rotate and per < CACHE_BYTES else 1
            self.Xs = [X0] + [X0.clone() for _ in range(self.R - 1)]
            self.Qs = [torch.empty(M, K, dtype=torch.uint8, device=dev) for _ in range(self.R)]
            self.Ss = [torch.empty(G, M, dtype=torch.uint8, device=dev) for _ in range(self.R)]   # group-major
            self.C = self.Qs[0]
            self.info = None
            self.fn = self.lib.dg_quant_mx
            self.args = [(h.h, M, K, self.Xs[i].data_ptr(), K, self.Qs[i].data_ptr(), K,
                          self.Ss[i].data_ptr(), M, self.stream) for i in range(self.R)]
            return
        self.A = t["A"].contiguous()
        self.SA = t["SA"].t().contiguous()          # group-major [K/32][M]
        B0 = dg.pack_e2m1(t["codes"])
        S0 = t["SB"].contiguous()                   # group-major [K/32][N]
        per = B0.numel() + S0.numel()
        self.R = -(-CACHE_BYTES // per) if rotate and per < CACHE_BYTES else 1
        self.Bs = [B0] + [B0.clone() for _ in range(self.R - 1)]
        self.Ss = [S0] + [S0.clone() for _ in range(self.R - 1)]
        self.C = torch.empty(M, N, dtype=torch.float16, device=dev)
        self.info = h.plan(M, N, K, "f8e4m3", "e2m1", "f16", dg.DG_COL_MAJOR, w.epilogue, group_k=32)
        self.ws = (torch.empty(self.info.workspace_bytes, dtype=torch.uint8, device=dev)
                   if self.info.workspace_bytes else None)
        self.epi = dg.dg_epilogue(dg.EPI[w.epilogue], 0, None, 1.0)
        self.fn = self.lib.dg_gemm_mx
        self.args = [(h.h, M, N, K, self.A.data_ptr(), K, self.SA.data_ptr(), M, self.Bs[i].data_ptr(),
                      K, self.Ss[i].data_ptr(), N, self.C.data_ptr(), dg.DG_F16, N, C.c_float(w.alpha),
                      C.byref(self.epi), None, self.ws.data_ptr() if self.ws is not None else None,
                      self.ws.numel() if self.ws is not None else 0, self.stream)
                     for i in range(self.R)]

    def launch(self, i=0):
        s = self.fn(*self.args[i % self.R])
        if s != 0:
            self.dg.check(s)


def prepare(h, name, dev, rotate):
    return (PreparedMx if name.startswith("mx") else Prepared)(h, name, dev, rotate)


def time_steps(p, steps, warmup, use_graph, min_warm_s=0.0):
    """Average milliseconds per step over `steps` steps (HIP events), after
    `warmup` untimed steps and, when min_warm_s > 0, untimed steps until at
    least that much time has passed (the clocks settle under sustained load)."""
    import torch
    if use_graph:
        # a graph of L consecutive steps (cycling through the B copies)
        L = max(p.R, 20)
        p.launch(0)
        torch.cuda.synchronize()
        eager = p.C.clone()
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            p.stream = s.cuda_stream
            p.args = [a[:-1] + (s.cuda_stream,) for a in p.args]
            with torch.cuda.graph(g, stream=s):
                for i in range(L):
                    p.launch(i)
        torch.cuda.current_stream().wait_stream(s)
        for _ in range(max(1, warmup // L)):
            g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < min_warm_s:
            g.replay()
            torch.cuda.synchronize()
        # the graph's result must equal the eager result
        if not torch.equal(p.C, eager):
            raise RuntimeError(f"graph replay differs from eager run for {p.w.name}")
        reps = max(1, -(-steps // L))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / (reps * L), reps * L
    for i in range(warmup):
        p.launch(i)
    torch.cuda.synchronize()
    t0, i = time.perf_counter(), warmup
    while time.perf_counter() - t0 < min_warm_s:
        for _ in range(20):
            p.launch(i)
            i += 1
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        p.launch(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps, steps


# Kernel sources whose text fixes the tiled kernel's code; a recorded traffic
# figure holds only for the sources it was measured on.
TILED_SOURCES = ["gemm_tiled.h", "gemm_tiled_i8.hip", "kcommon.h", "catalogue.h", "dg_args.h"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.txt")


def code_hash(texts):
    """Hash of source texts with comments and whitespace runs removed: a
    comment edit keeps it, any change to the code changes it."""
    import hashlib
    import re
    h = hashlib.sha256()
    for text in texts:
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def tiled_source_hash():
    """code_hash of the tiled kernel's sources: the recorded HBM counters stay
    valid while it matches."""
    texts = []
    for f in TILED_SOURCES:
        with open(os.path.join(ROOT, "tile_planned_generator_amd", "csrc", f), encoding="utf-8") as fh:
            texts.append(fh.read())
    return code_hash(texts)


def recorded_traffic(workload):
    """HBM bytes per launch measured with rocprofv3 counters for `workload`, or
    None when no record matches the current kernel sources."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    want = tiled_source_hash()
    with open(TRAFFIC_FILE) as fh:
        for line in fh:
            if line.startswith("#") or not line.strip():
                continue
            f = dict(kv.split("=", 1) for kv in line.split())
            if f.get("workload") == workload and f.get("sources") == want:
                return int(f["traffic_bytes"])
    return None


def report(p, ms):
    ops, byts = algorithmic(p.w)
    path = p.w.path
    tflops = ops / (ms * 1e-3) / 1e12
    gbps = byts / (ms * 1e-3) / 1e9
    i = p.info
    if path == "mxq":
        return {"ms": round(ms, 6), "GB/s": round(gbps, 1), "bound": "hbm",
                "frac_of_peak": round(gbps / HBM_PEAK, 4), "kernel": "quant_mx_kernel",
                "algorithmic_bytes": byts}
    bound = "hbm" if p.w.M <= 16 else "mfma"
    frac = gbps / HBM_PEAK if bound == "hbm" else tflops / PEAK[path]
    return {"ms": round(ms, 6), "TFLOP/s" if path != "i8" else "TOP/s": round(tflops, 2),
            "GB/s": round(gbps, 1), "bound": bound, "frac_of_peak": round(frac, 4),
            "kernel": i.kernel_name.decode(), "split_k": i.split_k,
            "tile": f"{i.m_tile}x{i.n_tile}", "algorithmic_bytes": byts, "ops": ops}


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def launch_pairs(p, n=100):
    """Median milliseconds of one launch bracketed by its own event pair (n
    launches): the kernel plus the overhead of an isolated launch."""
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(ev):
        a.record()
        p.launch(i)
        b.record()
    torch.cuda.synchronize()
    return sorted(a.elapsed_time(b) for a, b in ev)[n // 2]


def plan_record(info):
    """The headline plan's shape and resources: the compiler's register and LDS
    counts of the chosen kernel and the waves it runs per SIMD."""
    return {"kernel": info.kernel_name.decode(), "tile": [info.m_tile, info.n_tile],
            "mfma": [info.mfma_m, info.mfma_n, info.mfma_k], "waves_per_wg": info.waves_per_wg,
            "waves_per_simd": info.waves_per_simd, "vgpr": info.vgpr_est, "agpr": info.agpr_est,
            "lds_bytes": info.lds_bytes, "k_main": info.k_main, "n_main": info.n_main, "k_tail": info.k_tail,
            "split_k": info.split_k, "est_us": round(info.est_us, 2)}


def cpu_baseline(budget_s=12.0):
    """The oracle on leading rows of the int8 4096^3 workload; rows grow until
    about `budget_s` seconds of CPU work."""
    import oracle
    from tile_planned_generator_amd import synth
    w = synth.make(HEADLINE, M=4096)
    A = w.tensors["A"].numpy()
    B = w.tensors["B"].numpy()
    rows, spent = 8, 0.0
    while True:
        t0 = time.perf_counter()
        oracle.gemm_int(A[:rows], B)
        dt = time.perf_counter() - t0
        if dt * 4 > budget_s or rows >= 4096:
            break
        rows = min(4096, rows * 4)
        spent += dt
    ops = 2.0 * rows * w.N * w.K
    return {"value": round(ops / dt / 1e12, 6), "unit": "TOPS", "cores": oracle.max_threads(),
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"rows 0..{rows - 1} of the int8 4096x4096x4096 GEMM "
                      f"({rows}x4096x4096 multiply-adds, int64 accumulation), {dt:.2f} s"}


def stage_breakdown(h, p, launches=5):
    """Per-stage s_memtime ticks of the headline kernel from the library's stage
    clock (dg_set_stage_clock), on untimed launches after the timed ones: medians
    and maxima over the workgroups of the last launch, and the span from the first
    workgroup's entry to the last one's end."""
    import torch
    from tile_planned_generator_amd import dg
    grid = p.info.grid
    buf = torch.zeros(grid * 8, dtype=torch.int64, device="cuda:0")
    h.set_stage_clock(buf)
    try:
        for _ in range(launches):
            p.launch(0)
        torch.cuda.synchronize()
    finally:
        h.set_stage_clock(None)
    s = dg.stage_cycles(buf.cpu().numpy(), grid)
    tot = s["prologue"]["median"] + s["k_loop"]["median"] + s["epilogue"]["median"]
    s["frac"] = {k: round(s[k]["median"] / max(1, tot), 4) for k in ("prologue", "k_loop", "epilogue")}
    s.pop("span")   # the counters of different dies do not compare
    s["unit"] = "s_memtime ticks per workgroup"
    # The s_memtime counter runs at the MFMA clock (a 32x32x32 int8 MFMA issues
    # every 32 ticks back to back), and its rate over the K loop's real time is
    # the clock the loop ran at.  MFMA cycles each SIMD owes per K step: the
    # step's multiply-adds (tile x K step) over the CU's dense rate per clock
    # (the published peak over 256 CUs at 2.4 GHz: 4096 int8 multiply-adds,
    # whichever MFMA block the kernel uses).
    i = p.info
    macs_per_clk = PEAK[p.w.path] * 1e12 / 2 / 256 / 2.4e9
    per_step = i.m_tile * i.n_tile * i.k_main / macs_per_clk
    if s["k_loop"]["median"] > 0:
        s["k_loop_mfma_busy"] = round(per_step * s["k_steps"] / s["k_loop"]["median"], 4)
    if s.get("tick_ghz"):
        s["k_loop_clock_ghz"] = s["tick_ghz"]
        s["k_loop_peak_at_clock"] = round(PEAK["i8"] * s["tick_ghz"] / 2.4, 1)
    return s


def telemetry(p, ms_step, seconds=3.0):
    """Engine clock and package power while the headline kernel runs back to back
    for about `seconds`: the GPU metrics table of the AMD SMI library, sampled
    from a thread every 20 ms.  The firmware refreshes the table about once a
    second, so only samples taken after the first second of the loop and with a
    new firmware timestamp are kept.  `sclk_mhz` is the mean engine clock over the
    XCDs and those samples, `power_w` the mean socket power, and
    `power_limited_frac` the share of the loop the power limit (PPT) was
    throttling the clock (from the firmware's residency counters)."""
    import threading

    import torch
    try:
        import amdsmi
    except Exception as e:  # pragma: no cover - reported, not fatal
        return {"error": f"amdsmi not importable: {e}"}
    try:
        amdsmi.amdsmi_init()
        props = torch.cuda.get_device_properties(0)
        want = f"{props.pci_domain_id:04x}:{props.pci_bus_id:02x}:{props.pci_device_id:02x}"
        handle = None
        for x in amdsmi.amdsmi_get_processor_handles():
            if str(amdsmi.amdsmi_get_gpu_device_bdf(x)).lower().startswith(want):
                handle = x
        if handle is None:
            return {"error": f"no SMI device at {want}"}
        limit = amdsmi.amdsmi_get_power_info(handle).get("power_limit")
        samples, stop = [], threading.Event()

        def sample():
            while not stop.is_set():
                try:
                    m = amdsmi.amdsmi_get_gpu_metrics_info(handle)
                    samples.append((time.perf_counter(), m))
                except Exception:
                    pass
                time.sleep(0.02)

        n = max(1, int(seconds / (ms_step * 1e-3)))
        th = threading.Thread(target=sample, daemon=True)
        th.start()
        t0 = time.perf_counter()
        for i in range(n):
            p.launch(i)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        stop.set()
        th.join()
        kept, seen = [], set()
        for t, m in samples:
            stamp = m.get("firmware_timestamp")
            if t0 + 1.0 <= t <= t1 and stamp not in seen:
                seen.add(stamp)
                kept.append(m)
        out = {"loop_s": round(t1 - t0, 3), "launches": n, "samples": len(kept),
               "power_limit_w": round(limit / 1e6, 1) if isinstance(limit, (int, float)) and limit > 1e4
               else limit, "source": "amdsmi gpu metrics"}
        if not kept:
            out["error"] = "no refreshed sample inside the loop"
            return out

        def num(v):
            return isinstance(v, (int, float)) and not isinstance(v, bool)
        clks = [[c for c in m.get("current_gfxclks", []) if num(c) and c > 0] for m in kept]
        clks = [c for c in clks if c]
        if clks:
            out["sclk_mhz"] = round(sum(sum(c) / len(c) for c in clks) / len(clks), 1)
            out["sclk_mhz_per_xcd"] = [round(sum(c[i] for c in clks) / len(clks)) for i in range(len(clks[0]))]
        pw = [m.get("current_socket_power") for m in kept if num(m.get("current_socket_power"))]
        if pw:
            out["power_w"] = round(sum(pw) / len(pw), 1)
        first, last = kept[0], kept[-1]
        if all(num(x.get(k)) for x in (first, last) for k in ("ppt_residency_acc", "accumulation_counter")):
            da = last["accumulation_counter"] - first["accumulation_counter"]
            if da > 0:
                out["power_limited_frac"] = round((last["ppt_residency_acc"] - first["ppt_residency_acc"]) / da, 3)
        return out
    except Exception as e:  # pragma: no cover
        return {"error": f"{type(e).__name__}: {e}"}
    finally:
        try:
            amdsmi.amdsmi_shut_down()
        except Exception:
            pass


def versions():
    import torch
    rocm = None
    try:
        with open("/opt/rocm/.info/version") as fh:
            rocm = fh.read().strip()
    except OSError:
        pass
    return {"torch": torch.__version__, "hip": getattr(torch.version, "hip", None), "rocm": rocm}


def repeats(p, steps, n=5):
    """n more timed runs of `steps` back-to-back steps: median and minimum."""
    import torch
    ms = []
    for _ in range(n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for i in range(steps):
            p.launch(i)
        e1.record()
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1) / steps)
    srt = sorted(ms)
    return {"n": n, "steps": steps, "ms_median": round(srt[n // 2], 6), "ms_min": round(srt[0], 6),
            "all_ms": [round(x, 6) for x in ms]}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=300,
                    help="untimed launches first (the default, about 20 ms of the headline, runs past the "
                         "dip of the power management after an idle start)")
    ap.add_argument("--only-headline", action="store_true")
    ap.add_argument("--workloads", default="",
                    help="comma-separated subset of the other workloads to time")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-telemetry", action="store_true",
                    help="skip the clock and power record (a 3 s loop of the headline kernel)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first copy 256 MiB once (a plain copy kernel of known size, the "
                         "reference for scaling FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU: the planned GEMM is a single-GPU kernel here; "
              "--gpus above 1 is not supported", file=sys.stderr)
        sys.exit(2)
    import torch
    from tile_planned_generator_amd import dg
    dev = "cuda:0"
    torch.cuda.init()
    h = dg.Handle(0)
    props = torch.cuda.get_device_properties(0)

    if args.copy_calibration:
        src = torch.empty(256 * 2 ** 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # ---- headline
    p = Prepared(h, HEADLINE, dev, rotate=False)
    ms, steps = time_steps(p, args.steps, args.warmup, use_graph=False)
    head = report(p, ms)
    plan_info = p.info
    ops, _ = algorithmic(p.w)
    achieved_job = ops / (ms * 1e-3) / 1e12
    rep = repeats(p, steps)
    rep["launch_pair_ms_median"] = round(launch_pairs(p), 6)
    rep["TOP/s_median"] = round(ops / (rep["ms_median"] * 1e-3) / 1e12, 2)
    rep["TOP/s_best"] = round(ops / (rep["ms_min"] * 1e-3) / 1e12, 2)
    # the kernel's average duration over the timed region (one launch per step,
    # launched back to back): the mean of those launches in a kernel trace of
    # this command
    kernel_ms = ms
    achieved = ops / (kernel_ms * 1e-3) / 1e12
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK["i8"],
                "unit": "TOP/s", "frac": round(achieved / PEAK["i8"], 4),
                "traffic": recorded_traffic(HEADLINE), "kernel_ms": round(kernel_ms, 6), "launches": steps}
    stages = stage_breakdown(h, p)
    telem = None if args.no_telemetry else telemetry(p, ms)
    del p
    torch.cuda.empty_cache()

    workloads = {HEADLINE: head}
    if not args.only_headline:
        chosen = [w for w in args.workloads.split(",") if w] or SECONDARY
        for name in chosen:
            p = prepare(h, name, dev, rotate=True)
            small = p.info is None or p.info.est_us < 25
            ms_w, _ = time_steps(p, max(50, args.steps // 2), args.warmup, use_graph=small,
                                 min_warm_s=WORKLOAD_WARM_S)
            r = report(p, ms_w)
            if p.R > 1:
                r["rotated_copies"] = p.R
                pw = prepare(h, name, dev, rotate=False)
                ms_warm, _ = time_steps(pw, max(50, args.steps // 2), args.warmup, use_graph=small,
                                        min_warm_s=WORKLOAD_WARM_S)
                r["warm"] = report(pw, ms_warm)
                del pw
            r["graph"] = small
            workloads[name] = r
            del p
            torch.cuda.empty_cache()

    cpu = None if args.no_cpu_baseline else cpu_baseline()
    line = {
        "metric": METRIC, "value": round(achieved_job, 2), "unit": "TOPS", "n_gpus": 1,
        "steps": steps, "warmup": args.warmup, "ms_per_step": round(ms, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "i8",
        "data": "synthetic",
        "config": {"workload": HEADLINE, "M": 4096, "N": 4096, "K": 4096,
                   "a": "int8 row-major", "b": "int8 row-major (K x N)", "c": "int32",
                   "kernel": head["kernel"], "tile": head["tile"], "split_k": head["split_k"]},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "repeats": rep,
        "plan": plan_record(plan_info),
        "telemetry": telem,
        "stages": stages,
        "device": {"name": props.name, "cus": props.multi_processor_count},
        "versions": versions(),
        "workloads": workloads,
    }
    print(json.dumps(line), flush=True)
    h.close()


if __name__ == "__main__":
    main()
