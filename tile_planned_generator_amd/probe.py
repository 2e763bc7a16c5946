"""Hardware probe: measure the device and write the description the planner
plans with, as JSON (the pages' per-GPU hardware description, [generator]
section 3.2, step 1; the micro-benchmarks whose results feed candidate
generation, [overview] section 4.1, stage 1).

    python -m tile_planned_generator_amd.probe --out tile_planned_generator_amd/devices/gfx950.json

``dg_create`` reads ``<library directory>/devices/<arch>.json`` by itself, so
the committed file is what every device handle plans with.  The structural
fields come from the device properties; what the planner's cost model reads as
rates is measured with the library's probe kernels (dg_probe) and its own
GEMM kernels:

  hbm_gbps        streaming-read bandwidth of a buffer far larger than the
                  caches (16-byte non-temporal loads on every CU)
  mfma_tflops_f16 back-to-back independent 32x32x16 fp16 MFMAs on every SIMD,
                  and the engine clock that rate implies (mfma_clock_ghz)
  lds_conflict_stride_words
                  the smallest power-of-two word stride at which a wave's dword
                  LDS reads are as serialised as at a stride of 256 words (the
                  bank structure seen by dword accesses; 32 on MI355X), with the
                  ticks for every stride
  launch_us       an empty launch of the probe kernel on every CU
  l2_bytes_per_xcd, mall_bytes
                  cache capacities: repeated cached reads of buffers from 4 MiB
                  to 1 GiB (every CU a contiguous share, so each die reads its
                  own eighth); the read rate stays at the L2 rate while a die's
                  eighth fits its L2, then at the last-level (MALL) rate while
                  the whole buffer fits the MALL, then falls to HBM's
  int8_mfma_clock_by_data
                  the shader clock and MFMA busy share of back-to-back int8
                  MFMAs on random operands, on constant ones, with A zero, and
                  with LDS reads at the tiled kernel's fragment rate (random or
                  zero data): how much of the clock the data itself costs
                  (recorded, not read by the planner)
  tiled_efficiency, tiled_round_us
                  per compiled tiled kernel variant, from timings of its path's
                  M = N = 4096 problem at K = 4096 and 1024 on operands read
                  from HBM: the fraction of the probed MFMA rate (twice it for
                  int8 and the fp8 MFMA) one K step sustains, and the fixed
                  time of one round of workgroups (entry, epilogue, launch)

``load_desc(path)`` turns the JSON back into a ``dg_device_desc`` (for
``dg.Handle.set_device_desc`` or an offline handle); ``Handle.load_device_json``
loads all of it, efficiencies included.
"""
import argparse
import ctypes as C
import json
import math

from tile_planned_generator_amd import dg

DESC_FIELDS = ("cu_count", "xcd_count", "simd_per_cu", "wave_size", "lds_bytes_per_cu",
               "lds_bytes_per_wg", "vgpr_per_lane", "max_waves_per_simd", "clock_ghz", "hbm_gbps",
               "l2_bytes_per_xcd", "mall_bytes")
MEASURED_DESC = ("hbm_gbps", "mfma_tflops_f16", "launch_us", "lds_conflict_stride_words",
                 "l2_bytes_per_xcd", "mall_bytes")

# tiled variants of every path: (M tile, N tile, waves, K regions per step)
VARIANTS = {
    "f16": [(128, 256, 4, 1, 32), (256, 256, 8, 1, 32), (256, 128, 4, 1, 32), (128, 128, 4, 1, 32),
            (64, 64, 4, 1, 32), (256, 256, 4, 2, 32), (128, 256, 4, 2, 32), (256, 128, 4, 2, 32),
            (128, 128, 4, 2, 32), (64, 64, 4, 2, 32), (256, 256, 8, 1, 16)],
}
VARIANTS["bf16"] = VARIANTS["i8"] = VARIANTS["f16"]
VARIANTS["e2m1"] = [v for v in VARIANTS["f16"] if v[3] == 1]
VARIANTS["mx"] = VARIANTS["e2m1"]
REGION_K = {"f16": 32, "bf16": 32, "i8": 64, "e2m1": 32, "mx": 128}


def _timed(fn, reps):
    import torch
    fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps * 1e-3   # seconds per call


def cache_sizes(probe, buf, buf_bytes, cus, xcds):
    """(l2_bytes_per_xcd, mall_bytes, {MiB: GB/s}) from cached reads of buffers
    of growing size, each launch passing over its buffer repeatedly (about
    512 MiB read per launch, so the launch cost does not count); 0 where a
    level shows no step in the rate."""
    import torch
    mib = [m for m in (4, 8, 16, 24, 32, 48, 64, 96, 128, 160, 192, 224, 256, 320, 384, 512, 768, 1024)
           if m << 20 <= buf_bytes]   # never past the buffer
    grid = cus * 4
    sink = torch.zeros(grid, dtype=torch.int32, device=buf.device)
    rates = []
    for m in mib:
        nbytes = m << 20
        passes = max(1, min(4096, 512 // m))
        fn = lambda: probe(dg.DG_PROBE_STREAM, C.c_void_p(buf.data_ptr()), nbytes, 1 | (passes << 1), sink, grid)
        fn()
        t = min(_timed(fn, 5) for _ in range(3))
        rates.append(passes * nbytes / t / 1e9)
    by = {str(m): round(r, 1) for m, r in zip(mib, rates)}
    # L2: the leading run of sizes within 3/4 of the best small-buffer rate.
    # MALL: the run after it above the midpoint between its best rate and the
    # largest buffer's (HBM) rate, when that best rate is a tenth above HBM's.
    l2_rate, hbm_rate = max(rates[:3]), rates[-1]
    i = 0
    while i < len(mib) and rates[i] >= 0.75 * l2_rate:
        i += 1
    l2 = float((mib[i - 1] << 20) // xcds) if 0 < i < len(mib) else 0.0
    mall = 0.0
    if i < len(mib) and max(rates[i:]) >= 1.1 * hbm_rate:
        mid = 0.5 * (max(rates[i:]) + hbm_rate)
        j = i
        while j < len(mib) and rates[j] >= mid:
            j += 1
        if i < j < len(mib):
            mall = float(mib[j - 1] << 20)
    return l2, mall, by


def _operands(name, dev, copies=1, **size):
    """A workload's device operands, `copies` copies of each; returns (workload,
    make, output element size), make(h, opts, kmaj) giving (plan info, a call
    that enqueues the GEMM on the next copy in turn) - B stored N x K when kmaj
    (the e2m1 and MX operands are always so)."""
    import torch
    from tile_planned_generator_amd import synth
    w = synth.make(name, device=dev, **size)
    t = w.tensors

    def rep(x):
        return [x] + [x.clone() for _ in range(copies - 1)]

    def cycle(calls):
        it = [0]

        def call():
            calls[it[0] % len(calls)][1]()
            it[0] += 1
        return calls[0][0], call

    if w.path == "mx":
        As, SAs = rep(t["A"].contiguous()), rep(t["SA"].t().contiguous())
        Bs, SBs = rep(dg.pack_e2m1(t["codes"])), rep(t["SB"].contiguous())
        Cout = torch.empty(w.M, w.N, dtype=torch.float16, device=dev)
        return w, lambda h, o, kmaj=True: cycle([h.gemm_mx(As[i], SAs[i], Bs[i], SBs[i], Cout, opts=o,
                                                           prepared=True) for i in range(copies)]), 2
    out = {"f16": torch.float16, "bf16": torch.bfloat16, "i32": torch.int32}[w.out]
    Cout = torch.empty(w.M, w.N, dtype=out, device=dev)
    As = rep(t["A"].contiguous())
    if w.path == "e2m1":
        Bs, Ss = rep(dg.pack_e2m1(t["codes"])), rep(dg.scales_gn(t["scale"]))
        return w, lambda h, o, kmaj=True: cycle([h.gemm(As[i], Bs[i], Cout, b_scale=Ss[i], opts=o, prepared=True)
                                                 for i in range(copies)]), 2
    Bn = rep(t["B"].contiguous())
    Bk = []

    def make(h, o, kmaj=False):
        if kmaj and not Bk:
            Bk.extend(b.t().contiguous() for b in Bn)
        Bs = Bk if kmaj else Bn
        return cycle([h.gemm(As[i], Bs[i], Cout, b_layout=dg.DG_COL_MAJOR if kmaj else dg.DG_ROW_MAJOR,
                             opts=o, prepared=True) for i in range(copies)])
    return w, make, Cout.element_size()


# operand bytes the calibration cycles through: twice the L2s and the MALL
COLD_BYTES = 576 << 20


def calibrate(h, desc, dev, reps=40, rounds=3, paths=None, ks=(4096, 1024)):
    """Per tiled variant, from timings of the path's M = N = 4096 problem at two
    K lengths (operands cycled through copies that exceed the caches, so every
    launch reads them from HBM): the time of one K step and the fixed time of
    one round of workgroups, fitted to t = rounds * (round + steps * step).
    Returns ({kernel name: efficiency}, {kernel name: round us}, {kernel name:
    microseconds at each K}); the efficiency is the step time as a fraction of
    the probed MFMA rate (twice it for int8 and the fp8 MFMA), counting the
    workgroups a CU runs at once."""
    import torch
    work = [("f16_4096x4096x4096", "f16", (False, True)), ("i8_4096x4096x4096", "i8", (False, True)),
            ("bf16_16x4096x131072", "bf16", (False, True)), ("e2m1_4096x4096x4096", "e2m1", (True,)),
            ("mx_4096x4096x4096", "mx", (True,))]
    f16_cu_us = desc["mfma_tflops_f16"] * 1e6 / desc["cu_count"]
    eff, round_us, times = {}, {}, {}
    for name, path, layouts in work:
        if paths is not None and path not in paths:
            continue
        rate = f16_cu_us * (2 if path in ("i8", "mx") else 1)
        fits = {}   # kernel name -> [(rounds, steps, W, step ops, us)] per K
        for K in ks:
            from tile_planned_generator_amd import synth
            w0 = synth.make(name, M=8, N=8, K=K)
            per = sum(x.numel() * x.element_size() for x in w0.tensors.values()) * 4096 // 8
            copies = max(1, -(-COLD_BYTES // per))
            w, make, osz = _operands(name, dev, copies=copies, M=4096, N=4096, K=K)
            for kmaj in layouts:
                calls = []
                for bm, bn, nw, kr, ms in VARIANTS[path]:
                    o = dg.dg_plan_opts(force_m_tile=bm, force_n_tile=bn, force_waves=nw, force_split_k=1,
                                        force_k_tile=REGION_K[path] * kr, force_path=dg.DG_PATH_TILED,
                                        force_mfma=ms)
                    try:
                        calls.append(make(h, o, kmaj))
                    except dg.DGError:
                        continue
                meas = {i.kernel_name.decode(): [] for i, _ in calls}
                for _ in range(rounds):            # interleaved, so that drift hits all alike
                    for info, call in calls:
                        meas[info.kernel_name.decode()].append(_timed(call, reps) * 1e6)
                for info, call in calls:
                    nm = info.kernel_name.decode()
                    t_us = sorted(meas[nm])[len(meas[nm]) // 2]
                    wg_cu = max(1, info.waves_per_simd * desc["simd_per_cu"] // info.waves_per_wg)
                    rnds = math.ceil(info.grid / (desc["cu_count"] * wg_cu))
                    W = min(wg_cu, math.ceil(info.grid / desc["cu_count"]))
                    fits.setdefault(nm, []).append((rnds, info.n_main + info.n_tail, W,
                                                    2.0 * info.m_tile * info.n_tile * info.k_main, t_us))
                    times.setdefault(nm, {})[str(K)] = round(t_us, 2)
                del calls
            del w, make
            torch.cuda.empty_cache()
        for nm, pts in fits.items():
            (r1, s1, W, ops, t1), (r2, s2, _, _, t2) = pts[0], pts[-1]
            step = (t1 / r1 - t2 / r2) / (s1 - s2) if s1 != s2 else 0.0
            if step <= 0:   # no usable second point: the whole time is steps
                step = t1 / (r1 * s1)
            eff[nm] = round(min(1.5, W * ops / (rate * step)), 4)
            round_us[nm] = round(max(0.0, t1 / r1 - s1 * step), 3)
    return eff, round_us, times


# operand data of the MFMA data probe (DG_PROBE_MFMA_DATA's modes)
DATA_MODES = {0: "one_pair", 1: "random", 2: "random_lds_reads", 3: "zero_a", 4: "random_lds_zeros",
              5: "lds_reads_only"}


def mfma_data_clock(probe, device, cus, seconds=1.0, rounds=20000, seed=1234):
    """Per operand mode of DG_PROBE_MFMA_DATA (one workgroup of eight waves
    per CU, random int8 operands from a seeded generator): the shader clock
    the kernel ran at (s_memtime over s_memrealtime), the share of that clock
    the MFMAs were busy, and the int8 rate.  Each mode first runs for about
    `seconds` so that the clock settles."""
    import torch
    g = torch.Generator().manual_seed(seed)
    src = torch.randint(-2 ** 31, 2 ** 31 - 1, (1 << 22,), dtype=torch.int32, generator=g).to(device)
    out = torch.zeros(3 * cus, dtype=torch.int64, device=device)
    res = {}
    for mode, name in DATA_MODES.items():
        def call(mode=mode):
            probe(dg.DG_PROBE_MFMA_DATA, C.c_void_p(src.data_ptr()), src.numel() * 4, mode | (rounds << 3), out, cus)
        t1 = _timed(call, 1)
        _timed(call, max(1, int(seconds / t1)))          # settle
        t = _timed(call, max(3, int(seconds / t1)))
        o = out.view(cus, 3).cpu()
        ghz = o[:, 0].sum().item() / o[:, 1].sum().item() * 0.1
        row = {"shader_ghz": round(ghz, 3), "kernel_ms": round(t * 1e3, 3)}
        if mode != 5:
            cycles = 2 * rounds * 8 * 32                 # per SIMD: 2 waves x 8 MFMAs x 32 cycles a round
            row["mfma_busy"] = round(cycles / (t * ghz * 1e9), 3)
            row["int8_tops"] = round(cus * 8 * rounds * 8 * 2 * 32 * 32 * 32 / t / 1e12, 1)
        res[name] = row
    return res


def measure(device=0, stream_bytes=1 << 30, mfma_iters=4096, calibrate_tiles=True, data_clock=True):
    """Run the probes on HIP device ``device``; returns the JSON-ready dict."""
    import torch
    torch.cuda.set_device(device)
    h = dg.Handle(device)
    try:
        base = dg.dg_device_desc()
        dg.check(dg.dg_default_device_desc(C.byref(base)))
        props = torch.cuda.get_device_properties(device)
        cus = props.multi_processor_count
        stream = C.c_void_p(torch.cuda.current_stream().cuda_stream)

        def probe(kind, buf, nbytes, param, out, grid):
            dg.check(dg.dg_probe(h.h, kind, buf, nbytes, param, C.c_void_p(out.data_ptr()), grid, stream))

        # HBM streaming read
        buf = torch.ones(stream_bytes // 4, dtype=torch.int32, device=device)
        grid = cus * 16
        sink = torch.zeros(grid, dtype=torch.int32, device=device)
        t = _timed(lambda: probe(dg.DG_PROBE_STREAM, C.c_void_p(buf.data_ptr()), stream_bytes, 0, sink, grid), 20)
        hbm_gbps = stream_bytes / t / 1e9
        # cache capacities (cached re-reads of growing buffers)
        l2, mall, by_mib = cache_sizes(probe, buf, stream_bytes, cus, base.xcd_count)
        del buf

        # MFMA rate (two workgroups of four waves per CU: two waves per SIMD)
        mgrid = cus * 2
        fs = torch.zeros(mgrid, dtype=torch.float32, device=device)
        t_m = _timed(lambda: probe(dg.DG_PROBE_MFMA, None, 0, mfma_iters, fs, mgrid), 5)
        t_0 = _timed(lambda: probe(dg.DG_PROBE_MFMA, None, 0, 0, fs, mgrid), 20)
        flops = mgrid * 4 * mfma_iters * 8 * 2 * 32 * 32 * 16
        mfma_tflops = flops / max(t_m - t_0, 1e-9) / 1e12
        mfma_clock = mfma_tflops * 1e12 / (cus * 4 * 512 * 2) / 1e9   # 512 fp16 FMA per clock per SIMD

        # LDS bank structure
        ticks = torch.zeros(2, dtype=torch.int64, device=device)
        lds = {}
        for s in (1, 2, 4, 8, 16, 32, 64, 128, 256):
            vals = []
            for _ in range(3):
                probe(dg.DG_PROBE_LDS, None, 0, s, ticks, 1)
                torch.cuda.synchronize()
                vals.append(int(ticks[0].item()))
            lds[s] = min(vals)
        worst = lds[256]
        conflict_stride = min(s for s in lds if lds[s] >= 0.9 * worst)

        # the clock the MFMAs hold on random operands, with and without LDS traffic
        data = mfma_data_clock(probe, device, cus) if data_clock else None

        desc = {f: getattr(base, f) for f in DESC_FIELDS}
        desc.update(cu_count=cus, lds_bytes_per_cu=int(getattr(props, "shared_memory_per_multiprocessor", 0) or
                                                         desc["lds_bytes_per_cu"]),
                    hbm_gbps=round(hbm_gbps, 1))
        measured = {
            "hbm_gbps": round(hbm_gbps, 1),
            "mfma_tflops_f16": round(mfma_tflops, 1),
            "mfma_clock_ghz": round(mfma_clock, 3),
            "lds_conflict_stride_words": conflict_stride,
            "lds_ticks_by_stride": {str(k): v for k, v in lds.items()},
            "launch_us": round(t_0 * 1e6, 2),
            "l2_bytes_per_xcd": l2,
            "mall_bytes": mall,
            "cached_read_gbps_by_mib": {str(k): v for k, v in by_mib.items()},
        }
        if data is not None:
            measured["int8_mfma_clock_by_data"] = data
        out = {"arch": props.gcnArchName.split(":")[0], "name": props.name, "desc": desc, "measured": measured}
        if calibrate_tiles:
            cal = dict(desc, **{k: measured[k] for k in ("mfma_tflops_f16", "launch_us")})
            eff, round_us, times = calibrate(h, cal, device)
            out["tiled_efficiency"] = eff
            out["tiled_round_us"] = round_us
            out["tiled_us_by_k"] = times
    finally:
        h.close()
    return out


def load_desc(path_or_dict):
    """A dg_device_desc from a probe JSON file (or its dict): the structural
    fields, then the measured ones."""
    d = path_or_dict
    if not isinstance(d, dict):
        with open(d) as f:
            d = json.load(f)
    out = dg.dg_device_desc()
    dg.check(dg.dg_default_device_desc(C.byref(out)))
    out.arch = d.get("arch", "gfx950").encode()[:31]
    for f in DESC_FIELDS:
        if f in d["desc"]:
            setattr(out, f, type(getattr(out, f))(d["desc"][f]))
    for f in MEASURED_DESC:
        if f in d.get("measured", {}):
            setattr(out, f, type(getattr(out, f))(d["measured"][f]))
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--device", type=int, default=0)
    ap.add_argument("--out", default="")
    ap.add_argument("--no-calibrate", action="store_true", help="skip the per-variant GEMM timing")
    a = ap.parse_args()
    r = measure(a.device, calibrate_tiles=not a.no_calibrate)
    text = json.dumps(r, indent=1)
    if a.out:
        with open(a.out, "w") as f:
            f.write(text + "\n")
    print(text, flush=True)


if __name__ == "__main__":
    main()
