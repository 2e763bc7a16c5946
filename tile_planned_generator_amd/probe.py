"""Hardware probe: measure the device and write the description the planner
plans with, as JSON (the pages' per-GPU hardware description, [generator]
section 3.2, step 1; the hardware-aware first stage of [overview] section 4.1).

    python -m tile_planned_generator_amd.probe --out mi355x.json

The structural fields come from the device properties; what the planner's cost
model reads as rates is measured with the library's probe kernels (dg_probe):

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

``load_desc(path)`` turns the JSON back into a ``dg_device_desc`` (for
``dg.Handle.set_device_desc`` or an offline handle).  The measured peak clock
stays the device's published one: the planner's per-variant efficiencies
already fold in the clock under load.
"""
import argparse
import ctypes as C
import json

from tile_planned_generator_amd import dg

DESC_FIELDS = ("cu_count", "xcd_count", "simd_per_cu", "wave_size", "lds_bytes_per_cu",
               "lds_bytes_per_wg", "vgpr_per_lane", "max_waves_per_simd", "clock_ghz", "hbm_gbps",
               "l2_bytes_per_xcd")


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


def measure(device=0, stream_bytes=1 << 30, mfma_iters=4096):
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
    finally:
        h.close()

    desc = {f: getattr(base, f) for f in DESC_FIELDS}
    desc.update(cu_count=cus, lds_bytes_per_cu=int(getattr(props, "shared_memory_per_multiprocessor", 0) or
                                                     desc["lds_bytes_per_cu"]),
                hbm_gbps=round(hbm_gbps, 1))
    return {
        "arch": props.gcnArchName.split(":")[0],
        "name": props.name,
        "desc": desc,
        "measured": {
            "hbm_gbps": round(hbm_gbps, 1),
            "mfma_tflops_f16": round(mfma_tflops, 1),
            "mfma_clock_ghz": round(mfma_clock, 3),
            "lds_conflict_stride_words": conflict_stride,
            "lds_ticks_by_stride": {str(k): v for k, v in lds.items()},
            "launch_us": round(t_0 * 1e6, 2),
        },
    }


def load_desc(path_or_dict):
    """A dg_device_desc from a probe JSON file (or its dict)."""
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
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--device", type=int, default=0)
    ap.add_argument("--out", default="")
    a = ap.parse_args()
    r = measure(a.device)
    text = json.dumps(r, indent=1)
    if a.out:
        with open(a.out, "w") as f:
            f.write(text + "\n")
    print(text)


if __name__ == "__main__":
    main()
