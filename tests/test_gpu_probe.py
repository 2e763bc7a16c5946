"""GPU: the hardware probe (dg_probe, tile_planned_generator_amd.probe) gives
rates in the range the device's published peaks allow, a consistent LDS
bank-conflict curve and cache capacities, per-variant efficiencies from the
library's own kernels, and a description a device handle plans and computes
with correctly; dg_create plans with the shipped description of the device."""
import json
import os

import pytest

from tests.test_gpu_parity import h, run  # noqa: F401  (fixture and runner)
from tile_planned_generator_amd import dg, probe, synth

pytestmark = pytest.mark.gpu
SHIPPED = os.path.join(os.path.dirname(dg.LIB_PATH), "devices", "gfx950.json")


def test_probe_measures_the_device(h):  # noqa: F811
    r = probe.measure(0, stream_bytes=1 << 30, mfma_iters=1024, calibrate_tiles=False)
    m = r["measured"]
    print({k: v for k, v in m.items() if k != "lds_ticks_by_stride"})
    assert 1000 < m["hbm_gbps"] < 8000 * 1.05          # below the 8 TB/s peak
    assert 300 < m["mfma_tflops_f16"] < 2516.6 * 1.05  # below the fp16 dense peak
    assert 0.5 < m["mfma_clock_ghz"] < 2.5
    # LDS: more lanes per bank, more ticks; the stride reported is where that saturates
    t = {int(k): v for k, v in m["lds_ticks_by_stride"].items()}
    strides = sorted(t)
    assert all(t[b] >= 0.95 * t[a] for a, b in zip(strides, strides[1:]))
    assert t[256] > 2 * t[1]
    assert m["lds_conflict_stride_words"] == min(s for s in strides if t[s] >= 0.9 * t[256])
    assert m["lds_conflict_stride_words"] >= 16
    # caches: a per-die L2 of a few MiB and a last-level cache of some hundred
    # MiB, read faster than HBM
    assert 1 << 20 <= m["l2_bytes_per_xcd"] <= 16 << 20
    assert 64 << 20 <= m["mall_bytes"] <= 1 << 30
    rates = {int(k): v for k, v in m["cached_read_gbps_by_mib"].items()}
    assert rates[4] > 1.5 * rates[1024]
    assert r["desc"]["cu_count"] == 256 and r["desc"]["hbm_gbps"] == m["hbm_gbps"]
    # a device handle planning with the measured description still computes right
    h.set_device_desc(probe.load_desc(r))
    try:
        run(h, synth.make("bf16_1x4096x131072", K=4096))
        run(h, synth.make("f16_2048x2048x8192_bias_gelu", M=300, N=264, K=512))
    finally:
        h.load_device_json(SHIPPED)


def test_calibration_of_one_path(h, tmp_path):  # noqa: F811
    # every int8 variant timed at two K lengths: efficiencies in (0, 1.5] and
    # round times >= 0; with them loaded, the planner's estimate of each forced
    # variant at K = 4096 is the measured time (the fit passes through it)
    d = json.load(open(SHIPPED))
    desc = dict(d["desc"], mfma_tflops_f16=d["measured"]["mfma_tflops_f16"],
                launch_us=d["measured"]["launch_us"])
    eff, round_us, us = probe.calibrate(h, desc, "cuda:0", reps=10, rounds=1, paths=("i8",))
    assert len(eff) == 22 and all(0 < e <= 1.5 for e in eff.values())
    assert set(round_us) == set(eff) and all(r >= 0 for r in round_us.values())
    d2 = dict(d, tiled_efficiency=eff, tiled_round_us=round_us)
    (tmp_path / "cal.json").write_text(json.dumps(d2))
    off = dg.Handle(offline=dg.default_device_desc())
    off.load_device_json(str(tmp_path / "cal.json"))
    for nm in eff:
        parts = nm.split("_")[1:]
        ms = 16 if parts[-1] == "m16" else 32
        _, lay, mn, w, k = parts[:5]
        bm, bn = map(int, mn.split("x"))
        o = dg.dg_plan_opts(force_m_tile=bm, force_n_tile=bn, force_waves=2 * int(w[-1]) if w == "w2x4" else 4,
                            force_k_tile=int(k[1:]), force_split_k=1, force_path=dg.DG_PATH_TILED, force_mfma=ms)
        p = off.plan(4096, 4096, 4096, "i8", "i8", "i32", dg.DG_COL_MAJOR if lay == "k" else dg.DG_ROW_MAJOR,
                     opts=o)
        assert p.kernel_name.decode() == nm
        # (within a few per cent: the latency floor of a K step can bind for small tiles)
        assert abs(p.est_us - us[nm]["4096"]) <= 0.05 * us[nm]["4096"] + 1.0, (nm, p.est_us, us[nm])
    off.close()


def test_device_handle_plans_with_the_shipped_description(h, tmp_path):  # noqa: F811
    d = json.load(open(SHIPPED))
    got = h.device_desc()
    assert got.calibrated == len(d["tiled_efficiency"]) > 0
    assert got.mfma_tflops_f16 == d["measured"]["mfma_tflops_f16"]
    assert got.mall_bytes == d["measured"]["mall_bytes"]
    # another device's description is refused by a device handle, which keeps its own
    for change in ({"arch": "gfx942"}, {"desc": dict(d["desc"], cu_count=128)}):
        bad = dict(d, **change)
        (tmp_path / "other.json").write_text(json.dumps(bad))
        assert dg.dg_load_device_json(h.h, str(tmp_path / "other.json").encode()) == dg.DG_ERR_UNSUPPORTED
    assert h.device_desc().cu_count == 256 and h.device_desc().calibrated == got.calibrated


def test_mfma_data_probe(h):  # noqa: F811
    # every mode runs, the clock and busy share are in range, and MFMAs whose A
    # operands are all zero run at least as fast a clock as random ones
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    stream = dg.C.c_void_p(torch.cuda.current_stream().cuda_stream)

    def launch(kind, buf, nbytes, param, out, grid):
        dg.check(dg.dg_probe(h.h, kind, buf, nbytes, param, dg.C.c_void_p(out.data_ptr()), grid, stream))

    res = probe.mfma_data_clock(launch, 0, cus, seconds=0.3, rounds=4000)
    print(res)
    assert set(res) == set(probe.DATA_MODES.values())
    for name, row in res.items():
        assert 0.3 < row["shader_ghz"] < 2.6, (name, row)
        if name != "lds_reads_only":
            assert 0 < row["int8_tops"] < 5033 * 1.05
    for name in ("one_pair", "random", "zero_a"):
        assert 0.8 < res[name]["mfma_busy"] < 1.05, (name, res[name])
    assert res["zero_a"]["shader_ghz"] >= 0.95 * res["random"]["shader_ghz"]


def test_probe_argument_errors(h):  # noqa: F811
    assert dg.dg_probe(h.h, dg.DG_PROBE_STREAM, None, 16, 0, None, 1, None) == dg.DG_ERR_INVALID_ARG
    assert dg.dg_probe(h.h, 7, None, 0, 0, dg.C.c_void_p(1), 1, None) == dg.DG_ERR_INVALID_ARG
    assert dg.dg_probe(h.h, dg.DG_PROBE_LDS, None, 0, 0, dg.C.c_void_p(1), 1, None) == dg.DG_ERR_INVALID_ARG
    # the MFMA data probe: a source buffer, a known mode and at least one round
    one = dg.C.c_void_p(16)
    assert dg.dg_probe(h.h, dg.DG_PROBE_MFMA_DATA, None, 16, 1 | (8 << 3), one, 1, None) == dg.DG_ERR_INVALID_ARG
    assert dg.dg_probe(h.h, dg.DG_PROBE_MFMA_DATA, one, 16, 6 | (8 << 3), one, 1, None) == dg.DG_ERR_INVALID_ARG
    assert dg.dg_probe(h.h, dg.DG_PROBE_MFMA_DATA, one, 16, 1, one, 1, None) == dg.DG_ERR_INVALID_ARG
    assert dg.dg_probe(h.h, dg.DG_PROBE_MFMA_DATA, one, 24, 1 | (8 << 3), one, 1, None) == dg.DG_ERR_INVALID_ARG
    # a pass count past the limit is refused before launch
    assert dg.dg_probe(h.h, dg.DG_PROBE_STREAM, dg.C.c_void_p(16), 16, 1 | (4097 << 1), dg.C.c_void_p(1), 1,
                       None) == dg.DG_ERR_INVALID_ARG
