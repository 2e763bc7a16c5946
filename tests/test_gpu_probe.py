"""GPU: the hardware probe (dg_probe, tile_planned_generator_amd.probe) gives
rates in the range the device's published peaks allow, a consistent LDS
bank-conflict curve, and a description a device handle plans and computes with
correctly."""
import pytest

from tests.test_gpu_parity import h, run  # noqa: F401  (fixture and runner)
from tile_planned_generator_amd import dg, probe, synth

pytestmark = pytest.mark.gpu


def test_probe_measures_the_device(h):  # noqa: F811
    r = probe.measure(0, stream_bytes=1 << 29, mfma_iters=1024)
    m = r["measured"]
    print(r)
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
    assert r["desc"]["cu_count"] == 256 and r["desc"]["hbm_gbps"] == m["hbm_gbps"]
    # a device handle planning with the measured description still computes right
    h.set_device_desc(probe.load_desc(r))
    try:
        run(h, synth.make("bf16_1x4096x131072", K=4096))
        run(h, synth.make("f16_2048x2048x8192_bias_gelu", M=300, N=264, K=512))
    finally:
        h.set_device_desc(dg.default_device_desc())


def test_probe_argument_errors(h):  # noqa: F811
    assert dg.dg_probe(h.h, dg.DG_PROBE_STREAM, None, 16, 0, None, 1, None) == dg.DG_ERR_INVALID_ARG
    assert dg.dg_probe(h.h, 7, None, 0, 0, dg.C.c_void_p(1), 1, None) == dg.DG_ERR_INVALID_ARG
    assert dg.dg_probe(h.h, dg.DG_PROBE_LDS, None, 0, 0, dg.C.c_void_p(1), 1, None) == dg.DG_ERR_INVALID_ARG
