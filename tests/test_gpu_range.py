"""GPU: a plan over a K range (dg_plan_range) pins one kernel variant; dg_gemm
with those options runs every K of the range, each result checked against the
oracle (bit for bit for int8, the floating-point rule otherwise)."""
import pytest

from tests.test_gpu_parity import h, run  # noqa: F401  (fixture and runner)
from tile_planned_generator_amd import dg, synth

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("recipe,a,c,M,N,K_min,K_max,ks", [
    ("f16_2048x2048x8192_bias_gelu", "f16", "f16", 300, 264, 128, 512, (128, 192, 336, 512)),
    ("i8_4096x4096x4096", "i8", "i32", 257, 320, 128, 1024, (128, 416, 1024)),
    ("bf16_16x4096x131072", "bf16", "bf16", 16, 1024, 256, 8192, (256, 1056, 8192)),
])
def test_range_plan_runs_every_k(h, recipe, a, c, M, N, K_min, K_max, ks):  # noqa: F811
    ro, info, worst = h.plan_range(M, N, K_min, K_max, a, a, c,
                                   epilogue="bias_gelu_erf" if "gelu" in recipe else "none")
    assert worst >= 1.0
    for K in ks:
        w = synth.make(recipe, M=M, N=N, K=K)
        p, _ = run(h, w, opts=ro)
        if ro.force_path == dg.DG_PATH_TILED:
            assert (p.m_tile, p.n_tile, p.waves_per_wg) == (ro.force_m_tile, ro.force_n_tile, ro.force_waves)
