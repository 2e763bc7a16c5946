"""GPU: the stage clock (dg_set_stage_clock), the analogue of the generator's
profile option ([generator] section 3.2).  A launch with the clock on still
matches the oracle, every workgroup writes one consistent record, workgroups past
the buffer write nothing, and with the clock off nothing is written."""
import numpy as np
import pytest
import torch

from tests.test_gpu_parity import DEV, h, run  # noqa: F401  (fixture and runner)
from tile_planned_generator_amd import dg, synth

pytestmark = pytest.mark.gpu

SENTINEL = -12345


@pytest.mark.parametrize("bm,bn,nw,split", [(256, 256, 8, 1), (128, 128, 4, 2)])
def test_stage_clock_records(h, bm, bn, nw, split):  # noqa: F811
    w = synth.make("f16_2048x2048x8192_bias_gelu", M=600, N=520, K=7 * 32 + 16)
    o = dg.dg_plan_opts(force_m_tile=bm, force_n_tile=bn, force_waves=nw, force_split_k=split,
                        force_path=dg.DG_PATH_TILED)
    info = h.plan(w.M, w.N, w.K, "f16", "f16", "f16", dg.DG_ROW_MAJOR, w.epilogue, opts=o)
    grid = info.grid
    buf = torch.full((grid * 8 + 64,), SENTINEL, dtype=torch.int64, device=DEV)
    h.set_stage_clock(buf)
    try:
        run(h, w, opts=o)   # checked against the oracle with the clock on
    finally:
        h.set_stage_clock(None)
    torch.cuda.synchronize()
    r = buf.cpu().numpy()
    assert (r[grid * 8:] == SENTINEL).all()            # nothing past the grid
    rec = r[: grid * 8].reshape(grid, 8)
    assert (rec != SENTINEL).all()
    t = rec[:, :4]
    assert (np.diff(t, axis=1) >= 0).all()             # entry <= loop start <= loop end <= end
    die = rec[:, 5] & 0xFFFFFFFF
    assert (die >= 0).all() and (die < 8).all()        # die (XCC) index
    # real time of the K loop (100 MHz counter in the high halves of 4 and 5):
    # positive, and the s_memtime rate over it a plausible engine clock
    rt = (((rec[:, 5] >> 32) & 0xFFFFFFFF) - ((rec[:, 4] >> 32) & 0xFFFFFFFF)) % (1 << 32)
    assert (rt > 0).all()
    ghz = (rec[:, 2] - rec[:, 1]) / (rt * 10.0)
    assert (ghz > 0.3).all() and (ghz < 3.0).all(), ghz
    # K steps: a step is k_main long; the slices are k_slice long but the last
    steps = {-(-min(info.k_slice, w.K - s * info.k_slice) // info.k_main) for s in range(info.split_k)}
    assert set(rec[:, 6].tolist()) <= steps
    # grid coordinates: x + y * grid_x covers every workgroup once
    x, y = rec[:, 7] & 0xFFFFFFFF, rec[:, 7] >> 32
    gx = int(x.max()) + 1
    assert sorted((x + y * gx).tolist()) == list(range(grid))
    s = dg.stage_cycles(rec, grid)
    assert s["k_loop"]["median"] > 0 and s["span"] >= s["k_loop"]["max"]
    assert s["k_loop_us"] > 0 and 0.3 < s["tick_ghz"] < 3.0

    # clock off: the buffer stays as it is
    buf.fill_(SENTINEL)
    run(h, w, opts=o)
    torch.cuda.synchronize()
    assert (buf.cpu().numpy() == SENTINEL).all()


def test_stage_clock_short_buffer(h):  # noqa: F811
    # a buffer for two workgroups: the others write nothing
    w = synth.make("i8_4096x4096x4096", M=512, N=512, K=256)
    o = dg.dg_plan_opts(force_m_tile=128, force_n_tile=128, force_waves=4, force_path=dg.DG_PATH_TILED)
    buf = torch.full((64,), SENTINEL, dtype=torch.int64, device=DEV)
    st = dg.dg_set_stage_clock(h.h, dg.C.c_void_p(buf.data_ptr()), 16)
    assert st == dg.DG_OK
    try:
        info, _ = run(h, w, opts=o)
    finally:
        h.set_stage_clock(None)
    assert info.grid > 2
    r = buf.cpu().numpy()
    assert (r[:16] != SENTINEL).all() and (r[16:] == SENTINEL).all()
    assert dg.dg_set_stage_clock(h.h, None, 8) == dg.DG_ERR_INVALID_ARG
    assert dg.dg_set_stage_clock(h.h, dg.C.c_void_p(buf.data_ptr()), -1) == dg.DG_ERR_INVALID_ARG
