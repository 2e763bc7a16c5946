"""C-ABI and planner tests that need no GPU.

The library must load and export every function ``include/dg.h`` declares.
The planner runs on an offline handle (a described device, no HIP call), and
every plan it returns must satisfy the constraints it claims to enforce: LDS
and register budgets, the occupancy target, a K schedule whose steps sum to
the slice and are whole MFMA steps, slices that cover K, tiles that cover
M x N, and a Pareto set in which no candidate dominates another.  The error
catalogue of the pages maps onto status codes and is exercised here.
"""
import ctypes as C
import os
import re

import numpy as np

import pytest

from tile_planned_generator_amd import dg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(not os.path.exists(dg.LIB_PATH),
                                reason="libdg.so not built (run __graft_entry__.build())")


def header_functions():
    text = open(os.path.join(ROOT, "include", "dg.h")).read()
    return sorted(set(re.findall(r"^\s*(?:dg_status|const char \*)\s*(dg_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_symbol():
    lib = dg.load()
    names = header_functions()
    assert len(names) >= 9
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(dg.EXPORTS)


def test_status_strings():
    assert dg.dg_status_str(dg.DG_OK) == "DG_OK"
    assert dg.dg_status_str(dg.DG_ERR_NO_CANDIDATE) == "DG_ERR_NO_CANDIDATE"
    assert dg.dg_status_str(99) == "DG_UNKNOWN"


@pytest.fixture(scope="module")
def off():
    h = dg.Handle(offline=dg.default_device_desc())
    yield h
    h.close()


PROBLEMS = [
    # (M, N, K, a, b, c, epilogue)
    (256, 256, 256, "f16", "f16", "f16", "none"),
    (4096, 4096, 4096, "i8", "i8", "i32", "none"),
    (2048, 2048, 8192, "f16", "f16", "f16", "bias_gelu_erf"),
    (1, 4096, 131072, "bf16", "bf16", "bf16", "none"),
    (16, 4096, 131072, "bf16", "bf16", "bf16", "none"),
    (1, 256, 12800, "bf16", "bf16", "bf16", "none"),
    (1, 4096, 4096, "f16", "e2m1", "f16", "none"),
    (4096, 4096, 4096, "f16", "e2m1", "f16", "none"),
    (4096, 4096, 4096, "f16", "f16", "f16", "none"),
    (17, 40, 48, "f16", "f16", "f32", "none"),
    (300, 264, 4160, "bf16", "bf16", "bf16", "gelu_erf"),
    (5, 112, 96, "i8", "i8", "i8", "requant_i8"),
]


def _ksub(a, b):
    return 32 if a == "i8" or b == "e2m1" else 16


@pytest.mark.parametrize("M,N,K,a,b,c,epi", PROBLEMS)
def test_every_candidate_satisfies_constraints(off, M, N, K, a, b, c, epi):
    desc = dg.default_device_desc()
    cands = off.candidates(M, N, K, a, b, c, epilogue=epi)
    assert cands, "no candidate"
    # a ragged N with padded rows plans the same way
    if b != "e2m1" and N % 16 == 0:
        assert off.candidates(M, N - 7, K, a, b, c, epilogue=epi, ldb=N, ldc=N)
    for p in cands:
        assert p.lds_bytes <= desc.lds_bytes_per_wg
        assert p.vgpr_est <= 256 and p.agpr_est <= 256
        assert p.waves_per_simd >= 1
        # the K schedule of a slice: whole steps, summing to the slice
        assert p.n_main * p.k_main + p.n_tail * p.k_tail == p.k_slice or p.path == dg.DG_PATH_SKINNY
        if p.path == dg.DG_PATH_TILED:
            assert p.k_main % _ksub(a, b) == 0 and p.k_tail % _ksub(a, b) == 0
            assert p.n_tail in (0, 1) and p.k_tail < p.k_main
            tiles = -(-M // p.m_tile) * -(-N // p.n_tile)
            assert p.grid == tiles * p.split_k
        # slices cover K exactly once
        assert p.split_k >= 1
        assert p.split_k * p.k_slice >= K and (p.split_k - 1) * p.k_slice < K
        if p.split_k > 1:
            assert p.workspace_bytes == p.split_k * M * N * 4
        else:
            assert p.workspace_bytes == 0
        assert p.est_us > 0 and 0 < p.est_roof_fraction <= 1.0 + 1e-9
    # Pareto: nobody dominates anybody; best first
    def key(p):
        return (p.est_us, p.lds_bytes, p.vgpr_est + p.agpr_est)
    for i, x in enumerate(cands):
        for j, y in enumerate(cands):
            if i != j:
                kx, ky = key(x), key(y)
                assert not (all(u <= v for u, v in zip(ky, kx)) and ky != kx)
    assert [key(p)[0] for p in cands] == sorted(key(p)[0] for p in cands)
    # dg_plan picks the head of the Pareto list
    best = off.plan(M, N, K, a, b, c, epilogue=epi)
    assert best.kernel_name == cands[0].kernel_name and best.split_k == cands[0].split_k


def test_plan_is_deterministic_across_handles():
    h1 = dg.Handle(offline=dg.default_device_desc())
    h2 = dg.Handle(offline=dg.default_device_desc())
    for M, N, K, a, b, c, epi in PROBLEMS:
        p1 = h1.plan(M, N, K, a, b, c, epilogue=epi).as_dict()
        p2 = h2.plan(M, N, K, a, b, c, epilogue=epi).as_dict()
        assert p1 == p2
    h1.close()
    h2.close()


def test_pareto_matches_bruteforce_over_forced_plans(off):
    # every (tile, split) combination can be planned one at a time by forcing
    # it; the Pareto set must be exactly the non-dominated subset of those.
    M, N, K = 2048, 2048, 8192
    pareto = {(p.m_tile, p.n_tile, p.split_k, p.kernel_name) for p in off.candidates(M, N, K)}
    forced = []
    for mt, nt in [(256, 256), (128, 256), (256, 128), (128, 128), (64, 64)]:   # every compiled tile
        for s in (1, 2, 4, 8, 16, 32):
            o = dg.dg_plan_opts(force_m_tile=mt, force_n_tile=nt, force_split_k=s,
                                force_path=dg.DG_PATH_TILED)
            try:
                for p in off.candidates(M, N, K, opts=o):
                    forced.append(p)
            except dg.DGError:
                pass
    def key(p):
        return (p.est_us, p.lds_bytes, p.vgpr_est + p.agpr_est)
    nd = set()
    for x in forced:
        if not any(all(u <= v for u, v in zip(key(y), key(x))) and key(y) != key(x) for y in forced):
            nd.add((x.m_tile, x.n_tile, x.split_k, x.kernel_name))
    assert nd == pareto


def test_forced_tile_and_split(off):
    o = dg.dg_plan_opts(force_m_tile=128, force_n_tile=128, force_split_k=2)
    p = off.plan(1024, 1024, 1024, opts=o)
    assert (p.m_tile, p.n_tile, p.split_k) == (128, 128, 2)
    assert p.k_slice == 512 and p.n_main == 16 and p.n_tail == 0


def test_variable_k_schedule_tail(off):
    # K = 4096 + 48 with the 32-k step: 129 full steps and one tail step of 16
    # (one MFMA depth); with the 64-k step: 64 full steps and a tail of 48
    for kt, want in ((32, (32, 129, 16, 1)), (64, (64, 64, 48, 1))):
        o = dg.dg_plan_opts(force_path=dg.DG_PATH_TILED, force_split_k=1, force_k_tile=kt)
        p = off.plan(512, 512, 4096 + 48, opts=o)
        assert (p.k_main, p.n_main, p.k_tail, p.n_tail) == want
    # int8, K = 4096 + 96: 65 steps of 64 and a tail of 32, or 32 steps of 128
    # and a tail of 96
    for kt, want in ((64, (64, 65, 32, 1)), (128, (128, 32, 96, 1))):
        o = dg.dg_plan_opts(force_path=dg.DG_PATH_TILED, force_split_k=1, force_k_tile=kt)
        p = off.plan(512, 512, 4096 + 96, "i8", "i8", "i32", opts=o)
        assert (p.k_main, p.n_main, p.k_tail, p.n_tail) == want


def test_k_tile_is_a_planner_dimension(off):
    # the compiled K steps of each path are enumerated: the candidate set of a
    # large problem holds plans with different K steps, and a K step that no
    # variant of the path compiles is pruned
    for a, c, steps in (("f16", "f16", {32, 64}), ("bf16", "bf16", {32, 64}), ("i8", "i32", {64, 128})):
        seen = set()
        for kt in sorted(steps):
            o = dg.dg_plan_opts(force_path=dg.DG_PATH_TILED, force_k_tile=kt)
            for p in off.candidates(4096, 4096, 4096, a, a, c, opts=o):
                assert p.k_main == kt
                seen.add(p.k_main)
        assert seen == steps
        with pytest.raises(dg.DGError) as e:
            off.plan(4096, 4096, 4096, a, a, c, opts=dg.dg_plan_opts(force_k_tile=48))
        assert e.value.status == dg.DG_ERR_NO_CANDIDATE
    # e2m1 and MX compile one K step
    assert {p.k_main for p in off.candidates(4096, 4096, 4096, "f16", "e2m1", "f16",
                                             dg.DG_COL_MAJOR)} <= {32}


def test_skinny_shapes_choose_streaming_path(off):
    for M, N, K, a in [(1, 4096, 131072, "bf16"), (16, 4096, 131072, "bf16"), (1, 256, 12800, "bf16")]:
        p = off.plan(M, N, K, a, a, a)
        assert p.path == dg.DG_PATH_SKINNY, (M, N, K)
    p = off.plan(1, 4096, 4096, "f16", "e2m1", "f16")
    assert p.path == dg.DG_PATH_SKINNY and p.unit == dg.DG_UNIT_VALU
    p = off.plan(4096, 4096, 4096, "i8", "i8", "i32")
    assert p.path == dg.DG_PATH_TILED and p.unit == dg.DG_UNIT_MFMA


def test_unit_choice_mfma_vs_valu(off):
    # the pages choose plain FMA for tiny GEMMs (use_hmma false): both units
    # must be plannable for M = 1, and each request honoured
    pv = off.plan(1, 4096, 8192, "bf16", "bf16", "bf16", opts=dg.dg_plan_opts(unit=dg.DG_UNIT_VALU))
    pm = off.plan(1, 4096, 8192, "bf16", "bf16", "bf16", opts=dg.dg_plan_opts(unit=dg.DG_UNIT_MFMA))
    assert pv.unit == dg.DG_UNIT_VALU and pm.unit == dg.DG_UNIT_MFMA


# --------------------------------------------------------------- error catalogue
def _status(fn, *a, **k):
    try:
        fn(*a, **k)
    except dg.DGError as e:
        return e.status, str(e)
    return dg.DG_OK, ""


def test_no_candidate_after_pruning(off):
    s, msg = _status(off.plan, 4096, 4096, 4096, opts=dg.dg_plan_opts(lds_limit_bytes=1024))
    assert s == dg.DG_ERR_NO_CANDIDATE and "No valid candidate" in msg
    s, _ = _status(off.plan, 4096, 4096, 4096, opts=dg.dg_plan_opts(target_occupancy=1.0))
    assert s == dg.DG_ERR_NO_CANDIDATE


def test_k_not_aligned(off):
    s, msg = _status(off.plan, 64, 64, 4095)
    assert s == dg.DG_ERR_ALIGNMENT and "not aligned" in msg
    s, _ = _status(off.plan, 64, 64, 48, "i8", "i8", "i32")
    assert s == dg.DG_ERR_ALIGNMENT
    s, _ = _status(off.plan, 64, 64, 48, "f16", "e2m1", "f16")
    assert s == dg.DG_ERR_ALIGNMENT


def test_conflicting_compute_units(off):
    o = dg.dg_plan_opts(unit=dg.DG_UNIT_VALU, force_path=dg.DG_PATH_TILED)
    s, msg = _status(off.plan, 256, 256, 256, opts=o)
    assert s == dg.DG_ERR_CONFLICT and "conflicting compute units" in msg
    o = dg.dg_plan_opts(force_m_tile=128, force_path=dg.DG_PATH_SKINNY)
    assert _status(off.plan, 1, 256, 256, opts=o)[0] == dg.DG_ERR_CONFLICT


def test_mfma_block_option(off):
    # force_mfma picks the MFMA block of the tiled path: 16x16 exists for the
    # eight-wave 256x256 tile of every path, 32x32 for every tile
    probs = ((4096, 4096, 4096, "i8", "i8", "i32", dg.DG_ROW_MAJOR), (4096, 4096, 4096, "f16", "f16", "f16",
             dg.DG_COL_MAJOR), (2048, 2048, 8192, "bf16", "bf16", "bf16", dg.DG_ROW_MAJOR),
             (4096, 4096, 4096, "f16", "e2m1", "f16", dg.DG_COL_MAJOR))
    for M, N, K, a, b, c, lay in probs:
        for ms in (16, 32):
            p = off.plan(M, N, K, a, b, c, lay, opts=dg.dg_plan_opts(force_mfma=ms, force_path=dg.DG_PATH_TILED))
            assert p.mfma_m == p.mfma_n == ms and p.kernel_name.decode().endswith("_m16") == (ms == 16)
            if ms == 16:
                assert (p.m_tile, p.n_tile, p.waves_per_wg) == (256, 256, 8)
                assert p.mfma_k == {"i8": 64}.get(a, 32)
        # a 16x16 four-wave tile is not compiled
        o = dg.dg_plan_opts(force_mfma=16, force_waves=4)
        assert _status(off.plan, M, N, K, a, b, c, lay, opts=o)[0] == dg.DG_ERR_NO_CANDIDATE
    # only 16 and 32 are MFMA blocks; the option belongs to the tiled path
    o = dg.dg_plan_opts(force_mfma=8)
    assert _status(off.plan, 256, 256, 256, opts=o)[0] == dg.DG_ERR_INVALID_ARG
    o = dg.dg_plan_opts(force_mfma=16, force_path=dg.DG_PATH_SKINNY)
    assert _status(off.plan, 1, 4096, 4096, opts=o)[0] == dg.DG_ERR_CONFLICT
    # a streaming-shaped problem with the option set plans on the tiled path
    p = off.plan(1, 4096, 8192, "bf16", "bf16", "bf16", opts=dg.dg_plan_opts(force_mfma=32))
    assert p.path == dg.DG_PATH_TILED and p.mfma_m == 32


def test_forced_columns_pick_the_streaming_variant(off):
    # force_n_tile alone selects the streaming kernels' columns per workgroup
    for nt in (256, 512, 1024, 2048):
        o = dg.dg_plan_opts(force_n_tile=nt, force_path=dg.DG_PATH_SKINNY, unit=dg.DG_UNIT_VALU)
        p = off.plan(1, 4096, 131072, "bf16", "bf16", "bf16", opts=o)
        assert p.n_tile == nt and p.kernel_name.decode() == f"skinny_valu_bf16_mr1_lpr{nt // 32}"
    o = dg.dg_plan_opts(force_n_tile=512, force_path=dg.DG_PATH_SKINNY, unit=dg.DG_UNIT_MFMA)
    assert off.plan(16, 4096, 131072, "bf16", "bf16", "bf16", opts=o).kernel_name.decode() == "skinny_mfma_bf16"
    o = dg.dg_plan_opts(force_n_tile=16, force_path=dg.DG_PATH_SKINNY)
    p = off.plan(1, 4096, 4096, "f16", "e2m1", "f16", dg.DG_COL_MAJOR, opts=o)
    assert p.kernel_name.decode().startswith("skinny_e2m1") and p.n_tile == 16
    # no streaming kernel has 128 columns per workgroup
    o = dg.dg_plan_opts(force_n_tile=128, force_path=dg.DG_PATH_SKINNY)
    assert _status(off.plan, 1, 4096, 131072, "bf16", "bf16", "bf16", opts=o)[0] == dg.DG_ERR_NO_CANDIDATE
    # N = 256: only the 64-column waves keep all four waves of a workgroup busy
    assert off.plan(1, 256, 12800, "bf16", "bf16", "bf16").kernel_name.decode() == "skinny_valu_bf16_mr1_lpr8"


def test_unsupported_and_invalid(off):
    assert _status(off.plan, 64, 64, 64, "f16", "bf16", "f16")[0] == dg.DG_ERR_UNSUPPORTED
    assert _status(off.plan, 64, 64, 64, "f16", "f16", "bf16")[0] == dg.DG_ERR_UNSUPPORTED
    assert _status(off.plan, 64, 64, 64, "i8", "i8", "f32")[0] == dg.DG_ERR_UNSUPPORTED
    assert _status(off.plan, 64, 64, 64, "f16", "e2m1", "f16", b_layout=dg.DG_ROW_MAJOR)[0] == \
        dg.DG_ERR_UNSUPPORTED
    assert _status(off.plan, 64, 64, 64, "f16", "f16", "f16", epilogue="requant_i8")[0] == \
        dg.DG_ERR_UNSUPPORTED
    assert _status(off.plan, -1, 64, 64)[0] == dg.DG_ERR_INVALID_ARG
    assert _status(off.plan, 64, 64, 64, opts=dg.dg_plan_opts(pad_k=2))[0] == dg.DG_ERR_INVALID_ARG
    # leading dimension smaller than the matrix, or not 16-byte rows
    assert _status(off.plan, 64, 64, 64, lda=32)[0] == dg.DG_ERR_INVALID_ARG
    assert _status(off.plan, 64, 64, 64, ldb=68)[0] == dg.DG_ERR_ALIGNMENT


def test_offline_and_destroyed_handles_are_invalid_state():
    h = dg.Handle(offline=dg.default_device_desc())
    dt, lay = dg.Handle.problem("f16", "f16", "f16")
    one, zero = C.c_float(1.0), C.c_float(0.0)
    s = dg.dg_gemm(h.h, 16, 16, 16, C.byref(dt), C.byref(lay), 16, 16, None, 0, None, 16,
                   C.byref(one), C.byref(zero), None, None, None, 0, None)
    assert s == dg.DG_ERR_INVALID_STATE and "offline" in dg.dg_last_error()
    s = dg.dg_gemm_noalloc(h.h, 16, 16, 16, C.byref(dt), C.byref(lay), 16, 16, None, 0, None, 16,
                           C.byref(one), C.byref(zero), None, None, None)
    assert s == dg.DG_ERR_INVALID_STATE and "offline" in dg.dg_last_error()
    # the stage clock needs a device handle, and a consistent buffer size
    assert dg.dg_set_stage_clock(h.h, None, 0) == dg.DG_ERR_INVALID_STATE
    raw = C.c_void_p(h.h.value)
    h.close()
    assert dg.dg_set_stage_clock(raw, None, 0) == dg.DG_ERR_INVALID_STATE
    info = dg.dg_plan_info()
    s = dg.dg_plan(raw, 16, 16, 16, C.byref(dt), C.byref(lay), 0, 0, None, C.byref(info))
    assert s == dg.DG_ERR_INVALID_STATE
    assert dg.dg_destroy(raw) == dg.DG_ERR_INVALID_STATE
    assert dg.dg_destroy(None) == dg.DG_OK


def test_bad_offline_description():
    d = dg.default_device_desc()
    d.cu_count = 0
    h = C.c_void_p()
    assert dg.dg_create_offline(C.byref(h), C.byref(d)) == dg.DG_ERR_INVALID_ARG


def test_worked_example_shape_is_feasible_on_an_a100_like_description():
    # The pages' planner run (A100-SXM4, 2048 x 2048 x 8192 fp16, target
    # occupancy 0.8) lists a 64 x 64 tile with K step 32 first.  Its cost model
    # is not published, so the choice cannot be reproduced (parity unpinned);
    # what can be checked is that the 64 x 64 tile is a feasible plan under a
    # description with that GPU's shared memory and SM count.
    d = dg.default_device_desc()
    d.cu_count, d.lds_bytes_per_cu, d.lds_bytes_per_wg = 108, 164 * 1024, 164 * 1024
    d.clock_ghz, d.hbm_gbps = 1.41, 1555.0
    h = dg.Handle(offline=d)
    p = h.plan(2048, 2048, 8192, opts=dg.dg_plan_opts(force_m_tile=64, force_n_tile=64))
    assert (p.m_tile, p.n_tile) == (64, 64) and p.k_main % 16 == 0
    h.close()


def _resources():
    rows = []
    path = os.path.join(ROOT, "tile_planned_generator_amd", "csrc", "resources.inc")
    for line in open(path):
        if line.startswith("{"):
            rows.append([int(x) for x in line.strip().strip("{},").split(",")])
    return rows


def test_planner_uses_the_compiled_resource_usage(off):
    # the constraints are checked against the registers, LDS and occupancy the
    # compiler reported for each variant (no spills allowed at build time)
    rows = _resources()
    assert rows and all(r[-1] == 0 for r in rows)
    tiled = {tuple(r[1:9]): r for r in rows if r[0] == 0}
    names = {"f16": 0, "bf16": 1, "i8": 2, "e2m1": 3}
    region_k = {"f16": 32, "bf16": 32, "i8": 64, "e2m1": 32}
    for M, N, K, a, b, c, epi in PROBLEMS:
        for p in off.candidates(M, N, K, a, b, c, epilogue=epi):
            if p.path != dg.DG_PATH_TILED:
                continue
            nm = p.kernel_name.decode().split("_")
            ms = 16 if nm[-1] == "m16" else 32
            if ms == 16:
                nm = nm[:-1]
            wm, wn = map(int, nm[-2][1:].split("x"))
            kr = int(nm[-1][1:]) // region_k[nm[1]]
            assert p.k_main == int(nm[-1][1:])
            assert p.mfma_m == p.mfma_n == ms
            key = (names[nm[1]], 1 if nm[2] == "k" else 0, p.m_tile, p.n_tile, wm, wn, kr, ms)
            r = tiled[key]
            assert (p.vgpr_est, p.agpr_est, p.lds_bytes) == (r[9], r[10], r[11])
            assert p.waves_per_simd == r[12]
    # occupancy 2/8 keeps only variants the compiler gave >= 2 waves per SIMD
    o = dg.dg_plan_opts(force_m_tile=256, force_n_tile=256, target_occupancy=0.25)
    p = off.plan(2048, 2048, 2048, opts=o)
    assert "_w2x4_" in p.kernel_name.decode() and p.waves_per_simd >= 2
    for nw, part in ((4, "_w2x2_"), (8, "_w2x4_")):
        o = dg.dg_plan_opts(force_m_tile=256, force_waves=nw)
        p = off.plan(2048, 2048, 2048, opts=o)
        assert part in p.kernel_name.decode() and p.waves_per_wg == nw


def test_stage_cycles_summary():
    # four workgroups on two dies whose counters are offset: the span is per die
    r = np.zeros((4, 8), dtype=np.int64)
    r[:, 0] = [0, 10, 10**9, 10**9 + 30]
    r[:, 1] = r[:, 0] + [5, 7, 5, 5]
    r[:, 2] = r[:, 1] + 100
    r[:, 3] = r[:, 2] + [20, 20, 40, 20]
    r[:, 5] = [0, 0, 1, 1]
    r[:, 6] = 4
    s = dg.stage_cycles(r, 4)
    assert s["prologue"] == {"median": 5, "max": 7}
    assert s["k_loop"] == {"median": 100, "max": 100}
    assert s["epilogue"] == {"median": 20, "max": 40}
    assert s["span"] == 155 and s["k_steps"] == 4
    assert s["k_loop_us"] is None and s["tick_ghz"] is None     # no real-time stamps
    # real-time stamps (100 MHz) in the high halves of entries 4 and 5, one of
    # them across the 32-bit wrap: 100 ticks over 40 ns and 50 ns
    r[:, 4] = np.array([10, 20, 2**32 - 2, 30], dtype=np.int64) << 32
    r[:, 5] = (np.array([14, 25, 3, 34], dtype=np.int64) << 32) | np.array([0, 0, 1, 1])
    s = dg.stage_cycles(r, 4)
    assert s["span"] == 155                                         # dies still from the low halves
    assert s["k_loop_us"] == 0.045 and s["tick_ghz"] == 2.25


def test_probe_description_round_trip():
    # a probe result (JSON dict) becomes the description an offline handle plans with
    from tile_planned_generator_amd import probe
    base = dg.default_device_desc()
    d = {"arch": "gfx950", "desc": {f: getattr(base, f) for f in probe.DESC_FIELDS}}
    d["desc"].update(cu_count=128, hbm_gbps=6500.0)
    desc = probe.load_desc(d)
    assert desc.cu_count == 128 and desc.hbm_gbps == 6500.0 and desc.arch == b"gfx950"
    assert desc.lds_bytes_per_cu == base.lds_bytes_per_cu
    h = dg.Handle(offline=dg.default_device_desc())
    full = h.plan(1, 4096, 131072, "bf16", "bf16", "bf16")
    h.set_device_desc(desc)          # replaces the description, drops cached plans
    half = h.plan(1, 4096, 131072, "bf16", "bf16", "bf16")
    assert half.est_us > full.est_us  # fewer CUs and less bandwidth: a slower estimate
    bad = probe.load_desc(d)
    bad.hbm_gbps = 0.0
    assert dg.dg_set_device_desc(h.h, C.byref(bad)) == dg.DG_ERR_INVALID_ARG
    assert dg.dg_set_device_desc(h.h, None) == dg.DG_ERR_INVALID_ARG
    # the probe kernels need a device handle
    assert dg.dg_probe(h.h, dg.DG_PROBE_LDS, None, 0, 1, None, 1, None) == dg.DG_ERR_INVALID_STATE
    # the shipped MI355X description (written by the probe on the device) plans too
    shipped = probe.load_desc(os.path.join(ROOT, "tile_planned_generator_amd", "devices", "gfx950.json"))
    assert shipped.cu_count == 256 and 5000 < shipped.hbm_gbps < 8000
    h.set_device_desc(shipped)
    assert h.plan(4096, 4096, 4096, "i8", "i8", "i32").split_k == 1
    h.close()


def _probe_json(tmp_path, **measured):
    """A probe description (the shipped one's structure) with some measured
    fields replaced; returns its path."""
    import json
    with open(os.path.join(ROOT, "tile_planned_generator_amd", "devices", "gfx950.json")) as f:
        d = json.load(f)
    d.setdefault("measured", {}).update(measured)
    path = tmp_path / "dev.json"
    path.write_text(json.dumps(d))
    return str(path), d


def test_device_json_feeds_the_planner(tmp_path):
    # dg_load_device_json takes the probe's rates and variant efficiencies; the
    # planner's estimates and choices follow them
    path, d = _probe_json(tmp_path)
    h = dg.Handle(offline=dg.default_device_desc())
    h.load_device_json(path)
    got = h.device_desc()
    m = d["measured"]
    assert got.hbm_gbps == m["hbm_gbps"] and got.mfma_tflops_f16 == m["mfma_tflops_f16"]
    assert got.launch_us == m["launch_us"] and got.lds_conflict_stride_words == m["lds_conflict_stride_words"]
    assert got.calibrated == len(d.get("tiled_efficiency", {}))
    base = h.plan(4096, 4096, 4096, "i8", "i8", "i32")
    # a ten times slower MFMA makes every tiled estimate slower
    path2, _ = _probe_json(tmp_path, mfma_tflops_f16=m["mfma_tflops_f16"] / 10)
    h.load_device_json(path2)
    slow = h.plan(4096, 4096, 4096, "i8", "i8", "i32")
    assert slow.est_us > 3 * base.est_us
    # and the choices move with it: the tile and K split of a short, wide
    # problem, and the K split of the GELU workload's shape (at a faster MFMA
    # rate the partial sums' traffic of a split weighs more)
    for M, N, K, f in ((32, 4096, 8192, 1 / 50), (2048, 2048, 8192, 5.0)):
        got = []
        for tf in (m["mfma_tflops_f16"], m["mfma_tflops_f16"] * f):
            p, _ = _probe_json(tmp_path, mfma_tflops_f16=tf)
            h.load_device_json(p)
            q = h.plan(M, N, K, "bf16", "bf16", "bf16")
            got.append((q.kernel_name.decode(), q.split_k))
        assert got[0] != got[1], got
    h.close()


def test_device_json_errors(tmp_path):
    import json
    h = dg.Handle(offline=dg.default_device_desc())
    assert dg.dg_load_device_json(h.h, None) == dg.DG_ERR_INVALID_ARG
    assert dg.dg_load_device_json(h.h, str(tmp_path / "missing.json").encode()) == dg.DG_ERR_INVALID_ARG
    bad = tmp_path / "bad.json"
    for text in ("{", "[1, 2]", '{"desc": {}}', '{"arch": "gfx950", "desc": {"cu_count": -4}}',
                 '{"arch": "gfx950", "tiled_efficiency": {"tiled_i8_n_256x256_w2x4_k64": 7}}',
                 '{"arch": "gfx950", "desc": {"cu_count": 2.5}}'):
        bad.write_text(text)
        assert dg.dg_load_device_json(h.h, str(bad).encode()) == dg.DG_ERR_INVALID_ARG, text
    # a failed load leaves the description as it was
    assert h.device_desc().cu_count == 256 and h.device_desc().calibrated == 0
    ok = tmp_path / "ok.json"
    ok.write_text(json.dumps({"arch": "gfx950", "measured": {"launch_us": 5.5},
                              "tiled_efficiency": {"tiled_i8_n_256x256_w2x4_k64": 0.5}}))
    h.load_device_json(ok)
    assert h.device_desc().launch_us == 5.5 and h.device_desc().calibrated == 1
    h.close()


def test_pad_k_plans(off):
    # an aligned K: pad_k changes nothing
    a = off.plan(512, 512, 1024, opts=dg.dg_plan_opts(pad_k=1))
    b = off.plan(512, 512, 1024)
    assert a.split_k == b.split_k and a.workspace_bytes == b.workspace_bytes
    # K = 1000 (f16, 8 past a multiple of 16): the aligned part's slices plus one
    # tail slice, all reduced from the workspace
    # (leading dimensions stay 16-byte multiples: A's rows are padded)
    for (M, N, K, lda, a_t, c_t, unit) in ((512, 512, 1000, 1000, "f16", "f16", 16),
                                            (1, 4096, 4100, 4104, "bf16", "bf16", 16),
                                            (300, 208, 100, 112, "i8", "i32", 32), (64, 64, 7, 8, "f16", "f16", 16)):
        info = off.plan(M, N, K, a_t, a_t, c_t, opts=dg.dg_plan_opts(pad_k=1), lda=lda)
        main = off.plan(M, N, K - K % unit, a_t, a_t, c_t) if K >= unit else None
        slices = (main.split_k if main else 0) + 1
        assert info.split_k == slices
        assert info.workspace_bytes == slices * M * N * 4
        assert info.est_us > (main.est_us if main else 0)
    # e2m1 K must stay whole groups
    s, _ = _status(off.plan, 64, 64, 48, "f16", "e2m1", "f16", opts=dg.dg_plan_opts(pad_k=1))
    assert s == dg.DG_ERR_UNSUPPORTED


# ------------------------------------------------------------- MX block-scaled path
def _mx_dt(c=None):
    return dg.dg_dtypes(dg.DG_F8E4M3, dg.DG_E2M1, dg.DG_F16 if c is None else c, dg.DG_F32)


def _mx_lay():
    return dg.dg_layouts(dg.DG_ROW_MAJOR, dg.DG_COL_MAJOR, 0, 0, 0, 0)


@pytest.mark.parametrize("M,N,K", [(4096, 4096, 4096), (100, 200, 320), (1, 4096, 4096), (7, 9, 64)])
def test_mx_plans_satisfy_constraints(off, M, N, K):
    arr = (dg.dg_plan_info * 64)()
    cnt = C.c_int32()
    dg.check(dg.dg_plan_candidates(off.h, M, N, K, C.byref(_mx_dt()), C.byref(_mx_lay()), 32, 0, None,
                                   arr, 64, C.byref(cnt)))
    assert cnt.value >= 1
    for i in range(min(64, cnt.value)):
        p = arr[i]
        name = p.kernel_name.decode()
        assert name.startswith("tiled_mx_k_"), name
        # 32x32x64 or 16x16x128 block-scaled MFMAs
        assert (p.mfma_m, p.mfma_n, p.mfma_k) in ((32, 32, 64), (16, 16, 128))
        assert name.endswith("_m16") == (p.mfma_m == 16)
        assert p.lds_bytes <= 163840 and p.vgpr_est <= 256 and p.agpr_est <= 256
        # K steps of 128 (two block-scaled MFMAs); slices start on whole steps
        assert p.k_main == 128 and p.k_tail in (0, 64)
        if p.split_k > 1:
            assert p.k_slice % 128 == 0
        assert p.k_main * p.n_main + p.k_tail * p.n_tail == min(p.k_slice, K)


def test_mx_errors(off):
    info = dg.dg_plan_info()
    # K must be whole 64-element MFMA steps; pad_k is not offered
    assert dg.dg_plan(off.h, 64, 64, 96, C.byref(_mx_dt()), C.byref(_mx_lay()), 32, 0, None,
                      C.byref(info)) == dg.DG_ERR_ALIGNMENT
    o = dg.dg_plan_opts(pad_k=1)
    assert dg.dg_plan(off.h, 64, 64, 96, C.byref(_mx_dt()), C.byref(_mx_lay()), 32, 0, C.byref(o),
                      C.byref(info)) == dg.DG_ERR_UNSUPPORTED
    # fp8 A with a B that is not e2m1, or a row-major e2m1 B
    bad = dg.dg_dtypes(dg.DG_F8E4M3, dg.DG_F16, dg.DG_F16, dg.DG_F32)
    assert dg.dg_plan(off.h, 64, 64, 128, C.byref(bad), C.byref(_mx_lay()), 32, 0, None,
                      C.byref(info)) == dg.DG_ERR_UNSUPPORTED
    rm = dg.dg_layouts(dg.DG_ROW_MAJOR, dg.DG_ROW_MAJOR, 0, 0, 0, 0)
    assert dg.dg_plan(off.h, 64, 64, 128, C.byref(_mx_dt()), C.byref(rm), 32, 0, None,
                      C.byref(info)) == dg.DG_ERR_UNSUPPORTED
    # requantise epilogues and int outputs belong to the int8 path
    assert dg.dg_plan(off.h, 64, 64, 128, C.byref(_mx_dt()), C.byref(_mx_lay()), 32,
                      dg.DG_EPI_REQUANT_I8, None, C.byref(info)) == dg.DG_ERR_UNSUPPORTED
    assert dg.dg_plan(off.h, 64, 64, 128, C.byref(_mx_dt(dg.DG_I32)), C.byref(_mx_lay()), 32, 0, None,
                      C.byref(info)) == dg.DG_ERR_UNSUPPORTED
    # an offline handle launches nothing
    assert dg.dg_gemm_mx(off.h, 64, 64, 128, None, 0, None, 0, None, 0, None, 0, None, dg.DG_F16, 0,
                         1.0, None, None, None, 0, None) == dg.DG_ERR_INVALID_STATE
    assert dg.dg_quant_mx(off.h, 4, 64, None, 0, None, 0, None, 0, None) == dg.DG_ERR_INVALID_STATE
    # dg_gemm does not take MX operands (no scales for A)
    one = C.c_float(1.0)
    assert dg.dg_gemm(off.h, 64, 64, 128, C.byref(_mx_dt()), C.byref(_mx_lay()), None, None, None, 32,
                      None, None, C.byref(one), C.byref(one), None, None, None, 0,
                      None) == dg.DG_ERR_INVALID_STATE


def test_mx_plan_uses_fp8_rate_and_scale_bytes(off):
    i8 = off.plan(4096, 4096, 4096, "i8", "i8", "i32")
    mx = off.plan(4096, 4096, 4096, "f8e4m3", "e2m1", "f16", group_k=32)
    f16 = off.plan(4096, 4096, 4096, "f16", "f16", "f16")
    # the block-scaled fp8 x fp4 MFMA runs at the int8 / fp8 rate, twice fp16's
    assert mx.est_us < 0.75 * f16.est_us
    assert abs(mx.est_roof_fraction - i8.est_roof_fraction) < 0.25


# ------------------------------------------------------------------ K ranges
def _range_samples(K_min, K_max, unit):
    """The K samples dg_plan_range documents: both ends and the doublings between."""
    ks = [K_min]
    k = max(unit, K_min) * 2
    while k < K_max:
        ks.append(k // unit * unit)
        k *= 2
    if K_max != K_min:
        ks.append(K_max)
    return ks


# the compiled tiled variants of the 16-bit and int8 paths: (M tile, N tile,
# waves, K regions per step)
# (M tile, N tile, waves, K regions per step, MFMA block)
TILED_VARIANTS = ((128, 256, 4, 1, 32), (256, 256, 8, 1, 32), (256, 128, 4, 1, 32), (128, 128, 4, 1, 32),
                  (64, 64, 4, 1, 32), (256, 256, 4, 2, 32), (128, 256, 4, 2, 32), (256, 128, 4, 2, 32),
                  (128, 128, 4, 2, 32), (64, 64, 4, 2, 32), (256, 256, 8, 1, 16))


def _variants(off, path_b, bm_list=TILED_VARIANTS):
    region = 64 if path_b == "i8" else 32
    out = [dg.dg_plan_opts(force_path=dg.DG_PATH_TILED, force_m_tile=bm, force_n_tile=bn, force_waves=w,
                           force_k_tile=region * kr, force_mfma=ms)
           for bm, bn, w, kr, ms in bm_list]
    out.append(dg.dg_plan_opts(force_path=dg.DG_PATH_SKINNY))
    return out


@pytest.mark.parametrize("M,N,K_min,K_max,a,c", [(2048, 2048, 1024, 8192, "f16", "f16"),
                                                 (4096, 4096, 128, 512, "i8", "i32"),
                                                 (16, 4096, 128, 4096, "bf16", "bf16"),
                                                 (300, 200, 96, 1000, "f16", "f16")])
def test_plan_range_minimises_the_worst_ratio(off, M, N, K_min, K_max, a, c):
    # brute force over every variant: plan each sample with the variant pinned
    unit = 32 if a == "i8" else 16
    K_max = K_max // unit * unit
    ks = _range_samples(K_min, K_max, unit)
    best = [off.plan(M, N, k, a, a, c).est_us for k in ks]
    worst = {}
    for v in _variants(off, a):
        try:
            worst[(v.force_path, v.force_m_tile, v.force_n_tile, v.force_waves, v.force_k_tile, v.force_mfma)] = max(
                off.plan(M, N, k, a, a, c, opts=v).est_us / b for k, b in zip(ks, best))
        except dg.DGError:
            pass
    ro, info, w = off.plan_range(M, N, K_min, K_max, a, a, c)
    key = (ro.force_path, ro.force_m_tile, ro.force_n_tile, ro.force_waves, ro.force_k_tile, ro.force_mfma)
    assert key in worst and abs(worst[key] - w) < 1e-9
    assert w <= min(worst.values()) + 1e-9 and w >= 1.0 - 1e-12
    # the pinned variant plans every K of the range (on the MFMA depth)
    for k in range(K_min, K_max + 1, max(unit, (K_max - K_min) // 23 // unit * unit)):
        p = off.plan(M, N, k, a, a, c, opts=ro)
        assert p.kernel_name.decode() == info.kernel_name.decode() or ro.force_path == dg.DG_PATH_SKINNY


def test_plan_range_of_one_k_is_the_plan(off):
    for M, N, K in ((4096, 4096, 4096), (1, 4096, 131072), (600, 520, 256)):
        ro, info, w = off.plan_range(M, N, K, K)
        assert info.kernel_name.decode() == off.plan(M, N, K).kernel_name.decode() and w == 1.0


def test_plan_range_errors(off):
    dt, lay = dg.Handle.problem("f16", "f16", "f16")
    ro, info, w = dg.dg_plan_opts(), dg.dg_plan_info(), C.c_double()
    args = lambda kmin, kmax, o=None, r=C.byref(ro): (off.h, 256, 256, kmin, kmax, C.byref(dt), C.byref(lay), 0, 0,
                                                      C.byref(o) if o is not None else None, r, C.byref(info),
                                                      C.byref(w))
    assert dg.dg_plan_range(*args(512, 128)) == dg.DG_ERR_INVALID_ARG
    assert dg.dg_plan_range(*args(-16, 128)) == dg.DG_ERR_INVALID_ARG
    assert dg.dg_plan_range(*args(128, 512, r=None)) == dg.DG_ERR_INVALID_ARG
    assert dg.dg_plan_range(*args(128, 500)) == dg.DG_ERR_ALIGNMENT
    # with pad_k any K, but rows keep 16-byte leading dimensions (lda = 512 here)
    dt2, lay2 = dg.Handle.problem("f16", "f16", "f16", lda=512)
    assert dg.dg_plan_range(off.h, 256, 256, 128, 500, C.byref(dt2), C.byref(lay2), 0, 0,
                            C.byref(dg.dg_plan_opts(pad_k=1)), C.byref(ro), C.byref(info), C.byref(w)) == dg.DG_OK
    assert dg.dg_plan_range(*args(128, 500, dg.dg_plan_opts(pad_k=1))) == dg.DG_ERR_ALIGNMENT
    assert dg.dg_plan_range(*args(128, 512, dg.dg_plan_opts(force_m_tile=128))) == dg.DG_ERR_CONFLICT
    assert dg.dg_plan_range(None, 1, 1, 16, 32, C.byref(dt), C.byref(lay), 0, 0, None, C.byref(ro), None,
                            None) == dg.DG_ERR_INVALID_STATE


def test_transcript_tile_is_a_candidate_with_a100_budgets():
    """[generator] DeepGEMM generator article, section 3.2 (the worked planner
    run on an A100 for fp16 2048 x 2048 x 8192): the run keeps a handful of
    Pareto configurations and ranks a 64 x 64 tile with a 32-deep K step first.
    Its estimates cannot be reproduced (they equal the A100's peak rate, not a
    prediction), so this is a sanity check only: with the A100's budgets in the
    device description (108 SMs, 164 KB shared memory per SM and 163 KB per
    block, 1.41 GHz, 1555 GB/s, a 40 MB L2), the Pareto set still holds a
    64 x 64 tile stepping K by 32, and every candidate fits the described LDS
    and covers K."""
    a = dg.default_device_desc()
    a.arch = b"a100-budgets"
    a.cu_count, a.xcd_count = 108, 1
    a.lds_bytes_per_cu, a.lds_bytes_per_wg = 164 * 1024, 163 * 1024
    a.clock_ghz, a.hbm_gbps, a.l2_bytes_per_xcd = 1.41, 1555.0, 40.0 * 1024 * 1024
    h = dg.Handle(offline=a)
    try:
        M, N, K = 2048, 2048, 8192
        cands = h.candidates(M, N, K, "f16", "f16", "f16")
        assert any(p.m_tile == 64 and p.n_tile == 64 and p.k_main == 32 for p in cands)
        for p in cands:
            assert p.lds_bytes <= a.lds_bytes_per_wg
            assert p.k_main * p.n_main + p.k_tail * p.n_tail == -(-K // p.split_k)
    finally:
        h.close()


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), (["--gpus", "8"], {}), ([], {"WORLD_SIZE": "2"})])
def test_bench_refuses_more_than_one_gpu(argv, env):
    # the benchmark measures one GPU; asked for more it exits with status 2 and a
    # message, before it touches a device
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), *argv], capture_output=True, text=True,
                       timeout=120, env=dict(os.environ, **env))
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
