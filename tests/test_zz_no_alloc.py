"""dg_gemm_noalloc: dg_gemm for callers that cannot allocate device memory, with
the split-K partial sums in the library's static device scratch.

Each case calls dg_gemm (with a caller workspace) and dg_gemm_noalloc on the
same inputs and plan options, then compares: bit for bit for int8 (and the
integer result against the oracle), within the fp16 rule of tests/parity.py
for floating point (both against the oracle).  The calls come in pairs, the
second smaller than the first, so a partial sum left in the scratch by the
first call would show up in the second.  Plans whose partial sums exceed the
scratch are refused before anything is enqueued.
"""
import numpy as np
import pytest
import torch

import oracle
from tests.parity import bits, check_fp, say
from tile_planned_generator_amd import dg, synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def h():
    torch.cuda.init()
    hd = dg.Handle(0)
    yield hd
    hd.close()


def _int_pair(h, M, N, K, split, seed):
    say(f"[case] noalloc int8 M={M} N={N} K={K} split={split} seed={seed}")
    w = synth.make("i8_4096x4096x4096", M=M, N=N, K=K, seed=seed)
    A, B = w.tensors["A"].to(DEV), w.tensors["B"].to(DEV)
    o = dg.dg_plan_opts(force_split_k=split, force_path=dg.DG_PATH_TILED)
    C1 = torch.full((M, N), 7, dtype=torch.int32, device=DEV)
    C2 = torch.full((M, N), 7, dtype=torch.int32, device=DEV)
    info = h.gemm(A, B, C1, opts=o)
    assert info.split_k == split and info.workspace_bytes > 0
    h.gemm(A, B, C2, opts=o, noalloc=True)
    torch.cuda.synchronize()
    _, Cw, _ = oracle.gemm_int(w.tensors["A"].numpy(), w.tensors["B"].numpy())
    assert torch.equal(C1, C2)
    assert np.array_equal(C2.cpu().numpy(), Cw)


def test_int8_split_calls_in_a_row(h):
    _int_pair(h, 512, 384, 8192, 8, 211)
    _int_pair(h, 130, 96, 2048, 4, 212)


def _fp_pair(h, name, M, N, K, opts, seed):
    say(f"[case] noalloc {name} M={M} N={N} K={K} seed={seed}")
    w = synth.make(name, M=M, N=N, K=K, seed=seed)
    t = w.tensors
    A, B = t["A"].to(DEV), t["B"].to(DEV)
    bias = t["bias"].to(DEV) if "bias" in t else None
    out = {"f16": torch.float16, "bf16": torch.bfloat16}[w.out]
    C1 = torch.full((M, N), 7, dtype=out, device=DEV)
    C2 = torch.full((M, N), 7, dtype=out, device=DEV)
    info = h.gemm(A, B, C1, bias=bias, epilogue=w.epilogue, opts=opts)
    h.gemm(A, B, C2, bias=bias, epilogue=w.epilogue, opts=opts, noalloc=True)
    torch.cuda.synchronize()
    kind = "f16" if w.path == "f16" else "bf16"
    kw = dict(bias=bits(t["bias"]), bias_kind=kind) if bias is not None else {}
    R = oracle.gemm_real(bits(t["A"]), bits(t["B"]), a_kind=kind, b_kind=kind,
                         act=1 if "gelu" in w.epilogue else 0, **kw)
    tol = "bf16" if w.out == "bf16" else "f16"
    s1, s2 = check_fp(C1, R, tol), check_fp(C2, R, tol)
    say(f"       dg_gemm {info.kernel_name.decode()} S={info.split_k}: {s1}\n       noalloc: {s2}")
    return C1, C2


def test_bias_gelu_split_calls_in_a_row(h):
    o4 = dg.dg_plan_opts(force_split_k=4, force_path=dg.DG_PATH_TILED)
    C1, C2 = _fp_pair(h, "f16_2048x2048x8192_bias_gelu", 384, 320, 4096, o4, 311)
    assert torch.equal(C1, C2)   # same plan, same kernels: identical bits
    o2 = dg.dg_plan_opts(force_split_k=2, force_path=dg.DG_PATH_TILED)
    C1, C2 = _fp_pair(h, "f16_2048x2048x8192_bias_gelu", 100, 72, 1024, o2, 312)
    assert torch.equal(C1, C2)


def test_planner_keeps_plans_that_fit_the_scratch(h):
    # the bias + GELU workload at full size: dg_gemm's plan may split K into
    # partial sums larger than the scratch; dg_gemm_noalloc plans within it
    _fp_pair(h, "f16_2048x2048x8192_bias_gelu", 2048, 2048, 8192, None, 303)
    # the streaming path with a K split (M = 16 long K), then a smaller one
    _fp_pair(h, "bf16_16x4096x131072", 16, 4096, 32768, None, 405)
    _fp_pair(h, "bf16_1x4096x131072", 1, 1000, 8192, None, 404)


def test_plans_over_the_scratch_are_refused(h):
    A = torch.zeros(2048, 64, dtype=torch.float16, device=DEV)
    B = torch.zeros(64, 2048, dtype=torch.float16, device=DEV)
    C = torch.full((2048, 2048), 7, dtype=torch.float16, device=DEV)
    # four slices of 2048 x 2048 fp32 partial sums: 64 MiB
    with pytest.raises(dg.DGError) as e:
        h.gemm(A, B, C, opts=dg.dg_plan_opts(force_split_k=4, force_path=dg.DG_PATH_TILED), noalloc=True)
    assert e.value.status == dg.DG_ERR_WORKSPACE and "scratch" in str(e.value)
    # pad_k always adds a partial slice: 4096 x 4096 needs 128 MiB at least
    A = torch.zeros(4096, 112, dtype=torch.float16, device=DEV)
    B = torch.zeros(100, 4096, dtype=torch.float16, device=DEV)
    C = torch.full((4096, 4096), 7, dtype=torch.float16, device=DEV)
    with pytest.raises(dg.DGError) as e:
        h.gemm(A[:, :100], B, C, K=100, opts=dg.dg_plan_opts(pad_k=1), noalloc=True)
    assert e.value.status == dg.DG_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((C == 7).all())   # nothing was enqueued
