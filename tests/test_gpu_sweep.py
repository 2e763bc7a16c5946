"""GPU: a seeded sweep of random problems over every path, layout, epilogue,
K split and K tail, each checked against the oracle on every output (bit for
bit for int8, the floating-point rule of tests/parity.py otherwise).  The cases
are drawn once from a fixed seed, so a failure names a reproducible case."""
import numpy as np
import pytest

from tests.test_gpu_parity import h, run  # noqa: F401  (fixture and runner)
from tile_planned_generator_amd import dg, synth

pytestmark = pytest.mark.gpu

RECIPE = {"f16": "f16_2048x2048x8192_bias_gelu", "bf16": "bf16_16x4096x131072",
          "i8": "i8_4096x4096x4096", "e2m1": "e2m1_4096x4096x4096"}


def _cases(n=36, seed=20261202):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        path = ["f16", "bf16", "i8", "e2m1"][i % 4]
        unit = 32 if path in ("i8", "e2m1") else 16
        M = int(rng.choice([1, 2, 3, 5, 8, 11, 16, 33, 100, 257, 600]))
        N = int(rng.integers(1, 190)) * 8
        if path == "i8":
            N = (N + 15) // 16 * 16   # 16-byte rows of a row-major int8 B
        K = int(rng.integers(1, 96)) * unit
        pad_k = path != "e2m1" and rng.random() < 0.3
        if pad_k:
            K += int(rng.integers(1, unit))
        split = int(rng.choice([0, 0, 1, 2, 3, 5]))
        colmajor = path == "e2m1" or bool(rng.random() < 0.5)
        epi = {"f16": ["bias_gelu_erf", "bias"], "bf16": ["none", "gelu_erf"],
               "i8": ["none"], "e2m1": ["none"]}[path]
        epi = epi[int(rng.integers(0, len(epi)))]
        out_t = "f32" if path in ("f16", "bf16") and rng.random() < 0.25 else None
        pad = 8 if (pad_k or rng.random() < 0.3) else 0
        if path == "e2m1":
            pad = 0
        out.append((path, M, N, K, pad_k, split, colmajor, epi, out_t, pad, seed + i))
    return out


@pytest.mark.parametrize("case", _cases(), ids=lambda c: "{}-{}x{}x{}-pk{}-s{}-{}-{}".format(
    c[0], c[1], c[2], c[3], int(c[4]), c[5], "col" if c[6] else "row", c[7]))
def test_random_problem(h, case):  # noqa: F811
    path, M, N, K, pad_k, split, colmajor, epi, out_t, pad, seed = case
    w = synth.make(RECIPE[path], M=M, N=N, K=K, seed=seed)
    o = dg.dg_plan_opts(pad_k=1 if pad_k else 0, force_split_k=split)
    run(h, w, b_colmajor=colmajor and path != "e2m1", pad=pad, opts=o, epilogue=epi, out=out_t)
