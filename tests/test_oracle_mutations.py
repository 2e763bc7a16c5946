"""Mutation check of the oracle's pins (CPU only).

Each case plants one plausible mistake in a copy of the oracle's C source (a
transposed operand, a wrong index, an exponent off by one, a dropped term or
check), builds the copy with gcc in a temporary directory, and runs the pin
tests against it in a subprocess: at least one pin must fail (pytest exit
status 1, so a build or collection error does not count as a catch).  An
unmutated copy must pass the same run, which shows that the harness itself
works.  The oracle under ``oracle/`` is never modified.  Every mistake names the
exact source text it replaces; when the oracle changes so that the text no
longer occurs once, the case fails and the list has to follow the change.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# name: (source text, replacement)
MUTATIONS = {
    # real-valued GEMM (the f16 / bf16 / e2m1 paths)
    "B read transposed": ("double v = load_real(b_kind, B, k * N + n);",
                          "double v = load_real(b_kind, B, n * K + k);"),
    "dropped last k": ("/* k ascending for every element */\n            for (int64_t k = 0; k < K; ++k) {",
                       "/* k ascending for every element */\n            for (int64_t k = 0; k < K - 1; ++k) {"),
    "D read transposed": ("v += beta * load_real(d_kind, D, i * N + n);",
                          "v += beta * load_real(d_kind, D, n * M + i);"),
    "alpha-scaled bias": ("D, i * N + n);\n                if (bias) v += load_real(bias_kind, bias, n);",
                          "D, i * N + n);\n                if (bias) v += alpha * load_real(bias_kind, bias, n);"),
    "GELU argument times sqrt 2": ("erf(x * M_SQRT1_2)", "erf(x * M_SQRT2)"),
    "e2m1 exponent off by one": ("ldexp(1.0 + 0.5 * M, E - 1)", "ldexp(1.0 + 0.5 * M, E)"),
    "e2m1 scale group halved": ("scale[(k / group_k) * N + n]", "scale[(k / group_k / 2) * N + n]"),
    # integer GEMM
    "int8 B read unsigned": ("acc[n] += a * (int64_t)bk[n];", "acc[n] += a * (int64_t)(uint8_t)bk[n];"),
    # MX block-scaled GEMM, its decoders, encoder and quantiser
    "MX A-scale block": ("SA[i * G + k / 32]", "SA[i * G + (k / 64) * 2]"),
    "MX B-scale transposed": ("orc_e8m0_value(SB[(k / 32) * N + n])", "orc_e8m0_value(SB[n * (K / 32) + k / 32])"),
    "e8m0 bias off by one": ("ldexp(1.0, (int)code - 127)", "ldexp(1.0, (int)code - 126)"),
    "fp8 subnormal exponent": ("v = ldexp((double)M, -9);", "v = ldexp((double)M, -8);"),
    "fp8 encoder without saturation": ("    if (q > 448.0) q = 448.0;\n", ""),
    "quantiser exponent off by one": ("sc = (e2 - 1) - 8 + 127;", "sc = (e2 - 1) - 7 + 127;"),
    "quantiser block maximum over 16": (
        "            for (int t = 0; t < 32; ++t) {\n                double v = orc_f16_value(xb[t]);",
        "            for (int t = 0; t < 16; ++t) {\n                double v = orc_f16_value(xb[t]);"),
    # requantise
    "requant bias before the scale": ("volatile float v = a * alpha;\n            if (bias) v = v + bias[n];",
                                      "volatile float v = (bias ? a + bias[n] : a) * alpha;"),
    "requant rounds half away from zero": ("float r = rintf(v);", "float r = roundf(v);"),
}


def _copy_tree(dst):
    """The oracle and the pin tests, with the package linked (the pins use its
    seeded input generators)."""
    os.makedirs(os.path.join(dst, "oracle"))
    for f in os.listdir(os.path.join(ROOT, "oracle")):
        if f.endswith(".py") or f.endswith(".c"):
            shutil.copy(os.path.join(ROOT, "oracle", f), os.path.join(dst, "oracle", f))
    os.makedirs(os.path.join(dst, "tests"))
    for f in ("__init__.py", "conftest.py", "parity.py", "test_oracle_pins.py"):
        if os.path.exists(os.path.join(ROOT, "tests", f)):
            shutil.copy(os.path.join(ROOT, "tests", f), os.path.join(dst, "tests", f))
    shutil.copytree(os.path.join(ROOT, "tests", "golden"), os.path.join(dst, "tests", "golden"))
    os.symlink(os.path.join(ROOT, "tile_planned_generator_amd"), os.path.join(dst, "tile_planned_generator_amd"))


def _pins_status(dst):
    """Build the copy's oracle, run the pins against it; pytest's exit status."""
    env = dict(os.environ, PYTHONPATH=dst, PYTHONDONTWRITEBYTECODE="1")
    b = subprocess.run([sys.executable, "-c", "from oracle import build; build.build()"], cwd=dst, env=env,
                       capture_output=True, text=True, timeout=300)
    assert b.returncode == 0, b.stderr[-2000:]
    r = subprocess.run([sys.executable, "-m", "pytest", "tests/test_oracle_pins.py", "-x", "-q", "-m", "not gpu",
                        "-p", "no:cacheprovider"], cwd=dst, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode, r.stdout[-3000:]


def test_unmutated_copy_passes_the_pins(tmp_path):
    dst = str(tmp_path / "copy")
    _copy_tree(dst)
    rc, out = _pins_status(dst)
    assert rc == 0, out


@pytest.mark.parametrize("name", list(MUTATIONS))
def test_planted_mistake_is_caught(tmp_path, name):
    old, new = MUTATIONS[name]
    dst = str(tmp_path / "copy")
    _copy_tree(dst)
    src = os.path.join(dst, "oracle", "oracle.c")
    with open(src) as fh:
        text = fh.read()
    assert text.count(old) == 1, f"{name}: the source text no longer occurs exactly once"
    with open(src, "w") as fh:
        fh.write(text.replace(old, new))
    rc, out = _pins_status(dst)
    assert rc == 1, f"{name}: pins exit status {rc}\n{out}"
