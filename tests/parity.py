"""Parity helpers shared by the GPU tests, the smoke check and the benchmark.

Comparison rule (floating point): with r the unrounded binary64 oracle result
and s = RMS(r) over the compared outputs, the guarded relative error of an
output c is e = |c - r| / max(|r|, s).
  - fp16 and fp32 outputs: max e <= 2e-3;
  - bf16 outputs: ||c - r||_F / ||r||_F <= 2e-3 and max e <= 2^-7 (one bf16
    unit in the last place: bf16 keeps 8 significand bits, so even a
    correctly rounded bf16 output can sit 2^-8 from r, and an elementwise 2e-3
    is out of reach for any implementation);
  - e2m1-weight paths: max e <= 1e-2.
The guard max(|r|, s) keeps outputs near zero (where any rounding is a large
relative error) from deciding the verdict.  Integer outputs compare bit for
bit.
"""
import sys

import numpy as np
import torch

import oracle

TOL_F16 = 2e-3
TOL_BF16_NORM = 2e-3
TOL_BF16_ELT = 2.0 ** -7
TOL_E2M1 = 1e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bits(t: torch.Tensor) -> np.ndarray:
    """Host numpy view of a tensor's bit patterns (16-bit types as uint16)."""
    t = t.detach().contiguous().cpu()
    if t.dtype in (torch.float16, torch.bfloat16):
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def kind(t: torch.Tensor) -> str:
    return {torch.float16: "f16", torch.bfloat16: "bf16", torch.float32: "f32", torch.int8: "i8",
            torch.int32: "i32", torch.uint8: "e2m1"}[t.dtype]


def out_values(c: torch.Tensor) -> np.ndarray:
    return oracle.values(bits(c), kind(c))


def fp_errors(c: np.ndarray, r: np.ndarray) -> dict:
    c = np.asarray(c, np.float64)
    r = np.asarray(r, np.float64)
    s = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
    guard = np.maximum(np.abs(r), max(s, 1e-300))
    e = np.abs(c - r) / guard
    big = np.abs(r) >= s
    unguarded = float(np.max(np.abs(c - r)[big] / np.abs(r)[big])) if big.any() else 0.0
    nr = float(np.linalg.norm(r))
    norm = float(np.linalg.norm(c - r) / nr) if nr > 0 else float(np.linalg.norm(c - r))
    return {"max_guarded": float(e.max()) if e.size else 0.0, "max_unguarded": unguarded,
            "normwise": norm, "nonfinite": int((~np.isfinite(c)).sum()), "n": int(c.size)}


def check_fp(c_tensor: torch.Tensor, r: np.ndarray, tol: str) -> dict:
    c = out_values(c_tensor)
    st = fp_errors(c, r)
    assert st["nonfinite"] == 0, st
    if tol == "bf16":
        assert st["normwise"] <= TOL_BF16_NORM and st["max_guarded"] <= TOL_BF16_ELT, st
    elif tol == "e2m1":
        assert st["max_guarded"] <= TOL_E2M1, st
    else:
        assert st["max_guarded"] <= TOL_F16, st
    return st


def tol_for(path: str, out: str) -> str:
    if path == "e2m1":
        return "e2m1"
    return "bf16" if out == "bf16" else "f16"
