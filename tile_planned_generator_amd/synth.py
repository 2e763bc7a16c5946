"""Seeded synthetic inputs for the planned-GEMM workloads.

This module is the only code shared by the two sides of a parity check: it
draws input bit patterns, and both the CPU oracle and the HIP path consume the
same bits.  It holds none of the GEMM's arithmetic and imports nothing else
from this package.

Generator: SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom
number generators", OOPSLA 2014; constants as published by Vigna), used in its
counter form: draw i of a stream with seed s is mix(s + (i+1)*GAMMA).  Every
tensor has its own stream, seeded ``(workload_seed << 8) | tensor_id``.
Draws become values as:

  uniform[lo,hi)  lo + (hi-lo) * ((x >>> 11) * 2^-53)
  normal          Box-Muller, two draws per value:
                  sqrt(-2 ln u1) * cos(2 pi u2),
                  u1 = ((x0 >>> 11) + 1) * 2^-53,  u2 = (x1 >>> 11) * 2^-53
  int8            the top byte of x, as a signed value
  e2m1 code       the top 4 bits of x (uniform over the 16 codes)

Real values are rounded to the storage type in two steps, binary64 -> binary32
-> 16-bit, so the bits do not depend on the device that draws them (up to the
last bit of the transcendental functions in Box-Muller; a parity check always
hands the same drawn bits to both sides, whichever device drew them).

The workloads (shape, distribution, epilogue) follow the synthetic recipe of
the pages' workloads: the int8 4096^3 operator comparison ([overview] section
1), the FFN GEMM with a fused GELU ([overview] section 6.1), the skinny M=1 and
long-K inference shapes ([generator] section 2.1), the 4-bit weight x fp16
activation scheme ([overview] section 2.2), and a small alpha/beta check of the
"alpha * C + beta * D" epilogue ([generator] section 3.2).
"""
from dataclasses import dataclass, field

import torch

_GAMMA = 0x9E3779B97F4A7C15
_MIX1 = 0xBF58476D1CE4E5B9
_MIX2 = 0x94D049BB133111EB
_CHUNK = 1 << 25

# tensor ids within a workload
TID_A, TID_B, TID_D, TID_BIAS, TID_SCALE = 1, 2, 3, 4, 5


def _s64(x: int) -> int:
    x &= (1 << 64) - 1
    return x - (1 << 64) if x >= (1 << 63) else x


def _srl(x: torch.Tensor, s: int) -> torch.Tensor:
    """Logical right shift of int64 bit patterns."""
    return (x >> s) & ((1 << (64 - s)) - 1)


def splitmix64(seed: int, n: int, device="cpu", start: int = 0) -> torch.Tensor:
    """Draws start .. start+n-1 of the stream ``seed``, as int64 bit patterns."""
    i = torch.arange(start + 1, start + n + 1, dtype=torch.int64, device=device)
    z = i * _s64(_GAMMA) + _s64(seed)
    z = (z ^ _srl(z, 30)) * _s64(_MIX1)
    z = (z ^ _srl(z, 27)) * _s64(_MIX2)
    return z ^ _srl(z, 31)


def _chunked(n, fn, dtype, device):
    out = torch.empty(n, dtype=dtype, device=device)
    for s in range(0, n, _CHUNK):
        e = min(n, s + _CHUNK)
        out[s:e] = fn(s, e - s)
    return out


def _unit(x):
    return _srl(x, 11).to(torch.float64) * (2.0 ** -53)


def uniform(seed, n, lo, hi, device="cpu") -> torch.Tensor:
    """binary64 values in [lo, hi)."""
    return _chunked(n, lambda s, m: lo + (hi - lo) * _unit(splitmix64(seed, m, device, s)),
                    torch.float64, device)


def normal(seed, n, device="cpu") -> torch.Tensor:
    """binary64 standard normal values (Box-Muller, draws 2i and 2i+1)."""
    def f(s, m):
        x = splitmix64(seed, 2 * m, device, 2 * s)
        u1 = (_srl(x[0::2], 11) + 1).to(torch.float64) * (2.0 ** -53)
        u2 = _unit(x[1::2])
        return torch.sqrt(-2.0 * torch.log(u1)) * torch.cos((2.0 * torch.pi) * u2)
    return _chunked(n, f, torch.float64, device)


def int8_uniform(seed, n, device="cpu") -> torch.Tensor:
    """int8 values uniform over [-128, 127] (the top byte of each draw)."""
    return _chunked(n, lambda s, m: (splitmix64(seed, m, device, s) >> 56).to(torch.int8),
                    torch.int8, device)


def e2m1_codes(seed, n, device="cpu") -> torch.Tensor:
    """4-bit codes uniform over 0..15, one per uint8."""
    return _chunked(n, lambda s, m: _srl(splitmix64(seed, m, device, s), 60).to(torch.uint8),
                    torch.uint8, device)


def int_range(seed, n, lo, hi, device="cpu") -> torch.Tensor:
    """Integers uniform over [lo, hi] (the high 32 bits of each draw, modulo the
    range; the bias of the modulus is below 2^-24 for the small ranges used)."""
    span = hi - lo + 1
    return _chunked(n, lambda s, m: (_srl(splitmix64(seed, m, device, s), 32) % span + lo)
                    .to(torch.int32), torch.int32, device)


def fp8_codes(seed, n, device="cpu") -> torch.Tensor:
    """8-bit codes uniform over the 254 codes whose low seven bits are not all ones
    (in fp8 e4m3 those two codes are NaN), one per uint8."""
    return _chunked(n, lambda s, m: (lambda u: (u + (u >= 127).to(torch.int64)).to(torch.uint8))(
        _srl(splitmix64(seed, m, device, s), 32) % 254), torch.uint8, device)


def to_storage(x: torch.Tensor, dtype: torch.dtype) -> torch.Tensor:
    """binary64 -> binary32 -> 16-bit storage type (each step nearest-even)."""
    return x.to(torch.float32).to(dtype)


# ----------------------------------------------------------------- workloads
@dataclass
class Workload:
    name: str
    path: str                 # "f16", "bf16", "i8", "e2m1"
    M: int
    N: int
    K: int
    alpha: float = 1.0
    beta: float = 0.0
    epilogue: str = "none"    # "none", "bias", "gelu_erf", "bias_gelu_erf", "requant_i8", ...
    out: str = "f16"          # output storage type
    group_k: int = 32         # e2m1 scale group along K
    seed: int = 0
    tensors: dict = field(default_factory=dict)


# name -> (path, M, N, K, seed, alpha, beta, epilogue, out)
WORKLOADS = {
    "f16_256x256x256_alpha_beta_d": ("f16", 256, 256, 256, 101, 1.0, 0.5, "none", "f16"),
    "i8_4096x4096x4096": ("i8", 4096, 4096, 4096, 202, 1, 0, "none", "i32"),
    "f16_2048x2048x8192_bias_gelu": ("f16", 2048, 2048, 8192, 303, 1.0, 0.0, "bias_gelu_erf",
                                     "f16"),
    "bf16_1x4096x131072": ("bf16", 1, 4096, 131072, 404, 1.0, 0.0, "none", "bf16"),
    "bf16_16x4096x131072": ("bf16", 16, 4096, 131072, 405, 1.0, 0.0, "none", "bf16"),
    "bf16_1x256x12800": ("bf16", 1, 256, 12800, 406, 1.0, 0.0, "none", "bf16"),
    "e2m1_1x4096x4096": ("e2m1", 1, 4096, 4096, 501, 1.0, 0.0, "none", "f16"),
    "e2m1_4096x4096x4096": ("e2m1", 4096, 4096, 4096, 502, 1.0, 0.0, "none", "f16"),
    "f16_4096x4096x4096": ("f16", 4096, 4096, 4096, 901, 1.0, 0.0, "none", "f16"),
    "mx_4096x4096x4096": ("mx", 4096, 4096, 4096, 601, 1.0, 0.0, "none", "f16"),
    "mxq_4096x4096": ("mxq", 4096, 0, 4096, 602, 1.0, 0.0, "none", "u8"),
}


def _sid(seed, tid):
    return (seed << 8) | tid


def make(name: str, device="cpu", M=None, N=None, K=None, seed=None) -> Workload:
    """Draw the inputs of a named workload; M, N, K, seed may be overridden to get
    the same recipe at another size (parity cases)."""
    path, M0, N0, K0, seed0, alpha, beta, epi, out = WORKLOADS[name]
    M = M0 if M is None else M
    N = N0 if N is None else N
    K = K0 if K is None else K
    seed = seed0 if seed is None else seed
    w = Workload(name, path, M, N, K, alpha, beta, epi, out, seed=seed)
    t = w.tensors
    if name.startswith("f16_256"):
        t["A"] = to_storage(uniform(_sid(seed, TID_A), M * K, -1, 1, device), torch.float16).view(M, K)
        t["B"] = to_storage(uniform(_sid(seed, TID_B), K * N, -1, 1, device), torch.float16).view(K, N)
        t["D"] = to_storage(uniform(_sid(seed, TID_D), M * N, -1, 1, device), torch.float16).view(M, N)
    elif path == "i8":
        t["A"] = int8_uniform(_sid(seed, TID_A), M * K, device).view(M, K)
        t["B"] = int8_uniform(_sid(seed, TID_B), K * N, device).view(K, N)
    elif path in ("f16", "bf16"):
        dt = torch.float16 if path == "f16" else torch.bfloat16
        s = 1.0 / (K ** 0.5) if K > 0 else 1.0
        t["A"] = to_storage(normal(_sid(seed, TID_A), M * K, device) * s, dt).view(M, K)
        t["B"] = to_storage(normal(_sid(seed, TID_B), K * N, device) * s, dt).view(K, N)
        if "bias" in epi:
            t["bias"] = to_storage(uniform(_sid(seed, TID_BIAS), N, -0.1, 0.1, device), dt)
    elif path == "e2m1":
        G = K // w.group_k
        t["A"] = to_storage(normal(_sid(seed, TID_A), M * K, device), torch.float16).view(M, K)
        t["codes"] = e2m1_codes(_sid(seed, TID_B), K * N, device).view(K, N)
        t["scale"] = to_storage(uniform(_sid(seed, TID_SCALE), G * N, 0.01, 0.1, device),
                                torch.float16).view(G, N)
    elif path == "mx":
        # fp8 e4m3 activation codes with e8m0 scales 2^-15..2^-9 per 32 values of a
        # row, e2m1 weight codes with e8m0 scales 2^-8..2^-4 per 32 values of a
        # column: products stay near 1e-2 and the K sums well inside fp16's range.
        G = K // 32
        t["A"] = fp8_codes(_sid(seed, TID_A), M * K, device).view(M, K)
        t["SA"] = int_range(_sid(seed, TID_D), M * G, 112, 118, device).to(torch.uint8).view(M, G)
        t["codes"] = e2m1_codes(_sid(seed, TID_B), K * N, device).view(K, N)
        t["SB"] = int_range(_sid(seed, TID_SCALE), G * N, 119, 123, device).to(torch.uint8).view(G, N)
    elif path == "mxq":
        # fp16 activations for the MX quantiser: normal values times a per-row
        # magnitude 2^u, u uniform in [-6, 6], so blocks take many scale codes
        z = normal(_sid(seed, TID_A), M * K, device).view(M, K)
        u = int_range(_sid(seed, TID_SCALE), M, -6, 6, device).to(torch.float64)
        t["X"] = to_storage(z * torch.pow(2.0, u).view(M, 1), torch.float16)
    else:
        raise KeyError(name)
    return w
