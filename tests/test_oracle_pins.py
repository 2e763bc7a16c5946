"""Pins of the CPU oracle against things other than itself.

Each check is independent of the oracle's code: exact rational arithmetic
(``fractions.Fraction``) on small inputs drawn by the shared generator,
exhaustive codec comparisons against numpy's binary16 and a bit-level bfloat16
definition, closed forms (identity, permutation, rank one), invariants
(linearity in alpha and beta, GELU's odd-part identity, thread-count
determinism), a high-precision Taylor series for erf, and the fixtures under
``tests/golden/`` with their citations.  A dropped term, a wrong sign, a
swapped index or a transposed operand in the oracle fails one of them.
"""
import math
import os
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from tile_planned_generator_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------- helpers
def f16_exact(bits):
    """Exact rational value of a binary16 bit pattern (independent decoder)."""
    bits = int(bits)
    s = -1 if bits & 0x8000 else 1
    e = (bits >> 10) & 31
    f = bits & 1023
    assert e != 31
    if e == 0:
        return s * Fraction(f, 1 << 24)
    return s * Fraction(1024 + f, 1 << 10) * (Fraction(2) ** (e - 15))


def bf16_exact(bits):
    bits = int(bits)
    s = -1 if bits & 0x8000 else 1
    e = (bits >> 7) & 255
    f = bits & 127
    assert e != 255
    if e == 0:
        return s * Fraction(f, 128) * (Fraction(2) ** -126)
    return s * Fraction(128 + f, 128) * (Fraction(2) ** (e - 127))


def e2m1_golden():
    vals = {}
    with open(os.path.join(GOLDEN, "e2m1_values.txt")) as fh:
        for line in fh:
            if line.startswith("#") or not line.strip():
                continue
            c, v = line.split()
            vals[int(c)] = float(v)
    return vals


def bits16(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


# ------------------------------------------------------------------ codecs
def test_f16_decode_exhaustive_vs_numpy():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.f16_values(bits)
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_bf16_decode_exhaustive_vs_bit_definition():
    bits = np.arange(65536, dtype=np.uint32)
    ours = oracle.bf16_values(bits.astype(np.uint16))
    ref = (bits << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    # and against the independent rational decoder on all finite patterns
    for b in range(0, 65536, 97):
        if not nan[b] and not np.isinf(ref[b]):
            assert Fraction(ours[b]) == bf16_exact(b)


def test_f16_decode_matches_rational_decoder():
    for b in range(0, 65536, 13):
        if (b >> 10) & 31 == 31:
            continue
        assert Fraction(oracle.f16_values(np.array([b], np.uint16))[0]) == f16_exact(b)


def test_f16_rne_vs_numpy_random_and_ties():
    rng = np.random.default_rng(7)
    x = np.concatenate([
        rng.standard_normal(200000) * 10.0 ** rng.integers(-9, 5, 200000),
        rng.uniform(-70000, 70000, 20000),
        rng.uniform(-2.0 ** -14, 2.0 ** -14, 20000),            # subnormal range
    ])
    # exact midpoints between adjacent binary16 values (ties to even)
    h = np.arange(0, 0x7bff, 3, dtype=np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).view(np.float16).astype(np.float64)
    mids = (lo + hi) / 2
    x = np.concatenate([x, mids, -mids])
    ours = oracle.f16_rne(x)
    ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(ours, ref)


def test_f16_rne_handpicked():
    cases = {
        1 + 2.0 ** -11: 0x3C00,          # tie -> even (1.0)
        1 + 3 * 2.0 ** -11: 0x3C02,      # tie -> even (1 + 2^-9)
        65504.0: 0x7BFF,
        65519.99: 0x7BFF,
        65520.0: 0x7C00,                 # rounds past the largest finite -> inf
        2.0 ** -25: 0x0000,              # half the smallest subnormal -> even (0)
        3 * 2.0 ** -25: 0x0002,          # 1.5 * 2^-24 -> 2 * 2^-24
        2.0 ** -24: 0x0001,
        -0.0: 0x8000,
        6.103515625e-05: 0x0400,         # 2^-14, smallest normal
    }
    for x, b in cases.items():
        assert int(oracle.f16_rne(np.array([x]))[0]) == b, x


def test_bf16_rne_vs_torch_on_binary32_inputs():
    rng = np.random.default_rng(11)
    x32 = (rng.standard_normal(300000) * 10.0 ** rng.integers(-30, 30, 300000)).astype(np.float32)
    # exact midpoints between bfloat16 neighbours
    b = np.arange(0, 0x7F7F, 7, dtype=np.uint32)
    lo = (b << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    hi = ((b + 1) << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    mids = ((lo + hi) / 2).astype(np.float32)   # exact in binary32
    x32 = np.concatenate([x32, mids, -mids])
    ours = oracle.bf16_rne(x32.astype(np.float64))
    ref = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_e2m1_table_exhaustive():
    gold = e2m1_golden()
    got = oracle.e2m1_values(np.arange(16, dtype=np.uint8))
    for c in range(16):
        assert got[c] == gold[c]
        assert np.signbit(got[c]) == (c >= 8)
        # closed form of the fields: sign, exponent E (bias 1), mantissa M
        s, E, M = (c >> 3) & 1, (c >> 1) & 3, c & 1
        mag = Fraction(M, 2) if E == 0 else Fraction(2) ** (E - 1) * (1 + Fraction(M, 2))
        assert Fraction(abs(got[c])) == mag
        assert (-1 if s else 1) * mag == Fraction(got[c]) or mag == 0
    # only the low nibble is a code
    assert np.array_equal(oracle.e2m1_values(np.arange(16, 32, dtype=np.uint8)), got)


# ------------------------------------------------------------------ GELU / erf
def _erf_decimal(x: Decimal) -> Decimal:
    getcontext().prec = 60
    pi = Decimal("3.14159265358979323846264338327950288419716939937510582097494")
    s, term, n = Decimal(0), x, 0
    while True:
        t = term / (2 * n + 1)
        s += t if n % 2 == 0 else -t
        n += 1
        term = term * x * x / n
        if abs(term) < Decimal(10) ** -50:
            break
    return 2 / pi.sqrt() * s


def test_gelu_golden_and_identities():
    with open(os.path.join(GOLDEN, "gelu_values.txt")) as fh:
        rows = [l.split() for l in fh if l.strip() and not l.startswith("#")]
    for x, g in rows:
        got = oracle.gelu_erf(np.array([float(x)]))[0]
        assert abs(got - float(g)) <= 2 * np.spacing(abs(float(g)))
    assert oracle.gelu_erf(np.array([0.0]))[0] == 0.0
    x = np.linspace(-7, 7, 2001)
    d = oracle.gelu_erf(x) - oracle.gelu_erf(-x)
    assert np.max(np.abs(d - x)) <= 4 * np.spacing(7.0)
    big = np.linspace(8, 60, 101)
    assert np.max(np.abs(oracle.gelu_erf(big) - big) / big) < 1e-12
    # GELU(x) -> 0 from below as x -> -inf
    assert np.all(oracle.gelu_erf(-big) <= 0) and np.max(np.abs(oracle.gelu_erf(-big))) < 1e-12


def test_gelu_against_decimal_erf_series():
    getcontext().prec = 60
    r2 = Decimal(2).sqrt()
    for xv in np.linspace(-3, 3, 61):
        x = Decimal(repr(float(xv)))
        ref = x / 2 * (1 + _erf_decimal(x / r2))
        got = Decimal(repr(float(oracle.gelu_erf(np.array([float(xv)]))[0])))
        assert abs(got - ref) <= Decimal(4e-16) * max(Decimal(1), abs(ref)), xv


# ------------------------------------------------ GEMM: rational brute force
SHAPES = [(1, 1, 1), (2, 3, 5), (3, 5, 2), (5, 8, 17), (8, 17, 3), (17, 2, 8)]


def _frac_gemm(Av, Bv):
    M, K = len(Av), len(Av[0])
    N = len(Bv[0])
    return [[sum((Av[i][k] * Bv[k][j] for k in range(K)), Fraction(0)) for j in range(N)]
            for i in range(M)]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_f16_gemm_alpha_beta_d_exact(M, N, K):
    w = synth.make("f16_256x256x256_alpha_beta_d", M=M, N=N, K=K)
    A, B, D = (bits16(w.tensors[k]) for k in ("A", "B", "D"))
    R = oracle.gemm_real(A, B, a_kind="f16", b_kind="f16", alpha=1.0, beta=0.5, D=D, d_kind="f16")
    Av = [[f16_exact(A[i, k]) for k in range(K)] for i in range(M)]
    Bv = [[f16_exact(B[k, j]) for j in range(N)] for k in range(K)]
    S = _frac_gemm(Av, Bv)
    for i in range(M):
        for j in range(N):
            exact = S[i][j] + Fraction(1, 2) * f16_exact(D[i, j])
            # the sum of <= 17 products of binary16 values is exact in binary64, and
            # the beta*D addition is the only rounding: the result is correctly rounded
            assert R[i, j] == float(exact), (i, j)


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_bf16_gemm_bias_exact_within_rounding(M, N, K):
    w = synth.make("bf16_1x4096x131072", M=M, N=N, K=K)
    A, B = bits16(w.tensors["A"]), bits16(w.tensors["B"])
    bias = bits16(synth.to_storage(synth.uniform(99, N, -0.1, 0.1), torch.bfloat16))
    R = oracle.gemm_real(A, B, a_kind="bf16", b_kind="bf16", bias=bias, bias_kind="bf16",
                         alpha=2.0)
    Av = [[bf16_exact(A[i, k]) for k in range(K)] for i in range(M)]
    Bv = [[bf16_exact(B[k, j]) for j in range(N)] for k in range(K)]
    S = _frac_gemm(Av, Bv)
    for i in range(M):
        for j in range(N):
            exact = 2 * S[i][j] + bf16_exact(bias[j])
            mag = 2 * sum(abs(Av[i][k] * Bv[k][j]) for k in range(K)) + abs(bf16_exact(bias[j]))
            # at most K+1 binary64 roundings, each below 2^-53 of the running magnitude
            assert abs(Fraction(R[i, j]) - exact) <= (K + 2) * Fraction(1, 2 ** 53) * mag


@pytest.mark.parametrize("M,N,K", [(1, 1, 32), (2, 3, 32), (3, 5, 64), (4, 2, 96)])
def test_e2m1_gemm_exact(M, N, K):
    w = synth.make("e2m1_4096x4096x4096", M=M, N=N, K=K)
    A = bits16(w.tensors["A"])
    codes = w.tensors["codes"].numpy()
    scale = bits16(w.tensors["scale"])
    R = oracle.gemm_real(A, codes, a_kind="f16", b_kind="e2m1", scale=scale, group_k=32)
    gold = e2m1_golden()
    for i in range(M):
        for j in range(N):
            terms = [f16_exact(A[i, k]) * Fraction(gold[int(codes[k, j])]) *
                     f16_exact(scale[k // 32, j]) for k in range(K)]
            exact = sum(terms, Fraction(0))
            mag = sum(abs(t) for t in terms)
            assert abs(Fraction(R[i, j]) - exact) <= (K + 1) * Fraction(1, 2 ** 53) * mag


def test_e2m1_scale_group_index():
    # one non-zero weight per group: the result picks exactly that group's scale
    K, N = 96, 3
    codes = np.zeros((K, N), np.uint8)
    scale = np.zeros((K // 32, N), np.uint16)
    for g in range(K // 32):
        for j in range(N):
            scale[g, j] = oracle.f16_rne(np.array([2.0 ** -(g + 3 * j)]))[0]
    codes[40, 1] = 7        # 6.0 in group 1
    A = np.zeros((1, K), np.uint16)
    A[0, 40] = 0x3C00       # 1.0
    R = oracle.gemm_real(A, codes, a_kind="f16", b_kind="e2m1", scale=scale, group_k=32)
    assert R[0, 1] == 6.0 * 2.0 ** -(1 + 3)
    assert R[0, 0] == 0 and R[0, 2] == 0


@pytest.mark.parametrize("M,N,K", SHAPES + [(4, 7, 64)])
def test_int_gemm_vs_python_ints(M, N, K):
    w = synth.make("i8_4096x4096x4096", M=M, N=N, K=K)
    A, B = w.tensors["A"].numpy(), w.tensors["B"].numpy()
    D = np.arange(M * N, dtype=np.int32).reshape(M, N) * 7919 - 50000
    R, Cw, ov = oracle.gemm_int(A, B, alpha=3, beta=-2, D=D)
    assert ov == 0
    for i in range(M):
        for j in range(N):
            acc = sum(int(A[i, k]) * int(B[k, j]) for k in range(K))
            assert R[i, j] == 3 * acc - 2 * int(D[i, j])
            assert Cw[i, j] == R[i, j]


def test_int_overflow_flag_and_wrap():
    K = 131072
    A = np.full((1, K), -128, np.int8)
    B = np.full((K, 1), -128, np.int8)
    R, Cw, ov = oracle.gemm_int(A, B)
    assert R[0, 0] == 2 ** 31 and ov == 1
    assert Cw[0, 0] == -(2 ** 31)              # wrapped modulo 2^32
    # extremes inside the range
    A = np.full((1, 4096), 127, np.int8)
    B = np.full((4096, 1), -128, np.int8)
    R, Cw, ov = oracle.gemm_int(A, B)
    assert R[0, 0] == -66584576 and Cw[0, 0] == -66584576 and ov == 0
    A = np.full((1, 4096), -128, np.int8)
    R, Cw, ov = oracle.gemm_int(A, B)
    assert R[0, 0] == 2 ** 26 and ov == 0


# ------------------------------------------------ closed forms and invariants
@pytest.mark.parametrize("kind", ["f16", "bf16"])
def test_identity_and_permutation(kind):
    M, K = 9, 24
    dt = torch.float16 if kind == "f16" else torch.bfloat16
    A = bits16(synth.to_storage(synth.normal(5, M * K), dt).view(M, K))
    one = 0x3C00 if kind == "f16" else 0x3F80
    I = np.zeros((K, K), np.uint16)
    I[np.arange(K), np.arange(K)] = one
    R = oracle.gemm_real(A, I, a_kind=kind, b_kind=kind)
    assert np.array_equal(R, oracle.values(A, kind))
    perm = np.random.default_rng(3).permutation(K)
    P = np.zeros((K, K), np.uint16)
    P[np.arange(K), perm] = one          # (A.P)[:, perm[k]] = A[:, k]
    R = oracle.gemm_real(A, P, a_kind=kind, b_kind=kind)
    Av = oracle.values(A, kind)
    assert np.array_equal(R[:, perm], Av)


def test_rank_one_closed_form():
    M, N, K = 6, 5, 1000
    x = np.array([1, -2, 0.5, 4, -0.25, 3])
    y = np.array([2, -1, 0.125, -8, 1])
    A = np.repeat(oracle.f16_rne(x)[:, None], K, axis=1)
    B = np.repeat(oracle.f16_rne(y)[None, :], K, axis=0)
    R = oracle.gemm_real(A, B, a_kind="f16", b_kind="f16")
    assert np.array_equal(R, K * np.outer(x, y))
    # int8 rank one
    xi = np.array([127, -128, 1, 0], np.int8)
    yi = np.array([-128, 127, 5], np.int8)
    Ri, Ci, ov = oracle.gemm_int(np.repeat(xi[:, None], K, 1), np.repeat(yi[None, :], K, 0))
    assert np.array_equal(Ri, K * np.outer(xi.astype(np.int64), yi.astype(np.int64)))
    assert ov == 0


def test_alpha_beta_linearity_and_bias_gelu_order():
    w = synth.make("f16_256x256x256_alpha_beta_d", M=7, N=9, K=33)
    A, B, D = (bits16(w.tensors[k]) for k in ("A", "B", "D"))
    base = oracle.gemm_real(A, B, a_kind="f16", b_kind="f16")
    Dv = oracle.values(D, "f16")
    for alpha, beta in [(2.0, 0.25), (-0.5, 4.0), (1.0, -1.0)]:
        R = oracle.gemm_real(A, B, a_kind="f16", b_kind="f16", alpha=alpha, beta=beta, D=D)
        # power-of-two alpha and beta scale exactly; one rounding in the sum
        assert np.array_equal(R, alpha * base + beta * Dv)
    # beta = 0 does not read D
    R0 = oracle.gemm_real(A, B, a_kind="f16", b_kind="f16", beta=0.0, D=None)
    assert np.array_equal(R0, base)
    # the bias is added before the activation, unscaled by alpha
    bias = oracle.f16_rne(np.linspace(-1, 1, 9))
    Rb = oracle.gemm_real(A, B, a_kind="f16", b_kind="f16", alpha=2.0, bias=bias, act=1)
    pre = 2.0 * base + oracle.values(bias, "f16")[None, :]
    assert np.array_equal(Rb, oracle.gelu_erf(pre))


def _rne_fraction(x: Fraction, p: int, emin: int, maxv: Fraction):
    """Exact round-to-nearest-even of a rational to a binary format with p
    significand bits and minimum normal exponent emin (Python's round() on a
    Fraction rounds halves to even); None past the overflow threshold."""
    if x == 0:
        return Fraction(0)
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    ulp = Fraction(2) ** (max(e, emin) - (p - 1))
    q = round(a / ulp) * ulp
    if q > maxv:
        return None
    return q if x > 0 else -q


F32_MAX = (2 - Fraction(1, 2 ** 23)) * Fraction(2) ** 127


def _f32(x: Fraction) -> Fraction:
    return _rne_fraction(x, 24, -126, F32_MAX)


def _requant_exact(acc: int, alpha: Fraction, bias, out: str):
    """The requantise rule written out in exact rationals: v = f32(f32(f32(acc) *
    alpha) + bias), then int8: round half to even and saturate, or fp16: round
    half to even (as a rational, or +-inf)."""
    v = _f32(_f32(_f32(Fraction(acc)) * alpha) + (bias if bias is not None else 0))
    if out == "i8":
        return max(-128, min(127, round(v)))
    q = _rne_fraction(v, 11, -14, Fraction(65504))
    return q if q is not None else (math.inf if v > 0 else -math.inf)


def test_requant_against_exact_rational_steps():
    # Each binary32 step rounded exactly with Fractions (no floating-point
    # arithmetic of the host in the expected values): accumulators across the
    # whole int32 range, so f32(acc) and the product round; scales that are and
    # are not powers of two; a bias that does and does not change the rounding.
    acc = [int(v) for v in synth.int_range(91, 160, -2 ** 31, 2 ** 31 - 1).numpy()]
    acc[:8] = [5, 7, -5, 2049, 2051, 1000, 2 ** 24 + 1, -(2 ** 31)]
    bias_vals = [Fraction(float(b)) for b in np.float32(synth.uniform(92, 160, -3, 3).numpy())]
    for alpha in (0.5, 1.0, 3.0517578125e-05, 1.7e-6, 0.3):
        a32 = _f32(Fraction(alpha))
        A = np.array(acc, np.int32).reshape(16, 10)
        Bv = np.array([float(b) for b in bias_vals[:10]], np.float32)
        got_i8 = oracle.requant(A, alpha=alpha, bias=Bv, out="i8")
        got_f16 = oracle.f16_values(oracle.requant(A, alpha=alpha, out="f16"))
        for i in range(16):
            for j in range(10):
                want = _requant_exact(int(A[i, j]), a32, Fraction(float(Bv[j])), "i8")
                assert int(got_i8[i, j]) == want, (alpha, int(A[i, j]), float(Bv[j]))
                wf = _requant_exact(int(A[i, j]), a32, None, "f16")
                assert got_f16[i, j] == float(wf), (alpha, int(A[i, j]))


def test_requant_exact_cases_round_the_real_value_once():
    # With a power-of-two scale, |acc| < 2^24 and a bias on a coarse grid, every
    # binary32 step is exact: the result is the rounding of the real value
    # alpha * acc + bias itself - ties to even, saturation at -128 and 127, and
    # fp16 ties and overflow.
    acc = np.array([[5, 7, -5, -7, 1, 3, 1000, -1000, 255, -257, 2 ** 23, -(2 ** 23)]], np.int32)
    for k in (1, 2, 4):
        alpha = 2.0 ** -k
        for bias in (0.0, 0.25, -0.75, 1.5):
            q = oracle.requant(acc, alpha=alpha, bias=np.full(acc.shape[1], bias, np.float32), out="i8")
            for j, a in enumerate(acc[0].tolist()):
                exact = Fraction(a, 2 ** k) + Fraction(bias)
                assert int(q[0, j]) == max(-128, min(127, round(exact))), (a, k, bias)
    # ties to even and saturation, by hand
    q = oracle.requant(np.array([[5, 7, -5, 1000, -1000]], np.int32), alpha=0.5, out="i8")
    assert q.tolist() == [[2, 4, -2, 127, -128]]
    # fp16: 2049 and 2051 lie halfway between fp16 neighbours (spacing 2 above
    # 2048); 65519 rounds down to 65504 and 65520 up to infinity
    h = oracle.requant(np.array([[2049, 2051, 65519, 65520, -65520]], np.int32), alpha=1.0, out="f16")
    assert oracle.f16_values(h).tolist() == [[2048.0, 2052.0, 65504.0, math.inf, -math.inf]]


def test_thread_count_determinism():
    w = synth.make("f16_2048x2048x8192_bias_gelu", M=64, N=48, K=512)
    A, B, bias = (bits16(w.tensors[k]) for k in ("A", "B", "bias"))
    r1 = oracle.gemm_real(A, B, a_kind="f16", b_kind="f16", bias=bias, act=1, nthreads=1)
    r8 = oracle.gemm_real(A, B, a_kind="f16", b_kind="f16", bias=bias, act=1, nthreads=8)
    assert r1.tobytes() == r8.tobytes()
    wi = synth.make("i8_4096x4096x4096", M=33, N=65, K=300)
    a, b = wi.tensors["A"].numpy(), wi.tensors["B"].numpy()
    assert oracle.gemm_int(a, b, nthreads=1)[1].tobytes() == oracle.gemm_int(a, b, nthreads=7)[1].tobytes()


def test_empty_shapes():
    R = oracle.gemm_real(np.zeros((0, 4), np.uint16), np.zeros((4, 3), np.uint16),
                         a_kind="f16", b_kind="f16")
    assert R.shape == (0, 3)
    R = oracle.gemm_real(np.zeros((2, 0), np.uint16), np.zeros((0, 3), np.uint16),
                         a_kind="f16", b_kind="f16")
    assert np.array_equal(R, np.zeros((2, 3)))


# -------------------------------------------------- the shared input generator
def test_splitmix64_published_vector():
    # SplitMix64 seeded with 0: the first outputs of the reference generator
    x = synth.splitmix64(0, 3)
    got = [v & (2 ** 64 - 1) for v in x.tolist()]
    assert got == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_splitmix64_counter_form_matches_sequential_python():
    seed = (303 << 8) | 2
    mask = 2 ** 64 - 1
    state, seq = seed, []
    for _ in range(50):
        state = (state + 0x9E3779B97F4A7C15) & mask
        z = state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & mask
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & mask
        seq.append(z ^ (z >> 31))
    got = [v & mask for v in synth.splitmix64(seed, 50).tolist()]
    assert got == seq
    assert [v & mask for v in synth.splitmix64(seed, 20, start=30).tolist()] == seq[30:]


def test_generator_distributions():
    u = synth.uniform(1, 200000, -1, 1)
    assert u.min() >= -1 and u.max() < 1 and abs(float(u.mean())) < 0.01
    z = synth.normal(2, 200000)
    assert abs(float(z.mean())) < 0.01 and abs(float(z.std()) - 1) < 0.01
    i = synth.int8_uniform(3, 200000)
    assert int(i.min()) == -128 and int(i.max()) == 127
    c = synth.e2m1_codes(4, 160000)
    counts = torch.bincount(c.to(torch.int64), minlength=16)
    assert counts.numel() == 16 and int(counts.min()) > 9000


# ------------------------------------------------------- MX block-scaled path
def _fp8_torch(codes):
    """fp8 e4m3 values decoded by torch's float8_e4m3fn (an independent decoder)."""
    return torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(torch.float8_e4m3fn) \
        .to(torch.float64).numpy()


def test_fp8e4m3_decode_exhaustive_vs_torch():
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.fp8e4m3_values(codes)
    ref = _fp8_torch(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan) and set(np.flatnonzero(nan)) == {0x7F, 0xFF}
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), codes[~nan] >= 128)
    # the format's landmarks: 1.0, largest normal, smallest normal and subnormal
    assert got[0x38] == 1.0 and got[0x7E] == 448.0 and got[0x08] == 2.0 ** -6
    assert got[0x01] == 2.0 ** -9 and got[0x07] == 7 * 2.0 ** -9


def test_e8m0_decode_exhaustive_vs_torch():
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.e8m0_values(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert np.isnan(got[255]) and np.isnan(ref[255])
    assert np.array_equal(got[:255], ref[:255])
    assert got[127] == 1.0 and got[0] == 2.0 ** -127 and got[254] == 2.0 ** 127


def test_fp8_rne_sat_vs_torch_and_ties():
    z = synth.normal(71, 20000).numpy() * np.exp2(synth.int_range(72, 20000, -12, 8).numpy())
    z = z.astype(np.float32).astype(np.float64)          # torch converts from binary32
    inr = np.abs(z) <= 448
    got = oracle.fp8e4m3_rne_sat(z)
    ref = torch.from_numpy(z[inr].astype(np.float32)).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy()
    assert np.array_equal(got[inr], ref)
    assert np.all(got[(~inr) & (z > 0)] == 0x7E) and np.all(got[(~inr) & (z < 0)] == 0xFE)
    # ties go to the even mantissa; past the largest normal the result saturates
    cases = [(1 + 1 / 16, 0x38), (1 + 3 / 16, 0x3A), (-(1 + 1 / 16), 0xB8), (2.0 ** -10, 0x00),
             (3 * 2.0 ** -10, 0x02), (464.0, 0x7E), (1e6, 0x7E), (-1e6, 0xFE), (0.0, 0x00),
             (-0.0, 0x80)]
    for x, c in cases:
        assert int(oracle.fp8e4m3_rne_sat(np.array([x]))[0]) == c, x


def _mx_inputs(M, N, K, seed=601):
    w = synth.make("mx_4096x4096x4096", M=M, N=N, K=K, seed=seed)
    t = w.tensors
    return t["A"].numpy(), t["SA"].numpy(), t["codes"].numpy(), t["SB"].numpy()


@pytest.mark.parametrize("M,N,K", [(1, 1, 32), (2, 3, 64), (3, 5, 96), (4, 2, 128)])
def test_mx_gemm_exact(M, N, K):
    A, SA, Bc, SB = _mx_inputs(M, N, K)
    R = oracle.gemm_mx(A, SA, Bc, SB)
    av = _fp8_torch(A)
    gold = e2m1_golden()
    for i in range(M):
        for j in range(N):
            terms = [Fraction(av[i, k]) * Fraction(2) ** (int(SA[i, k // 32]) - 127) *
                     Fraction(gold[int(Bc[k, j])]) * Fraction(2) ** (int(SB[k // 32, j]) - 127)
                     for k in range(K)]
            exact = sum(terms, Fraction(0))
            mag = sum(abs(t) for t in terms)
            assert abs(Fraction(R[i, j]) - exact) <= (K + 1) * Fraction(1, 2 ** 53) * mag


def test_mx_scale_block_index():
    # one non-zero product per block: the result picks exactly that block's two scales
    K, M, N = 96, 2, 3
    A = np.zeros((M, K), np.uint8)
    Bc = np.zeros((K, N), np.uint8)
    SA = np.array([[127 + g + 3 * i for g in range(K // 32)] for i in range(M)], np.uint8)
    SB = np.array([[120 - g - 4 * j for j in range(N)] for g in range(K // 32)], np.uint8)
    A[1, 70] = 0x40            # 2.0, in block 2
    Bc[70, 2] = 7              # 6.0
    A[0, 40] = 0x38            # 1.0, in block 1 (an odd block, next to block 0)
    Bc[40, 0] = 2              # 1.0
    R = oracle.gemm_mx(A, SA, Bc, SB)
    assert R[1, 2] == 12.0 * 2.0 ** ((127 + 2 + 3) - 127) * 2.0 ** ((120 - 2 - 8) - 127)
    assert R[0, 0] == 2.0 ** ((127 + 1) - 127) * 2.0 ** ((120 - 1) - 127)
    assert np.count_nonzero(R) == 2


def test_mx_unit_scales_reduce_to_the_e2m1_gemm():
    # with every scale code 127 (2^0) the MX product is the e2m1 GEMM over fp16
    # activations holding the same values (fp8 e4m3 values are exact in fp16)
    A, SA, Bc, SB = _mx_inputs(5, 7, 96, seed=9)
    SA[:] = 127
    SB[:] = 127
    a16 = torch.from_numpy(_fp8_torch(A)).to(torch.float16).view(torch.int16).numpy() \
        .view(np.uint16)
    bias = bits16(synth.to_storage(synth.uniform(5, 7, -1, 1), torch.float16))
    R = oracle.gemm_mx(A, SA, Bc, SB, alpha=0.5, bias=bias, act=1)
    ones = np.full((3, 7), 0x3C00, np.uint16)
    ref = oracle.gemm_real(a16, Bc, a_kind="f16", b_kind="e2m1", scale=ones, group_k=32,
                           alpha=0.5, bias=bias, act=1)
    assert np.array_equal(R, ref)


def test_mx_quantiser_definition():
    w = synth.make("mxq_4096x4096", M=16, K=256)
    X = bits16(w.tensors["X"])
    X[3, 32:64] = 0                      # an all-zero block
    codes, scales = oracle.quant_mx(X)
    xv = oracle.f16_values(X)
    assert codes.shape == X.shape and scales.shape == (16, 8)
    assert scales[3, 1] == 0 and np.all(codes[3, 32:64] == 0)
    for i in range(16):
        for g in range(8):
            blk = xv[i, 32 * g:32 * g + 32]
            amax = np.abs(blk).max()
            if amax == 0:
                continue
            s = 2.0 ** (int(scales[i, g]) - 127)
            # the block maximum lands in the top binade of e4m3, [2^8, 2^9)
            assert 256 <= amax / s < 512
            q = blk / s
            ref = torch.from_numpy(np.clip(q, -448, 448).astype(np.float32)) \
                .to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            big = np.abs(q) > 448
            ref[big] = np.where(q[big] > 0, 0x7E, 0xFE)
            assert np.array_equal(codes[i, 32 * g:32 * g + 32], ref), (i, g)
    # values already on the grid come back unchanged: fp8 values times one power
    # of two, with the block maximum 448 * 2^-5
    v = _fp8_torch(synth.fp8_codes(73, 32).numpy())
    v = np.where(np.abs(v) > 448, 0, v) * 2.0 ** -5
    v[0] = 448 * 2.0 ** -5
    vb = oracle.f16_rne(v).reshape(1, 32)
    c2, s2 = oracle.quant_mx(vb)
    assert int(s2[0, 0]) == 127 - 5
    assert np.array_equal(_fp8_torch(c2[0]) * 2.0 ** -5, oracle.f16_values(vb)[0])


def test_mx_generators():
    c = synth.fp8_codes(5, 254 * 400)
    counts = torch.bincount(c.to(torch.int64), minlength=256)
    assert int(counts[0x7F]) == 0 and int(counts[0xFF]) == 0
    others = torch.cat([counts[:0x7F], counts[0x80:0xFF]])
    assert others.numel() == 254 and int(others.min()) > 300
    r = synth.int_range(6, 70000, 112, 118)
    assert int(r.min()) == 112 and int(r.max()) == 118
    assert int(torch.bincount(r.to(torch.int64) - 112).min()) > 9000
