"""GPU parity of the MX block-scaled path: dg_quant_mx and dg_gemm_mx against
the oracle on the same seeded bits.

The quantiser is byte work: codes and scales must match the oracle's bit for
bit.  The GEMM (fp8 e4m3 x e2m1 with e8m0 scales, fp32 accumulation) is compared
with the oracle's unrounded binary64 result under the fp16 rule of
``tests/parity.py`` (guarded relative error <= 2e-3): every product of the
path is exact, so only the fp32 summation and the final rounding separate the
two.  Small cases span several tiles, ragged edges, a half K step, forced tile
variants, K splits and padded leading dimensions; the full-size workload runs in
the benchmark's launch configuration and is checked on every output.
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


def padded(t, ld, fill=0):
    """2-D uint8/16-bit tensor on the GPU whose rows are `ld` elements apart."""
    buf = torch.full((t.shape[0], ld), fill, dtype=t.dtype, device=DEV)
    buf[:, : t.shape[1]] = t.to(DEV)
    return buf[:, : t.shape[1]]


def mx_operands(M, N, K, seed=601, pad=0, scale_fill=0xFF):
    """Seeded MX inputs: (host A, SA [M][K/32], codes [K][N], SB [K/32][N]) and
    their device layouts (A [M][K], SA group-major [K/32][lda], B packed [N][K/2],
    SB group-major [K/32][ldb]).  Scale rows are padded to a multiple of 4 bytes
    (plus `pad`), the padding holding the NaN scale code, which no output may
    see."""
    w = synth.make("mx_4096x4096x4096", M=M, N=N, K=K, seed=seed)
    t = w.tensors
    r4 = lambda n: (n + 3) // 4 * 4
    r16 = lambda n: (n + 15) // 16 * 16            # code rows start on 16-byte boundaries
    A = padded(t["A"], r16(K + pad))
    SA = padded(t["SA"].t().contiguous(), r4(M) + r4(pad), scale_fill)
    B = padded(dg.pack_e2m1(t["codes"]), r16(K // 2 + pad))
    SB = padded(t["SB"].contiguous(), r4(N) + r4(pad), scale_fill)
    host = (t["A"].numpy(), t["SA"].numpy(), t["codes"].numpy(), t["SB"].numpy())
    return host, (A, SA, B, SB)


def run_mx(h, M, N, K, *, seed=601, pad=0, opts=None, out=torch.float16, alpha=1.0,
           epilogue="none", bias_dtype=torch.float16, rows=None):
    say(f"[case] mx M={M} N={N} K={K} seed={seed} pad={pad} out={out} epi={epilogue} alpha={alpha} "
        f"opts={opts and {f: getattr(opts, f) for f, _ in opts._fields_}}")
    (A, SA, Bc, SB), (Ad, SAd, Bd, SBd) = mx_operands(M, N, K, seed, pad)
    bias = None
    if "bias" in epilogue:
        bias = synth.to_storage(synth.uniform(seed * 7 + 4, N, -0.1, 0.1), bias_dtype)
    # C inside a buffer whose row padding and three extra rows hold a sentinel
    Cbuf = torch.full((M + 3, N + pad), 7, dtype=out, device=DEV)
    Cd = Cbuf[:M, :N]
    info = h.gemm_mx(Ad, SAd, Bd, SBd, Cd, alpha=alpha, epilogue=epilogue,
                     bias=bias.to(DEV) if bias is not None else None, opts=opts)
    torch.cuda.synchronize()
    outside = torch.ones(Cbuf.shape, dtype=torch.bool)
    outside[:M, :N] = False
    assert int((Cbuf.cpu()[outside] != 7).sum()) == 0, "stores outside the output"
    rows = np.arange(M) if rows is None else np.asarray(rows)
    kind = {torch.float16: "f16", torch.bfloat16: "bf16", torch.float32: "f32"}[bias_dtype]
    R = oracle.gemm_mx(A[rows], SA[rows], Bc, SB, alpha=alpha,
                       bias=bits(bias) if bias is not None else None, bias_kind=kind,
                       act=1 if "gelu" in epilogue else 0)
    st = check_fp(Cd[torch.as_tensor(rows, device=DEV)], R, "f16")
    say(f"  {info.kernel_name.decode()} split={info.split_k} {st}")
    return info, st


# ------------------------------------------------------------------ quantiser
def quant_gpu(h, X, pad=0):
    """Codes [M][K] and scales as [M][K/32] (the device layout is group-major,
    [K/32][ld >= M]; transposed back here to compare with the oracle)."""
    M, K = X.shape
    Xd = padded(X, K + (pad + 7) // 8 * 8) if pad else X.to(DEV).contiguous()
    codes = padded(torch.zeros(M, K, dtype=torch.uint8), K + (pad + 15) // 16 * 16, 0xAA) if pad else \
        torch.full((M, K), 0xAA, dtype=torch.uint8, device=DEV)
    scales = padded(torch.zeros(K // 32, M, dtype=torch.uint8), M + pad, 0xAA) if pad else \
        torch.full((K // 32, M), 0xAA, dtype=torch.uint8, device=DEV)
    h.quant_mx(Xd, codes, scales)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.t().contiguous().cpu().numpy()


@pytest.mark.parametrize("M,K,pad", [(37, 96, 0), (64, 320, 5), (1, 32, 0)])
def test_quant_small_bit_exact(h, M, K, pad):
    say(f"[case] quant_mx M={M} K={K} pad={pad}")
    X = synth.make("mxq_4096x4096", M=M, K=K).tensors["X"]
    c, s = quant_gpu(h, X, pad)
    rc, rs = oracle.quant_mx(bits(X))
    assert np.array_equal(s, rs)
    assert np.array_equal(c, rc)


def test_quant_full_size_bit_exact(h):
    w = synth.make("mxq_4096x4096")
    say(f"[case] quant_mx {w.name} M={w.M} K={w.K}")
    X = w.tensors["X"]
    c, s = quant_gpu(h, X)
    rc, rs = oracle.quant_mx(bits(X))
    assert np.array_equal(s, rs)
    assert np.array_equal(c, rc)


def test_quant_edge_values(h):
    """Zero blocks (signed zeros), binary16 subnormals, saturation just below the
    next binade, exact ties of the e4m3 grid, and the largest binary16 values."""
    say("[case] quant_mx edge values")
    K = 32 * 8
    X = np.zeros((4, K), np.float64)
    X[0, 32:64] = -0.0
    X[0, 64:96] = np.arange(32) * 2.0 ** -24                     # subnormals only
    X[0, 96] = 511.0                                              # amax/scale = 511.0 -> 448
    X[0, 97:128] = np.linspace(-500, 500, 31)
    X[1, :32] = (1 + np.arange(32) / 16.0) * 2.0 ** 3             # ties at 1 + 1/16 steps
    X[1, 32:64] = 65504.0 * np.sign(np.arange(32) - 15.5)         # largest binary16
    X[1, 64:96] = np.linspace(-1, 1, 32) * 2.0 ** -14             # around the smallest normal
    z = synth.normal(17, 2 * K).numpy().reshape(2, K)
    X[2:] = z * 2.0 ** np.arange(-20, 12, 4).repeat(32)[None, :]
    Xb = torch.from_numpy(oracle.f16_rne(X).view(np.int16)).view(torch.float16)
    c, s = quant_gpu(h, Xb)
    rc, rs = oracle.quant_mx(bits(Xb))
    assert np.array_equal(s, rs)
    assert np.array_equal(c, rc)
    assert np.all(c[0, 32:64] == 0x80) and s[0, 0] == 0


def test_quant_non_finite_block(h):
    """A block holding an infinity or a NaN gets the NaN scale code and NaN codes
    (the interface's stated behaviour; the oracle rejects such input); the other
    blocks of the row are unaffected."""
    say("[case] quant_mx non-finite block")
    X = synth.make("mxq_4096x4096", M=2, K=128).tensors["X"].clone()
    X[0, 5] = float("inf")
    X[1, 70] = float("nan")
    c, s = quant_gpu(h, X)
    assert s[0, 0] == 255 and np.all(c[0, :32] == 0x7F)
    assert s[1, 2] == 255 and np.all(c[1, 64:96] == 0x7F)
    Y = X.clone()
    Y[0, :32] = 0
    Y[1, 64:96] = 0
    rc, rs = oracle.quant_mx(bits(Y))
    keep = np.ones((2, 4), bool)
    keep[0, 0] = keep[1, 2] = False
    assert np.array_equal(s[keep], rs[keep])
    ck = np.repeat(keep, 32, axis=1)
    assert np.array_equal(c[ck], rc[ck])


# ----------------------------------------------------------------------- GEMM
@pytest.mark.parametrize("M,N,K", [(256, 256, 256), (100, 200, 320), (1, 96, 64), (300, 130, 1024),
                                   (64, 64, 128), (513, 257, 192)])
def test_gemm_mx_small(h, M, N, K):
    run_mx(h, M, N, K)


@pytest.mark.parametrize("bm,bn,waves,ms", [(256, 256, 8, 32), (128, 256, 4, 32), (256, 128, 4, 32),
                                            (128, 128, 4, 32), (64, 64, 4, 32), (256, 256, 8, 16)])
def test_gemm_mx_every_variant(h, bm, bn, waves, ms):
    # a ragged problem with a half K step at the end, unsplit and split in 3
    for split in (1, 3):
        info, _ = run_mx(h, 300, 330, 448, opts=dg.dg_plan_opts(force_m_tile=bm, force_n_tile=bn, force_waves=waves,
                                                                force_mfma=ms, force_split_k=split))
        assert info.mfma_m == ms


@pytest.mark.parametrize("split", [2, 3, 8])
def test_gemm_mx_split_k_bias_gelu(h, split):
    run_mx(h, 96, 160, 1536, opts=dg.dg_plan_opts(force_split_k=split, force_path=dg.DG_PATH_TILED),
           epilogue="bias_gelu_erf")


@pytest.mark.parametrize("out,epi,bias_dtype,alpha", [
    (torch.float32, "bias", torch.float32, 0.5),
    (torch.float16, "gelu_erf", torch.float16, 2.0),
    (torch.float16, "bias_gelu_erf", torch.bfloat16, 1.0),
])
def test_gemm_mx_epilogues(h, out, epi, bias_dtype, alpha):
    run_mx(h, 192, 320, 512, out=out, epilogue=epi, bias_dtype=bias_dtype, alpha=alpha)


def test_gemm_mx_padded_leading_dimensions(h):
    run_mx(h, 130, 96, 384, pad=20)


def test_gemm_mx_empty_k(h):
    """K = 0: no products; the output is the epilogue of zero."""
    say("[case] mx K=0 bias")
    M, N = 40, 72
    bias = synth.to_storage(synth.uniform(3, N, -0.1, 0.1), torch.float16).to(DEV)
    Cd = torch.full((M, N), 7, dtype=torch.float16, device=DEV)
    h.gemm_mx(torch.zeros(M, 16, dtype=torch.uint8, device=DEV)[:, :0],
              torch.zeros(0, M, dtype=torch.uint8, device=DEV),
              torch.zeros(N, 16, dtype=torch.uint8, device=DEV)[:, :0],
              torch.zeros(0, N, dtype=torch.uint8, device=DEV), Cd, epilogue="bias", bias=bias)
    torch.cuda.synchronize()
    assert torch.equal(Cd.cpu(), bias.cpu().expand(M, N))


def test_gemm_mx_rejects_bad_arguments(h):
    (_, _, _, _), (A, SA, B, SB) = mx_operands(64, 64, 128)
    C = torch.empty(64, 64, dtype=torch.float16, device=DEV)
    with pytest.raises(dg.DGError) as e:     # K not a multiple of 64
        h.gemm_mx(A[:, :96], SA, B[:, :48], SB, C)
    assert e.value.status == dg.DG_ERR_ALIGNMENT
    with pytest.raises(dg.DGError) as e:     # scale rows not a multiple of 4 bytes
        h.gemm_mx(A, torch.zeros(4, 65, dtype=torch.uint8, device=DEV), B, SB, C)
    assert e.value.status == dg.DG_ERR_ALIGNMENT
    with pytest.raises(dg.DGError) as e:     # scale rows shorter than M
        h.gemm_mx(A, torch.zeros(4, 60, dtype=torch.uint8, device=DEV), B, SB, C)
    assert e.value.status == dg.DG_ERR_INVALID_ARG
    with pytest.raises(dg.DGError) as e:
        h.gemm_mx(A, SA, B, SB, torch.empty(64, 64, dtype=torch.int32, device=DEV))
    assert e.value.status == dg.DG_ERR_UNSUPPORTED


def test_gemm_mx_full_size_every_output(h):
    """The 4096^3 workload in the launch configuration the benchmark times,
    checked on every output."""
    info, st = run_mx(h, 4096, 4096, 4096)
    assert info.split_k == 1 and st["n"] == 4096 * 4096


@pytest.mark.parametrize("ms", [16, 32])
def test_gemm_mx_full_size_each_mfma_block(h, ms):
    """The 4096^3 workload with the eight-wave 256x256 tile on each MFMA block,
    every output against the oracle."""
    o = dg.dg_plan_opts(force_path=dg.DG_PATH_TILED, force_m_tile=256, force_n_tile=256, force_waves=8,
                        force_mfma=ms)
    info, st = run_mx(h, 4096, 4096, 4096, opts=o)
    assert info.mfma_m == ms and st["n"] == 4096 * 4096


def test_quant_then_gemm_end_to_end(h):
    """fp16 activations quantised on the GPU and multiplied by e2m1 weights,
    against the oracle's quantiser and MX GEMM on the same activations."""
    M, N, K = 160, 192, 640
    say(f"[case] quant_mx + gemm_mx M={M} N={N} K={K}")
    X = synth.make("mxq_4096x4096", M=M, K=K, seed=611).tensors["X"]
    w = synth.make("mx_4096x4096x4096", M=M, N=N, K=K, seed=612).tensors
    G = K // 32
    codes = torch.empty(M, K, dtype=torch.uint8, device=DEV)
    scales = torch.empty(G, (M + 3) // 4 * 4, dtype=torch.uint8, device=DEV)   # group-major
    h.quant_mx(X.to(DEV), codes, scales[:, :M])
    B = dg.pack_e2m1(w["codes"]).to(DEV)
    SB = padded(w["SB"].contiguous(), (N + 3) // 4 * 4)
    Cd = torch.empty(M, N, dtype=torch.float16, device=DEV)
    h.gemm_mx(codes, scales, B, SB, Cd)
    torch.cuda.synchronize()
    rc, rs = oracle.quant_mx(bits(X))
    R = oracle.gemm_mx(rc, rs, w["codes"].numpy(), w["SB"].numpy())
    st = check_fp(Cd, R, "f16")
    say(f"  {st}")


# ---------------------------------------------------------------- random sweep
def _mx_cases(n=16, seed=20261203):
    """Seeded random MX problems: ragged M and N, K in whole 64-element steps
    (half steps included), planner-chosen or forced K splits and tiles, every
    epilogue, fp16 or fp32 output, tight or padded leading dimensions."""
    rng = np.random.default_rng(seed)
    tiles = [(0, 0, 0), (256, 256, 8), (128, 256, 4), (256, 128, 4), (128, 128, 4), (64, 64, 4)]
    out = []
    for i in range(n):
        M = int(rng.choice([1, 3, 17, 64, 100, 257, 513]))
        N = int(rng.integers(1, 80)) * 8 + int(rng.choice([0, 0, 3]))
        K = int(rng.integers(1, 40)) * 64
        split = int(rng.choice([0, 0, 2, 3]))
        bm, bn, w = tiles[int(rng.integers(0, len(tiles)))]
        epi = ["none", "bias", "gelu_erf", "bias_gelu_erf"][int(rng.integers(0, 4))]
        out_t = torch.float32 if rng.random() < 0.25 else torch.float16
        pad = int(rng.choice([0, 0, 12]))
        alpha = float(rng.choice([1.0, 0.75]))
        out.append((M, N, K, split, bm, bn, w, epi, out_t, pad, alpha, seed + i))
    return out


@pytest.mark.parametrize("case", _mx_cases(), ids=lambda c: "{}x{}x{}-s{}-t{}x{}-{}".format(
    c[0], c[1], c[2], c[3], c[4], c[5], c[7]))
def test_gemm_mx_random_problem(h, case):
    M, N, K, split, bm, bn, w, epi, out_t, pad, alpha, seed = case
    o = dg.dg_plan_opts(force_split_k=split, force_m_tile=bm, force_n_tile=bn, force_waves=w,
                        force_path=dg.DG_PATH_TILED if split or bm else 0)
    run_mx(h, M, N, K, seed=seed, pad=pad, opts=o, out=out_t, alpha=alpha, epilogue=epi)
