"""GPU parity: the HIP path against the CPU oracle on the same seeded bits.

Every case draws its inputs with the shared generator, runs ``dg_gemm`` through
the C ABI (ctypes binding), and compares with the oracle: bit for bit for int8
-> int32 and the requantise epilogues, within the rule of ``tests/parity.py``
for floating point.  Small cases span several tiles with ragged edges and
padded leading dimensions; the full-size workloads run in the launch
configuration the benchmark times.  Every case is checked on every output, and
the output's row padding and a few rows past its end must keep a sentinel.
"""
import numpy as np
import pytest
import torch

import oracle
from tests.parity import bits, check_fp, out_values, say, tol_for
from tile_planned_generator_amd import dg, synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def h():
    torch.cuda.init()
    hd = dg.Handle(0)
    yield hd
    hd.close()


TORCH_OUT = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32,
             "i32": torch.int32, "i8": torch.int8}


def to_dev(t, pad=0):
    """2-D tensor on the GPU; with pad > 0 the rows are padded (leading dimension
    = columns + pad rounded up to 16 elements, so rows stay 16-byte aligned) and
    the kernels see a non-tight leading dimension."""
    t = t.to(DEV)
    if pad:
        ld = (t.shape[1] + pad + 15) // 16 * 16
        buf = torch.zeros(t.shape[0], ld, dtype=t.dtype, device=DEV)
        buf[:, : t.shape[1]] = t
        return buf[:, : t.shape[1]]
    return t.contiguous()


GUARD_ROWS = 3
SENTINEL = 7


def guarded_out(M, N, dtype, pad):
    """Output [M, N] inside a buffer whose row padding (pad > 0) and GUARD_ROWS
    extra rows hold SENTINEL: a store past column N or row M changes them.
    Returns (the [M, N] view, the whole buffer)."""
    ld = (N + pad + 15) // 16 * 16 if pad else N
    buf = torch.full((M + GUARD_ROWS, ld), SENTINEL, dtype=dtype, device=DEV)
    return buf[:M, :N], buf


def check_guards(buf, M, N):
    """Every element of `buf` outside [:M, :N] still holds SENTINEL."""
    host = buf.cpu()
    mask = torch.ones(host.shape, dtype=torch.bool)
    mask[:M, :N] = False
    bad = int((host[mask] != SENTINEL).sum())
    assert bad == 0, f"{bad} elements outside the output were written"


def _chunks(n, size):
    """Position slices of n columns, `size` at a time (one slice when size is 0)."""
    size = size or max(n, 1)
    return [slice(i, min(n, i + size)) for i in range(0, max(n, 1), size)]


def run(h, w, *, b_colmajor=False, pad=0, opts=None, out=None, epilogue=None, rows=None,
        cols=None, requant_scale=1.0, rq_bias=None, alpha=None, beta=None, col_chunk=0,
        c_ld=None, c_off=0):
    """Run workload ``w`` through dg_gemm and check it against the oracle on
    rows x cols (all by default; the oracle runs on column blocks of
    ``col_chunk`` columns when it is given, which bounds its binary64 copy of B).
    The output's row padding and a few rows past M are checked untouched.
    c_ld / c_off: C's leading dimension and its first element's offset (in
    elements) in its buffer, whose elements before C must stay untouched too.
    Returns (plan info, error stats)."""
    t = w.tensors
    M, N, K = w.M, w.N, w.K
    out = out or w.out
    epilogue = epilogue or w.epilogue
    alpha = w.alpha if alpha is None else alpha
    beta = w.beta if beta is None else beta
    say(f"[case] {w.name} M={M} N={N} K={K} seed={w.seed} out={out} epi={epilogue} "
        f"colmajor={b_colmajor} pad={pad} opts={opts and {f: getattr(opts, f) for f, _ in opts._fields_}}")
    A = to_dev(t["A"], pad)
    scale = None
    if w.path == "e2m1":
        Bd = to_dev(dg.pack_e2m1(t["codes"]), pad)
        scale = dg.scales_gn(t["scale"]).to(DEV)
        layout = dg.DG_COL_MAJOR
    elif b_colmajor:
        Bd = to_dev(t["B"].t().contiguous(), pad)
        layout = dg.DG_COL_MAJOR
    else:
        Bd = to_dev(t["B"], pad)
        layout = dg.DG_ROW_MAJOR
    if c_ld is None and not c_off:
        Cd, Cbuf = guarded_out(M, N, TORCH_OUT[out], pad)
        head = None
    else:
        ld = c_ld or N
        flat = torch.full((c_off + (M + GUARD_ROWS) * ld,), SENTINEL, dtype=TORCH_OUT[out], device=DEV)
        Cbuf = flat[c_off:].view(M + GUARD_ROWS, ld)
        Cd, head = Cbuf[:M, :N], flat[:c_off]
    D = to_dev(t["D"], pad) if "D" in t and beta != 0 else None
    bias = t.get("bias")
    if epilogue in ("requant_i8", "requant_f16"):
        bias = rq_bias
    bias = bias.to(DEV) if bias is not None else None
    info = h.gemm(A, Bd, Cd, alpha=alpha, beta=beta, D=D, bias=bias, epilogue=epilogue,
                  b_scale=scale, b_layout=layout, opts=opts, requant_scale=requant_scale)
    torch.cuda.synchronize()
    say(f"       plan {info.kernel_name.decode()} S={info.split_k} tile={info.m_tile}x{info.n_tile}")
    check_guards(Cbuf, M, N)
    if head is not None:
        assert bool((head.cpu() == SENTINEL).all()), "elements before C were written"
    del A, Bd, scale

    r_idx = torch.arange(M) if rows is None else torch.as_tensor(rows)
    c_idx = torch.arange(N) if cols is None else torch.as_tensor(cols)
    Csub = Cd.cpu()[r_idx][:, c_idx]
    Ah = t["A"][r_idx.to(t["A"].device)].cpu()
    if w.path == "i8":
        Dh = t["D"][r_idx][:, c_idx].cpu() if D is not None else None
        parts = []
        for pos in _chunks(len(c_idx), col_chunk):
            Bh = t["B"][:, c_idx[pos].to(t["B"].device)].cpu()
            Dc = bits(Dh[:, pos]) if Dh is not None else None
            parts.append(oracle.gemm_int(Ah.numpy(), Bh.numpy(), alpha=int(alpha), beta=int(beta), D=Dc))
        Cw = np.concatenate([p[1] for p in parts], axis=1)
        ov = sum(p[2] for p in parts)
        assert Cw.shape == (len(r_idx), len(c_idx))
        if epilogue in ("requant_i8", "requant_f16"):
            want = oracle.requant(Cw, alpha=requant_scale,
                                  bias=rq_bias.numpy()[c_idx.numpy()] if rq_bias is not None else None,
                                  out="i8" if epilogue == "requant_i8" else "f16")
            got = bits(Csub)
            assert np.array_equal(got, want), int((got != want).sum())
            return info, {"bitexact": True, "n": int(got.size)}
        got = Csub.numpy()
        assert np.array_equal(got, Cw), int((got != Cw).sum())
        say(f"       ok bit-exact on {got.size} outputs")
        return info, {"bitexact": True, "overflow": ov, "n": int(got.size)}
    a_kind = "f16" if w.path in ("f16", "e2m1") else "bf16"
    parts = []
    for pos in _chunks(len(c_idx), col_chunk):
        kw = {}
        cd = c_idx[pos].to(t["A"].device)
        if w.path == "e2m1":
            Bh = bits(t["codes"][:, cd])
            kw = dict(scale=bits(t["scale"][:, cd]), group_k=32)
            b_kind = "e2m1"
        else:
            Bh = bits(t["B"][:, cd])
            b_kind = a_kind
        if D is not None:
            kw.update(D=bits(t["D"][r_idx.to(t["D"].device)][:, cd]), d_kind=out)
        if bias is not None:
            kw.update(bias=bits(t["bias"][cd]), bias_kind=a_kind)
        act = 1 if "gelu" in epilogue else 0
        parts.append(oracle.gemm_real(bits(Ah), Bh, a_kind=a_kind, b_kind=b_kind, alpha=alpha,
                                      beta=beta, act=act, **kw))
        del Bh
    R = np.concatenate(parts, axis=1)
    st = check_fp(Csub, R, tol_for(w.path, out))
    say(f"       ok {st}")
    return info, st


# ------------------------------------------------------- exact special cases
def test_identity_and_permutation_are_bit_exact(h):
    # A . I = A and A . P permutes columns: one non-zero product per output,
    # exact in fp32, exact in the output type - any operand-layout or
    # output-layout slip in the MFMA fragments shows up as a wrong element.
    for dt, kd in ((torch.float16, "f16"), (torch.bfloat16, "bf16")):
        M, K = 96, 192
        A = synth.to_storage(synth.normal(77, M * K), dt).view(M, K)
        I = torch.eye(K, dtype=dt)
        perm = torch.randperm(K, generator=torch.Generator().manual_seed(1))
        P = I[:, perm].contiguous()          # (A.P)[:, j] = A[:, perm[j]]
        for colmajor in (False, True):
            for Bm, want in ((I, A), (P, A[:, perm])):
                Bd = Bm.t().contiguous().to(DEV) if colmajor else Bm.to(DEV)
                Cd = torch.empty(M, K, dtype=dt, device=DEV)
                h.gemm(A.to(DEV), Bd, Cd, b_layout=dg.DG_COL_MAJOR if colmajor else dg.DG_ROW_MAJOR)
                torch.cuda.synchronize()
                assert torch.equal(Cd.cpu(), want), (kd, colmajor)
    # int8: A . P with P a permutation gives A's columns exactly
    M, K = 64, 256
    A = synth.int8_uniform(78, M * K).view(M, K)
    perm = torch.randperm(K, generator=torch.Generator().manual_seed(2))
    P = torch.zeros(K, K, dtype=torch.int8)
    P[perm, torch.arange(K)] = 1
    for colmajor in (False, True):
        Bd = P.t().contiguous().to(DEV) if colmajor else P.to(DEV)
        Cd = torch.empty(M, K, dtype=torch.int32, device=DEV)
        h.gemm(A.to(DEV), Bd, Cd, b_layout=dg.DG_COL_MAJOR if colmajor else dg.DG_ROW_MAJOR)
        torch.cuda.synchronize()
        assert torch.equal(Cd.cpu(), A[:, perm].to(torch.int32)), colmajor


def test_e2m1_one_hot_decode_is_exact(h):
    # A = one-hot rows selects single weights: C[i][j] = e2m1(code[k_i][j]) *
    # scale[k_i/32][j]; with power-of-two scales every product is exact in fp16,
    # so all 16 codes, both nibbles and the group index are checked bit for bit.
    K, N = 64, 32
    codes = (torch.arange(K * N, dtype=torch.int64) % 16).to(torch.uint8).view(K, N)
    codes = codes[torch.randperm(K, generator=torch.Generator().manual_seed(3))]
    G = K // 32
    sc = torch.tensor([[2.0 ** (-(g + (j % 5))) for j in range(N)] for g in range(G)],
                      dtype=torch.float16)
    M = K
    A = torch.eye(K, dtype=torch.float16)
    gold = oracle.e2m1_values(codes.numpy()) * sc.double().numpy()[np.arange(K) // 32]
    for opts in (dg.dg_plan_opts(force_path=dg.DG_PATH_TILED), None):
        Cd = torch.empty(M, N, dtype=torch.float16, device=DEV)
        h.gemm(A.to(DEV), dg.pack_e2m1(codes).to(DEV), Cd, b_scale=dg.scales_gn(sc).to(DEV),
               opts=opts)
        torch.cuda.synchronize()
        assert np.array_equal(Cd.cpu().double().numpy(), gold)
    # the skinny path (M = 1) on each row of the one-hot
    for k in (0, 1, 33, 62):
        Cd = torch.empty(1, N, dtype=torch.float32, device=DEV)
        h.gemm(A[k:k + 1].contiguous().to(DEV), dg.pack_e2m1(codes).to(DEV), Cd,
               b_scale=dg.scales_gn(sc).to(DEV))
        torch.cuda.synchronize()
        assert np.array_equal(Cd.cpu().double().numpy()[0], gold[k])


def test_rank_one_closed_form_exact(h):
    # a[i][k] = x_i, b[k][j] = y_j: C = K x_i y_j, exact for small integers
    M, N, K = 130, 70, 512
    x = torch.tensor([(i % 7) - 3 for i in range(M)], dtype=torch.float16)
    y = torch.tensor([(j % 5) - 2 for j in range(N)], dtype=torch.float16)
    A = x[:, None].expand(M, K).contiguous()
    Bp = torch.zeros(K, 80, dtype=torch.float16)     # rows padded to 80 columns
    Bp[:, :N] = y[None, :].expand(K, N)
    Cd = torch.empty(M, N, dtype=torch.float32, device=DEV)
    h.gemm(A.to(DEV), Bp.to(DEV)[:, :N], Cd)
    torch.cuda.synchronize()
    assert torch.equal(Cd.cpu(), (K * x.float()[:, None] * y.float()[None, :]))
    # int8 extremes: 127 * -128 * 4096 and (-128)^2 * 4096 = 2^26
    A = torch.full((40, 4096), 127, dtype=torch.int8)
    A[20:] = -128
    B = torch.full((4096, 48), -128, dtype=torch.int8)
    Cd = torch.empty(40, 48, dtype=torch.int32, device=DEV)
    h.gemm(A.to(DEV), B.to(DEV), Cd)
    torch.cuda.synchronize()
    assert int(Cd[0, 0]) == -66584576 and int(Cd[39, 47]) == 2 ** 26


def test_int32_accumulation_wraps(h):
    # Sums past the int32 range: A = -128 everywhere and B[k][j] = -128 for the
    # first L_j rows of K (0 after), so C[i][j] = 16384 * L_j, from just below
    # 2^31 to about 1.28 * 2^31 across the columns (L_j = 131072 gives exactly
    # 2^31).  The 32-bit result wraps modulo 2^32 (the oracle's wrapped C), with
    # the whole K in one slice and split into slices reduced in 32 bits.
    M, N, K = 64, 96, 131072
    L = [K - 256 + 384 * j for j in range(N)]
    B = torch.zeros(K + 2048 * 32, N, dtype=torch.int8)
    for j, l in enumerate(L):
        B[:l, j] = -128
    for KK in (K, K + 2048 * 32):
        Ak = torch.full((M, KK), -128, dtype=torch.int8)
        Bk = B[:KK].contiguous()
        R, Cw, ov = oracle.gemm_int(Ak.numpy(), Bk.numpy())
        assert ov > 0 and int(R.max()) > 2 ** 31 - 1
        for split in (1, 4):
            say(f"[case] int32 wrap M={M} N={N} K={KK} split={split}")
            Cd = torch.empty(M, N, dtype=torch.int32, device=DEV)
            h.gemm(Ak.to(DEV), Bk.to(DEV), Cd,
                   opts=dg.dg_plan_opts(force_split_k=split, force_path=dg.DG_PATH_TILED))
            torch.cuda.synchronize()
            assert np.array_equal(Cd.cpu().numpy(), Cw)


def test_fp16_subnormal_inputs_not_flushed(h):
    # products of fp16 subnormals with 2^10 land in the normal range: flushing
    # either operand to zero would give 0
    M, N, K = 64, 64, 64
    A = torch.zeros(M, K, dtype=torch.float16)
    A[:, 0] = torch.tensor(2.0 ** -20, dtype=torch.float16)   # subnormal
    B = torch.zeros(K, N, dtype=torch.float16)
    B[0, :] = 1024.0
    Cd = torch.empty(M, N, dtype=torch.float32, device=DEV)
    h.gemm(A.to(DEV), B.to(DEV), Cd)
    torch.cuda.synchronize()
    assert torch.all(Cd.cpu() == 2.0 ** -10)


# --------------------------------------------------------- small full parity
def test_f16_alpha_beta_d_full_size(h):
    run(h, synth.make("f16_256x256x256_alpha_beta_d"))


@pytest.mark.parametrize("M,N,K,pad", [(257, 263, 272, 9), (300, 128, 1040, 0), (33, 65, 16, 15)])
def test_f16_alpha_beta_d_ragged(h, M, N, K, pad):
    # pad makes the row pitch a multiple of 8 elements (16 bytes)
    run(h, synth.make("f16_256x256x256_alpha_beta_d", M=M, N=N, K=K), pad=pad)


@pytest.mark.parametrize("name", ["f16_4096x4096x4096", "bf16_16x4096x131072"])
@pytest.mark.parametrize("tile", [(256, 256, 8, 16), (64, 64, 4, 32)])
@pytest.mark.parametrize("c_ld,c_off", [(268, 0), (264, 4), (265, 1)])
def test_16bit_c_pitch_and_alignment(h, name, tile, c_ld, c_off):
    # A plain 16-bit C goes eight columns per 16-byte store when its pitch is a
    # multiple of 8 elements and it is 16-byte aligned; a pitch of 4 mod 8, a
    # C 8 bytes past a 16-byte boundary, and an odd pitch with a 2-byte
    # aligned C take the element-wise stores (N = 264 is a whole number of
    # 8-column pieces, so only the pitch or the alignment decides)
    bm, bn, waves, ms = tile
    w = synth.make(name, M=300, N=264, K=512)
    o = dg.dg_plan_opts(force_path=dg.DG_PATH_TILED, force_m_tile=bm, force_n_tile=bn, force_waves=waves,
                        force_mfma=ms, force_split_k=1)
    run(h, w, opts=o, alpha=0.75, c_ld=c_ld, c_off=c_off)


@pytest.mark.parametrize("M,N,K", [(512, 384, 640), (300, 200, 96), (129, 257, 4160)])
@pytest.mark.parametrize("colmajor", [False, True])
def test_i8_bit_exact_small(h, M, N, K, colmajor):
    w = synth.make("i8_4096x4096x4096", M=M, N=N, K=K)
    run(h, w, b_colmajor=colmajor, pad=16 if N % 16 else 0)


@pytest.mark.parametrize("M,N,K", [(384, 320, 1024), (130, 200, 2112)])
def test_f16_bias_gelu_small(h, M, N, K):
    w = synth.make("f16_2048x2048x8192_bias_gelu", M=M, N=N, K=K)
    run(h, w, pad=8 if N % 8 else 0)
    run(h, w, out="f32", pad=8 if N % 8 else 0)


@pytest.mark.parametrize("M,N,K", [(256, 512, 1024), (100, 72, 320)])
@pytest.mark.parametrize("colmajor", [False, True])
def test_bf16_tiled_small(h, M, N, K, colmajor):
    w = synth.make("bf16_16x4096x131072", M=M, N=N, K=K)
    run(h, w, b_colmajor=colmajor)
    run(h, w, b_colmajor=colmajor, epilogue="gelu_erf", out="f32")


@pytest.mark.parametrize("M,N,K", [(256, 256, 512), (70, 96, 192)])
def test_e2m1_tiled_small(h, M, N, K):
    w = synth.make("e2m1_4096x4096x4096", M=M, N=N, K=K)
    run(h, w, opts=dg.dg_plan_opts(force_path=dg.DG_PATH_TILED))


@pytest.mark.parametrize("M,N,K,path", [(100, 257, 256, dg.DG_PATH_TILED), (300, 33, 1024, dg.DG_PATH_TILED),
                                        (1, 33, 512, dg.DG_PATH_SKINNY), (3, 129, 2048, dg.DG_PATH_SKINNY)])
def test_e2m1_odd_n(h, M, N, K, path):
    # odd N: the group-major scale rows are padded to N + 1 (scales_gn), and the
    # tiled kernel's paired scale loads cover a column past N
    w = synth.make("e2m1_4096x4096x4096", M=M, N=N, K=K)
    run(h, w, opts=dg.dg_plan_opts(force_path=path))


# compiled tiled variants: (M tile, N tile, waves, K regions per step, MFMA
# block); the double K step exists for the 16-bit and int8 paths, the 16x16
# MFMAs for those and e2m1
TILED_VARIANTS = ((128, 256, 4, 1, 32), (256, 256, 8, 1, 32), (256, 128, 4, 1, 32), (128, 128, 4, 1, 32),
                  (64, 64, 4, 1, 32), (256, 256, 4, 2, 32), (128, 256, 4, 2, 32), (256, 128, 4, 2, 32),
                  (128, 128, 4, 2, 32), (64, 64, 4, 2, 32), (256, 256, 8, 1, 16))


def test_every_tiled_variant_on_a_ragged_problem(h):
    # each compiled variant (tile shape, wave grid, K step, MFMA block), forced in turn, on a
    # problem with ragged M and N, a K tail and a K split: one K region per step
    # with K = 7 full steps + a half step (e2m1 K is whole 32-groups, so 8 full
    # steps), two regions per step with K = 3 full steps + a tail of one, two or
    # three substeps; split 2 gives slices with fewer steps than LDS stages
    for path, name, colm in (("f16", "f16_2048x2048x8192_bias_gelu", False),
                             ("f16", "f16_2048x2048x8192_bias_gelu", True),
                             ("bf16", "bf16_16x4096x131072", False),
                             ("i8", "i8_4096x4096x4096", False),
                             ("i8", "i8_4096x4096x4096", True),
                             ("e2m1", "e2m1_4096x4096x4096", True)):
        region = 64 if path == "i8" else 32
        for bm, bn, nw, kr, ms in TILED_VARIANTS:
            if kr > 1 and path == "e2m1":
                continue
            if kr == 1:
                ks = [8 * 32] if path == "e2m1" else [7 * region + region // 2]
            else:
                ks = [3 * 2 * region + t * region // 2 for t in (1, 2, 3)]
            for K in ks:
                w = synth.make(name, M=290, N=272, K=K)
                for s in (1, 2):
                    o = dg.dg_plan_opts(force_m_tile=bm, force_n_tile=bn, force_split_k=s,
                                        force_path=dg.DG_PATH_TILED, force_waves=nw, force_k_tile=region * kr,
                                        force_mfma=ms)
                    info, _ = run(h, w, b_colmajor=colm, opts=o)
                    assert info.k_main == region * kr and info.waves_per_wg == nw and info.mfma_m == ms


def test_split_k_and_schedule_tail(h):
    o = dg.dg_plan_opts(force_path=dg.DG_PATH_TILED, force_split_k=4)
    run(h, synth.make("f16_2048x2048x8192_bias_gelu", M=512, N=512, K=2048 + 48), opts=o)
    run(h, synth.make("i8_4096x4096x4096", M=512, N=512, K=2048 + 96), opts=o)
    # a K shorter than one full step: only a tail step
    run(h, synth.make("f16_256x256x256_alpha_beta_d", M=64, N=64, K=16))


# ------------------------------------------------------------- skinny paths
@pytest.mark.parametrize("M", [1, 2, 3, 5, 8])
@pytest.mark.parametrize("K", [1024, 2000])
def test_skinny_valu(h, M, K):
    for lpr_n in (4096, 1000, 256):
        w = synth.make("bf16_1x4096x131072", M=M, N=lpr_n, K=K)
        run(h, w, opts=dg.dg_plan_opts(unit=dg.DG_UNIT_VALU), pad=8 if lpr_n % 8 else 0)
    w = synth.make("f16_256x256x256_alpha_beta_d", M=M, N=520, K=K)
    run(h, w, opts=dg.dg_plan_opts(unit=dg.DG_UNIT_VALU, force_split_k=3))


@pytest.mark.parametrize("n_tile", [256, 512, 1024, 2048])
def test_skinny_valu_every_width(h, n_tile):
    # every column width of the VALU streaming kernel (64, 128, 256 or 512 columns
    # per wave), with slices that end in a partial batch of rows, ragged N and
    # padded leading dimensions
    for name in ("bf16_1x4096x131072", "f16_256x256x256_alpha_beta_d"):
        for M in (1, 3, 8):
            for K, S in ((2000, 3), (4144, 0), (144, 1)):
                w = synth.make(name, M=M, N=1000, K=K)
                o = dg.dg_plan_opts(force_n_tile=n_tile, force_split_k=S, force_path=dg.DG_PATH_SKINNY,
                                    unit=dg.DG_UNIT_VALU)
                info, _ = run(h, w, opts=o, pad=8)
                assert info.n_tile == n_tile and info.kernel_name.decode().endswith(f"lpr{n_tile // 32}")


@pytest.mark.parametrize("M", [1, 9, 16])
def test_skinny_mfma(h, M):
    w = synth.make("bf16_16x4096x131072", M=M, N=1000, K=4128)
    run(h, w, opts=dg.dg_plan_opts(unit=dg.DG_UNIT_MFMA, force_path=dg.DG_PATH_SKINNY), pad=8)
    w = synth.make("f16_256x256x256_alpha_beta_d", M=M, N=512, K=1040)
    run(h, w, opts=dg.dg_plan_opts(unit=dg.DG_UNIT_MFMA, force_path=dg.DG_PATH_SKINNY, force_split_k=5))


@pytest.mark.parametrize("M", [1, 2, 4, 7])
def test_skinny_e2m1(h, M):
    # one slice holds at most 32 KB of A (K * rows * 2 bytes): M > 4 needs two.
    # The longest slice each row count allows (16384 / MR, MR the rows the
    # kernel stages) takes the staging loops past their first batch.
    longest = {1: 16384, 2: 8192, 4: 4096, 7: 2048}[M]
    for K, S in ((4096, 1 if M <= 4 else 2), (4096, 4), (1056, 0), (longest, 1)):
        w = synth.make("e2m1_1x4096x4096", M=M, N=300, K=K)
        run(h, w, opts=dg.dg_plan_opts(force_path=dg.DG_PATH_SKINNY, force_split_k=S))


@pytest.mark.parametrize("M", [15, 16, 17])
def test_m_either_side_of_the_streaming_limit(h, M):
    # the streaming kernels take M <= 16: at 15 and 16 the 16-bit problems plan to
    # the skinny MFMA kernel, at 17 to the tiled one (int8 and e2m1 stay tiled);
    # N is ragged against every tile and the leading dimensions padded
    for name in ("bf16_16x4096x131072", "f16_256x256x256_alpha_beta_d"):
        run(h, synth.make(name, M=M, N=264, K=2080), pad=8)
    run(h, synth.make("i8_4096x4096x4096", M=M, N=208, K=640))
    run(h, synth.make("e2m1_4096x4096x4096", M=M, N=200, K=1024))


@pytest.mark.parametrize("name,K", [("f16_256x256x256_alpha_beta_d", 32), ("bf16_16x4096x131072", 32),
                                    ("i8_4096x4096x4096", 64), ("e2m1_4096x4096x4096", 32)])
def test_k_of_one_step(h, name, K):
    # K equal to one K step of the tiled kernels (the one-region step pinned, as
    # the planner may otherwise take the two-region step as one short tail):
    # one main step, no tail, no split
    info, _ = run(h, synth.make(name, M=130, N=96, K=K), opts=dg.dg_plan_opts(force_k_tile=K))
    assert info.n_main == 1 and info.n_tail == 0 and info.split_k == 1 and info.k_main == K


@pytest.mark.parametrize("name,M,N,K,split,path,pad", [
    # few outputs over many slices (32 to 160): the split-K reduction sums runs of
    # slices per group of four outputs, group counts 1024, 136, 65 (the last
    # workgroup partly empty), 128 and 256
    ("i8_4096x4096x4096", 64, 64, 8192, 64, "tiled", 0),
    ("i8_4096x4096x4096", 8, 68, 8192, 128, "tiled", 8),
    ("f16_256x256x256_alpha_beta_d", 1, 260, 12800, 160, "skinny", 8),
    ("f16_256x256x256_alpha_beta_d", 8, 64, 8192, 32, "skinny", 0),
    ("f16_256x256x256_alpha_beta_d", 16, 64, 8192, 64, "tiled", 0),
])
def test_reduce_many_runs(h, name, M, N, K, split, path, pad):
    w = synth.make(name, M=M, N=N, K=K)
    p = dg.DG_PATH_TILED if path == "tiled" else dg.DG_PATH_SKINNY
    info, _ = run(h, w, pad=pad, opts=dg.dg_plan_opts(force_split_k=split, force_path=p))
    assert info.split_k == split


def test_config_bf16_1x256x12800_full(h):
    run(h, synth.make("bf16_1x256x12800"))


def test_config_e2m1_1x4096x4096_full(h):
    run(h, synth.make("e2m1_1x4096x4096"))


# ------------------------------------------------------------ epilogues
def test_requantise_bit_exact(h):
    w = synth.make("i8_4096x4096x4096", M=130, N=96, K=512)
    rq_bias = synth.uniform(9, 96, -4, 4).to(torch.float32)
    for epi in ("requant_i8", "requant_f16"):
        for s_ in (1.0 / 4096, 3.1e-5):
            run(h, w, epilogue=epi, out="i8" if epi == "requant_i8" else "f16",
                requant_scale=s_, rq_bias=rq_bias if epi == "requant_i8" else None)
        run(h, w, epilogue=epi, out="i8" if epi == "requant_i8" else "f16", requant_scale=1 / 8192,
            opts=dg.dg_plan_opts(force_split_k=2, force_path=dg.DG_PATH_TILED))


def test_int_alpha_beta_d(h):
    w = synth.make("i8_4096x4096x4096", M=100, N=64, K=256)
    w.tensors["D"] = synth.int8_uniform(11, 100 * 64).view(100, 64).to(torch.int32) * 1000
    run(h, w, alpha=3, beta=-2)


@pytest.mark.parametrize("path,name,colm", [("f16", "f16_2048x2048x8192_bias_gelu", False),
                                            ("f16", "f16_2048x2048x8192_bias_gelu", True),
                                            ("bf16", "bf16_16x4096x131072", False),
                                            ("i8", "i8_4096x4096x4096", False),
                                            ("i8", "i8_4096x4096x4096", True),
                                            ("e2m1", "e2m1_4096x4096x4096", True)])
def test_small_tiles_with_beta_d(h, path, name, colm):
    # beta * D on every 64x64 tile (both K steps; the planner takes them for small
    # problems such as 256^3 with D), unsplit, with ragged M: N = 70 on padded
    # rows (the last, partial column group of a row goes element by element) and
    # N = 64 on tight ones.
    M, K = 100, 512
    region = 64 if path == "i8" else 32
    for kr in ((1,) if path == "e2m1" else (1, 2)):
        for N, pad in ((70, 2), (64, 0)):
            w = synth.make(name, M=M, N=N, K=K)
            if path == "i8":
                w.tensors["D"] = synth.int8_uniform(11, M * N).view(M, N).to(torch.int32) * 1000
                alpha, beta = 3, -2
            else:
                w.tensors["D"] = synth.to_storage(synth.uniform(7, M * N, -1, 1), TORCH_OUT[w.out]).view(M, N)
                alpha, beta = 1.25, 0.5
            o = dg.dg_plan_opts(force_path=dg.DG_PATH_TILED, force_m_tile=64, force_n_tile=64, force_waves=4,
                                force_k_tile=region * kr, force_split_k=1)
            info, st = run(h, w, opts=o, b_colmajor=colm, pad=pad, alpha=alpha, beta=beta)
            assert info.m_tile == 64 and info.n_tile == 64 and info.split_k == 1 and st["n"] == M * N


def test_pad_k(h):
    # K not a multiple of the MFMA depth: the aligned part runs as planned, a tail
    # kernel adds the rest as one more partial slice, the reduction applies the
    # epilogue.  Rows are padded to 16-byte leading dimensions.
    o = dg.dg_plan_opts(pad_k=1)
    # tiled f16, 7 full steps + 8, bias + GELU (applied by the reduction)
    run(h, synth.make("f16_2048x2048x8192_bias_gelu", M=300, N=264, K=7 * 32 + 8), opts=o, pad=8)
    # tiled f16 with a K split, then the tail
    run(h, synth.make("f16_2048x2048x8192_bias_gelu", M=512, N=512, K=2048 + 8),
        opts=dg.dg_plan_opts(pad_k=1, force_split_k=4, force_path=dg.DG_PATH_TILED), pad=8)
    # skinny bf16 (VALU at M=1, MFMA at M=16)
    run(h, synth.make("bf16_1x4096x131072", M=1, N=1000, K=4100), opts=o, pad=8)
    run(h, synth.make("bf16_16x4096x131072", M=16, N=512, K=1004), opts=o, pad=8)
    # int8, bit-exact, K = 3 * 32 + 4, B row- and column-major
    w = synth.make("i8_4096x4096x4096", M=300, N=200, K=100)
    run(h, w, opts=o, pad=16)
    run(h, w, opts=o, pad=16, b_colmajor=True)
    # fp16 with alpha, beta * D and only a tail (K < 16)
    run(h, synth.make("f16_256x256x256_alpha_beta_d", M=64, N=72, K=7), opts=o, pad=8)
    # the 16x16 MFMA tile with a half step, then the tail (fp16 and int8)
    o16 = dg.dg_plan_opts(pad_k=1, force_path=dg.DG_PATH_TILED, force_m_tile=256, force_n_tile=256,
                          force_waves=8, force_mfma=16)
    run(h, synth.make("f16_2048x2048x8192_bias_gelu", M=300, N=264, K=7 * 32 + 16 + 8), opts=o16, pad=8)
    run(h, synth.make("i8_4096x4096x4096", M=300, N=200, K=5 * 64 + 32 + 4), opts=o16, pad=16)


def test_k_zero_and_empty(h):
    # K = 0: the sum is empty and C = act(alpha*0 + beta*D + bias)
    run(h, synth.make("f16_256x256x256_alpha_beta_d", M=64, N=72, K=0))
    run(h, synth.make("f16_2048x2048x8192_bias_gelu", M=40, N=64, K=0))
    # every loop shape with an empty K range (eight-wave and four-wave tiles)
    # (the K step: regions of 32 k for 16-bit operands, 64 k for int8)
    for bm, bn, nw, kr, ms in ((256, 256, 8, 1, 32), (128, 256, 4, 1, 32), (128, 128, 4, 1, 32),
                               (256, 256, 4, 2, 32), (256, 256, 8, 1, 16)):
        for name, region in (("f16_256x256x256_alpha_beta_d", 32), ("i8_4096x4096x4096", 64)):
            o = dg.dg_plan_opts(force_m_tile=bm, force_n_tile=bn, force_path=dg.DG_PATH_TILED,
                                force_waves=nw, force_k_tile=region * kr, force_mfma=ms)
            run(h, synth.make(name, M=300, N=260, K=0), opts=o)
    # M = 0 or N = 0: nothing to do, nothing launched
    Ce = torch.empty(0, 64, dtype=torch.float16, device=DEV)
    h.gemm(torch.empty(0, 16, dtype=torch.float16, device=DEV),
           torch.zeros(16, 64, dtype=torch.float16, device=DEV), Ce)
    torch.cuda.synchronize()


def test_errors_on_device_handle(h):
    A = torch.zeros(64, 64, dtype=torch.float16, device=DEV)
    B = torch.zeros(64, 64, dtype=torch.float16, device=DEV)
    Cd = torch.zeros(64, 64, dtype=torch.float16, device=DEV)
    with pytest.raises(dg.DGError) as e:
        h.gemm(A, B, Cd, beta=1.0, D=None)
    assert e.value.status == dg.DG_ERR_INVALID_ARG
    with pytest.raises(dg.DGError) as e:
        h.gemm(A, B, Cd, epilogue="bias")
    assert e.value.status == dg.DG_ERR_INVALID_ARG
    o = dg.dg_plan_opts(force_split_k=4, force_path=dg.DG_PATH_TILED)
    with pytest.raises(dg.DGError) as e:
        h.gemm(A, B, Cd, opts=o, workspace=torch.empty(16, dtype=torch.uint8, device=DEV))
    assert e.value.status == dg.DG_ERR_WORKSPACE
    with pytest.raises(dg.DGError) as e:
        h.gemm(A[:, 1:], B[1:], Cd, K=63)
    assert e.value.status == dg.DG_ERR_ALIGNMENT


def test_operand_of_4_gib_is_refused_by_the_tiled_path(h):
    # The tiled kernels address operands with 32-bit offsets: an A of exactly
    # 4 GiB (32 rows of 2^26 fp16) is refused before anything is launched (the
    # operands are real allocations, so even a launch would stay inside them).
    K = 1 << 26
    A = torch.empty(32, K, dtype=torch.float16, device=DEV)
    B = torch.empty(K, 16, dtype=torch.float16, device=DEV)
    Cd = torch.empty(32, 16, dtype=torch.float16, device=DEV)
    with pytest.raises(dg.DGError) as e:
        h.gemm(A, B, Cd, opts=dg.dg_plan_opts(force_path=dg.DG_PATH_TILED))
    assert e.value.status == dg.DG_ERR_UNSUPPORTED and "4 GiB" in str(e.value)
    del A, B, Cd
    torch.cuda.empty_cache()


# ------------------------------------------------------ full-size workloads
@pytest.mark.parametrize("name,col_chunk", [("i8_4096x4096x4096", 0), ("f16_4096x4096x4096", 0),
                                            ("f16_2048x2048x8192_bias_gelu", 0),
                                            ("e2m1_4096x4096x4096", 0),
                                            ("bf16_1x4096x131072", 512), ("bf16_16x4096x131072", 512)])
def test_full_size_every_output(h, name, col_chunk):
    # the workload at its full size, in the launch configuration the benchmark
    # times (planner's choice), compared with the oracle on every output
    w = synth.make(name, device=DEV)
    info, st = run(h, w, col_chunk=col_chunk)
    assert st["n"] == w.M * w.N


@pytest.mark.parametrize("name,region", [("i8_4096x4096x4096", 64), ("f16_2048x2048x8192_bias_gelu", 32),
                                         ("bf16_16x4096x131072", 32)])
def test_short_k_on_the_16x16_tile(h, name, region):
    # The eight-wave 16x16 tile over a row-major B reads the next stage's B
    # fragments during the MFMAs: slices of one, two and three K steps (and a
    # split whose slices have one step each) take its prologue, its last step
    # and the steps in between, against the oracle.
    for steps, split in ((1, 1), (2, 1), (3, 1), (4, 4), (5, 1)):
        w = synth.make(name, M=300, N=264, K=steps * region)
        o = dg.dg_plan_opts(force_path=dg.DG_PATH_TILED, force_m_tile=256, force_n_tile=256, force_waves=8,
                            force_mfma=16, force_split_k=split)
        info, st = run(h, w, opts=o, pad=8)
        assert info.mfma_m == 16 and info.split_k == split and st["n"] == w.M * w.N


@pytest.mark.parametrize("name,ms", [("i8_4096x4096x4096", 16), ("i8_4096x4096x4096", 32),
                                     ("f16_4096x4096x4096", 16), ("f16_4096x4096x4096", 32),
                                     ("e2m1_4096x4096x4096", 16), ("e2m1_4096x4096x4096", 32)])
def test_full_size_each_mfma_block(h, name, ms):
    # the 4096^3 workloads with the eight-wave 256x256 tile on each MFMA block
    # (32x32 and 16x16), every output against the oracle
    w = synth.make(name, device=DEV)
    o = dg.dg_plan_opts(force_path=dg.DG_PATH_TILED, force_m_tile=256, force_n_tile=256, force_waves=8,
                        force_mfma=ms)
    info, st = run(h, w, opts=o)
    assert st["n"] == w.M * w.N and info.mfma_m == ms
