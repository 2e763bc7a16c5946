"""GPU: the C-ABI calls captured in a HIP graph and replayed.

A captured graph keeps the kernels of a call with their pointers, so each
replay computes on whatever the input buffers hold at that moment.  Every case
captures its calls once on a side stream; then, three times over, it rewrites
the inputs in place (eager work on the default stream, then a synchronisation),
replays the graph, and compares its outputs bit for bit with an eager call on
the same inputs: the kernels, their launch shapes and their order of additions
are the same, so the two results are identical.  The first eager result is
also checked against the oracle.  The cases are the configurations the
benchmark times through graphs (split-K partial sums with the ordered
reduction, the skinny streaming kernels, a small tiled GEMM reading D) plus
the MX quantiser feeding a split MX GEMM.
"""
import pytest
import torch

import oracle
from tests.parity import bits, check_fp, say, tol_for
from tile_planned_generator_amd import dg, synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
WS_BYTES = 64 << 20


@pytest.fixture(scope="module")
def h():
    torch.cuda.init()
    hd = dg.Handle(0)
    yield hd
    hd.close()


def f16(seed, n, dtype=torch.float16):
    return synth.to_storage(synth.normal(seed, n), dtype)


def case_skinny_bf16(h):
    # 1 x 256 x 12800: the skinny VALU kernel over 160 K slices, then the reduction
    M, N, K = 1, 256, 12800
    A = torch.empty(M, K, dtype=torch.bfloat16, device=DEV)
    B = torch.empty(K, N, dtype=torch.bfloat16, device=DEV)

    def refill(r):
        A.copy_(f16(900 + r, M * K, torch.bfloat16).view(M, K))
        B.copy_(f16(950 + r, K * N, torch.bfloat16).view(K, N))

    def launch(out, ws):
        return h.gemm(A, B, out[0], workspace=ws)

    def check(out):
        R = oracle.gemm_real(bits(A.cpu()), bits(B.cpu()), a_kind="bf16", b_kind="bf16")
        check_fp(out[0].cpu(), R, tol_for("bf16", "bf16"))

    return refill, launch, [torch.empty(M, N, dtype=torch.bfloat16, device=DEV)], check


def case_tiled_i8_split(h):
    # int8 -> int32, tiled, four K slices and the four-column reduction
    M, N, K = 256, 320, 4096
    A = torch.empty(M, K, dtype=torch.int8, device=DEV)
    B = torch.empty(K, N, dtype=torch.int8, device=DEV)
    opts = dg.dg_plan_opts(force_path=dg.DG_PATH_TILED, force_split_k=4)

    def refill(r):
        A.copy_(synth.int8_uniform(910 + r, M * K).view(M, K))
        B.copy_(synth.int8_uniform(960 + r, K * N).view(K, N))

    def launch(out, ws):
        info = h.gemm(A, B, out[0], opts=opts, workspace=ws)
        assert info.split_k == 4
        return info

    def check(out):
        _, Cw, _ = oracle.gemm_int(A.cpu().numpy(), B.cpu().numpy())
        assert (out[0].cpu().numpy() == Cw).all()

    return refill, launch, [torch.empty(M, N, dtype=torch.int32, device=DEV)], check


def case_tiled_f16_alpha_beta_d(h):
    # 256^3 fp16 with C = A.B + 0.5 D: the small tiled kernel reading D
    M = N = K = 256
    A = torch.empty(M, K, dtype=torch.float16, device=DEV)
    B = torch.empty(K, N, dtype=torch.float16, device=DEV)
    D = torch.empty(M, N, dtype=torch.float16, device=DEV)

    def refill(r):
        A.copy_(f16(920 + r, M * K).view(M, K))
        B.copy_(f16(970 + r, K * N).view(K, N))
        D.copy_(f16(990 + r, M * N).view(M, N))

    def launch(out, ws):
        return h.gemm(A, B, out[0], beta=0.5, D=D, workspace=ws)

    def check(out):
        R = oracle.gemm_real(bits(A.cpu()), bits(B.cpu()), a_kind="f16", b_kind="f16", beta=0.5,
                             D=bits(D.cpu()), d_kind="f16")
        check_fp(out[0].cpu(), R, tol_for("f16", "f16"))

    return refill, launch, [torch.empty(M, N, dtype=torch.float16, device=DEV)], check


def case_skinny_e2m1(h):
    # M = 1 fp16 activations x e2m1 weights with fp16 group scales (skinny e2m1)
    M, N, K = 1, 512, 4096
    w = synth.make("e2m1_1x4096x4096", M=M, N=N, K=K, seed=930).tensors
    A = torch.empty(M, K, dtype=torch.float16, device=DEV)
    B = dg.pack_e2m1(w["codes"]).to(DEV)
    S = dg.scales_gn(w["scale"]).to(DEV)

    def refill(r):
        A.copy_(f16(931 + r, M * K).view(M, K))

    def launch(out, ws):
        return h.gemm(A, B, out[0], b_scale=S, b_layout=dg.DG_COL_MAJOR, workspace=ws)

    def check(out):
        R = oracle.gemm_real(bits(A.cpu()), bits(w["codes"]), a_kind="f16", b_kind="e2m1",
                             scale=bits(w["scale"]), group_k=32)
        check_fp(out[0].cpu(), R, tol_for("e2m1", "f16"))

    return refill, launch, [torch.empty(M, N, dtype=torch.float16, device=DEV)], check


def case_quant_then_mx_split(h):
    # fp16 activations -> MX fp8 codes and e8m0 scales -> MX GEMM over two K slices
    M, N, K = 160, 192, 640
    w = synth.make("mx_4096x4096x4096", M=M, N=N, K=K, seed=940).tensors
    X = torch.empty(M, K, dtype=torch.float16, device=DEV)
    B = dg.pack_e2m1(w["codes"]).to(DEV)
    SB = torch.zeros(K // 32, (N + 3) // 4 * 4, dtype=torch.uint8, device=DEV)
    SB[:, :N] = w["SB"].to(DEV)
    opts = dg.dg_plan_opts(force_path=dg.DG_PATH_TILED, force_split_k=2)

    def refill(r):
        X.copy_(synth.make("mxq_4096x4096", M=M, K=K, seed=941 + r).tensors["X"])

    def launch(out, ws):
        codes, scales, C = out
        h.quant_mx(X, codes, scales[:, :M])
        info = h.gemm_mx(codes, scales, B, SB, C, opts=opts, workspace=ws)
        assert info.split_k == 2
        return info

    def check(out):
        codes, scales, C = (t.cpu() for t in out)
        rc, rs = oracle.quant_mx(bits(X.cpu()))
        assert (codes.numpy() == rc).all()
        assert (scales[:, :M].t().numpy() == rs).all()
        R = oracle.gemm_mx(rc, rs, w["codes"].numpy(), w["SB"].numpy())
        check_fp(C, R, "f16")

    outs = [torch.empty(M, K, dtype=torch.uint8, device=DEV),
            torch.zeros(K // 32, (M + 3) // 4 * 4, dtype=torch.uint8, device=DEV),
            torch.empty(M, N, dtype=torch.float16, device=DEV)]
    return refill, launch, outs, check


CASES = {
    "skinny_bf16_1x256x12800": case_skinny_bf16,
    "tiled_i8_split4": case_tiled_i8_split,
    "tiled_f16_256_alpha_beta_d": case_tiled_f16_alpha_beta_d,
    "skinny_e2m1_1x512x4096": case_skinny_e2m1,
    "quant_mx_then_gemm_mx_split2": case_quant_then_mx_split,
}


@pytest.mark.parametrize("name", list(CASES))
def test_graph_replays_match_eager(h, name):
    say(f"[case] graph {name}")
    refill, launch, outs_g, check = CASES[name](h)
    outs_e = [torch.empty_like(t) for t in outs_g]
    ws_g = torch.empty(WS_BYTES, dtype=torch.uint8, device=DEV)
    ws_e = torch.empty(WS_BYTES, dtype=torch.uint8, device=DEV)
    refill(0)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        launch(outs_g, ws_g)   # once outside the capture
        s.synchronize()
        with torch.cuda.graph(g, stream=s):
            launch(outs_g, ws_g)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()

    for r in range(3):
        refill(r)
        for t in outs_g + outs_e:   # (bytes the calls do not write stay equal)
            t.fill_(0x55 if t.dtype == torch.uint8 else 7)
        launch(outs_e, ws_e)
        torch.cuda.synchronize()
        if r == 0:
            check(outs_e)
        g.replay()
        torch.cuda.synchronize()
        for i, (t_g, t_e) in enumerate(zip(outs_g, outs_e)):
            assert torch.equal(t_g, t_e), (name, r, i)
        say(f"       replay {r} equal to the eager call")
