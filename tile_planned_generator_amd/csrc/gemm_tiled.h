// gemm_tiled.h - tiled MFMA GEMM kernel template for gfx950 (the compute-bound path).
//
// One workgroup computes a BM x BN tile of C over one K slice:
//   - global -> register -> LDS staging, double-buffered: the loads of K step
//     s+1 are issued before the MFMAs of step s and written to the other LDS
//     buffer after them, one barrier per step;
//   - LDS rows of 128 bytes (eight 16-byte chunks) with the chunk index XORed
//     by (row & 7), so that the 32 rows one fragment read touches spread over
//     all banks;
//   - B stored N-contiguous (row-major K x N) is transposed in registers while
//     it is staged (8x8 16-bit or 8x16 byte transposes with v_perm), so every
//     LDS row of B holds one column with K contiguous, which is what the MFMA
//     operand wants; B stored K-contiguous is copied as is;
//   - e2m1 codes are staged packed (two per byte) with their fp16 group scales
//     and decoded to fp16 when the fragment is read (v_cvt_scalef32_pk_f16_fp4
//     with a unit scale, then a packed fp16 multiply by the group scale);
//   - the accumulators stay in registers for the whole K range (32x32 MFMA
//     blocks: v_mfma_f32_32x32x16_f16/_bf16, v_mfma_i32_32x32x32_i8);
//   - the K schedule is n_main steps of the full step (64 k for 16-bit, 128 k
//     for int8) then at most one smaller tail step that still fills whole
//     MFMAs (the pages' variable K step, [generator] DeepGEMM article, kwkr.cn,
//     section 2.2, first layer);
//   - the epilogue (alpha, beta*D, bias, GELU, requantise, conversion) is
//     applied to the accumulators in registers and stored once; with a K split
//     the raw fp32 / int32 partials go to the workspace instead and a reduce
//     kernel applies the epilogue.
// Tiles are visited in a grouped order and every XCD gets a contiguous run of
// them, so tiles that share rows of A or columns of B share an L2.
#pragma once
#include "kcommon.h"
#include "catalogue.h"

namespace dg {

template <int PATH, int BKMAJ, int BM, int BN, int WM, int WN>
__global__ void __launch_bounds__(WM *WN * 64, 1) gemm_tiled_kernel(TiledArgs p)
{
    constexpr int NT = WM * WN * 64;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int FM = WTM / 32, FN = WTN / 32;
    constexpr bool IS_I8 = PATH == P_I8;
    constexpr bool IS_E2M1 = PATH == P_E2M1;
    constexpr int BKE = IS_I8 ? 128 : 64;   // k elements per full step
    constexpr int KSUB = IS_I8 ? 32 : 16;   // k elements per MFMA
    constexpr int NSUB = BKE / KSUB;        // MFMA k-substeps per full step
    constexpr int ESZ = IS_I8 ? 1 : 2;      // bytes per element of A (and of 16-bit / int8 B)
    constexpr int A_BYTES = BM * 128;
    constexpr int B_ROW = IS_E2M1 ? 40 : 128;
    constexpr int B_BYTES = BN * B_ROW;
    constexpr int S_BYTES = IS_E2M1 ? BN * 4 : 0;
    constexpr int STAGE = A_BYTES + B_BYTES + S_BYTES;
    static_assert(FM >= 1 && FN >= 1 && WTM % 32 == 0 && WTN % 32 == 0, "wave tile");
    static_assert((BM * 8) % NT == 0, "A staging");
    static_assert(2 * STAGE == tiled_lds_bytes(PATH, BM, BN), "LDS size");

    // staging counts per thread
    constexpr int A_IT = BM * 8 / NT;
    constexpr int BK_IT = BKMAJ ? (IS_E2M1 ? (BN * 2 + NT - 1) / NT : BN * 8 / NT) : 0;
    constexpr int BN_IT = BKMAJ ? 0 : (BN + NT - 1) / NT;  // transpose blocks
    constexpr int SC_IT = IS_E2M1 ? (BN * 2 + NT - 1) / NT : 0;

    __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int lr = lane & 31, kg = lane >> 5;

    // ---- tile coordinates: XCD-contiguous runs, grouped along M
    const int T = p.tiles_m * p.tiles_n;
    const int t = xcd_remap(blockIdx.x, T);
    const int per_group = p.group_m * p.tiles_n;
    const int grp = t / per_group;
    const int first_m = grp * p.group_m;
    const int gm = min(p.tiles_m - first_m, p.group_m);
    const int tl = t - grp * per_group;
    const int m0 = (first_m + tl % gm) * BM;
    const int n0 = (tl / gm) * BN;

    // ---- K slice and its schedule
    const int split = blockIdx.y;
    const int kbeg = split * p.k_slice;
    const int kend = min(p.K, kbeg + p.k_slice);
    const int nfull = (kend - kbeg) / BKE;
    const int tail = (kend - kbeg) - nfull * BKE;
    const int nsteps = nfull + (tail ? 1 : 0);

    const char *Ab = reinterpret_cast<const char *>(p.A);
    const char *Bb = reinterpret_cast<const char *>(p.B);
    const int64_t lda_b = p.lda * ESZ;
    const int64_t ldb_b = IS_E2M1 ? p.ldb / 2 : p.ldb * ESZ;
    const int M = p.M, N = p.N;

    u32x4 ra[A_IT];
    u32x4 rbk[BK_IT > 0 ? BK_IT : 1];
    u32x4 rbn[BN_IT > 0 ? BN_IT : 1][8];
    unsigned short rs[SC_IT > 0 ? SC_IT : 1];

    // Loads always target valid memory (clamped rows, columns and chunks); data
    // past the end of a tail step is staged but never read by an MFMA.
    auto load_stage = [&](int k0, int klen) {
        const int kbytes = klen * ESZ;
#pragma unroll
        for (int i = 0; i < A_IT; ++i) {
            const int q = tid + i * NT, r = q >> 3, c = q & 7;
            const int gr = min(m0 + r, M - 1);
            const int cb = (c * 16 < kbytes) ? c * 16 : 0;
            ra[i] = ld16(Ab + gr * lda_b + (int64_t)k0 * ESZ + cb);
        }
        if constexpr (BKMAJ && !IS_E2M1) {
#pragma unroll
            for (int i = 0; i < BK_IT; ++i) {
                const int q = tid + i * NT, r = q >> 3, c = q & 7;
                const int gn = min(n0 + r, N - 1);
                const int cb = (c * 16 < kbytes) ? c * 16 : 0;
                rbk[i] = ld16(Bb + gn * ldb_b + (int64_t)k0 * ESZ + cb);
            }
        }
        if constexpr (IS_E2M1) {
#pragma unroll
            for (int i = 0; i < BK_IT; ++i) {
                const int q = min(tid + i * NT, BN * 2 - 1), r = q >> 1, c = q & 1;
                const int gn = min(n0 + r, N - 1);
                const int cb = (c * 32 < klen) ? c * 16 : 0;
                rbk[i] = ld16(Bb + gn * ldb_b + (int64_t)(k0 >> 1) + cb);
            }
            const unsigned short *S = reinterpret_cast<const unsigned short *>(p.scale);
#pragma unroll
            for (int i = 0; i < SC_IT; ++i) {
                const int q = min(tid + i * NT, BN * 2 - 1), r = q >> 1, g = q & 1;
                const int gn = min(n0 + r, N - 1);
                rs[i] = S[gn * p.ld_scale + (k0 >> 5) + ((g * 32 < klen) ? g : 0)];
            }
        }
        if constexpr (!BKMAJ) {
            constexpr int CW = IS_I8 ? 16 : 8;   // columns per transpose block
            constexpr int NB = BN / CW;          // blocks along N
#pragma unroll
            for (int i = 0; i < BN_IT; ++i) {
                const int q = min(tid + i * NT, BN - 1);
                const int kb8 = q / NB, nb = q % NB;
                int col = n0 + nb * CW;
                if (col >= N) col = 0;
                const int kr = (kb8 * 8 < klen) ? k0 + kb8 * 8 : k0;
#pragma unroll
                for (int r = 0; r < 8; ++r)
                    rbn[i][r] = ld16(Bb + (int64_t)(kr + r) * ldb_b + col * ESZ);
            }
        }
    };

    auto store_stage = [&](int buf) {
        char *sA = smem + buf * STAGE;
        char *sB = sA + A_BYTES;
#pragma unroll
        for (int i = 0; i < A_IT; ++i) {
            const int q = tid + i * NT, r = q >> 3, c = q & 7;
            *reinterpret_cast<u32x4 *>(sA + r * 128 + ((c ^ (r & 7)) << 4)) = ra[i];
        }
        if constexpr (BKMAJ && !IS_E2M1) {
#pragma unroll
            for (int i = 0; i < BK_IT; ++i) {
                const int q = tid + i * NT, r = q >> 3, c = q & 7;
                *reinterpret_cast<u32x4 *>(sB + r * 128 + ((c ^ (r & 7)) << 4)) = rbk[i];
            }
        }
        if constexpr (IS_E2M1) {
#pragma unroll
            for (int i = 0; i < BK_IT; ++i) {
                const int q = tid + i * NT, r = q >> 1, c = q & 1;
                if (q < BN * 2) {
                    u32x2 *d = reinterpret_cast<u32x2 *>(sB + r * 40 + c * 16);
                    d[0] = u32x2{rbk[i][0], rbk[i][1]};
                    d[1] = u32x2{rbk[i][2], rbk[i][3]};
                }
            }
            unsigned short *sS = reinterpret_cast<unsigned short *>(sB + B_BYTES);
#pragma unroll
            for (int i = 0; i < SC_IT; ++i) {
                const int q = tid + i * NT;
                if (q < BN * 2) sS[q] = rs[i];
            }
        }
        if constexpr (!BKMAJ && !IS_I8) {
            constexpr int NB = BN / 8;
#pragma unroll
            for (int i = 0; i < BN_IT; ++i) {
                const int q = tid + i * NT;
                if (q < BN) {
                    const int kb8 = q / NB, nb = q % NB;
                    u32x4 o[8];
                    transpose8x8_b16(rbn[i], o);
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        *reinterpret_cast<u32x4 *>(sB + (nb * 8 + j) * 128 + ((kb8 ^ j) << 4)) = o[j];
                }
            }
        }
        if constexpr (!BKMAJ && IS_I8) {
            constexpr int NB = BN / 16;
#pragma unroll
            for (int i = 0; i < BN_IT; ++i) {
                const int q = tid + i * NT;
                if (q < BN) {
                    const int kb8 = q / NB, nb = q % NB;
                    u32x2 o[16];
                    transpose8x16_b8(rbn[i], o);
#pragma unroll
                    for (int j = 0; j < 16; ++j) {
                        const int n = nb * 16 + j;
                        *reinterpret_cast<u32x2 *>(sB + n * 128 + (((kb8 >> 1) ^ (n & 7)) << 4) +
                                                   ((kb8 & 1) << 3)) = o[j];
                    }
                }
            }
        }
    };

    using AccT = typename std::conditional<IS_I8, intx16, floatx16>::type;
    AccT acc[FM][FN];
#pragma unroll
    for (int mi = 0; mi < FM; ++mi)
#pragma unroll
        for (int ni = 0; ni < FN; ++ni)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[mi][ni][v] = 0;

    auto substep = [&](const char *sA, const char *sB, int s) {
        const int c = 2 * s + kg;
        u32x4 af[FM];
#pragma unroll
        for (int mi = 0; mi < FM; ++mi) {
            const int row = wm * WTM + mi * 32 + lr;
            af[mi] = *reinterpret_cast<const u32x4 *>(sA + row * 128 + ((c ^ (lr & 7)) << 4));
        }
        u32x4 bfr[FN];
#pragma unroll
        for (int ni = 0; ni < FN; ++ni) {
            const int row = wn * WTN + ni * 32 + lr;
            if constexpr (IS_E2M1) {
                const unsigned codes = *reinterpret_cast<const unsigned *>(sB + row * 40 + 8 * s + 4 * kg);
                const _Float16 sc =
                    reinterpret_cast<const _Float16 *>(sB + B_BYTES)[row * 2 + (s >> 1)];
                bfr[ni] = __builtin_bit_cast(u32x4, decode_e2m1x8(codes, sc));
            } else {
                bfr[ni] = *reinterpret_cast<const u32x4 *>(sB + row * 128 + ((c ^ (lr & 7)) << 4));
            }
        }
#pragma unroll
        for (int mi = 0; mi < FM; ++mi)
#pragma unroll
            for (int ni = 0; ni < FN; ++ni) {
                if constexpr (PATH == P_F16 || PATH == P_E2M1)
                    acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                        __builtin_bit_cast(half8, af[mi]), __builtin_bit_cast(half8, bfr[ni]),
                        acc[mi][ni], 0, 0, 0);
                else if constexpr (PATH == P_BF16)
                    acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        __builtin_bit_cast(bf16x8, af[mi]), __builtin_bit_cast(bf16x8, bfr[ni]),
                        acc[mi][ni], 0, 0, 0);
                else
                    acc[mi][ni] = __builtin_amdgcn_mfma_i32_32x32x32_i8(
                        __builtin_bit_cast(intx4, af[mi]), __builtin_bit_cast(intx4, bfr[ni]),
                        acc[mi][ni], 0, 0, 0);
            }
    };

    // ---- main loop
    if (nsteps > 0) {
        load_stage(kbeg, nfull > 0 ? BKE : tail);
        store_stage(0);
        __syncthreads();
    }
    for (int st = 0; st < nsteps; ++st) {
        const int cur = st & 1;
        const bool more = st + 1 < nsteps;
        if (more) load_stage(kbeg + (st + 1) * BKE, st + 1 < nfull ? BKE : tail);
        const char *sA = smem + cur * STAGE;
        const char *sB = sA + A_BYTES;
        const int nsub = st < nfull ? NSUB : tail / KSUB;
#pragma unroll
        for (int s = 0; s < NSUB; ++s)
            if (s < nsub) substep(sA, sB, s);
        if (more) store_stage(cur ^ 1);
        __syncthreads();
    }

    // ---- epilogue: each wave stages 32 rows of its accumulators in LDS at a time
    // and stores them row-contiguously (coalesced), applying the epilogue once.
    constexpr int RP = WTN + 4;   // padded row pitch (elements) of the staging area
    static_assert(WM * WN * 32 * RP * 4 <= 2 * STAGE, "epilogue staging");
    __syncthreads();   // every wave is done with the last K stage
    using ScalarT = typename std::conditional<IS_I8, int32_t, float>::type;
    ScalarT *sE = reinterpret_cast<ScalarT *>(smem) + wave * 32 * RP;
    constexpr int CPL = WTN >= 64 ? WTN / 64 : 1;   // columns per lane per row
    constexpr int RPI = WTN >= 64 ? 1 : 64 / WTN;   // rows per iteration
    const int lcol = (WTN >= 64 ? lane * CPL : lane % WTN);
    const int lrow = (WTN >= 64 ? 0 : lane / WTN);
#pragma unroll
    for (int mi = 0; mi < FM; ++mi) {
#pragma unroll
        for (int ni = 0; ni < FN; ++ni)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                sE[(8 * (v >> 2) + 4 * kg + (v & 3)) * RP + ni * 32 + lr] = acc[mi][ni][v];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const int row0 = m0 + wm * WTM + mi * 32;
        const int col0 = n0 + wn * WTN;
        for (int r = lrow; r < 32; r += RPI) {
            const int row = row0 + r;
            if (row >= M) break;
#pragma unroll
            for (int cc = 0; cc < CPL; ++cc) {
                const int c = lcol + cc;
                const int col = col0 + c;
                if (col < N) {
                    const ScalarT x = sE[r * RP + c];
                    if (p.split_k > 1) {
                        reinterpret_cast<ScalarT *>(p.ws)[((int64_t)split * M + row) * N + col] = x;
                    } else {
                        if constexpr (IS_I8)
                            epi_store_i(p.epi, row, col, x);
                        else
                            epi_store_f(p.epi, row, col, x);
                    }
                }
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
}

}  // namespace dg
