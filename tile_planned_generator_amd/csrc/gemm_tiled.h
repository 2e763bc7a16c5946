// gemm_tiled.h - tiled MFMA GEMM kernel template for gfx950 (the compute-bound path).
//
// One workgroup computes a BM x BN tile of C over one K slice.
//   - Operands go from HBM straight into LDS with buffer loads that write LDS
//     directly (buffer_load_dwordx4 ... lds): no staging registers and no LDS
//     store instructions.  Two LDS stages: while the MFMAs consume stage s, the
//     loads of step s+1 fill the other stage; one vmcnt wait and one barrier per
//     step.  The buffer range check returns zeros past the end of an operand, so
//     ragged rows and K tails need no clamping.
//   - A (and a K-contiguous B) is kept as rows of 128 bytes (eight 16-byte
//     chunks, one K step) whose chunk index is XORed with (row >> 1) & 7, so the
//     16 rows a 16-lane phase of a fragment read touches hit 16 distinct
//     16-byte bank groups of gfx950's 64-bank LDS.
//   - A row-major B (N contiguous) is kept as it is in memory, K rows of BN
//     columns, and read with the transposing LDS reads of gfx950
//     (ds_read_b64_tr_b16 / ds_read_b64_tr_b8): within each group of 16 lanes,
//     lane i = 4a+b (b16) receives element b of the 8-byte pieces addressed by
//     lanes a, a+4, a+8, a+12 (for b8: lane i = 8a+b, byte b of lanes a, a+2,
//     ..., a+14), so lanes that address 4 (8) consecutive K rows of 4 (8)
//     neighbouring columns hand every lane the consecutive K values of one
//     column - the MFMA B operand.  The 16-byte chunks of row k are XORed with
//     4*(k & 3) (b16) or 2*(k & 7) (b8) so those rows fall into distinct banks.
//   - e2m1 codes are staged packed (two per byte), chunk-major, with their
//     fp16 group scales, and decoded to fp16 when the fragment is read
//     (v_cvt_scalef32_pk_f16_fp4 with a unit scale, then a packed fp16 multiply
//     by the group scale).
//   - MFMA fragments are read from LDS one k-substep ahead of the MFMAs that use
//     them; accumulators stay in registers for the whole K range (32x32 blocks:
//     v_mfma_f32_32x32x16_f16/_bf16, v_mfma_i32_32x32x32_i8).
//   - The K schedule is n_main steps of the full step (64 k for 16-bit, 128 k
//     for int8) then at most one smaller tail step that still fills whole
//     MFMAs (the pages' variable K step, [generator] DeepGEMM article, kwkr.cn,
//     section 2.2, first layer).
//   - The epilogue (alpha, beta*D, bias, GELU, requantise, conversion) runs once
//     per output element after the K loop, four columns per lane with vector
//     loads and stores; with a K split the raw fp32 / int32 partials go to the
//     workspace and a reduce kernel applies the epilogue.
// Tiles are visited in a grouped order and every XCD gets a contiguous run of
// them, so tiles that share rows of A or columns of B share an L2.
#pragma once
#include "kcommon.h"
#include "catalogue.h"

namespace dg {

typedef short short4v __attribute__((ext_vector_type(4)));
typedef int int2v __attribute__((ext_vector_type(2)));
#define DG_LDS __attribute__((address_space(3)))

// Raw buffer descriptor over [base, base + bytes): loads at offsets at or past
// `bytes` return zero.
DG_DEV __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             0x00020000);
}

// 16 bytes per lane from buffer offset `off`, written to LDS at lds + 16 * lane
// (`lds` must be the same for the whole wave).
DG_DEV void buf_ld16_lds(__amdgpu_buffer_rsrc_t r, uint32_t off, void *lds)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (DG_LDS void *)lds, 16, (int)off, 0, 0, 0);
}

DG_DEV unsigned short buf_ld2(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
}

template <int PATH, int BKMAJ, int BM, int BN, int WM, int WN>
__global__ void __launch_bounds__(WM *WN * 64, 1) gemm_tiled_kernel(TiledArgs p)
{
    constexpr int NW = WM * WN;
    constexpr int NT = NW * 64;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int FM = WTM / 32, FN = WTN / 32;
    constexpr bool IS_I8 = PATH == P_I8;
    constexpr bool IS_E2M1 = PATH == P_E2M1;
    constexpr int BKE = IS_I8 ? 128 : 64;      // k elements per full step
    constexpr int KSUB = IS_I8 ? 32 : 16;      // k elements per MFMA
    constexpr int NSUB = BKE / KSUB;           // MFMA k-substeps per full step
    constexpr int ESZ = IS_I8 ? 1 : 2;         // bytes per element of A and of a 16-bit / int8 B
    constexpr int A_BYTES = BM * 128;
    constexpr int B_TILE = IS_E2M1 ? BN * 32 : BN * 128;   // e2m1: BKE/2 bytes of codes per column
    constexpr int S_BYTES = IS_E2M1 ? BN * 4 : 0;
    constexpr int STAGE = A_BYTES + B_TILE + S_BYTES;
    constexpr int RB = BN * ESZ;               // bytes per K row of a row-major B tile
    constexpr int CPR = RB / 16;               // 16-byte chunks per such row
    static_assert(FM >= 1 && FN >= 1 && WTM % 32 == 0 && WTN % 32 == 0, "wave tile");
    static_assert(2 * STAGE == tiled_lds_bytes(PATH, BM, BN), "LDS size");
    // direct-to-LDS loads: every wave instruction fills 1 KB (64 lanes x 16 B)
    constexpr int A_NL = A_BYTES / 1024, B_NL = B_TILE / 1024;   // 1 KB loads per step
    constexpr int A_LD = (A_NL + NW - 1) / NW;                   // per wave and step
    constexpr int B_LD = (B_NL + NW - 1) / NW;
    static_assert(A_NL * 1024 == A_BYTES && B_NL * 1024 == B_TILE, "tile not whole 1 KB loads");
    constexpr int SC_IT = IS_E2M1 ? (BN * 2 + NT - 1) / NT : 0;

    __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];

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

    const int M = p.M, N = p.N;
    const uint32_t lda_b = (uint32_t)(p.lda * ESZ);
    const uint32_t ldb_b = (uint32_t)(IS_E2M1 ? p.ldb / 2 : p.ldb * ESZ);
    // Operand extents, in bytes from the tile origin to the end of the last
    // valid element (a 16-byte chunk never straddles it: K and the column
    // blocks are 16-byte multiples).  The host checks they fit 32 bits.
    const char *Abase = reinterpret_cast<const char *>(p.A) + (int64_t)m0 * lda_b;
    const uint32_t a_bytes = (uint32_t)((M - m0 - 1) * (int64_t)lda_b + (int64_t)p.K * ESZ);
    const char *Bbase;
    uint32_t b_bytes;
    if constexpr (BKMAJ) {
        const int64_t rowb = IS_E2M1 ? p.K / 2 : (int64_t)p.K * ESZ;
        Bbase = reinterpret_cast<const char *>(p.B) + (int64_t)n0 * ldb_b;
        b_bytes = (uint32_t)((N - n0 - 1) * (int64_t)ldb_b + rowb);
    } else {
        const int64_t cpb = 16 / ESZ;                        // columns per 16-byte chunk
        const int64_t nr = ((int64_t)N + cpb - 1) / cpb * cpb;
        Bbase = reinterpret_cast<const char *>(p.B) + (int64_t)n0 * ESZ;
        b_bytes = (uint32_t)((p.K - 1) * (int64_t)ldb_b + (nr - n0) * ESZ);
    }
    const char *Sbase = IS_E2M1 ? reinterpret_cast<const char *>(p.scale) + (int64_t)n0 * p.ld_scale * 2
                                : nullptr;
    const uint32_t s_bytes = IS_E2M1 ? (uint32_t)((N - n0) * (int64_t)p.ld_scale * 2) : 0;

    // ---- per-lane source offsets of this wave's direct-to-LDS loads.  Load i of
    // wave w fills LDS bytes [(i*NW + w) * 1024, +1024) of the operand region;
    // lane l writes 16-byte chunk pc = (i*NW + w)*64 + l of it.  Rows past the
    // operand start at or beyond its extent, so their loads return zeros.
    uint32_t oa[A_LD];
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
        const int pc = (i * NW + wave) * 64 + lane;
        const int r = pc >> 3, c = (pc & 7) ^ ((r >> 1) & 7);
        oa[i] = r * lda_b + c * 16;
    }
    uint32_t ob[B_LD];
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
        const int pc = (i * NW + wave) * 64 + lane;
        if constexpr (IS_E2M1) {            // chunk-major: [chunk 0/1][BN columns][16 B]
            const int c = pc / BN, r = pc % BN;
            ob[i] = r * ldb_b + c * 16;
        } else if constexpr (BKMAJ) {       // as A, rows are columns of B
            const int r = pc >> 3, c = (pc & 7) ^ ((r >> 1) & 7);
            ob[i] = r * ldb_b + c * 16;
        } else {                            // K rows of BN columns
            const int k = pc / CPR, pcol = pc % CPR;
            const int sw = IS_I8 ? (2 * (k & 7)) % CPR : (4 * (k & 3)) % CPR;
            ob[i] = k * ldb_b + (pcol ^ sw) * 16;
        }
    }
    uint32_t os[SC_IT > 0 ? SC_IT : 1];
    if constexpr (IS_E2M1) {
#pragma unroll
        for (int i = 0; i < SC_IT; ++i) {
            const int q = min(tid + i * NT, BN * 2 - 1), r = q >> 1, g = q & 1;
            os[i] = (uint32_t)(r * p.ld_scale + g) * 2;
        }
    }
    unsigned short rs[SC_IT > 0 ? SC_IT : 1];

    // Issue the loads of the step starting at k0 into LDS stage `buf` (the e2m1
    // scales go through registers and are written by store_scales).
    auto load_stage = [&](int k0, int buf) {
        char *sA = smem + buf * STAGE;
        char *sB = sA + A_BYTES;
        const __amdgpu_buffer_rsrc_t rA =
            make_rsrc(Abase + (int64_t)k0 * ESZ, a_bytes - (uint32_t)(k0 * ESZ));
#pragma unroll
        for (int i = 0; i < A_LD; ++i)
            if (A_NL % NW == 0 || i * NW + wave < A_NL)   // wave-uniform
                buf_ld16_lds(rA, oa[i], sA + (i * NW + wave) * 1024);
        uint32_t kb;
        if constexpr (IS_E2M1) kb = (uint32_t)(k0 >> 1);
        else if constexpr (BKMAJ) kb = (uint32_t)(k0 * ESZ);
        else kb = (uint32_t)k0 * ldb_b;
        const __amdgpu_buffer_rsrc_t rB = make_rsrc(Bbase + kb, b_bytes - kb);
#pragma unroll
        for (int i = 0; i < B_LD; ++i)
            if (B_NL % NW == 0 || i * NW + wave < B_NL)   // wave-uniform
                buf_ld16_lds(rB, ob[i], sB + (i * NW + wave) * 1024);
        if constexpr (IS_E2M1) {
            const uint32_t sb = (uint32_t)(k0 >> 5) * 2;
            const __amdgpu_buffer_rsrc_t rS = make_rsrc(Sbase + sb, s_bytes - sb);
#pragma unroll
            for (int i = 0; i < SC_IT; ++i) rs[i] = buf_ld2(rS, os[i]);
        }
    };
    auto store_scales = [&](int buf) {
        if constexpr (IS_E2M1) {
            unsigned short *sS = reinterpret_cast<unsigned short *>(smem + buf * STAGE + A_BYTES + B_TILE);
#pragma unroll
            for (int i = 0; i < SC_IT; ++i) {
                const int q = tid + i * NT;
                if (q < BN * 2) sS[q] = rs[i];
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

    // fragments of one k-substep: FM A blocks and FN B blocks (16 bytes per lane each)
    struct Frag {
        u32x4 a[FM];
        u32x4 b[FN];
    };
    // transposing-read addressing of a row-major B tile: lane L of 16-lane group
    // g supplies K row (b16) kb + (L >> 2) at column 16*(g&1) + 4*(L&3), or (b8)
    // kb + (L >> 1) at column 16*(g&1) + 8*(L&1)
    const int grp16 = lane >> 4, L16 = lane & 15;
    auto read_frag = [&](const char *sA, const char *sB, int s, Frag &f) {
        const int c = 2 * s + kg;
#pragma unroll
        for (int mi = 0; mi < FM; ++mi) {
            const int row = wm * WTM + mi * 32 + lr;
            f.a[mi] = *reinterpret_cast<const u32x4 *>(sA + row * 128 + ((c ^ ((row >> 1) & 7)) << 4));
        }
#pragma unroll
        for (int ni = 0; ni < FN; ++ni) {
            const int col0 = wn * WTN + ni * 32;
            if constexpr (IS_E2M1) {
                const int row = col0 + lr;
                const int w = 2 * s + kg;   // 4-byte word of the column's 32 code bytes
                const unsigned codes =
                    *reinterpret_cast<const unsigned *>(sB + (w >> 2) * (BN * 16) + row * 16 + (w & 3) * 4);
                const _Float16 sc =
                    reinterpret_cast<const _Float16 *>(sB + B_TILE)[row * 2 + (s >> 1)];
                f.b[ni] = __builtin_bit_cast(u32x4, decode_e2m1x8(codes, sc));
            } else if constexpr (BKMAJ) {
                const int row = col0 + lr;
                f.b[ni] = *reinterpret_cast<const u32x4 *>(sB + row * 128 + ((c ^ ((row >> 1) & 7)) << 4));
            } else if constexpr (!IS_I8) {
                // two reads of 4 K rows each: K = 16s + 8*(g>>1) + {0..3, 4..7}
                const int col = col0 + 16 * (grp16 & 1) + 4 * (L16 & 3);
                const int kb = KSUB * s + 8 * (grp16 >> 1) + (L16 >> 2);
                const int cc = col >> 3, cb = (col & 7) * 2;
                const int k1 = kb, k2 = kb + 4;
                const short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (DG_LDS short4v *)(sB + k1 * RB + ((cc ^ ((4 * (k1 & 3)) % CPR)) << 4) + cb));
                const short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (DG_LDS short4v *)(sB + k2 * RB + ((cc ^ ((4 * (k2 & 3)) % CPR)) << 4) + cb));
                const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
                f.b[ni] = u32x4{l2.x, l2.y, h2.x, h2.y};
            } else {
                // two reads of 8 K rows each: K = 32s + 16*(g>>1) + {0..7, 8..15}
                const int col = col0 + 16 * (grp16 & 1) + 8 * (L16 & 1);
                const int kb = KSUB * s + 16 * (grp16 >> 1) + (L16 >> 1);
                const int cc = col >> 4, cb = col & 15;
                const int k1 = kb, k2 = kb + 8;
                const int2v lo = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                    (DG_LDS int2v *)(sB + k1 * RB + ((cc ^ ((2 * (k1 & 7)) % CPR)) << 4) + cb));
                const int2v hi = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                    (DG_LDS int2v *)(sB + k2 * RB + ((cc ^ ((2 * (k2 & 7)) % CPR)) << 4) + cb));
                f.b[ni] = u32x4{(unsigned)lo.x, (unsigned)lo.y, (unsigned)hi.x, (unsigned)hi.y};
            }
        }
    };
    auto mfmas = [&](const Frag &f) {
#pragma unroll
        for (int mi = 0; mi < FM; ++mi)
#pragma unroll
            for (int ni = 0; ni < FN; ++ni) {
                if constexpr (PATH == P_F16 || PATH == P_E2M1)
                    acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                        __builtin_bit_cast(half8, f.a[mi]), __builtin_bit_cast(half8, f.b[ni]),
                        acc[mi][ni], 0, 0, 0);
                else if constexpr (PATH == P_BF16)
                    acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        __builtin_bit_cast(bf16x8, f.a[mi]), __builtin_bit_cast(bf16x8, f.b[ni]),
                        acc[mi][ni], 0, 0, 0);
                else
                    acc[mi][ni] = __builtin_amdgcn_mfma_i32_32x32x32_i8(
                        __builtin_bit_cast(intx4, f.a[mi]), __builtin_bit_cast(intx4, f.b[ni]),
                        acc[mi][ni], 0, 0, 0);
            }
    };

    // ---- main loop: stage st & 1 is consumed while step st+1 streams into the other
    Frag fr[2];
    if (nsteps > 0) {
        load_stage(kbeg, 0);
        store_scales(0);
        __builtin_amdgcn_s_waitcnt(0);   // every counter at zero: the LDS-direct loads have landed
        __syncthreads();
        read_frag(smem, smem + A_BYTES, 0, fr[0]);
    }
    for (int st = 0; st < nsteps; ++st) {
        const int cur = st & 1;
        const bool more = st + 1 < nsteps;
        if (more) load_stage(kbeg + (st + 1) * BKE, cur ^ 1);
        const char *sA = smem + cur * STAGE;
        const char *sB = sA + A_BYTES;
        const int nsub = st < nfull ? NSUB : tail / KSUB;
#pragma unroll
        for (int s = 0; s < NSUB; ++s) {
            if (s < nsub) {
                if (s + 1 < nsub) read_frag(sA, sB, s + 1, fr[(s + 1) & 1]);
                mfmas(fr[s & 1]);
            }
        }
        if (more) {
            store_scales(cur ^ 1);
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            read_frag(smem + (cur ^ 1) * STAGE, smem + (cur ^ 1) * STAGE + A_BYTES, 0, fr[0]);
        }
    }

    // ---- epilogue: each wave stages 32 rows of its accumulators in LDS at a time
    // and stores them four columns per lane, row-contiguously.
    constexpr int RP = WTN + 4;   // padded row pitch (elements) of the staging area
    static_assert(NW * 32 * RP * 4 <= 2 * STAGE, "epilogue staging");
    __syncthreads();   // every wave is done with the last K stage
    using ScalarT = typename std::conditional<IS_I8, int32_t, float>::type;
    using Vec4 = typename std::conditional<IS_I8, intx4, floatx4>::type;
    ScalarT *sE = reinterpret_cast<ScalarT *>(smem) + wave * 32 * RP;
    constexpr int LPR = WTN / 4;    // lanes per row (4 columns each)
    constexpr int RPI = 64 / LPR;   // rows per iteration
    const int er = lane / LPR, ec = (lane % LPR) * 4;
    const bool vec_ok = epi_vec_ok(p.epi, p.split_k > 1, p.ws, N);
    // The store code (with the whole epilogue inlined) is too large to unroll FM
    // times, and a rolled loop must not index the accumulators at run time (that
    // demotes them all to private memory): the rolled loop stages block mi through
    // copies with constant indices instead.
#pragma unroll 1
    for (int mi = 0; mi < FM; ++mi) {
#pragma unroll
        for (int m = 0; m < FM; ++m) {
            if (m == mi) {
#pragma unroll
                for (int ni = 0; ni < FN; ++ni)
#pragma unroll
                    for (int v = 0; v < 16; ++v)
                        sE[(8 * (v >> 2) + 4 * kg + (v & 3)) * RP + ni * 32 + lr] = acc[m][ni][v];
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const int row0 = m0 + wm * WTM + mi * 32;
        const int col = n0 + wn * WTN + ec;
#pragma unroll 1
        for (int it = 0; it < 32 / RPI; ++it) {
            const int r = it * RPI + er;
            const int row = row0 + r;
            const Vec4 x = *reinterpret_cast<const Vec4 *>(sE + r * RP + ec);
            if (row < M) {
                if (vec_ok && col + 3 < N) {
                    if (p.split_k > 1)
                        *reinterpret_cast<Vec4 *>(reinterpret_cast<ScalarT *>(p.ws) +
                                                  ((int64_t)split * M + row) * N + col) = x;
                    else if constexpr (IS_I8)
                        epi_store4_i(p.epi, row, col, x);
                    else
                        epi_store4_f(p.epi, row, col, x);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        if (col + e < N) {
                            if (p.split_k > 1)
                                reinterpret_cast<ScalarT *>(p.ws)[((int64_t)split * M + row) * N + col + e] = x[e];
                            else if constexpr (IS_I8)
                                epi_store_i(p.epi, row, col + e, x[e]);
                            else
                                epi_store_f(p.epi, row, col + e, x[e]);
                        }
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
