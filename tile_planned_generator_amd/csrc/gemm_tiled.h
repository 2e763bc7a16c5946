// gemm_tiled.h - tiled MFMA GEMM kernel template for gfx950 (the compute-bound path).
//
// One workgroup computes a BM x BN tile of C over one K slice.
//   - Operands go from HBM straight into LDS with buffer loads that write LDS
//     directly (buffer_load_dwordx4 ... lds): no staging registers and no LDS
//     store instructions.  The buffer range check returns zeros past the end of
//     an operand, so ragged rows need no clamping.
//   - LDS stages of one K step each (two to five, as many as fit).  A K step is
//     one or two 64-byte K regions (KR, the K_tile the planner chooses: 32 or
//     64 k for 16-bit operands, 64 or 128 k for int8; 32 k for e2m1, 128 k for
//     MX), each region two MFMA k-substeps.  Step st runs its substeps with one
//     barrier before the last; the barrier is placed where every wave holds all
//     fragments of stage st in registers or in flight, so right after it the
//     loads of stage st+NBUF are issued into stage st's buffer.  Loads therefore
//     have NBUF-1 steps to land.  The barrier waits only for this wave's loads
//     of the next stage (vmcnt with the later stages still in flight) and for
//     its LDS reads; the workgroup fence of __syncthreads would wait for every
//     load.
//   - A (and a K-contiguous B) is kept as rows of 64 bytes per K region (four
//     16-byte chunks) whose chunk index is XORed with (row >> 2) & 3 for the
//     32x32 fragment reads and with (row >> 1) & 3 for the 16x16 ones: with
//     gfx950's LDS conflict counters, each is free of bank conflicts for its own
//     read (32 rows x one chunk, or 16 rows x four chunks, per instruction) and
//     costs the other twice the LDS cycles.
//   - A row-major B (N contiguous) is kept as it is in memory, K rows of BN
//     columns, and read with the transposing LDS reads of gfx950
//     (ds_read_b64_tr_b16 / ds_read_b64_tr_b8): within each group of 16 lanes,
//     lane i = 4a+b (b16) receives element b of the 8-byte pieces addressed by
//     lanes a, a+4, a+8, a+12 (for b8: lane i = 8a+b, byte b of lanes a, a+2,
//     ..., a+14), so lanes that address 4 (8) consecutive K rows of 4 (8)
//     neighbouring columns hand every lane the consecutive K values of one
//     column - the MFMA B operand.  The 16-byte chunks of row k are XORed with
//     4*(k & 3) (b16) or 2*(k & 7) (b8) so those rows fall into distinct banks;
//     the 16x16 reads, whose two half-waves read K rows 8 (b16) or 16 (b8)
//     apart, also take bit 3 (b16, as 2) or bit 4 (b8, as 1) of k, without which
//     the half-waves collide (measured: twice the LDS cycles).
//     These reads are issued from inline assembly: the compiler treats its own
//     transposing-read builtins as possibly aliasing every in-flight
//     direct-to-LDS load and would wait for all of them before each read.  Their
//     completion is awaited explicitly, tied to the fragment registers.
//   - e2m1 codes are staged packed (two per byte), 16 bytes per column and step,
//     with the column's fp16 group scale (the step's scales are contiguous in
//     the group-major scale array: whole-dword loads), and decoded to fp16
//     (v_cvt_scalef32_pk_f16_fp4 with a unit scale, then a packed fp16 multiply
//     by the group scale) before the MFMAs that take them: per substep with
//     32x32 blocks, and block by block between the MFMAs with 16x16 ones.
//   - MX (fp8 e4m3 A, e2m1 B, one e8m0 scale per 32 k on each): the operands
//     go to the block-scaled MFMA as stored, without decoding.  A step is 128 k:
//     two 64-byte fp8 rows per tile row (k 0-63 and 64-127 of the step, each
//     laid out and swizzled like an int8 A row), 64 bytes of codes per column
//     (laid out like a K-contiguous B), and per operand and group a 256-byte
//     chunk of scales (the scale arrays are group-major, so each chunk is one
//     contiguous load).  The scale register of lane group kg covers k 32kg .. +31
//     of one MFMA.
//   - Accumulators stay in registers for the whole K range.  MFMA blocks
//     (MS): 32x32 (v_mfma_f32_32x32x16_f16/_bf16, v_mfma_i32_32x32x32_i8,
//     v_mfma_scale_f32_32x32x64_f8f6f4; two per 64-byte region) or, on the
//     eight-wave tile, 16x16 (v_mfma_f32_16x16x32_f16/_bf16,
//     v_mfma_i32_16x16x64_i8, v_mfma_scale_f32_16x16x128_f8f6f4; one per
//     region and 16x16 block): the same work per clock, and on random operands
//     the 16x16 ones run at a higher clock under the power limit.
//   - The K schedule is n_main full steps then at most one shorter step of
//     1 .. 2KR-1 substeps for the tail (the pages' variable K step, [generator]
//     DeepGEMM article, kwkr.cn, section 2.2, first layer).
//   - The epilogue (alpha, beta*D, bias, GELU, requantise, conversion) runs once
//     per output element after the K loop, four columns per lane with vector
//     loads and stores (eight, one 16-byte store, for a plain 16-bit C); with a
//     K split the raw fp32 / int32 partials go to the workspace and a reduce
//     kernel applies the epilogue.
// Tiles are visited in a grouped order and every XCD gets a contiguous run of
// them, so tiles that share rows of A or columns of B share an L2.
#pragma once
#include "kcommon.h"
#include "catalogue.h"

namespace dg {

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

// 4 bytes per lane from buffer offset `off` (a multiple of 4), written to LDS at
// lds + 4 * lane.
DG_DEV void buf_ld4_lds(__amdgpu_buffer_rsrc_t r, uint32_t off, void *lds)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (DG_LDS void *)lds, 4, (int)off, 0, 0, 0);
}

// Transposing LDS reads at LDS byte address addr + OFF (see the header).
template <int OFF>
DG_DEV u32x2 lds_tr16(uint32_t addr)
{
    u32x2 v;
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "n"(OFF));
    return v;
}
template <int OFF>
DG_DEV u32x2 lds_tr8(uint32_t addr)
{
    u32x2 v;
    asm volatile("ds_read_b64_tr_b8 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "n"(OFF));
    return v;
}

// s_waitcnt immediate (gfx9 encoding): at most vm vector-memory and lgkm
// LDS/scalar operations outstanding, export counter not waited on.
constexpr int waitcnt_imm(int vm, int lgkm)
{
    return (vm & 0xF) | ((vm >> 4) << 14) | (0x7 << 4) | ((lgkm & 0xF) << 8);
}

// Wait until at most N of this wave's buffer loads are outstanding and all its
// LDS operations are done, then join the workgroup barrier.  The wait is the
// builtin, so the compiler's own wait insertion knows what it covers; the
// barrier is assembly with a memory clobber so that no LDS access moves across
// it (the barrier builtin alone does not order memory, and __syncthreads adds a
// fence that waits for every outstanding load).
template <int N>
DG_DEV void wait_vm_barrier()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(N, 0));
    asm volatile("s_barrier" : : : "memory");
}

// Calls f(integral_constant<int, i>) for i = 0 .. N-1 in order.
template <typename F, int... I>
DG_DEV void static_for_impl(F &&f, std::integer_sequence<int, I...>)
{
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
DG_DEV void static_for(F &&f)
{
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

template <int PATH, int BKMAJ, int BM, int BN, int WM, int WN, int KR, int MS = 32>
__global__ void __launch_bounds__(WM *WN * 64, 1) gemm_tiled_kernel(TiledArgs p)
{
    constexpr int NW = WM * WN;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int FM = WTM / 32, FN = WTN / 32;
    constexpr bool IS_I8 = PATH == P_I8;
    constexpr bool IS_E2M1 = PATH == P_E2M1;
    constexpr bool IS_MX = PATH == P_MX;
    constexpr bool FP4B = IS_E2M1 || IS_MX;            // B holds 4-bit codes, two per byte
    static_assert(!IS_MX || BKMAJ, "MX codes are stored N x K");
    constexpr bool B_TR = !BKMAJ && !FP4B;             // row-major B, transposing reads
    constexpr int BKE = tiled_bk_elems(PATH);          // k elements per K region
    constexpr int KSUB = tiled_ksub(PATH);             // k elements per MFMA
    static_assert(BKE == 2 * KSUB, "two substeps per region");
    static_assert(KR == 1 || PATH == P_F16 || PATH == P_BF16 || PATH == P_I8, "double K steps: 16-bit and int8");
    static_assert(KR == 1 || KR == 2, "one or two K regions per step");
    // MFMA block: 32x32 (two MFMAs of KSUB k per region and block) or 16x16
    // (one MFMA per 64-byte region and 16x16 block: v_mfma_i32_16x16x64_i8,
    // v_mfma_f32_16x16x32_f16/_bf16).  The 16x16 MFMAs do the same work per
    // clock and, on random operands, hold a higher clock under the power limit.
    constexpr bool M16 = MS == 16;
    static_assert(MS == 32 || MS == 16, "MFMA block size");
    static_assert(!M16 || (NW == 8 && KR == 1), "16x16 MFMAs: the eight-wave loop");
    constexpr int BKS = KR * BKE;                      // k elements per K step
    constexpr int NSUB = 2 * KR;                       // MFMA substeps per K step
    constexpr int NBUF = tiled_nbuf(PATH, BM, BN, WM, WN, KR);
    static_assert(NBUF >= 2, "LDS stages");
    constexpr int ESZ = (IS_I8 || IS_MX) ? 1 : 2;      // bytes per element of A and of a 16-bit / int8 B
    static_assert(BKE * ESZ == 64 * (IS_MX ? 2 : 1), "64-byte rows");
    constexpr int A_REG = (IS_MX ? 2 : 1) * KR;         // 64-byte A rows per tile row and step
    constexpr int A_BYTES = BM * 64;                    // one A region
    constexpr int A_ALL = A_REG * A_BYTES;
    constexpr int B_REG = IS_E2M1 ? BN * 16 : BN * 64;  // one B region (e2m1: BKE/2 bytes of codes per column)
    constexpr int B_TILE = KR * B_REG;
    // scales: e2m1 one fp16 per column (whole 256-byte loads); MX, per operand
    // and group of the step, one byte per row of A (column of B) in a 256-byte
    // chunk: [A g0..g3][B g0..g3], the chunks SBS bytes apart.  The 16x16
    // reads take the four groups' chunks at once (one per lane group): 256
    // bytes apart, their bytes of one row share a bank; 272 apart they do not
    // (measured with the LDS conflict counters).
    constexpr int SBS = IS_MX && M16 ? 272 : 256;
    constexpr int S_BYTES = IS_E2M1 ? (BN * 2 + 255) / 256 * 256 : (IS_MX ? 2304 : 0);
    static_assert(!IS_MX || (BM <= 256 && BN <= 256), "MX scale chunks hold 256 rows");
    constexpr int STAGE = A_ALL + B_TILE + S_BYTES;
    constexpr int RB = BN * ESZ;               // bytes per K row of a row-major B tile
    constexpr int CPR = RB / 16;               // 16-byte chunks per such row
    // chunk swizzles (see the header): 64-byte rows of A and of a K-major B,
    // and K rows of a row-major B
    auto rsw = [](int r) { return M16 ? (r >> 1) & 3 : (r >> 2) & 3; };
    auto ksw = [](int k) {
        return IS_I8 ? ((2 * (k & 7)) | (M16 ? (k >> 4) & 1 : 0)) % CPR
                     : ((4 * (k & 3)) | (M16 ? 2 * ((k >> 3) & 1) : 0)) % CPR;
    };
    static_assert(FM >= 1 && FN >= 1 && WTM % 32 == 0 && WTN % 32 == 0, "wave tile");
    constexpr int LDS_BYTES = tiled_lds_bytes(PATH, BM, BN, WM, WN, KR);
    static_assert(STAGE == tiled_stage_bytes(PATH, BM, BN, KR), "stage size");
    static_assert(STAGE % 1024 == 0 || IS_E2M1 || (IS_MX && STAGE % 256 == 0), "stage alignment");
    // direct-to-LDS loads: a 16-byte load fills 1 KB (64 lanes), a dword load 256 B.
    // Load i of an operand is issued by wave i % NW (the scale loads from the
    // last wave down, to even out the per-wave counts).
    constexpr int A_NL = A_ALL / 1024, B_NL = B_TILE / 1024, S_NL = IS_MX ? 8 : S_BYTES / 256;
    static_assert(A_NL * 1024 == A_ALL && B_NL * 1024 == B_TILE &&
                      (IS_MX ? (S_NL - 1) * SBS + 256 <= S_BYTES : S_NL * 256 == S_BYTES),
                  "tile not whole loads");
    constexpr int A_LD = (A_NL + NW - 1) / NW, B_LD = (B_NL + NW - 1) / NW, S_LD = (S_NL + NW - 1) / NW;
    constexpr int LPS = tiled_min_loads_per_wave(A_NL, B_NL, S_NL, NW);   // fewest loads a wave issues per stage
    static_assert(3 * LPS < 64, "vmcnt range");

    // Stage clock (the generator's profile option): s_memtime stamps at kernel
    // entry, loop start, loop end and kernel end, taken by wave 0 when a buffer
    // is given.
    const bool clk_on = p.clk != nullptr;
    unsigned long long ck0 = 0, ck1 = 0, ck2 = 0, rt1 = 0, rt2 = 0;   // rt: s_memrealtime (100 MHz)
    if (clk_on) ck0 = __builtin_amdgcn_s_memtime();

    __shared__ __attribute__((aligned(1024))) char smem[LDS_BYTES];
    const uint32_t lds0 = (uint32_t)(uintptr_t)(DG_LDS char *)smem;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar LDS bases
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
    const int nfull = (kend - kbeg) / BKS;
    const int tail = (kend - kbeg) - nfull * BKS;   // a multiple of KSUB below BKS (K is a multiple of KSUB)
    const int nsteps = nfull + (tail ? 1 : 0);
    const int nsub_last = tail ? tail / KSUB : NSUB;   // substeps the last step runs

    const int M = p.M, N = p.N;
    const uint32_t lda_b = (uint32_t)(p.lda * ESZ);
    const uint32_t ldb_b = (uint32_t)(FP4B ? p.ldb / 2 : p.ldb * ESZ);
    // Operand extents, in bytes from the tile origin to the end of the last
    // valid element (a 16-byte chunk never straddles it: K and the column
    // blocks are 16-byte multiples).  The host checks they fit 32 bits.
    const char *Abase = reinterpret_cast<const char *>(p.A) + (int64_t)m0 * lda_b;
    const uint32_t a_bytes = (uint32_t)((M - m0 - 1) * (int64_t)lda_b + (int64_t)p.K * ESZ);
    const char *Bbase;
    uint32_t b_bytes;
    if constexpr (BKMAJ) {
        const int64_t rowb = FP4B ? p.K / 2 : (int64_t)p.K * ESZ;
        Bbase = reinterpret_cast<const char *>(p.B) + (int64_t)n0 * ldb_b;
        b_bytes = (uint32_t)((N - n0 - 1) * (int64_t)ldb_b + rowb);
    } else {
        const int64_t cpb = 16 / ESZ;                        // columns per 16-byte chunk
        const int64_t nr = ((int64_t)N + cpb - 1) / cpb * cpb;
        Bbase = reinterpret_cast<const char *>(p.B) + (int64_t)n0 * ESZ;
        b_bytes = (uint32_t)((p.K - 1) * (int64_t)ldb_b + (nr - n0) * ESZ);
    }
    // e2m1 scales: group-major, fp16 scale (g, n) at element g * ld_scale + n
    // (ld_scale even, the pointer 4-byte aligned), so a K step's scales for the
    // tile's columns are contiguous and are fetched as whole dwords, two
    // columns each.  The range is the whole array: columns past N read the next
    // group's (discarded) or zeros.
    const char *Sbase = nullptr;
    uint32_t s_bytes = 0;
    if constexpr (IS_E2M1) {
        Sbase = reinterpret_cast<const char *>(p.scale);
        s_bytes = (uint32_t)((int64_t)(p.K / 32) * p.ld_scale * 2);
    }
    // MX scales: e8m0 bytes, group-major: row r of A, group g at scale_a +
    // g * ld_scale_a + r, column n of B, group g at scale + g * ld_scale + n (both
    // pitches multiples of 4, both pointers 4-byte aligned).  A stage fetches,
    // per operand and group, the 256 contiguous bytes from the tile's first row
    // (column): rows past the tile or M read other rows' scales or, past the
    // array, zeros, and are discarded.
    const char *SAbase = nullptr;
    uint32_t sa_bytes = 0;
    if constexpr (IS_MX) {
        SAbase = reinterpret_cast<const char *>(p.scale_a);
        Sbase = reinterpret_cast<const char *>(p.scale);
        sa_bytes = (uint32_t)((int64_t)(p.K / 32) * p.ld_scale_a);
        s_bytes = (uint32_t)((int64_t)(p.K / 32) * p.ld_scale);
    }

    // ---- per-lane source offsets of this wave's direct-to-LDS loads.  Load q of
    // an operand fills LDS bytes [q * 1024, +1024) of its region; lane l writes
    // 16-byte chunk pc = q * 64 + l of it.  Rows past the operand start at or
    // beyond its extent: their loads return zeros.
    // (MX: chunks past the first region fill the second, 64 k further on.)
    uint32_t oa[A_LD];
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
        const int pc0 = (i * NW + wave) * 64 + lane;
        const int reg = pc0 / (BM * 4), pc = pc0 % (BM * 4);
        const int r = pc >> 2, c = (pc & 3) ^ rsw(r);
        oa[i] = reg * 64 + r * lda_b + c * 16;
    }
    uint32_t ob[B_LD];
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
        const int pc = (i * NW + wave) * 64 + lane;
        if constexpr (IS_E2M1) {            // [BN columns][16 B]
            ob[i] = pc * ldb_b;
        } else if constexpr (BKMAJ) {       // as A, rows are columns of B (region reg: k + 64 bytes * reg)
            const int reg = pc / (BN * 4), q = pc % (BN * 4);
            const int r = q >> 2, c = (q & 3) ^ rsw(r);
            ob[i] = reg * 64 + r * ldb_b + c * 16;
        } else {                            // K rows of BN columns
            const int k = pc / CPR, pcol = pc % CPR;
            ob[i] = k * ldb_b + (pcol ^ ksw(k)) * 16;
        }
    }
    const int swave = NW - 1 - wave;        // scale loads go from the last wave down
    uint32_t os[S_LD > 0 ? S_LD : 1];
#pragma unroll
    for (int i = 0; i < S_LD; ++i) {
        const int col = (i * NW + swave) * 64 + lane;   // byte of scale (n0 + col, 0) from Sbase
        if constexpr (IS_MX) {   // load L = i NW + swave: operand L >> 2 (A, B), group L & 3
            const int L = i * NW + swave;
            os[i] = (uint32_t)(L & 3) * (uint32_t)((L >> 2) ? p.ld_scale : p.ld_scale_a) +
                    (uint32_t)((L >> 2) ? n0 : m0) + 4 * (uint32_t)lane;
        } else   // e2m1: dword `col` of the stage holds columns 2 col and 2 col + 1
            os[i] = 2 * (uint32_t)(n0 + 2 * col);
    }

    // Issue the loads of step j (k0 = kbeg + j * BKE) into LDS stage j % NBUF.
    // Steps past the last one issue the same loads over empty ranges: they only
    // write zeros into a stage nobody reads again, and keep every wave's count
    // of outstanding loads the same at each barrier.
    // Load i of step j: the A loads first, then B, then the e2m1 scales.
    auto load_one = [&](int j, int i) {
        const bool real = j < nsteps;
        const int k0 = real ? kbeg + j * BKS : 0;
        char *sb = smem + (j % NBUF) * STAGE;
        if (i < A_LD) {
            if (A_NL % NW == 0 || i * NW + wave < A_NL) {   // wave-uniform
                const __amdgpu_buffer_rsrc_t rA =
                    make_rsrc(Abase + (int64_t)k0 * ESZ, real ? a_bytes - (uint32_t)(k0 * ESZ) : 0u);
                buf_ld16_lds(rA, oa[i], sb + (i * NW + wave) * 1024);   // (both MX regions)
            }
        } else if (i < A_LD + B_LD) {
            const int q = i - A_LD;
            if (B_NL % NW == 0 || q * NW + wave < B_NL) {   // wave-uniform
                uint32_t kb;
                if constexpr (FP4B) kb = (uint32_t)(k0 >> 1);
                else if constexpr (BKMAJ) kb = (uint32_t)(k0 * ESZ);
                else kb = (uint32_t)k0 * ldb_b;
                const __amdgpu_buffer_rsrc_t rB = make_rsrc(Bbase + kb, real ? b_bytes - kb : 0u);
                buf_ld16_lds(rB, ob[q], sb + A_ALL + (q * NW + wave) * 1024);
            }
        } else if constexpr (IS_MX) {
            const int q = i - A_LD - B_LD;
            if (S_NL % NW == 0 || q * NW + swave < S_NL) {   // wave-uniform
                const bool rows = q * NW + swave < 4;   // wave-uniform: A's or B's scales
                const __amdgpu_buffer_rsrc_t rS =
                    make_rsrc(rows ? SAbase : Sbase, real ? (rows ? sa_bytes : s_bytes) : 0u);
                buf_ld4_lds(rS, os[q] + (uint32_t)(k0 >> 5) * (uint32_t)(rows ? p.ld_scale_a : p.ld_scale),
                            sb + A_ALL + B_TILE + (q * NW + swave) * SBS);
            }
        } else if constexpr (IS_E2M1) {
            const int q = i - A_LD - B_LD;
            if (S_NL % NW == 0 || q * NW + swave < S_NL) {   // wave-uniform
                const __amdgpu_buffer_rsrc_t rS = make_rsrc(Sbase, real ? s_bytes : 0u);
                buf_ld4_lds(rS, os[q] + 2 * (uint32_t)(k0 >> 5) * (uint32_t)p.ld_scale,
                            sb + A_BYTES + B_TILE + (q * NW + swave) * 256);
            }
        }
    };
    // All loads of step j (part 0: only A; part 1: only B and the scales).
    auto load_stage = [&](int j, int part = -1) {
#pragma unroll
        for (int i = 0; i < A_LD + B_LD + S_LD; ++i)
            if (part < 0 || (part == 0) == (i < A_LD)) load_one(j, i);
    };

    // Accumulators: per 32x32 block of the wave tile one 16-register tile, or
    // (16x16 MFMAs) four 4-register tiles, q = 2 * (row half) + (column half).
    using Acc32 = typename std::conditional<IS_I8, intx16, floatx16>::type;
    using Acc16 = typename std::conditional<IS_I8, intx4, floatx4>::type;
    using AccT = typename std::conditional<M16, Acc16, Acc32>::type;
    constexpr int NQ = M16 ? 4 : 1, NV = M16 ? 4 : 16;
    AccT acc[FM][FN][NQ];
#pragma unroll
    for (int mi = 0; mi < FM; ++mi)
#pragma unroll
        for (int ni = 0; ni < FN; ++ni)
#pragma unroll
            for (int q = 0; q < NQ; ++q)
#pragma unroll
                for (int v = 0; v < NV; ++v) acc[mi][ni][q][v] = 0;

    // fragments of one k-substep: FM A blocks and FN B blocks (16 bytes per lane
    // each; MX: 32 bytes of fp8 A per lane, and the lane's scale bytes of its A
    // row and B column in the low byte of sa / sb)
    using AFrag = typename std::conditional<IS_MX, u32x8, u32x4>::type;
    struct Frag {
        AFrag a[FM];
        u32x4 b[FN];
        unsigned sa[IS_MX ? FM : 1], sb[IS_MX ? FN : 1];
    };
    Frag f0, f1;
    // e2m1: substep 1's code word and the step's scale, taken by substep 0's read
    unsigned e2_next[IS_E2M1 ? FN : 1], e2_sh[IS_E2M1 ? FN : 1];
    // Per-lane LDS byte offsets (within a stage) of the fragment reads.
    //   A / K-major B: row `row`, logical chunk 2s + kg.
    //   row-major B (transposing reads): lane L of 16-lane group g supplies K row
    //   (b16) kb + (L >> 2) at column 16*(g&1) + 4*(L&3), or (b8) kb + (L >> 1) at
    //   column 16*(g&1) + 8*(L&1); kb = KSUB*s + 8*(g>>1) (b16) or 16*(g>>1) (b8).
    //   The two reads of a block cover K rows kb.. and kb+4.. (b16) / kb+8.. (b8);
    //   row k and k + 4 (k + 8) share their swizzle, as do substeps 0 and 1, so
    //   those reads differ by immediate offsets.
    //   16x16 MFMAs: A / K-major B row `row` (16 rows per block half), chunk
    //   lane >> 4 (the MFMA takes a whole 64-byte region); row-major B: lane L of
    //   group g supplies K row 8g + (L >> 2) at column 16 sn + 4 (L & 3) (b16), or
    //   16g + (L >> 1) at column 16 sn + 8 (L & 1) (b8), sn the column half.
    const int grp16 = lane >> 4, L16 = lane & 15;
    uint32_t boff[FN * (M16 ? 2 : 1)];
#pragma unroll
    for (int ni = 0; ni < FN; ++ni) {
#pragma unroll
        for (int sn = 0; sn < (M16 ? 2 : 1); ++sn) {
            const int col0 = wn * WTN + ni * 32 + 16 * sn;
            uint32_t o = 0;
            if constexpr (B_TR) {
                if constexpr (!IS_I8) {
                    const int col = col0 + (M16 ? 0 : 16 * (grp16 & 1)) + 4 * (L16 & 3);
                    const int k = (M16 ? 8 * grp16 : 8 * (grp16 >> 1)) + (L16 >> 2);
                    o = A_ALL + k * RB + (((col >> 3) ^ ksw(k)) << 4) + (col & 7) * 2;
                } else {
                    const int col = col0 + (M16 ? 0 : 16 * (grp16 & 1)) + 8 * (L16 & 1);
                    const int k = (M16 ? 16 * grp16 : 16 * (grp16 >> 1)) + (L16 >> 1);
                    o = A_ALL + k * RB + (((col >> 4) ^ ksw(k)) << 4) + (col & 15);
                }
            }
            boff[ni * (M16 ? 2 : 1) + sn] = o;
        }
    }

    // One fragment read: A block mi, or B block ni, of substep s of stage buf.
    // Substep s reads K region s / 2 (16-bit and int8 operands; MX and e2m1
    // steps are one region), chunk pair s % 2 of its 64-byte rows.
    auto read_a = [&](int buf, auto s_tag, int mi, Frag &f) {
        constexpr int s = decltype(s_tag)::value;
        const char *sA = smem + buf * STAGE;
        const int c = 2 * (s & 1) + kg;
        const int row = wm * WTM + mi * 32 + lr;
        if constexpr (IS_MX) {
            // Region s.  The 8-bit operand of the 32x32x64 block-scaled MFMA is
            // not 32 consecutive k per lane: lane group kg holds k 16kg .. +15 in
            // its first four registers and k 32 + 16kg .. +15 in its last four
            // (the 4-bit operand holds k 32kg .. +31), and the scale of lane
            // group kg applies to k 32kg .. +31 of both operands (probed on the
            // GPU with one-hot operands).  So the lane reads chunks kg and kg+2.
            // The lane's scale is byte `row` of the chunk of group 2s + kg.
            const char *rA = sA + s * A_BYTES + row * 64;
            const int sw = rsw(row);
            const u32x4 lo = *reinterpret_cast<const u32x4 *>(rA + ((kg ^ sw) << 4));
            const u32x4 hi = *reinterpret_cast<const u32x4 *>(rA + (((kg + 2) ^ sw) << 4));
            f.a[mi] = AFrag{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
            f.sa[mi] = *reinterpret_cast<const unsigned char *>(sA + A_ALL + B_TILE + (2 * s + kg) * SBS + row);
        } else {
            f.a[mi] = *reinterpret_cast<const u32x4 *>(sA + (s >> 1) * A_BYTES + row * 64 +
                                                        ((c ^ rsw(row)) << 4));
        }
    };
    auto read_b = [&](int buf, auto s_tag, int ni, Frag &f, int g) {
        constexpr int s = decltype(s_tag)::value;
        const char *sB = smem + buf * STAGE + A_ALL;
        const int c = IS_MX ? 2 * s + kg : 2 * (s & 1) + kg;
        const int col0 = wn * WTN + ni * 32;
        if constexpr (IS_E2M1) {
            // raw: the code word and the scale's bits; decode_b turns them into
            // the fp16 operand (in the MFMA phase, off the LDS-bound one).  Substep
            // 0 reads the column's whole 16-byte chunk (dword 2s + kg is substep
            // s's word for lane group kg): the 16 lanes of a read phase then cover
            // 256 contiguous bytes, where single-dword reads of 16-byte slots put
            // columns r and r + 16 in one bank.  Substep 1 takes its word and the
            // step's scale (one group per step) from that read; it always follows
            // substep 0 of the same stage.
            const int row = col0 + lr;
            if constexpr (s == 0) {
                const u32x4 raw = *reinterpret_cast<const u32x4 *>(sB + row * 16);
                const unsigned sh = *reinterpret_cast<const unsigned short *>(sB + B_TILE + row * 2);
                f.b[ni] = u32x4{kg ? raw.y : raw.x, sh, 0u, 0u};
                e2_next[ni] = kg ? raw.w : raw.z;
                e2_sh[ni] = sh;
            } else {
                f.b[ni] = u32x4{e2_next[ni], e2_sh[ni], 0u, 0u};
            }
        } else if constexpr (BKMAJ) {
            // (MX: chunk 2s + kg holds the 32 codes of k 64s + 32kg .. +31)
            const int row = col0 + lr;
            f.b[ni] = *reinterpret_cast<const u32x4 *>(sB + (IS_MX ? 0 : (s >> 1) * B_REG) + row * 64 +
                                                        ((c ^ rsw(row)) << 4));
            if constexpr (IS_MX)
                f.sb[ni] = *reinterpret_cast<const unsigned char *>(sB + B_TILE + 4 * SBS + (2 * s + kg) * SBS + row);
        } else {
            const uint32_t a = lds0 + (uint32_t)buf * STAGE + boff[M16 ? 2 * ni : ni];
            u32x2 lo, hi;
            if constexpr (!IS_I8) {
                lo = lds_tr16<KSUB * s * RB>(a);
                hi = lds_tr16<KSUB * s * RB + 4 * RB>(a);
            } else {
                lo = lds_tr8<KSUB * s * RB>(a);
                hi = lds_tr8<KSUB * s * RB + 8 * RB>(a);
            }
            f.b[ni] = u32x4{lo.x, lo.y, hi.x, hi.y};
        }
    };
    auto read_frag = [&](int buf, auto s_tag, Frag &f, int g) {
#pragma unroll
        for (int mi = 0; mi < FM; ++mi) read_a(buf, s_tag, mi, f);
#pragma unroll
        for (int ni = 0; ni < FN; ++ni) read_b(buf, s_tag, ni, f, g);
    };
    // The transposing reads are invisible to the compiler's wait insertion:
    // wait for all LDS reads, then tie the B registers to that point so the
    // MFMAs that use them cannot move above it.  The memory clobber keeps the
    // next reads below it.  Call it before issuing the reads of the next
    // fragments, or it would wait for those as well.
    auto settle = [&](Frag &f) {
        if constexpr (B_TR) {
            __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
#pragma unroll
            for (int ni = 0; ni < FN; ++ni) asm volatile("" : "+v"(f.b[ni]) : : "memory");
        }
    };
    // e2m1: decode the raw B fragments read by read_b (nothing to do otherwise)
    auto decode_b = [&](Frag &f) {
        if constexpr (IS_E2M1) {
#pragma unroll
            for (int ni = 0; ni < FN; ++ni) {
                const unsigned codes = f.b[ni].x;
                const unsigned short sh = (unsigned short)f.b[ni].y;
                f.b[ni] = __builtin_bit_cast(u32x4, decode_e2m1x8(codes, __builtin_bit_cast(_Float16, sh)));
            }
        }
    };
    // The B fragment goes in as the MFMA's first operand and the A fragment as
    // its second (each lane holds 8 consecutive k of one column of B, or of one
    // row of A, which is what either operand slot takes), so a block accumulates
    // the transposed product: lane l holds row lr of the block and, in registers
    // 4j .. 4j+3, its columns 8j + 4kg .. 8j + 4kg + 3.
    auto mfma1 = [&](const Frag &f, int mi, int ni) {
        if constexpr (M16)
            return;   // (16x16 tiles go through mfmas16)
        else if constexpr (PATH == P_F16 || PATH == P_E2M1)
            acc[mi][ni][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                __builtin_bit_cast(half8, f.b[ni]), __builtin_bit_cast(half8, f.a[mi]), acc[mi][ni][0], 0, 0, 0);
        else if constexpr (PATH == P_BF16)
            acc[mi][ni][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8, f.b[ni]), __builtin_bit_cast(bf16x8, f.a[mi]), acc[mi][ni][0], 0, 0, 0);
        else if constexpr (IS_MX)
            // first operand e2m1 (format 4, four registers used), second fp8 e4m3
            // (format 0); each scale is the low byte of its register
            acc[mi][ni][0] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                __builtin_bit_cast(intx8, u32x8{f.b[ni].x, f.b[ni].y, f.b[ni].z, f.b[ni].w, 0u, 0u, 0u, 0u}),
                __builtin_bit_cast(intx8, f.a[mi]), acc[mi][ni][0], 4, 0, 0, (int)f.sb[ni], 0, (int)f.sa[mi]);
        else
            acc[mi][ni][0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(
                __builtin_bit_cast(intx4, f.b[ni]), __builtin_bit_cast(intx4, f.a[mi]), acc[mi][ni][0], 0, 0, 0);
    };
    auto mfmas = [&](const Frag &f) {
#pragma unroll
        for (int mi = 0; mi < FM; ++mi)
#pragma unroll
            for (int ni = 0; ni < FN; ++ni) mfma1(f, mi, ni);
    };
    // ---- 16x16 MFMAs: the fragments of one K region are both row halves of
    // every 32-row A block and both column halves of every 32-column B block
    // (16 rows / columns each).  A lane reads chunk lane >> 4 of row (column)
    // lane & 15 of its half: the MFMA takes the whole 64-byte region.
    struct Frag16 {
        AFrag a[2][FM];
        u32x4 b[2][FN];
        unsigned sa[2][IS_MX ? FM : 1], sb[2][IS_MX ? FN : 1];
    };
    auto read_a16 = [&](int buf, int h, int mi, Frag16 &f) {
        const char *sA = smem + buf * STAGE;
        const int r16 = wm * WTM + mi * 32 + 16 * h + L16;
        const int sw = rsw(r16);
        if constexpr (IS_MX) {
            // 16x16x128 block-scaled MFMA: the 8-bit operand of lane group g
            // holds k 16g .. +15 in its first four registers and k 64 + 16g ..
            // +15 in its last four (probed on the GPU with one-hot operands), so
            // the lane reads chunk g of both 64-byte regions of its row; the
            // scale of lane group g applies to k 32g .. +31: byte `r16` of the
            // chunk of group g.
            const u32x4 lo = *reinterpret_cast<const u32x4 *>(sA + r16 * 64 + ((grp16 ^ sw) << 4));
            const u32x4 hi = *reinterpret_cast<const u32x4 *>(sA + A_BYTES + r16 * 64 + ((grp16 ^ sw) << 4));
            f.a[h][mi] = AFrag{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
            f.sa[h][mi] = *reinterpret_cast<const unsigned char *>(sA + A_ALL + B_TILE + grp16 * SBS + r16);
        } else {
            f.a[h][mi] = *reinterpret_cast<const u32x4 *>(sA + r16 * 64 + ((grp16 ^ sw) << 4));
        }
    };
    auto read_b16 = [&](int buf, int h, int ni, Frag16 &f) {
        const char *sB = smem + buf * STAGE + A_ALL;
        const int row = wn * WTN + ni * 32 + 16 * h + L16;   // column of the tile
        if constexpr (IS_E2M1) {
            // code dword g (k 8g .. +7) of the column and its scale; the 64
            // lanes of a read hit 64 distinct banks
            const unsigned codes = *reinterpret_cast<const unsigned *>(sB + row * 16 + 4 * grp16);
            const unsigned sh = *reinterpret_cast<const unsigned short *>(sB + B_TILE + row * 2);
            f.b[h][ni] = u32x4{codes, sh, 0u, 0u};
        } else if constexpr (IS_MX) {
            // the 4-bit operand of lane group g holds k 32g .. +31 of the step:
            // chunk g of the column's 64 bytes, and the column's scale of group g
            f.b[h][ni] = *reinterpret_cast<const u32x4 *>(sB + row * 64 + ((grp16 ^ rsw(row)) << 4));
            f.sb[h][ni] = *reinterpret_cast<const unsigned char *>(sB + B_TILE + 4 * SBS + grp16 * SBS + row);
        } else if constexpr (BKMAJ) {
            f.b[h][ni] = *reinterpret_cast<const u32x4 *>(sB + row * 64 + ((grp16 ^ rsw(row)) << 4));
        } else {
            // transposing reads, this half's own lane offsets; K rows from 0
            const uint32_t a = lds0 + (uint32_t)buf * STAGE + boff[2 * ni + h];
            u32x2 lo, hi;
            if constexpr (!IS_I8) {
                lo = lds_tr16<0>(a);
                hi = lds_tr16<4 * RB>(a);
            } else {
                lo = lds_tr8<0>(a);
                hi = lds_tr8<8 * RB>(a);
            }
            f.b[h][ni] = u32x4{lo.x, lo.y, hi.x, hi.y};
        }
    };
    // (as settle / tie for the 32x32 fragments)
    auto tie16 = [&](Frag16 &f) {
        if constexpr (B_TR) {
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int ni = 0; ni < FN; ++ni) asm volatile("" : "+v"(f.b[h][ni]) : : "memory");
        }
    };
    auto settle16 = [&](Frag16 &f) {
        if constexpr (B_TR) {
            __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
            tie16(f);
        }
    };
    // A final half step (keep false): the lanes holding k past its first half
    // (lane groups 2 and 3; for MX the upper halves of the 8-bit operands and
    // the 4-bit operands of lane groups 2 and 3, whose scales become 127, a
    // factor of one, since a scale byte past K may be the NaN code) contribute
    // 0 x 0.  Branch-free.
    auto keep16 = [&](Frag16 &f, bool keep) {
        const unsigned mb = (keep || grp16 < 2) ? ~0u : 0u;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int mi = 0; mi < FM; ++mi) {
                if constexpr (IS_MX) {
                    const unsigned mu = keep ? ~0u : 0u;
#pragma unroll
                    for (int e = 4; e < 8; ++e) f.a[h][mi][e] &= mu;
                    f.sa[h][mi] = (f.sa[h][mi] & mb) | (~mb & 127u);
                } else {
                    f.a[h][mi] &= mb;
                }
            }
#pragma unroll
            for (int ni = 0; ni < FN; ++ni) {
                f.b[h][ni] &= mb;
                if constexpr (IS_MX) f.sb[h][ni] = (f.sb[h][ni] & mb) | (~mb & 127u);
            }
        }
    };
    // MFMA q of a region, q = ((mi * 2 + sm) * FN + ni) * 2 + sn; B goes in
    // first as above, so lane l of a 16x16 tile holds row l & 15 and columns
    // 4 (l >> 4) .. +3.
    auto mfma16 = [&](const Frag16 &f, int q) {
        if constexpr (M16) {
            const int sn = q & 1, ni = (q >> 1) % FN, sm = (q / (2 * FN)) & 1, mi = q / (4 * FN);
            const AFrag a = f.a[sm][mi];
            const u32x4 b = f.b[sn][ni];
            AccT &c = acc[mi][ni][2 * sm + sn];
            if constexpr (IS_MX)
                // first operand e2m1 (format 4, four registers), second fp8 e4m3
                c = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    __builtin_bit_cast(intx8, u32x8{b.x, b.y, b.z, b.w, 0u, 0u, 0u, 0u}),
                    __builtin_bit_cast(intx8, a), c, 4, 0, 0, (int)f.sb[sn][ni], 0, (int)f.sa[sm][mi]);
            else if constexpr (PATH == P_F16 || PATH == P_E2M1)
                c = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, b), __builtin_bit_cast(half8, a),
                                                           c, 0, 0, 0);
            else if constexpr (PATH == P_BF16)
                c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, b),
                                                            __builtin_bit_cast(bf16x8, a), c, 0, 0, 0);
            else
                c = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(intx4, b), __builtin_bit_cast(intx4, a),
                                                          c, 0, 0, 0);
        }
    };
    // (A rows of half 0 first, in their read order)
    auto mfmas16 = [&](const Frag16 &f) {
#pragma unroll
        for (int sm = 0; sm < 2; ++sm)
#pragma unroll
            for (int mi = 0; mi < FM; ++mi)
#pragma unroll
                for (int b = 0; b < 2 * FN; ++b) mfma16(f, ((mi * 2 + sm) * FN + (b >> 1)) * 2 + (b & 1));
    };
    // e2m1: the compute phase decodes the B blocks one at a time, in four
    // pieces of two instructions (two conversions, or two fp16 products with
    // the scale: the arithmetic of decode_e2m1x8), each piece of block b+1
    // after one of block b's MFMAs.  Only block 0's decode precedes the first
    // MFMA; written as one run of decodes, all of them did.
    auto mfmas16_e2m1 = [&](Frag16 &f) {
        constexpr int NB = 2 * FN, NA = 2 * FM;
        half2v hv[4];
        half2v s2;
        auto piece = [&](auto b_tag, auto k_tag) {
            constexpr int b = decltype(b_tag)::value, k = decltype(k_tag)::value;
            constexpr int sn = b & 1, ni = b >> 1;
            const unsigned codes = f.b[sn][ni].x;
            if constexpr (k == 0) {
                const _Float16 sc = __builtin_bit_cast(_Float16, (unsigned short)f.b[sn][ni].y);
                s2 = half2v{sc, sc};
                hv[0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 0);
                hv[1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 1);
            } else if constexpr (k == 1) {
                hv[2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 2);
                hv[3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 3);
            } else if constexpr (k == 2) {
                hv[0] = hv[0] * s2;
                hv[1] = hv[1] * s2;
            } else {
                hv[2] = hv[2] * s2;
                hv[3] = hv[3] * s2;
                f.b[sn][ni] = u32x4{__builtin_bit_cast(unsigned, hv[0]), __builtin_bit_cast(unsigned, hv[1]),
                                    __builtin_bit_cast(unsigned, hv[2]), __builtin_bit_cast(unsigned, hv[3])};
            }
        };
        static_for<4>([&](auto k_tag) { piece(std::integral_constant<int, 0>{}, k_tag); });
        static_for<NB>([&](auto b_tag) {
            constexpr int b = decltype(b_tag)::value;
            static_for<NA>([&](auto a_tag) {
                constexpr int a = decltype(a_tag)::value;
                constexpr int sm = a / FM, mi = a % FM, sn = b & 1, ni = b >> 1;   // A rows of half 0 first
                __builtin_amdgcn_sched_barrier(0);
                mfma16(f, ((mi * 2 + sm) * FN + ni) * 2 + sn);
                if constexpr (b + 1 < NB && a < 4) {
                    __builtin_amdgcn_sched_barrier(0);
                    piece(std::integral_constant<int, b + 1>{}, a_tag);
                }
            });
        });
        __builtin_amdgcn_sched_barrier(0);
    };
    // A final half step runs its second substep on zeroed fragments (0 x 0 adds
    // nothing): the fragments are ANDed with a uniform mask, so the loop body has
    // no branch at all - a branch near the MFMAs makes the compiler copy every
    // accumulator on each step.
    // (MX: the scales become 127, a factor of one: a scale byte past K may be the
    // NaN code, and NaN times zero is not zero.)
    auto keep_if = [&](Frag &f, bool keep) {
        const unsigned m = keep ? ~0u : 0u;
#pragma unroll
        for (int mi = 0; mi < FM; ++mi) f.a[mi] &= m;
#pragma unroll
        for (int ni = 0; ni < FN; ++ni) f.b[ni] &= m;
        if constexpr (IS_MX) {
#pragma unroll
            for (int mi = 0; mi < FM; ++mi) f.sa[mi] = (f.sa[mi] & m) | (~m & 127u);
#pragma unroll
            for (int ni = 0; ni < FN; ++ni) f.sb[ni] = (f.sb[ni] & m) | (~m & 127u);
        }
    };
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    const int g0 = kbeg >> 5;   // e2m1 scale group of step 0

    // ---- main loop (four waves).  One step: [substep 0 of stage st, reads of
    // substep 1 in its shadow] barrier [loads of stage st+4, reads of substep 0
    // of stage st+1, substep 1 of stage st].  The barrier guarantees that stage st+1 has landed
    // for every wave (the loads of stages st+2 and st+3 may still be in flight)
    // and that no wave still reads stage st, whose buffer takes stage st+4.  The
    // body is branch-free.
    if constexpr (NW == 8) {
        static_assert(KR == 1, "the eight-wave loop takes one K region per step");
        // Eight waves: two groups of four (waves 0-3 and 4-7, one of each per
        // SIMD) alternate a memory phase (read both fragments of stage st, wait
        // for this wave's loads of stage st+1) and a compute phase (the MFMAs of
        // stage st), with a barrier after each phase.  The second group runs one
        // barrier behind, so on every SIMD one wave computes while the other does
        // its memory phase.  Stage st is read by the first group between barriers
        // 2st+1 and 2st+2 and by the second between 2st+2 and 2st+3, so its buffer
        // may be refilled by any phase that starts at or after barrier 2st+3.
        // The memory phase of step st issues the loads of stage st+NBUF-1, into
        // the buffer of stage st-1, and its wait leaves the NBUF-2 stages after
        // stage st+1 in flight.  With 16x16 MFMAs that wait is for the direct
        // loads only: the phase's fragment reads (B, then the A rows of each
        // half) are waited for in the compute phase, each before the first
        // MFMA that takes it.
        const bool lag = wave >= 4;
        auto bar = [] {
            __builtin_amdgcn_sched_barrier(0);
            asm volatile("s_barrier" : : : "memory");
            __builtin_amdgcn_sched_barrier(0);
        };
        auto tie = [&](Frag &f) {
            if constexpr (B_TR) {
#pragma unroll
                for (int ni = 0; ni < FN; ++ni) asm volatile("" : "+v"(f.b[ni]) : : "memory");
            }
        };
        constexpr int AHEAD = NBUF - 1;   // stages issued before the loop
#pragma unroll
        for (int j = 0; j < AHEAD; ++j) load_stage(j);
        __builtin_amdgcn_s_waitcnt(waitcnt_imm((AHEAD - 1) * LPS, 15));
        bar();
        if (lag) bar();
        // One step; the last one (LAST) issues no loads and masks its second
        // substep when it is a half step.
        Frag16 fr;   // (16x16 MFMAs)
        auto step = [&](int st, auto last_tag) {
            constexpr bool LAST = decltype(last_tag)::value;
            const int buf = st % NBUF;
            // memory phase: the fragment reads of stage st, with the loads of
            // stage st+NBUF-1 issued between them (LDS reads and buffer loads go
            // to different units)
            if constexpr (M16) {
                // the B reads first (e2m1: code words and scales, which block
                // 0's decode needs; row-major B: the transposing reads, which one
                // wait then covers), then the A rows of half 0 and of half 1, in
                // the order of the MFMAs that take them
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int ni = 0; ni < FN; ++ni) read_b16(buf, h, ni, fr);
#pragma unroll
                for (int mi = 0; mi < FM; ++mi) read_a16(buf, 0, mi, fr);
                if constexpr (!LAST) load_stage(st + AHEAD, 0);
#pragma unroll
                for (int mi = 0; mi < FM; ++mi) read_a16(buf, 1, mi, fr);
                if constexpr (!LAST) load_stage(st + AHEAD, 1);
                // only the direct loads are waited for before the barrier: the
                // fragment reads land while the other group's last MFMAs run,
                // and are waited for in the compute phase (stage st's buffer is
                // refilled only after the next barrier)
                __builtin_amdgcn_s_waitcnt(waitcnt_imm((AHEAD - 1) * LPS, 15));
            } else {
                read_frag(buf, S0{}, f0, g0 + st);
                if constexpr (!LAST) load_stage(st + AHEAD, 0);
                read_frag(buf, S1{}, f1, g0 + st);
                if constexpr (!LAST) load_stage(st + AHEAD, 1);
                __builtin_amdgcn_s_waitcnt(waitcnt_imm((AHEAD - 1) * LPS, 0));
                tie(f0);
                tie(f1);
                if constexpr (LAST) keep_if(f1, nfull == nsteps);   // a final half step adds 0 x 0
            }
            bar();
            // compute phase, at raised wave priority so that the SIMD's other
            // wave (in its memory phase) does not delay the MFMA issue
            __builtin_amdgcn_s_setprio(1);
            if constexpr (M16) {
                // (reads the compiler cannot see, the transposing ones, issued
                // before the 2 FM A reads, are waited for here; it waits for its
                // own ones where they are used)
                if constexpr (B_TR) __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 2 * FM));
                tie16(fr);
                if constexpr (LAST) keep16(fr, nfull == nsteps);
            }
            if constexpr (M16 && IS_E2M1) {
                mfmas16_e2m1(fr);
            } else if constexpr (M16) {
                mfmas16(fr);
            } else {
                decode_b(f0);
                mfmas(f0);
                decode_b(f1);
                mfmas(f1);
            }
            __builtin_amdgcn_s_setprio(0);
            bar();
        };
        if (clk_on) {
            ck1 = __builtin_amdgcn_s_memtime();
            rt1 = __builtin_amdgcn_s_memrealtime();
        }
        // no scalar memory result pending at the first step: such results return
        // out of order, and one in flight would make every wait for a fragment
        // read in the step a wait for all of them
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
        for (int st = 0; st < nsteps - 1; ++st) step(st, std::false_type{});
        // (with an empty K slice, stage 0 holds the zeros of out-of-range loads)
        step(nsteps > 0 ? nsteps - 1 : 0, std::true_type{});
        // (every fragment read in this loop is consumed in its own step; settling
        // here keeps the rule that no transposing read is left in flight)
        settle(f0);
        settle(f1);
        settle16(fr);
        if (!lag) bar();
    } else {
        // Four waves, one per SIMD: each wave hides its own LDS reads and buffer
        // loads behind its MFMAs, so the instruction order is fixed by hand
        // (sched_barrier after every MFMA).  A step runs NSUB substeps; the
        // fragment reads of substep s+1 go between the first two thirds of
        // substep s's MFMAs, so the last third covers their latency.  Every read
        // of stage st is issued by the end of substep NSUB-2, so the one barrier
        // of the step comes before the last substep: it finds those reads done,
        // stage st+1 landed, and frees stage st's buffer, into which the last
        // substep issues the loads of stage st+NBUF (between its last third of
        // MFMAs) while it reads substep 0 of stage st+1.
        constexpr int NM = FM * FN, NRD = FM + FN, NLD = A_LD + B_LD + S_LD;
        constexpr int QR = NM >= 3 ? 2 * NM / 3 : NM;
        auto read_slot = [](int r) { return r * QR / NRD; };
        auto load_slot = [](int i) {
            const int q = QR + i * (NM - QR) / NLD;
            return q < NM ? q : NM - 1;
        };
        auto read_item = [&](int buf, auto s_tag, int r, Frag &f, int g) {
            if (r < FM) read_a(buf, s_tag, r, f);
            else read_b(buf, s_tag, r - FM, f, g);
        };
        // One step; the last one (LAST) issues no loads and no reads ahead, needs
        // no barrier, and masks the substeps past the K tail.
        auto step = [&](int st, auto last_tag) {
            constexpr bool LAST = decltype(last_tag)::value;
            const int buf = st % NBUF;
            const int nxt = (st + 1) % NBUF;
            static_for<NSUB>([&](auto s_tag) {
                constexpr int s = decltype(s_tag)::value;
                Frag &F = (s & 1) ? f1 : f0;   // this substep's fragments
                Frag &G = (s & 1) ? f0 : f1;   // the next substep's
                if constexpr (!LAST && s == NSUB - 1) wait_vm_barrier<(NBUF - 2) * LPS>();
                settle(F);
                if constexpr (LAST && s > 0) keep_if(F, s < nsub_last);   // past the tail: 0 x 0
                decode_b(F);
#pragma unroll
                for (int q = 0; q < NM; ++q) {
                    mfma1(F, q / FN, q % FN);
                    if constexpr (s < NSUB - 1) {
#pragma unroll
                        for (int r = 0; r < NRD; ++r)
                            if (read_slot(r) == q)
                                read_item(buf, std::integral_constant<int, s + 1>{}, r, G, g0 + st);
                    } else if constexpr (!LAST) {
#pragma unroll
                        for (int r = 0; r < NRD; ++r)
                            if (read_slot(r) == q) read_item(nxt, S0{}, r, G, g0 + st + 1);
#pragma unroll
                        for (int i = 0; i < NLD; ++i)
                            if (load_slot(i) == q) load_one(st + NBUF, i);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            });
        };
#pragma unroll
        for (int j = 0; j < NBUF; ++j) load_stage(j);
        wait_vm_barrier<(NBUF - 1) * LPS>();
        read_frag(0, S0{}, f0, g0);
        if (clk_on) {
            ck1 = __builtin_amdgcn_s_memtime();
            rt1 = __builtin_amdgcn_s_memrealtime();
        }
        for (int st = 0; st < nsteps - 1; ++st) step(st, std::false_type{});
        // (with an empty K slice, stage 0 holds the zeros of out-of-range loads)
        step(nsteps > 0 ? nsteps - 1 : 0, std::true_type{});
        // (the last substep reads nothing ahead, and settling it waited for its
        // reads: no transposing read is in flight when the epilogue reuses
        // registers)
    }

    if (clk_on) {
        ck2 = __builtin_amdgcn_s_memtime();
        rt2 = __builtin_amdgcn_s_memrealtime();
    }

    // ---- epilogue: each wave stages 32 rows of its accumulators in LDS at a time
    // (a 16-byte write per four columns of a row: the blocks are transposed) and
    // stores them four columns per lane, row-contiguously.  Storing the
    // transposed blocks straight from registers instead (32 rows of 32 bytes per
    // store) took 2-4x longer.
    constexpr int RP = WTN + 4;   // padded row pitch (elements) of the staging area
    static_assert(NW * 32 * RP * 4 <= LDS_BYTES, "epilogue staging");
    __syncthreads();   // every wave is done with the last K stage
    using ScalarT = typename std::conditional<IS_I8, int32_t, float>::type;
    using Vec4 = typename std::conditional<IS_I8, intx4, floatx4>::type;
    ScalarT *sE = reinterpret_cast<ScalarT *>(smem) + wave * 32 * RP;
    constexpr int LPR = WTN / 4;    // lanes per row (4 columns each)
    constexpr int RPI = 64 / LPR;   // rows per read
    constexpr int NIT = 32 / RPI;   // reads per 32 rows
    const int er = lane / LPR, ec = (lane % LPR) * 4;
    const bool vec_ok = epi_vec_ok(p.epi, p.split_k > 1, p.ws, N);
    constexpr int EB = NIT < 4 ? NIT : 4;   // rows per batch (a larger batch makes the float epilogues spill)
    using DVec4 = typename std::conditional<IS_I8, intx4, floatx4>::type;
    // This lane's four columns are the same in every row: the bias is loaded once.
    const int col = n0 + wn * WTN + ec;
    const bool vec_col = vec_ok && col + 3 < N;
    const int mode = p.split_k > 1 ? 0 : (p.epi.d_read || p.epi.kind != E_NONE ? 2 : 1);
    // A plain 16-bit C (alpha * acc; no D, bias or activation) goes eight
    // columns per lane, one 16-byte store each, rather than four (8 bytes).
    constexpr int LPR8 = WTN / 8, RPI8 = 64 / LPR8, NIT8 = 32 / RPI8;
    constexpr int EB8 = NIT8 < 4 ? NIT8 : 4;
    static_assert(LPR8 * 8 == WTN && RPI8 * LPR8 == 64 && NIT8 * RPI8 == 32, "eight-column rows");
    const int er8 = lane / LPR8, ec8 = (lane % LPR8) * 8;
    const int col8 = n0 + wn * WTN + ec8;
    const bool wide16 = !IS_I8 && mode == 1 && p.epi.out_type != T_F32;
    const bool vec8 = aligned_to(p.epi.C, 16) && (p.epi.ldc & 7) == 0 && col8 + 7 < N;
    floatx4 bias4 = floatx4{0.f, 0.f, 0.f, 0.f};
    if (vec_col && p.split_k == 1) {
        if constexpr (IS_I8) bias4 = epi_bias4_i(p.epi, col);
        else bias4 = epi_bias4_f(p.epi, col);
    }
    // The store code (with the whole epilogue inlined) is too large to unroll FM
    // times, and a rolled loop must not index the accumulators at run time (that
    // demotes them all to private memory): the rolled loop stages row block mi
    // through copies with constant indices instead.
#pragma unroll 1
    for (int mi = 0; mi < FM; ++mi) {
#pragma unroll
        for (int m = 0; m < FM; ++m) {
            if (m == mi) {
#pragma unroll
                for (int ni = 0; ni < FN; ++ni) {
                    if constexpr (M16) {
                        // 16x16 tile q: row 16 (q >> 1) + (lane & 15), columns
                        // 16 (q & 1) + 4 (lane >> 4) .. +3
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            *reinterpret_cast<Vec4 *>(sE + (16 * (q >> 1) + L16) * RP + ni * 32 + 16 * (q & 1) +
                                                      4 * grp16) = acc[m][ni][q];
                    } else {
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            *reinterpret_cast<Vec4 *>(sE + lr * RP + ni * 32 + 8 * j + 4 * kg) =
                                Vec4{acc[m][ni][0][4 * j], acc[m][ni][0][4 * j + 1], acc[m][ni][0][4 * j + 2],
                                     acc[m][ni][0][4 * j + 3]};
                    }
                }
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // Rows go in batches of EB: the batch's LDS reads (and D loads) are issued
        // before its stores, so their latencies overlap.  Three separate bodies:
        // split-K partials, the plain alpha * acc, and the full epilogue.  The
        // plain one carries no code for D, bias or activation (the smaller code
        // alone saved several microseconds per launch), and only the full one
        // loads from memory inside the loop: a load waited for after a store waits
        // for that store too.
        const int row0 = m0 + wm * WTM + mi * 32;
        auto batch = [&](auto mode_tag, int it0) {
            constexpr int MODE = decltype(mode_tag)::value;
            Vec4 x[EB];
#pragma unroll
            for (int u = 0; u < EB; ++u)
                x[u] = *reinterpret_cast<const Vec4 *>(sE + ((it0 + u) * RPI + er) * RP + ec);
            DVec4 d[EB];
#pragma unroll
            for (int u = 0; u < EB; ++u) d[u] = DVec4{0, 0, 0, 0};
            if constexpr (MODE == 2) {
                if (p.epi.d_read) {
#pragma unroll
                    for (int u = 0; u < EB; ++u) {
                        const int row = min(row0 + (it0 + u) * RPI + er, M - 1);
                        if (vec_col) {
                            if constexpr (IS_I8)
                                d[u] = *reinterpret_cast<const intx4 *>(reinterpret_cast<const int32_t *>(p.epi.D) +
                                                                        (int64_t)row * p.epi.ldd + col);
                            else
                                d[u] = load4_f32(p.epi.D, p.epi.out_type, (int64_t)row * p.epi.ldd + col);
                        }
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < EB; ++u) {
                const int row = row0 + (it0 + u) * RPI + er;
                if (row >= M) continue;
                if constexpr (MODE == 0) {
                    ScalarT *w = reinterpret_cast<ScalarT *>(p.ws) + ((int64_t)split * M + row) * N;
                    if (vec_col) {
                        *reinterpret_cast<Vec4 *>(w + col) = x[u];
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (col + e < N) w[col + e] = x[u][e];
                    }
                } else if constexpr (MODE == 1) {
                    const int64_t c0 = (int64_t)row * p.epi.ldc + col;
                    if constexpr (IS_I8) {
                        intx4 v;
#pragma unroll
                        for (int e = 0; e < 4; ++e) v[e] = (int)((uint32_t)p.epi.ialpha * (uint32_t)x[u][e]);
                        if (vec_col) {
                            __builtin_nontemporal_store(v, reinterpret_cast<intx4 *>(
                                                               reinterpret_cast<int32_t *>(p.epi.C) + c0));
                        } else {
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                if (col + e < N) reinterpret_cast<int32_t *>(p.epi.C)[c0 + e] = v[e];
                        }
                    } else {
                        const floatx4 v = p.epi.alpha * x[u];
                        if (vec_col) {
                            store4_f32(p.epi.C, p.epi.out_type, c0, v);
                        } else {
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                if (col + e < N) store_f32(p.epi.C, p.epi.out_type, c0 + e, v[e]);
                        }
                    }
                } else {
                    if (vec_col) {
                        if constexpr (IS_I8)
                            epi_out4_i(p.epi, row, col, x[u], d[u], bias4);
                        else
                            epi_out4_f(p.epi, row, col, x[u], d[u], bias4);
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            if (col + e < N) {
                                if constexpr (IS_I8)
                                    epi_store_i(p.epi, row, col + e, x[u][e]);
                                else
                                    epi_store_f(p.epi, row, col + e, x[u][e]);
                            }
                        }
                    }
                }
            }
        };
        bool done = false;
        if constexpr (!IS_I8) {
            if (wide16) {
#pragma unroll 1
                for (int it0 = 0; it0 < NIT8; it0 += EB8) {
                    floatx4 x[EB8][2];
#pragma unroll
                    for (int u = 0; u < EB8; ++u) {
                        const float *src = sE + ((it0 + u) * RPI8 + er8) * RP + ec8;
                        x[u][0] = *reinterpret_cast<const floatx4 *>(src);
                        x[u][1] = *reinterpret_cast<const floatx4 *>(src + 4);
                    }
#pragma unroll
                    for (int u = 0; u < EB8; ++u) {
                        const int row = row0 + (it0 + u) * RPI8 + er8;
                        if (row >= M) continue;
                        const floatx4 lo = p.epi.alpha * x[u][0], hi = p.epi.alpha * x[u][1];
                        const int64_t c0 = (int64_t)row * p.epi.ldc + col8;
                        if (vec8) {
                            store8_f16x(p.epi.C, p.epi.out_type, c0, lo, hi);
                        } else {
#pragma unroll
                            for (int e = 0; e < 8; ++e)
                                if (col8 + e < N) store_f32(p.epi.C, p.epi.out_type, c0 + e, e < 4 ? lo[e] : hi[e - 4]);
                        }
                    }
                }
                done = true;
            }
        }
        if (!done) {
#pragma unroll 1
            for (int it0 = 0; it0 < NIT; it0 += EB) {
                if (mode == 0) batch(std::integral_constant<int, 0>{}, it0);
                else if (mode == 1) batch(std::integral_constant<int, 1>{}, it0);
                else batch(std::integral_constant<int, 2>{}, it0);
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }

    // Stage clock record of this workgroup (8 entries, written by lanes 0-7 of
    // wave 0 with vector stores): the four stamps, the hardware placement
    // (HW_ID: CU, shader array and engine; XCC_ID: die) with the low 32 bits of
    // the real-time counter at K-loop start and end in their high halves, the K
    // steps, and the workgroup's grid coordinates.  The end stamp follows the
    // issue of the last store, not its completion.
    if (clk_on) {
        const unsigned long long ck3 = __builtin_amdgcn_s_memtime();
        const long long wg = (long long)blockIdx.y * gridDim.x + blockIdx.x;
        if (wave == 0 && lane < 8 && wg < p.clk_wgs) {
            const unsigned hw_id = __builtin_amdgcn_s_getreg((31 << 11) | 4);
            const unsigned xcc_id = __builtin_amdgcn_s_getreg((31 << 11) | 20);
            unsigned long long v = lane == 0 ? ck0 : lane == 1 ? ck1 : lane == 2 ? ck2 : ck3;
            if (lane == 4) v = hw_id | ((rt1 & 0xffffffffull) << 32);
            if (lane == 5) v = xcc_id | ((rt2 & 0xffffffffull) << 32);
            if (lane == 6) v = (unsigned long long)nsteps;
            if (lane == 7) v = (unsigned long long)blockIdx.x | ((unsigned long long)blockIdx.y << 32);
            p.clk[wg * 8 + lane] = v;
        }
    }
}

}  // namespace dg
