// skinny.hip - split-K streaming GEMMs for small M (the HBM-bound path).
//
// The pages single out "thin-tall" shapes that template libraries do not cover
// (M = 1, N = 4096; K = 131072) and the M = 1, N = 256, K = 12800 shape whose
// K does not fit on chip ([generator] DeepGEMM article, kwkr.cn, section 2.1),
// and they pick plain vector FMA over the matrix units for tiny GEMMs
// ([overview] DeepGEMM article, section 5.3: use_hmma false).  Here every
// workgroup owns one range of columns and one K slice; B is read exactly once,
// with 16-byte non-temporal loads, so the time is HBM streaming; the per-slice
// partial sums go to a workspace and a reduce kernel adds them in slice order
// and applies the epilogue (or, with one slice, the epilogue is applied here).
#include "kcommon.h"
#include "catalogue.h"
#include "launch.h"

namespace dg {

DG_DEV void unpack8(int path, const u32x4 &b, float (&w)[8])
{
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        if (path == P_BF16) {
            w[2 * d] = __builtin_bit_cast(float, b[d] << 16);
            w[2 * d + 1] = __builtin_bit_cast(float, b[d] & 0xffff0000u);
        } else {
            w[2 * d] = (float)__builtin_bit_cast(_Float16, (unsigned short)(b[d] & 0xffffu));
            w[2 * d + 1] = (float)__builtin_bit_cast(_Float16, (unsigned short)(b[d] >> 16));
        }
    }
}

DG_DEV float elt16(int path, unsigned short h)
{
    return path == P_BF16 ? __builtin_bit_cast(float, (unsigned)h << 16)
                          : (float)__builtin_bit_cast(_Float16, h);
}

// ----------------------------------------------------------------- VALU path
// Four waves per workgroup, each on its own LPR*8 columns; within a wave,
// 64/LPR row groups take the K slice's rows U consecutive rows at a time (row
// group g: rows U*g .. U*g+U-1 of each batch of U*64/LPR rows; the rows after
// the last full batch interleave) and are summed by lane shuffles at the end.
// A's slice (MR rows) is staged in LDS.
constexpr int SKINNY_A_LDS = 32768;   // bytes of A staged per workgroup

template <int PATH, int MR, int LPR>
__global__ void __launch_bounds__(256) skinny_valu_kernel(SkinnyArgs p)
{
    constexpr int RPI = 64 / LPR;       // row groups per wave
    constexpr int WCOLS = LPR * 8;      // columns per wave
    constexpr int U = 8;                // rows per lane and batch
    __shared__ __attribute__((aligned(16))) unsigned short sA[SKINNY_A_LDS / 2];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane / LPR;
    const int col = blockIdx.x * (4 * WCOLS) + wave * WCOLS + (lane % LPR) * 8;
    const int split = blockIdx.y;
    const int kbeg = split * p.k_slice;
    const int kend = min(p.K, kbeg + p.k_slice);
    const int L = kend - kbeg;
    const int M = p.M;

    const char *Bb = reinterpret_cast<const char *>(p.B) + (int64_t)(col < p.N ? col : 0) * 2 +
                     (int64_t)kbeg * p.ldb * 2;
    const int64_t ldb_b = p.ldb * 2;
    // batches of U consecutive rows per lane (U * RPI rows per wave), then single rows
    const int nmain = L / (U * RPI);
    auto load_batch = [&](int it, u32x4 (&b)[U]) {
        const int r = U * g + it * U * RPI;
#pragma unroll
        for (int u = 0; u < U; ++u) b[u] = ld16_nt(Bb + (int64_t)(r + u) * ldb_b);
    };
    // the first batch of B is in flight while A is staged
    u32x4 b0[U], b1[U];
    if (nmain > 0) load_batch(0, b0);

    // stage A[0:M][kbeg:kend]
    const unsigned short *A = reinterpret_cast<const unsigned short *>(p.A);
    for (int idx = tid; idx < MR * L; idx += 256) {
        const int m = idx / L, k = idx - m * L;
        sA[idx] = m < M ? A[(int64_t)m * p.lda + kbeg + k] : (unsigned short)0;
    }
    __syncthreads();

    float acc[MR][8];
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[m][e] = 0.f;

    auto fma_batch = [&](int it, const u32x4 (&b)[U]) {
        const int r = U * g + it * U * RPI;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float w[8];
            unpack8(PATH, b[u], w);
#pragma unroll
            for (int m = 0; m < MR; ++m) {
                const float a = elt16(PATH, sA[m * L + r + u]);
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[m][e] += a * w[e];
            }
        }
    };
    // two register buffers: batch it+1 streams in while batch it is consumed.
    // The loop issues both of its loads unconditionally (the last batches are
    // peeled off below): a load under a branch makes the compiler's wait before
    // the following batch assume the branch not taken, so that it also waits
    // for the batch just issued.
    int it = 0;
    for (; it + 2 < nmain; it += 2) {
        load_batch(it + 1, b1);
        __builtin_amdgcn_sched_barrier(0);
        fma_batch(it, b0);
        load_batch(it + 2, b0);
        __builtin_amdgcn_sched_barrier(0);
        fma_batch(it + 1, b1);
    }
    if (it + 1 < nmain) {
        load_batch(it + 1, b1);
        __builtin_amdgcn_sched_barrier(0);
        fma_batch(it, b0);
        fma_batch(it + 1, b1);
    } else if (it < nmain) {
        fma_batch(it, b0);
    }
    // the rows after the last full batch (fewer than U per lane): all loaded at
    // once, then added in ascending row order
    {
        const int r0 = g + nmain * U * RPI;
        u32x4 bt[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            bt[u] = r0 + u * RPI < L ? ld16_nt(Bb + (int64_t)(r0 + u * RPI) * ldb_b) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int r = r0 + u * RPI;
            if (r >= L) break;
            float w[8];
            unpack8(PATH, bt[u], w);
#pragma unroll
            for (int m = 0; m < MR; ++m) {
                const float a = elt16(PATH, sA[m * L + r]);
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[m][e] += a * w[e];
            }
        }
    }

    // sum the row groups of the wave (fixed order)
#pragma unroll
    for (int off = 32; off >= LPR; off >>= 1)
#pragma unroll
        for (int m = 0; m < MR; ++m)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[m][e] += __shfl_xor(acc[m][e], off, 64);

    if (g != 0 || col >= p.N) return;
#pragma unroll
    for (int m = 0; m < MR; ++m) {
        if (m >= M) break;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int j = col + e;
            if (j >= p.N) break;
            if (p.split_k > 1)
                reinterpret_cast<float *>(p.ws)[((int64_t)split * M + m) * p.N + j] = acc[m][e];
            else
                epi_store_f(p.epi, m, j, acc[m][e]);
        }
    }
}

// ----------------------------------------------------------------- MFMA path
// M <= 16 with v_mfma_f32_16x16x32_{f16,bf16}.  Each wave covers 128 columns
// and 32 rows of K per step: lane (j, kg) loads rows k0+8kg .. k0+8kg+7 of
// columns c0+8j .. c0+8j+7 (16-byte loads, 16 lanes per 256-byte row segment),
// transposes the 8x8 block in registers and so holds, for each of 8 columns,
// the 8 consecutive k the MFMA B operand wants; MFMA t then computes output
// column c0 + 8j + t for j = 0..15.
template <int PATH>
__global__ void __launch_bounds__(256) skinny_mfma_kernel(SkinnyArgs p)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int j = lane & 15, kg = lane >> 4;
    const int c0 = blockIdx.x * 512 + wave * 128;
    const int col = c0 + 8 * j;
    const int split = blockIdx.y;
    const int kbeg = split * p.k_slice;
    const int kend = min(p.K, kbeg + p.k_slice);
    const int M = p.M;

    const char *Bb = reinterpret_cast<const char *>(p.B) + (int64_t)(col < p.N ? col : 0) * 2;
    const int64_t ldb_b = p.ldb * 2;
    const char *Ab = reinterpret_cast<const char *>(p.A) + (int64_t)min(j, M - 1) * p.lda * 2;

    floatx4 acc[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) acc[t] = floatx4{0.f, 0.f, 0.f, 0.f};

    // one step: 8 rows of 8 columns of B per lane and 8 k of A
    struct Tile {
        u32x4 b[8];
        u32x4 a;
    };
    auto load = [&](int k0, bool partial, Tile &t) {
        const int kr = k0 + 8 * kg;
        // one 64-bit row address per step, then the uniform row pitch per row
        // (a product per row costs three quarter-rate multiplies per load)
        const char *rp = Bb + (int64_t)kr * ldb_b;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            if (partial) {
                t.b[r] = ld16_nt(Bb + (int64_t)min(kr + r, kend - 1) * ldb_b);
                if (kr + r >= kend) t.b[r] = u32x4{0, 0, 0, 0};
            } else {
                t.b[r] = ld16_nt(rp + r * ldb_b);
            }
        }
        t.a = ld16(Ab + (int64_t)(partial ? min(kr, kend - 8) : kr) * 2);
        if (partial && kr >= kend) t.a = u32x4{0, 0, 0, 0};
    };
    auto compute = [&](const Tile &t) {
        u32x4 bt[8];
        transpose8x8_b16(t.b, bt);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            if constexpr (PATH == P_BF16)
                acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, t.a),
                                                                 __builtin_bit_cast(bf16x8, bt[q]),
                                                                 acc[q], 0, 0, 0);
            else
                acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, t.a),
                                                                __builtin_bit_cast(half8, bt[q]),
                                                                acc[q], 0, 0, 0);
        }
    };

    // two register buffers: step it+1 streams in while step it is consumed
    // (unconditional loads in the loop, the last steps peeled off, as in the
    // VALU kernel)
    const int nfull = (kend - kbeg) / 32;
    Tile t0, t1;
    if (nfull > 0) load(kbeg, false, t0);
    // (sched_barrier: the compiler would otherwise sink each load below the
    // step before it, and the loop would drain every iteration)
    int it = 0;
    for (; it + 2 < nfull; it += 2) {
        load(kbeg + (it + 1) * 32, false, t1);
        __builtin_amdgcn_sched_barrier(0);
        compute(t0);
        load(kbeg + (it + 2) * 32, false, t0);
        __builtin_amdgcn_sched_barrier(0);
        compute(t1);
    }
    if (it + 1 < nfull) {
        load(kbeg + (it + 1) * 32, false, t1);
        __builtin_amdgcn_sched_barrier(0);
        compute(t0);
        compute(t1);
    } else if (it < nfull) {
        compute(t0);
    }
    const int k0 = kbeg + nfull * 32;
    if (k0 < kend) {   // tail step: rows past the slice are zero
        load(k0, true, t1);
        compute(t1);
    }

    // lane holds rows 4*kg + v of columns c0 + 8j + t
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const int n = col + t;
        if (n >= p.N || col >= p.N) continue;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int m = 4 * kg + v;
            if (m >= M) continue;
            if (p.split_k > 1)
                reinterpret_cast<float *>(p.ws)[((int64_t)split * M + m) * p.N + n] = acc[t][v];
            else
                epi_store_f(p.epi, m, n, acc[t][v]);
        }
    }
}

// ----------------------------------------------------------------- e2m1 path
// B codes stored N x K (K contiguous, even k in the low nibble), scales G x N
// (group-major, ld_scale per group).
// Four columns per wave, 16 lanes each (16 columns per workgroup); lane q of a
// column takes the 32-code groups q, q+16, ... of the slice: one 16-byte load of
// codes, its fp16 scale, the group's dot product with A in fp32
// (v_cvt_scalef32_pk_f16_fp4 with a unit scale, then v_dot2_f32_f16), and the
// scale applied to the group sum.  A's slice and the slice's scales of the
// workgroup's 16 columns (one 32-byte piece per group row of the group-major
// scale array, fetched as dwords) are staged in LDS once per workgroup, their
// loads issued with the first codes; groups are taken GU at a time, all their
// loads issued before any arithmetic; the 16 lanes of a column are summed in a fixed
// order at the end.
constexpr int E2M1_COLS_PER_WG = 16;
constexpr int E2M1_A_LDS = 32768;   // bytes of A staged per workgroup
constexpr int E2M1_MAX_GROUPS = E2M1_A_LDS / 2 / 32;   // groups of the longest slice (MR = 1)

template <int MR>
__global__ void __launch_bounds__(256) skinny_e2m1_kernel(SkinnyArgs p)
{
    constexpr int GU = MR <= 2 ? 8 : 4;   // groups in flight per lane
    __shared__ __attribute__((aligned(16))) _Float16 sA[E2M1_A_LDS / 2];
    __shared__ __attribute__((aligned(16))) _Float16 sS[E2M1_MAX_GROUPS * E2M1_COLS_PER_WG];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int q = lane & 15;
    const int cw = wave * 4 + (lane >> 4);   // column within the workgroup
    const int n0 = blockIdx.x * E2M1_COLS_PER_WG;
    const int n = n0 + cw;
    const bool valid = n < p.N;
    const int nc = valid ? n : 0;   // columns past N read column 0 and store nothing
    const int split = blockIdx.y;
    const int kbeg = split * p.k_slice;
    const int kend = min(p.K, kbeg + p.k_slice);
    const int gbeg = kbeg >> 5, gend = kend >> 5;
    const int L = kend - kbeg;      // a multiple of 32
    const int M = p.M;

    const char *Bc = reinterpret_cast<const char *>(p.B) + (int64_t)nc * (p.ldb / 2);
    const _Float16 *A = reinterpret_cast<const _Float16 *>(p.A);

    u32x4 c[GU];
    int gcs[GU];
    auto load_groups = [&](int g0) {
#pragma unroll
        for (int u = 0; u < GU; ++u) {
            const int gi = g0 + 16 * u;
            gcs[u] = gi < gend ? gi : gbeg;   // a valid group; its terms are dropped below
            c[u] = ld16_nt(Bc + (int64_t)gcs[u] * 16);
        }
    };

    // Staging of the slice's scales of the workgroup's columns (group g,
    // columns n0 .. n0+15: 32 contiguous bytes, 8 dwords, of the group-major
    // array, rows of ld_scale fp16, ld_scale even) and of A[0:M][kbeg:kend]
    // (16-byte chunks; rows past M are zero).  The first SB dwords and AB
    // chunks per thread are requested together with the first codes, so that
    // one memory round trip serves all three; longer slices stage the rest
    // afterwards.  Buffer loads return 0 past the scale array's end; columns
    // past N are never used.
    constexpr int SB = 4, AB = 2 * MR;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void *>(p.scale), (short)0, (int)((int64_t)(p.K / 32) * p.ld_scale * 2), 0x00020000);
    unsigned *sSw = reinterpret_cast<unsigned *>(sS);
    const int ns = (gend - gbeg) * 8, L8 = L / 8, na = MR * L8;
    auto scale_off = [&](int idx) {
        return (int)(((int64_t)(gbeg + (idx >> 3)) * p.ld_scale + n0) * 2 + 4 * (idx & 7));
    };
    auto a_chunk = [&](int idx) {
        const int m = idx / L8, k8 = idx - m * L8;
        u32x4 v = u32x4{0u, 0u, 0u, 0u};
        if (m < M) v = ld16(A + (int64_t)m * p.lda + kbeg + 8 * k8);
        return v;
    };
    unsigned sv[SB];
    u32x4 av[AB];
#pragma unroll
    for (int j = 0; j < SB; ++j) {
        const int idx = tid + 256 * j;
        sv[j] = idx < ns ? __builtin_amdgcn_raw_buffer_load_b32(rs, scale_off(idx), 0, 0) : 0u;
    }
#pragma unroll
    for (int j = 0; j < AB; ++j) {
        const int idx = tid + 256 * j;
        av[j] = idx < na ? a_chunk(idx) : u32x4{0u, 0u, 0u, 0u};
    }
    // unconditional (lanes past the slice's groups load group gbeg, unused), so
    // that the staging writes below wait only for the staging loads
    load_groups(gbeg + q);
#pragma unroll
    for (int j = 0; j < SB; ++j) {
        const int idx = tid + 256 * j;
        if (idx < ns) sSw[idx] = sv[j];
    }
#pragma unroll
    for (int j = 0; j < AB; ++j) {
        const int idx = tid + 256 * j;
        if (idx < na) *reinterpret_cast<u32x4 *>(sA + 8 * idx) = av[j];
    }
    for (int idx = tid + 256 * SB; idx < ns; idx += 256)
        sSw[idx] = __builtin_amdgcn_raw_buffer_load_b32(rs, scale_off(idx), 0, 0);
    for (int idx = tid + 256 * AB; idx < na; idx += 256)
        *reinterpret_cast<u32x4 *>(sA + 8 * idx) = a_chunk(idx);
    __syncthreads();

    float acc[MR];
#pragma unroll
    for (int m = 0; m < MR; ++m) acc[m] = 0.f;

    for (int g0 = gbeg + q; g0 < gend; g0 += 16 * GU) {
        if (g0 != gbeg + q) load_groups(g0);
#pragma unroll
        for (int u = 0; u < GU; ++u) {
            half2v w[16];
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                w[4 * d + 0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c[u][d], 1.0f, 0);
                w[4 * d + 1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c[u][d], 1.0f, 1);
                w[4 * d + 2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c[u][d], 1.0f, 2);
                w[4 * d + 3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c[u][d], 1.0f, 3);
            }
#pragma unroll
            for (int m = 0; m < MR; ++m) {
                if (m >= M) break;
                const u32x4 *ar = reinterpret_cast<const u32x4 *>(sA + m * L + (gcs[u] - gbeg) * 32);
                float dsum = 0.f;
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    const u32x4 av = ar[h];
#pragma unroll
                    for (int d = 0; d < 4; ++d) {
                        // copy the element first: a bit_cast applied directly to a
                        // vector element with a loop index reads element 0 (clang)
                        const unsigned ad = av[d];
                        dsum = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2v, ad), w[4 * h + d],
                                                      dsum, false);
                    }
                }
                if (g0 + 16 * u < gend) acc[m] += (float)sS[(gcs[u] - gbeg) * E2M1_COLS_PER_WG + cw] * dsum;
            }
        }
    }
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int off = 8; off >= 1; off >>= 1) acc[m] += __shfl_xor(acc[m], off, 64);
    if (q != 0 || !valid) return;
#pragma unroll
    for (int m = 0; m < MR; ++m) {
        if (m >= M) break;
        if (p.split_k > 1)
            reinterpret_cast<float *>(p.ws)[((int64_t)split * M + m) * p.N + n] = acc[m];
        else
            epi_store_f(p.epi, m, n, acc[m]);
    }
}

// ---------------------------------------------------------------- launchers
struct SkinnyEntry {
    void (*fn)(SkinnyArgs);
};

#define DG_SV_ENTRY(path, mr, lpr) {skinny_valu_kernel<path, mr, lpr>},
#define DG_SM_ENTRY(path) {skinny_mfma_kernel<path>},
#define DG_SE_ENTRY(mr) {skinny_e2m1_kernel<mr>},

static const SkinnyEntry k_valu[] = {DG_SKINNY_VALU_CATALOGUE(DG_SV_ENTRY)};
static const SkinnyEntry k_mfma[] = {DG_SKINNY_MFMA_CATALOGUE(DG_SM_ENTRY)};
static const SkinnyEntry k_e2m1[] = {DG_SKINNY_E2M1_CATALOGUE(DG_SE_ENTRY)};
// rows of A each staging kernel holds in LDS (its MR)
#define DG_SV_MR(path, mr, lpr) mr,
#define DG_SE_MR(mr) mr,
static const int k_valu_mr[] = {DG_SKINNY_VALU_CATALOGUE(DG_SV_MR)};
static const int k_e2m1_mr[] = {DG_SKINNY_E2M1_CATALOGUE(DG_SE_MR)};

int skinny_valu_count() { return (int)(sizeof(k_valu) / sizeof(k_valu[0])); }
int skinny_mfma_count() { return (int)(sizeof(k_mfma) / sizeof(k_mfma[0])); }
int skinny_e2m1_count() { return (int)(sizeof(k_e2m1) / sizeof(k_e2m1[0])); }

static hipError_t launch_entry(const SkinnyEntry *tab, int count, int id, const SkinnyArgs &a,
                               int gx, int gy, hipStream_t s)
{
    if (id < 0 || id >= count) return hipErrorInvalidValue;
    hipLaunchKernelGGL(tab[id].fn, dim3(gx, gy, 1), dim3(256, 1, 1), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_skinny_valu(int id, const SkinnyArgs &a, int gx, int gy, hipStream_t s)
{
    // the A slice must fit the kernel's LDS staging area
    if (id >= 0 && id < skinny_valu_count() && (int64_t)a.k_slice * k_valu_mr[id] * 2 > SKINNY_A_LDS)
        return hipErrorInvalidValue;
    return launch_entry(k_valu, skinny_valu_count(), id, a, gx, gy, s);
}
hipError_t launch_skinny_mfma(int id, const SkinnyArgs &a, int gx, int gy, hipStream_t s)
{
    return launch_entry(k_mfma, skinny_mfma_count(), id, a, gx, gy, s);
}
hipError_t launch_skinny_e2m1(int id, const SkinnyArgs &a, int gx, int gy, hipStream_t s)
{
    // the A slice must fit the kernel's LDS staging area, in whole 32-k groups,
    // and every slice must start before K (the kernel reads a slice's first
    // group without a check)
    if (id >= 0 && id < skinny_e2m1_count() &&
        ((int64_t)a.k_slice * k_e2m1_mr[id] * 2 > E2M1_A_LDS || a.k_slice % 32 || a.k_slice <= 0 ||
         a.K <= 0 || (int64_t)(gy - 1) * a.k_slice >= a.K))
        return hipErrorInvalidValue;
    return launch_entry(k_e2m1, skinny_e2m1_count(), id, a, gx, gy, s);
}

// ------------------------------------------------------------ split-K reduce
// out[i][j] = epilogue( sum over the slices s of ws[s][i][j] ).  `lanes`
// consecutive lanes share an output: lane t adds slices [t*C, (t+1)*C) in
// ascending order (C = ceil(S / lanes)), eight loads in flight, and the lanes'
// sums are combined by a butterfly whose pairs add in the same order on both
// sides, so the result does not depend on timing.
__global__ void __launch_bounds__(256) reduce_kernel(ReduceArgs a)
{
    const int T = a.lanes;
    const int64_t MN = (int64_t)a.M * a.N;
    const int t = threadIdx.x & (T - 1);
    const int64_t idx = ((int64_t)blockIdx.x * 256 + threadIdx.x) / T;
    const bool ok = idx < MN;
    const int S = a.split_k;
    const int C = (S + T - 1) / T;
    const int s0 = min(S, t * C), s1 = min(S, s0 + C);
    const int64_t base = ok ? idx : 0;
    if (a.is_int) {
        const int32_t *w = reinterpret_cast<const int32_t *>(a.ws) + base;
        uint32_t acc = 0;
        int s = s0;
        for (; s + 8 <= s1; s += 8) {
            int32_t v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = ok ? w[(int64_t)(s + u) * MN] : 0;
#pragma unroll
            for (int u = 0; u < 8; ++u) acc += (uint32_t)v[u];
        }
        for (; s < s1; ++s) acc += ok ? (uint32_t)w[(int64_t)s * MN] : 0u;
        for (int off = T / 2; off >= 1; off >>= 1) acc += (uint32_t)__shfl_xor((int)acc, off, 64);
        if (t == 0 && ok) {
            const int i = (int)(idx / a.N), j = (int)(idx - (int64_t)i * a.N);
            epi_store_i(a.epi, i, j, (int32_t)acc);
        }
    } else {
        const float *w = reinterpret_cast<const float *>(a.ws) + base;
        float acc = 0.f;
        int s = s0;
        for (; s + 8 <= s1; s += 8) {
            float v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = ok ? w[(int64_t)(s + u) * MN] : 0.f;
#pragma unroll
            for (int u = 0; u < 8; ++u) acc += v[u];
        }
        for (; s < s1; ++s) acc += ok ? w[(int64_t)s * MN] : 0.f;
        for (int off = T / 2; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 64);
        if (t == 0 && ok) {
            const int i = (int)(idx / a.N), j = (int)(idx - (int64_t)i * a.N);
            epi_store_f(a.epi, i, j, acc);
        }
    }
}

// Few slices (lanes == 1) and N a multiple of 4: each thread sums four
// consecutive outputs of one row with 16-byte loads of every slice, in slice
// order, and stores them through the four-column epilogue when the output,
// D and bias allow it (else one element at a time).
__global__ void __launch_bounds__(256) reduce4_kernel(ReduceArgs a)
{
    const int64_t MN = (int64_t)a.M * a.N;
    const int64_t idx = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (idx >= MN) return;
    const int i = (int)(idx / a.N), j = (int)(idx - (int64_t)i * a.N);
    const bool vec = epi_vec_ok(a.epi, false, nullptr, a.N);
    if (a.is_int) {
        const int32_t *w = reinterpret_cast<const int32_t *>(a.ws) + idx;
        intx4 acc = intx4{0, 0, 0, 0};
        for (int k = 0; k < a.split_k; ++k) {
            const intx4 v = __builtin_nontemporal_load(reinterpret_cast<const intx4 *>(w + (int64_t)k * MN));
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[c] = (int)((uint32_t)acc[c] + (uint32_t)v[c]);
        }
        if (vec) {
            epi_store4_i(a.epi, i, j, acc);
        } else {
#pragma unroll
            for (int c = 0; c < 4; ++c) epi_store_i(a.epi, i, j + c, acc[c]);
        }
    } else {
        const float *w = reinterpret_cast<const float *>(a.ws) + idx;
        floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
        for (int k = 0; k < a.split_k; ++k)
            acc += __builtin_nontemporal_load(reinterpret_cast<const floatx4 *>(w + (int64_t)k * MN));
        if (vec) {
            epi_store4_f(a.epi, i, j, acc);
        } else {
#pragma unroll
            for (int c = 0; c < 4; ++c) epi_store_f(a.epi, i, j + c, acc[c]);
        }
    }
}

// Many slices and N a multiple of 4: R = lanes runs of slices per group of four
// consecutive outputs.  A workgroup holds 256 / R groups; thread (run r, group
// g) sums slices [r*C, (r+1)*C) of its four outputs in ascending order, with
// 16-byte loads that are contiguous across the threads of a run (up to 16 in
// flight per thread), and the R run
// sums are then added in run order through LDS.  The order of every addition is
// fixed, so the result does not depend on timing.
__global__ void __launch_bounds__(256) reduce_runs_kernel(ReduceArgs a)
{
    constexpr int RU = 16;   // loads in flight per thread: one round trip for runs of up to 16 slices
    const int R = a.lanes, G = 256 / R;
    const int t = threadIdx.x, g = t % G, r = t / G;
    const int64_t MN = (int64_t)a.M * a.N;
    const int64_t o4 = ((int64_t)blockIdx.x * G + g) * 4;
    const bool ok = o4 < MN;
    const int S = a.split_k;
    const int C = (S + R - 1) / R;
    const int s0 = min(S, r * C), s1 = min(S, s0 + C);
    __shared__ floatx4 part[256];
    if (a.is_int) {
        const int32_t *w = reinterpret_cast<const int32_t *>(a.ws) + (ok ? o4 : 0);
        intx4 acc = intx4{0, 0, 0, 0};
        for (int s = s0; s < s1; s += RU) {
            intx4 v[RU];
#pragma unroll
            for (int u = 0; u < RU; ++u)
                v[u] = (ok && s + u < s1)
                           ? __builtin_nontemporal_load(reinterpret_cast<const intx4 *>(w + (int64_t)(s + u) * MN))
                           : intx4{0, 0, 0, 0};
#pragma unroll
            for (int u = 0; u < RU; ++u)
#pragma unroll
                for (int c = 0; c < 4; ++c) acc[c] = (int)((uint32_t)acc[c] + (uint32_t)v[u][c]);
        }
        part[t] = __builtin_bit_cast(floatx4, acc);
        __syncthreads();
        if (r != 0 || !ok) return;
        for (int q = 1; q < R; ++q) {
            const intx4 v = __builtin_bit_cast(intx4, part[q * G + g]);
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[c] = (int)((uint32_t)acc[c] + (uint32_t)v[c]);
        }
        const int i = (int)(o4 / a.N), j = (int)(o4 - (int64_t)i * a.N);
        if (epi_vec_ok(a.epi, false, nullptr, a.N)) {
            epi_store4_i(a.epi, i, j, acc);
        } else {
#pragma unroll
            for (int c = 0; c < 4; ++c) epi_store_i(a.epi, i, j + c, acc[c]);
        }
    } else {
        const float *w = reinterpret_cast<const float *>(a.ws) + (ok ? o4 : 0);
        floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
        for (int s = s0; s < s1; s += RU) {
            floatx4 v[RU];
#pragma unroll
            for (int u = 0; u < RU; ++u)
                v[u] = (ok && s + u < s1)
                           ? __builtin_nontemporal_load(reinterpret_cast<const floatx4 *>(w + (int64_t)(s + u) * MN))
                           : floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int u = 0; u < RU; ++u) acc += v[u];
        }
        part[t] = acc;
        __syncthreads();
        if (r != 0 || !ok) return;
        for (int q = 1; q < R; ++q) acc += part[q * G + g];
        const int i = (int)(o4 / a.N), j = (int)(o4 - (int64_t)i * a.N);
        if (epi_vec_ok(a.epi, false, nullptr, a.N)) {
            epi_store4_f(a.epi, i, j, acc);
        } else {
#pragma unroll
            for (int c = 0; c < 4; ++c) epi_store_f(a.epi, i, j + c, acc[c]);
        }
    }
}

// pad_k tail: one thread per output, at most 31 products each (K past the
// MFMA-aligned part), summed in ascending k.  A handful of products per output:
// plain loads, coalesced along N for a row-major B.
__global__ void __launch_bounds__(256) tail_kernel(TailArgs a)
{
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (int64_t)a.M * a.N) return;
    const int m = (int)(idx / a.N), n = (int)(idx - (int64_t)m * a.N);
    if (a.path == P_I8) {
        const int8_t *A = reinterpret_cast<const int8_t *>(a.A) + (int64_t)m * a.lda;
        const int8_t *B = reinterpret_cast<const int8_t *>(a.B);
        uint32_t acc = 0;
        for (int k = a.k0; k < a.k1; ++k) {
            const int8_t b = a.b_kmajor ? B[(int64_t)n * a.ldb + k] : B[(int64_t)k * a.ldb + n];
            acc += (uint32_t)((int32_t)A[k] * (int32_t)b);
        }
        reinterpret_cast<int32_t *>(a.ws)[idx] = (int32_t)acc;
    } else {
        const unsigned short *A = reinterpret_cast<const unsigned short *>(a.A) + (int64_t)m * a.lda;
        const unsigned short *B = reinterpret_cast<const unsigned short *>(a.B);
        float acc = 0.f;
        for (int k = a.k0; k < a.k1; ++k) {
            const unsigned short b = a.b_kmajor ? B[(int64_t)n * a.ldb + k] : B[(int64_t)k * a.ldb + n];
            acc += elt16(a.path, A[k]) * elt16(a.path, b);
        }
        reinterpret_cast<float *>(a.ws)[idx] = acc;
    }
}

hipError_t launch_tail(const TailArgs &a, hipStream_t s)
{
    const int64_t grid = ((int64_t)a.M * a.N + 255) / 256;
    if (grid > 0x7fffffff || a.k1 - a.k0 > 31 || a.k0 < 0) return hipErrorInvalidValue;
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL(tail_kernel, dim3((unsigned)grid, 1, 1), dim3(256, 1, 1), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_reduce(const ReduceArgs &a, hipStream_t s)
{
    if (a.lanes < 1 || a.lanes > 64 || (a.lanes & (a.lanes - 1))) return hipErrorInvalidValue;
    const int64_t MN = (int64_t)a.M * a.N;
    if ((a.N & 3) == 0 && ((uintptr_t)a.ws & 15) == 0) {
        if (a.lanes == 1) {
            const int64_t grid4 = (MN / 4 + 255) / 256;
            if (grid4 > 0x7fffffff) return hipErrorInvalidValue;
            hipLaunchKernelGGL(reduce4_kernel, dim3((unsigned)grid4, 1, 1), dim3(256, 1, 1), 0, s, a);
            return hipGetLastError();
        }
        if (a.lanes <= 16) {
            const int64_t groups = 256 / a.lanes;
            const int64_t gridr = (MN / 4 + groups - 1) / groups;
            if (gridr > 0x7fffffff) return hipErrorInvalidValue;
            hipLaunchKernelGGL(reduce_runs_kernel, dim3((unsigned)gridr, 1, 1), dim3(256, 1, 1), 0, s, a);
            return hipGetLastError();
        }
    }
    const int64_t grid = (MN * a.lanes + 255) / 256;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(reduce_kernel, dim3((unsigned)grid, 1, 1), dim3(256, 1, 1), 0, s, a);
    return hipGetLastError();
}

}  // namespace dg
