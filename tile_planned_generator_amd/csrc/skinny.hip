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
// 64/LPR row groups interleave over the K slice and are summed by lane
// shuffles at the end.  A's slice (MR rows) is staged in LDS.
constexpr int SKINNY_A_LDS = 32768;   // bytes of A staged per workgroup

template <int PATH, int MR, int LPR>
__global__ void __launch_bounds__(256) skinny_valu_kernel(SkinnyArgs p)
{
    constexpr int RPI = 64 / LPR;       // row groups per wave
    constexpr int WCOLS = LPR * 8;      // columns per wave
    constexpr int U = 8;                // rows in flight per lane
    __shared__ __attribute__((aligned(16))) unsigned short sA[SKINNY_A_LDS / 2];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane / LPR;
    const int col = blockIdx.x * (4 * WCOLS) + wave * WCOLS + (lane % LPR) * 8;
    const int split = blockIdx.y;
    const int kbeg = split * p.k_slice;
    const int kend = min(p.K, kbeg + p.k_slice);
    const int L = kend - kbeg;
    const int M = p.M;

    // stage A[0:M][kbeg:kend]
    const unsigned short *A = reinterpret_cast<const unsigned short *>(p.A);
    for (int idx = tid; idx < MR * L; idx += 256) {
        const int m = idx / L, k = idx - m * L;
        sA[idx] = m < M ? A[(int64_t)m * p.lda + kbeg + k] : (unsigned short)0;
    }
    __syncthreads();

    const char *Bb = reinterpret_cast<const char *>(p.B) + (int64_t)(col < p.N ? col : 0) * 2;
    const int64_t ldb_b = p.ldb * 2;

    float acc[MR][8];
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[m][e] = 0.f;

    // K schedule of the slice: main steps of U*RPI rows, then single-row-group steps.
    const int nmain = L / (U * RPI);
    int r = g;
    for (int it = 0; it < nmain; ++it, r += U * RPI) {
        u32x4 b[U];
#pragma unroll
        for (int u = 0; u < U; ++u) b[u] = ld16_nt(Bb + (int64_t)(kbeg + r + u * RPI) * ldb_b);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float w[8];
            unpack8(PATH, b[u], w);
#pragma unroll
            for (int m = 0; m < MR; ++m) {
                const float a = elt16(PATH, sA[m * L + r + u * RPI]);
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[m][e] += a * w[e];
            }
        }
    }
    for (; r < L; r += RPI) {
        u32x4 b = ld16_nt(Bb + (int64_t)(kbeg + r) * ldb_b);
        float w[8];
        unpack8(PATH, b, w);
#pragma unroll
        for (int m = 0; m < MR; ++m) {
            const float a = elt16(PATH, sA[m * L + r]);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[m][e] += a * w[e];
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

    auto step = [&](int k0, bool partial) {
        const int kr = k0 + 8 * kg;
        u32x4 b[8], bt[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const int k = partial ? min(kr + r, kend - 1) : kr + r;
            b[r] = ld16_nt(Bb + (int64_t)k * ldb_b);
            if (partial && kr + r >= kend) b[r] = u32x4{0, 0, 0, 0};
        }
        u32x4 a = ld16(Ab + (int64_t)(partial ? min(kr, kend - 8) : kr) * 2);
        if (partial && kr >= kend) a = u32x4{0, 0, 0, 0};
        transpose8x8_b16(b, bt);
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            if constexpr (PATH == P_BF16)
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                                 __builtin_bit_cast(bf16x8, bt[t]),
                                                                 acc[t], 0, 0, 0);
            else
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, a),
                                                                __builtin_bit_cast(half8, bt[t]),
                                                                acc[t], 0, 0, 0);
        }
    };

    const int nfull = (kend - kbeg) / 32;
    int k0 = kbeg;
    for (int it = 0; it < nfull; ++it, k0 += 32) step(k0, false);
    if (k0 < kend) step(k0, true);   // tail step: rows past the slice are zero

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
// B codes stored N x K (K contiguous, even k in the low nibble), scales N x G.
// One wave per column; lane l takes 32-code groups l, l+64, ... of the slice:
// one 16-byte load of codes, one fp16 scale, the group's dot product with A in
// fp32 (v_cvt_scalef32_pk_f16_fp4 with a unit scale, then v_dot2_f32_f16), and
// the scale applied to the group sum.
template <int MR>
__global__ void __launch_bounds__(256) skinny_e2m1_kernel(SkinnyArgs p)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = blockIdx.x * 4 + wave;
    if (n >= p.N) return;
    const int split = blockIdx.y;
    const int kbeg = split * p.k_slice;
    const int kend = min(p.K, kbeg + p.k_slice);
    const int gbeg = kbeg >> 5, gend = kend >> 5;
    const int M = p.M;

    const char *Bc = reinterpret_cast<const char *>(p.B) + (int64_t)n * (p.ldb / 2);
    const _Float16 *S = reinterpret_cast<const _Float16 *>(p.scale) + (int64_t)n * p.ld_scale;
    const _Float16 *A = reinterpret_cast<const _Float16 *>(p.A);

    float acc[MR];
#pragma unroll
    for (int m = 0; m < MR; ++m) acc[m] = 0.f;

    for (int gi = gbeg + lane; gi < gend; gi += 64) {
        const u32x4 c = ld16_nt(Bc + (int64_t)gi * 16);
        const float s = (float)S[gi];
        half2v w[16];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            w[4 * d + 0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c[d], 1.0f, 0);
            w[4 * d + 1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c[d], 1.0f, 1);
            w[4 * d + 2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c[d], 1.0f, 2);
            w[4 * d + 3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c[d], 1.0f, 3);
        }
#pragma unroll
        for (int m = 0; m < MR; ++m) {
            if (m >= M) break;
            const u32x4 *ar = reinterpret_cast<const u32x4 *>(A + (int64_t)m * p.lda + gi * 32);
            float dsum = 0.f;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const u32x4 av = ar[q];
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    // copy the element first: a bit_cast applied directly to a
                    // vector element with a loop index reads element 0 (clang)
                    const unsigned ad = av[d];
                    dsum = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2v, ad), w[4 * q + d],
                                                  dsum, false);
                }
            }
            acc[m] += s * dsum;
        }
    }
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) acc[m] += __shfl_xor(acc[m], off, 64);
    if (lane != 0) return;
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
    return launch_entry(k_valu, skinny_valu_count(), id, a, gx, gy, s);
}
hipError_t launch_skinny_mfma(int id, const SkinnyArgs &a, int gx, int gy, hipStream_t s)
{
    return launch_entry(k_mfma, skinny_mfma_count(), id, a, gx, gy, s);
}
hipError_t launch_skinny_e2m1(int id, const SkinnyArgs &a, int gx, int gy, hipStream_t s)
{
    return launch_entry(k_e2m1, skinny_e2m1_count(), id, a, gx, gy, s);
}

// ------------------------------------------------------------ split-K reduce
// out[i][j] = epilogue( sum_{s = 0 .. S-1} ws[s][i][j] ), s ascending, so the
// result does not depend on the order in which the slices finished.
__global__ void __launch_bounds__(256) reduce_kernel(ReduceArgs a)
{
    const int64_t MN = (int64_t)a.M * a.N;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= MN) return;
    const int i = (int)(idx / a.N), j = (int)(idx - (int64_t)i * a.N);
    if (a.is_int) {
        const int32_t *w = reinterpret_cast<const int32_t *>(a.ws);
        uint32_t s = 0;
        for (int k = 0; k < a.split_k; ++k) s += (uint32_t)w[k * MN + idx];
        epi_store_i(a.epi, i, j, (int32_t)s);
    } else {
        const float *w = reinterpret_cast<const float *>(a.ws);
        float s = 0.f;
        for (int k = 0; k < a.split_k; ++k) s += w[k * MN + idx];
        epi_store_f(a.epi, i, j, s);
    }
}

hipError_t launch_reduce(const ReduceArgs &a, hipStream_t s)
{
    const int64_t MN = (int64_t)a.M * a.N;
    const int grid = (int)((MN + 255) / 256);
    hipLaunchKernelGGL(reduce_kernel, dim3(grid, 1, 1), dim3(256, 1, 1), 0, s, a);
    return hipGetLastError();
}

}  // namespace dg
