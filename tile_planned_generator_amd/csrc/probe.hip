// probe.hip - hardware probe kernels: the measured half of the device
// description the planner plans with ([overview] section 4.1, stage 1: the
// hardware-aware input to candidate generation; [generator] section 3.2,
// step 1: the per-GPU hardware description).  Each kernel measures one thing;
// the host side (dg_probe in api.cpp, tile_planned_generator_amd/probe.py)
// times it and turns the time into a rate.
#include <hip/hip_runtime.h>

#include "kcommon.h"
#include "launch.h"

namespace dg {

// Streams `n16` 16-byte chunks from `buf` `passes` times with non-temporal
// loads (plain, cached loads when PLAIN: repeated over a buffer that fits a
// cache level, they measure that level): workgroup w reads its own contiguous
// share, 256 consecutive chunks (4 KB) per load round and eight rounds in
// flight, and folds them into one word per workgroup so that no load is dead.
template <bool PLAIN>
DG_DEV u32x4 probe_load(const u32x4 *p)
{
    if constexpr (PLAIN) return *p;
    else return __builtin_nontemporal_load(p);
}

template <bool PLAIN>
__global__ void __launch_bounds__(256) probe_stream_kernel(const u32x4 *buf, int64_t n16, int passes,
                                                           unsigned *sink)
{
    unsigned acc = 0;
    const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
    const int64_t beg = (int64_t)blockIdx.x * per;
    const int64_t end = beg + per < n16 ? beg + per : n16;
    for (int pass = 0; pass < passes; ++pass) {
        asm volatile("" : : : "memory");   // every pass loads again
        int64_t i = beg + threadIdx.x;
        for (; i + 7 * 256 < end; i += 8 * 256) {
            u32x4 v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = probe_load<PLAIN>(buf + i + u * 256);
#pragma unroll
            for (int u = 0; u < 8; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
        }
        for (; i < end; i += 256) {
            const u32x4 v = probe_load<PLAIN>(buf + i);
            acc ^= v.x ^ v.y ^ v.z ^ v.w;
        }
        acc = (acc << 1) | (acc >> 31);   // passes do not cancel
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) acc ^= (unsigned)__shfl_xor((int)acc, off, 64);
    __shared__ unsigned w[4];
    if ((threadIdx.x & 63) == 0) w[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = w[0] ^ w[1] ^ w[2] ^ w[3];
}

// Back-to-back independent 32x32x16 fp16 MFMAs: `iters` rounds of 8 per wave.
__global__ void __launch_bounds__(256) probe_mfma_kernel(int iters, float *sink)
{
    floatx16 acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][v] = 0.f;
    half8 a, b;
#pragma unroll
    for (int v = 0; v < 8; ++v) {
        a[v] = (_Float16)((threadIdx.x & 7) * 0.001f);
        b[v] = (_Float16)(v * 0.01f);
    }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[i], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) s += acc[i][v];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
    __shared__ float w[4];
    if ((threadIdx.x & 63) == 0) w[threadIdx.x >> 6] = s;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = w[0] + w[1] + w[2] + w[3];
}

// One wave: 1024 dword LDS reads in which lane l reads word l * stride (plus a
// multiple of 256 words that changes per read and keeps the bank of any bank
// count up to 256), modulo the 16384 words of a 64 KB array; writes the
// s_memtime ticks they took.  Reads of lanes that fall in one bank are
// serialised, so the ticks grow with the number of lanes per bank.
__global__ void __launch_bounds__(64) probe_lds_kernel(int stride, unsigned long long *ticks)
{
    __shared__ unsigned lds[16384];
    const int lane = threadIdx.x;
    for (int i = lane; i < 16384; i += 64) lds[i] = (unsigned)i * 2654435761u;
    __syncthreads();
    const unsigned idx = ((unsigned)lane * (unsigned)stride) & 16383u;
    unsigned acc = 0;
    const unsigned long long t0 = __builtin_amdgcn_s_memtime();
    for (int r = 0; r < 64; ++r) {
        unsigned v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) v[u] = lds[(idx + (unsigned)(r * 16 + u) * 256u) & 16383u];
#pragma unroll
        for (int u = 0; u < 16; ++u) acc += v[u];
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): every read of the round is done
    }
    const unsigned long long t1 = __builtin_amdgcn_s_memtime();
    if (lane == 0) ticks[0] = t1 - t0;
    if (acc == 0x12345678u) ticks[1] = acc;   // keeps the reads live
}

// The clock the MFMAs hold on given operand data.  Eight waves per workgroup
// (two per SIMD, as in the 256x256 tiled kernel), each `rounds` rounds of 8
// independent int8 32x32x32 MFMAs whose operands are read once from `src`
// (n16 16-byte chunks, indexed modulo n16).  MODE:
//   0  one operand pair for every MFMA (no change of inputs between MFMAs)
//   1  eight operand pairs, a different one for each MFMA of a round
//   2  as 1, plus six 16-byte LDS reads per lane per round (0.75 KB per MFMA,
//      the fragment traffic of the tiled kernel's 128x64 wave tile), the LDS
//      filled from src; the reads of a round are issued one round ahead
//   3  as 1 with every A operand zero
//   4  as 2 with the LDS holding zeros
//   5  the LDS reads of 2 alone, no MFMAs
// Wave 0 of each workgroup writes its s_memtime ticks (the shader clock) and
// s_memrealtime ticks (100 MHz) from entry to exit, and the workgroup's
// checksum, to out[3 * workgroup + 0, 1, 2].
template <int MODE>
__global__ void __launch_bounds__(512) probe_mfma_data_kernel(const intx4 *src, int64_t n16, int rounds,
                                                              unsigned long long *out)
{
    const unsigned long long t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
    __shared__ intx4 lds[4096];   // 64 KB
    const int t = threadIdx.x;
    for (int i = t; i < 4096; i += 512)
        lds[i] = MODE == 4 ? intx4{0, 0, 0, 0} : src[((int64_t)blockIdx.x * 4096 + i) % n16];
    __syncthreads();
    intx4 a[8], b[8];
    const int64_t base = ((int64_t)blockIdx.x * 512 + t) * 16;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int k = MODE == 0 ? 0 : i;
        a[i] = MODE == 3 ? intx4{0, 0, 0, 0} : src[(base + k) % n16];
        b[i] = src[(base + 8 + k) % n16];
    }
    intx16 acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][v] = 0;
    constexpr bool READS = MODE == 2 || MODE == 4 || MODE == 5;
    intx4 fold = {0, 0, 0, 0}, cur[6], nxt[6];
    int off = t;
    if (READS) {
#pragma unroll
        for (int j = 0; j < 6; ++j) cur[j] = lds[(off + j * 577) & 4095];
    }
    for (int it = 0; it < rounds; ++it) {
        off = (off + 64) & 4095;
        if (READS) {
#pragma unroll
            for (int j = 0; j < 6; ++j) nxt[j] = lds[(off + j * 577) & 4095];
        }
        if (MODE != 5) {
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[i], b[i], acc[i], 0, 0, 0);
        }
        if (READS) {
#pragma unroll
            for (int j = 0; j < 6; ++j) { fold ^= cur[j]; cur[j] = nxt[j]; }
        }
    }
    int sum = fold[0] ^ fold[1] ^ fold[2] ^ fold[3];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) sum ^= acc[i][v];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) sum ^= __shfl_xor(sum, o, 64);
    __shared__ int w[8];
    if ((t & 63) == 0) w[t >> 6] = sum;
    __syncthreads();
    const unsigned long long t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
    if (t == 0) {
        int c = 0;
        for (int i = 0; i < 8; ++i) c ^= w[i];
        out[3 * blockIdx.x + 0] = t1 - t0;
        out[3 * blockIdx.x + 1] = r1 - r0;
        out[3 * blockIdx.x + 2] = (unsigned)c;
    }
}

hipError_t launch_probe(int kind, void *buf, size_t bytes, int param, void *out, int grid, hipStream_t s)
{
    if (kind == 0) {
        const int passes = (param >> 1) > 0 ? (param >> 1) : 1;
        if (bytes % 16 || grid <= 0 || param < 0 || passes > 4096) return hipErrorInvalidValue;
        if (param & 1)
            hipLaunchKernelGGL(probe_stream_kernel<true>, dim3(grid), dim3(256), 0, s,
                               reinterpret_cast<const u32x4 *>(buf), (int64_t)(bytes / 16), passes,
                               reinterpret_cast<unsigned *>(out));
        else
            hipLaunchKernelGGL(probe_stream_kernel<false>, dim3(grid), dim3(256), 0, s,
                               reinterpret_cast<const u32x4 *>(buf), (int64_t)(bytes / 16), passes,
                               reinterpret_cast<unsigned *>(out));
    } else if (kind == 1) {
        if (param < 0 || grid <= 0) return hipErrorInvalidValue;
        hipLaunchKernelGGL(probe_mfma_kernel, dim3(grid), dim3(256), 0, s, param, reinterpret_cast<float *>(out));
    } else if (kind == 2) {
        if (param < 1 || param > 16384) return hipErrorInvalidValue;
        hipLaunchKernelGGL(probe_lds_kernel, dim3(1), dim3(64), 0, s, param,
                           reinterpret_cast<unsigned long long *>(out));
    } else if (kind == 3) {
        const int mode = param & 7, rounds = param >> 3;
        if (!buf || bytes < 16 || bytes % 16 || grid <= 0 || mode > 5 || rounds < 1) return hipErrorInvalidValue;
        const intx4 *src = reinterpret_cast<const intx4 *>(buf);
        const int64_t n16 = (int64_t)(bytes / 16);
        unsigned long long *o = reinterpret_cast<unsigned long long *>(out);
        switch (mode) {
        case 0: hipLaunchKernelGGL(probe_mfma_data_kernel<0>, dim3(grid), dim3(512), 0, s, src, n16, rounds, o); break;
        case 1: hipLaunchKernelGGL(probe_mfma_data_kernel<1>, dim3(grid), dim3(512), 0, s, src, n16, rounds, o); break;
        case 2: hipLaunchKernelGGL(probe_mfma_data_kernel<2>, dim3(grid), dim3(512), 0, s, src, n16, rounds, o); break;
        case 3: hipLaunchKernelGGL(probe_mfma_data_kernel<3>, dim3(grid), dim3(512), 0, s, src, n16, rounds, o); break;
        case 4: hipLaunchKernelGGL(probe_mfma_data_kernel<4>, dim3(grid), dim3(512), 0, s, src, n16, rounds, o); break;
        default: hipLaunchKernelGGL(probe_mfma_data_kernel<5>, dim3(grid), dim3(512), 0, s, src, n16, rounds, o); break;
        }
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace dg
