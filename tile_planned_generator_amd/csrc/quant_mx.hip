// quant_mx.hip - binary16 activations -> MX fp8 e4m3 codes with one e8m0 scale
// per 32 consecutive values of a row (the OCP Microscaling v1.0 conversion), the
// activation side of the block-scaled 4-bit path (the pages' precision scheme
// with e2m1 weights, [overview] DeepGEMM article, section 2.2, second layer).
//
// Per block of 32 values x of one row:
//   amax  = max |x|
//   e     = floor(log2 amax) - 8     (8: the exponent of e4m3's largest normal, 448)
//   scale = 2^e, stored as the e8m0 code e + 127 (code 0 when amax is 0)
//   code  = e4m3(x / scale), nearest even, magnitudes above 448 saturating to 448
// x / scale is exact in binary32, so the conversion is the only rounding.  A
// block holding an infinity or a NaN gets the NaN scale code 255 and NaN codes
// 0x7f.
//
// Four lanes share a block: each lane loads 16 contiguous bytes (8 values), so
// one load instruction of a wave reads 1 KB of consecutive memory, the block
// maximum is combined over the four lanes with quad permutes, and each lane
// stores its 8 codes (8 contiguous bytes).  Each workgroup streams a contiguous
// share of the rows with the next round's loads in flight.
// HBM-bound: 2 bytes read and 1 + 1/32 bytes written per value.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kcommon.h"
#include "launch.h"

namespace dg {

// Four e4m3 codes (one dword, first value in the low byte) of binary32 values
// already divided by the block scale.  Clamping to +-448 first and then rounding
// to nearest even gives what rounding then saturating gives: every magnitude in
// (448, 464) rounds to 448 anyway, and larger ones saturate to it.  The
// conversion instruction rounds to nearest even and keeps e4m3's subnormals.
DG_DEV unsigned e4m3x4(float a, float b, float c, float d)
{
    const float lo = -448.0f, hi = 448.0f;
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_fmed3f(a, lo, hi), __builtin_amdgcn_fmed3f(b, lo, hi),
                                            0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_fmed3f(c, lo, hi), __builtin_amdgcn_fmed3f(d, lo, hi), w,
                                        true);
    return (unsigned)w;
}

constexpr int QU = 4;          // chunks of 8 values per thread and round
constexpr int QWG = 256;       // threads per workgroup
constexpr int QGRID = 2048;    // workgroups at most (eight per CU; measured on 4096x4096: 256, 512,
                               // 1024, 2048 workgroups take 20.0, 14.1, 12.5, 11.7 us: parallelism
                               // pays more than longer streams)

// Row and column (in chunks) of chunk c; 32-bit division whenever the chunk
// count fits (`narrow` is the same for the whole grid).
DG_DEV void chunk_rc(int64_t c, int64_t cpr, bool narrow, int64_t &row, int64_t &col)
{
    if (narrow) {
        const uint32_t q = (uint32_t)c / (uint32_t)cpr;
        row = q;
        col = c - (int64_t)q * cpr;
    } else {
        row = c / cpr;
        col = c - row * cpr;
    }
}

// Each workgroup streams a contiguous share of the chunks (`per` chunks, a
// multiple of QWG * QU) in rounds of QWG * QU; the loads of round r + 1 are
// issued before round r is converted.  Chunk of thread t, round r, item j:
// base + r * QWG * QU + j * QWG + t, so the four lanes 4q .. 4q+3 of a wave hold
// the four chunks of one block, and a block is in range for all four or for
// none (the chunk count is a multiple of 4): the swaps only mix lanes of one
// block.
__global__ void __launch_bounds__(QWG) quant_mx_kernel(QuantMxArgs p, int64_t per)
{
    const int64_t cpr = p.K / 8;                          // chunks per row (a multiple of 4)
    const int64_t nch = (int64_t)p.M * cpr;
    const bool narrow = nch + (int64_t)QWG * QU <= 0xffffffffLL;
    const int64_t base = (int64_t)blockIdx.x * per + threadIdx.x;
    const int64_t end = min(nch, (int64_t)(blockIdx.x + 1) * per);
    const int rounds = (int)(per / (QWG * QU));
    auto load = [&](int r, u32x4 (&raw)[QU]) {
#pragma unroll
        for (int j = 0; j < QU; ++j) {
            const int64_t c = base + (int64_t)r * QWG * QU + j * QWG;
            if (c < end) {
                int64_t row, col;
                chunk_rc(c, cpr, narrow, row, col);
                raw[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(
                    reinterpret_cast<const _Float16 *>(p.X) + row * p.ldx + col * 8));
            } else {
                raw[j] = u32x4{0u, 0u, 0u, 0u};
            }
        }
    };
    u32x4 cur[QU], nxt[QU];
    load(0, cur);
    for (int r = 0; r < rounds; ++r) {
        if (base + (int64_t)r * QWG * QU >= end) break;   // uniform over a block's lanes
        if (r + 1 < rounds) load(r + 1, nxt);
#pragma unroll
        for (int j = 0; j < QU; ++j) {
            const int64_t c = base + (int64_t)r * QWG * QU + j * QWG;
            const bool live = c < end;   // uniform over the four lanes of a block
            // The block maximum on the magnitude bits: for binary16, the order of
            // |x| is the integer order of its low 15 bits, infinities and NaN
            // above every finite value (0x7c00 and up), so one packed integer
            // maximum per dword finds both the maximum and any non-finite value.
            unsigned mx = 0;
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const unsigned w = cur[j][d] & 0x7fff7fffu;
                mx = __builtin_bit_cast(unsigned, __builtin_elementwise_max(__builtin_bit_cast(u16x2, mx),
                                                                            __builtin_bit_cast(u16x2, w)));
            }
            mx = max(mx & 0xffffu, mx >> 16);
            // lanes 4q .. 4q+3: swap neighbours, then pairs (quad permutes
            // [1,0,3,2] and [2,3,0,1], no LDS round trip)
            mx = max(mx, (unsigned)__builtin_amdgcn_update_dpp(0, (int)mx, 0xB1, 0xF, 0xF, true));
            mx = max(mx, (unsigned)__builtin_amdgcn_update_dpp(0, (int)mx, 0x4E, 0xF, 0xF, true));
            if (!live) continue;
            const bool bad = mx >= 0x7c00u;
            const float amax = (float)__builtin_bit_cast(_Float16, (unsigned short)mx);
            int64_t row, col;
            chunk_rc(c, cpr, narrow, row, col);
            unsigned sc;
            u32x2 out;
            if (bad) {
                sc = 255u;
                out = u32x2{0x7f7f7f7fu, 0x7f7f7f7fu};
            } else {
                // amax is a binary32 normal (binary16 subnormals are), so its
                // exponent field gives floor(log2 amax); e stays within -32 .. 7.
                const int e = amax == 0.0f ? -127 : (int)(__builtin_bit_cast(unsigned, amax) >> 23) - 127 - 8;
                sc = (unsigned)(e + 127);
                // 2^-e as a binary32 (e >= -32: a normal power of two); amax = 0
                // leaves every value zero, so any factor keeps the signs
                const float inv = amax == 0.0f ? 1.0f : __builtin_bit_cast(float, (unsigned)(127 - e) << 23);
                float f[8];
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    const unsigned w = cur[j][d];
                    f[2 * d] = (float)__builtin_bit_cast(_Float16, (unsigned short)(w & 0xffffu)) * inv;
                    f[2 * d + 1] = (float)__builtin_bit_cast(_Float16, (unsigned short)(w >> 16)) * inv;
                }
                out = u32x2{e4m3x4(f[0], f[1], f[2], f[3]), e4m3x4(f[4], f[5], f[6], f[7])};
            }
            __builtin_nontemporal_store(out, reinterpret_cast<u32x2 *>(
                reinterpret_cast<uint8_t *>(p.codes) + row * p.ldq + col * 8));
            // scales are group-major: block g of row `row` at g * ld_scale + row
            if ((col & 3) == 0) reinterpret_cast<uint8_t *>(p.scales)[(col / 4) * p.ld_scale + row] = (uint8_t)sc;
        }
#pragma unroll
        for (int j = 0; j < QU; ++j) cur[j] = nxt[j];
    }
}

hipError_t launch_quant_mx(const QuantMxArgs &a, hipStream_t s)
{
    const int64_t chunks = (int64_t)a.M * (a.K / 8);
    if (chunks == 0) return hipSuccess;
    constexpr int64_t R = (int64_t)QWG * QU;              // chunks per workgroup round
    int64_t grid = (chunks + R - 1) / R;
    if (grid > QGRID) grid = QGRID;
    const int64_t per = ((chunks + grid - 1) / grid + R - 1) / R * R;
    grid = (chunks + per - 1) / per;
    if (per / R > 0x7fffffff) return hipErrorInvalidValue;
    QuantMxArgs arg = a;
    int64_t per_arg = per;
    void *args[] = {&arg, &per_arg};
    hipError_t e = hipLaunchKernel(reinterpret_cast<void *>(quant_mx_kernel), dim3((unsigned)grid, 1, 1),
                                   dim3(QWG, 1, 1), args, 0, s);
    if (e != hipSuccess) return e;
    return hipGetLastError();
}

}  // namespace dg
