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
// x / scale is exact (a power of two within range), so the rounding to e4m3 is
// the only one.  A block holding an infinity or a NaN gets the NaN scale code
// 255 and NaN codes 0x7f.
//
// Four lanes share a block (a quad): each lane loads 16 contiguous bytes (8
// values), so a wave's load reads 1 KB of one row; the block maximum is combined
// over the quad with quad permutes; each lane stores its 8 codes.  A workgroup
// takes 16 rows x 16 groups and writes that tile's scales through LDS, 16
// contiguous bytes per group of the group-major scale array.  HBM-bound: 2 bytes
// read and 1 + 1/32 bytes written per value.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kcommon.h"
#include "launch.h"

namespace dg {

typedef short qs16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 qh16x2 __attribute__((ext_vector_type(2)));

// Four e4m3 codes (one dword, first value in the low byte) of the four binary16
// values in two dwords, each divided by the block scale.  gfx950's scaled
// conversion takes two binary16 values and a binary32 scale and writes two e4m3
// codes into one half of the destination; measured over every binary16 pattern
// and every scale 2^-32 .. 2^7, it divides exactly by the scale, rounds to
// nearest even and keeps e4m3's subnormals, but a quotient that rounds past 448
// gives the NaN code (0x7f, or 0xff when negative) instead of saturating.  The
// inputs here are finite, so every NaN code is such an overflow: it becomes
// +-448 (0x7e / 0xfe) by clearing the code's lowest bit.
DG_DEV unsigned e4m3x4(unsigned lo, unsigned hi, float scale)
{
    qs16x2 w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(qs16x2{0, 0}, __builtin_bit_cast(qh16x2, lo), scale, false);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(w, __builtin_bit_cast(qh16x2, hi), scale, true);
    const unsigned u = __builtin_bit_cast(unsigned, w);
    // a byte's low seven bits are 0x7f exactly when adding 1 sets its bit 7
    // (no carry leaves a byte: each is at most 0x7f)
    const unsigned nan = ((u & 0x7f7f7f7fu) + 0x01010101u) & 0x80808080u;
    return u ^ (nan >> 7);
}

constexpr int QWG = 256;   // threads per workgroup (four waves)
constexpr int QR = 16;     // rows per workgroup (four per wave)
constexpr int QG = 16;     // 32-value groups per workgroup (one 1 KB row segment)

// A workgroup quantises QR rows x QG groups.  Wave w takes rows 4w .. 4w+3 of
// the tile; for each, its 64 lanes read the row's 1 KB segment (lane l: group
// l / 4, chunk l % 4, so the four lanes of a block form one quad), and write the
// 512 bytes of codes.  The scales go through LDS: the tile's QG x QR scale bytes
// are written group-major, 16 contiguous bytes per group.
__global__ void __launch_bounds__(QWG) quant_mx_kernel(QuantMxArgs p)
{
    __shared__ uint8_t s_sc[QG][QR];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int G = p.K / 32;
    const int gtiles = (G + QG - 1) / QG;
    const int64_t rt = blockIdx.x / gtiles;
    const int g0 = (int)(blockIdx.x - rt * gtiles) * QG;
    const int64_t r0 = rt * QR;
    const int g = g0 + (lane >> 2), part = lane & 3;
    const bool g_ok = g < G;   // uniform over a quad
    u32x4 raw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t row = r0 + wave * 4 + i;
        raw[i] = u32x4{0u, 0u, 0u, 0u};
        if (row < p.M && g_ok)
            raw[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(
                reinterpret_cast<const _Float16 *>(p.X) + row * p.ldx + g * 32 + part * 8));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t row = r0 + wave * 4 + i;
        // The block maximum on the magnitude bits: for binary16, the order of |x|
        // is the integer order of its low 15 bits, infinities and NaN above every
        // finite value (0x7c00 and up), so one packed integer maximum per dword
        // finds both the maximum and any non-finite value.
        unsigned mx = 0;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const unsigned w = raw[i][d] & 0x7fff7fffu;
            mx = __builtin_bit_cast(unsigned, __builtin_elementwise_max(__builtin_bit_cast(u16x2, mx),
                                                                        __builtin_bit_cast(u16x2, w)));
        }
        mx = max(mx & 0xffffu, mx >> 16);
        // lanes 4q .. 4q+3: swap neighbours, then pairs (quad permutes [1,0,3,2]
        // and [2,3,0,1], no LDS round trip)
        mx = max(mx, (unsigned)__builtin_amdgcn_update_dpp(0, (int)mx, 0xB1, 0xF, 0xF, true));
        mx = max(mx, (unsigned)__builtin_amdgcn_update_dpp(0, (int)mx, 0x4E, 0xF, 0xF, true));
        if (row >= p.M || !g_ok) continue;
        const bool bad = mx >= 0x7c00u;
        const float amax = (float)__builtin_bit_cast(_Float16, (unsigned short)mx);
        unsigned sc;
        u32x2 out;
        if (bad) {
            sc = 255u;
            out = u32x2{0x7f7f7f7fu, 0x7f7f7f7fu};
        } else {
            // amax is a binary32 normal (binary16 subnormals are), so its exponent
            // field gives floor(log2 amax); e stays within -32 .. 7.
            const int e = amax == 0.0f ? -127 : (int)(__builtin_bit_cast(unsigned, amax) >> 23) - 127 - 8;
            sc = (unsigned)(e + 127);
            // 2^e as a binary32 (a normal power of two); amax = 0 leaves every
            // value zero, so any scale keeps the signs
            const float scale = amax == 0.0f ? 1.0f : __builtin_bit_cast(float, (unsigned)(e + 127) << 23);
            out = u32x2{e4m3x4(raw[i][0], raw[i][1], scale), e4m3x4(raw[i][2], raw[i][3], scale)};
        }
        __builtin_nontemporal_store(out, reinterpret_cast<u32x2 *>(
            reinterpret_cast<uint8_t *>(p.codes) + row * p.ldq + g * 32 + part * 8));
        if (part == 0) s_sc[lane >> 2][wave * 4 + i] = (uint8_t)sc;
    }
    __syncthreads();
    // group-major scales: block g of row r at g * ld_scale + r
    const int tg = threadIdx.x / QR, tr = threadIdx.x % QR;
    if (g0 + tg < G && r0 + tr < p.M)
        reinterpret_cast<uint8_t *>(p.scales)[(int64_t)(g0 + tg) * p.ld_scale + r0 + tr] = s_sc[tg][tr];
}

hipError_t launch_quant_mx(const QuantMxArgs &a, hipStream_t s)
{
    const int64_t G = a.K / 32;
    const int64_t grid = ((int64_t)a.M + QR - 1) / QR * ((G + QG - 1) / QG);
    if (grid == 0) return hipSuccess;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    QuantMxArgs arg = a;
    void *args[] = {&arg};
    hipError_t e = hipLaunchKernel(reinterpret_cast<void *>(quant_mx_kernel), dim3((unsigned)grid, 1, 1),
                                   dim3(QWG, 1, 1), args, 0, s);
    if (e != hipSuccess) return e;
    return hipGetLastError();
}

}  // namespace dg
