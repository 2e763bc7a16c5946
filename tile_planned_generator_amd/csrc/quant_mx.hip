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
// One thread per block: four 16-byte loads, two 16-byte code stores and one
// scale byte; consecutive threads take consecutive blocks of a row, so a wave
// reads and writes contiguous memory.  HBM-bound: 2 bytes read and 1 + 1/32
// bytes written per value.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kcommon.h"
#include "launch.h"

namespace dg {

// e4m3 code of a binary32 value v with |v| < 512 (or any v: magnitudes of 448
// and above give 448), nearest even.  Normal range: 3 mantissa bits kept from
// the binary32 significand with round-half-even on the 20 dropped bits (a carry
// out of the mantissa moves to the next exponent, which the code's bit layout
// absorbs).  Below 2^-6: the subnormal quantum is 2^-9, so the code is
// rint(|v| * 2^9) (8 is the smallest normal, code 0x08, again by the layout).
DG_DEV unsigned e4m3_rne_sat(float v)
{
    const unsigned u = __builtin_bit_cast(unsigned, v);
    const unsigned sign = (u >> 24) & 0x80u;
    const float a = __builtin_fabsf(v);
    unsigned code;
    if (a >= 448.0f) {
        code = 0x7eu;
    } else if (a < 0.015625f) {
        code = (unsigned)__builtin_rintf(a * 512.0f);
    } else {
        const unsigned ua = u & 0x7fffffffu;
        const int exp = (int)(ua >> 23) - 127;          // -6 .. 8
        const unsigned man = ua & 0x7fffffu;
        const unsigned keep = man >> 20, rem = man & 0xfffffu;
        const unsigned up = (rem > 0x80000u || (rem == 0x80000u && (keep & 1u))) ? 1u : 0u;
        code = ((unsigned)(exp + 7) << 3) + keep + up;
        if (code > 0x7eu) code = 0x7eu;
    }
    return sign | code;
}

__global__ void __launch_bounds__(256) quant_mx_kernel(QuantMxArgs p)
{
    const int G = p.K / 32;
    const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= (int64_t)p.M * G) return;
    const int row = (int)(b / G), g = (int)(b - (int64_t)row * G);
    const _Float16 *x = reinterpret_cast<const _Float16 *>(p.X) + (int64_t)row * p.ldx + g * 32;
    u32x4 raw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) raw[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(x) + i);
    float f[32];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const unsigned w = raw[i][j];
            f[8 * i + 2 * j] = (float)__builtin_bit_cast(_Float16, (unsigned short)(w & 0xffffu));
            f[8 * i + 2 * j + 1] = (float)__builtin_bit_cast(_Float16, (unsigned short)(w >> 16));
        }
    float amax = 0.0f;
    bool finite = true;
#pragma unroll
    for (int t = 0; t < 32; ++t) {
        const float a = __builtin_fabsf(f[t]);
        finite = finite && a <= 65504.0f;   // false for infinities and NaN
        amax = a > amax ? a : amax;
    }
    unsigned sc;
    u32x4 out[2];
    if (!finite) {
        sc = 255u;
        out[0] = out[1] = u32x4{0x7f7f7f7fu, 0x7f7f7f7fu, 0x7f7f7f7fu, 0x7f7f7f7fu};
    } else {
        // amax is a binary32 normal (binary16 subnormals are), so its exponent
        // field gives floor(log2 amax); e stays within -32 .. 7.
        const int e = amax == 0.0f ? -127 : (int)(__builtin_bit_cast(unsigned, amax) >> 23) - 127 - 8;
        sc = (unsigned)(e + 127);
        // 2^-e as a binary32 (e >= -32: a normal power of two); amax = 0 leaves
        // every value zero, so any factor keeps the signs
        const float inv = amax == 0.0f ? 1.0f : __builtin_bit_cast(float, (unsigned)(127 - e) << 23);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            unsigned w = 0;
#pragma unroll
            for (int t = 0; t < 4; ++t) w |= e4m3_rne_sat(f[4 * q + t] * inv) << (8 * t);
            out[q >> 2][q & 3] = w;
        }
    }
    u32x4 *dst = reinterpret_cast<u32x4 *>(reinterpret_cast<uint8_t *>(p.codes) + (int64_t)row * p.ldq + g * 32);
    __builtin_nontemporal_store(out[0], dst);
    __builtin_nontemporal_store(out[1], dst + 1);
    reinterpret_cast<uint8_t *>(p.scales)[(int64_t)row * p.ld_scale + g] = (uint8_t)sc;
}

hipError_t launch_quant_mx(const QuantMxArgs &a, hipStream_t s)
{
    const int64_t blocks = (int64_t)a.M * (a.K / 32);
    if (blocks == 0) return hipSuccess;
    const int64_t grid = (blocks + 255) / 256;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    QuantMxArgs arg = a;
    void *args[] = {&arg};
    hipError_t e = hipLaunchKernel(reinterpret_cast<void *>(quant_mx_kernel), dim3((unsigned)grid, 1, 1),
                                   dim3(256, 1, 1), args, 0, s);
    if (e != hipSuccess) return e;
    return hipGetLastError();
}

}  // namespace dg
