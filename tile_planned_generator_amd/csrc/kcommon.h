// kcommon.h - device-side types and helpers shared by the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <type_traits>

#include "dg_args.h"

namespace dg {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef int intx16 __attribute__((ext_vector_type(16)));
typedef int intx4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef int intx8 __attribute__((ext_vector_type(8)));

#define DG_DEV __device__ __forceinline__

DG_DEV u32x4 ld16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }
DG_DEV u32x4 ld16_nt(const void *p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}

// Byte permute: result byte i = pool[sel.byte i], pool = {lo bytes 0..3, hi bytes 4..7}.
DG_DEV unsigned perm(unsigned hi, unsigned lo, unsigned sel)
{
    return __builtin_amdgcn_perm(hi, lo, sel);
}

// Transpose an 8 x 8 block of 16-bit values held as 8 rows of 4 dwords:
// out[j] dword e = (in[2e] element j, in[2e+1] element j).
DG_DEV void transpose8x8_b16(const u32x4 (&in)[8], u32x4 (&out)[8])
{
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const unsigned sel = (j & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
        for (int e = 0; e < 4; ++e) out[j][e] = perm(in[2 * e + 1][j >> 1], in[2 * e][j >> 1], sel);
    }
}

// Transpose 4 dwords seen as a 4 x 4 byte matrix (row r = x[r]):
// y[t] = (x[0] byte t, x[1] byte t, x[2] byte t, x[3] byte t).
DG_DEV void transpose4x4_b8(unsigned x0, unsigned x1, unsigned x2, unsigned x3, unsigned &y0,
                            unsigned &y1, unsigned &y2, unsigned &y3)
{
    const unsigned p = perm(x1, x0, 0x05010400u);  // x0.b0 x1.b0 x0.b1 x1.b1
    const unsigned q = perm(x1, x0, 0x07030602u);  // x0.b2 x1.b2 x0.b3 x1.b3
    const unsigned r = perm(x3, x2, 0x05010400u);
    const unsigned s = perm(x3, x2, 0x07030602u);
    y0 = perm(r, p, 0x05040100u);
    y1 = perm(r, p, 0x07060302u);
    y2 = perm(s, q, 0x05040100u);
    y3 = perm(s, q, 0x07060302u);
}

// 8 rows of 16 bytes -> 16 rows of 8 bytes: out[j] = (in[0] byte j, ..., in[7] byte j).
DG_DEV void transpose8x16_b8(const u32x4 (&in)[8], u32x2 (&out)[16])
{
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            unsigned y0, y1, y2, y3;
            transpose4x4_b8(in[4 * h][d], in[4 * h + 1][d], in[4 * h + 2][d], in[4 * h + 3][d], y0,
                            y1, y2, y3);
            out[4 * d + 0][h] = y0;
            out[4 * d + 1][h] = y1;
            out[4 * d + 2][h] = y2;
            out[4 * d + 3][h] = y3;
        }
}

// e2m1 -> fp16 for the 8 codes of one dword (even k in the low nibble), times s.
// The conversion runs with a unit scale, so the decoded values are exact; the
// fp16 product with s is rounded to nearest even.
DG_DEV half8 decode_e2m1x8(unsigned codes, _Float16 s)
{
    half2v h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 0);
    half2v h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 1);
    half2v h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 2);
    half2v h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 3);
    half8 w = {h0.x, h0.y, h1.x, h1.y, h2.x, h2.y, h3.x, h3.y};
    return w * s;
}

// ------------------------------------------------------------------ epilogue
DG_DEV float load_f32(const void *p, int type, int64_t idx)
{
    if (type == T_F16) return (float)reinterpret_cast<const _Float16 *>(p)[idx];
    if (type == T_BF16) return (float)reinterpret_cast<const __bf16 *>(p)[idx];
    return reinterpret_cast<const float *>(p)[idx];
}

DG_DEV void store_f32(void *p, int type, int64_t idx, float v)
{
    if (type == T_F16)
        reinterpret_cast<_Float16 *>(p)[idx] = (_Float16)v;
    else if (type == T_BF16)
        reinterpret_cast<__bf16 *>(p)[idx] = (__bf16)v;
    else
        reinterpret_cast<float *>(p)[idx] = v;
}

// GELU, erf form: x/2 * (1 + erf(x / sqrt 2)); erff is the device math library's.
DG_DEV float gelu_erf(float x) { return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f)); }

// Floating-point epilogue of one element.
DG_DEV void epi_store_f(const EpiArgs &e, int64_t i, int64_t j, float acc)
{
    float v = e.alpha * acc;
    if (e.d_read) v += e.beta * load_f32(e.D, e.out_type, i * e.ldd + j);
    if (e.kind == E_BIAS || e.kind == E_BIAS_GELU) v += load_f32(e.bias, e.bias_type, j);
    if (e.kind == E_GELU || e.kind == E_BIAS_GELU) v = gelu_erf(v);
    store_f32(e.C, e.out_type, i * e.ldc + j, v);
}

// Integer epilogue of one element: wrapping alpha*acc + beta*D in 32 bits, or a
// requantisation whose steps are each rounded in binary32 (no contraction):
// v = (f32(acc) * scale) + bias[j].
DG_DEV void epi_store_i(const EpiArgs &e, int64_t i, int64_t j, int32_t acc)
{
    if (e.kind == E_RQ_I8 || e.kind == E_RQ_F16) {
        float v = __fmul_rn((float)acc, e.rq_scale);
        if (e.bias) v = __fadd_rn(v, reinterpret_cast<const float *>(e.bias)[j]);
        if (e.kind == E_RQ_I8) {
            float r = __builtin_rintf(v);
            r = r > 127.0f ? 127.0f : (r < -128.0f ? -128.0f : r);
            reinterpret_cast<int8_t *>(e.C)[i * e.ldc + j] = (int8_t)(int)r;
        } else {
            reinterpret_cast<_Float16 *>(e.C)[i * e.ldc + j] = (_Float16)v;
        }
        return;
    }
    uint32_t v = (uint32_t)e.ialpha * (uint32_t)acc;
    if (e.d_read) v += (uint32_t)e.ibeta * (uint32_t)reinterpret_cast<const int32_t *>(e.D)[i * e.ldd + j];
    reinterpret_cast<int32_t *>(e.C)[i * e.ldc + j] = (int32_t)v;
}

// ------------------------------------------------- vectorised epilogue (4 columns)
typedef _Float16 half4v __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4v __attribute__((ext_vector_type(4)));
typedef signed char i8x4v __attribute__((ext_vector_type(4)));

DG_DEV bool aligned_to(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

DG_DEV int elt_size(int t) { return (t == T_F16 || t == T_BF16) ? 2 : (t == T_I8 ? 1 : 4); }

// Whether 4 consecutive columns can go through 4-wide vector loads and stores:
// every pointer, and every row pitch, aligned to 4 elements.
DG_DEV bool epi_vec_ok(const EpiArgs &e, bool split, const void *ws, int N)
{
    if (split) return aligned_to(ws, 16) && (N & 3) == 0;
    const int os = elt_size(e.out_type);
    bool ok = aligned_to(e.C, 4 * os) && (e.ldc & 3) == 0;
    if (e.d_read) ok = ok && aligned_to(e.D, 4 * os) && (e.ldd & 3) == 0;
    if (e.bias) ok = ok && aligned_to(e.bias, 4 * elt_size(e.bias_type));
    return ok;
}

DG_DEV floatx4 load4_f32(const void *p, int type, int64_t idx)
{
    if (type == T_F16) {
        const half4v h = *reinterpret_cast<const half4v *>(reinterpret_cast<const _Float16 *>(p) + idx);
        return floatx4{(float)h.x, (float)h.y, (float)h.z, (float)h.w};
    }
    if (type == T_BF16) {
        const bf16x4v h = *reinterpret_cast<const bf16x4v *>(reinterpret_cast<const __bf16 *>(p) + idx);
        return floatx4{(float)h.x, (float)h.y, (float)h.z, (float)h.w};
    }
    return *reinterpret_cast<const floatx4 *>(reinterpret_cast<const float *>(p) + idx);
}

// Output stores are non-temporal: C is written once and not read back here.
DG_DEV void store4_f32(void *p, int type, int64_t idx, floatx4 v)
{
    if (type == T_F16)
        __builtin_nontemporal_store(half4v{(_Float16)v.x, (_Float16)v.y, (_Float16)v.z, (_Float16)v.w},
                                    reinterpret_cast<half4v *>(reinterpret_cast<_Float16 *>(p) + idx));
    else if (type == T_BF16)
        __builtin_nontemporal_store(bf16x4v{(__bf16)v.x, (__bf16)v.y, (__bf16)v.z, (__bf16)v.w},
                                    reinterpret_cast<bf16x4v *>(reinterpret_cast<__bf16 *>(p) + idx));
    else
        __builtin_nontemporal_store(v, reinterpret_cast<floatx4 *>(reinterpret_cast<float *>(p) + idx));
}

// Eight values to a 16-bit output (type T_F16 or T_BF16), nearest even, as one
// 16-byte store: idx a multiple of 8, p 16-byte aligned.
typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));
DG_DEV void store8_f16x(void *p, int type, int64_t idx, floatx4 lo, floatx4 hi)
{
    if (type == T_F16)
        __builtin_nontemporal_store(half8{(_Float16)lo.x, (_Float16)lo.y, (_Float16)lo.z, (_Float16)lo.w,
                                          (_Float16)hi.x, (_Float16)hi.y, (_Float16)hi.z, (_Float16)hi.w},
                                    reinterpret_cast<half8 *>(reinterpret_cast<_Float16 *>(p) + idx));
    else
        __builtin_nontemporal_store(bf16x8v{(__bf16)lo.x, (__bf16)lo.y, (__bf16)lo.z, (__bf16)lo.w,
                                            (__bf16)hi.x, (__bf16)hi.y, (__bf16)hi.z, (__bf16)hi.w},
                                    reinterpret_cast<bf16x8v *>(reinterpret_cast<__bf16 *>(p) + idx));
}

// epi_store_f on four consecutive columns j .. j+3 (the same arithmetic per
// element), on values already loaded: d holds D's four values (used when D is
// read), b the bias's four values (used by the bias kinds).
DG_DEV void epi_out4_f(const EpiArgs &e, int64_t i, int64_t j, floatx4 acc, floatx4 d, floatx4 b)
{
    floatx4 v = e.alpha * acc;
    if (e.d_read) v += e.beta * d;
    if (e.kind == E_BIAS || e.kind == E_BIAS_GELU) v += b;
    if (e.kind == E_GELU || e.kind == E_BIAS_GELU)
        v = floatx4{gelu_erf(v.x), gelu_erf(v.y), gelu_erf(v.z), gelu_erf(v.w)};
    store4_f32(e.C, e.out_type, i * e.ldc + j, v);
}

// The bias's four values at columns j .. j+3 for the float epilogue (zeros when
// the kind has no bias).
DG_DEV floatx4 epi_bias4_f(const EpiArgs &e, int64_t j)
{
    if (e.kind == E_BIAS || e.kind == E_BIAS_GELU) return load4_f32(e.bias, e.bias_type, j);
    return floatx4{0.f, 0.f, 0.f, 0.f};
}

DG_DEV void epi_store4_f(const EpiArgs &e, int64_t i, int64_t j, floatx4 acc)
{
    const floatx4 d = e.d_read ? load4_f32(e.D, e.out_type, i * e.ldd + j) : floatx4{0.f, 0.f, 0.f, 0.f};
    epi_out4_f(e, i, j, acc, d, epi_bias4_f(e, j));
}

// epi_store_i on four consecutive columns j .. j+3 (the same arithmetic per
// element), on values already loaded: d holds D's four values (used when D is
// read), b the requantisation bias's four values (used when there is a bias).
DG_DEV void epi_out4_i(const EpiArgs &e, int64_t i, int64_t j, intx4 acc, intx4 d, floatx4 b)
{
    if (e.kind == E_RQ_I8 || e.kind == E_RQ_F16) {
        floatx4 v;
#pragma unroll
        for (int c = 0; c < 4; ++c) v[c] = __fmul_rn((float)acc[c], e.rq_scale);
        if (e.bias) {
#pragma unroll
            for (int c = 0; c < 4; ++c) v[c] = __fadd_rn(v[c], b[c]);
        }
        if (e.kind == E_RQ_I8) {
            i8x4v q;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                float r = __builtin_rintf(v[c]);
                r = r > 127.0f ? 127.0f : (r < -128.0f ? -128.0f : r);
                q[c] = (signed char)(int)r;
            }
            *reinterpret_cast<i8x4v *>(reinterpret_cast<int8_t *>(e.C) + i * e.ldc + j) = q;
        } else {
            *reinterpret_cast<half4v *>(reinterpret_cast<_Float16 *>(e.C) + i * e.ldc + j) =
                half4v{(_Float16)v.x, (_Float16)v.y, (_Float16)v.z, (_Float16)v.w};
        }
        return;
    }
    intx4 v;
#pragma unroll
    for (int c = 0; c < 4; ++c) v[c] = (int)((uint32_t)e.ialpha * (uint32_t)acc[c]);
    if (e.d_read) {
#pragma unroll
        for (int c = 0; c < 4; ++c) v[c] = (int)((uint32_t)v[c] + (uint32_t)e.ibeta * (uint32_t)d[c]);
    }
    __builtin_nontemporal_store(v, reinterpret_cast<intx4 *>(reinterpret_cast<int32_t *>(e.C) + i * e.ldc + j));
}

// The requantisation bias's four values at columns j .. j+3 (zeros without one).
DG_DEV floatx4 epi_bias4_i(const EpiArgs &e, int64_t j)
{
    if ((e.kind == E_RQ_I8 || e.kind == E_RQ_F16) && e.bias)
        return *reinterpret_cast<const floatx4 *>(reinterpret_cast<const float *>(e.bias) + j);
    return floatx4{0.f, 0.f, 0.f, 0.f};
}

DG_DEV void epi_store4_i(const EpiArgs &e, int64_t i, int64_t j, intx4 acc)
{
    const intx4 d = e.d_read ? *reinterpret_cast<const intx4 *>(reinterpret_cast<const int32_t *>(e.D) + i * e.ldd + j)
                             : intx4{0, 0, 0, 0};
    epi_out4_i(e, i, j, acc, d, epi_bias4_i(e, j));
}

// Linear workgroup id -> tile index, keeping each accelerator die (XCD) on a
// contiguous run of tiles.  Workgroups are dispatched round-robin over the 8
// XCDs, so workgroup w runs on XCD w % 8; the run of XCD x starts at
// x*q + min(x, r) for T = 8q + r tiles.  A bijection on [0, T).
DG_DEV int xcd_remap(int w, int T)
{
    const int q = T >> 3, r = T & 7;
    const int x = w & 7, i = w >> 3;
    return x * q + (x < r ? x : r) + i;
}

}  // namespace dg
