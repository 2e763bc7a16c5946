// dg_args.h - argument blocks shared by the host launchers and the kernels.
//
// Internal to the library: the C ABI in include/dg.h is the only public surface.
#pragma once
#include <stddef.h>
#include <stdint.h>

namespace dg {

// Operand paths of the tiled kernel and the skinny kernels.
// P_MX: fp8 e4m3 A x e2m1 B with e8m0 block scales (one per 32 k) on both,
// fed to the block-scaled MFMA as they are stored.
enum Path : int { P_F16 = 0, P_BF16 = 1, P_I8 = 2, P_E2M1 = 3, P_MX = 4 };

// Storage types of outputs, D and bias.
enum Elt : int { T_F16 = 0, T_BF16 = 1, T_F32 = 2, T_I32 = 3, T_I8 = 4 };

// Fused epilogue kinds (same numbering as dg_epi_kind).
enum EpiKind : int {
    E_NONE = 0, E_BIAS = 1, E_GELU = 2, E_BIAS_GELU = 3, E_RQ_I8 = 4, E_RQ_F16 = 5
};

// Everything the epilogue needs: alpha*acc + beta*D + bias, activation, the
// conversion to the output type and the store.
struct EpiArgs {
    void *C;
    const void *D;
    const void *bias;
    int64_t ldc, ldd;
    float alpha, beta;        // floating-point compute
    int32_t ialpha, ibeta;    // integer compute
    float rq_scale;           // requantise multiplier
    int kind;                 // EpiKind
    int out_type;             // Elt of C (and of D)
    int bias_type;            // Elt of bias
    int d_read;               // beta != 0
};

// Tiled MFMA GEMM.
struct TiledArgs {
    const void *A, *B, *scale;
    int64_t lda, ldb, ld_scale;   // elements (codes for e2m1); ld_scale: per group row of the
                                  // scales (e2m1: elements; MX: bytes)
    const void *scale_a;          // MX: A's e8m0 scales, group-major [K/32][ld_scale_a]
    int64_t ld_scale_a;           // MX: bytes between group rows of scale_a (a multiple of 4)
    int M, N, K;
    int split_k, k_slice;         // K slices; every slice but the last has k_slice
    int tiles_m, tiles_n, group_m;
    void *ws;                     // split partials [split][M][N] (fp32 or int32)
    EpiArgs epi;
    unsigned long long *clk;      // stage clock: 8 entries per workgroup, or null
    int64_t clk_wgs;              // workgroups the stage-clock buffer holds
};

// Skinny split-K streaming GEMM (small M).
struct SkinnyArgs {
    const void *A, *B, *scale;
    int64_t lda, ldb, ld_scale;
    int M, N, K;
    int split_k, k_slice;
    void *ws;                     // split partials [split][M][N] fp32
    EpiArgs epi;
};

// pad_k tail: ws[m][n] = sum over k in [k0, k1) of A[m][k] * B[k][n], one more
// partial slice (fp32, or int32 for int8) for the split-K reduction.
struct TailArgs {
    const void *A, *B;
    int64_t lda, ldb;
    int M, N, k0, k1;
    int path;                     // P_F16, P_BF16 or P_I8
    int b_kmajor;                 // 1: B stored N x K
    void *ws;                     // the slice [M][N]
};

// MX quantiser: binary16 X (M x K, ldx elements) -> fp8 e4m3 codes (ldq bytes)
// and one e8m0 scale per 32 values of a row, group-major (block g of row r at
// g * ld_scale + r).
struct QuantMxArgs {
    const void *X;
    void *codes, *scales;
    int64_t ldx, ldq, ld_scale;
    int M, K;
};

// Split-K reduction: out = epilogue(sum of ws[s] over the slices s).  `lanes`
// lanes share one output (a power of two, at most 16): lane t sums a contiguous
// run of slices in ascending order and the runs are combined in a fixed pattern.
struct ReduceArgs {
    const void *ws;
    int split_k, M, N;
    int is_int;
    int lanes;
    EpiArgs epi;
};

}  // namespace dg
