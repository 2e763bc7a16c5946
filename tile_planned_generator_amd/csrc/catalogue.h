// catalogue.h - the compiled kernel variants the planner chooses among.
//
// Plain C++ (no HIP): included by the planner, which runs on any host, and by
// the kernel sources, which instantiate exactly these variants.  The pages'
// planner searches tile shape x layout x granularity ([overview] DeepGEMM
// article, section 4.1, stage 2); on gfx950 the tile shapes are multiples of
// the 32x32 MFMA output block, the granularity is the wave grid, and the MFMA
// block (32x32 or 16x16) is one more dimension.
#pragma once

namespace dg {

// Tiled MFMA GEMM: X(path, b_kmajor, BM, BN, WM, WN, KR, MS)
//   path      P_F16 / P_BF16 / P_I8 / P_E2M1 / P_MX
//   b_kmajor  1: B stored N x K (K contiguous); 0: K x N (N contiguous)
//   BM x BN   workgroup tile; WM x WN wave grid (each wave BM/WM x BN/WN)
//   KR        64-byte K regions per K step: the K step (K_tile) is KR x 32 k
//             (16-bit), KR x 64 k (int8); e2m1 and MX take KR = 1
//   MS        MFMA output block: 32 (32x32) or 16 (16x16)
#define DG_TILE_SHAPES(X, path, kmaj)  \
    X(path, kmaj, 128, 256, 2, 2, 1, 32)   \
    X(path, kmaj, 256, 256, 2, 4, 1, 32)   \
    X(path, kmaj, 256, 128, 2, 2, 1, 32)   \
    X(path, kmaj, 128, 128, 2, 2, 1, 32)   \
    X(path, kmaj, 64, 64, 2, 2, 1, 32)
// The double K step (two regions per LDS stage, four MFMA substeps per
// barrier), four-wave tiles only.
#define DG_TILE_SHAPES_K2(X, path, kmaj) \
    X(path, kmaj, 256, 256, 2, 2, 2, 32)     \
    X(path, kmaj, 128, 256, 2, 2, 2, 32)     \
    X(path, kmaj, 256, 128, 2, 2, 2, 32)     \
    X(path, kmaj, 128, 128, 2, 2, 2, 32)     \
    X(path, kmaj, 64, 64, 2, 2, 2, 32)
// 16x16 MFMAs (one per 64-byte K region and 16x16 block), the eight-wave tile.
#define DG_TILE_SHAPES_M16(X, path, kmaj) X(path, kmaj, 256, 256, 2, 4, 1, 16)

#define DG_TILED_CATALOGUE(X)          \
    DG_TILE_SHAPES(X, P_F16, 0)        \
    DG_TILE_SHAPES(X, P_F16, 1)        \
    DG_TILE_SHAPES(X, P_BF16, 0)       \
    DG_TILE_SHAPES(X, P_BF16, 1)       \
    DG_TILE_SHAPES(X, P_I8, 0)         \
    DG_TILE_SHAPES(X, P_I8, 1)         \
    DG_TILE_SHAPES(X, P_E2M1, 1)       \
    DG_TILE_SHAPES(X, P_MX, 1)         \
    DG_TILE_SHAPES_K2(X, P_F16, 0)     \
    DG_TILE_SHAPES_K2(X, P_F16, 1)     \
    DG_TILE_SHAPES_K2(X, P_BF16, 0)    \
    DG_TILE_SHAPES_K2(X, P_BF16, 1)    \
    DG_TILE_SHAPES_K2(X, P_I8, 0)      \
    DG_TILE_SHAPES_K2(X, P_I8, 1)      \
    DG_TILE_SHAPES_M16(X, P_F16, 0)    \
    DG_TILE_SHAPES_M16(X, P_F16, 1)    \
    DG_TILE_SHAPES_M16(X, P_BF16, 0)   \
    DG_TILE_SHAPES_M16(X, P_BF16, 1)   \
    DG_TILE_SHAPES_M16(X, P_I8, 0)     \
    DG_TILE_SHAPES_M16(X, P_I8, 1)     \
    DG_TILE_SHAPES_M16(X, P_E2M1, 1)   \
    DG_TILE_SHAPES_M16(X, P_MX, 1)

// Skinny VALU streaming GEMM over a row-major 16-bit B:
// X(path, MR, LPR): up to MR rows of A; LPR lanes span one row of B (8 columns each).
#define DG_SKINNY_VALU_MR(X, path, lpr) X(path, 1, lpr) X(path, 2, lpr) X(path, 4, lpr) X(path, 8, lpr)
#define DG_SKINNY_VALU_CATALOGUE(X)        \
    DG_SKINNY_VALU_MR(X, P_F16, 64)        \
    DG_SKINNY_VALU_MR(X, P_F16, 32)        \
    DG_SKINNY_VALU_MR(X, P_F16, 16)        \
    DG_SKINNY_VALU_MR(X, P_F16, 8)         \
    DG_SKINNY_VALU_MR(X, P_BF16, 64)       \
    DG_SKINNY_VALU_MR(X, P_BF16, 32)       \
    DG_SKINNY_VALU_MR(X, P_BF16, 16)       \
    DG_SKINNY_VALU_MR(X, P_BF16, 8)

// Skinny MFMA streaming GEMM (M <= 16) over a row-major 16-bit B: X(path)
#define DG_SKINNY_MFMA_CATALOGUE(X) X(P_F16) X(P_BF16)

// Skinny e2m1 GEMM (B codes N x K, K contiguous): X(MR)
#define DG_SKINNY_E2M1_CATALOGUE(X) X(1) X(2) X(4) X(8)

// Resource facts of the variants, used by the planner's constraints.
struct TiledShape {
    int path, b_kmajor, bm, bn, wm, wn, kr, ms;   // ms: MFMA block edge (32 or 16)
};

// Fewest direct-to-LDS loads any wave issues per stage when load i of an
// operand goes to wave i % nw (the scale loads counted from the last wave down).
constexpr int tiled_min_loads_per_wave(int a_nl, int b_nl, int s_nl, int nw)
{
    int m = 1 << 30;
    for (int w = 0; w < nw; ++w) {
        const int ws = nw - 1 - w;
        const int c = a_nl / nw + (w < a_nl % nw) + b_nl / nw + (w < b_nl % nw) + s_nl / nw +
                      (ws < s_nl % nw);
        m = c < m ? c : m;
    }
    return m;
}

// k elements per 64-byte K region (two MFMA substeps; a K step holds KR
// regions) and per MFMA.  MX: one 32x32x64 block-scaled MFMA per substep, so
// its one-region step is 128 k (two 64-byte rows of fp8 A per row of the tile).
constexpr int tiled_bk_elems(int path) { return path == 4 /*P_MX*/ ? 128 : (path == 2 /*P_I8*/ ? 64 : 32); }
constexpr int tiled_ksub(int path) { return path == 4 /*P_MX*/ ? 64 : (path == 2 /*P_I8*/ ? 32 : 16); }

// Sustained fraction of the published MFMA rate one K step of a tiled variant
// reaches on MI355X, measured with every variant forced on the 4096^3 and
// 2048x2048x8192 workloads (fp16; int8 and e2m1 relative to it).  It folds in
// what a peak-rate model leaves out: the engine clock under MFMA load (about
// 1.9-2.0 GHz, not 2.4), the LDS-bound fragment reads and the barriers.
constexpr double tiled_step_efficiency(int path, int bm, int bn, int waves, int kr = 1)
{
    (void)kr;
    const double base = waves == 8 ? 0.48
                      : bm * bn >= 256 * 128 ? 0.40
                      : bm * bn >= 128 * 128 ? 0.30 : 0.15;
    return base * (path == 2 /*P_I8*/ ? 0.95 : (path == 3 /*P_E2M1*/ ? 0.87 : 1.0));   // MX: as fp16
}

// LDS bytes of one stage (one K step) of a tiled variant.  A and a
// K-contiguous B take 64 bytes per row (per column of B), a row-major B 64 bytes
// per column (BN columns of a 32-k or 64-k step); e2m1 B takes 16 bytes of codes
// per column plus the step's fp16 scales (whole 256-byte loads).  MX: two 64-byte rows of fp8 A per tile
// row, 64 bytes of e2m1 codes per column, and 2 KB of e8m0 scales (a 256-byte
// chunk per operand and group of the step).
constexpr int tiled_stage_bytes(int path, int bm, int bn, int kr = 1)
{
    return path == 4 ? bm * 128 + bn * 64 + 2304
         : (path == 3 ? bm * 64 + bn * 16 + (bn * 2 + 255) / 256 * 256 : kr * (bm * 64 + bn * 64));
}
// LDS stages: five for the eight-wave variants when they fit gfx950's 160 KB
// (the loads of a stage are then issued a phase later, in the MFMA phase, with
// the same lookahead), four otherwise; MX stages and double K steps are
// larger: as many as fit, at most four (at least two for a double K step,
// three for MX).
constexpr int tiled_nbuf(int path, int bm, int bn, int wm, int wn, int kr = 1)
{
    return path == 4 ? (4 * tiled_stage_bytes(path, bm, bn) <= 163840 ? 4 : 3)
         : kr > 1   ? (4 * tiled_stage_bytes(path, bm, bn, kr) <= 163840
                           ? 4
                           : (3 * tiled_stage_bytes(path, bm, bn, kr) <= 163840 ? 3 : 2))
                    : (wm * wn == 8 && 5 * tiled_stage_bytes(path, bm, bn) <= 163840 ? 5 : 4);
}
// The epilogue reuses the LDS to stage 32 rows of every wave's accumulators
// (4-byte values, rows padded by 4): the allocation is the larger of the two.
constexpr int tiled_lds_bytes(int path, int bm, int bn, int wm, int wn, int kr = 1)
{
    return tiled_nbuf(path, bm, bn, wm, wn, kr) * tiled_stage_bytes(path, bm, bn, kr) >
                   wm * wn * 32 * (bn / wn + 4) * 4
               ? tiled_nbuf(path, bm, bn, wm, wn, kr) * tiled_stage_bytes(path, bm, bn, kr)
               : wm * wn * 32 * (bn / wn + 4) * 4;
}

}  // namespace dg
