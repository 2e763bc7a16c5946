/*
 * dg.h - C ABI of the planned dense GEMM for AMD MI355X (gfx950).
 *
 *   C = act( alpha * (A . B) + beta * D + bias )
 *
 * Page citations use two keys:
 *   [overview]  the DeepGEMM overview article (lqnn.cn, mirrored at discosf.com)
 *   [generator] the DeepGEMM generator article (kwkr.cn)
 *
 * The operation is the GEMM whose kernels the pages generate: the
 * "alpha * C + beta * D" epilogue ([generator] section 3.2, step 3), a bias
 * vector added in the epilogue ([generator] section 2.2, third layer), a fused
 * GELU ([overview] section 6.1), 16-bit inputs accumulated in fp32 and cast to
 * the output type ([overview] section 3.5, second lesson), int8 accumulated in
 * int32 and converted with round-to-nearest ([overview] section 4.3), and 4-bit
 * e2m1 weights with fp16 activations ([overview] section 2.2, second layer).
 * The tile shape, the K schedule (a K step that may change along K) and the
 * K split are chosen by a host-side constraint planner ([generator] section 2.2,
 * first layer: shared-memory, register and occupancy inequalities and a
 * Pareto-optimal set of tile shapes; here re-derived for gfx950's LDS, VGPR/AGPR
 * budget and MFMA geometry).
 *
 * Conventions for every function:
 *   - Every call returns a dg_status.  On failure, dg_last_error() returns a
 *     message for the last failing call on the calling thread.  No C++
 *     exception crosses this interface.  Nothing fails silently: a missing
 *     operand is DG_ERR_INVALID_ARG (the pages' runtime fails silently when an
 *     operand is left unbound, [overview] section 5.1, problem 3; this one
 *     does not).
 *   - Device buffers (A, B, scales, D, C, bias, workspace) belong to the
 *     caller and must stay valid until the work enqueued on the stream has
 *     finished.  The library never allocates device memory, never copies
 *     between host and device and never synchronises: dg_gemm validates on
 *     the host, enqueues its kernels on `stream` and returns.
 *   - A handle is used by one thread at a time; distinct handles are
 *     independent.  A handle holds only host state: the device description,
 *     the plan cache.
 *   - Sizes and leading dimensions are in elements (for e2m1, in 4-bit codes).
 */
#ifndef DG_H
#define DG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct dg_handle_s *dg_handle_t;
typedef void *dg_stream_t; /* a hipStream_t; NULL is the null stream */

/* Status codes.  The pages' failures map as: "No valid candidate found after
 * pruning" -> DG_ERR_NO_CANDIDATE; "K dimension not aligned" -> DG_ERR_ALIGNMENT;
 * "conflicting compute units" -> DG_ERR_CONFLICT; the runtime's
 * DGMM_ERROR_INVALID_STATE (module/hardware mismatch) -> DG_ERR_INVALID_STATE
 * ([overview] sections 3.5 and 5.1). */
typedef enum {
    DG_OK = 0,
    DG_ERR_INVALID_ARG = 1,    /* null operand, negative size, bad enum      */
    DG_ERR_UNSUPPORTED = 2,    /* dtype / layout / epilogue combination       */
    DG_ERR_ALIGNMENT = 3,      /* K or a leading dimension or pointer alignment */
    DG_ERR_NO_CANDIDATE = 4,   /* every tile candidate violates a constraint  */
    DG_ERR_CONFLICT = 5,       /* options that cannot hold together           */
    DG_ERR_INVALID_STATE = 6,  /* offline/destroyed handle, wrong device      */
    DG_ERR_WORKSPACE = 7,      /* workspace missing or smaller than planned   */
    DG_ERR_HIP = 8,            /* a HIP runtime call or kernel launch failed  */
    DG_ERR_INTERNAL = 9
} dg_status;

/* DG_F8E4M3: OCP MX fp8 e4m3 (sign, 4-bit exponent with bias 7, 3-bit mantissa;
 * largest finite 448, codes 0x7f and 0xff NaN).  DG_E8M0: OCP MX block scale, an
 * unsigned byte c meaning 2^(c - 127) (255 is NaN). */
typedef enum { DG_F16 = 0, DG_BF16 = 1, DG_F32 = 2, DG_I8 = 3, DG_I32 = 4, DG_E2M1 = 5,
               DG_F8E4M3 = 6, DG_E8M0 = 7 } dg_dtype;

/* DG_ROW_MAJOR: for A, M x K with K contiguous; for B, K x N with N contiguous.
 * DG_COL_MAJOR: for B only, stored N x K with K contiguous (the e2m1 layout). */
typedef enum { DG_ROW_MAJOR = 0, DG_COL_MAJOR = 1 } dg_layout;

typedef enum {
    DG_EPI_NONE = 0,           /* v = alpha*acc + beta*D                         */
    DG_EPI_BIAS = 1,           /* v = alpha*acc + beta*D + bias[j]               */
    DG_EPI_GELU_ERF = 2,       /* GELU(alpha*acc + beta*D), erf form             */
    DG_EPI_BIAS_GELU_ERF = 3,  /* GELU(alpha*acc + beta*D + bias[j])             */
    DG_EPI_REQUANT_I8 = 4,     /* int path: clamp(rint(f32(acc)*scale + bias[j])) to int8 */
    DG_EPI_REQUANT_F16 = 5     /* int path: fp16(f32(acc)*scale + bias[j]), nearest-even  */
} dg_epi_kind;

typedef enum { DG_UNIT_AUTO = 0, DG_UNIT_MFMA = 1, DG_UNIT_VALU = 2 } dg_unit;
typedef enum { DG_PATH_AUTO = 0, DG_PATH_TILED = 1, DG_PATH_SKINNY = 2 } dg_path;

/* Precision triple plus the accumulator type ([overview] section 2.2, second
 * layer: a precision scheme {weight, activation, output} is declared, not
 * guessed).  Supported:
 *   a=F16  b=F16  c=F16|F32  compute=F32
 *   a=BF16 b=BF16 c=BF16|F32 compute=F32
 *   a=I8   b=I8   c=I32      compute=I32   (c=I8 / F16 with the requantise epilogues)
 *   a=F16  b=E2M1 c=F16|F32  compute=F32   (b_scale: one fp16 per group_k codes)
 *   a=F8E4M3 b=E2M1 c=F16|F32 compute=F32  (the MX path: e8m0 scales on both
 *                                           operands, dg_gemm_mx only; dg_plan
 *                                           plans it with group_k 32)
 * D, when read, has the type of C (I32 for the int path). */
typedef struct {
    int32_t a, b, c, compute; /* dg_dtype */
} dg_dtypes;

/* Leading dimensions in elements; 0 means tightly packed.  A: row-major only.
 * B: row-major (f16, bf16, i8) or column-major (f16, bf16, i8, and e2m1, where
 * it is the only layout).  C and D are row-major.  A, B rows (columns for a
 * column-major B) must start on 16-byte boundaries: base pointers 16-byte
 * aligned and lda, ldb multiples of 16 bytes.  Every row of A and B must be
 * readable up to its next 16-byte boundary (any allocation of whole rows of
 * lda / ldb elements is).  The tiled MFMA path addresses each operand with
 * 32-bit offsets: M*lda, K*ldb (row-major B) or N*ldb (column-major B) times
 * the element size must stay below 4 GiB (DG_ERR_UNSUPPORTED otherwise). */
typedef struct {
    int32_t a, b;             /* dg_layout */
    int64_t lda, ldb, ldc, ldd;
} dg_layouts;

/* Epilogue.  bias: device pointer to N elements of bias_type (F16, BF16 or F32;
 * F32 for the requantise kinds), required by the kinds that name it and
 * optional for the requantise kinds.  scale: the requantise multiplier. */
typedef struct {
    int32_t kind;             /* dg_epi_kind */
    int32_t bias_type;        /* dg_dtype */
    const void *bias;
    float scale;
} dg_epilogue;

/* Planner options ([overview] section 3.2: constraints such as use_hmma and
 * sm_mem_limit; section 5.3: use_hmma false for small GEMMs).  Zero-initialised
 * options mean "planner decides". */
typedef struct {
    int32_t force_m_tile, force_n_tile, force_k_tile; /* tiled path tile (0 = free);
                                 * force_n_tile alone also picks the streaming
                                 * kernels' columns per workgroup (VALU: 256, 512,
                                 * 1024 or 2048; MFMA: 512; e2m1: 16) */
    int32_t force_split_k;    /* number of K slices (0 = free)                      */
    int32_t force_path;       /* dg_path (DG_PATH_AUTO = 0: planner decides)         */
    int32_t unit;             /* dg_unit: MFMA (matrix cores) or VALU (vector FMA)  */
    int32_t lds_limit_bytes;  /* LDS budget per workgroup (0 = device maximum)      */
    float target_occupancy;   /* minimum waves per SIMD as a fraction of 8 (0 = 0.125) */
    int32_t pad_k;            /* 1: K need not be a multiple of the MFMA depth (16 for
                                 16-bit inputs, 32 for int8): the planned kernels take the
                                 aligned part of K and write partial sums, a tail kernel
                                 adds the last K % depth products as one more partial,
                                 and the split-K reduction applies the epilogue (the
                                 pages' padding-aware kernel for such K, [overview]
                                 section 3.5, third lesson; section 5.1, case B).
                                 Leading dimensions must still be 16-byte multiples;
                                 e2m1 is not supported (DG_ERR_UNSUPPORTED).  0: such a
                                 K is DG_ERR_ALIGNMENT. */
    int32_t force_waves;      /* waves per workgroup of the tiled path (0 = free)    */
    int32_t force_mfma;       /* MFMA output block of the tiled path: 32 (32x32) or 16
                                 (16x16; every path, eight-wave tiles) (0 = free);
                                 other values are DG_ERR_INVALID_ARG */
} dg_plan_opts;

/* Description of the device the planner plans for.  dg_create fills it from
 * hipGetDeviceProperties and, when the hardware probe's JSON description is
 * present, from that (dg_load_device_json); dg_default_device_desc gives the
 * MI355X table (the analogue of the pages' per-GPU hardware JSON, [generator]
 * section 3.2, step 1, whose rates come from micro-benchmarks run before
 * candidate generation, [overview] section 4.1, stage 1).  The measured
 * fields are 0 when unknown: the planner then uses the published figures. */
typedef struct {
    char arch[32];            /* "gfx950" */
    int32_t cu_count;         /* compute units (256)                    */
    int32_t xcd_count;        /* accelerator dies sharing the CUs (8)   */
    int32_t simd_per_cu;      /* 4                                      */
    int32_t wave_size;        /* 64                                     */
    int32_t lds_bytes_per_cu; /* 163840                                 */
    int32_t lds_bytes_per_wg; /* largest LDS allocation of one workgroup */
    int32_t vgpr_per_lane;    /* unified VGPR+AGPR file per SIMD lane (512) */
    int32_t max_waves_per_simd; /* 8                                    */
    double clock_ghz;         /* peak engine clock (2.4)                */
    double hbm_gbps;          /* HBM read bandwidth, GB/s (8000 published; the probe's
                                 streaming-read rate when measured)    */
    double l2_bytes_per_xcd;  /* L2 per die (4 MiB; probed: where re-reads stop hitting it) */
    double mall_bytes;        /* last-level (MALL) cache, all dies (256 MiB; probed)      */
    double mfma_tflops_f16;   /* sustained fp16 MFMA rate of back-to-back MFMAs on every
                                 SIMD, TFLOP/s (0: 4096 flop per clock per CU at clock_ghz);
                                 int8 and the fp8 block-scaled MFMA run at twice it */
    double launch_us;         /* an empty kernel launch, microseconds (0: 2.0)            */
    int32_t lds_conflict_stride_words; /* smallest word stride at which a wave's dword LDS
                                 reads are fully serialised: half the bank count (0: 32) */
    int32_t calibrated;       /* number of tiled variants with a measured efficiency
                                 (dg_load_device_json; output of dg_get_device_desc only) */
} dg_device_desc;

/* What the planner chose (the pages' "Solution": tile shape and the estimate
 * behind the choice, [generator] section 3.2, step 2). */
typedef struct {
    int32_t path;             /* dg_path */
    int32_t unit;             /* dg_unit */
    int32_t mfma_m, mfma_n, mfma_k;   /* MFMA instruction shape (0 on VALU) */
    int32_t m_tile, n_tile;   /* workgroup tile (skinny path: M rows x N columns) */
    int32_t k_main, n_main;   /* K schedule of the first K slice: n_main steps of k_main */
    int32_t k_tail, n_tail;   /* then n_tail steps of k_tail (the smaller tail step) */
    int32_t split_k;          /* K slices; partials reduced in a fixed order (runs of
                                 consecutive slices summed in ascending order, the runs
                                 combined in a fixed pattern): run-to-run identical */
    int32_t k_slice;          /* K length of every slice but the last */
    int32_t waves_per_wg;
    int32_t lds_bytes;        /* LDS per workgroup */
    int32_t vgpr_est, agpr_est;       /* registers per lane (estimate) */
    int32_t waves_per_simd;   /* occupancy the estimate allows */
    int32_t grid;             /* workgroups launched by the main kernel */
    int64_t workspace_bytes;  /* workspace dg_gemm needs (0 if none) */
    double est_us;            /* model estimate of the kernel time */
    double est_roof_fraction; /* roofline time / estimate */
    int32_t kernel_id;
    char kernel_name[64];
} dg_plan_info;

/* Create a handle for HIP device `hip_device`: queries it and checks that it is
 * a gfx950 (DG_ERR_UNSUPPORTED otherwise, DG_ERR_HIP if the query fails). */
dg_status dg_create(dg_handle_t *out, int hip_device);

/* Planner-only handle for a described device (no HIP call is made).  dg_gemm on
 * it returns DG_ERR_INVALID_STATE.  `desc` is copied. */
dg_status dg_create_offline(dg_handle_t *out, const dg_device_desc *desc);

/* The MI355X description used by dg_create_offline callers and as the fallback
 * for fields the HIP query does not report. */
dg_status dg_default_device_desc(dg_device_desc *out);

/* Release a handle (NULL is accepted). */
dg_status dg_destroy(dg_handle_t h);

/* Plan one problem: enumerate tile candidates, prune by the constraints, score
 * with a roofline model, keep the Pareto set and pick the fastest estimate
 * ([generator] section 2.2, first layer; [overview] section 4.1, stage 2).  The
 * plan is cached in the handle.  `opts` and `out` may be NULL.  Errors:
 * DG_ERR_INVALID_ARG, DG_ERR_UNSUPPORTED, DG_ERR_ALIGNMENT, DG_ERR_CONFLICT,
 * DG_ERR_NO_CANDIDATE. */
dg_status dg_plan(dg_handle_t h, int64_t M, int64_t N, int64_t K,
                  const dg_dtypes *dt, const dg_layouts *lay, int32_t group_k,
                  int32_t epi_kind, const dg_plan_opts *opts, dg_plan_info *out);

/* The Pareto-optimal candidates (estimated time, LDS bytes, registers), best
 * first; at most `cap` are written, *count receives how many exist. */
dg_status dg_plan_candidates(dg_handle_t h, int64_t M, int64_t N, int64_t K,
                             const dg_dtypes *dt, const dg_layouts *lay, int32_t group_k,
                             int32_t epi_kind, const dg_plan_opts *opts,
                             dg_plan_info *out, int32_t cap, int32_t *count);

/* Plan for every K in [K_min, K_max] at once: the pages' range constraint
 * (K_min / K_max in the declaration instead of one K, so that one compact
 * kernel serves every layer whose K falls in the range, [overview] section
 * 5.3, the second stage of the service case).  K is sampled at both ends and at the
 * doublings between them; each compiled kernel variant of the problem's path
 * (tile, wave grid, K step and MFMA block, or the streaming path) is planned
 * at every sample, and
 * the variant whose largest ratio of estimated time to the best plan of that K
 * is smallest wins (ties: fewer LDS bytes, then fewer registers, then
 * catalogue order).
 *   opts         as for dg_plan, with tile, K step, waves, MFMA block and
 *                path left free
 *   range_opts   out: the options that pin the chosen variant; pass them to
 *                dg_gemm (or dg_plan) for any K of the range, where the planner
 *                still chooses the K split and schedule of that K
 *   out          nullable: the plan of the chosen variant at K_max
 *   worst_ratio  nullable: the chosen variant's largest estimated-time ratio
 * Errors: DG_ERR_INVALID_STATE, DG_ERR_INVALID_ARG (range_opts NULL, K_min < 0
 * or K_min > K_max), DG_ERR_CONFLICT (a forced tile, K step, wave count, MFMA
 * block or path), and
 * what dg_plan returns at either end of the range (DG_ERR_ALIGNMENT for an
 * unaligned end without pad_k); DG_ERR_NO_CANDIDATE when no variant is valid
 * for every sample. */
dg_status dg_plan_range(dg_handle_t h, int64_t M, int64_t N, int64_t K_min, int64_t K_max,
                        const dg_dtypes *dt, const dg_layouts *lay, int32_t group_k,
                        int32_t epi_kind, const dg_plan_opts *opts, dg_plan_opts *range_opts,
                        dg_plan_info *out, double *worst_ratio);

/* Enqueue C = act(alpha*(A.B) + beta*D + bias) on `stream` (the kernel argument
 * list of the pages' launch, A, B, C, alpha, beta, m, n, k, [generator] section
 * 3.2, step 4, plus the precision, layout and epilogue description).
 *   A       device, M x K (lda)
 *   B       device, K x N row-major (ldb) or N x K column-major (ldb); e2m1: two
 *           codes per byte, even k in the low nibble, N x K column-major
 *   b_scale e2m1 only: device fp16, group-major [K/group_k][ldsc] with ldsc = N
 *           rounded up to even (scale of group g, column n at g * ldsc + n: a
 *           K step's scales for consecutive columns are contiguous); 4-byte
 *           aligned
 *   group_k e2m1 only: 32
 *   D       device, M x N (ldd); read only when *beta != 0, may be NULL otherwise
 *   C       device, M x N (ldc)
 *   alpha, beta  host pointers to compute-type scalars (float for F32 compute,
 *           int32_t for I32 compute; the requantise kinds need alpha == 1 and
 *           beta == 0 and use epi->scale)
 *   epi     NULL means DG_EPI_NONE
 *   opts    the planner options (NULL: planner decides)
 *   workspace, workspace_bytes   device scratch of at least the planned
 *           workspace_bytes (may be NULL when the plan needs none)
 * Returns after enqueueing; errors in the arguments are reported before
 * anything is enqueued. */
dg_status dg_gemm(dg_handle_t h, int64_t M, int64_t N, int64_t K,
                  const dg_dtypes *dt, const dg_layouts *lay,
                  const void *A, const void *B, const void *b_scale, int32_t group_k,
                  const void *D, void *C, const void *alpha, const void *beta,
                  const dg_epilogue *epi, const dg_plan_opts *opts,
                  void *workspace, size_t workspace_bytes, dg_stream_t stream);

/* dg_gemm for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * arguments without the workspace.  The split-K partial sums go to the
 * library's static device scratch instead, DG_SCRATCH_BYTES per GPU (a
 * file-scope device array: each GPU the library runs on holds it from the
 * library's load until the process ends; its address on a device is taken by
 * dg_create).  The planner only considers plans whose partial sums fit it;
 * a forced K split (or a pad_k plan) needing more is DG_ERR_WORKSPACE, before
 * anything is enqueued.  Nothing is allocated, copied or synchronised.
 * Every call on a GPU shares that GPU's scratch, which keeps the last call's
 * partial sums (every K slice overwrites its whole partial, so nothing needs
 * clearing): calls that overlap on one GPU (concurrent streams, several
 * threads) race, and must be ordered by the caller.
 * Errors: as dg_gemm; DG_ERR_WORKSPACE when no plan fits the scratch. */
#define DG_SCRATCH_BYTES (32u << 20)
dg_status dg_gemm_noalloc(dg_handle_t h, int64_t M, int64_t N, int64_t K,
                          const dg_dtypes *dt, const dg_layouts *lay,
                          const void *A, const void *B, const void *b_scale, int32_t group_k,
                          const void *D, void *C, const void *alpha, const void *beta,
                          const dg_epilogue *epi, const dg_plan_opts *opts, dg_stream_t stream);

/* MX block-scaled GEMM: the 4-bit weight scheme of the pages (e2m1 weights with
 * a scale per group of 32 along K, [overview] section 2.2, second layer; the
 * in-register weight unpack of section 4.3) with the activations quantised to
 * fp8 as well, so both operands go to gfx950's block-scaled MFMA
 * (v_mfma_scale_f32_32x32x64_f8f6f4) without a decode step.  The element and
 * scale formats are those of the OCP Microscaling (MX) v1.0 specification:
 *   C[i][j] = act( alpha * sum_k a[i][k] * w[k][j] + bias[j] )
 *   a[i][k] = e4m3(A[i][k]) * 2^(a_scale[k/32][i] - 127)
 *   w[k][j] = e2m1(B[j][k]) * 2^(b_scale[k/32][j] - 127)
 * accumulated in fp32 (products and block sums inside the MFMA, then fp32
 * additions along K), rounded once to C's type.
 *   A          device, fp8 e4m3 codes, M x K row-major, lda bytes (0: K); 16-byte
 *              aligned, lda a multiple of 16
 *   a_scale    device, e8m0 codes, group-major [K/32][lda_scale] (the scale of
 *              row i, block g at g * lda_scale + i: a K step's scales for
 *              consecutive rows are contiguous), lda_scale >= M (0: M rounded up
 *              to a multiple of 4); 4-byte aligned, lda_scale a multiple of 4
 *   B          device, e2m1 codes N x K (K contiguous), two per byte with even k
 *              in the low nibble, ldb in codes (0: K, a multiple of 32); 16-byte
 *              aligned
 *   b_scale    device, e8m0 codes, group-major [K/32][ldb_scale] (column n,
 *              block g at g * ldb_scale + n), ldb_scale >= N (0: N rounded up to
 *              a multiple of 4); as a_scale
 *   C          device, M x N row-major, ldc elements (0: N), c_type F16 or F32
 *   alpha      the product's multiplier
 *   epi        NULL or DG_EPI_NONE / BIAS / GELU_ERF / BIAS_GELU_ERF (bias F16,
 *              BF16 or F32); no beta * D term
 *   opts, workspace, workspace_bytes, stream   as for dg_gemm
 * K must be a multiple of 64 (DG_ERR_ALIGNMENT; pad_k is DG_ERR_UNSUPPORTED).
 * Returns after enqueueing; errors are reported before anything is enqueued:
 * DG_ERR_INVALID_STATE, DG_ERR_INVALID_ARG, DG_ERR_UNSUPPORTED, DG_ERR_ALIGNMENT,
 * DG_ERR_NO_CANDIDATE, DG_ERR_WORKSPACE, DG_ERR_HIP. */
dg_status dg_gemm_mx(dg_handle_t h, int64_t M, int64_t N, int64_t K,
                     const void *A, int64_t lda, const void *a_scale, int64_t lda_scale,
                     const void *B, int64_t ldb, const void *b_scale, int64_t ldb_scale,
                     void *C, int32_t c_type, int64_t ldc, float alpha,
                     const dg_epilogue *epi, const dg_plan_opts *opts,
                     void *workspace, size_t workspace_bytes, dg_stream_t stream);

/* MX quantiser for the activation operand of dg_gemm_mx: binary16 X -> fp8 e4m3
 * codes and one e8m0 scale per 32 consecutive values of a row (the OCP MX v1.0
 * conversion).  Per block: amax = max |x|; e = floor(log2 amax) - 8 (8 is the
 * exponent of e4m3's largest normal); scale code e + 127 (0 when amax is 0);
 * code = e4m3(x * 2^-e), nearest even, magnitudes above 448 saturating to 448.
 * A block holding an infinity or a NaN gets scale code 255 and codes 0x7f.
 *   X        device binary16, M x K row-major, ldx elements (0: K); 16-byte
 *            aligned rows
 *   codes    device, M x K bytes, ldq bytes per row (0: K); 16-byte aligned rows
 *   scales   device, group-major [K/32][ld_scale] bytes (block g of row i at
 *            g * ld_scale + i: the layout dg_gemm_mx takes), ld_scale >= M (0: M)
 * K must be a multiple of 32 (DG_ERR_ALIGNMENT).  Enqueues one kernel on
 * `stream`.  Errors: DG_ERR_INVALID_STATE, DG_ERR_INVALID_ARG,
 * DG_ERR_UNSUPPORTED, DG_ERR_ALIGNMENT, DG_ERR_HIP. */
dg_status dg_quant_mx(dg_handle_t h, int64_t M, int64_t K, const void *X, int64_t ldx,
                      void *codes, int64_t ldq, void *scales, int64_t ld_scale, dg_stream_t stream);

/* Stage clock: the analogue of the generator's profile option, which reads the
 * clock inside the generated kernel and reports the cycles of each kernel stage
 * ([generator] section 3.2, the practical notes after the launch code).
 * While `buf` is set, every tiled-path launch through `h` has each workgroup w
 * (w = blockIdx.y * gridDim.x + blockIdx.x, for w < entries / 8) write 8
 * uint64 entries at buf[8w .. 8w+7]:
 *   0 kernel entry, 1 K-loop start, 2 K-loop end, 3 epilogue end (stores issued)
 *     - values of the s_memtime counter read by the workgroup's first wave (each
 *     die counts on its own, so only stamps from one die compare);
 *   4 HW_ID register (CU, shader array, shader engine) in bits 0-31, and in
 *     bits 32-63 the low 32 bits of the s_memrealtime counter (a constant
 *     100 MHz clock) at K-loop start;
 *   5 XCC_ID (die) in bits 0-31, and in bits 32-63 the low 32 bits of
 *     s_memrealtime at K-loop end (so entry 2 - entry 1 over the real-time
 *     difference is the rate s_memtime ticks at during the K loop);
 *   6 K steps of the workgroup's slice, 7 blockIdx.x | blockIdx.y << 32.
 *   h        a live device handle
 *   buf      device memory owned by the caller, NULL to switch the clock off
 *   entries  uint64 entries buf holds (>= 0); workgroups past entries / 8 write
 *            nothing
 * Skinny-path and reduce launches write nothing.  The setting belongs to the
 * handle: launches on several threads through one handle share it.  Errors:
 * DG_ERR_INVALID_STATE (handle NULL, destroyed or offline), DG_ERR_INVALID_ARG
 * (entries < 0, or buf NULL with entries > 0). */
dg_status dg_set_stage_clock(dg_handle_t h, uint64_t *buf, int64_t entries);

/* Hardware probe: the measured counterpart of dg_device_desc, the analogue of
 * the pages' hardware query that feeds candidate generation ([overview]
 * section 4.1, stage 1; [generator] section 3.2, step 1).  dg_probe enqueues
 * one probe kernel on `stream`; the caller times it and derives the rate
 * (tile_planned_generator_amd/probe.py writes the results as a JSON device
 * description).
 *   DG_PROBE_STREAM  reads `bytes` (a multiple of 16) of device memory `buf`
 *                    with 16-byte non-temporal loads (param bit 0 set: plain,
 *                    cached loads) on `grid` workgroups of 256 threads, each a
 *                    contiguous share, param >> 1 times (0: once; at most
 *                    4096); `out`: device uint32[grid] (a checksum)
 *   DG_PROBE_MFMA    `grid` workgroups of 4 waves, each wave `param` rounds of
 *                    8 independent 32x32x16 fp16 MFMAs (2*32*32*16 flops each);
 *                    `out`: device float[grid]
 *   DG_PROBE_LDS     one wave, 1024 dword LDS reads with lane l at word
 *                    l * param (1 <= param <= 16384); `out`: device uint64[2],
 *                    out[0] = s_memtime ticks of the reads
 *   DG_PROBE_MFMA_DATA  the clock the MFMAs hold on given data: `grid`
 *                    workgroups of 8 waves (two per SIMD), each wave param >> 3
 *                    (>= 1) rounds of 8 independent int8 32x32x32 MFMAs on
 *                    operands read once from `buf` (`bytes`, a multiple of 16,
 *                    indexed modulo its size).  param & 7 is the mode: 0 one
 *                    operand pair for every MFMA; 1 eight pairs, a different
 *                    one for each MFMA of a round; 2 as 1 plus LDS reads of
 *                    buf's data at 0.75 KB per MFMA (the tiled kernel's
 *                    fragment traffic); 3 as 1 with A zero; 4 as 2 with the LDS
 *                    holding zeros; 5 the LDS reads alone.  `out`: device
 *                    uint64[3 * grid]: per workgroup the s_memtime ticks (the
 *                    shader clock) and the 100 MHz s_memrealtime ticks of its
 *                    first wave from entry to exit, and a checksum
 * Errors: DG_ERR_INVALID_STATE (handle NULL, destroyed or offline; wrong current
 * device), DG_ERR_INVALID_ARG (NULL out, NULL buf for the stream probe, bad
 * size, grid or param), DG_ERR_HIP (launch failure). */
typedef enum { DG_PROBE_STREAM = 0, DG_PROBE_MFMA = 1, DG_PROBE_LDS = 2, DG_PROBE_MFMA_DATA = 3 } dg_probe_kind;
dg_status dg_probe(dg_handle_t h, int32_t kind, const void *buf, size_t bytes, int32_t param, void *out,
                   int32_t grid, dg_stream_t stream);

/* Replace the description a handle plans with (for instance one measured by the
 * probe), and drop its cached plans; measured variant efficiencies loaded
 * earlier stay.  Errors: DG_ERR_INVALID_STATE (handle NULL or destroyed),
 * DG_ERR_INVALID_ARG (desc NULL or a non-positive field, as for
 * dg_create_offline). */
dg_status dg_set_device_desc(dg_handle_t h, const dg_device_desc *desc);

/* Load a device description written by the hardware probe
 * (tile_planned_generator_amd/probe.py): a JSON object whose "desc" object holds
 * dg_device_desc fields by name, whose "measured" object holds the probed rates
 * (hbm_gbps, mfma_tflops_f16, launch_us, lds_conflict_stride_words, l2_bytes_per_xcd,
 * mall_bytes), whose "tiled_efficiency" object maps tiled kernel names (as in
 * dg_plan_info.kernel_name) to the fraction of the probed MFMA rate the variant
 * sustains per K step, and whose "tiled_round_us" object maps them to the fixed
 * time of one round of its workgroups (entry, epilogue, launch share), both
 * fitted from timings at two K lengths of each path's 4096 x 4096 problem on
 * operands not in the caches.  The planner then scores with these numbers
 * instead of its built-in fallbacks, and cached plans are dropped.  dg_create loads <library directory>/devices/<arch>.json by
 * itself when it exists and describes the device (the environment variable
 * DG_DEVICE_JSON names another file; set to an empty string it disables this).
 * Errors: DG_ERR_INVALID_STATE (handle), DG_ERR_INVALID_ARG (path NULL,
 * unreadable, not such a JSON object, or a field out of range),
 * DG_ERR_UNSUPPORTED (a device handle and a description of another
 * architecture or CU count). */
dg_status dg_load_device_json(dg_handle_t h, const char *path);

/* The description a handle plans with (after dg_create's own loading of the
 * probe's JSON, dg_load_device_json or dg_set_device_desc).  Errors:
 * DG_ERR_INVALID_STATE, DG_ERR_INVALID_ARG (out NULL). */
dg_status dg_get_device_desc(dg_handle_t h, dg_device_desc *out);

/* Thread-local message of the last failing call on this thread ("" if none). */
const char *dg_last_error(void);

/* Name of a status code. */
const char *dg_status_str(dg_status s);

#ifdef __cplusplus
}
#endif
#endif /* DG_H */
