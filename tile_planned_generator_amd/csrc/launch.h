// launch.h - host entry points of the kernel sources (internal).
#pragma once
#include <hip/hip_runtime.h>

#include "dg_args.h"

namespace dg {

// Tiled MFMA GEMM; `id` indexes DG_TILED_CATALOGUE.
int tiled_kernel_count();
hipError_t launch_tiled(int id, const TiledArgs &a, int grid_x, int grid_y, hipStream_t s);

// Skinny VALU GEMM; `id` indexes DG_SKINNY_VALU_CATALOGUE.
int skinny_valu_count();
hipError_t launch_skinny_valu(int id, const SkinnyArgs &a, int grid_x, int grid_y, hipStream_t s);

// Skinny MFMA GEMM (M <= 16); `id` indexes DG_SKINNY_MFMA_CATALOGUE.
int skinny_mfma_count();
hipError_t launch_skinny_mfma(int id, const SkinnyArgs &a, int grid_x, int grid_y, hipStream_t s);

// Skinny e2m1 GEMM; `id` indexes DG_SKINNY_E2M1_CATALOGUE.
int skinny_e2m1_count();
hipError_t launch_skinny_e2m1(int id, const SkinnyArgs &a, int grid_x, int grid_y, hipStream_t s);

// MX quantiser: binary16 -> fp8 e4m3 codes and e8m0 block scales.
hipError_t launch_quant_mx(const QuantMxArgs &a, hipStream_t s);

// Split-K reduction and epilogue.
hipError_t launch_reduce(const ReduceArgs &a, hipStream_t s);

// pad_k: the K tail past the aligned part, as one more partial slice.
hipError_t launch_tail(const TailArgs &a, hipStream_t s);

// Static device scratch of dg_gemm_noalloc (DG_SCRATCH_BYTES per GPU):
// scratch_init looks up its address on `device` (once; the device is made
// current for the lookup and restored), scratch_ptr returns it (NULL before).
hipError_t scratch_init(int device);
void *scratch_ptr(int device);

// Hardware probe kernels (dg_probe): kind 0 stream read, 1 MFMA, 2 LDS banks.
hipError_t launch_probe(int kind, void *buf, size_t bytes, int param, void *out, int grid, hipStream_t s);

}  // namespace dg
