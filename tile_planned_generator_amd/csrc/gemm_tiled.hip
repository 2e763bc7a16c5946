// gemm_tiled.hip - launcher of the tiled MFMA GEMM variants (the kernels are
// instantiated per operand path in gemm_tiled_{f16,bf16,i8,e2m1,mx}.hip).
#include <hip/hip_runtime.h>

#include "catalogue.h"
#include "launch.h"

namespace dg {

void *tiled_kernel_ptr_f16(int id);
void *tiled_kernel_ptr_bf16(int id);
void *tiled_kernel_ptr_i8(int id);
void *tiled_kernel_ptr_e2m1(int id);
void *tiled_kernel_ptr_mx(int id);

static const TiledShape k_shapes[] = {
#define DG_TS(path, kmaj, bm, bn, wm, wn, kr, ms) {path, kmaj, bm, bn, wm, wn, kr, ms},
    DG_TILED_CATALOGUE(DG_TS)
#undef DG_TS
};

int tiled_kernel_count() { return (int)(sizeof(k_shapes) / sizeof(k_shapes[0])); }

hipError_t launch_tiled(int id, const TiledArgs &a, int grid_x, int grid_y, hipStream_t s)
{
    if (id < 0 || id >= tiled_kernel_count()) return hipErrorInvalidValue;
    void *fn = nullptr;
    switch (k_shapes[id].path) {
    case P_F16: fn = tiled_kernel_ptr_f16(id); break;
    case P_BF16: fn = tiled_kernel_ptr_bf16(id); break;
    case P_I8: fn = tiled_kernel_ptr_i8(id); break;
    case P_E2M1: fn = tiled_kernel_ptr_e2m1(id); break;
    default: fn = tiled_kernel_ptr_mx(id); break;
    }
    if (!fn) return hipErrorInvalidDeviceFunction;
    TiledArgs arg = a;
    void *args[] = {&arg};
    const int threads = k_shapes[id].wm * k_shapes[id].wn * 64;
    hipError_t e = hipLaunchKernel(fn, dim3(grid_x, grid_y, 1), dim3(threads, 1, 1), args, 0, s);
    if (e != hipSuccess) return e;
    return hipGetLastError();
}

}  // namespace dg
