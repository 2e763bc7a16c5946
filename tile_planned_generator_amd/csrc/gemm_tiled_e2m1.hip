// gemm_tiled_e2m1.hip - instantiates the tiled kernel variants of the e2m1 path.
#include "gemm_tiled.h"

namespace dg {

template <int PATH, int KMAJ, int BM, int BN, int WM, int WN, int KR, int MS>
static void *pick_e2m1()
{
    if constexpr (PATH == P_E2M1)
        return reinterpret_cast<void *>(gemm_tiled_kernel<PATH, KMAJ, BM, BN, WM, WN, KR, MS>);
    else
        return nullptr;
}

#define DG_PICK(path, kmaj, bm, bn, wm, wn, kr, ms) pick_e2m1<path, kmaj, bm, bn, wm, wn, kr, ms>(),

// Kernel of catalogue entry id if it belongs to this path, else NULL.
void *tiled_kernel_ptr_e2m1(int id)
{
    static void *const table[] = {DG_TILED_CATALOGUE(DG_PICK)};
    const int n = (int)(sizeof(table) / sizeof(table[0]));
    return (id >= 0 && id < n) ? table[id] : nullptr;
}

}  // namespace dg
