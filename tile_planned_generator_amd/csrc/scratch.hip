// scratch.hip - the library's static device scratch, for dg_gemm_noalloc:
// the split-K partial sums of callers that cannot allocate device memory.
//
// The array is a file-scope __device__ variable: every GPU the library runs
// on holds its own copy (DG_SCRATCH_BYTES) from the module's load until the
// process ends.  In host code its name is only a host-side stand-in, never a
// device address: its address on a device is looked up once, with that device
// current, by scratch_init (called from dg_create), and that address is what
// the kernels receive.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/dg.h"
#include "launch.h"

namespace dg {

static __device__ __align__(256) char scratch[DG_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_ptr[kMaxDevices];
}  // namespace

hipError_t scratch_init(int device)
{
    if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(g_mu);
    if (g_ptr[device]) return hipSuccess;
    int prev = -1;
    hipError_t e = hipGetDevice(&prev);
    if (e != hipSuccess) return e;
    if (prev != device && (e = hipSetDevice(device)) != hipSuccess) return e;
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (prev != device) {
        const hipError_t e2 = hipSetDevice(prev);
        if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    g_ptr[device] = ptr;
    return hipSuccess;
}

void *scratch_ptr(int device)
{
    if (device < 0 || device >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lk(g_mu);
    return g_ptr[device];
}

}  // namespace dg
