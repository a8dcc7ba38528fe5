// The allocation-free variant of fq_linear keeps its workspace (the
// activation codes and per-token scales that pass from the prologue to the
// GEMM) in a fixed device array of this library instead of a caller buffer.
//
// `scratch` is a file-scope device array; each GPU the library runs on holds
// its own copy until the process ends.  In host code its name is only a
// host-side stand-in, never a device address: the address of a device's copy
// is taken once per device, with that device current, by hipGetSymbolAddress
// during the device's set-up (prepare_device), and only that address is ever
// passed to kernels.
#include <hip/hip_runtime.h>

#include "fq_internal.h"

namespace fq {
namespace {

static __device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

}  // namespace

hipError_t init_scratch_device(DeviceInfo& d) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    d.scratch = p;
    return hipSuccess;
}

}  // namespace fq
