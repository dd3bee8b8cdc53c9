// Device-memory placement helpers (dopt_vmm.h): thin wrappers over the HIP
// virtual-memory API, with the library's error convention.
#include <hip/hip_runtime.h>

#include <cstring>
#include <string>

#include "dopt_vmm.h"
#include "internal.h"

using namespace dopt;

namespace {

int hip_fail(hipError_t e, const char *what) {
    return fail(DOPT_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

hipMemAllocationProp device_prop(int32_t device) {
    hipMemAllocationProp p;
    std::memset(&p, 0, sizeof p);
    p.type = hipMemAllocationTypePinned;
    p.location.type = hipMemLocationTypeDevice;
    p.location.id = device;
    return p;
}

void *as_ptr(uint64_t v) { return reinterpret_cast<void *>(static_cast<uintptr_t>(v)); }

}  // namespace

extern "C" {

int dopt_vmm_granularity(int32_t device, size_t *out) {
    if (!out) return fail(DOPT_ERR_INVALID, "null output");
    hipMemAllocationProp p = device_prop(device);
    hipError_t e = hipMemGetAllocationGranularity(out, &p, hipMemAllocationGranularityRecommended);
    return e == hipSuccess ? DOPT_OK : hip_fail(e, "hipMemGetAllocationGranularity");
}

int dopt_vmm_reserve(size_t bytes, size_t align, uint64_t *va) {
    if (!va || bytes == 0) return fail(DOPT_ERR_INVALID, "null output or zero size");
    void *p = nullptr;
    hipError_t e = hipMemAddressReserve(&p, bytes, align, nullptr, 0);
    if (e != hipSuccess) return hip_fail(e, "hipMemAddressReserve");
    *va = static_cast<uint64_t>(reinterpret_cast<uintptr_t>(p));
    return DOPT_OK;
}

int dopt_vmm_free(uint64_t va, size_t bytes) {
    hipError_t e = hipMemAddressFree(as_ptr(va), bytes);
    return e == hipSuccess ? DOPT_OK : hip_fail(e, "hipMemAddressFree");
}

int dopt_vmm_create(int32_t device, size_t bytes, uint64_t *handle) {
    if (!handle || bytes == 0) return fail(DOPT_ERR_INVALID, "null output or zero size");
    hipMemAllocationProp p = device_prop(device);
    hipMemGenericAllocationHandle_t h;
    hipError_t e = hipMemCreate(&h, bytes, &p, 0);
    if (e != hipSuccess) return hip_fail(e, "hipMemCreate");
    static_assert(sizeof(h) <= sizeof(uint64_t), "allocation handle wider than 64 bits");
    *handle = 0;
    std::memcpy(handle, &h, sizeof h);
    return DOPT_OK;
}

int dopt_vmm_map(uint64_t va, size_t bytes, uint64_t handle) {
    hipMemGenericAllocationHandle_t h;
    std::memcpy(&h, &handle, sizeof h);
    hipError_t e = hipMemMap(as_ptr(va), bytes, 0, h, 0);
    return e == hipSuccess ? DOPT_OK : hip_fail(e, "hipMemMap");
}

int dopt_vmm_set_access(uint64_t va, size_t bytes, int32_t device) {
    hipMemAccessDesc d;
    std::memset(&d, 0, sizeof d);
    d.location.type = hipMemLocationTypeDevice;
    d.location.id = device;
    d.flags = hipMemAccessFlagsProtReadWrite;
    hipError_t e = hipMemSetAccess(as_ptr(va), bytes, &d, 1);
    return e == hipSuccess ? DOPT_OK : hip_fail(e, "hipMemSetAccess");
}

int dopt_vmm_unmap(uint64_t va, size_t bytes) {
    hipError_t e = hipMemUnmap(as_ptr(va), bytes);
    return e == hipSuccess ? DOPT_OK : hip_fail(e, "hipMemUnmap");
}

int dopt_vmm_release(uint64_t handle) {
    hipMemGenericAllocationHandle_t h;
    std::memcpy(&h, &handle, sizeof h);
    hipError_t e = hipMemRelease(h);
    return e == hipSuccess ? DOPT_OK : hip_fail(e, "hipMemRelease");
}

}  // extern "C"
