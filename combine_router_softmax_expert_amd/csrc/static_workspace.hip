// static_workspace.hip -- the dispatch workspace the library holds itself, for
// callers that cannot allocate device memory (code under graph capture, tight
// serving loops, harnesses that forbid hipMalloc): moe_dispatch_noalloc uses it
// in place of a caller-provided workspace.
//
// One file-scope device array per GPU, allocated with the code object when the
// library is loaded on that device and held until the process ends.  In host
// code the array's name is only a host-side stand-in, never a device address:
// the device address of each GPU's copy comes from hipGetSymbolAddress, taken
// once per device with that device current and kept per device, and only that
// address is handed to kernels.
//
// Every call on a GPU shares that GPU's copy, which keeps the last call's
// contents; no dispatch kernel reads a workspace word before writing it, so
// nothing needs clearing between calls.  A claim counter per device lets the
// library refuse a handle whose arrays a later dispatch on the same device has
// since overwritten.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "kernels.hpp"

namespace moe {
namespace {

constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kStaticWorkspaceBytes];

struct DeviceSlot {
    std::once_flag once;
    void* ptr = nullptr;
    hipError_t status = hipSuccess;
    std::atomic<uint64_t> claims{0};
};
DeviceSlot g_slots[kMaxDevices];

}  // namespace

hipError_t static_workspace(int* device, void** ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    DeviceSlot& slot = g_slots[dev];
    // first use on this device, with the device current: its copy's device address
    std::call_once(slot.once, [&slot] {
        void* p = nullptr;
        slot.status = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        slot.ptr = slot.status == hipSuccess ? p : nullptr;
    });
    if (slot.status != hipSuccess) return slot.status;
    *device = dev;
    *ptr = slot.ptr;
    return hipSuccess;
}

uint64_t static_workspace_claim(int device) { return g_slots[device].claims.fetch_add(1) + 1; }

uint64_t static_workspace_latest_claim(int device) { return g_slots[device].claims.load(); }

}  // namespace moe
