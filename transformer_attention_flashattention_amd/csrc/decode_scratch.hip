// Device-resident scratch for the allocation-free decode entry point
// (fa_decode_fwd_noalloc): the decode's partial-result workspace as a
// file-scope device array, so that a call allocates nothing.
//
// Each GPU the library runs on holds its own copy of `scratch` from the
// time the code object is loaded on it until the process ends.  Host code
// never passes the array's name to a kernel (on the host it only names a
// stand-in): the device address of each GPU's copy is looked up once per
// device with hipGetSymbolAddress, with that device current, and cached.
#include "fa_internal.h"

#include <mutex>

namespace fa {
namespace {

__device__ __attribute__((aligned(256))) char scratch[kDecodeScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_ptr[kMaxDevices];  // device address of `scratch` per device, once looked up

}  // namespace

hipError_t decode_scratch_address(int device, void **ptr) {
    if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[device]) {
        int cur = -1;
        hipError_t e = hipGetDevice(&cur);
        if (e != hipSuccess) return e;
        if (cur != device && (e = hipSetDevice(device)) != hipSuccess) return e;
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        const hipError_t er = (cur != device) ? hipSetDevice(cur) : hipSuccess;
        if (e != hipSuccess) return e;
        if (er != hipSuccess) return er;
        if (!p) return hipErrorInvalidSymbol;
        g_ptr[device] = p;
    }
    *ptr = g_ptr[device];
    return hipSuccess;
}

}  // namespace fa
