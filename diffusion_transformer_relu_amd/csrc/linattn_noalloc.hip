// sana_linattn_fwd_noalloc: the forward with the library's own static device
// scratch array in place of a caller's workspace, for callers that cannot
// allocate device memory.  The array is a __device__ object of this module, so
// each GPU the library runs on holds one copy for the life of the process.
// Host code never uses the array's name as an address: its device address is
// looked up once per device with hipGetSymbolAddress and only that address is
// passed to the kernels.
#include "sana_linattn.h"

#include <mutex>

#include "linattn_internal.h"

namespace {

static __device__ __align__(256) unsigned char scratch[SANA_LINATTN_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void* g_scratch[kMaxDevices];          // device address of `scratch` on each device
hipError_t g_lookup[kMaxDevices];      // result of the lookup on each device

// Device address of this device's copy of `scratch`, or nullptr with *err set.
void* scratch_address(hipError_t* err) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        *err = e != hipSuccess ? e : hipErrorInvalidDevice;
        return nullptr;
    }
    std::call_once(g_once[dev], [dev] {
        void* p = nullptr;
        g_lookup[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_scratch[dev] = g_lookup[dev] == hipSuccess ? p : nullptr;
    });
    *err = g_lookup[dev];
    return g_scratch[dev];
}

}  // namespace

extern "C" int sana_linattn_fwd_noalloc(const void* q, const void* k, const void* v, void* out, int in_dtype,
                                        int out_dtype, int B, int H, int N, int D, float eps, hipStream_t stream) {
    size_t need = 0;
    const int st = sana::forward_workspace(in_dtype, out_dtype, B, H, N, D, 0, &need);
    if (st != SANA_OK) return st;
    if (need > SANA_LINATTN_SCRATCH_BYTES) return SANA_ERR_SCRATCH;
    if (need == 0)   // an empty problem: nothing to enqueue, no scratch needed
        return sana::forward_call(q, k, v, out, in_dtype, out_dtype, B, H, N, D, 0, eps, nullptr, 0, stream);
    hipError_t err = hipSuccess;
    void* ws = scratch_address(&err);
    if (!ws) return SANA_ERR_HIP;
    return sana::forward_call(q, k, v, out, in_dtype, out_dtype, B, H, N, D, 0, eps, ws,
                              SANA_LINATTN_SCRATCH_BYTES, stream);
}
