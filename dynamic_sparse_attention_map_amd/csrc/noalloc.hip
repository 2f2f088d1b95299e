// crisp_prefill_noalloc: crisp_prefill on a scratch buffer that the library
// holds itself, for callers that cannot allocate device memory (code under
// HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
//
// The workspace is a file-scope device array, `scratch`, of
// CRISP_NOALLOC_SCRATCH_BYTES.  Each device the library runs on gets its own
// copy when the code object is loaded there, and keeps it until the process
// ends.  In host code the array's name is only a host-side stand-in, so its
// device address is looked up once per device (hipGetSymbolAddress, with
// that device current) on the first call there, and only that address is
// ever handed to the kernels.
//
// Every call on one device shares that device's array, and the array keeps
// whatever the last call left in it.  The kernels of the path clear what
// must start at zero (queue counters, histograms, pass counters) with small
// kernels of their own, so no call depends on the previous contents; but
// two calls that overlap in time on one device (different streams, or
// different host threads without ordering) race on the array.
#include <hip/hip_runtime.h>

#include <mutex>

#include "crisp.h"
#include "crisp_kernels.h"

namespace {

static __device__ __align__(256) unsigned char scratch[CRISP_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
void* g_ptr[kMaxDevices];
hipError_t g_err[kMaxDevices];
std::once_flag g_once[kMaxDevices];

// Device address of `scratch` on the calling thread's current device.
int scratch_address(void** out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return CRISP_ERR_HIP;
    std::call_once(g_once[dev], [dev]() {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_err[dev] = e;
        g_ptr[dev] = (e == hipSuccess) ? p : nullptr;
    });
    if (g_err[dev] != hipSuccess || g_ptr[dev] == nullptr) return CRISP_ERR_HIP;
    *out = g_ptr[dev];
    return CRISP_OK;
}

}  // namespace

extern "C" int crisp_prefill_noalloc(const void* q, const void* k, const void* v, int seq_len,
                                     int n_heads, int n_kv_heads, int head_dim, int block_size,
                                     float alpha, const crisp_opts* opts, void* out, void* stream)
{
    // every argument is checked before the device is touched
    size_t need = 0;
    int rc = crisp::validate_prefill(q, k, v, seq_len, n_heads, n_kv_heads, head_dim, block_size,
                                     alpha, opts, out, &need);
    if (rc) return rc;
    if (seq_len == 0) return CRISP_OK;
    if (need > (size_t)CRISP_NOALLOC_SCRATCH_BYTES) return CRISP_ERR_WORKSPACE;
    void* ws = nullptr;
    if ((rc = scratch_address(&ws))) return rc;
    return crisp_prefill(q, k, v, seq_len, n_heads, n_kv_heads, head_dim, block_size, alpha, opts,
                         ws, (size_t)CRISP_NOALLOC_SCRATCH_BYTES, out, stream);
}
