// loop_decode_noalloc.hip -- gdn_loop_decode_noalloc: the looped decode step
// on a library-held device scratch array, for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, harnesses
// that forbid hipMalloc).
//
// The scratch is a file-scope __device__ array: every GPU the library runs on
// holds its own copy until the process ends.  In host code the array's name is
// only a stand-in, so its device address is looked up once per device with
// hipGetSymbolAddress (with that device current) and kept; kernels receive
// that address, never the name.  All calls on one device share the array and
// its last contents.  Nothing in it needs to start at zero: the decode writes
// q, k, v, the gates and the bf16 operand of every loop before reading them.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/gdnloop.h"
#include "gdn_kernels.h"

static __device__ __align__(256) unsigned char scratch[GDN_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int MAX_DEVICES = 64;
void *g_scratch_ptr[MAX_DEVICES] = {};
std::mutex g_scratch_mu;

// Device address of this device's scratch array (looked up on first use, with
// the device current).  Returns nullptr and records the error on failure.
void *device_scratch(int *status) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= MAX_DEVICES) {
        *status = gdn::set_last_error(GDN_ERR_HIP, "gdn_loop_decode_noalloc: no usable current device");
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            *status = gdn::set_last_error(GDN_ERR_HIP, "gdn_loop_decode_noalloc: hipGetSymbolAddress failed");
            return nullptr;
        }
        g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" gdn_status gdn_loop_decode_noalloc(const gdn_desc *desc, const void *h_t, const void *Wpack,
                                              const float *rho, float *states, float *h_out, void *stream) {
    size_t need = 0;
    gdn_status st = gdn_workspace_bytes(desc, GDN_OP_LOOP_DECODE, &need);
    if (st != GDN_OK) return st;
    // a step whose channel-split projection partials do not fit runs unsplit
    // (gdn_loop_decode takes a workspace without that last region)
    const size_t part = gdn::decode_part_bytes(desc->act == GDN_F32, desc->B, desc->d, desc->H, desc->dk);
    if (part) need -= (part + 255) / 256 * 256;
    if (need > (size_t)GDN_NOALLOC_SCRATCH_BYTES)
        return (gdn_status)gdn::set_last_error(
            GDN_ERR_WORKSPACE, "gdn_loop_decode_noalloc: the step needs more scratch than the library's "
                               "GDN_NOALLOC_SCRATCH_BYTES; use gdn_loop_decode with a workspace");
    int status = GDN_OK;
    void *ws = device_scratch(&status);
    if (!ws) return (gdn_status)status;
    return gdn_loop_decode(desc, h_t, Wpack, rho, states, h_out, ws, (size_t)GDN_NOALLOC_SCRATCH_BYTES, stream);
}
