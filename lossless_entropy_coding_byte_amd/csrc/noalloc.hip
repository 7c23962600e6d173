// lecb_encode without allocation: the workspace lives in a static device
// array, for callers that cannot allocate device memory.
//
// The array's name is a host-side stand-in in host code; its device address
// is asked of the runtime once per device (hipGetSymbolAddress, with that
// device current) and only that address is handed to kernels.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "lecb.h"
#include "lecb_internal.hpp"

namespace {

__device__ __align__(256) uint8_t scratch[LECB_NOALLOC_SCRATCH_BYTES];

std::atomic<void*> scratch_addr[lecb::MAX_DEVICES];
std::mutex scratch_mu;

// Device address of `scratch` on the current device.
int scratch_of_current_device(void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= lecb::MAX_DEVICES) return LECB_ERR_HIP;
    void* p = scratch_addr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(scratch_mu);
        p = scratch_addr[dev].load(std::memory_order_relaxed);
        if (!p) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return LECB_ERR_HIP;
            scratch_addr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return LECB_OK;
}

}  // namespace

extern "C" int lecb_encode_noalloc(const uint8_t* d_in, uint64_t n, const void* d_blob, uint32_t chunk,
                                   uint8_t* d_out, uint64_t out_capacity, lecb_result* d_res, void* stream) {
    if (!lecb::valid_chunk(chunk)) return LECB_ERR_INVALID_ARG;
    if (lecb_workspace_bytes(n, chunk) > LECB_NOALLOC_SCRATCH_BYTES) return LECB_ERR_SCRATCH;
    void* ws = nullptr;
    int rc = scratch_of_current_device(&ws);
    if (rc != LECB_OK) return rc;
    if (n) {
        // the stream's workspace header (exit counter, accumulators, status)
        // starts at zero; the rest of the workspace is written before it is read
        rc = lecb::launch_fill_zero(ws, sizeof(lecb::WsHeader), stream);
        if (rc != LECB_OK) return rc;
    }
    return lecb_encode(d_in, n, d_blob, chunk, d_out, out_capacity, d_res, ws, LECB_NOALLOC_SCRATCH_BYTES,
                       stream);
}
