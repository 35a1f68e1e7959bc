// moe_forward_noalloc: the forward with its workspace in a static device
// array, for callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid allocation).
//
// The array, `scratch`, is a file-scope __device__ object of
// MOE_NOALLOC_SCRATCH_BYTES (32 MiB):
// the loader places one copy on every GPU the library's code object is
// loaded on, and it stays there until the process ends.  Host code never
// uses its name as an address (on the host the name is only a stand-in for
// the symbol): on its first call on a device, with that device current, the
// entry looks the array up with hipGetSymbolAddress and keeps the pointer per
// device; kernels receive that pointer as their workspace, exactly as they
// receive a caller's workspace from moe_forward.
//
// Every call on one GPU uses that GPU's single array, which keeps the last
// call's contents (no part of the workspace has to start zeroed: every
// buffer in it is fully written before it is read within one forward).
// Calls that overlap in time on one GPU -- two host threads, or two streams
// without ordering between them -- race on it.
#include "../../include/moe_mi355x.h"
#include "api_internal.h"

#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

namespace {

constexpr size_t kScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void *g_scratch[kMaxDevices] = {};

// This device's copy of `scratch`, looked up once per device.
moe_status scratch_of_current_device(void **out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        char msg[160];
        std::snprintf(msg, sizeof msg, "no-alloc forward: current device %d unusable (%s)", dev,
                      hipGetErrorString(e));
        return moe::set_error(MOE_ERR_HIP, msg);
    }
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            char msg[160];
            std::snprintf(msg, sizeof msg, "no-alloc forward: scratch lookup failed (%s)",
                          hipGetErrorString(e));
            return moe::set_error(MOE_ERR_HIP, msg);
        }
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return MOE_OK;
}

}  // namespace

extern "C" moe_status moe_forward_noalloc(const moe_layer *layer, const moe_tensor *x,
                                          const moe_tensor *router_logits,
                                          const moe_tensor *shared_output, moe_tensor *out,
                                          moe_routing_out *routing, void *stream)
{
    if (!layer || !x || !out)
        return moe::set_error(MOE_ERR_INVALID_ARGUMENT, "NULL argument");
    if (x->ndim < 2 || x->ndim > 3)
        return moe::set_error(MOE_ERR_SHAPE_MISMATCH, "x must be [T, H] or [B, S, H]");
    int64_t T = 1;
    for (int i = 0; i < x->ndim - 1; ++i) {
        if (x->shape[i] < 0) return moe::set_error(MOE_ERR_SHAPE_MISMATCH, "negative dim");
        T *= x->shape[i];
    }
    size_t need = 0;
    moe_status st = moe_workspace_size(layer, T, &need);
    if (st) return st;
    if (need > kScratchBytes) {
        char msg[200];
        std::snprintf(msg, sizeof msg,
                      "no-alloc forward: %lld tokens need %zu bytes of workspace, above the "
                      "%zu-byte static scratch (use moe_forward with a caller workspace)",
                      (long long)T, need, kScratchBytes);
        return moe::set_error(MOE_ERR_WORKSPACE, msg);
    }
    void *ws = nullptr;
    if ((st = scratch_of_current_device(&ws))) return st;
    return moe::forward_impl(layer, x, router_logits, shared_output, out, ws, kScratchBytes,
                             routing, stream, nullptr, false);
}
