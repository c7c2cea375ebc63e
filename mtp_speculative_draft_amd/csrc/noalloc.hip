// noalloc.hip -- mtp_draft_step_noalloc: the draft step with its scratch
// space in a static device array of the library instead of a caller's
// workspace, for callers that cannot allocate device memory.
//
// Each GPU the library runs on holds its own copy of `scratch` (the code
// object's), at its own address, until the process ends.  On the host the
// array's name is only a stand-in for the device symbol, so the kernels are
// given the device address that hipGetSymbolAddress returns, looked up once
// per device with that device current and kept in g_scratch.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/mtp.h"
#include "api_internal.hpp"

using namespace mtp;

namespace {

constexpr size_t kScratchBytes = MTP_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::once_flag g_once[kMaxDevices];
void* g_scratch[kMaxDevices];
hipError_t g_lookup[kMaxDevices];

// The device address of `scratch` on device dev (the current device).
hipError_t scratch_on(int dev, void** out) {
    std::call_once(g_once[dev], [dev] {
        void* ptr = nullptr;
        g_lookup[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        g_scratch[dev] = g_lookup[dev] == hipSuccess ? ptr : nullptr;
    });
    *out = g_scratch[dev];
    return g_lookup[dev];
}

}  // namespace

extern "C" {

mtp_status mtp_draft_step_noalloc(const mtp_layer* L, const float* e, const int32_t* tokens,
                                  const float* embed_table, const float* h, float* k_cache, float* v_cache,
                                  int32_t cache_len, int32_t capacity, int32_t m, int32_t* ids_out,
                                  float* hidden_out, float* logits_out, void* stream) {
    mtp_status s = check_draft_step_args(L, e, tokens, embed_table, h, k_cache, v_cache, cache_len, capacity, m,
                                         ids_out, hidden_out, logits_out);
    if (s) return s;
    const size_t need = mtp_draft_step_workspace_size(L, cache_len, m);
    if (need > kScratchBytes)
        return fail(MTP_ERR_WORKSPACE,
                    "mtp_draft_step_noalloc: this step needs %zu bytes of scratch, more than the static %zu "
                    "(MTP_NOALLOC_SCRATCH_BYTES); use mtp_draft_step with a workspace",
                    need, kScratchBytes);
    int dev = -1;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return hip_fail(err, "mtp_draft_step_noalloc hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices)
        return fail(MTP_ERR_UNSUPPORTED, "mtp_draft_step_noalloc: device %d (at most %d devices)", dev, kMaxDevices);
    if (stream) {
        int sdev = -1;
        if ((err = hipStreamGetDevice((hipStream_t)stream, &sdev)) != hipSuccess)
            return hip_fail(err, "mtp_draft_step_noalloc hipStreamGetDevice");
        if (sdev != dev)
            return fail(MTP_ERR_INVALID_ARG, "mtp_draft_step_noalloc: the stream is on device %d, the current device is %d",
                        sdev, dev);
    }
    void* ws = nullptr;
    if ((err = scratch_on(dev, &ws)) != hipSuccess) return hip_fail(err, "mtp_draft_step_noalloc hipGetSymbolAddress");
    // The first kernel of the step clears the argmax state at the scratch's
    // start; nothing else in it has to start at zero.
    return enqueue_draft_step(L, e, tokens, embed_table, h, k_cache, v_cache, cache_len, capacity, m, ids_out,
                              hidden_out, logits_out, ws, stream);
}

}  // extern "C"
