// api_internal.hpp -- pieces of api.cpp that other C-ABI sources of libmtp
// use (internal; the public interface is include/mtp.h).
#pragma once

#include <hip/hip_runtime.h>

#include "../../include/mtp.h"

namespace mtp {

// Record a message for mtp_last_error() (printf-style) and return s.
mtp_status fail(mtp_status s, const char* fmt, ...);
// MTP_ERR_HIP with "what: <HIP error string>".
mtp_status hip_fail(hipError_t e, const char* what);

// mtp_draft_step in two halves.  check_draft_step_args runs every check of
// the call except the workspace's on the host (no HIP call);
// enqueue_draft_step launches the step with ws of at least
// mtp_draft_step_workspace_size(L, cache_len, m) bytes, 256-byte aligned,
// on arguments that passed the checks.
mtp_status check_draft_step_args(const mtp_layer* L, const float* e, const int32_t* tokens,
                                 const float* embed_table, const float* h, float* k_cache, float* v_cache,
                                 int32_t cache_len, int32_t capacity, int32_t m, int32_t* ids_out,
                                 float* hidden_out, float* logits_out);
mtp_status enqueue_draft_step(const mtp_layer* L, const float* e, const int32_t* tokens, const float* embed_table,
                              const float* h, float* k_cache, float* v_cache, int32_t cache_len, int32_t capacity,
                              int32_t m, int32_t* ids_out, float* hidden_out, float* logits_out, void* ws,
                              void* stream);

}  // namespace mtp
