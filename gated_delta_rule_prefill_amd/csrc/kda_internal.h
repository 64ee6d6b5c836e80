// kda_internal.h -- host-side pieces of the C ABI shared between its source
// files (not part of the public interface).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <string>

#include "../../include/kda.h"

namespace kda {

// Sets the calling thread's kda_last_error_message() text.
void set_last_error(const std::string& msg);

// kda_prefill_ex with one more switch: with may_allocate false a NULL
// workspace is an error (KDA_ERR_WORKSPACE) instead of a stream-ordered
// allocation.
kda_status prefill_impl(const void* q, const void* k, const void* v, const float* log_alpha,
                        const float* beta, const float* initial_state, const int32_t* cu_seqlens,
                        int64_t total_tokens, int32_t num_seqs, int32_t H, int32_t dk, int32_t dv,
                        kda_dtype dtype, uint32_t flags, void* o, float* final_state,
                        float* chunk_states, void* workspace, size_t workspace_bytes,
                        bool may_allocate, void* stream_ptr);

}  // namespace kda
