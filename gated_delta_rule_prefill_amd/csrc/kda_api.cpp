// kda_api.cpp -- host side of libkda: argument validation, launch planning,
// workspace layout, error reporting and optional kernel timing.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/kda.h"
#include "kda_launch.h"


namespace {

thread_local std::string g_last_error;

kda_status fail(kda_status s, const std::string& msg) {
    g_last_error = msg;
    return s;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Workspace layout of one prefill call: one record per (chunk, head) slot,
// then the chunk table.
struct Plan {
    int64_t max_chunks = 0;
    size_t rec_bytes = 0;   // bytes of one (chunk, head) record
    size_t off_seq = 0;     // seq_chunk_start [N+1]
    size_t off_chunks = 0;  // ChunkInfo [max_chunks]
    size_t total = 0;
};

bool make_plan(int64_t T, int32_t N, int32_t H, int32_t dk, int32_t dv, kda_dtype dtype,
               Plan& p) {
    if (T < 0 || N <= 0 || H <= 0 || dk <= 0 || dv <= 0) return false;
    const int es = dtype == KDA_DTYPE_BF16 ? 2 : 4;
    p.max_chunks = (T + kda::CHUNK - 1) / kda::CHUNK + N;
    p.rec_bytes = kda::rec_layout(es, dk, dv).bytes;
    size_t at = align256((size_t)p.max_chunks * (size_t)H * p.rec_bytes);
    p.off_seq = at;
    at += align256(((size_t)N + 1) * 4);
    p.off_chunks = at;
    at += align256((size_t)p.max_chunks * sizeof(kda::ChunkInfo));
    p.total = at;
    return true;
}

bool supported_dim(int32_t d) { return d == 64 || d == 128; }

// Workspace of one backward call: the forward plan (chunk table and records for
// a recomputation), then the recomputed fp32
// chunk states, an output scratch for the recomputation, the per-slice
// partial gradients and the per-workgroup scratch.
struct BwdPlan {
    Plan fwd;
    size_t off_cs = 0, off_o = 0, off_part = 0, off_scratch = 0, total = 0;
};

bool make_bwd_plan(int64_t T, int32_t N, int32_t H, int32_t dk, int32_t dv, kda_dtype dtype,
                   BwdPlan& b) {
    if (dtype != KDA_DTYPE_F32 && dtype != KDA_DTYPE_BF16) return false;
    if (!make_plan(T, N, H, dk, dv, dtype, b.fwd)) return false;
    if (!supported_dim(dk) || !supported_dim(dv)) return false;
    const int es = dtype == KDA_DTYPE_BF16 ? 2 : 4;
    size_t at = b.fwd.total;
    b.off_cs = at;
    at += align256((size_t)b.fwd.max_chunks * H * dk * dv * 4);
    b.off_o = at;
    at += align256((size_t)T * H * dv * es);
    b.off_part = at;
    at += align256(kda::backward_partial_bytes(T, H, dk, dv));
    b.off_scratch = at;
    at += align256(kda::backward_scratch_bytes(N, H, dk, dv));
    b.total = at;
    return true;
}

constexpr uint32_t kFlagMask = KDA_FLAG_L2NORM_QK | KDA_FLAG_BETA_SIGMOID;

unsigned pre_flags(uint32_t flags) {
    return ((flags & KDA_FLAG_L2NORM_QK) ? kda::PRE_L2NORM_QK : 0u) |
           ((flags & KDA_FLAG_BETA_SIGMOID) ? kda::PRE_BETA_LOGIT : 0u);
}

// -- optional kernel timing ---------------------------------------------------
constexpr int kMaxTimed = 8;
std::mutex g_timing_mu;
bool g_timing = false;
hipEvent_t g_ev[kMaxTimed + 1] = {};
const char* g_names[kMaxTimed] = {};
int g_n_timed = -1;

struct Timer {
    bool on;
    int n = 0;
    hipStream_t stream;
    explicit Timer(hipStream_t s) : on(false), stream(s) {
        std::lock_guard<std::mutex> lk(g_timing_mu);
        on = g_timing;
        if (on) {
            for (int i = 0; i <= kMaxTimed; ++i)
                if (!g_ev[i] && hipEventCreate(&g_ev[i]) != hipSuccess) on = false;
            g_n_timed = -1;
        }
        if (on) hipEventRecord(g_ev[0], stream);
    }
    void mark(const char* name) {
        if (!on || n >= kMaxTimed) return;
        g_names[n] = name;
        hipEventRecord(g_ev[n + 1], stream);
        ++n;
    }
    ~Timer() {
        if (on) {
            std::lock_guard<std::mutex> lk(g_timing_mu);
            g_n_timed = n;
        }
    }
};

bool debug_sync() {
    static const bool on = [] {
        const char* e = std::getenv("KDA_DEBUG_SYNC");
        return e && e[0] && e[0] != '0';
    }();
    return on;
}

kda_status check_launch(hipError_t e, const char* what, hipStream_t stream) {
    if (e == hipSuccess && debug_sync()) e = hipStreamSynchronize(stream);
    if (e != hipSuccess)
        return fail(KDA_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
    return KDA_OK;
}

}  // namespace

extern "C" {

size_t kda_prefill_workspace_bytes(int64_t total_tokens, int32_t num_seqs, int32_t H,
                                   int32_t dk, int32_t dv, kda_dtype dtype) {
    Plan p;
    if (dtype != KDA_DTYPE_F32 && dtype != KDA_DTYPE_BF16) return 0;
    if (!make_plan(total_tokens, num_seqs, H, dk, dv, dtype, p)) return 0;
    return p.total;
}

kda_status kda_prefill(const void* q, const void* k, const void* v, const float* log_alpha,
                       const float* beta, const float* initial_state, const int32_t* cu_seqlens,
                       int64_t total_tokens, int32_t num_seqs, int32_t H, int32_t dk, int32_t dv,
                       kda_dtype dtype, void* o, float* final_state, void* workspace,
                       size_t workspace_bytes, void* stream_ptr) {
    return kda_prefill_ex(q, k, v, log_alpha, beta, initial_state, cu_seqlens, total_tokens,
                          num_seqs, H, dk, dv, dtype, 0u, o, final_state, nullptr, workspace,
                          workspace_bytes, stream_ptr);
}

kda_status kda_prefill_ex(const void* q, const void* k, const void* v, const float* log_alpha,
                          const float* beta, const float* initial_state,
                          const int32_t* cu_seqlens, int64_t total_tokens, int32_t num_seqs,
                          int32_t H, int32_t dk, int32_t dv, kda_dtype dtype, uint32_t flags,
                          void* o, float* final_state, float* chunk_states, void* workspace,
                          size_t workspace_bytes, void* stream_ptr) {
    try {
        if (dtype != KDA_DTYPE_F32 && dtype != KDA_DTYPE_BF16)
            return fail(KDA_ERR_INVALID_ARGUMENT, "dtype must be KDA_DTYPE_F32 or KDA_DTYPE_BF16");
        if (flags & ~kFlagMask) return fail(KDA_ERR_INVALID_ARGUMENT, "unknown flag bits");
        if (num_seqs <= 0) return fail(KDA_ERR_INVALID_ARGUMENT, "num_seqs must be >= 1");
        if (H <= 0 || H > 65535) return fail(KDA_ERR_INVALID_ARGUMENT, "H must be in [1, 65535]");
        if (total_tokens < 0 || total_tokens >= ((int64_t)1 << 31) - 2 * kda::CHUNK)
            return fail(KDA_ERR_INVALID_ARGUMENT, "total_tokens must be in [0, 2^31 - 128)");
        if (!supported_dim(dk) || !supported_dim(dv))
            return fail(KDA_ERR_UNSUPPORTED, "dk and dv must each be 64 or 128");
        if (!cu_seqlens && total_tokens % num_seqs != 0)
            return fail(KDA_ERR_INVALID_ARGUMENT,
                        "without cu_seqlens, total_tokens must be a multiple of num_seqs");
        if (total_tokens > 0 && (!q || !k || !v || !log_alpha || !beta || !o))
            return fail(KDA_ERR_INVALID_ARGUMENT, "q, k, v, log_alpha, beta and o must be non-NULL");
        const void* ptrs[] = {q, k, v, log_alpha, beta, initial_state, cu_seqlens, o,
                              final_state, chunk_states, workspace};
        for (const void* p : ptrs)
            if (p && !aligned16(p))
                return fail(KDA_ERR_INVALID_ARGUMENT, "every pointer must be 16-byte aligned");
        if (!workspace && workspace_bytes != 0)
            return fail(KDA_ERR_INVALID_ARGUMENT, "workspace_bytes given without a workspace");
        Plan plan;
        if (!make_plan(total_tokens, num_seqs, H, dk, dv, dtype, plan))
            return fail(KDA_ERR_INVALID_ARGUMENT, "invalid sizes");
        if (plan.max_chunks > 0x7fffffffLL / 2 || plan.max_chunks * H > 0x7fffffffLL)
            return fail(KDA_ERR_INVALID_ARGUMENT, "too many chunks (chunks * H must be < 2^31)");
        if (workspace && workspace_bytes < plan.total)
            return fail(KDA_ERR_WORKSPACE, "workspace too small: need " +
                                               std::to_string(plan.total) + " bytes");
        const long long state_blocks = ((long long)num_seqs * H + 7) / 8 * 8 * (dv / 16);
        if (state_blocks > 0x7fffffffLL)
            return fail(KDA_ERR_INVALID_ARGUMENT, "num_seqs * H too large");

        hipStream_t stream = reinterpret_cast<hipStream_t>(stream_ptr);
        const bool bf16 = dtype == KDA_DTYPE_BF16;
        unsigned char* ws = static_cast<unsigned char*>(workspace);
        bool owned = false;
        if (!ws) {
            hipError_t e = hipMallocAsync(reinterpret_cast<void**>(&ws), plan.total, stream);
            if (e != hipSuccess)
                return fail(KDA_ERR_HIP, std::string("hipMallocAsync: ") + hipGetErrorString(e));
            owned = true;
        }
        int32_t* seq_start = reinterpret_cast<int32_t*>(ws + plan.off_seq);
        kda::ChunkInfo* chunks = reinterpret_cast<kda::ChunkInfo*>(ws + plan.off_chunks);

        kda_status st = KDA_OK;
        {
            Timer timer(stream);
            // N equal rows need no chunk table: the kernels derive their chunks
            kda::ChunkSrc src{chunks, seq_start, cu_seqlens ? -1 : (int)(total_tokens / num_seqs),
                              num_seqs};
            if (cu_seqlens) {
                st = check_launch(kda::launch_chunk_table(cu_seqlens, total_tokens, num_seqs,
                                                          seq_start, chunks, (int)plan.max_chunks,
                                                          stream),
                                  "chunk table kernel", stream);
                timer.mark("chunk_table");
            }
            if (st == KDA_OK && total_tokens > 0) {
                st = check_launch(kda::launch_prefill_intra(q, k, v, log_alpha, beta, src,
                                                            (int)plan.max_chunks, H, dk, dv, bf16,
                                                            pre_flags(flags), ws, stream),
                                  "intra-chunk kernel", stream);
                timer.mark("prefill_intra");
            }
            if (st == KDA_OK) {
                st = check_launch(kda::launch_prefill_state(ws, src, initial_state, final_state, o,
                                                            chunk_states, H, dk, dv, bf16, stream),
                                  "state kernel", stream);
                timer.mark("prefill_state");
            }
        }
        if (owned) {
            hipError_t e = hipFreeAsync(ws, stream);
            if (st == KDA_OK && e != hipSuccess)
                st = fail(KDA_ERR_HIP, std::string("hipFreeAsync: ") + hipGetErrorString(e));
        }
        return st;
    } catch (...) {
        return fail(KDA_ERR_HIP, "unexpected C++ exception inside kda_prefill");
    }
}

size_t kda_backward_workspace_bytes(int64_t total_tokens, int32_t num_seqs, int32_t H,
                                    int32_t dk, int32_t dv, kda_dtype dtype) {
    BwdPlan b;
    if (!make_bwd_plan(total_tokens, num_seqs, H, dk, dv, dtype, b)) return 0;
    return b.total;
}

kda_status kda_backward(const void* q, const void* k, const void* v, const float* log_alpha,
                        const float* beta, const float* initial_state, const int32_t* cu_seqlens,
                        int64_t total_tokens, int32_t num_seqs, int32_t H, int32_t dk, int32_t dv,
                        kda_dtype dtype, const void* d_o, const float* d_final_state,
                        const float* chunk_states, void* dq, void* dk_out, void* dv_out,
                        float* dlog_alpha, float* dbeta, float* d_initial_state, void* workspace,
                        size_t workspace_bytes, void* stream_ptr) {
    try {
        if (dtype != KDA_DTYPE_F32 && dtype != KDA_DTYPE_BF16)
            return fail(KDA_ERR_INVALID_ARGUMENT, "dtype must be KDA_DTYPE_F32 or KDA_DTYPE_BF16");
        if (num_seqs <= 0) return fail(KDA_ERR_INVALID_ARGUMENT, "num_seqs must be >= 1");
        if (H <= 0 || H > 65535) return fail(KDA_ERR_INVALID_ARGUMENT, "H must be in [1, 65535]");
        if (total_tokens < 0 || total_tokens >= ((int64_t)1 << 31) - 2 * kda::CHUNK)
            return fail(KDA_ERR_INVALID_ARGUMENT, "total_tokens must be in [0, 2^31 - 128)");
        if (!supported_dim(dk) || !supported_dim(dv))
            return fail(KDA_ERR_UNSUPPORTED, "dk and dv must each be 64 or 128");
        if (!cu_seqlens && total_tokens % num_seqs != 0)
            return fail(KDA_ERR_INVALID_ARGUMENT,
                        "without cu_seqlens, total_tokens must be a multiple of num_seqs");
        if (total_tokens > 0 && (!q || !k || !v || !log_alpha || !beta || !d_o || !dq || !dk_out ||
                                 !dv_out || !dlog_alpha || !dbeta))
            return fail(KDA_ERR_INVALID_ARGUMENT,
                        "inputs, d_o and the gradient outputs must be non-NULL");
        const void* ptrs[] = {q, k, v, log_alpha, beta, initial_state, cu_seqlens, d_o,
                              d_final_state, chunk_states, dq, dk_out, dv_out, dlog_alpha, dbeta,
                              d_initial_state, workspace};
        for (const void* p : ptrs)
            if (p && !aligned16(p))
                return fail(KDA_ERR_INVALID_ARGUMENT, "every pointer must be 16-byte aligned");
        if (!workspace && workspace_bytes != 0)
            return fail(KDA_ERR_INVALID_ARGUMENT, "workspace_bytes given without a workspace");
        BwdPlan b;
        if (!make_bwd_plan(total_tokens, num_seqs, H, dk, dv, dtype, b))
            return fail(KDA_ERR_INVALID_ARGUMENT, "invalid sizes");
        const Plan& plan = b.fwd;
        if (plan.max_chunks > 0x7fffffffLL / 2 || plan.max_chunks * H > 0x7fffffffLL ||
            (long long)num_seqs * H * (dv / 16) > 0x7fffffffLL)
            return fail(KDA_ERR_INVALID_ARGUMENT, "sizes too large");
        if (workspace && workspace_bytes < b.total)
            return fail(KDA_ERR_WORKSPACE, "workspace too small: need " + std::to_string(b.total) +
                                               " bytes");

        hipStream_t stream = reinterpret_cast<hipStream_t>(stream_ptr);
        const bool bf16 = dtype == KDA_DTYPE_BF16;
        unsigned char* ws = static_cast<unsigned char*>(workspace);
        bool owned = false;
        if (!ws) {
            hipError_t e = hipMallocAsync(reinterpret_cast<void**>(&ws), b.total, stream);
            if (e != hipSuccess)
                return fail(KDA_ERR_HIP, std::string("hipMallocAsync: ") + hipGetErrorString(e));
            owned = true;
        }
        int32_t* seq_start = reinterpret_cast<int32_t*>(ws + plan.off_seq);
        kda::ChunkInfo* chunks = reinterpret_cast<kda::ChunkInfo*>(ws + plan.off_chunks);
        kda::ChunkSrc src{chunks, seq_start, cu_seqlens ? -1 : (int)(total_tokens / num_seqs),
                          num_seqs};
        kda_status st = KDA_OK;
        if (cu_seqlens)
            st = check_launch(kda::launch_chunk_table(cu_seqlens, total_tokens, num_seqs, seq_start,
                                                      chunks, (int)plan.max_chunks, stream),
                              "chunk table kernel", stream);
        const float* cs = chunk_states;
        if (st == KDA_OK && !cs && total_tokens > 0) {
            // forward recomputation: records, then the chain with its chunk states
            float* own_cs = reinterpret_cast<float*>(ws + b.off_cs);
            void* o_scratch = ws + b.off_o;
            st = check_launch(kda::launch_prefill_intra(q, k, v, log_alpha, beta, src,
                                                        (int)plan.max_chunks, H, dk, dv, bf16, 0u,
                                                        ws, stream),
                              "intra-chunk kernel", stream);
            if (st == KDA_OK)
                st = check_launch(kda::launch_prefill_state(ws, src, initial_state, nullptr,
                                                            o_scratch, own_cs, H, dk, dv, bf16,
                                                            stream),
                                  "state kernel", stream);
            cs = own_cs;
        }
        if (st == KDA_OK)
            st = check_launch(kda::launch_backward(q, k, v, log_alpha, beta, src, cs, d_o,
                                                   d_final_state, H, total_tokens, dk, dv, bf16, dq,
                                                   dk_out, dv_out, dlog_alpha, dbeta,
                                                   d_initial_state,
                                                   reinterpret_cast<float*>(ws + b.off_part),
                                                   reinterpret_cast<float*>(ws + b.off_scratch),
                                                   stream),
                              "backward kernels", stream);
        if (owned) {
            hipError_t e = hipFreeAsync(ws, stream);
            if (st == KDA_OK && e != hipSuccess)
                st = fail(KDA_ERR_HIP, std::string("hipFreeAsync: ") + hipGetErrorString(e));
        }
        return st;
    } catch (...) {
        return fail(KDA_ERR_HIP, "unexpected C++ exception inside kda_backward");
    }
}

kda_status kda_decode_tokens(float* state_pool, int32_t num_slots, const int32_t* state_indices,
                             const void* q, const void* k, const void* v, const float* log_alpha,
                             const float* beta, const int32_t* cu_seqlens, int64_t total_tokens,
                             int32_t num_seqs, int32_t H, int32_t dk, int32_t dv, kda_dtype dtype,
                             uint32_t flags, void* o, void* stream_ptr) {
    try {
        if (dtype != KDA_DTYPE_F32 && dtype != KDA_DTYPE_BF16)
            return fail(KDA_ERR_INVALID_ARGUMENT, "dtype must be KDA_DTYPE_F32 or KDA_DTYPE_BF16");
        if (flags & ~kFlagMask) return fail(KDA_ERR_INVALID_ARGUMENT, "unknown flag bits");
        if (num_seqs <= 0 || H <= 0 || num_slots <= 0)
            return fail(KDA_ERR_INVALID_ARGUMENT, "num_seqs, H and num_slots must be >= 1");
        if (total_tokens < 0 || total_tokens > 0x7fffffffLL)
            return fail(KDA_ERR_INVALID_ARGUMENT, "total_tokens must be in [0, 2^31)");
        const long long blocks = (long long)num_seqs * H;   // one workgroup per (sequence, head)
        if (blocks > 0x7fffffffLL || (long long)num_slots * H > 0x7fffffffLL)
            return fail(KDA_ERR_INVALID_ARGUMENT, "num_seqs * H or num_slots * H too large");
        if (!supported_dim(dk) || !supported_dim(dv))
            return fail(KDA_ERR_UNSUPPORTED, "dk and dv must each be 64 or 128");
        if (!cu_seqlens && total_tokens % num_seqs != 0)
            return fail(KDA_ERR_INVALID_ARGUMENT,
                        "without cu_seqlens, total_tokens must be a multiple of num_seqs");
        if (!state_indices && num_slots < num_seqs)
            return fail(KDA_ERR_INVALID_ARGUMENT, "without state_indices, num_slots must be >= num_seqs");
        if (!state_pool) return fail(KDA_ERR_INVALID_ARGUMENT, "state_pool must be non-NULL");
        if (total_tokens > 0 && (!q || !k || !v || !log_alpha || !beta || !o))
            return fail(KDA_ERR_INVALID_ARGUMENT, "q, k, v, log_alpha, beta and o must be non-NULL");
        const void* ptrs[] = {state_pool, state_indices, q, k, v, log_alpha, beta, cu_seqlens, o};
        for (const void* p : ptrs)
            if (p && !aligned16(p))
                return fail(KDA_ERR_INVALID_ARGUMENT, "every pointer must be 16-byte aligned");
        hipStream_t stream = reinterpret_cast<hipStream_t>(stream_ptr);
        const int rows = cu_seqlens ? -1 : (int)(total_tokens / num_seqs);
        return check_launch(kda::launch_recurrent(state_pool, num_slots, state_indices, q, k, v,
                                                  log_alpha, beta, cu_seqlens, rows, num_seqs, H,
                                                  dk, dv, dtype == KDA_DTYPE_BF16,
                                                  pre_flags(flags), o, stream),
                            "recurrent kernel", stream);
    } catch (...) {
        return fail(KDA_ERR_HIP, "unexpected C++ exception inside kda_decode_tokens");
    }
}

kda_status kda_decode_step(float* state, const void* q, const void* k, const void* v,
                           const float* log_alpha, const float* beta, int32_t num_seqs, int32_t H,
                           int32_t dk, int32_t dv, kda_dtype dtype, void* o, void* stream_ptr) {
    try {
        if (dtype != KDA_DTYPE_F32 && dtype != KDA_DTYPE_BF16)
            return fail(KDA_ERR_INVALID_ARGUMENT, "dtype must be KDA_DTYPE_F32 or KDA_DTYPE_BF16");
        if (num_seqs <= 0 || H <= 0)
            return fail(KDA_ERR_INVALID_ARGUMENT, "num_seqs and H must be >= 1");
        if ((long long)num_seqs * H > 0x7fffffffLL)
            return fail(KDA_ERR_INVALID_ARGUMENT, "num_seqs * H too large");
        if (!supported_dim(dk) || !supported_dim(dv))
            return fail(KDA_ERR_UNSUPPORTED, "dk and dv must each be 64 or 128");
        if (!state || !q || !k || !v || !log_alpha || !beta || !o)
            return fail(KDA_ERR_INVALID_ARGUMENT, "all pointers must be non-NULL");
        const void* ptrs[] = {state, q, k, v, log_alpha, beta, o};
        for (const void* p : ptrs)
            if (!aligned16(p))
                return fail(KDA_ERR_INVALID_ARGUMENT, "every pointer must be 16-byte aligned");
        hipStream_t stream = reinterpret_cast<hipStream_t>(stream_ptr);
        return check_launch(kda::launch_decode_step(state, q, k, v, log_alpha, beta, o,
                                                    num_seqs * H, dk, dv,
                                                    dtype == KDA_DTYPE_BF16, stream),
                            "decode kernel", stream);
    } catch (...) {
        return fail(KDA_ERR_HIP, "unexpected C++ exception inside kda_decode_step");
    }
}

const char* kda_status_string(kda_status s) {
    switch (s) {
        case KDA_OK: return "KDA_OK";
        case KDA_ERR_INVALID_ARGUMENT: return "KDA_ERR_INVALID_ARGUMENT";
        case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED";
        case KDA_ERR_WORKSPACE: return "KDA_ERR_WORKSPACE";
        case KDA_ERR_HIP: return "KDA_ERR_HIP";
    }
    return "unknown kda_status";
}

const char* kda_last_error_message(void) { return g_last_error.c_str(); }

int32_t kda_version(void) { return 100; }

kda_status kda_set_kernel_timing(int32_t enabled) {
    std::lock_guard<std::mutex> lk(g_timing_mu);
    g_timing = enabled != 0;
    return KDA_OK;
}

int32_t kda_prefill_kernel_times(float* ms, const char** names, int32_t max_kernels) {
    std::lock_guard<std::mutex> lk(g_timing_mu);
    if (g_n_timed < 0) return -1;
    if (hipEventSynchronize(g_ev[g_n_timed]) != hipSuccess) return -1;
    for (int i = 0; i < g_n_timed && i < max_kernels; ++i) {
        float t = 0.f;
        if (hipEventElapsedTime(&t, g_ev[i], g_ev[i + 1]) != hipSuccess) return -1;
        if (ms) ms[i] = t;
        if (names) names[i] = g_names[i];
    }
    return g_n_timed;
}

}  // extern "C"
