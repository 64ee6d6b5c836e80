// kda_api.cpp -- host side of libkda: argument validation, launch planning,
// workspace layout, error reporting and optional kernel timing.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdlib>
#include <algorithm>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/kda.h"
#include "kda_launch.h"
#include "kda_internal.h"


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
//
// Long batches of equal rows run in segments: token ranges of every sequence
// whose records together stay near the size of the 256 MB last-level cache,
// so that the sequential pass reads records the intra pass has just written
// instead of fetching them from HBM.  Only one segment's records exist at a
// time; the fp32 state passes from segment to segment through final_state
// (or, without it, a carry area at the end of the workspace).
// The record budget of one segment: 208 MiB, or KDA_SEGMENT_RECORD_BYTES from
// the environment (read once; for tests and tuning).
size_t segment_record_bytes() {
    static const size_t v = [] {
        const char* e = std::getenv("KDA_SEGMENT_RECORD_BYTES");
        const long long x = e ? std::atoll(e) : 0;
        return x > 0 ? (size_t)x : (size_t)208 << 20;
    }();
    return v;
}

struct Plan {
    int64_t max_chunks = 0;  // record slots per head (one segment's chunks)
    size_t rec_bytes = 0;    // bytes of one (chunk, head) record
    int seg_tokens = 0;      // equal rows: tokens per segment (== rows: one segment)
    size_t off_seq = 0;      // seq_chunk_start [N+1], then seq_order [N]
    size_t off_chunks = 0;   // ChunkInfo [max_chunks]
    size_t off_carry = 0;    // fp32 [N,H,dk,dv] state between segments (segmented only)
    size_t total = 0;
};

// segment: plan equal-row batches in segments (prefill); false keeps every
// chunk's record (the backward's recomputation reads them all at once).
bool make_plan(int64_t T, int32_t N, int32_t H, int32_t dk, int32_t dv, kda_dtype dtype,
               Plan& p, bool segment = false, bool equal_rows = false) {
    if (T < 0 || N <= 0 || H <= 0 || dk <= 0 || dv <= 0) return false;
    const int es = dtype == KDA_DTYPE_BF16 ? 2 : 4;
    p.rec_bytes = kda::rec_layout(es, dk, dv).bytes;
    p.max_chunks = (T + kda::CHUNK - 1) / kda::CHUNK + N;
    p.seg_tokens = 0;
    bool carry = false;
    if (segment && equal_rows && T % N == 0 && T / N > 0) {
        const int64_t rows = T / N, cps = (rows + kda::CHUNK - 1) / kda::CHUNK;
        const int64_t per_chunk = (int64_t)N * H * (int64_t)p.rec_bytes;
        const int64_t max_seg = std::max<int64_t>(1, (int64_t)segment_record_bytes() / per_chunk);
        const int64_t nseg = (cps + max_seg - 1) / max_seg;
        const int64_t seg_chunks = (cps + nseg - 1) / nseg;
        p.seg_tokens = (int)std::min<int64_t>(rows, seg_chunks * kda::CHUNK);
        p.max_chunks = (int64_t)N * seg_chunks;
        carry = nseg > 1;
    }
    size_t at = align256((size_t)p.max_chunks * (size_t)H * p.rec_bytes);
    p.off_seq = at;
    at += align256(((size_t)2 * N + 1) * 4);   // seq_chunk_start [N+1], then seq_order [N]
    p.off_chunks = at;
    at += align256((size_t)p.max_chunks * sizeof(kda::ChunkInfo));
    p.off_carry = at;
    if (carry) at += align256((size_t)N * H * dk * dv * 4);
    p.total = at;
    return true;
}

bool supported_dim(int32_t d) { return d == 64 || d == 128; }

// Workspace of one backward call: the forward plan (chunk table and records for
// a recomputation, reused for the reverse-chain records), then the recomputed
// fp32 chunk states, an output scratch for the recomputation, and one area
// that holds either the token-serial path's per-slice partial gradients and
// per-workgroup scratch or the chunkwise path's gradients leaving every chunk.
struct BwdPlan {
    Plan fwd;
    size_t off_cs = 0, off_o = 0, off_part = 0, off_scratch = 0, off_dsc = 0, total = 0;
};

// The chunkwise backward (reverse chain over per-chunk records, then one
// gradient workgroup per chunk) covers bf16 with dk = dv = 128; the other
// configurations walk the tokens.  KDA_BACKWARD_SERIAL=1 in the environment
// forces the token walk (read once; for tests and measurement).
bool chunkwise_backward(kda_dtype dtype, int32_t dk, int32_t dv) {
    static const bool serial = [] {
        const char* e = std::getenv("KDA_BACKWARD_SERIAL");
        return e && e[0] == '1';
    }();
    return !serial && dtype == KDA_DTYPE_BF16 && dk == 128 && dv == 128;
}

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
    b.off_dsc = at;
    const size_t serial = align256(kda::backward_partial_bytes(T, H, dk, dv)) +
                          align256(kda::backward_scratch_bytes(N, H, dk, dv));
    const size_t dsc = align256((size_t)b.fwd.max_chunks * H * dk * dv * 2);   // bf16
    b.off_scratch = at + align256(kda::backward_partial_bytes(T, H, dk, dv));
    at += std::max(serial, dsc);
    b.total = at;
    return true;
}

constexpr uint32_t kFlagMask = KDA_FLAG_L2NORM_QK | KDA_FLAG_BETA_SIGMOID;

unsigned pre_flags(uint32_t flags) {
    return ((flags & KDA_FLAG_L2NORM_QK) ? kda::PRE_L2NORM_QK : 0u) |
           ((flags & KDA_FLAG_BETA_SIGMOID) ? kda::PRE_BETA_LOGIT : 0u);
}

// -- optional kernel timing ---------------------------------------------------
// Per calling thread, like the error text: each thread that enables timing
// gets its own events (created on first use, kept until the process ends),
// and kda_prefill_kernel_times() reports the last call timed on that thread.
constexpr int kMaxTimed = 256;
struct TimingState {
    bool on = false;
    hipEvent_t ev[2 * kMaxTimed] = {};   // start and stop of each timed kernel
    const char* names[kMaxTimed] = {};
    int n_timed = -1;
};
thread_local TimingState t_timing;
thread_local kda::LaunchEvents t_launch;

// Each timed kernel gets its own pair of events, which the launcher hands to
// hipExtLaunchKernelGGL: they take the kernel's own start and end, so a
// kernel's time excludes the gap to the work before it.  The events are
// timing-only (no system-scope fence when one is recorded).
struct Timer {
    bool on;
    int n = 0;
    explicit Timer(hipStream_t) : on(t_timing.on) {
        if (on) {
            for (int i = 0; i < 2 * kMaxTimed; ++i)
                if (!t_timing.ev[i] && hipEventCreateWithFlags(&t_timing.ev[i],
                                                               hipEventDisableSystemFence) != hipSuccess)
                    on = false;
            t_timing.n_timed = -1;
        }
    }
    // before a kernel launch: the launch takes this kernel's events
    void arm() {
        if (on && n < kMaxTimed) t_launch = kda::LaunchEvents{t_timing.ev[2 * n], t_timing.ev[2 * n + 1]};
    }
    // after it: the kernel's name; the next launch is untimed until armed
    void mark(const char* name) {
        t_launch = kda::LaunchEvents{};
        if (!on || n >= kMaxTimed) return;
        t_timing.names[n] = name;
        ++n;
    }
    ~Timer() {
        t_launch = kda::LaunchEvents{};
        if (on) t_timing.n_timed = n;
    }
};

bool debug_sync() {
    static const bool on = [] {
        const char* e = std::getenv("KDA_DEBUG_SYNC");
        return e && e[0] && e[0] != '0';
    }();
    return on;
}

// KDA_DEBUG_SYNC: copy the device offsets to the host and check what the
// kernels take as a precondition (0 = c_0 <= c_1 <= ... <= c_N = T).
kda_status debug_check_cu_seqlens(const int32_t* cu, int32_t N, int64_t T, hipStream_t stream) {
    if (!cu || !debug_sync()) return KDA_OK;
    std::vector<int32_t> h((size_t)N + 1);
    hipError_t e = hipMemcpyAsync(h.data(), cu, ((size_t)N + 1) * sizeof(int32_t),
                                  hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess)
        return fail(KDA_ERR_HIP, std::string("KDA_DEBUG_SYNC copy of cu_seqlens: ") + hipGetErrorString(e));
    if (h[0] != 0) return fail(KDA_ERR_INVALID_ARGUMENT, "cu_seqlens[0] must be 0");
    for (int32_t i = 0; i < N; ++i)
        if (h[i + 1] < h[i])
            return fail(KDA_ERR_INVALID_ARGUMENT,
                        "cu_seqlens must be non-decreasing (entry " + std::to_string(i + 1) + ")");
    if ((int64_t)h[N] != T)
        return fail(KDA_ERR_INVALID_ARGUMENT, "cu_seqlens[N] must equal total_tokens");
    return KDA_OK;
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
    // the larger of the two layouts, so one size serves packed and equal-row calls
    Plan a, b;
    if (dtype != KDA_DTYPE_F32 && dtype != KDA_DTYPE_BF16) return 0;
    if (!make_plan(total_tokens, num_seqs, H, dk, dv, dtype, a)) return 0;
    if (!make_plan(total_tokens, num_seqs, H, dk, dv, dtype, b, true, true)) return 0;
    return std::max(a.total, b.total);
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
    return kda::prefill_impl(q, k, v, log_alpha, beta, initial_state, cu_seqlens, total_tokens,
                             num_seqs, H, dk, dv, dtype, flags, o, final_state, chunk_states,
                             workspace, workspace_bytes, true, stream_ptr);
}

}  // extern "C"

namespace kda {

void set_last_error(const std::string& msg) { g_last_error = msg; }

kda_status prefill_impl(const void* q, const void* k, const void* v, const float* log_alpha,
                        const float* beta, const float* initial_state, const int32_t* cu_seqlens,
                        int64_t total_tokens, int32_t num_seqs, int32_t H, int32_t dk, int32_t dv,
                        kda_dtype dtype, uint32_t flags, void* o, float* final_state,
                        float* chunk_states, void* workspace, size_t workspace_bytes,
                        bool may_allocate, void* stream_ptr) {
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
        if (!workspace && !may_allocate)
            return fail(KDA_ERR_WORKSPACE, "no workspace and no allocation allowed");
        Plan plan;
        if (!make_plan(total_tokens, num_seqs, H, dk, dv, dtype, plan, true, !cu_seqlens))
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
        if (kda_status dc = debug_check_cu_seqlens(cu_seqlens, num_seqs, total_tokens, stream))
            return dc;
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
            if (cu_seqlens) {
                kda::ChunkSrc src{chunks, seq_start, -1, num_seqs, 0, 0, seq_start + num_seqs + 1};
                timer.arm();
                st = check_launch(kda::launch_chunk_table(cu_seqlens, total_tokens, num_seqs,
                                                          seq_start, chunks, (int)plan.max_chunks,
                                                          seq_start + num_seqs + 1, stream),
                                  "chunk table kernel", stream);
                timer.mark("chunk_table");
                if (st == KDA_OK && total_tokens > 0) {
                    timer.arm();
                    st = check_launch(kda::launch_prefill_intra(q, k, v, log_alpha, beta, src,
                                                                (int)plan.max_chunks, H, dk, dv,
                                                                bf16, pre_flags(flags), ws, stream),
                                      "intra-chunk kernel", stream);
                    timer.mark("prefill_intra");
                }
                if (st == KDA_OK) {
                    timer.arm();
                    st = check_launch(kda::launch_prefill_state(ws, src, initial_state, final_state,
                                                                o, chunk_states, H, dk, dv, bf16,
                                                                stream),
                                      "state kernel", stream);
                    timer.mark("prefill_state");
                }
            } else {
                // N equal rows need no chunk table: the kernels derive their chunks.
                // Segments of seg_tokens rows of every sequence, in order; the
                // state leaving one segment enters the next in fp32.
                const int rows = (int)(total_tokens / num_seqs);
                const int seg = plan.seg_tokens > 0 ? plan.seg_tokens : rows;
                float* carry = final_state ? final_state
                                           : reinterpret_cast<float*>(ws + plan.off_carry);
                int off = 0;
                do {
                    const int len = std::min(seg, rows - off);
                    const bool first = off == 0, last = off + len >= rows;
                    kda::ChunkSrc src{chunks, seq_start, len, num_seqs, rows, off};
                    if (len > 0) {
                        timer.arm();
                    st = check_launch(kda::launch_prefill_intra(q, k, v, log_alpha, beta, src,
                                                                    (int)plan.max_chunks, H, dk,
                                                                    dv, bf16, pre_flags(flags), ws,
                                                                    stream),
                                          "intra-chunk kernel", stream);
                        timer.mark("prefill_intra");
                    }
                    if (st == KDA_OK) {
                        timer.arm();
                        st = check_launch(
                            kda::launch_prefill_state(ws, src, first ? initial_state : carry,
                                                      last ? final_state : carry, o, chunk_states,
                                                      H, dk, dv, bf16, stream),
                            "state kernel", stream);
                        timer.mark("prefill_state");
                    }
                    off += len;
                } while (st == KDA_OK && off < rows);
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

}  // namespace kda

extern "C" {

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
        if (kda_status dc = debug_check_cu_seqlens(cu_seqlens, num_seqs, total_tokens, stream))
            return dc;
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
        const int rows = cu_seqlens ? -1 : (int)(total_tokens / num_seqs);
        kda::ChunkSrc src{chunks, seq_start, rows, num_seqs, rows, 0,
                          cu_seqlens ? seq_start + num_seqs + 1 : nullptr};
        kda_status st = KDA_OK;
        if (cu_seqlens)
            st = check_launch(kda::launch_chunk_table(cu_seqlens, total_tokens, num_seqs, seq_start,
                                                      chunks, (int)plan.max_chunks,
                                                      seq_start + num_seqs + 1, stream),
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
        if (st == KDA_OK && chunkwise_backward(dtype, dk, dv)) {
            // reverse-chain records over the forward's, the chain (gradient
            // leaving every chunk, and entering each sequence), then the
            // per-chunk gradients
            void* dsc = ws + b.off_dsc;
            const int mc = (int)plan.max_chunks;
            st = check_launch(kda::launch_reverse_records(q, k, v, log_alpha, beta, d_o, src, mc, H,
                                                          dk, dv, ws, stream),
                              "reverse-record kernel", stream);
            if (st == KDA_OK)
                st = check_launch(kda::launch_reverse_chain(ws, src, d_final_state, d_initial_state,
                                                            dsc, H, dk, dv, stream),
                                  "reverse chain kernel", stream);
            if (st == KDA_OK)
                st = check_launch(kda::launch_chunk_grad(q, k, v, log_alpha, beta, d_o, src, mc, H,
                                                         dk, dv, ws, cs, dsc, dq, dk_out, dv_out,
                                                         dlog_alpha, dbeta, stream),
                                  "chunk gradient kernel", stream);
        } else if (st == KDA_OK)
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
        if (kda_status dc = debug_check_cu_seqlens(cu_seqlens, num_seqs, total_tokens, stream))
            return dc;
        const int rows = cu_seqlens ? -1 : (int)(total_tokens / num_seqs);
        // Exactly one token per sequence (equal rows of one, no options): the
        // decode step's kernel, which streams the state without the token
        // loop's staging.
        if (!cu_seqlens && rows == 1 && flags == 0)
            return check_launch(kda::launch_decode_slots(state_pool, num_slots, state_indices, q, k,
                                                         v, log_alpha, beta, o, num_seqs, H, dk, dv,
                                                         dtype == KDA_DTYPE_BF16, stream),
                                "decode kernel", stream);
        return check_launch(kda::launch_recurrent(state_pool, num_slots, state_indices, q, k, v,
                                                  log_alpha, beta, cu_seqlens, rows, num_seqs, H,
                                                  dk, dv, dtype == KDA_DTYPE_BF16,
                                                  pre_flags(flags), o, stream, total_tokens),
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
    t_timing.on = enabled != 0;
    return KDA_OK;
}

int32_t kda_prefill_kernel_times(float* ms, const char** names, int32_t max_kernels) {
    const TimingState& ts = t_timing;
    if (ts.n_timed < 0) return -1;
    for (int i = 0; i < ts.n_timed && i < max_kernels; ++i) {
        float t = 0.f;
        if (hipEventSynchronize(ts.ev[2 * i + 1]) != hipSuccess) return -1;
        if (hipEventElapsedTime(&t, ts.ev[2 * i], ts.ev[2 * i + 1]) != hipSuccess) return -1;
        if (ms) ms[i] = t;
        if (names) names[i] = ts.names[i];
    }
    return ts.n_timed;
}

}  // extern "C"

namespace kda {
LaunchEvents& launch_events() { return t_launch; }
}  // namespace kda
