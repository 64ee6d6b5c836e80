// kda_noalloc.hip -- kda_prefill_noalloc: kda_prefill whose workspace (the
// per-(chunk, head) records and the chunk table) lives in a fixed device array
// of this library instead of a caller buffer or a stream-ordered allocation.
//
// The array is a file-scope __device__ object: each GPU the library is loaded
// on holds its own copy from module load until the process ends.  Host code
// never passes the array's name to a kernel (in host code that name is only a
// stand-in); the first call on a device looks up the device address with
// hipGetSymbolAddress, with that device current, and keeps it per device.
// Nothing in the workspace has to start at zero: the chunk-table and
// intra-chunk kernels write every byte the sequential kernel reads.
#include <hip/hip_runtime.h>

#include <mutex>
#include <string>

#include "../../include/kda.h"
#include "kda_internal.h"

namespace {

__device__ __align__(256) unsigned char scratch[KDA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

kda_status fail(kda_status s, const std::string& msg) {
    kda::set_last_error(msg);
    return s;
}

// Device address of `scratch` on the device that `stream` belongs to.
kda_status scratch_for(hipStream_t stream, void** out) {
    int dev = -1;
    hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess)
        return fail(KDA_ERR_HIP, std::string("device of the stream: ") + hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(KDA_ERR_UNSUPPORTED, "device index too large");
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        int cur = -1;
        e = hipGetDevice(&cur);
        if (e == hipSuccess && cur != dev) e = hipSetDevice(dev);
        void* p = nullptr;
        if (e == hipSuccess) e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur >= 0 && cur != dev) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess || !p)
            return fail(KDA_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") +
                                         hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return KDA_OK;
}

}  // namespace

extern "C" kda_status kda_prefill_noalloc(const void* q, const void* k, const void* v,
                                          const float* log_alpha, const float* beta,
                                          const float* initial_state, const int32_t* cu_seqlens,
                                          int64_t total_tokens, int32_t num_seqs, int32_t H,
                                          int32_t dk, int32_t dv, kda_dtype dtype, void* o,
                                          float* final_state, void* stream_ptr) {
    try {
        // sizes first, on the host: the fixed array bounds what a call may need
        const size_t need = kda_prefill_workspace_bytes(total_tokens, num_seqs, H, dk, dv, dtype);
        if (need > KDA_NOALLOC_SCRATCH_BYTES)
            return fail(KDA_ERR_WORKSPACE,
                        "kda_prefill_noalloc: these sizes need " + std::to_string(need) +
                            " bytes of workspace; the fixed scratch array holds " +
                            std::to_string((size_t)KDA_NOALLOC_SCRATCH_BYTES) +
                            " (use kda_prefill with a workspace)");
        if (need == 0)   // invalid sizes or dtype: the full validation reports which
            return kda::prefill_impl(q, k, v, log_alpha, beta, initial_state, cu_seqlens,
                                     total_tokens, num_seqs, H, dk, dv, dtype, 0u, o, final_state,
                                     nullptr, nullptr, 0, false, stream_ptr);
        void* ws = nullptr;
        if (kda_status st = scratch_for(reinterpret_cast<hipStream_t>(stream_ptr), &ws)) return st;
        return kda::prefill_impl(q, k, v, log_alpha, beta, initial_state, cu_seqlens,
                                 total_tokens, num_seqs, H, dk, dv, dtype, 0u, o, final_state,
                                 nullptr, ws, KDA_NOALLOC_SCRATCH_BYTES, false, stream_ptr);
    } catch (...) {
        return fail(KDA_ERR_HIP, "unexpected C++ exception inside kda_prefill_noalloc");
    }
}
