// chunk_table.hip -- launch plan of the chunkwise prefill, built on the device.
//
// Splits every sequence of a packed batch into chunks of up to CHUNK tokens:
// chunks restart at each sequence start, never span two sequences, and the
// last chunk of a sequence may be partial.  Outputs
//   seq_chunk_start[N+1]  exclusive prefix of chunks per sequence
//   chunks[]              (sequence, first token, length) per chunk, in order
//   seq_order[N]          the sequences longest first (a chain kernel that runs
//                         the sequences in rounds starts the long ones first,
//                         so that the short ones fill in behind them)
// Reading cu_seqlens on the device avoids a host synchronisation.
#include <hip/hip_ext.h>

#include "kda_common.h"

namespace kda {

constexpr int TABLE_THREADS = 1024;

__device__ __forceinline__ void seq_bounds(const int32_t* cu, int64_t T, int N, int s,
                                           int64_t& a, int64_t& b)
{
    if (cu) {
        a = cu[s];
        b = cu[s + 1];
    } else {
        const int64_t len = T / N;
        a = (int64_t)s * len;
        b = a + len;
    }
}

__global__ __launch_bounds__(TABLE_THREADS) void chunk_table_kernel(
    const int32_t* __restrict__ cu, int64_t T, int N, int32_t* __restrict__ seq_chunk_start,
    ChunkInfo* __restrict__ chunks, int max_chunks, int32_t* __restrict__ seq_order)
{
    __shared__ int32_t s_scan[TABLE_THREADS];
    __shared__ int32_t s_base;
    const int tid = threadIdx.x;
    if (tid == 0) s_base = 0;
    __syncthreads();

    for (int base = 0; base < N; base += TABLE_THREADS) {
        const int s = base + tid;
        int32_t n = 0;
        if (s < N) {
            int64_t a, b;
            seq_bounds(cu, T, N, s, a, b);
            n = (int32_t)((b - a + CHUNK - 1) / CHUNK);
        }
        // inclusive Hillis-Steele scan over the block
        s_scan[tid] = n;
        __syncthreads();
        for (int off = 1; off < TABLE_THREADS; off <<= 1) {
            int32_t x = tid >= off ? s_scan[tid - off] : 0;
            __syncthreads();
            s_scan[tid] += x;
            __syncthreads();
        }
        if (s < N) seq_chunk_start[s] = s_base + s_scan[tid] - n;
        __syncthreads();
        if (tid == TABLE_THREADS - 1) s_base += s_scan[tid];
        __syncthreads();
    }
    if (tid == 0) seq_chunk_start[N] = s_base;
    __threadfence_block();
    __syncthreads();

    if (seq_order) {
        if (N <= SEQ_ORDER_MAX_N) {
            // rank of every sequence by (chunk count descending, index)
            for (int s = tid; s < N; s += TABLE_THREADS) s_scan[s] = seq_chunk_start[s + 1] - seq_chunk_start[s];
            __syncthreads();
            for (int s = tid; s < N; s += TABLE_THREADS) {
                const int n = s_scan[s];
                int rank = 0;
                for (int j = 0; j < N; ++j) rank += (s_scan[j] > n || (s_scan[j] == n && j < s)) ? 1 : 0;
                seq_order[rank] = s;
            }
        } else {
            for (int s = tid; s < N; s += TABLE_THREADS) seq_order[s] = s;
        }
    }

    const int total = s_base < max_chunks ? s_base : max_chunks;
    for (int c = tid; c < total; c += TABLE_THREADS) {
        // last sequence whose first chunk is <= c (skips empty sequences)
        int lo = 0, hi = N - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (seq_chunk_start[mid] <= c) lo = mid; else hi = mid - 1;
        }
        int64_t a, b;
        seq_bounds(cu, T, N, lo, a, b);
        const int64_t first = a + (int64_t)(c - seq_chunk_start[lo]) * CHUNK;
        const int64_t rem = b - first;
        ChunkInfo ci;
        ci.seq = lo;
        ci.start = (int32_t)first;
        ci.len = (int32_t)(rem < CHUNK ? rem : CHUNK);
        ci.pad = 0;
        chunks[c] = ci;
    }
}

hipError_t launch_chunk_table(const int32_t* cu, int64_t T, int N, int32_t* seq_chunk_start,
                              ChunkInfo* chunks, int max_chunks, int32_t* seq_order,
                              hipStream_t stream)
{
    hipExtLaunchKernelGGL(chunk_table_kernel, dim3(1), dim3(TABLE_THREADS), 0, stream, launch_events().start, launch_events().stop, 0, cu, T, N,
                       seq_chunk_start, chunks, max_chunks, seq_order);
    return hipGetLastError();
}

}  // namespace kda
