// kda_launch.h -- host-visible launchers of the libkda kernels and the chunk
// descriptor they share (no device code; included by the host API).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace kda {

constexpr int CHUNK = 64;  // tokens per chunk of the chunkwise prefill

// Chunk descriptor produced by the chunk-table kernel.
struct ChunkInfo {
    int32_t seq;    // sequence index
    int32_t start;  // first token (packed row index)
    int32_t len;    // 1..CHUNK
    int32_t pad;
};

hipError_t launch_chunk_table(const int32_t* cu, int64_t T, int N, int32_t* seq_chunk_start,
                              ChunkInfo* chunks, int max_chunks, hipStream_t stream);

// bufs: W, Qg, Kh, Aqk, Ut, gC (per-chunk intermediates in the workspace)
hipError_t launch_prefill_intra(const void* q, const void* k, const void* v, const float* la,
                                const float* beta, const ChunkInfo* chunks,
                                const int32_t* n_chunks, int max_chunks, int H, int dk, int dv,
                                bool bf16_io, void* const* bufs, hipStream_t stream);

hipError_t launch_prefill_state(void* const* bufs, const int32_t* seq_chunk_start,
                                const ChunkInfo* chunks, const float* S0, float* S_final,
                                void* o, int N, int H, int dk, int dv, bool bf16_io,
                                hipStream_t stream);

hipError_t launch_decode_step(float* state, const void* q, const void* k, const void* v,
                              const float* la, const float* beta, void* o, int units, int dk,
                              int dv, bool bf16_io, hipStream_t stream);

}  // namespace kda
