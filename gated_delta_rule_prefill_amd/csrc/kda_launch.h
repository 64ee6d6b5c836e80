// kda_launch.h -- host-visible launchers of the libkda kernels and the chunk
// descriptor they share (no device code; included by the host API).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace kda {

// Events that time the calling thread's next prefill kernel (set by the C ABI
// while kernel timing is on, both NULL otherwise): the launchers hand them to
// hipExtLaunchKernelGGL, which records the kernel's own start and end in them.
struct LaunchEvents {
    hipEvent_t start = nullptr, stop = nullptr;
};
LaunchEvents& launch_events();

constexpr int CHUNK = 64;  // tokens per chunk of the chunkwise prefill

// Chunk descriptor produced by the chunk-table kernel.
struct ChunkInfo {
    int32_t seq;    // sequence index
    int32_t start;  // first token (packed row index)
    int32_t len;    // 1..CHUNK
    int32_t pad;
};

// Where the kernels find the chunks of a batch: the chunk table (packed
// batches, rows < 0), or N equal sequences of `rows` tokens each, whose chunks
// follow arithmetically (no table, no extra kernel).
//
// In rows mode a launch may cover one token range [offset, offset + rows) of
// every sequence (the prefill processes long equal-row batches in such
// segments): sequence s's rows start at s * stride, and its chunk c in the
// launch is its chunk offset / CHUNK + c overall.
struct ChunkSrc {
    const ChunkInfo* chunks;          // [max_chunks], table mode
    const int32_t* seq_chunk_start;   // [N + 1], table mode
    int rows;                         // >= 0: tokens per sequence in this launch; < 0: table mode
    int N;
    int stride;                       // rows mode: tokens from one sequence to the next
    int offset;                       // rows mode: first token of the launch in each sequence
    const int32_t* seq_order = nullptr;   // table mode: the sequences longest first, or NULL
};

// Per-(chunk, head) record of the chunk intermediates in the workspace
// (byte offsets; es = element size of q/k/v, 2 or 4).  With entry state S,
// a chunk's state update and output are
//     S_next = Diag(gC) S + PM S + Hc,      O = QM S + OI
// (the chunk's transition and read-out folded in by the intra kernel):
//   PM   dk x dk    -Khat^T W, columns in perm32 order, stored in fragment
//                   order (frag_at: the A operands of the state product)
//   HCt  dv x dk    (Khat^T U)^T, columns in perm32 order, in planar fragment
//                   order: fragment (value slice j/16, block c/32); a value
//                   slice's fragments are one contiguous run
//   QM   [64][dk]   Qg - A_qk W, columns in perm32 order (row-major: it is
//                   written from the row mapping, where a row is contiguous)
//   OI   64 x dv    A_qk U, columns in perm32 order, in planar fragment order
//                   (slots 0..3 of the 64 lanes, then 4..7: value slice 2m is
//                   plane 0 of block m, slice 2m + 1 plane 1)
//   gC   [dk] fp32  e^{g_C}
struct RecLayout {
    size_t pm, hc, qm, oi, g, bytes;
};
constexpr RecLayout rec_layout(int es, int dk, int dv) {
    return RecLayout{0,
                     (size_t)dk * dk * es,
                     (size_t)dk * dk * es + (size_t)dv * dk * es,
                     (size_t)dk * dk * es + (size_t)dv * dk * es + (size_t)CHUNK * dk * es,
                     (size_t)dk * dk * es + (size_t)dv * dk * es + (size_t)CHUNK * dk * es +
                         (size_t)CHUNK * dv * es,
                     ((size_t)dk * dk * es + (size_t)dv * dk * es + (size_t)CHUNK * dk * es +
                      (size_t)CHUNK * dv * es + (size_t)dk * 4 + 255) & ~(size_t)255};
}

// Input preprocessing options (bits): L2-normalise q and k per (token, head);
// beta arrives as a logit and goes through a sigmoid.
constexpr unsigned PRE_L2NORM_QK = 1u, PRE_BETA_LOGIT = 2u;

// seq_order (or NULL): [N] the sequences by descending chunk count (ties by
// index) for N <= SEQ_ORDER_MAX_N, else in index order.
constexpr int SEQ_ORDER_MAX_N = 1024;
hipError_t launch_chunk_table(const int32_t* cu, int64_t T, int N, int32_t* seq_chunk_start,
                              ChunkInfo* chunks, int max_chunks, int32_t* seq_order,
                              hipStream_t stream);

// rec: [max_chunks * H] records of rec_layout() bytes
hipError_t launch_prefill_intra(const void* q, const void* k, const void* v, const float* la,
                                const float* beta, ChunkSrc src, int max_chunks, int H, int dk,
                                int dv, bool bf16_io, unsigned flags, void* rec,
                                hipStream_t stream);

// Sequential inter-chunk pass; it also forms every chunk's output O = QM S_c + OI.
// chunk_states (or NULL): every chunk-start state in fp32, [chunk][H][dk][dv].
hipError_t launch_prefill_state(const void* rec, ChunkSrc src, const float* S0, float* S_final,
                                void* o, float* chunk_states, int H, int dk, int dv, bool bf16_io,
                                hipStream_t stream);

// The same pass over two value slices per workgroup (bf16, dk = 128,
// dv = 64 or 128; see prefill_chain.hip).
hipError_t launch_prefill_chain2(const void* rec, ChunkSrc src, const float* S0, float* S_final,
                                 void* o, float* chunk_states, int H, int dk, int dv,
                                 hipStream_t stream);

// The backward pass's reverse chain (bf16, dk = dv = 128).  Records: for each
// (chunk, head) PM^T in PM's place, E = QM^T dO in Hc's place, gamma_C (intra
// kernel in its reverse-record mode, d_o the output gradient).  The chain
// then runs dS_in = Diag(gamma_C) dS + PM^T dS + E from the last chunk of
// each sequence to the first, starting from dS_last (the final-state
// gradient, NULL = 0); dS_chunks receives the gradient leaving every chunk
// ([chunk][H][dk][dv] bf16, chunk-state rows) and dS_first (or NULL, fp32)
// the gradient entering each sequence's first chunk.
hipError_t launch_reverse_records(const void* q, const void* k, const void* v, const float* la,
                                  const float* beta, const void* d_o, ChunkSrc src, int max_chunks,
                                  int H, int dk, int dv, void* rec, hipStream_t stream);
hipError_t launch_reverse_chain(const void* rec, ChunkSrc src, const float* dS_last,
                                float* dS_first, void* dS_chunks, int H, int dk, int dv,
                                hipStream_t stream);

// Per-chunk gradients of the chunkwise backward (bf16, dk = dv = 128): rec
// holds the reverse-chain records (for X, X^T and A_qk^T), chunk_states the
// state entering every chunk ([chunk][H][dk][dv] fp32) and dS_chunks the
// gradient leaving it ([chunk][H][dk][dv] bf16; rows = table chunks).  Writes
// dq, dk, dv, dlog_alpha and dbeta of every token.
hipError_t launch_chunk_grad(const void* q, const void* k, const void* v, const float* la,
                             const float* beta, const void* d_o, ChunkSrc src, int max_chunks,
                             int H, int dk, int dv, const void* rec, const float* chunk_states,
                             const void* dS_chunks, void* dq, void* dk_out, void* dv_out,
                             float* dla, float* dbeta, hipStream_t stream);

// Whether a configuration runs the LDS-ring sequential kernel (its ring fits),
// or the register-staged one (fp32 with dk = 128).
constexpr bool uses_ring_kernel(bool bf16_io, int dk) { return bf16_io || dk == 64; }

// Pooled paths walk the pool's slots in order (states streamed in address
// order) when the batch has at most this many sequences and the pool at most
// twice as many slots; otherwise they walk the sequences.
constexpr int SLOT_ORDER_MAX_SEQS = 4096;

// Recurrent tokens of a packed batch on pooled states (see kda_decode_tokens).
hipError_t launch_recurrent(float* pool, int num_slots, const int32_t* slots, const void* q,
                            const void* k, const void* v, const float* la, const float* beta,
                            const int32_t* cu, int rows, int N, int H, int dk, int dv,
                            bool bf16_io, unsigned flags, void* o, hipStream_t stream, int64_t T);

// Gradients of the recurrence (see backward.hip).  chunk_states: the fp32
// state entering every chunk, as kda_prefill_ex exports them.  part: the
// backward_partial_bytes() area; scratch: backward_scratch_bytes().
size_t backward_partial_bytes(int64_t T, int H, int dk, int dv);
size_t backward_scratch_bytes(int N, int H, int dk, int dv);
hipError_t launch_backward(const void* q, const void* k, const void* v, const float* la,
                           const float* beta, ChunkSrc src, const float* chunk_states,
                           const void* d_o, const float* d_final, int H, int64_t T, int dk, int dv,
                           bool bf16_io, void* dq, void* dk_out, void* dv_out, float* dla,
                           float* dbeta, float* d_initial, float* part, float* scratch,
                           hipStream_t stream);

hipError_t launch_decode_step(float* state, const void* q, const void* k, const void* v,
                              const float* la, const float* beta, void* o, int units, int dk,
                              int dv, bool bf16_io, hipStream_t stream);

// One token for each of N sequences on pooled states through slot indices
// (NULL = slot s for sequence s; a slot outside [0, num_slots) pads): the
// decode step's kernel with slot indirection.
hipError_t launch_decode_slots(float* pool, int num_slots, const int32_t* slots, const void* q,
                               const void* k, const void* v, const float* la, const float* beta,
                               void* o, int N, int H, int dk, int dv, bool bf16_io,
                               hipStream_t stream);

}  // namespace kda
