/*
 * kda.h -- C ABI of libkda: Kimi Delta Attention (KDA) prefill and decode on
 * AMD MI355X (gfx950).
 *
 * The operation (Kimi Linear paper notes, section 2 "KDA recurrence"): per
 * (sequence, head) a fixed dk x dv fp32 state S is updated token by token as
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *     o_t = S_t^T q_t
 *
 * where alpha_t = exp(log_alpha_t) is a per-key-channel decay vector and
 * beta_t the write strength.  kda_prefill evaluates whole sequences with the
 * chunkwise-parallel form (paper notes, section 3: dense WY/UT form of each
 * chunk's rank-1 transitions, inter-chunk plus intra-chunk output, only the
 * fixed-size state passed between chunks); kda_decode_step applies the
 * recurrence to one token (the fused recurrent decode path).  Both compute
 * the same function.
 *
 * Conventions shared by every call
 *   Layout     dense row-major.  Tokens of all sequences are packed along the
 *              first axis; head h of token t of a [T,H,d] tensor is row
 *              (t*H + h).  The state is [N,H,dk,dv], key channel major (row c
 *              of a head's state is key channel c).
 *   Dtypes     q, k, v and o share one dtype (KDA_DTYPE_F32 or KDA_DTYPE_BF16);
 *              log_alpha, beta and states are always fp32; accumulation is fp32.
 *   Sizes      dk, dv in {64, 128} (any pairing); H >= 1; num_seqs >= 1.
 *   Alignment  every pointer 16-byte aligned.
 *   Ownership  the caller owns every buffer (device memory).  The library
 *              keeps no pointer after a call returns.
 *   Streams    work is enqueued on `stream` (a hipStream_t; NULL = the null
 *              stream).  KDA_OK means "enqueued"; faults during execution
 *              surface at the caller's next synchronisation.
 *   Errors     a call returns a status and never aborts, prints or throws.
 *              Host-checkable argument errors are reported before any HIP
 *              call is made; kda_last_error_message() gives detail (per
 *              thread).  The contents of device-resident cu_seqlens are a
 *              precondition and are not read on the host, except with the
 *              environment variable KDA_DEBUG_SYNC=1: then every call copies
 *              them, returns KDA_ERR_INVALID_ARGUMENT unless
 *              0 = c_0 <= c_1 <= ... <= c_N = T, and synchronises the stream
 *              after each kernel so that execution faults surface as
 *              KDA_ERR_HIP from the call that caused them.
 *   Threads    calls are reentrant and may come from several threads.  The
 *              library keeps no mutable state shared between threads: the
 *              error text and the optional kernel timing are per thread.
 *   Values     log_alpha must be finite and <= 0 (alpha in (0, 1]).  Within
 *              every aligned 16-token block of a 64-token chunk the summed
 *              log_alpha of one channel must stay above -80; inside that range
 *              results match the recurrence up to rounding, outside it they
 *              are unspecified.  NaN/Inf inputs propagate.
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KDA_OK = 0,
    KDA_ERR_INVALID_ARGUMENT = 1, /* NULL/misaligned pointer, bad size or dtype */
    KDA_ERR_UNSUPPORTED = 2,      /* a head size the library has no kernels for */
    KDA_ERR_WORKSPACE = 3,        /* caller workspace smaller than required     */
    KDA_ERR_HIP = 4               /* a HIP runtime call or launch failed        */
} kda_status;

typedef enum { KDA_DTYPE_F32 = 0, KDA_DTYPE_BF16 = 1 } kda_dtype;

/*
 * Input preprocessing the layer may leave to the kernels (Kimi Linear paper
 * notes, section 3 on the FLA implementation: the layer L2-normalises q and
 * k and passes beta through a sigmoid, optionally inside the kernel).  Flags
 * for kda_prefill_ex and kda_decode_tokens; any other bit is rejected.
 *   KDA_FLAG_L2NORM_QK    q_t <- q_t / sqrt(q_t . q_t + 1e-6) per (token,
 *                         head) over the dk channels, the same for k_t
 *   KDA_FLAG_BETA_SIGMOID beta holds logits x; beta_t = 1 / (1 + exp(-x))
 */
enum { KDA_FLAG_L2NORM_QK = 1u, KDA_FLAG_BETA_SIGMOID = 2u };

/*
 * Device workspace kda_prefill needs for these sizes (bytes, 256-aligned).
 * It holds one record per (chunk, head) built from the chunk intermediates of
 * the chunkwise form (paper notes, section 3 and its list of chunk
 * intermediates: g, A_qk, A_kk, w, u, decayed q and k): the chunk's state
 * transition and read-out with W and U folded in, in the dtype of q/k/v, plus
 * the chunk-end decay in fp32; and the chunk table of the batch.  Returns 0
 * for invalid sizes.
 */
size_t kda_prefill_workspace_bytes(int64_t total_tokens, int32_t num_seqs, int32_t H,
                                   int32_t dk, int32_t dv, kda_dtype dtype);

/*
 * Chunkwise prefill of a packed batch (paper notes, sections 2-3).
 *
 *   q, k          [T,H,dk] dtype; v [T,H,dv] dtype      (device, read)
 *   log_alpha     [T,H,dk] fp32, log of the per-channel decay (device, read)
 *   beta          [T,H] fp32 write strength              (device, read)
 *   initial_state [N,H,dk,dv] fp32, or NULL = zero state (device, read)
 *   cu_seqlens    [N+1] int32 offsets 0 = c_0 <= c_1 <= ... <= c_N = T
 *                 (device; zero-length sequences allowed), or NULL = N equal
 *                 contiguous sequences of T/N tokens (T % N must be 0).  The
 *                 offsets are a precondition and are not read on the host.
 *   total_tokens  T >= 0; num_seqs N >= 1
 *   o             [T,H,dv] dtype (device, written; must not alias an input)
 *   final_state   [N,H,dk,dv] fp32 (device, written), or NULL.  May be the
 *                 same buffer as initial_state (state carried in place).
 *   workspace     device buffer of at least kda_prefill_workspace_bytes(), or
 *                 NULL with workspace_bytes 0: the library then allocates and
 *                 frees one stream-ordered on `stream`.
 * A sequence of length 0 writes final_state = initial_state (or zeros).
 */
kda_status kda_prefill(const void *q, const void *k, const void *v,
                       const float *log_alpha, const float *beta,
                       const float *initial_state, const int32_t *cu_seqlens,
                       int64_t total_tokens, int32_t num_seqs, int32_t H,
                       int32_t dk, int32_t dv, kda_dtype dtype,
                       void *o, float *final_state,
                       void *workspace, size_t workspace_bytes, void *stream);

/*
 * kda_prefill without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops and
 * harnesses that forbid hipMalloc.  The call allocates nothing (no hipMalloc,
 * no stream-ordered allocation, no allocating library routine).  Its
 * workspace is a fixed array of KDA_NOALLOC_SCRATCH_BYTES in the library's
 * device code: every GPU the library is loaded on holds one copy of it from
 * module load until the process ends.
 *   Limit    sizes for which kda_prefill_workspace_bytes() exceeds
 *            KDA_NOALLOC_SCRATCH_BYTES return KDA_ERR_WORKSPACE before any
 *            HIP call (at H = 32, dk = dv = 128, bf16 that is beyond 1,280
 *            tokens of one sequence; smaller H or head sizes allow more).
 *   Sharing  every call on one GPU uses that GPU's one array and leaves its
 *            contents behind; nothing in it needs to start at zero.  Calls
 *            that overlap on one GPU (concurrent streams, or threads without
 *            an order between them) race on the array: the caller must order
 *            them, e.g. by issuing them on one stream.
 * Arguments, results and errors otherwise as for kda_prefill.
 */
#define KDA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
kda_status kda_prefill_noalloc(const void *q, const void *k, const void *v,
                               const float *log_alpha, const float *beta,
                               const float *initial_state, const int32_t *cu_seqlens,
                               int64_t total_tokens, int32_t num_seqs, int32_t H,
                               int32_t dk, int32_t dv, kda_dtype dtype,
                               void *o, float *final_state, void *stream);

/*
 * kda_prefill with options.  The extra arguments:
 *   flags         KDA_FLAG_* bits (0 = kda_prefill)
 *   chunk_states  fp32 [NC,H,dk,dv] (device, written), or NULL: the state
 *                 entering every 64-token chunk of every sequence, i.e. after
 *                 64c of its tokens for c = 0 .. ceil(len/64) - 1 (c = 0 is
 *                 the initial state).  Rows run over the sequences in order,
 *                 ceil(len_s/64) rows for sequence s (none for an empty one):
 *                 NC = sum_s ceil(len_s/64) <= ceil(T/64) + N.  With
 *                 final_state, a caller can roll back to any 64-token boundary
 *                 of a sequence and prefill again from there (paper notes,
 *                 section 3: the chunk states h of the chunkwise form).
 */
kda_status kda_prefill_ex(const void *q, const void *k, const void *v,
                          const float *log_alpha, const float *beta,
                          const float *initial_state, const int32_t *cu_seqlens,
                          int64_t total_tokens, int32_t num_seqs, int32_t H,
                          int32_t dk, int32_t dv, kda_dtype dtype, uint32_t flags,
                          void *o, float *final_state, float *chunk_states,
                          void *workspace, size_t workspace_bytes, void *stream);

/*
 * One recurrent token for each of N sequences (fused recurrent decode,
 * paper notes, section 3; the state is the only memory a KDA layer keeps per
 * sequence).  The state is updated in place:
 *
 *   state      [N,H,dk,dv] fp32 (device, read and written)
 *   q, k       [N,H,dk] dtype; v [N,H,dv] dtype (device, read)
 *   log_alpha  [N,H,dk] fp32; beta [N,H] fp32   (device, read)
 *   o          [N,H,dv] dtype (device, written; must not alias an input)
 */
kda_status kda_decode_step(float *state, const void *q, const void *k, const void *v,
                           const float *log_alpha, const float *beta,
                           int32_t num_seqs, int32_t H, int32_t dk, int32_t dv,
                           kda_dtype dtype, void *o, void *stream);

/*
 * The recurrent form over a few tokens per sequence, on pooled states
 * (paper notes, section 3: FLA's fused recurrent mode, used for short inputs
 * and decoding; one fixed-size state per sequence).  Each sequence s runs
 * its tokens in order starting from state_pool[slot_s] and leaves its final
 * state there; the state never leaves the registers in between.
 *
 *   state_pool     [num_slots,H,dk,dv] fp32 (device, read and written)
 *   num_slots      >= 1
 *   state_indices  [N] int32 slot per sequence (device), or NULL = slot s for
 *                  sequence s (then num_slots >= N).  A slot outside
 *                  [0, num_slots) marks a padding sequence: its o rows are
 *                  zeroed and no state is read or written.  Sequences must
 *                  name distinct slots (with a repeated slot the results
 *                  are undefined).
 *   q, k, v, log_alpha, beta, cu_seqlens, total_tokens, num_seqs, flags:
 *                  as for kda_prefill_ex (tokens packed, cu_seqlens NULL = N
 *                  equal rows)
 *   o              [T,H,dv] dtype (device, written)
 * Meant for short runs (speculative verification, chunked decoding).  For
 * bf16 with dk = dv = 128 and more tokens than sequences the tokens of a
 * sequence are taken 16 at a time in the chunkwise form (section 3; bf16
 * products, fp32 state, the precision of kda_prefill); otherwise they are
 * processed one by one.  One token per sequence given as equal rows
 * (cu_seqlens NULL, total_tokens = num_seqs) with no flags runs
 * kda_decode_step's kernel through the slots: with identity slots its
 * results are kda_decode_step's, bit for bit.
 */
kda_status kda_decode_tokens(float *state_pool, int32_t num_slots, const int32_t *state_indices,
                             const void *q, const void *k, const void *v,
                             const float *log_alpha, const float *beta,
                             const int32_t *cu_seqlens, int64_t total_tokens, int32_t num_seqs,
                             int32_t H, int32_t dk, int32_t dv, kda_dtype dtype,
                             uint32_t flags, void *o, void *stream);

/*
 * Device workspace kda_backward needs for these sizes (bytes, 256-aligned;
 * 0 for invalid sizes).  It covers a forward recomputation of the chunk
 * states (used when the caller passes none) and either the per-chunk records
 * and bf16 gradients leaving every chunk of the chunkwise path or the
 * per-slice partial gradients and per-workgroup scratch of the token walk.
 */
size_t kda_backward_workspace_bytes(int64_t total_tokens, int32_t num_seqs, int32_t H,
                                    int32_t dk, int32_t dv, kda_dtype dtype);

/*
 * Gradients of kda_prefill (the recurrence of paper notes section 2; the
 * FLA implementation the pages describe trains through the chunkwise form
 * with a backward pass, section 3).  For a loss L with dL/do = d_o and
 * dL/dfinal_state = d_final_state it writes dL/dq, dL/dk, dL/dv, dL/dlog_alpha,
 * dL/dbeta and dL/dinitial_state.
 *
 *   q, k, v, log_alpha, beta, initial_state, cu_seqlens, total_tokens,
 *   num_seqs, H, dk, dv, dtype   as for kda_prefill (the forward's inputs;
 *                 no preprocessing flags: the gradients are with respect to
 *                 the q, k and beta the recurrence sees)
 *   d_o           [T,H,dv] dtype (device, read)
 *   d_final_state [N,H,dk,dv] fp32, or NULL = zero
 *   chunk_states  the forward's chunk states as kda_prefill_ex writes them
 *                 ([NC,H,dk,dv] fp32), or NULL: recomputed here
 *   dq, dk_out    [T,H,dk] dtype; dv_out [T,H,dv] dtype (device, written)
 *   dlog_alpha    [T,H,dk] fp32; dbeta [T,H] fp32 (device, written)
 *   d_initial_state [N,H,dk,dv] fp32 (device, written), or NULL
 *   workspace     at least kda_backward_workspace_bytes(), or NULL with 0
 *                 (then allocated stream-ordered on `stream`)
 * Outputs must not alias inputs.  The result is deterministic.  bf16 with
 * dk = dv = 128 runs the chunkwise backward: a reverse pass over the chunks
 * (the transpose of each chunk's transition, from the last chunk to the
 * first) gives the gradient leaving every chunk, then every chunk's input
 * gradients are formed in parallel from its entry state and that gradient.
 * Other configurations walk the tokens backwards (recomputed forward from the
 * chunk states, 8 tokens at a time).  KDA_BACKWARD_SERIAL=1 in the
 * environment selects the token walk for bf16 too.
 */
kda_status kda_backward(const void *q, const void *k, const void *v,
                        const float *log_alpha, const float *beta,
                        const float *initial_state, const int32_t *cu_seqlens,
                        int64_t total_tokens, int32_t num_seqs, int32_t H,
                        int32_t dk, int32_t dv, kda_dtype dtype,
                        const void *d_o, const float *d_final_state, const float *chunk_states,
                        void *dq, void *dk_out, void *dv_out, float *dlog_alpha, float *dbeta,
                        float *d_initial_state, void *workspace, size_t workspace_bytes,
                        void *stream);

/* Static description of a status code. */
const char *kda_status_string(kda_status status);

/* Detail of the last non-OK status returned on the calling thread ("" if none). */
const char *kda_last_error_message(void);

/* Library version, major*10000 + minor*100 + patch. */
int32_t kda_version(void);

/*
 * Kernel timing for measurement (not needed for normal use), per calling
 * thread.  While enabled on a thread, kda_prefill called from that thread
 * has each of its kernels record its own start and end in a pair of HIP
 * events (hipExtLaunchKernelGGL; timing-only events without a system-scope
 * fence, created on first use and kept until the process ends), so a
 * kernel's time excludes the gap to the work queued before it.
 * kda_prefill_kernel_times() waits for the events of the last call timed on
 * the calling thread and writes, for up to max_kernels kernels in launch
 * order, the elapsed milliseconds (ms) and a static kernel name (names, may
 * be NULL).  It returns the number of kernels of that call, or -1 when
 * nothing was recorded on this thread or a HIP call failed.
 */
kda_status kda_set_kernel_timing(int32_t enabled);
int32_t kda_prefill_kernel_times(float *ms, const char **names, int32_t max_kernels);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
