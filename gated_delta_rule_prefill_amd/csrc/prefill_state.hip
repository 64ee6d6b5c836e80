// prefill_state.hip -- sequential inter-chunk pass of the chunkwise KDA prefill.
//
// Only the fixed dk x dv state crosses chunk boundaries (Kimi Linear paper
// notes, section 3).  With the per-chunk W, U, Khat, Qg, A_qk and gamma_C from
// the intra kernel, each chunk in order applies
//
//   N = U - W S                    (values corrected by what S already predicts)
//   O = Qg S + A_qk N              (inter-chunk read-out + intra-chunk causal part)
//   S = Diag(gamma_C) S + Khat^T N
//
// One workgroup per (sequence, head, 16 value columns): the columns of S evolve
// independently, so a head's state is split over DV/16 workgroups that never
// communicate.  Roles inside the workgroup:
//   wave 0   the serial chain N, then S; it keeps the fp32 state tile (DK x 16)
//            in MFMA accumulator registers for the whole sequence;
//   wave 1   the output O of the same chunk, from the chunk-start state and N
//            that wave 0 hands over through a small LDS area;
//   wave 2   stages W into an LDS double buffer and touches the operands a
//            few chunks ahead so they sit in L2.
// Waves 0 and 1 load their other operand fragments straight from L2 into
// registers one chunk ahead (two register sets, loop unrolled by two).  The
// split keeps every wave under the 63 vector-memory operations one wave may
// have in flight, so loads for the next chunk never stall the current one.
//
// Every product takes its register-resident operand (S or N) straight from
// accumulator tiles: a 16x16 tile gives lane group g rows 4g..4g+3, the slot
// set that the perm32 storage order of W, Qg, Khat^T and A_qk matches.
#include "kda_common.h"

namespace kda {

constexpr int PREFETCH_DIST = 3;   // chunks between the L2 touch and the register load

template <typename E, int DK, int DV>
struct StateCfg {
    static constexpr int ES = sizeof(E);
    static constexpr int KS = DK / 32;   // contraction steps over key channels
    static constexpr int KT = DK / 16;   // accumulator tiles of S
    static constexpr int NSL = DV / 16;  // value slices per head
    static constexpr int FRAG = 8 * ES;  // bytes of one operand fragment per lane
    static constexpr int XFER = (KS + 2) * 64 * FRAG;   // chunk-start S and N
    static constexpr int W_RS = DK * ES + 16;           // padded LDS row stride of W
    static constexpr int W_BYTES = CHUNK * W_RS;
    static constexpr int W_UNITS = CHUNK * DK * ES / 16;
    static constexpr int W_PER_LANE = W_UNITS / 64;     // 16-byte units per loader lane
    static constexpr RecLayout RL = rec_layout(ES, DK, DV);
    static constexpr int LINES = (int)((RL.bytes + 127) / 128);
    // Two register sets of operands (load one chunk ahead) unless that would
    // spill: fp32 operands at dk = 128 use one set loaded at the chunk start.
    static constexpr bool TWO_SETS = ES == 2 || DK == 64;
};

// Operands of one chunk as seen by the serial wave (this lane's fragments).
template <typename E, int DK>
struct SerialOps {
    typename Vec<E>::v8 k[DK / 16][2];   // Khat^T rows 16t + ln
    f32x4 gc[DK / 16];                   // gamma_C rows 16t + 4g .. +3
    typename Vec<E>::v4 u[4];            // U^T[j0 + ln][16R + 4g .. +3]
};

// Operands of one chunk as seen by the output wave.
template <typename E, int DK>
struct OutputOps {
    typename Vec<E>::v8 q[4][DK / 32];   // Qg rows 16R + ln
    typename Vec<E>::v8 a[4][2];         // A_qk rows 16R + ln (steps ks <= R/2)
    int start, len;
};

template <typename E, int DK, int DV>
__device__ __forceinline__ void load_serial(SerialOps<E, DK>& op, const unsigned char* r, int g,
                                            int ln, int j0)
{
    using C = StateCfg<E, DK, DV>;
    using V8 = typename Vec<E>::v8;
    using V4 = typename Vec<E>::v4;
    const E* K = reinterpret_cast<const E*>(r + C::RL.k);
    const float* G = reinterpret_cast<const float*>(r + C::RL.g);
    const E* U = reinterpret_cast<const E*>(r + C::RL.u);
#pragma unroll
    for (int t = 0; t < C::KT; ++t) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) op.k[t][ks] = load_vec<V8>(K + (16 * t + ln) * CHUNK + 32 * ks + 8 * g);
        op.gc[t] = load_vec<f32x4>(G + 16 * t + 4 * g);
    }
#pragma unroll
    for (int R = 0; R < 4; ++R) op.u[R] = load_vec<V4>(U + (j0 + ln) * CHUNK + 16 * R + 4 * g);
}

template <typename E, int DK, int DV>
__device__ __forceinline__ void load_output(OutputOps<E, DK>& op, const unsigned char* r,
                                            const ChunkInfo* ci, int g, int ln)
{
    using C = StateCfg<E, DK, DV>;
    using V8 = typename Vec<E>::v8;
    const E* Q = reinterpret_cast<const E*>(r + C::RL.q);
    const E* A = reinterpret_cast<const E*>(r + C::RL.a);
#pragma unroll
    for (int R = 0; R < 4; ++R) {
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) op.q[R][ks] = load_vec<V8>(Q + (16 * R + ln) * DK + 32 * ks + 8 * g);
#pragma unroll
        for (int ks = 0; ks <= R / 2; ++ks) op.a[R][ks] = load_vec<V8>(A + (16 * R + ln) * CHUNK + 32 * ks + 8 * g);
    }
    op.start = ci->start;
    op.len = ci->len;
}

// Workgroups are grouped so that the DV/16 slices of one (sequence, head)
// have block indices congruent mod 8: blocks are dispatched round-robin over
// the 8 XCDs, so the slices that read the same chunk operands share one L2.
template <typename E, int DK, int DV>
__global__ __launch_bounds__(192) __attribute__((amdgpu_waves_per_eu(1, 1))) void prefill_state_kernel(
    const unsigned char* __restrict__ rec, const int32_t* __restrict__ seq_chunk_start,
    const ChunkInfo* __restrict__ chunks, const float* __restrict__ S0,
    float* __restrict__ S_final, E* __restrict__ o, int H, int n_pairs)
{
    using C = StateCfg<E, DK, DV>;
    using V4 = typename Vec<E>::v4;
    using V8 = typename Vec<E>::v8;
    constexpr int KS = C::KS, KT = C::KT, NSL = C::NSL;

    __shared__ __attribute__((aligned(16))) unsigned char xfer[C::XFER];
    __shared__ __attribute__((aligned(16))) unsigned char wbuf[2 * C::W_BYTES];

    const int b = blockIdx.x;
    const int xcd = b & 7, q8 = b >> 3;
    const int grp = q8 / NSL, slice = q8 % NSL;
    const int pair = grp * 8 + xcd;
    if (pair >= n_pairs) return;
    const int s = pair / H, h = pair % H;
    const int tid = threadIdx.x, wave = tid >> 6;
    const int l = tid & 63, g = l >> 4, ln = l & 15;
    const int j0 = slice * 16;
    const int c_begin = seq_chunk_start[s], c_end = seq_chunk_start[s + 1];
    const size_t sbase = (size_t)pair * DK * DV;
    auto record = [&](int cid) { return rec + ((size_t)cid * H + h) * C::RL.bytes; };
    E* xS = reinterpret_cast<E*>(xfer);                      // [KS][64 lanes][8]
    E* xN = reinterpret_cast<E*>(xfer + KS * 64 * C::FRAG);  // [2][64 lanes][8]

    if (wave == 0) {
        // ------------------------------------------------ serial wave
        f32x4 S[KT];
#pragma unroll
        for (int t = 0; t < KT; ++t) S[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (S0) {
#pragma unroll
            for (int t = 0; t < KT; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    S[t][i] = S0[sbase + (size_t)(16 * t + 4 * g + i) * DV + j0 + ln];
        }
        SerialOps<E, DK> opA, opB;
        if (C::TWO_SETS && c_begin < c_end) load_serial<E, DK, DV>(opA, record(c_begin), g, ln, j0);
        __syncthreads();   // W of the first chunk is in LDS

        auto step = [&](SerialOps<E, DK>& cur, SerialOps<E, DK>& nxt, int cid) {
            // The next chunk's loads are unconditional (the last chunk reloads
            // itself) so no branch makes the wait counters conservative.
            __builtin_amdgcn_sched_barrier(0);   // keep each chunk's work inside its step
            if constexpr (!C::TWO_SETS) load_serial<E, DK, DV>(cur, record(cid), g, ln, j0);
            else load_serial<E, DK, DV>(nxt, record(min(cid + 1, c_end - 1)), g, ln, j0);
            // S as an MFMA operand: slots of step ks = rows {32ks+4g..+3, 32ks+16+4g..+3}
            V8 Sf[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    Sf[ks][i] = from_f32<E>(S[2 * ks][i]);
                    Sf[ks][4 + i] = from_f32<E>(S[2 * ks + 1][i]);
                }
                store_vec(xS + (ks * 64 + l) * 8, Sf[ks]);
            }
            // N = U - W S   (N tile R: lane holds N[16R + 4g + i][j0 + ln])
            const unsigned char* wb = wbuf + ((cid - c_begin) & 1) * C::W_BYTES + ln * C::W_RS + 8 * g * C::ES;
            V8 wf[4][KS];
#pragma unroll
            for (int R = 0; R < 4; ++R)
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    wf[R][ks] = load_vec<V8>(reinterpret_cast<const E*>(wb + 16 * R * C::W_RS + 32 * ks * C::ES));
            f32x4 N[4];
#pragma unroll
            for (int R = 0; R < 4; ++R) N[R] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int R = 0; R < 4; ++R) N[R] = mma32(wf[R][ks], Sf[ks], N[R]);
            V8 Nf[2];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    Nf[ks][i] = from_f32<E>(to_f32(cur.u[2 * ks][i]) - N[2 * ks][i]);
                    Nf[ks][4 + i] = from_f32<E>(to_f32(cur.u[2 * ks + 1][i]) - N[2 * ks + 1][i]);
                }
                store_vec(xN + (ks * 64 + l) * 8, Nf[ks]);
            }
            __syncthreads();   // A: chunk-start S and N handed to the output wave
            // S = Diag(gamma_C) S + Khat^T N
#pragma unroll
            for (int t = 0; t < KT; ++t) S[t] *= cur.gc[t];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int t = 0; t < KT; ++t) S[t] = mma32(cur.k[t][ks], Nf[ks], S[t]);
            __syncthreads();   // B: the hand-over area is free again
            __builtin_amdgcn_sched_barrier(0);
        };
        int cid = c_begin;
        if constexpr (C::TWO_SETS) {
            for (; cid + 1 < c_end; cid += 2) {
                step(opA, opB, cid);
                step(opB, opA, cid + 1);
            }
        }
        for (; cid < c_end; ++cid) step(opA, opB, cid);

        if (S_final) {
#pragma unroll
            for (int t = 0; t < KT; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    S_final[sbase + (size_t)(16 * t + 4 * g + i) * DV + j0 + ln] = S[t][i];
        }
    } else if (wave == 1) {
        // ------------------------------------------------ output wave
        OutputOps<E, DK> opA, opB;
        if (C::TWO_SETS && c_begin < c_end) load_output<E, DK, DV>(opA, record(c_begin), chunks + c_begin, g, ln);
        __syncthreads();   // W of the first chunk is in LDS

        auto step = [&](OutputOps<E, DK>& cur, OutputOps<E, DK>& nxt, int cid) {
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (!C::TWO_SETS) load_output<E, DK, DV>(cur, record(cid), chunks + cid, g, ln);
            else {
                const int nx = min(cid + 1, c_end - 1);
                load_output<E, DK, DV>(nxt, record(nx), chunks + nx, g, ln);
            }
            __syncthreads();   // A
            V8 Sf[KS], Nf[2];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) Sf[ks] = load_vec<V8>(xS + (ks * 64 + l) * 8);
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) Nf[ks] = load_vec<V8>(xN + (ks * 64 + l) * 8);
            __syncthreads();   // B
            // O^T = S_start^T Qg^T + N^T A_qk^T   (tile R: lane holds O[16R + ln][j0 + 4g + i])
            f32x4 O[4];
#pragma unroll
            for (int R = 0; R < 4; ++R) O[R] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int R = 0; R < 4; ++R) O[R] = mma32(Sf[ks], cur.q[R][ks], O[R]);
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int R = 2 * ks; R < 4; ++R) O[R] = mma32(Nf[ks], cur.a[R][ks], O[R]);
#pragma unroll
            for (int R = 0; R < 4; ++R) {
                const int r = 16 * R + ln;
                if (r < cur.len) {
                    V4 w;
#pragma unroll
                    for (int i = 0; i < 4; ++i) w[i] = from_f32<E>(O[R][i]);
                    store_vec(o + ((size_t)(cur.start + r) * H + h) * DV + j0 + 4 * g, w);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        };
        int cid = c_begin;
        if constexpr (C::TWO_SETS) {
            for (; cid + 1 < c_end; cid += 2) {
                step(opA, opB, cid);
                step(opB, opA, cid + 1);
            }
        }
        for (; cid < c_end; ++cid) step(opA, opB, cid);
    } else {
        // ------------------------------------------------ W stager / L2 prefetch wave
        // W of chunk c sits in wbuf[c & 1] from barrier B of chunk c-1 on; the
        // stager holds chunk c+1 in registers and commits it during chunk c.
        // Each of the NSL slices of a head also touches every NSL-th 128-byte
        // line of the record PREFETCH_DIST chunks ahead; together they cover it.
        f32x4 wr[C::W_PER_LANE];
        auto wload = [&](int cid) {
            const f32x4* src = reinterpret_cast<const f32x4*>(record(cid) + C::RL.w);
#pragma unroll
            for (int i = 0; i < C::W_PER_LANE; ++i) wr[i] = src[l + 64 * i];
        };
        auto wcommit = [&](int it) {
            unsigned char* dst = wbuf + (it & 1) * C::W_BYTES;
            constexpr int UPR = DK * C::ES / 16;   // 16-byte units per row
#pragma unroll
            for (int i = 0; i < C::W_PER_LANE; ++i) {
                const int x = l + 64 * i;
                *reinterpret_cast<f32x4*>(dst + (x / UPR) * C::W_RS + 16 * (x % UPR)) = wr[i];
            }
        };
        if (c_begin < c_end) {
            wload(c_begin);
            wcommit(0);
            wload(min(c_begin + 1, c_end - 1));
        }
        __syncthreads();   // W of the first chunk is in LDS
        uint32_t sink = 0;
        for (int cid = c_begin; cid < c_end; ++cid) {
            const int it = cid - c_begin;
            const int pf = cid + PREFETCH_DIST;
            if (pf < c_end) {
                const unsigned char* r = record(pf);
                for (int line = slice + NSL * l; line < C::LINES; line += NSL * 64)
                    sink ^= *reinterpret_cast<const uint32_t*>(r + 128 * line);
            }
            __syncthreads();   // A
            if (cid + 1 < c_end) {
                wcommit(it + 1);                       // buffer freed by barrier B of chunk c-1
                wload(min(cid + 2, c_end - 1));
            }
            __syncthreads();   // B
        }
        if (n_pairs < 0) o[0] = from_f32<E>((float)sink);   // keeps the touches alive; never taken
    }
}

template <typename E, int DK, int DV>
static hipError_t launch_state_t(const void* rec, const int32_t* seq_chunk_start,
                                 const ChunkInfo* chunks, const float* S0, float* S_final,
                                 void* o, int N, int H, hipStream_t stream)
{
    const int n_pairs = N * H;
    const int groups = (n_pairs + 7) / 8;
    const long long blocks = (long long)groups * 8 * (DV / 16);
    hipLaunchKernelGGL((prefill_state_kernel<E, DK, DV>), dim3((unsigned)blocks), dim3(192), 0,
                       stream, (const unsigned char*)rec, seq_chunk_start, chunks, S0, S_final,
                       (E*)o, H, n_pairs);
    return hipGetLastError();
}

hipError_t launch_prefill_state(const void* rec, const int32_t* seq_chunk_start,
                                const ChunkInfo* chunks, const float* S0, float* S_final,
                                void* o, int N, int H, int dk, int dv, bool bf16_io,
                                hipStream_t stream)
{
#define KDA_STATE_CASE(E, DK_, DV_) \
    if (dk == DK_ && dv == DV_)     \
        return launch_state_t<E, DK_, DV_>(rec, seq_chunk_start, chunks, S0, S_final, o, N, H, stream);
    if (bf16_io) {
        KDA_STATE_CASE(bf16, 128, 128)
        KDA_STATE_CASE(bf16, 64, 64)
        KDA_STATE_CASE(bf16, 128, 64)
        KDA_STATE_CASE(bf16, 64, 128)
    } else {
        KDA_STATE_CASE(float, 128, 128)
        KDA_STATE_CASE(float, 64, 64)
        KDA_STATE_CASE(float, 128, 64)
        KDA_STATE_CASE(float, 64, 128)
    }
#undef KDA_STATE_CASE
    return hipErrorInvalidValue;
}

}  // namespace kda
