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
// communicate.  Wave 0 computes; it keeps the fp32 state tile (DK x 16) in MFMA
// accumulator registers for the whole sequence.  Waves 1-3 stage the next
// chunk's operands into an LDS double buffer while wave 0 works on the current
// one, so the serial loop never waits on HBM/L2 latency.
//
// Every product takes its register-resident operand (S or N) straight from
// accumulator tiles: a 16x16 tile gives lane group g rows 4g..4g+3, the slot
// set that the perm32 storage order of W, Qg, Khat^T and A_qk matches.
#include "kda_common.h"

namespace kda {

template <typename E>
struct ChunkBufsC {
    const E* W;
    const E* Qg;
    const E* Kh;
    const E* Aqk;
    const E* Ut;
    const float* gC;
};

// LDS image of one chunk's operands.  Rows are XOR-swizzled in 16-byte units
// so that the 16 rows a ds_read_b128 touches fall in distinct banks.
template <typename E, int DK, int DV>
struct StateLayout {
    static constexpr int ES = sizeof(E);
    static constexpr int W_RB = DK * ES;                    // row bytes of W / Qg
    static constexpr int K_RB = CHUNK * ES;                 // row bytes of Khat^T / A_qk / U^T
    static constexpr int OFF_W = 0;
    static constexpr int OFF_Q = OFF_W + CHUNK * W_RB;
    static constexpr int OFF_K = OFF_Q + CHUNK * W_RB;
    static constexpr int OFF_A = OFF_K + DK * K_RB;
    static constexpr int OFF_U = OFF_A + CHUNK * K_RB;      // this slice's 16 rows of U^T
    static constexpr int OFF_G = OFF_U + 16 * K_RB;
    static constexpr int BYTES = OFF_G + DK * 4;
    static constexpr int NBUF = 2 * BYTES <= 150 * 1024 ? 2 : 1;
    static constexpr int UNITS = BYTES / 16;
    static constexpr int LOADERS = 3;                       // waves 1..3
    static constexpr int PER_LANE = (UNITS + 64 * LOADERS - 1) / (64 * LOADERS);
};

__device__ __forceinline__ int swz(int row, int unit, int row_bytes) {
    const int units = row_bytes / 16;
    const int rows_per_256 = row_bytes >= 256 ? 1 : 256 / row_bytes;
    return row * row_bytes + 16 * (unit ^ ((row / rows_per_256) % units));
}

// 16-byte units of one chunk's operands, in LDS-image order:
// unit x -> (global source, LDS byte offset).
template <typename E, int DK, int DV>
__device__ __forceinline__ void unit_map(int x, const ChunkBufsC<E>& cb, size_t chh, int j0,
                                         const unsigned char*& src, int& dst)
{
    using L = StateLayout<E, DK, DV>;
    constexpr int UW = CHUNK * L::W_RB / 16, UK = DK * L::K_RB / 16, UA = CHUNK * L::K_RB / 16;
    constexpr int UU = 16 * L::K_RB / 16;
    if (x < UW) {
        src = (const unsigned char*)(cb.W + chh * CHUNK * DK) + 16 * x;
        dst = L::OFF_W + swz(x / (L::W_RB / 16), x % (L::W_RB / 16), L::W_RB);
    } else if ((x -= UW) < UW) {
        src = (const unsigned char*)(cb.Qg + chh * CHUNK * DK) + 16 * x;
        dst = L::OFF_Q + swz(x / (L::W_RB / 16), x % (L::W_RB / 16), L::W_RB);
    } else if ((x -= UW) < UK) {
        src = (const unsigned char*)(cb.Kh + chh * DK * CHUNK) + 16 * x;
        dst = L::OFF_K + swz(x / (L::K_RB / 16), x % (L::K_RB / 16), L::K_RB);
    } else if ((x -= UK) < UA) {
        src = (const unsigned char*)(cb.Aqk + chh * CHUNK * CHUNK) + 16 * x;
        dst = L::OFF_A + swz(x / (L::K_RB / 16), x % (L::K_RB / 16), L::K_RB);
    } else if ((x -= UA) < UU) {
        src = (const unsigned char*)(cb.Ut + (chh * DV + j0) * CHUNK) + 16 * x;
        dst = L::OFF_U + 16 * x;
    } else {
        x -= UU;
        src = (const unsigned char*)(cb.gC + chh * DK) + 16 * x;
        dst = L::OFF_G + 16 * x;
    }
}

template <typename E, int DK, int DV>
struct Stager {
    using L = StateLayout<E, DK, DV>;
    f32x4 reg[L::PER_LANE];
    int dst[L::PER_LANE];

    __device__ __forceinline__ void issue(const ChunkBufsC<E>& cb, size_t chh, int j0, int lt) {
#pragma unroll
        for (int i = 0; i < L::PER_LANE; ++i) {
            const int x = lt + 64 * L::LOADERS * i;
            dst[i] = -1;
            if (x < L::UNITS) {
                const unsigned char* src;
                unit_map<E, DK, DV>(x, cb, chh, j0, src, dst[i]);
                reg[i] = *reinterpret_cast<const f32x4*>(src);
            }
        }
    }
    __device__ __forceinline__ void commit(unsigned char* buf) {
#pragma unroll
        for (int i = 0; i < L::PER_LANE; ++i)
            if (dst[i] >= 0) *reinterpret_cast<f32x4*>(buf + dst[i]) = reg[i];
    }
};

// 8 operand elements at (row, element offset) of a swizzled LDS matrix
template <typename E>
__device__ __forceinline__ typename Vec<E>::v8 lds_frag(const unsigned char* base, int row,
                                                        int elem, int row_bytes)
{
    using V8 = typename Vec<E>::v8;
    if constexpr (sizeof(E) == 2) {
        return *reinterpret_cast<const V8*>(base + swz(row, elem * 2 / 16, row_bytes));
    } else {
        const f32x4 a = *reinterpret_cast<const f32x4*>(base + swz(row, elem * 4 / 16, row_bytes));
        const f32x4 b = *reinterpret_cast<const f32x4*>(base + swz(row, elem * 4 / 16 + 1, row_bytes));
        return V8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    }
}

// Workgroups are grouped so that the DV/16 slices of one (sequence, head)
// have block indices congruent mod 8: blocks are dispatched round-robin over
// the 8 XCDs, so the slices that read the same chunk operands share one L2.
template <typename E, int DK, int DV>
__global__ __launch_bounds__(256) void prefill_state_kernel(
    ChunkBufsC<E> cb, const int32_t* __restrict__ seq_chunk_start,
    const ChunkInfo* __restrict__ chunks, const float* __restrict__ S0,
    float* __restrict__ S_final, E* __restrict__ o, int H, int n_pairs)
{
    using L = StateLayout<E, DK, DV>;
    using V4 = typename Vec<E>::v4;
    using V8 = typename Vec<E>::v8;
    constexpr int NSL = DV / 16;  // value slices per head
    constexpr int KT = DK / 16;   // accumulator tiles of S
    constexpr int KS = DK / 32;   // contraction steps over key channels

    __shared__ __attribute__((aligned(16))) unsigned char smem[L::NBUF * L::BYTES];

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

    Stager<E, DK, DV> stage;
    const int lt = tid - 64;  // loader lane index 0..191
    if (wave > 0 && c_begin < c_end) {
        stage.issue(cb, (size_t)c_begin * H + h, j0, lt);
        stage.commit(smem);
    }

    // S tile t: lane holds S[16t + 4g + i][j0 + ln], i = 0..3 (wave 0 only)
    f32x4 S[KT];
    if (wave == 0) {
#pragma unroll
        for (int t = 0; t < KT; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) S[t][i] = 0.f;
        if (S0) {
#pragma unroll
            for (int t = 0; t < KT; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    S[t][i] = S0[sbase + (size_t)(16 * t + 4 * g + i) * DV + j0 + ln];
        }
    }
    __syncthreads();

    for (int cid = c_begin; cid < c_end; ++cid) {
        const int it = cid - c_begin;
        const unsigned char* buf = smem + (it % L::NBUF) * L::BYTES;
        if (wave == 0) {
            const ChunkInfo ci = chunks[cid];
            // S as an MFMA operand: slots of step ks = rows {32ks+4g..+3, 32ks+16+4g..+3}
            V8 Sf[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    Sf[ks][i] = from_f32<E>(S[2 * ks][i]);
                    Sf[ks][4 + i] = from_f32<E>(S[2 * ks + 1][i]);
                }

            // N = U - W S   (N tile R: lane holds N[16R + 4g + i][j0 + ln])
            f32x4 N[4];
#pragma unroll
            for (int R = 0; R < 4; ++R) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    acc = mma32(lds_frag<E>(buf + L::OFF_W, 16 * R + ln, 32 * ks + 8 * g, L::W_RB),
                                Sf[ks], acc);
                const V4 u = *reinterpret_cast<const V4*>(buf + L::OFF_U + ln * L::K_RB +
                                                         (16 * R + 4 * g) * L::ES);
#pragma unroll
                for (int i = 0; i < 4; ++i) N[R][i] = to_f32(u[i]) - acc[i];
            }
            V8 Nf[2];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    Nf[ks][i] = from_f32<E>(N[2 * ks][i]);
                    Nf[ks][4 + i] = from_f32<E>(N[2 * ks + 1][i]);
                }

            // S = Diag(gamma_C) S + Khat^T N   (the serial dependency: issue first)
#pragma unroll
            for (int t = 0; t < KT; ++t) {
                const f32x4 gc = *reinterpret_cast<const f32x4*>(buf + L::OFF_G + (16 * t + 4 * g) * 4);
                f32x4 acc = S[t] * gc;
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
                    acc = mma32(lds_frag<E>(buf + L::OFF_K, 16 * t + ln, 32 * ks + 8 * g, L::K_RB),
                                Nf[ks], acc);
                S[t] = acc;
            }

            // O^T = S0^T Qg^T + N^T A_qk^T with S0 the chunk-start state (held in Sf)
#pragma unroll
            for (int R = 0; R < 4; ++R) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    acc = mma32(Sf[ks], lds_frag<E>(buf + L::OFF_Q, 16 * R + ln, 32 * ks + 8 * g, L::W_RB),
                                acc);
#pragma unroll
                for (int ks = 0; ks <= R / 2; ++ks)
                    acc = mma32(Nf[ks], lds_frag<E>(buf + L::OFF_A, 16 * R + ln, 32 * ks + 8 * g, L::K_RB),
                                acc);
                const int r = 16 * R + ln;
                if (r < ci.len) {
                    V4 w;
#pragma unroll
                    for (int i = 0; i < 4; ++i) w[i] = from_f32<E>(acc[i]);
                    store_vec(o + ((size_t)(ci.start + r) * H + h) * DV + j0 + 4 * g, w);
                }
            }
        } else if (L::NBUF == 2 && cid + 1 < c_end) {
            stage.issue(cb, (size_t)(cid + 1) * H + h, j0, lt);
            stage.commit(smem + ((it + 1) % 2) * L::BYTES);
        }
        __syncthreads();
        if (L::NBUF == 1 && cid + 1 < c_end) {
            if (wave > 0) {
                stage.issue(cb, (size_t)(cid + 1) * H + h, j0, lt);
                stage.commit(smem);
            }
            __syncthreads();
        }
    }

    if (wave == 0 && S_final) {
#pragma unroll
        for (int t = 0; t < KT; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                S_final[sbase + (size_t)(16 * t + 4 * g + i) * DV + j0 + ln] = S[t][i];
    }
}

template <typename E, int DK, int DV>
static hipError_t launch_state_t(void* const* bufs, const int32_t* seq_chunk_start,
                                 const ChunkInfo* chunks, const float* S0, float* S_final,
                                 void* o, int N, int H, hipStream_t stream)
{
    const int n_pairs = N * H;
    const int groups = (n_pairs + 7) / 8;
    const long long blocks = (long long)groups * 8 * (DV / 16);
    ChunkBufsC<E> cb{(const E*)bufs[0], (const E*)bufs[1], (const E*)bufs[2],
                     (const E*)bufs[3], (const E*)bufs[4], (const float*)bufs[5]};
    hipLaunchKernelGGL((prefill_state_kernel<E, DK, DV>), dim3((unsigned)blocks), dim3(256), 0,
                       stream, cb, seq_chunk_start, chunks, S0, S_final, (E*)o, H, n_pairs);
    return hipGetLastError();
}

hipError_t launch_prefill_state(void* const* bufs, const int32_t* seq_chunk_start,
                                const ChunkInfo* chunks, const float* S0, float* S_final,
                                void* o, int N, int H, int dk, int dv, bool bf16_io,
                                hipStream_t stream)
{
#define KDA_STATE_CASE(E, DK_, DV_) \
    if (dk == DK_ && dv == DV_)     \
        return launch_state_t<E, DK_, DV_>(bufs, seq_chunk_start, chunks, S0, S_final, o, N, H, stream);
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
