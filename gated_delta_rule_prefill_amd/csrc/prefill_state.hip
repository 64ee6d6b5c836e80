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
// One wave per (sequence, head, 16 value columns): the columns of S evolve
// independently, so a head's state is split over DV/16 waves that never
// communicate.  The fp32 state tile (DK x 16) lives in MFMA accumulator
// registers for the whole sequence and is read from / written to HBM once.
// Every product takes its register-resident operand (S or N) directly from
// accumulator tiles: a tile's lane group g holds rows 4g..4g+3, which is the
// operand slot set that the perm32 storage order of W, Qg, Khat^T and A_qk
// matches, so no LDS round trip is needed inside the serial loop.
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

// Workgroups are grouped so that the DV/16 waves of one (sequence, head)
// have block indices congruent mod 8: blocks are dispatched round-robin over
// the 8 XCDs, so the waves that share a chunk's W/Qg/Khat/A_qk share one L2.
template <typename E, int DK, int DV>
__global__ __launch_bounds__(64) void prefill_state_kernel(
    ChunkBufsC<E> cb, const int32_t* __restrict__ seq_chunk_start,
    const ChunkInfo* __restrict__ chunks, const float* __restrict__ S0,
    float* __restrict__ S_final, E* __restrict__ o, int H, int n_pairs)
{
    using V4 = typename Vec<E>::v4;
    using V8 = typename Vec<E>::v8;
    constexpr int NSL = DV / 16;  // value slices per head
    constexpr int KT = DK / 16;   // accumulator tiles of S
    constexpr int KS = DK / 32;   // contraction steps over key channels

    const int b = blockIdx.x;
    const int xcd = b & 7, q8 = b >> 3;
    const int grp = q8 / NSL, slice = q8 % NSL;
    const int pair = grp * 8 + xcd;
    if (pair >= n_pairs) return;
    const int s = pair / H, h = pair % H;
    const int l = threadIdx.x, g = l >> 4, ln = l & 15;
    const int j0 = slice * 16;

    // S tile t: lane holds S[16t + 4g + i][j0 + ln], i = 0..3
    f32x4 S[KT];
    const size_t sbase = (size_t)pair * DK * DV;
#pragma unroll
    for (int t = 0; t < KT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            S[t][i] = S0 ? S0[sbase + (size_t)(16 * t + 4 * g + i) * DV + j0 + ln] : 0.f;

    const int c_begin = seq_chunk_start[s], c_end = seq_chunk_start[s + 1];
    for (int cid = c_begin; cid < c_end; ++cid) {
        const ChunkInfo ci = chunks[cid];
        const size_t chh = (size_t)cid * H + h;

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
            const E* wrow = cb.W + (chh * CHUNK + 16 * R + ln) * DK + 8 * g;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) acc = mma32(load_vec<V8>(wrow + 32 * ks), Sf[ks], acc);
            const V4 u = load_vec<V4>(cb.Ut + (chh * DV + j0 + ln) * CHUNK + 16 * R + 4 * g);
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

        // O^T = S^T Qg^T + N^T A_qk^T   (tile R: lane holds O[16R + ln][j0 + 4g + i])
#pragma unroll
        for (int R = 0; R < 4; ++R) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            const E* qrow = cb.Qg + (chh * CHUNK + 16 * R + ln) * DK + 8 * g;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) acc = mma32(Sf[ks], load_vec<V8>(qrow + 32 * ks), acc);
            const E* arow = cb.Aqk + (chh * CHUNK + 16 * R + ln) * CHUNK + 8 * g;
#pragma unroll
            for (int ks = 0; ks <= R / 2; ++ks) acc = mma32(Nf[ks], load_vec<V8>(arow + 32 * ks), acc);
            const int r = 16 * R + ln;
            if (r < ci.len) {
                V4 w;
#pragma unroll
                for (int i = 0; i < 4; ++i) w[i] = from_f32<E>(acc[i]);
                store_vec(o + ((size_t)(ci.start + r) * H + h) * DV + j0 + 4 * g, w);
            }
        }

        // S = Diag(gamma_C) S + Khat^T N
#pragma unroll
        for (int t = 0; t < KT; ++t) {
            const f32x4 gc = load_vec<f32x4>(cb.gC + chh * DK + 16 * t + 4 * g);
            S[t] *= gc;
            const E* krow = cb.Kh + (chh * DK + 16 * t + ln) * CHUNK + 8 * g;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) S[t] = mma32(load_vec<V8>(krow + 32 * ks), Nf[ks], S[t]);
        }
    }

    if (S_final) {
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
    hipLaunchKernelGGL((prefill_state_kernel<E, DK, DV>), dim3((unsigned)blocks), dim3(64), 0,
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
