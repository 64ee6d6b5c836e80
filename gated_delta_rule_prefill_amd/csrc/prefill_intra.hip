// prefill_intra.hip -- per-chunk work of the chunkwise KDA prefill.
//
// One workgroup (4 waves) per (chunk, head); chunks are independent, so the
// grid covers the whole batch at once.  For a chunk of C = 64 tokens
// r = 0..63 (rows past the sequence end are zero-padded, which makes every
// quantity below vanish for them) it computes, from the recurrence
// S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
// (Kimi Linear paper notes, section 2) folded over the chunk (section 3:
// WY/UT-style W and U, inter plus intra output; the listed chunk
// intermediates g_cumsum, Akk, Aqk, w, u, qg, kg):
//
//   g_r       = sum_{j<=r} log alpha_j             per channel (cumulative log-decay)
//   A_kk[r,i] = beta_r sum_c k_rc k_ic e^{g_rc - g_ic}, i < r
//   A_qk[r,i] =        sum_c q_rc k_ic e^{g_rc - g_ic}, i <= r
//   T         = (I + A_kk)^{-1} Diag(beta)         forward substitution in LDS
//   W         = T (e^g * K),   U = T V             MFMA
//   Khat      = e^{g_C - g} * K,  Qg = e^g * Q,  gamma_C = e^{g_C}
//
// and stores W, U, Khat^T, Qg, A_qk and gamma_C for the sequential state
// kernel.  The state kernel then needs, per chunk, only
//   N = U - W S,  O = Qg S + A_qk N,  S <- Diag(gamma_C) S + Khat^T N.
//
// Decay factors never form 1/gamma over a whole chunk: the chunk is cut into
// four 16-token blocks with reference log-decays B_R (g just before block R).
// Row factors e^{g_r - B_R} and cross-block factors e^{B_R - B_I} are <= 1;
// only the within-block factor e^{B_I - g_i} exceeds 1, bounded by the decay
// of at most 16 tokens.
#include "kda_common.h"

namespace kda {

template <typename E, int DK, int DV>
struct IntraLayout {
    static constexpr int ES = sizeof(E);
    static constexpr int PAD = 16 / ES;              // 16-byte row padding (elements)
    static constexpr int LK = DK + PAD;              // row stride of [64][DK] arrays
    static constexpr int LT = CHUNK + PAD;           // row stride of [d][64] / [64][64] arrays
    static constexpr int LA = CHUNK + 4;             // row stride of the fp32 A_kk array
    // phase 1 (A tiles): KP|QP and KD;  phase 2+ (W, U): kgT and vT in the same bytes
    static constexpr int P1_BYTES = 2 * CHUNK * LK * ES;
    static constexpr int P2_BYTES = (DK + DV) * LT * ES;
    static constexpr int U1_BYTES = P1_BYTES > P2_BYTES ? P1_BYTES : P2_BYTES;
    static constexpr int OFF_KP = 0;                         // also QP
    static constexpr int OFF_KD = CHUNK * LK * ES;
    static constexpr int OFF_KGT = 0;
    static constexpr int OFF_VT = DK * LT * ES;
    static constexpr int OFF_AL = (U1_BYTES + 255) & ~255;
    static constexpr int OFF_TL = OFF_AL + CHUNK * LA * 4;
    static constexpr int OFF_TAU = OFF_TL + ((CHUNK * LT * ES + 15) & ~15);
    static constexpr int OFF_BETA = OFF_TAU + 4 * DK * 4;
    static constexpr int BYTES = OFF_BETA + CHUNK * 4;
};

// Pointers to the per-(chunk, head) intermediates in the workspace.
template <typename E>
struct ChunkBufs {
    E* W;        // [NC*H][64][DK]   channels in perm32 order
    E* Qg;       // [NC*H][64][DK]   channels in perm32 order
    E* Kh;       // [NC*H][DK][64]   Khat^T, tokens in perm32 order
    E* Aqk;      // [NC*H][64][64]   key tokens in perm32 order
    E* Ut;       // [NC*H][DV][64]   U^T, natural token order
    float* gC;   // [NC*H][DK]       gamma_C = exp(g_C)
};

// 8 consecutive operand elements from LDS, optionally scaled per channel.
template <typename E>
__device__ __forceinline__ typename Vec<E>::v8 frag8(const E* p) {
    return load_vec<typename Vec<E>::v8>(p);
}
template <typename E>
__device__ __forceinline__ typename Vec<E>::v8 frag8_scaled(const E* p, const float (&f)[8]) {
    typename Vec<E>::v8 v = load_vec<typename Vec<E>::v8>(p);
#pragma unroll
    for (int m = 0; m < 8; ++m) v[m] = from_f32<E>(to_f32(v[m]) * f[m]);
    return v;
}

// Pairs (R, I) of 16-token blocks with I <= R, spread over the 4 waves.
__device__ __constant__ const int8_t kPairR[10] = {0, 1, 1, 2, 2, 2, 3, 3, 3, 3};
__device__ __constant__ const int8_t kPairI[10] = {0, 0, 1, 0, 1, 2, 0, 1, 2, 3};
__device__ __constant__ const int8_t kUpperR[6] = {0, 0, 0, 1, 1, 2};
__device__ __constant__ const int8_t kUpperI[6] = {1, 2, 3, 2, 3, 3};

template <typename E, int DK, int DV>
__global__ __launch_bounds__(256) void prefill_intra_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
    const float* __restrict__ log_alpha, const float* __restrict__ beta,
    const ChunkInfo* __restrict__ chunks, const int32_t* __restrict__ n_chunks_ptr, int H,
    ChunkBufs<E> out)
{
    using L = IntraLayout<E, DK, DV>;
    using V4 = typename Vec<E>::v4;
    using V8 = typename Vec<E>::v8;
    constexpr int CPT = DK / 64;   // key channels per thread in the row-block mapping
    constexpr int CPTV = DV / 64;  // value channels per thread
    constexpr int KS = DK / 32;    // contraction steps over key channels

    __shared__ __attribute__((aligned(16))) unsigned char smem[L::BYTES];
    E* sKP = reinterpret_cast<E*>(smem + L::OFF_KP);   // k*e^{g-B}  (phase 1a), then q*e^{g-B} (1b)
    E* sKD = reinterpret_cast<E*>(smem + L::OFF_KD);   // k*e^{B-g}
    E* sKGT = reinterpret_cast<E*>(smem + L::OFF_KGT); // (e^g * k)^T   (phase 2+)
    E* sVT = reinterpret_cast<E*>(smem + L::OFF_VT);   // v^T           (phase 2+)
    float* sAL = reinterpret_cast<float*>(smem + L::OFF_AL);
    E* sTL = reinterpret_cast<E*>(smem + L::OFF_TL);
    float* sTau = reinterpret_cast<float*>(smem + L::OFF_TAU);
    float* sBeta = reinterpret_cast<float*>(smem + L::OFF_BETA);

    const int cid = blockIdx.x;
    if (cid >= *n_chunks_ptr) return;
    const int h = blockIdx.y;
    const ChunkInfo ci = chunks[cid];
    const size_t chh = (size_t)cid * H + h;

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = t >> 6;     // also the 16-token block handled in the row mapping
    const int R = wave;
    const int g = lane >> 4, ln = lane & 15;
    const int c0 = lane * CPT;

    // ---- phase 0: cumulative log-decay inside each 16-token block -------------
    float ell[16][CPT];
    {
        float run[CPT];
#pragma unroll
        for (int e = 0; e < CPT; ++e) run[e] = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = 16 * R + r;
            if (row < ci.len) {
                const float* p = log_alpha + ((size_t)(ci.start + row) * H + h) * DK + c0;
#pragma unroll
                for (int e = 0; e < CPT; ++e) run[e] += p[e];
            }
#pragma unroll
            for (int e = 0; e < CPT; ++e) ell[r][e] = run[e];
        }
#pragma unroll
        for (int e = 0; e < CPT; ++e) sTau[R * DK + c0 + e] = run[e];
        if (wave == 0) sBeta[lane] = lane < ci.len ? beta[(size_t)(ci.start + lane) * H + h] : 0.f;
    }
    __syncthreads();

    float Bref[CPT], toEnd[CPT];   // B_R = g before block R;  g_C - B_R
#pragma unroll
    for (int e = 0; e < CPT; ++e) {
        float a = 0.f, b = 0.f;
#pragma unroll
        for (int Rp = 0; Rp < 4; ++Rp) {
            const float tv = sTau[Rp * DK + c0 + e];
            if (Rp < R) a += tv; else b += tv;
        }
        Bref[e] = a;
        toEnd[e] = b;
    }

    // keys: decayed operands for A_kk / A_qk, Khat^T and gamma_C to the workspace
    float kreg[16][CPT];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int row = 16 * R + r;
#pragma unroll
        for (int e = 0; e < CPT; ++e)
            kreg[r][e] = row < ci.len ? to_f32(k[((size_t)(ci.start + row) * H + h) * DK + c0 + e]) : 0.f;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int row = 16 * R + r;
#pragma unroll
        for (int e = 0; e < CPT; ++e) {
            const float P = fast_exp(ell[r][e]);
            const float iP = fast_exp(fminf(-ell[r][e], 80.f));
            sKP[row * L::LK + c0 + e] = from_f32<E>(kreg[r][e] * P);
            sKD[row * L::LK + c0 + e] = from_f32<E>(kreg[r][e] * iP);
        }
    }
#pragma unroll
    for (int e = 0; e < CPT; ++e) {
        E* dst = out.Kh + (chh * DK + c0 + e) * CHUNK;
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            V4 w;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 4 * r4 + i;
                w[i] = from_f32<E>(kreg[r][e] * fast_exp(toEnd[e] - ell[r][e]));
            }
            store_vec(dst + perm_index(16 * R + 4 * r4), w);
        }
        if (R == 0) out.gC[chh * DK + c0 + e] = fast_exp(toEnd[e]);
    }
    __syncthreads();

    // ---- phase 1a: A_kk tiles (rows r of block R, columns i of block I) --------
    // A operand k_r e^{g_r - B_R}; B operand k_i e^{B_I - g_i} * e^{B_R - B_I}.
    for (int p = wave; p < 10; p += 4) {
        const int PR = kPairR[p], PI = kPairI[p];
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const int cb = 32 * s + 8 * g;
            float f[8];
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                float d = 0.f;
                for (int Rp = PI; Rp < PR; ++Rp) d += sTau[Rp * DK + cb + m];
                f[m] = fast_exp(d);   // e^{B_R - B_I} <= 1
            }
            const V8 a = frag8<E>(sKP + (16 * PR + ln) * L::LK + cb);
            const V8 b = frag8_scaled<E>(sKD + (16 * PI + ln) * L::LK + cb, f);
            acc = mma32(a, b, acc);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 16 * PR + 4 * g + i, col = 16 * PI + ln;
            sAL[r * L::LA + col] = r > col ? sBeta[r] * acc[i] : 0.f;
        }
    }
    for (int u = wave - 2; u >= 0 && u < 6; u += 2) {   // waves 2 and 3 zero the upper tiles
        const int UR = kUpperR[u], UI = kUpperI[u];
#pragma unroll
        for (int i = 0; i < 4; ++i) sAL[(16 * UR + 4 * g + i) * L::LA + 16 * UI + ln] = 0.f;
    }
    __syncthreads();   // sKP no longer read

    // ---- phase 1b: queries -> q e^{g - B} (LDS) and Qg = q e^{g} (workspace) ----
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int row = 16 * R + r;
        typename Vec<E>::v2 qg2;
        float qv[CPT];
#pragma unroll
        for (int e = 0; e < CPT; ++e)
            qv[e] = row < ci.len ? to_f32(q[((size_t)(ci.start + row) * H + h) * DK + c0 + e]) : 0.f;
#pragma unroll
        for (int e = 0; e < CPT; ++e) {
            sKP[row * L::LK + c0 + e] = from_f32<E>(qv[e] * fast_exp(ell[r][e]));
            const E val = from_f32<E>(qv[e] * fast_exp(Bref[e] + ell[r][e]));
            if constexpr (CPT == 2) qg2[e] = val;
            else out.Qg[(chh * CHUNK + row) * DK + perm_index(c0 + e)] = val;
        }
        if constexpr (CPT == 2) store_vec(out.Qg + (chh * CHUNK + row) * DK + perm_index(c0), qg2);
    }
    __syncthreads();

    // ---- phase 1c: A_qk^T tiles (rows i of block I, columns r of block R) -------
    for (int p = wave; p < 10; p += 4) {
        const int PR = kPairR[p], PI = kPairI[p];
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const int cb = 32 * s + 8 * g;
            float f[8];
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                float d = 0.f;
                for (int Rp = PI; Rp < PR; ++Rp) d += sTau[Rp * DK + cb + m];
                f[m] = fast_exp(d);   // e^{B_R - B_I} <= 1
            }
            const V8 a = frag8_scaled<E>(sKD + (16 * PI + ln) * L::LK + cb, f);
            const V8 b = frag8<E>(sKP + (16 * PR + ln) * L::LK + cb);
            acc = mma32(a, b, acc);
        }
        const int r = 16 * PR + ln;
        V4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int col = 16 * PI + 4 * g + i;
            w[i] = from_f32<E>(r >= col ? acc[i] : 0.f);
        }
        store_vec(out.Aqk + (chh * CHUNK + r) * CHUNK + perm_index(16 * PI + 4 * g), w);
    }
    for (int u = wave - 2; u >= 0 && u < 6; u += 2) {
        const int UR = kUpperR[u], UI = kUpperI[u];
        V4 z;
#pragma unroll
        for (int i = 0; i < 4; ++i) z[i] = from_f32<E>(0.f);
        store_vec(out.Aqk + (chh * CHUNK + 16 * UR + ln) * CHUNK + perm_index(16 * UI + 4 * g), z);
    }
    __syncthreads();   // sKP / sKD dead: their bytes become kgT and vT

    // ---- phase 2: (e^g k)^T and v^T in LDS, token-contiguous ------------------
#pragma unroll
    for (int e = 0; e < CPT; ++e) {
        V8 lo, hi;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            lo[r] = from_f32<E>(kreg[r][e] * fast_exp(Bref[e] + ell[r][e]));
            hi[r] = from_f32<E>(kreg[r + 8][e] * fast_exp(Bref[e] + ell[r + 8][e]));
        }
        store_vec(sKGT + (c0 + e) * L::LT + 16 * R, lo);
        store_vec(sKGT + (c0 + e) * L::LT + 16 * R + 8, hi);
    }
    {
        const int cv0 = lane * CPTV;
#pragma unroll
        for (int e = 0; e < CPTV; ++e) {
            V8 lo, hi;
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const int row = 16 * R + r;
                lo[r] = row < ci.len ? v[((size_t)(ci.start + row) * H + h) * DV + cv0 + e] : from_f32<E>(0.f);
                hi[r] = row + 8 < ci.len ? v[((size_t)(ci.start + row + 8) * H + h) * DV + cv0 + e] : from_f32<E>(0.f);
            }
            store_vec(sVT + (cv0 + e) * L::LT + 16 * R, lo);
            store_vec(sVT + (cv0 + e) * L::LT + 16 * R + 8, hi);
        }
    }

    // ---- phase 3: T = (I + A_kk)^{-1} Diag(beta) by forward substitution -------
    // Lane j of wave 0 solves (I + A) x = e_j for column j of the inverse.
    if (wave == 0) {
        float x[CHUNK];
#pragma unroll
        for (int i = 0; i < CHUNK; ++i) x[i] = 0.f;
#pragma unroll
        for (int r = 0; r < CHUNK; ++r) {
            float acc = (r == lane) ? 1.f : 0.f;
#pragma unroll
            for (int i4 = 0; i4 < (r + 3) / 4; ++i4) {
                const f32x4 a = *reinterpret_cast<const f32x4*>(sAL + r * L::LA + 4 * i4);
                acc -= a[0] * x[4 * i4] + a[1] * x[4 * i4 + 1] + a[2] * x[4 * i4 + 2] + a[3] * x[4 * i4 + 3];
            }
            x[r] = acc;
        }
        const float bj = sBeta[lane];
#pragma unroll
        for (int r = 0; r < CHUNK; ++r) sTL[r * L::LT + lane] = from_f32<E>(x[r] * bj);
    }
    __syncthreads();

    // ---- phase 4: W^T = (e^g K)^T T^T and U = T V on MFMA ---------------------
    // T is lower triangular, so output block R' only needs key tokens < 16R'+16.
    for (int ct = wave; ct < DK / 16; ct += 4) {
#pragma unroll
        for (int Rq = 0; Rq < 4; ++Rq) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s <= Rq / 2; ++s) {
                const V8 a = frag8<E>(sKGT + (16 * ct + ln) * L::LT + 32 * s + 8 * g);
                const V8 b = frag8<E>(sTL + (16 * Rq + ln) * L::LT + 32 * s + 8 * g);
                acc = mma32(a, b, acc);
            }
            V4 w;
#pragma unroll
            for (int i = 0; i < 4; ++i) w[i] = from_f32<E>(acc[i]);
            const int r = 16 * Rq + ln;
            store_vec(out.W + (chh * CHUNK + r) * DK + perm_index(16 * ct + 4 * g), w);
        }
    }
    for (int ct = wave; ct < DV / 16; ct += 4) {
#pragma unroll
        for (int Rq = 0; Rq < 4; ++Rq) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s <= Rq / 2; ++s) {
                const V8 a = frag8<E>(sTL + (16 * Rq + ln) * L::LT + 32 * s + 8 * g);
                const V8 b = frag8<E>(sVT + (16 * ct + ln) * L::LT + 32 * s + 8 * g);
                acc = mma32(a, b, acc);
            }
            V4 w;
#pragma unroll
            for (int i = 0; i < 4; ++i) w[i] = from_f32<E>(acc[i]);
            store_vec(out.Ut + (chh * DV + 16 * ct + ln) * CHUNK + 16 * Rq + 4 * g, w);
        }
    }
}

template <typename E, int DK, int DV>
static hipError_t launch_intra_t(const void* q, const void* k, const void* v, const float* la,
                                 const float* beta, const ChunkInfo* chunks,
                                 const int32_t* n_chunks, int max_chunks, int H, void* const* bufs,
                                 hipStream_t stream)
{
    ChunkBufs<E> b{(E*)bufs[0], (E*)bufs[1], (E*)bufs[2], (E*)bufs[3], (E*)bufs[4], (float*)bufs[5]};
    hipLaunchKernelGGL((prefill_intra_kernel<E, DK, DV>), dim3(max_chunks, H), dim3(256), 0, stream,
                       (const E*)q, (const E*)k, (const E*)v, la, beta, chunks, n_chunks, H, b);
    return hipGetLastError();
}

// bufs: W, Qg, Kh, Aqk, Ut, gC
hipError_t launch_prefill_intra(const void* q, const void* k, const void* v, const float* la,
                                const float* beta, const ChunkInfo* chunks,
                                const int32_t* n_chunks, int max_chunks, int H, int dk, int dv,
                                bool bf16_io, void* const* bufs, hipStream_t stream)
{
#define KDA_INTRA_CASE(E, DK_, DV_)                                                               \
    if (dk == DK_ && dv == DV_)                                                                  \
        return launch_intra_t<E, DK_, DV_>(q, k, v, la, beta, chunks, n_chunks, max_chunks, H,   \
                                           bufs, stream);
    if (bf16_io) {
        KDA_INTRA_CASE(bf16, 128, 128)
        KDA_INTRA_CASE(bf16, 64, 64)
        KDA_INTRA_CASE(bf16, 128, 64)
        KDA_INTRA_CASE(bf16, 64, 128)
    } else {
        KDA_INTRA_CASE(float, 128, 128)
        KDA_INTRA_CASE(float, 64, 64)
        KDA_INTRA_CASE(float, 128, 64)
        KDA_INTRA_CASE(float, 64, 128)
    }
#undef KDA_INTRA_CASE
    return hipErrorInvalidValue;
}

}  // namespace kda
