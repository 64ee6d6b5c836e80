// prefill_intra.hip -- per-chunk work of the chunkwise KDA prefill.
//
// One workgroup (4 waves) per (chunk, head); chunks are independent, so the
// grid covers the whole batch at once.  For a chunk of C = 64 tokens
// r = 0..63 (only log_alpha and beta are zeroed past the sequence end, which
// makes every quantity below vanish or go unused for those rows) it computes,
// from the recurrence S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} +
// beta_t k_t v_t^T, o_t = S_t^T q_t (Kimi Linear paper notes, section 2)
// folded over the chunk (section 3: WY/UT-style W and U, inter- plus
// intra-chunk output, only the fixed-size state passed between chunks):
//
//   g_r       = sum_{j<=r} log alpha_j             per channel (cumulative log-decay)
//   A_kk[r,i] = beta_r sum_c k_rc k_ic e^{g_rc - g_ic}, i < r
//   A_qk[r,i] =        sum_c q_rc k_ic e^{g_rc - g_ic}, i <= r
//   T         = (I + A_kk)^{-1} Diag(beta)         blocked substitution in LDS
//   W         = T (e^g * K),   U = T V             MFMA
//   Khat      = e^{g_C - g} * K,   Qg = e^g * Q,   gamma_C = e^{g_C}
//
// With entry state S the chunk gives N = U - W S, O = Qg S + A_qk N and
// S' = Diag(gamma_C) S + Khat^T N.  This kernel folds W and U into the
// chunk's transition and read-out, so the sequential kernel only applies
//
//   S' = Diag(gamma_C) S + PM S + Hc,   O = QM S + OI
//   PM = -Khat^T W,  Hc = Khat^T U,  QM = Qg - A_qk W,  OI = A_qk U
//
// and writes PM, Hc^T, QM, OI and gamma_C as one record per chunk and head.
//
// The inverse of the unit lower-triangular I + A_kk is built blockwise: the
// four 16x16 diagonal blocks by forward substitution (one lane per column),
// then the off-diagonal blocks on fp32 MFMA, each wave walking down one
// column block with the blocks above it in registers, stored transposed in
// the unused upper triangle of A_kk.
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
    static constexpr int LA = CHUNK + 4;             // row stride of the fp32 A / X array
    // region U1: phase 1 KP|QP and KD; phase 3-4 kgT and vT; phase 5 QA (fp32 A_qk W)
    static constexpr int P1_BYTES = 2 * CHUNK * LK * ES;
    static constexpr int P2_BYTES = (DK + DV) * LT * ES;
    static constexpr int P5_BYTES = CHUNK * (DK + 4) * 4;
    static constexpr int U1_A = P1_BYTES > P2_BYTES ? P1_BYTES : P2_BYTES;
    static constexpr int U1_BYTES = U1_A > P5_BYTES ? U1_A : P5_BYTES;
    static constexpr int OFF_KP = 0;                         // also QP
    static constexpr int OFF_KD = CHUNK * LK * ES;
    static constexpr int OFF_KGT = 0;
    static constexpr int OFF_VT = DK * LT * ES;
    static constexpr int OFF_QA = 0;
    static constexpr int LQA = DK + 4;                       // row stride of QA (fp32)
    // region U2: A_kk / X (fp32) until T is formed, then Khat^T (perm32 token order)
    static constexpr int AL_BYTES = CHUNK * LA * 4;
    static constexpr int KHT_BYTES = DK * LT * ES;
    static constexpr int OFF_AL = (U1_BYTES + 255) & ~255;
    static constexpr int OFF_KHT = OFF_AL;
    static constexpr int U2_BYTES = AL_BYTES > KHT_BYTES ? AL_BYTES : KHT_BYTES;
    static constexpr int OFF_TL = OFF_AL + ((U2_BYTES + 15) & ~15);
    static constexpr int OFF_AQ = OFF_TL + ((CHUNK * LT * ES + 15) & ~15);   // A_qk, perm32 keys
    static constexpr int OFF_TAU = OFF_AQ + ((CHUNK * LT * ES + 15) & ~15);
    // phase 0b-1: q e^{g - B} ([64][LK]) over the T and A_qk areas, free until then
    static constexpr int OFF_QP = OFF_TL;
    static_assert(OFF_QP + CHUNK * LK * ES <= OFF_TAU, "q operand area");
    static constexpr int OFF_ETAB = OFF_TAU + 4 * DK * 4;
    static constexpr int OFF_BETA = OFF_ETAB + 6 * DK * 4;
    static constexpr int BYTES = OFF_BETA + CHUNK * 4;
};

// Pointers into one (chunk, head) record of the workspace (see rec_layout).
template <typename E, int DK, int DV>
struct ChunkOut {
    E* PM;
    E* HCt;
    E* QM;
    E* OI;
    float* gC;
    __device__ ChunkOut(unsigned char* rec, size_t chh) {
        constexpr RecLayout RL = rec_layout(sizeof(E), DK, DV);
        unsigned char* base = rec + chh * RL.bytes;
        PM = reinterpret_cast<E*>(base + RL.pm);
        HCt = reinterpret_cast<E*>(base + RL.hc);
        QM = reinterpret_cast<E*>(base + RL.qm);
        OI = reinterpret_cast<E*>(base + RL.oi);
        gC = reinterpret_cast<float*>(base + RL.g);
    }
};

// 8 consecutive operand elements from LDS, optionally scaled per channel.
template <typename E>
__device__ __forceinline__ typename Vec<E>::v8 frag8(const E* p) {
    return load_vec<typename Vec<E>::v8>(p);
}
template <typename E>
__device__ __forceinline__ typename Vec<E>::v8 frag8_scaled(const E* p, const float* f) {
    typename Vec<E>::v8 v = load_vec<typename Vec<E>::v8>(p);
    const f32x4 f0 = *reinterpret_cast<const f32x4*>(f);
    const f32x4 f1 = *reinterpret_cast<const f32x4*>(f + 4);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        v[m] = from_f32<E>(to_f32(v[m]) * f0[m]);
        v[m + 4] = from_f32<E>(to_f32(v[m + 4]) * f1[m]);
    }
    return v;
}

// CPT consecutive elements as floats (one vector load).  The inputs are read
// once: streaming loads keep them from displacing the records in the caches.
template <int CPT, typename E>
__device__ __forceinline__ void load_row(const E* p, float (&out)[CPT]) {
    if constexpr (CPT == 2) {
        const typename Vec<E>::v2 v = __builtin_nontemporal_load(reinterpret_cast<const typename Vec<E>::v2*>(p));
        out[0] = to_f32(v[0]);
        out[1] = to_f32(v[1]);
    } else {
        out[0] = to_f32(__builtin_nontemporal_load(p));
    }
}

// CPT consecutive elements to LDS (one store)
template <int CPT, typename E>
__device__ __forceinline__ void store_row(E* p, const E (&v)[CPT]) {
    if constexpr (CPT == 2) {
        typename Vec<E>::v2 w;
        w[0] = v[0];
        w[1] = v[1];
        *reinterpret_cast<typename Vec<E>::v2*>(p) = w;
    } else {
        p[0] = v[0];
    }
}

// An MFMA operand over 32 tokens (step s) from two stacked 16-token
// accumulator tiles: lane group g holds rows 4g..4g+3 of each, i.e. the
// perm32 slot order.
template <typename E>
__device__ __forceinline__ typename Vec<E>::v8 tiles_to_frag(const f32x4& lo, const f32x4& hi) {
    typename Vec<E>::v8 f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[i] = from_f32<E>(lo[i]);
        f[4 + i] = from_f32<E>(hi[i]);
    }
    return f;
}

// Pairs (R, I) of 16-token blocks, enumerated arithmetically (a table would be
// read from memory inside the loops).  All pairs with I <= R in the order
// (0,0) (1,0) (1,1) (2,0) (2,1) (2,2) (3,0) ...:
__device__ __forceinline__ int pair_r(int p) { return (p >= 1) + (p >= 3) + (p >= 6); }
__device__ __forceinline__ int pair_i(int p) { const int r = pair_r(p); return p - r * (r + 1) / 2; }
// the six pairs with I < R in the order (1,0) (2,0) (2,1) (3,0) (3,1) (3,2); the
// index of pair (R, I) is R(R-1)/2 + I, which is also its slot in the decay table
__device__ __forceinline__ int off_r(int p) { return 1 + (p >= 1) + (p >= 3); }
__device__ __forceinline__ int off_i(int p) { const int r = off_r(p); return p - r * (r - 1) / 2; }

// Element (r, c) of X = (I + A_kk)^{-1}: unit lower triangular, its strictly
// lower part stored transposed in the (otherwise zero) upper triangle of sAL.
template <int LA>
__device__ __forceinline__ float x_elem(const float* sAL, int r, int c) {
    return r == c ? 1.f : (r > c ? sAL[c * LA + r] : 0.f);
}

// Column block I of X below the diagonal, by one wave on fp32 MFMA:
//   X_RI = -X_RR * sum_{J=I}^{R-1} A_RJ X_JI,   R = I+1 .. 3,
// each block feeding the next from registers: an accumulator tile (lane
// group g holding rows 4g..4g+3) is the B operand whose slot (g, m) carries
// contraction index 4g + m.  Only the diagonal inverses X_RR and A come
// from LDS; the results go to the upper triangle of sAL, transposed.
template <int LA, int I>
__device__ __forceinline__ void x_column(float* sAL, int g, int ln) {
    f32x4 xc[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) xc[I][m] = x_elem<LA>(sAL, 16 * I + 4 * g + m, 16 * I + ln);
#pragma unroll
    for (int R = I + 1; R < 4; ++R) {
        float a[R - I][4], xr[4];
#pragma unroll
        for (int J = I; J < R; ++J)
#pragma unroll
            for (int m = 0; m < 4; ++m) a[J - I][m] = sAL[(16 * R + ln) * LA + 16 * J + 4 * g + m];
#pragma unroll
        for (int m = 0; m < 4; ++m) xr[m] = -x_elem<LA>(sAL, 16 * R + ln, 16 * R + 4 * g + m);
        f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int J = I; J < R; ++J)
#pragma unroll
            for (int m = 0; m < 4; ++m) z = __builtin_amdgcn_mfma_f32_16x16x4f32(a[J - I][m], xc[J][m], z, 0, 0, 0);
        f32x4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < 4; ++m) x = __builtin_amdgcn_mfma_f32_16x16x4f32(xr[m], z[m], x, 0, 0, 0);
        xc[R] = x;
#pragma unroll
        for (int i = 0; i < 4; ++i) sAL[(16 * I + ln) * LA + 16 * R + 4 * g + i] = x[i];
    }
}

// NORM: L2-normalise q and k rows first; beta_logit: beta arrives as a logit.
template <typename E, int DK, int DV, bool NORM>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void prefill_intra_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
    const float* __restrict__ log_alpha, const float* __restrict__ beta,
    const ChunkSrc src, int H, int beta_logit,
    unsigned char* __restrict__ rec)
{
    using L = IntraLayout<E, DK, DV>;
    using V4 = typename Vec<E>::v4;
    using V8 = typename Vec<E>::v8;
    constexpr int CPT = DK / 64;   // key channels per thread in the row-block mapping
    constexpr int CPTV = DV / 64;  // value channels per thread
    constexpr int KS = DK / 32;    // contraction steps over key channels
    constexpr int NWB = (DK / 16 + 3) / 4;   // key-column blocks per wave
    constexpr int NUB = (DV / 16 + 3) / 4;   // value-column blocks per wave

    __shared__ __attribute__((aligned(16))) unsigned char smem[L::BYTES];
    E* sKP = reinterpret_cast<E*>(smem + L::OFF_KP);   // k*e^{g-B}  (phase 0b-1)
    E* sKD = reinterpret_cast<E*>(smem + L::OFF_KD);   // k*e^{B-g}
    E* sKGT = reinterpret_cast<E*>(smem + L::OFF_KGT); // (e^g * k)^T   (phase 3-4)
    E* sVT = reinterpret_cast<E*>(smem + L::OFF_VT);   // v^T           (phase 3-4)
    float* sQA = reinterpret_cast<float*>(smem + L::OFF_QA);  // A_qk W (phase 5-6)
    float* sAL = reinterpret_cast<float*>(smem + L::OFF_AL);
    E* sKHT = reinterpret_cast<E*>(smem + L::OFF_KHT);  // Khat^T (phase 4+)
    E* sTL = reinterpret_cast<E*>(smem + L::OFF_TL);
    E* sAQ = reinterpret_cast<E*>(smem + L::OFF_AQ);
    E* sQP = reinterpret_cast<E*>(smem + L::OFF_QP);   // q*e^{g-B} (phase 0b-1)
    float* sTau = reinterpret_cast<float*>(smem + L::OFF_TAU);
    float* sEtab = reinterpret_cast<float*>(smem + L::OFF_ETAB);
    float* sBeta = reinterpret_cast<float*>(smem + L::OFF_BETA);

    int cid, h;
    chunk_head_of_block(H, true, cid, h);
    int n_chunks;
    ChunkInfo ci;
    chunk_of(src, cid, n_chunks, ci);
    if (cid >= n_chunks) return;
    const size_t chh = (size_t)cid * H + h;
    const ChunkOut<E, DK, DV> out(rec, chh);

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);   // also the 16-token block of the row mapping
    const int R = wave;
    const int g = lane >> 4, ln = lane & 15;
    const int c0 = lane * CPT;
    const int cv0 = lane * CPTV;

    // ---- phase 0: unconditional loads (rows past the end re-read the last row) -
    // Issued tensor by tensor in the order they are first needed: a wave's
    // loads complete in order, so the prefix sum waits only for log_alpha, the
    // decayed keys only for k, and v stays in flight until the transposes.
    float la[16][CPT], kr[16][CPT], qr[16][CPT], vr[16][CPTV];
    size_t rowoff[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int row = 16 * R + r;
        rowoff[r] = ((size_t)ci.start + (row < ci.len ? row : ci.len - 1)) * H + h;
    }
    // beta first: it is needed before the first barrier, and a wave's loads
    // complete in order, so a late beta load would make that barrier wait for
    // every input row (every wave loads it; wave 0 keeps it)
    const float bt = beta[((size_t)ci.start + (lane < ci.len ? lane : ci.len - 1)) * H + h];
#pragma unroll
    for (int r = 0; r < 16; ++r) load_row<CPT>(log_alpha + rowoff[r] * DK + c0, la[r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) load_row<CPT>(k + rowoff[r] * DK + c0, kr[r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) load_row<CPT>(q + rowoff[r] * DK + c0, qr[r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) load_row<CPTV>(v + rowoff[r] * DV + cv0, vr[r]);
    // cumulative log-decay inside each 16-token block; padded rows add nothing
    // (with beta = 0 there, their k, q, v never reach a stored result).
    float ell[16][CPT];
    {
        float run[CPT];
#pragma unroll
        for (int e = 0; e < CPT; ++e) run[e] = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const bool valid = 16 * R + r < ci.len;
#pragma unroll
            for (int e = 0; e < CPT; ++e) {
                run[e] += valid ? la[r][e] : 0.f;
                ell[r][e] = run[e];
            }
        }
#pragma unroll
        for (int e = 0; e < CPT; ++e) sTau[R * DK + c0 + e] = run[e];
        if (wave == 0) sBeta[lane] = lane < ci.len ? (beta_logit ? sigmoid(bt) : bt) : 0.f;
    }
    __syncthreads();

    // ---- phase 0b: block references, decay table, decayed keys and queries ----
    if constexpr (NORM) {
        l2_normalise_rows<CPT>(kr, lane);
        l2_normalise_rows<CPT>(qr, lane);
    }
    float eB[CPT], eTE[CPT];   // e^{B_R} (g before block R);  e^{g_C - B_R}
#pragma unroll
    for (int e = 0; e < CPT; ++e) {
        float a = 0.f, b = 0.f;
#pragma unroll
        for (int Rp = 0; Rp < 4; ++Rp) {
            const float tv = sTau[Rp * DK + c0 + e];
            if (Rp < R) a += tv; else b += tv;
        }
        eB[e] = fast_exp(a);
        eTE[e] = fast_exp(b);
    }
    // e^{B_R - B_I} for the six off-diagonal block pairs (all <= 1)
    for (int idx = t; idx < 6 * DK; idx += 256) {
        const int p = idx / DK, c = idx % DK;
        float d = 0.f;
        for (int Rp = off_i(p); Rp < off_r(p); ++Rp) d += sTau[Rp * DK + c];
        sEtab[idx] = fast_exp(d);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int row = 16 * R + r;
        E kp[CPT], kd[CPT], qp[CPT];
#pragma unroll
        for (int e = 0; e < CPT; ++e) {
            const float P = fast_exp(ell[r][e]);                   // e^{g_r - B_R} <= 1
            const float iP = fast_exp(fminf(-ell[r][e], 80.f));    // e^{B_R - g_r}
            kp[e] = from_f32<E>(kr[r][e] * P);
            kd[e] = from_f32<E>(kr[r][e] * iP);
            qp[e] = from_f32<E>(qr[r][e] * P);
            ell[r][e] = kr[r][e] * iP * eTE[e];                    // Khat: k e^{g_C - g_r}
            kr[r][e] *= P * eB[e];                                 // e^{g_r} k  (for W)
            qr[r][e] *= P * eB[e];                                 // Qg = e^{g_r} q
        }
        store_row<CPT>(sKP + row * L::LK + c0, kp);
        store_row<CPT>(sKD + row * L::LK + c0, kd);
        store_row<CPT>(sQP + row * L::LK + c0, qp);
    }
    if (R == 0) {
#pragma unroll
        for (int e = 0; e < CPT; ++e) out.gC[c0 + e] = eTE[e];
    }
    __syncthreads();

    // ---- phase 1: A_kk and A_qk^T tiles of each block pair (R, I), I <= R ----
    // A_kk: A operand k_r e^{g_r - B_R}, B operand k_i e^{B_I - g_i} e^{B_R - B_I};
    // A_qk^T: that same key operand as A, q_r e^{g_r - B_R} as B.  The decay
    // scaling of the key fragments is done once for both products, and the
    // diagonal test once per tile, so each path is straight code.  A_qk
    // tiles stay in registers until the barrier: their LDS area holds q.
    auto pair_tiles = [&](const int PR, const int PI, const bool diag) {
        const float* f = sEtab + (PR * (PR - 1) / 2 + PI) * DK;
        V8 a[KS], b[KS], qf[KS];
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const int cb = 32 * s + 8 * g;
            a[s] = frag8<E>(sKP + (16 * PR + ln) * L::LK + cb);
            b[s] = diag ? frag8<E>(sKD + (16 * PI + ln) * L::LK + cb)
                        : frag8_scaled<E>(sKD + (16 * PI + ln) * L::LK + cb, f + cb);
            qf[s] = frag8<E>(sQP + (16 * PR + ln) * L::LK + cb);
        }
        const f32x4 bt4 = *reinterpret_cast<const f32x4*>(sBeta + 16 * PR + 4 * g);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f}, aq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            acc = mma32(a[s], b[s], acc);
            aq = mma32(b[s], qf[s], aq);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 16 * PR + 4 * g + i, col = 16 * PI + ln;
            sAL[r * L::LA + col] = r > col ? bt4[i] * acc[i] : 0.f;
        }
        // A_qk^T tile: lane holds A_qk[16 PR + ln][16 PI + 4g + i] (causal mask)
        V4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            w[i] = from_f32<E>(16 * PR + ln >= 16 * PI + 4 * g + i ? aq[i] : 0.f);
        return w;
    };
    V4 qk[3];
#pragma unroll
    for (int k3 = 0; k3 < 3; ++k3) {
        const int p = wave + 4 * k3;
        if (p < 10) {
            const int PR = pair_r(p), PI = pair_i(p);
            qk[k3] = PR == PI ? pair_tiles(PR, PI, true) : pair_tiles(PR, PI, false);
        }
    }
    for (int u = wave - 2; u >= 0 && u < 6; u += 2) {   // waves 2 and 3 zero the upper tiles
        const int UR = off_i(u), UI = off_r(u);   // the transposed (upper) tile
#pragma unroll
        for (int i = 0; i < 4; ++i) sAL[(16 * UR + 4 * g + i) * L::LA + 16 * UI + ln] = 0.f;
    }
    __syncthreads();   // kp, kd, q operands dead: U1 becomes kgT / vT, the q area A_qk

    // A_qk[r][perm32(i)] for the read-out products; the upper tiles are zero
#pragma unroll
    for (int k3 = 0; k3 < 3; ++k3) {
        const int p = wave + 4 * k3;
        if (p < 10) {
            const int PR = pair_r(p), PI = pair_i(p);
            store_vec(sAQ + (16 * PR + ln) * L::LT + perm_index(16 * PI + 4 * g), qk[k3]);
        }
    }
    for (int u = wave - 2; u >= 0 && u < 6; u += 2) {
        const int UR = off_i(u), UI = off_r(u);   // the transposed (upper) tile
        V4 z;
#pragma unroll
        for (int i = 0; i < 4; ++i) z[i] = from_f32<E>(0.f);
        store_vec(sAQ + (16 * UR + ln) * L::LT + perm_index(16 * UI + 4 * g), z);
    }

    // ---- phase 3a: (e^g k)^T and v^T in LDS; diagonal 16x16 inverses ----------
#pragma unroll
    for (int e = 0; e < CPT; ++e) {
        V8 lo, hi;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            lo[r] = from_f32<E>(kr[r][e]);
            hi[r] = from_f32<E>(kr[r + 8][e]);
        }
        store_vec(sKGT + (c0 + e) * L::LT + 16 * R, lo);
        store_vec(sKGT + (c0 + e) * L::LT + 16 * R + 8, hi);
    }
#pragma unroll
    for (int e = 0; e < CPTV; ++e) {
        V8 lo, hi;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            lo[r] = from_f32<E>(vr[r][e]);
            hi[r] = from_f32<E>(vr[r + 8][e]);
        }
        store_vec(sVT + (cv0 + e) * L::LT + 16 * R, lo);
        store_vec(sVT + (cv0 + e) * L::LT + 16 * R + 8, hi);
    }
    if (wave == 0) {
        // lane (blk, j) solves (I + A_blk) x = e_j on diagonal block blk
        const int blk = lane >> 4, j = lane & 15;
        const float* Ab = sAL + 16 * blk * L::LA + 16 * blk;
        float x[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) x[i] = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float acc = (r == j) ? 1.f : 0.f;
#pragma unroll
            for (int i4 = 0; i4 < (r + 3) / 4; ++i4) {
                const f32x4 a = *reinterpret_cast<const f32x4*>(Ab + r * L::LA + 4 * i4);
                acc -= a[0] * x[4 * i4] + a[1] * x[4 * i4 + 1] + a[2] * x[4 * i4 + 2] +
                       a[3] * x[4 * i4 + 3];
            }
            x[r] = acc;
        }
        float* Xt = sAL + (16 * blk + j) * L::LA + 16 * blk;   // row j of the block, transposed store
#pragma unroll
        for (int r = 0; r < 16; ++r)
            if (r > j) Xt[r] = x[r];
    }
    __syncthreads();

    // ---- phase 3b: off-diagonal blocks of X, wave w down column block w ------
    if (wave == 0) x_column<L::LA, 0>(sAL, g, ln);
    else if (wave == 1) x_column<L::LA, 1>(sAL, g, ln);
    else if (wave == 2) x_column<L::LA, 2>(sAL, g, ln);
    __syncthreads();

    // ---- phase 3e: T = X Diag(beta) in the operand dtype ----------------------
    // lane = row r, wave w: column groups 2w, 2w + 1 (8 columns each, one
    // 16-byte store); X[r][c] for r > c sits transposed at sAL[c][r], so the
    // 64 lanes of one read touch 64 consecutive words.
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
        const int r = lane, c0 = 8 * (2 * wave + k2);
        const f32x4 b0 = *reinterpret_cast<const f32x4*>(sBeta + c0);
        const f32x4 b1 = *reinterpret_cast<const f32x4*>(sBeta + c0 + 4);
        float xv[8];
#pragma unroll
        for (int m = 0; m < 8; ++m) xv[m] = sAL[(c0 + m) * L::LA + r];
        V8 w;
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const int c = c0 + m;
            const float x = r > c ? xv[m] : (r == c ? 1.f : 0.f);
            w[m] = from_f32<E>(x * (m < 4 ? b0[m] : b1[m - 4]));
        }
        store_vec(sTL + r * L::LT + c0, w);
    }
    __syncthreads();   // X dead: its bytes become Khat^T

    // ---- phase 3f: Khat^T with tokens in perm32 order ---------------------------
#pragma unroll
    for (int e = 0; e < CPT; ++e) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            V4 w;
#pragma unroll
            for (int i = 0; i < 4; ++i) w[i] = from_f32<E>(ell[4 * r4 + i][e]);
            store_vec(sKHT + (c0 + e) * L::LT + perm_index(16 * R + 4 * r4), w);
        }
    }

    // ---- phase 4: W = T (e^g K) and U = T V on MFMA, kept in registers ---------
    // tile (Rq, column block): lane holds rows 16Rq + 4g + i, column 16cb + ln.
    // T is lower triangular, so token block Rq only needs key tokens < 16Rq+16.
    f32x4 Wt[NWB][4], Ut[NUB][4];
#pragma unroll
    for (int bw = 0; bw < NWB; ++bw) {
        const int ct = NWB * wave + bw;
        if (ct < DK / 16) {
            V8 a[4][2], b[2];
#pragma unroll
            for (int s = 0; s < 2; ++s) b[s] = frag8<E>(sKGT + (16 * ct + ln) * L::LT + 32 * s + 8 * g);
#pragma unroll
            for (int Rq = 0; Rq < 4; ++Rq)
#pragma unroll
                for (int s = 0; s <= Rq / 2; ++s) a[Rq][s] = frag8<E>(sTL + (16 * Rq + ln) * L::LT + 32 * s + 8 * g);
#pragma unroll
            for (int Rq = 0; Rq < 4; ++Rq) Wt[bw][Rq] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int Rq = 2 * s; Rq < 4; ++Rq) Wt[bw][Rq] = mma32(a[Rq][s], b[s], Wt[bw][Rq]);
        }
    }
#pragma unroll
    for (int bu = 0; bu < NUB; ++bu) {
        const int ct = NUB * wave + bu;
        if (ct < DV / 16) {
            V8 a[4][2], b[2];
#pragma unroll
            for (int s = 0; s < 2; ++s) b[s] = frag8<E>(sVT + (16 * ct + ln) * L::LT + 32 * s + 8 * g);
#pragma unroll
            for (int Rq = 0; Rq < 4; ++Rq)
#pragma unroll
                for (int s = 0; s <= Rq / 2; ++s) a[Rq][s] = frag8<E>(sTL + (16 * Rq + ln) * L::LT + 32 * s + 8 * g);
#pragma unroll
            for (int Rq = 0; Rq < 4; ++Rq) Ut[bu][Rq] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int Rq = 2 * s; Rq < 4; ++Rq) Ut[bu][Rq] = mma32(a[Rq][s], b[s], Ut[bu][Rq]);
        }
    }
    __syncthreads();   // kgT / vT dead: the region holds A_qk W from here on

    // ---- phase 5: transition and read-out products -------------------------
    //   PM^T (c', c) = -(W^T Khat)   Hc (c, j) = Khat^T U
    //   (A_qk W)^T (c', r)            OI^T (j, r) = U^T A_qk^T
    // W and U enter as operands straight from their accumulator tiles.  A wave
    // owns adjacent column tiles 2w, 2w + 1; in perm32 order their columns
    // 4g..4g+3 and 16+4g..16+4g+3 are the 8 consecutive slots 8g..8g+7 of the
    // 32-column block, so each lane writes 16 contiguous bytes.
    {
        static_assert(NWB == 1 || NWB == 2, "column tiles per wave");
        V8 wf[NWB][2];
#pragma unroll
        for (int bw = 0; bw < NWB; ++bw) {
            wf[bw][0] = tiles_to_frag<E>(Wt[bw][0], Wt[bw][1]);
            wf[bw][1] = tiles_to_frag<E>(Wt[bw][2], Wt[bw][3]);
        }
        const int ct0 = NWB * wave;
        if (ct0 < DK / 16) {
            // PM rows c = 16a + ln; columns 16 ct0 + 4g + i (and 16 (ct0 + 1) + 4g + i)
#pragma unroll
            for (int a = 0; a < DK / 16; ++a) {
                V8 kf[2];
#pragma unroll
                for (int s = 0; s < 2; ++s) kf[s] = frag8<E>(sKHT + (16 * a + ln) * L::LT + 32 * s + 8 * g);
                f32x4 acc[NWB];
#pragma unroll
                for (int bw = 0; bw < NWB; ++bw) {
                    acc[bw] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s = 0; s < 2; ++s) acc[bw] = mma32(wf[bw][s], kf[s], acc[bw]);
                }
                E* dst = out.PM + (16 * a + ln) * DK + perm_index(16 * ct0 + 4 * g);
                if constexpr (NWB == 2) {
                    V8 w;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        w[i] = from_f32<E>(-acc[0][i]);
                        w[4 + i] = from_f32<E>(-acc[1][i]);
                    }
                    store_vec(dst, w);
                } else {
                    V4 w;
#pragma unroll
                    for (int i = 0; i < 4; ++i) w[i] = from_f32<E>(-acc[0][i]);
                    store_vec(dst, w);
                }
            }
            // (A_qk W)[r][c'] for r = 16Rr + ln, c' = 16ct + 4g + i  (A_qk is causal)
#pragma unroll
            for (int Rr = 0; Rr < 4; ++Rr) {
                V8 af[2];
#pragma unroll
                for (int s = 0; s <= Rr / 2; ++s) af[s] = frag8<E>(sAQ + (16 * Rr + ln) * L::LT + 32 * s + 8 * g);
#pragma unroll
                for (int bw = 0; bw < NWB; ++bw) {
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s = 0; s <= Rr / 2; ++s) acc = mma32(wf[bw][s], af[s], acc);
                    *reinterpret_cast<f32x4*>(sQA + (16 * Rr + ln) * L::LQA + 16 * (ct0 + bw) + 4 * g) = acc;
                }
            }
        }
    }
    {
        static_assert(NUB == 1 || NUB == 2, "value tiles per wave");
        V8 uf[NUB][2];
#pragma unroll
        for (int bu = 0; bu < NUB; ++bu) {
            uf[bu][0] = tiles_to_frag<E>(Ut[bu][0], Ut[bu][1]);
            uf[bu][1] = tiles_to_frag<E>(Ut[bu][2], Ut[bu][3]);
        }
        const int ct0 = NUB * wave;
        if (ct0 < DV / 16) {
            // Hc rows c = 16a + 4g + i, column j = 16ct + ln  ->  Hc^T[j][perm(c)]:
            // row tiles a = 2m and 2m + 1 fill slots 32m + 8g .. +7
#pragma unroll
            for (int bu = 0; bu < NUB; ++bu) {
                const int ct = ct0 + bu;
#pragma unroll
                for (int m = 0; m < DK / 32; ++m) {
                    f32x4 acc[2];
#pragma unroll
                    for (int h2 = 0; h2 < 2; ++h2) {
                        const int a = 2 * m + h2;
                        acc[h2] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int s = 0; s < 2; ++s)
                            acc[h2] = mma32(frag8<E>(sKHT + (16 * a + ln) * L::LT + 32 * s + 8 * g), uf[bu][s], acc[h2]);
                    }
                    V8 w;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        w[i] = from_f32<E>(acc[0][i]);
                        w[4 + i] = from_f32<E>(acc[1][i]);
                    }
                    store_vec(out.HCt + (16 * ct + ln) * DK + 32 * m + 8 * g, w);
                }
            }
            // OI[r][perm(j)] for r = 16Rr + ln, j = 16ct + 4g + i
#pragma unroll
            for (int Rr = 0; Rr < 4; ++Rr) {
                V8 af[2];
#pragma unroll
                for (int s = 0; s <= Rr / 2; ++s) af[s] = frag8<E>(sAQ + (16 * Rr + ln) * L::LT + 32 * s + 8 * g);
                f32x4 acc[NUB];
#pragma unroll
                for (int bu = 0; bu < NUB; ++bu) {
                    acc[bu] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s = 0; s <= Rr / 2; ++s) acc[bu] = mma32(uf[bu][s], af[s], acc[bu]);
                }
                E* dst = out.OI + (16 * Rr + ln) * DV + perm_index(16 * ct0 + 4 * g);
                if constexpr (NUB == 2) {
                    V8 w;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        w[i] = from_f32<E>(acc[0][i]);
                        w[4 + i] = from_f32<E>(acc[1][i]);
                    }
                    store_vec(dst, w);
                } else {
                    V4 w;
#pragma unroll
                    for (int i = 0; i < 4; ++i) w[i] = from_f32<E>(acc[0][i]);
                    store_vec(dst, w);
                }
            }
        }
    }
    __syncthreads();

    // ---- phase 6: QM = Qg - A_qk W in the row mapping ------------------------
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int row = 16 * R + r;
        typename Vec<E>::v2 w2;
#pragma unroll
        for (int e = 0; e < CPT; ++e) {
            const E val = from_f32<E>(qr[r][e] - sQA[row * L::LQA + c0 + e]);
            if constexpr (CPT == 2) w2[e] = val;
            else out.QM[row * DK + perm_index(c0 + e)] = val;
        }
        if constexpr (CPT == 2) store_vec(out.QM + row * DK + perm_index(c0), w2);
    }
}

template <typename E, int DK, int DV>
static hipError_t launch_intra_t(const void* q, const void* k, const void* v, const float* la,
                                 const float* beta, ChunkSrc src, int max_chunks, int H,
                                 unsigned flags, void* rec, hipStream_t stream)
{
    const int beta_logit = (flags & PRE_BETA_LOGIT) ? 1 : 0;
    if (flags & PRE_L2NORM_QK)
        hipLaunchKernelGGL((prefill_intra_kernel<E, DK, DV, true>), dim3(max_chunks * H), dim3(256), 0,
                           stream, (const E*)q, (const E*)k, (const E*)v, la, beta, src, H,
                           beta_logit, (unsigned char*)rec);
    else
        hipLaunchKernelGGL((prefill_intra_kernel<E, DK, DV, false>), dim3(max_chunks * H), dim3(256), 0,
                           stream, (const E*)q, (const E*)k, (const E*)v, la, beta, src, H,
                           beta_logit, (unsigned char*)rec);
    return hipGetLastError();
}

hipError_t launch_prefill_intra(const void* q, const void* k, const void* v, const float* la,
                                const float* beta, ChunkSrc src, int max_chunks, int H, int dk,
                                int dv, bool bf16_io, unsigned flags, void* rec, hipStream_t stream)
{
#define KDA_INTRA_CASE(E, DK_, DV_)                                                               \
    if (dk == DK_ && dv == DV_)                                                                  \
        return launch_intra_t<E, DK_, DV_>(q, k, v, la, beta, src, max_chunks, H, flags, rec, stream);
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
