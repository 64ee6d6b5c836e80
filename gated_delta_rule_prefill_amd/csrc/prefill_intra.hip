// prefill_intra.hip -- per-chunk work of the chunkwise KDA prefill.
//
// One workgroup (8 waves) per (chunk, head); chunks are independent, so the
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
//   T         = (I + A_kk)^{-1} Diag(beta)         blockwise, see below
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
// four 16x16 diagonal blocks by forward substitution (one lane per column,
// by the wave that built the block), then the off-diagonal blocks on fp32
// MFMA, each wave walking down one column block with the blocks above it in
// registers, stored transposed in the unused upper triangle of A_kk.
//
// Wave w holds tokens 8w .. 8w + 7 in the row mapping (lane l: key channels
// l*dk/64 ..), so the per-token work of the loads, the decay factors and QM
// is spread over all eight waves; the MFMA phases split their tiles over
// the waves.  Eight waves of at most 128 registers, two workgroups per CU,
// keep 16 waves resident to cover the memory and MFMA latencies.
//
// Decay factors never form 1/gamma over a whole chunk: the chunk is cut into
// four 16-token blocks with reference log-decays B_R (g just before block R).
// Row factors e^{g_r - B_R} and cross-block factors e^{B_R - B_I} are <= 1;
// only the within-block factor e^{B_I - g_i} exceeds 1, bounded by the decay
// of at most 16 tokens.
#include <hip/hip_ext.h>

#include "kda_common.h"

namespace kda {

constexpr int INTRA_WAVES = 8;   // waves per workgroup

template <typename E, int DK, int DV>
struct IntraLayout {
    static constexpr int ES = sizeof(E);
    static constexpr int PAD = 16 / ES;              // 16-byte row padding (elements)
    static constexpr int LK = DK + PAD;              // row stride of [64][DK] arrays
    static constexpr int LT = CHUNK + PAD;           // row stride of [d][64] / [64][64] arrays
    static constexpr int LA = CHUNK + 4;             // row stride of the fp32 A / X array
    // region U1: phase 0b-1 KP and KD; phase 3-4 kgT and vT; phase 5-6 QA (fp32 A_qk W)
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
    // fp32 [8][DK]: log-decay summed over each wave's 8 tokens
    static constexpr int OFF_HALF = OFF_AQ + ((CHUNK * LT * ES + 15) & ~15);
    // phase 0b-1: q e^{g - B} ([64][LK]) over the T and A_qk areas, free until then
    static constexpr int OFF_QP = OFF_TL;
    static_assert(OFF_QP + CHUNK * LK * ES <= OFF_HALF, "q operand area");
    static constexpr int OFF_ETAB = OFF_HALF + 8 * DK * 4;
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

// CPT consecutive elements as loaded (one streaming load, kept packed), and
// element e of them.
template <typename E, int CPT> struct Raw { typedef typename Vec<E>::v2 type; };
template <typename E> struct Raw<E, 1> { typedef E type; };
template <int CPT, typename E>
__device__ __forceinline__ typename Raw<E, CPT>::type load_raw(const E* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const typename Raw<E, CPT>::type*>(p));
}
template <int CPT, typename T>
__device__ __forceinline__ auto raw_get(const T& v, int e) {
    if constexpr (CPT == 2) return v[e];
    else return v;
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

// Inverse of a unit lower-triangular diagonal block of I + A_kk by forward
// substitution from registers: lane (g, l) holds am = A[4g + i][l], i = 0..3
// (zero on and above the diagonal), and every lane solves (I + A) x = e_l,
// the row-r coefficients A[r][i] broadcast from the lane that holds them
// (v_readlane).  The substitution's only chain is one multiply-add per row.
// Lanes of group 0 store the strictly lower part of column l transposed,
// into the block's upper triangle at sX (= sAL + 16 blk LA + 16 blk).
template <int LA>
__device__ __forceinline__ void diag_inverse(const f32x4& am, float* sX, int g, int l) {
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        float acc = (r == l) ? 1.f : 0.f;
#pragma unroll
        for (int i = 0; i < r; ++i) acc -= read_lane(am[r & 3], 16 * (r >> 2) + i) * x[i];
        x[r] = acc;
    }
    if (g == 0) {
#pragma unroll
        for (int r = 1; r < 16; ++r)
            if (r > l) sX[l * LA + r] = x[r];
    }
}

// NORM: L2-normalise q and k rows first; beta_logit: beta arrives as a logit.
// bf16 operands fit 128 registers per lane (four waves per SIMD: two
// workgroups per CU, bounded by LDS); fp32 operands take up to 256.
// BWD: the record of the reverse chain of the backward pass instead (see the
// launcher): PM^T in PM's place, E = QM^T dO (dO: the output gradient) in
// Hc's place, gamma_C as before; QM's area takes X and X^T (64 x 64 each,
// row-major) and OI's area A_qk^T, which the gradient kernel reads.
template <typename E, int DK, int DV, bool NORM, bool BWD = false>
__global__ __launch_bounds__(64 * INTRA_WAVES)
__attribute__((amdgpu_waves_per_eu(sizeof(E) == 2 ? 4 : 2))) void prefill_intra_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
    const float* __restrict__ log_alpha, const float* __restrict__ beta,
    const ChunkSrc src, int H, int beta_logit,
    unsigned char* __restrict__ rec, const E* __restrict__ d_o = nullptr)
{
    using L = IntraLayout<E, DK, DV>;
    using V4 = typename Vec<E>::v4;
    using V8 = typename Vec<E>::v8;
    constexpr int CPT = DK / 64;   // key channels per lane in the row mapping
    constexpr int CPTV = DV / 64;  // value channels per lane
    constexpr int KS = DK / 32;    // contraction steps over key channels
    constexpr int NR = CHUNK / INTRA_WAVES;   // token rows per wave
    constexpr int NWP = DK / 32;   // pairs of 16-column tiles of W
    constexpr int NUP = DV / 32;   // ... and of U
    static_assert(NR == 8 && NWP + NUP <= INTRA_WAVES, "work split");
    using RK = typename Raw<E, CPT>::type;
    using RV = typename Raw<E, CPTV>::type;

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
    float* sHalf = reinterpret_cast<float*>(smem + L::OFF_HALF);
    float* sEtab = reinterpret_cast<float*>(smem + L::OFF_ETAB);
    float* sBeta = reinterpret_cast<float*>(smem + L::OFF_BETA);

    // chunks in descending order, so the sequential kernel (first chunk first)
    // finds the most recently written records first; the reverse chain starts
    // from the last chunk, so its records go in ascending order
    int cid, h;
    chunk_head_of_block(H, !BWD, cid, h);
    int n_chunks;
    ChunkInfo ci;
    chunk_of(src, cid, n_chunks, ci);
    if (cid >= n_chunks) return;
    const size_t chh = (size_t)cid * H + h;
    const ChunkOut<E, DK, DV> out(rec, chh);

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int R = wave >> 1;       // 16-token block of the wave's rows
    const int rb = NR * wave;      // first of the wave's rows
    const int g = lane >> 4, ln = lane & 15;
    const int c0 = lane * CPT;
    const int cv0 = lane * CPTV;

    // ---- phase 0: unconditional loads (rows past the end re-read the last row) -
    // Issued tensor by tensor in the order they are first needed: a wave's
    // loads complete in order, so the prefix sum waits only for log_alpha.
    // q, k and v stay packed until they are used.
    float la[NR][CPT];
    RK kraw[NR], qraw[NR];
    RV vraw[NR];
    size_t rowoff[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        const int row = rb + r;
        rowoff[r] = ((size_t)ci.start + (row < ci.len ? row : ci.len - 1)) * H + h;
    }
    // beta first: it is needed before the first barrier, and a wave's loads
    // complete in order (every wave loads it; wave 0 keeps it)
    const float bt = beta[((size_t)ci.start + (lane < ci.len ? lane : ci.len - 1)) * H + h];
#pragma unroll
    for (int r = 0; r < NR; ++r) load_row<CPT>(log_alpha + rowoff[r] * DK + c0, la[r]);
#pragma unroll
    for (int r = 0; r < NR; ++r) kraw[r] = load_raw<CPT>(k + rowoff[r] * DK + c0);
#pragma unroll
    for (int r = 0; r < NR; ++r) qraw[r] = load_raw<CPT>(q + rowoff[r] * DK + c0);
#pragma unroll
    for (int r = 0; r < NR; ++r) vraw[r] = load_raw<CPTV>(v + rowoff[r] * DV + cv0);
    // cumulative log-decay over the wave's rows; padded rows add nothing
    // (with beta = 0 there, their k, q, v never reach a stored result)
    float ell[NR][CPT];
    {
        float run[CPT];
#pragma unroll
        for (int e = 0; e < CPT; ++e) run[e] = 0.f;
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            const bool valid = rb + r < ci.len;
#pragma unroll
            for (int e = 0; e < CPT; ++e) {
                run[e] += valid ? la[r][e] : 0.f;
                ell[r][e] = run[e];
            }
        }
#pragma unroll
        for (int e = 0; e < CPT; ++e) sHalf[wave * DK + c0 + e] = run[e];
        if (wave == 0) sBeta[lane] = lane < ci.len ? (beta_logit ? sigmoid(bt) : bt) : 0.f;
    }
    __syncthreads();

    // ---- phase 0b: block references, decay table, decayed keys and queries ----
    float kr[NR][CPT], qr[NR][CPT];
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
        for (int e = 0; e < CPT; ++e) {
            kr[r][e] = to_f32(raw_get<CPT>(kraw[r], e));
            qr[r][e] = to_f32(raw_get<CPT>(qraw[r], e));
        }
    if constexpr (NORM) {
        l2_normalise_rows<NR, CPT>(kr, lane);
        l2_normalise_rows<NR, CPT>(qr, lane);
    }
    float eB[CPT], eTE[CPT];   // e^{B_R} (g before block R);  e^{g_C - B_R}
#pragma unroll
    for (int e = 0; e < CPT; ++e) {
        float a = 0.f, b = 0.f;
#pragma unroll
        for (int Rp = 0; Rp < 4; ++Rp) {
            const float tv = sHalf[2 * Rp * DK + c0 + e] + sHalf[(2 * Rp + 1) * DK + c0 + e];
            if (Rp < R) a += tv; else b += tv;
        }
        eB[e] = fast_exp(a);
        eTE[e] = fast_exp(b);
        if (wave & 1) {   // second half of block R: g_r - B_R includes the first half
            const float first = sHalf[(wave - 1) * DK + c0 + e];
#pragma unroll
            for (int r = 0; r < NR; ++r) ell[r][e] += first;
        }
    }
    // e^{B_R - B_I} for the six off-diagonal block pairs (all <= 1)
    for (int idx = t; idx < 6 * DK; idx += 64 * INTRA_WAVES) {
        const int p = idx / DK, c = idx % DK;
        float d = 0.f;
        for (int Rp = off_i(p); Rp < off_r(p); ++Rp) d += sHalf[2 * Rp * DK + c] + sHalf[(2 * Rp + 1) * DK + c];
        sEtab[idx] = fast_exp(d);
    }
    V8 kgt[CPT];       // e^g k, the wave's rows of key channel c0 + e  (W operand)
    V4 kht[CPT][2];    // Khat = k e^{g_C - g}, rows 4m .. 4m + 3
    RK qg[NR];         // Qg = e^g q in the operand dtype, until QM is formed
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        const int row = rb + r;
        E kp[CPT], kd[CPT], qp[CPT];
#pragma unroll
        for (int e = 0; e < CPT; ++e) {
            const float P = fast_exp(ell[r][e]);                   // e^{g_r - B_R} <= 1
            const float iP = fast_exp(fminf(-ell[r][e], 80.f));    // e^{B_R - g_r}
            kp[e] = from_f32<E>(kr[r][e] * P);
            kd[e] = from_f32<E>(kr[r][e] * iP);
            qp[e] = from_f32<E>(qr[r][e] * P);
            kht[e][r >> 2][r & 3] = from_f32<E>(kr[r][e] * iP * eTE[e]);
            const float PB = P * eB[e];                           // e^{g_r}
            kgt[e][r] = from_f32<E>(kr[r][e] * PB);
            if constexpr (CPT == 2) qg[r][e] = from_f32<E>(qr[r][e] * PB);
            else qg[r] = from_f32<E>(qr[r][e] * PB);
        }
        store_row<CPT>(sKP + row * L::LK + c0, kp);
        store_row<CPT>(sKD + row * L::LK + c0, kd);
        store_row<CPT>(sQP + row * L::LK + c0, qp);
    }
    // Qg stays packed from here to the QM phase: left free, the compiler
    // forms it there from the fp32 q rows and decays, which keeps twice the
    // registers alive across every phase and spills.
#pragma unroll
    for (int r = 0; r < NR; ++r) asm volatile("" : "+v"(qg[r]));
    V8 vt[CPTV];       // v, the wave's rows of value channel cv0 + e
#pragma unroll
    for (int e = 0; e < CPTV; ++e)
#pragma unroll
        for (int r = 0; r < NR; ++r) vt[e][r] = raw_get<CPTV>(vraw[r], e);
    if (wave == 0) {
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
    // Waves 0-3 take the diagonal pairs and invert their block of I + A_kk
    // right away from the tile's registers; waves 4-7 the six off-diagonal
    // pairs, whose A_kk tiles go to LDS.
    auto pair_tiles = [&](const int PR, const int PI, const bool diag, f32x4& am) {
        const float* f = sEtab + (PR * (PR - 1) / 2 + PI) * DK;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f}, aq = {0.f, 0.f, 0.f, 0.f};
        // two contraction steps per round of fragment loads (registers)
#pragma unroll
        for (int s0 = 0; s0 < KS; s0 += 2) {
            V8 a[2], b[2], qf[2];
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const int cb = 32 * (s0 + s) + 8 * g;
                a[s] = frag8<E>(sKP + (16 * PR + ln) * L::LK + cb);
                b[s] = diag ? frag8<E>(sKD + (16 * PI + ln) * L::LK + cb)
                            : frag8_scaled<E>(sKD + (16 * PI + ln) * L::LK + cb, f + cb);
                qf[s] = frag8<E>(sQP + (16 * PR + ln) * L::LK + cb);
            }
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                acc = mma32(a[s], b[s], acc);
                aq = mma32(b[s], qf[s], aq);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        const f32x4 bt4 = *reinterpret_cast<const f32x4*>(sBeta + 16 * PR + 4 * g);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 16 * PR + 4 * g + i, col = 16 * PI + ln;
            am[i] = r > col ? bt4[i] * acc[i] : 0.f;
            if (!diag) sAL[r * L::LA + col] = am[i];
        }
        // A_qk^T tile: lane holds A_qk[16 PR + ln][16 PI + 4g + i] (causal mask)
        V4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            w[i] = from_f32<E>(16 * PR + ln >= 16 * PI + 4 * g + i ? aq[i] : 0.f);
        return w;
    };
    // off-diagonal pairs of wave 4 + o: o = 0: 0, 1;  o = 1: 2, 3;  o = 2: 4;  o = 3: 5
    const int o = wave - 4;
    const int p0 = o < 2 ? 2 * o : o + 2;
    V4 qk[2];
    if (wave < 4) {
        f32x4 am;
        qk[0] = pair_tiles(wave, wave, true, am);
        diag_inverse<L::LA>(am, sAL + 16 * wave * L::LA + 16 * wave, g, ln);
    } else {
        f32x4 am;
        qk[0] = pair_tiles(off_r(p0), off_i(p0), false, am);
        if (o < 2) qk[1] = pair_tiles(off_r(p0 + 1), off_i(p0 + 1), false, am);
    }
    __syncthreads();   // kp, kd, q operands dead: U1 becomes kgT / vT, the q area A_qk

    // ---- phase 3: A_qk, (e^g k)^T and v^T to LDS; off-diagonal blocks of X ----
    // A_qk[r][perm32(i)] for the read-out products; the upper tiles are zero
    if (wave < 4) {
        store_vec(sAQ + (16 * wave + ln) * L::LT + perm_index(16 * wave + 4 * g), qk[0]);
    } else {
        store_vec(sAQ + (16 * off_r(p0) + ln) * L::LT + perm_index(16 * off_i(p0) + 4 * g), qk[0]);
        if (o < 2) {
            store_vec(sAQ + (16 * off_r(p0 + 1) + ln) * L::LT + perm_index(16 * off_i(p0 + 1) + 4 * g), qk[1]);
        } else {
            V4 z;
#pragma unroll
            for (int i = 0; i < 4; ++i) z[i] = from_f32<E>(0.f);
#pragma unroll
            for (int u = 3 * (o - 2); u < 3 * (o - 1); ++u)   // the transposed (upper) tiles
                store_vec(sAQ + (16 * off_i(u) + ln) * L::LT + perm_index(16 * off_r(u) + 4 * g), z);
        }
    }
#pragma unroll
    for (int e = 0; e < CPT; ++e) store_vec(sKGT + (c0 + e) * L::LT + rb, kgt[e]);
#pragma unroll
    for (int e = 0; e < CPTV; ++e) store_vec(sVT + (cv0 + e) * L::LT + rb, vt[e]);
    // X_RI for R > I: wave I walks down column block I
    if (wave == 0) x_column<L::LA, 0>(sAL, g, ln);
    else if (wave == 1) x_column<L::LA, 1>(sAL, g, ln);
    else if (wave == 2) x_column<L::LA, 2>(sAL, g, ln);
    __syncthreads();

    // ---- phase 3e: T = X Diag(beta) in the operand dtype ----------------------
    // lane = row r, wave w: columns 8w .. 8w + 7 (one 16-byte store); X[r][c]
    // for r > c sits transposed at sAL[c][r], so the 64 lanes of one read touch
    // 64 consecutive words.
    {
        const int r = lane, cg = 8 * wave;
        const f32x4 b0 = *reinterpret_cast<const f32x4*>(sBeta + cg);
        const f32x4 b1 = *reinterpret_cast<const f32x4*>(sBeta + cg + 4);
        float xv[8];
#pragma unroll
        for (int m = 0; m < 8; ++m) xv[m] = sAL[(cg + m) * L::LA + r];
        V8 w;
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const int c = cg + m;
            const float x = r > c ? xv[m] : (r == c ? 1.f : 0.f);
            w[m] = from_f32<E>(x * (m < 4 ? b0[m] : b1[m - 4]));
        }
        store_vec(sTL + r * L::LT + cg, w);
        if constexpr (BWD) {
            // X row-major (zeros above the unit diagonal) and X^T for the
            // gradient kernel, in the record's QM area: X[r][cg..cg+7] from
            // the values above, X^T[lane][8w..8w+7] = X[8w+m][lane] from row
            // `lane` of sAL
            V8 xr, xt;
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                const int c = cg + m;
                xr[m] = from_f32<E>(r > c ? xv[m] : (r == c ? 1.f : 0.f));
                const float a = sAL[r * L::LA + c];   // X[c][r] for c > r
                xt[m] = from_f32<E>(c > r ? a : (c == r ? 1.f : 0.f));
            }
            store_vec(out.QM + r * CHUNK + cg, xr);
            store_vec(out.QM + CHUNK * CHUNK + r * CHUNK + cg, xt);
        }
    }
    __syncthreads();   // X dead: its bytes become Khat^T

    // ---- phase 3f: Khat^T with tokens in perm32 order ---------------------------
#pragma unroll
    for (int e = 0; e < CPT; ++e)
#pragma unroll
        for (int m = 0; m < 2; ++m) store_vec(sKHT + (c0 + e) * L::LT + perm_index(rb + 4 * m), kht[e][m]);

    // ---- phase 4: W = T (e^g K) or U = T V on MFMA, kept in registers ---------
    // Waves 0 .. NWP-1 take the W column tiles 2p, 2p + 1, the next NUP waves
    // the U tiles.  Tile (Rq, column): lane holds rows 16Rq + 4g + i, column
    // 16ct + ln; T is lower triangular, so token block Rq only needs key tokens
    // < 16Rq + 16.  The tiles become MFMA operands over the tokens at once.
    const bool wside = wave < NWP, uside = !wside && wave < NWP + NUP;
    const int pr = wside ? wave : wave - NWP;   // column-tile pair
    const int ct0 = 2 * pr;
    V8 opf[2][2];   // [tile][32-token step]
    if (wside || uside) {
        const E* srcT = wside ? sKGT : sVT;
        V8 a[4][2];
#pragma unroll
        for (int Rq = 0; Rq < 4; ++Rq)
#pragma unroll
            for (int s = 0; s <= Rq / 2; ++s) a[Rq][s] = frag8<E>(sTL + (16 * Rq + ln) * L::LT + 32 * s + 8 * g);
#pragma unroll
        for (int bw = 0; bw < 2; ++bw) {
            V8 b[2];
#pragma unroll
            for (int s = 0; s < 2; ++s) b[s] = frag8<E>(srcT + (16 * (ct0 + bw) + ln) * L::LT + 32 * s + 8 * g);
            f32x4 acc[4];
#pragma unroll
            for (int Rq = 0; Rq < 4; ++Rq) acc[Rq] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int Rq = 2 * s; Rq < 4; ++Rq) acc[Rq] = mma32(a[Rq][s], b[s], acc[Rq]);
            opf[bw][0] = tiles_to_frag<E>(acc[0], acc[1]);
            opf[bw][1] = tiles_to_frag<E>(acc[2], acc[3]);
        }
    }
    __syncthreads();   // kgT / vT dead: the region holds A_qk W from here on

    // ---- phase 5: transition and read-out products -------------------------
    //   PM^T (c', c) = -(W^T Khat)   Hc (c, j) = Khat^T U
    //   (A_qk W)^T (c', r)            OI^T (j, r) = U^T A_qk^T
    // In perm32 order the columns 4g..4g+3 and 16+4g..16+4g+3 of a tile pair
    // are the 8 consecutive slots 8g..8g+7 of its 32-column block, so each
    // lane writes 16 contiguous bytes.
    if (wside && BWD) {
        // PM^T as A operands of the reverse chain: fragment (t, ks) holds, for
        // PM^T row 16t + ln (a PM column), PM rows 32ks + 4g + i and
        // 32ks + 16 + 4g + i -- two stacked accumulator tiles of K^T W with
        // K^T rows as the A operand and the W column tile t as the B operand
#pragma unroll
        for (int ks = 0; ks < DK / 32; ++ks) {
            f32x4 acc[2][2];   // [column tile bw][row tile 2ks + h2]
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                V8 kf[2];
#pragma unroll
                for (int s = 0; s < 2; ++s) kf[s] = frag8<E>(sKHT + (16 * (2 * ks + h2) + ln) * L::LT + 32 * s + 8 * g);
#pragma unroll
                for (int bw = 0; bw < 2; ++bw) {
                    acc[bw][h2] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s = 0; s < 2; ++s) acc[bw][h2] = mma32(kf[s], opf[bw][s], acc[bw][h2]);
                }
            }
#pragma unroll
            for (int bw = 0; bw < 2; ++bw) {
                V8 w;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    w[i] = from_f32<E>(-acc[bw][0][i]);
                    w[4 + i] = from_f32<E>(-acc[bw][1][i]);
                }
                store_frag(out.PM + frag_at<DK / 32>(ct0 + bw, ks), lane, w);
            }
        }
    }
    if (wside) {
        // PM rows c = 16a + ln; columns 16 ct0 + 4g + i and 16 (ct0 + 1) + 4g + i
#pragma unroll
        for (int a = 0; a < DK / 16 && !BWD; ++a) {
            V8 kf[2];
#pragma unroll
            for (int s = 0; s < 2; ++s) kf[s] = frag8<E>(sKHT + (16 * a + ln) * L::LT + 32 * s + 8 * g);
            f32x4 acc[2];
#pragma unroll
            for (int bw = 0; bw < 2; ++bw) {
                acc[bw] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < 2; ++s) acc[bw] = mma32(opf[bw][s], kf[s], acc[bw]);
            }
            V8 w;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                w[i] = from_f32<E>(-acc[0][i]);
                w[4 + i] = from_f32<E>(-acc[1][i]);
            }
            store_frag(out.PM + frag_at<DK / 32>(a, pr), lane, w);   // slots 8g .. 8g + 7 of block pr
        }
        // (A_qk W)[r][c'] for r = 16Rr + ln, c' = 16ct + 4g + i  (A_qk is causal)
#pragma unroll
        for (int Rr = 0; Rr < 4; ++Rr) {
            V8 af[2];
#pragma unroll
            for (int s = 0; s <= Rr / 2; ++s) af[s] = frag8<E>(sAQ + (16 * Rr + ln) * L::LT + 32 * s + 8 * g);
#pragma unroll
            for (int bw = 0; bw < 2; ++bw) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s <= Rr / 2; ++s) acc = mma32(opf[bw][s], af[s], acc);
                *reinterpret_cast<f32x4*>(sQA + (16 * Rr + ln) * L::LQA + 16 * (ct0 + bw) + 4 * g) = acc;
            }
        }
    } else if (uside && !BWD) {
        // Hc rows c = 16a + 4g + i, column j = 16ct + ln  ->  Hc^T[j][perm(c)]:
        // row tiles a = 2m and 2m + 1 fill slots 32m + 8g .. +7
#pragma unroll
        for (int m = 0; m < DK / 32; ++m) {
            f32x4 acc[2][2];   // [value tile][row tile 2m + h2]
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                V8 kf[2];
#pragma unroll
                for (int s = 0; s < 2; ++s) kf[s] = frag8<E>(sKHT + (16 * (2 * m + h2) + ln) * L::LT + 32 * s + 8 * g);
#pragma unroll
                for (int bu = 0; bu < 2; ++bu) {
                    acc[bu][h2] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s = 0; s < 2; ++s) acc[bu][h2] = mma32(kf[s], opf[bu][s], acc[bu][h2]);
                }
            }
#pragma unroll
            for (int bu = 0; bu < 2; ++bu) {
                V8 w;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    w[i] = from_f32<E>(acc[bu][0][i]);
                    w[4 + i] = from_f32<E>(acc[bu][1][i]);
                }
                store_frag_planar(out.HCt + frag_at<DK / 32>(ct0 + bu, m), lane, w);   // rows 2m, 2m + 1 as the planes
            }
        }
        // OI[r][perm(j)] for r = 16Rr + ln, j = 16ct + 4g + i
#pragma unroll
        for (int Rr = 0; Rr < 4; ++Rr) {
            V8 af[2];
#pragma unroll
            for (int s = 0; s <= Rr / 2; ++s) af[s] = frag8<E>(sAQ + (16 * Rr + ln) * L::LT + 32 * s + 8 * g);
            f32x4 acc[2];
#pragma unroll
            for (int bu = 0; bu < 2; ++bu) {
                acc[bu] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s <= Rr / 2; ++s) acc[bu] = mma32(opf[bu][s], af[s], acc[bu]);
            }
            V8 w;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                w[i] = from_f32<E>(acc[0][i]);
                w[4 + i] = from_f32<E>(acc[1][i]);
            }
            store_frag_planar(out.OI + frag_at<DV / 32>(Rr, pr), lane, w);   // slots 8g .. 8g + 7 of block pr
        }
    }
    __syncthreads();

    // ---- phase 6: QM = Qg - A_qk W in the row mapping ------------------------
    if constexpr (!BWD) {
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            const int row = rb + r;
            typename Vec<E>::v2 w2;
#pragma unroll
            for (int e = 0; e < CPT; ++e) {
                const E val = from_f32<E>(to_f32(raw_get<CPT>(qg[r], e)) - sQA[row * L::LQA + c0 + e]);
                if constexpr (CPT == 2) w2[e] = val;
                else out.QM[row * DK + perm_index(c0 + e)] = val;
            }
            if constexpr (CPT == 2) store_vec(out.QM + row * DK + perm_index(c0), w2);
        }
    } else {
        // ---- phases 6-7 of the reverse-chain record: E = QM^T dO ----------------
        // QM^T and dO^T go to LDS with the tokens contiguous (the rows of the
        // wave in order), over the area A_qk W occupied; rows past the end of the
        // sequence get dO = 0 so that they add nothing to E.
        V8 qmt[CPT], dot[CPTV];
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            const int row = rb + r;
#pragma unroll
            for (int e = 0; e < CPT; ++e)
                qmt[e][r] = from_f32<E>(to_f32(raw_get<CPT>(qg[r], e)) - sQA[row * L::LQA + c0 + e]);
            const RV dr = load_raw<CPTV>(d_o + rowoff[r] * DV + cv0);
#pragma unroll
            for (int e = 0; e < CPTV; ++e) dot[e][r] = row < ci.len ? raw_get<CPTV>(dr, e) : from_f32<E>(0.f);
        }
        __syncthreads();   // A_qk W dead: its area holds QM^T and dO^T
        E* sQMT = sKGT;    // [DK][LT], tokens in order
        E* sDOT = sVT;     // [DV][LT]
#pragma unroll
        for (int e = 0; e < CPT; ++e) store_vec(sQMT + (c0 + e) * L::LT + rb, qmt[e]);
#pragma unroll
        for (int e = 0; e < CPTV; ++e) store_vec(sDOT + (cv0 + e) * L::LT + rb, dot[e]);
        __syncthreads();
        // A_qk^T[i][r] (row-major, zero for r < i) for the gradient kernel, in
        // the record's OI area: thread (i, 8 tokens)
        {
            const int i = t >> 3, r0 = 8 * (t & 7);
            V8 w;
#pragma unroll
            for (int m = 0; m < 8; ++m) w[m] = sAQ[(r0 + m) * L::LT + perm_index(i)];
            store_vec(out.OI + i * CHUNK + r0, w);
        }
        // E tiles (row tile a = 2m + h2: key channels, column tile u: value
        // channels); wave w takes the tile pairs p = w, w + 8, ... of the
        // DK/32 x DV/16 pairs (m, u), each stored as one planar fragment of
        // E^T like Hc^T
        constexpr int PAIRS = (DK / 32) * (DV / 16);
        for (int p = wave; p < PAIRS; p += INTRA_WAVES) {
            const int m = p / (DV / 16), u = p % (DV / 16);
            V8 bf[2];
#pragma unroll
            for (int s = 0; s < 2; ++s) bf[s] = frag8<E>(sDOT + (16 * u + ln) * L::LT + 32 * s + 8 * g);
            f32x4 acc[2];
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                acc[h2] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < 2; ++s)
                    acc[h2] = mma32(frag8<E>(sQMT + (16 * (2 * m + h2) + ln) * L::LT + 32 * s + 8 * g), bf[s], acc[h2]);
            }
            V8 w;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                w[i] = from_f32<E>(acc[0][i]);
                w[4 + i] = from_f32<E>(acc[1][i]);
            }
            store_frag_planar(out.HCt + frag_at<DK / 32>(u, m), lane, w);
        }
    }
}

template <typename E, int DK, int DV>
static hipError_t launch_intra_t(const void* q, const void* k, const void* v, const float* la,
                                 const float* beta, ChunkSrc src, int max_chunks, int H,
                                 unsigned flags, void* rec, hipStream_t stream)
{
    const int beta_logit = (flags & PRE_BETA_LOGIT) ? 1 : 0;
    if (flags & PRE_L2NORM_QK)
        hipExtLaunchKernelGGL((prefill_intra_kernel<E, DK, DV, true>), dim3(max_chunks * H), dim3(64 * INTRA_WAVES), 0,
                           stream, launch_events().start, launch_events().stop, 0, (const E*)q, (const E*)k, (const E*)v, la, beta, src, H,
                           beta_logit, (unsigned char*)rec, (const E*)nullptr);
    else
        hipExtLaunchKernelGGL((prefill_intra_kernel<E, DK, DV, false>), dim3(max_chunks * H), dim3(64 * INTRA_WAVES), 0,
                           stream, launch_events().start, launch_events().stop, 0, (const E*)q, (const E*)k, (const E*)v, la, beta, src, H,
                           beta_logit, (unsigned char*)rec, (const E*)nullptr);
    return hipGetLastError();
}

hipError_t launch_reverse_records(const void* q, const void* k, const void* v, const float* la,
                                  const float* beta, const void* d_o, ChunkSrc src, int max_chunks,
                                  int H, int dk, int dv, void* rec, hipStream_t stream)
{
    if (dk != 128 || dv != 128) return hipErrorInvalidValue;
    hipExtLaunchKernelGGL((prefill_intra_kernel<bf16, 128, 128, false, true>), dim3(max_chunks * H),
                       dim3(64 * INTRA_WAVES), 0, stream, launch_events().start, launch_events().stop, 0, (const bf16*)q, (const bf16*)k,
                       (const bf16*)v, la, beta, src, H, 0, (unsigned char*)rec,
                       (const bf16*)d_o);
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
