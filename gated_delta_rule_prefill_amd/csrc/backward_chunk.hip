// backward_chunk.hip -- chunkwise gradients of the KDA prefill (bf16, dk = dv = 128).
//
// Reverse mode through one chunk of the chunkwise form (Kimi Linear paper
// notes, section 3: inside a chunk of C = 64 tokens the transitions fold into
// W = T (e^g K) and U = T V with T = (I + A_kk)^{-1} Diag(beta); the chunk
// reads the entering state S through O = Qg S + A_qk N, N = U - W S, and
// leaves S' = Diag(gamma_C) S + Khat^T N).  With S (the forward's chunk
// state) and dS (the gradient leaving the chunk, from the reverse chain, in
// bf16) every
// input gradient of the chunk is local to it:
//
//   dN  = A_qk^T dO + Khat dS             dQg = dO S^T      dKhat = N dS^T
//   dA_qk = tril(dO N^T)                  dW  = -dN S^T
//   dT  = tril(dW (e^g K)^T + dN V^T)     dKg = T^T dW      dV = T^T dN
//   dbeta_i = sum_r dT[r,i] X[r,i],   dA = -strict(X^T (dT Diag(beta)) X^T)
//   dL  = Diag(beta) dA,   dbeta_r += sum_i dA[r,i] L[r,i]   (A_kk = Diag(beta) L)
//
// and the decayed products A_qk[r,i] = sum_c q_rc k_ic e^{g_rc - g_ic} and
// L[r,i] (the same with k_r) pass dA_qk and dL back to q, k and g.  Their
// decay factors use the forward's 16-token block references B_R (g just
// before block R): e^{g_r - B_R} <= 1 and e^{B_R - B_I} <= 1 for I <= R, and
// only e^{B_I - g_i} inside one block exceeds 1.  The sum over i of
// dA[r,i] L[r,i] is taken as sum_c k_rc (dA-through product)[r,c], so L
// itself is never formed.  Then, with P = e^{g - B_R} per (row, channel),
//
//   dq = P (e^{B_R} dQg + XQ),   dk = P (e^{B_R} dKg + beta XL) + P^{-1} (e^{g_C - B_R} dKhat + Y)
//   dg = q dq + k (P (...) - P^{-1} (...)),   dlog_alpha = reverse cumsum of dg
//
// (XQ, XL: the dA_qk- and dA-through products over the key tokens i <= r;
// Y: the transposed ones over the rows r >= i), plus, for every row, the
// dependence of gamma_C and Khat on the chunk's last cumulative decay.
//
// One workgroup of 8 waves per (chunk, head).  Products whose output is
// [token][channel] are formed transposed (channel rows, token columns): wave w
// owns channel block w, the A operand is a per-channel run of 8 tokens or
// channels (gathered from LDS or read from memory), the B operand a token
// row read with one 16-byte LDS load, and each lane ends up with 4
// consecutive channels of one token.  The 64 x 64 products (dA_qk, dT, X^T dX,
// dA) split their 16 x 16 tiles over the waves.  S and dS are read once each
// with coalesced 16-byte loads and reach the MFMAs through a bf16 copy in LDS,
// from which every wave gathers them in the two orientations the products
// need.
#include "kda_common.h"

namespace kda {

namespace {

constexpr int CG_WAVES = 8;
constexpr int CG_LR = 136;   // row stride (elements) of bf16 [64][128] arrays
constexpr int CG_LT = 72;    // row stride of bf16 [64][64] arrays
constexpr int CG_LG = 132;   // row stride (floats) of fp32 [64][128] arrays
constexpr int CG_SLOT = 18432;   // a transient area: one [64][LR] or two [64][LT] arrays
// kept for the whole kernel
constexpr int CG_OFF_K = 0;                                  // k (rows past the end 0)
constexpr int CG_OFF_G = CG_OFF_K + CHUNK * CG_LR * 2;       // g, fp32
constexpr int CG_OFF_X = CG_OFF_G + CHUNK * CG_LG * 4;       // X row-major
constexpr int CG_OFF_XT = CG_OFF_X + CHUNK * CG_LT * 2;      // X^T row-major
constexpr int CG_OFF_BETA = CG_OFF_XT + CHUNK * CG_LT * 2;   // beta (0 past the end)
constexpr int CG_OFF_BREF = CG_OFF_BETA + CHUNK * 4;         // [5][128]: B_0..B_3, g_C
constexpr int CG_OFF_TOT = CG_OFF_BREF + 5 * 128 * 4;        // [4][128] per-block column sums
constexpr int CG_OFF_EXT = CG_OFF_TOT + 4 * 128 * 4;         // [2][128] per-channel last-row terms
constexpr int CG_OFF_DBC = CG_OFF_EXT + 2 * 128 * 4;         // [4][64] dbeta column partials
constexpr int CG_OFF_DBR = CG_OFF_DBC + 4 * 64 * 4;          // [8][64] dbeta row partials
// transient areas (see the phases)
constexpr int CG_OFF_S1 = CG_OFF_DBR + CG_WAVES * 64 * 4;
constexpr int CG_OFF_S2 = CG_OFF_S1 + CG_SLOT;
constexpr int CG_OFF_S3 = CG_OFF_S2 + CG_SLOT;
constexpr int CG_OFF_S4 = CG_OFF_S3 + CG_SLOT;
constexpr int CG_BYTES = CG_OFF_S4 + CG_SLOT;
static_assert(CG_OFF_S1 % 16 == 0 && CG_SLOT % 16 == 0, "16-byte aligned areas");
static_assert(CHUNK * CG_LR * 2 <= CG_SLOT && 2 * CHUNK * CG_LT * 2 <= CG_SLOT, "slot size");
static_assert(CHUNK * CG_LG * 4 <= 2 * CG_SLOT, "the scan area spans S3 and S4");
static_assert(CG_BYTES <= 160 * 1024, "LDS");

// 16x16 tile pairs (R, I) of a 64 x 64 matrix: slots 0..9 the lower ones
// (I <= R) in the order (0,0) (1,0) (1,1) (2,0) (2,1) (2,2) (3,0) ..., slots
// 10..15 the strictly upper ones (R < I).
struct TilePair { int R, I; };
__device__ __forceinline__ TilePair tile_pair(int p) {
    const int lr = (p >= 1) + (p >= 3) + (p >= 6);
    const int u = p - 10;   // (1,0) (2,0) (2,1) (3,0) (3,1) (3,2), transposed
    const int a = 1 + (u >= 1) + (u >= 3);
    return p < 10 ? TilePair{lr, p - lr * (lr + 1) / 2} : TilePair{u - a * (a - 1) / 2, a};
}

__device__ __forceinline__ bf16x8 lds8(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ f32x4 lds4f(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
// 8 elements down a column: p[0], p[ld], ..., p[7 ld]
__device__ __forceinline__ bf16x8 gather8(const bf16* p, int ld) {
    bf16x8 v;
#pragma unroll
    for (int m = 0; m < 8; ++m) v[m] = p[m * ld];
    return v;
}
__device__ __forceinline__ bf16x8 scale8(bf16x8 v, float f) {
#pragma unroll
    for (int m = 0; m < 8; ++m) v[m] = (bf16)((float)v[m] * f);
    return v;
}
__device__ __forceinline__ bf16x4 to_bf16x4(f32x4 a, float s = 1.f) {
    return bf16x4{(bf16)(s * a[0]), (bf16)(s * a[1]), (bf16)(s * a[2]), (bf16)(s * a[3])};
}
__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }
__device__ __forceinline__ float cexp(float x) { return fast_exp(fminf(x, 80.f)); }

// Sum over the 4 lane groups (lanes l, l ^ 16, l ^ 32, l ^ 48).
__device__ __forceinline__ float group4_sum(float x) {
    x += lane_xor<16>(x);
    return x + lane_xor<32>(x);
}

}  // namespace

__global__ __launch_bounds__(64 * CG_WAVES) void chunk_grad_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const float* __restrict__ log_alpha, const float* __restrict__ beta,
    const bf16* __restrict__ d_o, const ChunkSrc src, int H,
    const unsigned char* __restrict__ rec, const float* __restrict__ chunk_states,
    const bf16* __restrict__ dS_chunks, bf16* __restrict__ dq, bf16* __restrict__ dk,
    bf16* __restrict__ dv, float* __restrict__ dla, float* __restrict__ dbeta)
{
    constexpr int D = 128;
    constexpr int LR = CG_LR, LT = CG_LT, LG = CG_LG;
    __shared__ __attribute__((aligned(16))) unsigned char smem[CG_BYTES];
    bf16* sK = reinterpret_cast<bf16*>(smem + CG_OFF_K);
    float* sG = reinterpret_cast<float*>(smem + CG_OFF_G);
    bf16* sX = reinterpret_cast<bf16*>(smem + CG_OFF_X);
    bf16* sXT = reinterpret_cast<bf16*>(smem + CG_OFF_XT);
    float* sBeta = reinterpret_cast<float*>(smem + CG_OFF_BETA);
    float* sBref = reinterpret_cast<float*>(smem + CG_OFF_BREF);
    float* sTot = reinterpret_cast<float*>(smem + CG_OFF_TOT);
    float* sExt = reinterpret_cast<float*>(smem + CG_OFF_EXT);
    float* sDBC = reinterpret_cast<float*>(smem + CG_OFF_DBC);
    float* sDBR = reinterpret_cast<float*>(smem + CG_OFF_DBR);
    // S1: dO -> dW (row-major, dW = -dN S^T) -> q
    bf16* sDO = reinterpret_cast<bf16*>(smem + CG_OFF_S1);
    bf16* sDW = sDO;
    bf16* sQ = sDO;
    // S2: A_qk^T -> dA_qk, dA_qk^T
    bf16* sAqT = reinterpret_cast<bf16*>(smem + CG_OFF_S2);
    bf16* sDAq = sAqT;
    bf16* sDAqT = sAqT + CHUNK * LT;
    // S3: -W -> Khat -> dN -> dX^T, P
    bf16* sW = reinterpret_cast<bf16*>(smem + CG_OFF_S3);
    bf16* sKh = sW;
    bf16* sDN = sW;
    bf16* sDXT = sW;
    bf16* sP = sW + CHUNK * LT;
    // S4: N -> v -> e^g k -> dA, (Diag(beta) dA)^T
    bf16* sN = reinterpret_cast<bf16*>(smem + CG_OFF_S4);
    bf16* sV = sN;
    bf16* sKg = sN;
    bf16* sDA = sN;
    bf16* sDLT = sN + CHUNK * LT;
    // S3 + S4: dg for the reverse cumulative sum
    float* sScan = reinterpret_cast<float*>(smem + CG_OFF_S3);

    int cid, h;
    chunk_head_of_block(H, false, cid, h);
    int n_chunks;
    ChunkInfo ci;
    chunk_of(src, cid, n_chunks, ci);
    if (cid >= n_chunks) return;
    const int len = ci.len;
    const size_t chh = (size_t)cid * H + h;
    constexpr RecLayout RL = rec_layout(2, D, D);
    const bf16* rX = reinterpret_cast<const bf16*>(rec + chh * RL.bytes + RL.qm);
    const bf16* rXT = rX + CHUNK * CHUNK;
    const bf16* rAqT = reinterpret_cast<const bf16*>(rec + chh * RL.bytes + RL.oi);
    const float* Sg = chunk_states + chh * D * D;
    const bf16* dSg = dS_chunks + chh * D * D;   // bf16, as the reverse chain writes it
    const size_t r0 = (size_t)ci.start * H + h;
    const int HD = H * D;
    const bf16 *qB = q + r0 * D, *kB = k + r0 * D, *vB = v + r0 * D, *oB = d_o + r0 * D;
    const float* laB = log_alpha + r0 * D;

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);
    const int g = lane >> 4, ln = lane & 15;
    const int cw = 16 * w;          // the wave's channel block
    const int cl = cw + ln;         // the lane's channel as an A-operand row
    const int co = cw + 4 * g;      // the lane's 4 output channels

    // ---------------- phase 0: loads ------------------------------------------
    // Every global load of the phase goes out before the first wait (a wave's
    // loads complete in order, so each use below waits only for its own data
    // and those issued before it).  Token rows past the chunk's end re-read its
    // last row; their values are replaced by zeros where they are used.
    const int sc = t & (D - 1), sq = t >> 7;   // log_alpha: column sc, 16-row block sq
    const int last = len - 1;
    float lav[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) lav[u] = laB[min(16 * sq + u, last) * HD + sc];
    const float bet = beta[r0 + (size_t)min(t & (CHUNK - 1), last) * H];
    bf16x8 kv[2], dov[2];   // k and dO rows (t + 512e) >> 4, channels 8((t + 512e) & 15) ..
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const int u = t + 512 * e, r = min(u >> 4, last), c8 = 8 * (u & 15);
        kv[e] = *reinterpret_cast<const bf16x8*>(kB + r * HD + c8);
        dov[e] = *reinterpret_cast<const bf16x8*>(oB + r * HD + c8);
    }
    const int xr = t >> 3, x8 = 8 * (t & 7);   // X, X^T, A_qk^T from the record: row xr, columns x8 ..
    const bf16x8 xv = *reinterpret_cast<const bf16x8*>(rX + xr * CHUNK + x8);
    const bf16x8 xtv = *reinterpret_cast<const bf16x8*>(rXT + xr * CHUNK + x8);
    const bf16x8 aqv = *reinterpret_cast<const bf16x8*>(rAqT + xr * CHUNK + x8);
    // S and dS once each, coalesced: thread t takes rows (t >> 5) + 16e, columns
    // 4(t & 31) .. +3 (e = 0..7).  They reach the MFMAs through a bf16 copy in
    // LDS (S3 + S4, free until phase 1 writes -W), from which each wave
    // gathers its operands in both orientations.
    f32x4 sv[8];
    bf16x4 dsv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int at = ((t >> 5) + 16 * e) * D + 4 * (t & 31);
        sv[e] = *reinterpret_cast<const f32x4*>(Sg + at);
        dsv[e] = *reinterpret_cast<const bf16x4*>(dSg + at);
    }
    // v for the A operands over the tokens (for U): lane row j = cl, token
    // 32s + 8g + m; packed into operands after the S staging, so that its
    // waits come last
    bf16 vr[2][8];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int m = 0; m < 8; ++m) vr[s][m] = vB[min(32 * s + 8 * g + m, last) * HD + cl];

    // log_alpha: cumulative sum inside the thread's 16-row block
    float gl[16];
    {
        float run = 0.f;
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            // masked by a product, so that every load's value is used (a select
            // lets the compiler move the load under the condition)
            run = fmaf(lav[u], 16 * sq + u < len ? 1.f : 0.f, run);
            gl[u] = run;
        }
        sTot[sq * D + sc] = run;
    }
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const int u = t + 512 * e, r = u >> 4, c8 = 8 * (u & 15);
        *reinterpret_cast<bf16x8*>(sK + r * LR + c8) = r < len ? kv[e] : bf16x8{};
        *reinterpret_cast<bf16x8*>(sDO + r * LR + c8) = r < len ? dov[e] : bf16x8{};
    }
    *reinterpret_cast<bf16x8*>(sX + xr * LT + x8) = xv;
    *reinterpret_cast<bf16x8*>(sXT + xr * LT + x8) = xtv;
    *reinterpret_cast<bf16x8*>(sAqT + xr * LT + x8) = aqv;
    bf16* sSt = reinterpret_cast<bf16*>(smem + CG_OFF_S3);   // [128][LR] staging of S, then dS
    static_assert(D * CG_LR * 2 <= 2 * CG_SLOT, "S staging spans S3 and S4");
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int c = (t >> 5) + 16 * e;
        *reinterpret_cast<bf16x4*>(sSt + c * LR + 4 * (t & 31)) = to_bf16x4(sv[e]);
        float sd = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) sd += sv[e][i] * (float)dsv[e][i];
        sd = row16_sum(sd);
        sd += lane_xor<16>(sd);   // the 32 lanes of the row
        if ((t & 31) == 0) sExt[c] = sd;
    }
    if (t < CHUNK) sBeta[t] = t < len ? bet : 0.f;   // used from phase 1 on
    bf16x8 vop[2];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int m = 0; m < 8; ++m) vop[s][m] = 32 * s + 8 * g + m < len ? vr[s][m] : (bf16)0.f;
    __syncthreads();
    // S as A operands over the key channels c (for N; lane row = value channel
    // j = cl, slots c = 32s + 8g + m) and over the value channels j (for dQg,
    // dW; lane row = key channel c = cl, slots j = 32s + 8g + m)
    bf16x8 sN_op[4], sQ_op[4], dsN_op[4], dsQ_op[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        sN_op[s] = gather8(sSt + (32 * s + 8 * g) * LR + cl, LR);
        sQ_op[s] = lds8(sSt + cl * LR + 32 * s + 8 * g);
    }
    {
        float B = 0.f;
        for (int qd = 0; qd < sq; ++qd) B += sTot[qd * D + sc];
#pragma unroll
        for (int u = 0; u < 16; ++u) sG[(16 * sq + u) * LG + sc] = B + gl[u];
        sBref[sq * D + sc] = B;
        if (sq == 3) sBref[4 * D + sc] = B + sTot[3 * D + sc];
    }
    __syncthreads();
    // dS in S's place, its operands like S's (dKhat = N dS^T, dN = dS^T Khat^T)
#pragma unroll
    for (int e = 0; e < 8; ++e)
        *reinterpret_cast<bf16x4*>(sSt + ((t >> 5) + 16 * e) * LR + 4 * (t & 31)) = dsv[e];
    __syncthreads();
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        dsN_op[s] = gather8(sSt + (32 * s + 8 * g) * LR + cl, LR);
        dsQ_op[s] = lds8(sSt + cl * LR + 32 * s + 8 * g);
    }

    // T = X Diag(beta) as the B operand of token block R, step s: lane column
    // r = 16R + ln, slots i = 32s + 8g + m
    auto t_op = [&](int R, int s) {
        bf16x8 x = lds8(sX + (16 * R + ln) * LT + 32 * s + 8 * g);
        const f32x4 b0 = lds4f(sBeta + 32 * s + 8 * g), b1 = lds4f(sBeta + 32 * s + 8 * g + 4);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            x[m] = (bf16)((float)x[m] * b0[m]);
            x[4 + m] = (bf16)((float)x[4 + m] * b1[m]);
        }
        return x;
    };
    // T^T as the B operand of token block R (key tokens i = 16R + ln), slots
    // over the rows r = 32s + 8g + m: X[r][i] beta_i
    auto tt_op = [&](int R, int s) {
        return scale8(lds8(sXT + (16 * R + ln) * LT + 32 * s + 8 * g), sBeta[16 * R + ln]);
    };

    // ---------------- phase 1: W^T = (e^g K)^T T^T and U^T = V^T T^T -------------
    f32x4 accU[4];
    {
        f32x4 aws[4];
        bf16x8 kg[2];
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                const int i = 32 * s + 8 * g + m;
                kg[s][m] = (bf16)((float)sK[i * LR + cl] * fast_exp(sG[i * LG + cl]));
            }
#pragma unroll
        for (int R = 0; R < 4; ++R) {
            f32x4 aw = zero4(), au = zero4();
#pragma unroll
            for (int s = 0; s <= R / 2; ++s) {
                const bf16x8 tb = t_op(R, s);
                aw = mma32(kg[s], tb, aw);
                au = mma32(vop[s], tb, au);
            }
            accU[R] = au;
            aws[R] = aw;
        }
        __syncthreads();   // every wave has its dS operands: -W may overwrite the staging
#pragma unroll
        for (int R = 0; R < 4; ++R)   // lane: W[16R + ln][co + i]; stored negated for N = U - W S
            *reinterpret_cast<bf16x4*>(sW + (16 * R + ln) * LR + co) = to_bf16x4(aws[R], -1.f);
    }
    __syncthreads();

    // ---------------- phase 2: N^T = U^T - S^T W^T ---------------------------------
#pragma unroll
    for (int R = 0; R < 4; ++R) {
        f32x4 a = accU[R];
#pragma unroll
        for (int s = 0; s < 4; ++s) a = mma32(sN_op[s], lds8(sW + (16 * R + ln) * LR + 32 * s + 8 * g), a);
        *reinterpret_cast<bf16x4*>(sN + (16 * R + ln) * LR + co) = to_bf16x4(a);
    }
    __syncthreads();

    // ---------------- phase 3: dN^T = dO^T A_qk + dS^T Khat^T --------------------
    // Khat = e^{g_C - g} k, row-major, over -W
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const int u = t + 512 * e, r = u >> 4, c8 = 8 * (u & 15);
        const bf16x8 kv = lds8(sK + r * LR + c8);
        bf16x8 o;
#pragma unroll
        for (int m = 0; m < 8; ++m)
            o[m] = (bf16)((float)kv[m] * cexp(sBref[4 * D + c8 + m] - sG[r * LG + c8 + m]));
        *reinterpret_cast<bf16x8*>(sKh + r * LR + c8) = o;
    }
    f32x4 accN[4];
    {
        bf16x8 dop[2];   // dO as A operands over the tokens: lane row j = cl
#pragma unroll
        for (int s = 0; s < 2; ++s) dop[s] = gather8(sDO + (32 * s + 8 * g) * LR + cl, LR);
#pragma unroll
        for (int R = 0; R < 4; ++R) {
            f32x4 a = zero4();
            // A_qk[r][i] = 0 for r < i: token block R needs rows r >= 16R
#pragma unroll
            for (int s = R / 2; s < 2; ++s) a = mma32(dop[s], lds8(sAqT + (16 * R + ln) * LT + 32 * s + 8 * g), a);
            accN[R] = a;
        }
    }
    __syncthreads();
#pragma unroll
    for (int R = 0; R < 4; ++R)
#pragma unroll
        for (int s = 0; s < 4; ++s) accN[R] = mma32(dsN_op[s], lds8(sKh + (16 * R + ln) * LR + 32 * s + 8 * g), accN[R]);
    // v rows for dT, loaded now and stored once N's area is free
    bf16x8 vrow[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const int u = t + 512 * e, r = u >> 4, c8 = 8 * (u & 15);
        vrow[e] = bf16x8{};
        if (r < len) vrow[e] = *reinterpret_cast<const bf16x8*>(vB + r * HD + c8);
    }
    __syncthreads();
#pragma unroll
    for (int R = 0; R < 4; ++R)
        *reinterpret_cast<bf16x4*>(sDN + (16 * R + ln) * LR + co) = to_bf16x4(accN[R]);

    // ---------------- phase 4a: dQg^T = S dO^T, dKhat^T = dS N^T, dA_qk ------------
    f32x4 a1[4], a2[4], a3[4];   // see the header: dq = P a1, dk = P a2 + P^-1 a3
    {
        float ext[4] = {0.f, 0.f, 0.f, 0.f};
        const f32x4 gC4 = lds4f(sBref + 4 * D + co);
#pragma unroll
        for (int R = 0; R < 4; ++R) {
            f32x4 aq = zero4(), ak = zero4();
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                aq = mma32(sQ_op[s], lds8(sDO + (16 * R + ln) * LR + 32 * s + 8 * g), aq);
                ak = mma32(dsQ_op[s], lds8(sN + (16 * R + ln) * LR + 32 * s + 8 * g), ak);
            }
            const f32x4 B4 = lds4f(sBref + R * D + co);
            const f32x4 g4 = lds4f(sG + (16 * R + ln) * LG + co);
            const bf16x4 k4 = *reinterpret_cast<const bf16x4*>(sK + (16 * R + ln) * LR + co);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                a1[R][i] = fast_exp(B4[i]) * aq[i];
                a3[R][i] = fast_exp(gC4[i] - B4[i]) * ak[i];
                ext[i] += (float)k4[i] * cexp(gC4[i] - g4[i]) * ak[i];
            }
        }
        // per-channel sums over the 16 tokens of the lane row
#pragma unroll
        for (int i = 0; i < 4; ++i) ext[i] = row16_sum(ext[i]);
        if (ln == 0) *reinterpret_cast<f32x4*>(sExt + D + co) = f32x4{ext[0], ext[1], ext[2], ext[3]};
    }
    // dA_qk = tril(dO N^T): tile (Rr, Ri) with lane row r = 16Rr + 4g + i, column
    // i = 16Ri + ln; kept in both orientations (upper tiles zero)
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const TilePair tp = tile_pair(w + 8 * e);
        const int Rr = tp.R, Ri = tp.I;
        f32x4 a = zero4();
        if (Rr >= Ri) {
#pragma unroll
            for (int s = 0; s < 4; ++s)
                a = mma32(lds8(sDO + (16 * Rr + ln) * LR + 32 * s + 8 * g),
                          lds8(sN + (16 * Ri + ln) * LR + 32 * s + 8 * g), a);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (16 * Rr + 4 * g + i < 16 * Ri + ln) a[i] = 0.f;
        }
        *reinterpret_cast<bf16x4*>(sDAqT + (16 * Ri + ln) * LT + 16 * Rr + 4 * g) = to_bf16x4(a);
#pragma unroll
        for (int i = 0; i < 4; ++i) sDAq[(16 * Rr + 4 * g + i) * LT + 16 * Ri + ln] = (bf16)a[i];
    }
    __syncthreads();

    // ---------------- phase 4b: dW = -dN S^T --------------------------------------
#pragma unroll
    for (int R = 0; R < 4; ++R) {
        f32x4 a = zero4();
#pragma unroll
        for (int s = 0; s < 4; ++s) a = mma32(sQ_op[s], lds8(sDN + (16 * R + ln) * LR + 32 * s + 8 * g), a);
        *reinterpret_cast<bf16x4*>(sDW + (16 * R + ln) * LR + co) = to_bf16x4(a, -1.f);
    }
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const int u = t + 512 * e, r = u >> 4, c8 = 8 * (u & 15);
        *reinterpret_cast<bf16x8*>(sV + r * LR + c8) = vrow[e];
    }
    __syncthreads();

    // ---------------- phase 4c: dT (first term), dV, dKg ----------------------------
    f32x4 accT[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const TilePair tp = tile_pair(w + 8 * e);
        const int Rr = tp.R, Ri = tp.I;
        f32x4 a = zero4();
        if (Rr >= Ri) {
#pragma unroll
            for (int s = 0; s < 4; ++s)
                a = mma32(lds8(sDN + (16 * Rr + ln) * LR + 32 * s + 8 * g),
                          lds8(sV + (16 * Ri + ln) * LR + 32 * s + 8 * g), a);
        }
        accT[e] = a;
    }
    {
        bf16x8 dnop[2], dwop[2];   // dN and dW as A operands over the tokens: lane row = channel cl
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            dnop[s] = gather8(sDN + (32 * s + 8 * g) * LR + cl, LR);
            dwop[s] = gather8(sDW + (32 * s + 8 * g) * LR + cl, LR);
        }
#pragma unroll
        for (int R = 0; R < 4; ++R) {
            f32x4 av = zero4(), ag = zero4();
            // T[r][i] = 0 for r < i: key token block R needs rows r >= 16R
#pragma unroll
            for (int s = R / 2; s < 2; ++s) {
                const bf16x8 tb = tt_op(R, s);
                av = mma32(dnop[s], tb, av);
                ag = mma32(dwop[s], tb, ag);
            }
            const int r = 16 * R + ln;
            if (r < len) *reinterpret_cast<bf16x4*>(dv + r0 * D + r * HD + co) = to_bf16x4(av);
            const f32x4 B4 = lds4f(sBref + R * D + co);
#pragma unroll
            for (int i = 0; i < 4; ++i) a2[R][i] = fast_exp(B4[i]) * ag[i];
        }
    }
    __syncthreads();

    // ---------------- phase 4d: dT += dW (e^g K)^T ---------------------------------
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const int u = t + 512 * e, r = u >> 4, c8 = 8 * (u & 15);
        const bf16x8 kv = lds8(sK + r * LR + c8);
        bf16x8 o;
#pragma unroll
        for (int m = 0; m < 8; ++m) o[m] = (bf16)((float)kv[m] * fast_exp(sG[r * LG + c8 + m]));
        *reinterpret_cast<bf16x8*>(sKg + r * LR + c8) = o;
    }
    // q rows for the last phases, stored once dW's area is free
    bf16x8 qrow[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const int u = t + 512 * e, r = u >> 4, c8 = 8 * (u & 15);
        qrow[e] = bf16x8{};
        if (r < len) qrow[e] = *reinterpret_cast<const bf16x8*>(qB + r * HD + c8);
    }
    __syncthreads();
    // lane: dT[16Rr + 4g + i][16Ri + ln]; then dbeta's column term and dX^T
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const TilePair tp = tile_pair(w + 8 * e);
        const int Rr = tp.R, Ri = tp.I;
        f32x4 a = accT[e];
        if (Rr >= Ri) {
#pragma unroll
            for (int s = 0; s < 4; ++s)
                a = mma32(lds8(sDW + (16 * Rr + ln) * LR + 32 * s + 8 * g),
                          lds8(sKg + (16 * Ri + ln) * LR + 32 * s + 8 * g), a);
            float cs = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * Rr + 4 * g + i, col = 16 * Ri + ln;
                if (r < col) a[i] = 0.f;
                cs += a[i] * (float)sX[r * LT + col];
            }
            cs = group4_sum(cs);
            if (g == 0) sDBC[Rr * CHUNK + 16 * Ri + ln] = cs;
        }
        // dX = dT Diag(beta), stored transposed: dX^T[16Ri + ln][16Rr + 4g + i]
        *reinterpret_cast<bf16x4*>(sDXT + (16 * Ri + ln) * LT + 16 * Rr + 4 * g) =
            to_bf16x4(a, sBeta[16 * Ri + ln]);
    }
    __syncthreads();

    // ---------------- phase 5: P = X^T dX, dA = -strict(P X^T) -----------------------
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const int u = w + 8 * e, Ra = u >> 2, Rb = u & 3;
        f32x4 a = zero4();   // P^T tile: lane P[16Ra + ln][16Rb + 4g + i]
#pragma unroll
        for (int s = 0; s < 2; ++s)
            a = mma32(lds8(sDXT + (16 * Rb + ln) * LT + 32 * s + 8 * g),
                      lds8(sXT + (16 * Ra + ln) * LT + 32 * s + 8 * g), a);
        *reinterpret_cast<bf16x4*>(sP + (16 * Ra + ln) * LT + 16 * Rb + 4 * g) = to_bf16x4(a);
    }
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const int u = t + 512 * e, r = u >> 4, c8 = 8 * (u & 15);
        *reinterpret_cast<bf16x8*>(sQ + r * LR + c8) = qrow[e];
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const TilePair tp = tile_pair(w + 8 * e);
        const int Ra = tp.R, Rc = tp.I;
        f32x4 a = zero4();   // dA^T tile: lane dA[16Ra + ln][16Rc + 4g + i]
        if (Ra >= Rc) {
#pragma unroll
            for (int s = 0; s < 2; ++s)
                a = mma32(lds8(sX + (16 * Rc + ln) * LT + 32 * s + 8 * g),
                          lds8(sP + (16 * Ra + ln) * LT + 32 * s + 8 * g), a);
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = 16 * Ra + ln > 16 * Rc + 4 * g + i ? -a[i] : 0.f;
        }
        const int r = 16 * Ra + ln;
        *reinterpret_cast<bf16x4*>(sDA + r * LT + 16 * Rc + 4 * g) = to_bf16x4(a);
        const float br = sBeta[r];
#pragma unroll
        for (int i = 0; i < 4; ++i) sDLT[(16 * Rc + 4 * g + i) * LT + r] = (bf16)(br * a[i]);
    }
    __syncthreads();

    // ---------------- phase 6: the decayed products' gradients ------------------------
    // A operands over key tokens i = 32s + 8g + m for the lane's channel cl,
    // with the block reference of the lane's 16-token block (2s + g/2), kept
    // in fp32 and fed to the MFMA as a bf16 pair (high part, then the rounding
    // remainder).  The g-gradient of each decayed product enters dg twice
    // with opposite signs (at the row token and at the key token), and the
    // reverse cumulative sum keeps their difference only if both sides carry
    // the same values: one bf16 rounding of these operands leaves a residue of
    // the size of the pair terms, which under strong decay are large against
    // dlog_alpha itself.
    {
        float kb[2][8], qb[2][8], kr[2][8];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const float B = sBref[(2 * s + (g >> 1)) * D + cl];
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                const int i = 32 * s + 8 * g + m;
                const float gi = sG[i * LG + cl];
                const float kv = (float)sK[i * LR + cl];
                kb[s][m] = kv * cexp(B - gi);
                const float p = fast_exp(gi - B);
                kr[s][m] = kv * p;
                qb[s][m] = (float)sQ[i * LR + cl] * p;
            }
        }
        // f x (8 values) as the bf16 pair hi + lo
        auto split = [](const float (&x)[8], float f, bf16x8& hi, bf16x8& lo) {
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                const float y = x[m] * f;
                hi[m] = (bf16)y;
                lo[m] = (bf16)(y - (float)hi[m]);
            }
        };
        // the lane's key-token blocks (2s + g/2) as seen by its A-operand channel
        const float Bk0 = sBref[(g >> 1) * D + cl], Bk1 = sBref[(2 + (g >> 1)) * D + cl];
        // XQ, XL (row block R; key blocks I <= R) and Y (key block I; rows R >= I)
#pragma unroll
        for (int R = 0; R < 4; ++R) {
            f32x4 xq = zero4(), xl = zero4(), y = zero4();
            const float BR = sBref[R * D + cl];
#pragma unroll
            for (int s = 0; s <= R / 2; ++s) {
                const int I = 2 * s + (g >> 1);
                bf16x8 hi, lo;
                split(kb[s], I <= R ? fast_exp(BR - (s ? Bk1 : Bk0)) : 0.f, hi, lo);
                const bf16x8 aq = lds8(sDAq + (16 * R + ln) * LT + 32 * s + 8 * g);
                const bf16x8 al = lds8(sDA + (16 * R + ln) * LT + 32 * s + 8 * g);
                xq = mma32(hi, aq, xq);
                xq = mma32(lo, aq, xq);
                xl = mma32(hi, al, xl);
                xl = mma32(lo, al, xl);
            }
#pragma unroll
            for (int s = R / 2; s < 2; ++s) {
                const int Rk = 2 * s + (g >> 1);
                const float f = Rk >= R ? fast_exp((s ? Bk1 : Bk0) - BR) : 0.f;
                const bf16x8 at = lds8(sDAqT + (16 * R + ln) * LT + 32 * s + 8 * g);
                const bf16x8 lt = lds8(sDLT + (16 * R + ln) * LT + 32 * s + 8 * g);
                bf16x8 hi, lo;
                split(qb[s], f, hi, lo);
                y = mma32(hi, at, y);
                y = mma32(lo, at, y);
                split(kr[s], f, hi, lo);
                y = mma32(hi, lt, y);
                y = mma32(lo, lt, y);
            }
            // lane: token r = 16R + ln, channels co .. co + 3
            const int r = 16 * R + ln;
            const float br = sBeta[r];
            const f32x4 B4 = lds4f(sBref + R * D + co);
            const f32x4 g4 = lds4f(sG + r * LG + co);
            const bf16x4 k4 = *reinterpret_cast<const bf16x4*>(sK + r * LR + co);
            float db = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                a1[R][i] += xq[i];
                a2[R][i] += br * xl[i];
                a3[R][i] += y[i];
                db += (float)k4[i] * fast_exp(g4[i] - B4[i]) * xl[i];
            }
            db = group4_sum(db);
            if (g == 0) sDBR[w * CHUNK + r] = db;
        }
    }
    __syncthreads();

    // ---------------- phase 7: dq, dk, dg; dlog_alpha, dbeta -------------------------
#pragma unroll
    for (int R = 0; R < 4; ++R) {
        const int r = 16 * R + ln;
        const f32x4 B4 = lds4f(sBref + R * D + co);
        const f32x4 g4 = lds4f(sG + r * LG + co);
        const bf16x4 k4 = *reinterpret_cast<const bf16x4*>(sK + r * LR + co);
        const bf16x4 q4 = *reinterpret_cast<const bf16x4*>(sQ + r * LR + co);
        f32x4 dq4, dk4, dg4;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float P = fast_exp(g4[i] - B4[i]), Pi = cexp(B4[i] - g4[i]);
            const float kP = P * a2[R][i], kI = Pi * a3[R][i];
            dq4[i] = P * a1[R][i];
            dk4[i] = kP + kI;
            dg4[i] = r < len ? (float)q4[i] * dq4[i] + (float)k4[i] * (kP - kI) : 0.f;
        }
        if (r < len) {
            *reinterpret_cast<bf16x4*>(dq + r0 * D + r * HD + co) = to_bf16x4(dq4);
            *reinterpret_cast<bf16x4*>(dk + r0 * D + r * HD + co) = to_bf16x4(dk4);
        }
        *reinterpret_cast<f32x4*>(sScan + r * LG + co) = dg4;
    }
    __syncthreads();
    // reverse cumulative sum down each column (thread: column sc, rows 16 sq ..)
    {
        float suf[16], run = 0.f;
#pragma unroll
        for (int u = 15; u >= 0; --u) {
            run += sScan[(16 * sq + u) * LG + sc];
            suf[u] = run;
        }
        sTot[sq * D + sc] = run;
        __syncthreads();
        float later = fast_exp(sBref[4 * D + sc]) * sExt[sc] + sExt[D + sc];
        for (int qd = sq + 1; qd < 4; ++qd) later += sTot[qd * D + sc];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int r = 16 * sq + u;
            if (r < len) dla[r0 * D + r * HD + sc] = suf[u] + later;
        }
    }
    if (t < len) {
        float b = 0.f;
        for (int R = t >> 4; R < 4; ++R) b += sDBC[R * CHUNK + t];
#pragma unroll
        for (int x = 0; x < CG_WAVES; ++x) b += sDBR[x * CHUNK + t];
        dbeta[r0 + (size_t)t * H] = b;
    }
}

hipError_t launch_chunk_grad(const void* q, const void* k, const void* v, const float* la,
                             const float* beta, const void* d_o, ChunkSrc src, int max_chunks,
                             int H, int dk, int dv, const void* rec, const float* chunk_states,
                             const void* dS_chunks, void* dq, void* dk_out, void* dv_out,
                             float* dla, float* dbeta, hipStream_t stream)
{
    if (dk != 128 || dv != 128) return hipErrorInvalidValue;
    if (max_chunks <= 0) return hipSuccess;
    hipLaunchKernelGGL(chunk_grad_kernel, dim3((unsigned)max_chunks * H), dim3(64 * CG_WAVES), 0,
                       stream, (const bf16*)q, (const bf16*)k, (const bf16*)v, la, beta,
                       (const bf16*)d_o, src, H, (const unsigned char*)rec, chunk_states,
                       (const bf16*)dS_chunks, (bf16*)dq, (bf16*)dk_out, (bf16*)dv_out, dla, dbeta);
    return hipGetLastError();
}

}  // namespace kda
