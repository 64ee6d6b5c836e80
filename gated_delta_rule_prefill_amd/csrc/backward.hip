// backward.hip -- gradients of the KDA recurrence (reverse mode).
//
// One token of the recurrence (Kimi Linear paper notes, section 2), written
// in delta form:
//   X = Diag(a) S,   y = X^T k,   nu = beta (v - y),   S' = X + k nu^T,
//   o = S'^T q,      a = exp(log_alpha).
// Walking the tokens backwards with G = dL/dS' (plus q do^T from the
// read-out), the chain rule gives
//   dq = S' do,  dnu = G^T k,  dv = beta dnu,  dy = -beta dnu,
//   dbeta = dnu . (v - y),  dk = G nu + X dy,  G += k dy^T,
//   dlog_alpha_c = sum_j G[c,j] X[c,j],  dS = Diag(a) G.
//
// The state entering every 64-token chunk comes from the forward pass (the
// chunk states of the chunkwise prefill).  Inside a chunk the states are
// recomputed: a first forward sweep saves the state at every 8th token (to a
// per-workgroup scratch area, each lane its own values), then each 8-token
// piece, last first, is swept forward again keeping every state in
// registers, and walked backwards.  Only the 8-token loops are unrolled, so
// the code stays small.
//
// One workgroup of 4 waves per (sequence, head, 16 value columns): the
// columns of S and G evolve independently, so a head splits into DV/16
// chains.  Wave w owns 4 of the 16 columns for every key row (lane l: rows
// RPL*l .. RPL*l + RPL - 1, RPL = DK/64), so the products over key rows
// (y, dnu) are reduced inside the wave, with no barrier per token.  The sums
// over value columns (dq, dk, dlog_alpha, dbeta) are combined over the 4
// waves through LDS once per 8-token piece, giving one partial per
// workgroup; a second kernel sums the DV/16 partials in a fixed order, so
// the result is deterministic.
#include "kda_common.h"

namespace kda {

constexpr int BWD_COLS = 16;   // value columns per workgroup
constexpr int BWD_CW = 4;      // value columns per wave
constexpr int BWD_PIECE = 8;   // tokens per recomputed piece
constexpr int BWD_PIECES = CHUNK / BWD_PIECE;

// Totals over the 64 lanes of 4 values per lane (a transposing butterfly:
// the two permlane folds also halve the values, then a DPP row sum),
// returned uniform.
__device__ __forceinline__ void wave_sum4(const float (&a)[4], int lane, float (&t)[4]) {
    const float c = row16_sum(fold16(fold32(a[0], a[2]), fold32(a[1], a[3])));
    // lane 16 i now holds the total of value i
#pragma unroll
    for (int i = 0; i < 4; ++i) t[i] = read_lane(c, 16 * i);
}

// The LDS it stages holds the CU to one workgroup, one wave per SIMD: the
// compiler may spend registers on hiding latency.
template <typename E, int DK, int DV>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void backward_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
    const float* __restrict__ log_alpha, const float* __restrict__ beta,
    const ChunkSrc src, const float* __restrict__ chunk_states, const E* __restrict__ d_o,
    const float* __restrict__ d_final, int H, int T,
    E* __restrict__ dv_out, float* __restrict__ part, float* __restrict__ part_beta,
    float* __restrict__ d_initial, float* __restrict__ scratch)
{
    constexpr int RPL = DK / 64, NSL = DV / BWD_COLS, CW = BWD_CW;
    constexpr int NV = RPL * CW;   // state values per lane
    // Staged token i sits in row i + 1: rows 0 and CHUNK + 1 are never
    // written, so the look-ahead reads of tokens -1 and CHUNK (whose values
    // go unused) need no clamping.
    __shared__ __attribute__((aligned(16))) float sQ[CHUNK + 2][DK], sK[CHUNK + 2][DK], sA[CHUNK + 2][DK];
    __shared__ __attribute__((aligned(16))) float sV[CHUNK + 2][BWD_COLS], sDO[CHUNK + 2][BWD_COLS];
    __shared__ float sB[CHUNK + 2];
    __shared__ float comb[BWD_PIECE][4][3][DK];   // per-wave row sums of a piece: dq, dk, dlog_alpha
    __shared__ float combB[BWD_PIECE][4];

    const int slice = blockIdx.x % NSL;
    const int pair = blockIdx.x / NSL;   // sequence * H + head
    const int s = pair / H, h = pair % H;
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int r0 = RPL * lane;                 // first key row of this lane
    const int cw0 = wave * CW;                 // first column of this wave inside the slice
    const int j0 = slice * BWD_COLS + cw0;     // first value column of this wave
    int c_begin, n;
    seq_chunks(src, s, c_begin, n);

    // this workgroup's scratch: [piece][value][thread] (each thread its own values)
    float* const scr = scratch + (size_t)blockIdx.x * BWD_PIECES * NV * 256;
    float G[RPL][CW];
#pragma unroll
    for (int rr = 0; rr < RPL; ++rr)
#pragma unroll
        for (int e = 0; e < CW; ++e)
            G[rr][e] = d_final ? d_final[((size_t)pair * DK + r0 + rr) * DV + j0 + e] : 0.f;

    // A staged token's values as one lane uses them, read from LDS a token
    // ahead of their use so that the read is off the chain's critical path
    // (i from -1 to CHUNK).
    struct Tok {
        float a[RPL], k[RPL], q[RPL], v[CW], dov[CW], b;
    };
    auto tok = [&](int i, bool with_q) {
        ++i;
        Tok t;
#pragma unroll
        for (int rr = 0; rr < RPL; ++rr) {
            t.a[rr] = sA[i][r0 + rr];
            t.k[rr] = sK[i][r0 + rr];
            t.q[rr] = with_q ? sQ[i][r0 + rr] : 0.f;
        }
#pragma unroll
        for (int e = 0; e < CW; ++e) {
            t.v[e] = sV[i][cw0 + e];
            t.dov[e] = with_q ? sDO[i][cw0 + e] : 0.f;
        }
        t.b = sB[i];
        return t;
    };
    // one forward token on S; y and nu (uniform) returned
    auto fwd = [&](float (&S)[RPL][CW], const Tok& t, float (&y)[CW], float (&nu)[CW]) {
        float pp[CW];
#pragma unroll
        for (int e = 0; e < CW; ++e) pp[e] = 0.f;
#pragma unroll
        for (int rr = 0; rr < RPL; ++rr) {
#pragma unroll
            for (int e = 0; e < CW; ++e) {
                S[rr][e] *= t.a[rr];
                pp[e] += t.k[rr] * S[rr][e];
            }
        }
        wave_sum4(pp, lane, y);
#pragma unroll
        for (int e = 0; e < CW; ++e) nu[e] = t.b * (t.v[e] - y[e]);
#pragma unroll
        for (int rr = 0; rr < RPL; ++rr) {
#pragma unroll
            for (int e = 0; e < CW; ++e) S[rr][e] += t.k[rr] * nu[e];
        }
    };

    for (int c = n - 1; c >= 0; --c) {
        const ChunkInfo ci = chunk_desc(src, c_begin + c);
        const int L = ci.len;
        // the state entering the chunk (its columns of this lane), loaded with the inputs
        float Sc[RPL][CW];
        // ---- stage the chunk's inputs (fp32) ----
        // Every thread issues all of its loads (4 elements each) before
        // waiting on any, and before the barrier that frees the previous
        // chunk's staged values.  Rows past the chunk's end are staged as a
        // neutral token (alpha = 1, beta = 0, q = k = v = dO = 0), which
        // leaves S and G unchanged, so every piece runs all of its tokens.
        {
            using V4 = typename Vec<E>::v4;
            constexpr int NL = CHUNK * DK / 4 / 256;   // loads per thread per array
            static_assert(CHUNK * BWD_COLS == 4 * 256, "one load of v and dO per thread");
            V4 lq[NL], lk[NL];
            f32x4 la[NL];
#pragma unroll
            for (int m = 0; m < NL; ++m) {
                const int x = 4 * (m * 256 + tid), i = x / DK, r = x % DK;
                const size_t at = ((size_t)(ci.start + min(i, L - 1)) * H + h) * DK + r;
                lq[m] = load_vec<V4>(q + at);
                lk[m] = load_vec<V4>(k + at);
                la[m] = *reinterpret_cast<const f32x4*>(log_alpha + at);
            }
            const int iv = tid / 4, jv = 4 * (tid % 4);
            const size_t atv = ((size_t)(ci.start + min(iv, L - 1)) * H + h) * DV + slice * BWD_COLS + jv;
            const V4 lv = load_vec<V4>(v + atv), ld = load_vec<V4>(d_o + atv);
            const float lb = tid < CHUNK ? beta[(size_t)(ci.start + min(tid, L - 1)) * H + h] : 0.f;
            const float* cs = chunk_states + (chunk_state_row(src, s, c_begin, c) * H + h) * DK * DV + (size_t)r0 * DV + j0;
#pragma unroll
            for (int rr = 0; rr < RPL; ++rr)
#pragma unroll
                for (int e = 0; e < CW; ++e) Sc[rr][e] = cs[(size_t)rr * DV + e];
            __syncthreads();   // the previous chunk's staged values are no longer read
#pragma unroll
            for (int m = 0; m < NL; ++m) {
                const int x = 4 * (m * 256 + tid), i = x / DK, r = x % DK;
                const bool pad = i >= L;
                f32x4 fq, fk, fa;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    fq[e] = pad ? 0.f : to_f32(lq[m][e]);
                    fk[e] = pad ? 0.f : to_f32(lk[m][e]);
                    fa[e] = pad ? 1.f : __expf(la[m][e]);
                }
                *reinterpret_cast<f32x4*>(&sQ[i + 1][r]) = fq;
                *reinterpret_cast<f32x4*>(&sK[i + 1][r]) = fk;
                *reinterpret_cast<f32x4*>(&sA[i + 1][r]) = fa;
            }
            f32x4 fv, fd;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                fv[e] = iv < L ? to_f32(lv[e]) : 0.f;
                fd[e] = iv < L ? to_f32(ld[e]) : 0.f;
            }
            *reinterpret_cast<f32x4*>(&sV[iv + 1][jv]) = fv;
            *reinterpret_cast<f32x4*>(&sDO[iv + 1][jv]) = fd;
            if (tid < CHUNK) sB[tid + 1] = tid < L ? lb : 0.f;
        }
        __syncthreads();

        // ---- first sweep: the state entering every piece, to scratch ----
        const int npieces = (L + BWD_PIECE - 1) / BWD_PIECE;
        // The last piece's entry state stays in registers; the others go to
        // scratch and come back a piece ahead of their use.
        float Sn[RPL][CW];   // the state entering the piece walked next
        {
            float S[RPL][CW];
#pragma unroll
            for (int rr = 0; rr < RPL; ++rr)
#pragma unroll
                for (int e = 0; e < CW; ++e) S[rr][e] = Sc[rr][e];
            Tok t = tok(0, false);
            for (int p = 0; p + 1 < npieces; ++p) {
#pragma unroll
                for (int rr = 0; rr < RPL; ++rr)
#pragma unroll
                    for (int e = 0; e < CW; ++e) scr[(p * NV + rr * CW + e) * 256 + tid] = S[rr][e];
#pragma unroll
                for (int i = 0; i < BWD_PIECE; ++i) {
                    const Tok nx = tok(BWD_PIECE * p + i + 1, false);
                    float y[CW], nu[CW];
                    fwd(S, t, y, nu);
                    t = nx;
                }
            }
#pragma unroll
            for (int rr = 0; rr < RPL; ++rr)
#pragma unroll
                for (int e = 0; e < CW; ++e) Sn[rr][e] = S[rr][e];
        }
        // ---- pieces, last first: sweep forward keeping states, then backwards ----
        for (int p = npieces - 1; p >= 0; --p) {
            const int i0 = BWD_PIECE * p;
            const int np = min(BWD_PIECE, L - i0);
            float Sp[BWD_PIECE][RPL][CW];   // state before each token of the piece
            float yP[BWD_PIECE][CW], nuP[BWD_PIECE][CW];
            {
                float S[RPL][CW];
                const int pn = max(p - 1, 0);   // the next piece (p = 0: a load left unused)
#pragma unroll
                for (int rr = 0; rr < RPL; ++rr)
#pragma unroll
                    for (int e = 0; e < CW; ++e) {
                        S[rr][e] = Sn[rr][e];
                        Sn[rr][e] = scr[(pn * NV + rr * CW + e) * 256 + tid];
                    }
                Tok t = tok(i0, false);
#pragma unroll
                for (int i = 0; i < BWD_PIECE; ++i) {
                    const Tok nx = tok(i0 + i + 1, false);
#pragma unroll
                    for (int rr = 0; rr < RPL; ++rr)
#pragma unroll
                        for (int e = 0; e < CW; ++e) Sp[i][rr][e] = S[rr][e];
                    fwd(S, t, yP[i], nuP[i]);
                    t = nx;
                }
            }
            Tok tr = tok(i0 + BWD_PIECE - 1, true);
            // dv rows of the piece; every lane stores its column's value
            // (lanes 4 and up repeat lanes 0-3), so no lane mask is needed
            E* const dvp = dv_out + ((size_t)(ci.start + i0) * H + h) * DV + j0 + (lane & (CW - 1));
#pragma unroll
            for (int i = BWD_PIECE - 1; i >= 0; --i) {
                const int ti = i0 + i;
                const Tok t = tr;
                tr = tok(ti - 1, true);
                const float b = t.b;
                // dq = S' dO with S' = X + k nu^T: X dO + k (nu . dO)
                float dov[CW], vr[CW], bvr[CW], ndo = 0.f;
#pragma unroll
                for (int e = 0; e < CW; ++e) {
                    dov[e] = t.dov[e];
                    vr[e] = t.v[e] - yP[i][e];   // v - y
                    bvr[e] = b * vr[e];
                    ndo += nuP[i][e] * dov[e];
                }
                float X[RPL][CW], dq[RPL], gkp[CW];
#pragma unroll
                for (int e = 0; e < CW; ++e) gkp[e] = 0.f;
#pragma unroll
                for (int rr = 0; rr < RPL; ++rr) {
                    const float a = t.a[rr], kc = t.k[rr], qc = t.q[rr];
                    dq[rr] = kc * ndo;
#pragma unroll
                    for (int e = 0; e < CW; ++e) {
                        X[rr][e] = a * Sp[i][rr][e];
                        dq[rr] += X[rr][e] * dov[e];
                        G[rr][e] += qc * dov[e];
                        gkp[e] += G[rr][e] * kc;
                    }
                }
                float gk[CW], dy[CW];
                wave_sum4(gkp, lane, gk);
                float db = 0.f;
#pragma unroll
                for (int e = 0; e < CW; ++e) {
                    dy[e] = -b * gk[e];
                    db += gk[e] * vr[e];
                }
#pragma unroll
                for (int rr = 0; rr < RPL; ++rr) {
                    const float a = t.a[rr], kc = t.k[rr];
                    float dk = 0.f, dl = 0.f;
#pragma unroll
                    for (int e = 0; e < CW; ++e) {
                        dk += G[rr][e] * bvr[e] + X[rr][e] * dy[e];
                        G[rr][e] += kc * dy[e];
                        dl += G[rr][e] * X[rr][e];
                        G[rr][e] *= a;
                    }
                    comb[i][wave][0][r0 + rr] = dq[rr];
                    comb[i][wave][1][r0 + rr] = dk;
                    comb[i][wave][2][r0 + rr] = dl;
                }
                if (lane == 0) combB[i][wave] = db;
                if (i < np) {
                    // dv = beta dnu = -dy
                    float dve = -dy[0];
#pragma unroll
                    for (int e = 1; e < CW; ++e) dve = (lane & (CW - 1)) == e ? -dy[e] : dve;
                    dvp[(size_t)i * H * DV] = from_f32<E>(dve);
                }
            }
            __syncthreads();   // the piece's per-wave row sums are in LDS
            for (int x = tid; x < np * DK; x += 256) {
                const int i = x / DK, r = x % DK;
                const size_t t = (size_t)ci.start + i0 + i;
                float* pr = part + (((size_t)slice * T + t) * H + h) * DK + r;
                const size_t plane = (size_t)NSL * T * H * DK;
#pragma unroll
                for (int m = 0; m < 3; ++m)
                    pr[m * plane] = comb[i][0][m][r] + comb[i][1][m][r] + comb[i][2][m][r] + comb[i][3][m][r];
            }
            if (tid < np)
                part_beta[((size_t)slice * T + ci.start + i0 + tid) * H + h] =
                    combB[tid][0] + combB[tid][1] + combB[tid][2] + combB[tid][3];
            __syncthreads();   // comb is rewritten by the next piece
        }
    }
    if (d_initial) {
#pragma unroll
        for (int rr = 0; rr < RPL; ++rr)
#pragma unroll
            for (int e = 0; e < CW; ++e) d_initial[((size_t)pair * DK + r0 + rr) * DV + j0 + e] = G[rr][e];
    }
}

// Sums of the per-slice partials (fixed order): dq, dk in the q/k/v dtype,
// dlog_alpha and dbeta in fp32.
template <typename E, int DK, int NSL>
__global__ __launch_bounds__(256) void backward_reduce_kernel(
    const float* __restrict__ part, const float* __restrict__ part_beta, long long rows, int TH,
    E* __restrict__ dq, E* __restrict__ dk, float* __restrict__ dla, float* __restrict__ dbeta)
{
    const long long x = (long long)blockIdx.x * 256 + threadIdx.x;
    const long long plane = (long long)NSL * rows;
    if (x < rows) {
        float a = 0.f, b = 0.f, c = 0.f;
#pragma unroll
        for (int sl = 0; sl < NSL; ++sl) {
            a += part[sl * rows + x];
            b += part[plane + sl * rows + x];
            c += part[2 * plane + sl * rows + x];
        }
        dq[x] = from_f32<E>(a);
        dk[x] = from_f32<E>(b);
        dla[x] = c;
    }
    if (x < TH) {
        float d = 0.f;
#pragma unroll
        for (int sl = 0; sl < NSL; ++sl) d += part_beta[sl * (long long)TH + x];
        dbeta[x] = d;
    }
}

// Workspace of the backward kernels: per-slice partials of dq, dk,
// dlog_alpha ([3][DV/16][T][H][DK]) and dbeta ([DV/16][T][H]), then the
// per-workgroup scratch (DK x 16 fp32 per piece of a chunk).
size_t backward_partial_bytes(int64_t T, int H, int dk, int dv) {
    const size_t nsl = (size_t)dv / BWD_COLS;
    return (3 * nsl * (size_t)T * H * dk + nsl * (size_t)T * H) * sizeof(float);
}
size_t backward_scratch_bytes(int N, int H, int dk, int dv) {
    return (size_t)N * H * (dv / BWD_COLS) * BWD_PIECES * dk * BWD_COLS * sizeof(float);
}

template <typename E, int DK, int DV>
static hipError_t launch_bwd_t(const void* q, const void* k, const void* v, const float* la,
                               const float* beta, ChunkSrc src, const float* chunk_states,
                               const void* d_o, const float* d_final, int H, int64_t T, void* dq,
                               void* dk, void* dv, float* dla, float* dbeta, float* d_initial,
                               float* part, float* scratch, hipStream_t stream)
{
    constexpr int NSL = DV / BWD_COLS;
    float* part_beta = part + (size_t)3 * NSL * T * H * DK;
    const long long units = (long long)src.N * H * NSL;
    if (units > 0) {
        hipLaunchKernelGGL((backward_kernel<E, DK, DV>), dim3((unsigned)units), dim3(256), 0, stream,
                           (const E*)q, (const E*)k, (const E*)v, la, beta, src, chunk_states,
                           (const E*)d_o, d_final, H, (int)T, (E*)dv, part, part_beta, d_initial,
                           scratch);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const long long rows = T * H * DK;
    if (rows > 0) {
        hipLaunchKernelGGL((backward_reduce_kernel<E, DK, NSL>), dim3((unsigned)((rows + 255) / 256)),
                           dim3(256), 0, stream, part, part_beta, rows, (int)(T * H), (E*)dq, (E*)dk,
                           dla, dbeta);
        return hipGetLastError();
    }
    return hipSuccess;
}

hipError_t launch_backward(const void* q, const void* k, const void* v, const float* la,
                           const float* beta, ChunkSrc src, const float* chunk_states,
                           const void* d_o, const float* d_final, int H, int64_t T, int dk, int dv,
                           bool bf16_io, void* dq, void* dk_out, void* dv_out, float* dla,
                           float* dbeta, float* d_initial, float* part, float* scratch,
                           hipStream_t stream)
{
#define KDA_BWD_CASE(E, DK_, DV_)                                                                 \
    if (dk == DK_ && dv == DV_)                                                                  \
        return launch_bwd_t<E, DK_, DV_>(q, k, v, la, beta, src, chunk_states, d_o, d_final, H, T, \
                                         dq, dk_out, dv_out, dla, dbeta, d_initial, part, scratch, \
                                         stream);
    if (bf16_io) {
        KDA_BWD_CASE(bf16, 128, 128)
        KDA_BWD_CASE(bf16, 64, 64)
        KDA_BWD_CASE(bf16, 128, 64)
        KDA_BWD_CASE(bf16, 64, 128)
    } else {
        KDA_BWD_CASE(float, 128, 128)
        KDA_BWD_CASE(float, 64, 64)
        KDA_BWD_CASE(float, 128, 64)
        KDA_BWD_CASE(float, 64, 128)
    }
#undef KDA_BWD_CASE
    return hipErrorInvalidValue;
}

}  // namespace kda
