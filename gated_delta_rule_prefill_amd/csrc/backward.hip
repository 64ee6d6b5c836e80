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
// chains.  Wave w owns key rows RW*w .. RW*w + RW - 1 (RW = DK/4); lane l
// holds row RW*w + l % RW and CPL = RW/4 consecutive columns of group
// l / RW.  The products over key rows (y, dnu) are reduced across the
// workgroup every token; the sums over value columns (dq, dk, dlog_alpha,
// dbeta) are partial per workgroup and summed over the column slices by a
// second kernel in a fixed order, so the result is deterministic.
#include "kda_common.h"

namespace kda {

constexpr int BWD_COLS = 16;   // value columns per workgroup
constexpr int BWD_PIECE = 8;   // tokens per recomputed piece
constexpr int BWD_PIECES = CHUNK / BWD_PIECE;

template <int DK>
struct BwdCfg {
    static constexpr int RW = DK / 4;          // key rows per wave
    static constexpr int GROUPS = 64 / RW;     // column groups per wave
    static constexpr int CPL = BWD_COLS / GROUPS;   // columns per lane
    static_assert(CPL * GROUPS == BWD_COLS && CPL == RW / 4, "lane split");
};

// In-wave sum over the RW lanes of a column group (lane bits below log2(RW))
// of CPL values at once: lane l ends with the total of value (l >> 2) % CPL.
template <int RW, int CPL>
__device__ __forceinline__ float group_col_sum(const float (&a)[CPL], int lane) {
    float cur[CPL];
#pragma unroll
    for (int e = 0; e < CPL; ++e) cur[e] = a[e];
    int n = CPL;
#pragma unroll
    for (int m = RW / 2; m >= 1; m >>= 1) {
        if (n > 1) {
            const bool hi = lane & m;
#pragma unroll
            for (int j = 0; j < CPL / 2; ++j)
                if (j < n / 2)
                    cur[j] = (hi ? cur[n / 2 + j] : cur[j]) + __shfl_xor(hi ? cur[j] : cur[n / 2 + j], m);
            n >>= 1;
        } else {
            cur[0] += __shfl_xor(cur[0], m);
        }
    }
    return cur[0];
}

// Sum over the column groups of one row (lanes l, l + RW, ...): every lane of
// the row gets the total.
template <int RW>
__device__ __forceinline__ float row_sum(float x) {
#pragma unroll
    for (int m = RW; m < 64; m <<= 1) x += __shfl_xor(x, m);
    return x;
}

template <typename E, int DK, int DV>
__global__ __launch_bounds__(256) void backward_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
    const float* __restrict__ log_alpha, const float* __restrict__ beta,
    const ChunkSrc src, const float* __restrict__ chunk_states, const E* __restrict__ d_o,
    const float* __restrict__ d_final, int H, int T,
    E* __restrict__ dv_out, float* __restrict__ part, float* __restrict__ part_beta,
    float* __restrict__ d_initial, float* __restrict__ scratch)
{
    using C = BwdCfg<DK>;
    constexpr int RW = C::RW, CPL = C::CPL, NSL = DV / BWD_COLS;
    __shared__ float sQ[CHUNK][DK], sK[CHUNK][DK], sA[CHUNK][DK];
    __shared__ __attribute__((aligned(16))) float sV[CHUNK][BWD_COLS], sDO[CHUNK][BWD_COLS];
    __shared__ float sB[CHUNK];
    __shared__ float sNu[BWD_PIECE][BWD_COLS], sY[BWD_PIECE][BWD_COLS];
    __shared__ float red[2][4][BWD_COLS];

    const int slice = blockIdx.x % NSL;
    const int pair = blockIdx.x / NSL;   // sequence * H + head
    const int s = pair / H, h = pair % H;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int row = RW * wave + (lane % RW);
    const int cg = lane / RW;
    const int col0 = cg * CPL;              // first column of this lane inside the slice
    const int j0 = slice * BWD_COLS;        // first value column of the slice
    const int idx = (lane >> 2) % CPL;      // column this lane's group sums end on
    int c_begin, n;
    seq_chunks(src, s, c_begin, n);

    // this workgroup's scratch: [piece][value][thread] (each thread its own values)
    float* const scr = scratch + (size_t)blockIdx.x * BWD_PIECES * CPL * 256;
    float G[CPL];
#pragma unroll
    for (int e = 0; e < CPL; ++e)
        G[e] = d_final ? d_final[((size_t)pair * DK + row) * DV + j0 + col0 + e] : 0.f;

    int rb = 0;   // reduction buffer toggle: a buffer is rewritten two reductions later
    // sum over all key rows of CPL per-lane values; returns the lane's CPL column totals
    auto col_reduce = [&](const float (&a)[CPL], float (&out)[CPL]) {
        const float t = group_col_sum<RW, CPL>(a, lane);
        if ((lane & 3) == 0) red[rb][wave][col0 + idx] = t;
        __syncthreads();
#pragma unroll
        for (int e = 0; e < CPL; ++e)
            out[e] = red[rb][0][col0 + e] + red[rb][1][col0 + e] + red[rb][2][col0 + e] + red[rb][3][col0 + e];
        rb ^= 1;
    };
    // one forward token (index i of the staged chunk) on S; y and nu returned
    auto fwd = [&](float (&S)[CPL], int i, float (&y)[CPL], float (&nu)[CPL]) {
        const float a = sA[i][row], kc = sK[i][row];
        float pp[CPL];
#pragma unroll
        for (int e = 0; e < CPL; ++e) {
            S[e] *= a;
            pp[e] = kc * S[e];
        }
        col_reduce(pp, y);
        const float b = sB[i];
#pragma unroll
        for (int e = 0; e < CPL; ++e) {
            nu[e] = b * (sV[i][col0 + e] - y[e]);
            S[e] += kc * nu[e];
        }
    };

    for (int c = n - 1; c >= 0; --c) {
        const ChunkInfo ci = chunk_desc(src, c_begin + c);
        const int L = ci.len;
        // ---- stage the chunk's inputs (fp32) ----
        __syncthreads();   // the previous chunk's staged values are no longer read
        for (int x = tid; x < CHUNK * DK; x += 256) {
            const int i = x / DK, r = x % DK;
            const size_t at = ((size_t)(ci.start + min(i, L - 1)) * H + h) * DK + r;
            sQ[i][r] = to_f32(q[at]);
            sK[i][r] = to_f32(k[at]);
            sA[i][r] = __expf(log_alpha[at]);
        }
        for (int x = tid; x < CHUNK * BWD_COLS; x += 256) {
            const int i = x / BWD_COLS, j = x % BWD_COLS;
            const size_t at = ((size_t)(ci.start + min(i, L - 1)) * H + h) * DV + j0 + j;
            sV[i][j] = to_f32(v[at]);
            sDO[i][j] = to_f32(d_o[at]);
        }
        if (tid < CHUNK) sB[tid] = beta[(size_t)(ci.start + min(tid, L - 1)) * H + h];
        __syncthreads();

        // ---- first sweep: the state entering every piece, to scratch ----
        const int npieces = (L + BWD_PIECE - 1) / BWD_PIECE;
        {
            float S[CPL];
            const float* cs = chunk_states + ((size_t)(c_begin + c) * H + h) * DK * DV + (size_t)row * DV + j0 + col0;
#pragma unroll
            for (int e = 0; e < CPL; ++e) S[e] = cs[e];
            for (int p = 0; p < npieces; ++p) {
#pragma unroll
                for (int e = 0; e < CPL; ++e) scr[(p * CPL + e) * 256 + tid] = S[e];
                if (p + 1 < npieces) {   // the last piece's successors are not needed
#pragma unroll
                    for (int i = 0; i < BWD_PIECE; ++i) {
                        float y[CPL], nu[CPL];
                        fwd(S, BWD_PIECE * p + i, y, nu);
                    }
                }
            }
        }
        // ---- pieces, last first: sweep forward keeping states, then backwards ----
        for (int p = npieces - 1; p >= 0; --p) {
            const int i0 = BWD_PIECE * p;
            const int np = min(BWD_PIECE, L - i0);
            float Sp[BWD_PIECE][CPL];   // state before each token of the piece
            {
                float S[CPL];
#pragma unroll
                for (int e = 0; e < CPL; ++e) S[e] = scr[(p * CPL + e) * 256 + tid];
#pragma unroll
                for (int i = 0; i < BWD_PIECE; ++i) {
                    if (i < np) {
#pragma unroll
                        for (int e = 0; e < CPL; ++e) Sp[i][e] = S[e];
                        float y[CPL], nu[CPL];
                        fwd(S, i0 + i, y, nu);
                        if ((lane % RW) == 0 && wave == 0) {
#pragma unroll
                            for (int e = 0; e < CPL; ++e) {
                                sNu[i][col0 + e] = nu[e];
                                sY[i][col0 + e] = y[e];
                            }
                        }
                    }
                }
            }
            __syncthreads();   // sNu / sY of the piece visible
#pragma unroll
            for (int i = BWD_PIECE - 1; i >= 0; --i) {
                if (i >= np) continue;
                const int ti = i0 + i;
                const size_t t = (size_t)ci.start + ti;
                const float a = sA[ti][row], kc = sK[ti][row], qc = sQ[ti][row], b = sB[ti];
                float X[CPL], dq = 0.f;
#pragma unroll
                for (int e = 0; e < CPL; ++e) {
                    X[e] = a * Sp[i][e];
                    const float snew = X[e] + kc * sNu[i][col0 + e];
                    const float d = sDO[ti][col0 + e];
                    dq += snew * d;
                    G[e] += qc * d;
                }
                float gkp[CPL], gk[CPL];
#pragma unroll
                for (int e = 0; e < CPL; ++e) gkp[e] = G[e] * kc;
                col_reduce(gkp, gk);
                float dbp = 0.f, dkp = 0.f, dlp = 0.f;
                float dy[CPL];
#pragma unroll
                for (int e = 0; e < CPL; ++e) {
                    const float r = sV[ti][col0 + e] - sY[i][col0 + e];
                    dy[e] = -b * gk[e];
                    dbp += gk[e] * r;
                    dkp += b * G[e] * r + X[e] * dy[e];
                    G[e] += kc * dy[e];
                    dlp += G[e] * X[e];
                    G[e] *= a;
                }
                dq = row_sum<RW>(dq);
                dkp = row_sum<RW>(dkp);
                dlp = row_sum<RW>(dlp);
                dbp = row_sum<RW>(dbp);   // every row holds the slice's dbeta partial
                float* pr = part + (((size_t)slice * T + t) * H + h) * DK;
                const size_t plane = (size_t)NSL * T * H * DK;
                if (cg == 0) {
                    pr[row] = dq;
                    pr[plane + row] = dkp;
                    pr[2 * plane + row] = dlp;
                }
                if (wave == 0 && lane == 0) part_beta[((size_t)slice * T + t) * H + h] = dbp;
                if (wave == 0 && (lane % RW) == 0) {
#pragma unroll
                    for (int e = 0; e < CPL; ++e)
                        dv_out[(t * H + h) * DV + j0 + col0 + e] = from_f32<E>(-dy[e]);
                }
            }
            __syncthreads();   // sNu / sY rewritten by the next piece
        }
    }
    if (d_initial) {
#pragma unroll
        for (int e = 0; e < CPL; ++e) d_initial[((size_t)pair * DK + row) * DV + j0 + col0 + e] = G[e];
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
