// recurrent.hip -- fused recurrent path for a few tokens per sequence, on a
// pool of states addressed through a slot per sequence.
//
// The token-by-token form of the recurrence (Kimi Linear paper notes,
// section 2; the recurrent mode that the FLA implementation switches to for
// short inputs, section 3):
//
//   S' = Diag(alpha_t) S,  p = S'^T k_t,  nu = beta_t (v_t - p)
//   S  = S' + k_t nu^T,    o_t = S^T q_t = S'^T q_t + (q_t . k_t) nu
//
// One workgroup per (sequence, head, CB value columns) keeps its dk x CB
// slice of the fp32 state in registers across all of the sequence's tokens:
// the state is read from its slot once and written back once, however many
// tokens the sequence has.  Tokens are staged through LDS 16 at a time (q, k,
// alpha and the value slice, already widened to fp32), so each staged token
// costs one barrier.  A sequence whose slot lies outside the pool is padding:
// its output rows are zeroed and no state is touched.
#include "kda_common.h"

namespace kda {

constexpr int REC_COLS = 64;   // value columns per workgroup (as the decode step)
constexpr int REC_TB = 16;     // tokens staged per LDS fill

template <typename E, int DK, int DV, int CB, bool NORM>
__global__ __launch_bounds__(256) void recurrent_kernel(
    float* __restrict__ pool, int num_slots, const int32_t* __restrict__ slots,
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
    const float* __restrict__ log_alpha, const float* __restrict__ beta,
    const int32_t* __restrict__ cu, int rows, int H, int beta_logit, E* __restrict__ o)
{
    constexpr int NQ = CB / 4;       // column quads of the slice
    constexpr int RG = 256 / NQ;     // row groups
    constexpr int RPT = DK / RG;     // state rows per thread
    constexpr int WAVES = 4;
    constexpr int NPART = DV / CB;
    constexpr int TB = REC_TB;
    static_assert(DK % RG == 0 && RPT >= 1 && DV % CB == 0, "row / column split");

    __shared__ float s_q[TB][DK], s_k[TB][DK], s_a[TB][DK];
    __shared__ __attribute__((aligned(16))) float s_v[TB][CB];
    __shared__ float s_b[TB], s_qk[TB];
    __shared__ f32x4 s_p[2][WAVES][NQ], s_r[2][WAVES][NQ];

    const int u = blockIdx.x / NPART;          // sequence * H + head
    const int c0 = (blockIdx.x % NPART) * CB;  // first value column of the slice
    const int seq = u / H, h = u % H;
    const int t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    const int jq = t % NQ, rg = t / NQ;

    int t0, t1;
    if (cu) {
        t0 = cu[seq];
        t1 = cu[seq + 1];
    } else {
        t0 = seq * rows;
        t1 = t0 + rows;
    }
    const int slot = slots ? slots[seq] : seq;
    if (slot < 0 || slot >= num_slots) {   // padding sequence (uniform over the workgroup)
        for (int x = t; x < (t1 - t0) * CB; x += 256)
            o[((size_t)(t0 + x / CB) * H + h) * DV + c0 + x % CB] = from_f32<E>(0.f);
        return;
    }
    if (t1 <= t0) return;
    float* S = pool + ((size_t)slot * H + h) * DK * DV + c0;

    f32x4 s[RPT];
#pragma unroll
    for (int m = 0; m < RPT; ++m) s[m] = *(reinterpret_cast<const f32x4*>(S + (size_t)(rg + RG * m) * DV) + jq);

    for (int tb = t0; tb < t1; tb += TB) {
        const int nt = min(TB, t1 - tb);
        // ---- stage nt tokens (rows past the end re-read the last token) ----
        for (int x = t; x < TB * DK; x += 256) {
            const int i = x / DK, c = x % DK;
            const size_t row = ((size_t)(tb + min(i, nt - 1)) * H + h) * DK + c;
            s_q[i][c] = to_f32(q[row]);
            s_k[i][c] = to_f32(k[row]);
            s_a[i][c] = __expf(log_alpha[row]);
        }
        for (int x = t; x < TB * CB; x += 256) {
            const int i = x / CB, j = x % CB;
            s_v[i][j] = to_f32(v[((size_t)(tb + min(i, nt - 1)) * H + h) * DV + c0 + j]);
        }
        if (t < TB) {
            const float b = beta[(size_t)(tb + min(t, nt - 1)) * H + h];
            s_b[t] = beta_logit ? sigmoid(b) : b;
        }
        __syncthreads();
        // ---- per token: optional L2 normalisation of q and k, and q . k ----
        for (int i = wave; i < TB; i += WAVES) {
            float qq = 0.f, kk = 0.f, qk = 0.f;
            for (int c = lane; c < DK; c += 64) {
                const float a = s_q[i][c], b = s_k[i][c];
                qq += a * a;
                kk += b * b;
                qk += a * b;
            }
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) {
                qq += __shfl_xor(qq, off);
                kk += __shfl_xor(kk, off);
                qk += __shfl_xor(qk, off);
            }
            if constexpr (NORM) {
                const float iq = rsqrtf(qq + L2NORM_EPS), ik = rsqrtf(kk + L2NORM_EPS);
                for (int c = lane; c < DK; c += 64) {
                    s_q[i][c] *= iq;
                    s_k[i][c] *= ik;
                }
                qk *= iq * ik;
            }
            if (lane == 0) s_qk[i] = qk;
        }
        __syncthreads();
        // ---- the tokens in order, state in registers ----
        for (int i = 0; i < nt; ++i) {
            f32x4 p = {0.f, 0.f, 0.f, 0.f}, r = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int m = 0; m < RPT; ++m) {
                const int c = rg + RG * m;
                s[m] *= s_a[i][c];
                p += s_k[i][c] * s[m];
                r += s_q[i][c] * s[m];
            }
#pragma unroll
            for (int off = NQ; off < 64; off <<= 1) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    p[e] += __shfl_xor(p[e], off);
                    r[e] += __shfl_xor(r[e], off);
                }
            }
            // partials of token i go to buffer i & 1: the buffer written here was
            // last read before the previous token's barrier
            if (lane < NQ) {
                s_p[i & 1][wave][jq] = p;
                s_r[i & 1][wave][jq] = r;
            }
            __syncthreads();
            p = s_p[i & 1][0][jq];
            r = s_r[i & 1][0][jq];
#pragma unroll
            for (int w = 1; w < WAVES; ++w) {
                p += s_p[i & 1][w][jq];
                r += s_r[i & 1][w][jq];
            }
            const f32x4 vv = *reinterpret_cast<const f32x4*>(&s_v[i][4 * jq]);
            const f32x4 nu = s_b[i] * (vv - p);
            if (rg == 0) {
                typename Vec<E>::v4 ov;
                const f32x4 ot = r + s_qk[i] * nu;
#pragma unroll
                for (int e = 0; e < 4; ++e) ov[e] = from_f32<E>(ot[e]);
                store_vec(o + ((size_t)(tb + i) * H + h) * DV + c0 + 4 * jq, ov);
            }
#pragma unroll
            for (int m = 0; m < RPT; ++m) s[m] += s_k[i][rg + RG * m] * nu;
        }
        __syncthreads();   // the next fill overwrites the staged tokens
    }
#pragma unroll
    for (int m = 0; m < RPT; ++m) *(reinterpret_cast<f32x4*>(S + (size_t)(rg + RG * m) * DV) + jq) = s[m];
}

template <typename E, int DK, int DV>
static hipError_t launch_rec_t(float* pool, int num_slots, const int32_t* slots, const void* q,
                               const void* k, const void* v, const float* la, const float* beta,
                               const int32_t* cu, int rows, int N, int H, unsigned flags, void* o,
                               hipStream_t stream)
{
    constexpr int CB = REC_COLS < DV ? REC_COLS : DV;
    const dim3 grid((unsigned)((long long)N * H * (DV / CB)));
    const int beta_logit = (flags & PRE_BETA_LOGIT) ? 1 : 0;
    if (flags & PRE_L2NORM_QK)
        hipLaunchKernelGGL((recurrent_kernel<E, DK, DV, CB, true>), grid, dim3(256), 0, stream, pool,
                           num_slots, slots, (const E*)q, (const E*)k, (const E*)v, la, beta, cu,
                           rows, H, beta_logit, (E*)o);
    else
        hipLaunchKernelGGL((recurrent_kernel<E, DK, DV, CB, false>), grid, dim3(256), 0, stream, pool,
                           num_slots, slots, (const E*)q, (const E*)k, (const E*)v, la, beta, cu,
                           rows, H, beta_logit, (E*)o);
    return hipGetLastError();
}

hipError_t launch_recurrent(float* pool, int num_slots, const int32_t* slots, const void* q,
                            const void* k, const void* v, const float* la, const float* beta,
                            const int32_t* cu, int rows, int N, int H, int dk, int dv,
                            bool bf16_io, unsigned flags, void* o, hipStream_t stream)
{
#define KDA_REC_CASE(E, DK_, DV_) \
    if (dk == DK_ && dv == DV_)   \
        return launch_rec_t<E, DK_, DV_>(pool, num_slots, slots, q, k, v, la, beta, cu, rows, N, H, flags, o, stream);
    if (bf16_io) {
        KDA_REC_CASE(bf16, 128, 128)
        KDA_REC_CASE(bf16, 64, 64)
        KDA_REC_CASE(bf16, 128, 64)
        KDA_REC_CASE(bf16, 64, 128)
    } else {
        KDA_REC_CASE(float, 128, 128)
        KDA_REC_CASE(float, 64, 64)
        KDA_REC_CASE(float, 128, 64)
        KDA_REC_CASE(float, 64, 128)
    }
#undef KDA_REC_CASE
    return hipErrorInvalidValue;
}

}  // namespace kda
