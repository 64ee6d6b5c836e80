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
// One workgroup per (sequence, head) keeps the head's fp32 state in registers
// across all of the sequence's tokens: the state is read from its slot once
// and written back once, however many tokens the sequence has.  Wave w owns
// value columns 32w .. 32w + 31 for every key row; lane l holds columns
// 32w + 4(l & 7) .. +3 of the RPL = dk/8 consecutive rows starting at
// RPL (l >> 3), so the 8 lanes of a row group read whole 128-byte rows.  The
// sums over key rows stay inside the wave (a transposing butterfly over the
// 8 row groups), so the waves wait for each other only around the staging of
// up to 16 tokens in LDS (q, k, alpha and v, widened to fp32).  A sequence whose
// slot lies outside the pool is padding: its output rows are zeroed and no
// state is touched.
#include "kda_common.h"

namespace kda {

constexpr int REC_TB = 16;     // tokens staged per LDS fill

template <typename E, int DK, int DV, bool NORM>
__global__ __launch_bounds__(64 * (DV / 32)) void recurrent_kernel(
    float* __restrict__ pool, int num_slots, const int32_t* __restrict__ slots,
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
    const float* __restrict__ log_alpha, const float* __restrict__ beta,
    const int32_t* __restrict__ cu, int rows, int H, int beta_logit, E* __restrict__ o)
{
    constexpr int WAVES = DV / 32;
    constexpr int NT = 64 * WAVES;
    constexpr int RPL = DK / 8;      // key rows per lane
    constexpr int TB = REC_TB;

    __shared__ __attribute__((aligned(16))) float s_q[TB][DK], s_k[TB][DK], s_a[TB][DK];
    __shared__ __attribute__((aligned(16))) float s_v[TB][DV];
    __shared__ float s_b[TB], s_qk[TB];

    const int u = blockIdx.x;   // sequence * H + head
    const int seq = u / H, h = u % H;
    const int t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    const int quad = lane & 7, rg = lane >> 3;
    const int c0 = 32 * wave + 4 * quad;   // this lane's first value column
    const int r0 = RPL * rg;               // and first key row
    // value index of this lane after rowgroup_sum8: 0..3 -> p column, 4..7 -> r column
    const int vi = 4 * ((lane >> 5) & 1) + 2 * ((lane >> 4) & 1) + ((lane >> 3) & 1);

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
        for (int x = t; x < (t1 - t0) * DV; x += NT)
            o[((size_t)(t0 + x / DV) * H + h) * DV + x % DV] = from_f32<E>(0.f);
        return;
    }
    if (t1 <= t0) return;
    float* S = pool + ((size_t)slot * H + h) * DK * DV;

    f32x4 s[RPL];
#pragma unroll
    for (int m = 0; m < RPL; ++m) s[m] = *reinterpret_cast<const f32x4*>(S + (size_t)(r0 + m) * DV + c0);

    for (int tb = t0; tb < t1; tb += TB) {
        const int nt = min(TB, t1 - tb);
        // ---- stage nt tokens, 4 channels per load ----
        for (int x = t; x < nt * (DK / 4); x += NT) {
            const int i = x / (DK / 4), c = 4 * (x % (DK / 4));
            const size_t row = ((size_t)(tb + i) * H + h) * DK + c;
            const typename Vec<E>::v4 q4 = load_vec<typename Vec<E>::v4>(q + row);
            const typename Vec<E>::v4 k4 = load_vec<typename Vec<E>::v4>(k + row);
            const f32x4 l4 = *reinterpret_cast<const f32x4*>(log_alpha + row);
            f32x4 fq, fk, fa;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                fq[e] = to_f32(q4[e]);
                fk[e] = to_f32(k4[e]);
                fa[e] = __expf(l4[e]);
            }
            *reinterpret_cast<f32x4*>(&s_q[i][c]) = fq;
            *reinterpret_cast<f32x4*>(&s_k[i][c]) = fk;
            *reinterpret_cast<f32x4*>(&s_a[i][c]) = fa;
        }
        for (int x = t; x < nt * (DV / 4); x += NT) {
            const int i = x / (DV / 4), j = 4 * (x % (DV / 4));
            const typename Vec<E>::v4 v4 = load_vec<typename Vec<E>::v4>(v + ((size_t)(tb + i) * H + h) * DV + j);
            f32x4 fv;
#pragma unroll
            for (int e = 0; e < 4; ++e) fv[e] = to_f32(v4[e]);
            *reinterpret_cast<f32x4*>(&s_v[i][j]) = fv;
        }
        if (t < nt) {
            const float b = beta[(size_t)(tb + t) * H + h];
            s_b[t] = beta_logit ? sigmoid(b) : b;
        }
        __syncthreads();
        // ---- per token: optional L2 normalisation of q and k, and q . k ----
        for (int i = wave; i < nt; i += WAVES) {
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
        // ---- the tokens in order, state in registers, no barrier ----
        for (int i = 0; i < nt; ++i) {
            float kr[RPL];
            f32x4 p = {0.f, 0.f, 0.f, 0.f}, r = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int m4 = 0; m4 < RPL / 4; ++m4) {
                const f32x4 a4 = *reinterpret_cast<const f32x4*>(&s_a[i][r0 + 4 * m4]);
                const f32x4 k4 = *reinterpret_cast<const f32x4*>(&s_k[i][r0 + 4 * m4]);
                const f32x4 q4 = *reinterpret_cast<const f32x4*>(&s_q[i][r0 + 4 * m4]);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int m = 4 * m4 + e;
                    kr[m] = k4[e];
                    s[m] *= a4[e];
                    p += k4[e] * s[m];
                    r += q4[e] * s[m];
                }
            }
            const float part[8] = {p[0], p[1], p[2], p[3], r[0], r[1], r[2], r[3]};
            const float tot = rowgroup_sum8(part, lane);   // p (vi < 4) or r of column jv
            // lanes with vi < 4 hold p_j and form nu_j; the partner lane (xor 32)
            // holds r_j and forms the output
            const int jv = 4 * quad + (vi & 3) + 32 * wave;   // the column of tot
            const float nu = vi < 4 ? s_b[i] * (s_v[i][jv] - tot) : 0.f;
            const float nu_p = lane_xor<32>(nu);
            if (vi >= 4) o[((size_t)(tb + i) * H + h) * DV + jv] = from_f32<E>(tot + s_qk[i] * nu_p);
            // nu of this lane's 4 columns: from the lanes (quad, vi = 0..3)
            f32x4 nu4;
#pragma unroll
            for (int e = 0; e < 4; ++e) nu4[e] = __shfl(nu, quad + 8 * e);
#pragma unroll
            for (int m = 0; m < RPL; ++m) s[m] += kr[m] * nu4;
        }
        __syncthreads();   // the next fill overwrites the staged tokens
    }
#pragma unroll
    for (int m = 0; m < RPL; ++m) *reinterpret_cast<f32x4*>(S + (size_t)(r0 + m) * DV + c0) = s[m];
}

template <typename E, int DK, int DV>
static hipError_t launch_rec_t(float* pool, int num_slots, const int32_t* slots, const void* q,
                               const void* k, const void* v, const float* la, const float* beta,
                               const int32_t* cu, int rows, int N, int H, unsigned flags, void* o,
                               hipStream_t stream)
{
    const dim3 grid((unsigned)((long long)N * H));
    const int beta_logit = (flags & PRE_BETA_LOGIT) ? 1 : 0;
    if (flags & PRE_L2NORM_QK)
        hipLaunchKernelGGL((recurrent_kernel<E, DK, DV, true>), grid, dim3(64 * (DV / 32)), 0, stream, pool,
                           num_slots, slots, (const E*)q, (const E*)k, (const E*)v, la, beta, cu,
                           rows, H, beta_logit, (E*)o);
    else
        hipLaunchKernelGGL((recurrent_kernel<E, DK, DV, false>), grid, dim3(64 * (DV / 32)), 0, stream, pool,
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
