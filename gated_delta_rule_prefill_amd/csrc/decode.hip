// decode.hip -- fused single-token KDA step (the recurrent decode path).
//
// For each (sequence, head) the fp32 state S (dk x dv) is streamed from HBM
// exactly once, updated in registers and written back in place:
//
//   S' = Diag(alpha) S                      alpha = exp(log_alpha), per key channel
//   p  = S'^T k,   r = S'^T q               (one pass, two reductions over dk)
//   nu = beta (v - p)                       (delta-rule correction)
//   S  = S' + k nu^T
//   o  = S^T q = r + (q . k) nu
//
// which is the recurrence S_t = (I - beta k k^T) Diag(alpha) S_{t-1} + beta k v^T,
// o_t = S_t^T q_t (Kimi Linear paper notes, section 2) expanded so that the
// state is read once.  The kernel is bound by HBM bandwidth on the state.
#include "kda_common.h"

namespace kda {

// Value columns per workgroup (measured on MI355X with 256 x 32 heads of
// 128 x 128 fp32 state: 64 columns beat 128, 32 and 16).
constexpr int DECODE_COLS = 64;

// One workgroup of 256 threads per (sequence, head, CB value columns): the
// reductions over key channels are per value column, so column slices of a
// head are independent.  Thread t owns columns c0 + 4*(t % NQ) .. +3 and key
// rows rg, rg + RG, ... with rg = t / NQ, so each row of the slice is read by
// NQ consecutive threads as 16-byte vectors.  Smaller slices mean fewer rows
// per thread, fewer registers and more workgroups in flight per CU.
template <typename E, int DK, int DV, int CB>
__global__ __launch_bounds__(256) void decode_step_kernel(
    float* __restrict__ state, const E* __restrict__ q, const E* __restrict__ k,
    const E* __restrict__ v, const float* __restrict__ log_alpha,
    const float* __restrict__ beta, E* __restrict__ o)
{
    constexpr int NQ = CB / 4;       // column quads of the slice
    constexpr int RG = 256 / NQ;     // row groups
    constexpr int RPT = DK / RG;     // rows per thread
    constexpr int WAVES = 4;
    constexpr int NPART = DV / CB;   // slices per head
    static_assert(DK % RG == 0 && RPT >= 1 && DV % CB == 0, "row / column split");

    __shared__ float s_q[DK], s_k[DK], s_a[DK];
    __shared__ f32x4 s_p[WAVES][NQ], s_r[WAVES][NQ];
    __shared__ float s_qk;

    const int u = blockIdx.x / NPART;         // sequence * H + head
    const int c0 = (blockIdx.x % NPART) * CB; // first value column of the slice
    const int t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    const int jq = t % NQ, rg = t / NQ;
    float* S = state + (size_t)u * DK * DV + c0;

    // Issue the state loads first: they dominate and do not depend on q/k.
    // Plain (cached) loads and streaming stores measured fastest: 5.8 TB/s on
    // the 512 MiB state against 5.5 with streaming loads.
    f32x4 s[RPT];
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const int c = rg + RG * m;
        s[m] = *(reinterpret_cast<const f32x4*>(S + (size_t)c * DV) + jq);
    }

    for (int c = t; c < DK; c += 256) {
        s_q[c] = to_f32(q[(size_t)u * DK + c]);
        s_k[c] = to_f32(k[(size_t)u * DK + c]);
        s_a[c] = __expf(log_alpha[(size_t)u * DK + c]);
    }
    if (wave == 0) {
        float acc = 0.f;
        for (int c = lane; c < DK; c += 64)
            acc += to_f32(q[(size_t)u * DK + c]) * to_f32(k[(size_t)u * DK + c]);
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
        if (lane == 0) s_qk = acc;
    }
    __syncthreads();

    f32x4 p = {0.f, 0.f, 0.f, 0.f}, r = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const int c = rg + RG * m;
        s[m] *= s_a[c];
        p += s_k[c] * s[m];
        r += s_q[c] * s[m];
    }
    // Reduce over the row groups inside the wave (lanes that share jq) ...
#pragma unroll
    for (int off = NQ; off < 64; off <<= 1) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            p[i] += __shfl_xor(p[i], off);
            r[i] += __shfl_xor(r[i], off);
        }
    }
    // ... then across the four waves.
    if (lane < NQ) {
        s_p[wave][jq] = p;
        s_r[wave][jq] = r;
    }
    __syncthreads();
    p = s_p[0][jq];
    r = s_r[0][jq];
#pragma unroll
    for (int w = 1; w < WAVES; ++w) {
        p += s_p[w][jq];
        r += s_r[w][jq];
    }

    const float b = beta[u];
    const typename Vec<E>::v4 vv = load_vec<typename Vec<E>::v4>(v + (size_t)u * DV + c0 + 4 * jq);
    f32x4 nu;
#pragma unroll
    for (int i = 0; i < 4; ++i) nu[i] = b * (to_f32(vv[i]) - p[i]);

    if (rg == 0) {
        typename Vec<E>::v4 ov;
#pragma unroll
        for (int i = 0; i < 4; ++i) ov[i] = from_f32<E>(r[i] + s_qk * nu[i]);
        store_vec(o + (size_t)u * DV + c0 + 4 * jq, ov);
    }

#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const int c = rg + RG * m;
        f32x4 out = s[m] + s_k[c] * nu;
        __builtin_nontemporal_store(out, reinterpret_cast<f32x4*>(S + (size_t)c * DV) + jq);
    }
}

template <typename E, int DK, int DV>
static hipError_t launch_decode(float* state, const void* q, const void* k, const void* v,
                                const float* la, const float* beta, void* o, int units,
                                hipStream_t stream)
{
    constexpr int CB = DECODE_COLS < DV ? DECODE_COLS : DV;
    hipLaunchKernelGGL((decode_step_kernel<E, DK, DV, CB>), dim3(units * (DV / CB)), dim3(256), 0,
                       stream, state, (const E*)q, (const E*)k, (const E*)v, la, beta, (E*)o);
    return hipGetLastError();
}

hipError_t launch_decode_step(float* state, const void* q, const void* k, const void* v,
                              const float* la, const float* beta, void* o, int units, int dk,
                              int dv, bool bf16_io, hipStream_t stream)
{
#define KDA_DECODE_CASE(E, DK_, DV_) \
    if (dk == DK_ && dv == DV_) return launch_decode<E, DK_, DV_>(state, q, k, v, la, beta, o, units, stream);
    if (bf16_io) {
        KDA_DECODE_CASE(bf16, 128, 128)
        KDA_DECODE_CASE(bf16, 64, 64)
        KDA_DECODE_CASE(bf16, 128, 64)
        KDA_DECODE_CASE(bf16, 64, 128)
    } else {
        KDA_DECODE_CASE(float, 128, 128)
        KDA_DECODE_CASE(float, 64, 64)
        KDA_DECODE_CASE(float, 128, 64)
        KDA_DECODE_CASE(float, 64, 128)
    }
#undef KDA_DECODE_CASE
    return hipErrorInvalidValue;
}

}  // namespace kda
