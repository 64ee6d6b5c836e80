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

// One workgroup per (sequence, head), DV/32 waves: wave w owns value columns
// 32w .. 32w + 31 for every key row; lane l holds columns 32w + 4(l & 7) .. +3
// of the DK/8 consecutive rows starting at (DK/8)(l >> 3), so the 8 lanes of
// a row group read whole 128-byte rows of the state.  Each lane loads its own
// rows' alpha, k and q, and the sums over key rows (S'^T k, S'^T q for the
// lane's 4 columns, q . k) stay inside the wave: no LDS and no barrier, so
// every wave streams its part of the state independently.  Plain loads and
// streaming stores for the state (measured fastest; an earlier layout with
// one workgroup per 64 columns and partial sums over four waves reached
// 5.8 TB/s on the 512 MiB state, this one 6.2).
//
// slots (or NULL): the states are a pool and sequence s's state of head h is
// pool slot slots[s] (H heads per slot); a slot outside [0, num_slots) marks
// a padding sequence, whose output is zeroed and whose state is not touched.
// n_seqs > 0 (slot order): the grid walks the pool's slots instead of the
// sequences, workgroup b taking slot b / H and head b % H, so that the states
// stream in address order whatever order the slots are given in (a permuted
// order measured ≈17 % slower).  The workgroup finds the sequence holding its
// slot by one pass over the slot array; a slot no sequence holds is skipped,
// and the o rows of padding sequence s are zeroed by the workgroups of slot
// s mod num_slots.
template <typename E, int DK, int DV>
__global__ __launch_bounds__(64 * (DV / 32)) void decode_step_kernel(
    float* __restrict__ state, const E* __restrict__ q, const E* __restrict__ k,
    const E* __restrict__ v, const float* __restrict__ log_alpha,
    const float* __restrict__ beta, E* __restrict__ o,
    const int32_t* __restrict__ slots, int num_slots, int H, int n_seqs)
{
    constexpr int RPL = DK / 8;   // key rows per lane
    int u = blockIdx.x;           // sequence * H + head (slot * H + head in slot order)
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int quad = lane & 7, rg = lane >> 3;
    const int c0 = 32 * wave + 4 * quad, r0 = RPL * rg;
    // value index of this lane after the row-group sums: 0..3 -> p, 4..7 -> r
    const int vi = 4 * ((lane >> 5) & 1) + 2 * ((lane >> 4) & 1) + ((lane >> 3) & 1);
    float* S = state + (size_t)u * DK * DV;
    if (slots && n_seqs > 0) {   // slot order (uniform over the launch)
        __shared__ int sSeq;
        const int slot = u / H, h = u - slot * H;
        if (threadIdx.x == 0) sSeq = -1;
        __syncthreads();
        for (int i = threadIdx.x; i < n_seqs; i += blockDim.x) {
            const int si = slots[i];
            if (si == slot) sSeq = i;
            else if ((si < 0 || si >= num_slots) && i % num_slots == slot)
                for (int x = 0; x < DV; x += 4) {   // padding sequence i: zero its o row of head h
                    typename Vec<E>::v4 z;
#pragma unroll
                    for (int e = 0; e < 4; ++e) z[e] = from_f32<E>(0.f);
                    store_vec(o + ((size_t)i * H + h) * DV + x, z);
                }
        }
        __syncthreads();
        const int seq = sSeq;
        if (seq < 0) return;   // no sequence holds this slot (uniform over the workgroup)
        u = seq * H + h;
        S = state + ((size_t)slot * H + h) * DK * DV;
    } else if (slots) {
        const int seq = u / H, slot = slots[seq];
        if (slot < 0 || slot >= num_slots) {   // padding sequence (uniform over the workgroup)
            for (int x = threadIdx.x; x < DV; x += blockDim.x) o[(size_t)u * DV + x] = from_f32<E>(0.f);
            return;
        }
        S = state + ((size_t)slot * H + (u - seq * H)) * DK * DV;
    }

    // the state loads first: they dominate and depend on nothing else
    f32x4 s[RPL];
#pragma unroll
    for (int m = 0; m < RPL; ++m) s[m] = *reinterpret_cast<const f32x4*>(S + (size_t)(r0 + m) * DV + c0);
    float la[RPL], kk[RPL], qq[RPL];
#pragma unroll
    for (int m4 = 0; m4 < RPL / 4; ++m4) {
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(log_alpha + (size_t)u * DK + r0 + 4 * m4);
        const typename Vec<E>::v4 k4 = load_vec<typename Vec<E>::v4>(k + (size_t)u * DK + r0 + 4 * m4);
        const typename Vec<E>::v4 q4 = load_vec<typename Vec<E>::v4>(q + (size_t)u * DK + r0 + 4 * m4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            la[4 * m4 + e] = l4[e];
            kk[4 * m4 + e] = to_f32(k4[e]);
            qq[4 * m4 + e] = to_f32(q4[e]);
        }
    }
    const int jv = 32 * wave + 4 * quad + (vi & 3);   // the column of this lane's sum
    const float vj = to_f32(v[(size_t)u * DV + jv]);
    const float b = beta[u];

    f32x4 p = {0.f, 0.f, 0.f, 0.f}, r = {0.f, 0.f, 0.f, 0.f};
    float qk = 0.f;
#pragma unroll
    for (int m = 0; m < RPL; ++m) {
        s[m] *= __expf(la[m]);
        p += kk[m] * s[m];
        r += qq[m] * s[m];
        qk += qq[m] * kk[m];
    }
    qk += lane_xor<8>(qk);
    qk += lane_xor<16>(qk);
    qk += lane_xor<32>(qk);
    const float part[8] = {p[0], p[1], p[2], p[3], r[0], r[1], r[2], r[3]};
    const float tot = rowgroup_sum8(part, lane);
    // lanes with vi < 4 hold p_j and form nu_j; the partner lane (xor 32)
    // holds r_j and writes o_j = r_j + (q . k) nu_j
    const float nu = vi < 4 ? b * (vj - tot) : 0.f;
    const float nu_p = lane_xor<32>(nu);
    if (vi >= 4) o[(size_t)u * DV + jv] = from_f32<E>(tot + qk * nu_p);
    f32x4 nu4;   // nu of this lane's 4 columns, from the lanes (quad, vi = 0..3)
#pragma unroll
    for (int e = 0; e < 4; ++e) nu4[e] = __shfl(nu, quad + 8 * e);
#pragma unroll
    for (int m = 0; m < RPL; ++m)
        __builtin_nontemporal_store(s[m] + kk[m] * nu4, reinterpret_cast<f32x4*>(S + (size_t)(r0 + m) * DV + c0));
}

template <typename E, int DK, int DV>
static hipError_t launch_decode(float* state, const void* q, const void* k, const void* v,
                                const float* la, const float* beta, void* o, int units,
                                const int32_t* slots, int num_slots, int H, int n_seqs,
                                hipStream_t stream)
{
    hipLaunchKernelGGL((decode_step_kernel<E, DK, DV>), dim3(units), dim3(64 * (DV / 32)), 0, stream,
                       state, (const E*)q, (const E*)k, (const E*)v, la, beta, (E*)o, slots, num_slots,
                       H, n_seqs);
    return hipGetLastError();
}

static hipError_t launch_decode_any(float* state, const void* q, const void* k, const void* v,
                                    const float* la, const float* beta, void* o, int units,
                                    const int32_t* slots, int num_slots, int H, int n_seqs, int dk,
                                    int dv, bool bf16_io, hipStream_t stream)
{
#define KDA_DECODE_CASE(E, DK_, DV_) \
    if (dk == DK_ && dv == DV_)      \
        return launch_decode<E, DK_, DV_>(state, q, k, v, la, beta, o, units, slots, num_slots, H, n_seqs, stream);
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

hipError_t launch_decode_step(float* state, const void* q, const void* k, const void* v,
                              const float* la, const float* beta, void* o, int units, int dk,
                              int dv, bool bf16_io, hipStream_t stream)
{
    return launch_decode_any(state, q, k, v, la, beta, o, units, nullptr, 0, 1, 0, dk, dv, bf16_io, stream);
}

// One token for each of N sequences on pooled states (see kda_decode_tokens):
// the decode step with slot indirection.
hipError_t launch_decode_slots(float* pool, int num_slots, const int32_t* slots, const void* q,
                               const void* k, const void* v, const float* la, const float* beta,
                               void* o, int N, int H, int dk, int dv, bool bf16_io, hipStream_t stream)
{
    if (!slots) return launch_decode_any(pool, q, k, v, la, beta, o, N * H, nullptr, 0, 1, 0, dk, dv, bf16_io, stream);
    // slot order where the pool is not much larger than the batch (the grid
    // walks every slot) and one pass over the slot array stays short
    if (N <= SLOT_ORDER_MAX_SEQS && (long long)num_slots <= 2LL * N)
        return launch_decode_any(pool, q, k, v, la, beta, o, num_slots * H, slots, num_slots, H, N, dk, dv,
                                 bf16_io, stream);
    return launch_decode_any(pool, q, k, v, la, beta, o, N * H, slots, num_slots, H, 0, dk, dv, bf16_io, stream);
}

}  // namespace kda
