// prefill_output.hip -- output pass of the chunkwise KDA prefill.
//
// The output of a chunk is its read-out of the chunk-start state plus its
// intra-chunk term (Kimi Linear paper notes, section 3: inter- plus
// intra-chunk output).  With the chunk folded by the intra kernel,
//
//     O = QM S_c + OI,
//
// where S_c is the state entering the chunk, stored by the sequential kernel
// as bf16 (or fp32) MFMA operand slots.  Every (chunk, head) is independent,
// so the pass is one workgroup per (chunk, head), like the intra kernel.
#include "kda_common.h"

namespace kda {

typedef __attribute__((address_space(1))) void out_global_void;
typedef __attribute__((address_space(3))) void out_lds_void;

// LDS staging of one (chunk, head): the chunk-start state exactly as stored
// (operand slots, lane-contiguous) and QM with 16-byte padded rows.
template <typename E, int DK, int DV>
struct OutCfg {
    static constexpr int ES = sizeof(E);
    static constexpr int KS = DK / 32, NSL = DV / 16, SPW = NSL / 4;
    static constexpr int ST_UNITS = DK * DV * ES / 16;        // state, 16-byte units
    static constexpr int RW = DK * ES / 16;                   // units per QM row
    static constexpr int QM_UNITS = 64 * (RW + 1);            // padded rows
    static constexpr int UNITS = ST_UNITS + QM_UNITS;
    static constexpr int LOADS = (UNITS + 63) / 64;           // direct loads per block
    static constexpr int LOADS_W = (LOADS + 3) / 4;           // per wave
    static constexpr int OFF_QM = ST_UNITS * 16;
    static constexpr int QRS = (RW + 1) * 16;                 // padded QM row stride
    static constexpr int LDS_BYTES = LOADS_W * 4 * 1024;
};

// Wave w owns value slices SPW*w .. SPW*w + SPW - 1 (16 columns each) for all
// 64 rows; with two slices per wave their columns 4g..4g+3 are the 8
// consecutive perm32 slots 8g..8g+7 of OI.  The state and QM are moved into
// LDS once per workgroup by direct global->LDS loads, a quarter per wave.
template <typename E, int DK, int DV>
__global__ __launch_bounds__(256) void prefill_output_kernel(
    const unsigned char* __restrict__ rec, const E* __restrict__ states,
    const ChunkSrc src, int H, E* __restrict__ o)
{
    using C = OutCfg<E, DK, DV>;
    using V4 = typename Vec<E>::v4;
    using V8 = typename Vec<E>::v8;
    constexpr int KS = C::KS, SPW = C::SPW;
    static_assert(SPW == 1 || SPW == 2, "value slices per wave");
    constexpr RecLayout RL = rec_layout(sizeof(E), DK, DV);
    __shared__ __attribute__((aligned(1024))) unsigned char sm[C::LDS_BYTES];

    const int cid = blockIdx.x;
    int n_chunks;
    ChunkInfo ci;
    chunk_of(src, cid, n_chunks, ci);
    if (cid >= n_chunks) return;
    const int h = blockIdx.y;
    const size_t chh = (size_t)cid * H + h;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l = threadIdx.x & 63, g = l >> 4, ln = l & 15;
    const unsigned char* R0 = rec + chh * RL.bytes;
    const unsigned char* St = reinterpret_cast<const unsigned char*>(states + chh * DK * DV);

    // direct loads: units [0, ST_UNITS) copy the state, the rest fill QM's padded rows
    {
        const unsigned char* src[C::LOADS_W];
#pragma unroll
        for (int k = 0; k < C::LOADS_W; ++k) {
            const int u = 64 * (C::LOADS_W * wave + k) + l;
            if (u < C::ST_UNITS) {
                src[k] = St + 16 * (size_t)u;
            } else {
                const int v = u < C::UNITS ? u - C::ST_UNITS : 0;
                const int row = v / (C::RW + 1), col = v % (C::RW + 1);
                src[k] = R0 + RL.qm + (size_t)row * DK * sizeof(E) + (col < C::RW ? col : 0) * 16;
            }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k = 0; k < C::LOADS_W; ++k)
            if (C::LOADS_W * wave + k < C::LOADS)
                __builtin_amdgcn_global_load_lds((out_global_void*)src[k],
                                                 (out_lds_void*)(sm + 1024 * (C::LOADS_W * wave + k)), 16, 0, 0);
    }
    // OI[16R + ln][columns j0 + 4g .. +3 of each owned slice] (perm32 slots)
    float oi[4][SPW][4];
    const E* OI = reinterpret_cast<const E*>(R0 + RL.oi);
#pragma unroll
    for (int R = 0; R < 4; ++R) {
        const E* src = OI + (16 * R + ln) * DV + perm_index(16 * SPW * wave + 4 * g);
        if constexpr (SPW == 2) {
            const V8 v = load_vec<V8>(src);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                oi[R][0][i] = to_f32(v[i]);
                oi[R][1][i] = to_f32(v[4 + i]);
            }
        } else {
            const V4 v = load_vec<V4>(src);
#pragma unroll
            for (int i = 0; i < 4; ++i) oi[R][0][i] = to_f32(v[i]);
        }
    }
    __syncthreads();   // the workgroup's direct loads have landed

    const E* sst = reinterpret_cast<const E*>(sm);
    V8 sf[SPW][KS];
#pragma unroll
    for (int sp = 0; sp < SPW; ++sp)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) sf[sp][ks] = load_vec<V8>(sst + (((SPW * wave + sp) * KS + ks) * 64 + l) * 8);
#pragma unroll
    for (int R = 0; R < 4; ++R) {
        V8 q[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            q[ks] = load_vec<V8>(reinterpret_cast<const E*>(sm + C::OFF_QM + (16 * R + ln) * C::QRS) + 32 * ks + 8 * g);
        const int r = 16 * R + ln;
#pragma unroll
        for (int sp = 0; sp < SPW; ++sp) {
            // O^T tile: lane holds O[16R + ln][j0 + 4g + i]
            f32x4 acc = {oi[R][sp][0], oi[R][sp][1], oi[R][sp][2], oi[R][sp][3]};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) acc = mma32(sf[sp][ks], q[ks], acc);
            if (r < ci.len) {
                V4 w;
#pragma unroll
                for (int i = 0; i < 4; ++i) w[i] = from_f32<E>(acc[i]);
                const int j0 = 16 * (SPW * wave + sp);
                store_vec(o + ((size_t)(ci.start + r) * H + h) * DV + j0 + 4 * g, w);
            }
        }
    }
}

template <typename E, int DK, int DV>
static hipError_t launch_output_t(const void* rec, const void* states, ChunkSrc src, int max_chunks,
                                  int H, void* o, hipStream_t stream)
{
    hipLaunchKernelGGL((prefill_output_kernel<E, DK, DV>), dim3(max_chunks, H), dim3(256), 0, stream,
                       (const unsigned char*)rec, (const E*)states, src, H, (E*)o);
    return hipGetLastError();
}

hipError_t launch_prefill_output(const void* rec, const void* states, ChunkSrc src,
                                 int max_chunks, int H, int dk, int dv, bool bf16_io, void* o,
                                 hipStream_t stream)
{
#define KDA_OUT_CASE(E, DK_, DV_)   \
    if (dk == DK_ && dv == DV_)       \
        return launch_output_t<E, DK_, DV_>(rec, states, src, max_chunks, H, o, stream);
    if (bf16_io) {
        KDA_OUT_CASE(bf16, 128, 128)
        KDA_OUT_CASE(bf16, 64, 64)
        KDA_OUT_CASE(bf16, 128, 64)
        KDA_OUT_CASE(bf16, 64, 128)
    } else {
        KDA_OUT_CASE(float, 64, 64)
        KDA_OUT_CASE(float, 64, 128)
    }
#undef KDA_OUT_CASE
    return hipErrorInvalidValue;
}

}  // namespace kda
