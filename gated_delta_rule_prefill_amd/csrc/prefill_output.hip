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

// LDS holds only the chunk-start state, exactly as stored (operand slots,
// lane-contiguous), so several workgroups fit per CU.
template <typename E, int DK, int DV>
struct OutCfg {
    static constexpr int ES = sizeof(E);
    static constexpr int KS = DK / 32, NSL = DV / 16;
    static constexpr int ST_BYTES = DK * DV * ES;
    static constexpr int LOADS = ST_BYTES / 1024;             // direct loads per workgroup
    static constexpr int LOADS_W = (LOADS + 3) / 4;           // per wave
    static_assert(ST_BYTES % 1024 == 0, "state size");
};

// Wave w owns rows 16w .. 16w + 15 of the chunk for every value slice: its
// QM rows come straight into registers, the state comes from LDS (one direct
// load per 1 KiB, a quarter per wave).
template <typename E, int DK, int DV>
__global__ __launch_bounds__(256) void prefill_output_kernel(
    const unsigned char* __restrict__ rec, const E* __restrict__ states, const ChunkSrc src, int H,
    E* __restrict__ o)
{
    using C = OutCfg<E, DK, DV>;
    using V4 = typename Vec<E>::v4;
    using V8 = typename Vec<E>::v8;
    constexpr int KS = C::KS, NSL = C::NSL;
    constexpr RecLayout RL = rec_layout(sizeof(E), DK, DV);
    __shared__ __attribute__((aligned(1024))) unsigned char sm[C::LOADS_W * 4 * 1024];

    int cid, h;
    chunk_head_of_block(H, false, cid, h);
    int n_chunks;
    ChunkInfo ci;
    chunk_of(src, cid, n_chunks, ci);
    if (cid >= n_chunks) return;
    const size_t chh = (size_t)cid * H + h;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l = threadIdx.x & 63, g = l >> 4, ln = l & 15;
    const unsigned char* R0 = rec + chh * RL.bytes;
    const unsigned char* St = reinterpret_cast<const unsigned char*>(states + chh * DK * DV);

    {
        const unsigned char* srcp[C::LOADS_W];
#pragma unroll
        for (int k = 0; k < C::LOADS_W; ++k) srcp[k] = St + 1024 * (size_t)(C::LOADS_W * wave + k) + 16 * l;
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k = 0; k < C::LOADS_W; ++k)
            if (C::LOADS_W * wave + k < C::LOADS)
                __builtin_amdgcn_global_load_lds((out_global_void*)srcp[k],
                                                 (out_lds_void*)(sm + 1024 * (C::LOADS_W * wave + k)), 16, 0,
                                                 2 /* non-temporal: the state's only reader */);
    }
    const int r = 16 * wave + ln;   // this lane's row of the chunk
    const E* QM = reinterpret_cast<const E*>(R0 + RL.qm);
    const E* OI = reinterpret_cast<const E*>(R0 + RL.oi);
    V8 q[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) q[ks] = load_vec<V8>(QM + r * DK + 32 * ks + 8 * g);
    // OI[r][columns 16 sl + 4g .. +3] for every slice sl (perm32 slots: slices
    // 2m and 2m + 1 share one 16-byte group)
    float oi[NSL][4];
#pragma unroll
    for (int m = 0; m < NSL / 2; ++m) {
        const V8 v = load_frag(OI + frag_at<DV / 32>(wave, m), l);   // row r, slots 8g .. 8g + 7 of block m
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            oi[2 * m][i] = to_f32(v[i]);
            oi[2 * m + 1][i] = to_f32(v[4 + i]);
        }
    }
    __syncthreads();   // the workgroup's direct loads have landed

    const E* sst = reinterpret_cast<const E*>(sm);
#pragma unroll
    for (int sl = 0; sl < NSL; ++sl) {
        // O^T tile: lane holds O[16 wave + ln][16 sl + 4g + i]
        f32x4 acc = {oi[sl][0], oi[sl][1], oi[sl][2], oi[sl][3]};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            acc = mma32(load_vec<V8>(sst + ((sl * KS + ks) * 64 + l) * 8), q[ks], acc);
        if (r < ci.len) {
            V4 w;
#pragma unroll
            for (int i = 0; i < 4; ++i) w[i] = from_f32<E>(acc[i]);
            store_vec(o + ((size_t)(ci.start + r) * H + h) * DV + 16 * sl + 4 * g, w);
        }
    }
}

template <typename E, int DK, int DV>
static hipError_t launch_output_t(const void* rec, const void* states, ChunkSrc src, int max_chunks,
                                  int H, void* o, hipStream_t stream)
{
    hipLaunchKernelGGL((prefill_output_kernel<E, DK, DV>), dim3(max_chunks * H), dim3(256), 0, stream,
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
