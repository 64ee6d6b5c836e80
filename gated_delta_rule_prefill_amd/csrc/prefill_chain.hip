// prefill_chain.hip -- sequential inter-chunk pass of the chunkwise KDA
// prefill over two value slices per workgroup (bf16 q/k/v, dk = 128).
//
// Same chain as prefill_state.hip (Kimi Linear paper notes, section 3: only
// the fixed-size state crosses chunk boundaries), with entry state S each
// chunk in order applies
//
//   O  = QM S + OI,     S' = Diag(gamma_C) S + PM S + Hc,
//
// but one workgroup covers 32 value columns of a (sequence, head), and every
// compute wave does both halves of the work for its part:
//
//   compute wave w (w < 4)  owns rows 32w .. 32w + 31 of the fp32 state tile
//       (32 x 32, in MFMA accumulators for the whole sequence) and forms the
//       outputs of token tile w (16 tokens x 32 columns) of every chunk.  Per
//       chunk it reads the whole chunk-start state as bf16 operand slots from
//       LDS; those slots are the B operands of PM S and, unchanged, the A
//       operands of O^T = S^T QM^T (a slot holds 8 key rows of one value
//       column either way).  Its PM rows, Hc^T planes, gamma_C and OI planes
//       come straight from the record into a register ring of three chunk
//       sets, two chunks ahead; PM is fetched once for both value slices;
//   stager wave             moves QM (64 rows, padded stride) into a
//       three-slot LDS ring with direct global->LDS loads, two chunks ahead.
//
// One barrier per chunk.  Compared with one value slice per workgroup this
// halves the workgroups (and the CU time) of a chain while each CU moves
// about 62 KiB per chunk, and it needs 67 KiB of LDS and one wave per SIMD,
// so an intra-chunk workgroup fits beside it on the same CU.
#include <hip/hip_ext.h>

#include "kda_common.h"

namespace kda {

template <int DV>
struct Chain2Cfg {
    static constexpr int DK = 128, KS = 4, ES = 2;
    static constexpr int NPAIR = DV / 32;          // workgroups per (sequence, head)
    static constexpr int CW = 4;                   // compute waves
    static constexpr int WAVES = CW + 1;           // and the stager
    static constexpr int XSLOT = KS * 2 * 64 * 16; // chunk-start state slots: [ks][ct], 8 KiB
    static constexpr int NX = 2;
    static constexpr int RW = DK * ES / 16;        // 16-byte units per QM row
    static constexpr int RS = (RW + 1) * 16;       // padded LDS row stride of QM (bytes)
    static constexpr int QM_UNITS = CHUNK * (RW + 1);
    static constexpr int LOADS = (QM_UNITS + 63) / 64;   // direct loads per chunk
    static constexpr int SLOT = LOADS * 1024;
    static constexpr int NSLOT = 3;
    static constexpr RecLayout RL = rec_layout(ES, DK, DV);
    static_assert(2 * LOADS <= 60, "two chunks of direct loads must fit the counter");
};

// Operands of one chunk for a compute wave (this lane's fragments).
struct Chain2Ops {
    bf16x8 pm[2][4];   // PM rows 32w + 16h2 + ln, key block ks (A operands)
    bf16x4 hc[2][2];   // Hc[32w + 16h2 + 4g .. +3][j0 + 16ct + ln]
    f32x4 gc[2];       // gamma_C[32w + 16h2 + 4g .. +3]
    bf16x4 oi[2];      // OI[16w + ln][j0 + 16ct + 4g .. +3]
};

template <int DV>
__device__ __forceinline__ void chain2_load(Chain2Ops& op, const unsigned char* r, int w, int l,
                                            int j0)
{
    using C = Chain2Cfg<DV>;
    const bf16* PM = reinterpret_cast<const bf16*>(r + C::RL.pm);
    const bf16* HC = reinterpret_cast<const bf16*>(r + C::RL.hc);
    const bf16* OI = reinterpret_cast<const bf16*>(r + C::RL.oi);
    const float* G = reinterpret_cast<const float*>(r + C::RL.g);
    const int g = l >> 4;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) op.pm[h2][ks] = load_frag(PM + frag_at<4>(2 * w + h2, ks), l);
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)   // Hc^T fragment (value slice, key block w), plane h2
            op.hc[h2][ct] = load_plane(HC + frag_at<4>((j0 >> 4) + ct, w), l, h2);
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) op.gc[h2] = load_vec<f32x4>(G + 32 * w + 16 * h2 + 4 * g);
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)   // OI fragment (token tile w, value block j0/32), plane ct
        op.oi[ct] = load_plane(OI + frag_at<DV / 32>(w, j0 >> 5), l, ct);
}

// s_waitcnt immediate: at most n vector-memory operations of this wave outstanding.
constexpr int chain2_vmcnt(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

typedef __attribute__((address_space(1))) void c2_global_void;
typedef __attribute__((address_space(3))) void c2_lds_void;

// Barrier for waves whose direct loads must stay in flight across it: only
// their own LDS accesses are waited for (the workgroup fence of
// __syncthreads() would drain every outstanding load).
__device__ __forceinline__ void chain2_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

template <int DV>
__global__ __launch_bounds__(64 * Chain2Cfg<DV>::WAVES) void prefill_chain2_kernel(
    const unsigned char* __restrict__ rec, const ChunkSrc src, const float* __restrict__ S0,
    float* __restrict__ S_final, bf16* __restrict__ o, float* __restrict__ chunk_states, int H,
    int n_pairs)
{
    using C = Chain2Cfg<DV>;
    constexpr int DK = C::DK, NPAIR = C::NPAIR;
    __shared__ __attribute__((aligned(1024))) unsigned char ring[C::NSLOT * C::SLOT];
    __shared__ __attribute__((aligned(16))) unsigned char xfer[C::NX * C::XSLOT];

    const int b = blockIdx.x;
    const int xcd = b & 7, q8 = b >> 3;
    const int grp = q8 / NPAIR, ps = q8 % NPAIR;   // ps: which 32 value columns
    const int pair = grp * 8 + xcd;
    if (pair >= n_pairs) return;
    // the sequences longest first where the table gives their order: this
    // kernel runs the chains in rounds, and short ones then fill in behind
    const int s = src.seq_order ? src.seq_order[pair / H] : pair / H, h = pair % H;
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l = tid & 63, g = l >> 4, ln = l & 15;
    const int j0 = 32 * ps;
    int c_begin, n;
    seq_chunks(src, s, c_begin, n);
    const size_t sbase = ((size_t)s * H + h) * DK * DV;
    if (n == 0) {   // empty sequence: the final state is the initial one (or zero)
        if (S_final)
            for (int x = tid; x < DK * 32; x += blockDim.x) {
                const size_t at = sbase + (size_t)(x >> 5) * DV + j0 + (x & 31);
                S_final[at] = S0 ? S0[at] : 0.f;
            }
        return;   // uniform over the workgroup
    }
    auto record = [&](int it) {
        return rec + ((size_t)(c_begin + min(it, n - 1)) * H + h) * C::RL.bytes;
    };
    auto slot = [&](int it) { return ring + (it % C::NSLOT) * C::SLOT; };
    auto xslot = [&](int it) { return reinterpret_cast<bf16*>(xfer + (it % C::NX) * C::XSLOT); };

    if (wave < C::CW) {
        // ------------------------------------------------ compute waves
        const int w = wave;
        int n_all;
        ChunkInfo first, last;
        chunk_of(src, c_begin, n_all, first);
        chunk_of(src, c_begin + n - 1, n_all, last);
        const int seq_len = CHUNK * (n - 1) + last.len;
        // S[h2][ct]: lane holds S[32w + 16h2 + 4g + i][j0 + 16ct + ln]
        f32x4 S[2][2];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
                S[h2][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
                if (S0) {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        S[h2][ct][i] = S0[sbase + (size_t)(32 * w + 16 * h2 + 4 * g + i) * DV + j0 + 16 * ct + ln];
                }
            }
        // this wave's operand step (key block w) of the chunk-start state, to LDS
        auto put = [&](int it) {
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
                bf16x8 f;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    f[i] = (bf16)S[0][ct][i];
                    f[4 + i] = (bf16)S[1][ct][i];
                }
                store_vec(xslot(it) + ((w * 2 + ct) * 64 + l) * 8, f);
            }
        };
        Chain2Ops ops[3];
        chain2_load<DV>(ops[0], record(0), w, l, j0);
        chain2_load<DV>(ops[1], record(1), w, l, j0);
        put(0);
        chain2_barrier();
        // chunk it with operand set cur; set nxt (free since chunk it - 1) takes chunk it + 2
        auto step = [&](Chain2Ops& cur, Chain2Ops& nxt, int it) {
            const bf16* xs = xslot(it);
            const bf16* qrow = reinterpret_cast<const bf16*>(slot(it) + (16 * w + ln) * C::RS) + 8 * g;
            // key block 0's operands first; each block's LDS reads are issued
            // one block ahead of its products
            bf16x8 Sf[2][2], qf[2];
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) Sf[0][ct] = load_vec<bf16x8>(xs + (ct * 64 + l) * 8);
            qf[0] = load_vec<bf16x8>(qrow);
            __builtin_amdgcn_sched_barrier(0);
            chain2_load<DV>(nxt, record(it + 2), w, l, j0);
            __builtin_amdgcn_sched_barrier(0);
            if (chunk_states) {   // the chunk-start state in fp32, [chunk][H][DK][DV]
                float* cs = chunk_states + (chunk_state_row(src, s, c_begin, it) * H + h) * DK * DV + j0 + ln;
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            __builtin_nontemporal_store(S[h2][ct][i], cs + (size_t)(32 * w + 16 * h2 + 4 * g + i) * DV + 16 * ct);
            }
            // S' = Diag(gamma_C) S + Hc + PM S;  O^T tiles of token tile w
            // (lane holds O[16w + ln][j0 + 16ct + 4g + i]) = S^T QM^T + OI^T
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        S[h2][ct][i] = S[h2][ct][i] * cur.gc[h2][i] + (float)cur.hc[h2][ct][i];
            f32x4 O[2];
#pragma unroll
            for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                for (int i = 0; i < 4; ++i) O[ct][i] = (float)cur.oi[ct][i];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const int bq = ks & 1;
                if (ks + 1 < 4) {
#pragma unroll
                    for (int ct = 0; ct < 2; ++ct)
                        Sf[bq ^ 1][ct] = load_vec<bf16x8>(xs + (((ks + 1) * 2 + ct) * 64 + l) * 8);
                    qf[bq ^ 1] = load_vec<bf16x8>(qrow + 32 * (ks + 1));
                }
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                    for (int ct = 0; ct < 2; ++ct) S[h2][ct] = mma32(cur.pm[h2][ks], Sf[bq][ct], S[h2][ct]);
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) O[ct] = mma32(Sf[bq][ct], qf[bq], O[ct]);
            }
            const int r = CHUNK * it + 16 * w + ln;   // token of the sequence
            if (r < seq_len) {
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) {
                    bf16x4 v;
#pragma unroll
                    for (int i = 0; i < 4; ++i) v[i] = (bf16)O[ct][i];
                    store_vec(o + ((size_t)(first.start + r) * H + h) * DV + j0 + 16 * ct + 4 * g, v);
                }
            }
            if (it + 1 < n) put(it + 1);
            chain2_barrier();
        };
        // whole rounds of the ring without branches, then the remaining chunks
        int it0 = 0;
        for (; it0 + 3 <= n; it0 += 3) {
            step(ops[0], ops[2], it0);
            step(ops[1], ops[0], it0 + 1);
            step(ops[2], ops[1], it0 + 2);
        }
        if (it0 < n) step(ops[0], ops[2], it0);
        if (it0 + 1 < n) step(ops[1], ops[0], it0 + 1);
        if (S_final) {
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        S_final[sbase + (size_t)(32 * w + 16 * h2 + 4 * g + i) * DV + j0 + 16 * ct + ln] = S[h2][ct][i];
        }
    } else {
        // ------------------------------------------------ stager: QM rows into the ring
        // Unit u of a chunk: QM row u / (RW + 1), 16-byte column u % (RW + 1)
        // (the padding column re-reads column 0); past the last unit, the
        // record's gamma_C (never read from the slot's tail).
        uint32_t off[C::LOADS];
#pragma unroll
        for (int k = 0; k < C::LOADS; ++k) {
            const int u = 64 * k + l;
            int x;
            if (u < C::QM_UNITS) {
                const int row = u / (C::RW + 1), col = u % (C::RW + 1);
                x = (int)C::RL.qm + row * DK * 2 + (col < C::RW ? col : 0) * 16;
            } else {
                x = (int)C::RL.g;
            }
            off[k] = (uint32_t)x;
        }
        auto issue = [&](int c) {
            const unsigned char* r = record(c);
            unsigned char* dst = slot(c);
            const unsigned char* srcp[C::LOADS];
#pragma unroll
            for (int k = 0; k < C::LOADS; ++k) srcp[k] = r + off[k];
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int k = 0; k < C::LOADS; ++k)
                __builtin_amdgcn_global_load_lds((c2_global_void*)srcp[k], (c2_lds_void*)(dst + 1024 * k), 16, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        };
        issue(0);
        issue(1);
        __builtin_amdgcn_s_waitcnt(chain2_vmcnt(C::LOADS));   // chunk 0 has landed
        chain2_barrier();
        for (int it = 0; it < n; ++it) {
            if (it + 2 < n) {
                issue(it + 2);   // its slot was last read in iteration it - 1
                __builtin_amdgcn_s_waitcnt(chain2_vmcnt(C::LOADS));   // chunk it + 1 has landed
            } else {
                __builtin_amdgcn_s_waitcnt(chain2_vmcnt(0));
            }
            chain2_barrier();
        }
    }
}

template <int DV>
static hipError_t launch_chain2_t(const void* rec, ChunkSrc src, const float* S0, float* S_final,
                                  void* o, float* chunk_states, int H, hipStream_t stream)
{
    using C = Chain2Cfg<DV>;
    const int n_pairs = src.N * H;
    const long long blocks = (long long)((n_pairs + 7) / 8) * 8 * C::NPAIR;
    hipExtLaunchKernelGGL((prefill_chain2_kernel<DV>), dim3((unsigned)blocks), dim3(64 * C::WAVES), 0,
                       stream, launch_events().start, launch_events().stop, 0, (const unsigned char*)rec, src, S0, S_final, (bf16*)o, chunk_states,
                       H, n_pairs);
    return hipGetLastError();
}

hipError_t launch_prefill_chain2(const void* rec, ChunkSrc src, const float* S0, float* S_final,
                                 void* o, float* chunk_states, int H, int dk, int dv,
                                 hipStream_t stream)
{
    if (dk == 128 && dv == 128)
        return launch_chain2_t<128>(rec, src, S0, S_final, o, chunk_states, H, stream);
    if (dk == 128 && dv == 64)
        return launch_chain2_t<64>(rec, src, S0, S_final, o, chunk_states, H, stream);
    return hipErrorInvalidValue;
}

}  // namespace kda
