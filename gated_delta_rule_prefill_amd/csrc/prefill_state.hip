// prefill_state.hip -- sequential inter-chunk pass of the chunkwise KDA prefill.
//
// Only the fixed dk x dv state crosses chunk boundaries (Kimi Linear paper
// notes, section 3).  The intra kernel has folded each chunk into its
// transition and read-out, so with entry state S each chunk in order applies
//
//   O  = QM S + OI                              (inter- plus intra-chunk output)
//   S' = Diag(gamma_C) S + PM S + Hc            (state carried to the next chunk)
//
// One workgroup per (sequence, head, 16 value columns): the columns of S evolve
// independently, so a head's state is split over DV/16 workgroups that never
// communicate.  Roles inside the workgroup:
//   wave 0     the serial chain: it keeps the fp32 state tile (DK x 16) in MFMA
//              accumulator registers for the whole sequence, hands each
//              chunk-start state to wave 1 through LDS, and applies S';
//   wave 1     the output of the previous chunk (one chunk behind wave 0);
//   waves 2-3  stage PM into an LDS double buffer, two chunks ahead, and
//              touch each record a few chunks ahead so it is in L2.
// Waves 0 and 1 load their remaining operands straight from L2 into registers
// one chunk ahead (two register sets).  Every wave stays well under the 63
// vector-memory operations a wave may have in flight, so the loads for the
// next chunk never stall the current one, and one barrier per chunk orders
// all hand-overs.
//
// Every product takes the state straight from its accumulator tiles: a 16x16
// tile gives lane group g rows 4g..4g+3, the slot set that the perm32 column
// order of PM and QM matches.
#include "kda_common.h"

namespace kda {

constexpr int PREFETCH_DIST = 4;   // chunks between the L2 touch and the register load

template <typename E, int DK, int DV>
struct StateCfg {
    static constexpr int ES = sizeof(E);
    static constexpr int KS = DK / 32;   // contraction steps over key channels
    static constexpr int KT = DK / 16;   // accumulator tiles of S
    static constexpr int NSL = DV / 16;  // value slices per head
    static constexpr int FRAG = 8 * ES;  // bytes of one operand fragment per lane
    static constexpr int XSLOT = KS * 64 * FRAG;        // one chunk-start state hand-over
    static constexpr int PM_RS = DK * ES + 16;          // padded LDS row stride of PM
    static constexpr int PM_BYTES = DK * PM_RS;
    static constexpr int PM_UNITS = DK * DK * ES / 16;
    static constexpr int STAGERS = 2;                   // waves 2 and 3
    static constexpr int PM_PER_LANE = PM_UNITS / (64 * STAGERS);
    static constexpr RecLayout RL = rec_layout(ES, DK, DV);
    static constexpr int LINES = (int)(RL.bytes / 128);
};

// Operands of one chunk for the serial wave (this lane's fragments).
template <typename E, int DK>
struct SerialOps {
    typename Vec<E>::v4 hc[DK / 16];   // Hc^T[j0 + ln][16t + 4g .. +3] (perm32 slots)
    f32x4 gc[DK / 16];                 // gamma_C[16t + 4g .. +3]
};

// Operands of one chunk for the output wave.
template <typename E, int DK>
struct OutputOps {
    typename Vec<E>::v8 q[4][DK / 32];   // QM rows 16R + ln, slots of step ks
    typename Vec<E>::v4 oi[4];           // OI[16R + ln][j0 + 4g .. +3] (perm32 slots)
    int start, len;
};

template <typename E, int DK, int DV>
__device__ __forceinline__ void load_serial(SerialOps<E, DK>& op, const unsigned char* r, int g,
                                            int ln, int j0)
{
    using C = StateCfg<E, DK, DV>;
    using V4 = typename Vec<E>::v4;
    const E* HC = reinterpret_cast<const E*>(r + C::RL.hc);
    const float* G = reinterpret_cast<const float*>(r + C::RL.g);
#pragma unroll
    for (int t = 0; t < C::KT; ++t) {
        op.hc[t] = load_vec<V4>(HC + (j0 + ln) * DK + perm_index(16 * t + 4 * g));
        op.gc[t] = load_vec<f32x4>(G + 16 * t + 4 * g);
    }
}

template <typename E, int DK, int DV>
__device__ __forceinline__ void load_output(OutputOps<E, DK>& op, const unsigned char* r,
                                            const ChunkInfo* ci, int g, int ln, int j0)
{
    using C = StateCfg<E, DK, DV>;
    using V8 = typename Vec<E>::v8;
    using V4 = typename Vec<E>::v4;
    const E* QM = reinterpret_cast<const E*>(r + C::RL.qm);
    const E* OI = reinterpret_cast<const E*>(r + C::RL.oi);
#pragma unroll
    for (int R = 0; R < 4; ++R) {
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) op.q[R][ks] = load_vec<V8>(QM + (16 * R + ln) * DK + 32 * ks + 8 * g);
        op.oi[R] = load_vec<V4>(OI + (16 * R + ln) * DV + perm_index(j0 + 4 * g));
    }
    op.start = ci->start;
    op.len = ci->len;
}

// Workgroups are grouped so that the DV/16 slices of one (sequence, head)
// have block indices congruent mod 8: blocks are dispatched round-robin over
// the 8 XCDs, so the slices that read the same chunk records share one L2.
template <typename E, int DK, int DV>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void prefill_state_kernel(
    const unsigned char* __restrict__ rec, const int32_t* __restrict__ seq_chunk_start,
    const ChunkInfo* __restrict__ chunks, const float* __restrict__ S0,
    float* __restrict__ S_final, E* __restrict__ o, int H, int n_pairs)
{
    using C = StateCfg<E, DK, DV>;
    using V4 = typename Vec<E>::v4;
    using V8 = typename Vec<E>::v8;
    constexpr int KS = C::KS, KT = C::KT, NSL = C::NSL, ES = C::ES;

    __shared__ __attribute__((aligned(16))) unsigned char xfer[2 * C::XSLOT];
    __shared__ __attribute__((aligned(16))) unsigned char pmbuf[2 * C::PM_BYTES];

    const int b = blockIdx.x;
    const int xcd = b & 7, q8 = b >> 3;
    const int grp = q8 / NSL, slice = q8 % NSL;
    const int pair = grp * 8 + xcd;
    if (pair >= n_pairs) return;
    const int s = pair / H, h = pair % H;
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l = tid & 63, g = l >> 4, ln = l & 15;
    const int j0 = slice * 16;
    const int c_begin = seq_chunk_start[s];
    const int n = seq_chunk_start[s + 1] - c_begin;   // chunks of this sequence
    const size_t sbase = (size_t)pair * DK * DV;
    auto record = [&](int it) { return rec + ((size_t)(c_begin + it) * H + h) * C::RL.bytes; };
    auto xslot = [&](int it) { return reinterpret_cast<E*>(xfer + (it & 1) * C::XSLOT); };

    // Barrier schedule (every wave executes n + 2 barriers): one after the
    // prologue, then one closing each of n + 1 iterations; the serial wave
    // works on chunk `it` in iteration it, the output wave on chunk it - 1.
    if (wave == 0) {
        // ------------------------------------------------ serial wave
        // S tile t: lane holds S[16t + 4g + i][j0 + ln], i = 0..3
        f32x4 S[KT];
#pragma unroll
        for (int t = 0; t < KT; ++t) S[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (S0) {
#pragma unroll
            for (int t = 0; t < KT; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    S[t][i] = S0[sbase + (size_t)(16 * t + 4 * g + i) * DV + j0 + ln];
        }
        SerialOps<E, DK> opA, opB;
        if (n > 0) load_serial<E, DK, DV>(opA, record(0), g, ln, j0);
        const unsigned char* pm_lane = pmbuf + ln * C::PM_RS + 8 * g * ES;
        __syncthreads();

        auto step = [&](SerialOps<E, DK>& cur, SerialOps<E, DK>& nxt, int it) {
            __builtin_amdgcn_sched_barrier(0);
            // the next chunk's loads are unconditional (the last chunk reloads itself)
            load_serial<E, DK, DV>(nxt, record(min(it + 1, n - 1)), g, ln, j0);
            // chunk-start state as MFMA operand slots {32ks+4g..+3, 32ks+16+4g..+3}
            V8 Sf[KS];
            E* xs = xslot(it);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    Sf[ks][i] = from_f32<E>(S[2 * ks][i]);
                    Sf[ks][4 + i] = from_f32<E>(S[2 * ks + 1][i]);
                }
                store_vec(xs + (ks * 64 + l) * 8, Sf[ks]);
            }
            const unsigned char* pm = pm_lane + (it & 1) * C::PM_BYTES;
            V8 pf[KT][KS];
#pragma unroll
            for (int t = 0; t < KT; ++t)
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    pf[t][ks] = load_vec<V8>(reinterpret_cast<const E*>(pm + 16 * t * C::PM_RS + 32 * ks * ES));
            // S' = Diag(gamma_C) S + Hc + PM S
#pragma unroll
            for (int t = 0; t < KT; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) S[t][i] = S[t][i] * cur.gc[t][i] + to_f32(cur.hc[t][i]);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int t = 0; t < KT; ++t) S[t] = mma32(pf[t][ks], Sf[ks], S[t]);
            __syncthreads();
            __builtin_amdgcn_sched_barrier(0);
        };
        for (int it = 0; it < n; it += 2) {
            step(opA, opB, it);
            if (it + 1 < n) step(opB, opA, it + 1);
        }
        __syncthreads();   // iteration n: only the output wave works

        if (S_final) {
#pragma unroll
            for (int t = 0; t < KT; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    S_final[sbase + (size_t)(16 * t + 4 * g + i) * DV + j0 + ln] = S[t][i];
        }
    } else if (wave == 1) {
        // ------------------------------------------------ output wave (one chunk behind)
        OutputOps<E, DK> opA, opB;
        if (n > 0) load_output<E, DK, DV>(opA, record(0), chunks + c_begin, g, ln, j0);
        __syncthreads();
        __syncthreads();   // iteration 0: the serial wave hands over chunk 0's start state

        auto step = [&](OutputOps<E, DK>& cur, OutputOps<E, DK>& nxt, int it) {
            __builtin_amdgcn_sched_barrier(0);
            const int nx = min(it + 1, n - 1);
            load_output<E, DK, DV>(nxt, record(nx), chunks + c_begin + nx, g, ln, j0);
            const E* xs = xslot(it);
            V8 Sf[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) Sf[ks] = load_vec<V8>(xs + (ks * 64 + l) * 8);
            // O^T tile R: lane holds O[16R + ln][j0 + 4g + i];  O = QM S + OI
            f32x4 O[4];
#pragma unroll
            for (int R = 0; R < 4; ++R)
#pragma unroll
                for (int i = 0; i < 4; ++i) O[R][i] = to_f32(cur.oi[R][i]);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int R = 0; R < 4; ++R) O[R] = mma32(Sf[ks], cur.q[R][ks], O[R]);
#pragma unroll
            for (int R = 0; R < 4; ++R) {
                const int r = 16 * R + ln;
                if (r < cur.len) {
                    V4 w;
#pragma unroll
                    for (int i = 0; i < 4; ++i) w[i] = from_f32<E>(O[R][i]);
                    store_vec(o + ((size_t)(cur.start + r) * H + h) * DV + j0 + 4 * g, w);
                }
            }
            __syncthreads();
            __builtin_amdgcn_sched_barrier(0);
        };
        for (int it = 0; it < n; it += 2) {
            step(opA, opB, it);
            if (it + 1 < n) step(opB, opA, it + 1);
        }
    } else {
        // ------------------------------------------------ PM stagers / L2 touch
        // PM of chunk c sits in pmbuf[c & 1] from the barrier that ends
        // chunk c-1 on; each stager lane holds chunk c+1 in registers and
        // commits it while chunk c is processed.
        const int sl = tid - 128;   // stager lane 0..127
        f32x4 pr[C::PM_PER_LANE];
        auto pload = [&](int it) {
            const f32x4* src = reinterpret_cast<const f32x4*>(record(it) + C::RL.pm);
#pragma unroll
            for (int i = 0; i < C::PM_PER_LANE; ++i) pr[i] = src[sl + 128 * i];
        };
        auto pcommit = [&](int it) {
            unsigned char* dst = pmbuf + (it & 1) * C::PM_BYTES;
            constexpr int UPR = DK * ES / 16;   // 16-byte units per row
#pragma unroll
            for (int i = 0; i < C::PM_PER_LANE; ++i) {
                const int x = sl + 128 * i;
                *reinterpret_cast<f32x4*>(dst + (x / UPR) * C::PM_RS + 16 * (x % UPR)) = pr[i];
            }
        };
        if (n > 0) {
            pload(0);
            pcommit(0);
            pload(min(1, n - 1));
        }
        __syncthreads();
        uint32_t sink = 0;
        for (int it = 0; it <= n; ++it) {
            const int pf = it + PREFETCH_DIST;
            if (pf < n) {
                const unsigned char* r = record(pf);
                for (int line = slice + NSL * sl; line < C::LINES; line += NSL * 128)
                    sink ^= *reinterpret_cast<const uint32_t*>(r + 128 * line);
            }
            if (it + 1 < n) {
                pcommit(it + 1);                     // buffer freed by the previous barrier
                pload(min(it + 2, n - 1));
            }
            __syncthreads();
        }
        if (n_pairs < 0) o[0] = from_f32<E>((float)sink);   // keeps the touches alive; never taken
    }
}

// ---------------------------------------------------------------------------
// LDS-ring variant.  Same roles and barrier schedule as above, but the operands
// of the serial chain (PM, this slice's Hc^T rows and gamma_C) reach LDS by
// direct global->LDS loads (global_load_lds_dwordx4: no registers, no commit
// step) into a ring of three slots, two chunks ahead of their use:
//   wave 0  serial chain (reads PM, Hc, gamma_C of chunk it from slot it % 3)
//   wave 1  output one chunk behind; QM and OI come straight from global
//           memory into registers two chunks ahead (three register sets)
//   wave 2  the direct loads of chunk it + 2, then waits for chunk it + 1
//   wave 3  touches every line of chunk it + TOUCH_DIST so that the loads of
//           the other waves hit L2.  It is the only wave with loads whose
//           latency nobody waits for: a wave's vector-memory counter completes
//           in order, so touches issued by a loading wave would make that
//           wave's next wait cover them.
// A slot is written only after the barrier that ends the chunk which last
// read it, so every LDS hand-over is ordered by the one barrier per chunk.
template <typename E, int DK, int DV>
struct RingCfg {
    static constexpr int ES = sizeof(E);
    static constexpr int KS = DK / 32, KT = DK / 16, NSL = DV / 16;
    static constexpr int FRAG = 8 * ES;
    static constexpr int XSLOT = KS * 64 * FRAG;
    static constexpr int RW = DK * ES / 16;          // 16-byte units per PM / Hc^T row
    static constexpr int RS = (RW + 1) * 16;         // padded LDS row stride (bytes)
    static constexpr int PM_UNITS = DK * (RW + 1);
    static constexpr int HC_UNITS = 16 * (RW + 1);
    static constexpr int G_UNITS = DK / 4;
    static constexpr int UNITS = PM_UNITS + HC_UNITS + G_UNITS;
    static constexpr int LOADS = (UNITS + 63) / 64;  // direct loads per chunk (one wave)
    static constexpr int SLOT = LOADS * 1024;
    static constexpr int OFF_HC = PM_UNITS * 16;
    static constexpr int OFF_G = OFF_HC + HC_UNITS * 16;
    static constexpr int NSLOT = 3;
    static constexpr int LDS_BYTES = NSLOT * SLOT + 2 * XSLOT + 256;
    static constexpr RecLayout RL = rec_layout(ES, DK, DV);
    static constexpr int LINES = (int)(RL.bytes / 128);
    static constexpr int TOUCH_PER_LANE = (LINES + 64 * NSL - 1) / (64 * NSL);
    static_assert(LOADS <= 56, "direct loads of one chunk must fit the vector-memory counter");
};

constexpr int TOUCH_DIST = 5;   // chunks between the L2 touch and the first direct load

// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wave are outstanding (lgkm and exp counters left free).
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

typedef __attribute__((address_space(1))) void global_void;
typedef __attribute__((address_space(3))) void lds_void;

// Workgroup barrier for the waves that only issue direct global->LDS loads.
// __syncthreads() carries a workgroup release fence, which makes the wave wait
// for every outstanding direct load (they write LDS) -- including those meant
// for later chunks.  These waves order their LDS writes themselves with an
// explicit vector-memory wait, so they take a bare s_barrier; the empty asm
// statements only stop the compiler from moving memory accesses across it.
__device__ __forceinline__ void bare_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

template <typename E, int DK, int DV>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void prefill_state_ring_kernel(
    const unsigned char* __restrict__ rec, const int32_t* __restrict__ seq_chunk_start,
    const ChunkInfo* __restrict__ chunks, const float* __restrict__ S0,
    float* __restrict__ S_final, E* __restrict__ o, int H, int n_pairs)
{
    using C = RingCfg<E, DK, DV>;
    using V4 = typename Vec<E>::v4;
    using V8 = typename Vec<E>::v8;
    constexpr int KS = C::KS, KT = C::KT, NSL = C::NSL;

    __shared__ __attribute__((aligned(1024))) unsigned char ring[C::NSLOT * C::SLOT];
    __shared__ __attribute__((aligned(16))) unsigned char xfer[2 * C::XSLOT];
    __shared__ __attribute__((aligned(16))) unsigned char dump[256];   // touch destination, never read

    const int b = blockIdx.x;
    const int xcd = b & 7, q8 = b >> 3;
    const int grp = q8 / NSL, slice = q8 % NSL;
    const int pair = grp * 8 + xcd;
    if (pair >= n_pairs) return;
    const int s = pair / H, h = pair % H;
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l = tid & 63, g = l >> 4, ln = l & 15;
    const int j0 = slice * 16;
    const int c_begin = seq_chunk_start[s];
    const int n = seq_chunk_start[s + 1] - c_begin;   // chunks of this sequence
    const size_t sbase = (size_t)pair * DK * DV;
    auto record = [&](int it) { return rec + ((size_t)(c_begin + it) * H + h) * C::RL.bytes; };
    auto slot = [&](int it) { return ring + (it % C::NSLOT) * C::SLOT; };
    auto xslot = [&](int it) { return reinterpret_cast<E*>(xfer + (it & 1) * C::XSLOT); };

    if (wave == 0) {
        // ------------------------------------------------ serial wave
        f32x4 S[KT];   // tile t: lane holds S[16t + 4g + i][j0 + ln]
#pragma unroll
        for (int t = 0; t < KT; ++t) S[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (S0) {
#pragma unroll
            for (int t = 0; t < KT; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    S[t][i] = S0[sbase + (size_t)(16 * t + 4 * g + i) * DV + j0 + ln];
        }
        __syncthreads();
        for (int it = 0; it < n; ++it) {
            __builtin_amdgcn_sched_barrier(0);
            const unsigned char* sl = slot(it);
            const unsigned char* pm = sl + ln * C::RS + 8 * g * sizeof(E);
            V8 pf[KT][KS];
#pragma unroll
            for (int t = 0; t < KT; ++t)
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    pf[t][ks] = load_vec<V8>(reinterpret_cast<const E*>(pm + 16 * t * C::RS + 32 * ks * sizeof(E)));
            V4 hc[KT];
            f32x4 gc[KT];
#pragma unroll
            for (int t = 0; t < KT; ++t) {
                hc[t] = load_vec<V4>(reinterpret_cast<const E*>(sl + C::OFF_HC + ln * C::RS) + perm_index(16 * t + 4 * g));
                gc[t] = load_vec<f32x4>(reinterpret_cast<const float*>(sl + C::OFF_G) + 16 * t + 4 * g);
            }
            // chunk-start state as MFMA operand slots {32ks+4g..+3, 32ks+16+4g..+3}
            V8 Sf[KS];
            E* xs = xslot(it);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    Sf[ks][i] = from_f32<E>(S[2 * ks][i]);
                    Sf[ks][4 + i] = from_f32<E>(S[2 * ks + 1][i]);
                }
                store_vec(xs + (ks * 64 + l) * 8, Sf[ks]);
            }
            // S' = Diag(gamma_C) S + Hc + PM S
#pragma unroll
            for (int t = 0; t < KT; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) S[t][i] = S[t][i] * gc[t][i] + to_f32(hc[t][i]);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int t = 0; t < KT; ++t) S[t] = mma32(pf[t][ks], Sf[ks], S[t]);
            __syncthreads();
        }
        __syncthreads();   // iteration n: only the output wave works
        if (S_final) {
#pragma unroll
            for (int t = 0; t < KT; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    S_final[sbase + (size_t)(16 * t + 4 * g + i) * DV + j0 + ln] = S[t][i];
        }
    } else if (wave == 1) {
        // ------------------------------------------------ output wave (one chunk behind)
        OutputOps<E, DK> op0, op1, op2;
        if (n > 0) load_output<E, DK, DV>(op0, record(0), chunks + c_begin, g, ln, j0);
        __syncthreads();
        // iteration it: load chunk it + 1 into set (it + 1) % 3, output chunk it - 1
        auto step = [&](OutputOps<E, DK>& cur, OutputOps<E, DK>& nxt, int it) {
            __builtin_amdgcn_sched_barrier(0);
            const int nx = min(it + 1, n - 1);
            load_output<E, DK, DV>(nxt, record(nx), chunks + c_begin + nx, g, ln, j0);
            if (it > 0) {
                const E* xs = xslot(it - 1);
                V8 Sf[KS];
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) Sf[ks] = load_vec<V8>(xs + (ks * 64 + l) * 8);
                f32x4 O[4];   // O^T tile R: lane holds O[16R + ln][j0 + 4g + i];  O = QM S + OI
#pragma unroll
                for (int R = 0; R < 4; ++R)
#pragma unroll
                    for (int i = 0; i < 4; ++i) O[R][i] = to_f32(cur.oi[R][i]);
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                    for (int R = 0; R < 4; ++R) O[R] = mma32(Sf[ks], cur.q[R][ks], O[R]);
#pragma unroll
                for (int R = 0; R < 4; ++R) {
                    const int r = 16 * R + ln;
                    if (r < cur.len) {
                        V4 w;
#pragma unroll
                        for (int i = 0; i < 4; ++i) w[i] = from_f32<E>(O[R][i]);
                        store_vec(o + ((size_t)(cur.start + r) * H + h) * DV + j0 + 4 * g, w);
                    }
                }
            }
            __syncthreads();
        };
        // sets rotate: chunk c lives in set c % 3; iteration it outputs chunk it - 1
        for (int it = 0; it <= n; it += 3) {
            step(op2, op1, it);                         // outputs chunk it - 1 (set 2), loads it + 1
            if (it + 1 <= n) step(op0, op2, it + 1);    // outputs chunk it (set 0), loads it + 2
            if (it + 2 <= n) step(op1, op0, it + 2);    // outputs chunk it + 1 (set 1), loads it + 3
        }
    } else if (wave == 2) {
        // ------------------------------------------------ direct loads into the ring
        int off[C::LOADS];   // this lane's byte offset inside a record, per load
#pragma unroll
        for (int i = 0; i < C::LOADS; ++i) {
            const int u = 64 * i + l;
            int x;
            if (u < C::PM_UNITS) {
                const int row = u / (C::RW + 1), col = u % (C::RW + 1);
                x = (int)C::RL.pm + row * DK * (int)sizeof(E) + (col < C::RW ? col : 0) * 16;
            } else if (u < C::PM_UNITS + C::HC_UNITS) {
                const int v = u - C::PM_UNITS;
                const int row = v / (C::RW + 1), col = v % (C::RW + 1);
                x = (int)C::RL.hc + (j0 + row) * DK * (int)sizeof(E) + (col < C::RW ? col : 0) * 16;
            } else if (u < C::UNITS) {
                x = (int)C::RL.g + (u - C::PM_UNITS - C::HC_UNITS) * 16;
            } else {
                x = (int)C::RL.g;   // past the slot's data: lands in the slot's tail padding
            }
            off[i] = x;
        }
        auto issue = [&](int c) {
            const unsigned char* r = record(c);
            unsigned char* dst = slot(c);
#pragma unroll
            for (int i = 0; i < C::LOADS; ++i)
                __builtin_amdgcn_global_load_lds((global_void*)(r + off[i]), (lds_void*)(dst + 1024 * i),
                                                 16, 0, 0);
        };
        if (n > 0) {
            issue(0);
            issue(min(1, n - 1));
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(C::LOADS));   // chunk 0 has landed
        }
        bare_barrier();
        for (int it = 0; it <= n; ++it) {
            if (it + 2 < n) {
                issue(it + 2);   // its slot was last read in iteration it - 1
                __builtin_amdgcn_s_waitcnt(vmcnt_imm(C::LOADS));   // chunk it + 1 has landed
            } else {
                __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
            }
            bare_barrier();
        }
    } else {
        // ------------------------------------------------ L2 touches
        auto touch = [&](int c) {
            const unsigned char* r = record(c);
#pragma unroll
            for (int k = 0; k < C::TOUCH_PER_LANE; ++k) {
                const int line = slice + NSL * (l + 64 * k);
                if (line < C::LINES)
                    __builtin_amdgcn_global_load_lds((global_void*)(r + 128 * line), (lds_void*)dump, 4, 0, 0);
            }
        };
        for (int c = 2; c < min(TOUCH_DIST, n); ++c) touch(c);
        bare_barrier();
        for (int it = 0; it <= n; ++it) {
            if (it + TOUCH_DIST < n) touch(it + TOUCH_DIST);
            bare_barrier();
        }
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));   // no load may land after the workgroup ends
    }
}

template <typename E, int DK, int DV>
static hipError_t launch_state_ring_t(const void* rec, const int32_t* seq_chunk_start,
                                      const ChunkInfo* chunks, const float* S0, float* S_final,
                                      void* o, int N, int H, hipStream_t stream)
{
    const int n_pairs = N * H;
    const int groups = (n_pairs + 7) / 8;
    const long long blocks = (long long)groups * 8 * (DV / 16);
    hipLaunchKernelGGL((prefill_state_ring_kernel<E, DK, DV>), dim3((unsigned)blocks), dim3(256), 0,
                       stream, (const unsigned char*)rec, seq_chunk_start, chunks, S0, S_final,
                       (E*)o, H, n_pairs);
    return hipGetLastError();
}

template <typename E, int DK, int DV>
static hipError_t launch_state_t(const void* rec, const int32_t* seq_chunk_start,
                                 const ChunkInfo* chunks, const float* S0, float* S_final,
                                 void* o, int N, int H, hipStream_t stream)
{
    const int n_pairs = N * H;
    const int groups = (n_pairs + 7) / 8;
    const long long blocks = (long long)groups * 8 * (DV / 16);
    hipLaunchKernelGGL((prefill_state_kernel<E, DK, DV>), dim3((unsigned)blocks), dim3(256), 0,
                       stream, (const unsigned char*)rec, seq_chunk_start, chunks, S0, S_final,
                       (E*)o, H, n_pairs);
    return hipGetLastError();
}

hipError_t launch_prefill_state(const void* rec, const int32_t* seq_chunk_start,
                                const ChunkInfo* chunks, const float* S0, float* S_final,
                                void* o, int N, int H, int dk, int dv, bool bf16_io,
                                hipStream_t stream)
{
#define KDA_RING_CASE(E, DK_, DV_) \
    if (dk == DK_ && dv == DV_)     \
        return launch_state_ring_t<E, DK_, DV_>(rec, seq_chunk_start, chunks, S0, S_final, o, N, H, stream);
#define KDA_STATE_CASE(E, DK_, DV_) \
    if (dk == DK_ && dv == DV_)     \
        return launch_state_t<E, DK_, DV_>(rec, seq_chunk_start, chunks, S0, S_final, o, N, H, stream);
    // The ring needs three slots of (PM + 16 rows of Hc^T + gamma_C) in LDS; with
    // fp32 operands and dk = 128 they do not fit, and the register-staged kernel runs.
    if (bf16_io) {
        KDA_RING_CASE(bf16, 128, 128)
        KDA_RING_CASE(bf16, 64, 64)
        KDA_RING_CASE(bf16, 128, 64)
        KDA_RING_CASE(bf16, 64, 128)
    } else {
        KDA_STATE_CASE(float, 128, 128)
        KDA_RING_CASE(float, 64, 64)
        KDA_STATE_CASE(float, 128, 64)
        KDA_RING_CASE(float, 64, 128)
    }
#undef KDA_RING_CASE
#undef KDA_STATE_CASE
    return hipErrorInvalidValue;
}

}  // namespace kda
