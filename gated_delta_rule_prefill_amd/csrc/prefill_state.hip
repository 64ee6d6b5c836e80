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
// communicate.  Two kernels implement it:
//   prefill_state_ring_kernel  (bf16 q/k/v, and fp32 with dk = 64): DK/32
//       serial waves share the chain, PM streams into their registers, the
//       other operands through an LDS ring, and two output waves form O from
//       each chunk-start state in LDS (described above the kernel);
//   prefill_state_kernel  (fp32 with dk = 128, whose ring does not fit in
//       LDS): wave 0 runs the chain, wave 1 the output of the previous chunk
//       (one chunk behind), waves 2-3 stage PM into an LDS double buffer two
//       chunks ahead and touch each record a few chunks ahead so it is in L2;
//       waves 0 and 1 load their remaining operands straight from L2 into
//       registers one chunk ahead.
// One barrier per chunk orders all hand-overs.
//
// Every product takes the state straight from its accumulator tiles: a 16x16
// tile gives lane group g rows 4g..4g+3, the slot set that the perm32 column
// order of PM and QM matches.
#include <hip/hip_ext.h>

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
    static constexpr int PM_BYTES = DK * DK * ES;       // fragment order, as in the record
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
        op.hc[t] = load_plane(HC + frag_at<DK / 32>(j0 >> 4, t >> 1), 16 * g + ln, t & 1);   // row j0 + ln
        op.gc[t] = load_vec<f32x4>(G + 16 * t + 4 * g);
    }
}

template <typename E, int DK, int DV>
__device__ __forceinline__ void load_output(OutputOps<E, DK>& op, const unsigned char* r,
                                            const ChunkInfo ci, int g, int ln, int j0)
{
    using C = StateCfg<E, DK, DV>;
    using V8 = typename Vec<E>::v8;
    using V4 = typename Vec<E>::v4;
    const E* QM = reinterpret_cast<const E*>(r + C::RL.qm);
    const E* OI = reinterpret_cast<const E*>(r + C::RL.oi);
    const int l = 16 * g + ln;
#pragma unroll
    for (int R = 0; R < 4; ++R) {
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) op.q[R][ks] = load_vec<V8>(QM + (16 * R + ln) * DK + 32 * ks + 8 * g);
        // OI[16R + ln][perm_index(j0 + 4g) ..]: plane (j0/16) mod 2 of fragment (R, j0/32)
        op.oi[R] = load_plane(OI + frag_at<DV / 32>(R, j0 >> 5), l, (j0 >> 4) & 1);
    }
    op.start = ci.start;
    op.len = ci.len;
}

// Workgroups are grouped so that the DV/16 slices of one (sequence, head)
// have block indices congruent mod 8: blocks are dispatched round-robin over
// the 8 XCDs, so the slices that read the same chunk records share one L2.
template <typename E, int DK, int DV>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void prefill_state_kernel(
    const unsigned char* __restrict__ rec, const ChunkSrc src, const float* __restrict__ S0,
    float* __restrict__ S_final, E* __restrict__ o, float* __restrict__ chunk_states, int H,
    int n_pairs)
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
    int c_begin, n;   // first chunk and chunk count of this sequence
    seq_chunks(src, s, c_begin, n);
    const size_t sbase = (size_t)pair * DK * DV;
    if (n == 0) {   // empty sequence: the final state is the initial one (or zero)
        if (S_final)
            for (int x = tid; x < DK * 16; x += blockDim.x) {
                const size_t at = sbase + (size_t)(x >> 4) * DV + j0 + (x & 15);
                S_final[at] = S0 ? S0[at] : 0.f;
            }
        return;   // uniform over the workgroup: no barrier is skipped by part of it
    }
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
        __syncthreads();

        auto step = [&](SerialOps<E, DK>& cur, SerialOps<E, DK>& nxt, int it) {
            __builtin_amdgcn_sched_barrier(0);
            // the next chunk's loads are unconditional (the last chunk reloads itself)
            load_serial<E, DK, DV>(nxt, record(min(it + 1, n - 1)), g, ln, j0);
            if (chunk_states) {   // the chunk-start state, fp32 [chunk][H][DK][DV]
                float* cs = chunk_states + (chunk_state_row(src, s, c_begin, it) * H + h) * DK * DV + j0 + ln;
#pragma unroll
                for (int t = 0; t < KT; ++t)
#pragma unroll
                    for (int i = 0; i < 4; ++i) __builtin_nontemporal_store(S[t][i], cs + (size_t)(16 * t + 4 * g + i) * DV);
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
            const E* pm = reinterpret_cast<const E*>(pmbuf + (it & 1) * C::PM_BYTES);
            V8 pf[KT][KS];
#pragma unroll
            for (int t = 0; t < KT; ++t)
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) pf[t][ks] = load_frag(pm + frag_at<KS>(t, ks), l);
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
        if (n > 0) load_output<E, DK, DV>(opA, record(0), chunk_desc(src, c_begin), g, ln, j0);
        __syncthreads();
        __syncthreads();   // iteration 0: the serial wave hands over chunk 0's start state

        auto step = [&](OutputOps<E, DK>& cur, OutputOps<E, DK>& nxt, int it) {
            __builtin_amdgcn_sched_barrier(0);
            const int nx = min(it + 1, n - 1);
            load_output<E, DK, DV>(nxt, record(nx), chunk_desc(src, c_begin + nx), g, ln, j0);
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
            f32x4* dst = reinterpret_cast<f32x4*>(pmbuf + (it & 1) * C::PM_BYTES);
#pragma unroll
            for (int i = 0; i < C::PM_PER_LANE; ++i) dst[sl + 128 * i] = pr[i];
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
// LDS-ring variant, for every configuration whose ring fits in LDS.  It runs
// the sequential chain and forms every chunk's output from the chunk-start
// state while that state is in LDS.
//
// One workgroup per (sequence, head, 16 value columns): DK/32 serial waves, a
// touch wave, a stager wave and two output waves:
//   serial waves w < DK/32  own rows 32w..32w+31 of the fp32 state tile; per
//       chunk each applies S' = Diag(gamma_C) S + Hc + PM S to its rows (8
//       MFMAs), reading the whole chunk-start state as bf16 operand slots from
//       LDS and writing its own rows' slots for the next chunk to LDS.  A
//       16x16 accumulator tile gives lane group g rows 4g..4g+3, so the two
//       tiles of rows 32w.. are exactly operand step w of the next product.
//       Their PM rows (fragment order in the record, 1 KiB per fragment) come
//       straight from the record into a register ring PM_DIST - 1 chunks
//       ahead: nothing else in the workgroup reads them, and an LDS round
//       trip would cost the CU twice the bytes;
//   output waves  form O = QM S_c + OI for the chunk whose start state is in
//       LDS: row tiles 2ow, 2ow + 1 as O^T tiles, the state slots as A, QM rows
//       (ring slot) as B, the OI fragment halves as the accumulators' start;
//   touch wave  for chains of TOUCH_MIN_CHUNKS or more touches every line
//       the chain will read TOUCH_DIST chunks ahead so that the loads hit L2
//       (plain loads, folded into a value three chunks later), and with
//       chunk_states sends the fp32 chunk-start states to memory;
//   stager wave  moves this slice's Hc^T fragments, gamma_C, QM and the
//       slice's OI planes into a four-slot LDS ring by direct global->LDS loads
//       (global_load_lds_dwordx4), two chunks ahead.
// Every wave passes one barrier per chunk.  A ring slot or state slot is
// written only after the barrier that ends the chunk which last read it.
template <typename E, int DK, int DV>
struct RingCfg {
    static constexpr int ES = sizeof(E);
    static constexpr int KS = DK / 32, KT = DK / 16, NSL = DV / 16;
    static constexpr int NSER = KS;                  // serial waves
    static constexpr int NSTG = 1;                   // stager waves
    static constexpr int NOUT = 2;                   // output waves
    static constexpr int WAVES = NSER + 1 + NSTG + NOUT;   // + the touch wave
    static constexpr int FRAG = 8 * ES;
    static constexpr int XSLOT = KS * 64 * FRAG;     // one chunk-start state (operand slots)
    // state slots: it (serial waves read), it + 1 (written), it - 1 (output waves)
    static constexpr int NX = 3;
    static constexpr int RW = DK * ES / 16;          // 16-byte units per QM row
    static constexpr int RS = (RW + 1) * 16;         // padded LDS row stride of QM (bytes)
    static constexpr int HC_UNITS = DK * ES;         // this slice's Hc^T fragments (16 rows)
    static constexpr int G_UNITS = DK / 4;
    // QM rows (padded stride RS, against LDS bank conflicts) and this slice's planes of the OI fragments (R, j0/32)
    static constexpr int QM_UNITS = CHUNK * (RW + 1);
    static constexpr int OI_PLANE_UNITS = 256 * ES / 16;   // this slice's plane of one OI fragment
    static constexpr int OI_UNITS = (CHUNK / 16) * OI_PLANE_UNITS;
    static constexpr int UNITS = HC_UNITS + G_UNITS + QM_UNITS + OI_UNITS;
    static constexpr int LOADS = (UNITS + 63) / 64;  // direct loads per chunk
    static constexpr int LOADS_W = (LOADS + NSTG - 1) / NSTG;   // per stager wave
    static constexpr int LOADS_LAST = LOADS - (NSTG - 1) * LOADS_W;   // the last stager's share
    // the reverse chain forms no output: its stager moves only the E^T
    // fragments (in Hc^T's place) and gamma_C, the first units of the list
    static constexpr int LOADS_REV = (HC_UNITS + G_UNITS + 63) / 64;
    static constexpr int SLOT = LOADS * 1024;
    static constexpr int OFF_HC = 0;
    static constexpr int OFF_G = OFF_HC + HC_UNITS * 16;
    static constexpr int OFF_QM = OFF_G + G_UNITS * 16;
    static constexpr int OFF_OI = OFF_QM + QM_UNITS * 16;
    static constexpr int OUT_RPW = CHUNK / 16 / NOUT;   // row tiles per output wave
    static constexpr int NSLOT = 4;                  // it - 1 (output waves), it, it + 1, it + 2
    static constexpr int LDS_BYTES = NSLOT * SLOT + NX * XSLOT;
    static constexpr RecLayout RL = rec_layout(ES, DK, DV);
    static constexpr int TOUCH_LINES = DK * DK * ES / 128 / NSL + 16 * DK * ES / 128 + DK * 4 / 128;
    static constexpr int TOUCH_PER_LANE = (TOUCH_LINES + 63) / 64;
    static_assert(2 * LOADS_W <= 60, "two chunks of one stager's direct loads must fit its counter");
    static_assert(LOADS_LAST > 0 && LOADS_LAST <= LOADS_W, "stager split");
    static_assert(NSTG == 1 && LOADS_REV <= LOADS_W, "the reverse chain's loads are the first stager's first ones");
};

constexpr int TOUCH_DIST = 6;   // chunks between the L2 touch and the first direct load
// Chains shorter than this skip the touches: their records are mostly
// cache-resident already (the intra kernel's grid order), and the touches'
// own misses delay the workgroup's other loads (a CU returns data in order).
constexpr int TOUCH_MIN_CHUNKS = 256;

// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wave are outstanding (lgkm and exp counters left free).
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

typedef __attribute__((address_space(1))) void global_void;
typedef __attribute__((address_space(3))) void lds_void;

// Register ring of PM fragment sets per serial wave: chunk c's loads are
// issued while chunk c - PM_DIST + 1 is processed, PM_EARLY of its 2 DK/32
// fragments before that chunk's MFMAs.
constexpr int PM_DIST = 3;
constexpr int PM_EARLY = 4;

// Workgroup barrier for waves without LDS accesses of their own.
// __syncthreads() carries a workgroup release fence, which makes a wave wait
// for every outstanding direct load (they write LDS) -- including those meant
// for later chunks.  The stager waves order their LDS writes themselves with
// an explicit vector-memory wait, so they (and the touch wave) take a bare
// s_barrier; the empty asm statements only stop the compiler from moving
// memory accesses across it.
__device__ __forceinline__ void bare_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Barrier for the serial waves: their own LDS writes complete first, while
// their PM loads stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0); vmcnt and expcnt not waited on
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// reverse: walk each sequence's chunks from the last to the first (the
// backward pass's chain over reverse-chain records; o is then NULL and no
// output is formed, and chunk_states receives the state entering each step,
// i.e. the gradient leaving each chunk, at that chunk's row).
template <typename E, int DK, int DV>
__global__ __launch_bounds__((64 * RingCfg<E, DK, DV>::WAVES)) void prefill_state_ring_kernel(
    const unsigned char* __restrict__ rec, const ChunkSrc src, const float* __restrict__ S0,
    float* __restrict__ S_final, E* __restrict__ o, float* __restrict__ chunk_states, int H,
    int n_pairs, int reverse)
{
    using C = RingCfg<E, DK, DV>;
    using V4 = typename Vec<E>::v4;
    using V8 = typename Vec<E>::v8;
    constexpr int KS = C::KS, NSL = C::NSL, NSER = C::NSER;

    __shared__ __attribute__((aligned(1024))) unsigned char ring[C::NSLOT * C::SLOT];
    __shared__ __attribute__((aligned(16))) unsigned char xfer[C::NX * C::XSLOT];
    // fp32 chunk-start states for the chunk_states output, column-major
    // [slot][16 columns][DK rows (+4 padding)]; written by the serial waves with
    // 16-byte LDS stores, sent to memory row-major by the touch wave
    __shared__ __attribute__((aligned(16))) float cst[C::NX][16][DK + 4];

    const int b = blockIdx.x;
    const int xcd = b & 7, q8 = b >> 3;
    const int grp = q8 / NSL, slice = q8 % NSL;   // slice: 16 value columns
    const int pair = grp * 8 + xcd;
    if (pair >= n_pairs) return;
    const int s = pair / H, h = pair % H;
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l = tid & 63, g = l >> 4, ln = l & 15;
    const int j0 = slice * 16;
    int c_begin, n;   // first chunk and chunk count of this sequence
    seq_chunks(src, s, c_begin, n);
    const size_t sbase = (size_t)pair * DK * DV;
    if (n == 0) {   // empty sequence: the final state is the initial one (or zero)
        if (S_final)
            for (int x = tid; x < DK * 16; x += blockDim.x) {
                const size_t at = sbase + (size_t)(x >> 4) * DV + j0 + (x & 15);
                S_final[at] = S0 ? S0[at] : 0.f;
            }
        return;   // uniform over the workgroup: no barrier is skipped by part of it
    }
    auto chunk_at = [&](int it) { return reverse ? n - 1 - it : it; };   // chunk of step it
    auto record = [&](int it) { return rec + ((size_t)(c_begin + chunk_at(it)) * H + h) * C::RL.bytes; };
    auto slot = [&](int it) { return ring + (it % C::NSLOT) * C::SLOT; };
    auto xslot = [&](int it) { return reinterpret_cast<E*>(xfer + (it % C::NX) * C::XSLOT); };

    if (wave < NSER) {
        // ------------------------------------------------ serial waves
        const int w = wave;   // row group: rows 32w .. 32w + 31
        f32x4 S[2];   // S[h2]: lane holds S[32w + 16 h2 + 4g + i][j0 + ln]
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) S[h2] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (S0) {
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    S[h2][i] = S0[sbase + (size_t)(32 * w + 16 * h2 + 4 * g + i) * DV + j0 + ln];
        }
        // chunk-start state of chunk it, this wave's operand step, to LDS (and
        // its fp32 rows to the staging the touch wave sends to chunk_states)
        auto put = [&](int it) {
            V8 f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                f[i] = from_f32<E>(S[0][i]);
                f[4 + i] = from_f32<E>(S[1][i]);
            }
            store_vec(xslot(it) + (w * 64 + l) * 8, f);
            if (chunk_states) {
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2)
                    *reinterpret_cast<f32x4*>(&cst[it % C::NX][ln][32 * w + 16 * h2 + 4 * g]) = S[h2];
            }
        };
        // PM rows 32w .. 32w + 31 of chunk c (clamped): this lane's A fragments
        // of row tiles 2w, 2w + 1, straight from the record into a register
        // ring of PM_DIST sets
        using PmSet = V8[2][KS];
        constexpr int NSET = PM_DIST;
        // fragments f0 .. f1 - 1 of a set (f: row tile 2w + (f & 1), step f >> 1)
        auto pm_load = [&](PmSet& pf, int c, int f0, int f1) {
            const E* pm = reinterpret_cast<const E*>(record(min(c, n - 1)) + C::RL.pm);
#pragma unroll
            for (int f = 0; f < 2 * KS; ++f)
                if (f >= f0 && f < f1) pf[f & 1][f >> 1] = load_frag(pm + frag_at<KS>(2 * w + (f & 1), f >> 1), l);
        };
        PmSet pfr[NSET];
#pragma unroll
        for (int u = 0; u < PM_DIST - 1; ++u) pm_load(pfr[u], u, 0, 2 * KS);
        put(0);
        lds_barrier();
        // chunk it: the MFMAs take set pf; set pn (free since chunk it - 1)
        // takes chunk it + PM_DIST - 1, its loads issued in two parts so that
        // the CU's load path never holds a whole set of all serial waves at
        // once: the first while the LDS operands of this chunk are in flight,
        // the rest after the MFMAs
        auto step = [&](PmSet& pf, PmSet& pn, int it) {
            const unsigned char* sl = slot(it);
            const E* xs = xslot(it);
            V8 Sf[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) Sf[ks] = load_vec<V8>(xs + (ks * 64 + l) * 8);
            V4 hc[2];
            f32x4 gc[2];
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                const int t = 2 * w + h2;
                hc[h2] = load_plane(reinterpret_cast<const E*>(sl + C::OFF_HC) + 512 * w, l, h2);   // Hc^T[j0 + ln][perm_index(16t + 4g) ..]
                gc[h2] = load_vec<f32x4>(reinterpret_cast<const float*>(sl + C::OFF_G) + 16 * t + 4 * g);
            }
            __builtin_amdgcn_sched_barrier(0);   // LDS reads first, then the early loads
            pm_load(pn, it + PM_DIST - 1, 0, PM_EARLY);
            __builtin_amdgcn_sched_barrier(0);
            // S' = Diag(gamma_C) S + Hc + PM S
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                for (int i = 0; i < 4; ++i) S[h2][i] = S[h2][i] * gc[h2][i] + to_f32(hc[h2][i]);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2) S[h2] = mma32(pf[h2][ks], Sf[ks], S[h2]);
            pm_load(pn, it + PM_DIST - 1, PM_EARLY, 2 * KS);
            if (it + 1 < n) put(it + 1);
            lds_barrier();
        };
        // whole rounds of the register ring without branches (so that each
        // step waits only for its own set), then the remaining chunks
        int it0 = 0;
        for (; it0 + PM_DIST <= n; it0 += PM_DIST) {
#pragma unroll
            for (int u = 0; u < NSET; ++u) step(pfr[u], pfr[(u + NSET - 1) % NSET], it0 + u);
        }
#pragma unroll
        for (int u = 0; u < NSET - 1; ++u)
            if (it0 + u < n) step(pfr[u], pfr[(u + NSET - 1) % NSET], it0 + u);
        if (S_final) {
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    S_final[sbase + (size_t)(32 * w + 16 * h2 + 4 * g + i) * DV + j0 + ln] = S[h2][i];
        }
    } else if (wave == NSER) {
        // ------------------------------------------------ touch wave
        // Plain loads whose values are folded into `sink` three chunks later;
        // unconditional (clamped chunk index) so that each load writes its own
        // registers and the compiler has no reason to wait for it early.
        // Lines touched per chunk: 1/NSL of PM (shared by the workgroups of a
        // head), this workgroup's 16 rows of Hc^T, and gamma_C.
        using TouchSet = uint32_t[C::TOUCH_PER_LANE];
        uint32_t toff[C::TOUCH_PER_LANE];
#pragma unroll
        for (int k = 0; k < C::TOUCH_PER_LANE; ++k) {
            const int u = l + 64 * k;
            constexpr int PM_LINES = DK * DK * (int)sizeof(E) / 128;
            constexpr int HC_LINES = 16 * DK * (int)sizeof(E) / 128;
            constexpr int PM_MINE = PM_LINES / NSL;
            size_t x;
            if (u < PM_MINE) x = C::RL.pm + 128 * (size_t)(slice + NSL * u);
            else if (u < PM_MINE + HC_LINES) x = C::RL.hc + (size_t)j0 * DK * sizeof(E) + 128 * (size_t)(u - PM_MINE);
            else x = C::RL.g + 128 * (size_t)((u - PM_MINE - HC_LINES) % (DK * 4 / 128));
            toff[k] = (uint32_t)x;
        }
        const bool touching = n >= TOUCH_MIN_CHUNKS;   // uniform over the workgroup
        auto touch = [&](TouchSet& tv, int c) {
            const unsigned char* r = record(c);
#pragma unroll
            for (int k = 0; k < C::TOUCH_PER_LANE; ++k)
                tv[k] = touching ? *reinterpret_cast<const uint32_t*>(r + toff[k]) : 0u;
        };
        uint32_t sink = 0;
        TouchSet tv0, tv1, tv2;
        auto fold = [&](TouchSet& tv) {
#pragma unroll
            for (int k = 0; k < C::TOUCH_PER_LANE; ++k) sink ^= tv[k];
        };
        touch(tv0, min(TOUCH_DIST - 3, n - 1));
        touch(tv1, min(TOUCH_DIST - 2, n - 1));
        touch(tv2, min(TOUCH_DIST - 1, n - 1));
        bare_barrier();
        // chunk-start state `it` (in cst since the barrier that ended chunk it - 1;
        // rewritten only after the barrier that ends chunk it) to chunk_states,
        // fp32 [chunk][H][DK][DV]: 16-byte stores of 4 columns of a row
        // (the reverse chain's are gradients for the gradient kernel, which takes
        // them as bf16 MFMA operands: they go out in bf16)
        auto send_state = [&](int it) {
            const size_t at = (chunk_state_row(src, s, c_begin, chunk_at(it)) * H + h) * DK * DV + j0;
#pragma unroll
            for (int k = 0; k < DK * 4 / 64; ++k) {
                const int u = l + 64 * k, row = u >> 2, qd = u & 3;
                const f32x4 val = {cst[it % C::NX][4 * qd][row], cst[it % C::NX][4 * qd + 1][row],
                                   cst[it % C::NX][4 * qd + 2][row], cst[it % C::NX][4 * qd + 3][row]};
                // streaming stores: the records this kernel still has to read stay cached
                if (reverse) {
                    const bf16x4 b = {(bf16)val[0], (bf16)val[1], (bf16)val[2], (bf16)val[3]};
                    __builtin_nontemporal_store(b, reinterpret_cast<bf16x4*>(reinterpret_cast<bf16*>(chunk_states) + at +
                                                                             (size_t)row * DV + 4 * qd));
                } else {
                    __builtin_nontemporal_store(val, reinterpret_cast<f32x4*>(chunk_states + at + (size_t)row * DV + 4 * qd));
                }
            }
        };
        auto step = [&](TouchSet& tv, int it) {
            fold(tv);   // issued three chunks ago
            touch(tv, min(it + TOUCH_DIST, n - 1));
            if (chunk_states) send_state(it);
            bare_barrier();
        };
        for (int it = 0; it < n; it += 3) {
            step(tv0, it);
            if (it + 1 < n) step(tv1, it + 1);
            if (it + 2 < n) step(tv2, it + 2);
        }
        fold(tv0);
        fold(tv1);
        fold(tv2);
        if (n_pairs < 0) o[0] = from_f32<E>((float)sink);   // keeps the touches; never taken
    } else if (wave >= NSER + 1 + C::NSTG) {
        // ------------------------------------------------ output waves
        // O = QM S_c + OI for the chunk whose start state the serial waves
        // handed over last: output wave ow takes row tiles 2 ow, 2 ow + 1 as
        // O^T tiles (lane: row 16R + ln, columns j0 + 4g .. +3), the state
        // slots as A operands and QM rows (ring slot) as B.
        {
            const int ow = wave - (NSER + 1 + C::NSTG);
            constexpr int RPW = C::OUT_RPW;
            int n_all;
            ChunkInfo first, last;   // token range of the sequence
            chunk_of(src, c_begin, n_all, first);
            chunk_of(src, c_begin + n - 1, n_all, last);
            const int seq_len = CHUNK * (n - 1) + last.len;
            // chunk c's output is formed while the serial waves run chunk c + 1:
            // its ring slot and state slot live until the barrier that ends
            // chunk c + 1 (NSLOT = 4, NX = 3), so these waves never hold up a
            // barrier with work of the chunk the chain is on
            auto form = [&](int c) {
                if (o == nullptr) return;   // the reverse chain forms no output
                const unsigned char* sl = slot(c);
                const E* xs = xslot(c);
                V8 Sa[KS];
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) Sa[ks] = load_vec<V8>(xs + (ks * 64 + l) * 8);
#pragma unroll
                for (int rr = 0; rr < RPW; ++rr) {
                    const int R = RPW * ow + rr;
                    // OI[16R + ln][perm_index(j0 + 4g) ..]: this slice's plane of fragment (R, j0/32)
                    const V4 oi = load_plane(reinterpret_cast<const E*>(sl + C::OFF_OI) + 256 * R, l, 0);
                    f32x4 acc = {to_f32(oi[0]), to_f32(oi[1]), to_f32(oi[2]), to_f32(oi[3])};
                    const E* qrow = reinterpret_cast<const E*>(sl + C::OFF_QM + (16 * R + ln) * C::RS) + 8 * g;
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) acc = mma32(Sa[ks], load_vec<V8>(qrow + 32 * ks), acc);
                    const int r = CHUNK * c + 16 * R + ln;   // token of the sequence
                    if (r < seq_len) {
                        V4 w;
#pragma unroll
                        for (int i = 0; i < 4; ++i) w[i] = from_f32<E>(acc[i]);
                        store_vec(o + ((size_t)(first.start + r) * H + h) * DV + j0 + 4 * g, w);
                    }
                }
            };
            bare_barrier();
            for (int it = 0; it < n; ++it) {
                if (it > 0) form(it - 1);
                bare_barrier();   // every LDS read above was consumed before its store
            }
            form(n - 1);   // its slots are not rewritten after the last barrier
        }
    } else {
        // ------------------------------------------------ stager waves: direct loads into the ring
        const int sw = wave - NSER - 1;
        const int i0 = sw * C::LOADS_W;
        const int cnt = reverse ? C::LOADS_REV : min(C::LOADS_W, C::LOADS - i0);
        // This lane's byte offset inside a record, per load.
        uint32_t off[C::LOADS_W];
#pragma unroll
        for (int k = 0; k < C::LOADS_W; ++k) {
            const int u = 64 * (i0 + k) + l;
            int x;
            if (u < C::HC_UNITS) {
                x = (int)C::RL.hc + j0 * DK * (int)sizeof(E) + 16 * u;   // the slice's fragments
            } else if (u < C::HC_UNITS + C::G_UNITS) {
                x = (int)C::RL.g + (u - C::HC_UNITS) * 16;
            } else if (u < C::HC_UNITS + C::G_UNITS + C::QM_UNITS) {
                const int v = u - (C::HC_UNITS + C::G_UNITS);
                const int row = v / (C::RW + 1), col = v % (C::RW + 1);
                x = (int)C::RL.qm + row * DK * (int)sizeof(E) + (col < C::RW ? col : 0) * 16;
            } else if (u < C::UNITS) {
                const int v = u - (C::HC_UNITS + C::G_UNITS + C::QM_UNITS);
                const int R = v / C::OI_PLANE_UNITS, k = v % C::OI_PLANE_UNITS;
                x = (int)C::RL.oi + (frag_at<DV / 32>(R, j0 >> 5) + 256 * ((j0 >> 4) & 1)) * (int)sizeof(E) + 16 * k;
            } else {
                x = (int)C::RL.g;   // past the slot's data: lands in the slot's tail padding
            }
            off[k] = (uint32_t)x;
        }
        auto issue = [&](int c) {
            const unsigned char* r = record(c);
            unsigned char* dst = slot(c) + 1024 * i0;
            // all addresses first, then the loads: each load keeps its own address
            // registers, so no address is rewritten while a queued load still reads it
            const unsigned char* src[C::LOADS_W];
#pragma unroll
            for (int k = 0; k < C::LOADS_W; ++k) src[k] = r + off[k];
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int k = 0; k < C::LOADS_W; ++k)
                if (k < cnt)
                    __builtin_amdgcn_global_load_lds((global_void*)src[k], (lds_void*)(dst + 1024 * k), 16, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        };
        // wait until only the chunk issued last is in flight (cnt loads)
        auto wait_one_in_flight = [&]() {
            if (reverse) __builtin_amdgcn_s_waitcnt(vmcnt_imm(C::LOADS_REV));
            else if (cnt == C::LOADS_W) __builtin_amdgcn_s_waitcnt(vmcnt_imm(C::LOADS_W));
            else __builtin_amdgcn_s_waitcnt(vmcnt_imm(C::LOADS_LAST));
        };
        issue(0);
        issue(min(1, n - 1));
        wait_one_in_flight();   // chunk 0 has landed
        bare_barrier();
        for (int it = 0; it < n; ++it) {
            if (it + 2 < n) {
                issue(it + 2);   // its slot was last read in iteration it - 1
                wait_one_in_flight();   // chunk it + 1 has landed
            } else {
                __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
            }
            bare_barrier();
        }
    }
}

template <typename E, int DK, int DV>
static hipError_t launch_state_ring(const void* rec, ChunkSrc src, const float* S0, float* S_final,
                                    void* o, float* chunk_states, int H, hipStream_t stream)
{
    using C = RingCfg<E, DK, DV>;
    const int n_pairs = src.N * H;
    const int groups = (n_pairs + 7) / 8;
    const long long blocks = (long long)groups * 8 * C::NSL;
    hipExtLaunchKernelGGL((prefill_state_ring_kernel<E, DK, DV>), dim3((unsigned)blocks),
                       dim3(64 * C::WAVES), 0, stream, launch_events().start, launch_events().stop, 0, (const unsigned char*)rec, src, S0, S_final,
                       (E*)o, chunk_states, H, n_pairs, 0);
    return hipGetLastError();
}

hipError_t launch_reverse_chain(const void* rec, ChunkSrc src, const float* dS_last,
                                float* dS_first, void* dS_chunks, int H, int dk, int dv,
                                hipStream_t stream)
{
    if (dk != 128 || dv != 128) return hipErrorInvalidValue;
    using C = RingCfg<bf16, 128, 128>;
    const int n_pairs = src.N * H;
    const long long blocks = (long long)((n_pairs + 7) / 8) * 8 * C::NSL;
    hipExtLaunchKernelGGL((prefill_state_ring_kernel<bf16, 128, 128>), dim3((unsigned)blocks),
                       dim3(64 * C::WAVES), 0, stream, launch_events().start, launch_events().stop, 0, (const unsigned char*)rec, src, dS_last,
                       dS_first, (bf16*)nullptr, (float*)dS_chunks, H, n_pairs, 1);
    return hipGetLastError();
}

template <typename E, int DK, int DV>
static hipError_t launch_state_t(const void* rec, ChunkSrc src, const float* S0, float* S_final,
                                 void* o, float* chunk_states, int H, hipStream_t stream)
{
    const int n_pairs = src.N * H;
    const int groups = (n_pairs + 7) / 8;
    const long long blocks = (long long)groups * 8 * (DV / 16);
    hipExtLaunchKernelGGL((prefill_state_kernel<E, DK, DV>), dim3((unsigned)blocks), dim3(256), 0,
                       stream, launch_events().start, launch_events().stop, 0, (const unsigned char*)rec, src, S0, S_final, (E*)o, chunk_states, H,
                       n_pairs);
    return hipGetLastError();
}

// Compute units of the current device (queried once per device).
static int device_cu_count()
{
    static int cached[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int v = __atomic_load_n(&cached[dev], __ATOMIC_RELAXED);
    if (v <= 0) {
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
            v = 256;
        __atomic_store_n(&cached[dev], v, __ATOMIC_RELAXED);
    }
    return v;
}

hipError_t launch_prefill_state(const void* rec, ChunkSrc src, const float* S0, float* S_final,
                                void* o, float* chunk_states, int H, int dk, int dv, bool bf16_io,
                                hipStream_t stream)
{
#define KDA_RING_CASE(E, DK_, DV_) \
    if (dk == DK_ && dv == DV_)     \
        return launch_state_ring<E, DK_, DV_>(rec, src, S0, S_final, o, chunk_states, H, stream);
#define KDA_STATE_CASE(E, DK_, DV_) \
    if (dk == DK_ && dv == DV_)     \
        return launch_state_t<E, DK_, DV_>(rec, src, S0, S_final, o, chunk_states, H, stream);
    // More one-slice chains than CUs (they hold a CU each): two slices per
    // workgroup halve the rounds.
    if (bf16_io && dk == 128 && (long long)src.N * H * (dv / 16) > device_cu_count())
        return launch_prefill_chain2(rec, src, S0, S_final, o, chunk_states, H, dk, dv, stream);
    if (uses_ring_kernel(bf16_io, dk)) {
        if (bf16_io) {
            KDA_RING_CASE(bf16, 128, 128)
            KDA_RING_CASE(bf16, 64, 64)
            KDA_RING_CASE(bf16, 128, 64)
            KDA_RING_CASE(bf16, 64, 128)
        } else {
            KDA_RING_CASE(float, 64, 64)
            KDA_RING_CASE(float, 64, 128)
        }
    } else {
        KDA_STATE_CASE(float, 128, 128)
        KDA_STATE_CASE(float, 128, 64)
    }
#undef KDA_RING_CASE
#undef KDA_STATE_CASE
    return hipErrorInvalidValue;
}

}  // namespace kda
