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

// ---------------------------------------------------------------------------
// The chunkwise form of the same path (bf16, dk = dv = 128).  The paper notes
// (section 3) fold a run of tokens into dense products; here the run is at
// most RC = 16 tokens of one sequence.  For such a chunk with cumulative
// log-decay g (restarting at the chunk) and entering state S:
//
//   A_kk[t][t'] = beta_t sum_c k_tc k_t'c e^{g_tc - g_t'c}  (t' < t)
//   A_qk[t][t'] =        sum_c q_tc k_t'c e^{g_tc - g_t'c}  (t' <= t)
//   T = (I + A_kk)^{-1} Diag(beta),  W = T (e^g k),  U = T v
//   N = U - W S,  o = (e^g q) S + A_qk N,  S' = Diag(e^{g_C}) S + (e^{g_C - g} k)^T N
//
// (exact algebra of the recurrence, as in the chunkwise prefill; the decay
// factors e^{-g} span at most 16 tokens).  The fp32 state stays in MFMA
// accumulators: wave w of 8 owns value columns 16w .. 16w + 15, tile cb
// holding S[16cb + 4g + i][16w + (l & 15)].  The state is then touched
// once per chunk by VALU (the Diag(e^{g_C}) scaling and its bf16 operand
// copy) instead of four times per token, and the path is bound by the state's
// read and write.  Products over the chunk's tokens use the 16x16x32 MFMA
// with the upper 16 contraction slots zero.  The token data are staged by
// every thread alike (one token row, four channels), the cumulative decay
// summed across the lanes of a row; at under 80 registers per lane three
// workgroups share a CU.
constexpr int RC = 16;   // tokens per chunk

// Inclusive prefix sum over the 16 lanes of a row, in lane order (row shifts
// by 1, 2, 4 and 8; lanes before the row's start read 0).
template <int SH>
__device__ __forceinline__ float row_shr_or_0(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x110 + SH, 0xF, 0xF, false));
}
__device__ __forceinline__ float row16_scan(float x) {
    x += row_shr_or_0<1>(x);
    x += row_shr_or_0<2>(x);
    x += row_shr_or_0<4>(x);
    return x + row_shr_or_0<8>(x);
}

// Register budget: 80 per lane (six waves per SIMD, three workgroups per CU);
// the L2-normalising instance needs a few more and keeps the 128 of four.
// n_seqs > 0 (slot order): the grid walks the pool's slots, workgroup b taking
// slot b / H and head b % H, so that the states stream in address order
// whatever order the slots are given in; the workgroup finds the sequence
// holding its slot by one pass over the slot array (a slot no sequence holds
// is skipped), and the o rows of padding sequence s are zeroed by the
// workgroups of slot s mod num_slots.
template <bool NORM>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(NORM ? 4 : 6, NORM ? 4 : 6))) void recurrent_mfma_kernel(
    float* __restrict__ pool, int num_slots, const int32_t* __restrict__ slots,
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const float* __restrict__ log_alpha, const float* __restrict__ beta,
    const int32_t* __restrict__ cu, int rows, int H, int beta_logit, bf16* __restrict__ o, int n_seqs)
{
    constexpr int D = 128;
    constexpr int LK = D + 8;    // row stride of [RC][D] bf16 arrays (channels in perm32 order)
    constexpr int LT = RC + 8;   // row stride of [D][RC] and [RC][RC] bf16 arrays
    __shared__ __attribute__((aligned(16))) bf16 sW[RC * LK];   // -W
    __shared__ __attribute__((aligned(16))) bf16 sKg[RC * LK], sKi[RC * LK], sQg[RC * LK];
    __shared__ __attribute__((aligned(16))) bf16 sKgT[D * LT], sKhT[D * LT], sVT[D * LT];
    __shared__ __attribute__((aligned(16))) bf16 sT[RC * LT], sAq[RC * LT];
    __shared__ __attribute__((aligned(16))) float sBeta[RC], sGam[D];
    __shared__ float sNrm[2][8][RC];   // per-wave partial squared norms of the q and k rows

    const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    // Lane indices.  refresh() derives them anew from an opaque copy of the
    // thread index at the start of every chunk, so that the compiler does not
    // hoist the many values derived from them out of the chunk loop (held
    // across it, they would not fit the registers).
    int t, lane, g, ln, j, c4;
    auto refresh = [&]() {
        t = threadIdx.x;
        asm volatile("" : "+v"(t));
        lane = t & 63;
        g = lane >> 4;
        ln = lane & 15;
        j = 16 * w + ln;    // the lane's value column in the state tiles
        c4 = 4 * (t >> 4);  // staging: token row ln, channels c4 .. c4 + 3
    };
    refresh();

    // token range of sequence s
    auto range_of = [&](int s_, int& a, int& b) {
        if (cu) {
            a = cu[s_];
            b = cu[s_ + 1];
        } else {
            a = s_ * rows;
            b = a + rows;
        }
    };
    int seq, h, slot, t0, t1;
    if (n_seqs > 0) {   // slot order (uniform over the launch)
        __shared__ int sSeq;
        slot = blockIdx.x / H;
        h = blockIdx.x - slot * H;
        if (t == 0) sSeq = -1;
        __syncthreads();
        for (int i = t; i < n_seqs; i += 512) {
            const int si = slots[i];
            if (si == slot) {
                sSeq = i;
            } else if ((si < 0 || si >= num_slots) && i % num_slots == slot) {
                int a, b;   // padding sequence i: zero its o rows of head h
                range_of(i, a, b);
                for (int r = a; r < b; ++r)
                    for (int x = 0; x < D; x += 4)
                        *reinterpret_cast<bf16x4*>(o + ((size_t)r * H + h) * D + x) = bf16x4{};
            }
        }
        __syncthreads();
        seq = sSeq;
        if (seq < 0) return;   // no sequence holds this slot (uniform over the workgroup)
        range_of(seq, t0, t1);
    } else {
        seq = blockIdx.x / H;
        h = blockIdx.x % H;
        range_of(seq, t0, t1);
        slot = slots ? slots[seq] : seq;
        if (slot < 0 || slot >= num_slots) {   // padding sequence (uniform over the workgroup)
            for (int x = t; x < (t1 - t0) * D; x += 512)
                o[((size_t)(t0 + x / D) * H + h) * D + x % D] = (bf16)0.f;
            return;
        }
    }
    if (t1 <= t0) return;

    // A chunk's token data, loaded into registers ahead of the chunk: thread
    // (token row ln, channels c4 .. c4 + 3) holds its q, k, v and log_alpha
    // and the row's beta.  Rows past the chunk's end re-read its last row (and
    // count as zero).  Every thread loads the same kinds, so the wait for them
    // is exact on every path.
    bf16x4 qv, kv, vv;
    f32x4 lv;
    float bv;
    auto load_tokens = [&](int tb, int nt) {
        const size_t row = (size_t)(tb + min(ln, nt - 1)) * H + h;
        qv = *reinterpret_cast<const bf16x4*>(q + row * D + c4);
        kv = *reinterpret_cast<const bf16x4*>(k + row * D + c4);
        vv = *reinterpret_cast<const bf16x4*>(v + row * D + c4);
        lv = *reinterpret_cast<const f32x4*>(log_alpha + row * D + c4);
        bv = beta[row];
    };

    // The state through a buffer resource: the lane's part of each address in
    // one register, the row within a 16-row block as the immediate offset and
    // the block as the scalar offset.
    f32x4 st[8];   // st[cb]: lane holds S[16cb + 4g + i][j]
    const __amdgpu_buffer_rsrc_t srs =
        __builtin_amdgcn_make_buffer_rsrc(pool + ((size_t)slot * H + h) * D * D, (short)0, D * D * 4, 0x00020000);
    auto load_state = [&]() {
#pragma unroll
        for (int cb = 0; cb < 8; ++cb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                st[cb][i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                          srs, (4 * g * D + j + i * D) * 4, cb * 16 * D * 4, 0));
    };
    auto store_state = [&]() {
#pragma unroll
        for (int cb = 0; cb < 8; ++cb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float x = st[cb][i];   // a bit cast of a vector element in place reads element 0
                __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, x), srs,
                                                      (4 * g * D + j + i * D) * 4, cb * 16 * D * 4, 0);
            }
    };

    // operand of 4 consecutive tokens (slots 0..3) with the upper slots zero
    auto half8 = [](const bf16* p) {
        const bf16x4 a = *reinterpret_cast<const bf16x4*>(p);
        return bf16x8{a[0], a[1], a[2], a[3], (bf16)0.f, (bf16)0.f, (bf16)0.f, (bf16)0.f};
    };

    // One chunk [tb, tb + nt), its token data in the registers.
    auto chunk = [&](int tb, int nt) {
        __syncthreads();   // the previous chunk's operands are consumed
        // ---- decayed operands: thread (token row ln, channels c4 .. c4 + 3) ---------
        {
            const bool live = ln < nt;
            float qf[4], kf[4], gl[4], gc[4];
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                qf[m] = live ? (float)qv[m] : 0.f;
                kf[m] = live ? (float)kv[m] : 0.f;
                // cumulative log-decay over the chunk: the row's lanes hold tokens 0 .. 15
                gl[m] = row16_scan(live ? lv[m] : 0.f);
                gc[m] = __shfl(gl[m], (lane & 48) | 15);   // the chunk's total
            }
            if constexpr (NORM) {
                // squared norms over the row's 32 channel quads: lanes xor 16 and
                // 32 of the wave, then the 8 waves
                float sq = 0.f, sk = 0.f;
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    sq += qf[m] * qf[m];
                    sk += kf[m] * kf[m];
                }
                sq += lane_xor<16>(sq);
                sk += lane_xor<16>(sk);
                sq += lane_xor<32>(sq);
                sk += lane_xor<32>(sk);
                if (lane < RC) {
                    sNrm[0][w][lane] = sq;
                    sNrm[1][w][lane] = sk;
                }
                __syncthreads();
                float tq = 0.f, tk = 0.f;
#pragma unroll
                for (int x = 0; x < 8; ++x) {
                    tq += sNrm[0][x][ln];
                    tk += sNrm[1][x][ln];
                }
                const float iq = rsqrtf(tq + L2NORM_EPS), ik = rsqrtf(tk + L2NORM_EPS);
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    qf[m] *= iq;
                    kf[m] *= ik;
                }
            }
            bf16x4 kg, ki, qg;
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const float eg = fast_exp(gl[m]);
                kg[m] = (bf16)(kf[m] * eg);
                ki[m] = (bf16)(kf[m] * fast_exp(fminf(-gl[m], 80.f)));
                qg[m] = (bf16)(qf[m] * eg);
                const int c = c4 + m;
                sKgT[c * LT + ln] = kg[m];
                sKhT[c * LT + ln] = (bf16)(kf[m] * fast_exp(gc[m] - gl[m]));
                sVT[c * LT + ln] = live ? vv[m] : (bf16)0.f;
            }
            // channels c4 .. c4 + 3 sit together at perm_index(c4)
            const int p = ln * LK + perm_index(c4);
            *reinterpret_cast<bf16x4*>(sKg + p) = kg;
            *reinterpret_cast<bf16x4*>(sKi + p) = ki;
            *reinterpret_cast<bf16x4*>(sQg + p) = qg;
            if (ln == 0)
                *reinterpret_cast<f32x4*>(sGam + c4) =
                    f32x4{fast_exp(gc[0]), fast_exp(gc[1]), fast_exp(gc[2]), fast_exp(gc[3])};
            const float b = live ? (beta_logit ? sigmoid(bv) : bv) : 0.f;
            if (t < RC) sBeta[t] = b;
        }
        __syncthreads();
        // ---- A_kk and T (wave 0), A_qk (wave 1) ------------------------------------
        if (w < 2) {
            const bf16* A = w == 0 ? sKg : sQg;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};   // lane: [4g + i][ln]
#pragma unroll
            for (int s = 0; s < D / 32; ++s)
                acc = mma32(*reinterpret_cast<const bf16x8*>(A + ln * LK + 32 * s + 8 * g),
                            *reinterpret_cast<const bf16x8*>(sKi + ln * LK + 32 * s + 8 * g), acc);
            if (w == 0) {
                f32x4 am;
#pragma unroll
                for (int i = 0; i < 4; ++i) am[i] = 4 * g + i > ln ? sBeta[4 * g + i] * acc[i] : 0.f;
                // (I + A_kk) x = e_l by forward substitution, lane l = column l.
                // Rows from the chunk's end on hold no A_kk entries, so their
                // solution is e_l itself: the substitution stops at nt rows.
                const int nr = __builtin_amdgcn_readfirstlane(nt);
                float x[RC];
#pragma unroll
                for (int r = 0; r < RC; ++r) {
                    float a = r == ln ? 1.f : 0.f;
                    if (r < nr) {
#pragma unroll
                        for (int i = 0; i < r; ++i) a -= read_lane(am[r & 3], 16 * (r >> 2) + i) * x[i];
                    }
                    x[r] = a;
                }
                if (g == 0) {
                    const float bl = sBeta[ln];
#pragma unroll
                    for (int r = 0; r < RC; ++r) sT[r * LT + ln] = (bf16)(x[r] * bl);
                }
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    sAq[(4 * g + i) * LT + ln] = (bf16)(ln <= 4 * g + i ? acc[i] : 0.f);
            }
        }
        __syncthreads();
        // ---- W (negated, over g; wave w: key block w) and U (this wave's columns) ---------
        {
            const f32x4 a = mma32(half8(sKgT + (16 * w + ln) * LT + 4 * g), half8(sT + ln * LT + 4 * g),
                                  f32x4{0.f, 0.f, 0.f, 0.f});
            // lane: W[ln][16w + 4g + i]
            *reinterpret_cast<bf16x4*>(sW + ln * LK + perm_index(16 * w + 4 * g)) =
                bf16x4{(bf16)-a[0], (bf16)-a[1], (bf16)-a[2], (bf16)-a[3]};
        }
        // lane: [token 4g + i][j]
        f32x4 nacc = mma32(half8(sT + ln * LT + 4 * g), half8(sVT + j * LT + 4 * g), f32x4{0.f, 0.f, 0.f, 0.f});
        __syncthreads();
        // ---- N = U - W S, o = Qg S + A_qk N, S' = Diag(gamma) S + Khat^T N ---------------
        {
            f32x4 pacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                bf16x8 sf;   // perm32 slots of key rows 32s .. 32s + 31
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    sf[i] = (bf16)st[2 * s][i];
                    sf[4 + i] = (bf16)st[2 * s + 1][i];
                }
                nacc = mma32(*reinterpret_cast<const bf16x8*>(sW + ln * LK + 32 * s + 8 * g), sf, nacc);
                pacc = mma32(*reinterpret_cast<const bf16x8*>(sQg + ln * LK + 32 * s + 8 * g), sf, pacc);
            }
            const bf16x8 nb = {(bf16)nacc[0], (bf16)nacc[1], (bf16)nacc[2], (bf16)nacc[3],
                               (bf16)0.f, (bf16)0.f, (bf16)0.f, (bf16)0.f};
            pacc = mma32(half8(sAq + ln * LT + 4 * g), nb, pacc);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (4 * g + i < nt) o[((size_t)(tb + 4 * g + i) * H + h) * D + j] = (bf16)pacc[i];
#pragma unroll
            for (int cb = 0; cb < 8; ++cb) {
                const f32x4 gm = *reinterpret_cast<const f32x4*>(sGam + 16 * cb + 4 * g);
                f32x4 a = st[cb];
#pragma unroll
                for (int i = 0; i < 4; ++i) a[i] *= gm[i];
                st[cb] = mma32(half8(sKhT + (16 * cb + ln) * LT + 4 * g), nb, a);
            }
        }
    };

    // The first chunk's token data, then the state: a wave's loads complete in
    // order, so the chunk's operand work waits for its token data only, and
    // the state, first needed by the products, streams in behind it.
    load_tokens(t0, min(RC, t1 - t0));
    load_state();
    chunk(t0, min(RC, t1 - t0));
    for (int tb = t0 + RC; tb < t1; tb += RC) {
        refresh();
        load_tokens(tb, min(RC, t1 - tb));
        chunk(tb, min(RC, t1 - tb));
    }
    store_state();
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
                            bool bf16_io, unsigned flags, void* o, hipStream_t stream, int64_t T)
{
    // Chunkwise MFMA form for bf16 at d = 128 when some sequence has several
    // tokens; one token per sequence keeps the exact token step (it equals
    // the decode step).
    if (bf16_io && dk == 128 && dv == 128 && T > N) {
        // slot order where the pool is not much larger than the batch (the
        // grid walks every slot) and one pass over the slot array stays short
        const bool by_slot = slots && N <= SLOT_ORDER_MAX_SEQS && (long long)num_slots <= 2LL * N;
        const dim3 grid((unsigned)((long long)(by_slot ? num_slots : N) * H));
        const int n_seqs = by_slot ? N : 0;
        const int beta_logit = (flags & PRE_BETA_LOGIT) ? 1 : 0;
        if (flags & PRE_L2NORM_QK)
            hipLaunchKernelGGL(recurrent_mfma_kernel<true>, grid, dim3(512), 0, stream, pool, num_slots,
                               slots, (const bf16*)q, (const bf16*)k, (const bf16*)v, la, beta, cu, rows,
                               H, beta_logit, (bf16*)o, n_seqs);
        else
            hipLaunchKernelGGL(recurrent_mfma_kernel<false>, grid, dim3(512), 0, stream, pool, num_slots,
                               slots, (const bf16*)q, (const bf16*)k, (const bf16*)v, la, beta, cu, rows,
                               H, beta_logit, (bf16*)o, n_seqs);
        return hipGetLastError();
    }
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
