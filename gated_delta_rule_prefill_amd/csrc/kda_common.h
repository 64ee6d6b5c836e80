// kda_common.h -- device-side types and helpers shared by the libkda kernels
// (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kda_launch.h"

namespace kda {

typedef __bf16 bf16;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

// -- element type traits ----------------------------------------------------
// E is the storage type of q/k/v/o and of the chunk intermediates:
// __bf16 (bf16 inputs, bf16 MFMA) or float (fp32 inputs, fp32 MFMA).
template <typename E> struct Vec;
template <> struct Vec<bf16> {
    typedef bf16x2 v2;
    typedef bf16x4 v4;
    typedef bf16x8 v8;
};
template <> struct Vec<float> {
    typedef f32x2 v2;
    typedef f32x4 v4;
    typedef f32x8 v8;
};

__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(float x) { return x; }
template <typename E> __device__ __forceinline__ E from_f32(float x);
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }  // RNE
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }

// -- one 16x16 tile step over 32 contraction slots ----------------------------
// MFMA operand convention used throughout (16x16 output tiles, wave64):
//   A operand: lane l supplies row (l & 15) of A, 8 contraction slots
//              belonging to lane group g = l >> 4;
//   B operand: lane l supplies column (l & 15) of B, the same 8 slots of g;
//   D        : lane l holds D[4*g + i][l & 15], i = 0..3.
// Slot (g, m) of A is multiplied with slot (g, m) of B, so any assignment of
// the 32 contraction indices to slots works as long as A and B agree.
__device__ __forceinline__ f32x4 mma32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma32(f32x8 a, f32x8 b, f32x4 c) {
#pragma unroll
    for (int m = 0; m < 8; ++m) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[m], b[m], c, 0, 0, 0);
    return c;
}

// Storage order inside each 32-wide block of a contraction axis for matrices
// that the state kernel multiplies against register-resident accumulator
// tiles.  A 16x16 accumulator tile gives lane group g rows 4g..4g+3; two
// stacked tiles give slots {4g..4g+3, 16+4g..16+4g+3}.  Storing logical index
// x at perm32(x) puts exactly those 8 indices at 8g..8g+7, so one contiguous
// load per lane fetches the matching operand slots.
__device__ __forceinline__ int perm32(int x) {
    return 8 * ((x & 15) >> 2) + 4 * (x >> 4) + (x & 3);
}
__host__ __device__ constexpr int perm_index(int x) {  // any axis length, 32-aligned blocks
    return (x & ~31) + 8 * ((x & 15) >> 2) + 4 * ((x >> 4) & 1) + (x & 3);
}

// -- small vector helpers ---------------------------------------------------
// Vector loads and stores of up to 16 bytes use the vector type directly;
// 8 x fp32 is split in two 16-byte halves (addresses are 16-byte aligned,
// not necessarily 32).
template <typename V, typename E>
__device__ __forceinline__ V load_vec(const E* p) { return *reinterpret_cast<const V*>(p); }
template <typename V, typename E>
__device__ __forceinline__ void store_vec(E* p, V v) { *reinterpret_cast<V*>(p) = v; }
template <>
__device__ __forceinline__ f32x8 load_vec<f32x8, float>(const float* p) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p);
    const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
    return f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
template <>
__device__ __forceinline__ void store_vec<f32x8, float>(float* p, f32x8 v) {
    *reinterpret_cast<f32x4*>(p) = f32x4{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<f32x4*>(p + 4) = f32x4{v[4], v[5], v[6], v[7]};
}

// -- fragment-ordered storage ---------------------------------------------------
// A matrix that is only ever read as A operands of the 16x16x32 products
// (the chunk transition PM of the state recursion) is stored fragment by
// fragment in lane order: fragment (t, ks) -- rows 16t..16t+15, contraction
// block ks -- takes 512 elements from frag_at(t, ks); inside it lane l's 8
// slots are the 16 bytes at lane l (bf16), or two 16-byte planes of 64 lanes
// (fp32: slots 0..3, then 4..7).  Every 16-byte access of a wave then covers
// 1 KiB contiguously.
template <int KS>
__host__ __device__ constexpr int frag_at(int t, int ks) { return (t * KS + ks) * 512; }
__device__ __forceinline__ bf16x8 load_frag(const bf16* f, int l) {
    return *reinterpret_cast<const bf16x8*>(f + 8 * l);
}
__device__ __forceinline__ f32x8 load_frag(const float* f, int l) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(f + 4 * l);
    const f32x4 b = *reinterpret_cast<const f32x4*>(f + 256 + 4 * l);
    return f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
__device__ __forceinline__ void store_frag(bf16* f, int l, bf16x8 v) {
    *reinterpret_cast<bf16x8*>(f + 8 * l) = v;
}
// Planar fragments: slots 0..3 of all 64 lanes, then slots 4..7 (256
// elements each), for matrices whose readers take one half of each lane's
// slots (the fp32 fragment layout above is already planar).
__device__ __forceinline__ void store_frag_planar(bf16* f, int l, bf16x8 v) {
    *reinterpret_cast<bf16x4*>(f + 4 * l) = bf16x4{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<bf16x4*>(f + 256 + 4 * l) = bf16x4{v[4], v[5], v[6], v[7]};
}
__device__ __forceinline__ void store_frag_planar(float* f, int l, f32x8 v) {
    *reinterpret_cast<f32x4*>(f + 4 * l) = f32x4{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<f32x4*>(f + 256 + 4 * l) = f32x4{v[4], v[5], v[6], v[7]};
}
// slots 4h .. 4h + 3 of lane l from plane h of a planar fragment (h = 0, 1),
// or from a plane stored on its own (h = 0)
template <typename E>
__device__ __forceinline__ typename Vec<E>::v4 load_plane(const E* f, int l, int h) {
    return *reinterpret_cast<const typename Vec<E>::v4*>(f + 256 * h + 4 * l);
}
__device__ __forceinline__ void store_frag(float* f, int l, f32x8 v) {
    *reinterpret_cast<f32x4*>(f + 4 * l) = f32x4{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<f32x4*>(f + 256 + 4 * l) = f32x4{v[4], v[5], v[6], v[7]};
}

__device__ __forceinline__ float fast_exp(float x) { return __expf(x); }

// -- options of the layer's own input preprocessing ----------------------------
// In-call L2 normalisation of q and k (per token and head over the key
// channels, 1e-6 added to the squared norm) and beta given as a logit.
constexpr float L2NORM_EPS = 1e-6f;
__device__ __forceinline__ float sigmoid(float x) { return 1.f / (1.f + __expf(-x)); }

// Wave-wide sums of 8 values per lane at once (a transposing butterfly: 10
// lane exchanges instead of 8 x 6).  Lane l receives the total of
// a[row_of_lane(l)] over all 64 lanes, row_of_lane(l) = 4 b5 + 2 b4 + b3
// with b_i bit i of l; row_lane(r) is a lane that holds row r's total.
__host__ __device__ constexpr int row_lane(int r) {
    return (((r >> 2) & 1) << 5) | (((r >> 1) & 1) << 4) | ((r & 1) << 3);
}
// Exchanges across lane bits 4 and 5 on the VALU (CDNA4 permlane swaps).
// permlane32_swap(x, y) trades lanes 32-63 of x with lanes 0-31 of y, so x
// then holds (x low, y low) and y holds (x high, y high); their sum is, in
// the low half, x summed over lane bit 5 and, in the high half, y summed
// over it.  permlane16_swap does the same for lane bit 4 (odd rows of x
// with even rows of y).  The swapped halves are copied out of the result
// vector before the bit cast: a bit cast of a vector element in place
// compiles as element 0 here.
__device__ __forceinline__ float fold32(float x, float y) {
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x),
                                                    __builtin_bit_cast(unsigned, y), false, false);
    const unsigned r0 = r[0], r1 = r[1];
    return __builtin_bit_cast(float, r0) + __builtin_bit_cast(float, r1);
}
__device__ __forceinline__ float fold16(float x, float y) {
    const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, x),
                                                    __builtin_bit_cast(unsigned, y), false, false);
    const unsigned r0 = r[0], r1 = r[1];
    return __builtin_bit_cast(float, r0) + __builtin_bit_cast(float, r1);
}

// DPP move for patterns that read inside the lane's own row (rotations,
// mirrors, quad permutations): no lane is out of bounds, so bound_ctrl is
// free to set, which lets the compiler fold the move into the add using it.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}
// Value of lane l ^ M: quad permutations and the row rotation by 8 through
// DPP, xor 4 through a swizzle, 16 and 32 through the permlane swaps.
template <int M>
__device__ __forceinline__ float lane_xor(float x) {
    if constexpr (M == 1) return dpp<0xB1>(x);        // quad_perm 1,0,3,2
    else if constexpr (M == 2) return dpp<0x4E>(x);   // quad_perm 2,3,0,1
    else if constexpr (M == 8) return dpp<0x128>(x);  // row_ror 8
    else if constexpr (M == 4)
        return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), 0x1F | (4 << 10)));
    else {
        static_assert(M == 16 || M == 32, "lane_xor: 1, 2, 4, 8, 16 or 32");
        const unsigned v = __builtin_bit_cast(unsigned, x);
        const bool hi = __lane_id() & M;
        if constexpr (M == 16) {
            const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
            const unsigned r0 = r[0], r1 = r[1];
            return __builtin_bit_cast(float, hi ? r0 : r1);
        } else {
            const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
            const unsigned r0 = r[0], r1 = r[1];
            return __builtin_bit_cast(float, hi ? r0 : r1);
        }
    }
}
// Sum over the 8 lanes that share bits 3-5 of the lane index: the row
// half-mirror (lane i with 7 - i) and two quad permutations, all DPP.
__device__ __forceinline__ float group8_sum(float d) {
    d += dpp<0x141>(d);
    d += dpp<0x4E>(d);
    return d + dpp<0xB1>(d);
}
// Sum over the 16 lanes of a row (row rotations by 8 and 4, then the quads).
__device__ __forceinline__ float row16_sum(float d) {
    d += dpp<0x128>(d);
    d += dpp<0x124>(d);
    d += dpp<0x4E>(d);
    return d + dpp<0xB1>(d);
}

__device__ __forceinline__ float wave_sum8(const float (&a)[8], int lane) {
    const bool h3 = lane & 8;
    float b[4], c[2];
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = fold32(a[j], a[4 + j]);
#pragma unroll
    for (int j = 0; j < 2; ++j) c[j] = fold16(b[j], b[2 + j]);
    const float d = (h3 ? c[1] : c[0]) + lane_xor<8>(h3 ? c[0] : c[1]);
    return group8_sum(d);
}
// Sums of 8 values over the lanes that share bits 0-2 of the lane index
// (a transposing butterfly over lane bits 3-5: 7 exchanges).  Lane l gets
// the total of a[4 b5 + 2 b4 + b3] over its 8 lanes, b_i bit i of l.
__device__ __forceinline__ float rowgroup_sum8(const float (&a)[8], int lane) {
    const bool h3 = lane & 8;
    float b[4], c[2];
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = fold32(a[j], a[4 + j]);
#pragma unroll
    for (int j = 0; j < 2; ++j) c[j] = fold16(b[j], b[2 + j]);
    return (h3 ? c[1] : c[0]) + lane_xor<8>(h3 ? c[0] : c[1]);
}

__device__ __forceinline__ float read_lane(float x, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
}

// L2-normalise 8 rows held by a wave, CPT channels per lane (the lanes
// together hold every channel of each row).
template <int NR, int CPT>
__device__ __forceinline__ void l2_normalise_rows(float (&x)[NR][CPT], int lane) {
    static_assert(NR == 8, "rows per wave");
    float a[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        a[r] = 0.f;
#pragma unroll
        for (int e = 0; e < CPT; ++e) a[r] += x[r][e] * x[r][e];
    }
    const float inv = rsqrtf(wave_sum8(a, lane) + L2NORM_EPS);
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        const float sr = read_lane(inv, row_lane(r));
#pragma unroll
        for (int e = 0; e < CPT; ++e) x[r][e] *= sr;
    }
}

// Chunks of a batch (see ChunkSrc): from the table, or arithmetically for N
// equal sequences of src.rows tokens.
__device__ __forceinline__ int chunks_per_row(int rows) { return (rows + CHUNK - 1) / CHUNK; }

// Number of chunks and the descriptor of chunk cid (cid < gridDim.x entries of
// the table, so the table read is in bounds even past the last chunk; both
// table reads are issued together).
__device__ __forceinline__ void chunk_of(const ChunkSrc& src, int cid, int& n_chunks, ChunkInfo& ci) {
    if (src.rows >= 0) {
        const int cps = chunks_per_row(src.rows);
        n_chunks = src.N * cps;
        const int sq = cps > 0 ? cid / cps : 0, k = cps > 0 ? cid - sq * cps : 0;
        ci.seq = sq;
        ci.start = sq * src.stride + src.offset + CHUNK * k;
        ci.len = min(CHUNK, src.rows - CHUNK * k);
        ci.pad = 0;
    } else {
        n_chunks = src.seq_chunk_start[src.N];
        ci = src.chunks[cid];
    }
}

// Descriptor of chunk cid (cid must be a valid chunk).
__device__ __forceinline__ ChunkInfo chunk_desc(const ChunkSrc& src, int cid) {
    if (src.rows < 0) return src.chunks[cid];
    const int cps = chunks_per_row(src.rows);
    const int sq = cid / cps, k = cid - sq * cps;
    ChunkInfo ci;
    ci.seq = sq;
    ci.start = sq * src.stride + src.offset + CHUNK * k;
    ci.len = min(CHUNK, src.rows - CHUNK * k);
    ci.pad = 0;
    return ci;
}

// Workgroup -> (chunk, head) of the per-chunk kernels (one-dimensional grid
// of max_chunks * H workgroups).  Workgroups are dispatched round-robin over
// the 8 XCDs, and the sequential kernel reads head h's records on XCD h % 8
// (for H a multiple of 8): here too, so a head's records are written, read
// and re-read through one L2.  `descending` walks the chunks from the last:
// the intra kernel writes chunk 0 last, so the sequential kernel, which
// starts from chunk 0, finds the most recently written records first.
__device__ __forceinline__ void chunk_head_of_block(int H, bool descending, int& cid, int& h) {
    const int L = blockIdx.x, n = gridDim.x / H;
    int q;
    if ((H & 7) == 0) {
        const int hg = H >> 3;
        q = (L >> 3) / hg;
        h = (L & 7) + 8 * ((L >> 3) % hg);
    } else {
        q = L / H;
        h = L % H;
    }
    cid = descending ? n - 1 - q : q;
}

// Row of a chunk-state output for chunk `it` of sequence s in this launch
// (c_begin from seq_chunks): rows count the chunks of whole sequences.
__device__ __forceinline__ size_t chunk_state_row(const ChunkSrc& src, int s, int c_begin, int it) {
    if (src.rows < 0) return (size_t)c_begin + it;
    return (size_t)s * chunks_per_row(src.stride) + src.offset / CHUNK + it;
}

// First chunk and chunk count of sequence s.
__device__ __forceinline__ void seq_chunks(const ChunkSrc& src, int s, int& c_begin, int& n) {
    if (src.rows >= 0) {
        const int cps = chunks_per_row(src.rows);
        c_begin = s * cps;
        n = cps;
    } else {
        c_begin = src.seq_chunk_start[s];
        n = src.seq_chunk_start[s + 1] - c_begin;
    }
}

}  // namespace kda
