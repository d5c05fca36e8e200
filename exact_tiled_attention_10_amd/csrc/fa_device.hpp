// Device building blocks for the gfx950 (CDNA4) attention kernels.
//
// Matrix products use the 32x32x16 16-bit MFMA with fp32 accumulation.  Lane
// layout of v_mfma_f32_32x32x16_{bf16,f16} (checked on the device against a
// host matmul): with lane l, r = l % 32 and half = l / 32,
//   A (32 x 16, M x K): lane l holds A[r][8*half .. 8*half+7]
//   B (16 x 32, K x N): lane l holds B[8*half .. 8*half+7][r]
//   C (32 x 32)       : lane l, register i holds C[8*(i/4) + 4*half + i%4][r]
// So a C tile gives every lane one column and 16 of its rows, in four runs of
// four consecutive rows.  Feeding such a tile back as the B operand of the
// next product (the "P" of P.V and the "dS" of dS.K) is legal if the
// contraction index is renumbered consistently in both operands: for the
// k-step that covers rows 16*s .. 16*s+15 of the C tile, operand element j of
// lane half h stands for row 16*s + ROWPERM(h, j) with
//   ROWPERM(h, j) = 8*(j/4) + 4*h + j%4,
// i.e. the row order 0-3, 8-11 | 4-7, 12-15 inside each group of 16.  The
// other operand is stored in LDS with the same order (rows 4-7 and 8-11 of
// every 16 swapped), so each lane reads its eight values in one 16-byte load.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr float kNegInf = -__builtin_inff();

// C += A * B on one 32x32x16 MFMA; A and B are eight 16-bit values per lane.
template <bool BF16>
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
    if constexpr (BF16) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    } else {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(
            __builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
}

// Two fp32 values rounded to nearest even into one packed 16-bit pair
// (first value in the low half).
template <bool BF16>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    f32x2 v = {lo, hi};
    if constexpr (BF16) {
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
    } else {
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
    }
}

// One 16-bit value to fp32 (exact).
template <bool BF16>
__device__ __forceinline__ float to_f32(uint32_t bits16) {
    if constexpr (BF16) {
        return __uint_as_float(bits16 << 16);
    } else {
        return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
    }
}

// Combine a per-lane value with the lane 32 positions away (the other half
// of a wave that holds the same C-tile column).
__device__ __forceinline__ float max_halves(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
// A probability recomputed from the saved log-sum-exp, exp2(x) clamped to
// [0, 1] by the instruction's own output clamp (v_exp_f32 ... clamp, no extra
// instruction).  For every visible key x <= 0 up to rounding, so the clamp
// changes nothing but an overshoot of the last bit; for a key masked out of an
// edge tile the row's LSE does not cover its score, and without the clamp the
// exponential could overflow to +inf and meet a zero factor before the mask
// removes it.
__device__ __forceinline__ float exp2_prob(float x) {
    return __builtin_amdgcn_fmed3f(__builtin_amdgcn_exp2f(x), 0.f, 1.f);
}

// m folded with the 16 values of a C-tile register block as a chain of
// three-way maxima: one v_max3_f32 per pair, where a running max of pairwise
// maxima compiles to twice as many instructions.  The maximum of a set does
// not depend on the order it is taken in (no NaNs reach it).
__device__ __forceinline__ float max16(const f32x16& s, float m) {
#pragma unroll
    for (int i = 0; i < 16; i += 2) m = fmaxf(fmaxf(m, s[i]), s[i + 1]);
    return m;
}

// Position, inside a row of the permuted LDS layout, of the 4-element chunk
// holding rows 4*c .. 4*c+3 of a tile: chunks 1 and 2 of every 4 swap places.
__device__ __forceinline__ int perm_chunk_pos(int c) {
    const int cc = c & 3;
    const int pc = (cc == 1) ? 2 : (cc == 2) ? 1 : cc;
    return ((c >> 2) << 4) + (pc << 2);
}

// Transpose four rows of eight 16-bit values (r0..r3, element e of row k in
// half (e & 1) of word e / 2) into eight columns of four: out[e] holds
// element e of rows 0..3 in order.
__device__ __forceinline__ void transpose4x8(const u32x4& r0, const u32x4& r1, const u32x4& r2,
                                             const u32x4& r3, u32x2 out[8]) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        // v_perm_b32 selector bytes: 0-3 pick from the second operand, 4-7 from the first
        out[2 * w].x = __builtin_amdgcn_perm(r1[w], r0[w], 0x05040100u);
        out[2 * w].y = __builtin_amdgcn_perm(r3[w], r2[w], 0x05040100u);
        out[2 * w + 1].x = __builtin_amdgcn_perm(r1[w], r0[w], 0x07060302u);
        out[2 * w + 1].y = __builtin_amdgcn_perm(r3[w], r2[w], 0x07060302u);
    }
}

// ---------------------------------------------------------------------------
// Row-major LDS tiles filled by direct global -> LDS loads.
//
// A tile holds ROWS rows of D 16-bit values, unpadded.  The 16-byte chunk c of
// row r sits at slot c ^ swz(r): for 16 chunks per row the swizzle maps row
// bits (r % 4, (r / 4) % 4) to chunk bits (hi, lo), so the 16 consecutive rows
// an MFMA operand read (ds_read_b128, lane row r32, chunk 2 ks + half) touches
// land in 16 distinct slots, and the 8 rows x 4 chunks of a transposing read
// spread over all 16 slots (two lanes per bank word, the minimum for 512 B).
// ---------------------------------------------------------------------------
template <int CPR>
__device__ __forceinline__ int swz(int row) {
    // 32 chunks (512-byte rows): the same 4-bit permutation as for 16, on
    // the chunk's low bits (its high bit is kept)
    if constexpr (CPR == 16 || CPR == 32) return ((row & 3) << 2) | ((row >> 2) & 3);
    else return ((row & 3) << 1) | ((row >> 2) & 1);
}

// Direct loads go through a buffer resource (wave-uniform base address in
// scalar registers, a 32-bit byte offset per lane), not global_load_lds: the
// compiler takes an outstanding global_load_lds as a flat access that may
// also touch LDS, and while one is in flight it turns every LDS wait into a
// wait for all outstanding LDS reads, so operand reads issued ahead of their
// MFMAs would be waited for at once.  The buffer form leaves those waits
// exact.  Raw addressing (stride 0), no range limit (num_records at its
// maximum), 32-bit data format (a zero format would read zeros).
using rsrc_t = __amdgpu_buffer_rsrc_t;
__device__ __forceinline__ rsrc_t buffer_of(const void* base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, -1, 0x00020000);
}
// One direct load: each lane moves 16 bytes from src + byte_off to
// lds_dst + 16 * lane (lds_dst must be the same for the whole wave).
__device__ __forceinline__ void dma16(rsrc_t src, uint32_t byte_off, void* lds_dst) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (__attribute__((address_space(3))) void*)lds_dst, 16, byte_off,
                                             0, 0, 0);
}
// Same with 4 bytes per lane (256 B per instruction).
__device__ __forceinline__ void dma4(rsrc_t src, uint32_t byte_off, void* lds_dst) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (__attribute__((address_space(3))) void*)lds_dst, 4, byte_off,
                                             0, 0, 0);
}

// s_waitcnt with only vmcnt constrained (expcnt and lgkmcnt left at their
// maxima): vector memory operations, direct LDS loads included, still in
// flight <= N.  The 6-bit count is split over bits 3:0 and 15:14.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt immediate");
    __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// Workgroup barrier that waits only for this wave's LDS reads and writes
// (lgkmcnt(0)), not for its direct global -> LDS loads still in flight: the
// fence __syncthreads() carries counts those loads as LDS writes and would
// wait for all of them (vmcnt(0)), so a kernel that keeps tile loads in
// flight across barriers waits for them explicitly (wait_vmcnt) before the
// barrier that publishes the tile.  The empty asm statements keep the
// compiler from moving memory operations across the barrier.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt, expcnt at their maxima
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Per-lane offsets (in 16-bit elements inside the tile) of the transposing
// reads that build the A operand "X^T" of a 32x32x16 MFMA from a row-major
// tile X (rows = contraction index, columns = M index).  In every 16-lane
// group, lane 4r+c of ds_read_b64_tr_b16 receives element c of the 8-byte rows
// addressed by lanes r, r+4, r+8, r+12.  Lane j of group g therefore points at
// row 8*inst + 4*(g/2) + j/4 of the 16-row k-step and at columns
// 32*mb + 16*(g%2) + 4*(j%4) .. +3; the receiver's element 4*inst + j/4 is row
// ROWPERM(g/2, 4*inst + j/4) of the step, the order the B operand taken from an
// MFMA C tile uses.  off[inst][mb] for M blocks mb of 32 columns.
template <int D, int MB>
__device__ __forceinline__ void tr_offsets(int lane, int off[2][MB]) {
    constexpr int CPR = D / 8;
    const int g = lane >> 4, j = lane & 15;
#pragma unroll
    for (int inst = 0; inst < 2; ++inst) {
        const int rr = 8 * inst + 4 * (g >> 1) + (j >> 2);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const int col = 32 * mb + 16 * (g & 1) + 4 * (j & 3);
            off[inst][mb] = rr * D + (((col >> 3) ^ swz<CPR>(rr)) * 8) + (col & 7);
        }
    }
}

// The A operand X^T for k-step `ks` (rows 16 ks .. 16 ks + 15) and M block mb.
template <int D, int MB>
__device__ __forceinline__ u32x4 read_tr(const uint16_t* tile, int ks, int mb, const int off[2][MB]) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tile + ks * 16 * D + off[0][mb]));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tile + ks * 16 * D + off[1][mb]));
    const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
    return u32x4{l2.x, l2.y, h2.x, h2.y};
}

// ---------------------------------------------------------------------------
// Dropout keep decisions.
//
// Element (sequence b, query head h, query row i, key j) is kept iff byte
// (j mod 4) of word (i mod 4) of the Philox4x32-10 block at counter
// (j / 4, i / 4, h, b), keyed by the 64-bit seed, is below the threshold T.
// Philox4x32-10 is the counter-based generator of Salmon, Moraes, Dror and
// Shaw ("Parallel random numbers: as easy as 1, 2, 3", SC 2011): ten rounds
// of two 32 x 32 -> 64-bit products, the key advanced by two Weyl constants
// between rounds.
//
// In either MFMA C layout a lane holds one row (or column) of a 32 x 32 block
// and four runs of four consecutive columns (or rows), and the four lanes of a
// quad (consecutive lanes, same half) share the 4 x 4 sub-blocks of those
// runs.  So each lane draws one block (its run = its index in the quad) and the
// quad exchanges words (quad_transpose) to give every lane the words of its
// own row in all four runs.
// ---------------------------------------------------------------------------
__device__ __forceinline__ u32x4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                               uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r > 0) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
        const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
        c1 = (uint32_t)p1;
        c3 = (uint32_t)p0;
        c0 = n0;
        c2 = n2;
    }
    return u32x4{c0, c1, c2, c3};
}

// One round of quad_transpose: lane t receives, from lane (t + R) mod 4, that
// lane's word t, and stores it as out[(t + R) mod 4].
template <int R>
__device__ __forceinline__ void quad_round(const u32x4& w, u32x4& out, int t) {
    // quad_perm control: lane k of the quad reads lane (k + R) mod 4
    constexpr int kPerm = ((0 + R) & 3) | (((1 + R) & 3) << 2) | (((2 + R) & 3) << 4) | (((3 + R) & 3) << 6);
    const int si = (t - R) & 3;  // the word lane (t - R) mod 4 wants from this lane
    const uint32_t x = si == 0 ? w[0] : si == 1 ? w[1] : si == 2 ? w[2] : w[3];
    const uint32_t y = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kPerm, 0xF, 0xF, false);
    const int di = (t + R) & 3;
    out[0] = di == 0 ? y : out[0];
    out[1] = di == 1 ? y : out[1];
    out[2] = di == 2 ? y : out[2];
    out[3] = di == 3 ? y : out[3];
}

// Lane t of every quad holds words w[0..3]; returns, for each g, word t of the
// quad's lane g (a 4 x 4 transpose across the quad).
__device__ __forceinline__ u32x4 quad_transpose(u32x4 w) {
    const int t = threadIdx.x & 3;
    u32x4 out = w;  // out[t] = w[t] already; the other three come from the rounds
    quad_round<1>(w, out, t);
    quad_round<2>(w, out, t);
    quad_round<3>(w, out, t);
    return out;
}

// 4 x 4 byte transpose inside a lane: byte e of out[k] = byte k of w[e].
__device__ __forceinline__ u32x4 byte_transpose(u32x4 w) {
    // v_perm_b32 selector bytes: 0-3 pick from the second operand, 4-7 from the first
    const uint32_t a = __builtin_amdgcn_perm(w[1], w[0], 0x05010400u);  // w0b0 w1b0 w0b1 w1b1
    const uint32_t b = __builtin_amdgcn_perm(w[1], w[0], 0x07030602u);  // w0b2 w1b2 w0b3 w1b3
    const uint32_t c = __builtin_amdgcn_perm(w[3], w[2], 0x05010400u);  // w2b0 w3b0 w2b1 w3b1
    const uint32_t d = __builtin_amdgcn_perm(w[3], w[2], 0x07030602u);  // w2b2 w3b2 w2b3 w3b3
    return u32x4{__builtin_amdgcn_perm(c, a, 0x05040100u), __builtin_amdgcn_perm(c, a, 0x07060302u),
                 __builtin_amdgcn_perm(d, b, 0x05040100u), __builtin_amdgcn_perm(d, b, 0x07060302u)};
}

// Byte e of a word, compared with the keep threshold.
__device__ __forceinline__ bool keep_byte(uint32_t w, int e, uint32_t thresh) {
    return ((w >> (8 * e)) & 0xFFu) < thresh;
}

// Geometry of one (batch, head) problem slice: packed (cu_seqlens), fixed
// length, or fixed layout with fewer valid rows (used_q / used_k: padded
// batches, lengths clamped to the layout).
#ifndef FA_XCD_GROUPS
#define FA_XCD_GROUPS 1
#endif
// Column of this workgroup in a grid (columns, rows[, z]) dispatched row after
// row.  The GPU hands workgroup i to XCD i % 8 and, inside the XCD, to its four
// shader engines in a fixed rotation by i / 8 (read back from the hardware id
// register).  When 8 divides the column count n and n / 8 is even, a column's
// engine slot repeats every row or every other row: with 32 columns, columns
// 8 s .. 8 s + 7 land in slot s on every row, and when some columns have no
// work (the shorter sequences of a packed batch, past their end) the same
// engines idle row after row while the others queue the real workgroups.
// Shifting the columns by 8 per row then moves each column one slot further
// per row and keeps it on its XCD (its L2 keeps serving it).  For other n the
// slot already advances with the row, and the columns are left in place.
__device__ __forceinline__ int rotated_column() {
    const unsigned n = gridDim.x;
    const unsigned shift = (n % 8u == 0u && (n / 8u) % 2u == 0u) ? 8u : 0u;
    return (int)((blockIdx.x + shift * blockIdx.y) % n);
}

// (batch, query head) of workgroup column x in a grid over batch * heads.
// The GPU hands workgroups to its 8 XCDs (each with its own L2) in turn, so
// columns x and x + 8 run on the same XCD.  When the g = heads / kv_heads
// query heads reading one kv head can all share an XCD (g > 1 and the
// batch * kv_heads groups a multiple of 8), group G goes to XCD G % 8 and
// its heads to columns G % 8 + 8 ((G / 8) g + r), r = 0 .. g-1: the group's
// K and V are then fetched into one L2.  Otherwise x = b * heads + h.  A
// bijection either way.
__device__ __forceinline__ void xcd_head(int x, int batch, int heads, int kv_heads, int& b, int& h) {
    const int g = heads / kv_heads, groups = batch * kv_heads;
    if (FA_XCD_GROUPS && g > 1 && (groups & 7) == 0) {
        const int xcd = x & 7, p = x >> 3;
        const int grp = (p / g) * 8 + xcd;
        b = grp / kv_heads;
        h = (grp % kv_heads) * g + p % g;
    } else {
        b = x / heads;
        h = x % heads;
    }
}

struct Seq {
    int64_t q_start, k_start;  // first row of the sequence in the tensor
    int len_q, len_k;          // valid rows
    int off;                   // len_k - len_q: bottom-right alignment
};

__device__ __forceinline__ Seq seq_of(int b, const int32_t* cu_q, const int32_t* cu_k, const int32_t* used_q,
                                      const int32_t* used_k, int seqlen_q, int seqlen_k) {
    Seq s;
    if (cu_q) {
        const int q0 = cu_q[b], q1 = cu_q[b + 1], k0 = cu_k[b], k1 = cu_k[b + 1];
        s.q_start = q0; s.k_start = k0; s.len_q = q1 - q0; s.len_k = k1 - k0;
    } else {
        s.q_start = (int64_t)b * seqlen_q; s.k_start = (int64_t)b * seqlen_k;
        s.len_q = used_q ? min(max(used_q[b], 0), seqlen_q) : seqlen_q;
        s.len_k = used_k ? min(max(used_k[b], 0), seqlen_k) : seqlen_k;
    }
    s.off = s.len_k - s.len_q;
    return s;
}

// Mask parameters: key j visible for query i iff j < len_k and
// lo(i) <= j <= hi(i), lo(i) = i + off - left (left >= 0), hi(i) = i + off
// (causal) or i + off + right (right >= 0).
struct Mask {
    int causal, left, right;
    __device__ __forceinline__ int hi_of(int i, const Seq& s) const {
        int hi = s.len_k - 1;
        if (causal) hi = min(hi, i + s.off);
        if (right >= 0) hi = min(hi, i + s.off + right);
        return hi;
    }
    __device__ __forceinline__ int lo_of(int i, const Seq& s) const {
        return left >= 0 ? max(0, i + s.off - left) : 0;
    }
};

}  // namespace fa
