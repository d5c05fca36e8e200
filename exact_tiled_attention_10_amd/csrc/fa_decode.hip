// Decode: exact attention of a short block of new query tokens over a long
// key/value cache (the KV-cache entry of the FlashAttention-2 overview page,
// lshu.cn/news/55956, section 3.3), split over the keys and merged through
// the online-softmax statistics (same page, section 2.2).
//
// The work is bound by reading the cache once, so the kernel is organised for
// memory-level parallelism rather than matrix-core rate:
//   * the g query heads sharing a kv head and the Nq new tokens are packed
//     into blocks of 32 rows (row r = (head r / Nq, token r % Nq)), so a
//     cache byte is read once per kv head (per 32 such rows), not once per
//     query head;
//   * a segment is one (sequence b, row block).  The visible 32-key steps of
//     all segments, laid end to end, are divided evenly over groups of
//     kv_heads waves, whatever the sequence lengths; wave hk of a group
//     takes kv head hk.  The waves of a group read neighbouring pieces of
//     the same cache rows at the same time (kept in step by their equal
//     work), which keeps DRAM pages open.  A group's range may span the end
//     of one segment and the start of the next; each wave writes one partial
//     result (O normalised, LSE) per piece.  Piece (group j, segment s) of
//     kv head hk goes to slot (j + s) * kv_heads + hk: groups and segments
//     both advance along the same axis, so no two pieces share a slot;
//   * inside a piece the loads of K and V run kDecAhead steps (one at width 256) ahead into
//     registers (coalesced 16-byte loads; the register file is far larger
//     than LDS, so many bytes are in flight per CU); at its turn a step is
//     written to the wave's own LDS tiles, from which the matrix-core
//     operands are read (V^T by transposing reads).  LDS operations of one
//     wave execute in order, so no barrier is needed;
//   * per step: S^T = K Q^T on the matrix cores, the online softmax per query
//     column (lazy rescale, as in the forward kernel), O^T += V^T P^T;
//   * a second kernel merges, for every output row, the pieces of its
//     segment: LSE = log sum_p e^{LSE_p}, O = sum_p e^{LSE_p - LSE} O_p.
// Head dimension as in the forward: tiles D = 64 or 128 wide run any head_dim
// dh that is a multiple of 8 up to D (q zero past dh, cache loads repeat the
// row's last valid chunk past dh, columns past dh not stored).
// Masking, alignment and empty-row conventions are those of the forward
// (bottom-right causal alignment, inclusive windows, O = 0 and LSE = -inf
// for a row without visible keys).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {

namespace {

constexpr float kDecLazyLog2 = 8.0f;
constexpr int kDecBK = 32;    // keys per step
constexpr int kDecAhead = 3;  // steps whose loads are in flight

template <int D>
struct DecCfg {
    static constexpr int CPR = D / 8;                  // 16-byte chunks per cache row
    static constexpr int tileElems = kDecBK * D;       // one K or V tile
    static constexpr int kLd = tileElems * 2 / 1024;   // 16-byte loads per lane per tile
    static constexpr int kRowsPerLd = 1024 / (2 * D);  // cache rows per wave load
    // steps in flight: at width 256 one step's K and V already take 128
    // registers per lane
    static constexpr int kAhead = D > 128 ? 1 : kDecAhead;
};

// Valid keys of sequence b.
__device__ __forceinline__ int dec_len(const DecArgs& a, int b) {
    const int len = a.cache_lens ? a.cache_lens[b] : a.seqlen_k;
    return min(max(len, 0), a.seqlen_k);
}

__device__ __forceinline__ Seq dec_seq(const DecArgs& a, int b, int len) {
    Seq s;
    s.q_start = (int64_t)b * a.seqlen_q;
    s.k_start = (int64_t)b * a.seqlen_k;
    s.len_q = a.seqlen_q;
    s.len_k = len;
    s.off = len - a.seqlen_q;
    return s;
}

// Steps a segment of sequence b walks: from the 32-key step holding the first
// key any new token sees to the one holding the last (tokens 0 and Nq-1 bound
// the range, the visible interval moving right with the token).
__device__ __forceinline__ void dec_steps(const DecArgs& a, int b, int& st_lo, int& n) {
    const Seq s = dec_seq(a, b, dec_len(a, b));
    const Mask mk{a.causal, a.left, a.right};
    const int lo = mk.lo_of(0, s), hi = mk.hi_of(a.seqlen_q - 1, s);
    st_lo = lo / kDecBK;
    n = lo <= hi ? hi / kDecBK + 1 - st_lo : 0;
}

// Even division of the T steps of the step axis over G groups: the first R
// groups take Q + 1 steps, the others Q (Q = T / G, R = T % G).  T < 2^31 is
// guaranteed by the host.
struct DecPart {
    int T, G, Q, R;
    __device__ __forceinline__ DecPart(int T_, int G_) : T(T_), G(G_), Q(T_ / G_), R(T_ % G_) {}
    __device__ __forceinline__ int start(int j) const { return j * Q + min(j, R); }
    __device__ __forceinline__ bool empty(int j) const { return Q == 0 && j >= R; }
    // group holding position pos (0 <= pos < T)
    __device__ __forceinline__ int group_of(int pos) const {
        const int big = R * (Q + 1);
        return pos < big ? pos / (Q + 1) : R + (pos - big) / Q;
    }
};

// Inclusive prefix sum over the wave's lanes.
__device__ __forceinline__ int64_t wave_scan(int64_t x, int lane) {
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int64_t y = __shfl_up(x, d, 64);
        x += lane >= d ? y : 0;
    }
    return x;
}

template <bool BF16, int D>
__global__ __launch_bounds__(64) void decode_split_kernel(DecArgs a) {
    using C = DecCfg<D>;
    constexpr int KS = D / 16, DB = D / 32;
    __shared__ __attribute__((aligned(16))) uint16_t kt[C::tileElems];
    __shared__ __attribute__((aligned(16))) uint16_t vt[C::tileElems];

    const int lane = threadIdx.x;
    const int r32 = lane & 31, half = lane >> 5;
    const int grp = blockIdx.x / a.kv_heads, hk = blockIdx.x % a.kv_heads;
    const int G = a.waves / a.kv_heads;  // groups
    const int HR = a.row_blocks;          // segments per sequence

    // ---- this wave's range of the step axis -----------------------------------
    // Sum of steps over the sequences, then (second pass) the sequence holding
    // the range's first step.  The first wave also records the prefix sums of
    // the per-sequence step counts for the merge kernel.
    int n_first = 0;  // first 64 sequences: kept for the second pass
    {
        int st_lo;
        if (lane < a.batch) dec_steps(a, lane, st_lo, n_first);
    }
    int64_t total = n_first;
    for (int c0 = 64; c0 < a.batch; c0 += 64) {
        int st_lo = 0, n = 0;
        if (c0 + lane < a.batch) dec_steps(a, c0 + lane, st_lo, n);
        total += n;
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) total += __shfl_xor(total, d, 64);
    const DecPart part((int)(total * HR), G);
    const int pos0 = part.start(grp), pos1 = part.start(grp + 1);
    int b = -1;
    int seq_base = 0;  // step-axis position of sequence b's first segment
    {
        int64_t carry = 0;
        for (int c0 = 0; c0 < a.batch; c0 += 64) {
            const int bb = c0 + lane;
            int st_lo = 0, n = n_first;
            if (c0 > 0 && bb < a.batch) dec_steps(a, bb, st_lo, n);
            const int64_t incl = carry + wave_scan(n, lane), excl = incl - n;
            if (blockIdx.x == 0 && bb < a.batch) a.prefix[bb] = excl;
            const bool here = bb < a.batch && n > 0 && excl * HR <= pos0 && pos0 < incl * HR;
            const uint64_t m = __builtin_amdgcn_ballot_w64(here);
            if (b < 0 && m) {
                const int src = __builtin_ctzll(m);
                b = c0 + src;
                seq_base = (int)(__shfl(excl, src, 64) * HR);
            }
            carry = __shfl(incl, 63, 64);
        }
        if (blockIdx.x == 0 && lane == 0) a.prefix[a.batch] = carry;
    }
    if (pos0 >= pos1) return;  // empty range (more groups than steps)

    // ---- per-lane constants ------------------------------------------------------
    const int g = a.heads / a.kv_heads;
    const int nq = a.seqlen_q;
    const int rows = g * nq;
    const Mask mk{a.causal, a.left, a.right};
    const int dh = a.head_dim;  // multiple of 8, at most D
    const int kv_stride = a.kv_heads * dh;
    const float c = a.scale_log2;
    // load i of a tile: lane reads chunk lane % CPR of row i * kRowsPerLd + lane / CPR
    // and later writes it to that row's swizzled slot in LDS
    const int ld_r = lane / C::CPR, ld_c = lane % C::CPR;
    const int ld_cg = min(ld_c, dh / 8 - 1);  // chunk read from the global row
    int st_off[C::kLd];
#pragma unroll
    for (int i = 0; i < C::kLd; ++i) {
        const int row = i * C::kRowsPerLd + ld_r;
        st_off[i] = row * D + ((ld_c ^ swz<C::CPR>(row)) * 8);
    }
    int k_rd[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) k_rd[ks] = r32 * D + (((2 * ks + half) ^ swz<C::CPR>(r32)) * 8);
    int v_rd[2][DB];
    tr_offsets<D, DB>(lane, v_rd);

    // ---- pieces -------------------------------------------------------------------
    int st_lo, n;
    dec_steps(a, b, st_lo, n);
    int pos = pos0;
    int seg = (pos - seq_base) / n;  // segment (row block) inside sequence b
    int off = (pos - seq_base) % n;  // first step inside it
    while (true) {
        const int cnt = min(n - off, pos1 - pos);
        const int rb = seg;
        const int64_t slot = ((int64_t)grp + (int64_t)b * HR + seg) * a.kv_heads + hk;

        const int len_k = dec_len(a, b);
        const Seq s = dec_seq(a, b, len_k);
        // this lane's row: query head hq, token t
        const int rr = rb * 32 + r32;
        const bool live = rr < rows;
        const int t = live ? rr % nq : 0;
        const int hq = hk * g + (live ? rr / nq : 0);
        const int lo_q = mk.lo_of(t, s), hi_q = live ? mk.hi_of(t, s) : -1;
        // no row of the block needs a mask inside [full_lo, full_hi] (uniform)
        const int full_lo = mk.lo_of(nq - 1, s), full_hi = mk.hi_of(0, s);

        u32x4 qf[KS];
        {
            const uint16_t* qrow = (const uint16_t*)a.q + ((s.q_start + t) * a.heads + hq) * dh;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                qf[ks] = live && ks * 16 + 8 * half < dh ? *(const u32x4*)(qrow + ks * 16 + 8 * half)
                                                         : u32x4{0, 0, 0, 0};
        }
        const uint16_t* kbase = (const uint16_t*)a.kc + (s.k_start * a.kv_heads + hk) * dh;
        const uint16_t* vbase = (const uint16_t*)a.vc + (s.k_start * a.kv_heads + hk) * dh;

        f32x16 acc[DB];
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[db] = f32x16{0};
        float m_run = kNegInf, l_part = 0.f;

        // registers of the steps in flight
        u32x4 kr[C::kAhead][C::kLd], vr[C::kAhead][C::kLd];
        auto load = [&](int st, u32x4 (&kx)[C::kLd], u32x4 (&vx)[C::kLd]) {
            const int key0 = st * kDecBK;
#pragma unroll
            for (int i = 0; i < C::kLd; ++i) {
                // rows past the end (the look-ahead of the last steps) re-read the last row
                const int row = min(key0 + i * C::kRowsPerLd + ld_r, len_k - 1);
                const int64_t o = (int64_t)row * kv_stride + ld_cg * 8;
                kx[i] = *(const u32x4*)(kbase + o);
                vx[i] = *(const u32x4*)(vbase + o);
            }
        };
        auto stage = [&](const u32x4 (&kx)[C::kLd], const u32x4 (&vx)[C::kLd]) {
#pragma unroll
            for (int i = 0; i < C::kLd; ++i) {
                *(u32x4*)(kt + st_off[i]) = kx[i];
                *(u32x4*)(vt + st_off[i]) = vx[i];
            }
        };
        auto compute = [&](int st) {
            const int key0 = st * kDecBK;
            f32x16 sacc = f32x16{0};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) sacc = mfma32<BF16>(*(const u32x4*)(kt + k_rd[ks]), qf[ks], sacc);
            if (!(key0 >= full_lo && key0 + kDecBK - 1 <= full_hi)) {  // uniform: edge steps only
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int key = key0 + 8 * (i / 4) + 4 * half + (i % 4);
                    sacc[i] = (key < lo_q || key > hi_q) ? kNegInf : sacc[i];
                }
            }
            float mx = max_halves(max16(sacc, kNegInf));
            const bool up = (mx > m_run) & ((m_run == kNegInf) | ((mx - m_run) * c > kDecLazyLog2));
            if (__builtin_amdgcn_ballot_w64(up)) {
                const float alpha = !up ? 1.f : (m_run == kNegInf ? 0.f : fast_exp2((m_run - mx) * c));
                m_run = up ? mx : m_run;
                l_part *= alpha;
#pragma unroll
                for (int db = 0; db < DB; ++db) acc[db] *= alpha;
            }
            const float mc = m_run == kNegInf ? 0.f : m_run * c;
            uint32_t pk[8];
            float lsum = 0.f;
#pragma unroll
            for (int i = 0; i < 16; i += 2) {
                const float p0 = fast_exp2(__builtin_fmaf(sacc[i], c, -mc));
                const float p1 = fast_exp2(__builtin_fmaf(sacc[i + 1], c, -mc));
                lsum += p0 + p1;
                pk[i / 2] = pack2<BF16>(p0, p1);
            }
            l_part += lsum;
#pragma unroll
            for (int hs = 0; hs < 2; ++hs) {
                const u32x4 pb = u32x4{pk[4 * hs], pk[4 * hs + 1], pk[4 * hs + 2], pk[4 * hs + 3]};
#pragma unroll
                for (int db = 0; db < DB; ++db)
                    acc[db] = mfma32<BF16>(read_tr<D, DB>(vt, hs, db, v_rd), pb, acc[db]);
            }
        };

        const int sa = st_lo + off, se = sa + cnt;
#pragma unroll
        for (int j = 0; j < C::kAhead; ++j) load(sa + j, kr[j], vr[j]);
        // Whole groups of C::kAhead steps (each step's registers fixed, one
        // exit), then the last < C::kAhead steps, which load nothing more.
        int st = sa;
        const int groups = cnt / C::kAhead;
        for (int it = 0; it < groups; ++it, st += C::kAhead) {
#pragma unroll
            for (int j = 0; j < C::kAhead; ++j) {
                stage(kr[j], vr[j]);
                load(st + j + C::kAhead, kr[j], vr[j]);
                compute(st + j);
            }
        }
#pragma unroll
        for (int j = 0; j < C::kAhead - 1; ++j) {
            if (st + j < se) {
                stage(kr[j], vr[j]);
                compute(st + j);
            }
        }

        // partial O (normalised, fp32) and LSE of this piece, live rows only
        const float l = sum_halves(l_part);
        if (live) {
            const int64_t prow = slot * 32 + r32;
            const float inv = l > 0.f ? 1.f / l : 0.f;
            float* orow = a.ws_o + prow * D;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int gq = 0; gq < 4; ++gq) {
                    float4 v;
                    v.x = acc[db][4 * gq] * inv;
                    v.y = acc[db][4 * gq + 1] * inv;
                    v.z = acc[db][4 * gq + 2] * inv;
                    v.w = acc[db][4 * gq + 3] * inv;
                    *(float4*)(orow + db * 32 + 8 * gq + 4 * half) = v;
                }
            if (half == 0) a.ws_lse[prow] = l > 0.f ? m_run * a.scale + logf(l) : kNegInf;
        }

        pos += cnt;
        if (pos >= pos1) break;
        // next segment with steps: the next row block, else the next
        // sequence that has any (one exists: pos < T)
        off = 0;
        if (++seg == HR) {
            seg = 0;
            do {
                ++b;
                dec_steps(a, b, st_lo, n);
            } while (n == 0);
        }
    }
    // loads issued past a piece's end have landed before the wave ends
    wait_vmcnt<0>();
}

// One workgroup of D threads per (batch, query head, token): merge the pieces
// of the row's segment.  Thread d merges column d; the pieces are taken in
// batches of kMergeBatch whose loads (LSE, broadcast, and O) are all issued
// before any is used, so a typical row costs one round trip to memory after
// the prefix sums.
constexpr int kMergeBatch = 16;

template <bool BF16, int D>
__global__ __launch_bounds__(D) void decode_combine_kernel(DecArgs a) {
    const int row = blockIdx.x;  // ((b * heads) + hq) * nq + t, below 2^31 (host check)
    const int nq = a.seqlen_q;
    const int d = threadIdx.x;
    const int t = row % nq;
    const int bh = row / nq;
    const int hq = bh % a.heads;
    const int b = bh / a.heads;
    const int g = a.heads / a.kv_heads;
    const int hk = hq / g;
    const int r = (hq - hk * g) * nq + t;  // row inside the kv head's packed rows
    const int rb = r / 32, r32 = r % 32;
    const int HR = a.row_blocks;
    const int G = a.waves / a.kv_heads;
    const int pb = (int)a.prefix[b];
    const DecPart part((int)a.prefix[a.batch] * HR, G);
    const int n = (int)a.prefix[b + 1] - pb;  // steps of each segment of sequence b
    float o = 0.f, lse = kNegInf;
    if (n > 0) {
        const int p0 = pb * HR + rb * n, p1 = p0 + n - 1;  // the segment's first and last step
        const int j0 = part.group_of(p0), j1 = part.group_of(p1);
        const int64_t s = (int64_t)b * HR + rb;
        float mx = kNegInf, wsum = 0.f;
        for (int jb = j0; jb <= j1; jb += kMergeBatch) {
            float ls[kMergeBatch], ov[kMergeBatch];
#pragma unroll
            for (int i = 0; i < kMergeBatch; ++i) {
                const int j = jb + i;
                // past the segment's last group, or a group with an empty range
                // (more groups than steps): no piece, never read
                const bool has = j <= j1 && !part.empty(j);
                const int64_t prow = ((j + s) * a.kv_heads + hk) * 32 + r32;
                ls[i] = has ? a.ws_lse[prow] : kNegInf;
                ov[i] = has ? a.ws_o[prow * D + d] : 0.f;
            }
            float m2 = mx;
#pragma unroll
            for (int i = 0; i < kMergeBatch; ++i) m2 = fmaxf(m2, ls[i]);
            if (m2 == kNegInf) continue;
            const float f = mx == kNegInf ? 0.f : __expf(mx - m2);  // rescale what came before
            wsum *= f;
            o *= f;
#pragma unroll
            for (int i = 0; i < kMergeBatch; ++i) {
                if (ls[i] == kNegInf) continue;
                const float wt = __expf(ls[i] - m2);
                wsum += wt;
                o = __builtin_fmaf(wt, ov[i], o);
            }
            mx = m2;
        }
        if (mx != kNegInf) {
            o /= wsum;
            lse = mx + __logf(wsum);
        }
    }
    uint16_t* out = (uint16_t*)a.o + (((int64_t)b * nq + t) * a.heads + hq) * a.head_dim;
    if (d < a.head_dim) {
        if constexpr (BF16) {
            const __bf16 hv = (__bf16)o;
            out[d] = __builtin_bit_cast(uint16_t, hv);
        } else {
            const _Float16 hv = (_Float16)o;
            out[d] = __builtin_bit_cast(uint16_t, hv);
        }
    }
    if (d == 0) a.lse[row] = lse;
}

template <bool BF16, int D>
int launch_decode_t(const DecArgs& a, hipStream_t stream) {
    if (a.batch == 0 || a.seqlen_q == 0) return 0;
    hipLaunchKernelGGL((decode_split_kernel<BF16, D>), dim3(a.waves), dim3(64), 0, stream, a);
    if (hipGetLastError() != hipSuccess) return 1;
    const int64_t nrows = (int64_t)a.batch * a.heads * a.seqlen_q;
    hipLaunchKernelGGL((decode_combine_kernel<BF16, D>), dim3((unsigned)nrows), dim3(D), 0, stream, a);
    return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // namespace

int launch_decode(const DecArgs& a, hipStream_t stream) {
    if (a.head_dim > 128) return a.bf16 ? launch_decode_t<true, 256>(a, stream) : launch_decode_t<false, 256>(a, stream);
    if (a.bf16)
        return a.head_dim > 64 ? launch_decode_t<true, 128>(a, stream) : launch_decode_t<true, 64>(a, stream);
    return a.head_dim > 64 ? launch_decode_t<false, 128>(a, stream) : launch_decode_t<false, 64>(a, stream);
}

}  // namespace fa
