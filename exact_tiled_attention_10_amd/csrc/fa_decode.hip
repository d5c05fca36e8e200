// Decode: exact attention of a short block of new query tokens over a long
// key/value cache (the KV-cache entry of the FlashAttention-2 overview page,
// lshu.cn/news/55956, section 3.3), split over the keys.
//
// The work is bound by reading the cache once, so the kernel is organised for
// memory-level parallelism rather than matrix-core rate:
//   * one wave per (batch, kv head, key split, row block); the g query heads
//     that share the kv head and the Nq new tokens are packed into blocks of
//     32 rows (row r = (head r / Nq, token r % Nq)), so a cache byte is read
//     once per kv head (per 32 such rows), not once per query head;
//   * each wave streams its split in 32-key steps through its own two LDS
//     stages with direct global -> LDS loads, waiting only on its own loads
//     (no workgroup barriers);
//   * per step: S^T = K Q^T on the matrix cores, the online softmax per query
//     column (lazy rescale, as in the forward kernel), O^T += V^T P^T with V^T
//     from transposing LDS reads;
//   * each split writes its normalised partial O (fp32) and LSE; a second
//     kernel merges the splits by their LSE: LSE = log sum_s e^{LSE_s},
//     O = sum_s e^{LSE_s - LSE} O_s.
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
constexpr int kDecWaves = 4;  // splits per workgroup, one per wave
constexpr int kDecBK = 32;    // keys per step

template <int D>
struct DecCfg {
    static constexpr int CPR = D / 8;
    static constexpr int tileElems = kDecBK * D;          // one K or V tile
    static constexpr int kDma = tileElems * 2 / 1024;     // 1 KiB direct loads per tile
    static constexpr int kRowsPerBlock = 1024 / (2 * D);  // cache rows per direct load
};

template <bool BF16, int D>
__global__ __launch_bounds__(64 * kDecWaves) void decode_split_kernel(DecArgs a) {
    using C = DecCfg<D>;
    constexpr int KS = D / 16, DB = D / 32;
    // Two stages per tensor as separate objects (one slice per wave): reads of
    // one stage are then known not to touch the loads in flight into the other.
    __shared__ __attribute__((aligned(16))) uint16_t kst0[kDecWaves][C::tileElems];
    __shared__ __attribute__((aligned(16))) uint16_t kst1[kDecWaves][C::tileElems];
    __shared__ __attribute__((aligned(16))) uint16_t vst0[kDecWaves][C::tileElems];
    __shared__ __attribute__((aligned(16))) uint16_t vst1[kDecWaves][C::tileElems];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r32 = lane & 31, half = lane >> 5;
    const int b = blockIdx.x / a.kv_heads, hk = blockIdx.x % a.kv_heads;
    const int sp = blockIdx.y * kDecWaves + wave;
    const int rb = blockIdx.z;
    if (sp >= a.nsplit) return;  // whole wave; no barrier below
    auto kst = [&](int p) { return p ? kst1[wave] : kst0[wave]; };
    auto vst = [&](int p) { return p ? vst1[wave] : vst0[wave]; };

    const int g = a.heads / a.kv_heads;
    const int nq = a.seqlen_q;
    const int rows = g * nq;
    int len_k = a.cache_lens ? a.cache_lens[b] : a.seqlen_k;
    len_k = min(max(len_k, 0), a.seqlen_k);
    Seq s;
    s.q_start = (int64_t)b * nq;
    s.k_start = (int64_t)b * a.seqlen_k;
    s.len_q = nq;
    s.len_k = len_k;
    s.off = len_k - nq;
    const Mask mk{a.causal, a.left, a.right};

    // this lane's row: query head hq, token t
    const int rr = rb * 32 + r32;
    const bool live = rr < rows;
    const int t = live ? rr % nq : 0;
    const int hq = hk * g + (live ? rr / nq : 0);
    const int lo_q = mk.lo_of(t, s), hi_q = live ? mk.hi_of(t, s) : -1;
    // This sequence's keys split in whole 32-key steps over the nsplit waves,
    // so every split of a sequence does the same work whatever its length.
    const int chunk = kDecBK * (((len_k + kDecBK - 1) / kDecBK + a.nsplit - 1) / a.nsplit);
    const int k_begin = sp * chunk;
    const int k_end = min(k_begin + chunk, len_k);  // exclusive
    const int vis_lo = max(k_begin, mk.lo_of(0, s));
    const int vis_hi = min(k_end - 1, mk.hi_of(nq - 1, s));
    // no row of the block needs a mask inside [full_lo, full_hi] (uniform)
    const int full_lo = max(k_begin, mk.lo_of(nq - 1, s));
    const int full_hi = min(k_end - 1, mk.hi_of(0, s));

    const int kv_stride = a.kv_heads * D;
    u32x4 qf[KS];
    {
        const uint16_t* qrow = (const uint16_t*)a.q + ((s.q_start + t) * a.heads + hq) * D;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qf[ks] = live ? *(const u32x4*)(qrow + ks * 16 + 8 * half) : u32x4{0, 0, 0, 0};
    }
    const uint16_t* kbase = (const uint16_t*)a.kc + (s.k_start * a.kv_heads + hk) * D;
    const uint16_t* vbase = (const uint16_t*)a.vc + (s.k_start * a.kv_heads + hk) * D;

    // direct loads: block i covers cache rows i * kRowsPerBlock + lane / CPR
    const int dma_r = lane / C::CPR;
    int dma_off[C::kDma];
#pragma unroll
    for (int i = 0; i < C::kDma; ++i) {
        const int row = i * C::kRowsPerBlock + dma_r;
        dma_off[i] = ((lane % C::CPR) ^ swz<C::CPR>(row)) * 8;
    }
    int k_rd[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) k_rd[ks] = r32 * D + (((2 * ks + half) ^ swz<C::CPR>(r32)) * 8);
    int v_rd[2][DB];
    tr_offsets<D, DB>(lane, v_rd);

    f32x16 acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] = f32x16{0};
    float m_run = kNegInf, l_part = 0.f;
    const float c = a.scale_log2;

    auto issue = [&](int st, int p) {
        const int key0 = st * kDecBK;
#pragma unroll
        for (int i = 0; i < C::kDma; ++i) {
            const int row = min(key0 + i * C::kRowsPerBlock + dma_r, len_k - 1);  // clamp: in bounds
            const int64_t off = (int64_t)row * kv_stride + dma_off[i];
            dma16(kbase + off, kst(p) + i * 512);
            dma16(vbase + off, vst(p) + i * 512);
        }
    };

    auto compute = [&](int st, int p) {
        const int key0 = st * kDecBK;
        const uint16_t* kt = kst(p);
        const uint16_t* vt = vst(p);
        f32x16 sacc = f32x16{0};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) sacc = mfma32<BF16>(*(const u32x4*)(kt + k_rd[ks]), qf[ks], sacc);
        if (!(key0 >= full_lo && key0 + kDecBK - 1 <= full_hi)) {  // uniform: edge steps only
            const int klo = max(lo_q, k_begin), khi = min(hi_q, k_end - 1);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int key = key0 + 8 * (i / 4) + 4 * half + (i % 4);
                sacc[i] = (key < klo || key > khi) ? kNegInf : sacc[i];
            }
        }
        float mx = kNegInf;
#pragma unroll
        for (int i = 0; i < 16; i += 2) mx = fmaxf(mx, fmaxf(sacc[i], sacc[i + 1]));
        mx = max_halves(mx);
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
            for (int db = 0; db < DB; ++db) acc[db] = mfma32<BF16>(read_tr<D, DB>(vt, hs, db, v_rd), pb, acc[db]);
        }
    };

    if (vis_lo <= vis_hi) {
        const int st_lo = vis_lo / kDecBK, st_hi = vis_hi / kDecBK + 1;
        // Two steps per iteration so the stage index stays a constant.  The
        // first DMA is issued inside the loop (the compute of the step
        // before st_lo is skipped); loads past the last step read the
        // clamped last cache row and are drained before the wave exits.
        int st = st_lo - 1;  // step held in stage 1
        for (;;) {
            issue(st + 1, 0);
            wait_vmcnt<2 * C::kDma>();
            if (st >= st_lo) compute(st, 1);
            if (st + 1 >= st_hi) break;
            issue(st + 2, 1);
            wait_vmcnt<2 * C::kDma>();
            compute(st + 1, 0);
            st += 2;
            if (st >= st_hi) break;
        }
        wait_vmcnt<0>();
    }

    // partial O (normalised, fp32) and LSE of this split
    const float l = sum_halves(l_part);
    if (!live) return;
    const int64_t prow = (((int64_t)sp * a.batch + b) * a.heads + hq) * nq + t;
    const float inv = l > 0.f ? 1.f / l : 0.f;
    float* orow = a.ws_o + prow * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
            float4 w;
            w.x = acc[db][4 * gq] * inv;
            w.y = acc[db][4 * gq + 1] * inv;
            w.z = acc[db][4 * gq + 2] * inv;
            w.w = acc[db][4 * gq + 3] * inv;
            *(float4*)(orow + db * 32 + 8 * gq + 4 * half) = w;
        }
    if (half == 0) a.ws_lse[prow] = l > 0.f ? m_run * a.scale + logf(l) : kNegInf;
}

// One workgroup of D threads per (batch, query head, token): merge the splits.
template <bool BF16, int D>
__global__ __launch_bounds__(D) void decode_combine_kernel(DecArgs a) {
    const int64_t row = blockIdx.x;  // ((b * heads) + hq) * nq + t
    const int nq = a.seqlen_q;
    const int64_t nrows = (int64_t)a.batch * a.heads * nq;
    const int d = threadIdx.x;
    float mx = kNegInf;
    for (int sp = 0; sp < a.nsplit; ++sp) mx = fmaxf(mx, a.ws_lse[sp * nrows + row]);
    float wsum = 0.f, o = 0.f;
    if (mx != kNegInf) {
        for (int sp = 0; sp < a.nsplit; ++sp) {
            const float ls = a.ws_lse[sp * nrows + row];
            const float w = ls == kNegInf ? 0.f : expf(ls - mx);
            wsum += w;
            o += w * a.ws_o[(sp * nrows + row) * D + d];
        }
        o /= wsum;
    }
    const int t = (int)(row % nq);
    const int64_t bh = row / nq;
    const int hq = (int)(bh % a.heads);
    const int64_t bb = bh / a.heads;
    uint16_t* out = (uint16_t*)a.o + ((bb * nq + t) * a.heads + hq) * D;
    if constexpr (BF16) {
        const __bf16 hv = (__bf16)o;
        out[d] = __builtin_bit_cast(uint16_t, hv);
    } else {
        const _Float16 hv = (_Float16)o;
        out[d] = __builtin_bit_cast(uint16_t, hv);
    }
    if (d == 0) a.lse[row] = mx == kNegInf ? kNegInf : mx + logf(wsum);
}

template <bool BF16, int D>
int launch_decode_t(const DecArgs& a, hipStream_t stream) {
    if (a.batch == 0 || a.seqlen_q == 0) return 0;
    dim3 grid(a.batch * a.kv_heads, (a.nsplit + kDecWaves - 1) / kDecWaves, a.row_blocks);
    hipLaunchKernelGGL((decode_split_kernel<BF16, D>), grid, dim3(64 * kDecWaves), 0, stream, a);
    if (hipGetLastError() != hipSuccess) return 1;
    const int64_t nrows = (int64_t)a.batch * a.heads * a.seqlen_q;
    hipLaunchKernelGGL((decode_combine_kernel<BF16, D>), dim3((unsigned)nrows), dim3(D), 0, stream, a);
    return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // namespace

int launch_decode(const DecArgs& a, hipStream_t stream) {
    if (a.bf16)
        return a.head_dim == 128 ? launch_decode_t<true, 128>(a, stream) : launch_decode_t<true, 64>(a, stream);
    return a.head_dim == 128 ? launch_decode_t<false, 128>(a, stream) : launch_decode_t<false, 64>(a, stream);
}

}  // namespace fa
