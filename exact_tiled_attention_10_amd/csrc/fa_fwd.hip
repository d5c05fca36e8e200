// Forward of exact tiled attention on gfx950.
//
// One workgroup = one (batch, query head) and a tile of BM = 32 * QB * NW
// query rows; NW waves, each owning QB column blocks of 32 rows.  The kernel
// streams the visible K/V tiles (BN keys each) through two LDS buffers: while
// the waves compute on one buffer, the next tile is in flight to the other by
// direct global -> LDS loads that bypass registers entirely (the
// asynchronous double buffering of the FlashAttention-2 overview page,
// lshu.cn/news/55956, section 2.2, third innovation).  Per tile and wave:
//
//   S^T = K Q^T            (keys x queries; Q^T held in registers)
//   online softmax          per query column: running max m and sum l
//                           (same page, section 2.2, second innovation)
//   O^T += V^T P^T          (d x queries; P^T taken straight from the S^T
//                           registers, V^T gathered from the row-major V tile
//                           by the transposing LDS reads of gfx950)
//
// The N x N score matrix never leaves registers (first innovation, tiled
// fusion).  Working in the transposed orientation puts one query per lane
// column, so the row max needs one swap between wave halves and the rescale
// factor is one value per lane.
//
// The running max used as the exponent offset is only moved when the true
// row max exceeds it by more than 2^kLazyLog2 in p (log2 units); below that
// the factors exp(s - m) stay <= 2^kLazyLog2, far from fp32 / fp16 overflow,
// and the final O = acc / l and LSE = m + ln l are the same numbers.  This
// skips the rescale of the accumulator registers on almost every tile.
//
// Dropout (DROP): after the exponent each probability is kept or zeroed by
// its Philox draw (fa_device.hpp) before it enters P.V; the row sum l keeps
// every probability, and the kept ones are scaled by 256 / T in the epilogue,
// so O = (P o M) V * 256 / T and LSE is that of the undropped softmax.
//
// Head dimension: the kernels are built for tile widths D = 64 and 128 and
// run any head_dim dh that is a multiple of 8 up to D.  Global rows are dh
// long; the resident Q^T fragments hold zeros past dh, and the direct loads
// of K and V fill the columns past dh with a copy of the row's last valid
// chunk (finite values that only ever meet those zeros in S, and only reach
// the columns of O past dh, which are not stored).
//
// Masked scores are set to -inf before the exponent; the host clamps
// scale*log2(e) to at least the smallest normal float, so -inf * c stays -inf
// and exp2 gives an exact 0 even for softmax_scale == 0 (where every finite
// score then maps to exp2(0) = 1, the uniform weights that scale means).
#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {

namespace {

constexpr float kLazyLog2 = 8.0f;

template <int D, int NW, int BN>
struct FwdCfg {
    static constexpr int kThreads = 64 * NW;
    // K and V tiles: BN rows (keys) of D 16-bit values each, unpadded; the
    // 16-byte chunk c of row r sits at slot c ^ swz(r).  Both are filled by
    // direct global -> LDS loads, each writing 1 KiB (64 lanes x 16 B) in lane
    // order, so a load instruction covers 1024 / (2 D) whole rows.
    static constexpr int CPR = D / 8;
    static constexpr int tileElems = BN * D;
    static constexpr int kDmaBlocks = BN * D * 2 / 1024;
    static constexpr int kDmaPerWave = kDmaBlocks / NW;
    static constexpr int kRowsPerBlock = 1024 / (D * 2);
    static constexpr int stageElems = 2 * tileElems;  // K then V
    static_assert(kDmaBlocks % NW == 0, "tiles must split evenly into 1 KiB blocks per wave");
};

template <bool BF16, int D, int NW, int QB, int BN, int WPE, bool DROP>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * NW, 64 * NW), amdgpu_waves_per_eu(WPE, WPE)))
void fwd_kernel(FwdArgs a) {
    using C = FwdCfg<D, NW, BN>;
    constexpr int KS = D / 16;  // k-steps of S over d
    constexpr int DB = D / 32;  // 32-row blocks of O^T over d
    constexpr int KB = BN / 32; // 32-key blocks per tile
    constexpr int BM = 32 * QB * NW;
    constexpr int RW = 32 * QB;  // rows per wave
    // Two LDS stages as separate objects: the compiler can then tell that reads
    // of one stage never touch the direct loads in flight into the other, and
    // does not wait for those loads before the transposing reads.
    __shared__ __attribute__((aligned(16))) uint16_t lds0[C::stageElems];
    __shared__ __attribute__((aligned(16))) uint16_t lds1[C::stageElems];
    auto stage = [&](int buf) { return buf ? lds1 : lds0; };

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches below
    const int r32 = lane & 31, half = lane >> 5;
    int b, h;
    xcd_head(rotated_column(), a.batch, a.heads, a.kv_heads, b, h);
    const int ntiles = gridDim.y;
    const int qt = a.causal ? (ntiles - 1 - (int)blockIdx.y) : (int)blockIdx.y;
    const Seq s = seq_of(b, a.cu_q, a.cu_k, a.used_q, a.used_k, a.seqlen_q, a.seqlen_k);
    const int i0 = qt * BM;
    if (i0 >= s.len_q) return;
    const Mask mk{a.causal, a.left, a.right};
    const int hk = h / (a.heads / a.kv_heads);

    const int dh = a.head_dim;  // multiple of 8, at most D
    const int64_t q_row_stride = (int64_t)a.heads * dh;
    const int kv_row_stride = a.kv_heads * dh;
    const uint16_t* qbase = (const uint16_t*)a.q + (s.q_start * a.heads + h) * dh;
    const uint16_t* kbase = (const uint16_t*)a.k + (s.k_start * a.kv_heads + hk) * dh;
    const uint16_t* vbase = (const uint16_t*)a.v + (s.k_start * a.kv_heads + hk) * dh;
    uint16_t* obase = (uint16_t*)a.o + (s.q_start * a.heads + h) * dh;
    float* lsebase = a.cu_q ? a.lse + (int64_t)h * a.cu_q[a.batch] + s.q_start
                            : a.lse + ((int64_t)b * a.heads + h) * a.seqlen_q;

    // Key range of the whole workgroup, as whole tiles.
    const int i_last = min(i0 + BM, s.len_q) - 1;
    const int key_lo = mk.lo_of(i0, s);
    const int key_hi = mk.hi_of(i_last, s);  // inclusive
    const int t_lo = key_lo / BN;
    const int t_hi = key_hi >= key_lo ? key_hi / BN + 1 : t_lo;

    // This wave's rows and the key range any of them can see (all uniform).
    const int wq0 = i0 + RW * wave;
    const int wq1 = min(wq0 + RW, s.len_q) - 1;
    const bool wave_live = wq0 < s.len_q;
    const int w_key_lo = wave_live ? mk.lo_of(wq0, s) : 0;
    const int w_key_hi = wave_live ? mk.hi_of(wq1, s) : -1;
    // Tiles inside [w_full_lo, w_full_hi] need no mask for any row of the wave.
    const int w_full_lo = wave_live ? mk.lo_of(wq1, s) : 0;
    const int w_full_hi = wave_live ? mk.hi_of(wq0, s) : -1;

    // Q^T fragments (B operand of S^T = K Q^T), resident for the whole loop.
    u32x4 qf[QB][KS];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int row = wq0 + 32 * qb + r32;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qf[qb][ks] = row < s.len_q && ks * 16 + 8 * half < dh
                             ? *(const u32x4*)(qbase + (int64_t)row * q_row_stride + ks * 16 + 8 * half)
                             : u32x4{0, 0, 0, 0};
    }

    // ---- per-thread constant offsets -----------------------------------------------
    // Direct loads: block bi = wave * kDmaPerWave + i covers rows
    // bi * kRowsPerBlock + lane / CPR; lane slot lane % CPR receives chunk slot ^ swz(row).
    int dma_goff[C::kDmaPerWave];  // element offset inside the tile (row * stride + chunk * 8)
    int dma_row[C::kDmaPerWave];
#pragma unroll
    for (int i = 0; i < C::kDmaPerWave; ++i) {
        const int bi = wave * C::kDmaPerWave + i;
        const int row = bi * C::kRowsPerBlock + lane / C::CPR;
        const int slot = lane % C::CPR;
        dma_row[i] = row;
        const int chunk = min(slot ^ swz<C::CPR>(row), dh / 8 - 1);  // columns past dh: last chunk again
        dma_goff[i] = row * kv_row_stride + chunk * 8;
    }
    // S^T operand reads of K: lane (r32, half) reads row kb*32 + r32, chunk 2 ks + half.
    int k_rd[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) k_rd[ks] = r32 * D + (((2 * ks + half) ^ swz<C::CPR>(r32)) * 8);
    // V^T operand reads: transposing LDS reads of the row-major V tile.
    int v_rd[2][DB];
    tr_offsets<D, DB>(lane, v_rd);

    f32x16 acc[DB][QB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) acc[db][qb] = f32x16{0};
    float m_run[QB], l_part[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) { m_run[qb] = kNegInf; l_part[qb] = 0.f; }
    const float c = a.scale_log2;

    // Issue the loads of tile t straight into LDS buffer `buf` (K, then V).
    auto issue_tile = [&](int t, int buf) {
        const int key0 = t * BN;
        const bool tail = key0 + BN > s.len_k;  // uniform
        const int last = s.len_k - 1 - key0;
        const int64_t tile_off = (int64_t)key0 * kv_row_stride;
        uint16_t* kl = stage(buf);
        const rsrc_t ksrc = buffer_of(kbase + tile_off), vsrc = buffer_of(vbase + tile_off);
#pragma unroll
        for (int i = 0; i < C::kDmaPerWave; ++i) {
            int off = dma_goff[i];
            if (tail && dma_row[i] > last) off += (last - dma_row[i]) * kv_row_stride;  // clamp to the last key
            uint16_t* dst = kl + (wave * C::kDmaPerWave + i) * 512;
            dma16(ksrc, (uint32_t)off * 2u, dst);
            dma16(vsrc, (uint32_t)off * 2u, dst + C::tileElems);
        }
    };

    // One K/V tile on LDS buffer `buf` for this wave.
    auto compute_tile = [&](int t, int buf) {
        const int key0 = t * BN;
        if (!(wave_live && key0 <= w_key_hi && key0 + BN - 1 >= w_key_lo)) return;
        const uint16_t* ks_lds = stage(buf);
        const uint16_t* vs_lds = ks_lds + C::tileElems;
        // ---- S^T = K Q^T -------------------------------------------------
        f32x16 sacc[KB][QB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) sacc[kb][qb] = f32x16{0};
        // K fragments are read one k-step ahead of the MFMAs that use them.
        u32x4 kf[2][KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) kf[0][kb] = *(const u32x4*)(ks_lds + kb * 32 * D + k_rd[0]);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if (ks + 1 < KS) {
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) kf[(ks + 1) & 1][kb] = *(const u32x4*)(ks_lds + kb * 32 * D + k_rd[ks + 1]);
            }
            __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of these MFMAs
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) sacc[kb][qb] = mfma32<BF16>(kf[ks & 1][kb], qf[qb][ks], sacc[kb][qb]);
            __builtin_amdgcn_sched_barrier(0);
        }
        // ---- mask (edge tiles only; uniform branch) --------------------------
        if (key0 < w_full_lo || key0 + BN - 1 > w_full_hi) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                const int qi = wq0 + 32 * qb + r32;
                const int lo = mk.lo_of(qi, s) - key0, hi = mk.hi_of(qi, s) - key0;
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int kk = kb * 32 + 8 * (i / 4) + 4 * half + (i % 4);
                        sacc[kb][qb][i] = (kk < lo || kk > hi) ? kNegInf : sacc[kb][qb][i];
                    }
            }
        }
        // Dropout: this lane's keep words, one per 32 x 32 block: word g holds the
        // draws of its query row for keys 8 g + 4 half + 0..3 of the block.
        u32x4 kw[DROP ? KB : 1][DROP ? QB : 1];
        if constexpr (DROP) {
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) {
                    const uint32_t jq = (uint32_t)(key0 + 32 * kb) / 4 + 2 * (r32 & 3) + half;
                    const uint32_t iq = (uint32_t)(wq0 + 32 * qb + r32) / 4;
                    kw[kb][qb] = quad_transpose(philox4x32_10(jq, iq, h, b, a.seed_lo, a.seed_hi));
                }
        }
        // V^T fragments of the first key step: read now, used after the softmax.
        auto read_vt = [&](int kk, int db) { return read_tr<D, DB>(vs_lds, kk, db, v_rd); };
        u32x4 vf0[DB];
#pragma unroll
        for (int db = 0; db < DB; ++db) vf0[db] = read_vt(0, db);
        // ---- online softmax ------------------------------------------------
        uint32_t pk[KB][QB][8];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            float mx = kNegInf;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) mx = max16(sacc[kb][qb], mx);
            mx = max_halves(mx);
            const float m_old = m_run[qb];
            const bool up = mx > m_old && (m_old == kNegInf || (mx - m_old) * c > kLazyLog2);
            if (__builtin_amdgcn_ballot_w64(up)) {
                const float alpha = !up ? 1.f : (m_old == kNegInf ? 0.f : fast_exp2((m_old - mx) * c));
                m_run[qb] = up ? mx : m_old;
                l_part[qb] *= alpha;
#pragma unroll
                for (int db = 0; db < DB; ++db) acc[db][qb] *= alpha;
            }
            const float mc = m_run[qb] == kNegInf ? 0.f : m_run[qb] * c;
            float lsum = 0.f;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int i = 0; i < 16; i += 2) {
                    float p0 = fast_exp2(__builtin_fmaf(sacc[kb][qb][i], c, -mc));
                    float p1 = fast_exp2(__builtin_fmaf(sacc[kb][qb][i + 1], c, -mc));
                    lsum += p0 + p1;
                    if constexpr (DROP) {
                        const uint32_t w = kw[kb][qb][i / 4];
                        p0 = keep_byte(w, i % 4, a.drop_t) ? p0 : 0.f;
                        p1 = keep_byte(w, (i + 1) % 4, a.drop_t) ? p1 : 0.f;
                    }
                    pk[kb][qb][i / 2] = pack2<BF16>(p0, p1);
                }
            l_part[qb] += lsum;
        }
        // ---- O^T += V^T P^T --------------------------------------------------
#pragma unroll
        for (int kk = 0; kk < BN / 16; ++kk) {
            const int kb = kk / 2, hs = kk % 2;
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const u32x4 vf = kk == 0 ? vf0[db] : read_vt(kk, db);
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) {
                    const u32x4 pb = u32x4{pk[kb][qb][4 * hs], pk[kb][qb][4 * hs + 1],
                                           pk[kb][qb][4 * hs + 2], pk[kb][qb][4 * hs + 3]};
                    acc[db][qb] = mfma32<BF16>(vf, pb, acc[db][qb]);
                }
            }
        }
    };

    // One pipeline step: prefetch tile t+1 into the other buffer, compute tile t.
    auto step = [&](int t, int buf) {
        const bool has_next = t + 1 < t_hi;
        if (has_next) issue_tile(t + 1, buf ^ 1);
        compute_tile(t, buf);
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): direct K loads have landed
        __syncthreads();
    };

    if (t_lo < t_hi) {
        issue_tile(t_lo, 0);
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();
        for (int t = t_lo; t < t_hi; t += 2) {
            step(t, 0);
            if (t + 1 < t_hi) step(t + 1, 1);
        }
    }

    // ---- epilogue: O = acc / l, LSE = scale * m + ln l ------------------------------
    if (!wave_live) return;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int row = wq0 + 32 * qb + r32;
        const float l = sum_halves(l_part[qb]);
        const float inv = l > 0.f ? (DROP ? a.drop_scale : 1.f) / l : 0.f;
        if (row < s.len_q) {
            uint16_t* orow = obase + (int64_t)row * q_row_stride;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int col = db * 32 + 8 * g + 4 * half;  // four columns, all below dh or none
                    if (col >= dh) continue;
                    u32x2 w;
                    w.x = pack2<BF16>(acc[db][qb][4 * g] * inv, acc[db][qb][4 * g + 1] * inv);
                    w.y = pack2<BF16>(acc[db][qb][4 * g + 2] * inv, acc[db][qb][4 * g + 3] * inv);
                    *(u32x2*)(orow + col) = w;
                }
            if (half == 0)
                lsebase[row] = l > 0.f ? m_run[qb] * a.scale + logf(l) : kNegInf;
        }
    }
}

template <bool BF16, int D, int NW, int QB, int BN, int WPE>
int launch_fwd_t(const FwdArgs& a, hipStream_t stream) {
    constexpr int BM = 32 * QB * NW;
    using C = FwdCfg<D, NW, BN>;
    const int ntiles = (a.seqlen_q + BM - 1) / BM;
    if (ntiles == 0 || a.batch == 0) return 0;
    auto kern = a.drop_t < 256 ? fwd_kernel<BF16, D, NW, QB, BN, WPE, true>
                               : fwd_kernel<BF16, D, NW, QB, BN, WPE, false>;
    dim3 grid(a.batch * a.heads, ntiles);
    hipLaunchKernelGGL(kern, grid, dim3(C::kThreads), 0, stream, a);
    return hipGetLastError() == hipSuccess ? 0 : 1;
}

// Launch shapes (measured on MI355X, bf16 causal).  d = 128: 8 waves of 32
// query rows (two waves per SIMD, all state in arch VGPRs) beat 4 waves of 64
// rows, whose accumulators spill into AGPR traffic; 64-key tiles.  An 8-wave
// workgroup fills a CU, so a grid of fewer than four of them per CU ends in
// a long tail: such grids run 4-wave workgroups of the same kind, two per CU
// (same results: every query row is computed alike).  d = 64:
// fewer registers per wave, so 4 waves of 32 rows with three workgroups per
// CU (three waves per SIMD) and 64-key tiles.  Overridable at build time for
// tuning.
#ifndef FA_FWD_NW
#define FA_FWD_NW 8
#endif
#ifndef FA_FWD_QB
#define FA_FWD_QB 1
#endif
#ifndef FA_FWD_BN128
#define FA_FWD_BN128 64
#endif
#ifndef FA_FWD_WPE
#define FA_FWD_WPE 2
#endif
#ifndef FA_FWD64_NW
#define FA_FWD64_NW 4
#endif
#ifndef FA_FWD_BN64
#define FA_FWD_BN64 64
#endif
#ifndef FA_FWD64_WPE
#define FA_FWD64_WPE 3
#endif

}  // namespace

int launch_fwd(const FwdArgs& a, hipStream_t stream) {
    constexpr int NW = FA_FWD_NW, QB = FA_FWD_QB, W = FA_FWD_WPE, B1 = FA_FWD_BN128;
    constexpr int NW2 = FA_FWD64_NW, W2 = FA_FWD64_WPE, B2 = FA_FWD_BN64;
    // tile width: the smallest of 64, 128, 256 holding head_dim.  At 256 the
    // O accumulators (128 per lane) and the resident Q^T (64) need more than
    // half the register file: 4 waves at one per SIMD, 64-key tiles (K and V
    // of a tile 64 KiB, two stages in 128 KiB of LDS; measured 6-8% faster
    // than 32-key tiles at 8K, one register spilled).
    if (a.head_dim > 128)
        return a.bf16 ? launch_fwd_t<true, 256, 4, 1, 64, 1>(a, stream)
                      : launch_fwd_t<false, 256, 4, 1, 64, 1>(a, stream);
    if (a.head_dim > 64) {
        const long long wgs = (long long)a.batch * a.heads * ((a.seqlen_q + 32 * NW * QB - 1) / (32 * NW * QB));
        if (NW == 8 && wgs < 4LL * a.cus)
            return a.bf16 ? launch_fwd_t<true, 128, 4, QB, B1, W>(a, stream)
                          : launch_fwd_t<false, 128, 4, QB, B1, W>(a, stream);
        return a.bf16 ? launch_fwd_t<true, 128, NW, QB, B1, W>(a, stream)
                      : launch_fwd_t<false, 128, NW, QB, B1, W>(a, stream);
    }
    return a.bf16 ? launch_fwd_t<true, 64, NW2, QB, B2, W2>(a, stream)
                  : launch_fwd_t<false, 64, NW2, QB, B2, W2>(a, stream);
}

}  // namespace fa
