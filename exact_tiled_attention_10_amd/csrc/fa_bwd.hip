// Backward of exact tiled attention on gfx950.
//
// The scores are recomputed from Q, K and the saved LSE instead of being read
// back (install guide page yfxerp.com/news/195771, section 1; the overview
// page lshu.cn/news/55956, section 2.1, second anti-pattern, is the cost of
// not doing so).  With P_ij = exp(scale q_i.k_j - LSE_i) and
// D_i = dO_i . O_i (equal to sum_j P_ij dP_ij):
//
//   dP = dO V^T,  dS = P o (dP - D),  dV = P^T dO,  dK = scale dS^T Q,
//   dQ = scale dS K.
//
// With dropout (DROP; keep decisions as in the forward, fa_device.hpp), P
// below is the undropped softmax, M the keep mask and s = 256 / T:
//   dV = (P o M)^T dO * s,  dS = P o (M o dP * s - D),  D_i = dO_i . O_i
// (O being the dropped output, D needs no change).
//
// Head dimension: as in the forward, tiles are D = 64 or 128 wide and any
// head_dim dh that is a multiple of 8 up to D runs in them: global rows are dh
// long, register-resident fragments are zero past dh, direct loads repeat the
// row's last valid chunk past dh, and columns past dh are not stored.
//
// Three kernels on one stream:
//   bwd_rowdot   D_i = dO_i . O_i and LSE_i * log2(e) into the workspace
//   bwd_dkdv     per key tile (outer) and every visible query tile of every
//                query head of the GQA group (inner): dK, dV accumulated in
//                registers, no atomics
//   bwd_dq       per query tile (outer) over the visible key tiles (inner):
//                the separate dQ accumulation pass, no atomics
// or, on the atomic dQ path (head_dim up to 128, when the caller allows a
// summation order that varies from call to call):
//   bwd_rowdot   as above, and zeroes a float32 dQ accumulator
//   bwd_dkdv     also forms dQ += dS K for each 32-row block over the
//                workgroup's 128 keys and adds it into the accumulator with
//                float32 atomics, so the scores and dP are computed once
//                (five products per visible pair instead of seven)
//   bwd_dq_cvt   dQ = scale * accumulator, rounded to the 16-bit type
// Both main kernels stream their tiles row-major into LDS with direct
// global -> LDS loads (double-buffered) and build every transposed MFMA
// operand (dO^T, Q^T, K^T) with the transposing LDS reads of gfx950, so no
// tile is ever transposed through registers.  Operand orientation follows the
// MFMA C layout (fa_device.hpp): the dK/dV pass computes S = Q K^T with one key
// per lane column, so P and dS feed dV^T = dO^T P and dK^T = Q^T dS directly;
// the dQ pass computes S^T = K Q^T with one query per lane column, so dS^T
// feeds dQ^T = K^T dS^T.
#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {

namespace {

constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------------------
// D_i = dO_i . O_i  and  lse2_i = LSE_i * log2(e)
// ---------------------------------------------------------------------------
template <bool BF16, int D>
__global__ __launch_bounds__(256) void bwd_rowdot_kernel(BwdArgs a) {
    constexpr int LPR = D / 8;               // lanes per (row, head), 16 B each
    constexpr int RPB = 256 / LPR;           // (row, head) pairs per block
    const int tid = threadIdx.x;
    const int64_t item = (int64_t)blockIdx.x * RPB + tid / LPR;
    const int part = tid % LPR;
    const int64_t rows = a.cu_q ? (int64_t)a.cu_q[a.batch] : (int64_t)a.batch * a.seqlen_q;
    const int64_t t = item / a.heads;  // packed row
    const int h = (int)(item % a.heads);
    float acc = 0.f;
    const bool live = t < rows;
    if (live && part * 8 < a.head_dim) {
        const int64_t off = (t * a.heads + h) * a.head_dim + part * 8;
        const u32x4 o4 = *(const u32x4*)((const uint16_t*)a.o + off);
        const u32x4 d4 = *(const u32x4*)((const uint16_t*)a.dout + off);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            acc += to_f32<BF16>(o4[w] & 0xffffu) * to_f32<BF16>(d4[w] & 0xffffu);
            acc += to_f32<BF16>(o4[w] >> 16) * to_f32<BF16>(d4[w] >> 16);
        }
    }
#pragma unroll
    for (int m = LPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, LPR);
    if (live && part == 0) {
        int64_t idx;
        if (a.cu_q) {
            idx = (int64_t)h * rows + t;
        } else {
            const int64_t b = t / a.seqlen_q, i = t % a.seqlen_q;
            idx = (b * a.heads + h) * a.seqlen_q + i;
        }
        a.dsum[idx] = acc;
        // a row without visible keys (LSE = -inf) gets +inf, so that every
        // recomputed probability of it is exp2(-inf) = 0 rather than inf
        const float l = a.lse[idx];
        a.lse2[idx] = l == kNegInf ? __builtin_inff() : l * kLog2e;
    }
    if (a.dq_acc && live) {  // atomic dQ path: clear the accumulator row (all D columns)
        f32x4* z = (f32x4*)(a.dq_acc + (t * a.heads + h) * D + part * 8);
        z[0] = f32x4{0.f, 0.f, 0.f, 0.f};
        z[1] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
}

// Atomic dQ path: dq = scale * dq_acc, rounded to the 16-bit type (columns
// below head_dim only).
template <bool BF16, int D>
__global__ __launch_bounds__(256) void bwd_dq_cvt_kernel(BwdArgs a) {
    constexpr int LPR = D / 8;
    constexpr int RPB = 256 / LPR;
    const int tid = threadIdx.x;
    const int64_t item = (int64_t)blockIdx.x * RPB + tid / LPR;
    const int part = tid % LPR;
    const int64_t rows = a.cu_q ? (int64_t)a.cu_q[a.batch] : (int64_t)a.batch * a.seqlen_q;
    const int64_t t = item / a.heads;
    const int h = (int)(item % a.heads);
    if (t >= rows || part * 8 >= a.head_dim) return;
    const f32x4* src = (const f32x4*)(a.dq_acc + (t * a.heads + h) * D + part * 8);
    const f32x4 x0 = src[0], x1 = src[1];
    const float sc = a.scale;
    u32x4 w;
    w[0] = pack2<BF16>(x0[0] * sc, x0[1] * sc);
    w[1] = pack2<BF16>(x0[2] * sc, x0[3] * sc);
    w[2] = pack2<BF16>(x1[0] * sc, x1[1] * sc);
    w[3] = pack2<BF16>(x1[2] * sc, x1[3] * sc);
    *(u32x4*)((uint16_t*)a.dq + (t * a.heads + h) * a.head_dim + part * 8) = w;
}

// Direct loads of ROWS rows of a [rows, heads, D] tensor (row stride `stride`
// elements, rows past `last` clamped to it) into a swizzled LDS tile, split
// over NW waves: block bi = wave * PER + i covers 1024 bytes.
template <int D, int ROWS, int NW>
struct TileDma {
    static constexpr int CPR = D / 8;
    static constexpr int kBlocks = ROWS * D * 2 / 1024;
    static constexpr int kPerWave = kBlocks / NW;
    static constexpr int kRowsPerBlock = 1024 / (D * 2);
    static_assert(kBlocks % NW == 0, "tile must split evenly into 1 KiB blocks per wave");
    // The lane's row in block i is row0 + i * kRowsPerBlock; its offsets are
    // recomputed at each issue (a few integer operations) rather than kept in
    // registers for the whole kernel.
    int row0, slot, last_chunk;
    // dh: the tensor's row length (multiple of 8, at most D); slots past it
    // receive the row's last valid chunk again
    __device__ __forceinline__ void init(int wave, int lane, int dh) {
        row0 = wave * kPerWave * kRowsPerBlock + lane / CPR;
        slot = lane % CPR;
        last_chunk = dh / 8 - 1;
    }
    // g: first row of the tile in global memory; last: last valid row index
    // relative to g (rows beyond are clamped); tail: whether clamping applies.
    __device__ __forceinline__ void issue(const uint16_t* g, uint16_t* tile, int wave, int stride,
                                          bool tail, int last) const {
        const rsrc_t src = buffer_of(g);
#pragma unroll
        for (int i = 0; i < kPerWave; ++i) {
            const int r = row0 + i * kRowsPerBlock;
            const int rg = tail && r > last ? last : r;
            const int off = rg * stride + min(slot ^ swz<CPR>(r), last_chunk) * 8;
            dma16(src, (uint32_t)off * 2u, tile + (wave * kPerWave + i) * 512);
        }
    }
};

// ---------------------------------------------------------------------------
// dQ: one workgroup per (batch, query head, BM-row tile); NW waves x 32 rows,
// WPE waves per SIMD (launch shapes at launch_dq).  Per key tile and wave:
//   S^T = K Q^T, dP^T = V dO^T     (A from the K / V tiles, B resident)
//   P^T = exp2(c S^T - lse2), dS^T = P^T o (dP^T - D)   (one query per lane)
//   dQ^T += K^T dS^T              (K^T from transposing reads of the K tile)
// ---------------------------------------------------------------------------
template <int D, int NW, int BN>
struct DqCfg {
    static constexpr int tileElems = BN * D;
    static constexpr int stageElems = 2 * tileElems;  // K then V
};

template <bool BF16, int D, int NW, int BN, bool DROP, int WPE>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * NW, 64 * NW), amdgpu_waves_per_eu(WPE, WPE)))
void bwd_dq_kernel(BwdArgs a) {
    using C = DqCfg<D, NW, BN>;
    using Dma = TileDma<D, BN, NW>;
    constexpr int KS = D / 16, DB = D / 32, KB = BN / 32, CPR = D / 8;
    constexpr int BM = 32 * NW;
    // separate objects per stage (no waits on the other stage's direct loads)
    __shared__ __attribute__((aligned(16))) uint16_t lds0[C::stageElems];
    __shared__ __attribute__((aligned(16))) uint16_t lds1[C::stageElems];
    auto stage = [&](int buf) { return buf ? lds1 : lds0; };

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
    const int dh = a.head_dim;
    const int64_t q_stride = (int64_t)a.heads * dh;
    const int kv_stride = a.kv_heads * dh;
    const uint16_t* qbase = (const uint16_t*)a.q + (s.q_start * a.heads + h) * dh;
    const uint16_t* dobase = (const uint16_t*)a.dout + (s.q_start * a.heads + h) * dh;
    const uint16_t* kbase = (const uint16_t*)a.k + (s.k_start * a.kv_heads + hk) * dh;
    const uint16_t* vbase = (const uint16_t*)a.v + (s.k_start * a.kv_heads + hk) * dh;
    const int64_t rowidx0 = a.cu_q ? (int64_t)h * a.cu_q[a.batch] + s.q_start
                                   : ((int64_t)b * a.heads + h) * a.seqlen_q;

    const int i_last = min(i0 + BM, s.len_q) - 1;
    const int key_lo = mk.lo_of(i0, s), key_hi = mk.hi_of(i_last, s);
    const int t_lo = key_lo / BN;
    const int t_hi = key_hi >= key_lo ? key_hi / BN + 1 : t_lo;

    const int wq0 = i0 + 32 * wave;
    const int wq1 = min(wq0 + 31, s.len_q - 1);
    const bool wave_live = wq0 < s.len_q;
    const int w_key_lo = wave_live ? mk.lo_of(wq0, s) : 0;
    const int w_key_hi = wave_live ? mk.hi_of(wq1, s) : -1;
    const int w_full_lo = wave_live ? mk.lo_of(wq1, s) : 0;
    const int w_full_hi = wave_live ? mk.hi_of(wq0, s) : -1;

    const int row = wq0 + r32;
    const bool row_ok = row < s.len_q;
    u32x4 qf[KS], dof[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const bool ok = row_ok && ks * 16 + 8 * half < dh;
        qf[ks] = ok ? *(const u32x4*)(qbase + (int64_t)row * q_stride + ks * 16 + 8 * half) : u32x4{0, 0, 0, 0};
        dof[ks] = ok ? *(const u32x4*)(dobase + (int64_t)row * q_stride + ks * 16 + 8 * half) : u32x4{0, 0, 0, 0};
    }
    const float lse2 = row_ok ? a.lse2[rowidx0 + row] : __builtin_inff();  // +inf: P = 0 on padding rows
    const float dsum = row_ok ? a.dsum[rowidx0 + row] : 0.f;
    const int row_lo = mk.lo_of(row, s), row_hi = mk.hi_of(row, s);

    Dma dma;
    dma.init(wave, lane, dh);
    int k_rd[KS];  // A operand reads of the K / V tiles: row r32, chunk 2 ks + half
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) k_rd[ks] = r32 * D + (((2 * ks + half) ^ swz<CPR>(r32)) * 8);
    int kt_rd[2][DB];  // K^T operand (transposing reads)
    tr_offsets<D, DB>(lane, kt_rd);

    f32x16 dq[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) dq[db] = f32x16{0};
    const float c = a.scale_log2;

    auto issue_tile = [&](int t, int buf) {
        const int key0 = t * BN;
        const bool tail = key0 + BN > s.len_k;
        const int last = s.len_k - 1 - key0;
        uint16_t* st = stage(buf);
        const int64_t toff = (int64_t)key0 * kv_stride;
        dma.issue(kbase + toff, st, wave, kv_stride, tail, last);
        dma.issue(vbase + toff, st + C::tileElems, wave, kv_stride, tail, last);
    };

    // One key tile, as KB blocks of 32 keys in a three-stage pipeline of
    // phases: phase ph multiplies S^T, dP^T of block ph, computes P^T, dS^T of
    // block ph-1 and accumulates dQ^T += K^T dS^T of block ph-2, one k-step at a
    // time (each k-step: one S/dP product pair, one dQ product, and a slice of
    // the exponentials), so the matrix cores and the vector ALU of one wave
    // work side by side.  Operands are read one k-step ahead of their products.
    auto compute = [&](int t, int buf) {
        const int key0 = t * BN;
        if (!(wave_live && key0 <= w_key_hi && key0 + BN - 1 >= w_key_lo)) return;
        const uint16_t* kt = stage(buf);
        const uint16_t* vt = kt + C::tileElems;
        // lane column = query row; register i = key key0 + kb*32 + 8(i/4) + 4 half + i%4
        const bool masked = key0 < w_full_lo || key0 + BN - 1 > w_full_hi;  // uniform
        const int lo = row_lo - key0, hi = row_hi - key0;
        constexpr int KPM = KS > 8 ? KS / 8 : 1;   // k-steps per slot of exponentials
        constexpr int MPS = KS >= 8 ? 1 : 8 / KS;  // register pairs per slot
        static_assert(2 * DB == KS, "one dQ product per k-step");
        f32x16 sacc[KB], dpacc[KB];
        uint32_t dsp[KB][8];
        u32x4 ka[2], va[2], tq[2];  // S / dP operands and dQ operands, double-buffered
        u32x4 kw;                   // dropout keep words of the block in the exponential stage
        auto load_sd = [&](int kb, int ks, int slot) {
            ka[slot] = *(const u32x4*)(kt + kb * 32 * D + k_rd[ks]);
            va[slot] = *(const u32x4*)(vt + kb * 32 * D + k_rd[ks]);
        };
        // dQ product j of block kb: key k-step 2 kb + j / DB, output block j % DB
        auto load_q = [&](int kb, int j, int slot) {
            tq[slot] = read_tr<D, DB>(kt, 2 * kb + j / DB, j % DB, kt_rd);
        };
        auto pair = [&](int kb, int m) {  // P, dS of registers 2m, 2m + 1 of block kb
            const int i = 2 * m;
            float p0 = exp2_prob(__builtin_fmaf(sacc[kb][i], c, -lse2));
            float p1 = exp2_prob(__builtin_fmaf(sacc[kb][i + 1], c, -lse2));
            if (masked) {
                const int k0 = kb * 32 + 8 * (i / 4) + 4 * half + (i % 4);
                p0 = (k0 < lo || k0 > hi) ? 0.f : p0;
                p1 = (k0 + 1 < lo || k0 + 1 > hi) ? 0.f : p1;
            }
            float dp0 = dpacc[kb][i], dp1 = dpacc[kb][i + 1];
            if constexpr (DROP) {
                dp0 = keep_byte(kw[i / 4], i % 4, a.drop_t) ? dp0 * a.drop_scale : 0.f;
                dp1 = keep_byte(kw[i / 4], (i + 1) % 4, a.drop_t) ? dp1 * a.drop_scale : 0.f;
            }
            dsp[kb][m] = pack2<BF16>(p0 * (dp0 - dsum), p1 * (dp1 - dsum));
        };
#pragma unroll
        for (int ph = 0; ph <= KB + 1; ++ph) {
            const int bs = ph, bv = ph - 1, bp = ph - 2;  // S/dP, exponential and dQ blocks
            const bool hs = bs < KB, hv = bv >= 0 && bv < KB, hp = bp >= 0;
            if constexpr (DROP) {
                if (hv) {  // keep words of this lane's query row, as in the forward
                    const uint32_t jq = (uint32_t)(key0 + 32 * bv) / 4 + 2 * (r32 & 3) + half;
                    kw = quad_transpose(philox4x32_10(jq, (uint32_t)row / 4, h, b, a.seed_lo, a.seed_hi));
                }
            }
            if (hs) load_sd(bs, 0, 0);
            if (hp) load_q(bp, 0, 0);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                if (hs && ks + 1 < KS) load_sd(bs, ks + 1, (ks + 1) & 1);
                if (hp && ks + 1 < KS) load_q(bp, ks + 1, (ks + 1) & 1);
                __builtin_amdgcn_sched_barrier(0);
                if (hs) {
                    sacc[bs] = mfma32<BF16>(ka[ks & 1], qf[ks], ks ? sacc[bs] : f32x16{0});
                    dpacc[bs] = mfma32<BF16>(va[ks & 1], dof[ks], ks ? dpacc[bs] : f32x16{0});
                }
                if (hp) {
                    const int j = ks, hsel = j / DB, db = j % DB;
                    const u32x4 sb = u32x4{dsp[bp][4 * hsel], dsp[bp][4 * hsel + 1], dsp[bp][4 * hsel + 2],
                                           dsp[bp][4 * hsel + 3]};
                    dq[db] = mfma32<BF16>(tq[ks & 1], sb, dq[db]);
                }
                if (hv && ks % KPM == 0) {
                    const int m0 = (ks / KPM) * MPS;
#pragma unroll
                    for (int m = m0; m < m0 + MPS; ++m) pair(bv, m);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };

    auto step = [&](int t, int buf) {
        const bool has_next = t + 1 < t_hi;
        if (has_next) issue_tile(t + 1, buf ^ 1);
        compute(t, buf);
        wait_vmcnt<0>();  // this wave's direct loads have landed
        __syncthreads();
    };
    if (t_lo < t_hi) {
        issue_tile(t_lo, 0);
        wait_vmcnt<0>();
        __syncthreads();
        for (int t = t_lo; t < t_hi; t += 2) {
            step(t, 0);
            if (t + 1 < t_hi) step(t + 1, 1);
        }
    }
    if (!row_ok) return;
    uint16_t* dqrow = (uint16_t*)a.dq + ((s.q_start + row) * a.heads + h) * dh;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
            const int col = db * 32 + 8 * gq + 4 * half;  // four columns, all below dh or none
            if (col >= dh) continue;
            u32x2 w;
            w.x = pack2<BF16>(dq[db][4 * gq] * a.scale, dq[db][4 * gq + 1] * a.scale);
            w.y = pack2<BF16>(dq[db][4 * gq + 2] * a.scale, dq[db][4 * gq + 3] * a.scale);
            *(u32x2*)(dqrow + col) = w;
        }
}

// ---------------------------------------------------------------------------
// dK, dV: one workgroup per (batch, kv head, 128-key tile); 4 waves x 32 keys,
// one wave per SIMD (the dK/dV accumulators live beside resident K^T / V^T
// operand fragments).  Per streamed 128-row query tile (four 32-row blocks) and wave:
//   S = Q K^T, dP = dO V^T      (A from the Q / dO tiles, B resident)
//   P = exp2(c S - lse2), dS = P o (dP - D)      (one key per lane column)
//   dV^T += dO^T P, dK^T += Q^T dS   (A from transposing reads of the tiles)
// ---------------------------------------------------------------------------
constexpr int kKvWaves = 4;
constexpr int kKvBN = 32 * kKvWaves;  // keys per workgroup
constexpr int kKvBM = 128;            // query rows per streamed tile
constexpr int kKvQB = kKvBM / 32;     // 32-row blocks per tile

// dK/dV waves per SIMD at width 64: two (with one k-step of operand reads
// ahead, 256 registers), measured faster than one at 128 + 126 AGPRs.
#ifndef FA_DKDV64_WPE
#define FA_DKDV64_WPE 2
#endif
#ifndef FA_DKDV_PF_2W
#define FA_DKDV_PF_2W 1
#endif

template <int D, int BMR>
struct DkdvCfg {
    static constexpr int tileElems = BMR * D;
    // per stage: Q tile, dO tile (16-bit), then lse2[BMR], D[BMR] (fp32)
    static constexpr int stageBytes = 2 * tileElems * 2 + 2 * BMR * 4;
};

// D: tile width of the contraction over head_dim (S, dP); DO: the dK / dV
// columns one workgroup accumulates, columns DO * blockIdx.z .. + DO - 1
// (DO = D, except at width 256, where the accumulators of all 256 columns and
// the resident K^T / V^T do not fit the register file together: two
// workgroups per key tile, each recomputing S and dP); BMR: query rows per
// streamed tile (64 at width 256, so that two stages fit in LDS).
template <bool BF16, int D, bool DROP, int DO, int BMR, int WPE>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(WPE, WPE)))
void bwd_dkdv_kernel(BwdArgs a) {
    using C = DkdvCfg<D, BMR>;
    using Dma = TileDma<D, BMR, kKvWaves>;
    constexpr int KS = D / 16, DB = DO / 32, CPR = D / 8;
    const int c0 = (int)blockIdx.z * DO;  // first dK / dV column of this workgroup
    // separate objects per stage (no waits on the other stage's direct loads)
    __shared__ __attribute__((aligned(16))) uint8_t lds0[C::stageBytes];
    __shared__ __attribute__((aligned(16))) uint8_t lds1[C::stageBytes];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r32 = lane & 31, half = lane >> 5;
    const int g = a.heads / a.kv_heads;
    const int col = rotated_column();
    const int b = col / a.kv_heads, hk = col % a.kv_heads;
    const Seq s = seq_of(b, a.cu_q, a.cu_k, a.used_q, a.used_k, a.seqlen_q, a.seqlen_k);
    const int j0 = blockIdx.y * kKvBN;
    if (j0 >= s.len_k) return;
    const Mask mk{a.causal, a.left, a.right};
    const int j1 = min(j0 + kKvBN, s.len_k) - 1;

    const int dh = a.head_dim;
    const int q_stride = a.heads * dh, kv_stride = a.kv_heads * dh;
    const uint16_t* kbase = (const uint16_t*)a.k + (s.k_start * a.kv_heads + hk) * dh;
    const uint16_t* vbase = (const uint16_t*)a.v + (s.k_start * a.kv_heads + hk) * dh;
    const int64_t total_q = a.cu_q ? (int64_t)a.cu_q[a.batch] : 0;

    // Query rows that see any key of this tile.
    int i_lo = 0, i_hi = s.len_q - 1;
    if (a.causal) i_lo = max(i_lo, j0 - s.off);
    if (a.right >= 0) i_lo = max(i_lo, j0 - s.off - a.right);
    if (a.left >= 0) i_hi = min(i_hi, j1 - s.off + a.left);
    const int it_lo = i_lo / BMR;
    const int it_hi = i_hi >= i_lo ? i_hi / BMR + 1 : it_lo;
    const int nt = it_hi - it_lo;  // tiles per head

    // This wave's keys and, per lane, the query rows that see its key.
    const int kw0 = j0 + 32 * wave;
    const int kw1 = min(kw0 + 31, s.len_k - 1);
    const bool wave_live = kw0 < s.len_k;
    const int key = kw0 + r32;
    int q_lo = 0, q_hi = s.len_q - 1;  // visible iff q_lo <= query <= q_hi
    if (a.causal) q_lo = max(q_lo, key - s.off);
    if (a.right >= 0) q_lo = max(q_lo, key - s.off - a.right);
    if (a.left >= 0) q_hi = min(q_hi, key - s.off + a.left);
    if (key >= s.len_k) q_hi = -1;
    u32x4 kf[KS], vf[KS];  // K^T, V^T B operands: lane column = key
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const bool ok = key < s.len_k && ks * 16 + 8 * half < dh;
        kf[ks] = ok ? *(const u32x4*)(kbase + (int64_t)key * kv_stride + ks * 16 + 8 * half) : u32x4{0, 0, 0, 0};
        vf[ks] = ok ? *(const u32x4*)(vbase + (int64_t)key * kv_stride + ks * 16 + 8 * half) : u32x4{0, 0, 0, 0};
    }
    f32x16 dk[DB], dv[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) { dk[db] = f32x16{0}; dv[db] = f32x16{0}; }
    const float c = a.scale_log2;

    Dma dma;
    dma.init(wave, lane, dh);
    int q_rd[KS];  // A operand reads of the Q / dO tiles: row r32 (+32 qb), chunk 2 ks + half
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) q_rd[ks] = r32 * D + (((2 * ks + half) ^ swz<CPR>(r32)) * 8);
    int t_rd[2][DB];  // Q^T / dO^T operands (transposing reads) of columns c0 ..
    tr_offsets<D, DB>(lane, t_rd);
#pragma unroll
    for (int inst = 0; inst < 2; ++inst)
#pragma unroll
        for (int db = 0; db < DB; ++db) t_rd[inst][db] += c0;  // c0 / 8 is a multiple of 16: above the swizzle

    auto q_lds = [&](int buf) { return (uint16_t*)(buf ? lds1 : lds0); };
    auto lse_lds = [&](int buf) { return (float*)((buf ? lds1 : lds0) + 2 * C::tileElems * 2); };

    // Flattened (query head in group, query tile) sequence n = 0 .. g*nt-1.
    auto issue_step = [&](int n, int buf) {
        const int h = hk * g + n / nt;
        const int row0 = (it_lo + n % nt) * BMR;
        const bool tail = row0 + BMR > s.len_q;
        const int last = s.len_q - 1 - row0;
        const int64_t hoff = (s.q_start * a.heads + h) * dh + (int64_t)row0 * q_stride;
        uint16_t* qt = q_lds(buf);
        dma.issue((const uint16_t*)a.q + hoff, qt, wave, q_stride, tail, last);
        dma.issue((const uint16_t*)a.dout + hoff, qt + C::tileElems, wave, q_stride, tail, last);
        constexpr int kRowLoads = BMR / 64;  // 4-byte direct loads (64 rows each) per array
        static_assert(2 * kRowLoads <= kKvWaves, "one row-term load per wave");
        if (wave < 2 * kRowLoads) {  // lse2 rows, then D rows
            const int arr = wave / kRowLoads, part = wave % kRowLoads;
            const int64_t idx0 = a.cu_q ? (int64_t)h * total_q + s.q_start + row0
                                        : ((int64_t)b * a.heads + h) * a.seqlen_q + row0;
            const float* src = (arr == 0 ? a.lse2 : a.dsum) + idx0;
            dma4(buffer_of(src), (uint32_t)min(64 * part + lane, last) * 4u, lse_lds(buf) + arr * BMR + 64 * part);
        }
    };

    // One step covers a BMR-row query tile as (BMR / 32) blocks of 32 rows,
    // software-pipelined over the blocks: phase ph multiplies S, dP of block
    // ph and dV, dK of block ph-2 beside the softmax arithmetic (P, dS) of
    // block ph-1, so the matrix cores and the vector ALU work side by side and
    // no MFMA waits on an LDS read issued just before it (operands are read
    // kPf k-steps ahead; the next phase's first reads and the row terms of the
    // next softmax block are issued during the current phase).  Scheduling
    // fences keep this order.  P and dS are computed unmasked; on tiles where
    // not every (row, key) pair is visible (full == false, uniform) the packed
    // 16-bit words are ANDed with the visibility mask before their products, a
    // branch that touches nothing but those words.  Masked entries of rows
    // without any visible key give inf or NaN before the AND, never after.
    auto compute = [&](int n, int buf, bool full) {
        constexpr int QBS = (BMR / 32);
        // k-steps of operand reads ahead of their MFMAs (one when a second
        // wave per SIMD hides the LDS latency and the registers are short)
        constexpr int kPf = WPE > 1 ? FA_DKDV_PF_2W : 2;
        constexpr int NJ = 4 * DB;      // dV, dK products per block
        constexpr int JPS = NJ / KS;    // dV, dK products per k-step
        constexpr int KPM = KS > 8 ? KS / 8 : 1;  // k-steps per softmax slot
        constexpr int MPS = KS >= 8 ? 1 : 8 / KS;  // softmax register pairs per slot
        const int row0 = (it_lo + n % nt) * BMR;
        const uint16_t* qt = q_lds(buf);
        const uint16_t* dot = qt + C::tileElems;
        const float* lses = lse_lds(buf);
        const float* dss = lses + BMR;
        const int lo = q_lo - row0, hi = q_hi - row0;

        const int hq = hk * g + n / nt;  // query head of this step
        // Dropout keep words of the softmax block: word g_ holds the draws of
        // this lane's key for query rows 8 g_ + 4 half + 0..3 of the block, one
        // byte per row.
        u32x4 kwd;
        auto keep_words = [&](int qb) {
            const uint32_t iq = (uint32_t)(row0 + 32 * qb) / 4 + 2 * (r32 & 3) + half;
            return quad_transpose(
                byte_transpose(philox4x32_10((uint32_t)key / 4, iq, hq, b, a.seed_lo, a.seed_hi)));
        };
        f32x16 sacc[QBS], dpacc[QBS];
        u32x4 qa[QBS][KS], da[QBS][KS];  // A operands Q, dO of each block (row r32, k-step ks)
        f32x4 l4[QBS][4], d4[QBS][4];    // lse2 and D of the rows of register group gq
        uint32_t pp[QBS][8], dsp[QBS][8];
        u32x4 tra[QBS][NJ];              // X^T operands of the dV, dK products, in issue order

        auto load_ops = [&](int qb, int ks) {
            qa[qb][ks] = *(const u32x4*)(qt + qb * 32 * D + q_rd[ks]);
            da[qb][ks] = *(const u32x4*)(dot + qb * 32 * D + q_rd[ks]);
        };
        auto load_rows = [&](int qb, int gq) {
            const int rb = qb * 32 + 8 * gq + 4 * half;
            l4[qb][gq] = *(const f32x4*)(lses + rb);
            d4[qb][gq] = *(const f32x4*)(dss + rb);
        };
        // product j of a block: k-step kk = 2 qb + j / (2 DB), M block (j / 2) % DB,
        // even j: dV^T += dO^T P, odd j: dK^T += Q^T dS
        auto load_tr = [&](int qb, int j) {
            const int kk = 2 * qb + j / (2 * DB), db = (j / 2) % DB;
            tra[qb][j] = read_tr<D, DB>((j & 1) ? qt : dot, kk, db, t_rd);
        };
        auto prod = [&](int qb, int j) {
            const int hs = j / (2 * DB), db = (j / 2) % DB;
            const uint32_t* src = (j & 1) ? dsp[qb] : pp[qb];
            const u32x4 bop = u32x4{src[4 * hs], src[4 * hs + 1], src[4 * hs + 2], src[4 * hs + 3]};
            if (j & 1) dk[db] = mfma32<BF16>(tra[qb][j], bop, dk[db]);
            else dv[db] = mfma32<BF16>(tra[qb][j], bop, dv[db]);
        };
        auto sdp = [&](int qb, int ks) {
            sacc[qb] = mfma32<BF16>(qa[qb][ks], kf[ks], ks ? sacc[qb] : f32x16{0});
            dpacc[qb] = mfma32<BF16>(da[qb][ks], vf[ks], ks ? dpacc[qb] : f32x16{0});
        };
        // P and dS of registers 2m, 2m + 1 (register i: query row
        // 32 qb + 8 (i / 4) + 4 half + i % 4 of the tile, lane column = key)
        auto softmax_pair = [&](int qb, int m) {
            float pv[2], dv2[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int i = 2 * m + t;
                const float pr = exp2_prob(__builtin_fmaf(sacc[qb][i], c, -l4[qb][i / 4][i % 4]));
                if constexpr (DROP) {
                    const bool kp = keep_byte(kwd[i / 4], i % 4, a.drop_t);
                    pv[t] = kp ? pr : 0.f;
                    dv2[t] = pr * ((kp ? dpacc[qb][i] * a.drop_scale : 0.f) - d4[qb][i / 4][i % 4]);
                } else {
                    pv[t] = pr;
                    dv2[t] = pr * (dpacc[qb][i] - d4[qb][i / 4][i % 4]);
                }
            }
            pp[qb][m] = pack2<BF16>(pv[0], pv[1]);
            dsp[qb][m] = pack2<BF16>(dv2[0], dv2[1]);
        };
        auto mask_block = [&](int qb) {
            // Empty, emits nothing; its side effect keeps the compiler from
            // speculating this edge-tile work out of its branch into every tile.
            asm volatile("");
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                const int r0 = qb * 32 + 8 * (m / 2) + 4 * half + 2 * (m % 2);  // rows of registers 2m, 2m + 1
                const uint32_t keep = ((r0 >= lo && r0 <= hi) ? 0x0000FFFFu : 0u) |
                                      ((r0 + 1 >= lo && r0 + 1 <= hi) ? 0xFFFF0000u : 0u);
                pp[qb][m] &= keep;
                dsp[qb][m] &= keep;
            }
        };

#pragma unroll
        for (int ks = 0; ks < kPf; ++ks) load_ops(0, ks);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ph = 0; ph <= QBS + 1; ++ph) {
            const int bs = ph, bv = ph - 1, bp = ph - 2;  // S/dP, softmax and dV/dK blocks
            const bool hs = bs < QBS, hv = bv >= 0 && bv < QBS, hp = bp >= 0;
            if (hp && !full) mask_block(bp);
            if constexpr (DROP) {
                if (hv) kwd = keep_words(bv);
            }
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                if (hs) sdp(bs, ks);
                if (hp) {
#pragma unroll
                    for (int jj = 0; jj < JPS; ++jj) prod(bp, ks * JPS + jj);
                }
                if (hs && ks + kPf < KS) load_ops(bs, ks + kPf);
                if (hp && ks + kPf < KS) {
#pragma unroll
                    for (int jj = 0; jj < JPS; ++jj) load_tr(bp, (ks + kPf) * JPS + jj);
                }
                // row terms of the softmax block: group gq serves pairs 2 gq, 2 gq + 1,
                // read one group ahead of its first use
                if (ks % KPM == 0) {
                    const int m0 = (ks / KPM) * MPS;  // first pair of this slot
                    if (hv && m0 % 2 == 0 && m0 / 2 + 1 < 4) load_rows(bv, m0 / 2 + 1);
                    if (hv) {
#pragma unroll
                        for (int m = m0; m < m0 + MPS; ++m) softmax_pair(bv, m);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            // first operand reads of the next phase: S/dP of block ph+1, dV/dK of block ph-1
            if (ph + 1 < QBS) {
#pragma unroll
                for (int ks = 0; ks < kPf; ++ks) load_ops(ph + 1, ks);
            }
            if (ph - 1 >= 0 && ph - 1 < QBS) {
#pragma unroll
                for (int j = 0; j < kPf * JPS; ++j) load_tr(ph - 1, j);
            }
            if (ph < QBS) load_rows(ph, 0);  // first row group of the next softmax block
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    const int total = g * nt;
    auto step = [&](int n, int buf) {
        const bool has_next = n + 1 < total;
        if (has_next) issue_step(n + 1, buf ^ 1);
        const int row0 = (it_lo + n % nt) * BMR;
        const int row1 = min(row0 + BMR, s.len_q) - 1;
        // any visible pair between rows [row0, row1] and keys [kw0, kw1]?  (uniform)
        if (wave_live && mk.hi_of(row1, s) >= kw0 && mk.lo_of(row0, s) <= kw1) {
            // all visible: the first row sees the last key and the last row the first key
            const bool full = row0 + BMR <= s.len_q && kw0 + 31 < s.len_k &&
                              mk.hi_of(row0, s) >= kw0 + 31 && mk.lo_of(row0 + BMR - 1, s) <= kw0;
            compute(n, buf, full);
        }
        wait_vmcnt<0>();
        __syncthreads();
    };
    if (total > 0) {
        issue_step(0, 0);
        wait_vmcnt<0>();
        __syncthreads();
        for (int n = 0; n < total; n += 2) {
            step(n, 0);
            if (n + 1 < total) step(n + 1, 1);
        }
    }

    // store dK = scale * dK^T, dV = dV^T (lane column = key, registers = d)
    if (!wave_live || key >= s.len_k) return;
    uint16_t* dkrow = (uint16_t*)a.dk + ((s.k_start + key) * a.kv_heads + hk) * dh;
    uint16_t* dvrow = (uint16_t*)a.dv + ((s.k_start + key) * a.kv_heads + hk) * dh;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
            const int col = c0 + db * 32 + 8 * gq + 4 * half;  // four columns, all below dh or none
            if (col >= dh) continue;
            u32x2 wk, wv;
            wk.x = pack2<BF16>(dk[db][4 * gq] * a.scale, dk[db][4 * gq + 1] * a.scale);
            wk.y = pack2<BF16>(dk[db][4 * gq + 2] * a.scale, dk[db][4 * gq + 3] * a.scale);
            const float sv = DROP ? a.drop_scale : 1.f;
            wv.x = pack2<BF16>(dv[db][4 * gq] * sv, dv[db][4 * gq + 1] * sv);
            wv.y = pack2<BF16>(dv[db][4 * gq + 2] * sv, dv[db][4 * gq + 3] * sv);
            *(u32x2*)(dkrow + col) = wk;
            *(u32x2*)(dvrow + col) = wv;
        }
}

// ---------------------------------------------------------------------------
// dK, dV (and on the atomic path dQ) with producer and consumer waves.
//
// One workgroup per (batch, kv head, 128-key tile), 8 waves, two per SIMD.
// Waves p = 0..3 (producers) and c = p + 4 (consumers) share the 32 keys
// j0 + 32 p ..; the workgroup streams 64-row query tiles (Q, dO and the row
// terms) through three LDS stages and handles them as 32-row blocks, one
// block per iteration, the consumers one block behind the producers:
//   producer, block n:   S = Q K^T, dP = dO V^T        (K^T, V^T resident)
//                        P = exp2(c S - lse2), dS = P o (dP - D), masked,
//                        stored transposed (key rows) into LDS
//   consumer, block n-1: dV^T += dO^T P, dK^T += Q^T dS (accumulators
//                        resident; P, dS read back as B operands)
//                        atomic path: dQ[32 rows][its d-block] = dS K over
//                        the keys of its key group (dS by transposing reads,
//                        K resident), added into dq_acc with float32 atomics
// and one barrier per iteration.  A wave keeps only its role's state, so two
// fit a SIMD (256 registers each) and the SIMD overlaps one wave's softmax
// arithmetic with the other's matrix products.  Only producers load tiles
// (their vmcnt waits count direct loads only); only consumers issue atomics.
// ---------------------------------------------------------------------------
constexpr int kPcBM = 64;  // query rows per streamed tile (two blocks)
#ifndef FA_PC_DET
#define FA_PC_DET 0
#endif
#ifndef FA_PC_PF
#define FA_PC_PF 1
#endif

template <int D>
struct PcCfg {
    static constexpr int tileElems = kPcBM * D;                        // Q or dO tile (16-bit)
    static constexpr int stageBytes = 2 * tileElems * 2 + 2 * kPcBM * 4;  // Q, dO, lse2, D
    static constexpr int xElems = kKvBN * 32;  // P^T or dS^T of one block: [128 keys][32 rows]
    static_assert(2 * tileElems * 2 >= kKvBN * D * 2, "the key tile passes through one stage");
};

// Offset (16-bit elements) of rows 8 g + 4 h .. + 3 of key row kt in a
// [128 keys][32 rows] exchange tile: 16-byte chunk g at slot g ^ ((kt >> 2) & 3),
// and its 8-byte halves swapped on odd 16-key groups.  The 8-byte accesses of
// one half-wave (32 lanes: 32 keys, one h) then cover all 64 banks once.
__device__ __forceinline__ int xch_off(int kt, int g, int h) {
    return kt * 32 + ((g ^ ((kt >> 2) & 3)) * 8) + 4 * (h ^ ((kt >> 4) & 1));
}

template <bool BF16, int D, bool DROP, bool ADQ>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void bwd_pc_kernel(BwdArgs a) {
    using C = PcCfg<D>;
    using Dma = TileDma<D, kPcBM, 4>;  // issued by the four producers
    using KDma = TileDma<D, kKvBN, 4>;
    constexpr int KS = D / 16, DB = D / 32, CPR = D / 8;
    // three stages, separate objects (reads of one never wait on loads into another)
    __shared__ __attribute__((aligned(16))) uint8_t st0[C::stageBytes];
    __shared__ __attribute__((aligned(16))) uint8_t st1[C::stageBytes];
    __shared__ __attribute__((aligned(16))) uint8_t st2[C::stageBytes];
    // P^T and dS^T of a block, by block parity
    __shared__ __attribute__((aligned(16))) uint16_t pt0[C::xElems];
    __shared__ __attribute__((aligned(16))) uint16_t pt1[C::xElems];
    __shared__ __attribute__((aligned(16))) uint16_t dt0[C::xElems];
    __shared__ __attribute__((aligned(16))) uint16_t dt1[C::xElems];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kw = wave & 3;  // key block of this wave
    const int r32 = lane & 31, half = lane >> 5;
    const int g = a.heads / a.kv_heads;
    const int col = rotated_column();
    const int b = col / a.kv_heads, hk = col % a.kv_heads;
    const Seq s = seq_of(b, a.cu_q, a.cu_k, a.used_q, a.used_k, a.seqlen_q, a.seqlen_k);
    const int j0 = blockIdx.y * kKvBN;
    if (j0 >= s.len_k) return;
    const Mask mk{a.causal, a.left, a.right};
    const int j1 = min(j0 + kKvBN, s.len_k) - 1;

    const int dh = a.head_dim;
    const int q_stride = a.heads * dh, kv_stride = a.kv_heads * dh;
    const uint16_t* kbase = (const uint16_t*)a.k + (s.k_start * a.kv_heads + hk) * dh;
    const uint16_t* vbase = (const uint16_t*)a.v + (s.k_start * a.kv_heads + hk) * dh;
    const int64_t total_q = a.cu_q ? (int64_t)a.cu_q[a.batch] : 0;

    // Query rows that see any key of this tile, as whole 64-row tiles.
    int i_lo = 0, i_hi = s.len_q - 1;
    if (a.causal) i_lo = max(i_lo, j0 - s.off);
    if (a.right >= 0) i_lo = max(i_lo, j0 - s.off - a.right);
    if (a.left >= 0) i_hi = min(i_hi, j1 - s.off + a.left);
    const int it_lo = i_lo / kPcBM;
    const int nt = i_hi >= i_lo ? i_hi / kPcBM + 1 - it_lo : 0;  // tiles per query head
    const int ntiles = g * nt;                                      // over the GQA group
    const int nblocks = 2 * ntiles;

    const int kw0 = j0 + 32 * kw;
    const int key = kw0 + r32;
    int q_lo = 0, q_hi = s.len_q - 1;  // this lane's key is visible to rows q_lo .. q_hi
    if (a.causal) q_lo = max(q_lo, key - s.off);
    if (a.right >= 0) q_lo = max(q_lo, key - s.off - a.right);
    if (a.left >= 0) q_hi = min(q_hi, key - s.off + a.left);
    if (key >= s.len_k) q_hi = -1;

    auto stage = [&](int i) -> uint8_t* { return i == 0 ? st0 : (i == 1 ? st1 : st2); };
    auto q_tile = [&](int i) { return (const uint16_t*)stage(i); };
    auto do_tile = [&](int i) { return (const uint16_t*)stage(i) + C::tileElems; };
    auto rows_lds = [&](int i) { return (const float*)(stage(i) + 2 * C::tileElems * 2); };
    auto ptile = [&](int par) { return par ? pt1 : pt0; };
    auto dtile = [&](int par) { return par ? dt1 : dt0; };
    // (query head, first row) of tile t of the sequence; t past the last is
    // clamped to it (its loads then only refill a free stage)
    auto tile_head = [&](int t) { return hk * g + min(t, ntiles - 1) / nt; };
    auto tile_row0 = [&](int t) { return (it_lo + min(t, ntiles - 1) % nt) * kPcBM; };

    if (wave < 4) {
        // =========================== producer ===========================
        Dma dma;
        dma.init(wave, lane, dh);
        const int p = wave;
        u32x4 kf[KS], vf[KS];  // K^T, V^T B operands: lane column = key
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const bool ok = key < s.len_k && ks * 16 + 8 * half < dh;
            kf[ks] = ok ? *(const u32x4*)(kbase + (int64_t)key * kv_stride + ks * 16 + 8 * half) : u32x4{0, 0, 0, 0};
            vf[ks] = ok ? *(const u32x4*)(vbase + (int64_t)key * kv_stride + ks * 16 + 8 * half) : u32x4{0, 0, 0, 0};
        }
        int q_rd[KS];  // A operand reads of the Q / dO tiles: row r32 (+32 blk), chunk 2 ks + half
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) q_rd[ks] = r32 * D + (((2 * ks + half) ^ swz<CPR>(r32)) * 8);
        int x_wr[4];
        const int kt = 32 * p + r32;
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) x_wr[gq] = xch_off(kt, gq, half);
        const float c = a.scale_log2;

        // Tile t into stage st: Q, dO, and the row terms (lse2 by producers 0 and
        // 2, D by 1 and 3: the duplicates write the same bytes, so that every
        // producer issues the same number of loads per tile).
        auto issue_tile = [&](int t, int st) {
            const int h = tile_head(t), row0 = tile_row0(t);
            const bool tail = row0 + kPcBM > s.len_q;
            const int last = s.len_q - 1 - row0;
            const int64_t hoff = (s.q_start * a.heads + h) * dh + (int64_t)row0 * q_stride;
            uint16_t* qt = (uint16_t*)stage(st);
            dma.issue((const uint16_t*)a.q + hoff, qt, p, q_stride, tail, last);
            dma.issue((const uint16_t*)a.dout + hoff, qt + C::tileElems, p, q_stride, tail, last);
            const int64_t idx0 = a.cu_q ? (int64_t)h * total_q + s.q_start + row0
                                        : ((int64_t)b * a.heads + h) * a.seqlen_q + row0;
            const float* src = ((p & 1) ? a.dsum : a.lse2) + idx0;
            dma4(buffer_of(src), (uint32_t)min(lane, last) * 4u, (float*)(stage(st) + 2 * C::tileElems * 2) + (p & 1) * kPcBM);
        };
        constexpr int kOps = 2 * Dma::kPerWave + 1;  // direct loads per tile and producer

        // S = Q K^T and dP = dO V^T of block n (tile n / 2 in stage st, rows
        // 32 (n % 2) .. of it), one k-step per call: operands read two k-steps ahead.
        struct Sdp {
            f32x16 s, dp;
        };
        constexpr int kPfP = FA_PC_PF;  // k-steps of operand reads ahead of their products
        u32x4 qa[KS], da[KS];
        auto sdp_load = [&](int n, int st, int ks) {
            const int blk = n & 1;
            qa[ks] = *(const u32x4*)(q_tile(st) + blk * 32 * D + q_rd[ks]);
            da[ks] = *(const u32x4*)(do_tile(st) + blk * 32 * D + q_rd[ks]);
        };
        auto sdp_step = [&](Sdp& x, int ks) {
            x.s = mfma32<BF16>(qa[ks], kf[ks], ks ? x.s : f32x16{0});
            x.dp = mfma32<BF16>(da[ks], vf[ks], ks ? x.dp : f32x16{0});
        };
        // Iteration n of the producer: S, dP of block n + 1 (when there is one)
        // on the matrix cores, interleaved k-step by k-step with P, dS of block
        // n (from the S, dP the previous iteration left in `cur`) on the vector
        // ALU, so one wave keeps both busy; then block n's P, dS, masked, go to
        // the exchange tiles of parity par.
        auto produce = [&](int n, int st, int st_next, int par, Sdp& cur, Sdp& nxt, bool has_next) {
            // Opaque per iteration: LDS objects past 64 KiB cannot take the
            // instruction's 16-bit offset, so each (lane offset, object) sum
            // costs a register if the compiler hoists it out of the loop;
            // this keeps the additions next to their reads.
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) asm volatile("" : "+v"(q_rd[ks]));
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) asm volatile("" : "+v"(x_wr[gq]));
            const int t = n >> 1, blk = n & 1;
            const int hq = tile_head(t), row0 = tile_row0(t) + 32 * blk;
            const float* lses = rows_lds(st) + 32 * blk;
            const float* dss = lses + kPcBM;
            // row terms of this lane's 16 rows 8 gq + 4 half + 0..3, group gq read
            // one group ahead of its first pair (pairs 2 gq, 2 gq + 1)
            f32x4 l4[4], d4[4];
            auto load_rows = [&](int gq) {
                l4[gq] = *(const f32x4*)(lses + 8 * gq + 4 * half);
                d4[gq] = *(const f32x4*)(dss + 8 * gq + 4 * half);
            };
            load_rows(0);
            u32x4 kwd;
            if constexpr (DROP) {
                const uint32_t iq = (uint32_t)row0 / 4 + 2 * (r32 & 3) + half;
                kwd = quad_transpose(byte_transpose(philox4x32_10((uint32_t)key / 4, iq, hq, b, a.seed_lo, a.seed_hi)));
            }
            uint32_t pp[8], dsp[8];
            // P, dS of register pair m (register i: row 8 (i / 4) + 4 half + i % 4)
            auto pair = [&](int m) {
                if (m % 2 == 0 && m / 2 + 1 < 4) load_rows(m / 2 + 1);
                float pv[2], dv2[2];
#pragma unroll
                for (int t2 = 0; t2 < 2; ++t2) {
                    const int i = 2 * m + t2;
                    const float pr = exp2_prob(__builtin_fmaf(cur.s[i], c, -l4[i / 4][i % 4]));
                    if constexpr (DROP) {
                        const bool kp = keep_byte(kwd[i / 4], i % 4, a.drop_t);
                        pv[t2] = kp ? pr : 0.f;
                        dv2[t2] = pr * ((kp ? cur.dp[i] * a.drop_scale : 0.f) - d4[i / 4][i % 4]);
                    } else {
                        pv[t2] = pr;
                        dv2[t2] = pr * (cur.dp[i] - d4[i / 4][i % 4]);
                    }
                }
                pp[m] = pack2<BF16>(pv[0], pv[1]);
                dsp[m] = pack2<BF16>(dv2[0], dv2[1]);
            };
            constexpr int MPS = 8 / KS > 0 ? 8 / KS : 1;  // softmax pairs per k-step
            // Without a next block the products still run, on this block's own
            // (valid) stage, and their result is never used: no branch splits
            // the k-steps, so the products and the vector work interleave.
            const int nn = has_next ? n + 1 : n;
            const int sn = has_next ? st_next : st;
#pragma unroll
            for (int ks = 0; ks < kPfP && ks < KS; ++ks) sdp_load(nn, sn, ks);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                if (ks + kPfP < KS) sdp_load(nn, sn, ks + kPfP);
                sdp_step(nxt, ks);
#pragma unroll
                for (int m = ks * MPS; m < (ks + 1) * MPS && m < 8; ++m) pair(m);
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int m = KS * MPS; m < 8; ++m) pair(m);
            // visibility: all pairs visible, or AND the words with the mask
            const int lo = q_lo - row0, hi = q_hi - row0;
            const bool full = lo <= 0 && hi >= 31;  // this lane's key sees all 32 rows
            if (__builtin_amdgcn_ballot_w64(!full) != 0) {  // uniform
#pragma unroll
                for (int m = 0; m < 8; ++m) {
                    const int r0 = 8 * (m / 2) + 4 * half + 2 * (m % 2);
                    const uint32_t keep = ((r0 >= lo && r0 <= hi) ? 0x0000FFFFu : 0u) |
                                          ((r0 + 1 >= lo && r0 + 1 <= hi) ? 0xFFFF0000u : 0u);
                    pp[m] &= keep;
                    dsp[m] &= keep;
                }
            }
            uint16_t* ptw = ptile(par);
            uint16_t* dtw = dtile(par);
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                *(u32x2*)(ptw + x_wr[gq]) = u32x2{pp[2 * gq], pp[2 * gq + 1]};
                *(u32x2*)(dtw + x_wr[gq]) = u32x2{dsp[2 * gq], dsp[2 * gq + 1]};
            }
        };

        // prologue: the key tile through stage 2 for the consumers' K operands
        KDma kd;
        kd.init(p, lane, dh);
        kd.issue(kbase + (int64_t)j0 * kv_stride, (uint16_t*)st2, p, kv_stride, j0 + kKvBN > s.len_k, s.len_k - 1 - j0);
        wait_vmcnt<0>();
        lds_barrier();  // (1) key tile in LDS
        lds_barrier();  // (2) consumers have read it
        Sdp sa, sb;     // S, dP of the next block to soften: by iteration parity
        if (ntiles > 0) {
            issue_tile(0, 0);
            issue_tile(1, 1);
            wait_vmcnt<kOps>();  // tile 0 landed
            lds_barrier();       // (3) ... for every producer
            // S, dP of block 0
#pragma unroll
            for (int ks = 0; ks < 2 && ks < KS; ++ks) sdp_load(0, 0, ks);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                if (ks + 2 < KS) sdp_load(0, 0, ks + 2);
                sdp_step(sa, ks);
            }
        } else {
            lds_barrier();  // (3)
        }
        // Iteration n: P, dS of block n (n < nblocks) and S, dP of block n + 1.
        // Tile X (blocks 2X, 2X + 1, stage X % 3) is loaded from odd iteration
        // 2X - 3 (its stage's previous tile was last read in iteration 2X - 4)
        // and waited for at the end of iteration 2X - 2, before its first S, dP
        // in iteration 2X - 1.  Unrolled by 6 so stages and parities are static.
        for (int n0 = 0; n0 <= nblocks; n0 += 6) {
#pragma unroll
            for (int u = 0; u < 6; ++u) {
                const int n = n0 + u;
                if (n > nblocks) break;
                if (u & 1) issue_tile((n + 3) >> 1, ((u + 3) >> 1) % 3);
                if (n < nblocks) {
                    Sdp& cur = (u & 1) ? sb : sa;
                    Sdp& nxt = (u & 1) ? sa : sb;
                    produce(n, (u >> 1) % 3, ((u + 1) >> 1) % 3, u & 1, cur, nxt, n + 1 < nblocks);
                }
                if (!(u & 1)) wait_vmcnt<0>();  // tile n / 2 + 1 (the last one issued) landed
                lds_barrier();
            }
        }
    } else {
        // =========================== consumer ===========================
        const int cw = wave - 4;
        int t_rd[2][DB];  // transposing reads (X^T operands) of a row-major tile
        tr_offsets<D, DB>(lane, t_rd);
        f32x16 dk[DB], dv[DB];
#pragma unroll
        for (int db = 0; db < DB; ++db) { dk[db] = f32x16{0}; dv[db] = f32x16{0}; }
        int x_rd[2][2];  // B operand reads of P^T / dS^T: k-step kk, chunk 2 kk + e
        {
            const int kt = 32 * cw + r32;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int e = 0; e < 2; ++e) x_rd[kk][e] = xch_off(kt, 2 * kk + e, half);
        }
        // atomic dQ: d-block and key group of this wave, K operands, dS reads
        const int dqb = cw % DB, dkg = cw / DB;
        u32x4 kq[ADQ ? KS : 1];
        int dq_rd[2][2];  // [parity of the 16-key k-step][instruction]
        lds_barrier();  // (1)
        if constexpr (ADQ) {
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) kq[kk] = read_tr<D, DB>((const uint16_t*)st2, KS * dkg + kk, dqb, t_rd);
            const int g4 = lane >> 4, jl = lane & 15;
#pragma unroll
            for (int par = 0; par < 2; ++par)
#pragma unroll
                for (int inst = 0; inst < 2; ++inst) {
                    // key row 16 k + rr, query rows col .. col + 3 (xch_off's layout)
                    const int rr = 8 * inst + 4 * (g4 >> 1) + (jl >> 2);
                    const int col = 16 * (g4 & 1) + 4 * (jl & 3);
                    dq_rd[par][inst] = rr * 32 + (((col >> 3) ^ ((rr >> 2) & 3)) * 8) + 4 * (((col >> 2) & 1) ^ par);
                }
        }
        lds_barrier();  // (2) (waits for the reads above)
        lds_barrier();  // (3)
        const int64_t dq_row_stride = (int64_t)a.heads * D;
        const uint32_t dq_lane = (uint32_t)(4 * half * dq_row_stride) + 32 * dqb + r32;

        auto consume = [&](int m, int st, int par) {
            // lane offsets opaque per iteration (as in the producer)
#pragma unroll
            for (int inst = 0; inst < 2; ++inst)
#pragma unroll
                for (int db = 0; db < DB; ++db) asm volatile("" : "+v"(t_rd[inst][db]));
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int e = 0; e < 2; ++e) asm volatile("" : "+v"(x_rd[kk][e]));
            const int t = m >> 1, blk = m & 1;
            const int hq = tile_head(t), row0 = tile_row0(t) + 32 * blk;
            const uint16_t* qt = q_tile(st);
            const uint16_t* dot = do_tile(st);
            const uint16_t* ptr = ptile(par);
            const uint16_t* dtr = dtile(par);
            auto xread = [&](const uint16_t* x, int kk) {
                const u32x2 lo = *(const u32x2*)(x + x_rd[kk][0]);
                const u32x2 hi = *(const u32x2*)(x + x_rd[kk][1]);
                return u32x4{lo.x, lo.y, hi.x, hi.y};
            };
            auto dsa_read = [&](int kk) {
                typedef short s16x4 __attribute__((ext_vector_type(4)));
                typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
                const int kst = KS * dkg + kk;  // 16-key k-step of the tile
                const uint16_t* x = dtr + kst * 16 * 32;
                const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(x + dq_rd[kst & 1][0]));
                const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(x + dq_rd[kst & 1][1]));
                const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
                return u32x4{l2.x, l2.y, h2.x, h2.y};
            };
            f32x16 dqa = f32x16{0};
            // two k-steps of 16 rows; per k-step DB dV and DB dK products, and
            // (atomic path) KS / 2 dQ products interleaved with them
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const u32x4 pb = xread(ptr, kk), sb = xread(dtr, kk);
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const u32x4 ta = read_tr<D, DB>(dot, 2 * blk + kk, db, t_rd);
                    const u32x4 tb = read_tr<D, DB>(qt, 2 * blk + kk, db, t_rd);
                    dv[db] = mfma32<BF16>(ta, pb, dv[db]);
                    dk[db] = mfma32<BF16>(tb, sb, dk[db]);
                    if constexpr (ADQ) {
                        const int j = kk * DB + db;  // dQ k-step, 0 .. 2 DB - 1 = KS - 1
                        dqa = mfma32<BF16>(dsa_read(j), kq[j], dqa);
                    }
                }
            }
            if constexpr (ADQ) {
                float* dqh = a.dq_acc + ((s.q_start + row0) * a.heads + hq) * (int64_t)D;
                const int last_row = s.len_q - 1 - row0;
                if (31 <= last_row) {
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        unsafeAtomicAdd(dqh + (int64_t)(8 * (i / 4) + (i % 4)) * dq_row_stride + dq_lane, dqa[i]);
                } else {  // tail block: rows past the sequence (dS zero there) clamped to its last row
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int r = min(8 * (i / 4) + 4 * half + (i % 4), last_row);
                        unsafeAtomicAdd(dqh + (int64_t)r * dq_row_stride + 32 * dqb + r32, dqa[i]);
                    }
                }
            }
        };

        for (int n0 = 0; n0 <= nblocks; n0 += 6) {
#pragma unroll
            for (int u = 0; u < 6; ++u) {
                const int n = n0 + u;
                if (n > nblocks) break;
                // block n - 1: tile (n - 1) / 2, stage ((u + 5) % 6 / 2) % 3, parity (n - 1) & 1
                if (n >= 1) consume(n - 1, ((u + 5) % 6) >> 1, (u + 1) & 1);
                lds_barrier();
            }
        }

        // store dK = scale * dK^T, dV = dV^T (lane column = key, registers = d)
        if (kw0 >= s.len_k || key >= s.len_k) return;
        uint16_t* dkrow = (uint16_t*)a.dk + ((s.k_start + key) * a.kv_heads + hk) * dh;
        uint16_t* dvrow = (uint16_t*)a.dv + ((s.k_start + key) * a.kv_heads + hk) * dh;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                const int col = db * 32 + 8 * gq + 4 * half;  // four columns, all below dh or none
                if (col >= dh) continue;
                u32x2 wk, wv;
                wk.x = pack2<BF16>(dk[db][4 * gq] * a.scale, dk[db][4 * gq + 1] * a.scale);
                wk.y = pack2<BF16>(dk[db][4 * gq + 2] * a.scale, dk[db][4 * gq + 3] * a.scale);
                const float sv = DROP ? a.drop_scale : 1.f;
                wv.x = pack2<BF16>(dv[db][4 * gq] * sv, dv[db][4 * gq + 1] * sv);
                wv.y = pack2<BF16>(dv[db][4 * gq + 2] * sv, dv[db][4 * gq + 3] * sv);
                *(u32x2*)(dkrow + col) = wk;
                *(u32x2*)(dvrow + col) = wv;
            }
    }
}

// dQ launch shapes (measured on MI355X, bf16 causal): NW waves of 32 query
// rows, BN-key tiles, WPE waves per SIMD.  Width 128: 4 waves at two per SIMD
// (two workgroups per CU), 64-key tiles: as fast as 8 waves on large grids and
// faster on small ones, which 8-wave workgroups (one per CU) fill unevenly.
// Width 64 without dropout: 4 waves at three per SIMD (168
// registers), 64-key tiles; with dropout that shape spills, so it keeps 8
// waves at two per SIMD with 128-key tiles.  Width 256: 4 waves at one per
// SIMD (the resident Q, dO and the dQ accumulators take 256 registers per
// lane), 64-key tiles (two stages in 128 KiB of LDS; 3% faster than 32-key
// tiles at 8K).  Overridable at build time for tuning.
#ifndef FA_DQ_NW
#define FA_DQ_NW 4
#endif
#ifndef FA_DQ64_NW
#define FA_DQ64_NW 4
#endif
#ifndef FA_DQ64_BN
#define FA_DQ64_BN 64
#endif
#ifndef FA_DQ64_WPE
#define FA_DQ64_WPE 3
#endif

template <int D, bool DROP>
struct DqShape {
    static constexpr bool kNarrow = D == 64 && !DROP;
    static constexpr int NW = D > 128 ? 4 : (kNarrow ? FA_DQ64_NW : (D == 64 ? 8 : FA_DQ_NW));
    static constexpr int BN = D > 128 ? 64 : (kNarrow ? FA_DQ64_BN : (D == 128 ? 64 : 128));
    static constexpr int WPE = D > 128 ? 1 : (kNarrow ? FA_DQ64_WPE : 2);
};

template <bool BF16, int D, bool DROP>
int launch_dq(const BwdArgs& a, hipStream_t stream) {
    using S = DqShape<D, DROP>;
    constexpr int BM = 32 * S::NW;
    const int ntiles = (a.seqlen_q + BM - 1) / BM;
    if (ntiles == 0 || a.batch == 0) return 0;
    hipLaunchKernelGGL((bwd_dq_kernel<BF16, D, S::NW, S::BN, DROP, S::WPE>), dim3(a.batch * a.heads, ntiles),
                       dim3(64 * S::NW), 0, stream, a);
    return hipGetLastError() == hipSuccess ? 0 : 1;
}

template <bool BF16, int D>
int launch_bwd_t(const BwdArgs& a, int stage, hipStream_t stream) {
    if (stage == 0) {  // D_i = dO_i . O_i, lse2_i
        constexpr int RPB = 256 / (D / 8);
        const int64_t items = (int64_t)a.batch * a.seqlen_q * a.heads;
        const int64_t blocks = (items + RPB - 1) / RPB;
        if (blocks > 0) {
            hipLaunchKernelGGL((bwd_rowdot_kernel<BF16, D>), dim3((unsigned)blocks), dim3(256), 0, stream, a);
            if (hipGetLastError() != hipSuccess) return 1;
        }
        return 0;
    }
    if (stage == 1) {  // dK, dV (and dQ into dq_acc on the atomic path)
        const int ntiles = (a.seqlen_k + kKvBN - 1) / kKvBN;
        if (ntiles > 0 && a.batch > 0) {
            // The separate-dQ path runs the one-wave-per-SIMD kernel (measured
            // faster than the producer / consumer kernel without dQ); the atomic
            // path runs the producer / consumer kernel, which forms dQ as well.
            if constexpr (D <= 128) {
                if (a.dq_acc) {
                    auto kern = a.drop_t < 256 ? bwd_pc_kernel<BF16, D, true, true> : bwd_pc_kernel<BF16, D, false, true>;
                    hipLaunchKernelGGL(kern, dim3(a.batch * a.kv_heads, ntiles), dim3(512), 0, stream, a);
                    return hipGetLastError() == hipSuccess ? 0 : 1;
                }
                if (FA_PC_DET) {  // build-time switch for measurement: the separate-dQ path on the same kernel
                    auto kern = a.drop_t < 256 ? bwd_pc_kernel<BF16, D, true, false> : bwd_pc_kernel<BF16, D, false, false>;
                    hipLaunchKernelGGL(kern, dim3(a.batch * a.kv_heads, ntiles), dim3(512), 0, stream, a);
                    return hipGetLastError() == hipSuccess ? 0 : 1;
                }
            }
            constexpr int DO = D > 128 ? 128 : D, BMR = D > 128 ? 64 : kKvBM;
            constexpr int WPE = D == 64 ? FA_DKDV64_WPE : 1;
            auto kern = a.drop_t < 256 ? bwd_dkdv_kernel<BF16, D, true, DO, BMR, WPE>
                                       : bwd_dkdv_kernel<BF16, D, false, DO, BMR, WPE>;
            hipLaunchKernelGGL(kern, dim3(a.batch * a.kv_heads, ntiles, D / DO), dim3(256), 0, stream, a);
            if (hipGetLastError() != hipSuccess) return 1;
        }
        return 0;
    }
    if (a.dq_acc) {  // stage 2 of the atomic path: dq = scale * dq_acc
        constexpr int RPB = 256 / (D / 8);
        const int64_t items = (int64_t)a.batch * a.seqlen_q * a.heads;
        const int64_t blocks = (items + RPB - 1) / RPB;
        if (blocks > 0) {
            hipLaunchKernelGGL((bwd_dq_cvt_kernel<BF16, D>), dim3((unsigned)blocks), dim3(256), 0, stream, a);
            if (hipGetLastError() != hipSuccess) return 1;
        }
        return 0;
    }
    // stage 2: dQ
    return a.drop_t < 256 ? launch_dq<BF16, D, true>(a, stream) : launch_dq<BF16, D, false>(a, stream);
}

}  // namespace

int launch_bwd(const BwdArgs& a, int stage, hipStream_t stream) {
    // tile width: the smallest of 64, 128, 256 holding head_dim
    if (a.head_dim > 128)
        return a.bf16 ? launch_bwd_t<true, 256>(a, stage, stream) : launch_bwd_t<false, 256>(a, stage, stream);
    if (a.bf16)
        return a.head_dim > 64 ? launch_bwd_t<true, 128>(a, stage, stream) : launch_bwd_t<true, 64>(a, stage, stream);
    return a.head_dim > 64 ? launch_bwd_t<false, 128>(a, stage, stream) : launch_bwd_t<false, 64>(a, stage, stream);
}

}  // namespace fa
