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
// Three kernels on one stream:
//   bwd_rowdot   D_i = dO_i . O_i                         (HBM-bound)
//   bwd_dkdv     per key tile (outer) and every visible query tile of every
//                query head of the GQA group (inner): dK, dV accumulated in
//                registers, no atomics
//   bwd_dq       per query tile (outer) over the visible key tiles (inner):
//                the separate dQ accumulation pass, no atomics
// Both main kernels double-buffer their streamed tiles in LDS like the
// forward.  Operand orientation follows the MFMA C layout (fa_device.hpp):
// the dK/dV pass computes S = Q K^T with one key per lane column, so P and dS
// feed dV^T = dO^T P and dK^T = Q^T dS directly; the dQ pass computes
// S^T = K Q^T with one query per lane column, so dS^T feeds dQ^T = K^T dS^T.
#include <type_traits>

#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {

namespace {

constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------------------
// D_i = dO_i . O_i
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
    if (live) {
        const int64_t off = (t * a.heads + h) * D + part * 8;
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
    }
}

// Loads a 64-row x D tile of a row-major [rows, heads, D] tensor as
// (4-row x 8-column) pieces: thread -> rows 4*rc .. 4*rc+3, columns 8*dc ..
// 8*dc+7.  Rows outside [0, nrows) read as zero.
template <int D, int ROWS>
struct Piece {
    static constexpr int kRowChunks = ROWS / 4;
    static constexpr int kItems = kRowChunks * (D / 8);
    static_assert(kItems <= 256, "one piece per thread");
    u32x4 r[4];
    __device__ __forceinline__ void load(const uint16_t* base, int64_t stride, int row0, int nrows, int tid) {
        if (tid >= kItems) return;
        const int rc = tid % kRowChunks, dc = tid / kRowChunks;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int row = row0 + 4 * rc + k;
            r[k] = row < nrows ? *(const u32x4*)(base + (int64_t)row * stride + dc * 8) : u32x4{0, 0, 0, 0};
        }
    }
    // row-major copy: lds[row * stride + col]
    __device__ __forceinline__ void store_rows(uint16_t* lds, int stride, int tid) const {
        if (tid >= kItems) return;
        const int rc = tid % kRowChunks, dc = tid / kRowChunks;
#pragma unroll
        for (int k = 0; k < 4; ++k) *(u32x4*)(lds + (4 * rc + k) * stride + dc * 8) = r[k];
    }
    // transposed copy in the permuted row order: lds[col * stride + perm(row)]
    __device__ __forceinline__ void store_cols(uint16_t* lds, int stride, int tid) const {
        if (tid >= kItems) return;
        const int rc = tid % kRowChunks, dc = tid / kRowChunks;
        u32x2 cols[8];
        transpose4x8(r[0], r[1], r[2], r[3], cols);
        const int pos = perm_chunk_pos(rc);
#pragma unroll
        for (int e = 0; e < 8; ++e) *(u32x2*)(lds + (dc * 8 + e) * stride + pos) = cols[e];
    }
};

// ---------------------------------------------------------------------------
// dK, dV: one workgroup per (batch, kv head, 128-key tile); 4 waves x 32 keys
// ---------------------------------------------------------------------------
constexpr int kKvWaves = 4;
constexpr int kKvBN = 32 * kKvWaves;  // keys per workgroup
constexpr int kKvBM = 64;             // query rows per streamed tile

template <int D>
struct DkdvSmem {
    static constexpr int rStride = D + 8;        // row-major Q / dO
    static constexpr int cStride = kKvBM + 8;    // transposed Q^T / dO^T (per d)
    static constexpr int rElems = kKvBM * rStride;
    static constexpr int cElems = D * cStride;
    // per stage: Q, dO (row-major), Q^T, dO^T (permuted), LSE*log2e, D
    static constexpr int stageBytes = (2 * rElems + 2 * cElems) * 2 + 2 * kKvBM * 4;
    static constexpr int bytes = 2 * stageBytes;
};

template <bool BF16, int D>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void bwd_dkdv_kernel(BwdArgs a) {
    using SM = DkdvSmem<D>;
    using P = Piece<D, kKvBM>;
    constexpr int KS = D / 16, DB = D / 32;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem_raw[];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r32 = lane & 31, half = lane >> 5;
    const int g = a.heads / a.kv_heads;
    const int b = blockIdx.x / a.kv_heads, hk = blockIdx.x % a.kv_heads;
    const Seq s = seq_of(b, a.cu_q, a.cu_k, a.seqlen_q, a.seqlen_k);
    const int j0 = blockIdx.y * kKvBN;
    if (j0 >= s.len_k) return;
    const Mask mk{a.causal, a.left, a.right};
    const int j1 = min(j0 + kKvBN, s.len_k) - 1;

    const int64_t q_stride = (int64_t)a.heads * D, kv_stride = (int64_t)a.kv_heads * D;
    const uint16_t* kbase = (const uint16_t*)a.k + (s.k_start * a.kv_heads + hk) * D;
    const uint16_t* vbase = (const uint16_t*)a.v + (s.k_start * a.kv_heads + hk) * D;
    const int64_t total_q = a.cu_q ? (int64_t)a.cu_q[a.batch] : 0;

    // Query rows that see any key of this tile.
    int i_lo = 0, i_hi = s.len_q - 1;
    if (a.causal) i_lo = max(i_lo, j0 - s.off);
    if (a.right >= 0) i_lo = max(i_lo, j0 - s.off - a.right);
    if (a.left >= 0) i_hi = min(i_hi, j1 - s.off + a.left);
    const int it_lo = i_lo / kKvBM;
    const int it_hi = i_hi >= i_lo ? i_hi / kKvBM + 1 : it_lo;
    const int nt = it_hi - it_lo;  // tiles per head

    // This wave's keys, resident as B operands (K^T and V^T fragments).
    const int kw0 = j0 + 32 * wave;
    const int kw1 = min(kw0 + 31, s.len_k - 1);
    const bool wave_live = kw0 < s.len_k;
    u32x4 kf[KS], vf[KS];
    {
        const int key = kw0 + r32;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const bool ok = key < s.len_k;
            kf[ks] = ok ? *(const u32x4*)(kbase + (int64_t)key * kv_stride + ks * 16 + 8 * half) : u32x4{0, 0, 0, 0};
            vf[ks] = ok ? *(const u32x4*)(vbase + (int64_t)key * kv_stride + ks * 16 + 8 * half) : u32x4{0, 0, 0, 0};
        }
    }
    f32x16 dk[DB], dv[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) { dk[db] = f32x16{0}; dv[db] = f32x16{0}; }
    const float c = a.scale_log2;

    auto stage_ptr = [&](int buf) { return smem_raw + buf * SM::stageBytes; };
    auto q_lds = [&](uint8_t* st) { return (uint16_t*)st; };
    auto do_lds = [&](uint8_t* st) { return (uint16_t*)st + SM::rElems; };
    auto qt_lds = [&](uint8_t* st) { return (uint16_t*)st + 2 * SM::rElems; };
    auto dot_lds = [&](uint8_t* st) { return (uint16_t*)st + 2 * SM::rElems + SM::cElems; };
    auto lse_lds = [&](uint8_t* st) { return (float*)((uint16_t*)st + 2 * SM::rElems + 2 * SM::cElems); };
    auto ds_lds = [&](uint8_t* st) { return lse_lds(st) + kKvBM; };

    P pq, pdo;
    float st_lse = 0.f, st_d = 0.f;
    // Flattened (head in group, query tile) sequence n = 0 .. g*nt-1.
    auto load_stage = [&](int n) {
        const int h = hk * g + n / nt;
        const int row0 = (it_lo + n % nt) * kKvBM;
        const uint16_t* qb = (const uint16_t*)a.q + (s.q_start * a.heads + h) * D;
        const uint16_t* dob = (const uint16_t*)a.dout + (s.q_start * a.heads + h) * D;
        pq.load(qb, q_stride, row0, s.len_q, tid);
        pdo.load(dob, q_stride, row0, s.len_q, tid);
        if (tid < 2 * kKvBM) {
            const int row = row0 + (tid % kKvBM);
            const int64_t idx = a.cu_q ? (int64_t)h * total_q + s.q_start + row
                                       : ((int64_t)b * a.heads + h) * a.seqlen_q + row;
            if (tid < kKvBM)  // rows past the end get LSE = +inf, so P = 0 there
                st_lse = row < s.len_q ? a.lse[idx] * kLog2e : __builtin_inff();
            else
                st_d = row < s.len_q ? a.dsum[idx] : 0.f;
        }
    };
    auto store_stage = [&](uint8_t* st) {
        pq.store_rows(q_lds(st), SM::rStride, tid);
        pdo.store_rows(do_lds(st), SM::rStride, tid);
        pq.store_cols(qt_lds(st), SM::cStride, tid);
        pdo.store_cols(dot_lds(st), SM::cStride, tid);
        if (tid < kKvBM) lse_lds(st)[tid] = st_lse;
        else if (tid < 2 * kKvBM) ds_lds(st)[tid - kKvBM] = st_d;
    };

    // One streamed query tile against this wave's 32 keys.
    auto tile = [&](auto masked, int row0, uint8_t* st) {
        const uint16_t* qs = q_lds(st);
        const uint16_t* dos = do_lds(st);
        const uint16_t* qts = qt_lds(st);
        const uint16_t* dots = dot_lds(st);
        const float* lses = lse_lds(st);
        const float* dss = ds_lds(st);
        uint32_t pp[2][8], dsp[2][8];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            f32x16 sacc = f32x16{0}, dpacc = f32x16{0};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const u32x4 qa = *(const u32x4*)(qs + (qb * 32 + r32) * SM::rStride + ks * 16 + 8 * half);
                const u32x4 da = *(const u32x4*)(dos + (qb * 32 + r32) * SM::rStride + ks * 16 + 8 * half);
                sacc = mfma32<BF16>(qa, kf[ks], sacc);
                dpacc = mfma32<BF16>(da, vf[ks], dpacc);
            }
            // lane column = key kw0 + r32; register i = query row qb*32 + 8(i/4) + 4 half + i%4
            const int key = kw0 + r32;
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                const int rbase = qb * 32 + 8 * gq + 4 * half;
                const float4 l4 = *(const float4*)(lses + rbase);
                const float4 d4 = *(const float4*)(dss + rbase);
                const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
                const float dvv[4] = {d4.x, d4.y, d4.z, d4.w};
                float pv[4], dsv[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i = 4 * gq + e;
                    float p = fast_exp2(__builtin_fmaf(sacc[i], c, -lv[e]));
                    if constexpr (decltype(masked)::value) {
                        const int qi = row0 + rbase + e;
                        if (key < mk.lo_of(qi, s) || key > mk.hi_of(qi, s)) p = 0.f;
                    }
                    pv[e] = p;
                    dsv[e] = p * (dpacc[i] - dvv[e]);
                }
                pp[qb][2 * gq] = pack2<BF16>(pv[0], pv[1]);
                pp[qb][2 * gq + 1] = pack2<BF16>(pv[2], pv[3]);
                dsp[qb][2 * gq] = pack2<BF16>(dsv[0], dsv[1]);
                dsp[qb][2 * gq + 1] = pack2<BF16>(dsv[2], dsv[3]);
            }
        }
        // dV^T += dO^T P, dK^T += Q^T dS over the 64 rows (4 k-steps of 16)
#pragma unroll
        for (int kk = 0; kk < kKvBM / 16; ++kk) {
            const int qb = kk / 2, hs = kk % 2;
            const u32x4 pb = u32x4{pp[qb][4 * hs], pp[qb][4 * hs + 1], pp[qb][4 * hs + 2], pp[qb][4 * hs + 3]};
            const u32x4 sb = u32x4{dsp[qb][4 * hs], dsp[qb][4 * hs + 1], dsp[qb][4 * hs + 2], dsp[qb][4 * hs + 3]};
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const u32x4 doa = *(const u32x4*)(dots + (db * 32 + r32) * SM::cStride + kk * 16 + 8 * half);
                const u32x4 qa = *(const u32x4*)(qts + (db * 32 + r32) * SM::cStride + kk * 16 + 8 * half);
                dv[db] = mfma32<BF16>(doa, pb, dv[db]);
                dk[db] = mfma32<BF16>(qa, sb, dk[db]);
            }
        }
    };

    const int total = g * nt;
    if (total > 0) {
        load_stage(0);
        store_stage(stage_ptr(0));
        __syncthreads();
        for (int n = 0; n < total; ++n) {
            const int buf = n & 1;
            const bool has_next = n + 1 < total;
            if (has_next) load_stage(n + 1);
            const int row0 = (it_lo + n % nt) * kKvBM;
            const int row1 = min(row0 + kKvBM, s.len_q) - 1;
            // any visible pair between rows [row0, row1] and keys [kw0, kw1]?
            const bool on = wave_live && mk.hi_of(row1, s) >= kw0 && mk.lo_of(row0, s) <= kw1 &&
                            mk.hi_of(row1, s) >= mk.lo_of(row0, s);
            if (on) {
                // all pairs visible when the first row sees the last key and the
                // last row sees the first key
                const bool full = mk.hi_of(row0, s) >= kw1 && mk.lo_of(row1, s) <= kw0 &&
                                  kw0 + 31 < s.len_k;
                if (full)
                    tile(std::false_type{}, row0, stage_ptr(buf));
                else
                    tile(std::true_type{}, row0, stage_ptr(buf));
            }
            if (has_next) store_stage(stage_ptr(buf ^ 1));
            __syncthreads();
        }
    }

    // store dK = scale * dK^T, dV = dV^T (lane column = key, registers = d)
    const int key = kw0 + r32;
    if (!wave_live || key >= s.len_k) return;
    uint16_t* dkrow = (uint16_t*)a.dk + ((s.k_start + key) * a.kv_heads + hk) * D;
    uint16_t* dvrow = (uint16_t*)a.dv + ((s.k_start + key) * a.kv_heads + hk) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
            const int col = db * 32 + 8 * gq + 4 * half;
            u32x2 wk, wv;
            wk.x = pack2<BF16>(dk[db][4 * gq] * a.scale, dk[db][4 * gq + 1] * a.scale);
            wk.y = pack2<BF16>(dk[db][4 * gq + 2] * a.scale, dk[db][4 * gq + 3] * a.scale);
            wv.x = pack2<BF16>(dv[db][4 * gq], dv[db][4 * gq + 1]);
            wv.y = pack2<BF16>(dv[db][4 * gq + 2], dv[db][4 * gq + 3]);
            *(u32x2*)(dkrow + col) = wk;
            *(u32x2*)(dvrow + col) = wv;
        }
}

// ---------------------------------------------------------------------------
// dQ: one workgroup per (batch, query head, 128-row tile); 4 waves x 32 rows
// ---------------------------------------------------------------------------
constexpr int kQWaves = 4;
constexpr int kQBM = 32 * kQWaves;
constexpr int kQBN = 64;

template <int D>
struct DqSmem {
    static constexpr int rStride = D + 8;      // row-major K, V
    static constexpr int cStride = kQBN + 8;   // K^T (permuted key order)
    static constexpr int rElems = kQBN * rStride;
    static constexpr int cElems = D * cStride;
    static constexpr int stageElems = 2 * rElems + cElems;
    static constexpr int bytes = 2 * stageElems * 2;
};

template <bool BF16, int D>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void bwd_dq_kernel(BwdArgs a) {
    using SM = DqSmem<D>;
    using P = Piece<D, kQBN>;
    constexpr int KS = D / 16, DB = D / 32;
    extern __shared__ __attribute__((aligned(16))) uint16_t smem[];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r32 = lane & 31, half = lane >> 5;
    const int b = blockIdx.x / a.heads, h = blockIdx.x % a.heads;
    const int ntiles = gridDim.y;
    const int qt = a.causal ? (ntiles - 1 - (int)blockIdx.y) : (int)blockIdx.y;
    const Seq s = seq_of(b, a.cu_q, a.cu_k, a.seqlen_q, a.seqlen_k);
    const int i0 = qt * kQBM;
    if (i0 >= s.len_q) return;
    const Mask mk{a.causal, a.left, a.right};
    const int hk = h / (a.heads / a.kv_heads);
    const int64_t q_stride = (int64_t)a.heads * D, kv_stride = (int64_t)a.kv_heads * D;
    const uint16_t* qbase = (const uint16_t*)a.q + (s.q_start * a.heads + h) * D;
    const uint16_t* dobase = (const uint16_t*)a.dout + (s.q_start * a.heads + h) * D;
    const uint16_t* kbase = (const uint16_t*)a.k + (s.k_start * a.kv_heads + hk) * D;
    const uint16_t* vbase = (const uint16_t*)a.v + (s.k_start * a.kv_heads + hk) * D;
    const int64_t rowidx0 = a.cu_q ? (int64_t)h * a.cu_q[a.batch] + s.q_start
                                   : ((int64_t)b * a.heads + h) * a.seqlen_q;

    const int i_last = min(i0 + kQBM, s.len_q) - 1;
    const int key_lo = mk.lo_of(i0, s), key_hi = mk.hi_of(i_last, s);
    const int t_lo = key_lo / kQBN;
    const int t_hi = key_hi >= key_lo ? key_hi / kQBN + 1 : t_lo;

    const int wq0 = i0 + 32 * wave;
    const int wq1 = min(wq0 + 31, s.len_q - 1);
    const bool wave_live = wq0 < s.len_q;
    const int row = wq0 + r32;
    const bool row_ok = row < s.len_q;
    u32x4 qf[KS], dof[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        qf[ks] = row_ok ? *(const u32x4*)(qbase + (int64_t)row * q_stride + ks * 16 + 8 * half) : u32x4{0, 0, 0, 0};
        dof[ks] = row_ok ? *(const u32x4*)(dobase + (int64_t)row * q_stride + ks * 16 + 8 * half) : u32x4{0, 0, 0, 0};
    }
    const float lse2 = row_ok ? a.lse[rowidx0 + row] * kLog2e : __builtin_inff();
    const float dsum = row_ok ? a.dsum[rowidx0 + row] : 0.f;
    const int row_lo = mk.lo_of(row, s), row_hi = mk.hi_of(row, s);
    f32x16 dq[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) dq[db] = f32x16{0};
    const float c = a.scale_log2;

    P pk, pv;
    auto tile = [&](auto masked, int key0, const uint16_t* ks_lds) {
        const uint16_t* vs_lds = ks_lds + SM::rElems;
        const uint16_t* kts = ks_lds + 2 * SM::rElems;
        uint32_t dsp[2][8];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            f32x16 sacc = f32x16{0}, dpacc = f32x16{0};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const u32x4 ka = *(const u32x4*)(ks_lds + (kb * 32 + r32) * SM::rStride + ks * 16 + 8 * half);
                const u32x4 va = *(const u32x4*)(vs_lds + (kb * 32 + r32) * SM::rStride + ks * 16 + 8 * half);
                sacc = mfma32<BF16>(ka, qf[ks], sacc);
                dpacc = mfma32<BF16>(va, dof[ks], dpacc);
            }
            // lane column = query row; register i = key kb*32 + 8(i/4) + 4 half + i%4
#pragma unroll
            for (int i = 0; i < 16; i += 2) {
                float p0 = fast_exp2(__builtin_fmaf(sacc[i], c, -lse2));
                float p1 = fast_exp2(__builtin_fmaf(sacc[i + 1], c, -lse2));
                if constexpr (decltype(masked)::value) {
                    const int k0 = key0 + kb * 32 + 8 * (i / 4) + 4 * half + (i % 4);
                    if (k0 < row_lo || k0 > row_hi) p0 = 0.f;
                    if (k0 + 1 < row_lo || k0 + 1 > row_hi) p1 = 0.f;
                }
                dsp[kb][i / 2] = pack2<BF16>(p0 * (dpacc[i] - dsum), p1 * (dpacc[i + 1] - dsum));
            }
        }
        // dQ^T += K^T dS^T over the 64 keys (4 k-steps of 16)
#pragma unroll
        for (int kk = 0; kk < kQBN / 16; ++kk) {
            const int kb = kk / 2, hs = kk % 2;
            const u32x4 sb = u32x4{dsp[kb][4 * hs], dsp[kb][4 * hs + 1], dsp[kb][4 * hs + 2], dsp[kb][4 * hs + 3]};
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const u32x4 ka = *(const u32x4*)(kts + (db * 32 + r32) * SM::cStride + kk * 16 + 8 * half);
                dq[db] = mfma32<BF16>(ka, sb, dq[db]);
            }
        }
    };

    const int w_key_lo = wave_live ? mk.lo_of(wq0, s) : 0;
    const int w_key_hi = wave_live ? mk.hi_of(wq1, s) : -1;
    const int w_full_lo = wave_live ? mk.lo_of(wq1, s) : 0;
    const int w_full_hi = wave_live ? mk.hi_of(wq0, s) : -1;
    if (t_lo < t_hi) {
        pk.load(kbase, kv_stride, t_lo * kQBN, s.len_k, tid);
        pv.load(vbase, kv_stride, t_lo * kQBN, s.len_k, tid);
        pk.store_rows(smem, SM::rStride, tid);
        pv.store_rows(smem + SM::rElems, SM::rStride, tid);
        pk.store_cols(smem + 2 * SM::rElems, SM::cStride, tid);
        __syncthreads();
        for (int t = t_lo; t < t_hi; ++t) {
            const int buf = (t - t_lo) & 1;
            uint16_t* st = smem + buf * SM::stageElems;
            const bool has_next = t + 1 < t_hi;
            if (has_next) {
                pk.load(kbase, kv_stride, (t + 1) * kQBN, s.len_k, tid);
                pv.load(vbase, kv_stride, (t + 1) * kQBN, s.len_k, tid);
            }
            const int key0 = t * kQBN;
            if (wave_live && key0 <= w_key_hi && key0 + kQBN - 1 >= w_key_lo) {
                if (key0 < w_full_lo || key0 + kQBN - 1 > w_full_hi)
                    tile(std::true_type{}, key0, st);
                else
                    tile(std::false_type{}, key0, st);
            }
            if (has_next) {
                uint16_t* nx = smem + (buf ^ 1) * SM::stageElems;
                pk.store_rows(nx, SM::rStride, tid);
                pv.store_rows(nx + SM::rElems, SM::rStride, tid);
                pk.store_cols(nx + 2 * SM::rElems, SM::cStride, tid);
            }
            __syncthreads();
        }
    }
    if (!row_ok) return;
    uint16_t* dqrow = (uint16_t*)a.dq + ((s.q_start + row) * a.heads + h) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
            u32x2 w;
            w.x = pack2<BF16>(dq[db][4 * gq] * a.scale, dq[db][4 * gq + 1] * a.scale);
            w.y = pack2<BF16>(dq[db][4 * gq + 2] * a.scale, dq[db][4 * gq + 3] * a.scale);
            *(u32x2*)(dqrow + db * 32 + 8 * gq + 4 * half) = w;
        }
}

template <typename K>
bool set_smem(K kernel, int bytes) {
    return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                               hipFuncAttributeMaxDynamicSharedMemorySize, bytes) == hipSuccess;
}

template <bool BF16, int D>
int launch_bwd_t(const BwdArgs& a, int stage, hipStream_t stream) {
    if (stage == 0) {  // D_i = dO_i . O_i
        constexpr int RPB = 256 / (D / 8);
        const int64_t items = (int64_t)a.batch * a.seqlen_q * a.heads;
        const int64_t blocks = (items + RPB - 1) / RPB;
        if (blocks > 0) {
            hipLaunchKernelGGL((bwd_rowdot_kernel<BF16, D>), dim3((unsigned)blocks), dim3(256), 0, stream, a);
            if (hipGetLastError() != hipSuccess) return 1;
        }
        return 0;
    }
    if (stage == 1) {  // dK, dV
        const int ntiles = (a.seqlen_k + kKvBN - 1) / kKvBN;
        if (ntiles > 0 && a.batch > 0) {
            static const bool ok = set_smem(bwd_dkdv_kernel<BF16, D>, DkdvSmem<D>::bytes);
            if (!ok) return 1;
            hipLaunchKernelGGL((bwd_dkdv_kernel<BF16, D>), dim3(a.batch * a.kv_heads, ntiles), dim3(256),
                               DkdvSmem<D>::bytes, stream, a);
            if (hipGetLastError() != hipSuccess) return 1;
        }
        return 0;
    }
    // stage 2: dQ
    const int ntiles = (a.seqlen_q + kQBM - 1) / kQBM;
    if (ntiles > 0 && a.batch > 0) {
        static const bool ok = set_smem(bwd_dq_kernel<BF16, D>, DqSmem<D>::bytes);
        if (!ok) return 1;
        hipLaunchKernelGGL((bwd_dq_kernel<BF16, D>), dim3(a.batch * a.heads, ntiles), dim3(256),
                           DqSmem<D>::bytes, stream, a);
        if (hipGetLastError() != hipSuccess) return 1;
    }
    return 0;
}

}  // namespace

int launch_bwd(const BwdArgs& a, int stage, hipStream_t stream) {
    if (a.bf16)
        return a.head_dim == 128 ? launch_bwd_t<true, 128>(a, stage, stream) : launch_bwd_t<true, 64>(a, stage, stream);
    return a.head_dim == 128 ? launch_bwd_t<false, 128>(a, stage, stream) : launch_bwd_t<false, 64>(a, stage, stream);
}

}  // namespace fa
