// Forward of exact tiled attention on gfx950.
//
// One workgroup = one (batch, query head) and a tile of BM = 256 query rows;
// four waves, each owning 64 rows as two 32-row column blocks.  The kernel
// streams the visible K/V tiles (BN = 64 keys) through two LDS buffers: while
// the waves compute on one buffer, the next tile's global loads are in flight
// into registers and are written to the other buffer afterwards (the
// asynchronous double buffering of the FlashAttention-2 overview page,
// lshu.cn/news/55956, section 2.2, third innovation).  Per tile and wave:
//
//   S^T = K Q^T            (keys x queries; Q^T held in registers)
//   online softmax          per query column: running max m and sum l
//                           (same page, section 2.2, second innovation)
//   O^T += V^T P^T          (d x queries; P^T taken straight from the S^T
//                           registers, V^T read from a transposed LDS copy)
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
// skips the rescale of the 64..128 accumulator registers on almost every
// tile.
#include <type_traits>

#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kQB = 2;                  // 32-row query blocks per wave
constexpr int kBM = 32 * kQB * kWaves;  // query rows per workgroup
constexpr int kBN = 64;                 // keys per tile
constexpr int kKB = kBN / 32;           // 32-key blocks per tile
constexpr float kLazyLog2 = 8.0f;

template <int D>
struct FwdSmem {
    static constexpr int kStride = D + 8;      // K rows, 16-bit elements (16 B pad)
    static constexpr int vStride = kBN + 8;    // V^T rows (one per d), 16-bit elements
    static constexpr int kElems = kBN * kStride;
    static constexpr int vElems = D * vStride;
    static constexpr int stageElems = kElems + vElems;
    static constexpr int bytes = 2 * stageElems * 2;
};

template <int D>
struct KVStage {
    // K: 64 rows x D, as (row, 16-byte chunk) pieces spread over the threads.
    static constexpr int kChunksPerRow = D / 8;
    static constexpr int kPieces = kBN * kChunksPerRow / kThreads;  // per thread
    // V: 4-key x 8-d pieces, transposed on the way to LDS.
    static constexpr int vItems = (kBN / 4) * (D / 8);
    u32x4 k[kPieces];
    u32x4 v[4];
};

template <int D>
__device__ __forceinline__ void load_kv(KVStage<D>& st, const uint16_t* __restrict__ kbase,
                                        const uint16_t* __restrict__ vbase, int64_t row_stride,
                                        int key0, int len_k, int tid) {
    constexpr int CPR = KVStage<D>::kChunksPerRow;
#pragma unroll
    for (int p = 0; p < KVStage<D>::kPieces; ++p) {
        const int c = tid + p * kThreads;
        const int row = c / CPR, ch = c % CPR;
        const int key = key0 + row;
        if (key < len_k)
            st.k[p] = *(const u32x4*)(kbase + (int64_t)key * row_stride + ch * 8);
        else
            st.k[p] = u32x4{0, 0, 0, 0};
    }
    if (tid < KVStage<D>::vItems) {
        const int kc = tid % (kBN / 4), dc = tid / (kBN / 4);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int key = key0 + 4 * kc + r;
            if (key < len_k)
                st.v[r] = *(const u32x4*)(vbase + (int64_t)key * row_stride + dc * 8);
            else
                st.v[r] = u32x4{0, 0, 0, 0};
        }
    }
}

template <int D>
__device__ __forceinline__ void store_kv(const KVStage<D>& st, uint16_t* ks, uint16_t* vts, int tid) {
    using SM = FwdSmem<D>;
    constexpr int CPR = KVStage<D>::kChunksPerRow;
#pragma unroll
    for (int p = 0; p < KVStage<D>::kPieces; ++p) {
        const int c = tid + p * kThreads;
        const int row = c / CPR, ch = c % CPR;
        *(u32x4*)(ks + row * SM::kStride + ch * 8) = st.k[p];
    }
    if (tid < KVStage<D>::vItems) {
        const int kc = tid % (kBN / 4), dc = tid / (kBN / 4);
        u32x2 cols[8];
        transpose4x8(st.v[0], st.v[1], st.v[2], st.v[3], cols);
        const int pos = perm_chunk_pos(kc);
#pragma unroll
        for (int e = 0; e < 8; ++e)
            *(u32x2*)(vts + (dc * 8 + e) * SM::vStride + pos) = cols[e];
    }
}

template <bool BF16, int D>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(1, 1)))
void fwd_kernel(FwdArgs a) {
    using SM = FwdSmem<D>;
    constexpr int KS = D / 16;  // k-steps of S over d
    constexpr int DB = D / 32;  // 32-row blocks of O^T over d
    extern __shared__ __attribute__((aligned(16))) uint16_t smem[];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r32 = lane & 31, half = lane >> 5;
    const int hb = blockIdx.x;
    const int b = hb / a.heads, h = hb % a.heads;
    const int ntiles = gridDim.y;
    const int qt = a.causal ? (ntiles - 1 - (int)blockIdx.y) : (int)blockIdx.y;
    const Seq s = seq_of(b, a.cu_q, a.cu_k, a.seqlen_q, a.seqlen_k);
    const int i0 = qt * kBM;
    if (i0 >= s.len_q) return;
    const Mask mk{a.causal, a.left, a.right};
    const int hk = h / (a.heads / a.kv_heads);

    const int64_t q_row_stride = (int64_t)a.heads * D;
    const int64_t kv_row_stride = (int64_t)a.kv_heads * D;
    const uint16_t* qbase = (const uint16_t*)a.q + (s.q_start * a.heads + h) * D;
    const uint16_t* kbase = (const uint16_t*)a.k + (s.k_start * a.kv_heads + hk) * D;
    const uint16_t* vbase = (const uint16_t*)a.v + (s.k_start * a.kv_heads + hk) * D;
    uint16_t* obase = (uint16_t*)a.o + (s.q_start * a.heads + h) * D;
    float* lsebase = a.cu_q ? a.lse + (int64_t)h * a.cu_q[a.batch] + s.q_start
                            : a.lse + ((int64_t)b * a.heads + h) * a.seqlen_q;

    // Key range of the whole workgroup, as whole tiles.
    const int i_last = min(i0 + kBM, s.len_q) - 1;
    const int key_lo = mk.lo_of(i0, s);
    const int key_hi = mk.hi_of(i_last, s);  // inclusive
    const int t_lo = key_lo / kBN;
    const int t_hi = key_hi >= key_lo ? key_hi / kBN + 1 : t_lo;

    // This wave's rows and the key range any of them can see.
    const int wq0 = i0 + 64 * wave;
    const int wq1 = min(wq0 + 64, s.len_q) - 1;
    const bool wave_live = wq0 < s.len_q;
    const int w_key_lo = wave_live ? mk.lo_of(wq0, s) : 0;
    const int w_key_hi = wave_live ? mk.hi_of(wq1, s) : -1;
    // Tiles inside [w_full_lo, w_full_hi] need no mask for any row of the wave.
    const int w_full_lo = wave_live ? mk.lo_of(wq1, s) : 0;
    const int w_full_hi = wave_live ? mk.hi_of(wq0, s) : -1;

    // Q^T fragments (B operand of S^T = K Q^T), resident for the whole loop.
    u32x4 qf[kQB][KS];
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
        const int row = wq0 + 32 * qb + r32;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if (row < s.len_q)
                qf[qb][ks] = *(const u32x4*)(qbase + (int64_t)row * q_row_stride + ks * 16 + 8 * half);
            else
                qf[qb][ks] = u32x4{0, 0, 0, 0};
        }
    }

    f32x16 acc[DB][kQB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb) acc[db][qb] = f32x16{0};
    float m_run[kQB], l_part[kQB];
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) { m_run[qb] = kNegInf; l_part[qb] = 0.f; }
    const float c = a.scale_log2;

    // One K/V tile for this wave; `masked` selects the edge-tile variant.
    auto tile = [&](auto masked, const int key0, const uint16_t* ks_lds, const uint16_t* vt_lds) {
            // ---- S^T = K Q^T -------------------------------------------------
            f32x16 sacc[kKB][kQB];
#pragma unroll
            for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
                for (int qb = 0; qb < kQB; ++qb) sacc[kb][qb] = f32x16{0};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                u32x4 kf[kKB];
#pragma unroll
                for (int kb = 0; kb < kKB; ++kb)
                    kf[kb] = *(const u32x4*)(ks_lds + (kb * 32 + r32) * SM::kStride + ks * 16 + 8 * half);
#pragma unroll
                for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
                    for (int qb = 0; qb < kQB; ++qb)
                        sacc[kb][qb] = mfma32<BF16>(kf[kb], qf[qb][ks], sacc[kb][qb]);
            }
            // ---- mask (edge tiles only) ---------------------------------------
            if constexpr (decltype(masked)::value) {
#pragma unroll
                for (int qb = 0; qb < kQB; ++qb) {
                    const int qi = wq0 + 32 * qb + r32;
                    const int lo = mk.lo_of(qi, s), hi = mk.hi_of(qi, s);
#pragma unroll
                    for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
                        for (int i = 0; i < 16; ++i) {
                            const int key = key0 + kb * 32 + 8 * (i / 4) + 4 * half + (i % 4);
                            if (key < lo || key > hi) sacc[kb][qb][i] = kNegInf;
                        }
                }
            }
            // ---- online softmax ------------------------------------------------
            uint32_t pk[kKB][kQB][8];
#pragma unroll
            for (int qb = 0; qb < kQB; ++qb) {
                float mx = kNegInf;
#pragma unroll
                for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
                    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][qb][i]);
                mx = max_halves(mx);
                const float m_old = m_run[qb];
                const bool up = mx > m_old && (m_old == kNegInf || (mx - m_old) * c > kLazyLog2);
                if (__builtin_amdgcn_ballot_w64(up)) {
                    const float alpha = !up ? 1.f : (m_old == kNegInf ? 0.f : fast_exp2((m_old - mx) * c));
                    if (up) m_run[qb] = mx;
                    l_part[qb] *= alpha;
#pragma unroll
                    for (int db = 0; db < DB; ++db) acc[db][qb] *= alpha;
                }
                const float mc = m_run[qb] == kNegInf ? 0.f : m_run[qb] * c;
                float lsum = 0.f;
#pragma unroll
                for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
                    for (int i = 0; i < 16; i += 2) {
                        float p0 = fast_exp2(__builtin_fmaf(sacc[kb][qb][i], c, -mc));
                        float p1 = fast_exp2(__builtin_fmaf(sacc[kb][qb][i + 1], c, -mc));
                        if constexpr (decltype(masked)::value) {
                            // exact zero for masked keys, also when scale == 0
                            p0 = sacc[kb][qb][i] == kNegInf ? 0.f : p0;
                            p1 = sacc[kb][qb][i + 1] == kNegInf ? 0.f : p1;
                        }
                        lsum += p0 + p1;
                        pk[kb][qb][i / 2] = pack2<BF16>(p0, p1);
                    }
                l_part[qb] += lsum;
            }
            // ---- O^T += V^T P^T --------------------------------------------------
#pragma unroll
            for (int kk = 0; kk < kBN / 16; ++kk) {
                const int kb = kk / 2, hs = kk % 2;
                u32x4 pb[kQB];
#pragma unroll
                for (int qb = 0; qb < kQB; ++qb)
                    pb[qb] = u32x4{pk[kb][qb][4 * hs], pk[kb][qb][4 * hs + 1],
                                   pk[kb][qb][4 * hs + 2], pk[kb][qb][4 * hs + 3]};
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const u32x4 vf = *(const u32x4*)(vt_lds + (db * 32 + r32) * SM::vStride + kk * 16 + 8 * half);
#pragma unroll
                    for (int qb = 0; qb < kQB; ++qb) acc[db][qb] = mfma32<BF16>(vf, pb[qb], acc[db][qb]);
                }
            }
    };

    if (t_lo < t_hi) {
        KVStage<D> st;
        load_kv<D>(st, kbase, vbase, kv_row_stride, t_lo * kBN, s.len_k, tid);
        store_kv<D>(st, smem, smem + SM::kElems, tid);
        __syncthreads();

        for (int t = t_lo; t < t_hi; ++t) {
            const int buf = (t - t_lo) & 1;
            const uint16_t* ks_lds = smem + buf * SM::stageElems;
            const uint16_t* vt_lds = ks_lds + SM::kElems;
            const bool has_next = t + 1 < t_hi;
            if (has_next) load_kv<D>(st, kbase, vbase, kv_row_stride, (t + 1) * kBN, s.len_k, tid);

            const int key0 = t * kBN;
            const bool wave_on = wave_live && key0 <= w_key_hi && key0 + kBN - 1 >= w_key_lo;
            if (wave_on) {
                if (key0 < w_full_lo || key0 + kBN - 1 > w_full_hi)
                    tile(std::true_type{}, key0, ks_lds, vt_lds);
                else
                    tile(std::false_type{}, key0, ks_lds, vt_lds);
            }
            if (has_next) store_kv<D>(st, smem + (buf ^ 1) * SM::stageElems,
                                      smem + (buf ^ 1) * SM::stageElems + SM::kElems, tid);
            __syncthreads();
        }
    }

    // ---- epilogue: O = acc / l, LSE = scale * m + ln l ------------------------------
    if (!wave_live) return;
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
        const int row = wq0 + 32 * qb + r32;
        const float l = sum_halves(l_part[qb]);
        const float inv = l > 0.f ? 1.f / l : 0.f;
        if (row < s.len_q) {
            uint16_t* orow = obase + (int64_t)row * q_row_stride;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    u32x2 w;
                    w.x = pack2<BF16>(acc[db][qb][4 * g] * inv, acc[db][qb][4 * g + 1] * inv);
                    w.y = pack2<BF16>(acc[db][qb][4 * g + 2] * inv, acc[db][qb][4 * g + 3] * inv);
                    *(u32x2*)(orow + db * 32 + 8 * g + 4 * half) = w;
                }
            if (half == 0)
                lsebase[row] = l > 0.f ? m_run[qb] * a.scale + logf(l) : kNegInf;
        }
    }
}

template <bool BF16, int D>
int launch_fwd_t(const FwdArgs& a, hipStream_t stream) {
    const int ntiles = (a.seqlen_q + kBM - 1) / kBM;
    if (ntiles == 0 || a.batch == 0) return 0;
    static const bool smem_ok =
        hipFuncSetAttribute(reinterpret_cast<const void*>(fwd_kernel<BF16, D>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, FwdSmem<D>::bytes) == hipSuccess;
    if (!smem_ok) return 1;
    dim3 grid(a.batch * a.heads, ntiles);
    hipLaunchKernelGGL((fwd_kernel<BF16, D>), grid, dim3(kThreads), FwdSmem<D>::bytes, stream, a);
    return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // namespace

int launch_fwd(const FwdArgs& a, hipStream_t stream) {
    if (a.bf16) return a.head_dim == 128 ? launch_fwd_t<true, 128>(a, stream) : launch_fwd_t<true, 64>(a, stream);
    return a.head_dim == 128 ? launch_fwd_t<false, 128>(a, stream) : launch_fwd_t<false, 64>(a, stream);
}

}  // namespace fa
