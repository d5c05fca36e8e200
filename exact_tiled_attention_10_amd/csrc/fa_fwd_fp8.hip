// FP8 forward of exact tiled attention on gfx950: Q, K, V in the 8-bit E4M3
// format with one scale per tensor (the FP8 path the FlashAttention-2
// overview page, lshu.cn/news/55956, section 5.2, describes for H100), O in
// bf16 or fp16, LSE in fp32.
//
// The structure is the 16-bit forward's (fa_fwd.hip): one workgroup per
// (batch, query head) and 128 query rows, 4 waves of 32 rows, the visible
// K/V tiles streamed through two LDS stages by direct global -> LDS loads,
// S^T = K Q^T and O^T += V^T P^T on the matrix cores, the online softmax in
// fp32 in between.  What changes with 8-bit operands:
//
// * Products.  v_mfma_scale_f32_32x32x64_f8f6f4 (scales fixed at 1.0)
//   contracts 64 elements per lane pair: lane l of an operand holds 32 bytes
//   of row (A) or column (B) l % 32, and the hardware pairs byte b of A lane
//   l with byte b of B lane l' when l / 32 == l' / 32.  The order of the 64
//   elements inside is irrelevant as long as both operands use the same one:
//   for S, lane half h holds d = 64 ks + 32 h .. + 31 of both K and Q; for
//   P.V, lane half h holds the 32 keys its S^T registers already hold
//   (rows 8 g + 4 h + r of each 32-key block), in the same byte order for the
//   P^T operand (packed from the registers) and the V^T operand (gathered by
//   8-bit transposing LDS reads).
// * P in FP8.  The probabilities are rounded to E4M3 (round to nearest even)
//   before P.V; the row sum l uses the unrounded fp32 values.  To keep them
//   inside the format's range and away from its subnormals, the exponent
//   offset is lowered by kShiftLog2: p' = 2^(s c - m c + kShiftLog2), with the
//   running max m moved whenever the row max exceeds it by more than
//   kLazyLog2 (in log2 units), so p' <= 2^(kLazyLog2 + kShiftLog2) = 256 < 448
//   and l, O = acc / l and LSE = m scale + ln l - kShiftLog2 ln 2 are the same
//   numbers as without the offset.
// * Scales.  The descales of Q and K fold into the softmax scale (the host
//   passes scale = softmax_scale * dq * dk), the descale of V into the
//   epilogue (O = dv * acc / l).
// * Tiles.  64 keys per tile (one 64-key step of P.V), 1 byte per element:
//   two stages of K and V take 32 KiB at d = 128.  K and V have their own
//   XOR swizzles of 16-byte chunks: the K operand reads (16 B per lane) and
//   the transposing V reads (8 B per lane, 8 rows per 16 lanes) each spread
//   over distinct bank groups.
//
// head_dim is any multiple of 16 up to 128, run in tiles 64 or 128 wide, as
// the 16-bit forward runs its head dims: rows are head_dim bytes long, the
// resident Q^T fragments hold zeros past head_dim, the direct loads of K and V
// fill the chunks past it with a copy of the row's last valid chunk (finite
// values that only meet those zeros in S and only reach columns of O past
// head_dim, which are not stored).
#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

constexpr float kLazyLog2F8 = 4.0f;
constexpr float kShiftLog2F8 = 4.0f;
constexpr float kLn2 = 0.69314718055994530942f;

// Swizzles of the 16-byte chunks of a K / V tile row (CPR chunks per row).
// K: the operand read of lane (row r32, chunk c) puts 16 consecutive rows of
// one chunk into 16 distinct (row parity, slot) bank groups.
template <int CPR>
__device__ __forceinline__ int swz_k(int r) {
    if constexpr (CPR == 8) return (r >> 1) & 7;
    else return (r >> 2) & 3;
}
// V: a transposing read of 16 lanes touches rows {4 h + 0..3, 8 + 4 h + 0..3}
// (mod 16) of one chunk, the neighbouring 16 lanes the next chunk; the
// swizzle keeps the chunk's parity and separates rows 2 or 8 apart.
template <int CPR>
__device__ __forceinline__ int swz_v(int r) {
    if constexpr (CPR == 8) return (((r >> 1) & 1) << 1) | (((r >> 3) & 1) << 2);
    else return ((r >> 3) & 1) << 1;
}

__device__ __forceinline__ f32x16 mfma_f8(const i32x8& a, const i32x8& b, const f32x16& c) {
    // format 0 = E4M3 for both operands, E8M0 scales 127 = 1.0
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// Four fp32 values -> four E4M3 bytes (round to nearest even), byte i = x_i.
__device__ __forceinline__ int pack4_e4m3(float x0, float x1, float x2, float x3) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
    return __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, w, true);
}

template <int D, int NW, int BN>
struct F8Cfg {
    static constexpr int kThreads = 64 * NW;
    static constexpr int CPR = D / 16;                 // 16-byte chunks per row
    static constexpr int tileBytes = BN * D;
    static constexpr int kDmaBlocks = tileBytes / 1024;  // 1 KiB per wave load
    static constexpr int kDmaPerWave = kDmaBlocks / NW;
    static constexpr int kRowsPerBlock = 1024 / D;
    static_assert(kDmaBlocks % NW == 0, "tiles must split evenly into 1 KiB blocks per wave");
};

template <bool BF16, int D, int NW, int BN, int WPE>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * NW, 64 * NW), amdgpu_waves_per_eu(WPE, WPE)))
void fwd_fp8_kernel(Fp8Args a8) {
    using C = F8Cfg<D, NW, BN>;
    constexpr int KS = D / 64;   // k-steps of S over d
    constexpr int DB = D / 32;   // 32-row blocks of O^T over d
    constexpr int KB = BN / 32;  // 32-key blocks per tile
    constexpr int KK = BN / 64;  // 64-key steps of P.V
    constexpr int BM = 32 * NW;
    constexpr int CPR = C::CPR;
    const FwdArgs& a = a8.f;
    __shared__ __attribute__((aligned(16))) uint8_t lds0[2 * C::tileBytes];
    __shared__ __attribute__((aligned(16))) uint8_t lds1[2 * C::tileBytes];
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

    const int dh = a.head_dim;  // multiple of 16, at most D
    const int64_t q_row_stride = (int64_t)a.heads * dh;  // bytes
    const int kv_row_stride = a.kv_heads * dh;
    const uint8_t* qbase = (const uint8_t*)a.q + (s.q_start * a.heads + h) * dh;
    const uint8_t* kbase = (const uint8_t*)a.k + (s.k_start * a.kv_heads + hk) * dh;
    const uint8_t* vbase = (const uint8_t*)a.v + (s.k_start * a.kv_heads + hk) * dh;
    uint16_t* obase = (uint16_t*)a.o + (s.q_start * a.heads + h) * dh;
    float* lsebase = a.cu_q ? a.lse + (int64_t)h * a.cu_q[a.batch] + s.q_start
                            : a.lse + ((int64_t)b * a.heads + h) * a.seqlen_q;

    // Key range of the workgroup as whole tiles, and of this wave.
    const int i_last = min(i0 + BM, s.len_q) - 1;
    const int key_lo = mk.lo_of(i0, s);
    const int key_hi = mk.hi_of(i_last, s);
    const int t_lo = key_lo / BN;
    const int t_hi = key_hi >= key_lo ? key_hi / BN + 1 : t_lo;
    const int wq0 = i0 + 32 * wave;
    const int wq1 = min(wq0 + 32, s.len_q) - 1;
    const bool wave_live = wq0 < s.len_q;
    const int w_key_lo = wave_live ? mk.lo_of(wq0, s) : 0;
    const int w_key_hi = wave_live ? mk.hi_of(wq1, s) : -1;
    const int w_full_lo = wave_live ? mk.lo_of(wq1, s) : 0;
    const int w_full_hi = wave_live ? mk.hi_of(wq0, s) : -1;

    // Q^T fragments: per k-step, bytes d = 64 ks + 32 half .. + 31 of query row r32.
    i32x8 qf[KS];
    {
        const int row = wq0 + r32;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            u32x4 lo = {0, 0, 0, 0}, hi = {0, 0, 0, 0};
            const int c0 = 64 * ks + 32 * half;  // first byte of this lane's two 16-byte chunks
            if (row < s.len_q) {
                const uint8_t* src = qbase + (int64_t)row * q_row_stride + c0;
                if (c0 < dh) lo = *(const u32x4*)src;
                if (c0 + 16 < dh) hi = *(const u32x4*)(src + 16);
            }
            qf[ks] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        }
    }

    // Direct loads: block bi = wave * kDmaPerWave + i covers tile rows
    // bi * kRowsPerBlock + lane / CPR; lane slot lane % CPR receives chunk slot ^ swz(row).
    int dk_off[C::kDmaPerWave], dv_off[C::kDmaPerWave], dma_row[C::kDmaPerWave];
#pragma unroll
    for (int i = 0; i < C::kDmaPerWave; ++i) {
        const int bi = wave * C::kDmaPerWave + i;
        const int row = bi * C::kRowsPerBlock + lane / CPR;
        const int slot = lane % CPR;
        dma_row[i] = row;
        // chunks past head_dim: the row's last valid chunk again
        dk_off[i] = row * kv_row_stride + min(slot ^ swz_k<CPR>(row), dh / 16 - 1) * 16;
        dv_off[i] = row * kv_row_stride + min(slot ^ swz_v<CPR>(row), dh / 16 - 1) * 16;
    }
    // K operand reads: lane (r32, half) reads row 32 kb + r32, chunks 4 ks + 2 half + e.
    int k_rd[KS][2];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int e = 0; e < 2; ++e) k_rd[ks][e] = r32 * D + (((4 * ks + 2 * half + e) ^ swz_k<CPR>(r32)) * 16);
    // V^T operand reads (ds_read_b64_tr_b8): in each 16-lane group G, lane u
    // receives byte (u % 8) of the 8-byte pieces addressed by lanes u / 8 + 2 j,
    // j = 0..7, as its bytes j.  Lane u addresses key row
    // 8 (j / 4) + 4 half + j % 4 (j = u / 2; plus 64 kk + 32 kbh + 16 gp) and the
    // piece of columns 32 db + 16 (G % 2) + 8 (u % 2) .. + 7, so that lane
    // (r32, half) receives V[keys 8 g + 4 half + 0..3][32 db + r32] for
    // g = 2 gp, 2 gp + 1: the bytes its P^T operand holds for those keys.
    int v_rd[DB];
    {
        const int G = lane >> 4, u = lane & 15, j = u >> 1, rp = u & 1;
        const int rl = 8 * (j >> 2) + 4 * half + (j & 3);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const int ch = 2 * db + (G & 1);
            v_rd[db] = rl * D + ((ch ^ swz_v<CPR>(rl)) * 16) + 8 * rp;
        }
    }

    f32x16 acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] = f32x16{0};
    float m_run = kNegInf, l_part = 0.f;
    const float c = a.scale_log2;

    auto issue_tile = [&](int t, int buf) {
        const int key0 = t * BN;
        const bool tail = key0 + BN > s.len_k;  // uniform
        const int last = s.len_k - 1 - key0;
        const int64_t tile_off = (int64_t)key0 * kv_row_stride;
        uint8_t* kl = stage(buf);
        const rsrc_t ksrc = buffer_of(kbase + tile_off), vsrc = buffer_of(vbase + tile_off);
#pragma unroll
        for (int i = 0; i < C::kDmaPerWave; ++i) {
            int ok = dk_off[i], ov = dv_off[i];
            if (tail && dma_row[i] > last) {  // rows past the sequence: the last key again
                const int adj = (last - dma_row[i]) * kv_row_stride;
                ok += adj;
                ov += adj;
            }
            uint8_t* dst = kl + (wave * C::kDmaPerWave + i) * 1024;
            dma16(ksrc, (uint32_t)ok, dst);
            dma16(vsrc, (uint32_t)ov, dst + C::tileBytes);
        }
    };

    auto compute_tile = [&](int t, int buf) {
        const int key0 = t * BN;
        if (!(wave_live && key0 <= w_key_hi && key0 + BN - 1 >= w_key_lo)) return;
        const uint8_t* ks_lds = stage(buf);
        const uint8_t* vs_lds = ks_lds + C::tileBytes;
        // ---- S^T = K Q^T ------------------------------------------------------
        f32x16 sacc[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) sacc[kb] = f32x16{0};
        auto read_k = [&](int kb, int ks) {
            const u32x4 lo = *(const u32x4*)(ks_lds + kb * 32 * D + k_rd[ks][0]);
            const u32x4 hi = *(const u32x4*)(ks_lds + kb * 32 * D + k_rd[ks][1]);
            return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        };
        i32x8 kf[2][KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kf[0][ks] = read_k(0, ks);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            if (kb + 1 < KB) {
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) kf[(kb + 1) & 1][ks] = read_k(kb + 1, ks);
            }
            __builtin_amdgcn_sched_barrier(0);  // operand reads one block ahead of their MFMAs
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) sacc[kb] = mfma_f8(kf[kb & 1][ks], qf[ks], sacc[kb]);
            __builtin_amdgcn_sched_barrier(0);
        }
        // ---- mask (edge tiles only; uniform branch) -----------------------------
        if (key0 < w_full_lo || key0 + BN - 1 > w_full_hi) {
            const int qi = wq0 + r32;
            const int lo = mk.lo_of(qi, s) - key0, hi = mk.hi_of(qi, s) - key0;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int kk = kb * 32 + 8 * (i / 4) + 4 * half + (i % 4);
                    sacc[kb][i] = (kk < lo || kk > hi) ? kNegInf : sacc[kb][i];
                }
        }
        // ---- online softmax, P rounded to E4M3 ----------------------------------------
        float mx = kNegInf;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) mx = max16(sacc[kb], mx);
        mx = max_halves(mx);
        const float m_old = m_run;
        const bool up = mx > m_old && (m_old == kNegInf || (mx - m_old) * c > kLazyLog2F8);
        if (__builtin_amdgcn_ballot_w64(up)) {
            const float alpha = !up ? 1.f : (m_old == kNegInf ? 0.f : fast_exp2((m_old - mx) * c));
            m_run = up ? mx : m_old;
            l_part *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db) acc[db] *= alpha;
        }
        const float mc = m_run == kNegInf ? 0.f : m_run * c - kShiftLog2F8;
        int pk[KB][4];  // dword (kb, g): E4M3 bytes of keys 32 kb + 8 g + 4 half + 0..3
        float lsum = 0.f;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const float p0 = fast_exp2(__builtin_fmaf(sacc[kb][4 * g], c, -mc));
                const float p1 = fast_exp2(__builtin_fmaf(sacc[kb][4 * g + 1], c, -mc));
                const float p2 = fast_exp2(__builtin_fmaf(sacc[kb][4 * g + 2], c, -mc));
                const float p3 = fast_exp2(__builtin_fmaf(sacc[kb][4 * g + 3], c, -mc));
                lsum += (p0 + p1) + (p2 + p3);
                pk[kb][g] = pack4_e4m3(p0, p1, p2, p3);
            }
        l_part += lsum;
        // ---- O^T += V^T P^T, 64 keys per product -------------------------------------
        typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            const i32x8 pb = i32x8{pk[2 * kk][0], pk[2 * kk][1], pk[2 * kk][2], pk[2 * kk][3],
                                   pk[2 * kk + 1][0], pk[2 * kk + 1][1], pk[2 * kk + 1][2], pk[2 * kk + 1][3]};
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                i32x8 va;
#pragma unroll
                for (int kbh = 0; kbh < 2; ++kbh)
#pragma unroll
                    for (int gp = 0; gp < 2; ++gp) {
                        const uint8_t* p = vs_lds + (64 * kk + 32 * kbh + 16 * gp) * D + v_rd[db];
                        const i32x2 x = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)p);
                        va[4 * kbh + 2 * gp] = x[0];
                        va[4 * kbh + 2 * gp + 1] = x[1];
                    }
                acc[db] = mfma_f8(va, pb, acc[db]);
            }
        }
    };

    auto step = [&](int t, int buf) {
        if (t + 1 < t_hi) issue_tile(t + 1, buf ^ 1);
        compute_tile(t, buf);
        wait_vmcnt<0>();  // the next tile's direct loads have landed
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

    // ---- epilogue: O = dv * acc / l, LSE = m scale + ln l - kShiftLog2 ln 2 -------------
    if (!wave_live) return;
    const int row = wq0 + r32;
    const float l = sum_halves(l_part);
    const float inv = l > 0.f ? a8.v_scale / l : 0.f;
    if (row < s.len_q) {
        uint16_t* orow = obase + (int64_t)row * q_row_stride;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int col = db * 32 + 8 * g + 4 * half;  // four columns, all below dh or none
                if (col >= dh) continue;
                u32x2 w;
                w.x = pack2<BF16>(acc[db][4 * g] * inv, acc[db][4 * g + 1] * inv);
                w.y = pack2<BF16>(acc[db][4 * g + 2] * inv, acc[db][4 * g + 3] * inv);
                *(u32x2*)(orow + col) = w;
            }
        if (half == 0) lsebase[row] = l > 0.f ? m_run * a.scale + (logf(l) - kShiftLog2F8 * kLn2) : kNegInf;
    }
}

// Launch shape (measured on MI355X, causal, 8K, d = 128): 4 waves of 32 query
// rows with 64-key tiles, three workgroups per CU (three waves per SIMD, 168
// registers), against 8 waves at two per SIMD with 128-key tiles.
// Overridable at build time for tuning.
#ifndef FA_F8_NW
#define FA_F8_NW 4
#endif
#ifndef FA_F8_BN
#define FA_F8_BN 64
#endif
#ifndef FA_F8_WPE
#define FA_F8_WPE 3
#endif

template <bool BF16, int D>
int launch_fp8_t(const Fp8Args& a8, hipStream_t stream) {
    constexpr int NW = FA_F8_NW, BN = FA_F8_BN, WPE = FA_F8_WPE, BM = 32 * NW;
    const FwdArgs& a = a8.f;
    const int ntiles = (a.seqlen_q + BM - 1) / BM;
    if (ntiles == 0 || a.batch == 0) return 0;
    dim3 grid(a.batch * a.heads, ntiles);
    hipLaunchKernelGGL((fwd_fp8_kernel<BF16, D, NW, BN, WPE>), grid, dim3(64 * NW), 0, stream, a8);
    return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // namespace

int launch_fwd_fp8(const Fp8Args& a8, hipStream_t stream) {
    const bool bf16 = a8.f.bf16 != 0;
    // tile width: the smaller of 64, 128 holding head_dim
    if (a8.f.head_dim > 64) return bf16 ? launch_fp8_t<true, 128>(a8, stream) : launch_fp8_t<false, 128>(a8, stream);
    return bf16 ? launch_fp8_t<true, 64>(a8, stream) : launch_fp8_t<false, 64>(a8, stream);
}

}  // namespace fa
