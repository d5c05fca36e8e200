// C-ABI front end of the attention library: argument validation, the device
// check and dispatch to the kernel launchers.  Declared in include/fa.h.
//
// Every argument check runs before the first HIP call, so misuse is reported
// the same way on a host without a GPU.  The device check is cached per
// device ordinal.
#include <hip/hip_runtime_api.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>

#include "../../include/fa.h"
#include "fa_launch.hpp"

namespace {

constexpr int kVersion = 10000;  // 1.0.0
constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_state[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other
std::atomic<int> g_cus[kMaxDevices];         // compute units, valid once the state is known

bool aligned(const void* p, size_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

// Supported head dimensions: multiples of 8 (16-byte rows) up to 256; the
// kernels run them in tiles 64, 128 or 256 wide.
bool head_dim_ok(int d) { return d >= 8 && d <= 256 && d % 8 == 0; }
int tile_width(int d) { return d > 128 ? 256 : (d > 64 ? 128 : 64); }

// The backward accumulates dQ with float32 atomics inside the dK/dV pass when
// the caller does not ask for bitwise repeatable results and the head fits a
// tile of 64 or 128 columns; otherwise it runs the separate dQ pass.
bool atomic_dq(int deterministic, int head_dim) { return deterministic == 0 && head_dim <= 128; }
// Bytes of the dQ accumulator ([rows, heads, tile width] float32), rounded up
// to 256 so the arrays after it stay aligned.
size_t dq_acc_bytes(size_t rows_heads, int head_dim) {
    return (rows_heads * (size_t)tile_width(head_dim) * sizeof(float) + 255) & ~(size_t)255;
}

int check_common(int batch, int heads, int kv_heads, int seqlen_q, int seqlen_k, int head_dim,
                 int causal, int window_left, int window_right, float softmax_scale, int dtype,
                 const int32_t* cu_q, const int32_t* cu_k) {
    if (batch < 0 || heads < 1 || kv_heads < 1 || seqlen_q < 0 || seqlen_k < 0) return FA_ERR_INVALID_ARG;
    if (heads % kv_heads != 0) return FA_ERR_INVALID_ARG;
    if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
    if (window_left < -1 || window_right < -1) return FA_ERR_INVALID_ARG;
    if (!std::isfinite(softmax_scale) || softmax_scale < 0.f) return FA_ERR_INVALID_ARG;
    if ((cu_q == nullptr) != (cu_k == nullptr)) return FA_ERR_INVALID_ARG;
    if (cu_q && (!aligned(cu_q, 4) || !aligned(cu_k, 4))) return FA_ERR_INVALID_ARG;
    // indices are 32-bit inside a sequence, 64-bit across the batch
    if ((long long)batch * heads > (1LL << 31) - 1) return FA_ERR_INVALID_ARG;
    // byte offsets inside a tile (up to 256 rows of heads * head_dim 16-bit values) are 32-bit
    if ((long long)heads * head_dim >= (1LL << 23)) return FA_ERR_INVALID_ARG;
    if (dtype != FA_DTYPE_F16 && dtype != FA_DTYPE_BF16) return FA_ERR_UNSUPPORTED;
    if (!head_dim_ok(head_dim)) return FA_ERR_UNSUPPORTED;
    return FA_OK;
}

// The current device must be a gfx950; *cus (if given) receives its compute
// unit count.  Both are looked up once per device.
int check_arch(int* cus = nullptr) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
        (void)hipGetLastError();
        return FA_ERR_ARCH;
    }
    if (dev < kMaxDevices) {
        const int st = g_arch_state[dev].load(std::memory_order_acquire);
        if (st == 1) {
            if (cus) *cus = g_cus[dev].load(std::memory_order_relaxed);
            return FA_OK;
        }
        if (st == 2) return FA_ERR_ARCH;
    }
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
        (void)hipGetLastError();
        return FA_ERR_ARCH;
    }
    const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 &&
                    (prop.gcnArchName[6] == '\0' || prop.gcnArchName[6] == ':');
    if (dev < kMaxDevices) {
        g_cus[dev].store(prop.multiProcessorCount, std::memory_order_relaxed);
        g_arch_state[dev].store(ok ? 1 : 2, std::memory_order_release);
    }
    if (cus) *cus = prop.multiProcessorCount;
    return ok ? FA_OK : FA_ERR_ARCH;
}

// softmax_scale * log2(e), at least the smallest normal float: keeps -inf
// scores at -inf (exp2 -> exact 0) when softmax_scale == 0, where any finite
// score still maps to exp2(~0) = 1.
float log2e_scaled(float s) {
    const float c = (float)((double)s * 1.4426950408889634074);
    return c < 1.17549435e-38f ? 1.17549435e-38f : c;
}

// Padded-batch lengths: device int32[batch] arrays, only with the fixed
// layout (not together with cu_seqlens).
bool seqused_ok(const int32_t* used_q, const int32_t* used_k, const int32_t* cu_q) {
    if ((used_q || used_k) && cu_q) return false;
    return aligned(used_q, 4) && aligned(used_k, 4);
}

// Dropout threshold T (elements kept iff their 8-bit draw is below T) and
// the scale of kept probabilities, 256 / T (0 when T = 0).  p must lie in
// [0, 1).
bool dropout_params(float p, uint32_t& t, float& scale_kept) {
    if (!std::isfinite(p) || p < 0.f || p >= 1.f) return false;
    double tt = std::floor((1.0 - (double)p) * 256.0 + 0.5);
    tt = tt < 0.0 ? 0.0 : (tt > 256.0 ? 256.0 : tt);
    t = (uint32_t)tt;
    scale_kept = t > 0 ? (float)(256.0 / tt) : 0.f;
    return true;
}

}  // namespace

extern "C" {

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
           const int32_t* seqused_q, const int32_t* seqused_k,
           int batch, int heads, int kv_heads, int seqlen_q, int seqlen_k,
           int head_dim, int causal, int window_left, int window_right,
           float softmax_scale, float dropout_p, uint64_t dropout_seed, int dtype, void* stream) {
    int rc = check_common(batch, heads, kv_heads, seqlen_q, seqlen_k, head_dim, causal, window_left,
                          window_right, softmax_scale, dtype, cu_seqlens_q, cu_seqlens_k);
    if (rc != FA_OK) return rc;
    uint32_t drop_t;
    float drop_scale;
    if (!dropout_params(dropout_p, drop_t, drop_scale)) return FA_ERR_INVALID_ARG;
    if (!seqused_ok(seqused_q, seqused_k, cu_seqlens_q)) return FA_ERR_INVALID_ARG;
    const bool has_q = (long long)batch * seqlen_q > 0, has_k = (long long)batch * seqlen_k > 0;
    if ((has_q && (!q || !o || !lse)) || (has_k && (!k || !v))) return FA_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4))
        return FA_ERR_INVALID_ARG;
    int cus = 0;
    rc = check_arch(&cus);
    if (rc != FA_OK) return rc;
    fa::FwdArgs a;
    a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
    a.cu_q = cu_seqlens_q; a.cu_k = cu_seqlens_k;
    a.used_q = seqused_q; a.used_k = seqused_k;
    a.batch = batch; a.heads = heads; a.kv_heads = kv_heads;
    a.seqlen_q = seqlen_q; a.seqlen_k = seqlen_k; a.head_dim = head_dim;
    a.causal = causal; a.left = window_left; a.right = window_right;
    a.scale = softmax_scale; a.scale_log2 = log2e_scaled(softmax_scale);
    a.bf16 = dtype == FA_DTYPE_BF16;
    a.drop_t = drop_t; a.drop_scale = drop_scale;
    a.seed_lo = (uint32_t)dropout_seed; a.seed_hi = (uint32_t)(dropout_seed >> 32);
    a.cus = cus;
    if (fa::launch_fwd(a, (hipStream_t)stream) != 0) return FA_ERR_LAUNCH;
    if (seqused_q && fa::launch_pad_fill(o, lse, seqused_q, batch, seqlen_q, heads, head_dim,
                                         (hipStream_t)stream) != 0)
        return FA_ERR_LAUNCH;
    return FA_OK;
}

int fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
               const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
               const int32_t* seqused_q, const int32_t* seqused_k,
               int batch, int heads, int kv_heads, int seqlen_q, int seqlen_k,
               int head_dim, int causal, int window_left, int window_right, float softmax_scale,
               float descale_q, float descale_k, float descale_v, int out_dtype, void* stream) {
    for (float d : {descale_q, descale_k, descale_v})
        if (!std::isfinite(d) || d < 0.f) return FA_ERR_INVALID_ARG;
    if (!std::isfinite(softmax_scale) || softmax_scale < 0.f) return FA_ERR_INVALID_ARG;
    const float sc = softmax_scale * descale_q * descale_k;  // scale of the raw E4M3 dot products
    int rc = check_common(batch, heads, kv_heads, seqlen_q, seqlen_k, head_dim, causal, window_left,
                          window_right, sc, out_dtype, cu_seqlens_q, cu_seqlens_k);
    if (rc != FA_OK) return rc;
    if (head_dim % 16 != 0 || head_dim > 128) return FA_ERR_UNSUPPORTED;  // 16-byte chunks of E4M3 rows
    if (!seqused_ok(seqused_q, seqused_k, cu_seqlens_q)) return FA_ERR_INVALID_ARG;
    const bool has_q = (long long)batch * seqlen_q > 0, has_k = (long long)batch * seqlen_k > 0;
    if ((has_q && (!q || !o || !lse)) || (has_k && (!k || !v))) return FA_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4))
        return FA_ERR_INVALID_ARG;
    int cus = 0;
    rc = check_arch(&cus);
    if (rc != FA_OK) return rc;
    fa::Fp8Args a8;
    fa::FwdArgs& a = a8.f;
    a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
    a.cu_q = cu_seqlens_q; a.cu_k = cu_seqlens_k;
    a.used_q = seqused_q; a.used_k = seqused_k;
    a.batch = batch; a.heads = heads; a.kv_heads = kv_heads;
    a.seqlen_q = seqlen_q; a.seqlen_k = seqlen_k; a.head_dim = head_dim;
    a.causal = causal; a.left = window_left; a.right = window_right;
    a.scale = sc; a.scale_log2 = log2e_scaled(sc);
    a.bf16 = out_dtype == FA_DTYPE_BF16;
    a.drop_t = 256; a.drop_scale = 1.f; a.seed_lo = 0; a.seed_hi = 0;
    a.cus = cus;
    a8.v_scale = descale_v;
    if (fa::launch_fwd_fp8(a8, (hipStream_t)stream) != 0) return FA_ERR_LAUNCH;
    if (seqused_q && fa::launch_pad_fill(o, lse, seqused_q, batch, seqlen_q, heads, head_dim,
                                         (hipStream_t)stream) != 0)
        return FA_ERR_LAUNCH;
    return FA_OK;
}

size_t fa_bwd_workspace_size(int batch, int heads, int seqlen_q, int head_dim, int dtype, int deterministic) {
    if (batch < 0 || heads < 1 || seqlen_q < 0) return 0;
    if (!head_dim_ok(head_dim)) return 0;
    if (dtype != FA_DTYPE_F16 && dtype != FA_DTYPE_BF16) return 0;
    if (deterministic != 0 && deterministic != 1) return 0;
    const size_t rows = (size_t)batch * (size_t)seqlen_q * (size_t)heads;
    // sizes whose byte count would not fit a size_t are invalid
    if (batch > 0 && heads > 0 && seqlen_q > 0 &&
        ((size_t)batch * (size_t)heads > SIZE_MAX / (size_t)seqlen_q || rows > SIZE_MAX / (2 * 4 + 128 * 4 + 256)))
        return 0;
    // two float arrays (D and LSE * log2 e), one entry per query row and head;
    // on the atomic dQ path first a float32 dQ accumulator, tile width wide
    size_t n = 2 * rows * sizeof(float);
    if (atomic_dq(deterministic, head_dim)) n += dq_acc_bytes(rows, head_dim);
    return n > 0 ? n : 4;  // never zero for valid sizes, so a null workspace is an error
}

}  // extern "C"

namespace {

int bwd_common(int stage_lo, int stage_hi,
               const void* q, const void* k, const void* v, const void* o,
               const float* lse, const void* dout, void* dq, void* dk, void* dv,
               void* workspace, size_t workspace_bytes,
               const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
               const int32_t* seqused_q, const int32_t* seqused_k,
               int batch, int heads, int kv_heads, int seqlen_q, int seqlen_k,
               int head_dim, int causal, int window_left, int window_right,
               float softmax_scale, float dropout_p, uint64_t dropout_seed, int dtype, int deterministic,
               void* stream) {
    int rc = check_common(batch, heads, kv_heads, seqlen_q, seqlen_k, head_dim, causal, window_left,
                          window_right, softmax_scale, dtype, cu_seqlens_q, cu_seqlens_k);
    if (rc != FA_OK) return rc;
    if (deterministic != 0 && deterministic != 1) return FA_ERR_INVALID_ARG;
    uint32_t drop_t;
    float drop_scale;
    if (!dropout_params(dropout_p, drop_t, drop_scale)) return FA_ERR_INVALID_ARG;
    if (!seqused_ok(seqused_q, seqused_k, cu_seqlens_q)) return FA_ERR_INVALID_ARG;
    const bool has_q = (long long)batch * seqlen_q > 0, has_k = (long long)batch * seqlen_k > 0;
    if ((has_q && (!q || !o || !lse || !dout || !dq)) || (has_k && (!k || !v || !dk || !dv)) || !workspace)
        return FA_ERR_INVALID_ARG;
    const void* p16[] = {q, k, v, o, dout, dq, dk, dv, workspace};
    for (const void* p : p16)
        if (!aligned(p, 16)) return FA_ERR_INVALID_ARG;
    if (!aligned(lse, 4)) return FA_ERR_INVALID_ARG;
    const size_t need = fa_bwd_workspace_size(batch, heads, seqlen_q, head_dim, dtype, deterministic);
    if (need == 0) return FA_ERR_INVALID_ARG;  // sizes past what a size_t counts
    if (workspace_bytes < need) return FA_ERR_WORKSPACE;
    rc = check_arch();
    if (rc != FA_OK) return rc;
    const size_t rows = (size_t)batch * (size_t)heads * (size_t)seqlen_q;
    fa::BwdArgs a;
    a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse; a.dout = dout;
    a.dq = dq; a.dk = dk; a.dv = dv;
    const bool adq = atomic_dq(deterministic, head_dim);
    a.dq_acc = adq ? (float*)workspace : nullptr;
    a.dsum = (float*)((char*)workspace + (adq ? dq_acc_bytes(rows, head_dim) : 0));
    a.lse2 = a.dsum + rows;
    a.cu_q = cu_seqlens_q; a.cu_k = cu_seqlens_k;
    a.used_q = seqused_q; a.used_k = seqused_k;
    a.batch = batch; a.heads = heads; a.kv_heads = kv_heads;
    a.seqlen_q = seqlen_q; a.seqlen_k = seqlen_k; a.head_dim = head_dim;
    a.causal = causal; a.left = window_left; a.right = window_right;
    a.scale = softmax_scale; a.scale_log2 = log2e_scaled(softmax_scale);
    a.bf16 = dtype == FA_DTYPE_BF16;
    a.drop_t = drop_t; a.drop_scale = drop_scale;
    a.seed_lo = (uint32_t)dropout_seed; a.seed_hi = (uint32_t)(dropout_seed >> 32);
    hipStream_t st_ = (hipStream_t)stream;
    for (int st = stage_lo; st <= stage_hi; ++st) {
        if (fa::launch_bwd(a, st, st_) != 0) return FA_ERR_LAUNCH;
        // padded rows of the stage's outputs
        if (st == 1 && seqused_k &&
            (fa::launch_pad_fill(dk, nullptr, seqused_k, batch, seqlen_k, kv_heads, head_dim, st_) != 0 ||
             fa::launch_pad_fill(dv, nullptr, seqused_k, batch, seqlen_k, kv_heads, head_dim, st_) != 0))
            return FA_ERR_LAUNCH;
        if (st == 2 && seqused_q &&
            fa::launch_pad_fill(dq, nullptr, seqused_q, batch, seqlen_q, heads, head_dim, st_) != 0)
            return FA_ERR_LAUNCH;
    }
    return FA_OK;
}

}  // namespace

extern "C" {

int fa_bwd(const void* q, const void* k, const void* v, const void* o,
           const float* lse, const void* dout, void* dq, void* dk, void* dv,
           void* workspace, size_t workspace_bytes,
           const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
           const int32_t* seqused_q, const int32_t* seqused_k,
           int batch, int heads, int kv_heads, int seqlen_q, int seqlen_k,
           int head_dim, int causal, int window_left, int window_right,
           float softmax_scale, float dropout_p, uint64_t dropout_seed, int dtype, int deterministic,
           void* stream) {
    return bwd_common(0, 2, q, k, v, o, lse, dout, dq, dk, dv, workspace, workspace_bytes,
                      cu_seqlens_q, cu_seqlens_k, seqused_q, seqused_k, batch, heads, kv_heads, seqlen_q, seqlen_k, head_dim,
                      causal, window_left, window_right, softmax_scale, dropout_p, dropout_seed, dtype,
                      deterministic, stream);
}

int fa_bwd_stage(int stage, const void* q, const void* k, const void* v, const void* o,
                 const float* lse, const void* dout, void* dq, void* dk, void* dv,
                 void* workspace, size_t workspace_bytes,
                 const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                 const int32_t* seqused_q, const int32_t* seqused_k,
                 int batch, int heads, int kv_heads, int seqlen_q, int seqlen_k,
                 int head_dim, int causal, int window_left, int window_right,
                 float softmax_scale, float dropout_p, uint64_t dropout_seed, int dtype, int deterministic,
                 void* stream) {
    if (stage < 0 || stage > 2) return FA_ERR_INVALID_ARG;
    return bwd_common(stage, stage, q, k, v, o, lse, dout, dq, dk, dv, workspace, workspace_bytes,
                      cu_seqlens_q, cu_seqlens_k, seqused_q, seqused_k, batch, heads, kv_heads, seqlen_q, seqlen_k, head_dim,
                      causal, window_left, window_right, softmax_scale, dropout_p, dropout_seed, dtype,
                      deterministic, stream);
}

}  // extern "C"

namespace {

// Work split of a decode call: `row_blocks` blocks of 32 packed (query head,
// token) rows per kv head; a segment is one (sequence, row block), so there
// are batch * row_blocks segments, and the visible steps of all of them are
// divided evenly over `waves / kv_heads` groups of kv_heads waves (one per
// kv head).  num_splits > 0 asks for num_splits waves per (sequence, kv
// head, row block) on average; otherwise about kDecAutoWaves waves, two per
// CU, which measured faster than filling every SIMD: the split pass is
// bound by HBM, and fewer concurrent streams keep more DRAM pages open.
// Never more groups than segment-steps at full capacity, and at most 65536
// waves.
constexpr long long kDecAutoWaves = 512;
struct DecPlan {
    int waves, row_blocks;
    long long segments;  // batch * row_blocks
};

DecPlan dec_plan(int batch, int heads, int kv_heads, int seqlen_q, int seqlen_k, int head_dim, int num_splits) {
    DecPlan p;
    const long long rows = (long long)(heads / kv_heads) * seqlen_q;
    p.row_blocks = (int)((rows + 31) / 32);
    p.segments = (long long)batch * p.row_blocks;
    long long groups = num_splits > 0 ? (long long)num_splits * p.segments
                                      : kDecAutoWaves / kv_heads;
    const long long max_useful = p.segments * ((seqlen_k + 31) / 32);
    if (groups > max_useful) groups = max_useful;
    if (groups > 65536 / kv_heads) groups = 65536 / kv_heads;
    if (groups < 1) groups = 1;
    p.waves = (int)(groups * kv_heads);
    return p;
}

// Workspace layout: partial O [slots, 32, head_dim] floats, partial LSE
// [slots, 32] floats, prefix sums [batch + 1] int64, with
// slots = (groups + segments) * kv_heads.
size_t dec_slots(const DecPlan& p, int kv_heads) {
    return (size_t)(p.waves / kv_heads + p.segments) * (size_t)kv_heads;
}
size_t dec_ws_o_elems(const DecPlan& p, int kv_heads, int head_dim) {
    return dec_slots(p, kv_heads) * 32 * (size_t)head_dim;
}
size_t dec_ws_lse_elems(const DecPlan& p, int kv_heads) { return dec_slots(p, kv_heads) * 32; }

}  // namespace

extern "C" {

size_t fa_fwd_kvcache_workspace_size(int batch, int heads, int kv_heads, int seqlen_q, int seqlen_k,
                                     int head_dim, int num_splits) {
    if (batch < 0 || heads < 1 || kv_heads < 1 || heads % kv_heads != 0 || seqlen_q < 0 || seqlen_k < 0)
        return 0;
    if (!head_dim_ok(head_dim)) return 0;
    const DecPlan p = dec_plan(batch, heads, kv_heads, seqlen_q, seqlen_k, head_dim, num_splits);
    return (dec_ws_o_elems(p, kv_heads, tile_width(head_dim)) + dec_ws_lse_elems(p, kv_heads)) * sizeof(float) +
           ((size_t)batch + 1) * sizeof(int64_t);
}

int fa_fwd_kvcache(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                   const int32_t* cache_seqlens, void* workspace, size_t workspace_bytes,
                   int batch, int heads, int kv_heads, int seqlen_q, int seqlen_k,
                   int head_dim, int causal, int window_left, int window_right,
                   float softmax_scale, int dtype, int num_splits, void* stream) {
    int rc = check_common(batch, heads, kv_heads, seqlen_q, seqlen_k, head_dim, causal, window_left,
                          window_right, softmax_scale, dtype, nullptr, nullptr);
    if (rc != FA_OK) return rc;
    const bool has_q = (long long)batch * seqlen_q > 0, has_k = (long long)batch * seqlen_k > 0;
    if ((has_q && (!q || !o || !lse || !workspace)) || (has_k && (!k_cache || !v_cache)))
        return FA_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(o, 16) ||
        !aligned(lse, 4) || !aligned(cache_seqlens, 4) || !aligned(workspace, 16))
        return FA_ERR_INVALID_ARG;
    // the kernels count steps of the split axis and output rows in 32 bits
    const long long rblocks = ((long long)(heads / kv_heads) * seqlen_q + 31) / 32;
    if ((long long)batch * rblocks * ((seqlen_k + 31) / 32) >= (1LL << 31) ||
        (long long)batch * heads * seqlen_q >= (1LL << 31))
        return FA_ERR_INVALID_ARG;
    if (has_q && workspace_bytes < fa_fwd_kvcache_workspace_size(batch, heads, kv_heads, seqlen_q, seqlen_k,
                                                                 head_dim, num_splits))
        return FA_ERR_WORKSPACE;
    rc = check_arch();
    if (rc != FA_OK) return rc;
    if (!has_q) return FA_OK;
    const DecPlan p = dec_plan(batch, heads, kv_heads, seqlen_q, seqlen_k, head_dim, num_splits);
    fa::DecArgs a;
    a.q = q; a.kc = k_cache; a.vc = v_cache; a.o = o; a.lse = lse;
    a.cache_lens = cache_seqlens;
    a.ws_o = (float*)workspace;
    a.ws_lse = a.ws_o + dec_ws_o_elems(p, kv_heads, tile_width(head_dim));
    a.prefix = (int64_t*)(a.ws_lse + dec_ws_lse_elems(p, kv_heads));
    a.batch = batch; a.heads = heads; a.kv_heads = kv_heads;
    a.seqlen_q = seqlen_q; a.seqlen_k = seqlen_k; a.head_dim = head_dim;
    a.causal = causal; a.left = window_left; a.right = window_right;
    a.scale = softmax_scale; a.scale_log2 = log2e_scaled(softmax_scale);
    a.bf16 = dtype == FA_DTYPE_BF16;
    a.waves = p.waves; a.row_blocks = p.row_blocks;
    return fa::launch_decode(a, (hipStream_t)stream) == 0 ? FA_OK : FA_ERR_LAUNCH;
}

int fa_fwd_kvcache_splits(int batch, int heads, int kv_heads, int seqlen_q, int seqlen_k, int head_dim,
                          int num_splits) {
    if (batch < 0 || heads < 1 || kv_heads < 1 || heads % kv_heads != 0 || seqlen_q < 0 || seqlen_k < 0)
        return 0;
    if (!head_dim_ok(head_dim)) return 0;
    return dec_plan(batch, heads, kv_heads, seqlen_q, seqlen_k, head_dim, num_splits).waves;
}

const char* fa_strerror(int status) {
    switch (status) {
        case FA_OK: return "ok";
        case FA_ERR_INVALID_ARG: return "invalid argument";
        case FA_ERR_UNSUPPORTED: return "unsupported head_dim (a multiple of 8 from 8 to 256; FP8: of 16 up to 128) or dtype";
        case FA_ERR_ARCH: return "no gfx950 (MI355X) device is current";
        case FA_ERR_WORKSPACE: return "workspace too small";
        case FA_ERR_LAUNCH: return "kernel launch failed";
        default: return "unknown status";
    }
}

int fa_version(void) { return kVersion; }

}  // extern "C"
