// Host-side argument blocks and launchers shared by the C-ABI front end and
// the kernel files.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace fa {

struct FwdArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    const int32_t* cu_q;
    const int32_t* cu_k;
    const int32_t* used_q;  // padded batches: valid rows per sequence, or null
    const int32_t* used_k;
    int batch, heads, kv_heads, seqlen_q, seqlen_k, head_dim;
    int causal, left, right;
    float scale;       // softmax scale
    float scale_log2;  // softmax scale * log2(e)
    int bf16;
    // dropout: keep iff the element's 8-bit draw < drop_t (256: no dropout);
    // kept probabilities are scaled by drop_scale = 256 / drop_t
    uint32_t drop_t;
    float drop_scale;
    uint32_t seed_lo, seed_hi;
    int cus;  // compute units of the device (launch-shape choice on the host; 0: unknown)
};

struct Fp8Args {
    FwdArgs f;
    float v_scale;  // descale of V: O = v_scale * sum_j p_j v_j / l
};

struct BwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* o;
    const float* lse;
    const void* dout;
    void* dq;
    void* dk;
    void* dv;
    float* dsum;  // workspace: D_i = dO_i . O_i, laid out like lse
    float* lse2;  // workspace: LSE_i * log2(e), laid out like lse
    // workspace of the atomic dQ path, or null (separate dQ pass): unscaled
    // dQ in float32, [rows, heads, W] with W the tile width (64 or 128) and
    // rows as in dq
    float* dq_acc;
    const int32_t* cu_q;
    const int32_t* cu_k;
    const int32_t* used_q;  // as in FwdArgs
    const int32_t* used_k;
    int batch, heads, kv_heads, seqlen_q, seqlen_k, head_dim;
    int causal, left, right;
    float scale;
    float scale_log2;
    int bf16;
    uint32_t drop_t;     // as in FwdArgs
    float drop_scale;
    uint32_t seed_lo, seed_hi;
};

struct DecArgs {
    const void* q;       // [batch, seqlen_q, heads, D]
    const void* kc;      // [batch, seqlen_k, kv_heads, D] (seqlen_k = cache capacity)
    const void* vc;
    void* o;             // like q
    float* lse;          // [batch, heads, seqlen_q]
    const int32_t* cache_lens;  // [batch] valid cache rows, or null (all seqlen_k)
    // workspace: one slot of 32 rows per piece and kv head
    // ((groups + segments) * kv_heads slots)
    float* ws_o;         // [slots, 32, D] partial O, normalised (D: the tile width)
    float* ws_lse;       // [slots, 32] partial LSE
    int64_t* prefix;     // [batch + 1] prefix sums of the per-sequence step counts
    int batch, heads, kv_heads, seqlen_q, seqlen_k, head_dim;
    int causal, left, right;
    float scale;
    float scale_log2;
    int bf16;
    int waves;           // waves of the split pass: groups of kv_heads waves, one per
                         // kv head, share out the step axis evenly
    int row_blocks;      // ceil(heads / kv_heads * seqlen_q / 32)
};

// Each returns 0 when every launch was accepted, 1 otherwise.  Backward
// stages: 0 = D_i = dO_i . O_i (and, on the atomic dQ path, dq_acc = 0),
// 1 = dK/dV pass (on the atomic dQ path it also adds dQ into dq_acc),
// 2 = dQ pass (atomic dQ path: dq = scale * dq_acc in the 16-bit type).
int launch_fwd(const FwdArgs& a, hipStream_t stream);
// FP8 forward: f.q/k/v hold E4M3 bytes, f.scale = softmax_scale * dq * dk
// (f.scale_log2 likewise), f.o is bf16 or fp16 (f.bf16); no dropout.
int launch_fwd_fp8(const Fp8Args& a, hipStream_t stream);
int launch_bwd(const BwdArgs& a, int stage, hipStream_t stream);
int launch_decode(const DecArgs& a, hipStream_t stream);

// Padded batches: for each sequence b and row r with used[b] <= r < seqlen of
// a [batch, seqlen, heads, dh] 16-bit tensor, zero the row of every head and,
// when lse is given ([batch, heads, seqlen] float32), set its LSE to -inf.
int launch_pad_fill(void* t, float* lse, const int32_t* used, int batch, int seqlen, int heads, int dh,
                    hipStream_t stream);

}  // namespace fa
