// Allocation-free backward entry point: fa_bwd with its workspace in a
// file-scope device array instead of caller memory, for callers that cannot
// allocate device memory (code being captured into a HIP graph, serving
// loops, harnesses that forbid allocation).  Declared in include/fa.h.
//
// The array lives on every device the library runs on until the process
// ends.  In host code its name only stands in for it, so its device address
// is looked up once per device (hipGetSymbolAddress, with that device
// current) and that address, never the name, is what the kernels get.  All
// calls on one device share the array: calls that overlap on one GPU (other
// streams, other threads) race on it.  Nothing in it needs to start at zero:
// the first kernel of the backward writes every entry the later ones read.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/fa.h"

namespace {

constexpr size_t kScratchBytes = (size_t)16 << 20;  // D and LSE * log2(e): 2^21 (row, head) pairs
constexpr int kMaxDevices = 64;

}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

std::mutex g_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device ordinal

// The array's device address on the current device (null on failure).
void* scratch_ptr() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return nullptr;
    }
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            (void)hipGetLastError();
            return nullptr;
        }
        g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                   const float* lse, const void* dout, void* dq, void* dk, void* dv,
                   const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                   const int32_t* seqused_q, const int32_t* seqused_k,
                   int batch, int heads, int kv_heads, int seqlen_q, int seqlen_k,
                   int head_dim, int causal, int window_left, int window_right,
                   float softmax_scale, float dropout_p, uint64_t dropout_seed, int dtype, void* stream) {
    // argument checks first, before any HIP call (as every entry point does):
    // with no workspace, a call whose arguments are valid stops at the
    // workspace check, anything else returns its own code
    static unsigned char no_workspace alignas(256)[16];
    const int rc = fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, no_workspace, 0, cu_seqlens_q, cu_seqlens_k, seqused_q,
                          seqused_k, batch, heads, kv_heads, seqlen_q, seqlen_k, head_dim, causal, window_left,
                          window_right, softmax_scale, dropout_p, dropout_seed, dtype, 1, stream);
    if (rc != FA_ERR_WORKSPACE) return rc;
    // sizes beyond the array: batch * heads * seqlen_q above 2^21
    if (fa_bwd_workspace_size(batch, heads, seqlen_q, head_dim, dtype, 1) > kScratchBytes) return FA_ERR_WORKSPACE;
    void* ws = scratch_ptr();
    if (!ws) return FA_ERR_ARCH;
    return fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, ws, kScratchBytes, cu_seqlens_q, cu_seqlens_k, seqused_q,
                  seqused_k, batch, heads, kv_heads, seqlen_q, seqlen_k, head_dim, causal, window_left, window_right,
                  softmax_scale, dropout_p, dropout_seed, dtype, 1, stream);
}

}  // extern "C"
