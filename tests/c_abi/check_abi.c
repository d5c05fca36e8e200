/* Plain C11 client of libfa.so: include/fa.h must compile as C, and the
 * argument checks must answer before any HIP call (this program runs on a
 * host without a GPU).  Prints one line per check; exits non-zero on the
 * first mismatch. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "fa.h"

static int fails = 0;

static void expect(const char* what, int got, int want) {
    printf("%-48s %d (want %d)\n", what, got, want);
    if (got != want) ++fails;
}

int main(void) {
    /* fake, aligned, never dereferenced: validation rejects the calls first */
    void* p = (void*)(uintptr_t)0x10000;
    float* lse = (float*)(uintptr_t)0x20000;
    expect("fa_version >= 1.0.0", fa_version() >= 10000, 1);
    expect("fa_strerror(FA_OK) is \"ok\"", strcmp(fa_strerror(FA_OK), "ok") == 0, 1);
    expect("fwd: heads % kv_heads != 0",
           fa_fwd(p, p, p, p, lse, NULL, NULL, NULL, NULL, 1, 6, 4, 128, 128, 128, 1, -1, -1, 0.125f, 0.0f, 0,
                  FA_DTYPE_BF16, NULL),
           FA_ERR_INVALID_ARG);
    expect("fwd: head_dim 100",
           fa_fwd(p, p, p, p, lse, NULL, NULL, NULL, NULL, 1, 4, 2, 128, 128, 100, 1, -1, -1, 0.125f, 0.0f, 0,
                  FA_DTYPE_BF16, NULL),
           FA_ERR_UNSUPPORTED);
    expect("fwd: dropout_p = 1",
           fa_fwd(p, p, p, p, lse, NULL, NULL, NULL, NULL, 1, 4, 2, 128, 128, 128, 1, -1, -1, 0.125f, 1.0f, 0,
                  FA_DTYPE_BF16, NULL),
           FA_ERR_INVALID_ARG);
    expect("fwd_fp8: head_dim 40 (not a multiple of 16)",
           fa_fwd_fp8(p, p, p, p, lse, NULL, NULL, NULL, NULL, 1, 4, 2, 128, 128, 40, 1, -1, -1, 0.125f, 1.0f, 1.0f,
                      1.0f, FA_DTYPE_BF16, NULL),
           FA_ERR_UNSUPPORTED);
    expect("bwd: workspace too small",
           fa_bwd(p, p, p, p, lse, p, p, p, p, p, 16, NULL, NULL, NULL, NULL, 1, 4, 2, 128, 128, 128, 1, -1, -1,
                  0.125f, 0.0f, 0, FA_DTYPE_BF16, 1, NULL),
           FA_ERR_WORKSPACE);
    expect("bwd_stage: stage 3",
           fa_bwd_stage(3, p, p, p, p, lse, p, p, p, p, p, 1 << 20, NULL, NULL, NULL, NULL, 1, 4, 2, 128, 128, 128,
                        1, -1, -1, 0.125f, 0.0f, 0, FA_DTYPE_BF16, 0, NULL),
           FA_ERR_INVALID_ARG);
    expect("bwd: deterministic = 2",
           fa_bwd(p, p, p, p, lse, p, p, p, p, p, 1 << 20, NULL, NULL, NULL, NULL, 1, 4, 2, 128, 128, 128, 1, -1,
                  -1, 0.125f, 0.0f, 0, FA_DTYPE_BF16, 2, NULL),
           FA_ERR_INVALID_ARG);
    expect("bwd workspace size: 2 float arrays of B*H*N",
           (int)fa_bwd_workspace_size(2, 4, 100, 128, FA_DTYPE_BF16, 1), 2 * 2 * 4 * 100 * 4);
    expect("bwd workspace size, atomic dQ: + B*N*H*128 floats",
           (int)fa_bwd_workspace_size(2, 4, 100, 128, FA_DTYPE_BF16, 0), 2 * 2 * 4 * 100 * 4 + 2 * 100 * 4 * 128 * 4);
    expect("kvcache workspace size > 0", fa_fwd_kvcache_workspace_size(2, 8, 2, 1, 4096, 128, 0) > 0, 1);
    expect("kvcache: head_dim 7 (size 0)", (int)fa_fwd_kvcache_workspace_size(2, 8, 2, 1, 4096, 7, 0), 0);
    printf("%s\n", fails ? "FAILED" : "all checks passed");
    return fails ? 1 : 0;
}
