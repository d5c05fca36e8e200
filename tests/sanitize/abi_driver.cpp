// Drives every entry point of include/fa.h through valid and invalid
// arguments with real host buffers, under ASan/UBSan, against the stubs of
// abi_stubs.cpp.  Exits non-zero on the first unexpected status.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "fa.h"

extern int g_stub_device;
extern const char* g_stub_arch;
extern int g_launches[8];
extern const char* g_ws_lo;
extern const char* g_ws_hi;

static int fails = 0;
static void expect(const char* what, int got, int want) {
    if (got != want) {
        std::printf("FAIL %-56s got %d want %d\n", what, got, want);
        ++fails;
    }
}

struct Buf {  // 256-byte aligned host buffer of n bytes
    void* p = nullptr;
    explicit Buf(size_t n) { p = std::aligned_alloc(256, (n + 255) / 256 * 256 + 256); }
    ~Buf() { std::free(p); }
};

int main() {
    const int B = 2, H = 8, HK = 2, N = 100, NK = 130;
    for (int d : {8, 64, 96, 128, 200, 256}) {
        Buf q(B * N * H * d * 2), k(B * NK * HK * d * 2), v(B * NK * HK * d * 2), o(B * N * H * d * 2);
        Buf lse(B * H * N * 4), dq(B * N * H * d * 2), dk(B * NK * HK * d * 2), dv(B * NK * HK * d * 2);
        for (int dtype : {FA_DTYPE_F16, FA_DTYPE_BF16}) {
            expect("fwd valid", fa_fwd(q.p, k.p, v.p, o.p, (float*)lse.p, nullptr, nullptr, nullptr, nullptr, B, H,
                                       HK, N, NK, d, 1, -1, -1, 0.1f, 0.f, 0, dtype, nullptr), FA_OK);
            for (int det : {0, 1}) {
                const size_t ws = fa_bwd_workspace_size(B, H, N, d, dtype, det);
                Buf w(ws);
                g_ws_lo = (const char*)w.p;
                g_ws_hi = g_ws_lo + ws;
                expect("bwd valid", fa_bwd(q.p, k.p, v.p, o.p, (const float*)lse.p, o.p, dq.p, dk.p, dv.p, w.p, ws,
                                           nullptr, nullptr, nullptr, nullptr, B, H, HK, N, NK, d, 1, 100, 0,
                                           0.1f, 0.1f, 7, dtype, det, nullptr), FA_OK);
                expect("bwd one byte short", fa_bwd(q.p, k.p, v.p, o.p, (const float*)lse.p, o.p, dq.p, dk.p,
                                                    dv.p, w.p, ws - 1, nullptr, nullptr, nullptr, nullptr, B, H,
                                                    HK, N, NK, d, 1, -1, -1, 0.1f, 0.f, 0, dtype, det, nullptr),
                       FA_ERR_WORKSPACE);
                for (int st = 0; st < 3; ++st)
                    expect("bwd stage", fa_bwd_stage(st, q.p, k.p, v.p, o.p, (const float*)lse.p, o.p, dq.p, dk.p,
                                                     dv.p, w.p, ws, nullptr, nullptr, nullptr, nullptr, B, H, HK,
                                                     N, NK, d, 0, -1, -1, 0.f, 0.f, 0, dtype, det, nullptr),
                           FA_OK);
            }
            for (int splits : {0, 1, 7}) {
                const size_t ws = fa_fwd_kvcache_workspace_size(B, H, HK, 3, NK, d, splits);
                Buf w(ws);
                g_ws_lo = (const char*)w.p;
                g_ws_hi = g_ws_lo + ws;
                expect("kvcache valid", fa_fwd_kvcache(q.p, k.p, v.p, o.p, (float*)lse.p, nullptr, w.p, ws, B, H, HK,
                                                       3, NK, d, 1, -1, -1, 0.1f, dtype, splits, nullptr), FA_OK);
            }
        }
        if (d % 16 == 0 && d <= 128)
            expect("fp8 valid", fa_fwd_fp8(q.p, k.p, v.p, o.p, (float*)lse.p, nullptr, nullptr, nullptr, nullptr, B,
                                           H, HK, N, NK, d, 0, 5, 5, 0.1f, 0.5f, 0.25f, 2.f, FA_DTYPE_BF16, nullptr),
                   FA_OK);
    }
    // invalid arguments, each rejected before the device check
    Buf x(1 << 16);
    float* l = (float*)x.p;
    expect("heads % kv_heads", fa_fwd(x.p, x.p, x.p, x.p, l, nullptr, nullptr, nullptr, nullptr, 1, 6, 4, 8, 8, 64, 0,
                                      -1, -1, 0.1f, 0.f, 0, 1, nullptr), FA_ERR_INVALID_ARG);
    expect("dropout nan", fa_fwd(x.p, x.p, x.p, x.p, l, nullptr, nullptr, nullptr, nullptr, 1, 4, 4, 8, 8, 64, 0,
                                 -1, -1, 0.1f, 0.f / 0.f, 0, 1, nullptr), FA_ERR_INVALID_ARG);
    expect("huge sizes", fa_fwd(x.p, x.p, x.p, x.p, l, nullptr, nullptr, nullptr, nullptr, 1 << 20, 1 << 12, 1,
                                1 << 30, 1 << 30, 256, 1, -1, -1, 0.1f, 0.f, 0, 1, nullptr), FA_ERR_INVALID_ARG);
    expect("bwd deterministic 2", fa_bwd(x.p, x.p, x.p, x.p, l, x.p, x.p, x.p, x.p, x.p, 1 << 16, nullptr, nullptr,
                                         nullptr, nullptr, 1, 4, 4, 8, 8, 64, 0, -1, -1, 0.1f, 0.f, 0, 1, 2, nullptr),
           FA_ERR_INVALID_ARG);
    expect("workspace size overflow-free", fa_bwd_workspace_size(1 << 20, 1 << 10, 1 << 20, 128, 1, 0) > 0, 1);
    expect("strerror", fa_strerror(12345) != nullptr, 1);
    // device checks: no device, then another architecture
    g_stub_device = -1;
    expect("no device", fa_fwd(x.p, x.p, x.p, x.p, l, nullptr, nullptr, nullptr, nullptr, 1, 4, 4, 8, 8, 64, 0, -1,
                               -1, 0.1f, 0.f, 0, 1, nullptr), FA_ERR_ARCH);
    g_stub_device = 1;
    g_stub_arch = "gfx942";
    expect("other arch", fa_fwd(x.p, x.p, x.p, x.p, l, nullptr, nullptr, nullptr, nullptr, 1, 4, 4, 8, 8, 64, 0, -1,
                                -1, 0.1f, 0.f, 0, 1, nullptr), FA_ERR_ARCH);
    expect("launches happened", g_launches[0] > 0 && g_launches[2] > 0 && g_launches[3] > 0 && g_launches[4] > 0 &&
                                    g_launches[5] > 0, 1);
    std::printf("%s\n", fails ? "FAILED" : "abi: all checks passed");
    return fails ? 1 : 0;
}
