// Host-only stand-ins for the HIP runtime calls and the kernel launchers that
// the C-ABI front end (fa_api.cpp) makes, so that the front end can be built
// with AddressSanitizer and UndefinedBehaviorSanitizer and run on a host with
// no GPU.  The device "is" a gfx950 unless the driver says otherwise; the
// launchers launch nothing: they check that every region they were handed
// lies inside the workspace the caller passed, and count their calls.
#include <hip/hip_runtime_api.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "../../exact_tiled_attention_10_amd/csrc/fa_launch.hpp"

int g_stub_device = 0;             // -1: hipGetDevice fails
const char* g_stub_arch = "gfx950:sramecc+:xnack-";
int g_launches[8];
const char* g_ws_lo = nullptr;     // the workspace the driver passed
const char* g_ws_hi = nullptr;

extern "C" hipError_t hipGetDevice(int* d) {
    if (g_stub_device < 0) return hipErrorNoDevice;
    *d = g_stub_device;
    return hipSuccess;
}
extern "C" hipError_t hipGetDeviceProperties(hipDeviceProp_t* p, int) {
    std::memset(p, 0, sizeof(*p));
    std::snprintf(p->gcnArchName, sizeof(p->gcnArchName), "%s", g_stub_arch);
    return hipSuccess;
}
extern "C" hipError_t hipGetLastError(void) { return hipSuccess; }

static void inside(const void* p, size_t bytes, const char* what) {
    const char* c = (const char*)p;
    if (!g_ws_lo || c < g_ws_lo || c + bytes > g_ws_hi) {
        std::fprintf(stderr, "workspace region %s outside the caller's workspace\n", what);
        std::abort();
    }
}

namespace fa {
int launch_fwd(const FwdArgs&, hipStream_t) { ++g_launches[0]; return 0; }
int launch_fwd_fp8(const Fp8Args&, hipStream_t) { ++g_launches[1]; return 0; }
int launch_bwd(const BwdArgs& a, int stage, hipStream_t) {
    ++g_launches[2 + stage];
    const size_t rows = (size_t)a.batch * a.heads * a.seqlen_q;
    inside(a.dsum, rows * sizeof(float), "dsum");
    inside(a.lse2, rows * sizeof(float), "lse2");
    if (a.dq_acc) inside(a.dq_acc, rows * (a.head_dim > 64 ? 128 : 64) * sizeof(float), "dq_acc");
    return 0;
}
int launch_decode(const DecArgs& a, hipStream_t) {
    ++g_launches[5];
    inside(a.prefix, ((size_t)a.batch + 1) * sizeof(int64_t), "prefix");
    inside(a.ws_o, sizeof(float), "ws_o");
    inside(a.ws_lse, sizeof(float), "ws_lse");
    return 0;
}
int launch_pad_fill(void*, float*, const int32_t*, int, int, int, int, hipStream_t) {
    ++g_launches[6];
    return 0;
}
}  // namespace fa
