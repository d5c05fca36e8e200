// Padded batches: the attention kernels treat sequence b of a fixed-layout
// batch as its first used[b] rows and never write the rows past them; this
// pass makes the outputs complete by writing those rows as a sequence
// without them defines them: zero (O, dQ, dK, dV) and, for O, LSE = -inf
// (a row with no visible key).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {

namespace {

constexpr int kFillRows = 4;  // rows per workgroup

__device__ __forceinline__ void fill_rows(uint16_t* t, float* lse, const int32_t* used, int b, int seqlen,
                                          int heads, int dh) {
    const int u = min(max(used[b], 0), seqlen);
    const int r0 = blockIdx.x * kFillRows;
    const int rlo = max(r0, u), rhi = min(r0 + kFillRows, seqlen);
    if (rlo >= rhi) return;
    // rows rlo .. rhi-1 of sequence b are contiguous: heads * dh values each, dh a multiple of 8
    const int64_t n16 = (int64_t)(rhi - rlo) * heads * dh / 8;
    u32x4* base = (u32x4*)(t + ((int64_t)b * seqlen + rlo) * heads * dh);
    for (int64_t i = threadIdx.x; i < n16; i += 256) base[i] = u32x4{0, 0, 0, 0};
    if (lse) {
        for (int i = threadIdx.x; i < (rhi - rlo) * heads; i += 256) {
            const int r = rlo + i / heads, h = i % heads;
            lse[((int64_t)b * heads + h) * seqlen + r] = kNegInf;
        }
    }
}

constexpr int kMaxGridY = 65535;

// Workgroup (x, y) covers rows [kFillRows x, kFillRows (x + 1)) of sequences
// y, y + gridDim.y, ...; rows below used[b] are left alone.
__global__ __launch_bounds__(256) void pad_fill_kernel(uint16_t* t, float* lse, const int32_t* used, int batch,
                                                       int seqlen, int heads, int dh) {
    for (int b = blockIdx.y; b < batch; b += gridDim.y) fill_rows(t, lse, used, b, seqlen, heads, dh);
}

}  // namespace

int launch_pad_fill(void* t, float* lse, const int32_t* used, int batch, int seqlen, int heads, int dh,
                    hipStream_t stream) {
    if (batch == 0 || seqlen == 0) return 0;
    dim3 grid((seqlen + kFillRows - 1) / kFillRows, min(batch, kMaxGridY));
    hipLaunchKernelGGL(pad_fill_kernel, grid, dim3(256), 0, stream, (uint16_t*)t, lse, used, batch, seqlen, heads,
                       dh);
    return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // namespace fa
