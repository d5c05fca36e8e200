// Calibration kernel for the HBM byte counters: a plain streaming copy of a
// known number of bytes, with the same 16-byte-per-lane loads and stores of
// whole 128-byte lines that the attention kernels issue.  Built into its own
// small library (libfacalib.so), outside the attention interface; the
// profiling entry point runs it under `rocprofv3 --pmc` to learn how many
// bytes the read and write counters report per byte moved.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Wave w copies 16-byte units [w * per_wave, (w + 1) * per_wave), 16 loads
// of 1 KiB in flight per step.
__global__ __launch_bounds__(64) void calib_copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                        int64_t per_wave) {
    const int64_t base = (int64_t)blockIdx.x * per_wave + threadIdx.x;
    for (int64_t n = 0; n < per_wave; n += 16 * 64) {
        u32x4 v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) v[u] = src[base + n + u * 64];
#pragma unroll
        for (int u = 0; u < 16; ++u) dst[base + n + u * 64] = v[u];
    }
}

}  // namespace

extern "C" {

// Copies `bytes` bytes from src to dst (device buffers that do not overlap)
// with `waves` waves.  bytes must be a multiple of waves * 16 KiB.  Returns 0
// when the launch was accepted, 1 for bad arguments, 2 for a failed launch.
int fa_calib_copy(const void* src, void* dst, size_t bytes, int waves, void* stream) {
    if (!src || !dst || waves < 1 || bytes == 0 || bytes % ((size_t)waves * 16384) != 0) return 1;
    const int64_t per_wave = (int64_t)(bytes / 16 / (size_t)waves);
    hipLaunchKernelGGL(calib_copy_kernel, dim3(waves), dim3(64), 0, (hipStream_t)stream,
                       (const u32x4*)src, (u32x4*)dst, per_wave);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
