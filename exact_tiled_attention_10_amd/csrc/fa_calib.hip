// Calibration kernels for the hardware counters, built into their own small
// library (libfacalib.so), outside the attention interface; the profiling
// entry point runs them under `rocprofv3 --pmc`.
//  * HBM: a plain streaming copy of a known number of bytes, with the same
//    16-byte-per-lane loads and stores of whole 128-byte lines that the
//    attention kernels issue, to learn how many bytes the read and write
//    counters report per byte moved.
//  * LDS: conflict-free LDS reads of a known number of bytes, as many as the
//    CUs can serve, to learn the unit of the LDS activity counter and the read
//    bandwidth the LDS sustains.
//  * Matrix cores: independent chains of the 32x32 MFMAs the kernels use
//    (bf16 32x32x16, fp8 32x32x64 with unit scales) on every SIMD, with the
//    shader clock read beside the fixed 100 MHz real-time counter: the
//    matrix-core rate the chip sustains under load, and its clock, as a
//    measured denominator next to the published peak.
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

// Each wave reads 1 KiB of LDS per step (64 lanes x 16 bytes, or two
// transposing reads of 64 x 8 bytes), 8 steps per iteration, over 64 blocks of
// 1 KiB; 512 threads and 64 KiB of LDS per workgroup.
template <bool TR>
__global__ __launch_bounds__(512) void calib_lds_kernel(uint32_t* __restrict__ out, int iters) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    __shared__ __attribute__((aligned(16))) unsigned char lds[65536];
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    for (int i = t; i < 65536 / 16; i += 512) ((u32x4*)lds)[i] = u32x4{(uint32_t)i, i * 3u, i * 5u, i * 7u};
    __syncthreads();
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int blk = (it * 8 + u + w * 3) & 63;
            if constexpr (!TR) {
                acc ^= *(const u32x4*)(lds + blk * 1024 + lane * 16);
            } else {
                const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(lds + blk * 1024 + lane * 8));
                const s16x4 hi =
                    __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(lds + blk * 1024 + 512 + lane * 8));
                const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
                acc ^= u32x4{l2.x, l2.y, h2.x, h2.y};
            }
        }
    }
    out[(int64_t)blockIdx.x * 512 + t] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

// Each wave runs `iters` rounds of NACC independent accumulator chains (one
// MFMA per chain per round), so the matrix core of its SIMD never waits on a
// result; two waves per SIMD.  Wave 0 of each workgroup records the shader
// clock counter (s_memtime) and the 100 MHz real-time counter at its start
// and end.  The accumulators go to `sink` so the chains are not removed.
template <bool FP8>
__global__ __launch_bounds__(512) void calib_mfma_kernel(float* __restrict__ sink, uint64_t* __restrict__ clocks,
                                                         int iters) {
    constexpr int NACC = 4;
    const int t = threadIdx.x;
    uint64_t c0 = 0, r0 = 0;
    if (t == 0) {
        c0 = __builtin_amdgcn_s_memtime();
        r0 = __builtin_amdgcn_s_memrealtime();
    }
    f32x16 acc[NACC];
#pragma unroll
    for (int i = 0; i < NACC; ++i) acc[i] = f32x16{0};
    // operands differ per lane and stay finite: small integers in bf16 / E4M3
    const uint32_t x = 0x3F803F80u ^ ((uint32_t)(t & 7) << 16);  // 1.0, 1.x in bf16
    if constexpr (!FP8) {
        const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{x, x, x, x});
        const bf16x8 b = __builtin_bit_cast(bf16x8, u32x4{x ^ 1u, x, x, x});
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int i = 0; i < NACC; ++i) acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[i], 0, 0, 0);
        }
    } else {
        const int w = 0x38383838 ^ (t & 3);  // E4M3 1.0 and neighbours
        const i32x8 a = {w, w, w, w, w, w, w, w};
        const i32x8 b = {w ^ 1, w, w, w, w, w, w, w};
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int i = 0; i < NACC; ++i)
                acc[i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[i], 0, 0, 0, 127, 0, 127);
        }
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < NACC; ++i)
#pragma unroll
        for (int j = 0; j < 16; ++j) s += acc[i][j];
    sink[(int64_t)blockIdx.x * 512 + t] = s;
    if (t == 0) {
        const uint64_t c1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
        clocks[4 * blockIdx.x + 0] = c0;
        clocks[4 * blockIdx.x + 1] = c1;
        clocks[4 * blockIdx.x + 2] = r0;
        clocks[4 * blockIdx.x + 3] = r1;
    }
}

}  // namespace

extern "C" {

// Runs the matrix-core calibration: `workgroups` workgroups of 8 waves, each
// wave `iters` x 4 MFMAs (bf16 32x32x16: 32768 FLOP each; fp8 32x32x64:
// 131072 FLOP each).  sink (device) receives workgroups * 512 floats, clocks
// (device) workgroups * 4 uint64: shader clock at start and end, real-time
// counter (100 MHz) at start and end, of wave 0.  Returns 0 when the launch
// was accepted, 1 for bad arguments, 2 for a failed launch.
int fa_calib_mfma(float* sink, uint64_t* clocks, int workgroups, int iters, int fp8, void* stream) {
    if (!sink || !clocks || workgroups < 1 || iters < 1 || (fp8 != 0 && fp8 != 1)) return 1;
    if (fp8)
        hipLaunchKernelGGL(calib_mfma_kernel<true>, dim3(workgroups), dim3(512), 0, (hipStream_t)stream, sink, clocks,
                           iters);
    else
        hipLaunchKernelGGL(calib_mfma_kernel<false>, dim3(workgroups), dim3(512), 0, (hipStream_t)stream, sink,
                           clocks, iters);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

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

// Reads workgroups * 8 waves * iters * 8 KiB from LDS (b128 reads, or
// transposing b64 reads when `transposing` is 1); out (device) receives
// workgroups * 512 uint32.  Returns 0 when the launch was accepted, 1 for bad
// arguments, 2 for a failed launch.
int fa_calib_lds(uint32_t* out, int workgroups, int iters, int transposing, void* stream) {
    if (!out || workgroups < 1 || iters < 1 || (transposing != 0 && transposing != 1)) return 1;
    if (transposing)
        hipLaunchKernelGGL(calib_lds_kernel<true>, dim3(workgroups), dim3(512), 0, (hipStream_t)stream, out, iters);
    else
        hipLaunchKernelGGL(calib_lds_kernel<false>, dim3(workgroups), dim3(512), 0, (hipStream_t)stream, out, iters);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
