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
//  * Matrix cores fed from LDS: every MFMA takes its A operand from a 1 KiB
//    LDS read of its own, the ratio of the attention kernels' products for 32
//    query rows per wave, with one or two waves per SIMD and the reads issued
//    1, 2 or 4 MFMAs ahead.
//  * Pipe mix: the two waves of each SIMD given different work (idle, MFMA
//    chains from registers or from LDS, independent FMA chains, independent
//    exp2 chains), to see which pairs overlap and at what vector rate one and
//    two waves issue.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

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

// Records the shader clock and the 100 MHz real-time counter at the start and
// end of wave 0 of the workgroup (the kernel's clock under its own load).
struct ClockPair {
    uint64_t c0 = 0, r0 = 0;
    __device__ void start() {
        if (threadIdx.x == 0) {
            c0 = __builtin_amdgcn_s_memtime();
            r0 = __builtin_amdgcn_s_memrealtime();
        }
    }
    __device__ void stop(uint64_t* clocks) {
        if (threadIdx.x == 0) {
            const uint64_t c1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
            clocks[4 * blockIdx.x + 0] = c0;
            clocks[4 * blockIdx.x + 1] = c1;
            clocks[4 * blockIdx.x + 2] = r0;
            clocks[4 * blockIdx.x + 3] = r1;
        }
    }
};

// 64 KiB of LDS as 64 blocks of 1 KiB, filled with bf16 values near 1.
__device__ __forceinline__ void fill_lds(uint32_t* lds) {
    for (int i = threadIdx.x; i < 16384; i += blockDim.x) lds[i] = 0x3F803F80u ^ (uint32_t)(i & 7);
    __syncthreads();
}
// Wave w's 16-byte operand of step s: block (s + 5 w) mod 64, lane order
// (conflict-free).
__device__ __forceinline__ u32x4 lds_operand(const uint32_t* lds, int s, int w, int lane) {
    return *(const u32x4*)&lds[(((s + w * 5) & 63) * 256) + lane * 4];
}

// 4 WPE waves (WPE per SIMD), each `iters` x 16 MFMAs over 4 accumulator
// chains; MFMA k takes A from LDS read k, issued PF MFMAs earlier.
template <int WPE, int PF>
__global__ __attribute__((amdgpu_flat_work_group_size(256 * WPE, 256 * WPE), amdgpu_waves_per_eu(WPE, WPE)))
void calib_lds_mfma_kernel(float* __restrict__ sink, uint64_t* __restrict__ clocks, int iters) {
    __shared__ __attribute__((aligned(16))) uint32_t lds[16384];
    ClockPair ck;
    ck.start();
    fill_lds(lds);
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    f32x16 acc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = f32x16{0};
    const bf16x8 b = __builtin_bit_cast(bf16x8, u32x4{0x3F803F80u, 0x3F803F81u, 0x3F803F80u, 0x3F803F80u});
    u32x4 ring[PF + 1];
#pragma unroll
    for (int p = 0; p < PF; ++p) ring[p] = lds_operand(lds, p, w, lane);
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int s = 0; s < 16; ++s) {
            ring[(s + PF) % (PF + 1)] = lds_operand(lds, it * 16 + s + PF, w, lane);
            acc[s % 4] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ring[s % (PF + 1)]), b,
                                                                 acc[s % 4], 0, 0, 0);
        }
    }
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 16; ++j) sum += acc[i][j];
    sink[(int64_t)blockIdx.x * 512 + t] = sum;
    ck.stop(clocks);
}

// The same with the 16x16x32 MFMA: 4 WPE waves, each `iters` x 32 MFMAs
// (16384 FLOP each, the FLOP of 16 of the 32x32x16 form) over 8 accumulator
// chains; MFMA k takes A from LDS read k, issued 4 MFMAs earlier.  A 1 KiB
// operand then feeds half the work it feeds in the 32x32x16 form.
template <int WPE>
__global__ __attribute__((amdgpu_flat_work_group_size(256 * WPE, 256 * WPE), amdgpu_waves_per_eu(WPE, WPE)))
void calib_lds_mfma16_kernel(float* __restrict__ sink, uint64_t* __restrict__ clocks, int iters) {
    constexpr int PF = 4;
    __shared__ __attribute__((aligned(16))) uint32_t lds[16384];
    ClockPair ck;
    ck.start();
    fill_lds(lds);
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    f32x4 acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    const bf16x8 b = __builtin_bit_cast(bf16x8, u32x4{0x3F803F80u, 0x3F803F81u, 0x3F803F80u, 0x3F803F80u});
    u32x4 ring[PF + 1];
#pragma unroll
    for (int p = 0; p < PF; ++p) ring[p] = lds_operand(lds, p, w, lane);
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int s = 0; s < 32; ++s) {
            ring[(s + PF) % (PF + 1)] = lds_operand(lds, it * 32 + s + PF, w, lane);
            acc[s % 8] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ring[s % (PF + 1)]), b,
                                                                 acc[s % 8], 0, 0, 0);
        }
    }
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) sum += acc[i][j];
    sink[(int64_t)blockIdx.x * 1024 + t] = sum;
    ck.stop(clocks);
}

// Waves 0-3 run role RA, waves 4-7 (the same four SIMDs) role RB:
//   0 idle; 1 MFMA, register operands, 4 chains, iters_m x 16 MFMAs;
//   2 the same with a 1 KiB LDS read per MFMA, 4 ahead;
//   3 16 independent FMA chains, iters_v x 16 FMAs;
//   4 16 independent exp2 chains, iters_v x 16 exponentials;
//   5 roles 1 and 3 in one wave: each MFMA followed by iters_v / iters_m FMAs
//     (the same totals, interleaved in one instruction stream);
//   6 the same with exp2 in place of the FMAs;
//   7, 8 roles 5, 6 with each MFMA's A operand a 1 KiB LDS read, 4 ahead.
template <int RA, int RB>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void calib_mix_kernel(float* __restrict__ sink, uint64_t* __restrict__ clocks, int iters_m, int iters_v, float c) {
    __shared__ __attribute__((aligned(16))) uint32_t lds[16384];
    ClockPair ck;
    ck.start();
    fill_lds(lds);
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int role = w < 4 ? RA : RB;
    float out = 0.f;
    if (role == 1 || role == 2) {
        f32x16 acc[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = f32x16{0};
        const bf16x8 b = __builtin_bit_cast(bf16x8, u32x4{0x3F803F80u, 0x3F803F81u, 0x3F803F80u, 0x3F803F80u});
        const u32x4 areg = {0x3F803F80u, 1u, 2u, 3u};
        u32x4 ring[5];
#pragma unroll
        for (int p = 0; p < 4; ++p) ring[p] = role == 2 ? lds_operand(lds, p, w, lane) : areg;
        for (int it = 0; it < iters_m; ++it) {
#pragma unroll
            for (int s = 0; s < 16; ++s) {
                if (role == 2) ring[(s + 4) % 5] = lds_operand(lds, it * 16 + s + 4, w, lane);
                const u32x4 a = role == 2 ? ring[s % 5] : areg;
                acc[s % 4] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), b, acc[s % 4], 0,
                                                                     0, 0);
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 16; ++j) out += acc[i][j];
    } else if (role >= 5 && role <= 8) {
        f32x16 acc[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = f32x16{0};
        const bf16x8 b = __builtin_bit_cast(bf16x8, u32x4{0x3F803F80u, 0x3F803F81u, 0x3F803F80u, 0x3F803F80u});
        const u32x4 areg = {0x3F803F80u, 1u, 2u, 3u};
        const bool from_lds = role >= 7, fma_work = role == 5 || role == 7;
        u32x4 ring[5];
#pragma unroll
        for (int p = 0; p < 4; ++p) ring[p] = from_lds ? lds_operand(lds, p, w, lane) : areg;
        float x[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) x[i] = lane * 0.001f + i;
        constexpr int PER = 4;  // vector instructions per MFMA (iters_v = 4 iters_m)
        for (int it = 0; it < iters_m; ++it) {
#pragma unroll
            for (int s = 0; s < 16; ++s) {
                // step s issues the operand read of step s + 4; fences keep each
                // step's MFMA and vector work together and the reads ahead
                if (from_lds) ring[(s + 4) % 5] = lds_operand(lds, it * 16 + s + 4, w, lane);
                __builtin_amdgcn_sched_barrier(0);
                const u32x4 a = from_lds ? ring[s % 5] : areg;
                acc[s % 4] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), b, acc[s % 4], 0,
                                                                     0, 0);
#pragma unroll
                for (int v = 0; v < PER; ++v) {
                    float& y = x[(s * PER + v) % 16];
                    y = fma_work ? __builtin_fmaf(y, c, 0.5f) : __builtin_amdgcn_exp2f(y);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 16; ++j) out += acc[i][j];
#pragma unroll
        for (int i = 0; i < 16; ++i) out += x[i];
    } else if (role == 3 || role == 4) {
        float x[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) x[i] = lane * 0.001f + i;
        for (int it = 0; it < iters_v; ++it) {
#pragma unroll
            for (int i = 0; i < 16; ++i) x[i] = role == 3 ? __builtin_fmaf(x[i], c, 0.5f) : __builtin_amdgcn_exp2f(x[i]);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) out += x[i];
    }
    sink[(int64_t)blockIdx.x * 512 + t] = out;
    ck.stop(clocks);
}

template <int RA>
int launch_mix(int rb, float* sink, uint64_t* clocks, int workgroups, int iters_m, int iters_v, hipStream_t st) {
    void (*k)(float*, uint64_t*, int, int, float) = rb == 0   ? calib_mix_kernel<RA, 0>
                                                    : rb == 3 ? calib_mix_kernel<RA, 3>
                                                    : rb == 4 ? calib_mix_kernel<RA, 4>
                                                    : rb == 5 ? calib_mix_kernel<RA, 5>
                                                    : rb == 6 ? calib_mix_kernel<RA, 6>
                                                    : rb == 7 ? calib_mix_kernel<RA, 7>
                                                              : calib_mix_kernel<RA, 8>;
    hipLaunchKernelGGL(k, dim3(workgroups), dim3(512), 0, st, sink, clocks, iters_m, iters_v, 0.999f);
    return hipGetLastError() == hipSuccess ? 0 : 2;
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

// Matrix cores fed from LDS: `workgroups` workgroups of 4 * waves_per_simd
// waves (1 or 2 per SIMD), each wave `iters` x 16 bf16 32x32x16 MFMAs, every
// MFMA's A operand a 1 KiB LDS read of its own issued `prefetch` (1, 2 or 4)
// MFMAs ahead.  sink (device): workgroups * 512 floats; clocks (device):
// workgroups * 4 uint64 as for fa_calib_mfma.  Returns 0 when the launch was
// accepted, 1 for bad arguments, 2 for a failed launch.
int fa_calib_lds_mfma(float* sink, uint64_t* clocks, int workgroups, int iters, int waves_per_simd, int prefetch,
                      void* stream) {
    if (!sink || !clocks || workgroups < 1 || iters < 1) return 1;
    if (waves_per_simd != 1 && waves_per_simd != 2) return 1;
    if (prefetch != 1 && prefetch != 2 && prefetch != 4) return 1;
    void (*k)(float*, uint64_t*, int) =
        waves_per_simd == 1 ? (prefetch == 1 ? calib_lds_mfma_kernel<1, 1>
                               : prefetch == 2 ? calib_lds_mfma_kernel<1, 2>
                                               : calib_lds_mfma_kernel<1, 4>)
                            : (prefetch == 1 ? calib_lds_mfma_kernel<2, 1>
                               : prefetch == 2 ? calib_lds_mfma_kernel<2, 2>
                                               : calib_lds_mfma_kernel<2, 4>);
    hipLaunchKernelGGL(k, dim3(workgroups), dim3(256 * waves_per_simd), 0, (hipStream_t)stream, sink, clocks, iters);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

// LDS-fed 16x16x32 MFMA calibration: `workgroups` workgroups of 4 x
// waves_per_simd waves (1..4 per SIMD), each iters x 32 MFMAs with a 1 KiB LDS
// read per MFMA, 4 ahead.  sink (device) receives workgroups * 1024 floats,
// clocks as for fa_calib_mfma.  Returns 0 when the launch was accepted, 1 for
// bad arguments, 2 for a failed launch.
int fa_calib_lds_mfma16(float* sink, uint64_t* clocks, int workgroups, int iters, int waves_per_simd,
                        void* stream) {
    if (!sink || !clocks || workgroups < 1 || iters < 1 || waves_per_simd < 1 || waves_per_simd > 4) return 1;
    void (*k)(float*, uint64_t*, int) = waves_per_simd == 1   ? calib_lds_mfma16_kernel<1>
                                        : waves_per_simd == 2 ? calib_lds_mfma16_kernel<2>
                                        : waves_per_simd == 3 ? calib_lds_mfma16_kernel<3>
                                                              : calib_lds_mfma16_kernel<4>;
    hipLaunchKernelGGL(k, dim3(workgroups), dim3(256 * waves_per_simd), 0, (hipStream_t)stream, sink, clocks, iters);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

// Pipe mix: `workgroups` workgroups of 8 waves; waves 0-3 take role_a, waves
// 4-7 (same SIMDs) role_b.  Roles: 0 idle, 1 MFMA from registers and 2 MFMA
// with an LDS read each (iters_m x 16 bf16 32x32x16 MFMAs per wave), 3 FMA
// and 4 exp2 chains (iters_v x 16 per wave), 5 and 6 role 1 with the FMAs
// (exp2s) of role 3 (4) interleaved in the same wave (iters_v must be
// 4 iters_m), 7 and 8 the same with role 2's LDS reads.  role_a in 0..8,
// role_b in 0 or 3..8.  sink and clocks
// as for fa_calib_lds_mfma.  Returns 0 when the launch was accepted, 1 for
// bad arguments, 2 for a failed launch.
int fa_calib_mix(float* sink, uint64_t* clocks, int workgroups, int iters_m, int iters_v, int role_a, int role_b,
                 void* stream) {
    if (!sink || !clocks || workgroups < 1 || iters_m < 0 || iters_v < 0) return 1;
    if (role_a < 0 || role_a > 8 || role_b < 0 || role_b > 8 || role_b == 1 || role_b == 2) return 1;
    if ((role_a >= 5 || role_b >= 5) && iters_v != 4 * iters_m) return 1;
    hipStream_t st = (hipStream_t)stream;
    switch (role_a) {
        case 0: return launch_mix<0>(role_b, sink, clocks, workgroups, iters_m, iters_v, st);
        case 1: return launch_mix<1>(role_b, sink, clocks, workgroups, iters_m, iters_v, st);
        case 2: return launch_mix<2>(role_b, sink, clocks, workgroups, iters_m, iters_v, st);
        case 3: return launch_mix<3>(role_b, sink, clocks, workgroups, iters_m, iters_v, st);
        case 4: return launch_mix<4>(role_b, sink, clocks, workgroups, iters_m, iters_v, st);
        case 5: return launch_mix<5>(role_b, sink, clocks, workgroups, iters_m, iters_v, st);
        case 6: return launch_mix<6>(role_b, sink, clocks, workgroups, iters_m, iters_v, st);
        case 7: return launch_mix<7>(role_b, sink, clocks, workgroups, iters_m, iters_v, st);
        default: return launch_mix<8>(role_b, sink, clocks, workgroups, iters_m, iters_v, st);
    }
}

}  // extern "C"
