// probes.hip -- microbenchmarks that measure ceilings of the MI355X for the rooflines
// reported next to the attention kernels (built into libprobes.so, not into
// libattn.so; bench.py and the profiling runs load it):
//  * read_kernel: streaming 16-byte loads over a buffer, each XCD always reading its own
//    contiguous eighth, so that a buffer whose eighth fits an XCD's L2 (4 MiB) is
//    served by L2, one whose eighth exceeds it but that fits the memory-side cache
//    (MALL, 256 MiB) by the MALL, and a larger one by HBM;
//  * mfma_kernel: independent chains of v_mfma_f32_32x32x16_bf16, timed by the shader
//    clock counter (s_memtime) and the constant 100 MHz counter (s_memrealtime) on
//    each wave, whose ratio is the engine clock under MFMA load;
//  * mfma_chain_kernel: one wave per SIMD running 1, 2 or 4 independent chains of
//    dependent MFMAs, to measure how fast a dependent MFMA issues behind its predecessor;
//  * trans_kernel: independent chains of v_log_f32 followed by v_exp_f32 (the pair the
//    general-power epilogue x^p = exp2(p log2 x) issues per element);
//  * lds_kernel: LDS read throughput of ds_read_b128 (16 bytes per lane) or of the
//    transposing ds_read_b64_tr_b16 (8 bytes per lane), bank-conflict-free addresses,
//    timed by the shader clock on each wave.
// Every loop is bounded by its arguments and every access stays inside its buffer.
#include <hip/hip_runtime.h>
#include <stdint.h>

#define PROBE_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr uint32_t kNever = 0x9e3779b9u;  // a value the reductions below practically never take

// n elements of 16 bytes (n a multiple of 8), grid a multiple of 8.  Workgroups are
// dealt to the 8 XCDs round-robin, so workgroup w runs on XCD w % 8; the workgroups of
// XCD x read the contiguous eighth x of the buffer, thread t of the XCD's workgroup
// number w / 8 reading its elements t + k*stride in every pass (four loads in flight).
__global__ __launch_bounds__(256) void read_kernel(const u32x4 *__restrict__ buf, int64_t n,
                                                   int passes, uint32_t *__restrict__ sink) {
    const int64_t per_xcd = n / 8;
    const u32x4 *part = buf + (int64_t)(blockIdx.x & 7) * per_xcd;
    const int64_t stride = (int64_t)(gridDim.x / 8) * 256;
    const int64_t first = (int64_t)(blockIdx.x >> 3) * 256 + threadIdx.x;
    uint32_t acc = 0;
    for (int p = 0; p < passes; ++p) {
        int64_t i = first;
        for (; i + 3 * stride < per_xcd; i += 4 * stride) {
            const u32x4 a = part[i], b = part[i + stride], c = part[i + 2 * stride],
                        d = part[i + 3 * stride];
            const u32x4 x = a ^ b ^ c ^ d;
            acc ^= x.x ^ x.y ^ x.z ^ x.w;
        }
        for (; i < per_xcd; i += stride) {
            const u32x4 a = part[i];
            acc ^= a.x ^ a.y ^ a.z ^ a.w;
        }
    }
    if (acc == kNever) sink[0] = acc;
}

// Four independent accumulators per wave; clk[2*w] = shader clock cycles and
// clk[2*w + 1] = 100 MHz ticks spent by wave w in the loop.
__global__ __launch_bounds__(256) void mfma_kernel(int iters, float *__restrict__ sink,
                                                   uint64_t *__restrict__ clk) {
    const int lane = threadIdx.x & 63;
    bf16x8 a, b;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        a[t] = (__bf16)(0.001f * (float)(lane + t));
        b[t] = (__bf16)(0.002f * (float)(lane - t));
    }
    f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    const uint64_t t0 = __builtin_amdgcn_s_memtime();
    const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
    for (int i = 0; i < iters; ++i) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
    if (s == 1234.5f) sink[0] = s;
    const int w = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (lane == 0) {
        clk[2 * w] = t1 - t0;
        clk[2 * w + 1] = r1 - r0;
    }
}

// One wave per SIMD (a single-wave workgroup, one workgroup per SIMD of the chip) running
// CH independent chains of dependent v_mfma_f32_32x32x16_bf16 (each accumulating into its
// own registers), to see how fast back-to-back dependent MFMAs issue.
template <int CH>
__global__ __launch_bounds__(64) void mfma_chain_kernel(int iters, float *__restrict__ sink) {
    const int lane = threadIdx.x & 63;
    bf16x8 a, b;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        a[t] = (__bf16)(0.001f * (float)(lane + t));
        b[t] = (__bf16)(0.002f * (float)(lane - t));
    }
    f32x16 c[CH];
#pragma unroll
    for (int j = 0; j < CH; ++j) c[j] = f32x16{};
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int j = 0; j < CH; ++j) c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[j], 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < CH; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += c[j][r];
    if (s == 1234.5f) sink[0] = s;
}

// Eight independent chains per lane of x <- 2^-|log2 |x||, which stays in (0, 1]:
// each step is one v_log_f32 and one v_exp_f32 with input modifiers only.
__global__ __launch_bounds__(256) void trans_kernel(int iters, float *__restrict__ sink) {
    float x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = 0.3f + 0.01f * (float)((threadIdx.x + j) & 31);
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
            x[j] = __builtin_amdgcn_exp2f(-__builtin_fabsf(__builtin_amdgcn_logf(__builtin_fabsf(x[j]))));
    }
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) s += x[j];
    if (s == 1234.5f) sink[0] = s;
}

// Each workgroup fills a 32 KiB LDS buffer, then each wave reads it `iters` times 8
// reads per iteration: MODE 0 ds_read_b128 with lane l at 16-byte chunk (l + 64 j + 512 s)
// mod 2048 (16 consecutive lanes cover the 64 banks once), MODE 1 ds_read_b64_tr_b16 with
// lane l at 8-byte chunk (l + 64 j + 512 s) mod 4096.  clk as in mfma_kernel.
typedef short v4i16 __attribute__((ext_vector_type(4)));
template <int MODE>
__global__ __launch_bounds__(256) void lds_kernel(int iters, uint32_t *__restrict__ sink,
                                                  uint64_t *__restrict__ clk) {
    __shared__ __attribute__((aligned(16))) u32x4 buf[2048];
    for (int k = threadIdx.x; k < 2048; k += 256)
        buf[k] = u32x4{(uint32_t)k, (uint32_t)k * 3u, (uint32_t)k * 5u, (uint32_t)k * 7u};
    __syncthreads();
    const int lane = threadIdx.x & 63;
    u32x4 acc = {0u, 0u, 0u, 0u};
    const uint64_t t0 = __builtin_amdgcn_s_memtime();
    const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
    for (int i = 0; i < iters; ++i) {
        const int s = 512 * (i & 3);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if constexpr (MODE == 0) {
                acc ^= buf[(lane + 64 * j + s) & 2047];
            } else {
                const int c = (lane + 64 * j + s) & 4095;
                const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) v4i16 *)((__attribute__((address_space(3))) uint8_t *)buf + 8 * c));
                acc[j & 3] ^= (uint32_t)(uint16_t)v[0] | ((uint32_t)(uint16_t)v[1] << 16);
                acc[(j + 1) & 3] ^= (uint32_t)(uint16_t)v[2] | ((uint32_t)(uint16_t)v[3] << 16);
            }
        }
    }
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
    if ((acc[0] ^ acc[1] ^ acc[2] ^ acc[3]) == kNever) sink[0] = acc[0];
    const int w = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (lane == 0) {
        clk[2 * w] = t1 - t0;
        clk[2 * w + 1] = r1 - r0;
    }
}

}  // namespace

// Streaming read of `bytes` (a multiple of 128) at `buf`, `passes` times, by `grid`
// workgroups of 256 threads (a multiple of 8).  Returns the HIP launch status.
PROBE_EXPORT int probe_read(const void *buf, int64_t bytes, int passes, int grid, void *sink,
                            void *stream) {
    if (!buf || !sink || bytes < 128 || (bytes & 127) || passes < 1 || grid < 8 || (grid & 7))
        return -1;
    hipLaunchKernelGGL(read_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream,
                       (const u32x4 *)buf, bytes / 16, passes, (uint32_t *)sink);
    return (int)hipGetLastError();
}

// `iters` iterations of 4 MFMAs (32x32x16 bf16, 32768 FLOPs each) per wave, `grid`
// workgroups of 4 waves; clk holds 2 uint64 per wave (shader cycles, 100 MHz ticks).
PROBE_EXPORT int probe_mfma(int iters, int grid, void *sink, void *clk, void *stream) {
    if (!sink || !clk || iters < 1 || grid < 1) return -1;
    hipLaunchKernelGGL(mfma_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, iters,
                       (float *)sink, (uint64_t *)clk);
    return (int)hipGetLastError();
}

// `iters` MFMAs per chain, `chains` (1, 2 or 4) independent chains per wave, one wave per
// workgroup, `grid` workgroups.
PROBE_EXPORT int probe_mfma_chains(int iters, int chains, int grid, void *sink, void *stream) {
    if (!sink || iters < 1 || grid < 1) return -1;
    if (chains == 1)
        hipLaunchKernelGGL(mfma_chain_kernel<1>, dim3(grid), dim3(64), 0, (hipStream_t)stream, iters, (float *)sink);
    else if (chains == 2)
        hipLaunchKernelGGL(mfma_chain_kernel<2>, dim3(grid), dim3(64), 0, (hipStream_t)stream, iters, (float *)sink);
    else if (chains == 4)
        hipLaunchKernelGGL(mfma_chain_kernel<4>, dim3(grid), dim3(64), 0, (hipStream_t)stream, iters, (float *)sink);
    else
        return -1;
    return (int)hipGetLastError();
}

// `iters` iterations of 8 (log, exp) pairs per lane, `grid` workgroups of 256 threads.
PROBE_EXPORT int probe_trans(int iters, int grid, void *sink, void *stream) {
    if (!sink || iters < 1 || grid < 1) return -1;
    hipLaunchKernelGGL(trans_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, iters,
                       (float *)sink);
    return (int)hipGetLastError();
}

// `iters` iterations of 8 LDS reads per wave (mode 0: ds_read_b128, 1 KiB per read and
// wave; mode 1: ds_read_b64_tr_b16, 512 bytes), `grid` workgroups of 4 waves; clk holds
// 2 uint64 per wave (shader cycles, 100 MHz ticks).
PROBE_EXPORT int probe_lds(int iters, int mode, int grid, void *sink, void *clk, void *stream) {
    if (!sink || !clk || iters < 1 || grid < 1 || (mode != 0 && mode != 1)) return -1;
    if (mode == 0)
        hipLaunchKernelGGL(lds_kernel<0>, dim3(grid), dim3(256), 0, (hipStream_t)stream, iters,
                           (uint32_t *)sink, (uint64_t *)clk);
    else
        hipLaunchKernelGGL(lds_kernel<1>, dim3(grid), dim3(256), 0, (hipStream_t)stream, iters,
                           (uint32_t *)sink, (uint64_t *)clk);
    return (int)hipGetLastError();
}
