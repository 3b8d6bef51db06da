// Measurement probes (not part of the attention ABI; a library of their own,
// libsta_probe.so, that the benchmark loads beside libsta).
//
// 1. exp_rate_kernel: the rate of the hardware base-2 exponential,
//    v_exp_f32, which the attention forward issues once per score of its
//    online softmax.  Every thread runs `iters` rounds of 16 independent
//    exponential chains (so that issue, not latency, limits the rate), each
//    round replacing every x by 2^-x (one v_exp_f32 with a negated source;
//    the values stay in [0.5, 1]), and writes one sum so that no work is
//    dropped.  A launch issues blocks * 256 * iters * 16 exponentials.
//
// 2. copy_probe_kernel: a plain streaming copy of n 16-byte granules, every
//    source byte read once and every destination byte written once, so its
//    HBM traffic is known exactly (2 * 16 * n bytes).  The hardware traffic
//    counters (FETCH_SIZE, WRITE_SIZE) of the attention kernels are scaled
//    by what they read for this launch.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__global__ __launch_bounds__(256) void exp_rate_kernel(float *__restrict__ out, int iters, float seed)
{
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = (float)((threadIdx.x + 17 * i) & 255) * (1.0f / 256.0f) + seed;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < 16; ++i) x[i] = __builtin_amdgcn_exp2f(-x[i]);
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) s += x[i];
    out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// grid-stride copy: granule i of src to granule i of dst
__global__ __launch_bounds__(256) void copy_probe_kernel(const u32x4 *__restrict__ src, u32x4 *__restrict__ dst,
                                                         int64_t n)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

}  // namespace

extern "C" {

// Enqueues one exponential-rate launch of `blocks` workgroups of 256 threads
// on `stream`; out holds blocks * 256 floats (device).  Returns 0, or the HIP
// error code of the launch (1 for a non-positive size).
int sta_probe_exp(float *out, int blocks, int iters, void *stream)
{
    if (blocks <= 0 || iters < 0) return 1;
    hipLaunchKernelGGL(exp_rate_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, out, iters, 0.0f);
    return (int)hipGetLastError();
}

// Enqueues one copy of `bytes` bytes (a positive multiple of 16; both
// buffers on the device, 16-byte aligned, not overlapping) on `stream`.
// Returns 0, or the HIP error code of the launch (1 for a bad size).
int sta_probe_copy(const void *src, void *dst, int64_t bytes, void *stream)
{
    if (bytes <= 0 || bytes % 16 != 0) return 1;
    const int64_t n = bytes / 16;
    hipLaunchKernelGGL(copy_probe_kernel, dim3(4096), dim3(256), 0, (hipStream_t)stream, (const u32x4 *)src,
                       (u32x4 *)dst, n);
    return (int)hipGetLastError();
}

}  // extern "C"
