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
//
// 3. mfma_rate_kernel: the sustained rate of v_mfma_f32_32x32x16_bf16, the
//    matrix instruction of the bf16 attention kernels, with nothing else
//    issued.  Every wave runs `iters` rounds of 16 MFMAs over 4 independent
//    accumulators; their operands rotate over 4 register sets of
//    pseudo-random bf16 values, so that the operand data changes from one
//    instruction to the next as it does in a real product (constant
//    operands draw less power and would let the clock rise).  A launch
//    executes blocks * 4 waves * iters * 16 MFMAs of 32*32*16*2 flop.
//
// 4. lds_rate_kernel: the rate of plain 16-byte LDS reads (ds_read_b128), the
//    row reads the attention kernels feed their MFMAs with.  Each workgroup
//    fills a 32 KB LDS tile, then every thread runs `iters` rounds of 16
//    reads, consecutive lanes on consecutive 16-byte granules (no bank
//    conflicts), the granule moving by one per round so that no read is
//    loop-invariant; the XOR of what it read is written out.  A launch reads
//    blocks * 256 * iters * 16 * 16 bytes.
//
// 5. block_copy_kernel: the attention kernels' key/value block copies with
//    nothing else issued.  A workgroup of 4 waves moves 16 KB blocks (32 rows
//    of K and V at D = 128) from global memory into a 2-slot LDS ring with
//    16-byte buffer-to-LDS loads, waits for them and meets at a barrier, as
//    the kernels do once per key block.  The blocks come in turn from a
//    source region of `bytes` bytes: a few MB stay in L2, a large region
//    streams from HBM.  A launch copies blocks * iters * 16 KB.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mfma.h"

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
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// a value in [-1, 1) from an integer (a 32-bit mixing function)
__device__ inline float mix_unit(uint32_t x)
{
    x ^= x >> 16;
    x *= 0x7feb352dU;
    x ^= x >> 15;
    x *= 0x846ca68bU;
    x ^= x >> 16;
    return (float)(x & 0xffff) * (2.0f / 65536.0f) - 1.0f;
}

__global__ __launch_bounds__(256, 2) void mfma_rate_kernel(float *__restrict__ out, int iters)
{
    const uint32_t t = blockIdx.x * 256u + threadIdx.x;
    bf16x8 a[4], b[4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            a[m][i] = (__bf16)mix_unit(t * 64u + m * 8u + i);
            b[m][i] = (__bf16)mix_unit(t * 64u + 32u + m * 8u + i + 0x9e3779b9u);
        }
    f32x16 acc[4] = {};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int m = 0; m < 4; ++m)
                acc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(u + m) & 3], b[(u + 2 * m + 1) & 3], acc[m], 0, 0,
                                                                 0);
    }
    float s = 0.f;
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int i = 0; i < 16; ++i) s += acc[m][i];
    out[t] = s;
}

// grid-stride copy: granule i of src to granule i of dst
__global__ __launch_bounds__(256) void copy_probe_kernel(const u32x4 *__restrict__ src, u32x4 *__restrict__ dst,
                                                         int64_t n)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

__global__ __launch_bounds__(256) void lds_rate_kernel(uint32_t *__restrict__ out, int iters)
{
    constexpr int G = 2048;                          // 16-byte granules: 32 KB
    __shared__ u32x4 tile[G];
    for (int i = threadIdx.x; i < G; i += 256) tile[i] = (u32x4){(uint32_t)i, (uint32_t)i * 3u, ~(uint32_t)i, 7u};
    __syncthreads();
    u32x4 x = {0u, 0u, 0u, 0u};
    int g = threadIdx.x;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int k = 0; k < 16; ++k) x ^= tile[(g + (G / 16) * k) & (G - 1)];   // 16 distinct granules
        g = (g + 1) & (G - 1);
    }
    out[blockIdx.x * 256u + threadIdx.x] = x[0] ^ x[1] ^ x[2] ^ x[3];
}

__global__ __launch_bounds__(256) void block_copy_kernel(const char *__restrict__ src, int region_blocks, int iters,
                                                         int32_t *__restrict__ out)
{
    constexpr int BLOCK = 16384;
    __shared__ __attribute__((aligned(1024))) char ring[2][BLOCK];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int off = (wave * 64 + lane) * 16;             // this lane's granule of each 4 KB quarter
    int b = (int)(blockIdx.x % (unsigned)region_blocks);
    for (int it = 0; it < iters; ++it) {
        const auto rs = sta::make_rsrc(src + (int64_t)b * BLOCK, BLOCK);
        char *dst = ring[it & 1];
#pragma unroll
        for (int i = 0; i < 4; ++i) sta::b2lds16(rs, off + i * 4096, dst + (i * 4 + wave) * 1024);
        sta::wait_vmem<0>();
        sta::barrier_nofence();
        b = b + 1 == region_blocks ? 0 : b + 1;
    }
    __syncthreads();
    out[blockIdx.x * 256u + tid] = ((const int32_t *)ring[0])[tid] ^ ((const int32_t *)ring[1])[tid];
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

// Enqueues one LDS read-rate launch of `blocks` workgroups of 256 threads
// on `stream`; out holds blocks * 256 uint32 (device).  Returns 0, or the HIP
// error code of the launch (1 for a non-positive size).
int sta_probe_lds(uint32_t *out, int blocks, int iters, void *stream)
{
    if (blocks <= 0 || iters < 0) return 1;
    hipLaunchKernelGGL(lds_rate_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, out, iters);
    return (int)hipGetLastError();
}

// Enqueues one matrix-core rate launch of `blocks` workgroups of 256
// threads on `stream`; out holds blocks * 256 floats (device).  Returns 0, or
// the HIP error code of the launch (1 for a non-positive size).
int sta_probe_mfma(float *out, int blocks, int iters, void *stream)
{
    if (blocks <= 0 || iters < 0) return 1;
    hipLaunchKernelGGL(mfma_rate_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, out, iters);
    return (int)hipGetLastError();
}

// Enqueues one block-copy launch of `blocks` workgroups of 256 threads on
// `stream`: each copies `iters` 16 KB blocks of the source region (device,
// `bytes` a positive multiple of 16384, 16-byte aligned) into LDS; out holds
// blocks * 256 int32 (device).  Returns 0, or the HIP error code of the
// launch (1 for a bad size).
int sta_probe_block_copy(const void *src, int64_t bytes, int blocks, int iters, int32_t *out, void *stream)
{
    if (bytes < 16384 || bytes % 16384 != 0 || bytes / 16384 > INT32_MAX || blocks <= 0 || iters < 1) return 1;
    hipLaunchKernelGGL(block_copy_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                       (const char *)src, (int)(bytes / 16384), iters, out);
    return (int)hipGetLastError();
}

}  // extern "C"
