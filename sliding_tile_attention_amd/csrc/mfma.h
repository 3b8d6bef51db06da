// MFMA fragment conventions shared by the bf16 attention kernels (gfx950).
//
// v_mfma_f32_32x32x16_bf16 computes C[32x32] += A[32x16] * B[16x32].
// Lane l (0..63) supplies row i = l%32 of A and column j = l%32 of B, each
// as 8 bf16 values of the reduction index; lanes 0-31 and 32-63 supply the
// two halves of the 16-long reduction.  Which physical k a value maps to
// does not matter as long as A and B agree, so every kernel picks the
// reduction order that makes its operand loads contiguous.
// The result lane l, register r holds C[i][j] with
//     j = l % 32,   i = 8*(r/4) + 4*(l/32) + r%4.
//
// Row permutation sigma: if the A rows fed to an MFMA are permuted by
// sigma (swap bits 2 and 3 of the row index), the 16 result registers of
// lane l hold rows 16*(r/8) + 8*(l/32) + r%8 -- i.e. registers 8k..8k+7
// are 8 CONSECUTIVE rows, which is exactly the operand shape the next MFMA
// needs when those rows become its reduction index.
#pragma once

#include <hip/hip_runtime.h>

namespace sta {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ inline int sigma32(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

// Row of the result held by register r of lane l (unpermuted A rows).
__device__ inline int mfma_row(int lane, int r) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

// Row held by register r of lane l when the A rows were permuted by sigma.
__device__ inline int mfma_row_sigma(int lane, int r) { return 16 * (r >> 3) + 8 * (lane >> 5) + (r & 7); }

__device__ inline f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ inline bf16x8 zero8() { return __builtin_bit_cast(bf16x8, (u32x4){0u, 0u, 0u, 0u}); }

__device__ inline bf16x8 ld8(const __bf16 *p) { return *(const bf16x8 *)p; }

// max / sum of x over lanes l and l^32 (v_permlane32_swap: each lane gets
// its own value and its partner's, in some order).
__device__ inline float max_pair32(float x)
{
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float sum_pair32(float x)
{
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// LDS transpose read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lane i receives element (i%4) of the 8-byte chunks addressed by lanes
// 4j + i/4 of its group, j = 0..3.  If lane s = 4j + c of a group points at
// row (r0 + j), columns (c0 + 4c .. c0 + 4c + 3) of a row-major bf16 matrix,
// lane i of the group receives rows r0..r0+3 of column c0 + i.
__device__ inline bf16x4 ld_tr4(const __bf16 *p)
{
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(p));
}

__device__ inline bf16x8 cat8(bf16x4 a, bf16x4 b)
{
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Sum of the 8 bf16 values of v, accumulated in fp32 onto acc (v_dot2 with 1s).
__device__ inline float sum8(bf16x8 v, float acc)
{
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 0, 1), one, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 2, 3), one, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 4, 5), one, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 6, 7), one, acc, false);
    return acc;
}

// Wait until at most N vector-memory operations of this wave are in flight
// (lgkm and export counters untouched).
template <int N>
__device__ inline void wait_vmem()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Workgroup barrier without the release fence of __syncthreads() (which
// waits for every outstanding memory operation, LDS copies in flight
// included).  Callers make the LDS data they hand over visible themselves:
// LDS reads are complete once their results are used, and asynchronous
// global -> LDS copies are waited for with wait_vmem.  The empty asm
// statements keep the compiler from moving memory accesses across it.
__device__ inline void barrier_nofence()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Buffer descriptor over `bytes` bytes from `base` (raw addressing: loads at
// offsets >= bytes return zero).
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, bytes, 0x00020000);
}

// Asynchronous 16-byte buffer -> LDS copy: lane l's 16 bytes at descriptor
// offset voffset + soffset land at lds_base + 16*l (lds_base and soffset
// wave-uniform).  The per-lane offset is a plain register that can stay
// loop-invariant.
__device__ inline void b2lds16(__amdgpu_buffer_rsrc_t r, int voffset, void *lds_base, int soffset = 0)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds_base, 16, voffset,
                                             soffset, 0, 0);
}

}  // namespace sta
