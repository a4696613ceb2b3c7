// Device helpers shared by the gfx950 kernels of the decode layer step.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/dl.h"

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));

#define DL_WAVE 64

// ------------------------------------------------------------------ numbers
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16, round to nearest even (inputs are finite).
__device__ __forceinline__ uint16_t f32_to_bf16(float f)
{
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Two OCP e4m3fn codes (bytes 0,1 or 2,3 of w) -> fp32 with the gfx950 converter.
__device__ __forceinline__ v2f fp8x2_lo(uint32_t w) { return __builtin_amdgcn_cvt_pk_f32_fp8(w, false); }
__device__ __forceinline__ v2f fp8x2_hi(uint32_t w) { return __builtin_amdgcn_cvt_pk_f32_fp8(w, true); }

// Round two fp32 values to e4m3fn codes (|v| already <= 448), packed into the low 16 bits.
__device__ __forceinline__ uint32_t f32x2_to_fp8(float a, float b)
{
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}

// Byte offset of key byte i of item `row` in an index-key cache of DI bytes per item: row-major, or the tiled
// layout (per 16 consecutive items: [DI / 64 chunks][4 groups of 16 bytes][16 items][16 bytes]).
__host__ __device__ __forceinline__ long key_offset(long row, int i, int DI, bool tiles)
{
    return tiles ? (row & ~15L) * DI + (i >> 6) * 1024 + ((i >> 4) & 3) * 256 + (row & 15) * 16 + (i & 15)
                 : row * DI + i;
}

__device__ __forceinline__ float act_load(const void *p, int dt, long i)
{
    return dt == DL_BF16 ? bf16_to_f32(((const uint16_t *)p)[i]) : ((const float *)p)[i];
}

// ------------------------------------------------------------- wave reductions
__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}
__device__ __forceinline__ double wave_sum_d(double v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}
__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}
__device__ __forceinline__ int wave_max_i(int v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o, 64));
    return v;
}
__device__ __forceinline__ int wave_sum_i(int v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// Device-scope accesses (coherent across the eight XCDs' L2 caches: stores write through, loads do not hit a
// line another XCD may have changed) for data handed between workgroups inside one launch.
__device__ __forceinline__ float ld_dev(const float *p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ int ld_dev(const int *p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ unsigned long long ld_dev(const unsigned long long *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(float *p, float v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ void st_dev(uint16_t *p, uint16_t v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ void st_dev(unsigned *p, unsigned v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ void st_dev(unsigned long long *p, unsigned long long v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Coherent (device-scope) load of data other workgroups of the same launch wrote with atomics.
__device__ __forceinline__ int ld_agent(const int *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned ld_agent_u(const unsigned *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ v4i ldg16(const void *p) { return *(const v4i *)p; }
