// Device helpers shared by the gfx950 kernels of the MoE-layer forward.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));

// bf16 bit pattern -> fp32 (exact)
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16 bit pattern, round to nearest even (finite values)
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Split v into bf16 hi + bf16 lo with hi + lo == v to 16 significant bits; returns bit patterns.
__device__ __forceinline__ void split_bf16(float v, uint32_t &hi, uint32_t &lo) {
    hi = f32_to_bf16_rne(v);
    lo = f32_to_bf16_rne(v - __uint_as_float(hi << 16));
}

// acc + a.lo*b.lo + a.hi*b.hi for two packed bf16 pairs (v_dot2c_f32_bf16)
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), acc,
                                           false);
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Read of a value that no kernel of the launch writes, through the constant address space: with a
// wave-uniform index it becomes a scalar-unit load, which leaves the vector-memory counter (and so the
// weight loads in flight) alone.
__device__ __forceinline__ int32_t ld_const(const int32_t *p, long i) {
    return ((const __attribute__((address_space(4))) int32_t *)p)[i];
}

// Raw buffer loads: an offset at or beyond the descriptor's byte count returns zeros without touching
// memory, so loads that may fall outside their row stay branch-free and keep many requests in flight.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOOB = 0x80000000u;  // offset that is always out of range
// Every buffer a kernel addresses through a descriptor stays below kOOB bytes: the marker is then out of range
// for every descriptor, and no valid offset reaches it.  The host rejects shapes that would pass this.
constexpr long kMaxDescBytes = 1L << 31;
constexpr int kRsrcWord3 = 0x00020000;  // gfx9-family raw buffer descriptor, 32-bit data

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, kRsrcWord3);
}

__device__ __forceinline__ uint4 buf_load16(rsrc_t r, uint32_t off) {
    typedef int i32x4 __attribute__((ext_vector_type(4)));
    const i32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
    return make_uint4((uint32_t)v.x, (uint32_t)v.y, (uint32_t)v.z, (uint32_t)v.w);
}

__device__ __forceinline__ double buf_load_f64(rsrc_t r, uint32_t off) {
    typedef int i32x2 __attribute__((ext_vector_type(2)));
    const i32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0);
    return __builtin_bit_cast(double, v);
}

__device__ __forceinline__ uint32_t buf_load4(rsrc_t r, uint32_t off) {
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}

__device__ __forceinline__ uint16_t buf_load2(rsrc_t r, uint32_t off) {
    return (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
}

}  // namespace moe
