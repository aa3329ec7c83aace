// Shared device helpers for the gfx950 kernels (wave64, bf16 MFMA).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "spark_attn.h"

namespace spark {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kMaxBlocks = 16384;  // largest M the select / attention LDS tables are sized for

// Maximum of v over lanes l and l ^ 32 (the two 32-lane halves of the wave), in one VALU swap
// (v_permlane32_swap) instead of a round trip through the LDS crossbar.  Whichever way the swap
// assigns its two results, together they hold v of both lanes.
__device__ __forceinline__ float half_max(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// A route entry read from caller memory, clamped to the key blocks [0, Mk): a bad entry then selects
// a wrong block rather than reading or writing out of bounds.
__device__ __forceinline__ int clamp_block(int J, int Mk) { return min(max(J, 0), Mk - 1); }

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// Eight consecutive input elements (bf16 or fp32) widened to fp32.
template <typename T> struct In;
template <> struct In<__bf16> {
    static constexpr int kBytes = 2;
    __device__ __forceinline__ static void load8(const __bf16* p, float (&v)[8]) {
        const u32x4 u = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[2 * j] = bf16_bits_to_f32(u[j] & 0xffffu);
            v[2 * j + 1] = bf16_bits_to_f32(u[j] >> 16);
        }
    }
};
template <> struct In<float> {
    static constexpr int kBytes = 4;
    __device__ __forceinline__ static void load8(const float* p, float (&v)[8]) {
        const f32x4 a = *reinterpret_cast<const f32x4*>(p);
        const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) { v[j] = a[j]; v[4 + j] = b[j]; }
    }
};

// Eight consecutive input elements kept as raw bits (loaded now, widened later), so that a
// thread can have all of its loads in flight before it needs any value.
template <typename T> struct Raw8;
template <> struct Raw8<__bf16> {
    u32x4 u;
    __device__ __forceinline__ void load(const __bf16* p) { u = *reinterpret_cast<const u32x4*>(p); }
    __device__ __forceinline__ void widen(float (&v)[8]) const {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[2 * j] = bf16_bits_to_f32(u[j] & 0xffffu);
            v[2 * j + 1] = bf16_bits_to_f32(u[j] >> 16);
        }
    }
};
template <> struct Raw8<float> {
    f32x4 a, b;
    __device__ __forceinline__ void load(const float* p) {
        a = *reinterpret_cast<const f32x4*>(p);
        b = *reinterpret_cast<const f32x4*>(p + 4);
    }
    __device__ __forceinline__ void widen(float (&v)[8]) const {
#pragma unroll
        for (int j = 0; j < 4; ++j) { v[j] = a[j]; v[4 + j] = b[j]; }
    }
};

// Eight consecutive elements as packed bf16 (16 bytes), rounding fp32 to nearest even.
__device__ __forceinline__ u32x4 pack8_bf16(const float (&v)[8]) {
    u32x4 r;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const __bf16 lo = (__bf16)v[2 * j], hi = (__bf16)v[2 * j + 1];
        r[j] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
    }
    return r;
}

template <typename T> __device__ __forceinline__ u32x4 load8_as_bf16(const T* p);
template <> __device__ __forceinline__ u32x4 load8_as_bf16<__bf16>(const __bf16* p) {
    return *reinterpret_cast<const u32x4*>(p);
}
template <> __device__ __forceinline__ u32x4 load8_as_bf16<float>(const float* p) {
    float v[8];
    In<float>::load8(p, v);
    return pack8_bf16(v);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

// amax = max(amax, v) for a non-negative float v held as its bits (non-negative floats order as
// unsigned integers).  The atomic is skipped when the current value is already as large: once the
// running maximum is reached, most callers only read it, so many workgroups raising one value do
// not queue on its atomic unit (a stale read only costs an extra atomic).
__device__ __forceinline__ void raise_max_bits(uint32_t* amax, float v) {
    const uint32_t b = __float_as_uint(v);
    if (b > __hip_atomic_load(amax, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) atomicMax(amax, b);
}

__device__ __forceinline__ int wave_sum_int(int v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

__device__ __forceinline__ uint64_t lanemask_lt() {
    const int lane = threadIdx.x & 63;
    return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

}  // namespace spark
