// swa_device.hpp - device-side helpers shared by the libswa kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace swa {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// bfloat16 values travel as raw 16-bit patterns.
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h16) {
    return __uint_as_float(h16 << 16);
}

// Round-to-nearest-even float -> bfloat16 (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
    __bf16 h = (__bf16)x;
    return __builtin_bit_cast(uint16_t, h);
}

// Two floats -> one dword holding two bfloat16 (lo = a, hi = b).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    f32x2_t f = {a, b};
    bf16x2_t h = __builtin_convertvector(f, bf16x2_t);
    return __builtin_bit_cast(uint32_t, h);
}

// Two floats -> one dword holding two float16, round to nearest even (v_cvt_pk_f16_f32).
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
    f32x2_t f = {a, b};
    f16x2_t h = __builtin_convertvector(f, f16x2_t);
    return __builtin_bit_cast(uint32_t, h);
}

// Element access for the two supported element types (0 = float32, 1 = bfloat16).
template <int DT> struct Elem;
template <> struct Elem<0> {
    typedef float storage;
    __device__ __forceinline__ static float load(const void *p, int64_t i) {
        return static_cast<const float *>(p)[i];
    }
    __device__ __forceinline__ static void store(void *p, int64_t i, float x) {
        static_cast<float *>(p)[i] = x;
    }
};
template <> struct Elem<1> {
    typedef uint16_t storage;
    __device__ __forceinline__ static float load(const void *p, int64_t i) {
        return bf16_bits_to_f32(static_cast<const uint16_t *>(p)[i]);
    }
    __device__ __forceinline__ static void store(void *p, int64_t i, float x) {
        static_cast<uint16_t *>(p)[i] = f32_to_bf16_bits(x);
    }
};

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
    return x;
}

// Quiet NaN used to flag outputs of queries whose position could not be served.
__device__ __forceinline__ float qnan() { return __uint_as_float(0x7fc00000u); }

}  // namespace swa
