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

// 16-byte loads and stores in the global address space (device pointers that the compiler
// cannot trace back to a kernel argument would otherwise become flat accesses).
typedef unsigned int u32x4_ev __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const u32x4_ev global_cu4;
typedef __attribute__((address_space(1))) u32x4_ev global_u4;
__device__ __forceinline__ uint4 ldg16(const void *p) {
    const u32x4_ev x = *(global_cu4 *)p;
    return make_uint4(x[0], x[1], x[2], x[3]);
}
__device__ __forceinline__ void stg16(void *p, uint4 x) {
    const u32x4_ev v = {x.x, x.y, x.z, x.w};
    *(global_u4 *)p = v;
}

// Eight bf16 values (16 bytes) -> eight float16 values, round to nearest even.
__device__ __forceinline__ uint4 convert_bf16x8_to_f16x8(uint4 x) {
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
    uint32_t r[4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
        r[m] = pack_f16x2(__uint_as_float(w[m] << 16), __uint_as_float(w[m] & 0xffff0000u));
    return make_uint4(r[0], r[1], r[2], r[3]);
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

__device__ __forceinline__ float4 as_float4(uint4 x) {
    return make_float4(__uint_as_float(x.x), __uint_as_float(x.y), __uint_as_float(x.z),
                       __uint_as_float(x.w));
}

// Eight consecutive elements (16-byte aligned) as floats, and back: one 16-byte access for
// bf16, two for float32.
template <int DT>
__device__ __forceinline__ void load8f(const void *base, int64_t off, float (&x)[8]) {
    if (DT == 1) {
        const uint4 u = ldg16(static_cast<const uint16_t *>(base) + off);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            x[2 * m] = __uint_as_float(w[m] << 16);
            x[2 * m + 1] = __uint_as_float(w[m] & 0xffff0000u);
        }
    } else {
        const uint4 a = ldg16(static_cast<const float *>(base) + off);
        const uint4 b = ldg16(static_cast<const float *>(base) + off + 4);
        const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int m = 0; m < 8; ++m) x[m] = __uint_as_float(w[m]);
    }
}
template <int DT>
__device__ __forceinline__ void store8f(void *base, int64_t off, const float (&x)[8]) {
    if (DT == 1) {
        stg16(static_cast<uint16_t *>(base) + off,
              make_uint4(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]),
                         pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7])));
    } else {
        stg16(static_cast<float *>(base) + off,
              make_uint4(__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]),
                         __float_as_uint(x[3])));
        stg16(static_cast<float *>(base) + off + 4,
              make_uint4(__float_as_uint(x[4]), __float_as_uint(x[5]), __float_as_uint(x[6]),
                         __float_as_uint(x[7])));
    }
}

// Rotate four interleaved pairs by the angles (cos, sin) in t0 = (c0, s0, c1, s1) and t1.
__device__ __forceinline__ void rotate8(float (&x)[8], float4 t0, float4 t1) {
    const float c[4] = {t0.x, t0.z, t1.x, t1.z}, sn[4] = {t0.y, t0.w, t1.y, t1.w};
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const float a = x[2 * m], b = x[2 * m + 1];
        x[2 * m] = fmaf(-b, sn[m], a * c[m]);
        x[2 * m + 1] = fmaf(a, sn[m], b * c[m]);
    }
}

template <int CTRL>
__device__ __forceinline__ float dpp_f(float x);

// Wavefront-wide sum / max: DPP within each row of 16 lanes, then the four row results
// combined through scalar reads (no LDS permute round trips).
__device__ __forceinline__ float row16_max(float x);
__device__ __forceinline__ float row16_sum(float x);
__device__ __forceinline__ float wave_sum(float x) {
    x = row16_sum(x);
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
    return (r0 + r1) + (r2 + r3);
}
__device__ __forceinline__ float wave_max(float x) {
    x = row16_max(x);
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
    return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// Sums over aligned groups of 8 or 16 lanes with DPP lane permutations (no LDS traffic):
// xor-1 and xor-2 quad permutes, then the half-row and row mirrors. Every lane of the group
// ends with the group's total.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float group8_sum(float x) {
    x += dpp_f<0xB1>(x);    // quad_perm [1,0,3,2]
    x += dpp_f<0x4E>(x);    // quad_perm [2,3,0,1]
    x += dpp_f<0x141>(x);   // row_half_mirror: lane i <- lane 7 - i within each 8
    return x;
}
__device__ __forceinline__ float group16_sum(float x) {
    x = group8_sum(x);
    x += dpp_f<0x140>(x);   // row_mirror: lane i <- lane 15 - i within each 16
    return x;
}
__device__ __forceinline__ float row16_sum(float x) { return group16_sum(x); }
__device__ __forceinline__ float row16_max(float x) {
    x = fmaxf(x, dpp_f<0xB1>(x));
    x = fmaxf(x, dpp_f<0x4E>(x));
    x = fmaxf(x, dpp_f<0x141>(x));
    x = fmaxf(x, dpp_f<0x140>(x));
    return x;
}

// The general vector kernels spread one head vector over a wavefront: element c sits in
// lane c % 64, register c / 64.
constexpr int kMaxPerLane = 4;  // d <= 256 over 64 lanes

// Rotate a lane-distributed head vector by the RoPE angles of position pos (sgn = 1) or by
// their negatives (sgn = -1, the transpose R(pos)^T). Pair (2u, 2u+1) lives in adjacent
// lanes; the partner value comes from lane ^ 1. rope: [rows, d/2, 2] (cos, sin).
__device__ __forceinline__ void rotate_lanes(float (&x)[kMaxPerLane], int lane, int d,
                                             const float *rope, int64_t pos, float sgn = 1.0f) {
    const int half = d >> 1;
#pragma unroll
    for (int t = 0; t < kMaxPerLane; ++t) {
        const float partner = __shfl_xor(x[t], 1, 64);
        const int c = lane + 64 * t;
        if (c < d) {
            const float2 cs = reinterpret_cast<const float2 *>(rope)[pos * half + (c >> 1)];
            const float sn = sgn * cs.y;
            x[t] = (c & 1) ? fmaf(partner, sn, x[t] * cs.x) : fmaf(-partner, sn, x[t] * cs.x);
        }
    }
}

// Quiet NaN used to flag outputs of queries whose position could not be served.
__device__ __forceinline__ float qnan() { return __uint_as_float(0x7fc00000u); }

}  // namespace swa
