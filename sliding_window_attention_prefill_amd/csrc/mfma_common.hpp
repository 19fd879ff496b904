// mfma_common.hpp - pieces shared by the matrix-core attention kernels (gfx950): tile
// constants, buffer resources, float16 operand conversion and rotation, buffer-to-LDS
// transfers, the band's edge mask on a 32x32 score block and the ALiBi bias operands.
#pragma once

#include "swa_device.hpp"

namespace swa {
namespace {

constexpr int BK = 64;  // keys per tile
constexpr float LOG2E = 1.4426950408889634f;
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef short s16x4_t __attribute__((__vector_size__(4 * sizeof(short))));
typedef short s16x8_t __attribute__((__vector_size__(8 * sizeof(short))));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

constexpr int cmax(int a, int b) { return a > b ? a : b; }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             0x00020000);
}

__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const u32x4_t x = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
    return make_uint4(x[0], x[1], x[2], x[3]);
}

__device__ __forceinline__ float4 buf_load16f(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const u32x4_t x = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
    return make_float4(__uint_as_float(x[0]), __uint_as_float(x[1]), __uint_as_float(x[2]),
                       __uint_as_float(x[3]));
}


// Two floats -> two float16 operands that saturate at +-65504, the largest finite float16,
// where a plain conversion would overflow to infinity: an input operand past the float16
// range enters the products clamped, and the outputs stay finite.
constexpr float F16_MAX = 65504.0f;
__device__ __forceinline__ uint32_t pack_f16x2_sat(float a, float b) {
    return pack_f16x2(__builtin_amdgcn_fmed3f(a, -F16_MAX, F16_MAX),
                      __builtin_amdgcn_fmed3f(b, -F16_MAX, F16_MAX));
}

// A dword of two bf16 inputs -> two float16 matrix operands, rotated by (c, s) or not.
__device__ __forceinline__ uint32_t rotate_pair(uint32_t w, float c, float s) {
    const float a = __uint_as_float(w << 16);
    const float b = __uint_as_float(w & 0xffff0000u);
    return pack_f16x2_sat(fmaf(-b, s, a * c), fmaf(a, s, b * c));
}
__device__ __forceinline__ uint32_t to_f16_pair(uint32_t w) {
    return pack_f16x2_sat(__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u));
}
__device__ __forceinline__ uint4 rotate_chunk(uint4 x, float4 t0, float4 t1) {
    return make_uint4(rotate_pair(x.x, t0.x, t0.y), rotate_pair(x.y, t0.z, t0.w),
                      rotate_pair(x.z, t1.x, t1.y), rotate_pair(x.w, t1.z, t1.w));
}
__device__ __forceinline__ uint4 convert_chunk(uint4 x) {
    return make_uint4(to_f16_pair(x.x), to_f16_pair(x.y), to_f16_pair(x.z), to_f16_pair(x.w));
}
// The same with every value multiplied by f before the single rounding to float16.
__device__ __forceinline__ uint4 rotate_chunk_scaled(uint4 x, float4 t0, float4 t1, float f) {
    return make_uint4(rotate_pair(x.x, t0.x * f, t0.y * f), rotate_pair(x.y, t0.z * f, t0.w * f),
                      rotate_pair(x.z, t1.x * f, t1.y * f), rotate_pair(x.w, t1.z * f, t1.w * f));
}
__device__ __forceinline__ uint32_t to_f16_pair_scaled(uint32_t w, float f) {
    return pack_f16x2_sat(__uint_as_float(w << 16) * f, __uint_as_float(w & 0xffff0000u) * f);
}
__device__ __forceinline__ uint4 convert_chunk_scaled(uint4 x, float f) {
    return make_uint4(to_f16_pair_scaled(x.x, f), to_f16_pair_scaled(x.y, f),
                      to_f16_pair_scaled(x.z, f), to_f16_pair_scaled(x.w, f));
}

// Four output values at element offset off of a float32 or bf16 output. STREAM: streaming
// (non-temporal) stores, for outputs the kernel does not read again whose stores cover
// whole cache lines: they stay out of L2, which is left to the K/V tiles other workgroups
// still read. Scattered partial-line stores are better merged in L2 (plain stores).
template <bool STREAM>
__device__ __forceinline__ void store_out4(void *out, bool bf16, int64_t off, float a, float b,
                                           float c, float d) {
    if (bf16) {
        const uint64_t v = (uint64_t)pack_bf16x2(a, b) | ((uint64_t)pack_bf16x2(c, d) << 32);
        uint64_t *dst = reinterpret_cast<uint64_t *>(static_cast<uint16_t *>(out) + off);
        if (STREAM) __builtin_nontemporal_store(v, dst);
        else *dst = v;
    } else {
        float *dst = static_cast<float *>(out) + off;
        if (STREAM) {
            __builtin_nontemporal_store(a, dst);
            __builtin_nontemporal_store(b, dst + 1);
            __builtin_nontemporal_store(c, dst + 2);
            __builtin_nontemporal_store(d, dst + 3);
        } else {
            *reinterpret_cast<float4 *>(dst) = make_float4(a, b, c, d);
        }
    }
}

// Buffer -> LDS transfers: ROUNDS rounds of 1 KB per wavefront; lane l of round i lands at
// bytes 16 l of that round's kilobyte (wavefront wave fills kilobytes wave * ROUNDS + i).
// off[i] is this lane's source offset.
template <int ROUNDS>
__device__ __forceinline__ void dma_rounds(uint16_t *__restrict__ dst, __amdgpu_buffer_rsrc_t r,
                                           uint32_t base, const uint32_t *off, int wave) {
#pragma unroll
    for (int i = 0; i < ROUNDS; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            r, (lds_void_t *)(dst + (wave * ROUNDS + i) * 512), 16, base + off[i], 0, 0, 0);
}

// The same transfers when round i reads at off + i * stride: one offset register per lane.
// A stride of 1 KB (consecutive kilobytes of a tile image) rides in the instruction's
// immediate offset, which moves the LDS destination by the same amount, so every round
// names the wavefront's first kilobyte; other strides are added per round.
template <int ROUNDS>
__device__ __forceinline__ void dma_rounds_strided(uint16_t *__restrict__ dst,
                                                   __amdgpu_buffer_rsrc_t r, uint32_t off,
                                                   uint32_t stride, int wave) {
#pragma unroll
    for (int i = 0; i < ROUNDS; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            r, (lds_void_t *)(dst + (wave * ROUNDS + i) * 512), 16, off + i * stride, 0, 0, 0);
}
template <int ROUNDS>
__device__ __forceinline__ void dma_rounds_kb(uint16_t *__restrict__ dst, __amdgpu_buffer_rsrc_t r,
                                              uint32_t off, int wave) {
    static_assert(ROUNDS >= 1 && ROUNDS <= 4, "the immediate offset holds at most 4095 bytes");
    lds_void_t *const d = (lds_void_t *)(dst + wave * ROUNDS * 512);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, d, 16, off, 0, 0, 0);
    if constexpr (ROUNDS > 1) __builtin_amdgcn_raw_ptr_buffer_load_lds(r, d, 16, off, 0, 1024, 0);
    if constexpr (ROUNDS > 2) __builtin_amdgcn_raw_ptr_buffer_load_lds(r, d, 16, off, 0, 2048, 0);
    if constexpr (ROUNDS > 3) __builtin_amdgcn_raw_ptr_buffer_load_lds(r, d, 16, off, 0, 3072, 0);
}

// Key offset (from j0 + 4g) of accumulator element e of score block kb.
__device__ __forceinline__ constexpr int key_of(int kb, int e) {
    return kb * 32 + 8 * (e >> 2) + (e & 3);
}

// Exclude the keys of an edge tile that are outside the key set: their scores become fill
// (-inf for a logit, +inf for the sigmoid's negated logit: weight 0 either way). Element (kb, e) is key j = jb + key_of(kb, e) with
// i - j = dq - key_of(kb, e). w is the window's extent in positions; with a dilation r (a
// power of two, dmask = r - 1) only every r-th of them is a key. SINKS adds the keys j < s
// at or before the query.
template <bool SINKS>
__device__ __forceinline__ void mask_tile(f32x16_t (&sacc)[2], int dq, int jb, int w, int s,
                                          int dmask = 0, float fill = -INFINITY) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int dij = dq - key_of(kb, e);
            bool ok = ((unsigned)dij < (unsigned)w) & ((dij & dmask) == 0);   // 0 <= i - j < w
            if (SINKS) ok = ok | ((dij >= 0) & (jb + key_of(kb, e) < s));
            sacc[kb][e] = ok ? sacc[kb][e] : fill;
        }
}

// mask_tile for one 32-key block kb of the tile.
template <bool SINKS>
__device__ __forceinline__ void mask_block(f32x16_t &x, int kb, int dq, int jb, int w, int s,
                                           float fill) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const int dij = dq - key_of(kb, e);
        bool ok = (unsigned)dij < (unsigned)w;   // 0 <= i - j < w
        if (SINKS) ok = ok | ((dij >= 0) & (jb + key_of(kb, e) < s));
        x[e] = ok ? x[e] : fill;
    }
}

// x = keep ? x : fill, written in x's own register (an instruction with the result tied to
// its input), so that a conditionally masked accumulator needs no copy where the masked and
// the unmasked paths meet.
__device__ __forceinline__ float keep_or_fill(float x, bool keep, float fill) {
    const uint64_t m = __builtin_amdgcn_ballot_w64(keep);
    asm("v_cndmask_b32_e64 %0, %1, %0, %2" : "+v"(x) : "v"(fill), "s"(m));
    return x;
}

// mask_tile in place; with all_out every key is excluded (a tile that meets none of this
// wavefront's key sets).
template <bool SINKS>
__device__ __forceinline__ void mask_tile_inplace(f32x16_t (&sacc)[2], int dq, int jb, int w,
                                                  int s, int dmask, float fill, bool all_out) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int dij = dq - key_of(kb, e);
            bool ok = ((unsigned)dij < (unsigned)w) & ((dij & dmask) == 0);
            if (SINKS) ok = ok | ((dij >= 0) & (jb + key_of(kb, e) < s));
            sacc[kb][e] = keep_or_fill(sacc[kb][e], ok & !all_out, fill);
        }
}

// The two one-sided cuts of an edge tile, one compare each: keys after the query (causal
// edge, i - j < 0) and keys that left the window (i - j >= w; dqw = dq - w).
__device__ __forceinline__ void mask_causal(f32x16_t (&sacc)[2], int dq, float fill) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) sacc[kb][e] = key_of(kb, e) <= dq ? sacc[kb][e] : fill;
}
__device__ __forceinline__ void mask_far(f32x16_t (&sacc)[2], int dqw, float fill) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) sacc[kb][e] = key_of(kb, e) > dqw ? sacc[kb][e] : fill;
}

// Operands of one extra matrix instruction per 32-key block that puts the key part of the
// ALiBi bias into the score accumulator: with r = slope log2(e) / cs split as
// 2^a (hi + lo) in float16, A row m holds (2^a kappa, 2^a kappa) and every B column
// (-hi, -lo) in k = 0, 1, so the product is -r kappa for the key kappa = 32 kb + m of the
// tile (kappa 2^a is exact in float16, and hi + lo carries r to about 22 bits).
//
// With qterm the same instruction also carries a per-query term r u (u = i - j0, refreshed
// per tile by query_term): k = 2, 3 hold 2^c in A and the two-term float16 split of
// r u 2^-c in B (query_term's dword), c = min(a + 12, 15). Then |r u 2^-c| < 2^13 for
// u < 2^24 (no float16 overflow) and >= 2^-12 for u >= 1 (normal float16); a term past
// the float16 range (only for |r| >= 16) is clamped, where the sigmoid has saturated.
struct BiasOperands {
    f16x8_t a[2];
    f16x8_t b;
    float qmul;  // r 2^-c (qterm only)
};

__device__ __forceinline__ BiasOperands bias_operands(float r, int lane, bool qterm = false) {
    int ex = 0;
    (void)frexpf(r, &ex);                      // |r| = m 2^ex, m in [0.5, 1)
    int a = ex - 1;
    a = a < -24 ? -24 : (a > 9 ? 9 : a);       // kappa 2^a stays exact for kappa < 64
    const float rs = ldexpf(r, -a);
    const _Float16 hi = (_Float16)rs;
    const _Float16 lo = (_Float16)(rs - (float)hi);
    const int c = a + 12 < 15 ? a + 12 : 15;
    BiasOperands bo;
    const f16x8_t z = {};
    bo.a[0] = z; bo.a[1] = z; bo.b = z;
    bo.qmul = qterm ? ldexpf(r, -c) : 0.0f;
    if (lane < 32) {
        const _Float16 k0 = (_Float16)ldexpf((float)lane, a);
        const _Float16 k1 = (_Float16)ldexpf((float)(lane + 32), a);
        bo.a[0][0] = k0; bo.a[0][1] = k0;
        bo.a[1][0] = k1; bo.a[1][1] = k1;
        bo.b[0] = -hi; bo.b[1] = -lo;
        if (qterm) {
            const _Float16 pc = (_Float16)ldexpf(1.0f, c);
            bo.a[0][2] = pc; bo.a[0][3] = pc;
            bo.a[1][2] = pc; bo.a[1][3] = pc;
        }
    }
    return bo;
}

// The bias B operand for a tile whose query offset is u = i - j0: the two-term float16
// split of qmul u in k = 2, 3 (lanes of k >= 8 carry it too; their A entries are zero).
__device__ __forceinline__ f16x8_t query_term(const BiasOperands &bo, int u) {
    float v = bo.qmul * (float)u;
    v = fminf(fmaxf(v, -65000.0f), 65000.0f);
    const float vh = (float)(_Float16)v;
    f16x8_t b = bo.b;
    b[2] = (_Float16)vh;
    b[3] = (_Float16)(v - vh);
    return b;
}

// S^T = K Q^T for the 64 keys of one LDS tile (two 32-key blocks, whose chains alternate);
// koff[ks] is this lane's element offset of its row's chunk for k-step ks. With ALiBi each
// block starts from the bias instruction (A from bo, B = bb).
template <int D, bool ALIBI>
__device__ __forceinline__ void qk_tile_off(const uint16_t *__restrict__ kl, const int (&koff)[D / 16],
                                            const BiasOperands &bo, const f16x8_t &bb,
                                            const f16x8_t (&qreg)[D / 16], const f32x16_t &init,
                                            f32x16_t (&sacc)[2]) {
    constexpr int KS = D / 16;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
        sacc[kb] = ALIBI ? __builtin_amdgcn_mfma_f32_32x32x16_f16(bo.a[kb], bb, init, 0, 0, 0) : init;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const f16x8_t a = *reinterpret_cast<const f16x8_t *>(kl + kb * 32 * D + koff[ks]);
            sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, qreg[ks], sacc[kb], 0, 0, 0);
        }
}

template <int D, bool ALIBI>
__device__ __forceinline__ void qk_tile_off(const uint16_t *__restrict__ kl, const int (&koff)[D / 16],
                                            const BiasOperands &bo, const f16x8_t &bb,
                                            const f16x8_t (&qreg)[D / 16], f32x16_t (&sacc)[2]) {
    const f32x16_t zero = {};
    qk_tile_off<D, ALIBI>(kl, koff, bo, bb, qreg, zero, sacc);
}

template <int D, bool ALIBI>
__device__ __forceinline__ void qk_tile_off(const uint16_t *__restrict__ kl, const int (&koff)[D / 16],
                                            const BiasOperands &bo, const f16x8_t (&qreg)[D / 16],
                                            f32x16_t (&sacc)[2]) {
    qk_tile_off<D, ALIBI>(kl, koff, bo, bo.b, qreg, sacc);
}

}  // namespace
}  // namespace swa
