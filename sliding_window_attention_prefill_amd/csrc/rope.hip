// rope.hip - RoPE angle table and in-place rotation.
//
// Rotation R(p) of a head vector: the interleaved pairs (2t, 2t+1) turn by the angle
// p * theta^(-2t/d) (SWAT: Sliding Window Attention Training, symbol map and "RoPE"; the
// RoFormer rotation it cites). Angles are evaluated in float64 so that positions up to
// 2^24 keep full float32 accuracy in the table.
#include "swa_device.hpp"
#include "swa_kernels.hpp"

namespace swa {
namespace {

__global__ __launch_bounds__(256) void rope_table_kernel(float *__restrict__ table, int64_t n_pos,
                                                         int64_t d, double theta) {
    const int64_t half = d / 2;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= n_pos * half) return;
    const int64_t pos = idx / half, t = idx % half;
    const double freq = pow(theta, -2.0 * (double)t / (double)d);
    const double ang = (double)pos * freq;
    double sn, cs;
    sincos(ang, &sn, &cs);
    reinterpret_cast<float2 *>(table)[idx] = make_float2((float)cs, (float)sn);
}

template <int DT>
__global__ __launch_bounds__(256) void rope_apply_kernel(void *__restrict__ x, int64_t B, int64_t N,
                                                         int64_t H, int64_t d,
                                                         const int32_t *__restrict__ pos0,
                                                         const float *__restrict__ rope,
                                                         int64_t rope_rows) {
    const int64_t half = d / 2;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= B * N * H * half) return;
    const int64_t t = idx % half;
    const int64_t n = (idx / (half * H)) % N;
    const int64_t b = idx / (half * H * N);
    const int64_t pos = (int64_t)pos0[b] + n;
    const int64_t e = 2 * idx;  // element index of the pair's first value
    float a = Elem<DT>::load(x, e), c = Elem<DT>::load(x, e + 1);
    if (pos < 0 || pos >= rope_rows) {
        a = c = qnan();
    } else {
        const float2 cs = reinterpret_cast<const float2 *>(rope)[pos * half + t];
        const float ra = fmaf(-c, cs.y, a * cs.x);
        const float rc = fmaf(a, cs.y, c * cs.x);
        a = ra;
        c = rc;
    }
    Elem<DT>::store(x, e, a);
    Elem<DT>::store(x, e + 1, c);
}

// Vector form for d % 8 == 0 and a 16-byte aligned tensor: a thread rotates one 8-element
// chunk (four pairs) with 16-byte accesses.
template <int DT>
__global__ __launch_bounds__(256) void rope_apply8_kernel(void *__restrict__ x, int64_t B, int64_t N,
                                                          int64_t H, int64_t d,
                                                          const int32_t *__restrict__ pos0,
                                                          const float *__restrict__ rope,
                                                          int64_t rope_rows) {
    const int64_t c8 = d / 8;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= B * N * H * c8) return;
    const int64_t ch = idx % c8;
    const int64_t n = (idx / (c8 * H)) % N;
    const int64_t b = idx / (c8 * H * N);
    const int64_t pos = (int64_t)pos0[b] + n;
    float v[8];
    load8f<DT>(x, 8 * idx, v);
    if (pos < 0 || pos >= rope_rows) {
#pragma unroll
        for (int m = 0; m < 8; ++m) v[m] = qnan();
    } else {
        const float *t = rope + (pos * (d / 2) + 4 * ch) * 2;
        rotate8(v, as_float4(ldg16(t)), as_float4(ldg16(t + 4)));
    }
    store8f<DT>(x, 8 * idx, v);
}

}  // namespace

hipError_t launch_rope_table(float *table, int64_t n_pos, int64_t d, double theta,
                             hipStream_t st) {
    const int64_t n = n_pos * (d / 2);
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                       table, n_pos, d, theta);
    return hipGetLastError();
}

hipError_t launch_rope_apply(void *x, int64_t B, int64_t N, int64_t H, int64_t d,
                             const int32_t *pos0, const float *rope, int64_t rope_rows, int dt,
                             hipStream_t st) {
    const int64_t n = B * N * H * (d / 2);
    if (n == 0) return hipSuccess;
    if (d % 8 == 0 && (reinterpret_cast<uintptr_t>(x) & 15) == 0 &&
        (reinterpret_cast<uintptr_t>(rope) & 15) == 0) {
        const dim3 grid8((unsigned)((n / 4 + 255) / 256));
        if (dt == 0)
            hipLaunchKernelGGL(rope_apply8_kernel<0>, grid8, dim3(256), 0, st, x, B, N, H, d, pos0,
                               rope, rope_rows);
        else
            hipLaunchKernelGGL(rope_apply8_kernel<1>, grid8, dim3(256), 0, st, x, B, N, H, d, pos0,
                               rope, rope_rows);
        return hipGetLastError();
    }
    const dim3 grid((unsigned)((n + 255) / 256));
    if (dt == 0)
        hipLaunchKernelGGL(rope_apply_kernel<0>, grid, dim3(256), 0, st, x, B, N, H, d, pos0,
                           rope, rope_rows);
    else
        hipLaunchKernelGGL(rope_apply_kernel<1>, grid, dim3(256), 0, st, x, B, N, H, d, pos0,
                           rope, rope_rows);
    return hipGetLastError();
}

}  // namespace swa
