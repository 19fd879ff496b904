// prefill_simt.hip - general vector prefill kernel.
//
// Covers every shape the C ABI accepts (float32 or bfloat16 in/out, any even d <= 256):
// one wavefront evaluates one query row, walking the row's key set in order (sinks not in
// the window, then the window) with an online softmax or the plain sigmoid sum. It is the
// path for float32 inputs and for head dims the matrix-core kernel does not cover.
//
// Definition followed (SWAT: Sliding Window Attention Training, "Balanced ALiBi" attention
// equation and "Sigmoid" equation; Sliding Window Attention glossary, band mask; sinks per
// Sliding-window beats linear attention, SWA(w, s)):
//   x_ij = scale * (R(i) q_i).(R(j) k_j) + slope_h (i - j),  j in K(i)
//   sigmoid: o_i = sum sigma(x_ij) v_j ; softmax: o_i = sum softmax_j(x_ij) v_j
#include "swa_device.hpp"
#include "swa_kernels.hpp"

namespace swa {
namespace {

struct SimtParams {
    int64_t B, Hq, Hkv, N, d, w, s, dil;
    int mode;
    float scale;
    const float *slopes;
    const float *rope;
    float *lse;  // softmax row log-normalisers [B, Hq, N], or null
};

template <int IN, int OUT>
__global__ __launch_bounds__(256) void prefill_simt_kernel(SimtParams p, const void *__restrict__ q,
                                                           const void *__restrict__ k,
                                                           const void *__restrict__ v,
                                                           void *__restrict__ o) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= p.B * p.N * p.Hq) return;  // whole wavefront leaves together
    const int64_t h = row % p.Hq;
    const int64_t i = (row / p.Hq) % p.N;
    const int64_t b = row / (p.Hq * p.N);
    const int64_t hk = h / (p.Hq / p.Hkv);
    const int d = (int)p.d;
    const float slope = p.slopes ? p.slopes[h] : 0.0f;

    float qv[kMaxPerLane], acc[kMaxPerLane];
    const int64_t qbase = ((b * p.N + i) * p.Hq + h) * d;
#pragma unroll
    for (int t = 0; t < kMaxPerLane; ++t) {
        const int c = lane + 64 * t;
        qv[t] = c < d ? Elem<IN>::load(q, qbase + c) : 0.0f;
        acc[t] = 0.0f;
    }
    if (p.rope) rotate_lanes(qv, lane, d, p.rope, i);

    // the window spans positions [lo, i]; with a dilation only every dil-th of them is a key
    const int64_t span = p.w - 1 >= i ? i : p.dil * (p.w - 1);
    const int64_t lo = i - span > 0 ? i - span : 0;
    const int64_t n_sink = p.s < lo ? p.s : lo;
    const int64_t n_keys = n_sink + (i - lo + 1);
    float m = -INFINITY, l = 0.0f;

    for (int64_t e = 0; e < n_keys; ++e) {
        const int64_t j = e < n_sink ? e : lo + (e - n_sink);
        if (e >= n_sink && (i - j) % p.dil != 0 && j >= p.s) continue;   // wave-uniform
        const int64_t kbase = ((b * p.N + j) * p.Hkv + hk) * d;
        float kv[kMaxPerLane];
#pragma unroll
        for (int t = 0; t < kMaxPerLane; ++t) {
            const int c = lane + 64 * t;
            kv[t] = c < d ? Elem<IN>::load(k, kbase + c) : 0.0f;
        }
        if (p.rope) rotate_lanes(kv, lane, d, p.rope, j);
        float part = 0.0f;
#pragma unroll
        for (int t = 0; t < kMaxPerLane; ++t) part = fmaf(qv[t], kv[t], part);
        const float x = fmaf(wave_sum(part), p.scale, slope * (float)(i - j));

        float wgt, corr = 1.0f;
        if (p.mode == 0) {
            wgt = 1.0f / (1.0f + expf(-x));
        } else {
            const float m_new = fmaxf(m, x);
            corr = expf(m - m_new);
            wgt = expf(x - m_new);
            l = fmaf(l, corr, wgt);
            m = m_new;
        }
#pragma unroll
        for (int t = 0; t < kMaxPerLane; ++t) {
            const int c = lane + 64 * t;
            const float vv = c < d ? Elem<IN>::load(v, kbase + c) : 0.0f;
            acc[t] = fmaf(wgt, vv, acc[t] * corr);
        }
    }
    if (p.mode == 1 && p.lse && lane == 0) p.lse[(b * p.Hq + h) * p.N + i] = m + logf(l);
    const float inv = p.mode == 1 ? 1.0f / l : 1.0f;
#pragma unroll
    for (int t = 0; t < kMaxPerLane; ++t) {
        const int c = lane + 64 * t;
        if (c < d) Elem<OUT>::store(o, qbase + c, acc[t] * inv);
    }
}

template <int IN, int OUT>
hipError_t launch_t(const PrefillArgs &a, const void *q, const void *k, const void *v, void *o,
                    float *lse, hipStream_t st) {
    SimtParams p{a.B, a.Hq, a.Hkv, a.N, a.d, a.w, a.s, a.dil, a.mode, a.scale, a.slopes, a.rope,
                 lse};
    const int64_t rows = a.B * a.N * a.Hq;
    const int64_t blocks = (rows + 3) / 4;
    hipLaunchKernelGGL((prefill_simt_kernel<IN, OUT>), dim3((unsigned)blocks), dim3(256), 0, st,
                       p, q, k, v, o);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_simt(const PrefillArgs &a, const void *q, const void *k,
                               const void *v, void *o, hipStream_t st, float *lse) {
    if (a.B * a.N * a.Hq == 0) return hipSuccess;
    if (a.in_dt == 0 && a.out_dt == 0) return launch_t<0, 0>(a, q, k, v, o, lse, st);
    if (a.in_dt == 0 && a.out_dt == 1) return launch_t<0, 1>(a, q, k, v, o, lse, st);
    if (a.in_dt == 1 && a.out_dt == 0) return launch_t<1, 0>(a, q, k, v, o, lse, st);
    return launch_t<1, 1>(a, q, k, v, o, lse, st);
}

}  // namespace swa
