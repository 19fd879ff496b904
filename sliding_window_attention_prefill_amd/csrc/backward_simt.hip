// backward_simt.hip - general vector backward of the sliding-window prefill.
//
// Covers every shape the general forward covers (float32 or bfloat16 inputs, any even
// d <= 256, any dilation): the gradients of SWAT: Sliding Window Attention Training,
// "Putting It Together" (the layer trains end to end), for the score of the "Balanced
// ALiBi" attention equation with the "Sigmoid" equation's logistic weights or softmax ones:
//   p_ij = sigma(x_ij)  or  exp(x_ij - lse_i),   dP_ij = dout_i . v_j
//   dX_ij = dP_ij p_ij (1 - p_ij)   or   p_ij (dP_ij - delta_i),  delta_i = sum_j p_ij dP_ij
//   dv_j = sum_i p_ij dout_i
//   dq_i = scale R(i)^T sum_j dX_ij R(j) k_j,   dk_j = scale R(j)^T sum_i dX_ij R(i) q_i
// delta_i (softmax) equals dout_i . o_i for the exact o; summing it over the key set instead
// keeps the rounding of a bfloat16 o out of the gradients.
// Two kernels, each gradient row owned by one wavefront (no atomics, deterministic):
// bwd_simt_dq_kernel walks the key set K(i) of one query row as the forward does (softmax:
// twice, first for delta_i, which it leaves in the workspace); bwd_simt_dkv_kernel walks,
// for one key row j, every query i with j in K(i) and every query head of the key's group,
// accumulating dk and dv.
#include "swa_device.hpp"
#include "swa_kernels.hpp"

namespace swa {
namespace {

struct SimtBwdParams {
    int64_t B, Hq, Hkv, N, d, w, s, dil;
    int mode;
    float scale;
    const float *slopes;
    const float *rope;
    const float *lse;  // softmax: [B, Hq, N]
    float *delta;      // softmax: [B, Hq, N], written by the dq kernel, read by the dk/dv one
};

template <int DT>
__device__ __forceinline__ void load_row(float (&x)[kMaxPerLane], const void *src, int64_t base,
                                         int lane, int d) {
#pragma unroll
    for (int t = 0; t < kMaxPerLane; ++t) {
        const int c = lane + 64 * t;
        x[t] = c < d ? Elem<DT>::load(src, base + c) : 0.0f;
    }
}

__device__ __forceinline__ float dot_lanes(const float (&a)[kMaxPerLane],
                                           const float (&b)[kMaxPerLane]) {
    float part = 0.0f;
#pragma unroll
    for (int t = 0; t < kMaxPerLane; ++t) part = fmaf(a[t], b[t], part);
    return wave_sum(part);
}

// Weight p and score gradient dX of one (query, key) pair from the score x, the value
// product dP, the row's lse and delta (softmax).
__device__ __forceinline__ void weight_and_grad(int mode, float x, float dP, float lse,
                                                float delta, float &p, float &dx) {
    if (mode == 0) {
        p = 1.0f / (1.0f + expf(-x));
        dx = dP * p * (1.0f - p);
    } else {
        p = expf(x - lse);
        dx = p * (dP - delta);
    }
}

// One wavefront per query row (b, i, h): dq_i.
template <int IN, int OUT>
__global__ __launch_bounds__(256) void bwd_simt_dq_kernel(SimtBwdParams p,
                                                          const void *__restrict__ q,
                                                          const void *__restrict__ k,
                                                          const void *__restrict__ v,
                                                          const void *__restrict__ dout,
                                                          void *__restrict__ dq) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= p.B * p.N * p.Hq) return;  // whole wavefront leaves together
    const int64_t h = row % p.Hq;
    const int64_t i = (row / p.Hq) % p.N;
    const int64_t b = row / (p.Hq * p.N);
    const int64_t hk = h / (p.Hq / p.Hkv);
    const int d = (int)p.d;
    const float slope = p.slopes ? p.slopes[h] : 0.0f;
    const int64_t qbase = ((b * p.N + i) * p.Hq + h) * d;

    float qv[kMaxPerLane], gv[kMaxPerLane], acc[kMaxPerLane];
    load_row<IN>(qv, q, qbase, lane, d);
    load_row<OUT>(gv, dout, qbase, lane, d);
    if (p.rope) rotate_lanes(qv, lane, d, p.rope, i);
    const int64_t srow = (b * p.Hq + h) * p.N + i;
    const float lse = p.mode == 1 ? p.lse[srow] : 0.0f;
    float delta = 0.0f;
#pragma unroll
    for (int t = 0; t < kMaxPerLane; ++t) acc[t] = 0.0f;

    // key set of row i: sinks below the window, then the window [lo, i] (every dil-th
    // position, sink positions inside it always)
    const int64_t span = p.w - 1 >= i ? i : p.dil * (p.w - 1);
    const int64_t lo = i - span > 0 ? i - span : 0;
    const int64_t n_sink = p.s < lo ? p.s : lo;
    const int64_t n_keys = n_sink + (i - lo + 1);
    // softmax: pass 0 sums delta_i, pass 1 accumulates dq; sigmoid: pass 1 only
    for (int pass = p.mode == 1 ? 0 : 1; pass < 2; ++pass) {
        for (int64_t e = 0; e < n_keys; ++e) {
            const int64_t j = e < n_sink ? e : lo + (e - n_sink);
            if (e >= n_sink && (i - j) % p.dil != 0 && j >= p.s) continue;   // wave-uniform
            const int64_t kbase = ((b * p.N + j) * p.Hkv + hk) * d;
            float kv[kMaxPerLane], vv[kMaxPerLane];
            load_row<IN>(kv, k, kbase, lane, d);
            load_row<IN>(vv, v, kbase, lane, d);
            if (p.rope) rotate_lanes(kv, lane, d, p.rope, j);
            const float x = fmaf(dot_lanes(qv, kv), p.scale, slope * (float)(i - j));
            const float dP = dot_lanes(gv, vv);
            float w, dx;
            weight_and_grad(p.mode, x, dP, lse, delta, w, dx);
            if (pass == 0) {
                delta = fmaf(w, dP, delta);
            } else {
#pragma unroll
                for (int t = 0; t < kMaxPerLane; ++t) acc[t] = fmaf(dx, kv[t], acc[t]);
            }
        }
    }
    if (p.mode == 1 && lane == 0) p.delta[srow] = delta;
#pragma unroll
    for (int t = 0; t < kMaxPerLane; ++t) acc[t] *= p.scale;
    if (p.rope) rotate_lanes(acc, lane, d, p.rope, i, -1.0f);
#pragma unroll
    for (int t = 0; t < kMaxPerLane; ++t) {
        const int c = lane + 64 * t;
        if (c < d) Elem<OUT>::store(dq, qbase + c, acc[t]);
    }
}

// One wavefront per key row (b, j, hk): dk_j and dv_j over every query head of the group.
template <int IN, int OUT>
__global__ __launch_bounds__(256) void bwd_simt_dkv_kernel(SimtBwdParams p,
                                                           const void *__restrict__ q,
                                                           const void *__restrict__ k,
                                                           const void *__restrict__ v,
                                                           const void *__restrict__ dout,
                                                           void *__restrict__ dk,
                                                           void *__restrict__ dv) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= p.B * p.N * p.Hkv) return;  // whole wavefront leaves together
    const int64_t hk = row % p.Hkv;
    const int64_t j = (row / p.Hkv) % p.N;
    const int64_t b = row / (p.Hkv * p.N);
    const int64_t G = p.Hq / p.Hkv;
    const int d = (int)p.d;
    const int64_t kbase = ((b * p.N + j) * p.Hkv + hk) * d;

    float kv[kMaxPerLane], vv[kMaxPerLane], dk_acc[kMaxPerLane], dv_acc[kMaxPerLane];
    load_row<IN>(kv, k, kbase, lane, d);
    load_row<IN>(vv, v, kbase, lane, d);
    if (p.rope) rotate_lanes(kv, lane, d, p.rope, j);
#pragma unroll
    for (int t = 0; t < kMaxPerLane; ++t) dk_acc[t] = dv_acc[t] = 0.0f;

    // queries that see key j: every i >= j for a sink, else i = j + dil t with t < w
    const int64_t t_last = (p.N - 1 - j) / p.dil;
    const bool sink = j < p.s;
    const int64_t n_q = sink ? p.N - j : 1 + (p.w - 1 < t_last ? p.w - 1 : t_last);
    for (int64_t e = 0; e < n_q; ++e) {
        const int64_t i = sink ? j + e : j + p.dil * e;
        for (int64_t g = 0; g < G; ++g) {
            const int64_t h = hk * G + g;
            const int64_t qbase = ((b * p.N + i) * p.Hq + h) * d;
            float qv[kMaxPerLane], gv[kMaxPerLane];
            load_row<IN>(qv, q, qbase, lane, d);
            load_row<OUT>(gv, dout, qbase, lane, d);
            if (p.rope) rotate_lanes(qv, lane, d, p.rope, i);
            float lse = 0.0f, delta = 0.0f;
            if (p.mode == 1) {
                lse = p.lse[(b * p.Hq + h) * p.N + i];
                delta = p.delta[(b * p.Hq + h) * p.N + i];
            }
            const float slope = p.slopes ? p.slopes[h] : 0.0f;
            const float x = fmaf(dot_lanes(qv, kv), p.scale, slope * (float)(i - j));
            const float dP = dot_lanes(gv, vv);
            float w, dx;
            weight_and_grad(p.mode, x, dP, lse, delta, w, dx);
#pragma unroll
            for (int t = 0; t < kMaxPerLane; ++t) {
                dv_acc[t] = fmaf(w, gv[t], dv_acc[t]);
                dk_acc[t] = fmaf(dx, qv[t], dk_acc[t]);
            }
        }
    }
#pragma unroll
    for (int t = 0; t < kMaxPerLane; ++t) dk_acc[t] *= p.scale;
    if (p.rope) rotate_lanes(dk_acc, lane, d, p.rope, j, -1.0f);
#pragma unroll
    for (int t = 0; t < kMaxPerLane; ++t) {
        const int c = lane + 64 * t;
        if (c < d) {
            Elem<OUT>::store(dk, kbase + c, dk_acc[t]);
            Elem<OUT>::store(dv, kbase + c, dv_acc[t]);
        }
    }
}

template <int IN, int OUT>
hipError_t launch_t(const PrefillArgs &a, const void *q, const void *k, const void *v,
                    const float *lse, const void *dout, void *dq, void *dk, void *dv, void *ws,
                    hipStream_t st) {
    SimtBwdParams p{a.B, a.Hq, a.Hkv, a.N, a.d, a.w, a.s, a.dil, a.mode, a.scale, a.slopes,
                    a.rope, lse, static_cast<float *>(ws)};
    const int64_t q_rows = a.B * a.N * a.Hq, k_rows = a.B * a.N * a.Hkv;
    hipLaunchKernelGGL((bwd_simt_dq_kernel<IN, OUT>), dim3((unsigned)((q_rows + 3) / 4)),
                       dim3(256), 0, st, p, q, k, v, dout, dq);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_simt_dkv_kernel<IN, OUT>), dim3((unsigned)((k_rows + 3) / 4)),
                       dim3(256), 0, st, p, q, k, v, dout, dk, dv);
    return hipGetLastError();
}

}  // namespace

size_t prefill_bwd_simt_workspace_bytes(const PrefillArgs &a) {
    return a.mode == 1 ? (size_t)(a.B * a.Hq * a.N) * sizeof(float) : 0;
}

hipError_t launch_prefill_bwd_simt(const PrefillArgs &a, const void *q, const void *k,
                                   const void *v, const float *lse, const void *dout, void *dq,
                                   void *dk, void *dv, void *ws, hipStream_t st) {
    if (a.B * a.N == 0) return hipSuccess;
    if (a.in_dt == 0 && a.out_dt == 0) return launch_t<0, 0>(a, q, k, v, lse, dout, dq, dk, dv, ws, st);
    if (a.in_dt == 0 && a.out_dt == 1) return launch_t<0, 1>(a, q, k, v, lse, dout, dq, dk, dv, ws, st);
    if (a.in_dt == 1 && a.out_dt == 0) return launch_t<1, 0>(a, q, k, v, lse, dout, dq, dk, dv, ws, st);
    return launch_t<1, 1>(a, q, k, v, lse, dout, dq, dk, dv, ws, st);
}

}  // namespace swa
