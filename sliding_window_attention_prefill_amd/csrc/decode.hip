// decode.hip - ring-buffer KV cache: append and single-token decode.
//
// The cache keeps w slots per (sequence, kv head); position p lives in slot p mod w and
// overwrites the oldest entry (Sliding Window Attention glossary, ring-buffer paragraph).
// Positions 0..s-1 are also kept in a sink store beside the ring (Sliding Window Attention
// glossary, "attention sink"; Sliding-window beats linear attention, SWA(64, 4)). Keys are
// stored rotated at their own absolute position, so a decode step only rotates its query.
#include "swa_device.hpp"
#include "swa_kernels.hpp"

namespace swa {
namespace {

// One block per (sequence, token, kv head); thread t handles the pair (2t, 2t+1).
template <int DT>
__global__ __launch_bounds__(128) void kv_append_kernel(CacheArgs c, const void *__restrict__ k_new,
                                                        const void *__restrict__ v_new,
                                                        const int32_t *__restrict__ pos0,
                                                        int64_t n_new, const float *__restrict__ rope,
                                                        int64_t rope_rows) {
    const int64_t row = blockIdx.x;
    const int64_t hk = row % c.Hkv;
    const int64_t n = (row / c.Hkv) % n_new;
    const int64_t sq = row / (c.Hkv * n_new);
    const int64_t p0 = pos0[sq];
    if (p0 < 0) return;
    const int64_t p = p0 + n;
    // A token of this call that a later token of the same call overwrites is skipped, so
    // every slot has exactly one writer.
    const bool to_ring = n >= n_new - c.w;
    const bool to_sink = p < c.s;
    if (!to_ring && !to_sink) return;
    const int64_t half = c.d / 2;
    for (int64_t t = threadIdx.x; t < half; t += blockDim.x) {
        const int64_t src = ((sq * n_new + n) * c.Hkv + hk) * c.d + 2 * t;
        float ka = Elem<DT>::load(k_new, src), kb = Elem<DT>::load(k_new, src + 1);
        const float va = Elem<DT>::load(v_new, src), vb = Elem<DT>::load(v_new, src + 1);
        if (rope) {
            if (p >= rope_rows) {
                ka = kb = qnan();
            } else {
                const float2 cs = reinterpret_cast<const float2 *>(rope)[p * half + t];
                const float ra = fmaf(-kb, cs.y, ka * cs.x);
                kb = fmaf(ka, cs.y, kb * cs.x);
                ka = ra;
            }
        }
        if (to_ring) {
            const int64_t dst = ((sq * c.Hkv + hk) * c.w + p % c.w) * c.d + 2 * t;
            Elem<DT>::store(c.k_ring, dst, ka);
            Elem<DT>::store(c.k_ring, dst + 1, kb);
            Elem<DT>::store(c.v_ring, dst, va);
            Elem<DT>::store(c.v_ring, dst + 1, vb);
        }
        if (to_sink) {
            const int64_t dst = ((sq * c.Hkv + hk) * c.s + p) * c.d + 2 * t;
            Elem<DT>::store(c.k_sink, dst, ka);
            Elem<DT>::store(c.k_sink, dst + 1, kb);
            Elem<DT>::store(c.v_sink, dst, va);
            Elem<DT>::store(c.v_sink, dst + 1, vb);
        }
    }
}

// General decode: one block of 256 threads per (sequence, kv head) serves the G query heads
// of the group. Keys are walked in chunks of KC staged in LDS as float32: sinks the window
// no longer covers first, then ring positions max(0, p-w+1)..p in order.
struct DecodeGen {
    int64_t S, Hq, Hkv, w, s, d;
    int mode;
    float scale;
    const float *slopes;
    const float *rope;
    int64_t rope_rows;
    const void *k_ring, *v_ring, *k_sink, *v_sink;
};

template <int DT, int OUT>
__global__ __launch_bounds__(256) void decode_general_kernel(DecodeGen a, const void *__restrict__ q,
                                                             const int32_t *__restrict__ q_pos,
                                                             void *__restrict__ o, int KC) {
    extern __shared__ float lds[];
    const int64_t G = a.Hq / a.Hkv;
    const int64_t sq = blockIdx.x / a.Hkv;
    const int64_t hk = blockIdx.x % a.Hkv;
    const int d = (int)a.d, half = d / 2;
    const int tid = threadIdx.x;
    const int KS = d + 1;  // padded LDS row (float32)
    float *qs = lds;                       // [G][d]
    float *ks = qs + G * d;                // [KC][d+1]
    float *vs = ks + KC * KS;              // [KC][d+1]
    float *sc = vs + KC * KS;              // [G][KC]
    float *os = sc + G * KC;               // [G][d]
    float *ml = os + G * d;                // [G] max, [G] sum, [G] correction
    int *kpos = reinterpret_cast<int *>(ml + 3 * G);  // [KC] position, [KC] source row

    const int64_t p = q_pos[sq];
    const bool valid = p >= 0 && (!a.rope || p < a.rope_rows);
    if (!valid) {
        for (int64_t idx = tid; idx < G * d; idx += blockDim.x) {
            const int64_t h = hk * G + idx / d;
            Elem<OUT>::store(o, (sq * a.Hq + h) * d + idx % d, qnan());
        }
        return;
    }
    for (int64_t idx = tid; idx < G * half; idx += blockDim.x) {
        const int64_t g = idx / half, t = idx % half;
        const int64_t src = (sq * a.Hq + hk * G + g) * d + 2 * t;
        float x0 = Elem<DT>::load(q, src), x1 = Elem<DT>::load(q, src + 1);
        if (a.rope) {
            const float2 cs = reinterpret_cast<const float2 *>(a.rope)[p * half + t];
            const float r0 = fmaf(-x1, cs.y, x0 * cs.x);
            x1 = fmaf(x0, cs.y, x1 * cs.x);
            x0 = r0;
        }
        qs[g * d + 2 * t] = x0;
        qs[g * d + 2 * t + 1] = x1;
    }
    for (int64_t idx = tid; idx < G * d; idx += blockDim.x) os[idx] = 0.0f;
    for (int64_t g = tid; g < G; g += blockDim.x) {
        ml[g] = -INFINITY;
        ml[G + g] = 0.0f;
    }
    const int64_t lo = p - a.w + 1 > 0 ? p - a.w + 1 : 0;
    const int64_t n_sink = a.s < lo ? a.s : lo;
    const int64_t n_keys = n_sink + (p - lo + 1);
    __syncthreads();

    for (int64_t c0 = 0; c0 < n_keys; c0 += KC) {
        const int nk = (int)(n_keys - c0 < KC ? n_keys - c0 : KC);
        for (int e = tid; e < nk; e += blockDim.x) {
            const int64_t ee = c0 + e;
            kpos[e] = (int)(ee < n_sink ? ee : lo + (ee - n_sink));
        }
        __syncthreads();
        for (int64_t idx = tid; idx < (int64_t)nk * d; idx += blockDim.x) {
            const int e = (int)(idx / d), c = (int)(idx % d);
            const int64_t ee = c0 + e;
            const int64_t P = kpos[e];
            int64_t src;
            const void *kb, *vb;
            if (ee < n_sink) {
                src = ((sq * a.Hkv + hk) * a.s + P) * d + c;
                kb = a.k_sink;
                vb = a.v_sink;
            } else {
                src = ((sq * a.Hkv + hk) * a.w + P % a.w) * d + c;
                kb = a.k_ring;
                vb = a.v_ring;
            }
            ks[e * KS + c] = Elem<DT>::load(kb, src);
            vs[e * KS + c] = Elem<DT>::load(vb, src);
        }
        __syncthreads();
        for (int64_t idx = tid; idx < G * nk; idx += blockDim.x) {
            const int64_t g = idx / nk;
            const int e = (int)(idx % nk);
            float acc = 0.0f;
            for (int c = 0; c < d; ++c) acc = fmaf(qs[g * d + c], ks[e * KS + c], acc);
            const float slope = a.slopes ? a.slopes[hk * G + g] : 0.0f;
            sc[g * KC + e] = fmaf(acc, a.scale, slope * (float)(p - kpos[e]));
        }
        __syncthreads();
        // weights: one wavefront per head
        for (int64_t g = tid >> 6; g < G; g += blockDim.x >> 6) {
            const int lane = tid & 63;
            if (a.mode == 0) {
                for (int e = lane; e < nk; e += 64) {
                    const float x = sc[g * KC + e];
                    sc[g * KC + e] = 1.0f / (1.0f + expf(-x));
                }
            } else {
                float mx = -INFINITY;
                for (int e = lane; e < nk; e += 64) mx = fmaxf(mx, sc[g * KC + e]);
                mx = wave_max(mx);
                const float m_old = ml[g];
                const float m_new = fmaxf(m_old, mx);
                float sum = 0.0f;
                for (int e = lane; e < nk; e += 64) {
                    const float pe = expf(sc[g * KC + e] - m_new);
                    sc[g * KC + e] = pe;
                    sum += pe;
                }
                sum = wave_sum(sum);
                if (lane == 0) {
                    const float corr = expf(m_old - m_new);
                    ml[G + g] = ml[G + g] * corr + sum;
                    ml[2 * G + g] = corr;
                    ml[g] = m_new;
                }
            }
        }
        __syncthreads();
        for (int64_t idx = tid; idx < G * d; idx += blockDim.x) {
            const int64_t g = idx / d;
            const int c = (int)(idx % d);
            float acc = a.mode == 1 ? os[idx] * ml[2 * G + g] : os[idx];
            for (int e = 0; e < nk; ++e) acc = fmaf(sc[g * KC + e], vs[e * KS + c], acc);
            os[idx] = acc;
        }
        __syncthreads();
    }
    for (int64_t idx = tid; idx < G * d; idx += blockDim.x) {
        const int64_t g = idx / d;
        const float inv = a.mode == 1 ? 1.0f / ml[G + g] : 1.0f;
        Elem<OUT>::store(o, (sq * a.Hq + hk * G + g) * d + idx % d, os[idx] * inv);
    }
}

size_t decode_general_lds(int64_t G, int64_t d, int KC) {
    return sizeof(float) * (size_t)(G * d + 2 * KC * (d + 1) + G * KC + G * d + 3 * G) +
           sizeof(int) * (size_t)KC;
}

}  // namespace

hipError_t launch_kv_append(const CacheArgs &c, const void *k_new, const void *v_new,
                            const int32_t *pos0, int64_t n_new, const float *rope,
                            int64_t rope_rows, hipStream_t st) {
    const int64_t rows = c.S * n_new * c.Hkv;
    if (rows == 0) return hipSuccess;
    if (c.dt == 0)
        hipLaunchKernelGGL(kv_append_kernel<0>, dim3((unsigned)rows), dim3(128), 0, st, c, k_new,
                           v_new, pos0, n_new, rope, rope_rows);
    else
        hipLaunchKernelGGL(kv_append_kernel<1>, dim3((unsigned)rows), dim3(128), 0, st, c, k_new,
                           v_new, pos0, n_new, rope, rope_rows);
    return hipGetLastError();
}

size_t decode_workspace_bytes(const DecodeArgs &, const CacheArgs &) { return 0; }

hipError_t launch_decode(const DecodeArgs &a, const CacheArgs &c, const void *q,
                         const int32_t *q_pos, void *o, void *, size_t, hipStream_t st) {
    if (c.S == 0) return hipSuccess;
    const int64_t G = a.Hq / c.Hkv;
    int KC = 64;
    while (KC > 8 && decode_general_lds(G, c.d, KC) > 64 * 1024) KC /= 2;
    const size_t lds = decode_general_lds(G, c.d, KC);
    if (lds > 64 * 1024) return hipErrorNotSupported;
    DecodeGen g{c.S, a.Hq, c.Hkv, c.w, c.s, c.d, a.mode, a.scale, a.slopes, a.rope, a.rope_rows,
                c.k_ring, c.v_ring, c.k_sink, c.v_sink};
    const dim3 grid((unsigned)(c.S * c.Hkv));
    if (c.dt == 0 && a.out_dt == 0)
        hipLaunchKernelGGL((decode_general_kernel<0, 0>), grid, dim3(256), lds, st, g, q, q_pos, o, KC);
    else if (c.dt == 0 && a.out_dt == 1)
        hipLaunchKernelGGL((decode_general_kernel<0, 1>), grid, dim3(256), lds, st, g, q, q_pos, o, KC);
    else if (c.dt == 1 && a.out_dt == 0)
        hipLaunchKernelGGL((decode_general_kernel<1, 0>), grid, dim3(256), lds, st, g, q, q_pos, o, KC);
    else
        hipLaunchKernelGGL((decode_general_kernel<1, 1>), grid, dim3(256), lds, st, g, q, q_pos, o, KC);
    return hipGetLastError();
}

}  // namespace swa
