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

// Vector form for d % 8 == 0 and 16-byte aligned tensors: a thread moves one 8-element chunk
// of one (sequence, token, kv head) row with 16-byte accesses; same writers as above.
template <int DT>
__global__ __launch_bounds__(256) void kv_append8_kernel(CacheArgs c, const void *__restrict__ k_new,
                                                         const void *__restrict__ v_new,
                                                         const int32_t *__restrict__ pos0,
                                                         int64_t n_new, const float *__restrict__ rope,
                                                         int64_t rope_rows) {
    const int64_t c8 = c.d / 8;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= c.S * n_new * c.Hkv * c8) return;
    const int64_t ch = idx % c8;
    const int64_t row = idx / c8;   // (sq, n, hk)
    const int64_t hk = row % c.Hkv;
    const int64_t n = (row / c.Hkv) % n_new;
    const int64_t sq = row / (c.Hkv * n_new);
    const int64_t p0 = pos0[sq];
    if (p0 < 0) return;
    const int64_t p = p0 + n;
    const bool to_ring = n >= n_new - c.w;
    const bool to_sink = p < c.s;
    if (!to_ring && !to_sink) return;
    float kx[8], vx[8];
    load8f<DT>(k_new, 8 * idx, kx);
    load8f<DT>(v_new, 8 * idx, vx);
    if (rope) {
        if (p >= rope_rows) {
#pragma unroll
            for (int m = 0; m < 8; ++m) kx[m] = qnan();
        } else {
            const float *t = rope + (p * (c.d / 2) + 4 * ch) * 2;
            rotate8(kx, as_float4(ldg16(t)), as_float4(ldg16(t + 4)));
        }
    }
    if (to_ring) {
        const int64_t dst = ((sq * c.Hkv + hk) * c.w + p % c.w) * c.d + 8 * ch;
        store8f<DT>(c.k_ring, dst, kx);
        store8f<DT>(c.v_ring, dst, vx);
    }
    if (to_sink) {
        const int64_t dst = ((sq * c.Hkv + hk) * c.s + p) * c.d + 8 * ch;
        store8f<DT>(c.k_sink, dst, kx);
        store8f<DT>(c.v_sink, dst, vx);
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

// Fast decode for a bf16 cache, d in {64, 128}, up to 8 query heads per kv head. One block
// of 256 threads per (sequence, kv head) issues every K and V load of a 128-key chunk before
// any arithmetic, so the whole working set of the step is in flight at once:
//   score pass: 4 threads per key, each a quarter of the row, reduced with two shuffles;
//   weights:    one wavefront per head, keys across lanes (wavefront max / sum reductions);
//   value pass: thread (key group, 8-column chunk) accumulates 8 columns for every head,
//               then the key groups are summed through LDS.
// With APPEND the block first writes the new token (rotated key, value) to its ring slot
// and sink entry, keeps it in LDS and uses that copy for position q_pos, so the slot it
// wrote is never read back within the launch.
// Split-KV: with nsplit > 1 the key list of a query is cut into nsplit contiguous, chunk-
// aligned ranges, one block each; a block writes its unnormalised partial output with its
// running maximum and sum to the workspace, and decode_combine_kernel merges the partials
// (log-sum-exp rescaling for softmax, a plain sum for sigmoid). Only the block whose range
// holds the query's own position appends the new token.
struct DecodeFast {
    int S, Hq, Hkv, G, w, s, mode;
    int nsplit;          // key ranges per (sequence, kv head); 1 = no split
    float *part;         // workspace: [S, Hkv, nsplit, G] x (D outputs, max, sum), or null
    float cs;            // scale * log2(e): scores are kept in base-2 units
    const float *slopes;
    const float *rope;
    int64_t rope_rows;
    uint16_t *k_ring, *v_ring, *k_sink, *v_sink;
};

constexpr int DEC_KC = 128;  // keys per chunk

template <int D>
struct DecLds {
    static constexpr int C8 = D / 8;          // 16-byte chunks per row
    static constexpr int KG = 256 / C8;       // key groups of the value pass
    static constexpr int VK = DEC_KC / KG;    // keys per thread in the value pass
    static constexpr int QE = D / 4;          // elements per thread in the score pass
    // a head's query is kept as four quarters of QE values, each padded by 4 floats, so the
    // four quarters that one wavefront reads at once sit in different banks
    static constexpr int QQ = QE + 4;         // floats per stored quarter
    static constexpr int QG = 4 * QQ;         // floats per stored head
};

template <int D>
size_t decode_fast_lds(int G) {
    using L = DecLds<D>;
    return sizeof(float) * ((size_t)G * L::QG + (size_t)G * DEC_KC + 2 * D + 3 * 8 +
                            (size_t)L::KG * G * D);
}

__device__ __forceinline__ uint4 ld16(const uint16_t *p) { return *reinterpret_cast<const uint4 *>(p); }

// Block barrier that orders LDS accesses only: global loads in flight stay in flight.
__device__ __forceinline__ void lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <int D, int G, int OUT, bool APPEND>
__global__ __launch_bounds__(256) void decode_fast_kernel(DecodeFast a, const uint16_t *__restrict__ q,
                                                          const int32_t *__restrict__ q_pos,
                                                          void *__restrict__ o,
                                                          const uint16_t *__restrict__ k_new,
                                                          const uint16_t *__restrict__ v_new) {
    using L = DecLds<D>;
    extern __shared__ float lds[];
    float *qs = lds;                    // [G][4][QQ] rotated queries * scale * log2(e)
    float *sc = qs + G * L::QG;         // [G][KC] scores, then weights
    float *kn = sc + G * DEC_KC;        // [D] appended key (as stored)
    float *vn = kn + D;                 // [D] appended value
    float *ml = vn + D;                 // [3][8] max, sum, correction per head
    float *red = ml + 24;               // [KG][G][D] partial outputs

    const int split = blockIdx.x % a.nsplit, bsh = blockIdx.x / a.nsplit;
    const int sq = bsh / a.Hkv, hk = bsh % a.Hkv;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int p = q_pos[sq];
    const bool valid = p >= 0 && (!a.rope || (int64_t)p < a.rope_rows);
    if (!valid) {
        // the combine kernel flags split outputs itself
        if (a.nsplit == 1)
            for (int idx = tid; idx < G * D; idx += 256)
                Elem<OUT>::store(o, ((int64_t)sq * a.Hq + hk * G) * D + idx, qnan());
        return;
    }
    // this block's range of the query's key list (sinks first, then the window)
    const int lo_w = p - a.w + 1 > 0 ? p - a.w + 1 : 0;
    const int n_all = (a.s < lo_w ? a.s : lo_w) + (p - lo_w + 1);
    const int per = ((n_all + a.nsplit - 1) / a.nsplit + DEC_KC - 1) / DEC_KC * DEC_KC;
    const int k_begin = split * per < n_all ? split * per : n_all;
    const int k_end = k_begin + per < n_all ? k_begin + per : n_all;
    const bool owns_new = k_begin <= n_all - 1 && n_all - 1 < k_end;   // the query's own key
    const int64_t ring_base = ((int64_t)sq * a.Hkv + hk) * a.w * D;
    const int64_t sink_base = ((int64_t)sq * a.Hkv + hk) * a.s * D;
    const int half = D / 2;

    // ---- the new token (fused append) and the queries, rotated at position p
    if (APPEND && owns_new && tid < half) {
        const int64_t src = ((int64_t)sq * a.Hkv + hk) * D + 2 * tid;
        float k0 = bf16_bits_to_f32(k_new[src]), k1 = bf16_bits_to_f32(k_new[src + 1]);
        const uint32_t vv = *reinterpret_cast<const uint32_t *>(v_new + src);
        if (a.rope) {
            const float2 cs = reinterpret_cast<const float2 *>(a.rope)[(int64_t)p * half + tid];
            const float r0 = fmaf(-k1, cs.y, k0 * cs.x);
            k1 = fmaf(k0, cs.y, k1 * cs.x);
            k0 = r0;
        }
        const uint32_t kk = pack_bf16x2(k0, k1);
        *reinterpret_cast<uint32_t *>(a.k_ring + ring_base + (int64_t)(p % a.w) * D + 2 * tid) = kk;
        *reinterpret_cast<uint32_t *>(a.v_ring + ring_base + (int64_t)(p % a.w) * D + 2 * tid) = vv;
        if (p < a.s) {
            *reinterpret_cast<uint32_t *>(a.k_sink + sink_base + (int64_t)p * D + 2 * tid) = kk;
            *reinterpret_cast<uint32_t *>(a.v_sink + sink_base + (int64_t)p * D + 2 * tid) = vv;
        }
        kn[2 * tid] = bf16_bits_to_f32(kk & 0xffffu);
        kn[2 * tid + 1] = bf16_bits_to_f32(kk >> 16);
        vn[2 * tid] = bf16_bits_to_f32(vv & 0xffffu);
        vn[2 * tid + 1] = bf16_bits_to_f32(vv >> 16);
    }
    for (int idx = tid; idx < G * half; idx += 256) {
        const int g = idx / half, t = idx % half;
        const int64_t src = ((int64_t)sq * a.Hq + hk * G + g) * D + 2 * t;
        float x0 = bf16_bits_to_f32(q[src]), x1 = bf16_bits_to_f32(q[src + 1]);
        if (a.rope) {
            const float2 cs = reinterpret_cast<const float2 *>(a.rope)[(int64_t)p * half + t];
            const float r0 = fmaf(-x1, cs.y, x0 * cs.x);
            x1 = fmaf(x0, cs.y, x1 * cs.x);
            x0 = r0;
        }
        const int col = 2 * t;   // a quarter holds QE consecutive columns
        qs[g * L::QG + (col / L::QE) * L::QQ + col % L::QE] = x0 * a.cs;
        qs[g * L::QG + (col / L::QE) * L::QQ + col % L::QE + 1] = x1 * a.cs;
    }
    if (tid < 8) {
        ml[tid] = -INFINITY;
        ml[8 + tid] = 0.0f;
        ml[16 + tid] = 1.0f;
    }
    const int lo = lo_w;
    const int n_sink = a.s < lo ? a.s : lo;
    const int n_keys = k_end;
    // ring slot of window position lo + m (0 <= m < w): lo mod w + m, less w past the end
    // (rows past the key list, which are never read, get slot 0)
    const int slot_lo = lo % a.w;
    auto ring_slot = [&](int P) {
        const int sl = slot_lo + (P - lo);
        return sl < a.w ? sl : (sl - a.w < a.w ? sl - a.w : 0);
    };

    // value-pass ownership: 8 columns, keys kg, kg + KG, ...
    const int c8 = tid % L::C8, kg = tid / L::C8;
    float acc[G][8];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[g][c] = 0.0f;
    __syncthreads();

    // K rows of the next chunk are requested as soon as this chunk's scores are formed, V rows
    // as soon as its values are added; the block barriers inside a chunk order LDS only, so
    // those loads stay in flight across them.
    uint4 kx[2][L::QE / 8];
    int kpos[2];
    uint4 vx[L::VK];
    int vpos[L::VK];
    auto load_k = [&](int cc) {
        const int nk = n_keys - cc < DEC_KC ? n_keys - cc : DEC_KC;
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int slot = tid + 256 * r, e = slot / 4, qq = slot % 4;
            const int ee = cc + e;
            const int P = ee < n_sink ? ee : lo + (ee - n_sink);
            kpos[r] = P;
            const bool from_mem = e < nk && !(APPEND && P == p);
            const uint16_t *row = ee < n_sink ? a.k_sink + sink_base + (int64_t)P * D
                                              : a.k_ring + ring_base + (int64_t)ring_slot(P) * D;
#pragma unroll
            for (int u = 0; u < L::QE / 8; ++u)
                kx[r][u] = from_mem ? ld16(row + qq * L::QE + 8 * u) : make_uint4(0, 0, 0, 0);
        }
    };
    auto load_v = [&](int cc) {
        const int nk = n_keys - cc < DEC_KC ? n_keys - cc : DEC_KC;
#pragma unroll
        for (int r = 0; r < L::VK; ++r) {
            const int e = kg + L::KG * r, ee = cc + e;
            const int P = ee < n_sink ? ee : lo + (ee - n_sink);
            vpos[r] = P;
            const bool from_mem = e < nk && !(APPEND && P == p);
            const uint16_t *row = ee < n_sink ? a.v_sink + sink_base + (int64_t)P * D
                                              : a.v_ring + ring_base + (int64_t)ring_slot(P) * D;
            vx[r] = from_mem ? ld16(row + 8 * c8) : make_uint4(0, 0, 0, 0);
        }
    };
    if (k_begin < n_keys) {
        load_k(k_begin);
        load_v(k_begin);
    }
    for (int c0 = k_begin; c0 < n_keys; c0 += DEC_KC) {
        const int nk = n_keys - c0 < DEC_KC ? n_keys - c0 : DEC_KC;
        const bool more = c0 + DEC_KC < n_keys;
        // -- scores (base 2): q.k * scale log2e + slope log2e (p - P)
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int slot = tid + 256 * r, e = slot / 4, qq = slot % 4;
            const int P = kpos[r];
            float kf[L::QE];
#pragma unroll
            for (int u = 0; u < L::QE / 8; ++u) {
                const uint32_t w4[4] = {kx[r][u].x, kx[r][u].y, kx[r][u].z, kx[r][u].w};
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    kf[8 * u + 2 * m] = __uint_as_float(w4[m] << 16);
                    kf[8 * u + 2 * m + 1] = __uint_as_float(w4[m] & 0xffff0000u);
                }
            }
            if (APPEND && P == p && e < nk) {
#pragma unroll
                for (int c = 0; c < L::QE; ++c) kf[c] = kn[qq * L::QE + c];
            }
            float part[G];
#pragma unroll
            for (int g = 0; g < G; ++g) {
                float acc_d = 0.0f;
#pragma unroll
                for (int c = 0; c < L::QE; ++c) acc_d = fmaf(qs[g * L::QG + qq * L::QQ + c], kf[c], acc_d);
                part[g] = acc_d;
            }
#pragma unroll
            for (int g = 0; g < G; ++g) {
                part[g] += __shfl_xor(part[g], 1, 64);
                part[g] += __shfl_xor(part[g], 2, 64);
            }
            if (qq == 0 && e < nk) {
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    const float slope = a.slopes ? a.slopes[hk * G + g] * 1.4426950408889634f : 0.0f;
                    sc[g * DEC_KC + e] = fmaf(slope, (float)(p - P), part[g]);
                }
            }
        }
        if (more) load_k(c0 + DEC_KC);
        lds_sync();
        // -- weights: one wavefront per head, keys across lanes
        for (int g = wave; g < G; g += 4) {
            float x0 = lane < nk ? sc[g * DEC_KC + lane] : -INFINITY;
            float x1 = lane + 64 < nk ? sc[g * DEC_KC + lane + 64] : -INFINITY;
            if (a.mode == 0) {
                x0 = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-x0));
                x1 = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-x1));
            } else {
                const float m_old = ml[g];
                const float m_new = fmaxf(m_old, wave_max(fmaxf(x0, x1)));
                x0 = __builtin_amdgcn_exp2f(x0 - m_new);
                x1 = __builtin_amdgcn_exp2f(x1 - m_new);
                const float sum = wave_sum(x0 + x1);
                if (lane == 0) {
                    const float corr = __builtin_amdgcn_exp2f(m_old - m_new);
                    ml[8 + g] = ml[8 + g] * corr + sum;
                    ml[16 + g] = corr;
                    ml[g] = m_new;
                }
            }
            if (lane < nk) sc[g * DEC_KC + lane] = x0;
            if (lane + 64 < nk) sc[g * DEC_KC + lane + 64] = x1;
        }
        lds_sync();
        // -- values: acc[g][c] = acc * corr + sum_e w[g][e] v[e][8 c8 + c]
        if (a.mode == 1) {
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const float corr = ml[16 + g];
#pragma unroll
                for (int c = 0; c < 8; ++c) acc[g][c] *= corr;
            }
        }
#pragma unroll
        for (int r = 0; r < L::VK; ++r) {
            const int e = kg + L::KG * r;
            if (e < nk) {
                float vf[8];
                const uint32_t w4[4] = {vx[r].x, vx[r].y, vx[r].z, vx[r].w};
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    vf[2 * m] = __uint_as_float(w4[m] << 16);
                    vf[2 * m + 1] = __uint_as_float(w4[m] & 0xffff0000u);
                }
                if (APPEND && vpos[r] == p) {
#pragma unroll
                    for (int c = 0; c < 8; ++c) vf[c] = vn[8 * c8 + c];
                }
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    const float wgt = sc[g * DEC_KC + e];
#pragma unroll
                    for (int c = 0; c < 8; ++c) acc[g][c] = fmaf(wgt, vf[c], acc[g][c]);
                }
            }
        }
        if (more) load_v(c0 + DEC_KC);
        lds_sync();
    }
    // ---- sum the key groups and normalise
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int c = 0; c < 8; ++c) red[(kg * G + g) * D + 8 * c8 + c] = acc[g][c];
    __syncthreads();
    float *pp = a.nsplit > 1 ? a.part + (((int64_t)bsh * a.nsplit + split) * G) * (D + 2) : nullptr;
    for (int idx = tid; idx < G * D; idx += 256) {
        const int g = idx / D, col = idx % D;
        float sum = 0.0f;
        for (int r = 0; r < L::KG; ++r) sum += red[(r * G + g) * D + col];
        if (a.nsplit > 1) {
            pp[g * (D + 2) + col] = sum;
        } else {
            if (a.mode == 1) sum /= ml[8 + g];
            Elem<OUT>::store(o, ((int64_t)sq * a.Hq + hk * G + g) * D + col, sum);
        }
    }
    if (a.nsplit > 1 && tid < G) {
        pp[tid * (D + 2) + D] = ml[tid];          // running maximum (base 2), -inf if empty
        pp[tid * (D + 2) + D + 1] = ml[8 + tid];  // running sum
    }
}

// Merge of the split partials of decode_fast_kernel: one block per (sequence, kv head).
// softmax: o = sum_k acc_k 2^(m_k - M) / sum_k l_k 2^(m_k - M) with M the largest m_k;
// sigmoid: o = sum_k acc_k. A query whose position cannot be served gets NaN.
template <int D, int G, int OUT>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeFast a,
                                                             const int32_t *__restrict__ q_pos,
                                                             void *__restrict__ o) {
    const int bsh = blockIdx.x, sq = bsh / a.Hkv, hk = bsh % a.Hkv;
    const int p = q_pos[sq];
    const bool valid = p >= 0 && (!a.rope || (int64_t)p < a.rope_rows);
    const float *pp = a.part + (int64_t)bsh * a.nsplit * G * (D + 2);
    for (int idx = threadIdx.x; idx < G * D; idx += 256) {
        const int g = idx / D, col = idx % D;
        float out;
        if (!valid) {
            out = qnan();
        } else if (a.mode == 0) {
            out = 0.0f;
            for (int k = 0; k < a.nsplit; ++k) out += pp[(k * G + g) * (D + 2) + col];
        } else {
            float M = -INFINITY;
            for (int k = 0; k < a.nsplit; ++k) M = fmaxf(M, pp[(k * G + g) * (D + 2) + D]);
            float num = 0.0f, den = 0.0f;
            for (int k = 0; k < a.nsplit; ++k) {
                const float *e = pp + (k * G + g) * (D + 2);
                const float f = __builtin_amdgcn_exp2f(e[D] - M);  // empty range: 2^-inf = 0
                num = fmaf(e[col], f, num);
                den = fmaf(e[D + 1], f, den);
            }
            out = num / den;
        }
        Elem<OUT>::store(o, ((int64_t)sq * a.Hq + hk * G + g) * D + col, out);
    }
}

// Whole-window decode for a bf16 cache when the ring and the sink store together hold at
// most 128 rows (w + s <= 128, e.g. SWA(64, 4)). The rows a query can read are then known
// without its position: every ring slot and every sink entry. So the block issues all of
// its loads - queries, every K and V row, the new token - before the position arrives, and
// only then decides which rows count (ring slot t holds position p - ((p - t) mod w) when
// that is >= 0; sink j counts when the window no longer covers it) and what bias each gets.
// Thread (row group, 16-byte column chunk) owns the same chunk of up to NS rows; scores are
// reduced over the chunks of a row with lane shuffles, weights per head by one wavefront,
// and value partials over rows with lane shuffles and one LDS pass.
template <int D, int NT>
struct WinCfg {
    static constexpr int C8 = D / 8;           // 16-byte chunks per row: 8 or 16
    static constexpr int RPP = NT / C8;        // rows per pass of the block
    static constexpr int NS = 128 / RPP;       // passes for 128 rows
    static constexpr int NW = NT / 64;         // wavefronts
};

template <int D, int G, int OUT, bool APPEND, int NT>
__global__ __launch_bounds__(NT) void decode_window_kernel(DecodeFast a, const uint16_t *__restrict__ q,
                                                            const int32_t *__restrict__ q_pos,
                                                            void *__restrict__ o,
                                                            const uint16_t *__restrict__ k_new,
                                                            const uint16_t *__restrict__ v_new) {
    using C = WinCfg<D, NT>;
    __shared__ float sc[G][128];
    __shared__ __attribute__((aligned(16))) float red[C::RPP][G][D];
    __shared__ float lsum[G];
    const int sq = blockIdx.x / a.Hkv, hk = blockIdx.x % a.Hkv;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int col = tid % C::C8, rbase = tid / C::C8;
    const int NK = a.w + a.s;
    const int ns = (NK + C::RPP - 1) / C::RPP;   // row passes that hold any row
    const int64_t ring_base = ((int64_t)sq * a.Hkv + hk) * a.w * D;
    const int64_t sink_base = ((int64_t)sq * a.Hkv + hk) * a.s * D;

    // ---- everything that does not depend on the position, in flight at once
    const int p = q_pos[sq];
    uint4 qx[G];
#pragma unroll
    for (int g = 0; g < G; ++g)
        qx[g] = *reinterpret_cast<const uint4 *>(q + ((int64_t)sq * a.Hq + hk * G + g) * D + 8 * col);
    uint4 kx[C::NS], vx[C::NS];
#pragma unroll
    for (int r = 0; r < C::NS; ++r) {
        const int e = rbase + C::RPP * r;   // row: ring slot e, or sink entry e - w
        const int64_t off = e < a.w ? ring_base + (int64_t)e * D : sink_base + (int64_t)(e - a.w) * D;
        const uint16_t *kb = e < a.w ? a.k_ring : a.k_sink;
        const uint16_t *vb = e < a.w ? a.v_ring : a.v_sink;
        kx[r] = e < NK ? ldg16(kb + off + 8 * col) : make_uint4(0, 0, 0, 0);
        vx[r] = e < NK ? ldg16(vb + off + 8 * col) : make_uint4(0, 0, 0, 0);
    }
    uint4 knx = make_uint4(0, 0, 0, 0), vnx = make_uint4(0, 0, 0, 0);
    if (APPEND) {
        const int64_t src = ((int64_t)sq * a.Hkv + hk) * D + 8 * col;
        knx = *reinterpret_cast<const uint4 *>(k_new + src);
        vnx = *reinterpret_cast<const uint4 *>(v_new + src);
    }

    const bool valid = p >= 0 && (!a.rope || (int64_t)p < a.rope_rows);
    if (!valid) {
        for (int idx = tid; idx < G * D; idx += NT)
            Elem<OUT>::store(o, ((int64_t)sq * a.Hq + hk * G) * D + idx, qnan());
        return;
    }
    // ---- rotation of this thread's 4 pairs at position p
    float cs8[8] = {1.f, 0.f, 1.f, 0.f, 1.f, 0.f, 1.f, 0.f};
    if (a.rope) {
        const float4 *t = reinterpret_cast<const float4 *>(a.rope + ((int64_t)p * (D / 2) + 4 * col) * 2);
        const float4 t0 = t[0], t1 = t[1];
        cs8[0] = t0.x; cs8[1] = t0.y; cs8[2] = t0.z; cs8[3] = t0.w;
        cs8[4] = t1.x; cs8[5] = t1.y; cs8[6] = t1.z; cs8[7] = t1.w;
    }
    auto unpack = [](uint4 x, float (&f)[8]) {
        const uint32_t w4[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            f[2 * m] = __uint_as_float(w4[m] << 16);
            f[2 * m + 1] = __uint_as_float(w4[m] & 0xffff0000u);
        }
    };
    float qf[G][8];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        float f[8];
        unpack(qx[g], f);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const float c = cs8[2 * m], sn = cs8[2 * m + 1];
            qf[g][2 * m] = fmaf(-f[2 * m + 1], sn, f[2 * m] * c) * a.cs;
            qf[g][2 * m + 1] = fmaf(f[2 * m], sn, f[2 * m + 1] * c) * a.cs;
        }
    }
    const int slot_new = p % a.w;
    if (APPEND) {
        // rotate the new key, round it as the cache stores it, write the ring slot (and the
        // sink entry), and put it in place of the slot's old row
        float f[8];
        unpack(knx, f);
        uint32_t kk[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const float c = cs8[2 * m], sn = cs8[2 * m + 1];
            kk[m] = pack_bf16x2(fmaf(-f[2 * m + 1], sn, f[2 * m] * c), fmaf(f[2 * m], sn, f[2 * m + 1] * c));
        }
        knx = make_uint4(kk[0], kk[1], kk[2], kk[3]);
#pragma unroll
        for (int r = 0; r < C::NS; ++r) {
            if (rbase + C::RPP * r == slot_new) {
                kx[r] = knx;
                vx[r] = vnx;
                *reinterpret_cast<uint4 *>(a.k_ring + ring_base + (int64_t)slot_new * D + 8 * col) = knx;
                *reinterpret_cast<uint4 *>(a.v_ring + ring_base + (int64_t)slot_new * D + 8 * col) = vnx;
            }
        }
        if (p < a.s && rbase == 0) {
            *reinterpret_cast<uint4 *>(a.k_sink + sink_base + (int64_t)p * D + 8 * col) = knx;
            *reinterpret_cast<uint4 *>(a.v_sink + sink_base + (int64_t)p * D + 8 * col) = vnx;
        }
    }
    // ---- scores of my rows: partial dot over my chunk, reduced across the row's chunks
    const int lo = p - a.w + 1 > 0 ? p - a.w + 1 : 0;
    for (int g = tid; g < G * 128; g += NT) sc[g / 128][g % 128] = -INFINITY;
    __syncthreads();
#pragma unroll
    for (int r = 0; r < C::NS; ++r) {
        if (r >= ns) break;   // uniform: rows past the key set
        const int e = rbase + C::RPP * r;
        float f[8];
        unpack(kx[r], f);
        float part[G];
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float acc = 0.0f;
#pragma unroll
            for (int c = 0; c < 8; ++c) acc = fmaf(qf[g][c], f[c], acc);
            part[g] = acc;
        }
#pragma unroll
        for (int g = 0; g < G; ++g) part[g] = C::C8 == 16 ? group16_sum(part[g]) : group8_sum(part[g]);
        if (col == 0 && e < 128) {
            // position held by row e, and whether it belongs to the key set
            int P;
            bool inset;
            if (e < a.w) {
                // ring slot e holds p - ((p - e) mod w); with slot_new = p mod w and e < w
                // that distance is slot_new - e, or slot_new - e + w when negative
                const int dist = slot_new >= e ? slot_new - e : slot_new - e + a.w;
                P = p - dist;
                inset = e < NK && P >= 0;
            } else {
                P = e - a.w;
                inset = e < NK && P < lo;
            }
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const float slope = a.slopes ? a.slopes[hk * G + g] * 1.4426950408889634f : 0.0f;
                sc[g][e] = inset ? fmaf(slope, (float)(p - P), part[g]) : -INFINITY;
            }
        }
    }
    __syncthreads();
    // ---- weights: one wavefront per head, two rows per lane
    for (int g = wave; g < G; g += C::NW) {
        float x0 = sc[g][lane], x1 = sc[g][lane + 64];
        if (a.mode == 0) {
            x0 = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-x0));
            x1 = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-x1));
        } else {
            const float m = wave_max(fmaxf(x0, x1));
            x0 = __builtin_amdgcn_exp2f(x0 - m);
            x1 = __builtin_amdgcn_exp2f(x1 - m);
            const float l = wave_sum(x0 + x1);
            if (lane == 0) lsum[g] = l;
        }
        sc[g][lane] = x0;
        sc[g][lane + 64] = x1;
    }
    __syncthreads();
    // ---- values: my chunk of every row I own, summed over rows
    float acc[G][8];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[g][c] = 0.0f;
#pragma unroll
    for (int r = 0; r < C::NS; ++r) {
        if (r >= ns) break;
        const int e = rbase + C::RPP * r;
        if (e < NK) {
            float f[8];
            unpack(vx[r], f);
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const float wgt = sc[g][e];
#pragma unroll
                for (int c = 0; c < 8; ++c) acc[g][c] = fmaf(wgt, f[c], acc[g][c]);
            }
        }
    }
    // partial sums of the RPP row groups, added through LDS
#pragma unroll
    for (int g = 0; g < G; ++g) {
        float4 *dst = reinterpret_cast<float4 *>(&red[rbase][g][8 * col]);
        dst[0] = make_float4(acc[g][0], acc[g][1], acc[g][2], acc[g][3]);
        dst[1] = make_float4(acc[g][4], acc[g][5], acc[g][6], acc[g][7]);
    }
    __syncthreads();
    for (int idx = tid; idx < G * D; idx += NT) {
        const int g = idx / D, cc = idx % D;
        float sum = 0.0f;
#pragma unroll
        for (int r = 0; r < C::RPP; ++r) sum += red[r][g][cc];
        if (a.mode == 1) sum /= lsum[g];
        Elem<OUT>::store(o, ((int64_t)sq * a.Hq + hk * G + g) * D + cc, sum);
    }
}

template <int D, int G, int OUT, bool APPEND>
hipError_t launch_fast_t(const DecodeFast &f, const void *q, const int32_t *q_pos, void *o,
                         const void *k_new, const void *v_new, hipStream_t st) {
    if (f.w + f.s <= 128 && G <= 4) {
        hipLaunchKernelGGL((decode_window_kernel<D, G, OUT, APPEND, 512>), dim3((unsigned)(f.S * f.Hkv)),
                           dim3(512), 0, st, f, static_cast<const uint16_t *>(q), q_pos, o,
                           static_cast<const uint16_t *>(k_new), static_cast<const uint16_t *>(v_new));
        return hipGetLastError();
    }
    if (f.w + f.s <= 128) {
        hipLaunchKernelGGL((decode_window_kernel<D, G, OUT, APPEND, 256>), dim3((unsigned)(f.S * f.Hkv)),
                           dim3(256), 0, st, f, static_cast<const uint16_t *>(q), q_pos, o,
                           static_cast<const uint16_t *>(k_new), static_cast<const uint16_t *>(v_new));
        return hipGetLastError();
    }
    const size_t lds = decode_fast_lds<D>(G);
    hipLaunchKernelGGL((decode_fast_kernel<D, G, OUT, APPEND>), dim3((unsigned)(f.S * f.Hkv * f.nsplit)),
                       dim3(256), lds, st, f, static_cast<const uint16_t *>(q), q_pos, o,
                       static_cast<const uint16_t *>(k_new), static_cast<const uint16_t *>(v_new));
    if (f.nsplit > 1) {
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((decode_combine_kernel<D, G, OUT>), dim3((unsigned)(f.S * f.Hkv)),
                           dim3(256), 0, st, f, q_pos, o);
    }
    return hipGetLastError();
}

template <int D, int G>
hipError_t launch_fast_g(const DecodeFast &f, int out_dt, const void *q, const int32_t *q_pos,
                         void *o, const void *k_new, const void *v_new, hipStream_t st) {
    const bool app = k_new != nullptr;
    if (out_dt == 0) return app ? launch_fast_t<D, G, 0, true>(f, q, q_pos, o, k_new, v_new, st)
                                : launch_fast_t<D, G, 0, false>(f, q, q_pos, o, k_new, v_new, st);
    return app ? launch_fast_t<D, G, 1, true>(f, q, q_pos, o, k_new, v_new, st)
               : launch_fast_t<D, G, 1, false>(f, q, q_pos, o, k_new, v_new, st);
}

template <int D>
hipError_t launch_fast_d(const DecodeFast &f, int out_dt, const void *q, const int32_t *q_pos,
                         void *o, const void *k_new, const void *v_new, hipStream_t st) {
    switch (f.G) {
        case 1: return launch_fast_g<D, 1>(f, out_dt, q, q_pos, o, k_new, v_new, st);
        case 2: return launch_fast_g<D, 2>(f, out_dt, q, q_pos, o, k_new, v_new, st);
        case 4: return launch_fast_g<D, 4>(f, out_dt, q, q_pos, o, k_new, v_new, st);
        default: return launch_fast_g<D, 8>(f, out_dt, q, q_pos, o, k_new, v_new, st);
    }
}

bool decode_fast_ok(const DecodeArgs &a, const CacheArgs &c) {
    const int64_t G = a.Hq / c.Hkv;
    if (c.dt != 1 || (c.d != 64 && c.d != 128) || (G != 1 && G != 2 && G != 4 && G != 8)) return false;
    if (c.S * c.Hkv * 64 > 0x7fffffff || c.w > (1 << 30) || c.s > (1 << 30)) return false;
    const size_t lds = c.d == 64 ? decode_fast_lds<64>((int)G) : decode_fast_lds<128>((int)G);
    return lds <= 64 * 1024;
}

// Key ranges per (sequence, kv head) for the chunked decode: about two blocks per CU in
// total, and at least 512 keys per range.
int64_t decode_nsplit(const CacheArgs &c) {
    if (c.w + c.s <= 128) return 1;            // whole-window kernel
    const int64_t bh = c.S * c.Hkv;
    if (bh <= 0) return 1;
    int64_t ns = (512 + bh - 1) / bh;
    const int64_t by_keys = (c.w + c.s) / 512;
    if (ns > by_keys) ns = by_keys;
    if (ns > 64) ns = 64;
    return ns < 1 ? 1 : ns;
}

hipError_t launch_decode_fast(const DecodeArgs &a, const CacheArgs &c, const void *q,
                              const int32_t *q_pos, void *o, const void *k_new, const void *v_new,
                              void *ws, hipStream_t st) {
    DecodeFast f;
    f.S = (int)c.S; f.Hq = (int)a.Hq; f.Hkv = (int)c.Hkv; f.G = (int)(a.Hq / c.Hkv);
    f.w = (int)c.w; f.s = (int)c.s; f.mode = a.mode;
    f.nsplit = (int)decode_nsplit(c);
    f.part = static_cast<float *>(ws);
    f.cs = a.scale * 1.4426950408889634f;
    f.slopes = a.slopes; f.rope = a.rope; f.rope_rows = a.rope_rows;
    f.k_ring = static_cast<uint16_t *>(c.k_ring); f.v_ring = static_cast<uint16_t *>(c.v_ring);
    f.k_sink = static_cast<uint16_t *>(c.k_sink); f.v_sink = static_cast<uint16_t *>(c.v_sink);
    if (c.d == 64) return launch_fast_d<64>(f, a.out_dt, q, q_pos, o, k_new, v_new, st);
    return launch_fast_d<128>(f, a.out_dt, q, q_pos, o, k_new, v_new, st);
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
    const uintptr_t bits = reinterpret_cast<uintptr_t>(k_new) | reinterpret_cast<uintptr_t>(v_new) |
                           reinterpret_cast<uintptr_t>(c.k_ring) | reinterpret_cast<uintptr_t>(c.v_ring) |
                           reinterpret_cast<uintptr_t>(c.k_sink) | reinterpret_cast<uintptr_t>(c.v_sink) |
                           reinterpret_cast<uintptr_t>(rope);
    if (c.d % 8 == 0 && (bits & 15) == 0) {
        const int64_t n = rows * (c.d / 8);
        const dim3 grid((unsigned)((n + 255) / 256));
        if (c.dt == 0)
            hipLaunchKernelGGL(kv_append8_kernel<0>, grid, dim3(256), 0, st, c, k_new, v_new, pos0,
                               n_new, rope, rope_rows);
        else
            hipLaunchKernelGGL(kv_append8_kernel<1>, grid, dim3(256), 0, st, c, k_new, v_new, pos0,
                               n_new, rope, rope_rows);
        return hipGetLastError();
    }
    if (c.dt == 0)
        hipLaunchKernelGGL(kv_append_kernel<0>, dim3((unsigned)rows), dim3(128), 0, st, c, k_new,
                           v_new, pos0, n_new, rope, rope_rows);
    else
        hipLaunchKernelGGL(kv_append_kernel<1>, dim3((unsigned)rows), dim3(128), 0, st, c, k_new,
                           v_new, pos0, n_new, rope, rope_rows);
    return hipGetLastError();
}

size_t decode_workspace_bytes(const DecodeArgs &a, const CacheArgs &c) {
    if (c.S == 0 || !decode_fast_ok(a, c)) return 0;
    const int64_t ns = decode_nsplit(c);
    if (ns <= 1) return 0;
    return sizeof(float) * (size_t)(c.S * c.Hkv * ns * (a.Hq / c.Hkv) * (c.d + 2));
}

hipError_t launch_decode(const DecodeArgs &a, const CacheArgs &c, const void *q,
                         const int32_t *q_pos, void *o, void *ws, size_t, hipStream_t st) {
    if (c.S == 0) return hipSuccess;
    if (decode_fast_ok(a, c)) return launch_decode_fast(a, c, q, q_pos, o, nullptr, nullptr, ws, st);
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

hipError_t launch_decode_append(const DecodeArgs &a, const CacheArgs &c, const void *q,
                                const void *k_new, const void *v_new, const int32_t *q_pos,
                                void *o, void *ws, size_t ws_bytes, hipStream_t st) {
    if (c.S == 0) return hipSuccess;
    if (decode_fast_ok(a, c)) return launch_decode_fast(a, c, q, q_pos, o, k_new, v_new, ws, st);
    // general shapes: the append kernel, then the decode kernel, in stream order
    const hipError_t e = launch_kv_append(c, k_new, v_new, q_pos, 1, a.rope, a.rope_rows, st);
    if (e != hipSuccess) return e;
    return launch_decode(a, c, q, q_pos, o, ws, ws_bytes, st);
}

}  // namespace swa
