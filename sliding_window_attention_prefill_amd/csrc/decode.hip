// decode.hip - ring-buffer KV cache: append and single-token decode.
//
// The cache keeps w slots per (sequence, kv head); position p lives in slot p mod w and
// overwrites the oldest entry (Sliding Window Attention glossary, ring-buffer paragraph).
// Positions 0..s-1 are also kept in a sink store beside the ring (Sliding Window Attention
// glossary, "attention sink"; Sliding-window beats linear attention, SWA(64, 4)). Keys are
// stored rotated at their own absolute position, so a decode step only rotates its query.
#include "mfma_common.hpp"
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

// Decode for a bf16 cache, d in {64, 128}, G = H_q / H_kv in {1, 2, 4, 8}: the whole-window
// kernels (w + s <= 128: decode_wmfma_kernel at d = 128 with four or eight query heads per kv
// head, decode_window_kernel otherwise) and the split matrix-core kernel (longer windows)
// below share these arguments.
// With APPEND a block first writes the new token (rotated key, value) to its ring slot and
// sink entry, keeps it in LDS and uses that copy for position q_pos, so the slot it wrote is
// never read back within the launch.
// Split-KV: with nsplit > 1 the key list of a query is cut into nsplit contiguous ranges, one
// block each; a block writes its unnormalised partial output with its running maximum and
// sum to the workspace, and decode_combine_kernel merges the partials (log-sum-exp
// rescaling for softmax, a plain sum for sigmoid). Only the block whose range holds the
// query's own position appends the new token.
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

// Block barrier that orders LDS accesses only: global loads in flight stay in flight.
__device__ __forceinline__ void lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Merge of the split partials of decode_mfma_kernel: one block per (sequence, kv head).
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
            // one pass, online: the loads of every range are independent of the running
            // maximum, so they are all in flight together
            float M = -INFINITY, num = 0.0f, den = 0.0f;
#pragma unroll 8
            for (int k = 0; k < a.nsplit; ++k) {
                const float *e = pp + (k * G + g) * (D + 2);
                const float m = e[D], x = e[col], l = e[D + 1];
                const float M2 = fmaxf(M, m);
                const float fo = __builtin_amdgcn_exp2f(M - M2);   // 2^-inf = 0 at the start
                const float fn = __builtin_amdgcn_exp2f(m - M2);
                num = fmaf(num, fo, x * fn);
                den = fmaf(den, fo, l * fn);
                M = M2;
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
    // block: (sequence, kv head, head part); the kv head's a.G query heads are split into
    // parts of G heads, each block reading the whole window for its part
    const int hs = blockIdx.x % (a.G / G), bsh = blockIdx.x / (a.G / G);
    const int sq = bsh / a.Hkv, hk = bsh % a.Hkv;
    const int hbase = hk * a.G + hs * G;
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
        qx[g] = *reinterpret_cast<const uint4 *>(q + ((int64_t)sq * a.Hq + hbase + g) * D + 8 * col);
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
            Elem<OUT>::store(o, ((int64_t)sq * a.Hq + hbase) * D + idx, qnan());
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
        // every head part uses the new token; the first one writes it
#pragma unroll
        for (int r = 0; r < C::NS; ++r) {
            if (rbase + C::RPP * r == slot_new) {
                kx[r] = knx;
                vx[r] = vnx;
                if (hs == 0) {
                    *reinterpret_cast<uint4 *>(a.k_ring + ring_base + (int64_t)slot_new * D + 8 * col) = knx;
                    *reinterpret_cast<uint4 *>(a.v_ring + ring_base + (int64_t)slot_new * D + 8 * col) = vnx;
                }
            }
        }
        if (p < a.s && rbase == 0 && hs == 0) {
            *reinterpret_cast<uint4 *>(a.k_sink + sink_base + (int64_t)p * D + 8 * col) = knx;
            *reinterpret_cast<uint4 *>(a.v_sink + sink_base + (int64_t)p * D + 8 * col) = vnx;
        }
    }
    // ---- scores of my rows: partial dot over my chunk, reduced across the row's chunks;
    // every row below NK gets its logit (or -inf outside the key set), rows past NK are
    // never read
    const int lo = p - a.w + 1 > 0 ? p - a.w + 1 : 0;
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
        if (col == 0 && e < NK) {
            // position held by row e, and whether it belongs to the key set
            int P;
            bool inset;
            if (e < a.w) {
                // ring slot e holds p - ((p - e) mod w); with slot_new = p mod w and e < w
                // that distance is slot_new - e, or slot_new - e + w when negative
                const int dist = slot_new >= e ? slot_new - e : slot_new - e + a.w;
                P = p - dist;
                inset = P >= 0;
            } else {
                P = e - a.w;
                inset = P < lo;
            }
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const float slope = a.slopes ? a.slopes[hbase + g] * 1.4426950408889634f : 0.0f;
                sc[g][e] = inset ? fmaf(slope, (float)(p - P), part[g]) : -INFINITY;
            }
        }
    }
    __syncthreads();
    // ---- weights: one wavefront per head, two rows per lane
    for (int g = wave; g < G; g += C::NW) {
        float x0 = lane < NK ? sc[g][lane] : -INFINITY;
        float x1 = lane + 64 < NK ? sc[g][lane + 64] : -INFINITY;
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
        Elem<OUT>::store(o, ((int64_t)sq * a.Hq + hbase + g) * D + cc, sum);
    }
}

// Matrix-core decode for long windows (bf16 cache, d in {64, 128}). One block of four
// wavefronts per (sequence, kv head, key range), with the key ranges of the split scheme
// above; each wavefront walks its own 32-key tiles of the range (tiles wave, wave + 4, ...)
// with no block barrier inside the walk, and the four partial results are merged at the end.
//   scores  S^T = K Q^T with v_mfma_f32_32x32x16_bf16: the K rows are the A operand exactly
//           as stored, loaded from memory straight into registers. Column n of the B operand
//           holds, for n < G, the bf16 part hi of query head n (rotated, times scale log2 e)
//           and, for G <= n < 2G, the bf16 remainder lo of head n - G, so that hi + lo keeps
//           about 16 bits of the query; a lane exchange adds the two columns, after which both
//           lanes of a head hold its full base-2 logit.
//   weights ALiBi, the end-of-range cut and the running maximum (lazy rescale, as in the
//           prefill kernels) on the vector unit.
//   values  O^T += V^T P^T: V rows go buffer -> LDS (two tiles per wavefront, 16-byte chunks
//           XOR-swizzled by row) and come back through transposing LDS reads; the weights
//           enter as bf16 hi / lo columns again, so both products are exact up to float32
//           accumulation.
// Sink keys and window keys form separate tiles, so that each tile reads a single store.
template <int D>
struct DecM {
    static constexpr int KS = D / 16;              // k-steps of the score product
    static constexpr int DB = D / 32;              // 32-row blocks of O^T
    static constexpr int C = D / 8;                // 16-byte chunks per row
    static constexpr int TE = 32 * D;              // bf16 elements of one V tile
    static constexpr int ROUNDS = TE * 2 / 1024;   // 1 KB transfers per tile and wavefront
};

// Chunk c of V tile row r sits at chunk c ^ dec_vswz(r), which spreads the transposing reads
// over all banks.
template <int D>
__device__ __forceinline__ constexpr int dec_vswz(int r) {
    return D == 64 ? ((r >> 1) & 1) << 2 : (r & 3) << 2;
}

// V tiles (4 wavefronts x 2 x 32 rows x d bf16), reused by the merge for 4 x 2G x d floats;
// then the appended key and value (d bf16 each), 4 x 8 x 2 floats of running state and the
// query operand (d / 16 k-steps x 64 lanes x 16 bytes).
__host__ __device__ constexpr size_t decode_mfma_vbytes(int d, int G) {
    return (size_t)4 * 2 * 32 * d * 2 > (size_t)4 * 2 * G * d * 4 ? (size_t)4 * 2 * 32 * d * 2
                                                                   : (size_t)4 * 2 * G * d * 4;
}
size_t decode_mfma_lds(int d, int G) {
    return decode_mfma_vbytes(d, G) + (size_t)4 * d + 4 * 8 * 2 * 4 + (size_t)d / 16 * 64 * 16;
}

// Buffer offsets are 32-bit: each (sequence, kv head) slice of the ring and of the sink
// store stays below 2 GB.
bool decode_mfma_fits(int64_t w, int64_t s, int d) {
    return w * d * 2 < ((int64_t)1 << 31) && s * d * 2 < ((int64_t)1 << 31);
}

constexpr uint32_t DEC_OOB = 0x80000000u;  // past every store: buffer reads return zero

// One 32-key tile of a query's key list: sink tiles first, then window tiles.
struct DecTile {
    bool sink;  // rows come from the sink store
    int base;   // sink index / window offset of row 0
    int lim;    // rows below lim hold keys
    int u0;     // p - (position of row 0)
};

struct DecCtx {
    __amdgpu_buffer_rsrc_t rk_ring, rv_ring, rk_sink, rv_sink;
    uint32_t row_bytes;
    int w, slot_lo, n_sink, n_win, n_st, p;
    int t_end;          // tiles at or past t_end are empty (no rows, no transfers)
    int lane, col, half;
    bool qcol, lo_part;
    float slope_l2;

    __device__ __forceinline__ DecTile tile(int tt) const {
        DecTile t;
        t.sink = tt < n_st;
        t.base = t.sink ? 32 * tt : 32 * (tt - n_st);
        t.lim = tt < t_end ? (t.sink ? n_sink : n_win) - t.base : 0;
        t.u0 = t.sink ? p - t.base : n_win - 1 - t.base;
        return t;
    }
    // byte offset of tile row r in its store (DEC_OOB past the key list)
    __device__ __forceinline__ uint32_t row_off(const DecTile &t, int r) const {
        int slot = t.base + r;
        if (!t.sink) {
            slot += slot_lo;
            if (slot >= w) slot -= w;
        }
        return r < t.lim ? (uint32_t)slot * row_bytes : DEC_OOB;
    }
};

// V tile rows -> LDS: round i moves slots 64 i .. 64 i + 63 (slot = row * C + stored chunk
// position), lane l the slot 64 i + l.
template <int D>
__device__ __forceinline__ void dec_load_v(const DecCtx &cx, uint16_t *dst, const DecTile &t) {
    using M = DecM<D>;
    const __amdgpu_buffer_rsrc_t r = t.sink ? cx.rv_sink : cx.rv_ring;
#pragma unroll
    for (int i = 0; i < M::ROUNDS; ++i) {
        const int slot = 64 * i + cx.lane, row = slot / M::C;
        const int c = (slot % M::C) ^ dec_vswz<D>(row);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t *)(dst + 512 * i), 16,
                                                 cx.row_off(t, row) + 16 * c, 0, 0, 0);
    }
}
// K tile as the A operand: lane l holds row l % 32, chunk 2 ks + l / 32 for k-step ks.
template <int D>
__device__ __forceinline__ void dec_load_k(const DecCtx &cx, bf16x8_t (&kr)[D / 16], const DecTile &t) {
    const __amdgpu_buffer_rsrc_t r = t.sink ? cx.rk_sink : cx.rk_ring;
    const uint32_t o0 = cx.row_off(t, cx.col) + 16 * cx.half;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
        kr[ks] = __builtin_bit_cast(bf16x8_t, buf_load16(r, o0 + 32 * ks));
}

// Wait until only the KS + ROUNDS transfers this step started are outstanding, whatever
// order they were issued in: the current tile's V rows have landed. The memory clobber
// keeps the LDS reads below the wait.
template <int D>
__device__ __forceinline__ void wait_own_tile() {
    using M = DecM<D>;
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(M::KS + M::ROUNDS) : "memory");
}

// One tile of a wavefront's walk: start the transfers of the next tile (V into v_fill, K into
// k_next; past the range they are out-of-range reads that move nothing, so every step issues
// the same count), then scores, weights and the value product of this tile (K in k_cur, V in
// v_cur). The two V buffers are distinct restrict pointers, so that reads of v_cur do not
// wait for the transfer into v_fill.
template <int D, int G, bool APPEND>
__device__ __forceinline__ void dec_step(const DecCtx &cx, uint16_t *__restrict__ v_cur,
                                         uint16_t *__restrict__ v_fill, bf16x8_t (&k_cur)[D / 16],
                                         bf16x8_t (&k_next)[D / 16], const uint4 *qop,
                                         f32x16_t (&oacc)[D / 32], float &m_run, float &l_run,
                                         int mode, int tt, int t_new,
                                         const uint32_t *knew, const uint32_t *vnew) {
    using M = DecM<D>;
    const DecTile t = cx.tile(tt);
    // the previous step's reads of v_fill are complete before its refill starts
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    {
        const DecTile tn = cx.tile(tt + 4);
        dec_load_v<D>(cx, v_fill, tn);
        dec_load_k<D>(cx, k_next, tn);
    }
    // the appended token replaces what its ring slot held before this launch
    const bool has_new = APPEND && tt == t_new;
    const int r_new = cx.n_win - 1 - t.base;
    if (has_new && cx.col == r_new) {
#pragma unroll
        for (int ks = 0; ks < M::KS; ++ks) {
            const uint32_t *kp = knew + 4 * (2 * ks + cx.half);
            k_cur[ks] = __builtin_bit_cast(bf16x8_t, make_uint4(kp[0], kp[1], kp[2], kp[3]));
        }
    }
    f32x16_t s = {};
#pragma unroll
    for (int ks = 0; ks < M::KS; ++ks)
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k_cur[ks], __builtin_bit_cast(bf16x8_t, qop[64 * ks + cx.lane]),
                                                    s, 0, 0, 0);
    // hi + lo columns, then ALiBi and the cut: element e is row 8 (e / 4) + 4 half + e % 4
    const int partner = cx.lo_part ? cx.lane - G : cx.lane + G;
    const float u0 = (float)(t.u0 - 4 * cx.half);
    const int lim = t.lim - 4 * cx.half;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const int kr = 8 * (e >> 2) + (e & 3);
        const float full = s[e] + __shfl(s[e], partner, 64);
        s[e] = kr < lim ? fmaf(cx.slope_l2, u0 - (float)kr, full) : -INFINITY;
    }
    if (mode == 0) {
#pragma unroll
        for (int e = 0; e < 16; ++e)
            s[e] = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-s[e]));
    } else {
        float mt = s[0];
#pragma unroll
        for (int e = 1; e < 16; ++e) mt = fmaxf(mt, s[e]);
        mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
        const float m_new = fmaxf(m_run, mt);
        // keep a stale maximum while the new one exceeds it by less than 8 (weights stay
        // below 2^8); the merge uses the same maximum
        const bool need = m_new > m_run + 8.0f;
        if (__any(need)) {
            const float corr = need ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
#pragma unroll
            for (int db = 0; db < M::DB; ++db)
#pragma unroll
                for (int e = 0; e < 16; ++e) oacc[db][e] *= corr;
            l_run *= corr;
            m_run = need ? m_new : m_run;
        }
        float ls = 0.0f;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            s[e] = __builtin_amdgcn_exp2f(s[e] - m_run);
            ls += s[e];
        }
        l_run += ls;
    }
    // P^T operand of step j (keys 16 j + 4 half + {0..3, 8..11}): elements 8 j .. 8 j + 7,
    // as bf16 hi (columns < G) or lo (columns G .. 2G - 1)
    uint4 pk[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        float x[8];
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const float v = s[8 * j + m];
            const float hi = bf16_bits_to_f32(f32_to_bf16_bits(v));
            x[m] = cx.lo_part ? v - hi : v;
        }
        const uint4 pp = make_uint4(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]),
                                    pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7]));
        pk[j] = cx.qcol ? pp : make_uint4(0, 0, 0, 0);
    }
    wait_own_tile<D>();
    if (has_new) {
        // the tile's own transfer has landed: the new value over its row
        if (cx.lane < M::C) {
            const int pos = (r_new * M::C + (cx.lane ^ dec_vswz<D>(r_new))) * 8;
            const uint32_t *vp = vnew + 4 * cx.lane;
            *reinterpret_cast<uint4 *>(v_cur + pos) = make_uint4(vp[0], vp[1], vp[2], vp[3]);
        }
    }
    // transposing read: lane (G4, rr, a) supplies row 4 (G4 / 2) + rr and column group
    // 16 (G4 % 2) + 4 a of the 8 x 32 block one read covers
    const int G4 = cx.lane >> 4, rr = (cx.lane >> 2) & 3, a = cx.lane & 3;
    const int row_l = 4 * (G4 >> 1) + rr, cb = 2 * (G4 & 1) + (a >> 1);
    const int fq = dec_vswz<D>(rr) >> 2;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int db = 0; db < M::DB; ++db) {
            const int vo = row_l * D + (4 * (db ^ fq) + cb) * 8 + 4 * (a & 1);
            const s16x4_t lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)(v_cur + 16 * j * D + vo));
            const s16x4_t hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)(v_cur + (16 * j + 8) * D + vo));
            const s16x8_t a8 = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
            oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a8),
                                                               __builtin_bit_cast(bf16x8_t, pk[j]),
                                                               oacc[db], 0, 0, 0);
        }
}

// Whole-window decode on the matrix cores, d = 128 with four query heads per block and at most
// 128 window + sink rows (e.g. SWA(64, 4)). As in decode_window_kernel, every K and V row a
// query can read is known without its position, so all loads are issued first. One block of
// four wavefronts per (sequence, kv head, head part); wavefront t owns storage rows
// 32 t .. 32 t + 31 (ring slots, then sink entries):
//   scores  S^T = K Q^T with v_mfma_f32_32x32x16_bf16, the K rows as loaded in the A operand
//           layout (exact) and the query in bf16 hi / lo columns (as in decode_mfma_kernel,
//           about 16 bits); the position then decides which rows count and their bias.
//   weights per wavefront: sigmoid directly, softmax against the wavefront's own maximum.
//   values  O^T += V^T P^T with V staged in LDS and read transposed, P in hi / lo columns.
// The four partial results (and, for softmax, their maxima and sums) meet in LDS once.
template <int OUT, bool APPEND>
__global__ __launch_bounds__(256) void decode_wmfma_kernel(DecodeFast a, const uint16_t *__restrict__ q,
                                                           const int32_t *__restrict__ q_pos,
                                                           void *__restrict__ o,
                                                           const uint16_t *__restrict__ k_new,
                                                           const uint16_t *__restrict__ v_new) {
    constexpr int D = 128, G = 4, KS = D / 16, DB = D / 32, C = D / 8;
    __shared__ __attribute__((aligned(16))) uint16_t vt[4][32 * D];   // V rows, chunk-swizzled
    __shared__ __attribute__((aligned(16))) uint4 qop[KS * 64];       // query operand, columns < 2G
    __shared__ __attribute__((aligned(16))) uint16_t knr[D];          // appended key, rotated
    __shared__ __attribute__((aligned(16))) float red[4][2 * G][D];   // partial O^T per wavefront
    __shared__ float mls[4][G][2];                                     // (maximum, sum) per wavefront

    // grid (sequence, kv head, head part): no division by a runtime count before the loads
    const int sq = blockIdx.x, hk = blockIdx.y, hs = blockIdx.z;
    const int p = q_pos[sq];
    const int hbase = hk * a.G + hs * G;
    const int tid = threadIdx.x, lane = tid & 63, t = tid >> 6;
    const int col = lane & 31, half = lane >> 5;
    const int NK = a.w + a.s;
    const int64_t ring_base = ((int64_t)sq * a.Hkv + hk) * a.w * D;
    const int64_t sink_base = ((int64_t)sq * a.Hkv + hk) * a.s * D;
    auto row_ptr = [&](const uint16_t *ring, const uint16_t *sink, int e) {
        return e < a.w ? ring + ring_base + (int64_t)e * D : sink + sink_base + (int64_t)(e - a.w) * D;
    };

    // ---- loads that do not depend on the position, all in flight together
    const bool live = 32 * t < NK;                 // uniform: the wavefront owns any row
    const int er = 32 * t + col;                   // this lane's K row
    uint4 kx[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        kx[ks] = er < NK ? ldg16(row_ptr(a.k_ring, a.k_sink, er) + 8 * (2 * ks + half)) : make_uint4(0, 0, 0, 0);
    // V rows in the LDS layout of decode_mfma_kernel's tiles: slot 64 i + lane holds row
    // slot / C, stored chunk slot % C, which is chunk (slot % C) ^ dec_vswz(row)
    uint4 vx[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int slot = 64 * i + lane, r = slot / C, c = (slot % C) ^ dec_vswz<D>(r);
        const int e = 32 * t + r;
        vx[i] = e < NK ? ldg16(row_ptr(a.v_ring, a.v_sink, e) + 8 * c) : make_uint4(0, 0, 0, 0);
    }
    // the query pair this thread rotates: head tid / 64, dimensions 2 (tid % 64) + {0, 1}
    const int qh = tid >> 6, qj = tid & 63;
    const uint32_t qw = *reinterpret_cast<const uint32_t *>(q + ((int64_t)sq * a.Hq + hbase + qh) * D + 2 * qj);
    uint32_t kw = 0;
    uint4 vn = make_uint4(0, 0, 0, 0);
    if (APPEND) {
        const int64_t src = ((int64_t)sq * a.Hkv + hk) * D;
        if (tid < D / 2) kw = *reinterpret_cast<const uint32_t *>(k_new + src + 2 * tid);
        if (lane < C) vn = *reinterpret_cast<const uint4 *>(v_new + src + 8 * lane);
    }

    const bool valid = p >= 0 && (!a.rope || (int64_t)p < a.rope_rows);
    if (!valid) {
        for (int idx = tid; idx < G * D; idx += 256)
            Elem<OUT>::store(o, ((int64_t)sq * a.Hq + hbase) * D + idx, qnan());
        return;
    }
    float cs = 1.0f, sn = 0.0f;
    if (a.rope) {
        const float2 cw = *reinterpret_cast<const float2 *>(a.rope + ((int64_t)p * (D / 2) + qj) * 2);
        cs = cw.x; sn = cw.y;
    }
    const int slot_new = p % a.w;
    {
        // query operand: column qh carries the bf16 part hi of the rotated, scaled query and
        // column G + qh its remainder lo; dimension d sits in k-step d / 16, lane half
        // (d % 16) / 8, element d % 8
        const float x0 = bf16_bits_to_f32(qw & 0xffffu), x1 = bf16_bits_to_f32(qw >> 16);
        const float r0 = fmaf(-x1, sn, x0 * cs) * a.cs, r1 = fmaf(x0, sn, x1 * cs) * a.cs;
        const float h0 = bf16_bits_to_f32(f32_to_bf16_bits(r0)), h1 = bf16_bits_to_f32(f32_to_bf16_bits(r1));
        const int d = 2 * qj, ks = d >> 4, hf = (d >> 3) & 1, el = d & 7;
        uint32_t *qo = reinterpret_cast<uint32_t *>(qop);
        qo[((64 * ks + 32 * hf + qh) * 8 + el) >> 1] = pack_bf16x2(h0, h1);
        qo[((64 * ks + 32 * hf + G + qh) * 8 + el) >> 1] = pack_bf16x2(r0 - h0, r1 - h1);
    }
    if (APPEND && tid < D / 2) {
        // the appended key, rotated and rounded as the cache stores it
        const float x0 = bf16_bits_to_f32(kw & 0xffffu), x1 = bf16_bits_to_f32(kw >> 16);
        const uint32_t kr = pack_bf16x2(fmaf(-x1, sn, x0 * cs), fmaf(x0, sn, x1 * cs));
        reinterpret_cast<uint32_t *>(knr)[tid] = kr;
        if (hs == 0) {
            *reinterpret_cast<uint32_t *>(a.k_ring + ring_base + (int64_t)slot_new * D + 2 * tid) = kr;
            if (p < a.s) *reinterpret_cast<uint32_t *>(a.k_sink + sink_base + (int64_t)p * D + 2 * tid) = kr;
        }
    }
    if (APPEND && hs == 0 && t == 0 && lane < C) {
        *reinterpret_cast<uint4 *>(a.v_ring + ring_base + (int64_t)slot_new * D + 8 * lane) = vn;
        if (p < a.s) *reinterpret_cast<uint4 *>(a.v_sink + sink_base + (int64_t)p * D + 8 * lane) = vn;
    }
    // V rows into this wavefront's LDS tile; then the appended value over its slot's row (the
    // same wavefront, later in program order)
    uint16_t *const vl = vt[t];
#pragma unroll
    for (int i = 0; i < 8; ++i) *reinterpret_cast<uint4 *>(vl + (64 * i + lane) * 8) = vx[i];
    if (APPEND && (slot_new >> 5) == t && lane < C) {
        const int r = slot_new & 31;
        *reinterpret_cast<uint4 *>(vl + (r * C + (lane ^ dec_vswz<D>(r))) * 8) = vn;
    }
    __syncthreads();

    f32x16_t oacc[DB];
    float m_w = -INFINITY, l_w = 0.0f;
    if (live) {
        if (APPEND && er == slot_new) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) kx[ks] = *reinterpret_cast<const uint4 *>(knr + 8 * (2 * ks + half));
        }
        const bool qcol = col < 2 * G, lo_part = col >= G;
        // every operand read first, then two independent product chains
        uint4 qb[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qb[ks] = qcol ? qop[64 * ks + lane] : make_uint4(0, 0, 0, 0);
        f32x16_t sacc = {}, sacc2 = {};
#pragma unroll
        for (int ks = 0; ks < KS; ks += 2) {
            sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, kx[ks]),
                                                           __builtin_bit_cast(bf16x8_t, qb[ks]), sacc, 0, 0, 0);
            sacc2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, kx[ks + 1]),
                                                            __builtin_bit_cast(bf16x8_t, qb[ks + 1]), sacc2, 0, 0, 0);
        }
#pragma unroll
        for (int e = 0; e < 16; ++e) sacc[e] += sacc2[e];
        // hi + lo columns; element e is storage row 32 t + 8 (e / 4) + 4 half + e % 4, which
        // counts when it holds a position of the key set: ring slot r holds
        // p - ((slot_new - r) mod w), sink entry j position j while the window no longer
        // covers it; the bias is slope (p - position)
        const int partner = lo_part ? lane - G : lane + G;
        const int hg = lo_part ? col - G : col;
        const float slope = (a.slopes && qcol) ? a.slopes[hbase + hg] * 1.4426950408889634f : 0.0f;
        const int lo = p - a.w + 1 > 0 ? p - a.w + 1 : 0;
        float s[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int r = 32 * t + 8 * (e >> 2) + 4 * half + (e & 3);
            const float full = sacc[e] + __shfl(sacc[e], partner, 64);
            int dist;
            bool inset;
            if (r < a.w) {
                dist = slot_new >= r ? slot_new - r : slot_new - r + a.w;
                inset = dist <= p;
            } else {
                dist = p - (r - a.w);
                inset = r < NK && r - a.w < lo;
            }
            s[e] = inset ? fmaf(slope, (float)dist, full) : -INFINITY;
        }
        if (a.mode == 0) {
#pragma unroll
            for (int e = 0; e < 16; ++e) s[e] = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-s[e]));
        } else {
            float mt = s[0];
#pragma unroll
            for (int e = 1; e < 16; ++e) mt = fmaxf(mt, s[e]);
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt), __float_as_uint(mt), false, false);
            mt = fmaxf(mt, fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])));
            m_w = mt;
            const float mref = mt == -INFINITY ? 0.0f : mt;   // a wavefront with no row of the set
            float ls = 0.0f;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                s[e] = __builtin_amdgcn_exp2f(s[e] - mref);
                ls += s[e];
            }
            const auto sl = __builtin_amdgcn_permlane32_swap(__float_as_uint(ls), __float_as_uint(ls), false, false);
            l_w = __uint_as_float(sl[0]) + __uint_as_float(sl[1]);
        }
        // P^T operand of k-step j (rows 16 j + 4 half + {0..3, 8..11}): bf16 hi (columns < G)
        // or lo (columns G .. 2G - 1)
        uint4 pk[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            float x[8];
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                const float v = s[8 * j + m];
                const float h = bf16_bits_to_f32(f32_to_bf16_bits(v));
                x[m] = lo_part ? v - h : v;
            }
            const uint4 pp = make_uint4(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]),
                                        pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7]));
            pk[j] = qcol ? pp : make_uint4(0, 0, 0, 0);
        }
        // transposing read: lane (G4, rr, a) supplies row 4 (G4 / 2) + rr and column group
        // 16 (G4 % 2) + 4 a of the 8 x 32 block one read covers
        const int G4 = lane >> 4, rr = (lane >> 2) & 3, aa = lane & 3;
        const int row_l = 4 * (G4 >> 1) + rr, cb = 2 * (G4 & 1) + (aa >> 1);
        const int fq = dec_vswz<D>(rr) >> 2;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            oacc[db] = f32x16_t{};
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int vo = row_l * D + (4 * (db ^ fq) + cb) * 8 + 4 * (aa & 1);
                const s16x4_t lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)(vl + 16 * j * D + vo));
                const s16x4_t hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t *)(vl + (16 * j + 8) * D + vo));
                const s16x8_t a8 = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
                oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a8),
                                                                   __builtin_bit_cast(bf16x8_t, pk[j]),
                                                                   oacc[db], 0, 0, 0);
            }
        }
        // partial O^T: element e of block db is dimension 32 db + 8 (e / 4) + 4 half + e % 4
        if (qcol) {
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    *reinterpret_cast<float4 *>(&red[t][col][32 * db + 8 * u + 4 * half]) =
                        make_float4(oacc[db][4 * u], oacc[db][4 * u + 1], oacc[db][4 * u + 2], oacc[db][4 * u + 3]);
        }
        if (lane < G) {
            mls[t][lane][0] = m_w;
            mls[t][lane][1] = l_w;
        }
    }
    __syncthreads();
    // ---- merge of the wavefronts that own rows: sigmoid adds; softmax rescales each partial
    // by 2^(m_t - M)
    const int nt = (NK + 31) >> 5;
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const int idx = tid + 256 * it;
        const int g = idx / D, d = idx % D;
        // every read of the (at most four) wavefronts first, then the arithmetic
        float x[4], m[4], l[4];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            const bool in = tt < nt;
            x[tt] = in ? red[tt][g][d] + red[tt][G + g][d] : 0.0f;
            m[tt] = in ? mls[tt][g][0] : -INFINITY;
            l[tt] = in ? mls[tt][g][1] : 0.0f;
        }
        float sum = 0.0f;
        if (a.mode == 0) {
            sum = (x[0] + x[1]) + (x[2] + x[3]);
        } else {
            const float M = fmaxf(fmaxf(m[0], m[1]), fmaxf(m[2], m[3]));
            float den = 0.0f;
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                const float f = m[tt] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m[tt] - M);
                sum = fmaf(x[tt], f, sum);
                den = fmaf(l[tt], f, den);
            }
            sum *= __builtin_amdgcn_rcpf(den);
        }
        // streaming (non-temporal) stores: the outputs are not read again by this launch, and
        // the launch's end waits for them (0.33 us less per SWA(64, 4) step than plain stores)
        const int64_t off = ((int64_t)sq * a.Hq + hbase + g) * D + d;
        if (OUT == 0)
            __builtin_nontemporal_store(sum, static_cast<float *>(o) + off);
        else
            __builtin_nontemporal_store(f32_to_bf16_bits(sum), static_cast<uint16_t *>(o) + off);
    }
}

// Two wavefronts per SIMD: two blocks per CU keep 16 tiles of transfers in flight.
template <int D, int G, int OUT, bool APPEND>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void decode_mfma_kernel(DecodeFast a, const uint16_t *__restrict__ q,
                                                          const int32_t *__restrict__ q_pos,
                                                          void *__restrict__ o,
                                                          const uint16_t *__restrict__ k_new,
                                                          const uint16_t *__restrict__ v_new) {
    using M = DecM<D>;
    extern __shared__ uint4 dlds4[];
    uint16_t *lds = reinterpret_cast<uint16_t *>(dlds4);
    const size_t vbytes = decode_mfma_vbytes(D, G);
    uint32_t *knew = reinterpret_cast<uint32_t *>(lds + vbytes / 2);   // [D / 2] bf16 pairs
    uint32_t *vnew = knew + D / 2;
    float *mls = reinterpret_cast<float *>(vnew + D / 2);               // [4][G][2]
    uint4 *qop = reinterpret_cast<uint4 *>(mls + 4 * 8 * 2);            // [D / 16][64]

    const int split = blockIdx.x % a.nsplit, bsh = blockIdx.x / a.nsplit;
    const int sq = bsh / a.Hkv, hk = bsh % a.Hkv;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int p = q_pos[sq];
    const bool valid = p >= 0 && (!a.rope || (int64_t)p < a.rope_rows);
    if (!valid) {
        // the combine kernel flags split outputs itself
        if (a.nsplit == 1)
            for (int idx = tid; idx < G * D; idx += 256)
                Elem<OUT>::store(o, ((int64_t)sq * a.Hq + hk * G) * D + idx, qnan());
        return;
    }
    // the key list: n_sink sinks, then window positions lo .. p; its tiles, and this block's
    // range of them
    const int lo = p - a.w + 1 > 0 ? p - a.w + 1 : 0;
    const int n_sink = a.s < lo ? a.s : lo, n_win = p - lo + 1;
    const int n_st = (n_sink + 31) / 32, n_t = n_st + (n_win + 31) / 32;
    const int per = (n_t + a.nsplit - 1) / a.nsplit;
    const int t_begin = split * per < n_t ? split * per : n_t;
    const int t_end = t_begin + per < n_t ? t_begin + per : n_t;
    const bool owns_new = t_begin <= n_t - 1 && n_t - 1 < t_end;   // the query's own key
    const int64_t ring_base = ((int64_t)sq * a.Hkv + hk) * a.w * D;
    const int64_t sink_base = ((int64_t)sq * a.Hkv + hk) * a.s * D;
    const int half_d = D / 2;

    // ---- the new token (fused append): ring slot and sink entry, and a copy in LDS
    if (APPEND && owns_new && tid < half_d) {
        const int64_t src = ((int64_t)sq * a.Hkv + hk) * D + 2 * tid;
        float k0 = bf16_bits_to_f32(k_new[src]), k1 = bf16_bits_to_f32(k_new[src + 1]);
        const uint32_t vv = *reinterpret_cast<const uint32_t *>(v_new + src);
        if (a.rope) {
            const float2 cs = reinterpret_cast<const float2 *>(a.rope)[(int64_t)p * half_d + tid];
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
        knew[tid] = kk;
        vnew[tid] = vv;
    }

    DecCtx cx;
    cx.row_bytes = 2 * D;
    cx.rk_ring = make_rsrc(a.k_ring + ring_base, (uint32_t)(a.w * D * 2));
    cx.rv_ring = make_rsrc(a.v_ring + ring_base, (uint32_t)(a.w * D * 2));
    cx.rk_sink = make_rsrc(a.s > 0 ? a.k_sink + sink_base : a.k_ring, (uint32_t)(a.s * D * 2));
    cx.rv_sink = make_rsrc(a.s > 0 ? a.v_sink + sink_base : a.v_ring, (uint32_t)(a.s * D * 2));
    cx.w = a.w; cx.slot_lo = lo % a.w; cx.n_sink = n_sink; cx.n_win = n_win; cx.n_st = n_st;
    cx.p = p;
    cx.t_end = t_end;
    cx.lane = lane; cx.col = lane & 31; cx.half = lane >> 5;
    cx.qcol = cx.col < 2 * G; cx.lo_part = cx.col >= G;
    const int g = cx.col & (G - 1);
    cx.slope_l2 = a.slopes ? a.slopes[hk * G + g] * 1.4426950408889634f : 0.0f;

    // ---- this wavefront's tiles, padded to an even count with an empty tile; the first
    // transfers are in flight while the query is formed
    const int first = t_begin + wave;
    const int n_my = first < t_end ? (t_end - first + 3) / 4 : 0;
    const int n_pad = (n_my + 1) & ~1;
    uint16_t *vb0 = lds + wave * 2 * M::TE, *vb1 = vb0 + M::TE;
    bf16x8_t ka[M::KS], kb[M::KS];
    {
        const DecTile t0 = cx.tile(first);   // empty past the range
        dec_load_v<D>(cx, vb0, t0);
        dec_load_k<D>(cx, ka, t0);
    }

    // ---- B operand of the score product, kept in LDS for the four wavefronts: column
    // n = lane % 32, k-slice 8 (lane / 32) of each k-step; rotated at p, times scale log2(e),
    // split into bf16 hi / lo. Wavefront wave forms k-steps wave, wave + 4, ...
    {
        constexpr int KW = (M::KS + 3) / 4;   // k-steps per wavefront
        const uint16_t *qrow = q + ((int64_t)sq * a.Hq + hk * G + g) * D;
        const float4 *trow = a.rope ? reinterpret_cast<const float4 *>(a.rope + (int64_t)p * D) : nullptr;
        uint4 xq[KW];
        float4 t0[KW], t1[KW];
#pragma unroll
        for (int u = 0; u < KW; ++u) {
            const int ks = wave + 4 * u;
            if (ks < M::KS) {
                xq[u] = ldg16(qrow + 16 * ks + 8 * cx.half);
                if (trow) {
                    t0[u] = trow[4 * ks + 2 * cx.half];
                    t1[u] = trow[4 * ks + 2 * cx.half + 1];
                }
            }
        }
#pragma unroll
        for (int u = 0; u < KW; ++u) {
            const int ks = wave + 4 * u;
            if (ks >= M::KS) continue;
            const uint32_t wq[4] = {xq[u].x, xq[u].y, xq[u].z, xq[u].w};
            float x[8];
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                x[2 * m] = bf16_bits_to_f32(wq[m] & 0xffffu);
                x[2 * m + 1] = bf16_bits_to_f32(wq[m] >> 16);
            }
            if (trow) rotate8(x, t0[u], t1[u]);
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                const float v = x[m] * a.cs;
                const float hi = bf16_bits_to_f32(f32_to_bf16_bits(v));
                x[m] = cx.lo_part ? v - hi : v;
            }
            const uint4 pq = make_uint4(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]),
                                        pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7]));
            qop[64 * ks + lane] = cx.qcol ? pq : make_uint4(0, 0, 0, 0);
        }
    }

    f32x16_t oacc[M::DB];
#pragma unroll
    for (int db = 0; db < M::DB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[db][e] = 0.0f;
    float m_run = -1e30f, l_run = 0.0f;
    const int t_new = APPEND && owns_new ? n_t - 1 : -1;
    lds_sync();   // the query operand and the appended token (tile transfers stay in flight)

    for (int i = 0; i < n_pad; i += 2) {
        dec_step<D, G, APPEND>(cx, vb0, vb1, ka, kb, qop, oacc, m_run, l_run, a.mode,
                               first + 4 * i, t_new, knew, vnew);
        dec_step<D, G, APPEND>(cx, vb1, vb0, kb, ka, qop, oacc, m_run, l_run, a.mode,
                               first + 4 * (i + 1), t_new, knew, vnew);
    }

    // ---- merge the four wavefronts: per head g, columns g (hi) and g + G (lo)
    l_run += __shfl_xor(l_run, 32, 64);   // lanes l and l + 32 saw different keys
    __syncthreads();                      // every V tile has been read
    float *red = reinterpret_cast<float *>(lds);   // [4][2G][D]
    if (cx.qcol) {
#pragma unroll
        for (int db = 0; db < M::DB; ++db)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                red[(wave * 2 * G + cx.col) * D + 32 * db + 8 * (e >> 2) + 4 * cx.half + (e & 3)] = oacc[db][e];
    }
    if (cx.col < G && cx.half == 0) {
        mls[(wave * G + cx.col) * 2] = m_run;
        mls[(wave * G + cx.col) * 2 + 1] = l_run;
    }
    __syncthreads();
    float *pp = a.nsplit > 1 ? a.part + (((int64_t)bsh * a.nsplit + split) * G) * (D + 2) : nullptr;
    for (int idx = tid; idx < G * D; idx += 256) {
        const int hg = idx / D, c = idx % D;
        float mx = mls[hg * 2];
#pragma unroll
        for (int wv = 1; wv < 4; ++wv) mx = fmaxf(mx, mls[(wv * G + hg) * 2]);
        float sum = 0.0f, den = 0.0f;
#pragma unroll
        for (int wv = 0; wv < 4; ++wv) {
            const float f = a.mode == 1 ? __builtin_amdgcn_exp2f(mls[(wv * G + hg) * 2] - mx) : 1.0f;
            sum = fmaf(red[(wv * 2 * G + hg) * D + c] + red[(wv * 2 * G + G + hg) * D + c], f, sum);
            den = fmaf(mls[(wv * G + hg) * 2 + 1], f, den);
        }
        if (a.nsplit > 1) {
            pp[hg * (D + 2) + c] = sum;
            if (c == 0) {
                pp[hg * (D + 2) + D] = mx;        // running maximum (base 2)
                pp[hg * (D + 2) + D + 1] = den;   // running sum
            }
        } else {
            if (a.mode == 1) sum /= den;
            Elem<OUT>::store(o, ((int64_t)sq * a.Hq + hk * G + hg) * D + c, sum);
        }
    }
}

template <int D, int G, int OUT, bool APPEND>
hipError_t launch_fast_t(const DecodeFast &f, const void *q, const int32_t *q_pos, void *o,
                         const void *k_new, const void *v_new, hipStream_t st) {
    if (f.w + f.s <= 128) {
        // up to four query heads per block; eight heads per kv head take two blocks, each
        // reading the window for its four heads (splitting four heads over two blocks
        // measured slower: 11.9 against 8.6 us per SWA(64, 4) step)
        constexpr int GB = G < 4 ? G : 4;
        // d = 128 with four heads per block on the matrix cores (its grid is (sequences,
        // kv heads, head parts): y stays within 65535, x times 256 threads within 2^32)
        if (D == 128 && GB == 4 && f.Hkv <= 65535 && f.S <= (1 << 24)) {
            hipLaunchKernelGGL((decode_wmfma_kernel<OUT, APPEND>), dim3((unsigned)f.S, (unsigned)f.Hkv, (unsigned)(G / GB)),
                               dim3(256), 0, st, f, static_cast<const uint16_t *>(q), q_pos, o,
                               static_cast<const uint16_t *>(k_new), static_cast<const uint16_t *>(v_new));
            return hipGetLastError();
        }
        hipLaunchKernelGGL((decode_window_kernel<D, GB, OUT, APPEND, 512>), dim3((unsigned)(f.S * f.Hkv * (G / GB))),
                           dim3(512), 0, st, f, static_cast<const uint16_t *>(q), q_pos, o,
                           static_cast<const uint16_t *>(k_new), static_cast<const uint16_t *>(v_new));
        return hipGetLastError();
    }
    hipLaunchKernelGGL((decode_mfma_kernel<D, G, OUT, APPEND>), dim3((unsigned)(f.S * f.Hkv * f.nsplit)),
                       dim3(256), decode_mfma_lds(D, G), st, f, static_cast<const uint16_t *>(q),
                       q_pos, o, static_cast<const uint16_t *>(k_new), static_cast<const uint16_t *>(v_new));
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
    // whole-window kernel for windows of up to 128 keys; matrix-core kernel beyond
    return c.w + c.s <= 128 ? true : decode_mfma_fits(c.w, c.s, (int)c.d);
}

// Key ranges per (sequence, kv head) for the matrix-core decode: about two blocks per CU in
// total (the kernel's register use allows two), and at least 512 keys per range.
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

// The fast kernels read q, the cache rows, the appended token and the rotation angles with
// 16-byte vector loads and buffer-to-LDS transfers, store the fused append in 4-byte words and
// keep the split partials as float32: every tensor they touch must sit on a 16-byte boundary.
// Calls with a tensor off that boundary take the general kernel (which needs no workspace).
bool decode_fast_aligned(const DecodeArgs &a, const CacheArgs &c, const void *q, const void *o,
                         const void *k_new, const void *v_new, const void *ws) {
    const uintptr_t bits = reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(o) |
                           reinterpret_cast<uintptr_t>(k_new) | reinterpret_cast<uintptr_t>(v_new) |
                           reinterpret_cast<uintptr_t>(c.k_ring) | reinterpret_cast<uintptr_t>(c.v_ring) |
                           reinterpret_cast<uintptr_t>(c.k_sink) | reinterpret_cast<uintptr_t>(c.v_sink) |
                           reinterpret_cast<uintptr_t>(a.rope) |
                           (decode_nsplit(c) > 1 ? reinterpret_cast<uintptr_t>(ws) : 0);
    return (bits & 15) == 0;
}

hipError_t launch_decode(const DecodeArgs &a, const CacheArgs &c, const void *q,
                         const int32_t *q_pos, void *o, void *ws, size_t, hipStream_t st) {
    if (c.S == 0) return hipSuccess;
    if (decode_fast_ok(a, c) && decode_fast_aligned(a, c, q, o, nullptr, nullptr, ws))
        return launch_decode_fast(a, c, q, q_pos, o, nullptr, nullptr, ws, st);
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
    if (decode_fast_ok(a, c) && decode_fast_aligned(a, c, q, o, k_new, v_new, ws))
        return launch_decode_fast(a, c, q, q_pos, o, k_new, v_new, ws, st);
    // general shapes: the append kernel, then the decode kernel, in stream order
    const hipError_t e = launch_kv_append(c, k_new, v_new, q_pos, 1, a.rope, a.rope_rows, st);
    if (e != hipSuccess) return e;
    return launch_decode(a, c, q, q_pos, o, ws, ws_bytes, st);
}

}  // namespace swa
