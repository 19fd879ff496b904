// prefill_mfma.hip - banded matrix-core prefill for bfloat16 inputs, d in {64, 128}.
//
// What it computes (SWAT: Sliding Window Attention Training, "Balanced ALiBi" attention
// equation, "Sigmoid" equation; Sliding Window Attention glossary, band mask; sinks per
// Sliding-window beats linear attention, SWA(w, s)):
//   o_i = sum_{j in K(i)} p(x_ij) v_j,  x_ij = scale (R(i)q_i).(R(j)k_j) + slope_h (i - j),
//   K(i) = { j <= i : i - j < w or j < s },  p = sigmoid (no normalisation) or softmax.
//
// How (gfx950):
//   * One workgroup (4 wavefronts) owns 128 query rows: 128/GP positions x GP query heads
//     that share one kv head (grouped-query packing), so each K/V tile is staged once for
//     the whole group.
//   * It walks only the key tiles that intersect its band [q0 - w + 1, q0 + 127] plus the
//     sink tiles the window no longer covers; every other tile is skipped (the block
//     skipping the glossary describes for windowed exact-attention kernels). Tiles that are
//     fully inside every row's key set skip the element predicate.
//   * Matrix operands are float16: the bf16 inputs are widened, rotated in float32 and
//     rounded once to float16 (11-bit significand), and the weights are rounded to float16
//     (they are at most 2^8). Both products run at the same matrix rate as bf16 and the
//     rounding error is several times smaller. Inputs must stay within the float16 range
//     (|x| < 65504), which attention activations do.
//   * K tiles are rotated on the way into LDS; V tiles are stored transposed in LDS with a
//     key permutation that matches the register layout of the score accumulators, so the
//     probabilities feed the second product straight from registers.
//   * Each wavefront computes S^T = K Q^T (32 keys x 32 queries per v_mfma_f32_32x32x16_f16)
//     so that a lane holds one query's scores; the weights (sigmoid, or an online softmax
//     with lazily rescaled accumulators) are computed on the VALU in the base-2 domain, and
//     O^T += V^T P^T accumulates in float32.
//   * LDS is double-buffered: the next tile's global loads are issued before the current
//     tile's math and written to the other buffer after it.
//   * Workgroups are numbered so that each of the 8 XCDs walks a contiguous run of query
//     tiles of the same (batch, kv head), keeping shared K/V tiles in that XCD's L2.
#include "swa_device.hpp"
#include "swa_kernels.hpp"

namespace swa {
namespace {

constexpr int BK = 64;         // keys per tile
constexpr float LOG2E = 1.4426950408889634f;

template <int D>
struct Tile {
    static constexpr int KSTR = D + 8;             // bf16 per K row in LDS (16 B pad)
    static constexpr int VSTR = BK + 8;            // bf16 per V^T row in LDS (16 B pad)
    static constexpr int K_ELEMS = BK * KSTR;
    static constexpr int V_ELEMS = D * VSTR;
    static constexpr int BUF = K_ELEMS + V_ELEMS;  // one buffer, bf16 elements
    static constexpr int C8 = D / 8;               // 16-byte chunks per row
    static constexpr int K_CHUNKS = BK * C8;       // 512 or 1024
    static constexpr int K_PER_T = K_CHUNKS / 256; // 2 or 4
    static constexpr int V_UNITS = (BK / 4) * C8;  // 4 keys x 8 columns each: 128 or 256
};

struct MfmaParams {
    int64_t B, Hq, Hkv, N, w, s;
    int64_t G;         // query heads per kv head
    int64_t n_qtiles, n_hgroups;
    float cs;          // scale * log2(e)
    const float *slopes;
    const float *rope;
    int out_bf16;
};

// Storage column of key kk inside a V^T row: bits 2 and 3 swapped, which makes the eight
// keys one lane contributes to one P.V step contiguous.
__device__ __forceinline__ int vperm(int kk) {
    return (kk & ~12) | ((kk & 4) << 1) | ((kk & 8) >> 1);
}

// A dword of two bf16 inputs -> two float16 matrix operands, rotated by (c, s) or not.
__device__ __forceinline__ uint32_t rotate_pair(uint32_t w, float c, float s) {
    const float a = bf16_bits_to_f32(w & 0xffffu);
    const float b = bf16_bits_to_f32(w >> 16);
    return pack_f16x2(fmaf(-b, s, a * c), fmaf(a, s, b * c));
}
__device__ __forceinline__ uint32_t to_f16_pair(uint32_t w) {
    return pack_f16x2(bf16_bits_to_f32(w & 0xffffu), bf16_bits_to_f32(w >> 16));
}

// x holds 8 bf16 = 4 rotation pairs; t0, t1 hold (cos, sin) of those 4 pairs.
__device__ __forceinline__ uint4 rotate_chunk(uint4 x, float4 t0, float4 t1) {
    return make_uint4(rotate_pair(x.x, t0.x, t0.y), rotate_pair(x.y, t0.z, t0.w),
                      rotate_pair(x.z, t1.x, t1.y), rotate_pair(x.w, t1.z, t1.w));
}
__device__ __forceinline__ uint4 convert_chunk(uint4 x) {
    return make_uint4(to_f16_pair(x.x), to_f16_pair(x.y), to_f16_pair(x.z), to_f16_pair(x.w));
}

template <int D>
struct Stage {
    uint4 kraw[Tile<D>::K_PER_T];
    float4 kcs[Tile<D>::K_PER_T][2];
    uint4 vraw[4];
};

// Issue the global loads of one K/V tile (rows j0..j0+63 of kv head hkv) into registers.
template <int D>
__device__ __forceinline__ void stage_load(Stage<D> &st, const uint16_t *__restrict__ k,
                                           const uint16_t *__restrict__ v, const MfmaParams &p,
                                           int64_t b, int64_t hkv, int64_t j0, int tid,
                                           bool rope) {
    using T = Tile<D>;
    const uint4 zero = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int r = 0; r < T::K_PER_T; ++r) {
        const int c = tid + 256 * r;
        const int row = c / T::C8, c8 = c % T::C8;
        const int64_t j = j0 + row;
        if (j < p.N) {
            st.kraw[r] = *reinterpret_cast<const uint4 *>(k + ((b * p.N + j) * p.Hkv + hkv) * D + c8 * 8);
            if (rope) {
                const float4 *t = reinterpret_cast<const float4 *>(p.rope + (j * (D / 2) + c8 * 4) * 2);
                st.kcs[r][0] = t[0];
                st.kcs[r][1] = t[1];
            }
        } else {
            st.kraw[r] = zero;
            st.kcs[r][0] = make_float4(1.f, 0.f, 1.f, 0.f);
            st.kcs[r][1] = make_float4(1.f, 0.f, 1.f, 0.f);
        }
    }
    if (tid < T::V_UNITS) {
        const int kq = tid / T::C8, c8 = tid % T::C8;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t j = j0 + 4 * kq + r;
            st.vraw[r] = j < p.N ? *reinterpret_cast<const uint4 *>(v + ((b * p.N + j) * p.Hkv + hkv) * D + c8 * 8)
                                 : zero;
        }
    }
}

// Rotate K and write K (row-major) and V^T (permuted keys) into one LDS buffer.
template <int D>
__device__ __forceinline__ void stage_store(const Stage<D> &st, uint16_t *buf, int tid, bool rope) {
    using T = Tile<D>;
    uint16_t *kl = buf;
    uint16_t *vl = buf + T::K_ELEMS;
#pragma unroll
    for (int r = 0; r < T::K_PER_T; ++r) {
        const int c = tid + 256 * r;
        const int row = c / T::C8, c8 = c % T::C8;
        uint4 x = st.kraw[r];
        x = rope ? rotate_chunk(x, st.kcs[r][0], st.kcs[r][1]) : convert_chunk(x);
        *reinterpret_cast<uint4 *>(kl + row * T::KSTR + c8 * 8) = x;
    }
    if (tid < T::V_UNITS) {
        const int kq = tid / T::C8, c8 = tid % T::C8;
        const int col = vperm(4 * kq);
        const uint32_t v0[4] = {st.vraw[0].x, st.vraw[0].y, st.vraw[0].z, st.vraw[0].w};
        const uint32_t v1[4] = {st.vraw[1].x, st.vraw[1].y, st.vraw[1].z, st.vraw[1].w};
        const uint32_t v2[4] = {st.vraw[2].x, st.vraw[2].y, st.vraw[2].z, st.vraw[2].w};
        const uint32_t v3[4] = {st.vraw[3].x, st.vraw[3].y, st.vraw[3].z, st.vraw[3].w};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            // column 2m takes the low halves, column 2m+1 the high halves, as float16
            const uint2 lo = make_uint2(pack_f16x2(__uint_as_float(v0[m] << 16), __uint_as_float(v1[m] << 16)),
                                        pack_f16x2(__uint_as_float(v2[m] << 16), __uint_as_float(v3[m] << 16)));
            const uint2 hi = make_uint2(pack_f16x2(__uint_as_float(v0[m] & 0xffff0000u), __uint_as_float(v1[m] & 0xffff0000u)),
                                        pack_f16x2(__uint_as_float(v2[m] & 0xffff0000u), __uint_as_float(v3[m] & 0xffff0000u)));
            *reinterpret_cast<uint2 *>(vl + (c8 * 8 + 2 * m) * T::VSTR + col) = lo;
            *reinterpret_cast<uint2 *>(vl + (c8 * 8 + 2 * m + 1) * T::VSTR + col) = hi;
        }
    }
}

template <int D, int GP, int MODE, bool ALIBI>
__global__ __launch_bounds__(256) void prefill_mfma_kernel(MfmaParams p, const uint16_t *__restrict__ q,
                                                           const uint16_t *__restrict__ k,
                                                           const uint16_t *__restrict__ v,
                                                           void *__restrict__ o) {
    using T = Tile<D>;
    constexpr int QP = 128 / GP;  // query positions per workgroup
    constexpr int WPH = 4 / GP;   // wavefronts per query head
    constexpr int KS = D / 16;    // k-steps of the score product
    constexpr int DB = D / 32;    // 32-row blocks of the output
    __shared__ __attribute__((aligned(16))) uint16_t lds[2 * T::BUF];

    // ---- workgroup -> (batch, kv head, head group, query tile), XCD-contiguous
    const int64_t nb = gridDim.x, bid = blockIdx.x;
    const int64_t per = nb / 8, rem = nb % 8, xcd = bid % 8, local = bid / 8;
    const int64_t logical = xcd < rem ? xcd * (per + 1) + local
                                      : rem * (per + 1) + (xcd - rem) * per + local;
    const int64_t qt = logical % p.n_qtiles;
    int64_t rest = logical / p.n_qtiles;
    const int64_t hg = rest % p.n_hgroups;
    rest /= p.n_hgroups;
    const int64_t hkv = rest % p.Hkv;
    const int64_t b = rest / p.Hkv;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int qc = lane & 31, g = lane >> 5;
    const int hp = wave / WPH, pb = wave % WPH;
    const int64_t h = hkv * p.G + hg * GP + hp;
    const int64_t q0 = qt * QP;
    const int64_t qa = q0 + 32 * pb;                 // this wavefront's first query
    const int64_t i = qa + qc;                       // this lane's query
    const int64_t qe = (q0 + QP < p.N ? q0 + QP : p.N) - 1;
    const int64_t qb = (qa + 31 < p.N ? qa + 31 : p.N - 1);
    const bool rope = p.rope != nullptr;

    // ---- this lane's query fragment (B operand of S^T = K Q^T), rotated, bf16
    f16x8_t qreg[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        uint4 x = make_uint4(0, 0, 0, 0);
        if (i < p.N) {
            x = *reinterpret_cast<const uint4 *>(q + ((b * p.N + i) * p.Hq + h) * D + ks * 16 + g * 8);
            if (rope) {
                const float4 *t = reinterpret_cast<const float4 *>(p.rope + (i * (D / 2) + ks * 8 + g * 4) * 2);
                x = rotate_chunk(x, t[0], t[1]);
            } else {
                x = convert_chunk(x);
            }
        }
        qreg[ks] = __builtin_bit_cast(f16x8_t, x);
    }
    const float slope_l2 = ALIBI ? p.slopes[h] * LOG2E : 0.0f;

    // ---- band of key tiles: sink tiles the window no longer covers, then the window
    const int64_t lo_wg = q0 - p.w + 1 > 0 ? q0 - p.w + 1 : 0;
    const int64_t tw_begin = lo_wg / BK, tw_end = qe / BK;
    const int64_t n_sink_keys = p.s < lo_wg ? p.s : lo_wg;
    int64_t ts_end = (n_sink_keys + BK - 1) / BK;
    if (ts_end > tw_begin) ts_end = tw_begin;
    const int64_t n_tiles = ts_end + (tw_end - tw_begin + 1);

    f32x16_t oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[db][e] = 0.0f;
    float m_run = -1e30f, l_run = 0.0f;

    Stage<D> st;
    stage_load<D>(st, k, v, p, b, hkv, (ts_end > 0 ? 0 : tw_begin) * BK, tid, rope);
    stage_store<D>(st, lds, tid, rope);
    __syncthreads();

    for (int64_t it = 0; it < n_tiles; ++it) {
        const int64_t j0 = (it < ts_end ? it : tw_begin + (it - ts_end)) * BK;
        if (it + 1 < n_tiles) {
            const int64_t jn = (it + 1 < ts_end ? it + 1 : tw_begin + (it + 1 - ts_end)) * BK;
            stage_load<D>(st, k, v, p, b, hkv, jn, tid, rope);
        }
        const uint16_t *kl = lds + (it & 1) * T::BUF;
        const uint16_t *vl = kl + T::K_ELEMS;

        // classify this tile for the wavefront's queries [qa, qb]
        const bool active = qa < p.N;
        const bool any_sink = j0 < p.s;
        const bool empty = !active || j0 > qb || (qa - (j0 + BK - 1) >= p.w && !any_sink);
        const bool full = (j0 + BK - 1 <= qa) && (qb - j0 < p.w || j0 + BK - 1 < p.s);

        if (!empty) {
            f32x16_t sacc[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                for (int e = 0; e < 16; ++e) sacc[kb][e] = 0.0f;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const f16x8_t a = *reinterpret_cast<const f16x8_t *>(kl + (kb * 32 + qc) * T::KSTR + ks * 16 + g * 8);
                    sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, qreg[ks], sacc[kb], 0, 0, 0);
                }
            }
            // scores -> base-2 logits. Element (kb, e) of this lane is key
            // j0 + 4g + kb*32 + 8(e/4) + (e%4) for query i.
            const int dq = (int)(i - j0) - 4 * g;  // i - (j0 + 4g)
            const float base = slope_l2 * (float)dq;
            float x[2][16];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int ce = kb * 32 + 8 * (e >> 2) + (e & 3);
                    float xv = ALIBI ? fmaf(sacc[kb][e], p.cs, fmaf(-slope_l2, (float)ce, base))
                                     : sacc[kb][e] * p.cs;
                    if (!full) {
                        const int dij = dq - ce;                      // i - j
                        const int64_t j = j0 + 4 * g + ce;
                        const bool ok = dij >= 0 && (dij < p.w || j < p.s);
                        if (!ok) xv = -INFINITY;  // weight 0 in both modes
                    }
                    x[kb][e] = xv;
                }
            float pr[2][16];
            if (MODE == 0) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        // sigma(x) = 1 / (1 + e^-x) = 1 / (1 + 2^(-x log2 e)); x = -inf -> 0
                        const float t = __builtin_amdgcn_exp2f(-x[kb][e]);
                        pr[kb][e] = __builtin_amdgcn_rcpf(1.0f + t);
                    }
            } else {
                float mt = -INFINITY;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int e = 0; e < 16; ++e) mt = fmaxf(mt, x[kb][e]);
                mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
                const float m_new = fmaxf(m_run, mt);
                // lazy rescale: keep the stale maximum while the new one exceeds it by less
                // than 8 (weights stay below 2^8); the final division uses the same maximum.
                const bool need = m_new > m_run + 8.0f;
                if (__any(need)) {
                    const float corr = need ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
#pragma unroll
                    for (int db = 0; db < DB; ++db)
#pragma unroll
                        for (int e = 0; e < 16; ++e) oacc[db][e] *= corr;
                    l_run *= corr;
                    m_run = need ? m_new : m_run;
                }
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        pr[kb][e] = __builtin_amdgcn_exp2f(x[kb][e] - m_run);
                        l_run += pr[kb][e];
                    }
            }
            // P^T fragments: step t uses this lane's elements (t/2, 8(t%2) + 0..7)
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int kb = t >> 1, e0 = 8 * (t & 1);
                uint4 pk;
                pk.x = pack_f16x2(pr[kb][e0 + 0], pr[kb][e0 + 1]);
                pk.y = pack_f16x2(pr[kb][e0 + 2], pr[kb][e0 + 3]);
                pk.z = pack_f16x2(pr[kb][e0 + 4], pr[kb][e0 + 5]);
                pk.w = pack_f16x2(pr[kb][e0 + 6], pr[kb][e0 + 7]);
                const f16x8_t bp = __builtin_bit_cast(f16x8_t, pk);
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const f16x8_t a = *reinterpret_cast<const f16x8_t *>(vl + (db * 32 + qc) * T::VSTR + 16 * t + 8 * g);
                    oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, bp, oacc[db], 0, 0, 0);
                }
            }
        }
        if (it + 1 < n_tiles) stage_store<D>(st, lds + ((it + 1) & 1) * T::BUF, tid, rope);
        __syncthreads();
    }

    // ---- epilogue: lane holds query i, rows 32 db + 8 r + 4 g + (0..3) of the output
    // the two lanes of a query hold disjoint halves of its row sum
    const float l_tot = MODE == 1 ? l_run + __shfl_xor(l_run, 32, 64) : 1.0f;
    if (i < p.N) {
        const float inv = MODE == 1 ? 1.0f / l_tot : 1.0f;
        const int64_t obase = ((b * p.N + i) * p.Hq + h) * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int d0 = 32 * db + 8 * r + 4 * g;
                const float a0 = oacc[db][4 * r] * inv, a1 = oacc[db][4 * r + 1] * inv;
                const float a2 = oacc[db][4 * r + 2] * inv, a3 = oacc[db][4 * r + 3] * inv;
                if (p.out_bf16) {
                    *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(o) + obase + d0) =
                        make_uint2(pack_bf16x2(a0, a1), pack_bf16x2(a2, a3));
                } else {
                    *reinterpret_cast<float4 *>(static_cast<float *>(o) + obase + d0) =
                        make_float4(a0, a1, a2, a3);
                }
            }
    }
}

template <int D, int GP, int MODE, bool ALIBI>
hipError_t launch_t(const MfmaParams &mp, int64_t nblocks, const void *q, const void *k,
                    const void *v, void *o, hipStream_t st) {
    hipLaunchKernelGGL((prefill_mfma_kernel<D, GP, MODE, ALIBI>), dim3((unsigned)nblocks),
                       dim3(256), 0, st, mp, static_cast<const uint16_t *>(q),
                       static_cast<const uint16_t *>(k), static_cast<const uint16_t *>(v), o);
    return hipGetLastError();
}

template <int D, int GP>
hipError_t launch_d(const MfmaParams &mp, int64_t nb, int mode, bool alibi, const void *q,
                    const void *k, const void *v, void *o, hipStream_t st) {
    if (mode == 0)
        return alibi ? launch_t<D, GP, 0, true>(mp, nb, q, k, v, o, st)
                     : launch_t<D, GP, 0, false>(mp, nb, q, k, v, o, st);
    return alibi ? launch_t<D, GP, 1, true>(mp, nb, q, k, v, o, st)
                 : launch_t<D, GP, 1, false>(mp, nb, q, k, v, o, st);
}

int pack_of(int64_t G) { return G % 4 == 0 ? 4 : (G % 2 == 0 ? 2 : 1); }

}  // namespace

bool prefill_mfma_supported(const PrefillArgs &a) {
    if (a.in_dt != 1 || (a.d != 64 && a.d != 128)) return false;
    if (a.B * a.N == 0) return true;
    const int64_t G = a.Hq / a.Hkv;
    const int GP = pack_of(G);
    const int64_t nb = a.B * a.Hkv * (G / GP) * ((a.N + 128 / GP - 1) / (128 / GP));
    return nb <= 0x7fffffff && a.N < (int64_t(1) << 24);
}

hipError_t launch_prefill_mfma(const PrefillArgs &a, const void *q, const void *k,
                               const void *v, void *o, hipStream_t st) {
    if (a.B * a.N == 0) return hipSuccess;
    const int64_t G = a.Hq / a.Hkv;
    const int GP = pack_of(G);
    const int64_t QP = 128 / GP;
    MfmaParams mp;
    mp.B = a.B; mp.Hq = a.Hq; mp.Hkv = a.Hkv; mp.N = a.N; mp.w = a.w; mp.s = a.s;
    mp.G = G;
    mp.n_qtiles = (a.N + QP - 1) / QP;
    mp.n_hgroups = G / GP;
    mp.cs = a.scale * LOG2E;
    mp.slopes = a.slopes;
    mp.rope = a.rope;
    mp.out_bf16 = a.out_dt == 1;
    const int64_t nb = a.B * a.Hkv * mp.n_hgroups * mp.n_qtiles;
    const bool alibi = a.slopes != nullptr;
    if (a.d == 64) {
        if (GP == 4) return launch_d<64, 4>(mp, nb, a.mode, alibi, q, k, v, o, st);
        if (GP == 2) return launch_d<64, 2>(mp, nb, a.mode, alibi, q, k, v, o, st);
        return launch_d<64, 1>(mp, nb, a.mode, alibi, q, k, v, o, st);
    }
    if (GP == 4) return launch_d<128, 4>(mp, nb, a.mode, alibi, q, k, v, o, st);
    if (GP == 2) return launch_d<128, 2>(mp, nb, a.mode, alibi, q, k, v, o, st);
    return launch_d<128, 1>(mp, nb, a.mode, alibi, q, k, v, o, st);
}

}  // namespace swa
