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
//     skipping the glossary describes for windowed exact-attention kernels). Tiles inside
//     every row's key set run without the element predicate.
//   * Matrix operands are float16: the bf16 inputs are widened, rotated in float32 and
//     rounded once to float16 (11-bit significand), and the weights are rounded to float16
//     (they are at most 2^8). Both products run at the same matrix rate as bf16 and the
//     rounding error is several times smaller. Inputs must stay within the float16 range
//     (|x| < 65504), which attention activations do.
//   * K tiles are rotated on the way into LDS; V tiles are stored transposed in LDS with a
//     key permutation that matches the register layout of the score accumulators, so the
//     weights feed the second product straight from registers.
//   * Each wavefront computes S^T = K Q^T (32 keys x 32 queries per v_mfma_f32_32x32x16_f16)
//     so that a lane holds one query's scores. The scale and the ALiBi bias fold into two
//     FMAs per score in base-2 units. Weights are computed in base 2: sigmoid as 1/(1 + 2^t), softmax online with lazily
//     rescaled accumulators. O^T += V^T P^T accumulates in float32.
//   * K/V tiles are fetched with buffer loads whose range check returns zeros past the
//     sequence end; LDS is double-buffered with the next tile's loads issued before the
//     current tile's math.
//   * The output goes through LDS so that every global store writes whole rows.
//   * Workgroups are numbered so that each of the 8 XCDs walks a contiguous run of query
//     tiles of the same (batch, kv head), keeping shared K/V tiles in that XCD's L2.
#include "swa_device.hpp"
#include "swa_kernels.hpp"

namespace swa {
namespace {

constexpr int BK = 64;  // keys per tile
constexpr float LOG2E = 1.4426950408889634f;
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

template <int D>
struct Tile {
    static constexpr int KSTR = D + 8;             // f16 per K row in LDS (16 B pad)
    static constexpr int VSTR = BK + 8;            // f16 per V^T row in LDS (16 B pad)
    static constexpr int K_ELEMS = BK * KSTR;
    static constexpr int V_ELEMS = D * VSTR;
    static constexpr int BUF = K_ELEMS + V_ELEMS;  // one buffer, 16-bit elements
    static constexpr int C8 = D / 8;               // 16-byte chunks per row
    static constexpr int K_PER_T = BK * C8 / 256;  // K chunks per thread: 2 or 4
    static constexpr int KPU = BK * C8 / 256;      // keys per V unit (one unit per thread)
    static constexpr int KG = BK / KPU;            // key groups per tile: 32 or 16
    static constexpr int OSTR = D + 4;             // floats per output row staged in LDS
};

struct MfmaParams {
    const uint16_t *q, *k, *v;
    void *o;
    const float *slopes;
    const float *rope;
    int64_t N, Hq, Hkv, G;
    int n_qtiles, n_hgroups;
    int w, s;                 // clamped to N
    float cs;                 // scale * log2(e)
    uint32_t kv_bytes;        // bytes of one (batch, kv head) K or V slice, rows [0, N)
    uint32_t row_bytes;       // bytes between consecutive positions of K/V
    uint32_t rope_bytes;      // bytes of the rotation table
    int out_bf16;
};

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

// Storage column of key kk inside a V^T row: bits 2 and 3 swapped, which makes the eight
// keys one lane contributes to one P.V step contiguous.
__device__ __forceinline__ int vperm(int kk) {
    return (kk & ~12) | ((kk & 4) << 1) | ((kk & 8) >> 1);
}

// A dword of two bf16 inputs -> two float16 matrix operands, rotated by (c, s) or not.
__device__ __forceinline__ uint32_t rotate_pair(uint32_t w, float c, float s) {
    const float a = __uint_as_float(w << 16);
    const float b = __uint_as_float(w & 0xffff0000u);
    return pack_f16x2(fmaf(-b, s, a * c), fmaf(a, s, b * c));
}
__device__ __forceinline__ uint32_t to_f16_pair(uint32_t w) {
    return pack_f16x2(__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u));
}
__device__ __forceinline__ uint4 rotate_chunk(uint4 x, float4 t0, float4 t1) {
    return make_uint4(rotate_pair(x.x, t0.x, t0.y), rotate_pair(x.y, t0.z, t0.w),
                      rotate_pair(x.z, t1.x, t1.y), rotate_pair(x.w, t1.z, t1.w));
}
__device__ __forceinline__ uint4 convert_chunk(uint4 x) {
    return make_uint4(to_f16_pair(x.x), to_f16_pair(x.y), to_f16_pair(x.z), to_f16_pair(x.w));
}

template <int D>
struct Stage {
    uint4 k[Tile<D>::K_PER_T];
    float4 kcs[Tile<D>::K_PER_T][2];
    uint4 v[Tile<D>::KPU];
};

struct Rsrc {
    __amdgpu_buffer_rsrc_t k, v, t;
};

// Global -> registers for the tile of keys j0..j0+63 (rows past the end read as zero).
template <int D>
__device__ __forceinline__ void stage_load(Stage<D> &st, const Rsrc &rs, uint32_t row_bytes,
                                           int j0, int tid, bool rope) {
    using T = Tile<D>;
#pragma unroll
    for (int r = 0; r < T::K_PER_T; ++r) {
        const int c = tid + 256 * r;
        const int j = j0 + c / T::C8, c8 = c % T::C8;
        st.k[r] = buf_load16(rs.k, (uint32_t)j * row_bytes + c8 * 16);
        if (rope) {
            const uint32_t toff = ((uint32_t)j * (D / 2) + c8 * 4) * 8;
            st.kcs[r][0] = buf_load16f(rs.t, toff);
            st.kcs[r][1] = buf_load16f(rs.t, toff + 16);
        }
    }
    const int kg = tid % T::KG, c8 = tid / T::KG;
#pragma unroll
    for (int r = 0; r < T::KPU; ++r)
        st.v[r] = buf_load16(rs.v, (uint32_t)(j0 + kg * T::KPU + r) * row_bytes + c8 * 16);
}

__device__ __forceinline__ uint32_t dword_of(const uint4 &x, int m) {
    return m == 0 ? x.x : m == 1 ? x.y : m == 2 ? x.z : x.w;
}

// Registers -> LDS: K rotated (or converted) row-major, V converted and transposed.
template <int D>
__device__ __forceinline__ void stage_store(const Stage<D> &st, uint16_t *buf, int tid, bool rope) {
    using T = Tile<D>;
    uint16_t *kl = buf;
    uint16_t *vl = buf + T::K_ELEMS;
#pragma unroll
    for (int r = 0; r < T::K_PER_T; ++r) {
        const int c = tid + 256 * r;
        const int row = c / T::C8, c8 = c % T::C8;
        const uint4 x = rope ? rotate_chunk(st.k[r], st.kcs[r][0], st.kcs[r][1]) : convert_chunk(st.k[r]);
        *reinterpret_cast<uint4 *>(kl + row * T::KSTR + c8 * 8) = x;
    }
    const int kg = tid % T::KG, c8 = tid / T::KG;
    const int col = vperm(kg * T::KPU);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        // element 2m (low half) and 2m+1 (high half) of each key, as float32
        float lo[T::KPU], hi[T::KPU];
#pragma unroll
        for (int r = 0; r < T::KPU; ++r) {
            const uint32_t w = dword_of(st.v[r], m);
            lo[r] = __uint_as_float(w << 16);
            hi[r] = __uint_as_float(w & 0xffff0000u);
        }
        uint16_t *row_lo = vl + (c8 * 8 + 2 * m) * T::VSTR + col;
        uint16_t *row_hi = row_lo + T::VSTR;
        if constexpr (T::KPU == 2) {
            *reinterpret_cast<uint32_t *>(row_lo) = pack_f16x2(lo[0], lo[1]);
            *reinterpret_cast<uint32_t *>(row_hi) = pack_f16x2(hi[0], hi[1]);
        } else {
            *reinterpret_cast<uint2 *>(row_lo) = make_uint2(pack_f16x2(lo[0], lo[1]), pack_f16x2(lo[2], lo[3]));
            *reinterpret_cast<uint2 *>(row_hi) = make_uint2(pack_f16x2(hi[0], hi[1]), pack_f16x2(hi[2], hi[3]));
        }
    }
}

// Key offset (from j0 + 4g) of accumulator element e of score block kb.
__device__ __forceinline__ constexpr int key_of(int kb, int e) {
    return kb * 32 + 8 * (e >> 2) + (e & 3);
}

// Exclude the keys of an edge tile that are outside the key set: their logits become -inf
// (weight 0 in both modes). Element (kb, e) is key j = jb + key_of(kb, e) with
// i - j = dq - key_of(kb, e). SINKS adds the keys j < s at or before the query.
template <bool SINKS>
__device__ __forceinline__ void mask_tile(f32x16_t (&sacc)[2], int dq, int jb, int w, int s) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int dij = dq - key_of(kb, e);
            bool ok = (unsigned)dij < (unsigned)w;   // 0 <= i - j < w
            if (SINKS) ok = ok | ((dij >= 0) & (jb + key_of(kb, e) < s));
            sacc[kb][e] = ok ? sacc[kb][e] : -INFINITY;
        }
}

// One 64-key tile for one wavefront: S^T = K Q^T, weights, O^T += V^T P^T.
// kind: 0 = every pair in the key set, 1 = cut by the window edges, 2 = also holds sinks.
template <int D, int MODE, bool ALIBI>
__device__ __forceinline__ void tile_math(const uint16_t *kl, const uint16_t *vl,
                                          const f16x8_t (&qreg)[D / 16], f32x16_t (&oacc)[D / 32],
                                          float &m_run, float &l_run, float cs, float slope_l2,
                                          int kind, int dq, int jb, int w, int s, int qc, int g) {
    using T = Tile<D>;
    constexpr int KS = D / 16, DB = D / 32;
    f32x16_t sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        const f16x8_t a0 = *reinterpret_cast<const f16x8_t *>(kl + (kb * 32 + qc) * T::KSTR + g * 8);
        const f32x16_t zero = {};
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0, qreg[0], zero, 0, 0, 0);
#pragma unroll
        for (int ks = 1; ks < KS; ++ks) {
            const f16x8_t a = *reinterpret_cast<const f16x8_t *>(kl + (kb * 32 + qc) * T::KSTR + ks * 16 + g * 8);
            sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, qreg[ks], sacc[kb], 0, 0, 0);
        }
    }
    if (kind == 1) mask_tile<false>(sacc, dq, jb, w, s);
    else if (kind == 2) mask_tile<true>(sacc, dq, jb, w, s);

    const float bias0 = slope_l2 * (float)dq;  // slope log2(e) (i - j) for key_of = 0
    if (MODE == 0) {
        // sigma(x) = 1 / (1 + 2^t) with t = -x log2(e); an excluded key has t = +inf -> 0
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                // -x log2(e) = -(cs * score + slope log2(e) (i - j)), i - j = dq - key_of
                const float nb = ALIBI ? fmaf(slope_l2, (float)key_of(kb, e), -bias0) : 0.0f;
                const float t = fmaf(sacc[kb][e], -cs, nb);
                sacc[kb][e] = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(t));
            }
    } else {
        // base-2 logits x = cs * score + slope log2(e) (i - j); excluded keys stay -inf
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                sacc[kb][e] = ALIBI ? fmaf(sacc[kb][e], cs, fmaf(-slope_l2, (float)key_of(kb, e), bias0))
                                    : sacc[kb][e] * cs;
        float mx[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
            mx[u] = fmaxf(fmaxf(sacc[0][4 * u], sacc[0][4 * u + 1]), fmaxf(sacc[0][4 * u + 2], sacc[0][4 * u + 3]));
#pragma unroll
        for (int u = 0; u < 4; ++u)
            mx[u] = fmaxf(mx[u], fmaxf(fmaxf(sacc[1][4 * u], sacc[1][4 * u + 1]), fmaxf(sacc[1][4 * u + 2], sacc[1][4 * u + 3])));
        float mt = fmaxf(fmaxf(mx[0], mx[1]), fmaxf(mx[2], mx[3]));
        mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
        const float m_new = fmaxf(m_run, mt);
        // lazy rescale: keep the stale maximum while the new one exceeds it by less than 8
        // (weights stay below 2^8); the final division uses the same maximum.
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
        float ls[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const float pe = __builtin_amdgcn_exp2f(sacc[kb][e] - m_run);
                ls[e & 3] += pe;
                sacc[kb][e] = pe;
            }
        l_run += (ls[0] + ls[1]) + (ls[2] + ls[3]);
    }
    // O^T += V^T P^T; P^T step t uses this lane's elements (t/2, 8(t%2) + 0..7)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int kb = t >> 1, e0 = 8 * (t & 1);
        uint4 pk;
        pk.x = pack_f16x2(sacc[kb][e0 + 0], sacc[kb][e0 + 1]);
        pk.y = pack_f16x2(sacc[kb][e0 + 2], sacc[kb][e0 + 3]);
        pk.z = pack_f16x2(sacc[kb][e0 + 4], sacc[kb][e0 + 5]);
        pk.w = pack_f16x2(sacc[kb][e0 + 6], sacc[kb][e0 + 7]);
        const f16x8_t bp = __builtin_bit_cast(f16x8_t, pk);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const f16x8_t a = *reinterpret_cast<const f16x8_t *>(vl + (db * 32 + qc) * T::VSTR + 16 * t + 8 * g);
            oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, bp, oacc[db], 0, 0, 0);
        }
    }
}

// Register budget: 3 wavefronts per SIMD at d = 64, 2 at d = 128 (the LDS double buffer
// allows 4 and 2 workgroups per CU respectively).
template <int D, int GP, int MODE, bool ALIBI>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(D == 64 ? 3 : 2)))
void prefill_mfma_kernel(MfmaParams p) {
    using T = Tile<D>;
    constexpr int QP = 128 / GP;  // query positions per workgroup
    constexpr int WPH = 4 / GP;   // wavefronts per query head
    constexpr int KS = D / 16;    // k-steps of the score product
    constexpr int DB = D / 32;    // 32-row blocks of the output
    __shared__ __attribute__((aligned(16))) uint16_t lds[2 * T::BUF];

    // ---- workgroup -> (batch, kv head, head group, query tile), XCD-contiguous
    const int nb = gridDim.x, bid = blockIdx.x;
    const int per = nb / 8, rem = nb % 8, xcd = bid % 8, local = bid / 8;
    const int logical = xcd < rem ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
    const int qt = logical % p.n_qtiles;
    int rest = logical / p.n_qtiles;
    const int hg = rest % p.n_hgroups;
    rest /= p.n_hgroups;
    const int hkv = rest % (int)p.Hkv;
    const int b = rest / (int)p.Hkv;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int qc = lane & 31, g = lane >> 5;
    const int hp = wave / WPH, pb = wave % WPH;
    const int64_t h = (int64_t)hkv * p.G + hg * GP + hp;
    const int N = (int)p.N;
    const int q0 = qt * QP;
    const int qa = q0 + 32 * pb;                   // this wavefront's first query
    const int i = qa + qc;                         // this lane's query
    const int qe = (q0 + QP < N ? q0 + QP : N) - 1;
    const int qb = (qa + 31 < N ? qa + 31 : N - 1);
    const bool rope = p.rope != nullptr;

    Rsrc rs;
    const int64_t kvoff = ((int64_t)b * p.N * p.Hkv + hkv) * D;
    rs.k = make_rsrc(p.k + kvoff, p.kv_bytes);
    rs.v = make_rsrc(p.v + kvoff, p.kv_bytes);
    rs.t = make_rsrc(p.rope, rope ? p.rope_bytes : 0);

    // ---- this lane's query fragment (B operand of S^T = K Q^T): rotated, float16
    f16x8_t qreg[KS];
    {
        const uint16_t *qrow = p.q + (((int64_t)b * p.N + i) * p.Hq + h) * D;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            uint4 x = make_uint4(0, 0, 0, 0);
            if (i < N) {
                x = *reinterpret_cast<const uint4 *>(qrow + ks * 16 + g * 8);
                if (rope) {
                    const float4 *t = reinterpret_cast<const float4 *>(p.rope + ((int64_t)i * (D / 2) + ks * 8 + g * 4) * 2);
                    x = rotate_chunk(x, t[0], t[1]);
                } else {
                    x = convert_chunk(x);
                }
            }
            qreg[ks] = __builtin_bit_cast(f16x8_t, x);
        }
    }

    const float slope_l2 = ALIBI ? p.slopes[h] * LOG2E : 0.0f;  // bias in base-2 units

    // ---- band of key tiles: sink tiles the window no longer covers, then the window
    const int lo_wg = q0 - p.w + 1 > 0 ? q0 - p.w + 1 : 0;
    const int tw_begin = lo_wg / BK, tw_end = qe / BK;
    const int n_sink_keys = p.s < lo_wg ? p.s : lo_wg;
    int ts_end = (n_sink_keys + BK - 1) / BK;
    if (ts_end > tw_begin) ts_end = tw_begin;
    const int n_tiles = ts_end + (tw_end - tw_begin + 1);

    f32x16_t oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[db][e] = 0.0f;
    float m_run = -1e30f, l_run = 0.0f;
    const float cs = p.cs;

    Stage<D> st;
    stage_load<D>(st, rs, p.row_bytes, (ts_end > 0 ? 0 : tw_begin) * BK, tid, rope);
    stage_store<D>(st, lds, tid, rope);
    __syncthreads();

    for (int it = 0; it < n_tiles; ++it) {
        const int j0 = (it < ts_end ? it : tw_begin + (it - ts_end)) * BK;
        if (it + 1 < n_tiles) {
            const int jn = (it + 1 < ts_end ? it + 1 : tw_begin + (it + 1 - ts_end)) * BK;
            stage_load<D>(st, rs, p.row_bytes, jn, tid, rope);
        }
        const uint16_t *kl = lds + (it & 1) * T::BUF;
        const uint16_t *vl = kl + T::K_ELEMS;

        // classify the tile for this wavefront's queries [qa, qb] (wave-uniform)
        const bool empty = qa >= N || j0 > qb || (qa - (j0 + BK - 1) >= p.w && j0 >= p.s);
        const bool full = (j0 + BK - 1 <= qa) && (qb - j0 < p.w || j0 + BK - 1 < p.s);

        if (!empty) {
            const int dq = i - j0 - 4 * g;   // element (kb, e) has i - j = dq - key_of(kb, e)
            const int jb = j0 + 4 * g;       // and key j = jb + key_of(kb, e)
            const int kind = full ? 0 : (j0 >= p.s ? 1 : 2);
            tile_math<D, MODE, ALIBI>(kl, vl, qreg, oacc, m_run, l_run, cs, slope_l2, kind, dq,
                                      jb, p.w, p.s, qc, g);
        }
        if (it + 1 < n_tiles) stage_store<D>(st, lds + ((it + 1) & 1) * T::BUF, tid, rope);
        __syncthreads();
    }

    // ---- epilogue: normalise, stage O row-major in LDS, store whole rows
    const float l_tot = MODE == 1 ? l_run + __shfl_xor(l_run, 32, 64) : 1.0f;
    const float inv = MODE == 1 ? 1.0f / l_tot : 1.0f;
    float *ol = reinterpret_cast<float *>(lds) + wave * (32 * T::OSTR);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int d0 = 32 * db + 8 * r + 4 * g;
            *reinterpret_cast<float4 *>(ol + qc * T::OSTR + d0) =
                make_float4(oacc[db][4 * r] * inv, oacc[db][4 * r + 1] * inv,
                            oacc[db][4 * r + 2] * inv, oacc[db][4 * r + 3] * inv);
        }
    __syncthreads();
    constexpr int C4 = D / 4;  // 4-float chunks per row
#pragma unroll
    for (int rr = 0; rr < 32 * C4 / 64; ++rr) {
        const int ch = lane + 64 * rr;
        const int qrow = ch / C4, c4 = ch % C4;
        const int iq = qa + qrow;
        if (iq < N) {
            const float4 x = *reinterpret_cast<const float4 *>(ol + qrow * T::OSTR + 4 * c4);
            const int64_t off = (((int64_t)b * p.N + iq) * p.Hq + h) * D + 4 * c4;
            if (p.out_bf16)
                *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(p.o) + off) =
                    make_uint2(pack_bf16x2(x.x, x.y), pack_bf16x2(x.z, x.w));
            else
                *reinterpret_cast<float4 *>(static_cast<float *>(p.o) + off) = x;
        }
    }
}

template <int D, int GP, int MODE, bool ALIBI>
hipError_t launch_t(const MfmaParams &mp, int nblocks, hipStream_t st) {
    hipLaunchKernelGGL((prefill_mfma_kernel<D, GP, MODE, ALIBI>), dim3((unsigned)nblocks),
                       dim3(256), 0, st, mp);
    return hipGetLastError();
}

template <int D, int GP>
hipError_t launch_d(const MfmaParams &mp, int nb, int mode, bool alibi, hipStream_t st) {
    if (mode == 0)
        return alibi ? launch_t<D, GP, 0, true>(mp, nb, st) : launch_t<D, GP, 0, false>(mp, nb, st);
    return alibi ? launch_t<D, GP, 1, true>(mp, nb, st) : launch_t<D, GP, 1, false>(mp, nb, st);
}

int pack_of(int64_t G) { return G % 4 == 0 ? 4 : (G % 2 == 0 ? 2 : 1); }

}  // namespace

bool prefill_mfma_supported(const PrefillArgs &a) {
    if (a.in_dt != 1 || (a.d != 64 && a.d != 128)) return false;
    if (a.B * a.N == 0) return true;
    const int64_t G = a.Hq / a.Hkv;
    const int GP = pack_of(G);
    const int64_t nb = a.B * a.Hkv * (G / GP) * ((a.N + 128 / GP - 1) / (128 / GP));
    // 32-bit block ids and buffer offsets: one K/V slice and the table stay below 2 GiB
    const int64_t slice = (a.N * a.Hkv) * a.d * 2;
    const int64_t table = a.rope ? a.rope_rows * a.d * 4 : 0;
    return nb <= 0x7fffffff && slice < (int64_t(1) << 31) && table < (int64_t(1) << 31) &&
           a.N < (int64_t(1) << 24);
}

hipError_t launch_prefill_mfma(const PrefillArgs &a, const void *q, const void *k,
                               const void *v, void *o, hipStream_t st) {
    if (a.B * a.N == 0) return hipSuccess;
    const int64_t G = a.Hq / a.Hkv;
    const int GP = pack_of(G);
    const int64_t QP = 128 / GP;
    MfmaParams mp;
    mp.q = static_cast<const uint16_t *>(q);
    mp.k = static_cast<const uint16_t *>(k);
    mp.v = static_cast<const uint16_t *>(v);
    mp.o = o;
    mp.slopes = a.slopes;
    mp.rope = a.rope;
    mp.N = a.N; mp.Hq = a.Hq; mp.Hkv = a.Hkv; mp.G = G;
    mp.n_qtiles = (int)((a.N + QP - 1) / QP);
    mp.n_hgroups = (int)(G / GP);
    mp.w = (int)(a.w < a.N ? a.w : a.N);
    mp.s = (int)(a.s < a.N ? a.s : a.N);
    mp.cs = a.scale * LOG2E;
    mp.kv_bytes = (uint32_t)(((a.N - 1) * a.Hkv + 1) * a.d * 2);
    mp.row_bytes = (uint32_t)(a.Hkv * a.d * 2);
    mp.rope_bytes = (uint32_t)(a.rope ? a.rope_rows * a.d * 4 : 0);
    mp.out_bf16 = a.out_dt == 1;
    const int nb = (int)(a.B * a.Hkv * mp.n_hgroups * mp.n_qtiles);
    const bool alibi = a.slopes != nullptr;
    if (a.d == 64) {
        if (GP == 4) return launch_d<64, 4>(mp, nb, a.mode, alibi, st);
        if (GP == 2) return launch_d<64, 2>(mp, nb, a.mode, alibi, st);
        return launch_d<64, 1>(mp, nb, a.mode, alibi, st);
    }
    if (GP == 4) return launch_d<128, 4>(mp, nb, a.mode, alibi, st);
    if (GP == 2) return launch_d<128, 2>(mp, nb, a.mode, alibi, st);
    return launch_d<128, 1>(mp, nb, a.mode, alibi, st);
}

}  // namespace swa
