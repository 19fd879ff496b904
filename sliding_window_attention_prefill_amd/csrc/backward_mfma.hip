// backward_mfma.hip - gradients of the banded matrix-core prefill (bfloat16 inputs, d in
// {64, 128}).
//
// What it computes (SWAT: Sliding Window Attention Training, "Putting It Together" attention
// equation, differentiated; "Sigmoid: Dense Attention Without Suppression" for the weights):
// for j in K(i), with p_ij the forward weights and x_ij the logits,
//   dP_ij = dout_i . v_j
//   dX_ij = dP_ij p_ij (1 - p_ij)                (sigmoid: the logistic derivative)
//         = p_ij (dP_ij - dout_i . o_i)          (softmax: the row Jacobian)
//   dv_j = sum_i p_ij dout_i,  dq~_i = scale sum_j dX_ij k~_j,  dk~_j = scale sum_i dX_ij q~_i
// with q~ = R(i) q, k~ = R(j) k; dq = R(i)^T dq~ and dk = R(j)^T dk~ (R is orthogonal).
// Key and value gradients sum over the query heads of their group.
//
// How (gfx950):
//   * Pre-passes write float16 tile images of the rotated keys and queries, of the values
//     and of the output gradient, with a chunk swizzle that serves both the row reads and the
//     transposing reads; for softmax every row also gets its base-2 log-normaliser (from the
//     forward) and dout . o.
//   * dq: one workgroup per (batch, kv head, head group, query tile) walks the key tiles of
//     its band as the forward does, one 32-key block at a time: S^T = K Q^T and
//     dP^T = V dO^T from LDS rows, dX^T in registers (one query per lane), then
//     dQ^T += K^T dX^T with K read transposed.
//   * dk, dv: one workgroup per (batch, kv head, 128 keys) walks the query tiles whose window
//     reaches its keys, for every query head of the group: S = Q K^T and dP = dO V^T with K
//     and V held in registers (one key per lane), then dV^T += dO^T P and dK^T += Q^T dX with
//     dO and Q read transposed. Queries that see a sink key only through the sink rule are
//     taken by extra workgroups, each storing its share in a slot of its own; the key
//     block's own workgroup adds the slots in split order, so the result is the same bits on
//     every run.
//   * All products take float16 operands with float32 accumulation; values past the float16
//     range saturate at +-65504.
#include "mfma_common.hpp"
#include "swa_kernels.hpp"

namespace swa {
namespace {

// Chunk c of tile row r is stored at chunk c ^ bswz(r). A row read serves 16 rows at one
// chunk per group of 16 lanes; a transposing read serves 4 consecutive rows x 4 adjacent
// chunks per group of 32 lanes. This swizzle keeps both free of LDS bank conflicts: it is a
// permutation of 16 consecutive rows (of 8 rows per row parity at d = 64, where two rows
// share a 256-byte bank line), and it sends the 4 rows of a transposing read to 4 different
// aligned groups of 4 chunks.
template <int D>
__host__ __device__ __forceinline__ constexpr int bswz(int r) {
    return D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3))
                    : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}

template <int D>
struct BT {
    static constexpr int C = D / 8;                        // 16-byte chunks per row
    static constexpr int IMG = BK * D;                     // 16-bit elements of a tile
    static constexpr int IMG_BYTES = IMG * 2;
    static constexpr int NW = 4;                           // wavefronts per workgroup
    static constexpr int DMA_W = IMG_BYTES / (NW * 1024);  // 1 KB transfers per wavefront
    static constexpr int KPT = BK * C / 256;               // chunks per thread of a pre-pass
    static constexpr int KP = 32 * NW;                     // keys per dk/dv workgroup
    static constexpr int OSTR = D + 4;                     // floats per staged output row
};

// Element offset in a tile image of chunk c of row r.
template <int D>
__device__ __forceinline__ int slot_of(int r, int c) {
    return (r * BT<D>::C + (c ^ bswz<D>(r))) * 8;
}

// Eight output-dtype values -> float.
template <int OUT>
__device__ __forceinline__ void load8(const void *base, int64_t off, float (&x)[8]) {
    if (OUT == 1) {
        const uint4 u = ldg16(static_cast<const uint16_t *>(base) + off);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            x[2 * m] = __uint_as_float(w[m] << 16);
            x[2 * m + 1] = __uint_as_float(w[m] & 0xffff0000u);
        }
    } else {
        const float4 a = as_float4(ldg16(static_cast<const float *>(base) + off));
        const float4 b = as_float4(ldg16(static_cast<const float *>(base) + off + 4));
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
        x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    }
}

// ---------------------------------------------------------------------------------------
// Pre-passes.
struct PackKV {
    const uint16_t *k, *v;
    uint16_t *kimg, *vimg;
    const float *rope;
    int64_t N, Hkv;
    int n_tiles;
};

// One block per (batch, 64-position tile, up to four kv heads): rotated keys and values as
// float16 images. Rows past N are zero.
template <int D, bool ROT>
__global__ __launch_bounds__(256) void bwd_pack_kv_kernel(PackKV p) {
    using T = BT<D>;
    const int n_hg = (int)((p.Hkv + 3) / 4);
    const int hg = blockIdx.x % n_hg;
    const int rest = blockIdx.x / n_hg;
    const int jt = rest % p.n_tiles;
    const int64_t b = rest / p.n_tiles;
    const int64_t h0 = (int64_t)hg * 4;
    const int nh = p.Hkv - h0 < 4 ? (int)(p.Hkv - h0) : 4;
#pragma unroll
    for (int r = 0; r < T::KPT; ++r) {
        const int cidx = threadIdx.x + 256 * r, row = cidx / T::C, c = cidx % T::C;
        const int64_t j = (int64_t)jt * BK + row;
        const bool in = j < p.N;
        float4 t0 = make_float4(1.f, 0.f, 1.f, 0.f), t1 = t0;
        if (ROT && in) {
            const float *t = p.rope + (j * (D / 2) + c * 4) * 2;
            t0 = as_float4(ldg16(t));
            t1 = as_float4(ldg16(t + 4));
        }
        const int slot = slot_of<D>(row, c);
        // the row's loads for every head first, then its stores
        uint4 xk[4], xv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            xk[e] = xv[e] = make_uint4(0, 0, 0, 0);
            if (in && e < nh) {
                const int64_t off = ((b * p.N + j) * p.Hkv + h0 + e) * D + c * 8;
                xk[e] = ldg16(p.k + off);
                xv[e] = ldg16(p.v + off);
            }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if (e >= nh) break;
            const int64_t img = ((b * p.Hkv + h0 + e) * p.n_tiles + jt) * T::IMG;
            stg16(p.kimg + img + slot, ROT ? rotate_chunk(xk[e], t0, t1) : convert_chunk(xk[e]));
            stg16(p.vimg + img + slot, convert_chunk(xv[e]));
        }
    }
}

struct PackQ {
    const uint16_t *q;
    const void *dout, *o;
    const float *lse;
    uint16_t *qimg, *gimg;
    float *stats;      // [B, Hq, n_tiles * 64, 2]: (base-2 log-normaliser, dout . o)
    const float *rope;
    int64_t N, Hq;
    int n_tiles;
    float qs;          // factor on the query image: -scale log2(e) for sigmoid, else 1
};

// One block per (batch, 64-position tile, part of the tile, up to four query heads), each
// thread one 16-byte chunk per head: rotated queries and the output gradient as float16
// images; for softmax the row statistics (rows past N get an infinite log-normaliser, so
// their weights vanish). Tile parts give the grid several rounds of blocks, whose loads and
// stores overlap.
template <int D, bool ROT, int OUT, int MODE>
__global__ __launch_bounds__(256) void bwd_pack_q_kernel(PackQ p) {
    using T = BT<D>;
    const int n_hg = (int)((p.Hq + 3) / 4);
    const int hg = blockIdx.x % n_hg;
    const int rest0 = blockIdx.x / n_hg;
    const int pt = rest0 % T::KPT;   // this block's chunks: 256 pt .. 256 pt + 255
    const int rest = rest0 / T::KPT;
    const int it = rest % p.n_tiles;
    const int64_t b = rest / p.n_tiles;
    const int64_t h0 = (int64_t)hg * 4;
    const int nh = p.Hq - h0 < 4 ? (int)(p.Hq - h0) : 4;
    {
        const int cidx = threadIdx.x + 256 * pt, row = cidx / T::C, c = cidx % T::C;
        const int64_t i = (int64_t)it * BK + row;
        const bool in = i < p.N;
        float4 t0 = make_float4(1.f, 0.f, 1.f, 0.f), t1 = t0;
        if (ROT && in) {
            const float *t = p.rope + (i * (D / 2) + c * 4) * 2;
            t0 = as_float4(ldg16(t));
            t1 = as_float4(ldg16(t + 4));
        }
        const int slot = slot_of<D>(row, c);
        // the row's loads for every head first (queries, output gradients, outputs and
        // log-normalisers), then its conversions and stores
        uint4 xq[4];
        float g8[4][8], o8[4][8], lsev[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            xq[e] = make_uint4(0, 0, 0, 0);
            lsev[e] = 0.0f;
#pragma unroll
            for (int m = 0; m < 8; ++m) g8[e][m] = o8[e][m] = 0.0f;
            if (in && e < nh) {
                const int64_t off = ((b * p.N + i) * p.Hq + h0 + e) * D + c * 8;
                xq[e] = ldg16(p.q + off);
                load8<OUT>(p.dout, off, g8[e]);
                if (MODE == 1) {
                    load8<OUT>(p.o, off, o8[e]);
                    if (c == 0) lsev[e] = p.lse[(b * p.Hq + h0 + e) * p.N + i];
                }
            }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if (e >= nh) break;
            const int64_t h = h0 + e;
            const int64_t img = ((b * p.Hq + h) * p.n_tiles + it) * T::IMG;
            // sigmoid: the query image carries -scale log2(e), so that the score product is
            // the negated base-2 logit (the dk/dv kernels undo the factor on dK)
            if (MODE == 0)
                stg16(p.qimg + img + slot, ROT ? rotate_chunk_scaled(xq[e], t0, t1, p.qs)
                                               : convert_chunk_scaled(xq[e], p.qs));
            else
                stg16(p.qimg + img + slot, ROT ? rotate_chunk(xq[e], t0, t1) : convert_chunk(xq[e]));
            stg16(p.gimg + img + slot,
                  make_uint4(pack_f16x2_sat(g8[e][0], g8[e][1]), pack_f16x2_sat(g8[e][2], g8[e][3]),
                             pack_f16x2_sat(g8[e][4], g8[e][5]), pack_f16x2_sat(g8[e][6], g8[e][7])));
            if (MODE == 1) {
                float dot = 0.0f;
#pragma unroll
                for (int m = 0; m < 8; ++m) dot = fmaf(g8[e][m], o8[e][m], dot);
                // the C chunks of a row sit in C consecutive lanes
                dot = T::C == 8 ? group8_sum(dot) : group16_sum(dot);
                if (c == 0) {
                    float2 st;
                    st.x = in ? lsev[e] * LOG2E : INFINITY;
                    st.y = in ? dot : 0.0f;
                    reinterpret_cast<float2 *>(p.stats)[(b * p.Hq + h) * (int64_t)p.n_tiles * BK + i] = st;
                }
            }
        }
    }
}

__global__ void zero_kernel(float *x, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) x[i] = 0.0f;
}

// ---------------------------------------------------------------------------------------
struct BwdParams {
    const uint16_t *kimg, *vimg, *qimg, *gimg;
    const float *stats, *slopes, *rope;
    void *dq, *dk, *dv;
    // partial dk~, dv of the sink blocks from the extra workgroups, one slot per split:
    // [B, Hkv, n_splits, sink_blocks * 128, D] float32 each
    float *sink_k, *sink_v;
    int64_t N, Hq, Hkv, G;
    int n_tiles;             // 64-row tiles of every image slice
    int n_qtiles, n_hgroups; // dq grid
    int n_kblocks;           // dk/dv grid: 128-key blocks per (batch, kv head)
    int sink_blocks, n_splits, split_tiles;
    int w, s;
    float cs, scale;
    int out_bf16;
};

// Element offset of key j's row in split sp's slot of the sink partials (times D).
template <int D>
__device__ __forceinline__ int64_t sink_slot_d(const BwdParams &p, int b, int hkv, int sp, int j) {
    const int64_t sk = (int64_t)p.sink_blocks * 128;
    return ((((int64_t)b * p.Hkv + hkv) * p.n_splits + sp) * sk + j) * D;
}

// Transposing-read offsets: lane (G4, rr, a) supplies row 8 h + 4 (G4 / 2) + rr of an 8 x 32
// block and the column group 16 (G4 % 2) + 4 a of 32-column block db.
template <int D>
__device__ __forceinline__ void tr_offsets(int lane, int (&off)[2][D / 32]) {
    const int G4 = lane >> 4, rr = (lane >> 2) & 3, a = lane & 3;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
        const int row = 8 * h2 + 4 * (G4 >> 1) + rr;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
            const int cl = 4 * db + 2 * (G4 & 1) + (a >> 1);
            off[h2][db] = row * D + ((cl ^ bswz<D>(row)) * 8) + 4 * (a & 1);
        }
    }
}

// acc^T += M^T X^T over the 32 rows 32 xb .. 32 xb + 31 of an LDS tile, in two steps of 16
// rows: X is one 32-row block of scores in the accumulator layout, and step t2 uses
// x[8 t2 + 0..7], rows 32 xb + 16 t2 + 4 g + {0..3, 8..11}, which is the order in which the
// two transposing reads deliver M^T.
template <int D>
__device__ __forceinline__ void acc_tr(const uint16_t *__restrict__ ml, int xb,
                                       const int (&off)[2][D / 32], const f32x16_t &x,
                                       f32x16_t (&acc)[D / 32]) {
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) {
        const int e0 = 8 * t2, row0 = 32 * xb + 16 * t2;
        uint4 pk;
        pk.x = pack_f16x2(x[e0 + 0], x[e0 + 1]);
        pk.y = pack_f16x2(x[e0 + 2], x[e0 + 3]);
        pk.z = pack_f16x2(x[e0 + 4], x[e0 + 5]);
        pk.w = pack_f16x2(x[e0 + 6], x[e0 + 7]);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
            const s16x4_t lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_s16x4_t *)(ml + row0 * D + off[0][db]));
            const s16x4_t hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_s16x4_t *)(ml + row0 * D + off[1][db]));
            const s16x8_t a8 = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
            acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                __builtin_bit_cast(f16x8_t, a8), __builtin_bit_cast(f16x8_t, pk), acc[db], 0, 0, 0);
        }
    }
}

// Workgroup id -> logical id, so that each XCD walks a contiguous run of logical ids.
__device__ __forceinline__ int xcd_logical() {
    const int nb = gridDim.x, bid = blockIdx.x;
    const int per = nb / 8, rem = nb % 8, xcd = bid % 8, local = bid / 8;
    return xcd < rem ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
}

// (i, j) -> rotated-frame gradient pair (a, b) at position pos turned back by R(pos)^T.
__device__ __forceinline__ float2 unrotate(float a, float b, float2 cs) {
    return make_float2(fmaf(b, cs.y, a * cs.x), fmaf(-a, cs.y, b * cs.x));
}

// ---------------------------------------------------------------------------------------
// dq. Register budget: 2 wavefronts per SIMD.
template <int D, int GP, int MODE, bool ALIBI>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void bwd_dq_kernel(BwdParams p) {
    using T = BT<D>;
    constexpr int QP = 32 * T::NW / GP;   // query positions per workgroup
    constexpr int WPH = T::NW / GP;       // wavefronts per query head
    constexpr int KS = D / 16, DB = D / 32;
    constexpr int LDS_ELEMS = cmax(4 * T::IMG, T::NW * 32 * T::OSTR * 2);
    __shared__ __attribute__((aligned(16))) uint16_t lds[LDS_ELEMS];
    // K tiles at lds + buf * IMG, V tiles at lds + (2 + buf) * IMG

    const int logical = xcd_logical();
    // query tile order as in the forward: the tiles whose bands the sequence start cuts short
    // come last, longest first
    int rot = (p.w - 1 + QP - 1) / QP;
    if (rot > p.n_qtiles) rot = p.n_qtiles;
    const int lt = logical % p.n_qtiles;
    const int qt = lt < p.n_qtiles - rot ? lt + rot : p.n_qtiles - 1 - lt;
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
    const int qa = q0 + 32 * pb;
    const int qb = qa + 31 < N ? qa + 31 : N - 1;
    const int i = qa + qc;
    const int qe = (q0 + QP < N ? q0 + QP : N) - 1;

    // band of key tiles (as the forward walks it)
    const int lo_wg = q0 - p.w + 1 > 0 ? q0 - p.w + 1 : 0;
    const int tw_begin = lo_wg / BK, tw_end = qe / BK;
    const int n_sink_keys = p.s < lo_wg ? p.s : lo_wg;
    int ts_end = (n_sink_keys + BK - 1) / BK;
    if (ts_end > tw_begin) ts_end = tw_begin;
    const int n_walk = ts_end + (tw_end - tw_begin + 1);
    auto j0_of = [&](int t) { return (t < ts_end ? t : tw_begin + (t - ts_end)) * BK; };
    // 0: every pair in the key set, 1: window edges, 2: also sinks, -1: none (this wavefront)
    auto kind_of = [&](int j0) {
        if (qa >= N || j0 > qb || (qa - (j0 + BK - 1) >= p.w && j0 >= p.s)) return -1;
        if ((j0 + BK - 1 <= qa) && (qb - j0 < p.w || j0 + BK - 1 < p.s)) return 0;
        return j0 >= p.s ? 1 : 2;
    };

    const int64_t kvslice = ((int64_t)b * p.Hkv + hkv) * p.n_tiles * T::IMG;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(p.kimg + kvslice, (uint32_t)p.n_tiles * T::IMG_BYTES);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.vimg + kvslice, (uint32_t)p.n_tiles * T::IMG_BYTES);
    uint32_t dimg[T::DMA_W];
#pragma unroll
    for (int r = 0; r < T::DMA_W; ++r) dimg[r] = (uint32_t)((wave * T::DMA_W + r) * 64 + lane) * 16;
    int koff[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) koff[ks] = slot_of<D>(qc, 2 * ks + g);
    int toff[2][DB];
    tr_offsets<D>(lane, toff);

    // this lane's query and output-gradient fragments (B operands), rotated float16
    // (every load in flight at once: a lane past the end reads the last row and drops it)
    f16x8_t qreg[KS], greg[KS];
    const bool in = i < N;
    const int ic = in ? i : N - 1;
    {
        const int64_t qslice = ((int64_t)b * p.Hq + h) * p.n_tiles * T::IMG;
        const int it = ic / BK, ri = ic % BK;
        uint4 xq[KS], xg[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int64_t off = qslice + (int64_t)it * T::IMG + slot_of<D>(ri, 2 * ks + g);
            xq[ks] = ldg16(p.qimg + off);
            xg[ks] = ldg16(p.gimg + off);
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            qreg[ks] = __builtin_bit_cast(f16x8_t, in ? xq[ks] : make_uint4(0, 0, 0, 0));
            greg[ks] = __builtin_bit_cast(f16x8_t, in ? xg[ks] : make_uint4(0, 0, 0, 0));
        }
    }
    float l2 = 0.0f, dl = 0.0f;
    if (MODE == 1) {
        const float2 st = reinterpret_cast<const float2 *>(p.stats)[((int64_t)b * p.Hq + h) * p.n_tiles * BK + ic];
        l2 = in ? st.x : 0.0f;
        dl = in ? st.y : 0.0f;
    }
    const float slope_l2 = ALIBI ? p.slopes[h] * LOG2E : 0.0f;
    // softmax: key part -(slope log2(e) / cs) kappa of the unscaled product; sigmoid (query
    // image scaled by -cs): the whole bias of the negated logit, key and query parts
    const BiasOperands bo = MODE == 0 ? bias_operands(ALIBI ? -slope_l2 : 0.0f, lane, ALIBI)
                                      : bias_operands(ALIBI ? slope_l2 / p.cs : 0.0f, lane);

    f32x16_t acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[db][e] = 0.0f;

    auto load = [&](int t, int buf) {
        const uint32_t base = (uint32_t)(j0_of(t) / BK) * T::IMG_BYTES;
        dma_rounds<T::DMA_W>(lds + buf * T::IMG, rk, base, dimg, wave);
        dma_rounds<T::DMA_W>(lds + (2 + buf) * T::IMG, rv, base, dimg, wave);
    };
    load(0, 0);
    __syncthreads();
    for (int t = 0; t < n_walk; ++t) {
        const int cur = t & 1;
        if (t + 1 < n_walk) load(t + 1, cur ^ 1);
        const int j0 = j0_of(t);
        const int kind = kind_of(j0);
        if (kind >= 0) {
            const uint16_t *kl = lds + cur * T::IMG, *vl = lds + (2 + cur) * T::IMG;
            const f16x8_t bb = (MODE == 0 && ALIBI) ? query_term(bo, i - j0) : bo.b;
            constexpr float fill = MODE == 0 ? INFINITY : -INFINITY;
            const float bq = slope_l2 * (float)(i - j0);
            // one 32-key block at a time: S^T and dP^T (their chains alternate), dX^T, then
            // dQ^T += K^T dX^T; the next block's products overlap this block's vector work
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const f32x16_t zero = {};
                f32x16_t sa = ALIBI ? __builtin_amdgcn_mfma_f32_32x32x16_f16(bo.a[kb], bb, zero, 0, 0, 0) : zero;
                f32x16_t da = zero;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const f16x8_t ak = *reinterpret_cast<const f16x8_t *>(kl + kb * 32 * D + koff[ks]);
                    const f16x8_t av = *reinterpret_cast<const f16x8_t *>(vl + kb * 32 * D + koff[ks]);
                    sa = __builtin_amdgcn_mfma_f32_32x32x16_f16(ak, qreg[ks], sa, 0, 0, 0);
                    da = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, greg[ks], da, 0, 0, 0);
                }
                {
                    // rows read four products ahead of their use
                    constexpr int NR = 2 * KS, AH = 4;
                    __builtin_amdgcn_sched_group_barrier(0x100, AH, 0);  // LDS reads
                    if (ALIBI) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
#pragma unroll
                    for (int u = 0; u < NR - AH; ++u) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // matrix
                        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                    }
                    __builtin_amdgcn_sched_group_barrier(0x008, AH, 0);
                }
                if (kind == 1) mask_block<false>(sa, kb, i - j0 - 4 * g, j0 + 4 * g, p.w, p.s, fill);
                else if (kind == 2) mask_block<true>(sa, kb, i - j0 - 4 * g, j0 + 4 * g, p.w, p.s, fill);
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    if (MODE == 0) {
                        const float pe = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(sa[e]));
                        sa[e] = da[e] * fmaf(-pe, pe, pe);   // dP p (1 - p)
                    } else {
                        const float pe = __builtin_amdgcn_exp2f(fmaf(sa[e], p.cs, bq) - l2);
                        sa[e] = pe * (da[e] - dl);
                    }
                }
                acc_tr<D>(kl, kb, toff, sa, acc);
            }
        }
        __syncthreads();
    }

    // ---- epilogue: dq = R(i)^T (scale dq~), staged through LDS as whole rows
    float *ol = reinterpret_cast<float *>(lds) + wave * (32 * T::OSTR);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int d0 = 32 * db + 8 * r + 4 * g;   // this lane holds d0 .. d0 + 3
            float v0 = acc[db][4 * r] * p.scale, v1 = acc[db][4 * r + 1] * p.scale;
            float v2 = acc[db][4 * r + 2] * p.scale, v3 = acc[db][4 * r + 3] * p.scale;
            if (p.rope != nullptr && i < N) {
                const float4 c = as_float4(ldg16(p.rope + ((int64_t)i * (D / 2) + d0 / 2) * 2));
                const float2 u0 = unrotate(v0, v1, make_float2(c.x, c.y));
                const float2 u1 = unrotate(v2, v3, make_float2(c.z, c.w));
                v0 = u0.x; v1 = u0.y; v2 = u1.x; v3 = u1.y;
            }
            *reinterpret_cast<float4 *>(ol + qc * T::OSTR + d0) = make_float4(v0, v1, v2, v3);
        }
    __syncthreads();
    constexpr int C4 = D / 4;
#pragma unroll
    for (int rr = 0; rr < 32 * C4 / 64; ++rr) {
        const int ch = lane + 64 * rr;
        const int row = ch / C4, c4 = ch % C4;
        const int iq = qa + row;
        if (iq < N) {
            const float4 x = *reinterpret_cast<const float4 *>(ol + row * T::OSTR + 4 * c4);
            const int64_t off = (((int64_t)b * p.N + iq) * p.Hq + h) * D + 4 * c4;
            store_out4<false>(p.dq, p.out_bf16, off, x.x, x.y, x.z, x.w);
        }
    }
}

// ---------------------------------------------------------------------------------------
// dk, dv. One wavefront owns 32 keys (one per lane column); the workgroup's four wavefronts
// share the query tiles staged in LDS. SINK: the workgroup is one of the extra ones that
// take the queries past every window pair of a sink key block.
template <int D, int MODE, bool ALIBI, bool SINK>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(D == 64 ? 2 : 1)))
void bwd_dkv_kernel(BwdParams p) {
    using T = BT<D>;
    constexpr int KS = D / 16, DB = D / 32;
    constexpr int STAGE = 2 * T::IMG + 256;   // Q tile, dO tile, 64 x (log-normaliser, dout.o)
    __shared__ __attribute__((aligned(16))) uint16_t lds[2 * STAGE];

    int b, hkv, kblk, split = 0;
    {
        const int logical = xcd_logical();
        int rest = logical;
        if (SINK) {
            split = rest % p.n_splits;
            rest /= p.n_splits;
            kblk = rest % p.sink_blocks;
            rest /= p.sink_blocks;
        } else {
            kblk = rest % p.n_kblocks;
            rest /= p.n_kblocks;
        }
        hkv = rest % (int)p.Hkv;
        b = rest / (int)p.Hkv;
    }
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int g = lane >> 5;
    const int N = (int)p.N;
    const int j0 = kblk * T::KP;                  // the workgroup's first key
    const int jw = j0 + 32 * wave;                // this wavefront's first key
    const int j = jw + (lane & 31);               // this lane's key
    // queries this workgroup answers for: [qlo, qhi)
    const int win_end = j0 + T::KP - 1 + p.w < N ? j0 + T::KP - 1 + p.w : N;
    int qlo, qhi;
    if (SINK) {
        qlo = win_end + split * p.split_tiles * BK;
        qhi = qlo + p.split_tiles * BK < N ? qlo + p.split_tiles * BK : N;
        if (qlo >= N) return;
    } else {
        qlo = j0;
        qhi = win_end;
    }
    const int t_lo = qlo / BK, t_hi = (qhi - 1) / BK;
    const int n_steps = (t_hi - t_lo + 1) * (int)p.G;
    const bool active = !SINK || jw < p.s;        // sink workgroups: only waves holding sinks

    const uint32_t qslice_bytes = (uint32_t)p.n_tiles * T::IMG_BYTES;
    uint32_t dimg[T::DMA_W];
#pragma unroll
    for (int r = 0; r < T::DMA_W; ++r) dimg[r] = (uint32_t)((wave * T::DMA_W + r) * 64 + lane) * 16;
    int qoff[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qoff[ks] = slot_of<D>(lane & 31, 2 * ks + g);
    int toff[2][DB];
    tr_offsets<D>(lane, toff);

    // this lane's key and value fragments (B operands of S = Q K^T and dP = dO V^T)
    // (every load in flight at once: a lane past the end reads the last row and drops it)
    f16x8_t kreg[KS], vreg[KS];
    {
        const bool jin = j < N;
        const int jc = jin ? j : N - 1;
        const int64_t slice = ((int64_t)b * p.Hkv + hkv) * p.n_tiles * T::IMG;
        const int jt = jc / BK, rj = jc % BK;
        uint4 xk[KS], xv[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int64_t off = slice + (int64_t)jt * T::IMG + slot_of<D>(rj, 2 * ks + g);
            xk[ks] = ldg16(p.kimg + off);
            xv[ks] = ldg16(p.vimg + off);
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            kreg[ks] = __builtin_bit_cast(f16x8_t, jin ? xk[ks] : make_uint4(0, 0, 0, 0));
            vreg[ks] = __builtin_bit_cast(f16x8_t, jin ? xv[ks] : make_uint4(0, 0, 0, 0));
        }
    }

    f32x16_t dk[DB], dv[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) { dk[db][e] = 0.0f; dv[db][e] = 0.0f; }

    auto load = [&](int n, int buf) {
        const int qt = t_lo + n / (int)p.G;
        const int64_t hq = (int64_t)hkv * p.G + n % (int)p.G;
        const int64_t slice = ((int64_t)b * p.Hq + hq) * p.n_tiles * T::IMG;
        const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.qimg + slice, qslice_bytes);
        const __amdgpu_buffer_rsrc_t rg = make_rsrc(p.gimg + slice, qslice_bytes);
        uint16_t *st = lds + buf * STAGE;
        dma_rounds<T::DMA_W>(st, rq, (uint32_t)qt * T::IMG_BYTES, dimg, wave);
        dma_rounds<T::DMA_W>(st + T::IMG, rg, (uint32_t)qt * T::IMG_BYTES, dimg, wave);
        if (MODE == 1 && wave == 0 && lane < 32) {
            const float *src = p.stats + (((int64_t)b * p.Hq + hq) * p.n_tiles * BK + (int64_t)qt * BK) * 2;
            const __amdgpu_buffer_rsrc_t rs = make_rsrc(src, 512);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t *)(st + 2 * T::IMG), 16,
                                                     (uint32_t)lane * 16, 0, 0, 0);
        }
    };

    load(0, 0);
    __syncthreads();
    for (int n = 0; n < n_steps; ++n) {
        const int cur = n & 1;
        if (n + 1 < n_steps) load(n + 1, cur ^ 1);
        const int qt = t_lo + n / (int)p.G;
        const int64_t hq = (int64_t)hkv * p.G + n % (int)p.G;
        const int i0 = qt * BK;
        // pairs of this wavefront's keys with the tile's queries: none, all, or some
        const int ilo = i0 > qlo ? i0 : qlo, ihi = (i0 + BK < qhi ? i0 + BK : qhi) - 1;
        const bool any = active && ilo <= ihi && ihi >= jw &&
                         ((ilo - (jw + 31) < p.w) || jw < p.s);
        // uniform by construction; read back as a scalar so that the per-element masking below
        // branches once per step, not per element under an execution mask
        const bool all = __builtin_amdgcn_readfirstlane((int)(ilo == i0 && ihi == i0 + BK - 1 && i0 >= jw + 31 &&
                             ((i0 + BK - 1 - jw < p.w) || jw + 31 < p.s) && jw + 31 < N)) != 0;
        if (any) {
            const uint16_t *ql = lds + cur * STAGE;
            const uint16_t *gl = ql + T::IMG;
            const float *stl = reinterpret_cast<const float *>(ql + 2 * T::IMG);
            const float slope_l2 = ALIBI ? p.slopes[hq] * LOG2E : 0.0f;
            // rows are queries here: softmax adds (slope log2(e) / cs) m for query offset m;
            // sigmoid (query tiles scaled by -cs) the whole bias -slope log2(e) (i0 + m - j)
            const BiasOperands bo = MODE == 0 ? bias_operands(ALIBI ? slope_l2 : 0.0f, lane, ALIBI)
                                              : bias_operands(ALIBI ? -slope_l2 / p.cs : 0.0f, lane);
            const f16x8_t bb = (MODE == 0 && ALIBI) ? query_term(bo, j - i0) : bo.b;
            const float lb = slope_l2 * (float)(i0 - j);   // key part of the bias (softmax)
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                const f32x16_t zero = {};
                f32x16_t sacc = ALIBI ? __builtin_amdgcn_mfma_f32_32x32x16_f16(bo.a[qb], bb, zero, 0, 0, 0) : zero;
                f32x16_t dacc = zero;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const f16x8_t aq = *reinterpret_cast<const f16x8_t *>(ql + qb * 32 * D + qoff[ks]);
                    const f16x8_t ag = *reinterpret_cast<const f16x8_t *>(gl + qb * 32 * D + qoff[ks]);
                    sacc = __builtin_amdgcn_mfma_f32_32x32x16_f16(aq, kreg[ks], sacc, 0, 0, 0);
                    dacc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ag, vreg[ks], dacc, 0, 0, 0);
                }
                // edge steps: pairs outside the key sets get the fill that makes their weight
                // zero, in place (one branch per row block)
                if (!all) {
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int iq = i0 + 32 * qb + 8 * (e >> 2) + 4 * g + (e & 3);
                        const int dij = iq - j;
                        const bool ok = (iq >= qlo) & (iq < qhi) & (iq < N) & (j < N) & (dij >= 0) &
                                        ((dij < p.w) | (j < p.s));
                        sacc[e] = keep_or_fill(sacc[e], ok, MODE == 0 ? INFINITY : -INFINITY);
                    }
                }
                // weights into sacc, dX into dacc
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int r0 = 32 * qb + 8 * u + 4 * g;   // rows r0 .. r0 + 3 of the tile
                    float4 st0 = make_float4(0.f, 0.f, 0.f, 0.f), st1 = st0;
                    if (MODE == 1) {
                        st0 = *reinterpret_cast<const float4 *>(stl + 2 * r0);
                        st1 = *reinterpret_cast<const float4 *>(stl + 2 * r0 + 4);
                    }
                    const float l2v[4] = {st0.x, st0.z, st1.x, st1.z};
                    const float dlv[4] = {st0.y, st0.w, st1.y, st1.w};
#pragma unroll
                    for (int e4 = 0; e4 < 4; ++e4) {
                        const int e = 4 * u + e4;
                        const float x = sacc[e];
                        float pe, dxe;
                        if (MODE == 0) {
                            pe = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(x));
                            dxe = dacc[e] * fmaf(-pe, pe, pe);   // dP p (1 - p)
                        } else {
                            pe = __builtin_amdgcn_exp2f(fmaf(x, p.cs, lb) - l2v[e4]);
                            dxe = pe * (dacc[e] - dlv[e4]);
                        }
                        sacc[e] = pe;
                        dacc[e] = dxe;
                    }
                }
                acc_tr<D>(gl, qb, toff, sacc, dv);   // dV^T += dO^T P
                acc_tr<D>(ql, qb, toff, dacc, dk);   // dK~^T += Q~^T dX
            }
        }
        __syncthreads();
    }

    // ---- epilogue
    if (SINK) {
        // this split's partial into its own slot (no atomics: the block's own workgroup sums
        // the slots in split order, so the result does not depend on timing)
        if (!active) return;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int d = 32 * db + 8 * (e >> 2) + 4 * g + (e & 3);
                const int64_t off = sink_slot_d<D>(p, b, hkv, split, j) + d;
                p.sink_k[off] = dk[db][e];
                p.sink_v[off] = dv[db][e];
            }
        return;
    }
    if (j >= N) return;
    if (p.sink_k != nullptr && kblk < p.sink_blocks) {
        f32x16_t sk_[DB], sv_[DB];
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int e = 0; e < 16; ++e) sk_[db][e] = sv_[db][e] = 0.0f;
        for (int sp = 0; sp < p.n_splits; ++sp)
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int d = 32 * db + 8 * (e >> 2) + 4 * g + (e & 3);
                    const int64_t off = sink_slot_d<D>(p, b, hkv, sp, j) + d;
                    sk_[db][e] += p.sink_k[off];
                    sv_[db][e] += p.sink_v[off];
                }
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                dk[db][e] += sk_[db][e];
                dv[db][e] += sv_[db][e];
            }
    }
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int d0 = 32 * db + 8 * r + 4 * g;
            // sigmoid accumulated dK against the query image scaled by -cs
            const float dks = MODE == 0 ? -p.scale / p.cs : p.scale;
            float k0 = dk[db][4 * r] * dks, k1 = dk[db][4 * r + 1] * dks;
            float k2 = dk[db][4 * r + 2] * dks, k3 = dk[db][4 * r + 3] * dks;
            if (p.rope != nullptr) {
                const float4 c = as_float4(ldg16(p.rope + ((int64_t)j * (D / 2) + d0 / 2) * 2));
                const float2 u0 = unrotate(k0, k1, make_float2(c.x, c.y));
                const float2 u1 = unrotate(k2, k3, make_float2(c.z, c.w));
                k0 = u0.x; k1 = u0.y; k2 = u1.x; k3 = u1.y;
            }
            const int64_t off = (((int64_t)b * p.N + j) * p.Hkv + hkv) * D + d0;
            store_out4<false>(p.dk, p.out_bf16, off, k0, k1, k2, k3);
            store_out4<false>(p.dv, p.out_bf16, off, dv[db][4 * r], dv[db][4 * r + 1], dv[db][4 * r + 2],
                       dv[db][4 * r + 3]);
        }
}

// ---------------------------------------------------------------------------------------
// dk, dv with each 32-key block's work split over two wavefronts (eight per workgroup, two
// per SIMD): wavefront w < 4 forms the scores and weights P of its keys, publishes P (float16)
// in LDS and accumulates dV^T += dO^T P; wavefront w + 4 forms dP = dO V^T, takes P from LDS,
// forms dX and accumulates dK~^T += Q~^T dX. Each role holds one fragment (K or V) and one
// accumulator, half the registers of the single-wavefront form, so two wavefronts share a SIMD.
template <int D, int MODE, bool ALIBI, bool SINK>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2)))
void bwd_dkv2_kernel(BwdParams p) {
    using T = BT<D>;
    constexpr int KS = D / 16, DB = D / 32;
    constexpr int NWG = 8;
    constexpr int DMA_R = T::IMG_BYTES / (NWG * 1024);   // 1 KB transfers per wavefront
    constexpr int STAGE = 2 * T::IMG + 256;              // Q tile, dO tile, 64 row statistics
    constexpr int PX = 4 * 2 * 64 * 16;                  // P: 4 key blocks x 2 row blocks x 64 lanes x 16
    // the dX role runs one step behind the P role: three stages (the P role's, the dX role's
    // and the one being loaded) and two P buffers
    __shared__ __attribute__((aligned(16))) uint16_t lds[3 * STAGE + 2 * PX];
    uint16_t *const px0 = lds + 3 * STAGE;

    int b, hkv, kblk, split = 0;
    {
        int rest = xcd_logical();
        if (SINK) {
            split = rest % p.n_splits;
            rest /= p.n_splits;
            kblk = rest % p.sink_blocks;
            rest /= p.sink_blocks;
        } else {
            kblk = rest % p.n_kblocks;
            rest /= p.n_kblocks;
        }
        hkv = rest % (int)p.Hkv;
        b = rest / (int)p.Hkv;
    }
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int g = lane >> 5;
    const bool role_p = wave < 4;                 // P and dV; else dP, dX and dK
    const int kw = wave & 3;                      // this wavefront's 32-key block
    const int N = (int)p.N;
    const int j0 = kblk * T::KP;
    const int jw = j0 + 32 * kw;
    const int j = jw + (lane & 31);
    const int win_end = j0 + T::KP - 1 + p.w < N ? j0 + T::KP - 1 + p.w : N;
    int qlo, qhi;
    if (SINK) {
        qlo = win_end + split * p.split_tiles * BK;
        qhi = qlo + p.split_tiles * BK < N ? qlo + p.split_tiles * BK : N;
        if (qlo >= N) return;
    } else {
        qlo = j0;
        qhi = win_end;
    }
    const int t_lo = qlo / BK, t_hi = (qhi - 1) / BK;
    const int n_steps = (t_hi - t_lo + 1) * (int)p.G;
    const bool active = !SINK || jw < p.s;

    const uint32_t qslice_bytes = (uint32_t)p.n_tiles * T::IMG_BYTES;
    uint32_t dimg[DMA_R];
#pragma unroll
    for (int r = 0; r < DMA_R; ++r) dimg[r] = (uint32_t)((wave * DMA_R + r) * 64 + lane) * 16;
    int qoff[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qoff[ks] = slot_of<D>(lane & 31, 2 * ks + g);
    int toff[2][DB];
    tr_offsets<D>(lane, toff);

    // this lane's key (P role) or value (dX role) fragment
    f16x8_t kv[KS];
    {
        // every load in flight at once: a lane past the end reads the last row and drops it
        const uint16_t *img = role_p ? p.kimg : p.vimg;
        const bool jin = j < N;
        const int jc = jin ? j : N - 1;
        const int64_t slice = ((int64_t)b * p.Hkv + hkv) * p.n_tiles * T::IMG;
        const int jt = jc / BK, rj = jc % BK;
        uint4 x[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) x[ks] = ldg16(img + slice + (int64_t)jt * T::IMG + slot_of<D>(rj, 2 * ks + g));
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kv[ks] = __builtin_bit_cast(f16x8_t, jin ? x[ks] : make_uint4(0, 0, 0, 0));
    }
    f32x16_t acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[db][e] = 0.0f;

    auto load = [&](int n, uint16_t *__restrict__ st) {
        const int qt = t_lo + n / (int)p.G;
        const int64_t hq = (int64_t)hkv * p.G + n % (int)p.G;
        const int64_t slice = ((int64_t)b * p.Hq + hq) * p.n_tiles * T::IMG;
        const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.qimg + slice, qslice_bytes);
        const __amdgpu_buffer_rsrc_t rg = make_rsrc(p.gimg + slice, qslice_bytes);
        dma_rounds<DMA_R>(st, rq, (uint32_t)qt * T::IMG_BYTES, dimg, wave);
        dma_rounds<DMA_R>(st + T::IMG, rg, (uint32_t)qt * T::IMG_BYTES, dimg, wave);
        if (MODE == 1 && wave == 0 && lane < 32) {
            const float *src = p.stats + (((int64_t)b * p.Hq + hq) * p.n_tiles * BK + (int64_t)qt * BK) * 2;
            const __amdgpu_buffer_rsrc_t rs = make_rsrc(src, 512);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t *)(st + 2 * T::IMG), 16,
                                                     (uint32_t)lane * 16, 0, 0, 0);
        }
    };

    // One step of one role. The three stages and the P buffers are passed as distinct restrict
    // pointers, so the compiler knows that the transfers into the next stage cannot touch what
    // this step reads from LDS and does not wait for them before those reads.
    auto work = [&](int n, int my, uint16_t *__restrict__ fill, const uint16_t *__restrict__ ql,
                    uint16_t *__restrict__ pxw) {
        if (n + 1 < n_steps) load(n + 1, fill);
        const int qt = t_lo + my / (int)p.G;
        const int64_t hq = (int64_t)hkv * p.G + my % (int)p.G;
        const int i0 = qt * BK;
        const int ilo = i0 > qlo ? i0 : qlo, ihi = (i0 + BK < qhi ? i0 + BK : qhi) - 1;
        const bool any = active && ilo <= ihi && ihi >= jw &&
                         ((ilo - (jw + 31) < p.w) || jw < p.s);
        // uniform by construction; read back as a scalar so that the per-element masking below
        // branches once per step, not per element under an execution mask
        const bool all = __builtin_amdgcn_readfirstlane((int)(ilo == i0 && ihi == i0 + BK - 1 && i0 >= jw + 31 &&
                             ((i0 + BK - 1 - jw < p.w) || jw + 31 < p.s) && jw + 31 < N)) != 0;
        const uint16_t *gl = ql + T::IMG;
        const float *stl = reinterpret_cast<const float *>(ql + 2 * T::IMG);
        f32x16_t sd[2];                                       // P (P role) or dP (dX role)
        if (any) {
            const float slope_l2 = ALIBI ? p.slopes[hq] * LOG2E : 0.0f;
            // as in bwd_dkv_kernel: softmax adds (slope log2(e) / cs) m, sigmoid the whole
            // bias of the negated logit
            const BiasOperands bo = MODE == 0 ? bias_operands(ALIBI ? slope_l2 : 0.0f, lane, ALIBI)
                                              : bias_operands(ALIBI ? -slope_l2 / p.cs : 0.0f, lane);
            const f16x8_t bb = (MODE == 0 && ALIBI) ? query_term(bo, j - i0) : bo.b;
            const float lb = slope_l2 * (float)(i0 - j);   // key part of the bias (softmax)
            const uint16_t *al = role_p ? ql : gl;          // A rows: Q for S, dO for dP
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                const f32x16_t zero = {};
                f32x16_t a = (ALIBI && role_p) ? __builtin_amdgcn_mfma_f32_32x32x16_f16(bo.a[qb], bb, zero, 0, 0, 0) : zero;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const f16x8_t ar = *reinterpret_cast<const f16x8_t *>(al + qb * 32 * D + qoff[ks]);
                    a = __builtin_amdgcn_mfma_f32_32x32x16_f16(ar, kv[ks], a, 0, 0, 0);
                }
                sd[qb] = a;
            }
            if (role_p) {
                // edge steps: pairs outside the key sets get the fill that makes their weight
                // zero, in place (one branch per step)
                if (!all) {
#pragma unroll
                    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                        for (int e = 0; e < 16; ++e) {
                            const int iq = i0 + 32 * qb + 8 * (e >> 2) + 4 * g + (e & 3);
                            const int dij = iq - j;
                            const bool ok = (iq >= qlo) & (iq < qhi) & (iq < N) & (j < N) & (dij >= 0) &
                                            ((dij < p.w) | (j < p.s));
                            sd[qb][e] = keep_or_fill(sd[qb][e], ok, MODE == 0 ? INFINITY : -INFINITY);
                        }
                }
#pragma unroll
                for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const int r0 = 32 * qb + 8 * u + 4 * g;
                        float4 st0 = make_float4(0.f, 0.f, 0.f, 0.f), st1 = st0;
                        if (MODE == 1) {
                            st0 = *reinterpret_cast<const float4 *>(stl + 2 * r0);
                            st1 = *reinterpret_cast<const float4 *>(stl + 2 * r0 + 4);
                        }
                        const float l2v[4] = {st0.x, st0.z, st1.x, st1.z};
#pragma unroll
                        for (int e4 = 0; e4 < 4; ++e4) {
                            const int e = 4 * u + e4;
                            const float x = sd[qb][e];
                            sd[qb][e] = MODE == 0
                                ? __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(x))
                                : __builtin_amdgcn_exp2f(fmaf(x, p.cs, lb) - l2v[e4]);
                        }
                    }
                    uint4 w0, w1;
                    w0.x = pack_f16x2(sd[qb][0], sd[qb][1]);   w0.y = pack_f16x2(sd[qb][2], sd[qb][3]);
                    w0.z = pack_f16x2(sd[qb][4], sd[qb][5]);   w0.w = pack_f16x2(sd[qb][6], sd[qb][7]);
                    w1.x = pack_f16x2(sd[qb][8], sd[qb][9]);   w1.y = pack_f16x2(sd[qb][10], sd[qb][11]);
                    w1.z = pack_f16x2(sd[qb][12], sd[qb][13]); w1.w = pack_f16x2(sd[qb][14], sd[qb][15]);
                    *reinterpret_cast<uint4 *>(pxw + qb * 64 * 16) = w0;
                    *reinterpret_cast<uint4 *>(pxw + qb * 64 * 16 + 64 * 8) = w1;
                }
            }
        }
        if (any) {
            if (role_p) {
                acc_tr<D>(gl, 0, toff, sd[0], acc);   // dV^T += dO^T P
                acc_tr<D>(gl, 1, toff, sd[1], acc);
            } else {
#pragma unroll
                for (int qb = 0; qb < 2; ++qb) {
                    const uint4 w0 = *reinterpret_cast<const uint4 *>(pxw + qb * 64 * 16);
                    const uint4 w1 = *reinterpret_cast<const uint4 *>(pxw + qb * 64 * 16 + 64 * 8);
                    const uint32_t wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const int r0 = 32 * qb + 8 * u + 4 * g;
                        float4 st0 = make_float4(0.f, 0.f, 0.f, 0.f), st1 = st0;
                        if (MODE == 1) {
                            st0 = *reinterpret_cast<const float4 *>(stl + 2 * r0);
                            st1 = *reinterpret_cast<const float4 *>(stl + 2 * r0 + 4);
                        }
                        const float dlv[4] = {st0.y, st0.w, st1.y, st1.w};
#pragma unroll
                        for (int e4 = 0; e4 < 4; ++e4) {
                            const int e = 4 * u + e4;
                            const f16x2_t h2 = __builtin_bit_cast(f16x2_t, wv[e >> 1]);
                            const float pe = (float)h2[e & 1];
                            sd[qb][e] = MODE == 0 ? sd[qb][e] * fmaf(-pe, pe, pe)
                                                  : pe * (sd[qb][e] - dlv[e4]);
                        }
                    }
                    acc_tr<D>(ql, qb, toff, sd[qb], acc);   // dK~^T += Q~^T dX
                }
            }
        }
    };

    load(0, lds);
    __syncthreads();
    // iteration n: the P role forms and publishes P of step n and adds dV; the dX role takes
    // step n - 1, whose P was published before the last barrier; stage n + 1 loads meanwhile.
    // One barrier per iteration: it publishes P(n) and frees stage n - 1 and P buffer n - 1.
    for (int n = 0; n <= n_steps; ++n) {
        const int my = role_p ? n : n - 1;   // the step this wavefront works on
        uint16_t *const fill = lds + ((n + 1) % 3) * STAGE;
        if (my < 0 || my >= n_steps) {
            if (n + 1 < n_steps) load(n + 1, fill);
            __syncthreads();
            continue;
        }
        // this lane's P of row block qb: values 0..7 at pxw + qb * 1024, 8..15 at + 512
        work(n, my, fill, lds + (my % 3) * STAGE, px0 + (my & 1) * PX + (kw * 2) * 64 * 16 + lane * 8);
        __syncthreads();
    }

    // ---- epilogue: the P role owns dv, the dX role dk
    float *sink = role_p ? p.sink_v : p.sink_k;
    if (SINK) {
        // this split's partial into its own slot, summed in split order below
        if (!active) return;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int d = 32 * db + 8 * (e >> 2) + 4 * g + (e & 3);
                sink[sink_slot_d<D>(p, b, hkv, split, j) + d] = acc[db][e];
            }
        return;
    }
    if (j >= N) return;
    if (sink != nullptr && kblk < p.sink_blocks) {
        f32x16_t part[DB];
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int e = 0; e < 16; ++e) part[db][e] = 0.0f;
        for (int sp = 0; sp < p.n_splits; ++sp)
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int d = 32 * db + 8 * (e >> 2) + 4 * g + (e & 3);
                    part[db][e] += sink[sink_slot_d<D>(p, b, hkv, sp, j) + d];
                }
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[db][e] += part[db][e];
    }
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int d0 = 32 * db + 8 * r + 4 * g;
            float x0 = acc[db][4 * r], x1 = acc[db][4 * r + 1];
            float x2 = acc[db][4 * r + 2], x3 = acc[db][4 * r + 3];
            if (!role_p) {
                // sigmoid accumulated dK against the query image scaled by -cs
                const float dks = MODE == 0 ? -p.scale / p.cs : p.scale;
                x0 *= dks; x1 *= dks; x2 *= dks; x3 *= dks;
                if (p.rope != nullptr) {
                    const float4 c = as_float4(ldg16(p.rope + ((int64_t)j * (D / 2) + d0 / 2) * 2));
                    const float2 u0 = unrotate(x0, x1, make_float2(c.x, c.y));
                    const float2 u1 = unrotate(x2, x3, make_float2(c.z, c.w));
                    x0 = u0.x; x1 = u0.y; x2 = u1.x; x3 = u1.y;
                }
            }
            void *dst = role_p ? p.dv : p.dk;
            const int64_t off = (((int64_t)b * p.N + j) * p.Hkv + hkv) * D + d0;
            store_out4<false>(dst, p.out_bf16, off, x0, x1, x2, x3);
        }
}

// ---------------------------------------------------------------------------------------
// Host side.
struct BwdPlan {
    int64_t n_tiles;
    size_t kv_img, q_img, stats, sink;   // bytes of each workspace part
    int sink_blocks, n_splits, split_tiles;
};

BwdPlan bwd_plan(const PrefillArgs &a) {
    BwdPlan pl;
    pl.n_tiles = (a.N + BK - 1) / BK;
    pl.kv_img = (size_t)(a.B * a.Hkv * pl.n_tiles) * BK * (size_t)a.d * 2;
    pl.q_img = (size_t)(a.B * a.Hq * pl.n_tiles) * BK * (size_t)a.d * 2;
    pl.stats = a.mode == 1 ? (size_t)(a.B * a.Hq * pl.n_tiles) * BK * 2 * sizeof(float) : 0;
    const int64_t KP = 128;
    const int64_t w = a.w < a.N ? a.w : a.N, s = a.s < a.N ? a.s : a.N;
    // queries past every window pair of sink block 0 (the longest such range)
    const int64_t beyond = a.N - (KP - 1 + w);
    pl.sink_blocks = 0; pl.n_splits = 0; pl.split_tiles = 16;
    if (s > 0 && beyond > 0) {
        pl.sink_blocks = (int)((s + KP - 1) / KP);
        pl.n_splits = (int)((beyond + pl.split_tiles * BK - 1) / (pl.split_tiles * BK));
    }
    // one partial per split (summed in split order: deterministic)
    pl.sink = pl.sink_blocks ? 2 * (size_t)(a.B * a.Hkv * pl.n_splits * pl.sink_blocks * KP) *
                                   a.d * sizeof(float)
                             : 0;
    return pl;
}

int gp_of(int64_t G) { return G % 4 == 0 ? 4 : (G % 2 == 0 ? 2 : 1); }

template <int D, int MODE, bool ALIBI>
hipError_t launch_kernels(const BwdParams &bp, int n_dq, int n_dkv, int n_sink, int GP,
                          hipStream_t st) {
    if (D == 128) {
        // two wavefronts per 32-key block (see bwd_dkv2_kernel)
        if (n_sink > 0)
            hipLaunchKernelGGL((bwd_dkv2_kernel<D, MODE, ALIBI, true>), dim3((unsigned)n_sink),
                               dim3(512), 0, st, bp);
        hipLaunchKernelGGL((bwd_dkv2_kernel<D, MODE, ALIBI, false>), dim3((unsigned)n_dkv),
                           dim3(512), 0, st, bp);
    } else {
        if (n_sink > 0)
            hipLaunchKernelGGL((bwd_dkv_kernel<D, MODE, ALIBI, true>), dim3((unsigned)n_sink),
                               dim3(256), 0, st, bp);
        hipLaunchKernelGGL((bwd_dkv_kernel<D, MODE, ALIBI, false>), dim3((unsigned)n_dkv),
                           dim3(256), 0, st, bp);
    }
    if constexpr (!(D == 128 && ALIBI)) {   // (the host never picks four heads there)
        if (GP == 4) {
            hipLaunchKernelGGL((bwd_dq_kernel<D, 4, MODE, ALIBI>), dim3((unsigned)n_dq), dim3(256), 0, st, bp);
            return hipGetLastError();
        }
    }
    if (GP == 2)
        hipLaunchKernelGGL((bwd_dq_kernel<D, 2, MODE, ALIBI>), dim3((unsigned)n_dq), dim3(256), 0, st, bp);
    else
        hipLaunchKernelGGL((bwd_dq_kernel<D, 1, MODE, ALIBI>), dim3((unsigned)n_dq), dim3(256), 0, st, bp);
    return hipGetLastError();
}

template <int D>
hipError_t launch_bwd_d(const PrefillArgs &a, const BwdPlan &pl, const void *q, const void *k,
                        const void *v, const void *o, const float *lse, const void *dout,
                        void *dq, void *dk, void *dv, void *ws, hipStream_t st) {
    uint8_t *w8 = static_cast<uint8_t *>(ws);
    uint16_t *kimg = reinterpret_cast<uint16_t *>(w8);
    uint16_t *vimg = reinterpret_cast<uint16_t *>(w8 + pl.kv_img);
    uint16_t *qimg = reinterpret_cast<uint16_t *>(w8 + 2 * pl.kv_img);
    uint16_t *gimg = reinterpret_cast<uint16_t *>(w8 + 2 * pl.kv_img + pl.q_img);
    float *stats = pl.stats ? reinterpret_cast<float *>(w8 + 2 * pl.kv_img + 2 * pl.q_img) : nullptr;
    float *sink = pl.sink ? reinterpret_cast<float *>(w8 + 2 * pl.kv_img + 2 * pl.q_img + pl.stats)
                          : nullptr;
    const bool rot = a.rope != nullptr;
    const int nt = (int)pl.n_tiles;
    {
        PackKV pk = {};
        pk.k = static_cast<const uint16_t *>(k); pk.v = static_cast<const uint16_t *>(v);
        pk.kimg = kimg; pk.vimg = vimg; pk.rope = a.rope; pk.N = a.N; pk.Hkv = a.Hkv;
        pk.n_tiles = nt;
        const unsigned nb = (unsigned)(a.B * nt * ((a.Hkv + 3) / 4));
        if (rot) hipLaunchKernelGGL((bwd_pack_kv_kernel<D, true>), dim3(nb), dim3(256), 0, st, pk);
        else hipLaunchKernelGGL((bwd_pack_kv_kernel<D, false>), dim3(nb), dim3(256), 0, st, pk);
    }
    {
        PackQ pq = {};
        pq.q = static_cast<const uint16_t *>(q); pq.dout = dout; pq.o = o; pq.lse = lse;
        pq.qimg = qimg; pq.gimg = gimg; pq.stats = stats; pq.rope = a.rope; pq.N = a.N;
        pq.Hq = a.Hq; pq.n_tiles = nt;
        pq.qs = a.mode == 0 ? -a.scale * LOG2E : 1.0f;
        const unsigned nb = (unsigned)(a.B * nt * ((a.Hq + 3) / 4) * BT<D>::KPT);
#define SWA_PACKQ(R, O, M) hipLaunchKernelGGL((bwd_pack_q_kernel<D, R, O, M>), dim3(nb), dim3(256), 0, st, pq)
        if (a.mode == 1) {
            if (rot) { if (a.out_dt == 1) SWA_PACKQ(true, 1, 1); else SWA_PACKQ(true, 0, 1); }
            else { if (a.out_dt == 1) SWA_PACKQ(false, 1, 1); else SWA_PACKQ(false, 0, 1); }
        } else {
            if (rot) { if (a.out_dt == 1) SWA_PACKQ(true, 1, 0); else SWA_PACKQ(true, 0, 0); }
            else { if (a.out_dt == 1) SWA_PACKQ(false, 1, 0); else SWA_PACKQ(false, 0, 0); }
        }
#undef SWA_PACKQ
    }
    if (sink) {
        const int64_t n = (int64_t)(pl.sink / sizeof(float));
        hipLaunchKernelGGL(zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, sink, n);
    }
    const int64_t G = a.Hq / a.Hkv;
    // four query heads per dq workgroup at d = 128 with ALiBi would keep more state than its
    // registers hold (it spilled 19-24 registers to scratch): two heads per workgroup there
    const int GP = (D == 128 && a.slopes != nullptr && gp_of(G) == 4) ? 2 : gp_of(G);
    const int64_t QP = 32 * 4 / GP;
    BwdParams bp = {};
    bp.kimg = kimg; bp.vimg = vimg; bp.qimg = qimg; bp.gimg = gimg; bp.stats = stats;
    bp.slopes = a.slopes; bp.rope = a.rope;
    bp.dq = dq; bp.dk = dk; bp.dv = dv;
    bp.sink_k = sink;
    bp.sink_v = sink ? sink + pl.sink / sizeof(float) / 2 : nullptr;
    bp.N = a.N; bp.Hq = a.Hq; bp.Hkv = a.Hkv; bp.G = G;
    bp.n_tiles = nt;
    bp.n_qtiles = (int)((a.N + QP - 1) / QP);
    bp.n_hgroups = (int)(G / GP);
    bp.n_kblocks = (int)((a.N + 127) / 128);
    bp.sink_blocks = pl.sink_blocks; bp.n_splits = pl.n_splits; bp.split_tiles = pl.split_tiles;
    bp.w = (int)(a.w < a.N ? a.w : a.N);
    bp.s = (int)(a.s < a.N ? a.s : a.N);
    bp.cs = a.scale * LOG2E;
    bp.scale = a.scale;
    bp.out_bf16 = a.out_dt == 1;
    const int n_dq = (int)(a.B * a.Hkv * bp.n_hgroups * bp.n_qtiles);
    const int n_dkv = (int)(a.B * a.Hkv * bp.n_kblocks);
    const int n_sink = (int)(a.B * a.Hkv * pl.sink_blocks * pl.n_splits);
    const bool alibi = a.slopes != nullptr;
    if (a.mode == 1)
        return alibi ? launch_kernels<D, 1, true>(bp, n_dq, n_dkv, n_sink, GP, st)
                     : launch_kernels<D, 1, false>(bp, n_dq, n_dkv, n_sink, GP, st);
    return alibi ? launch_kernels<D, 0, true>(bp, n_dq, n_dkv, n_sink, GP, st)
                 : launch_kernels<D, 0, false>(bp, n_dq, n_dkv, n_sink, GP, st);
}

}  // namespace

size_t prefill_bwd_workspace_bytes(const PrefillArgs &a) {
    if (a.B * a.N == 0) return 0;
    const BwdPlan pl = bwd_plan(a);
    return 2 * pl.kv_img + 2 * pl.q_img + pl.stats + pl.sink;
}

hipError_t launch_prefill_bwd(const PrefillArgs &a, const void *q, const void *k,
                              const void *v, const void *o, const float *lse, const void *dout,
                              void *dq, void *dk, void *dv, void *ws, hipStream_t st) {
    if (a.B * a.N == 0) return hipSuccess;
    const BwdPlan pl = bwd_plan(a);
    return a.d == 64 ? launch_bwd_d<64>(a, pl, q, k, v, o, lse, dout, dq, dk, dv, ws, st)
                     : launch_bwd_d<128>(a, pl, q, k, v, o, lse, dout, dq, dk, dv, ws, st);
}

}  // namespace swa
