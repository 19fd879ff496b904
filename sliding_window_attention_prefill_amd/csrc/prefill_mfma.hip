// prefill_mfma.hip - banded matrix-core prefill for bfloat16 inputs, d in {64, 128}.
//
// What it computes (SWAT: Sliding Window Attention Training, "Putting It Together" attention
// equation with the balanced ALiBi bias, "Sigmoid: Dense Attention Without Suppression";
// Sliding Window Attention glossary, band mask; Sliding-window beats linear attention,
// SWA(w, s)):
//   o_i = sum_{j in K(i)} p(x_ij) v_j,  x_ij = scale (R(i)q_i).(R(j)k_j) + slope_h (i - j),
//   K(i) = { j <= i : i - j < w or j < s },  p = sigmoid (no normalisation) or softmax.
//
// How (gfx950):
//   * One workgroup of 4 wavefronts owns 32 query rows per wavefront: positions x GP query
//     heads that share one kv head, so each K/V tile in LDS serves the whole group and is
//     fetched by fewer workgroups.
//   * It walks only the 64-key tiles that intersect its band of keys, plus the sink tiles the
//     window no longer covers (the block skipping the glossary describes for windowed
//     exact-attention kernels). Tiles inside every row's key set run without the element
//     predicate.
//   * Each wavefront computes S^T = K Q^T (32 keys x 32 queries per 32x32x16 matrix
//     instruction), so a lane holds one query's scores; q enters scaled by scale x log2(e)
//     (negated for sigmoid), so the product is a base-2 logit; sigmoid is 1 / (1 + 2^t),
//     softmax is online with a lazily rescaled accumulator. O^T += V^T P^T takes the
//     weights straight from registers.
//   * Score operands are float16: q and k are widened from bf16, rotated in float32 and
//     rounded once; values past the float16 range saturate at +-65504.
//   * A pre-pass rotates every key once into float16 tile images laid out exactly as LDS
//     holds them (for softmax it also stores V transposed, as float16 images of V^T); the
//     main kernel copies tiles with buffer-to-LDS transfers, which take no registers and no
//     vector instructions. Sigmoid reads V rows as stored (bf16) with the same transfers,
//     and its second product runs in bf16 with the weights rounded to bf16; those rows stay
//     row-major in LDS and the transposing LDS read (ds_read_b64_tr_b16) delivers them in
//     the operand layout of the second product. Softmax's second product runs in float16 and
//     reads the V^T tile with plain 16-byte LDS reads (twice the bytes per read of the
//     transposing one), its keys stored in the order of the score registers.
//   * ALiBi: the key part of the bias enters the score accumulator through one more matrix
//     instruction per 32-key block (exact key offsets against a two-term float16 split of
//     the slope). Softmax adds the query part with one add per score; sigmoid carries it in
//     two more k-slots of the same instruction, so its scores need no vector work before
//     the weights.
//   * LDS rows are XOR-swizzled in 16-byte chunks so that the row reads of K and the
//     transposing reads of V are free of bank conflicts; the register path, the transfers
//     and the pre-pass all write that swizzle.
//   * LDS is double-buffered: the next tile's loads are issued before the current tile's
//     math.
//   * The output goes through LDS so that every global store writes whole rows.
//   * Workgroups are numbered so that each of the 8 XCDs walks a contiguous run of query
//     tiles of the same (batch, kv head), keeping shared K/V tiles in that XCD's L2. Within
//     a run the tiles go in sequence order, so workgroups dispatched one after another read
//     each K/V tile a short time apart, except that the first tiles of the sequence (whose
//     bands the sequence start cuts short) come last, longest first: short work then fills
//     the end of the grid instead of its start.
#include "mfma_common.hpp"
#include "swa_kernels.hpp"

namespace swa {
namespace {

template <int D>
struct Tile {
    static constexpr int NW = 4;                         // wavefronts per workgroup
    static constexpr bool PIPE = D == 128;               // software-pipelined tile loop
    static constexpr int C = D / 8;                      // 16-byte chunks per row
    static constexpr int IMG = BK * D;                   // 16-bit elements of a K or V tile
    static constexpr int IMG_BYTES = IMG * 2;
    static constexpr int DMA_W = IMG_BYTES / (NW * 1024); // 1 KB transfers per wavefront
    static constexpr int KPT = BK * C / 256;             // chunks per thread of the pre-pass
    static constexpr int OSTR = D + 4;                   // floats per output row in LDS
    // four wavefronts stage their output rows at a time
    static constexpr int LDS_BYTES = cmax(2 * 2 * IMG_BYTES, 4 * 32 * OSTR * 4);
};

// Chunk swizzles: chunk c of tile row r is stored at chunk c ^ swz(r) of that row.
// K rows are read 16 rows at one chunk; V is read 4 rows x 4 chunks per 32 lanes.
template <int D>
__host__ __device__ __forceinline__ constexpr int kswz(int r) {
    return D == 64 ? (r >> 1) & 7 : r & 15;
}
template <int D>
__host__ __device__ __forceinline__ constexpr int vswz(int r) {
    return D == 64 ? ((r >> 1) & 1) << 2 : (r & 3) << 2;
}

// Transposed value tiles (softmax): V^T, one row of the 64 keys per head dimension d,
// float16. The second product takes V^T as its A operand, 8 consecutive k per lane, and
// the k order of a 16-key step t must be the key order of the weights, which the score
// registers hold as keys 16 t + 4 g + {0..3, 8..11} for lane half g. So within each
// 16-key group the row stores the keys in the order 0-3, 8-11, 4-7, 12-15: stored position
// p holds key vt_key(p), and lane half g of step t reads the 16 bytes at position 16 t + 8 g.
// Chunk c (8 positions) of row d sits at chunk c ^ vtswz(d): the 16 rows one read covers at
// one chunk then fall on 16 distinct bank groups.
__host__ __device__ __forceinline__ constexpr int vt_key(int p) {
    return (p & ~15) + ((p >> 3) & 1) * 4 + (p & 3) + ((p >> 2) & 1) * 8;
}
__host__ __device__ __forceinline__ constexpr int vtswz(int d) { return (d >> 1) & 7; }
// element offset of chunk c of row d in a transposed tile image
__host__ __device__ __forceinline__ constexpr int vt_slot(int d, int c) {
    return (d * 8 + (c ^ vtswz(d))) * 8;
}

// A chunked call (prefill over the ring cache): sequence b owns the packed rows
// cu[b] .. cu[b+1]-1, the tokens at positions pos0[b], pos0[b] + 1, ...
struct ChunkGeom {
    const int32_t *cu, *pos0;
    int64_t T;        // packed rows of q, k_new, v_new and o
    int max_q;        // rows of the longest sequence the launch covers
    int pos_limit;    // positions must stay below this (rotation table rows, float-exact)
    int w;            // window (clamped to the position range)
    int ns_img;       // sink tiles at the front of every sequence's tile images
};

// Where sequence b's rows and key tiles are. Its images hold the sink tiles [0, ns_img)
// (whole 64-position tiles) and then the window tiles the chunk's queries can reach,
// [max(lo, ns_img), hi) with lo the tile of position p0 - w + 1 and hi the tile past the
// chunk's last position; window tile t >= ns_img is image tile t - shift.
struct ChunkSeq {
    bool rows_ok;     // the row range lies inside [0, T): rows may be written
    bool valid;       // the sequence runs (else its rows become NaN, its cache is untouched)
    int p0, n;
    int64_t row0;
    int shift, n_img;
};

__device__ __forceinline__ ChunkSeq chunk_seq(const ChunkGeom &g, int64_t b) {
    ChunkSeq c;
    const int64_t c0 = g.cu[b], c1 = g.cu[b + 1], p0 = g.pos0[b];
    c.rows_ok = c0 >= 0 && c0 <= c1 && c1 <= g.T;
    c.valid = c.rows_ok && p0 >= 0 && c1 - c0 <= g.max_q && p0 + (c1 - c0) <= g.pos_limit;
    c.p0 = (int)p0;
    c.n = (int)(c1 - c0);
    c.row0 = c0;
    c.shift = 0;
    c.n_img = 0;
    if (c.valid) {
        const int lo_pos = c.p0 - g.w + 1 > 0 ? c.p0 - g.w + 1 : 0;
        const int lo = lo_pos / BK > g.ns_img ? lo_pos / BK : g.ns_img;
        const int hi = (c.p0 + c.n + BK - 1) / BK;
        c.shift = lo - g.ns_img;
        c.n_img = g.ns_img + (hi > lo ? hi - lo : 0);
    }
    return c;
}

struct MfmaParams {
    const uint16_t *q, *k, *v;
    const uint16_t *kimg, *vimg;  // packed tile images, or null
    void *o;
    const float *slopes;
    const float *rope;
    int64_t N, Hq, Hkv, G;
    int n_qtiles, n_hgroups, n_ktiles;
    int w, s;                 // window extent in positions and sinks, clamped to N
    int dmask;                // dilation - 1 (the window keeps every dilation-th position)
    float cs;                 // scale * log2(e)
    uint32_t kv_bytes;        // bytes of one (batch, kv head) K or V slice, rows [0, N)
    uint32_t row_bytes;       // bytes between consecutive positions of K/V
    int out_bf16;
    int chunked;              // 1: rows and positions per sequence from cg; V from vimg
    ChunkGeom cg;
    float *lse;               // softmax row log-normalisers [B, Hq, N_mem] (natural log), or null
    // whole sequences: query/key i is memory row b N_mem + pos_off + pos_stride i at position
    // pos_off + pos_stride i, and ALiBi slopes are multiplied by slope_mul (one residue class
    // of a dilated window: pos_stride = r, slope_mul = r; else 0, 1, N, 1)
    int64_t N_mem;
    int pos_off, pos_stride;
    float slope_mul;
};

struct PackParams {
    const uint16_t *k, *v;
    uint16_t *kimg, *vimg;
    const float *rope;
    int64_t N, Hkv;
    int n_ktiles;
    // key j of the (strided) sequence is memory row b N_mem + pos_off + pos_stride j and
    // position pos_off + pos_stride j (a residue class of a dilated window; else 0, 1, N)
    int64_t N_mem;
    int pos_off, pos_stride;
};

// ---------------------------------------------------------------------------------------
// Pre-pass: every 64-key tile, once, into its LDS image. One block per (batch, tile, part of
// the tile, group of up to four kv heads), each thread one 16-byte chunk per head: the
// rotation angles of a position are read once for the group, and the grid holds several
// rounds of blocks, so that the loads of later blocks overlap the stores of earlier ones.
// K image: rotated (or converted) float16; V image (PACK_V): converted float16. Rows past
// the sequence end are zero.
constexpr int PACK_HG = 4;  // kv heads per pre-pass block

template <int D, bool ROT, bool PACK_V>
__global__ __launch_bounds__(256) void prefill_pack_kernel(PackParams p) {
    using T = Tile<D>;
    const int n_hg = (int)((p.Hkv + PACK_HG - 1) / PACK_HG);
    const int bid = blockIdx.x, tid = threadIdx.x;
    const int hg = bid % n_hg;
    const int rest0 = bid / n_hg;
    const int pt = rest0 % T::KPT;           // this block's chunks: 256 pt .. 256 pt + 255
    const int rest = rest0 / T::KPT;
    const int jt = rest % p.n_ktiles;
    const int64_t b = rest / p.n_ktiles;
    const int64_t h0 = (int64_t)hg * PACK_HG;
    const int nh = p.Hkv - h0 < PACK_HG ? (int)(p.Hkv - h0) : PACK_HG;
    constexpr int R = 1;
    if constexpr (!PACK_V) {
        // keys only: every load of the block is issued before the first store (the images
        // may not be assumed disjoint from the inputs, so a store would order later loads
        // after it)
        uint4 xk[R][PACK_HG];
        float4 t0[R], t1[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int cidx = tid + 256 * (r + pt), row = cidx / T::C, c = cidx % T::C;
            const int64_t j = (int64_t)jt * BK + row;
            const bool in = j < p.N;
            t0[r] = make_float4(1.f, 0.f, 1.f, 0.f);
            t1[r] = t0[r];
            const int64_t pos = p.pos_off + (int64_t)p.pos_stride * j;
            if (ROT && in) {
                const float *t = p.rope + (pos * (D / 2) + c * 4) * 2;
                t0[r] = as_float4(ldg16(t));
                t1[r] = as_float4(ldg16(t + 4));
            }
#pragma unroll
            for (int u = 0; u < PACK_HG; ++u) {
                xk[r][u] = make_uint4(0, 0, 0, 0);
                if (in && u < nh) xk[r][u] = ldg16(p.k + ((b * p.N_mem + pos) * p.Hkv + h0 + u) * D + c * 8);
            }
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int cidx = tid + 256 * (r + pt), row = cidx / T::C, c = cidx % T::C;
            const int kslot = (row * T::C + (c ^ kswz<D>(row))) * 8;
#pragma unroll
            for (int u = 0; u < PACK_HG; ++u) {
                if (u >= nh) break;
                const int64_t img = ((b * p.Hkv + h0 + u) * p.n_ktiles + jt) * T::IMG;
                stg16(p.kimg + img + kslot, ROT ? rotate_chunk(xk[r][u], t0[r], t1[r]) : convert_chunk(xk[r][u]));
            }
        }
    } else {
        // keys as above; values transposed through LDS: this block's part holds head
        // dimensions [DP pt, DP pt + DP) of all 64 keys
        constexpr int DP = D / T::KPT;               // 32 head dimensions per part
        constexpr int TPR = DP / 8;                  // threads per key row (16-byte chunks)
        __shared__ __attribute__((aligned(16))) uint16_t tr[PACK_HG][DP][BK];
        {
            const int cidx = tid + 256 * pt, row = cidx / T::C, c = cidx % T::C;
            const int64_t j = (int64_t)jt * BK + row;
            const bool in = j < p.N;
            const int64_t pos = p.pos_off + (int64_t)p.pos_stride * j;
            float4 t0 = make_float4(1.f, 0.f, 1.f, 0.f), t1 = t0;
            if (ROT && in) {
                const float *t = p.rope + (pos * (D / 2) + c * 4) * 2;
                t0 = as_float4(ldg16(t));
                t1 = as_float4(ldg16(t + 4));
            }
            const int vr = tid / TPR, vd = DP * pt + 8 * (tid % TPR);   // value row, dims
            const int64_t jv = (int64_t)jt * BK + vr;
            uint4 xk[PACK_HG], xv[PACK_HG];
#pragma unroll
            for (int u = 0; u < PACK_HG; ++u) {
                xk[u] = xv[u] = make_uint4(0, 0, 0, 0);
                const int64_t posv = p.pos_off + (int64_t)p.pos_stride * jv;
                if (u < nh && in) xk[u] = ldg16(p.k + ((b * p.N_mem + pos) * p.Hkv + h0 + u) * D + c * 8);
                if (u < nh && jv < p.N) xv[u] = ldg16(p.v + ((b * p.N_mem + posv) * p.Hkv + h0 + u) * D + vd);
            }
            const int kslot = (row * T::C + (c ^ kswz<D>(row))) * 8;
#pragma unroll
            for (int u = 0; u < PACK_HG; ++u) {
                if (u >= nh) break;
                const int64_t img = ((b * p.Hkv + h0 + u) * p.n_ktiles + jt) * T::IMG;
                stg16(p.kimg + img + kslot, ROT ? rotate_chunk(xk[u], t0, t1) : convert_chunk(xk[u]));
                const uint4 f = convert_chunk(xv[u]);
                const uint32_t w4[4] = {f.x, f.y, f.z, f.w};
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    tr[u][vd - DP * pt + 2 * m][vr] = (uint16_t)(w4[m] & 0xffffu);
                    tr[u][vd - DP * pt + 2 * m + 1][vr] = (uint16_t)(w4[m] >> 16);
                }
            }
        }
        __syncthreads();
        {
            // thread: head dimension DP pt + tid / 8, stored chunk tid % 8 (positions 8 c ..
            // 8 c + 7: keys 16 (c / 2) + 4 (c % 2) + {0..3, 8..11})
            const int dl = tid / 8, c = tid % 8;
            const int k0 = 16 * (c >> 1) + 4 * (c & 1);
            const int d = DP * pt + dl;
#pragma unroll
            for (int u = 0; u < PACK_HG; ++u) {
                if (u >= nh) break;
                const uint2 lo = *reinterpret_cast<const uint2 *>(&tr[u][dl][k0]);
                const uint2 hi = *reinterpret_cast<const uint2 *>(&tr[u][dl][k0 + 8]);
                const int64_t img = ((b * p.Hkv + h0 + u) * p.n_ktiles + jt) * T::IMG;
                stg16(p.vimg + img + vt_slot(d, c), make_uint4(lo.x, lo.y, hi.x, hi.y));
            }
        }
    }
}

// ---------------------------------------------------------------------------------------
// Chunked calls. The gather pre-pass builds each sequence's tile images from three sources:
// position j >= p0 is the chunk's own row (key rotated here), p0 - w <= j < p0 is the ring
// slot j mod w (keys stored rotated), j < s the sink store; anything else (positions no query
// of the chunk can see, or past the chunk) is zero. K images are float16 with the K swizzle;
// V images are float16 with the V swizzle (softmax) or bf16 row-major without swizzle
// (sigmoid, read by the same transfers as V input rows).
struct GatherParams {
    ChunkGeom cg;
    const uint16_t *k_new, *v_new;    // [T, Hkv, D]
    const uint16_t *k_ring, *v_ring;  // [S, Hkv, w_ring, D]
    const uint16_t *k_sink, *v_sink;  // [S, Hkv, s, D]
    uint16_t *kimg, *vimg;
    const float *rope;
    int64_t Hkv, w_ring, s;
    int n_ktiles;                      // image tiles per (sequence, kv head)
};

template <int D, bool ROT, bool VF16>
__global__ __launch_bounds__(256) void chunk_gather_kernel(GatherParams p) {
    using T = Tile<D>;
    // softmax: the values of each head go through LDS to be stored transposed
    __shared__ __attribute__((aligned(16))) uint16_t tr[VF16 ? PACK_HG : 1][VF16 ? D : 1][BK];
    const int n_hg = (int)((p.Hkv + PACK_HG - 1) / PACK_HG);
    const int bid = blockIdx.x, tid = threadIdx.x;
    const int hg = bid % n_hg;
    const int rest = bid / n_hg;
    const int u = rest % p.n_ktiles;
    const int64_t b = rest / p.n_ktiles;
    const ChunkSeq cs = chunk_seq(p.cg, b);
    if (!cs.valid || u >= cs.n_img) return;
    const int64_t t = u < p.cg.ns_img ? u : u + cs.shift;
    const int64_t h0 = (int64_t)hg * PACK_HG;
    const int nh = p.Hkv - h0 < PACK_HG ? (int)(p.Hkv - h0) : PACK_HG;
#pragma unroll
    for (int r = 0; r < T::KPT; ++r) {
        const int cidx = tid + 256 * r, row = cidx / T::C, c = cidx % T::C;
        const int64_t j = t * BK + row;
        // 0: zero, 1: chunk row, 2: ring slot, 3: sink entry
        const int src = j >= cs.p0 + cs.n ? 0
                        : j >= cs.p0 ? 1
                        : (j >= cs.p0 - p.w_ring && j >= 0) ? 2
                        : j < p.s ? 3 : 0;
        float4 t0 = make_float4(1.f, 0.f, 1.f, 0.f), t1 = t0;
        if (ROT && src == 1) {
            const float *tb = p.rope + (j * (D / 2) + c * 4) * 2;
            t0 = as_float4(ldg16(tb));
            t1 = as_float4(ldg16(tb + 4));
        }
        const int kslot = (row * T::C + (c ^ kswz<D>(row))) * 8;
        const int vslot = (row * T::C + c) * 8;
        // the row's loads for every head first, then its stores
        const uint16_t *ksrc = src == 1 ? p.k_new : src == 2 ? p.k_ring : p.k_sink;
        const uint16_t *vsrc = src == 1 ? p.v_new : src == 2 ? p.v_ring : p.v_sink;
        uint4 xk[PACK_HG], xv[PACK_HG];
#pragma unroll
        for (int e = 0; e < PACK_HG; ++e) {
            const int64_t hkv = h0 + e;
            xk[e] = xv[e] = make_uint4(0, 0, 0, 0);
            if (src != 0 && e < nh) {
                const int64_t off =
                    src == 1 ? ((cs.row0 + (j - cs.p0)) * p.Hkv + hkv) * D + c * 8
                    : src == 2 ? ((b * p.Hkv + hkv) * p.w_ring + j % p.w_ring) * D + c * 8
                               : ((b * p.Hkv + hkv) * p.s + j) * D + c * 8;
                xk[e] = ldg16(ksrc + off);
                xv[e] = ldg16(vsrc + off);
            }
        }
#pragma unroll
        for (int e = 0; e < PACK_HG; ++e) {
            if (e >= nh) break;
            // chunk rows are rotated here; ring and sink keys are stored rotated
            const uint4 k = (ROT && src == 1) ? rotate_chunk(xk[e], t0, t1) : convert_chunk(xk[e]);
            const int64_t img = ((b * p.Hkv + h0 + e) * p.n_ktiles + u) * T::IMG;
            stg16(p.kimg + img + kslot, k);
            if constexpr (VF16) {
                const uint4 f = convert_chunk(xv[e]);
                const uint32_t w4[4] = {f.x, f.y, f.z, f.w};
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    tr[e][8 * c + 2 * m][row] = (uint16_t)(w4[m] & 0xffffu);
                    tr[e][8 * c + 2 * m + 1][row] = (uint16_t)(w4[m] >> 16);
                }
            } else {
                stg16(p.vimg + img + vslot, xv[e]);
            }
        }
    }
    if constexpr (VF16) {
        // the transposed value images: D rows of 8 stored chunks per head
        __syncthreads();
#pragma unroll
        for (int r = 0; r < D * 8 / 256; ++r) {
            const int oc = tid + 256 * r, d = oc / 8, c = oc % 8;
            const int k0 = 16 * (c >> 1) + 4 * (c & 1);
#pragma unroll
            for (int e = 0; e < PACK_HG; ++e) {
                if (e >= nh) break;
                const uint2 lo = *reinterpret_cast<const uint2 *>(&tr[e][d][k0]);
                const uint2 hi = *reinterpret_cast<const uint2 *>(&tr[e][d][k0 + 8]);
                const int64_t img = ((b * p.Hkv + h0 + e) * p.n_ktiles + u) * T::IMG;
                stg16(p.vimg + img + vt_slot(d, c), make_uint4(lo.x, lo.y, hi.x, hi.y));
            }
        }
    }
}

// After the attention, the chunk joins the cache: row r of a sequence with n rows goes to
// ring slot (p0 + r) mod w when it is among the last w rows (a later row of the same call
// would overwrite it), and to the sink store when p0 + r < s. Keys are rotated at their
// position in float32 and rounded once to bf16, as the single-token append stores them.
// Eight blocks per (sequence, 64 rows), taking interleaved runs of the tile's 16-byte chunks;
// a thread moves 8 elements of one (row, kv head) per chunk.
struct ChunkAppendParams {
    ChunkGeom cg;
    const uint16_t *k_new, *v_new;
    uint16_t *k_ring, *v_ring, *k_sink, *v_sink;
    const float *rope;
    int64_t Hkv, w_ring, s;
    int n_rtiles;                      // 64-row tiles per sequence in the grid
    int n_parts;                       // blocks per (sequence, 64-row tile)
};

__device__ __forceinline__ uint32_t rotate_pair_bf16(uint32_t w, float c, float s) {
    const float a = __uint_as_float(w << 16);
    const float b = __uint_as_float(w & 0xffff0000u);
    return pack_bf16x2(fmaf(-b, s, a * c), fmaf(a, s, b * c));
}

template <int D>
__global__ __launch_bounds__(256) void chunk_append_kernel(ChunkAppendParams p) {
    constexpr int C = D / 8;
    constexpr int U = 4;   // elements per thread whose loads are in flight together
    const int part = blockIdx.x % p.n_parts;
    const int64_t b = blockIdx.x / p.n_parts / p.n_rtiles;
    const int rt = (blockIdx.x / p.n_parts) % p.n_rtiles;
    const ChunkSeq cs = chunk_seq(p.cg, b);
    if (!cs.valid || rt * BK >= cs.n) return;
    const int rows = cs.n - rt * BK < BK ? cs.n - rt * BK : BK;
    const int64_t per_row = p.Hkv * C;
    const int64_t total = rows * per_row;
    // the parts of a tile take interleaved runs of 256 U elements
    for (int64_t e0 = (int64_t)part * 256 * U + threadIdx.x; e0 < total; e0 += (int64_t)p.n_parts * 256 * U) {
        // loads of U elements first (the ring and sink stores may not be assumed disjoint
        // from the chunk, so a store would hold back the loads behind it)
        uint4 xk[U], xv[U];
        float4 t0[U], t1[U];
        bool live[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t e = e0 + 256 * u;
            const int r = rt * BK + (int)(e / per_row);
            const int64_t pos = (int64_t)cs.p0 + r;
            live[u] = e < total && (r >= cs.n - p.w_ring || pos < p.s);
            xk[u] = xv[u] = make_uint4(0, 0, 0, 0);
            t0[u] = make_float4(1.f, 0.f, 1.f, 0.f);
            t1[u] = t0[u];
            if (live[u]) {
                const int64_t hkv = (e % per_row) / C;
                const int c = (int)(e % C);
                const int64_t src = ((cs.row0 + r) * p.Hkv + hkv) * D + c * 8;
                xk[u] = ldg16(p.k_new + src);
                xv[u] = ldg16(p.v_new + src);
                if (p.rope) {
                    t0[u] = as_float4(ldg16(p.rope + (pos * (D / 2) + c * 4) * 2));
                    t1[u] = as_float4(ldg16(p.rope + (pos * (D / 2) + c * 4) * 2 + 4));
                }
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (!live[u]) continue;
            const int64_t e = e0 + 256 * u;
            const int r = rt * BK + (int)(e / per_row);
            const int64_t hkv = (e % per_row) / C;
            const int c = (int)(e % C);
            const int64_t pos = (int64_t)cs.p0 + r;
            uint4 k = xk[u];
            if (p.rope)
                k = make_uint4(rotate_pair_bf16(k.x, t0[u].x, t0[u].y), rotate_pair_bf16(k.y, t0[u].z, t0[u].w),
                               rotate_pair_bf16(k.z, t1[u].x, t1[u].y), rotate_pair_bf16(k.w, t1[u].z, t1[u].w));
            if (r >= cs.n - p.w_ring) {
                const int64_t dst = ((b * p.Hkv + hkv) * p.w_ring + pos % p.w_ring) * D + c * 8;
                stg16(p.k_ring + dst, k);
                stg16(p.v_ring + dst, xv[u]);
            }
            if (pos < p.s) {
                const int64_t dst = ((b * p.Hkv + hkv) * p.s + pos) * D + c * 8;
                stg16(p.k_sink + dst, k);
                stg16(p.v_sink + dst, xv[u]);
            }
        }
    }
}

// ---------------------------------------------------------------------------------------
// Main kernel pieces.

// Per-lane offsets, fixed for the whole kernel.
template <int D>
struct LaneOffsets {
    int k[D / 16];                   // LDS element offset of the K row read of score step ks
    int v[D / 32];                   // LDS element offset of the V transposing read, block db
    int vt[4];                       // LDS element offset of the V^T read of step t (block 0)
    uint32_t dimg;    // source byte offset of the first transfer in a packed tile image
    uint32_t dvraw;   // source byte offset of the first transfer in the V input rows
    uint32_t dvstep;  // bytes between the V input rows of consecutive transfers
};

// S^T = K Q^T for the 64 keys of one tile at j0 (i: this lane's query). For sigmoid the
// product is the negated base-2 logit t = -x log2(e) itself: q enters scaled by -cs and
// the bias instruction adds -slope log2(e) (i - j), its query part refreshed per tile.
template <int D, int MODE, bool ALIBI>
__device__ __forceinline__ void qk_tile(const uint16_t *__restrict__ kl, const LaneOffsets<D> &lo,
                                        const BiasOperands &bo, const f16x8_t (&qreg)[D / 16],
                                        f32x16_t (&sacc)[2], int i, int j0) {
    if (MODE == 0 && ALIBI) qk_tile_off<D, ALIBI>(kl, lo.k, bo, query_term(bo, i - j0), qreg, sacc);
    else qk_tile_off<D, ALIBI>(kl, lo.k, bo, qreg, sacc);
}

// The largest of three floats in one v_max3_f32. Written as an instruction because the
// compiler would otherwise first quiet each operand (one v_max per operand) when they come
// straight from a matrix instruction; none of them is a signalling NaN here.
__device__ __forceinline__ float max3f(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

// Softmax: the largest base-2 logit of one tile for this lane's query (both lane halves).
// Three-operand steps in four independent chains; the scores come straight from the matrix
// unit and v_max3 takes them as they are.
__device__ __forceinline__ float tile_max(const f32x16_t (&sacc)[2]) {
    float mx[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        mx[u] = max3f(sacc[0][4 * u], sacc[0][4 * u + 1], sacc[0][4 * u + 2]);
        mx[u] = max3f(mx[u], sacc[0][4 * u + 3], sacc[1][4 * u]);
        mx[u] = max3f(mx[u], sacc[1][4 * u + 1], sacc[1][4 * u + 2]);
    }
    float mt = max3f(max3f(mx[0], mx[1], mx[2]), mx[3], sacc[1][3]);
    mt = max3f(mt, sacc[1][7], sacc[1][11]);
    mt = fmaxf(mt, sacc[1][15]);
    // the other lane half holds the query's other 32 keys: exchange the halves in registers
    // (v_permlane32_swap swaps lanes 32..63 of one operand with lanes 0..31 of the other, so
    // the larger of its two results is the maximum over lanes l and l ^ 32)
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt), __float_as_uint(mt),
                                                     false, false);
    return max3f(__uint_as_float(sw[0]), __uint_as_float(sw[1]), mt);
}

// Softmax: fold a tile maximum into the running one. The stale maximum stays while the new
// one exceeds it by less than 8 (weights stay below 2^8); the final division uses the same
// maximum.
template <int D>
__device__ __forceinline__ void fold_max(float mt, f32x16_t (&oacc)[D / 32], float &m_run,
                                         float &l_run) {
    const float m_new = fmaxf(m_run, mt);
    const bool need = m_new > m_run + 8.0f;
    if (__any(need)) {
        const float corr = need ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int e = 0; e < 16; ++e) oacc[db][e] *= corr;
        l_run *= corr;
        m_run = need ? m_new : m_run;
    }
}

// Scores of one tile made ready for weighting (run in the step that formed them): edge
// masking (sigmoid scores are negated logits, so an excluded key gets +inf), and for
// softmax the base-2 logits x log2(e) = acc + bias_q (the product of q scaled by cs; bias_q =
// slope log2(e) (i - j0), zero without ALiBi) with the running maximum and the lazy rescale
// of the accumulator.
template <int D, int MODE, bool ALIBI, bool DIL>
__device__ __forceinline__ void prep_scores(f32x16_t (&sacc)[2], f32x16_t (&oacc)[D / 32],
                                            float &m_run, float &l_run, float cs, float bias_q,
                                            int kind, int dq, int jb, int w, int s, int dmask) {
    // the stride test exists only in the dilated instantiations
    constexpr float fill = MODE == 0 ? INFINITY : -INFINITY;
    if (D == 64 && kind == 3) mask_causal(sacc, dq, fill);
    else if (D == 64 && kind == 4) mask_far(sacc, dq - w, fill);
    else if (kind == 1) mask_tile<false>(sacc, dq, jb, w, s, DIL ? dmask : 0, fill);
    else if (kind == 2) mask_tile<true>(sacc, dq, jb, w, s, DIL ? dmask : 0, fill);
    if (MODE == 1) {
        // the product already is cs x (q.k) minus the bias's key part (q entered scaled by
        // cs); the bias's query part is one add. Excluded keys stay -inf.
        if (ALIBI) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int e = 0; e < 16; ++e) sacc[kb][e] += bias_q;
        }
        fold_max<D>(tile_max(sacc), oacc, m_run, l_run);
    }
}

// Weights of one prepared tile, packed as the B operand of the second product (step t =
// keys 16t..16t+15: this lane's P^T elements are sacc[t/2][8(t%2) + 0..7] = keys
// 16t + 4g + {0..3, 8..11}); for softmax the row sum, taken from the packed weights as the
// second product sees them (float16), two per instruction.
template <int MODE, bool VF16>
__device__ __forceinline__ void tile_weights(f32x16_t (&sacc)[2], float m_run, float &l_run,
                                             uint4 (&pk)[4]) {
    if (MODE == 0) {
        // sigma(x) = 1 / (1 + 2^t); the scores already are t = -x log2(e) (an excluded key
        // has t = +inf -> 0)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                sacc[kb][e] = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(sacc[kb][e]));
    } else {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int e = 0; e < 16; ++e) sacc[kb][e] = __builtin_amdgcn_exp2f(sacc[kb][e] - m_run);
    }
    float ls[2] = {0.0f, 0.0f};
    const f16x2_t ones = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int kb = t >> 1, e0 = 8 * (t & 1);
        if (VF16) {
            pk[t].x = pack_f16x2(sacc[kb][e0 + 0], sacc[kb][e0 + 1]);
            pk[t].y = pack_f16x2(sacc[kb][e0 + 2], sacc[kb][e0 + 3]);
            pk[t].z = pack_f16x2(sacc[kb][e0 + 4], sacc[kb][e0 + 5]);
            pk[t].w = pack_f16x2(sacc[kb][e0 + 6], sacc[kb][e0 + 7]);
            if (MODE == 1) {
                ls[0] = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, pk[t].x), ones, ls[0], false);
                ls[1] = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, pk[t].y), ones, ls[1], false);
                ls[0] = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, pk[t].z), ones, ls[0], false);
                ls[1] = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, pk[t].w), ones, ls[1], false);
            }
        } else {
            pk[t].x = pack_bf16x2(sacc[kb][e0 + 0], sacc[kb][e0 + 1]);
            pk[t].y = pack_bf16x2(sacc[kb][e0 + 2], sacc[kb][e0 + 3]);
            pk[t].z = pack_bf16x2(sacc[kb][e0 + 4], sacc[kb][e0 + 5]);
            pk[t].w = pack_bf16x2(sacc[kb][e0 + 6], sacc[kb][e0 + 7]);
        }
    }
    if (MODE == 1) l_run += ls[0] + ls[1];
}

// O^T += V^T P^T with the packed weights of one tile: the two transposing reads (bf16 V rows)
// or the one 16-byte read (float16 V^T image) deliver V^T in the key order of the weights.
template <int D, bool VF16>
__device__ __forceinline__ void tile_pv(const uint16_t *__restrict__ vl, const LaneOffsets<D> &lo,
                                        const uint4 (&pk)[4], f32x16_t (&oacc)[D / 32]) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
            if constexpr (VF16) {
                // V^T rows 32 db .. 32 db + 31 of the transposed tile: one 16-byte read
                const f16x8_t a = *reinterpret_cast<const f16x8_t *>(vl + 32 * db * BK + lo.vt[t]);
                oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                    a, __builtin_bit_cast(f16x8_t, pk[t]), oacc[db], 0, 0, 0);
            } else {
                const s16x4_t lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_s16x4_t *)(vl + 16 * t * D + lo.v[db]));
                const s16x4_t hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_s16x4_t *)(vl + (16 * t + 8) * D + lo.v[db]));
                const s16x8_t a8 = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
                oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    __builtin_bit_cast(bf16x8_t, a8), __builtin_bit_cast(bf16x8_t, pk[t]), oacc[db], 0, 0, 0);
            }
        }
    }
}

// Weights of one prepared tile, then O^T += V^T P^T.
template <int D, int MODE, bool VF16>
__device__ __forceinline__ void weigh_pv(const uint16_t *__restrict__ vl, const LaneOffsets<D> &lo,
                                         f32x16_t (&sacc)[2], f32x16_t (&oacc)[D / 32],
                                         float m_run, float &l_run) {
    uint4 pk[4];
    tile_weights<MODE, VF16>(sacc, m_run, l_run, pk);
    tile_pv<D, VF16>(vl, lo, pk, oacc);
}

struct TileCtx {
    __amdgpu_buffer_rsrc_t rk, rv;
    uint32_t row_bytes;
    int tid, wave, qa, qb, i, g, w, s, N;
    int dmask;                      // dilation - 1 (a power of two minus one; 0: contiguous)
    int n_tiles, ts_end, tw_begin;  // the walk: sink tiles [0, ts_end), then window tiles
    int ns_img, shift;              // tile t of the key positions is image tile img_of(t)
    uint32_t vtile_bytes;           // bytes between V tiles read as rows
    float cs, slope_l2;

    __device__ __forceinline__ uint32_t img_of(int j0) const {
        const int t = j0 / BK;
        return (uint32_t)(t >= ns_img ? t - shift : t);
    }

    __device__ __forceinline__ int j0_of(int t) const {
        return (t < ts_end ? t : tw_begin + (t - ts_end)) * BK;
    }
    // 0 = every pair in the key set, 1 = cut by the window edges, 2 = also holds sinks,
    // 3 = cut by the causal edge only, 4 = cut by the far window edge only (3 and 4 with
    // ONE_SIDED, for contiguous windows), -1 = no pair in the key set (wave-uniform: this
    // wavefront's queries [qa, qb])
    template <bool ONE_SIDED>
    __device__ __forceinline__ int kind_of(int j0) const {
        if (qa >= N || j0 > qb || (qa - (j0 + BK - 1) >= w && j0 >= s)) return -1;
        const bool causal_ok = j0 + BK - 1 <= qa, far_ok = qb - j0 < w;
        if (causal_ok && ((far_ok && dmask == 0) || j0 + BK - 1 < s)) return 0;
        if (j0 < s) return 2;
        if (ONE_SIDED && dmask == 0 && far_ok) return 3;
        if (ONE_SIDED && dmask == 0 && causal_ok) return 4;
        return 1;
    }
};

// Transfers into a K or V tile buffer: packed images, or V straight from the input rows.
template <int D>
__device__ __forceinline__ void load_k(uint16_t *__restrict__ dst, const TileCtx &cx,
                                       const LaneOffsets<D> &lo, int j0) {
    dma_rounds_kb<Tile<D>::DMA_W>(dst, cx.rk, cx.img_of(j0) * Tile<D>::IMG_BYTES + lo.dimg, cx.wave);
}
template <int D, bool VF16>
__device__ __forceinline__ void load_v(uint16_t *__restrict__ dst, const TileCtx &cx,
                                       const LaneOffsets<D> &lo, int j0) {
    if (VF16)
        dma_rounds_kb<Tile<D>::DMA_W>(dst, cx.rv, cx.img_of(j0) * Tile<D>::IMG_BYTES + lo.dimg, cx.wave);
    else
        dma_rounds_strided<Tile<D>::DMA_W>(dst, cx.rv, cx.img_of(j0) * cx.vtile_bytes + lo.dvraw,
                                           lo.dvstep, cx.wave);
}

// Edge masking of a freshly formed tile at j, in place (the masked scores stay in the
// registers of the unmasked ones, so the rare masked path costs the common one no copies).
// kind < 0 (no tile, or one that meets none of this wavefront's key sets) excludes every
// key, so that weighing the tile adds nothing.
template <int D, int MODE, bool DIL>
__device__ __forceinline__ void mask_scores(f32x16_t (&sacc)[2], const TileCtx &cx, int j,
                                            int kind) {
    constexpr float fill = MODE == 0 ? INFINITY : -INFINITY;
    if (kind != 0) {
        const int dq = cx.i - j - 4 * cx.g, jb = j + 4 * cx.g;
        if (kind == 2)
            mask_tile_inplace<true>(sacc, dq, jb, cx.w, cx.s, DIL ? cx.dmask : 0, fill, false);
        else
            mask_tile_inplace<false>(sacc, dq, jb, cx.w, cx.s, DIL ? cx.dmask : 0, fill, kind < 0);
    }
}

// Step t of the software pipeline (d = 128). On entry s_cur holds the prepared scores of
// tile t, K buffer k_next holds tile t + 1 and V buffer v_cur tile t. The step starts the
// transfers of K tile t + 2 (into k_fill, free since tile t's scores were formed) and V tile
// t + 1 (into v_fill, free since tile t - 1's product), forms the scores of tile t + 1 while
// it weighs tile t, and prepares tile t + 1's scores. The scores of tile t + 1 are formed
// whether or not that tile exists or meets this wavefront's queries (one definition keeps
// them in place across the steps); unused, they are never weighed (sigmoid) or are masked out
// whole (softmax). Softmax masks tile t + 1 in place right after forming it (edge tiles only)
// and takes its maximum after tile t's product; sigmoid weighs tile t first. Each order
// measured faster for its mode.
// The four buffers are distinct restrict pointers, so no LDS read here waits for the
// transfers this step starts.
template <int D, int MODE, bool ALIBI, bool VF16, bool DIL>
__device__ __forceinline__ void pipe_step(uint16_t *__restrict__ k_fill,
                                          uint16_t *__restrict__ v_fill,
                                          const uint16_t *__restrict__ k_next,
                                          const uint16_t *__restrict__ v_cur, const TileCtx &cx,
                                          const LaneOffsets<D> &lo, const BiasOperands &bo,
                                          const f16x8_t (&qreg)[D / 16], f32x16_t (&s_cur)[2],
                                          f32x16_t (&s_next)[2], f32x16_t (&oacc)[D / 32],
                                          float &m_run, float &l_run, int t) {
    const bool has1 = t + 1 < cx.n_tiles;
    if (t + 2 < cx.n_tiles) load_k<D>(k_fill, cx, lo, cx.j0_of(t + 2));
    const int j1 = cx.j0_of(t + 1);
    if (has1) load_v<D, VF16>(v_fill, cx, lo, j1);
    const int kind1 = has1 ? cx.template kind_of<false>(j1) : -1;
    qk_tile<D, MODE, ALIBI>(k_next, lo, bo, qreg, s_next, cx.i, j1);
    {
        // K rows read four products ahead of their use (the compiler's own order issues each
        // pair of reads right before its products)
        constexpr int NR = 2 * (D / 16), AH = 4;
        __builtin_amdgcn_sched_group_barrier(0x100, AH, 0);  // LDS reads
#pragma unroll
        for (int u = 0; u < NR - AH; ++u) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // matrix
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, AH, 0);
    }
    if constexpr (MODE == 0) {
        if (cx.template kind_of<false>(cx.j0_of(t)) >= 0)
            weigh_pv<D, MODE, VF16>(v_cur, lo, s_cur, oacc, m_run, l_run);
        if (kind1 >= 0)
            prep_scores<D, MODE, ALIBI, DIL>(s_next, oacc, m_run, l_run, cx.cs, 0.0f, kind1,
                                             cx.i - j1 - 4 * cx.g, j1 + 4 * cx.g, cx.w, cx.s,
                                             cx.dmask);
    } else {
        mask_scores<D, MODE, DIL>(s_next, cx, j1, kind1);
        weigh_pv<D, MODE, VF16>(v_cur, lo, s_cur, oacc, m_run, l_run);
        if (ALIBI) {
            const float bq = cx.slope_l2 * (float)(cx.i - j1);
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int e = 0; e < 16; ++e) s_next[kb][e] += bq;
        }
        fold_max<D>(tile_max(s_next), oacc, m_run, l_run);
    }
}

// Step t without pipelining: start the transfers of tile t + 1 (K and V) into the other
// buffer pair, then form, prepare and weigh tile t. Fewer live registers than pipe_step.
template <int D, int MODE, bool ALIBI, bool VF16, bool DIL>
__device__ __forceinline__ void plain_step(uint16_t *__restrict__ k_fill,
                                           uint16_t *__restrict__ v_fill,
                                           const uint16_t *__restrict__ k_cur,
                                           const uint16_t *__restrict__ v_cur, const TileCtx &cx,
                                           const LaneOffsets<D> &lo, const BiasOperands &bo,
                                           const f16x8_t (&qreg)[D / 16], f32x16_t (&oacc)[D / 32],
                                           float &m_run, float &l_run, int t) {
    if (t + 1 < cx.n_tiles) {
        const int j1 = cx.j0_of(t + 1);
        load_k<D>(k_fill, cx, lo, j1);
        load_v<D, VF16>(v_fill, cx, lo, j1);
    }
    const int j0 = cx.j0_of(t);
    const int kind = cx.template kind_of<D == 64>(j0);
    if (kind >= 0) {
        f32x16_t sacc[2];
        const float bq = cx.slope_l2 * (float)(cx.i - j0);
        qk_tile<D, MODE, ALIBI>(k_cur, lo, bo, qreg, sacc, cx.i, j0);
        prep_scores<D, MODE, ALIBI, DIL>(sacc, oacc, m_run, l_run, cx.cs, bq, kind,
                                    cx.i - j0 - 4 * cx.g, j0 + 4 * cx.g, cx.w, cx.s, cx.dmask);
        weigh_pv<D, MODE, VF16>(v_cur, lo, sacc, oacc, m_run, l_run);
    }
}

// Rows of a sequence a chunked call cannot serve: NaN for this workgroup's query heads
// h_first .. h_first + GP - 1, on the query tiles qt0, qt0 + QP * n_qtiles, ...
template <int D, int GP>
__device__ void nan_rows(const MfmaParams &p, const ChunkSeq &cs, int r_first, int QP,
                         int64_t h_first) {
    const int64_t stride = (int64_t)p.n_qtiles * QP;
    for (int64_t r0 = r_first; r0 < cs.n; r0 += stride) {
        const int rows = cs.n - r0 < QP ? (int)(cs.n - r0) : QP;
        for (int e = threadIdx.x; e < rows * GP * D; e += blockDim.x) {
            const int rr = e / (GP * D), hp = (e / D) % GP, c = e % D;
            const int64_t off = ((cs.row0 + r0 + rr) * p.Hq + h_first + hp) * D + c;
            if (p.out_bf16) static_cast<uint16_t *>(p.o)[off] = 0x7fc0;
            else static_cast<float *>(p.o)[off] = qnan();
        }
    }
}

// Register budget: 4 wavefronts per SIMD at d = 64 (3 with four heads per workgroup, which
// keeps more per-head state), 2 at d = 128.
template <int D, int GP, int MODE, bool ALIBI, bool VF16, bool DIL>
__global__ __launch_bounds__(64 * Tile<D>::NW)
__attribute__((amdgpu_waves_per_eu(D == 64 ? (GP < 4 ? 4 : 3) : 2)))
void prefill_mfma_kernel(MfmaParams p) {
    using T = Tile<D>;
    constexpr int QP = 32 * T::NW / GP;  // query positions per workgroup
    constexpr int WPH = T::NW / GP;      // wavefronts per query head
    constexpr int KS = D / 16;    // k-steps of the score product
    constexpr int DB = D / 32;    // 32-row blocks of the output
    __shared__ __attribute__((aligned(16))) uint16_t lds[T::LDS_BYTES / 2];
    uint16_t *const kbuf0 = lds, *const kbuf1 = lds + T::IMG;
    uint16_t *const vbuf0 = lds + 2 * T::IMG, *const vbuf1 = lds + 3 * T::IMG;

    // ---- workgroup -> (batch, kv head, head group, query tile), XCD-contiguous
    const int nb = gridDim.x, bid = blockIdx.x;
    const int per = nb / 8, rem = nb % 8, xcd = bid % 8, local = bid / 8;
    const int logical = xcd < rem ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
    // query tiles [rot, n) in order, then the rot tiles with shortened bands, longest first
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
    // query rows: positions [qpos0, N) at memory rows qrow0 + rstep (position - qpos0)
    int qpos0 = 0, nq = (int)p.N, shift = 0, ns_img = 0;
    int64_t qrow0 = (int64_t)b * p.N_mem + p.pos_off;   // memory row of query qpos0
    int rstep = p.pos_stride;                           // memory rows between queries
    if (p.chunked) {
        const ChunkSeq cs = chunk_seq(p.cg, b);
        if (!cs.rows_ok) return;
        if (!cs.valid) {
            nan_rows<D, GP>(p, cs, qt * QP, QP, h - hp);
            return;
        }
        if (qt * QP >= cs.n) return;
        qpos0 = cs.p0; nq = cs.n; qrow0 = cs.row0; shift = cs.shift; ns_img = p.cg.ns_img;
        rstep = 1;
    }
    const int N = qpos0 + nq;
    const int q0 = qpos0 + qt * QP;
    const int qa = q0 + 32 * pb;                   // this wavefront's first query
    const int i = qa + qc;                         // this lane's query
    const int qe = (q0 + QP < N ? q0 + QP : N) - 1;
    const bool rope = p.rope != nullptr;

    // ---- band of key tiles: sink tiles the window no longer covers, then the window
    const int lo_wg = q0 - p.w + 1 > 0 ? q0 - p.w + 1 : 0;
    const int tw_begin = lo_wg / BK, tw_end = qe / BK;
    const int n_sink_keys = p.s < lo_wg ? p.s : lo_wg;
    int ts_end = (n_sink_keys + BK - 1) / BK;
    if (ts_end > tw_begin) ts_end = tw_begin;

    TileCtx cx;
    {
        const int64_t kvoff = (((int64_t)b * p.N_mem + p.pos_off) * p.Hkv + hkv) * D;
        const int64_t imoff = ((int64_t)b * p.Hkv + hkv) * p.n_ktiles * T::IMG;
        const uint32_t imbytes = (uint32_t)p.n_ktiles * T::IMG_BYTES;
        cx.rk = make_rsrc(p.kimg + imoff, imbytes);
        cx.rv = (VF16 || p.chunked) ? make_rsrc(p.vimg + imoff, imbytes)
                                    : make_rsrc(p.v + kvoff, p.kv_bytes);
        cx.row_bytes = p.row_bytes;
        cx.ns_img = ns_img; cx.shift = shift;
        cx.vtile_bytes = p.chunked ? (uint32_t)T::IMG_BYTES : (uint32_t)BK * p.row_bytes;
        // the wavefront index is uniform: keep it (and the LDS addresses of the transfers) scalar
        cx.tid = tid; cx.wave = __builtin_amdgcn_readfirstlane(wave); cx.qa = qa; cx.qb = qa + 31 < N ? qa + 31 : N - 1;
        cx.i = i; cx.g = g; cx.w = p.w; cx.s = p.s; cx.N = N; cx.dmask = p.dmask;
        cx.n_tiles = ts_end + (tw_end - tw_begin + 1);
        cx.ts_end = ts_end; cx.tw_begin = tw_begin;
        cx.cs = p.cs;
        cx.slope_l2 = 0.0f;  // set below, once its load has joined the others
    }

    LaneOffsets<D> lo;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) lo.k[ks] = qc * D + (((2 * ks + g) ^ kswz<D>(qc)) * 8);
    {
        // transposing read: lane (G4, rr, a) supplies the row 4 (G4 / 2) + rr and the column
        // group 16 (G4 % 2) + 4 a of the 8 x 32 block that one read covers
        const int G4 = lane >> 4, rr = (lane >> 2) & 3, a = lane & 3;
        const int row_l = 4 * (G4 >> 1) + rr, cb = 2 * (G4 & 1) + (a >> 1);
        const int fq = vswz<D>(rr) >> 2;   // the V swizzle depends on row bits the lane fixes
#pragma unroll
        for (int db = 0; db < DB; ++db) lo.v[db] = row_l * D + (4 * (db ^ fq) + cb) * 8 + 4 * (a & 1);
    }
    // V^T read of step t: row qc (plus 32 db), stored chunk 2 t + g (the swizzle of row
    // 32 db + qc equals that of row qc)
#pragma unroll
    for (int t = 0; t < 4; ++t) lo.vt[t] = vt_slot(qc, 2 * t + g);
    {
        // transfer r of this wavefront fills the 16-byte slots (wave DMA_W + r) 64 + lane of
        // the tile image: 512 / D rows per transfer, and the swizzle of a lane's row does not
        // depend on r (it takes only row bits below 512 / D)
        const uint32_t vrow = p.chunked ? (uint32_t)(2 * D) : p.row_bytes;
        const int slot = wave * T::DMA_W * 64 + lane;
        const int row = slot / T::C, c = (slot % T::C) ^ vswz<D>(row);
        static_assert(vswz<D>(512 / D) == 0 && vswz<D>(2 * (512 / D)) == 0, "swizzle period");
        lo.dimg = (uint32_t)slot * 16;
        lo.dvraw = (uint32_t)row * vrow + c * 16;
        lo.dvstep = (uint32_t)(512 / D) * vrow;
    }

    // ---- first transfers: K tile 0 (and 1 when pipelined) and V tile 0, in flight while the
    // query fragment and the slope load
    const float slope = ALIBI ? p.slopes[h] * p.slope_mul : 0.0f;
    load_k<D>(kbuf0, cx, lo, cx.j0_of(0));
    load_v<D, VF16>(vbuf0, cx, lo, cx.j0_of(0));
    if (T::PIPE && cx.n_tiles > 1) load_k<D>(kbuf1, cx, lo, cx.j0_of(1));

    // ---- this lane's query fragment (B operand of S^T = K Q^T): rotated, float16; for
    // sigmoid scaled by -cs first, so that the product is the negated base-2 logit. Every
    // load is issued before the first use (a lane past the end reads the last row and
    // drops it), so the fragment costs one memory round trip.
    f16x8_t qreg[KS];
    {
        const bool in = i < N;
        const int ic = in ? i : N - 1;
        const uint16_t *qrow = p.q + ((qrow0 + (int64_t)(ic - qpos0) * rstep) * p.Hq + h) * D;
        // rotation angles at the query's position (chunked: the position itself; a residue
        // class: pos_off + r i)
        const int64_t qpos = p.chunked ? (int64_t)ic : p.pos_off + (int64_t)p.pos_stride * ic;
        const float4 *trow = rope ? reinterpret_cast<const float4 *>(p.rope + qpos * D) : nullptr;
        uint4 xq[KS];
        float4 t0[KS], t1[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            xq[ks] = *reinterpret_cast<const uint4 *>(qrow + ks * 16 + g * 8);
            if (rope) {
                t0[ks] = trow[ks * 4 + g * 2];
                t1[ks] = trow[ks * 4 + g * 2 + 1];
            }
        }
        // sigmoid: the negated base-2 logit, so q times -cs; softmax: the base-2 logit, q
        // times cs
        const float qs = MODE == 0 ? -p.cs : p.cs;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            uint4 x;
            if (rope) x = rotate_chunk_scaled(xq[ks], t0[ks], t1[ks], qs);
            else x = convert_chunk_scaled(xq[ks], qs);
            qreg[ks] = __builtin_bit_cast(f16x8_t, in ? x : make_uint4(0, 0, 0, 0));
        }
    }

    // ALiBi bias in base-2 units. Softmax: the key part -slope log2(e) kappa (the query part
    // is one add per score); sigmoid: the whole bias of the negated logit, key part
    // slope log2(e) kappa plus the query part
    if (ALIBI) cx.slope_l2 = slope * LOG2E;
    const BiasOperands bo = MODE == 0 ? bias_operands(ALIBI ? -cx.slope_l2 : 0.0f, lane, ALIBI)
                                      : bias_operands(ALIBI ? cx.slope_l2 : 0.0f, lane);

    f32x16_t oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[db][e] = 0.0f;
    float m_run = -1e30f, l_run = 0.0f;

    if constexpr (T::PIPE) {
        // ---- prologue: K tiles 0 and 1, V tile 0; scores of tile 0
        f32x16_t sa[2], sb[2];
        __syncthreads();
        {
            const int j0 = cx.j0_of(0), kind0 = cx.template kind_of<false>(j0);
            qk_tile<D, MODE, ALIBI>(kbuf0, lo, bo, qreg, sa, i, j0);
            if (MODE == 0) {
                if (kind0 >= 0)
                    prep_scores<D, MODE, ALIBI, DIL>(sa, oacc, m_run, l_run, cx.cs, 0.0f, kind0,
                                                     i - j0 - 4 * g, j0 + 4 * g, cx.w, cx.s,
                                                     cx.dmask);
            } else {
                mask_scores<D, MODE, DIL>(sa, cx, j0, kind0);
                if (ALIBI) {
                    const float bq = cx.slope_l2 * (float)(i - j0);
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                        for (int e = 0; e < 16; ++e) sa[kb][e] += bq;
                }
                fold_max<D>(tile_max(sa), oacc, m_run, l_run);
            }
        }
        __syncthreads();

        // ---- tile t lives in K/V buffer t % 2; two steps per trip keep the score registers
        for (int t = 0; t < cx.n_tiles; t += 2) {
            pipe_step<D, MODE, ALIBI, VF16, DIL>(kbuf0, vbuf1, kbuf1, vbuf0, cx, lo, bo, qreg, sa, sb,
                                                 oacc, m_run, l_run, t);
            __syncthreads();
            if (t + 1 >= cx.n_tiles) break;
            pipe_step<D, MODE, ALIBI, VF16, DIL>(kbuf1, vbuf0, kbuf0, vbuf1, cx, lo, bo, qreg, sb, sa,
                                                 oacc, m_run, l_run, t + 1);
            __syncthreads();
        }
    } else {
        __syncthreads();
        for (int t = 0; t < cx.n_tiles; t += 2) {
            plain_step<D, MODE, ALIBI, VF16, DIL>(kbuf1, vbuf1, kbuf0, vbuf0, cx, lo, bo, qreg, oacc,
                                             m_run, l_run, t);
            __syncthreads();
            if (t + 1 >= cx.n_tiles) break;
            plain_step<D, MODE, ALIBI, VF16, DIL>(kbuf0, vbuf0, kbuf1, vbuf1, cx, lo, bo, qreg, oacc,
                                             m_run, l_run, t + 1);
            __syncthreads();
        }
    }

    // ---- epilogue: normalise, stage O row-major in LDS (four wavefronts at a time), store
    // whole rows. The loop holds every register, so the lane's indices are formed again here
    // from the scalar wavefront index and the lane id rather than kept across it.
    int elane;  // the lane id, read here (an asm statement the compiler cannot hoist)
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(elane));
    const int ew = cx.wave;
    const int eqc = elane & 31, eg = elane >> 5;
    const int64_t eh = (int64_t)hkv * p.G + hg * GP + ew / WPH;
    const int eqa = q0 + 32 * (ew % WPH), ei = eqa + eqc;
    float l_tot = 1.0f;
    if (MODE == 1) {
        // the sum over both lane halves (lanes l and l ^ 32 saw the query's two key halves)
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run),
                                                         __float_as_uint(l_run), false, false);
        l_tot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    }
    const float inv = MODE == 1 ? 1.0f / l_tot : 1.0f;
    if (MODE == 1 && p.lse != nullptr && eg == 0 && ei < N)
        p.lse[((int64_t)b * p.Hq + eh) * p.N_mem + p.pos_off + (int64_t)p.pos_stride * ei] =
            (m_run + log2f(l_tot)) * 0.6931471805599453f;
    float *ol = reinterpret_cast<float *>(lds) + (ew & 3) * (32 * T::OSTR);
    constexpr int C4 = D / 4;  // 4-float chunks per row
#pragma unroll
    for (int round = 0; round < T::NW / 4; ++round) {
        if ((ew >> 2) == round) {
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int d0 = 32 * db + 8 * r + 4 * eg;
                    *reinterpret_cast<float4 *>(ol + eqc * T::OSTR + d0) =
                        make_float4(oacc[db][4 * r] * inv, oacc[db][4 * r + 1] * inv,
                                    oacc[db][4 * r + 2] * inv, oacc[db][4 * r + 3] * inv);
                }
        }
        __syncthreads();
        if ((ew >> 2) == round) {
            // this wavefront's 32 rows start at element obase; row r lies r * rstep * Hq * D further
            // (32-bit offsets: Hq * D * 32 < 2^31 is a launch condition)
            const int64_t obase = ((qrow0 + (int64_t)(eqa - qpos0) * rstep) * p.Hq + eh) * D;
            void *ob = p.out_bf16 ? static_cast<void *>(static_cast<uint16_t *>(p.o) + obase)
                                  : static_cast<void *>(static_cast<float *>(p.o) + obase);
            const int rstride = rstep * (int)p.Hq * D;
#pragma unroll
            for (int rr = 0; rr < 32 * C4 / 64; ++rr) {
                const int ch = elane + 64 * rr;
                const int qrow = ch / C4, c4 = ch % C4;
                if (eqa + qrow < N) {
                    const float4 x = *reinterpret_cast<const float4 *>(ol + qrow * T::OSTR + 4 * c4);
                    store_out4<true>(ob, p.out_bf16, qrow * rstride + 4 * c4, x.x, x.y, x.z, x.w);  // whole rows
                }
            }
        }
        if (round + 1 < T::NW / 4) __syncthreads();
    }
}

template <int D, int GP, int MODE, bool VF16>
hipError_t launch_main(const MfmaParams &mp, int nblocks, bool alibi, hipStream_t st) {
    const dim3 grid((unsigned)nblocks), block(64 * Tile<D>::NW);
    if (mp.dmask != 0) {
        if (alibi) hipLaunchKernelGGL((prefill_mfma_kernel<D, GP, MODE, true, VF16, true>), grid, block, 0, st, mp);
        else hipLaunchKernelGGL((prefill_mfma_kernel<D, GP, MODE, false, VF16, true>), grid, block, 0, st, mp);
    } else {
        if (alibi) hipLaunchKernelGGL((prefill_mfma_kernel<D, GP, MODE, true, VF16, false>), grid, block, 0, st, mp);
        else hipLaunchKernelGGL((prefill_mfma_kernel<D, GP, MODE, false, VF16, false>), grid, block, 0, st, mp);
    }
    return hipGetLastError();
}

// Softmax packs V to float16 as well (float16 second product); sigmoid reads V as stored.
template <int D, int GP>
hipError_t launch_gp(const MfmaParams &mp, int nb, int mode, bool alibi, hipStream_t st) {
    if (mode == 1) return launch_main<D, GP, 1, true>(mp, nb, alibi, st);
    return launch_main<D, GP, 0, false>(mp, nb, alibi, st);
}

// nblocks: (batch, tile, kv-head group) triples; each gets KPT blocks.
template <int D>
hipError_t launch_pack(const PackParams &pp, int nblocks, bool rot, bool pack_v, hipStream_t st) {
    nblocks *= Tile<D>::KPT;
    if (rot) {
        if (pack_v) hipLaunchKernelGGL((prefill_pack_kernel<D, true, true>), dim3((unsigned)nblocks), dim3(256), 0, st, pp);
        else hipLaunchKernelGGL((prefill_pack_kernel<D, true, false>), dim3((unsigned)nblocks), dim3(256), 0, st, pp);
    } else {
        if (pack_v) hipLaunchKernelGGL((prefill_pack_kernel<D, false, true>), dim3((unsigned)nblocks), dim3(256), 0, st, pp);
        else hipLaunchKernelGGL((prefill_pack_kernel<D, false, false>), dim3((unsigned)nblocks), dim3(256), 0, st, pp);
    }
    return hipGetLastError();
}

int pack_of(int64_t G) { return G % 4 == 0 ? 4 : (G % 2 == 0 ? 2 : 1); }

struct Plan {
    bool vf16;
    int64_t n_ktiles;
    size_t img_bytes;  // one full set of K (or V) tile images
};

Plan plan_of(const PrefillArgs &a) {
    Plan pl;
    pl.vf16 = a.mode == 1;
    pl.n_ktiles = (a.N + BK - 1) / BK;
    pl.img_bytes = (size_t)(a.B * a.Hkv * pl.n_ktiles) * BK * (size_t)a.d * 2;
    return pl;
}

}  // namespace

// Dilated windows without sinks run as one plain window per residue class of positions;
// past MAX_CLASSES classes (two launches each) the single in-kernel stride test is cheaper.
constexpr int64_t MAX_CLASSES = 64;
bool class_path(const PrefillArgs &a) { return a.dil > 1 && a.s == 0 && a.dil <= MAX_CLASSES; }

bool prefill_mfma_supported(const PrefillArgs &a) {
    if (a.in_dt != 1 || (a.d != 64 && a.d != 128)) return false;
    // dilated windows: without sinks a dilation up to MAX_CLASSES runs as residue classes
    // (strided rows: dilation x Hq x d x 32 elements of output per wavefront stay below
    // 2^31); otherwise the in-kernel stride test, which needs a power of two
    if (a.dil > (int64_t(1) << 24)) return false;
    if (class_path(a)) {
        if (a.dil * a.Hq * a.d * 32 >= (int64_t(1) << 31)) return false;
    } else if ((a.dil & (a.dil - 1)) != 0) {
        return false;
    }
    if (a.B * a.N == 0) return true;
    const int64_t G = a.Hq / a.Hkv;
    const int GP = pack_of(G);
    const int64_t QP = 32 * (a.d == 128 ? Tile<128>::NW : Tile<64>::NW) / GP;
    const int64_t nb = a.B * a.Hkv * (G / GP) * ((a.N + QP - 1) / QP);
    const int64_t n_kt = (a.N + BK - 1) / BK;
    // 32-bit block ids and buffer offsets: one K/V slice, one slice of tile images and the
    // table stay below 2 GiB
    const int64_t slice = (a.N * a.Hkv) * a.d * 2;
    const int64_t img_slice = n_kt * BK * a.d * 2;
    const int64_t table = a.rope ? a.rope_rows * a.d * 4 : 0;
    const int64_t pack_blocks = a.B * n_kt * ((a.Hkv + PACK_HG - 1) / PACK_HG) * Tile<128>::KPT;
    return nb <= 0x7fffffff && a.B * a.Hkv * n_kt <= 0x7fffffff && pack_blocks <= 0x7fffffff &&
           slice < (int64_t(1) << 31) &&
           img_slice < (int64_t(1) << 31) && table < (int64_t(1) << 31) && a.N < (int64_t(1) << 24) &&
           a.Hq * a.d * 32 < (int64_t(1) << 31);
}

size_t prefill_mfma_workspace_bytes(const PrefillArgs &a) {
    if (a.B * a.N == 0) return 0;
    const Plan pl = plan_of(a);
    return pl.img_bytes + (pl.vf16 ? pl.img_bytes : 0);
}

// One pre-pass + main kernel pair over the (strided) sequence of n positions: memory rows and
// positions pos_off + r j, j < n; ALiBi slopes times r; dmask the in-kernel stride test
// (dilation - 1) of the general form, 0 when the positions are one residue class.
hipError_t launch_prefill_pair(const PrefillArgs &a, const void *q, const void *k,
                               const void *v, void *o, void *ws, hipStream_t st, float *lse,
                               int64_t n, int pos_off, int r, int64_t w_ext, int dmask) {
    const bool vf16 = a.mode == 1;
    const int64_t n_ktiles = (n + BK - 1) / BK;
    // the workspace holds the images of the whole sequence; a class uses its front part
    const size_t img_bytes = plan_of(a).img_bytes;
    const int64_t G = a.Hq / a.Hkv;
    const int GP = pack_of(G);
    const int64_t QP = 32 * (a.d == 128 ? Tile<128>::NW : Tile<64>::NW) / GP;
    MfmaParams mp = {};  // chunked = 0: whole sequences, no chunk geometry
    mp.q = static_cast<const uint16_t *>(q);
    mp.k = static_cast<const uint16_t *>(k);
    mp.v = static_cast<const uint16_t *>(v);
    mp.kimg = static_cast<const uint16_t *>(ws);
    mp.vimg = vf16 ? static_cast<const uint16_t *>(ws) + img_bytes / 2 : nullptr;
    mp.o = o;
    mp.slopes = a.slopes;
    mp.rope = a.rope;
    mp.N = n; mp.Hq = a.Hq; mp.Hkv = a.Hkv; mp.G = G;
    mp.n_qtiles = (int)((n + QP - 1) / QP);
    mp.n_hgroups = (int)(G / GP);
    mp.n_ktiles = (int)n_ktiles;
    mp.w = (int)(w_ext < n ? w_ext : n);
    mp.dmask = dmask;
    mp.s = (int)(a.s < n ? a.s : n);
    mp.cs = a.scale * LOG2E;
    // bytes from this sequence's first V row to past its last one (raw V reads)
    mp.kv_bytes = (uint32_t)(((n - 1) * r * a.Hkv + 1) * a.d * 2);
    mp.row_bytes = (uint32_t)(r * a.Hkv * a.d * 2);
    mp.out_bf16 = a.out_dt == 1;
    mp.lse = lse;
    mp.N_mem = a.N; mp.pos_off = pos_off; mp.pos_stride = r;
    mp.slope_mul = (float)r;

    {
        PackParams pp = {};
        pp.k = mp.k; pp.v = mp.v;
        pp.kimg = static_cast<uint16_t *>(ws);
        pp.vimg = vf16 ? static_cast<uint16_t *>(ws) + img_bytes / 2 : nullptr;
        pp.rope = a.rope; pp.N = n; pp.Hkv = a.Hkv; pp.n_ktiles = (int)n_ktiles;
        pp.N_mem = a.N; pp.pos_off = pos_off; pp.pos_stride = r;
        const int npb = (int)(a.B * n_ktiles * ((a.Hkv + PACK_HG - 1) / PACK_HG));
        const hipError_t e = a.d == 64 ? launch_pack<64>(pp, npb, a.rope != nullptr, vf16, st)
                                       : launch_pack<128>(pp, npb, a.rope != nullptr, vf16, st);
        if (e != hipSuccess) return e;
    }
    const bool alibi = a.slopes != nullptr;
    const int nb = (int)(a.B * a.Hkv * mp.n_hgroups * mp.n_qtiles);
    if (a.d == 64) {
        if (GP == 4) return launch_gp<64, 4>(mp, nb, a.mode, alibi, st);
        if (GP == 2) return launch_gp<64, 2>(mp, nb, a.mode, alibi, st);
        return launch_gp<64, 1>(mp, nb, a.mode, alibi, st);
    }
    if (GP == 4) return launch_gp<128, 4>(mp, nb, a.mode, alibi, st);
    if (GP == 2) return launch_gp<128, 2>(mp, nb, a.mode, alibi, st);
    return launch_gp<128, 1>(mp, nb, a.mode, alibi, st);
}

hipError_t launch_prefill_mfma(const PrefillArgs &a, const void *q, const void *k,
                               const void *v, void *o, void *ws, hipStream_t st, float *lse) {
    if (a.B * a.N == 0) return hipSuccess;
    if (class_path(a)) {
        // a dilated window without sinks is the plain window of w keys on each residue class
        // of positions mod r: run the classes one after another, each over the strided rows
        // (keys and queries rotated at their true positions, slopes times r); the classes
        // share the workspace, in stream order
        const int r = a.dil < a.N ? (int)a.dil : (int)a.N;
        for (int c = 0; c < r; ++c) {
            const int64_t n = (a.N - c + r - 1) / r;
            const hipError_t e = launch_prefill_pair(a, q, k, v, o, ws, st, lse, n, c, r, a.w, 0);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
    // positions the window spans (w - 1 < N keeps the product small)
    const int64_t extent = a.w - 1 >= a.N ? a.N : a.dil * (a.w - 1) + 1;
    return launch_prefill_pair(a, q, k, v, o, ws, st, lse, a.N, 0, 1, extent, (int)(a.dil - 1));
}

}  // namespace swa

// ---------------------------------------------------------------------------------------
// Chunked prefill over the ring cache: gather, banded attention, append.
namespace swa {
namespace {

constexpr int64_t POS_LIMIT = int64_t(1) << 24;  // positions stay float-exact integers

struct ChunkPlan {
    int w_k, s_k;        // window and sinks clamped to the position range
    int64_t ns_img;      // sink tiles at the front of each sequence's images
    int64_t n_ktiles;    // image tiles per (sequence, kv head)
    int64_t pos_limit;
    size_t img_bytes;    // one full set of K (or V) images
};

ChunkPlan chunk_plan(const DecodeArgs &a, const CacheArgs &c, int64_t max_q) {
    ChunkPlan pl;
    pl.w_k = (int)(c.w < POS_LIMIT + BK ? c.w : POS_LIMIT + BK);
    pl.s_k = (int)(c.s < POS_LIMIT + BK ? c.s : POS_LIMIT + BK);
    pl.pos_limit = a.rope && a.rope_rows < POS_LIMIT ? a.rope_rows : POS_LIMIT;
    pl.ns_img = (pl.s_k + BK - 1) / BK;
    // window tiles a chunk can reach: fewer than (max_q + w - 1) / 64 + 2, and never more
    // than the tiles of all admissible positions
    const int64_t by_window = (max_q + pl.w_k + 62) / BK + 1;
    const int64_t by_pos = (pl.pos_limit + BK - 1) / BK;
    pl.n_ktiles = pl.ns_img + (by_window < by_pos ? by_window : by_pos);
    pl.img_bytes = (size_t)(c.S * c.Hkv * pl.n_ktiles) * BK * (size_t)c.d * 2;
    return pl;
}

int64_t chunk_qp(const CacheArgs &c, int64_t G) {
    return 32 * (c.d == 128 ? Tile<128>::NW : Tile<64>::NW) / pack_of(G);
}

template <int D>
hipError_t launch_gather(const GatherParams &gp, int nblocks, bool rot, bool vf16, hipStream_t st) {
    if (rot) {
        if (vf16) hipLaunchKernelGGL((chunk_gather_kernel<D, true, true>), dim3((unsigned)nblocks), dim3(256), 0, st, gp);
        else hipLaunchKernelGGL((chunk_gather_kernel<D, true, false>), dim3((unsigned)nblocks), dim3(256), 0, st, gp);
    } else {
        if (vf16) hipLaunchKernelGGL((chunk_gather_kernel<D, false, true>), dim3((unsigned)nblocks), dim3(256), 0, st, gp);
        else hipLaunchKernelGGL((chunk_gather_kernel<D, false, false>), dim3((unsigned)nblocks), dim3(256), 0, st, gp);
    }
    return hipGetLastError();
}

}  // namespace

bool prefill_chunk_supported(const DecodeArgs &a, const CacheArgs &c, int64_t T, int64_t max_q) {
    if (c.dt != 1 || (c.d != 64 && c.d != 128)) return false;
    if (c.S == 0 || T == 0 || max_q == 0) return true;
    if (max_q >= POS_LIMIT) return false;
    const ChunkPlan pl = chunk_plan(a, c, max_q);
    const int64_t G = a.Hq / c.Hkv;
    const int64_t QP = chunk_qp(c, G);
    const int64_t nb = c.S * c.Hkv * (G / pack_of(G)) * ((max_q + QP - 1) / QP);
    const int64_t ngather = c.S * pl.n_ktiles * ((c.Hkv + PACK_HG - 1) / PACK_HG);
    const int64_t nappend = c.S * ((max_q + BK - 1) / BK);
    const int64_t img_slice = pl.n_ktiles * BK * c.d * 2;
    const int64_t table = a.rope ? a.rope_rows * c.d * 4 : 0;
    return nb <= 0x7fffffff && ngather <= 0x7fffffff && nappend <= 0x7fffffff &&
           a.Hq * c.d * 32 < (int64_t(1) << 31) &&
           img_slice < (int64_t(1) << 31) && table < (int64_t(1) << 31);
}

size_t prefill_chunk_workspace_bytes(const DecodeArgs &a, const CacheArgs &c, int64_t T,
                                     int64_t max_q) {
    if (c.S == 0 || T == 0 || max_q == 0) return 0;
    return 2 * chunk_plan(a, c, max_q).img_bytes;
}

hipError_t launch_prefill_chunk(const DecodeArgs &a, const CacheArgs &c, const void *q,
                                const void *k_new, const void *v_new, const int32_t *cu,
                                const int32_t *pos0, int64_t T, int64_t max_q, void *o,
                                void *ws, hipStream_t st) {
    if (c.S == 0 || T == 0 || max_q == 0) return hipSuccess;
    const ChunkPlan pl = chunk_plan(a, c, max_q);
    const int64_t G = a.Hq / c.Hkv;
    const int GP = pack_of(G);
    const int64_t QP = chunk_qp(c, G);
    const bool vf16 = a.mode == 1;
    uint16_t *kimg = static_cast<uint16_t *>(ws);
    uint16_t *vimg = kimg + pl.img_bytes / 2;

    ChunkGeom cg = {};
    cg.cu = cu; cg.pos0 = pos0; cg.T = T; cg.max_q = (int)max_q;
    cg.pos_limit = (int)pl.pos_limit; cg.w = pl.w_k; cg.ns_img = (int)pl.ns_img;
    {
        GatherParams gp = {};
        gp.cg = cg;
        gp.k_new = static_cast<const uint16_t *>(k_new);
        gp.v_new = static_cast<const uint16_t *>(v_new);
        gp.k_ring = static_cast<const uint16_t *>(c.k_ring);
        gp.v_ring = static_cast<const uint16_t *>(c.v_ring);
        gp.k_sink = static_cast<const uint16_t *>(c.k_sink);
        gp.v_sink = static_cast<const uint16_t *>(c.v_sink);
        gp.kimg = kimg; gp.vimg = vimg;
        gp.rope = a.rope;
        gp.Hkv = c.Hkv; gp.w_ring = c.w; gp.s = c.s;
        gp.n_ktiles = (int)pl.n_ktiles;
        const int nb = (int)(c.S * pl.n_ktiles * ((c.Hkv + PACK_HG - 1) / PACK_HG));
        const hipError_t e = c.d == 64 ? launch_gather<64>(gp, nb, a.rope != nullptr, vf16, st)
                                       : launch_gather<128>(gp, nb, a.rope != nullptr, vf16, st);
        if (e != hipSuccess) return e;
    }
    {
        MfmaParams mp = {};
        mp.q = static_cast<const uint16_t *>(q);
        mp.kimg = kimg; mp.vimg = vimg;
        mp.o = o;
        mp.slopes = a.slopes;
        mp.rope = a.rope;
        mp.N = 0; mp.Hq = a.Hq; mp.Hkv = c.Hkv; mp.G = G;
        mp.N_mem = 0; mp.pos_off = 0; mp.pos_stride = 1; mp.slope_mul = 1.0f;
        mp.n_qtiles = (int)((max_q + QP - 1) / QP);
        mp.n_hgroups = (int)(G / GP);
        mp.n_ktiles = (int)pl.n_ktiles;
        mp.w = pl.w_k; mp.s = pl.s_k;
        mp.cs = a.scale * LOG2E;
        mp.out_bf16 = a.out_dt == 1;
        mp.chunked = 1;
        mp.cg = cg;
        const int nb = (int)(c.S * c.Hkv * mp.n_hgroups * mp.n_qtiles);
        const bool alibi = a.slopes != nullptr;
        hipError_t e;
        if (c.d == 64)
            e = GP == 4 ? launch_gp<64, 4>(mp, nb, a.mode, alibi, st)
              : GP == 2 ? launch_gp<64, 2>(mp, nb, a.mode, alibi, st)
                        : launch_gp<64, 1>(mp, nb, a.mode, alibi, st);
        else
            e = GP == 4 ? launch_gp<128, 4>(mp, nb, a.mode, alibi, st)
              : GP == 2 ? launch_gp<128, 2>(mp, nb, a.mode, alibi, st)
                        : launch_gp<128, 1>(mp, nb, a.mode, alibi, st);
        if (e != hipSuccess) return e;
    }
    ChunkAppendParams ap = {};
    ap.cg = cg;
    ap.k_new = static_cast<const uint16_t *>(k_new);
    ap.v_new = static_cast<const uint16_t *>(v_new);
    ap.k_ring = static_cast<uint16_t *>(c.k_ring);
    ap.v_ring = static_cast<uint16_t *>(c.v_ring);
    ap.k_sink = static_cast<uint16_t *>(c.k_sink);
    ap.v_sink = static_cast<uint16_t *>(c.v_sink);
    ap.rope = a.rope;
    ap.Hkv = c.Hkv; ap.w_ring = c.w; ap.s = c.s;
    ap.n_rtiles = (int)((max_q + BK - 1) / BK);
    // several blocks per tile (a tile holds 64 H_kv d / 8 chunks, 8192 at H_kv 8, d 128), so
    // that the grid fills the chip; one block per tile if the grid would outgrow 32-bit ids
    ap.n_parts = c.S * ap.n_rtiles * 8 <= 0x7fffffff ? 8 : 1;
    const int nb = (int)(c.S * ap.n_rtiles * ap.n_parts);
    if (c.d == 64) hipLaunchKernelGGL(chunk_append_kernel<64>, dim3((unsigned)nb), dim3(256), 0, st, ap);
    else hipLaunchKernelGGL(chunk_append_kernel<128>, dim3((unsigned)nb), dim3(256), 0, st, ap);
    return hipGetLastError();
}

}  // namespace swa
