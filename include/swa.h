/*
 * swa.h - libswa: causal sliding-window attention on AMD MI355X (gfx950).
 *
 * The operation (SWAT: Sliding Window Attention Training, "Balanced ALiBi" attention
 * equation; Sliding Window Attention glossary, the band mask and the ring buffer;
 * Sliding-window beats linear attention, SWA(w, s) with sink tokens):
 *
 *   For batch b, query head h (kv head hk = h / (H_q / H_kv)) and query position i:
 *     K(i)  = { j : 0 <= j <= i  and  (i - j < w  or  j < s) }
 *     x_ij  = scale * (R(i) q_i) . (R(j) k_j) + slope_h * (i - j)
 *     p_ij  = 1 / (1 + exp(-x_ij))                       SWA_SIGMOID (no normalisation)
 *           = exp(x_ij) / sum_{j' in K(i)} exp(x_ij')    SWA_SOFTMAX
 *     o_i   = sum_{j in K(i)} p_ij v_j
 *   R(p) rotates the interleaved pairs (2t, 2t+1) of a head vector by the angle
 *   p * theta^(-2t/d) (RoPE); the angles come from a table built by swa_rope_table.
 *   Positions are absolute 0-based token indices everywhere, sinks included.
 *
 * Conventions shared by every entry point:
 *   - Pointers are caller-owned DEVICE memory unless a comment says "host". The library
 *     allocates nothing, frees nothing and keeps no pointer after returning.
 *   - Tensors are dense, row-major, innermost dimension last, with the layouts given
 *     below. Element types are float32 (SWA_F32) or bfloat16 (SWA_BF16).
 *   - Arguments are validated on the host before anything is launched; on an error
 *     nothing is written and nothing is launched. A failed launch returns SWA_ERR_HIP
 *     (the HIP error code is then available from swa_last_hip_error()).
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the default
 *     stream). The caller synchronises. Calls on different streams may run concurrently.
 *   - The library holds no state: positions and cache contents are always explicit.
 *   - Device values that cannot be checked on the host (positions, table coverage of a
 *     position) are checked by the kernels: an out-of-range position produces NaN
 *     outputs for the affected query instead of an out-of-bounds access.
 */
#ifndef LIBSWA_SWA_H
#define LIBSWA_SWA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SWA_OK = 0,
    SWA_ERR_INVALID_ARGUMENT = 1, /* a null pointer, a negative size, H_q % H_kv != 0, ... */
    SWA_ERR_UNSUPPORTED = 2,      /* a valid combination this build does not implement     */
    SWA_ERR_HIP = 3               /* a HIP runtime call or a kernel launch failed          */
} swa_status;

typedef enum { SWA_SIGMOID = 0, SWA_SOFTMAX = 1 } swa_mode;
typedef enum { SWA_F32 = 0, SWA_BF16 = 1 } swa_dtype;

/*
 * Prefill over one batch of whole sequences: query row n sits at position n.
 *   q, o : [B, N, H_q, d]    k, v : [B, N, H_kv, d]
 * Requirements: B, N >= 0; H_q, H_kv >= 1; H_q % H_kv == 0; d even, 2 <= d <= 256;
 * w >= 1; s >= 0; mode is a swa_mode; in_dtype/out_dtype are swa_dtype values.
 * scale <= 0 selects 1/sqrt(d). alibi_slopes: device float[H_q] of signed slopes, or NULL
 * for no bias (a zero slope also means no bias on that head). rope_table: device float
 * [rope_rows, d/2, 2] from swa_rope_table, or NULL for no rotation; rope_rows >= N.
 * Dilated window (the dilated-window member of the sparse-attention family the Sliding
 * Window Attention glossary lists beside SWA): with dilation r > 1 the window keeps every
 * r-th position, K(i) = { j <= i : ((i - j) mod r = 0 and (i - j) / r < w) or j < s }, so w
 * keys span r (w - 1) + 1 positions; the sinks are unchanged. On the matrix cores a dilated
 * window without sinks and r <= 64 runs as the plain window on each residue class of
 * positions mod r, one pre-pass and main kernel pair per class on the strided rows (2 r
 * launches on the stream); with sinks, or past r = 64, r must be a power of two (other r
 * run on the general kernel). The cache entry points take no dilation.
 * bf16 inputs with d in {64, 128}, H_q * d below 2^26 and 16-byte aligned tensors run on the
 * matrix cores, which form the score product from float16 operands (rotated q and k; for
 * sigmoid q is also multiplied by -scale * log2(e) before its rounding, and the ALiBi term
 * enters the product through float16 splits of the slope and of the query offset) and the
 * value product from float16 (softmax) or bf16 (sigmoid) operands, with float32
 * accumulation, and |slope| / scale below 2^24. Every operand taken as float16 saturates
 * at +-65504, the largest finite float16, instead of overflowing: the rotated keys, the
 * rotated queries (for sigmoid after the factor -scale * log2(e)) and, for softmax, the
 * values. Inputs past that range thus give the attention of the saturated operands, with
 * finite outputs; inputs within it are exact up to the float16 rounding. Other shapes run
 * on a general float32 vector kernel, where nothing saturates.
 */
typedef struct swa_prefill_params {
    int64_t B, H_q, H_kv, N, d;
    int64_t w;                 /* window length, counting the query itself            */
    int64_t s;                 /* number of sink tokens (positions 0..s-1)             */
    int32_t mode;              /* swa_mode                                             */
    int32_t in_dtype;          /* swa_dtype of q, k, v                                 */
    int32_t out_dtype;         /* swa_dtype of o                                       */
    float scale;               /* <= 0: 1/sqrt(d)                                      */
    const float *alibi_slopes; /* device float[H_q] or NULL                            */
    const float *rope_table;   /* device float[rope_rows][d/2][2] (cos, sin) or NULL   */
    int64_t rope_rows;
    int64_t dilation;          /* 0 or 1: contiguous window; r > 1: dilated (below)    */
} swa_prefill_params;

/*
 * workspace: device scratch of at least swa_prefill_workspace_bytes(p) bytes, 16-byte
 * aligned (may be NULL when that is 0). The matrix-core path uses it for the keys, rotated
 * once into float16 tile images, and for softmax also the values converted to float16:
 * B * H_kv * ceil(N / 64) * 64 * d * 2 bytes each. Its contents on entry do not matter;
 * calls that share a workspace must not overlap. A workspace that is too small or
 * misaligned for a call that needs one is rejected with SWA_ERR_INVALID_ARGUMENT.
 */
swa_status swa_prefill(const swa_prefill_params *p, const void *q, const void *k,
                       const void *v, void *o, void *workspace, size_t workspace_bytes,
                       void *stream);

/* Bytes of workspace swa_prefill needs for these parameters (0 when it needs none, or when
 * the parameters are invalid). */
size_t swa_prefill_workspace_bytes(const swa_prefill_params *p);

/*
 * Training pair: the forward for training and its backward (SWAT: Sliding Window Attention
 * Training, "Putting It Together": the layer is trained end to end, so its inputs need
 * gradients). They take every shape swa_prefill takes. bf16 q, k, v with d in {64, 128}, a
 * contiguous window (dilation 0 or 1) and 16-byte aligned tensors (q, k, v, o, dout, dq, dk,
 * dv, rope_table) run on the matrix cores, with operands as in swa_prefill (float16
 * products, float32 accumulation; the float16 operands of the inputs, dout among them,
 * saturate at +-65504 as in swa_prefill, and v is taken as float16 in both modes); every
 * other shape, dilated windows included, runs on general float32 vector kernels. Each call
 * picks its path by these rules alone, so a forward and a backward may take different
 * paths: lse and o mean the same on both.
 *
 * swa_prefill_train: swa_prefill, plus for softmax the natural-log normaliser of every row,
 *   lse[b][h][i] = log sum_{j in K(i)} exp(x_ij), device float [B, H_q, N] (NULL allowed
 *   for sigmoid, which has no normaliser). Workspace as for swa_prefill.
 */
swa_status swa_prefill_train(const swa_prefill_params *p, const void *q, const void *k,
                             const void *v, void *o, float *lse, void *workspace,
                             size_t workspace_bytes, void *stream);

/*
 * swa_prefill_backward: gradients of a loss L given dout = dL/do [B, N, H_q, d]:
 *   dP_ij = dout_i . v_j
 *   dX_ij = dP_ij p_ij (1 - p_ij)            sigmoid (the logistic derivative)
 *         = p_ij (dP_ij - dout_i . o_i)      softmax (the row Jacobian; the general path
 *                                            sums dout_i . o_i as sum_j p_ij dP_ij, which
 *                                            keeps a bf16 o's rounding out)
 *   dv_j = sum_i p_ij dout_i,  dq_i = scale R(i)^T sum_j dX_ij R(j) k_j,
 *   dk_j = scale R(j)^T sum_i dX_ij R(i) q_i
 * over j in K(i); key and value gradients sum over the query heads of their group; the
 * ALiBi slopes get no gradient. dq [B, N, H_q, d], dk, dv [B, N, H_kv, d] are written
 * entirely (no accumulation into them). o, dout, dq, dk, dv have p->out_dtype; o and lse
 * (from swa_prefill_train with the same parameters and inputs) are read for softmax only
 * and may be NULL for sigmoid. workspace: swa_prefill_backward_workspace_bytes(p) bytes,
 * 16-byte aligned. The matrix-core path keeps float16 images of k, v, q and dout there
 * (B * N_tiles * 64 * d * 2 bytes for each of H_kv, H_kv, H_q and H_q heads, N_tiles =
 * ceil(N / 64)), for softmax 8 bytes of row statistics per (b, h, row), and with sinks a
 * float32 partial gradient of the sink keys; the general path, for softmax, one float per
 * (b, h, row) (none for sigmoid). With dilation > 1 the window is the dilated K(i) of
 * swa_prefill.
 */
swa_status swa_prefill_backward(const swa_prefill_params *p, const void *q, const void *k,
                                const void *v, const void *o, const float *lse,
                                const void *dout, void *dq, void *dk, void *dv,
                                void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of workspace swa_prefill_backward needs on whichever path it takes (0 when none,
 * or when the parameters are invalid). */
size_t swa_prefill_backward_workspace_bytes(const swa_prefill_params *p);

/*
 * RoPE angle table (SWAT: Sliding Window Attention Training, "RoPE: Stabilizing Sigmoid
 * Attention Training"; the RoFormer rotation it cites):
 *   table[pos][t] = (cos(pos * theta^(-2t/d)), sin(pos * theta^(-2t/d))), pos in
 *   [0, n_pos), t in [0, d/2), evaluated in float64 on the device and rounded to float32.
 * table: device float[n_pos * d/2 * 2]. Requires n_pos >= 0, d even >= 2, theta > 0.
 */
swa_status swa_rope_table(float *table, int64_t n_pos, int64_t d, double theta, void *stream);

/*
 * In-place rotation of x [B, N, H, d] (dtype), row n of batch b at position pos0[b] + n.
 * pos0: device int32[B]. rope_table: device [rope_rows, d/2, 2]. A row whose position is
 * outside [0, rope_rows) is set to NaN.
 */
swa_status swa_rope_apply(void *x, int64_t B, int64_t N, int64_t H, int64_t d,
                          const int32_t *pos0, const float *rope_table, int64_t rope_rows,
                          int32_t dtype, void *stream);

/*
 * Ring-buffer KV cache for num_seqs sequences (Sliding Window Attention glossary, ring
 * buffer: w slots, position i in slot i mod w, the oldest entry overwritten), plus a sink
 * store for positions 0..s-1 (Sliding-window beats linear attention, SWA(64, 4)).
 *   k_ring, v_ring : [num_seqs, H_kv, w, d]   keys stored rotated at their own position
 *   k_sink, v_sink : [num_seqs, H_kv, s, d]   NULL when s == 0
 * After positions 0..p of a sequence have been appended, slot t holds position
 * p - ((p - t) mod w) when that is >= 0; the cache itself stores no positions.
 */
typedef struct swa_cache {
    int64_t num_seqs, H_kv, w, s, d;
    int32_t dtype;             /* swa_dtype of every cache tensor                      */
    int32_t reserved;
    void *k_ring, *v_ring;
    void *k_sink, *v_sink;
} swa_cache;

/*
 * Append n_new tokens per sequence: token n of sequence q has position pos0[q] + n; its key
 * is rotated at that position (when rope_table is not NULL) and written with its value to
 * slot position mod w; positions below s are also written to the sink store. When
 * n_new > w, only the last w tokens reach the ring (the result equals appending one token
 * at a time). k_new, v_new : [num_seqs, n_new, H_kv, d] (cache dtype); pos0: device
 * int32[num_seqs]. A sequence whose pos0 is negative is skipped (nothing is written for
 * it), which lets one call serve a subset of the sequences. A key whose position lies
 * outside the rotation table is written as NaN.
 */
swa_status swa_kv_append(const swa_cache *c, const void *k_new, const void *v_new,
                         const int32_t *pos0, int64_t n_new, const float *rope_table,
                         int64_t rope_rows, void *stream);

/*
 * One query token per sequence over the ring cache. The query of sequence q sits at
 * position q_pos[q] and its own token must already be appended. Its keys are the ring
 * slots holding positions max(0, q_pos - w + 1) .. q_pos and the sink entries j < s that
 * the window no longer covers; scores, bias and weights are as in swa_prefill.
 *   q, o : [num_seqs, H_q, d]   (q not yet rotated; rotated here at q_pos)
 * H_q % cache->H_kv == 0. workspace: device memory of at least
 * swa_decode_workspace_bytes(p, c) bytes (may be NULL when that is 0).
 * Paths: a bf16 cache with d in {64, 128} and H_q / H_kv in {1, 2, 4, 8} runs on vector
 * kernels that read with 16-byte loads; they need q, o, the four cache tensors, the rotation
 * table and (when the call splits the window into key ranges) the workspace on 16-byte
 * boundaries. A call with any of them off that boundary, and every other shape, runs on a
 * general float32 kernel with element accesses, which needs no workspace: the result is
 * the same up to rounding.
 */
typedef struct swa_decode_params {
    int64_t H_q;
    int32_t mode;              /* swa_mode                                             */
    int32_t out_dtype;         /* swa_dtype of o                                       */
    float scale;               /* <= 0: 1/sqrt(d)                                      */
    int32_t reserved;
    const float *alibi_slopes; /* device float[H_q] or NULL                            */
    const float *rope_table;   /* device [rope_rows, d/2, 2] or NULL                   */
    int64_t rope_rows;
} swa_decode_params;

swa_status swa_decode(const swa_decode_params *p, const swa_cache *c, const void *q,
                      const int32_t *q_pos, void *o, void *workspace, size_t workspace_bytes,
                      void *stream);

/*
 * One decode step with the new token's append fused in. For each sequence q, the token at
 * position q_pos[q] - key k_new[q] (not yet rotated) and value v_new[q], both [num_seqs,
 * H_kv, d] in the cache dtype - is written to the ring (and to the sink store when
 * q_pos[q] < s) exactly as swa_kv_append with n_new = 1 writes it, and query q[q] is then
 * answered as swa_decode answers it. The append costs no launch of its own: the workgroup
 * whose key range holds q_pos writes the token and uses it without reading it back (long
 * windows over few sequences add the merge launch that swa_decode also uses).
 * A sequence whose q_pos is invalid (negative, or outside the rotation table) gets NaN
 * outputs and its cache is left untouched. Other arguments as in swa_decode; the alignment
 * rule there covers k_new and v_new too (off a 16-byte boundary, the append and the query
 * run as two launches on the general kernels).
 */
swa_status swa_decode_append(const swa_decode_params *p, const swa_cache *c, const void *q,
                             const void *k_new, const void *v_new, const int32_t *q_pos,
                             void *o, void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of workspace swa_decode needs for this problem (0 when it needs none). */
size_t swa_decode_workspace_bytes(const swa_decode_params *p, const swa_cache *c);

/*
 * swa_decode_append for callers that cannot allocate device memory or pass a workspace
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same computation and the same kernels, with the split partials kept in a 4 MiB device
 * array inside the library instead of a workspace. Each GPU the library runs on holds its own
 * copy of that array from the first call on that device until the process ends; the first
 * call on a device looks up the array's address (no allocation). The call allocates and frees
 * nothing. Every call on one GPU shares that GPU's array, so calls that overlap in time on
 * one GPU (on different streams, or from several threads) race and must not be issued.
 * A problem whose swa_decode_workspace_bytes exceeds 4 MiB is rejected with
 * SWA_ERR_UNSUPPORTED before anything is launched (use swa_decode_append with a workspace).
 * Arguments, layouts and errors otherwise as swa_decode_append.
 */
swa_status swa_decode_append_static(const swa_decode_params *p, const swa_cache *c,
                                    const void *q, const void *k_new, const void *v_new,
                                    const int32_t *q_pos, void *o, void *stream);

/*
 * Chunked prefill over the ring cache, variable-length batch (a new chunk of each sequence
 * attends to its cached history and to itself; Sliding Window Attention glossary: the ring
 * buffer keeps the last w tokens, which is all a chunk's window can reach besides the sinks).
 * Sequence q owns the packed rows cu_seqlens[q] .. cu_seqlens[q+1]-1 of q, k_new, v_new
 * and o; row cu_seqlens[q] + r is the token at position pos0[q] + r. The cache must hold
 * positions 0 .. pos0[q]-1 of that sequence, appended earlier (swa_kv_append, an earlier
 * chunk, or decode steps). Every query i of the chunk is answered over the key set K(i)
 * of swa_prefill, reading keys j < pos0[q] from the ring or the sink store and keys
 * j >= pos0[q] from the chunk; scores, bias and weights are as in swa_prefill. After the
 * attention the chunk is appended to the cache exactly as swa_kv_append would append it.
 *   q, o         : [total_rows, H_q, d]    (q not rotated)
 *   k_new, v_new : [total_rows, H_kv, d]   (cache dtype, keys not rotated)
 *   cu_seqlens   : device int32[num_seqs + 1]   pos0: device int32[num_seqs]
 *   max_seqlen   : host bound on cu_seqlens[q+1] - cu_seqlens[q]
 * p: as for swa_decode (its out_dtype is the dtype of o). A sequence with no rows is a no-op.
 * A sequence whose pos0 is negative, whose row count exceeds max_seqlen, or whose last
 * position lies outside the rotation table gets NaN rows and its cache is left untouched;
 * rows outside [0, total_rows) are never written (such a sequence is skipped). Sequences'
 * row ranges must not overlap.
 * Requirements: a bf16 cache with d in {64, 128} and 16-byte aligned tensors (else
 * SWA_ERR_UNSUPPORTED). The attention runs on the matrix cores as in swa_prefill, with the
 * same operand ranges. workspace: device scratch of swa_prefill_chunk_workspace_bytes bytes,
 * 16-byte aligned, holding float16 tile images of each sequence's sinks and of the window
 * positions the chunk can reach: about 2 * num_seqs * H_kv * (s + w + max_seqlen) * d * 2
 * bytes (fewer when the rotation table bounds the positions).
 */
swa_status swa_prefill_chunk(const swa_decode_params *p, const swa_cache *c, const void *q,
                             const void *k_new, const void *v_new, const int32_t *cu_seqlens,
                             const int32_t *pos0, int64_t total_rows, int64_t max_seqlen,
                             void *o, void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of workspace swa_prefill_chunk needs (0 when it needs none or the arguments are
 * invalid or unsupported). */
size_t swa_prefill_chunk_workspace_bytes(const swa_decode_params *p, const swa_cache *c,
                                         int64_t total_rows, int64_t max_seqlen);

/* Static, human-readable text for a status code. */
const char *swa_status_string(swa_status s);

/* The hipError_t of the most recent SWA_ERR_HIP returned on this thread (0 if none). */
int swa_last_hip_error(void);

/* Version of this interface: major * 10000 + minor * 100 + patch. */
int swa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBSWA_SWA_H */
