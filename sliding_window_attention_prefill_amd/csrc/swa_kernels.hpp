// swa_kernels.hpp - host-side launch interface between the C ABI layer and the kernels.
// Arguments here are already validated; each launcher only enqueues work on the stream.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace swa {

struct PrefillArgs {
    int64_t B, Hq, Hkv, N, d, w, s;
    int mode;           // 0 sigmoid, 1 softmax
    int in_dt, out_dt;  // 0 float32, 1 bfloat16
    float scale;        // resolved (> 0)
    const float *slopes;
    const float *rope;  // [rope_rows, d/2, 2] or null
    int64_t rope_rows;
    int64_t dil;        // window dilation (1: contiguous)
};

struct CacheArgs {
    int64_t S, Hkv, w, s, d;
    int dt;
    void *k_ring, *v_ring, *k_sink, *v_sink;
};

struct DecodeArgs {
    int64_t Hq;
    int mode, out_dt;
    float scale;
    const float *slopes;
    const float *rope;
    int64_t rope_rows;
};

// General vector kernel: any even d <= 256, float32 or bfloat16 in/out. lse (softmax only,
// may be null): the log-normaliser of every row, [B, Hq, N] float32.
hipError_t launch_prefill_simt(const PrefillArgs &a, const void *q, const void *k,
                               const void *v, void *o, hipStream_t st, float *lse = nullptr);

// Backward of the general kernel (any shape it takes): dq, dk, dv in the out dtype from
// dout (out dtype) and, for softmax, lse. ws: prefill_bwd_simt_workspace_bytes(a) bytes,
// 4-byte aligned (softmax: one float per row for sum_j p_ij dP_ij).
size_t prefill_bwd_simt_workspace_bytes(const PrefillArgs &a);
hipError_t launch_prefill_bwd_simt(const PrefillArgs &a, const void *q, const void *k,
                                   const void *v, const float *lse, const void *dout, void *dq,
                                   void *dk, void *dv, void *ws, hipStream_t st);

// Matrix-core kernel: bfloat16 inputs, d in {64, 128}; prefill_mfma_supported tells
// whether a shape is covered (the caller otherwise uses the general kernel). ws must hold
// prefill_mfma_workspace_bytes(a) bytes (packed K/V tile images), 16-byte aligned.
bool prefill_mfma_supported(const PrefillArgs &a);
size_t prefill_mfma_workspace_bytes(const PrefillArgs &a);
// lse (softmax only, may be null): the log-normaliser of every row, [B, Hq, N] float32.
hipError_t launch_prefill_mfma(const PrefillArgs &a, const void *q, const void *k,
                               const void *v, void *o, void *ws, hipStream_t st,
                               float *lse = nullptr);

// Backward of the matrix-core prefill (bf16 inputs, d in {64, 128}): gradients dq, dk, dv
// (out dtype) from dout (out dtype), the forward output o and, for softmax, the forward's
// lse. ws holds prefill_bwd_workspace_bytes(a) bytes, 16-byte aligned.
size_t prefill_bwd_workspace_bytes(const PrefillArgs &a);
hipError_t launch_prefill_bwd(const PrefillArgs &a, const void *q, const void *k,
                              const void *v, const void *o, const float *lse, const void *dout,
                              void *dq, void *dk, void *dv, void *ws, hipStream_t st);

hipError_t launch_rope_table(float *table, int64_t n_pos, int64_t d, double theta,
                             hipStream_t st);
hipError_t launch_rope_apply(void *x, int64_t B, int64_t N, int64_t H, int64_t d,
                             const int32_t *pos0, const float *rope, int64_t rope_rows, int dt,
                             hipStream_t st);

hipError_t launch_kv_append(const CacheArgs &c, const void *k_new, const void *v_new,
                            const int32_t *pos0, int64_t n_new, const float *rope,
                            int64_t rope_rows, hipStream_t st);

size_t decode_workspace_bytes(const DecodeArgs &a, const CacheArgs &c);
hipError_t launch_decode(const DecodeArgs &a, const CacheArgs &c, const void *q,
                         const int32_t *q_pos, void *o, void *ws, size_t ws_bytes,
                         hipStream_t st);
// Chunked prefill over the ring cache (packed rows, cu/pos0 per sequence): a gather
// pre-pass builds float16 tile images from sinks, ring and chunk, the matrix-core kernel
// attends, then the chunk is appended. bf16 caches with d in {64, 128} only; ws must hold
// prefill_chunk_workspace_bytes bytes, 16-byte aligned.
bool prefill_chunk_supported(const DecodeArgs &a, const CacheArgs &c, int64_t T, int64_t max_q);
size_t prefill_chunk_workspace_bytes(const DecodeArgs &a, const CacheArgs &c, int64_t T,
                                     int64_t max_q);
hipError_t launch_prefill_chunk(const DecodeArgs &a, const CacheArgs &c, const void *q,
                                const void *k_new, const void *v_new, const int32_t *cu,
                                const int32_t *pos0, int64_t T, int64_t max_q, void *o,
                                void *ws, hipStream_t st);

// Append one token per sequence at q_pos, then decode (one launch where possible).
hipError_t launch_decode_append(const DecodeArgs &a, const CacheArgs &c, const void *q,
                                const void *k_new, const void *v_new, const int32_t *q_pos,
                                void *o, void *ws, size_t ws_bytes, hipStream_t st);

// The device scratch array for callers that cannot allocate: its size, and its address on
// the current device (looked up once per device; *ptr is the address kernels may use).
size_t decode_scratch_bytes();
hipError_t decode_scratch(void **ptr);

}  // namespace swa
