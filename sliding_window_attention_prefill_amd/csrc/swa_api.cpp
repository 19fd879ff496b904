// swa_api.cpp - the libswa C ABI: argument validation and kernel dispatch.
//
// Every entry point validates its arguments on the host before anything is enqueued, so
// a rejected call touches no memory. Launch failures are reported as SWA_ERR_HIP with the
// HIP error kept per thread for swa_last_hip_error().
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <initializer_list>

#include "../../include/swa.h"
#include "swa_kernels.hpp"

namespace {

thread_local int g_last_hip_error = 0;

swa_status hip_status(hipError_t e) {
    if (e == hipSuccess) return SWA_OK;
    g_last_hip_error = (int)e;
    return SWA_ERR_HIP;
}

bool valid_dtype(int32_t dt) { return dt == SWA_F32 || dt == SWA_BF16; }
bool valid_mode(int32_t m) { return m == SWA_SIGMOID || m == SWA_SOFTMAX; }

float resolve_scale(float scale, int64_t d) {
    return scale > 0.0f ? scale : (float)(1.0 / std::sqrt((double)d));
}

}  // namespace

extern "C" {

int swa_version(void) { return 500; }

const char *swa_status_string(swa_status s) {
    switch (s) {
        case SWA_OK: return "ok";
        case SWA_ERR_INVALID_ARGUMENT: return "invalid argument";
        case SWA_ERR_UNSUPPORTED: return "unsupported combination";
        case SWA_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

int swa_last_hip_error(void) { return g_last_hip_error; }

// Host-side checks shared by swa_prefill and swa_prefill_workspace_bytes.
static swa_status check_prefill(const swa_prefill_params *p) {
    if (!p) return SWA_ERR_INVALID_ARGUMENT;
    if (p->B < 0 || p->N < 0 || p->H_q < 1 || p->H_kv < 1 || p->H_q % p->H_kv != 0)
        return SWA_ERR_INVALID_ARGUMENT;
    if (p->d < 2 || p->d % 2 != 0 || p->w < 1 || p->s < 0) return SWA_ERR_INVALID_ARGUMENT;
    if (!valid_mode(p->mode) || !valid_dtype(p->in_dtype) || !valid_dtype(p->out_dtype))
        return SWA_ERR_INVALID_ARGUMENT;
    if (!std::isfinite(p->scale)) return SWA_ERR_INVALID_ARGUMENT;
    if (p->rope_table && p->rope_rows < p->N) return SWA_ERR_INVALID_ARGUMENT;
    if (p->dilation < 0) return SWA_ERR_INVALID_ARGUMENT;
    if (p->d > 256) return SWA_ERR_UNSUPPORTED;
    // positions travel as float-exact integers and 32-bit grid dimensions
    if (p->N > (int64_t(1) << 24)) return SWA_ERR_UNSUPPORTED;
    return SWA_OK;
}

static swa::PrefillArgs prefill_args(const swa_prefill_params *p) {
    return swa::PrefillArgs{p->B, p->H_q, p->H_kv, p->N, p->d, p->w, p->s, p->mode,
                            p->in_dtype, p->out_dtype, resolve_scale(p->scale, p->d),
                            p->alibi_slopes, p->rope_table, p->rope_table ? p->rope_rows : 0,
                            // a dilation of at least N keeps only i - j = 0 in the window;
                            // 2^24 >= N stands for every larger one
                            p->dilation > 1 ? std::min<int64_t>(p->dilation, int64_t(1) << 24)
                                            : 1};
}

size_t swa_prefill_workspace_bytes(const swa_prefill_params *p) {
    if (check_prefill(p) != SWA_OK) return 0;
    const swa::PrefillArgs a = prefill_args(p);
    return swa::prefill_mfma_supported(a) ? swa::prefill_mfma_workspace_bytes(a) : 0;
}

swa_status swa_prefill(const swa_prefill_params *p, const void *q, const void *k,
                       const void *v, void *o, void *workspace, size_t workspace_bytes,
                       void *stream) {
    const swa_status chk = check_prefill(p);
    if (chk != SWA_OK) return chk;
    const int64_t elems = p->B * p->N;
    if (elems > 0 && (!q || !k || !v || !o)) return SWA_ERR_INVALID_ARGUMENT;

    const swa::PrefillArgs a = prefill_args(p);
    hipStream_t st = static_cast<hipStream_t>(stream);
    // the matrix-core kernel moves 16-byte vectors: it needs 16-byte aligned tensors
    const bool aligned = ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) |
                           reinterpret_cast<uintptr_t>(v) | reinterpret_cast<uintptr_t>(o) |
                           reinterpret_cast<uintptr_t>(p->rope_table)) & 15) == 0;
    if (aligned && swa::prefill_mfma_supported(a)) {
        const size_t need = swa::prefill_mfma_workspace_bytes(a);
        if (need > 0 && (!workspace || workspace_bytes < need ||
                         (reinterpret_cast<uintptr_t>(workspace) & 15) != 0))
            return SWA_ERR_INVALID_ARGUMENT;
        return hip_status(swa::launch_prefill_mfma(a, q, k, v, o, workspace, st));
    }
    if ((a.B * a.N * a.Hq + 3) / 4 > 0x7fffffff) return SWA_ERR_UNSUPPORTED;
    return hip_status(swa::launch_prefill_simt(a, q, k, v, o, st));
}

// The training pair runs on the matrix cores for bf16 inputs, d in {64, 128}, a contiguous
// window and 16-byte aligned tensors, and on the general vector kernels otherwise.
static bool train_on_mfma(const swa::PrefillArgs &a, const swa_prefill_params *p,
                          std::initializer_list<const void *> ptrs) {
    if (!swa::prefill_mfma_supported(a) || a.dil != 1) return false;
    uintptr_t bits = reinterpret_cast<uintptr_t>(p->rope_table);
    for (const void *x : ptrs) bits |= reinterpret_cast<uintptr_t>(x);
    return (bits & 15) == 0;
}

swa_status swa_prefill_train(const swa_prefill_params *p, const void *q, const void *k,
                             const void *v, void *o, float *lse, void *workspace,
                             size_t workspace_bytes, void *stream) {
    const swa_status chk = check_prefill(p);
    if (chk != SWA_OK) return chk;
    const int64_t elems = p->B * p->N;
    if (elems > 0 && (!q || !k || !v || !o)) return SWA_ERR_INVALID_ARGUMENT;
    if (elems > 0 && p->mode == SWA_SOFTMAX && !lse) return SWA_ERR_INVALID_ARGUMENT;
    const swa::PrefillArgs a = prefill_args(p);
    hipStream_t st = static_cast<hipStream_t>(stream);
    float *row_lse = p->mode == SWA_SOFTMAX ? lse : nullptr;
    if (train_on_mfma(a, p, {q, k, v, o})) {
        const size_t need = swa::prefill_mfma_workspace_bytes(a);
        if (need > 0 && (!workspace || workspace_bytes < need ||
                         (reinterpret_cast<uintptr_t>(workspace) & 15) != 0))
            return SWA_ERR_INVALID_ARGUMENT;
        return hip_status(swa::launch_prefill_mfma(a, q, k, v, o, workspace, st, row_lse));
    }
    if ((a.B * a.N * a.Hq + 3) / 4 > 0x7fffffff) return SWA_ERR_UNSUPPORTED;
    return hip_status(swa::launch_prefill_simt(a, q, k, v, o, st, row_lse));
}

// Workspace for whichever path a call takes: the matrix-core need (when that path can be
// taken) covers the general path's (4 bytes per softmax row against at least 8).
size_t swa_prefill_backward_workspace_bytes(const swa_prefill_params *p) {
    if (check_prefill(p) != SWA_OK) return 0;
    const swa::PrefillArgs a = prefill_args(p);
    const size_t gen = swa::prefill_bwd_simt_workspace_bytes(a);
    if (!swa::prefill_mfma_supported(a) || a.dil != 1) return gen;
    const size_t mf = swa::prefill_bwd_workspace_bytes(a);
    return mf > gen ? mf : gen;
}

swa_status swa_prefill_backward(const swa_prefill_params *p, const void *q, const void *k,
                                const void *v, const void *o, const float *lse,
                                const void *dout, void *dq, void *dk, void *dv,
                                void *workspace, size_t workspace_bytes, void *stream) {
    const swa_status chk = check_prefill(p);
    if (chk != SWA_OK) return chk;
    const int64_t elems = p->B * p->N;
    if (elems > 0 && (!q || !k || !v || !dout || !dq || !dk || !dv))
        return SWA_ERR_INVALID_ARGUMENT;
    if (elems > 0 && p->mode == SWA_SOFTMAX && (!o || !lse)) return SWA_ERR_INVALID_ARGUMENT;
    const swa::PrefillArgs a = prefill_args(p);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (train_on_mfma(a, p, {q, k, v, o, dout, dq, dk, dv})) {
        const size_t need = swa::prefill_bwd_workspace_bytes(a);
        if (need > 0 && (!workspace || workspace_bytes < need ||
                         (reinterpret_cast<uintptr_t>(workspace) & 15) != 0))
            return SWA_ERR_INVALID_ARGUMENT;
        return hip_status(
            swa::launch_prefill_bwd(a, q, k, v, o, lse, dout, dq, dk, dv, workspace, st));
    }
    if ((a.B * a.N * a.Hq + 3) / 4 > 0x7fffffff) return SWA_ERR_UNSUPPORTED;
    const size_t need = swa::prefill_bwd_simt_workspace_bytes(a);
    if (need > 0 && (!workspace || workspace_bytes < need ||
                     (reinterpret_cast<uintptr_t>(workspace) & 15) != 0))
        return SWA_ERR_INVALID_ARGUMENT;
    return hip_status(
        swa::launch_prefill_bwd_simt(a, q, k, v, lse, dout, dq, dk, dv, workspace, st));
}

swa_status swa_rope_table(float *table, int64_t n_pos, int64_t d, double theta, void *stream) {
    if (n_pos < 0 || d < 2 || d % 2 != 0 || !(theta > 0.0) || !std::isfinite(theta))
        return SWA_ERR_INVALID_ARGUMENT;
    if (n_pos > 0 && !table) return SWA_ERR_INVALID_ARGUMENT;
    if ((n_pos * (d / 2) + 255) / 256 > 0x7fffffff) return SWA_ERR_UNSUPPORTED;
    return hip_status(swa::launch_rope_table(table, n_pos, d, theta, static_cast<hipStream_t>(stream)));
}

swa_status swa_rope_apply(void *x, int64_t B, int64_t N, int64_t H, int64_t d,
                          const int32_t *pos0, const float *rope_table, int64_t rope_rows,
                          int32_t dtype, void *stream) {
    if (B < 0 || N < 0 || H < 1 || d < 2 || d % 2 != 0 || !valid_dtype(dtype) || rope_rows < 0)
        return SWA_ERR_INVALID_ARGUMENT;
    if (B * N > 0 && (!x || !pos0 || !rope_table)) return SWA_ERR_INVALID_ARGUMENT;
    if ((B * N * H * (d / 2) + 255) / 256 > 0x7fffffff) return SWA_ERR_UNSUPPORTED;
    return hip_status(swa::launch_rope_apply(x, B, N, H, d, pos0, rope_table, rope_rows, dtype,
                                             static_cast<hipStream_t>(stream)));
}

static swa_status check_cache(const swa_cache *c) {
    if (!c) return SWA_ERR_INVALID_ARGUMENT;
    if (c->num_seqs < 0 || c->H_kv < 1 || c->w < 1 || c->s < 0 || c->d < 2 || c->d % 2 != 0 ||
        !valid_dtype(c->dtype))
        return SWA_ERR_INVALID_ARGUMENT;
    if (c->num_seqs > 0 && (!c->k_ring || !c->v_ring)) return SWA_ERR_INVALID_ARGUMENT;
    if (c->num_seqs > 0 && c->s > 0 && (!c->k_sink || !c->v_sink)) return SWA_ERR_INVALID_ARGUMENT;
    if (c->d > 256) return SWA_ERR_UNSUPPORTED;
    return SWA_OK;
}

static swa::CacheArgs cache_args(const swa_cache *c) {
    return swa::CacheArgs{c->num_seqs, c->H_kv, c->w, c->s, c->d, c->dtype,
                          c->k_ring, c->v_ring, c->k_sink, c->v_sink};
}

swa_status swa_kv_append(const swa_cache *c, const void *k_new, const void *v_new,
                         const int32_t *pos0, int64_t n_new, const float *rope_table,
                         int64_t rope_rows, void *stream) {
    swa_status st = check_cache(c);
    if (st != SWA_OK) return st;
    if (n_new < 0 || (rope_table && rope_rows < 0)) return SWA_ERR_INVALID_ARGUMENT;
    if (c->num_seqs * n_new > 0 && (!k_new || !v_new || !pos0)) return SWA_ERR_INVALID_ARGUMENT;
    if (c->num_seqs * n_new * c->H_kv > 0x7fffffff) return SWA_ERR_UNSUPPORTED;
    return hip_status(swa::launch_kv_append(cache_args(c), k_new, v_new, pos0, n_new, rope_table,
                                            rope_table ? rope_rows : 0,
                                            static_cast<hipStream_t>(stream)));
}

static swa_status check_decode(const swa_decode_params *p, const swa_cache *c) {
    swa_status st = check_cache(c);
    if (st != SWA_OK) return st;
    if (!p || p->H_q < 1 || p->H_q % c->H_kv != 0 || !valid_mode(p->mode) ||
        !valid_dtype(p->out_dtype) || !std::isfinite(p->scale))
        return SWA_ERR_INVALID_ARGUMENT;
    if (p->rope_table && p->rope_rows < 0) return SWA_ERR_INVALID_ARGUMENT;
    if (p->H_q / c->H_kv > 64) return SWA_ERR_UNSUPPORTED;
    return SWA_OK;
}

static swa::DecodeArgs decode_args(const swa_decode_params *p, int64_t d) {
    return swa::DecodeArgs{p->H_q, p->mode, p->out_dtype, resolve_scale(p->scale, d),
                           p->alibi_slopes, p->rope_table, p->rope_table ? p->rope_rows : 0};
}

size_t swa_decode_workspace_bytes(const swa_decode_params *p, const swa_cache *c) {
    if (check_decode(p, c) != SWA_OK) return 0;
    return swa::decode_workspace_bytes(decode_args(p, c->d), cache_args(c));
}

swa_status swa_decode(const swa_decode_params *p, const swa_cache *c, const void *q,
                      const int32_t *q_pos, void *o, void *workspace, size_t workspace_bytes,
                      void *stream) {
    swa_status st = check_decode(p, c);
    if (st != SWA_OK) return st;
    if (c->num_seqs > 0 && (!q || !q_pos || !o)) return SWA_ERR_INVALID_ARGUMENT;
    const swa::DecodeArgs a = decode_args(p, c->d);
    const swa::CacheArgs ca = cache_args(c);
    const size_t need = swa::decode_workspace_bytes(a, ca);
    if (need > 0 && (!workspace || workspace_bytes < need)) return SWA_ERR_INVALID_ARGUMENT;
    if (c->num_seqs * c->H_kv > 0x7fffffff) return SWA_ERR_UNSUPPORTED;
    const hipError_t e = swa::launch_decode(a, ca, q, q_pos, o, workspace, workspace_bytes,
                                            static_cast<hipStream_t>(stream));
    if (e == hipErrorNotSupported) return SWA_ERR_UNSUPPORTED;
    return hip_status(e);
}

swa_status swa_decode_append(const swa_decode_params *p, const swa_cache *c, const void *q,
                             const void *k_new, const void *v_new, const int32_t *q_pos,
                             void *o, void *workspace, size_t workspace_bytes, void *stream) {
    swa_status st = check_decode(p, c);
    if (st != SWA_OK) return st;
    if (c->num_seqs > 0 && (!q || !q_pos || !o || !k_new || !v_new)) return SWA_ERR_INVALID_ARGUMENT;
    const swa::DecodeArgs a = decode_args(p, c->d);
    const swa::CacheArgs ca = cache_args(c);
    const size_t need = swa::decode_workspace_bytes(a, ca);
    if (need > 0 && (!workspace || workspace_bytes < need)) return SWA_ERR_INVALID_ARGUMENT;
    if (c->num_seqs * c->H_kv > 0x7fffffff) return SWA_ERR_UNSUPPORTED;
    const hipError_t e = swa::launch_decode_append(a, ca, q, k_new, v_new, q_pos, o, workspace,
                                                   workspace_bytes, static_cast<hipStream_t>(stream));
    if (e == hipErrorNotSupported) return SWA_ERR_UNSUPPORTED;
    return hip_status(e);
}

swa_status swa_decode_append_static(const swa_decode_params *p, const swa_cache *c,
                                    const void *q, const void *k_new, const void *v_new,
                                    const int32_t *q_pos, void *o, void *stream) {
    swa_status st = check_decode(p, c);
    if (st != SWA_OK) return st;
    if (c->num_seqs > 0 && (!q || !q_pos || !o || !k_new || !v_new)) return SWA_ERR_INVALID_ARGUMENT;
    if (c->num_seqs * c->H_kv > 0x7fffffff) return SWA_ERR_UNSUPPORTED;
    const swa::DecodeArgs a = decode_args(p, c->d);
    const swa::CacheArgs ca = cache_args(c);
    // the split partials must fit the library's scratch array (checked before any HIP call)
    const size_t need = swa::decode_workspace_bytes(a, ca);
    if (need > swa::decode_scratch_bytes()) return SWA_ERR_UNSUPPORTED;
    if (c->num_seqs == 0) return SWA_OK;
    void *ws = nullptr;
    if (need > 0) {
        const hipError_t e = swa::decode_scratch(&ws);
        if (e != hipSuccess) return hip_status(e);
    }
    const hipError_t e = swa::launch_decode_append(a, ca, q, k_new, v_new, q_pos, o, ws, need,
                                                   static_cast<hipStream_t>(stream));
    if (e == hipErrorNotSupported) return SWA_ERR_UNSUPPORTED;
    return hip_status(e);
}

static bool aligned16(std::initializer_list<const void *> ptrs) {
    uintptr_t bits = 0;
    for (const void *x : ptrs) bits |= reinterpret_cast<uintptr_t>(x);
    return (bits & 15) == 0;
}

static swa_status check_chunk(const swa_decode_params *p, const swa_cache *c, int64_t total_rows,
                              int64_t max_seqlen) {
    swa_status st = check_decode(p, c);
    if (st != SWA_OK) return st;
    if (total_rows < 0 || max_seqlen < 0) return SWA_ERR_INVALID_ARGUMENT;
    if (total_rows > 0x7fffffff) return SWA_ERR_UNSUPPORTED;  // rows are int32 offsets
    if (!swa::prefill_chunk_supported(decode_args(p, c->d), cache_args(c), total_rows, max_seqlen))
        return SWA_ERR_UNSUPPORTED;
    return SWA_OK;
}

size_t swa_prefill_chunk_workspace_bytes(const swa_decode_params *p, const swa_cache *c,
                                         int64_t total_rows, int64_t max_seqlen) {
    if (check_chunk(p, c, total_rows, max_seqlen) != SWA_OK) return 0;
    return swa::prefill_chunk_workspace_bytes(decode_args(p, c->d), cache_args(c), total_rows,
                                              max_seqlen);
}

swa_status swa_prefill_chunk(const swa_decode_params *p, const swa_cache *c, const void *q,
                             const void *k_new, const void *v_new, const int32_t *cu_seqlens,
                             const int32_t *pos0, int64_t total_rows, int64_t max_seqlen,
                             void *o, void *workspace, size_t workspace_bytes, void *stream) {
    swa_status st = check_chunk(p, c, total_rows, max_seqlen);
    if (st != SWA_OK) return st;
    if (c->num_seqs > 0 && (!cu_seqlens || !pos0)) return SWA_ERR_INVALID_ARGUMENT;
    if (c->num_seqs > 0 && total_rows > 0 && (!q || !k_new || !v_new || !o))
        return SWA_ERR_INVALID_ARGUMENT;
    // 16-byte vector moves on every tensor
    if (!aligned16({q, k_new, v_new, o, c->k_ring, c->v_ring, c->k_sink, c->v_sink,
                    p->rope_table}))
        return SWA_ERR_UNSUPPORTED;
    const swa::DecodeArgs a = decode_args(p, c->d);
    const swa::CacheArgs ca = cache_args(c);
    const size_t need = swa::prefill_chunk_workspace_bytes(a, ca, total_rows, max_seqlen);
    if (need > 0 && (!workspace || workspace_bytes < need ||
                     (reinterpret_cast<uintptr_t>(workspace) & 15) != 0))
        return SWA_ERR_INVALID_ARGUMENT;
    return hip_status(swa::launch_prefill_chunk(a, ca, q, k_new, v_new, cu_seqlens, pos0,
                                                total_rows, max_seqlen, o, workspace,
                                                static_cast<hipStream_t>(stream)));
}

}  // extern "C"
