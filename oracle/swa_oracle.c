/*
 * swa_oracle.c - CPU oracle for causal sliding-window attention.
 *
 * TEST INFRASTRUCTURE ONLY. The tests, the smoke check and the bench's CPU-baseline leg
 * call this file; the product path (HIP kernels behind the libswa C ABI) never does, and
 * the two share no code, header, table or constant.
 *
 * Everything here is the plain definition evaluated in float64, one query row at a time,
 * from the same (already rounded) input values the GPU reads:
 *
 *   key set    K(i) = { j : 0 <= j <= i  and  (i - j < w  or  j < s) }
 *                 - the causal band: each token sees itself and the w-1 tokens before it
 *                   (Sliding Window Attention glossary, the boolean band mask example);
 *                 - s sink tokens kept beside the window (Sliding Window Attention glossary,
 *                   "attention sink" entry; Sliding-window beats linear attention, SWA(64,4)).
 *   rotation   R(p): pairs (2t, 2t+1) rotated by the angle p * theta^(-2t/d)
 *                 (SWAT: Sliding Window Attention Training, symbol map and "RoPE"; the
 *                 RoFormer rotation it cites).
 *   score      x_ij = scale * (R(i) q_i) . (R(j) k_j) + slope_h * (i - j)
 *                 (SWAT page, "Balanced ALiBi" attention equation; scale = 1/sqrt(d)).
 *   weights    sigmoid: p_ij = 1 / (1 + exp(-x_ij)), no normalisation (SWAT page,
 *                 "Sigmoid" equation); softmax: p_ij = exp(x_ij - m_i) / sum_K exp(x - m_i)
 *                 with m_i the row maximum over K(i) (SWAT page, "Why this exists").
 *   output     o_i = sum_{j in K(i)} p_ij v_j.
 *
 * Decode keeps an explicit ring of w slots per (sequence, kv head) holding
 * (position, rotated key, value): position p is written to slot p mod w, overwriting the
 * oldest entry (Sliding Window Attention glossary, ring-buffer paragraph), and a sink store
 * of s entries. Keys are stored rotated at their own absolute position.
 *
 * Layouts (row-major, innermost last): q/o [B, N, H_q, d]; k/v [B, N, H_kv, d];
 * query head h reads kv head h / (H_q / H_kv).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_SIGMOID 0
#define ORACLE_SOFTMAX 1

int swa_oracle_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* cos/sin of the rotation angle p * theta^(-2t/d), for positions [0, P) and t in [0, d/2). */
static void rope_table(int64_t P, int64_t d, double theta, double *cs, double *sn) {
    int64_t half = d / 2;
    for (int64_t p = 0; p < P; ++p) {
        for (int64_t t = 0; t < half; ++t) {
            double freq = pow(theta, -2.0 * (double)t / (double)d);
            double phi = (double)p * freq;
            cs[p * half + t] = cos(phi);
            sn[p * half + t] = sin(phi);
        }
    }
}

/* y = R(p) x, with the rotation read from a row of the table. */
static void rotate(const double *x, double *y, int64_t d, const double *c, const double *s) {
    for (int64_t t = 0; t < d / 2; ++t) {
        double a = x[2 * t], b = x[2 * t + 1];
        y[2 * t] = a * c[t] - b * s[t];
        y[2 * t + 1] = a * s[t] + b * c[t];
    }
}

/* Same rotation, angle computed directly (used by decode, one position at a time). */
static void rotate_direct(const double *x, double *y, int64_t d, int64_t p, double theta) {
    for (int64_t t = 0; t < d / 2; ++t) {
        double freq = pow(theta, -2.0 * (double)t / (double)d);
        double phi = (double)p * freq;
        double c = cos(phi), s = sin(phi);
        double a = x[2 * t], b = x[2 * t + 1];
        y[2 * t] = a * c - b * s;
        y[2 * t + 1] = a * s + b * c;
    }
}

static double dot(const double *a, const double *b, int64_t d) {
    double acc = 0.0;
    for (int64_t c = 0; c < d; ++c) acc += a[c] * b[c];
    return acc;
}

/* Weights from scores, in place: sigmoid elementwise, or softmax over the n entries. */
static void weights(double *x, int64_t n, int mode) {
    if (mode == ORACLE_SIGMOID) {
        for (int64_t e = 0; e < n; ++e) x[e] = 1.0 / (1.0 + exp(-x[e]));
        return;
    }
    double m = -INFINITY;
    for (int64_t e = 0; e < n; ++e) if (x[e] > m) m = x[e];
    double z = 0.0;
    for (int64_t e = 0; e < n; ++e) { x[e] = exp(x[e] - m); z += x[e]; }
    for (int64_t e = 0; e < n; ++e) x[e] /= z;
}

/*
 * Prefill. rows == NULL: every query row i in [0, N) is computed and o is [B, N, H_q, d].
 * Otherwise only the listed rows are computed and o is [B, n_rows, H_q, d], in list order.
 * slopes: float64[H_q] signed ALiBi slopes, or NULL for no bias. theta <= 0: no rotation.
 * scale <= 0 means 1/sqrt(d). Returns 0, or -1 on bad arguments / allocation failure.
 */
/*
 * K(i) written out as an ascending list of key positions: the sinks below the window
 * [0, min(s, lo)), then the window. With dil = 1 the window is [lo, i], lo = max(0, i-w+1)
 * (the band mask of the Sliding Window Attention glossary, sinks per the SWA(w, s) rule of
 * Sliding-window beats linear attention); with dil > 1 it keeps i, i - dil, ...,
 * i - dil (w - 1) and every sink position inside it. Returns the count.
 */
static int64_t key_set(int64_t i, int64_t w, int64_t s, int64_t dil, int64_t *key) {
    int64_t n = 0;
    int64_t lo = i - dil * (w - 1) > 0 ? i - dil * (w - 1) : 0;
    for (int64_t j = 0; j < s && j < lo; ++j) key[n++] = j;
    for (int64_t j = lo; j <= i; ++j)
        if ((i - j) % dil == 0 || j < s) key[n++] = j;
    return n;
}

static int prefill_impl(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d, int64_t w,
                        int64_t s, int64_t dil, int mode, double scale, const double *slopes,
                        double theta, const double *q, const double *k, const double *v,
                        const int64_t *rows, int64_t n_rows, double *o) {
    if (B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || N < 0 || d <= 0 || w < 1 || s < 0 ||
        dil < 1)
        return -1;
    if (theta > 0.0 && d % 2 != 0) return -1;
    if (scale <= 0.0) scale = 1.0 / sqrt((double)d);
    int64_t nr = rows ? n_rows : N;
    if (rows) {
        for (int64_t r = 0; r < n_rows; ++r) if (rows[r] < 0 || rows[r] >= N) return -1;
    }
    int64_t P = 0;
    for (int64_t r = 0; r < nr; ++r) {
        int64_t i = rows ? rows[r] : r;
        if (i + 1 > P) P = i + 1;
    }
    int64_t half = d / 2;
    double *cs = NULL, *sn = NULL;
    if (theta > 0.0 && P > 0) {
        cs = (double *)malloc(sizeof(double) * (size_t)(P * half));
        sn = (double *)malloc(sizeof(double) * (size_t)(P * half));
        if (!cs || !sn) { free(cs); free(sn); return -1; }
        rope_table(P, d, theta, cs, sn);
    }
    int64_t group = Hq / Hkv;
    int64_t total = B * nr * Hq;
    int fail = 0;

#pragma omp parallel
    {
        double *qt = (double *)malloc(sizeof(double) * (size_t)d);
        double *kt = (double *)malloc(sizeof(double) * (size_t)d);
        /* a key set has at most min(i + 1, w + s) entries; N + s + 1 also holds any list
           that repeats the sinks, so a planted mistake fails a pin instead of a write */
        double *x = (double *)malloc(sizeof(double) * (size_t)(N + s + 1));
        int64_t *key = (int64_t *)malloc(sizeof(int64_t) * (size_t)(N + s + 1));
        if (!qt || !kt || !x || !key) {
#pragma omp atomic write
            fail = 1;
        } else {
#pragma omp for schedule(dynamic, 16)
            for (int64_t idx = 0; idx < total; ++idx) {
                int64_t h = idx % Hq;
                int64_t r = (idx / Hq) % nr;
                int64_t b = idx / (Hq * nr);
                int64_t i = rows ? rows[r] : r;
                int64_t hk = h / group;
                const double *qi = q + ((b * N + i) * Hq + h) * d;
                if (cs) rotate(qi, qt, d, cs + i * half, sn + i * half);
                else memcpy(qt, qi, sizeof(double) * (size_t)d);

                int64_t n = key_set(i, w, s, dil, key);

                for (int64_t e = 0; e < n; ++e) {
                    int64_t j = key[e];
                    const double *kj = k + ((b * N + j) * Hkv + hk) * d;
                    if (cs) rotate(kj, kt, d, cs + j * half, sn + j * half);
                    else memcpy(kt, kj, sizeof(double) * (size_t)d);
                    double bias = slopes ? slopes[h] * (double)(i - j) : 0.0;
                    x[e] = scale * dot(qt, kt, d) + bias;
                }
                weights(x, n, mode);

                double *oi = o + ((b * nr + r) * Hq + h) * d;
                for (int64_t c = 0; c < d; ++c) oi[c] = 0.0;
                for (int64_t e = 0; e < n; ++e) {
                    const double *vj = v + ((b * N + key[e]) * Hkv + hk) * d;
                    for (int64_t c = 0; c < d; ++c) oi[c] += x[e] * vj[c];
                }
            }
        }
        free(qt); free(kt); free(x); free(key);
    }
    free(cs); free(sn);
    return fail ? -1 : 0;
}

int swa_oracle_prefill(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d, int64_t w,
                       int64_t s, int mode, double scale, const double *slopes, double theta,
                       const double *q, const double *k, const double *v,
                       const int64_t *rows, int64_t n_rows, double *o) {
    return prefill_impl(B, Hq, Hkv, N, d, w, s, 1, mode, scale, slopes, theta, q, k, v, rows,
                        n_rows, o);
}

/*
 * Dilated prefill (the dilated-window member of the sparse-attention family the Sliding
 * Window Attention glossary lists beside SWA): the window keeps every dil-th position,
 *   K(i) = { j <= i : ((i - j) mod dil = 0 and (i - j) / dil < w)  or  j < s },
 * so the window spans dil (w - 1) + 1 positions with w keys; the sinks are unchanged.
 * dil = 1 is swa_oracle_prefill. Everything else as there.
 */
int swa_oracle_prefill_dilated(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d,
                               int64_t w, int64_t s, int64_t dil, int mode, double scale,
                               const double *slopes, double theta, const double *q,
                               const double *k, const double *v, const int64_t *rows,
                               int64_t n_rows, double *o) {
    return prefill_impl(B, Hq, Hkv, N, d, w, s, dil, mode, scale, slopes, theta, q, k, v, rows,
                        n_rows, o);
}

/*
 * Append n_new tokens per sequence to the ring, one token at a time in position order, so
 * a later token overwrites an earlier one in the same slot. Token n of sequence q sits at
 * position pos0[q] + n: its key is rotated at that position and written with its value to
 * slot position mod w, and the slot's position is recorded in ring_pos; a token whose
 * position is below s is also written to the sink store at index position. A sequence
 * whose pos0 is negative receives nothing.
 * k_new/v_new [S, n_new, H_kv, d]; rings [S, H_kv, w, d]; ring_pos [S, w];
 * sinks [S, H_kv, s, d] (may be NULL when s == 0).
 */
int swa_oracle_append(int64_t S, int64_t Hkv, int64_t w, int64_t s, int64_t d, double theta,
                      double *k_ring, double *v_ring, int64_t *ring_pos, double *k_sink,
                      double *v_sink, const double *k_new, const double *v_new,
                      const int64_t *pos0, int64_t n_new) {
    if (S < 0 || Hkv <= 0 || w < 1 || s < 0 || d <= 0 || n_new < 0) return -1;
    if (s > 0 && (!k_sink || !v_sink)) return -1;
    double *kt = (double *)malloc(sizeof(double) * (size_t)d);
    if (!kt) return -1;
    for (int64_t q = 0; q < S; ++q) {
        if (pos0[q] < 0) continue;  /* a sequence with a negative start is left untouched */
        for (int64_t n = 0; n < n_new; ++n) {
            int64_t p = pos0[q] + n;
            int64_t slot = p % w;
            ring_pos[q * w + slot] = p;
            for (int64_t hk = 0; hk < Hkv; ++hk) {
                const double *kn = k_new + ((q * n_new + n) * Hkv + hk) * d;
                const double *vn = v_new + ((q * n_new + n) * Hkv + hk) * d;
                if (theta > 0.0) rotate_direct(kn, kt, d, p, theta);
                else memcpy(kt, kn, sizeof(double) * (size_t)d);
                memcpy(k_ring + ((q * Hkv + hk) * w + slot) * d, kt, sizeof(double) * (size_t)d);
                memcpy(v_ring + ((q * Hkv + hk) * w + slot) * d, vn, sizeof(double) * (size_t)d);
                if (p < s) {
                    memcpy(k_sink + ((q * Hkv + hk) * s + p) * d, kt, sizeof(double) * (size_t)d);
                    memcpy(v_sink + ((q * Hkv + hk) * s + p) * d, vn, sizeof(double) * (size_t)d);
                }
            }
        }
    }
    free(kt);
    return 0;
}

/* Positions a ring of w slots holds after positions 0..p_last were appended in order
 * (-1 for a slot never written): a plain simulation of the ring writes. */
void swa_oracle_ring_fill_positions(int64_t p_last, int64_t w, int64_t *pos_out) {
    for (int64_t t = 0; t < w; ++t) pos_out[t] = -1;
    for (int64_t p = 0; p <= p_last; ++p) pos_out[p % w] = p;
}

/*
 * One decode query per sequence at position q_pos[q] (its own token already appended).
 * Key set: ring slots holding a position P with 0 <= q_pos - P < w, plus sink entries
 * j < s that the window no longer covers (j < q_pos - w + 1). q [S, H_q, d] is not yet
 * rotated; ring and sink keys are stored rotated. o [S, H_q, d].
 */
int swa_oracle_decode(int64_t S, int64_t Hq, int64_t Hkv, int64_t d, int64_t w, int64_t s,
                      int mode, double scale, const double *slopes, double theta,
                      const double *q, const int64_t *q_pos, const double *k_ring,
                      const double *v_ring, const int64_t *ring_pos, const double *k_sink,
                      const double *v_sink, double *o) {
    if (S < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || d <= 0 || w < 1 || s < 0) return -1;
    if (s > 0 && (!k_sink || !v_sink)) return -1;
    if (scale <= 0.0) scale = 1.0 / sqrt((double)d);
    int64_t group = Hq / Hkv;
    double *qt = (double *)malloc(sizeof(double) * (size_t)d);
    double *x = (double *)malloc(sizeof(double) * (size_t)(w + s));
    const double **vv = (const double **)malloc(sizeof(double *) * (size_t)(w + s));
    int64_t *slot_of = (int64_t *)malloc(sizeof(int64_t) * (size_t)w);
    if (!qt || !x || !vv || !slot_of) { free(qt); free(x); free(vv); free(slot_of); return -1; }
    for (int64_t sq = 0; sq < S; ++sq) {
        int64_t p = q_pos[sq];
        int64_t lo = p - w + 1 > 0 ? p - w + 1 : 0;
        /* which slot records each position lo..p (-1: none); a position recorded by two
         * slots is not a ring state */
        for (int64_t e = 0; e < w; ++e) slot_of[e] = -1;
        for (int64_t t = 0; t < w; ++t) {
            int64_t P = ring_pos[sq * w + t];
            if (P < lo || P > p) continue;
            if (slot_of[P - lo] >= 0) { free(qt); free(x); free(vv); free(slot_of); return -1; }
            slot_of[P - lo] = t;
        }
        for (int64_t h = 0; h < Hq; ++h) {
            int64_t hk = h / group;
            const double *qh = q + (sq * Hq + h) * d;
            if (theta > 0.0) rotate_direct(qh, qt, d, p, theta);
            else memcpy(qt, qh, sizeof(double) * (size_t)d);
            int64_t n = 0;
            for (int64_t j = 0; j < s && j < lo; ++j) {
                const double *kj = k_sink + ((sq * Hkv + hk) * s + j) * d;
                double bias = slopes ? slopes[h] * (double)(p - j) : 0.0;
                x[n] = scale * dot(qt, kj, d) + bias;
                vv[n] = v_sink + ((sq * Hkv + hk) * s + j) * d;
                ++n;
            }
            /* ring entries in position order lo..p */
            for (int64_t P = lo; P <= p; ++P) {
                int64_t t = slot_of[P - lo];
                if (t < 0) continue;
                const double *kj = k_ring + ((sq * Hkv + hk) * w + t) * d;
                double bias = slopes ? slopes[h] * (double)(p - P) : 0.0;
                x[n] = scale * dot(qt, kj, d) + bias;
                vv[n] = v_ring + ((sq * Hkv + hk) * w + t) * d;
                ++n;
            }
            weights(x, n, mode);
            double *oh = o + (sq * Hq + h) * d;
            for (int64_t c = 0; c < d; ++c) oh[c] = 0.0;
            for (int64_t e = 0; e < n; ++e)
                for (int64_t c = 0; c < d; ++c) oh[c] += x[e] * vv[e][c];
        }
    }
    free(qt); free(x); free(vv); free(slot_of);
    return 0;
}

/*
 * Chunked prefill over the ring (a serving step between whole-sequence prefill and
 * single-token decode; Sliding Window Attention glossary, ring-buffer paragraph: the cache
 * keeps the last w tokens, so a new chunk needs nothing older than that besides the sinks).
 * Sequence q contributes the packed rows cu[q] .. cu[q+1]-1 of q, k_new, v_new and o; row
 * cu[q] + r is the token at position pos0[q] + r. Query i of the chunk attends to the key set
 * K(i) of the prefill definition; key j is read from
 *   - the chunk itself when j >= pos0[q] (row cu[q] + j - pos0[q], rotated at j here),
 *   - else the ring slot j mod w when that slot records position j,
 *   - else the sink store when j < s.
 * A key found in none of them means the cache does not hold the sequence's history: the
 * call fails (-2). The ring is only read here (appending the chunk is a separate step).
 * q [T, H_q, d]; k_new, v_new [T, H_kv, d]; rings and sinks as in swa_oracle_append.
 * rows == NULL: o is [T, H_q, d]; otherwise only the listed packed rows are computed and o
 * is [n_rows, H_q, d] in list order. pos0[q] >= 0 for every sequence.
 * Returns 0, -1 on bad arguments, -2 on missing history.
 */
int swa_oracle_chunk(int64_t S, int64_t Hq, int64_t Hkv, int64_t d, int64_t w, int64_t s,
                     int mode, double scale, const double *slopes, double theta,
                     const double *q, const double *k_new, const double *v_new,
                     const int64_t *cu, const int64_t *pos0, int64_t T, const double *k_ring,
                     const double *v_ring, const int64_t *ring_pos, const double *k_sink,
                     const double *v_sink, const int64_t *rows, int64_t n_rows, double *o) {
    if (S < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || d <= 0 || w < 1 || s < 0 || T < 0)
        return -1;
    if (rows) {
        for (int64_t r = 0; r < n_rows; ++r) if (rows[r] < 0 || rows[r] >= T) return -1;
    }
    if (theta > 0.0 && d % 2 != 0) return -1;
    if (s > 0 && (!k_sink || !v_sink)) return -1;
    for (int64_t sq = 0; sq < S; ++sq)
        if (pos0[sq] < 0 || cu[sq] < 0 || cu[sq] > cu[sq + 1] || cu[sq + 1] > T) return -1;
    if (scale <= 0.0) scale = 1.0 / sqrt((double)d);
    int64_t group = Hq / Hkv;
    int64_t nr = rows ? n_rows : T;
    int64_t total = nr * Hq;
    int status = 0;

#pragma omp parallel
    {
        double *qt = (double *)malloc(sizeof(double) * (size_t)d);
        double *kt = (double *)malloc(sizeof(double) * (size_t)d);
        double *x = (double *)malloc(sizeof(double) * (size_t)(w + s + 1));
        const double **vv = (const double **)malloc(sizeof(double *) * (size_t)(w + s + 1));
        if (!qt || !kt || !x || !vv) {
#pragma omp atomic write
            status = -1;
        } else {
#pragma omp for schedule(dynamic, 16)
            for (int64_t idx = 0; idx < total; ++idx) {
                int64_t h = idx % Hq, r_out = idx / Hq;
                int64_t row = rows ? rows[r_out] : r_out;
                int64_t sq = -1;
                for (int64_t t = 0; t < S; ++t)
                    if (cu[t] <= row && row < cu[t + 1]) { sq = t; break; }
                if (sq < 0) continue;  /* a row no sequence claims is left as it is */
                int64_t p0 = pos0[sq];
                int64_t i = p0 + (row - cu[sq]);
                int64_t hk = h / group;
                const double *qi = q + (row * Hq + h) * d;
                if (theta > 0.0) rotate_direct(qi, qt, d, i, theta);
                else memcpy(qt, qi, sizeof(double) * (size_t)d);

                /* K(i) as two disjoint ranges: sinks [0, min(s, lo)) and window [lo, i]. */
                int64_t lo = i - w + 1 > 0 ? i - w + 1 : 0;
                int64_t n_sink = s < lo ? s : lo;
                int64_t n = 0;
                int missing = 0;
                for (int64_t e = 0; e < n_sink + (i - lo + 1); ++e) {
                    int64_t j = e < n_sink ? e : lo + (e - n_sink);
                    const double *kj;
                    if (j >= p0) {
                        int64_t src = cu[sq] + (j - p0);
                        const double *kn = k_new + (src * Hkv + hk) * d;
                        if (theta > 0.0) rotate_direct(kn, kt, d, j, theta);
                        else memcpy(kt, kn, sizeof(double) * (size_t)d);
                        kj = kt;
                        vv[n] = v_new + (src * Hkv + hk) * d;
                    } else if (ring_pos[sq * w + j % w] == j) {
                        int64_t slot = j % w;
                        kj = k_ring + ((sq * Hkv + hk) * w + slot) * d;
                        vv[n] = v_ring + ((sq * Hkv + hk) * w + slot) * d;
                    } else if (j < s) {
                        kj = k_sink + ((sq * Hkv + hk) * s + j) * d;
                        vv[n] = v_sink + ((sq * Hkv + hk) * s + j) * d;
                    } else {
                        missing = 1;
                        break;
                    }
                    double bias = slopes ? slopes[h] * (double)(i - j) : 0.0;
                    x[n] = scale * dot(qt, kj, d) + bias;
                    ++n;
                }
                if (missing) {
#pragma omp atomic write
                    status = -2;
                    continue;
                }
                weights(x, n, mode);
                double *oi = o + (r_out * Hq + h) * d;
                for (int64_t c = 0; c < d; ++c) oi[c] = 0.0;
                for (int64_t e = 0; e < n; ++e)
                    for (int64_t c = 0; c < d; ++c) oi[c] += x[e] * vv[e][c];
            }
        }
        free(qt); free(kt); free(x); free(vv);
    }
    return status;
}

/*
 * Backward pass of prefill (the gradients SWAT training needs; SWAT page, "Putting It
 * Together": the forward is differentiated as written). Given dout = dL/do, for every
 * (b, h, i) and j in K(i), with x_ij, p_ij as in the forward and q~ = R(i) q, k~ = R(j) k:
 *   dP_ij = dout_i . v_j
 *   dX_ij = dP_ij * p_ij * (1 - p_ij)                 sigmoid (the logistic derivative)
 *         = p_ij * (dP_ij - sum_{j'} p_ij' dP_ij')     softmax (the row Jacobian)
 *   dv_j += p_ij dout_i,  dq~_i += scale dX_ij k~_j,  dk~_j += scale dX_ij q~_i
 * and dq_i = R(i)^T dq~_i, dk_j = R(j)^T dk~_j (the rotation is orthogonal; its transpose
 * rotates by the opposite angle). Key and value gradients sum over the query heads of their
 * group. The slopes are fixed (no gradient). Layouts as in swa_oracle_prefill; dq like q,
 * dk/dv like k. Returns 0, or -1 on bad arguments / allocation failure.
 */
static int backward_impl(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d, int64_t w,
                         int64_t s, int64_t dil, int mode, double scale, const double *slopes,
                         double theta, const double *q, const double *k, const double *v,
                         const double *dout, double *dq, double *dk, double *dv) {
    if (B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || N < 0 || d <= 0 || w < 1 || s < 0 ||
        dil < 1)
        return -1;
    if (theta > 0.0 && d % 2 != 0) return -1;
    if (scale <= 0.0) scale = 1.0 / sqrt((double)d);
    int64_t half = d / 2, group = Hq / Hkv;
    double *cs = NULL, *sn = NULL;
    if (theta > 0.0 && N > 0) {
        cs = (double *)malloc(sizeof(double) * (size_t)(N * half));
        sn = (double *)malloc(sizeof(double) * (size_t)(N * half));
        if (!cs || !sn) { free(cs); free(sn); return -1; }
        rope_table(N, d, theta, cs, sn);
    }
    memset(dq, 0, sizeof(double) * (size_t)(B * N * Hq * d));
    memset(dk, 0, sizeof(double) * (size_t)(B * N * Hkv * d));
    memset(dv, 0, sizeof(double) * (size_t)(B * N * Hkv * d));
    int fail = 0;

    /* one (batch, kv head) slice per task: its key and value gradients have one writer */
#pragma omp parallel
    {
        double *qt = (double *)malloc(sizeof(double) * (size_t)d);
        double *x = (double *)malloc(sizeof(double) * (size_t)(N + s + 1));
        double *dp = (double *)malloc(sizeof(double) * (size_t)(N + s + 1));
        int64_t *key = (int64_t *)malloc(sizeof(int64_t) * (size_t)(N + s + 1));
        double *kr = (double *)malloc(sizeof(double) * (size_t)((N > 0 ? N : 1) * d));
        double *dkr = (double *)malloc(sizeof(double) * (size_t)((N > 0 ? N : 1) * d));
        double *dqr = (double *)malloc(sizeof(double) * (size_t)d);
        if (!qt || !x || !dp || !key || !kr || !dkr || !dqr) {
#pragma omp atomic write
            fail = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t bh = 0; bh < B * Hkv; ++bh) {
                int64_t b = bh / Hkv, hk = bh % Hkv;
                /* rotated keys of this slice, and their gradients in the rotated frame */
                for (int64_t j = 0; j < N; ++j) {
                    const double *kj = k + ((b * N + j) * Hkv + hk) * d;
                    if (cs) rotate(kj, kr + j * d, d, cs + j * half, sn + j * half);
                    else memcpy(kr + j * d, kj, sizeof(double) * (size_t)d);
                }
                memset(dkr, 0, sizeof(double) * (size_t)(N * d));
                for (int64_t h = hk * group; h < (hk + 1) * group; ++h) {
                    for (int64_t i = 0; i < N; ++i) {
                        const double *qi = q + ((b * N + i) * Hq + h) * d;
                        const double *gi = dout + ((b * N + i) * Hq + h) * d;
                        if (cs) rotate(qi, qt, d, cs + i * half, sn + i * half);
                        else memcpy(qt, qi, sizeof(double) * (size_t)d);
                        int64_t n = key_set(i, w, s, dil, key);
                        for (int64_t e = 0; e < n; ++e) {
                            int64_t j = key[e];
                            double bias = slopes ? slopes[h] * (double)(i - j) : 0.0;
                            x[e] = scale * dot(qt, kr + j * d, d) + bias;
                            dp[e] = dot(gi, v + ((b * N + j) * Hkv + hk) * d, d);
                        }
                        weights(x, n, mode);   /* x now holds p */
                        double rowsum = 0.0;
                        if (mode == ORACLE_SOFTMAX)
                            for (int64_t e = 0; e < n; ++e) rowsum += x[e] * dp[e];
                        for (int64_t c = 0; c < d; ++c) dqr[c] = 0.0;
                        for (int64_t e = 0; e < n; ++e) {
                            int64_t j = key[e];
                            double p = x[e];
                            double dx = mode == ORACLE_SIGMOID ? dp[e] * p * (1.0 - p)
                                                               : p * (dp[e] - rowsum);
                            double *dvj = dv + ((b * N + j) * Hkv + hk) * d;
                            for (int64_t c = 0; c < d; ++c) {
                                dvj[c] += p * gi[c];
                                dqr[c] += scale * dx * kr[j * d + c];
                                dkr[j * d + c] += scale * dx * qt[c];
                            }
                        }
                        double *dqi = dq + ((b * N + i) * Hq + h) * d;
                        if (cs) {
                            /* R^T: rotation by the opposite angle */
                            for (int64_t t = 0; t < half; ++t) {
                                double a = dqr[2 * t], bb = dqr[2 * t + 1];
                                double c = cs[i * half + t], sv = sn[i * half + t];
                                dqi[2 * t] = a * c + bb * sv;
                                dqi[2 * t + 1] = -a * sv + bb * c;
                            }
                        } else {
                            memcpy(dqi, dqr, sizeof(double) * (size_t)d);
                        }
                    }
                }
                for (int64_t j = 0; j < N; ++j) {
                    double *dkj = dk + ((b * N + j) * Hkv + hk) * d;
                    const double *g = dkr + j * d;
                    if (cs) {
                        for (int64_t t = 0; t < half; ++t) {
                            double a = g[2 * t], bb = g[2 * t + 1];
                            double c = cs[j * half + t], sv = sn[j * half + t];
                            dkj[2 * t] = a * c + bb * sv;
                            dkj[2 * t + 1] = -a * sv + bb * c;
                        }
                    } else {
                        memcpy(dkj, g, sizeof(double) * (size_t)d);
                    }
                }
            }
        }
        free(qt); free(x); free(dp); free(key); free(kr); free(dkr); free(dqr);
    }
    free(cs); free(sn);
    return fail ? -1 : 0;
}

int swa_oracle_backward(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d, int64_t w,
                        int64_t s, int mode, double scale, const double *slopes, double theta,
                        const double *q, const double *k, const double *v, const double *dout,
                        double *dq, double *dk, double *dv) {
    return backward_impl(B, Hq, Hkv, N, d, w, s, 1, mode, scale, slopes, theta, q, k, v, dout,
                         dq, dk, dv);
}

/* Backward of the dilated prefill: the same gradients over the dilated K(i) of
 * swa_oracle_prefill_dilated. dil = 1 is swa_oracle_backward. */
int swa_oracle_backward_dilated(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d,
                                int64_t w, int64_t s, int64_t dil, int mode, double scale,
                                const double *slopes, double theta, const double *q,
                                const double *k, const double *v, const double *dout,
                                double *dq, double *dk, double *dv) {
    return backward_impl(B, Hq, Hkv, N, d, w, s, dil, mode, scale, slopes, theta, q, k, v, dout,
                         dq, dk, dv);
}
