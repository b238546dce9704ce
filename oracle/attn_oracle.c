/*
 * attn_oracle.c -- plain, slow, fp64 CPU oracle for multi-head scaled-dot-product
 * attention (prefill and single-token decode).
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the reference that the GPU library is
 * checked against.  Only the test suite, the smoke check and the CPU-baseline leg
 * of the benchmark load it.  It shares no code, header, table or helper with the
 * GPU library, and the GPU library never calls it.
 *
 * What it computes (the exact definition, written out, three passes per row):
 *
 *   For batch item b, query head h, query row i:
 *     kv head       kh  = h / (q_heads / kv_heads)     (grouped KV heads: contiguous
 *                                                       groups of query heads share one
 *                                                       K/V head; ferrum-kernels `Backend`
 *                                                       page, `split_qkv` and
 *                                                       `split_qkv_norm_rope` shapes)
 *     query pos     p   = pos_offset + i               (ferrum-kernels `Backend` page,
 *                                                       `qk_norm_rope`: token 0 sits at
 *                                                       pos_offset, token i at pos_offset+i)
 *     valid keys    L   = clamp(seq_lens[b], 0, kv_len) or kv_len without seq_lens
 *     row is padding when p >= L: output 0            (ripvec-core `Driver` page,
 *                                                       `unpad_from_batch`: padded rows
 *                                                       are discarded)
 *     key set J = { j < L : (!causal || j <= p) && in_band(p, j) }
 *       in_band: window == 0             -> every key
 *                causal, window w        -> p - j < w  (the last w positions, ferrum-kernels
 *                                           `Backend` page, `flash_attention_batched_per_cache`,
 *                                           sliding_window)
 *                bidirectional, window w -> |p - j| <= floor(w / 2) (ripvec-core `Driver`
 *                                           page, `fused_scale_mask_softmax_windowed`)
 *     J empty: output 0 (realizar `cached/attention.rs`, `batched_causal_softmax`:
 *              a row is only normalised when its exponential sum is positive)
 *     pass 1  s_j  = scale * sum_d q[d] * k[j][d]          for j in J
 *     pass 2  pi_j = exp(s_j - max s) / sum_J exp(s - max s)
 *     pass 3  out[d] = sum_J pi_j * v[j][d]
 *   (ripvec-core `Driver` page, `fused_scale_mask_softmax`: softmax(scores*scale + mask)
 *   per head; realizar `cached/attention.rs`, `parallel_multihead_attention_gpu_cached`:
 *   per-head Q.K^T, times 1/sqrt(head_dim), masked softmax, times V.)
 *
 *   Masked keys are excluded (weight exactly 0).  This equals the pages' additive
 *   -10000 / -inf masks on every row that has at least one valid key.
 *
 *   Decode is the q_len = 1 causal case over a head-major cache
 *   [batch, kv_heads, capacity, head_dim] of which the first kv_len slots are filled
 *   (ferrum-kernels `Backend` page, `kv_cache_append_head_major` and
 *   `flash_attention_batched_per_cache`).  With per-item kv_lens the query sits at
 *   position kv_lens[b] - 1 and sees L = min(kv_lens[b], kv_len) keys; without them
 *   the query sits at pos_offset and sees keys j < kv_len, j <= pos_offset.
 *
 * Inputs are read exactly: fp32 values as stored, bf16 values widened bit-exactly
 * (a bf16 is the upper 16 bits of an fp32), fp16 values decoded from their fields.  All arithmetic is in double; the output
 * is double and is never rounded.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#define ORACLE_F32 0
#define ORACLE_BF16 1
#define ORACLE_F16 2

/* IEEE 754 binary16 bits -> double, from the format's definition: sign bit 15, biased
 * exponent bits 14..10 (bias 15), fraction bits 9..0; exponent 0 is subnormal
 * (fraction * 2^-24), exponent 31 is infinity (fraction 0) or NaN. */
static double half_to_double(uint16_t h) {
    const int sign = (h >> 15) & 1;
    const int expo = (h >> 10) & 0x1f;
    const int frac = h & 0x3ff;
    double mag;
    if (expo == 0)
        mag = ldexp((double)frac, -24);
    else if (expo == 31)
        mag = frac == 0 ? INFINITY : NAN;
    else
        mag = ldexp(1024.0 + frac, expo - 25);
    return sign ? -mag : mag;
}

/* Read element `idx` of a tensor stored as fp32, bf16 or fp16, widened to double. */
static double load_elem(const void* base, int dtype, int64_t idx) {
    if (dtype == ORACLE_F32) {
        return (double)((const float*)base)[idx];
    }
    if (dtype == ORACLE_F16) return half_to_double(((const uint16_t*)base)[idx]);
    uint32_t bits = (uint32_t)((const uint16_t*)base)[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* The shape of one problem; every pointer is a host pointer. */
typedef struct {
    const void* q;   /* [batch, q_heads, q_len, head_dim]                      */
    const void* k;   /* [batch, kv_heads, kv_stride, head_dim]                  */
    const void* v;   /* [batch, kv_heads, kv_stride, head_dim]                  */
    int dtype;
    int batch, q_heads, kv_heads, q_len, kv_len, kv_stride, head_dim;
    int pos_offset;
    const int32_t* seq_lens; /* [batch] valid key count per item, or NULL     */
    int window, causal;
    double scale;
    int decode;              /* 1: seq_lens are decode kv_lens (query at len-1) */
} problem_t;

/* Query position and valid key count of row i of batch item b. */
static void row_geometry(const problem_t* P, int b, int i, int64_t* pos, int64_t* nvalid) {
    if (P->decode) {
        if (P->seq_lens) {
            int64_t len = P->seq_lens[b];
            if (len < 0) len = 0;
            if (len > P->kv_len) len = P->kv_len;
            *nvalid = len;
            *pos = len - 1;
        } else {
            *nvalid = P->kv_len;
            *pos = P->pos_offset;
        }
        return;
    }
    int64_t len = P->kv_len;
    if (P->seq_lens) {
        len = P->seq_lens[b];
        if (len < 0) len = 0;
        if (len > P->kv_len) len = P->kv_len;
    }
    *nvalid = len;
    *pos = (int64_t)P->pos_offset + i;
}

/* Is key j in the key set of a query at position p with nvalid valid keys? */
static int key_allowed(const problem_t* P, int64_t p, int64_t nvalid, int64_t j) {
    if (j < 0 || j >= nvalid) return 0;
    if (p >= nvalid) return 0; /* padded query row */
    int causal = P->decode ? 1 : P->causal;
    if (causal && j > p) return 0;
    if (P->window > 0) {
        if (causal) {
            if (p - j >= P->window) return 0;
        } else {
            int64_t half = P->window / 2;
            int64_t d = p - j;
            if (d < 0) d = -d;
            if (d > half) return 0;
        }
    }
    return 1;
}

/*
 * One output row, three passes.  `probs` (length kv_len, may be NULL) receives the
 * softmax weights pi_j (0 for keys outside J).  `scores` is caller scratch of length
 * kv_len.  Returns the size of the key set.
 */
static int64_t attend_row(const problem_t* P, int b, int h, int i, double* out,
                          double* probs, double* scores) {
    const int D = P->head_dim;
    const int group = P->q_heads / P->kv_heads;
    const int kh = h / group;
    int64_t pos, nvalid;
    row_geometry(P, b, i, &pos, &nvalid);

    const int64_t q_row = (((int64_t)b * P->q_heads + h) * P->q_len + i) * D;
    const int64_t kv_head_base = ((int64_t)b * P->kv_heads + kh) * P->kv_stride;

    for (int d = 0; d < D; ++d) out[d] = 0.0;
    if (probs) for (int64_t j = 0; j < P->kv_len; ++j) probs[j] = 0.0;

    /* pass 1: scaled scores of the keys in J */
    int64_t count = 0;
    double m = -INFINITY;
    for (int64_t j = 0; j < P->kv_len; ++j) {
        if (!key_allowed(P, pos, nvalid, j)) continue;
        double dot = 0.0;
        const int64_t k_row = (kv_head_base + j) * D;
        for (int d = 0; d < D; ++d)
            dot += load_elem(P->q, P->dtype, q_row + d) * load_elem(P->k, P->dtype, k_row + d);
        scores[j] = P->scale * dot;
        if (scores[j] > m) m = scores[j];
        ++count;
    }
    if (count == 0) return 0;

    /* pass 2: softmax over J */
    double z = 0.0;
    for (int64_t j = 0; j < P->kv_len; ++j) {
        if (!key_allowed(P, pos, nvalid, j)) continue;
        scores[j] = exp(scores[j] - m);
        z += scores[j];
    }

    /* pass 3: probability-weighted sum of V rows */
    for (int64_t j = 0; j < P->kv_len; ++j) {
        if (!key_allowed(P, pos, nvalid, j)) continue;
        const double pj = scores[j] / z;
        if (probs) probs[j] = pj;
        const int64_t v_row = (kv_head_base + j) * D;
        for (int d = 0; d < D; ++d) out[d] += pj * load_elem(P->v, P->dtype, v_row + d);
    }
    return count;
}

/* ---- work distribution over host threads: rows are independent ---- */

typedef struct {
    const problem_t* P;
    const int32_t* rows; /* NULL: all rows in order; else n_rows (b, h, i) triples */
    int64_t n_rows;
    double* out;         /* [n_rows, head_dim] */
    int64_t next;        /* shared cursor, guarded by mu */
    pthread_mutex_t mu;
} job_t;

static void row_triple(const job_t* J, int64_t r, int* b, int* h, int* i) {
    if (J->rows) {
        *b = J->rows[3 * r];
        *h = J->rows[3 * r + 1];
        *i = J->rows[3 * r + 2];
    } else {
        const int64_t per_b = (int64_t)J->P->q_heads * J->P->q_len;
        *b = (int)(r / per_b);
        *h = (int)((r % per_b) / J->P->q_len);
        *i = (int)(r % J->P->q_len);
    }
}

static void* worker(void* arg) {
    job_t* J = (job_t*)arg;
    double* scores = (double*)malloc(sizeof(double) * (size_t)(J->P->kv_len > 0 ? J->P->kv_len : 1));
    if (!scores) return (void*)1;
    const int64_t chunk = 16;
    for (;;) {
        pthread_mutex_lock(&J->mu);
        int64_t start = J->next;
        J->next += chunk;
        pthread_mutex_unlock(&J->mu);
        if (start >= J->n_rows) break;
        int64_t end = start + chunk < J->n_rows ? start + chunk : J->n_rows;
        for (int64_t r = start; r < end; ++r) {
            int b, h, i;
            row_triple(J, r, &b, &h, &i);
            attend_row(J->P, b, h, i, J->out + r * J->P->head_dim, NULL, scores);
        }
    }
    free(scores);
    return NULL;
}

static int run_rows(const problem_t* P, const int32_t* rows, int64_t n_rows, double* out,
                    int nthreads) {
    if (nthreads <= 0) nthreads = (int)sysconf(_SC_NPROCESSORS_ONLN);
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    job_t J;
    J.P = P;
    J.rows = rows;
    J.n_rows = n_rows;
    J.out = out;
    J.next = 0;
    pthread_mutex_init(&J.mu, NULL);
    pthread_t tid[256];
    int started = 0, failed = 0;
    for (int t = 0; t < nthreads; ++t) {
        if (pthread_create(&tid[t], NULL, worker, &J) != 0) break;
        ++started;
    }
    if (started == 0) failed |= worker(&J) != NULL;
    for (int t = 0; t < started; ++t) {
        void* ret = NULL;
        pthread_join(tid[t], &ret);
        failed |= ret != NULL;
    }
    pthread_mutex_destroy(&J.mu);
    return failed ? -2 : nthreads;
}

static int check_shape(const problem_t* P) {
    if (P->batch < 0 || P->q_heads < 1 || P->kv_heads < 1 || P->q_len < 0 || P->kv_len < 0 ||
        P->head_dim < 1 || P->window < 0)
        return -1;
    if (P->q_heads % P->kv_heads != 0) return -1;
    if (P->dtype != ORACLE_F32 && P->dtype != ORACLE_BF16 && P->dtype != ORACLE_F16) return -1;
    if (P->kv_stride < P->kv_len) return -1;
    return 0;
}

/* ---- exported entry points (return the thread count used, or < 0 on error) ---- */

/* Full prefill: out [batch, q_heads, q_len, head_dim] in double. */
int oracle_prefill(const void* q, const void* k, const void* v, double* out, int dtype, int batch,
                   int q_heads, int kv_heads, int q_len, int kv_len, int head_dim, int pos_offset,
                   const int32_t* seq_lens, int window, int causal, double scale, int nthreads) {
    problem_t P = {q, k, v, dtype, batch, q_heads, kv_heads, q_len, kv_len, kv_len, head_dim,
                   pos_offset, seq_lens, window, causal, scale, 0};
    if (check_shape(&P)) return -1;
    return run_rows(&P, NULL, (int64_t)batch * q_heads * q_len, out, nthreads);
}

/* Selected prefill rows: rows = n_rows (b, h, i) triples; out [n_rows, head_dim]. */
int oracle_prefill_rows(const void* q, const void* k, const void* v, double* out, int dtype,
                        int batch, int q_heads, int kv_heads, int q_len, int kv_len, int head_dim,
                        int pos_offset, const int32_t* seq_lens, int window, int causal,
                        double scale, const int32_t* rows, int64_t n_rows, int nthreads) {
    problem_t P = {q, k, v, dtype, batch, q_heads, kv_heads, q_len, kv_len, kv_len, head_dim,
                   pos_offset, seq_lens, window, causal, scale, 0};
    if (check_shape(&P)) return -1;
    for (int64_t r = 0; r < n_rows; ++r)
        if (rows[3 * r] < 0 || rows[3 * r] >= batch || rows[3 * r + 1] < 0 ||
            rows[3 * r + 1] >= q_heads || rows[3 * r + 2] < 0 || rows[3 * r + 2] >= q_len)
            return -1;
    return run_rows(&P, rows, n_rows, out, nthreads);
}

/* Decode: q [batch, q_heads, head_dim]; caches [batch, kv_heads, capacity, head_dim];
 * out [batch, q_heads, head_dim] in double.  rows/n_rows as above with i = 0 (rows may
 * be NULL for every (b, h)). */
int oracle_decode(const void* q, const void* k_cache, const void* v_cache, double* out, int dtype,
                  int batch, int q_heads, int kv_heads, int kv_len, int capacity, int head_dim,
                  int pos_offset, const int32_t* kv_lens, int window, double scale,
                  const int32_t* rows, int64_t n_rows, int nthreads) {
    problem_t P = {q, k_cache, v_cache, dtype, batch, q_heads, kv_heads, 1, kv_len, capacity,
                   head_dim, pos_offset, kv_lens, window, 1, scale, 1};
    if (check_shape(&P)) return -1;
    if (!rows) n_rows = (int64_t)batch * q_heads;
    else
        for (int64_t r = 0; r < n_rows; ++r)
            if (rows[3 * r] < 0 || rows[3 * r] >= batch || rows[3 * r + 1] < 0 ||
                rows[3 * r + 1] >= q_heads || rows[3 * r + 2] != 0)
                return -1;
    return run_rows(&P, rows, n_rows, out, nthreads);
}

/* Softmax weights of one prefill row: probs [kv_len] (0 outside the key set) and the
 * row's output [head_dim].  Returns the key-set size.  Inspection entry for tests. */
int64_t oracle_prefill_probs(const void* q, const void* k, const void* v, double* probs,
                             double* out_row, int dtype, int batch, int q_heads, int kv_heads,
                             int q_len, int kv_len, int head_dim, int pos_offset,
                             const int32_t* seq_lens, int window, int causal, double scale, int b,
                             int h, int i) {
    problem_t P = {q, k, v, dtype, batch, q_heads, kv_heads, q_len, kv_len, kv_len, head_dim,
                   pos_offset, seq_lens, window, causal, scale, 0};
    if (check_shape(&P)) return -1;
    if (b < 0 || b >= batch || h < 0 || h >= q_heads || i < 0 || i >= q_len) return -1;
    double* scores = (double*)malloc(sizeof(double) * (size_t)(kv_len > 0 ? kv_len : 1));
    if (!scores) return -2;
    int64_t n = attend_row(&P, b, h, i, out_row, probs, scores);
    free(scores);
    return n;
}
