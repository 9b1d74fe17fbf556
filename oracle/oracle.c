/*
 * oracle.c -- the slow, plain CPU oracle for the prefill attention core.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no source,
 * header, table or constant with the HIP library, and the HIP library never
 * calls it.
 *
 * Everything is computed in double precision, straight from the definitions,
 * with no tiling, no online softmax and no fusion.  Work is split over
 * independent (token, head) or (query row, head) units with pthreads; every
 * unit is computed sequentially by one thread, so results do not depend on the
 * thread count.
 *
 * Sources (the pages' own words are paraphrased, never quoted):
 *  - memra-engine 0.130.0 src/forward.rs, `Model::forward`, QK-norm block: the
 *    Q and K projections are normalised per (token, head) over head_dim rows of
 *    the token-major buffer, each row then multiplied by the learned
 *    q_norm / k_norm vector of length head_dim.
 *  - same page, RoPE block: NeoX rotation of Q and K at positions 0..T-1 with
 *    head_dim, the rotated-dimension count and the frequency base as arguments.
 *  - needle-core v3/model.rs, `rope_at` / `rope`: half = rotated dims / 2,
 *    frequency of pair i is base^(-2i / rotated dims), angle = position x
 *    frequency, and the cos/sin of that angle rotate the pair.
 *  - memra-engine 0.130.0 src/forward.rs, SDPA block: causal grouped-query
 *    attention with n_head query heads over n_head_kv K/V heads, T_q = T_kv = T,
 *    scale = 1/sqrt(head_dim).
 *  - memra-engine 0.101.0 src/spec.rs, `full_attn_verify`, per-row fallback:
 *    row r of a block attends base_len + r + 1 keys, i.e. itself and every
 *    earlier key (the diagonal is visible).
 *  - same function: a block of t new rows over a cache that already holds
 *    base_len rows is normalised and rotated at the positions of the new rows,
 *    its K and V are appended to the cache, and row r then attends cache rows
 *    0 .. base_len + r (the chunk entry points below; base_len = 0 is plain
 *    prefill).
 *  - needle-core v3/model.rs, cache fill after the prefill: what a cache keeps
 *    are the normalised, rotated keys and the values.
 *  - memra-engine 0.101.0 src/spec.rs, sliding-window layers of the step35 MTP
 *    path: once a sequence holds more than `window` keys, a new token attends
 *    only the last `window` of them, itself included (needle-core v3/model.rs
 *    passes a per-layer attention span to its attention for the same purpose):
 *    row i sees key j when i - window < j <= i.
 *  - needle-core v3/model.rs, gated attention output: every element of the
 *    attention output is multiplied by the logistic sigmoid of the matching
 *    element of a gate tensor before the output projection; memra-engine
 *    0.101.0 src/spec.rs does the same with the gate split off the Q
 *    projection, and its step35 layers with one gate value per head.
 *  - needle-core v3/model.rs, 8-bit activation quantisation of a session
 *    (`quant_rows`, `quantize_rows` and the 8-bit K/V store): after RoPE the
 *    query, key and value rows are quantised per (token, head) with 8 bits,
 *    the store keeps integer rows with one scale per row, and its reader takes
 *    the scale outside the dot product (which is algebraically the dot product
 *    of the dequantised rows); quantising twice changes nothing.
 *
 * Readings taken where the pages are silent (each one is listed with its
 * reason in the design notes of the repository):
 *  - RMSNorm puts eps inside the root: y = x / sqrt(mean(x^2) + eps) * w.
 *  - Rotate-half pairing (j, j + n/2); the exponent uses n = rope_dim; the
 *    dimensions from rope_dim to head_dim - 1 pass through unchanged.
 *  - Query head h reads K/V head floor(h / (n_head / n_head_kv)).
 *  - Packed sequences never attend across their boundaries and their positions
 *    restart at 0.
 *  - 8-bit quantisation is symmetric with the row's largest magnitude on the
 *    top code: scale = max|x| / 127, code = x / scale rounded to the nearest
 *    integer, ties to even, within -127..127; a row of zeros gets scale 0 and
 *    codes 0.  These are integer decisions, so they are taken in single
 *    precision, the precision of the values being quantised.  The pages print
 *    neither the tie direction nor the divisor: for those two details the
 *    8-bit rule is parity unpinned against the pages (its pins hold it to the
 *    rule as stated here).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#define ORACLE_OK 0
#define ORACLE_BAD_ARG -1
#define ORACLE_NO_MEM -2

/* ------------------------------------------------------------------------ */
/* sequences                                                                  */

/* Index of the packed sequence that holds token t: the s with
 * offsets[s] <= t < offsets[s+1].  offsets has n_seqs + 1 entries. */
static int seq_of_token(const int32_t* offsets, int n_seqs, int64_t t) {
    for (int s = 0; s < n_seqs; ++s)
        if (t >= offsets[s] && t < offsets[s + 1]) return s;
    return -1;
}

static int check_offsets(const int32_t* offsets, int n_seqs, int64_t T) {
    if (n_seqs < 1 || offsets[0] != 0 || offsets[n_seqs] != T) return 0;
    for (int s = 0; s < n_seqs; ++s)
        if (offsets[s + 1] < offsets[s]) return 0;
    return 1;
}

/* ------------------------------------------------------------------------ */
/* a tiny work pool: units 0..n_units-1 handed out one at a time             */

typedef void (*unit_fn)(void* ctx, int64_t unit, double* scratch);

typedef struct {
    unit_fn fn;
    void* ctx;
    int64_t n_units;
    int64_t next;
    size_t scratch_len;
    pthread_mutex_t lock;
    int failed;
} pool_t;

static void* pool_worker(void* arg) {
    pool_t* p = (pool_t*)arg;
    double* scratch = NULL;
    if (p->scratch_len) {
        scratch = (double*)malloc(p->scratch_len * sizeof(double));
        if (!scratch) {
            pthread_mutex_lock(&p->lock);
            p->failed = 1;
            pthread_mutex_unlock(&p->lock);
            return NULL;
        }
    }
    for (;;) {
        pthread_mutex_lock(&p->lock);
        int64_t u = p->next++;
        pthread_mutex_unlock(&p->lock);
        if (u >= p->n_units) break;
        p->fn(p->ctx, u, scratch);
    }
    free(scratch);
    return NULL;
}

static int run_pool(unit_fn fn, void* ctx, int64_t n_units, size_t scratch_len, int n_threads) {
    if (n_threads <= 0) {
        long nc = sysconf(_SC_NPROCESSORS_ONLN);
        n_threads = nc > 0 ? (int)nc : 1;
    }
    if (n_threads > 256) n_threads = 256;
    if ((int64_t)n_threads > n_units) n_threads = n_units > 0 ? (int)n_units : 1;
    pool_t p;
    p.fn = fn;
    p.ctx = ctx;
    p.n_units = n_units;
    p.next = 0;
    p.scratch_len = scratch_len;
    p.failed = 0;
    pthread_mutex_init(&p.lock, NULL);
    pthread_t th[256];
    int started = 0;
    for (int i = 0; i < n_threads; ++i) {
        if (pthread_create(&th[i], NULL, pool_worker, &p) != 0) break;
        ++started;
    }
    if (started == 0) pool_worker(&p); /* no threads available: run inline */
    for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
    pthread_mutex_destroy(&p.lock);
    return p.failed ? ORACLE_NO_MEM : ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* O1 -- per-(token, head) RMSNorm over head_dim with a learned scale         */

/* y[c] = x[c] * w[c] / sqrt((1/d) * sum_c x[c]^2 + eps), c = 0..d-1. */
static void rms_norm_row(const double* x, const double* w, int d, double eps, double* y) {
    double ss = 0.0;
    for (int c = 0; c < d; ++c) ss += x[c] * x[c];
    double ms = ss / (double)d;
    double r = 1.0 / sqrt(ms + eps);
    for (int c = 0; c < d; ++c) y[c] = x[c] * r * w[c];
}

/* ------------------------------------------------------------------------ */
/* O2 -- NeoX (rotate-half) rotary embedding of one head row, in place        */

/* For j < n/2: theta = pos * base^(-2j/n); the pair (y[j], y[j + n/2]) turns
 * by theta.  Dimensions n..d-1 are left alone. */
static void rope_neox_row(double* y, int d, int n, double base, int64_t pos) {
    int half = n / 2;
    for (int j = 0; j < half; ++j) {
        double freq = pow(base, -2.0 * (double)j / (double)n);
        double theta = (double)pos * freq;
        double c = cos(theta), s = sin(theta);
        double a = y[j], b = y[j + half];
        y[j] = a * c - b * s;
        y[j + half] = a * s + b * c;
    }
    (void)d;
}

typedef struct {
    const float* x;     /* [T, heads*d] */
    const float* w;     /* [d] */
    double* out;        /* [T, heads*d] */
    const int32_t* offsets;
    const int64_t* pos0; /* position of each sequence's first row; NULL: all 0 */
    int n_seqs, heads, d, n;
    double base, eps;
} qknorm_ctx;

static void qknorm_unit(void* vctx, int64_t unit, double* scratch) {
    qknorm_ctx* c = (qknorm_ctx*)vctx;
    int64_t t = unit / c->heads;
    int h = (int)(unit % c->heads);
    int s = seq_of_token(c->offsets, c->n_seqs, t);
    int64_t pos = t - c->offsets[s];
    if (c->pos0) pos += c->pos0[s];
    double* x = scratch;         /* d */
    double* w = scratch + c->d;  /* d */
    const float* src = c->x + (t * c->heads + h) * (int64_t)c->d;
    for (int i = 0; i < c->d; ++i) {
        x[i] = (double)src[i];
        w[i] = (double)c->w[i];
    }
    double* y = c->out + (t * c->heads + h) * (int64_t)c->d;
    rms_norm_row(x, w, c->d, c->eps, y);
    rope_neox_row(y, c->d, c->n, c->base, pos);
}

/* O1 then O2 on every head row of Q (n_head heads, scale wq) and K (n_head_kv
 * heads, scale wk).  Inputs are f32 as the GPU receives them; outputs are f64.
 * seq_offsets may be NULL (one sequence [0, T)).  Row r of sequence s sits at
 * position pos0[s] + r (pos0 NULL: r). */
int oracle_qknorm_rope_from(const float* q, const float* k, const float* wq, const float* wk,
                            const int32_t* seq_offsets, int n_seqs, const int64_t* pos0,
                            int64_t T, int n_head, int n_head_kv, int head_dim, int rope_dim,
                            double base, double eps, double* q_out, double* k_out,
                            int n_threads) {
    int32_t one[2];
    if (T < 0 || n_head <= 0 || n_head_kv <= 0 || head_dim <= 0 || rope_dim < 0 ||
        rope_dim > head_dim || (rope_dim & 1) || !(base > 0.0) || eps < 0.0)
        return ORACLE_BAD_ARG;
    if (T == 0) return ORACLE_OK;
    if (!seq_offsets) {
        one[0] = 0;
        one[1] = (int32_t)T;
        seq_offsets = one;
        n_seqs = 1;
    }
    if (!check_offsets(seq_offsets, n_seqs, T)) return ORACLE_BAD_ARG;
    for (int s = 0; pos0 && s < n_seqs; ++s)
        if (pos0[s] < 0) return ORACLE_BAD_ARG;
    qknorm_ctx c = {q, wq, q_out, seq_offsets, pos0, n_seqs, n_head, head_dim, rope_dim, base,
                    eps};
    int rc = run_pool(qknorm_unit, &c, T * n_head, 2 * (size_t)head_dim, n_threads);
    if (rc) return rc;
    qknorm_ctx ck = {k, wk, k_out, seq_offsets, pos0, n_seqs, n_head_kv, head_dim, rope_dim,
                     base, eps};
    return run_pool(qknorm_unit, &ck, T * n_head_kv, 2 * (size_t)head_dim, n_threads);
}

/* As oracle_qknorm_rope_from with every sequence starting at position 0. */
int oracle_qknorm_rope(const float* q, const float* k, const float* wq, const float* wk,
                       const int32_t* seq_offsets, int n_seqs, int64_t T, int n_head,
                       int n_head_kv, int head_dim, int rope_dim, double base, double eps,
                       double* q_out, double* k_out, int n_threads) {
    return oracle_qknorm_rope_from(q, k, wq, wk, seq_offsets, n_seqs, NULL, T, n_head,
                                   n_head_kv, head_dim, rope_dim, base, eps, q_out, k_out,
                                   n_threads);
}

/* ------------------------------------------------------------------------ */
/* O3 -- causal grouped-query attention, one (query row, head) per unit       */

typedef struct {
    const double *q, *k, *v; /* [T_q, H*d], [T_kv, Hkv*d], [T_kv, Hkv*d] */
    double* out;             /* [n_rows, H*d] */
    const int64_t* rows;     /* NULL: row r of out is query row r */
    const int32_t* offsets;    /* query rows of each sequence */
    const int32_t* kv_offsets; /* key rows of each sequence (the same for plain prefill) */
    int n_seqs, H, Hkv, d, causal;
    int64_t window;            /* causal only: keys visible per row, the row's own included; 0: all */
    const double* gate;        /* NULL, or [T_q, H*d] (per element) / [T_q, H] (per head) */
    int gate_per_head;
    double scale;
} attn_ctx;

static void attn_unit(void* vctx, int64_t unit, double* e) {
    attn_ctx* c = (attn_ctx*)vctx;
    int64_t r = unit / c->H;
    int h = (int)(unit % c->H);
    int64_t i = c->rows ? c->rows[r] : r;
    int s = seq_of_token(c->offsets, c->n_seqs, i);
    /* the sequence's keys: its base rows already cached, then one per query row;
     * the query row sits at the key of its own position, `last` */
    int64_t lo = c->kv_offsets[s];
    int64_t base = ((int64_t)c->kv_offsets[s + 1] - lo) - (c->offsets[s + 1] - c->offsets[s]);
    int64_t last = lo + base + (i - c->offsets[s]);
    int64_t hi = c->causal ? last : (int64_t)c->kv_offsets[s + 1] - 1; /* inclusive */
    if (c->causal && c->window > 0 && last - c->window + 1 > lo) lo = last - c->window + 1;
    int g = c->H / c->Hkv;
    int kv = h / g;
    int d = c->d;
    const double* qi = c->q + (i * c->H + h) * (int64_t)d;
    double* o = c->out + (r * c->H + h) * (int64_t)d;

    /* scores over the visible keys and their maximum */
    double m = -INFINITY;
    for (int64_t j = lo; j <= hi; ++j) {
        const double* kj = c->k + (j * c->Hkv + kv) * (int64_t)d;
        double dot = 0.0;
        for (int x = 0; x < d; ++x) dot += qi[x] * kj[x];
        double sj = c->scale * dot;
        e[j - lo] = sj;
        if (sj > m) m = sj;
    }
    /* softmax weights (max-subtracted) and their sum */
    double Z = 0.0;
    for (int64_t j = lo; j <= hi; ++j) {
        e[j - lo] = exp(e[j - lo] - m);
        Z += e[j - lo];
    }
    /* weighted sum of the visible values */
    for (int x = 0; x < d; ++x) o[x] = 0.0;
    for (int64_t j = lo; j <= hi; ++j) {
        const double* vj = c->v + (j * c->Hkv + kv) * (int64_t)d;
        double wgt = e[j - lo];
        for (int x = 0; x < d; ++x) o[x] += wgt * vj[x];
    }
    for (int x = 0; x < d; ++x) o[x] /= Z;
    /* gated output: o * sigmoid(gate) */
    if (c->gate) {
        for (int x = 0; x < d; ++x) {
            double g = c->gate_per_head ? c->gate[i * c->H + h] : c->gate[(i * c->H + h) * (int64_t)d + x];
            o[x] *= 1.0 / (1.0 + exp(-g));
        }
    }
}

/* Attention of query rows over a K/V cache.  Sequence s owns query rows
 * q_offsets[s] .. q_offsets[s+1]-1 and cache rows kv_offsets[s] ..
 * kv_offsets[s+1]-1, at least as many as queries: its first base_s cache rows
 * were there before, the query rows are the last ones.  out[r, h, :] =
 * softmax_j(scale * q[i,h,:] . k[j,kv,:]) v[j,kv,:] over the visible keys j of
 * row i = rows[r] (or r when rows is NULL): the keys of i's sequence, and when
 * causal only those up to i's own position (base_s + i - q_offsets[s]) and, with
 * window > 0, not more than window of them (the latest); with a gate, the row's
 * output is then multiplied by sigmoid(gate) per element (gate [T_q, H*d]) or per
 * head (gate [T_q, H]).  All arithmetic in f64.  NULL offsets (both): one
 * sequence. */
int oracle_chunk_attn(const double* q, const double* k, const double* v,
                      const int32_t* q_offsets, const int32_t* kv_offsets, int n_seqs,
                      int64_t T_q, int64_t T_kv, int n_head, int n_head_kv, int head_dim,
                      double scale, int causal, int64_t window, const double* gate,
                      int gate_per_head, const int64_t* rows, int64_t n_rows, double* out,
                      int n_threads) {
    int32_t one_q[2], one_kv[2];
    if (T_q < 0 || T_kv < 0 || n_head <= 0 || n_head_kv <= 0 || head_dim <= 0 ||
        n_head % n_head_kv || (!q_offsets) != (!kv_offsets) || window < 0 ||
        (window > 0 && !causal))
        return ORACLE_BAD_ARG;
    if (!q_offsets) {
        one_q[0] = 0;
        one_q[1] = (int32_t)T_q;
        one_kv[0] = 0;
        one_kv[1] = (int32_t)T_kv;
        q_offsets = one_q;
        kv_offsets = one_kv;
        n_seqs = 1;
    }
    if (!check_offsets(q_offsets, n_seqs, T_q) || !check_offsets(kv_offsets, n_seqs, T_kv))
        return ORACLE_BAD_ARG;
    for (int s = 0; s < n_seqs; ++s)
        if (kv_offsets[s + 1] - kv_offsets[s] < q_offsets[s + 1] - q_offsets[s])
            return ORACLE_BAD_ARG;
    if (T_q == 0) return ORACLE_OK;
    if (!rows) n_rows = T_q;
    for (int64_t r = 0; rows && r < n_rows; ++r)
        if (rows[r] < 0 || rows[r] >= T_q) return ORACLE_BAD_ARG;
    attn_ctx c = {q, k, v, out, rows, q_offsets, kv_offsets, n_seqs, n_head, n_head_kv,
                  head_dim, causal ? 1 : 0, window, gate, gate_per_head ? 1 : 0, scale};
    return run_pool(attn_unit, &c, n_rows * n_head, (size_t)T_kv, n_threads); /* scores: <= T_kv */
}

/* out[r, h, :] = softmax_j(scale * q[i,h,:] . k[j,kv,:]) v[j,kv,:] over the
 * visible keys j of row i = rows[r] (or r when rows is NULL).  Visible: same
 * sequence as i and, when causal, j <= i.  All arithmetic in f64.  (The chunk
 * case with nothing cached before: each sequence's keys are its query rows.) */
int oracle_gqa_attn(const double* q, const double* k, const double* v,
                    const int32_t* seq_offsets, int n_seqs, int64_t T, int n_head,
                    int n_head_kv, int head_dim, double scale, int causal,
                    const int64_t* rows, int64_t n_rows, double* out, int n_threads) {
    return oracle_chunk_attn(q, k, v, seq_offsets, seq_offsets, n_seqs, T, T, n_head,
                             n_head_kv, head_dim, scale, causal, 0, NULL, 0, rows, n_rows,
                             out, n_threads);
}

/* 8-bit quantisation of n_rows rows of len floats each (needle-core v3/model.rs,
 * `quant_rows` per (token, head) row; `quantize_rows` returning the integer rows
 * and one scale per row).  codes[r, i] * scales[r] (rounded to float) is the
 * fake-quantised value, written to deq when deq is not NULL.  Single precision
 * throughout: scale = max|x| / 127, code = nearest integer to x / scale (ties to
 * even), clamped to -127..127. */
int oracle_quant_rows(const float* x, int64_t n_rows, int len, int8_t* codes, float* scales,
                      float* deq) {
    if (n_rows < 0 || len <= 0 || (n_rows > 0 && (!x || !codes || !scales)))
        return ORACLE_BAD_ARG;
    for (int64_t r = 0; r < n_rows; ++r) {
        const float* xr = x + r * len;
        float amax = 0.0f;
        for (int i = 0; i < len; ++i) {
            const float m = fabsf(xr[i]);
            if (m > amax) amax = m;
        }
        const float scale = amax / 127.0f;
        scales[r] = scale;
        for (int i = 0; i < len; ++i) {
            float c = scale > 0.0f ? rintf(xr[i] / scale) : 0.0f;
            if (c > 127.0f) c = 127.0f;
            if (c < -127.0f) c = -127.0f;
            codes[r * len + i] = (int8_t)c;
            if (deq) deq[r * len + i] = c * scale;
        }
    }
    return ORACLE_OK;
}

const char* oracle_version(void) { return "pfa-oracle 1 (f64, plain loops)"; }
