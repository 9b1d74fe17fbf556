/* oracle_driver.c -- runs the CPU oracle's entry points on small packed inputs under
 * AddressSanitizer and UBSan: every array is heap-allocated at its exact size, so a read
 * or write past one (a wrong index, a wrong row count) is reported.  Covers QK-norm +
 * RoPE (from position 0 and from start positions), prefill attention, chunks over cached
 * prefixes with a window and both gate layouts, row subsets, and 8-bit quantisation.
 * Also checks a few exact facts of the results, so a silent no-op cannot pass.
 * Exit status 0 when everything holds. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_qknorm_rope_from(const float* q, const float* k, const float* wq, const float* wk,
                            const int32_t* seq_offsets, int n_seqs, const int64_t* pos0,
                            int64_t T, int n_head, int n_head_kv, int head_dim, int rope_dim,
                            double base, double eps, double* q_out, double* k_out,
                            int n_threads);
int oracle_chunk_attn(const double* q, const double* k, const double* v,
                      const int32_t* q_offsets, const int32_t* kv_offsets, int n_seqs,
                      int64_t T_q, int64_t T_kv, int n_head, int n_head_kv, int head_dim,
                      double scale, int causal, int64_t window, const double* gate,
                      int gate_per_head, const int64_t* rows, int64_t n_rows, double* out,
                      int n_threads);
int oracle_gqa_attn(const double* q, const double* k, const double* v,
                    const int32_t* seq_offsets, int n_seqs, int64_t T, int n_head,
                    int n_head_kv, int head_dim, double scale, int causal,
                    const int64_t* rows, int64_t n_rows, double* out, int n_threads);
int oracle_quant_rows(const float* x, int64_t n_rows, int len, int8_t* codes, float* scales,
                      float* deq);

static int failures = 0;
static void expect(int ok, const char* what) {
    if (!ok) {
        fprintf(stderr, "FAILED: %s\n", what);
        ++failures;
    }
}

static uint64_t state = 88172645463325252ull;
static double unif(void) { /* xorshift64 in [-1, 1) */
    state ^= state << 13;
    state ^= state >> 7;
    state ^= state << 17;
    return (double)(state >> 11) / (double)(1ull << 52) - 1.0;
}

static float* fvec(size_t n) {
    float* a = malloc(sizeof(float) * n);
    for (size_t i = 0; i < n; ++i) a[i] = (float)unif();
    return a;
}
static double* dvec(size_t n) {
    double* a = malloc(sizeof(double) * n);
    for (size_t i = 0; i < n; ++i) a[i] = unif();
    return a;
}

int main(void) {
    /* packed sequences (an empty one, a one-row one), 6 query heads over 2 K/V heads */
    const int n_seqs = 4, H = 6, Hkv = 2, d = 64, n = 48;
    int32_t* offs = malloc(sizeof(int32_t) * (n_seqs + 1));
    const int lens[4] = {9, 0, 1, 14};
    offs[0] = 0;
    for (int s = 0; s < n_seqs; ++s) offs[s + 1] = offs[s] + lens[s];
    const int T = offs[n_seqs];
    float *q = fvec((size_t)T * H * d), *k = fvec((size_t)T * Hkv * d);
    float *wq = fvec(d), *wk = fvec(d);
    double *qo = malloc(sizeof(double) * T * H * d), *ko = malloc(sizeof(double) * T * Hkv * d);
    int64_t* pos0 = malloc(sizeof(int64_t) * n_seqs);
    for (int s = 0; s < n_seqs; ++s) pos0[s] = 100 * s;
    for (int threads = 1; threads <= 3; threads += 2) {
        expect(oracle_qknorm_rope_from(q, k, wq, wk, offs, n_seqs, NULL, T, H, Hkv, d, n, 1e4,
                                       1e-6, qo, ko, threads) == 0, "qknorm_rope");
        expect(oracle_qknorm_rope_from(q, k, wq, wk, offs, n_seqs, pos0, T, H, Hkv, d, n, 1e4,
                                       1e-6, qo, ko, threads) == 0, "qknorm_rope_from");
    }
    double *v = dvec((size_t)T * Hkv * d), *out = malloc(sizeof(double) * T * H * d);
    expect(oracle_gqa_attn(qo, ko, v, offs, n_seqs, T, H, Hkv, d, 0.125, 1, NULL, 0, out, 2) == 0,
           "gqa_attn");
    /* the first row of a sequence equals its V exactly */
    for (int h = 0; h < H; ++h)
        for (int c = 0; c < d; ++c)
            expect(out[(size_t)(offs[3] * H + h) * d + c] == v[(size_t)(offs[3] * Hkv + h / 3) * d + c],
                   "first row is V");
    int64_t* rows = malloc(sizeof(int64_t) * 3);
    rows[0] = 0;
    rows[1] = 9;
    rows[2] = T - 1;
    double* out3 = malloc(sizeof(double) * 3 * H * d);
    expect(oracle_gqa_attn(qo, ko, v, offs, n_seqs, T, H, Hkv, d, 0.125, 0, rows, 3, out3, 1) == 0,
           "gqa_attn rows");
    /* chunks: each sequence keeps `base` earlier rows before its queries */
    int32_t* kv_offs = malloc(sizeof(int32_t) * (n_seqs + 1));
    kv_offs[0] = 0;
    for (int s = 0; s < n_seqs; ++s) kv_offs[s + 1] = kv_offs[s] + lens[s] + 5 * s;
    const int T_kv = kv_offs[n_seqs];
    double *kc = dvec((size_t)T_kv * Hkv * d), *vc = dvec((size_t)T_kv * Hkv * d);
    double *g_elem = dvec((size_t)T * H * d), *g_head = dvec((size_t)T * H);
    for (int64_t window = 0; window <= 4; window += 4) {
        expect(oracle_chunk_attn(qo, kc, vc, offs, kv_offs, n_seqs, T, T_kv, H, Hkv, d, 0.125, 1,
                                 window, g_elem, 0, NULL, 0, out, 3) == 0, "chunk, gate per element");
        expect(oracle_chunk_attn(qo, kc, vc, offs, kv_offs, n_seqs, T, T_kv, H, Hkv, d, 0.125, 1,
                                 window, g_head, 1, rows, 3, out3, 1) == 0, "chunk, gate per head");
    }
    /* bad arguments are refused, not read past */
    expect(oracle_chunk_attn(qo, kc, vc, kv_offs, offs, n_seqs, T_kv, T, H, Hkv, d, 0.125, 1, 0,
                             NULL, 0, NULL, 0, out, 1) != 0, "cache shorter than queries");
    rows[2] = T;
    expect(oracle_gqa_attn(qo, ko, v, offs, n_seqs, T, H, Hkv, d, 0.125, 1, rows, 3, out3, 1) != 0,
           "row out of range");
    /* 8-bit quantisation, with and without the fake-quantised copy */
    const int qr = 37, ql = 33;
    float *x = fvec((size_t)qr * ql), *sc = malloc(sizeof(float) * qr);
    float* deq = malloc(sizeof(float) * qr * ql);
    int8_t* codes = malloc((size_t)qr * ql);
    for (int i = 0; i < ql; ++i) x[5 * ql + i] = 0.0f; /* a zero row */
    expect(oracle_quant_rows(x, qr, ql, codes, sc, deq) == 0, "quant_rows");
    expect(oracle_quant_rows(x, qr, ql, codes, sc, NULL) == 0, "quant_rows without deq");
    expect(sc[5] == 0.0f, "zero row has scale 0");
    for (int r = 0; r < qr; ++r) {
        int top = 0;
        for (int i = 0; i < ql; ++i) top |= abs(codes[r * ql + i]) == 127;
        expect(r == 5 || top, "every nonzero row reaches the top code");
    }
    free(offs); free(q); free(k); free(wq); free(wk); free(qo); free(ko); free(pos0);
    free(v); free(out); free(rows); free(out3); free(kv_offs); free(kc); free(vc);
    free(g_elem); free(g_head); free(x); free(sc); free(deq); free(codes);
    printf("oracle driver: %d failures\n", failures);
    return failures ? 1 : 0;
}
