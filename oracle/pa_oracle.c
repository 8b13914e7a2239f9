/*
 * CPU oracle for paged-attention decode (and prefill over a paged context, see
 * orc_prefill at the end).  TEST INFRASTRUCTURE ONLY: the tests,
 * the smoke check and the CPU-baseline leg of the benchmark call it; the
 * product path never does.  It shares no code, header or constant with the
 * GPU library.
 *
 * What it computes is the plain definition the paged-attention pages reduce
 * to.  The page of commit 87a19d2 (paged_attention_v2_triton.py, the
 * online-softmax fix) identifies its tiled update as the flash-attention
 * online softmax, and the page of commit 8d26e23 (docs, the attention_partial
 * compound type) gives the partition combine the same math; both are exact
 * re-orderings of
 *
 *     out[s,h,:] = sum_t softmax_t( scale * q[s,h,:] . K[t,:] ) * V[t,:]
 *
 * where token t of sequence s lives in physical page block_tables[s][t/bs]
 * at slot t%bs (commit b80fd2b, paged_attn.py, rewrite item 1: K/V are
 * gathered from the caches by block id), and query head h reads KV head
 * h / (num_heads/num_kv_heads) (commit 8d26e23, grid on num_kv_heads: one
 * block serves all query heads that share a KV head).  Everything is
 * evaluated in double precision, one (sequence, query head) at a time, with
 * no blocking or reordering.
 *
 * Layouts:
 *   q            [S][Hq][D]              16-bit (f16 or bf16 bit patterns)
 *   key_cache    [NB][Hkv][bs][D]        16-bit
 *   value_cache  [NB][Hkv][bs][D]        16-bit
 *   block_tables [S][MB]                 int32
 *   seq_lens     [S]                     int32
 *   out          [S][Hq][D]              double
 *
 * Return codes: 0 ok, -1 bad shape, -2 page id outside [0, NB),
 * -3 seq_len larger than MB*bs, -4 out of memory.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_F16 0
#define ORC_BF16 1

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
static double orc_from_f16(uint16_t h) {
    int sign = h >> 15;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);                 /* subnormal: f * 2^-24 */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(f + 1024), e - 25);     /* (1 + f/2^10) * 2^(e-15) */
    return sign ? -v : v;
}

/* bfloat16 is the upper half of an IEEE 754 binary32. */
static double orc_from_bf16(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double orc_val(uint16_t x, int dtype) {
    return dtype == ORC_BF16 ? orc_from_bf16(x) : orc_from_f16(x);
}

/* exported so a test can compare the conversion with library conversions */
void orc_convert(const uint16_t* in, double* out, int64_t n, int dtype) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_val(in[i], dtype);
}

/* Address of element (token t, dim 0) of KV head kvh for sequence s, or NULL
 * with *err set when the table points outside the pool. */
static const uint16_t* orc_token(const uint16_t* cache, const int32_t* bt, int s, int t,
                                 int kvh, int Hkv, int bs, int D, int NB, int MB,
                                 int* err) {
    int32_t page = bt[(int64_t)s * MB + t / bs];
    if (page < 0 || page >= NB) {
        *err = -2;
        return NULL;
    }
    int slot = t % bs;
    return cache + (((int64_t)page * Hkv + kvh) * bs + slot) * (int64_t)D;
}

static int orc_check(int S, int Hq, int Hkv, int D, int bs, int NB, int MB,
                     const int32_t* seq_lens) {
    if (S < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || bs <= 0 || NB < 0 || MB < 0) return -1;
    if (Hq % Hkv) return -1;
    for (int s = 0; s < S; ++s)
        if (seq_lens[s] > (int64_t)MB * bs) return -3;
    return 0;
}

/* One (sequence, query head) row of the definition.  x has room for L doubles. */
static int orc_row(double* out, const uint16_t* q, const uint16_t* kc, const uint16_t* vc,
                   const int32_t* bt, int L, int s, int h, int Hq, int Hkv, int D, int bs,
                   int NB, int MB, double scale, int dtype, double* x) {
    int g = Hq / Hkv;
    int kvh = h / g;
    int err = 0;
    for (int d = 0; d < D; ++d) out[d] = 0.0;
    if (L <= 0) return 0;
    const uint16_t* qrow = q + ((int64_t)s * Hq + h) * D;
    /* logits x_t = scale * sum_d q_d k_{t,d}, summed over d in increasing order */
    double m = -INFINITY;
    for (int t = 0; t < L; ++t) {
        const uint16_t* k = orc_token(kc, bt, s, t, kvh, Hkv, bs, D, NB, MB, &err);
        if (!k) return err;
        double acc = 0.0;
        for (int d = 0; d < D; ++d) acc += orc_val(qrow[d], dtype) * orc_val(k[d], dtype);
        x[t] = scale * acc;
        if (x[t] > m) m = x[t];
    }
    /* softmax weights w_t = exp(x_t - m), Z = sum_t w_t; out = sum_t w_t V_t / Z */
    double Z = 0.0;
    for (int t = 0; t < L; ++t) {
        double w = exp(x[t] - m);
        Z += w;
        const uint16_t* v = orc_token(vc, bt, s, t, kvh, Hkv, bs, D, NB, MB, &err);
        if (!v) return err;
        for (int d = 0; d < D; ++d) out[d] += w * orc_val(v[d], dtype);
    }
    for (int d = 0; d < D; ++d) out[d] /= Z;
    return 0;
}

/* Full decode.  nthreads <= 0 uses the OpenMP default. Returns the thread count
 * actually used through *used_threads when it is not NULL. */
int orc_decode(double* out, const uint16_t* q, const uint16_t* kc, const uint16_t* vc,
               const int32_t* bt, const int32_t* seq_lens, int S, int Hq, int Hkv, int D,
               int bs, int NB, int MB, double scale, int dtype, int nthreads,
               int* used_threads) {
    int rc = orc_check(S, Hq, Hkv, D, bs, NB, MB, seq_lens);
    if (rc) return rc;
    int64_t maxL = 1;
    for (int s = 0; s < S; ++s)
        if (seq_lens[s] > maxL) maxL = seq_lens[s];
    int status = 0;
    int used = 1;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#endif
#pragma omp parallel
    {
#ifdef _OPENMP
#pragma omp single
        used = omp_get_num_threads();
#endif
        double* x = (double*)malloc(sizeof(double) * maxL);
        if (!x) {
#pragma omp atomic write
            status = -4;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < (int64_t)S * Hq; ++r) {
            if (!x) continue;
            int s = (int)(r / Hq), h = (int)(r % Hq);
            int e = orc_row(out + r * D, q, kc, vc, bt, seq_lens[s], s, h, Hq, Hkv, D, bs,
                            NB, MB, scale, dtype, x);
            if (e) {
#pragma omp atomic write
                status = e;
            }
        }
        free(x);
    }
    if (used_threads) *used_threads = used;
    return status;
}

/* Selected rows only: rows[2*i] = sequence, rows[2*i+1] = query head;
 * out is [n_rows][D]. */
int orc_decode_rows(double* out, const int32_t* rows, int n_rows, const uint16_t* q,
                    const uint16_t* kc, const uint16_t* vc, const int32_t* bt,
                    const int32_t* seq_lens, int S, int Hq, int Hkv, int D, int bs, int NB,
                    int MB, double scale, int dtype, int nthreads) {
    int rc = orc_check(S, Hq, Hkv, D, bs, NB, MB, seq_lens);
    if (rc) return rc;
    int64_t maxL = 1;
    for (int i = 0; i < n_rows; ++i) {
        int s = rows[2 * i];
        if (s < 0 || s >= S || rows[2 * i + 1] < 0 || rows[2 * i + 1] >= Hq) return -1;
        if (seq_lens[s] > maxL) maxL = seq_lens[s];
    }
    int status = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#endif
#pragma omp parallel
    {
        double* x = (double*)malloc(sizeof(double) * maxL);
        if (!x) {
#pragma omp atomic write
            status = -4;
        }
#pragma omp for schedule(dynamic, 1)
        for (int i = 0; i < n_rows; ++i) {
            if (!x) continue;
            int s = rows[2 * i], h = rows[2 * i + 1];
            int e = orc_row(out + (int64_t)i * D, q, kc, vc, bt, seq_lens[s], s, h, Hq, Hkv,
                            D, bs, NB, MB, scale, dtype, x);
            if (e) {
#pragma omp atomic write
                status = e;
            }
        }
        free(x);
    }
    return status;
}

/* Gather by block table: k_out/v_out [S][Hkv][Lcap][D] receive the raw 16-bit
 * values of tokens t < seq_lens[s]; other slots are left untouched. */
int orc_gather(uint16_t* k_out, uint16_t* v_out, const uint16_t* kc, const uint16_t* vc,
               const int32_t* bt, const int32_t* seq_lens, int S, int Hkv, int D, int bs,
               int NB, int MB, int Lcap) {
    int rc = orc_check(S, Hkv, Hkv, D, bs, NB, MB, seq_lens);
    if (rc) return rc;
    for (int s = 0; s < S; ++s) {
        int L = seq_lens[s];
        if (L > Lcap) return -1;
        for (int kvh = 0; kvh < Hkv; ++kvh)
            for (int t = 0; t < L; ++t) {
                int err = 0;
                const uint16_t* k = orc_token(kc, bt, s, t, kvh, Hkv, bs, D, NB, MB, &err);
                const uint16_t* v = orc_token(vc, bt, s, t, kvh, Hkv, bs, D, NB, MB, &err);
                if (!k || !v) return err;
                int64_t o = (((int64_t)s * Hkv + kvh) * Lcap + t) * D;
                memcpy(k_out + o, k, sizeof(uint16_t) * D);
                memcpy(v_out + o, v, sizeof(uint16_t) * D);
            }
    }
    return 0;
}

/* Per-partition partials by definition (commit 8d26e23, the attention_partial
 * compound type: max_score, exp_sum, weighted_v).  Partition p of sequence s covers tokens
 * [p*P, min(L, (p+1)*P)).  For each (s, h, p):
 *   m   = max_t x_t                       (x_t = scale * q.k_t, natural-log units)
 *   l   = sum_t exp(x_t - m)
 *   acc = sum_t exp(x_t - m) V_t / l      (the partition's own normalised output)
 * Partitions past the end of a sequence hold the identity (-inf, 0, 0).
 * m, l: [S][Hq][NP]; acc: [S][Hq][NP][D]. */
int orc_partials(double* m_out, double* l_out, double* acc_out, const uint16_t* q,
                 const uint16_t* kc, const uint16_t* vc, const int32_t* bt,
                 const int32_t* seq_lens, int S, int Hq, int Hkv, int D, int bs, int NB,
                 int MB, double scale, int dtype, int P, int NP) {
    int rc = orc_check(S, Hq, Hkv, D, bs, NB, MB, seq_lens);
    if (rc) return rc;
    if (P <= 0 || NP < 0) return -1;
    int g = Hq / Hkv;
    for (int s = 0; s < S; ++s) {
        int L = seq_lens[s];
        if (L > 0 && (L + P - 1) / P > NP) return -1;
        for (int h = 0; h < Hq; ++h) {
            int kvh = h / g;
            const uint16_t* qrow = q + ((int64_t)s * Hq + h) * D;
            for (int p = 0; p < NP; ++p) {
                int64_t base = ((int64_t)s * Hq + h) * NP + p;
                double* acc = acc_out + base * D;
                for (int d = 0; d < D; ++d) acc[d] = 0.0;
                int t0 = p * P, t1 = (p + 1) * P < L ? (p + 1) * P : L;
                if (t0 >= t1) {
                    m_out[base] = -INFINITY;
                    l_out[base] = 0.0;
                    continue;
                }
                double m = -INFINITY;
                int err = 0;
                for (int t = t0; t < t1; ++t) {
                    const uint16_t* k = orc_token(kc, bt, s, t, kvh, Hkv, bs, D, NB, MB, &err);
                    if (!k) return err;
                    double a = 0.0;
                    for (int d = 0; d < D; ++d) a += orc_val(qrow[d], dtype) * orc_val(k[d], dtype);
                    if (scale * a > m) m = scale * a;
                }
                double l = 0.0;
                for (int t = t0; t < t1; ++t) {
                    const uint16_t* k = orc_token(kc, bt, s, t, kvh, Hkv, bs, D, NB, MB, &err);
                    const uint16_t* v = orc_token(vc, bt, s, t, kvh, Hkv, bs, D, NB, MB, &err);
                    if (!k || !v) return err;
                    double a = 0.0;
                    for (int d = 0; d < D; ++d) a += orc_val(qrow[d], dtype) * orc_val(k[d], dtype);
                    double w = exp(scale * a - m);
                    l += w;
                    for (int d = 0; d < D; ++d) acc[d] += w * orc_val(v[d], dtype);
                }
                for (int d = 0; d < D; ++d) acc[d] /= l;
                m_out[base] = m;
                l_out[base] = l;
            }
        }
    }
    return 0;
}

/*
 * Prefill over a paged context: the prefix path of the page of commit b80fd2b
 * (paged_attn.py: _forward_prefix_pytorch runs one online softmax over the
 * context gathered from the caches by block id, then over the current chunk's
 * own keys under the causal mask; rewrite item 1 gathers the context once).
 * By definition, for sequence s with C = ctx_lens[s] cached tokens and new
 * tokens n = 0 .. Qn-1 (Qn = qstart[s+1] - qstart[s]) held at rows
 * r = qstart[s] + n of q, k_new and v_new, query head h attends to the context
 * tokens t < C (in the caches through block_tables, as in decode) and to the new
 * tokens j <= n:
 *
 *     out[r,h,:] = sum_u softmax_u( scale * q[r,h,:] . K_u ) * V_u
 *
 * evaluated in double precision with the keys in the order context, then new.
 * C <= 0 means no context.
 *
 * Layouts: q, out [T][Hq][D]; k_new, v_new [T][Hkv][D]; qstart [S+1] with
 * qstart[0] = 0 and T = qstart[S]; caches and tables as above.
 * rows: NULL for every (row, head), else n_rows pairs (row, query head) and out
 * is [n_rows][D].
 */
static int orc_prefill_row(double* out, const uint16_t* q, const uint16_t* kn,
                           const uint16_t* vn, const uint16_t* kc, const uint16_t* vc,
                           const int32_t* bt, int C, int r0, int n, int s, int h, int Hq,
                           int Hkv, int D, int bs, int NB, int MB, double scale, int dtype,
                           double* x) {
    int g = Hq / Hkv;
    int kvh = h / g;
    int err = 0;
    int r = r0 + n;
    if (C < 0) C = 0;
    const uint16_t* qrow = q + ((int64_t)r * Hq + h) * D;
    int L = C + n + 1;
    double m = -INFINITY;
    for (int u = 0; u < L; ++u) {
        const uint16_t* k = u < C ? orc_token(kc, bt, s, u, kvh, Hkv, bs, D, NB, MB, &err)
                                  : kn + ((int64_t)(r0 + u - C) * Hkv + kvh) * D;
        if (!k) return err;
        double acc = 0.0;
        for (int d = 0; d < D; ++d) acc += orc_val(qrow[d], dtype) * orc_val(k[d], dtype);
        x[u] = scale * acc;
        if (x[u] > m) m = x[u];
    }
    for (int d = 0; d < D; ++d) out[d] = 0.0;
    double Z = 0.0;
    for (int u = 0; u < L; ++u) {
        double w = exp(x[u] - m);
        Z += w;
        const uint16_t* v = u < C ? orc_token(vc, bt, s, u, kvh, Hkv, bs, D, NB, MB, &err)
                                  : vn + ((int64_t)(r0 + u - C) * Hkv + kvh) * D;
        if (!v) return err;
        for (int d = 0; d < D; ++d) out[d] += w * orc_val(v[d], dtype);
    }
    for (int d = 0; d < D; ++d) out[d] /= Z;
    return 0;
}

int orc_prefill(double* out, const int32_t* rows, int n_rows, const uint16_t* q,
                const uint16_t* kn, const uint16_t* vn, const uint16_t* kc, const uint16_t* vc,
                const int32_t* bt, const int32_t* ctx_lens, const int32_t* qstart, int S,
                int Hq, int Hkv, int D, int bs, int NB, int MB, double scale, int dtype,
                int nthreads, int* used_threads) {
    if (S < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || bs <= 0 || NB < 0 || MB < 0) return -1;
    if (Hq % Hkv) return -1;
    if (qstart[0] != 0) return -1;
    int64_t maxL = 1;
    for (int s = 0; s < S; ++s) {
        if (qstart[s + 1] < qstart[s]) return -1;
        if (ctx_lens[s] > (int64_t)MB * bs) return -3;
        int64_t L = (ctx_lens[s] > 0 ? ctx_lens[s] : 0) + (qstart[s + 1] - qstart[s]);
        if (L > maxL) maxL = L;
    }
    int T = qstart[S];
    /* sequence of every row */
    int* seq = (int*)malloc(sizeof(int) * (T > 0 ? T : 1));
    if (!seq) return -4;
    for (int s = 0; s < S; ++s)
        for (int r = qstart[s]; r < qstart[s + 1]; ++r) seq[r] = s;
    int64_t total = rows ? n_rows : (int64_t)T * Hq;
    int status = 0;
    int used = 1;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#endif
#pragma omp parallel
    {
#ifdef _OPENMP
#pragma omp single
        used = omp_get_num_threads();
#endif
        double* x = (double*)malloc(sizeof(double) * maxL);
        if (!x) {
#pragma omp atomic write
            status = -4;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < total; ++i) {
            if (!x) continue;
            int r = rows ? rows[2 * i] : (int)(i / Hq);
            int h = rows ? rows[2 * i + 1] : (int)(i % Hq);
            int e;
            if (r < 0 || r >= T || h < 0 || h >= Hq) {
                e = -1;
            } else {
                int s = seq[r];
                e = orc_prefill_row(out + i * D, q, kn, vn, kc, vc, bt, ctx_lens[s], qstart[s],
                                    r - qstart[s], s, h, Hq, Hkv, D, bs, NB, MB, scale, dtype, x);
            }
            if (e) {
#pragma omp atomic write
                status = e;
            }
        }
        free(x);
    }
    free(seq);
    if (used_threads) *used_threads = used;
    return status;
}
