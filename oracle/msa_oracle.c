/*
 * msa_oracle.c -- plain fp64 CPU reference of the MSA hot path.
 * TEST INFRASTRUCTURE ONLY (tests, smoke check, CPU-baseline leg of the bench).
 * Definitions and sources are documented in msa_oracle.h.
 * Build: gcc -O2 -ffp-contract=off -fPIC -shared -pthread (no fast-math; plain C99).
 */
#define _POSIX_C_SOURCE 200809L
#include "msa_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- bf16 --- */

double orc_bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

uint16_t orc_bf16_from_double(double x)
{
    /* bf16 = 1 sign, 8 exponent, 7 fraction bits: 8 significant bits for
     * normal numbers, and a fixed spacing of 2^-133 below 2^-126.  Round to
     * that grid with nearbyint (round-half-even in the default mode). */
    if (isnan(x)) return 0x7FC0;
    if (x == 0.0) return signbit(x) ? 0x8000 : 0x0000;
    if (isinf(x)) return signbit(x) ? 0xFF80 : 0x7F80;
    int e;
    frexp(x, &e);                 /* |x| = m * 2^e, m in [0.5, 1) */
    int q = e - 8;                /* spacing of an 8-bit significand */
    if (q < -133) q = -133;       /* subnormal spacing */
    double y = ldexp(nearbyint(ldexp(x, -q)), q);
    if (fabs(y) > 3.3895313892515355e38) /* largest finite bf16 (0x7F7F) */
        return signbit(x) ? 0xFF80 : 0x7F80;
    float f = (float)y;           /* exact: y is on the bf16 grid */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

/* ------------------------------------------------- document offset tables */

void orc_group_ids(const int64_t* doc_ids, int64_t n, int64_t* group_ids)
{
    /* [P2 5.3] The tokens of one document are consecutive, so the document ids form
     * maximal runs of equal values; every run is one group, and the groups are
     * numbered 1, 2, 3, ... in the order the runs appear. */
    int64_t run = 0;
    int64_t i = 0;
    while (i < n) {
        int64_t j = i;
        run += 1;
        while (j < n && doc_ids[j] == doc_ids[i]) group_ids[j++] = run;
        i = j;
    }
}

int64_t orc_doc_tok_offsets(const int64_t* doc_ids, int64_t n, int64_t* doc_tok_off)
{
    int64_t* gid = (int64_t*)malloc((size_t)(n > 0 ? n : 1) * sizeof(int64_t));
    orc_group_ids(doc_ids, n, gid);
    int64_t n_groups = 0;
    for (int64_t i = 0; i < n; ++i) {
        if (gid[i] != n_groups) {      /* first token of group gid[i] */
            doc_tok_off[n_groups] = i;
            n_groups = gid[i];
        }
    }
    doc_tok_off[n_groups] = n;
    free(gid);
    return n_groups;
}

int64_t orc_block_offsets(const int64_t* doc_tok_off, int32_t n_docs,
                          int64_t* doc_blk_off, int32_t* max_doc_blocks)
{
    int32_t mx = 0;
    doc_blk_off[0] = 0;
    for (int32_t d = 0; d < n_docs; ++d) {
        int64_t len = doc_tok_off[d + 1] - doc_tok_off[d];
        int64_t nb = (len + ORC_BLOCK - 1) / ORC_BLOCK;
        doc_blk_off[d + 1] = doc_blk_off[d] + nb;
        if (nb > mx) mx = (int32_t)nb;
    }
    if (max_doc_blocks) *max_doc_blocks = mx;
    return doc_blk_off[n_docs];
}

/* ---------------------------------------------------------------- pooling */

void orc_pool(int32_t n_layers, const uint16_t* x, int64_t n_tok,
              const int64_t* doc_tok_off, const int64_t* doc_blk_off, int32_t n_docs,
              int64_t n_blk, uint16_t* xbar)
{
    for (int32_t l = 0; l < n_layers; ++l) {
        const uint16_t* xl = x + (size_t)l * (size_t)n_tok * ORC_ROW;
        uint16_t* ol = xbar + (size_t)l * (size_t)n_blk * ORC_ROW;
        for (int32_t d = 0; d < n_docs; ++d) {
            int64_t s = doc_tok_off[d], e = doc_tok_off[d + 1];
            for (int64_t j = 0; doc_blk_off[d] + j < doc_blk_off[d + 1]; ++j) {
                int64_t t0 = s + ORC_BLOCK * j;
                int64_t t1 = t0 + ORC_BLOCK < e ? t0 + ORC_BLOCK : e;
                uint16_t* out = ol + (size_t)(doc_blk_off[d] + j) * ORC_ROW;
                for (int c = 0; c < ORC_ROW; ++c) {
                    double sum = 0.0;
                    for (int64_t t = t0; t < t1; ++t)
                        sum += orc_bf16_to_double(xl[(size_t)t * ORC_ROW + c]);
                    out[c] = orc_bf16_from_double(sum / (double)(t1 - t0));
                }
            }
        }
    }
}

void orc_head_norms(const uint16_t* rows, int64_t n_rows, double* norms)
{
    for (int64_t r = 0; r < n_rows; ++r)
        for (int h = 0; h < ORC_H; ++h) {
            double ss = 0.0;
            for (int i = 0; i < ORC_D; ++i) {
                double v = orc_bf16_to_double(rows[(size_t)r * ORC_ROW + h * ORC_D + i]);
                ss += v * v;
            }
            norms[r * ORC_H + h] = sqrt(ss);
        }
}

/* ---------------------------------------------------------------- routing */

static double cosine(const uint16_t* a, const uint16_t* b)
{
    double ab = 0.0, aa = 0.0, bb = 0.0;
    for (int i = 0; i < ORC_D; ++i) {
        double x = orc_bf16_to_double(a[i]), y = orc_bf16_to_double(b[i]);
        ab += x * y;
        aa += x * x;
        bb += y * y;
    }
    double na = sqrt(aa), nb = sqrt(bb);
    if (na < 1e-8) na = 1e-8;
    if (nb < 1e-8) nb = 1e-8;
    return ab / (na * nb);
}

double orc_block_score(const uint16_t* q_row, const uint16_t* k_row)
{
    double s = 0.0;
    for (int h = 0; h < ORC_H; ++h) s += cosine(q_row + h * ORC_D, k_row + h * ORC_D);
    return s / ORC_H;
}

void orc_doc_scores(int32_t T, const uint16_t* qr, const uint16_t* krbar,
                    const int64_t* doc_blk_off, int32_t n_docs, double* S)
{
    for (int32_t d = 0; d < n_docs; ++d) {
        double best = -INFINITY;
        for (int64_t b = doc_blk_off[d]; b < doc_blk_off[d + 1]; ++b)
            for (int32_t t = 0; t < T; ++t) {
                double s = orc_block_score(qr + (size_t)t * ORC_ROW, krbar + (size_t)b * ORC_ROW);
                if (s > best) best = s;
            }
        S[d] = best;
    }
}

/* ------------------------------------------------- threaded drivers (no arithmetic)
 * The documents are cut into contiguous ranges of about equal work and each
 * thread runs the unchanged single-threaded function on one range.  Offsets are
 * absolute indices into the row arrays, so a range is the same call on a slice of
 * the offset table; every output value is produced by the same code, in the same
 * operation order, as in one single-threaded call. */

typedef struct {
    int kind;                                   /* 0: doc scores, 1: pooling */
    int32_t T, n_layers, n_docs;
    const uint16_t *qr, *krbar, *x;
    int64_t n_tok, n_blk;
    const int64_t *doc_tok_off, *doc_blk_off;   /* already offset to the range's first doc */
    double* S;
    uint16_t* xbar;
} orc_range;

static void* orc_run_range(void* arg)
{
    orc_range* r = (orc_range*)arg;
    if (r->n_docs <= 0) return NULL;
    if (r->kind == 0)
        orc_doc_scores(r->T, r->qr, r->krbar, r->doc_blk_off, r->n_docs, r->S);
    else
        orc_pool(r->n_layers, r->x, r->n_tok, r->doc_tok_off, r->doc_blk_off, r->n_docs, r->n_blk, r->xbar);
    return NULL;
}

/* First document of range i of n when work[d] = off[d+1] - off[d] is split evenly. */
static int32_t orc_range_start(const int64_t* off, int32_t n_docs, int32_t i, int32_t n)
{
    if (i <= 0) return 0;
    if (i >= n) return n_docs;
    int64_t target = off[0] + (int64_t)((double)(off[n_docs] - off[0]) * i / n);
    int32_t lo = 0, hi = n_docs;                 /* first d with off[d] >= target */
    while (lo < hi) {
        int32_t mid = lo + (hi - lo) / 2;
        if (off[mid] < target) lo = mid + 1; else hi = mid;
    }
    return lo;
}

static void orc_run_ranges(orc_range base, const int64_t* split_off, int32_t n_docs, int32_t n_threads)
{
    if (n_threads < 1) n_threads = 1;
    if (n_threads > 256) n_threads = 256;
    orc_range rs[256];
    pthread_t th[256];
    int started[256];
    for (int32_t i = 0; i < n_threads; ++i) {
        int32_t d0 = orc_range_start(split_off, n_docs, i, n_threads);
        int32_t d1 = orc_range_start(split_off, n_docs, i + 1, n_threads);
        rs[i] = base;
        rs[i].n_docs = d1 - d0;
        rs[i].doc_blk_off = base.doc_blk_off + d0;
        if (base.doc_tok_off) rs[i].doc_tok_off = base.doc_tok_off + d0;
        if (base.S) rs[i].S = base.S + d0;
        started[i] = i > 0 && pthread_create(&th[i], NULL, orc_run_range, &rs[i]) == 0;
        if (i > 0 && !started[i]) orc_run_range(&rs[i]);   /* no thread: run it here */
    }
    orc_run_range(&rs[0]);
    for (int32_t i = 1; i < n_threads; ++i)
        if (started[i]) pthread_join(th[i], NULL);
}

void orc_doc_scores_mt(int32_t T, const uint16_t* qr, const uint16_t* krbar,
                       const int64_t* doc_blk_off, int32_t n_docs, double* S, int32_t n_threads)
{
    orc_range b;
    memset(&b, 0, sizeof b);
    b.kind = 0;
    b.T = T;
    b.qr = qr;
    b.krbar = krbar;
    b.doc_blk_off = doc_blk_off;
    b.S = S;
    orc_run_ranges(b, doc_blk_off, n_docs, n_threads);
}

void orc_pool_mt(int32_t n_layers, const uint16_t* x, int64_t n_tok,
                 const int64_t* doc_tok_off, const int64_t* doc_blk_off, int32_t n_docs,
                 int64_t n_blk, uint16_t* xbar, int32_t n_threads)
{
    orc_range b;
    memset(&b, 0, sizeof b);
    b.kind = 1;
    b.n_layers = n_layers;
    b.x = x;
    b.n_tok = n_tok;
    b.n_blk = n_blk;
    b.doc_tok_off = doc_tok_off;
    b.doc_blk_off = doc_blk_off;
    b.xbar = xbar;
    orc_run_ranges(b, doc_tok_off, n_docs, n_threads);
}

/* ------------------------------------------------------------------ top-k */

typedef struct { double s; int32_t id; } scored;

static int by_score_desc_id_asc(const void* pa, const void* pb)
{
    const scored* a = (const scored*)pa;
    const scored* b = (const scored*)pb;
    if (a->s > b->s) return -1;
    if (a->s < b->s) return 1;
    return (a->id > b->id) - (a->id < b->id);
}

void orc_topk(const double* S, int32_t n_docs, int32_t k, int32_t* ids, double* scores)
{
    scored* all = (scored*)malloc((size_t)(n_docs > 0 ? n_docs : 1) * sizeof(scored));
    for (int32_t d = 0; d < n_docs; ++d) { all[d].s = S[d]; all[d].id = d; }
    qsort(all, (size_t)n_docs, sizeof(scored), by_score_desc_id_asc);
    for (int32_t j = 0; j < k; ++j) { ids[j] = all[j].id; scores[j] = all[j].s; }
    free(all);
}

/* ----------------------------------------------------------------- gather */

int64_t orc_gather(const int32_t* ids, int32_t k, const int64_t* doc_blk_off,
                   const uint16_t* kbar, const uint16_t* vbar,
                   uint16_t* ctx_k, uint16_t* ctx_v)
{
    int64_t r = 0;
    for (int32_t j = 0; j < k; ++j) {
        int32_t d = ids[j];
        for (int64_t b = doc_blk_off[d]; b < doc_blk_off[d + 1]; ++b, ++r) {
            memcpy(ctx_k + (size_t)r * ORC_ROW, kbar + (size_t)b * ORC_ROW, ORC_ROW * sizeof(uint16_t));
            memcpy(ctx_v + (size_t)r * ORC_ROW, vbar + (size_t)b * ORC_ROW, ORC_ROW * sizeof(uint16_t));
        }
    }
    return r;
}

/* ----------------------------------------------------------------- decode */

void orc_decode(int32_t Hq, const uint16_t* q,
                const uint16_t* ctx_k, const uint16_t* ctx_v, int64_t n_ctx,
                const uint16_t* loc_k, const uint16_t* loc_v, int64_t n_loc,
                double scale, double* out)
{
    int32_t group = Hq / ORC_H;
    int64_t n = n_ctx + n_loc;
    double* s = (double*)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
    for (int32_t hq = 0; hq < Hq; ++hq) {
        int32_t g = hq / group;
        const uint16_t* qh = q + (size_t)hq * ORC_D;
        double* o = out + (size_t)hq * ORC_D;
        for (int i = 0; i < ORC_D; ++i) o[i] = 0.0;
        if (n == 0) continue;
        /* pass 1: scores and their maximum */
        double m = -INFINITY;
        for (int64_t j = 0; j < n; ++j) {
            const uint16_t* kr = j < n_ctx ? ctx_k + (size_t)j * ORC_ROW
                                           : loc_k + (size_t)(j - n_ctx) * ORC_ROW;
            double dot = 0.0;
            for (int i = 0; i < ORC_D; ++i)
                dot += orc_bf16_to_double(qh[i]) * orc_bf16_to_double(kr[g * ORC_D + i]);
            s[j] = scale * dot;
            if (s[j] > m) m = s[j];
        }
        /* pass 2: normaliser and weighted values */
        double z = 0.0;
        for (int64_t j = 0; j < n; ++j) {
            const uint16_t* vr = j < n_ctx ? ctx_v + (size_t)j * ORC_ROW
                                           : loc_v + (size_t)(j - n_ctx) * ORC_ROW;
            double w = exp(s[j] - m);
            z += w;
            for (int i = 0; i < ORC_D; ++i) o[i] += w * orc_bf16_to_double(vr[g * ORC_D + i]);
        }
        for (int i = 0; i < ORC_D; ++i) o[i] /= z;
    }
    free(s);
}

/* ---------------------------------------------------------------- prefill */

void orc_prefill(int32_t T, int32_t Hq, const uint16_t* q,
                 const uint16_t* ctx_k, const uint16_t* ctx_v, int64_t n_ctx,
                 const uint16_t* loc_k, const uint16_t* loc_v, int64_t n_loc,
                 double scale, double* out)
{
    for (int32_t t = 0; t < T; ++t) {
        /* local rows visible to token t: 0 .. n_loc - T + t */
        int64_t vis = n_loc - T + t + 1;
        if (vis < 0) vis = 0;
        if (vis > n_loc) vis = n_loc;
        orc_decode(Hq, q + (size_t)t * Hq * ORC_D, ctx_k, ctx_v, n_ctx, loc_k, loc_v, vis, scale,
                   out + (size_t)t * Hq * ORC_D);
    }
}

/* ----------------------------------------------------------------- encode */

void orc_encode(int32_t H, const uint16_t* x, int64_t n_tok,
                const uint16_t* w_k, const uint16_t* w_v, const uint16_t* w_kr, const uint16_t* w_norm,
                double eps, double theta,
                const int64_t* doc_tok_off, const int64_t* doc_blk_off, int32_t n_docs, int64_t n_blk,
                uint16_t* kbar, uint16_t* vbar, uint16_t* krbar)
{
    double* k = (double*)malloc(ORC_ROW * sizeof(double));
    double* v = (double*)malloc(ORC_ROW * sizeof(double));
    double* r = (double*)malloc(ORC_ROW * sizeof(double));
    double* sk = (double*)malloc(ORC_ROW * sizeof(double));
    double* sv = (double*)malloc(ORC_ROW * sizeof(double));
    double* sr = (double*)malloc(ORC_ROW * sizeof(double));
    (void)n_tok;
    (void)n_blk;
    for (int32_t d = 0; d < n_docs; ++d) {
        int64_t s = doc_tok_off[d], e = doc_tok_off[d + 1];
        for (int64_t j = 0; doc_blk_off[d] + j < doc_blk_off[d + 1]; ++j) {
            int64_t t0 = s + ORC_BLOCK * j;
            int64_t t1 = t0 + ORC_BLOCK < e ? t0 + ORC_BLOCK : e;
            for (int c = 0; c < ORC_ROW; ++c) sk[c] = sv[c] = sr[c] = 0.0;
            for (int64_t t = t0; t < t1; ++t) {
                const uint16_t* xt = x + (size_t)t * H;
                /* the three projections */
                for (int c = 0; c < ORC_ROW; ++c) k[c] = v[c] = r[c] = 0.0;
                for (int32_t i = 0; i < H; ++i) {
                    double xi = orc_bf16_to_double(xt[i]);
                    if (xi == 0.0) continue;
                    const uint16_t* wk = w_k + (size_t)i * ORC_ROW;
                    const uint16_t* wv = w_v + (size_t)i * ORC_ROW;
                    const uint16_t* wr = w_kr + (size_t)i * ORC_ROW;
                    for (int c = 0; c < ORC_ROW; ++c) {
                        k[c] += xi * orc_bf16_to_double(wk[c]);
                        v[c] += xi * orc_bf16_to_double(wv[c]);
                        r[c] += xi * orc_bf16_to_double(wr[c]);
                    }
                }
                /* key: per-head RMS normalisation, then the document-wise rotation */
                double p = (double)(t - s);
                for (int h = 0; h < ORC_H; ++h) {
                    double* kh = k + h * ORC_D;
                    double ms = 0.0;
                    for (int i = 0; i < ORC_D; ++i) ms += kh[i] * kh[i];
                    double inv = 1.0 / sqrt(ms / ORC_D + eps);
                    for (int i = 0; i < ORC_D; ++i) kh[i] *= inv * orc_bf16_to_double(w_norm[i]);
                    for (int i = 0; i < ORC_D / 2; ++i) {
                        double ang = p * pow(theta, -(double)i / (ORC_D / 2));
                        double c0 = cos(ang), s0 = sin(ang);
                        double a = kh[i], b = kh[i + ORC_D / 2];
                        kh[i] = a * c0 - b * s0;
                        kh[i + ORC_D / 2] = b * c0 + a * s0;
                    }
                }
                for (int c = 0; c < ORC_ROW; ++c) {
                    sk[c] += k[c];
                    sv[c] += v[c];
                    sr[c] += r[c];
                }
            }
            size_t o = (size_t)(doc_blk_off[d] + j) * ORC_ROW;
            double n = (double)(t1 - t0);
            for (int c = 0; c < ORC_ROW; ++c) {
                kbar[o + c] = orc_bf16_from_double(sk[c] / n);
                vbar[o + c] = orc_bf16_from_double(sv[c] / n);
                krbar[o + c] = orc_bf16_from_double(sr[c] / n);
            }
        }
    }
    free(k); free(v); free(r); free(sk); free(sv); free(sr);
}

