/*
 * sv_oracle.c — plain, slow, fp64 CPU definition of the speculative-sampling
 * verify step.  TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the
 * benchmark's CPU-baseline leg call it; the GPU library never does, and the
 * two share no code, header, table or helper.
 *
 * Sources (web pages, cited by title and section):
 *   [OPTIQ]  deniz.in, "Üç düzeltmeden sonra Qwen3.5 ve Qwen3.6 MTP head,
 *            Apple Silicon'da 1.4 kata ulaştı"
 *              - section "Örnekleme altında doğrulama yanlıştı"
 *                (greedy check against the target argmax; rejection sampling
 *                with acceptance min(1, p/q) and a fresh draw from the clipped,
 *                rescaled difference of the two distributions on rejection)
 *              - section "Kesme her iki tarafta eşleşmek zorunda"
 *                (both distributions get the same top_k / top_p truncation)
 *   [MTPLX]  text-matrix.pages.dev, "MTPLX：让模型用上自己的 MTP 头——Apple
 *            Silicon 上的原生投机解码", section 3.3 (精确拒绝采样): accept with
 *            min(1, p/q), otherwise sample (p-q)+; output law equals plain
 *            decoding from the target.
 *   [TINYCTO] tinycto.tv, "Spekülatif Kod Çözme (Speculative Decoding): Taslak
 *            Modeller, VRAM Yönetimi ve 3 Kat Çıkarım Hızı", section
 *            "1. Temel Çalışma Mekanizması": drafts are tested in order, the
 *            first rejection resamples from (p-q)+ and cancels the rest.
 *
 * Where the pages leave a step open, this file takes these readings (each is
 * restated next to the code that uses it):
 *   R1  order of operations: temperature, then top_k, then renormalise, then
 *       the top_p walk over the renormalised top_k, then renormalise again.
 *   R2  ranking key: logit descending, token id ascending (raw logits).
 *   R3  the top_p walk keeps a token iff the mass strictly before it is
 *       < top_p; the token that crosses the threshold is kept; top_p >= 1
 *       disables the cut.
 *   R4  top_k <= 0 or top_k >= V disables top_k.
 *   R5  T == 0 is a greedy row (argmax compare, lowest id on ties).
 *   R6  q(x) == 0: accept iff p(x) > 0.
 *   R7  accept iff u < a (strict), u in [0, 1).
 *   R8  uniforms[b][k] for the accept test at draft position k (0-based),
 *       uniforms[b][K] for the single final draw (residual or bonus).
 *   R9  inverse CDF in ascending token id; returns the first id with
 *       w > 0 and u*W < running sum.
 *   R10 residual mass W <= 0 falls back to sampling p.
 *   R11 bonus token: when every draft is accepted, draw from the target row at
 *       position L (0-based), i.e. one past the last draft.
 *   R12 rows are ragged: positions at or after draft_len are never read.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Per-row sampler parameters as laid out in memory (16 bytes). */
typedef struct {
    float temperature;
    int32_t top_k;
    float top_p;
    int32_t reserved;
} or_params;

typedef struct {
    double logit;
    int32_t id;
} or_item;

/* Exact widening of one stored logit to fp64.  dtype 0 = fp32, 1 = bf16. */
static double or_load(const void* base, int dtype, size_t idx) {
    if (dtype == 0) return (double)((const float*)base)[idx];
    uint32_t bits = (uint32_t)((const uint16_t*)base)[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* R2: better = higher logit, then lower id. qsort puts better first. */
static int or_cmp(const void* a, const void* b) {
    const or_item* x = (const or_item*)a;
    const or_item* y = (const or_item*)b;
    if (x->logit > y->logit) return -1;
    if (x->logit < y->logit) return 1;
    return (x->id < y->id) ? -1 : (x->id > y->id);
}

/*
 * The truncated, tempered distribution of one logits row (R1-R4), written
 * into prob[0..V-1] (zero outside the kept set).  Returns 0, or -1 when the
 * row has no finite logit.  *cut_margin receives the distance of the top_p
 * walk's two closest decisions to top_p (+inf when no cut is applied).
 * [OPTIQ] "Kesme her iki tarafta eşleşmek zorunda": the same top_k and top_p
 * are applied to target and draft alike; each keeps its own set.
 */
static int or_dist(const double* logit, int V, double T, int top_k, double top_p,
                   or_item* items, double* w, double* prob, double* cut_margin) {
    *cut_margin = INFINITY;
    for (int i = 0; i < V; i++) {
        items[i].logit = logit[i];
        items[i].id = i;
    }
    qsort(items, (size_t)V, sizeof(or_item), or_cmp);
    const double lmax = items[0].logit;
    if (!(lmax > -INFINITY)) return -1;

    int n = V; /* R4 */
    if (top_k > 0 && top_k < V) n = top_k;

    double zk = 0.0;
    for (int j = 0; j < n; j++) {
        w[j] = exp((items[j].logit - lmax) / T);
        zk += w[j];
    }

    int keep = n;
    if (top_p < 1.0) { /* R3 */
        double cum = 0.0;
        keep = 0;
        double last_kept_before = 0.0;
        while (keep < n && cum < top_p) {
            last_kept_before = cum;
            cum += w[keep] / zk;
            keep++;
        }
        double m = top_p - last_kept_before;
        if (keep < n) {
            double d = cum - top_p;
            if (d < m) m = d;
        }
        *cut_margin = m;
    }

    double zs = 0.0;
    for (int j = 0; j < keep; j++) zs += w[j];
    for (int i = 0; i < V; i++) prob[i] = 0.0;
    for (int j = 0; j < keep; j++) prob[items[j].id] = w[j] / zs;
    return 0;
}

/*
 * R9: inverse CDF in ascending id order.  Returns the token and writes the
 * chosen bin's lower/upper edges (as fractions of the total) and the margin
 * of u to the nearer edge.
 */
static int or_invcdf(const double* wgt, int V, double u, double* lo, double* hi,
                     double* margin) {
    double W = 0.0;
    for (int i = 0; i < V; i++) W += wgt[i];
    const double target = u * W;
    double S = 0.0;
    int last_pos = -1;
    double last_before = 0.0;
    for (int i = 0; i < V; i++) {
        if (!(wgt[i] > 0.0)) continue;
        double before = S;
        S += wgt[i];
        last_pos = i;
        last_before = before;
        if (target < S) {
            *lo = before / W;
            *hi = S / W;
            double a = u - *lo, b = *hi - u;
            *margin = a < b ? a : b;
            return i;
        }
    }
    /* Not reachable for u in [0, 1); kept so the function is total. */
    *lo = last_before / W;
    *hi = 1.0;
    *margin = 0.0;
    return last_pos;
}

static int or_argmax(const double* logit, int V) {
    int best = 0;
    for (int i = 1; i < V; i++)
        if (logit[i] > logit[best]) best = i;
    return best;
}

typedef struct {
    double* logit;
    or_item* items;
    double* w;
    double* p;
    double* q;
    double* r;
} or_scratch;

static void or_load_row(const void* base, int dtype, size_t row_off, int V, double* out) {
    for (int i = 0; i < V; i++) out[i] = or_load(base, dtype, row_off + (size_t)i);
}

static void or_fill_nan(double* d, int n) {
    for (int i = 0; i < n; i++) d[i] = NAN;
}

/*
 * One row of the verify step.  Returns the accept length, or -1 for a row
 * whose inputs are invalid (then every output token is -1).
 */
static int or_verify_row(const void* target, const void* draft, int dtype, int K, int V,
                         int64_t t_stride, int64_t d_stride, int b,
                         const int32_t* tokens, int L, const or_params* prm,
                         const float* u, int32_t* out_tok, double* diag,
                         double* cut_margin_out, or_scratch* s) {
    for (int k = 0; k <= K; k++) out_tok[k] = -1;
    if (diag) or_fill_nan(diag, 4 * (K + 1));
    *cut_margin_out = INFINITY;

    const double T = (double)prm->temperature;
    const double top_p = (double)prm->top_p;
    if (!(T >= 0.0) || !(T < INFINITY)) return -1;
    if (!(top_p > 0.0)) return -1;
    if (L < 0 || L > K) return -1;
    for (int k = 0; k < L; k++)
        if (tokens[k] < 0 || tokens[k] >= V) return -1;

    const size_t trow0 = (size_t)b * (size_t)(K + 1);
    const size_t drow0 = (size_t)b * (size_t)K;

    /* R5 and [OPTIQ] "Örnekleme altında doğrulama yanlıştı": a greedy row
     * accepts a draft iff it equals the target argmax at that position. */
    if (T == 0.0) {
        for (int k = 0; k <= L; k++) {
            or_load_row(target, dtype, (trow0 + (size_t)k) * (size_t)t_stride, V, s->logit);
            int g = or_argmax(s->logit, V);
            if (k == L || tokens[k] != g) {
                for (int j = 0; j < k; j++) out_tok[j] = tokens[j];
                out_tok[k] = g;
                return k;
            }
        }
        return -1; /* unreachable */
    }

    for (int k = 0; k <= L; k++) {
        double cm;
        or_load_row(target, dtype, (trow0 + (size_t)k) * (size_t)t_stride, V, s->logit);
        if (or_dist(s->logit, V, T, prm->top_k, top_p, s->items, s->w, s->p, &cm) != 0)
            return -1;
        if (cm < *cut_margin_out) *cut_margin_out = cm;

        if (k == L) {
            /* R11: every draft accepted -> bonus draw from p at position L. */
            double lo, hi, mg;
            int y = or_invcdf(s->p, V, (double)u[K], &lo, &hi, &mg);
            for (int j = 0; j < k; j++) out_tok[j] = tokens[j];
            out_tok[k] = y;
            if (diag) {
                diag[4 * K + 0] = s->p[y];
                diag[4 * K + 1] = lo;
                diag[4 * K + 2] = hi;
                diag[4 * K + 3] = mg;
            }
            return k;
        }

        or_load_row(draft, dtype, (drow0 + (size_t)k) * (size_t)d_stride, V, s->logit);
        if (or_dist(s->logit, V, T, prm->top_k, top_p, s->items, s->w, s->q, &cm) != 0)
            return -1;
        if (cm < *cut_margin_out) *cut_margin_out = cm;

        /* [MTPLX] 3.3 / [TINYCTO] mechanism: accept with min(1, p/q). R6, R7. */
        const int x = tokens[k];
        const double px = s->p[x], qx = s->q[x];
        double a;
        if (qx > 0.0) {
            a = px / qx;
            if (a > 1.0) a = 1.0;
        } else {
            a = (px > 0.0) ? 1.0 : 0.0;
        }
        const double uk = (double)u[k];
        if (diag) {
            diag[4 * k + 0] = px;
            diag[4 * k + 1] = qx;
            diag[4 * k + 2] = a;
            diag[4 * k + 3] = fabs(uk - a);
        }
        if (uk < a) continue;

        /* Rejection: resample from the normalised (p - q)+ (R9, R10) and
         * drop the remaining drafts. */
        double W = 0.0;
        for (int i = 0; i < V; i++) {
            double d = s->p[i] - s->q[i];
            s->r[i] = d > 0.0 ? d : 0.0;
            W += s->r[i];
        }
        const double* wgt = (W > 0.0) ? s->r : s->p;
        double lo, hi, mg;
        int y = or_invcdf(wgt, V, (double)u[K], &lo, &hi, &mg);
        for (int j = 0; j < k; j++) out_tok[j] = tokens[j];
        out_tok[k] = y;
        if (diag) {
            double Wn = 0.0;
            for (int i = 0; i < V; i++) Wn += wgt[i];
            diag[4 * K + 0] = wgt[y] / Wn;
            diag[4 * K + 1] = lo;
            diag[4 * K + 2] = hi;
            diag[4 * K + 3] = mg;
        }
        return k;
    }
    return -1; /* unreachable */
}

/*
 * Batch entry point (host pointers).
 *   target  [B][K+1] rows of V logits, row r at r * t_stride elements
 *   draft   [B][K]   rows of V logits, row r at r * d_stride elements
 *   dtype   0 = fp32, 1 = bf16 (raw 16-bit patterns)
 *   tokens  [B][K] int32; draft_len [B] int32 or NULL (= K for every row)
 *   params  [B] or_params; uniforms [B][K+1] fp32 in [0, 1)
 *   out_tokens [B][K+1] (-1 padded), out_accept_len [B] (-1 = invalid row)
 *   diag [B][K+1][4] fp64 or NULL: slots 0..K-1 = (p(x), q(x), a, |u - a|)
 *        for evaluated accept tests; slot K = (probability of the drawn token
 *        under the final distribution, bin lower edge, bin upper edge, margin
 *        of u to the nearer edge).  NaN where nothing was evaluated.
 *   cut_margin [B] fp64 or NULL: smallest top_p walk margin of the row.
 *   nthreads: OpenMP threads (<= 0: runtime default).
 * Returns the number of threads used, or -1 on a null required pointer.
 */
int sv_oracle_verify(const void* target, const void* draft, int dtype, int B, int K, int V,
                     int64_t t_stride, int64_t d_stride, const int32_t* tokens,
                     const int32_t* draft_len, const void* params, const float* uniforms,
                     int32_t* out_tokens, int32_t* out_accept_len, double* diag,
                     double* cut_margin, int nthreads) {
    if (!target || !tokens || !params || !uniforms || !out_tokens || !out_accept_len) return -1;
    if (K > 0 && !draft) return -1;
    if (B <= 0 || K < 0 || V < 1) return -1;
    if (t_stride < V || (K > 0 && d_stride < V)) return -1;
    const or_params* prm = (const or_params*)params;
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
        or_scratch s;
        s.logit = (double*)malloc(sizeof(double) * (size_t)V);
        s.items = (or_item*)malloc(sizeof(or_item) * (size_t)V);
        s.w = (double*)malloc(sizeof(double) * (size_t)V);
        s.p = (double*)malloc(sizeof(double) * (size_t)V);
        s.q = (double*)malloc(sizeof(double) * (size_t)V);
        s.r = (double*)malloc(sizeof(double) * (size_t)V);
#pragma omp for schedule(dynamic, 1)
        for (int b = 0; b < B; b++) {
            int L = draft_len ? draft_len[b] : K;
            double cm;
            int a = or_verify_row(target, draft, dtype, K, V, t_stride, d_stride, b,
                                  tokens + (size_t)b * (size_t)K, L, prm + b,
                                  uniforms + (size_t)b * (size_t)(K + 1),
                                  out_tokens + (size_t)b * (size_t)(K + 1),
                                  diag ? diag + (size_t)b * 4 * (size_t)(K + 1) : NULL, &cm, &s);
            if (a < 0) {
                for (int k = 0; k <= K; k++) out_tokens[(size_t)b * (size_t)(K + 1) + k] = -1;
                if (diag) or_fill_nan(diag + (size_t)b * 4 * (size_t)(K + 1), 4 * (K + 1));
            }
            out_accept_len[b] = a;
            if (cut_margin) cut_margin[b] = cm;
        }
        free(s.logit);
        free(s.items);
        free(s.w);
        free(s.p);
        free(s.q);
        free(s.r);
    }
    return used;
}

/* The truncated distribution of one fp64 logits row (tests use it to draw
 * draft tokens from q and to state closed forms).  Returns 0 or -1. */
int sv_oracle_dist(const double* logit, int V, double T, int top_k, double top_p,
                   double* prob, double* cut_margin) {
    if (!logit || !prob || V < 1 || !(T > 0.0)) return -1;
    or_item* items = (or_item*)malloc(sizeof(or_item) * (size_t)V);
    double* w = (double*)malloc(sizeof(double) * (size_t)V);
    double cm;
    int rc = or_dist(logit, V, T, top_k, top_p, items, w, prob, &cm);
    if (cut_margin) *cut_margin = cm;
    free(items);
    free(w);
    return rc;
}

/*
 * The decisions the verify rule takes along one given outcome of a row, for
 * judging an outcome that differs from the oracle's own: does some uniform
 * vector within a small distance of the given one lead the rule to it?
 * The outcome is an accept length acc in [0, L] and a final token y.  Along
 * it, for j = 0 .. min(acc, L - 1): a_out[j], px_out[j], qx_out[j] are the
 * accept probability min(1, p_j(x_j) / q_j(x_j)) (R6 for q = 0) and its two
 * probabilities (the outcome accepts draft j for j < acc and rejects draft
 * acc when acc < L).  The final distribution is the residual (p - q)+ at acc
 * (R10: p itself when its mass is 0) when acc < L, p at position L (R11)
 * otherwise; *lo and *hi are the edges of y's bin of its inverse CDF in
 * ascending id order (R9), as fractions of its total, and *py the probability
 * of y under it (0 when y carries no weight).  Slots past the path are NaN.
 * Returns 0, 1 for a greedy row (T = 0: no uniform takes part, nothing to
 * explain), -1 for an invalid row or an outcome outside [0, L] x [0, V).
 * [OPTIQ] "Örnekleme altında doğrulama yanlıştı", [MTPLX] 3.3: the same
 * accept test and residual as or_verify_row, evaluated on a forced path.
 */
static int or_explain_row(const void* target, const void* draft, int dtype, int K, int V,
                          int64_t t_stride, int64_t d_stride, int b, const int32_t* tokens,
                          int L, const or_params* prm, int acc, int y, double* a_out,
                          double* px_out, double* qx_out, double* lo, double* hi, double* py,
                          or_scratch* s) {
    or_fill_nan(a_out, K);
    or_fill_nan(px_out, K);
    or_fill_nan(qx_out, K);
    *lo = *hi = *py = NAN;
    const double T = (double)prm->temperature;
    const double top_p = (double)prm->top_p;
    if (!(T >= 0.0) || !(T < INFINITY) || !(top_p > 0.0) || L < 0 || L > K) return -1;
    for (int k = 0; k < L; k++)
        if (tokens[k] < 0 || tokens[k] >= V) return -1;
    if (T == 0.0) return 1;
    if (acc < 0 || acc > L || y < 0 || y >= V) return -1;
    const size_t trow0 = (size_t)b * (size_t)(K + 1);
    const size_t drow0 = (size_t)b * (size_t)K;
    const int last = acc < L ? acc : L - 1;
    double cm;
    for (int k = 0; k <= last; k++) {
        or_load_row(target, dtype, (trow0 + (size_t)k) * (size_t)t_stride, V, s->logit);
        if (or_dist(s->logit, V, T, prm->top_k, top_p, s->items, s->w, s->p, &cm) != 0)
            return -1;
        or_load_row(draft, dtype, (drow0 + (size_t)k) * (size_t)d_stride, V, s->logit);
        if (or_dist(s->logit, V, T, prm->top_k, top_p, s->items, s->w, s->q, &cm) != 0)
            return -1;
        const int x = tokens[k];
        const double px = s->p[x], qx = s->q[x];
        double a;
        if (qx > 0.0) {
            a = px / qx;
            if (a > 1.0) a = 1.0;
        } else {
            a = (px > 0.0) ? 1.0 : 0.0;
        }
        a_out[k] = a;
        px_out[k] = px;
        qx_out[k] = qx;
    }
    const double* wgt;
    if (acc < L) {
        /* s->p and s->q hold position acc (the last one evaluated above) */
        double W = 0.0;
        for (int i = 0; i < V; i++) {
            double d = s->p[i] - s->q[i];
            s->r[i] = d > 0.0 ? d : 0.0;
            W += s->r[i];
        }
        wgt = (W > 0.0) ? s->r : s->p;
    } else {
        or_load_row(target, dtype, (trow0 + (size_t)L) * (size_t)t_stride, V, s->logit);
        if (or_dist(s->logit, V, T, prm->top_k, top_p, s->items, s->w, s->p, &cm) != 0)
            return -1;
        wgt = s->p;
    }
    double W = 0.0, before = 0.0;
    for (int i = 0; i < V; i++) {
        if (i == y) before = W;
        W += wgt[i];
    }
    *lo = before / W;
    *hi = (before + wgt[y]) / W;
    *py = wgt[y] / W;
    return 0;
}

/*
 * Batch form of or_explain_row over rows laid out as for sv_oracle_verify
 * (K = 0 allowed: draft may then be NULL and the outcome is the one draw).
 * acc [B], y [B]: the outcomes to explain; a_out, px_out, qx_out [B][K];
 * lo, hi, py [B]; status [B] (the row's return code).  Returns the number of
 * threads used, or -1 on a null required pointer.
 */
int sv_oracle_explain(const void* target, const void* draft, int dtype, int B, int K, int V,
                      int64_t t_stride, int64_t d_stride, const int32_t* tokens,
                      const int32_t* draft_len, const void* params, const int32_t* acc,
                      const int32_t* y, double* a_out, double* px_out, double* qx_out,
                      double* lo, double* hi, double* py, int32_t* status, int nthreads) {
    if (!target || !tokens || !params || !acc || !y || !a_out || !px_out || !qx_out || !lo ||
        !hi || !py || !status)
        return -1;
    if (K > 0 && !draft) return -1;
    if (B <= 0 || K < 0 || V < 1 || t_stride < V || (K > 0 && d_stride < V)) return -1;
    const or_params* prm = (const or_params*)params;
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
        or_scratch s;
        s.logit = (double*)malloc(sizeof(double) * (size_t)V);
        s.items = (or_item*)malloc(sizeof(or_item) * (size_t)V);
        s.w = (double*)malloc(sizeof(double) * (size_t)V);
        s.p = (double*)malloc(sizeof(double) * (size_t)V);
        s.q = (double*)malloc(sizeof(double) * (size_t)V);
        s.r = (double*)malloc(sizeof(double) * (size_t)V);
#pragma omp for schedule(dynamic, 1)
        for (int b = 0; b < B; b++) {
            const int L = draft_len ? draft_len[b] : K;
            status[b] = or_explain_row(target, draft, dtype, K, V, t_stride, d_stride, b,
                                       tokens + (size_t)b * (size_t)K, L, prm + b, acc[b], y[b],
                                       a_out + (size_t)b * (size_t)K,
                                       px_out + (size_t)b * (size_t)K,
                                       qx_out + (size_t)b * (size_t)K, lo + b, hi + b, py + b,
                                       &s);
        }
        free(s.logit);
        free(s.items);
        free(s.w);
        free(s.p);
        free(s.q);
        free(s.r);
    }
    return used;
}

/* ---------------------------------------------------------------------------
 * Tree / multi-candidate verify.
 *
 * [TINYCTO], question "Medusa / Eagle spekülatif taslak mekanizması nedir?":
 * draft heads propose candidate tokens; the pages give no rule for checking
 * several candidates at one position.  This oracle takes the reading that
 * keeps the output law equal to the target's when the candidates at a node
 * are drawn independently from q at that node: recursive rejection.
 *   R17 nodes: node 0 is the committed context; node c >= 1 carries the
 *       candidate token tok[c-1], drawn at its parent par[c-1] < c.  Target
 *       row v is the target's logits after node v's path, draft row v
 *       (v < K) the draft's logits there (its children were drawn from it).
 *   R18 at node v the children c_1 < ... < c_m (ascending node index) are
 *       tested in turn against r, which starts as p_v: candidate x is
 *       accepted iff u[c-1] < min(1, r(x) / q_v(x)) (R6 for q_v(x) = 0);
 *       after a rejection r becomes (r - q_v)+ normalised (unchanged when
 *       that has no mass, R10).  An accepted child becomes v.
 *   R19 when every child of v is rejected, or v has none, the final token
 *       is drawn from r with uniform u[K] (R9): the residual after the
 *       rejections, p_v itself at a leaf (the bonus token, R11).
 *   R20 greedy rows accept the first child whose token is the argmax of
 *       target row v and otherwise emit that argmax.
 * With one child per node (par[c-1] = c-1) this is or_verify_row exactly.
 * ------------------------------------------------------------------------- */

/* Children of v among nodes 1..n-1, ascending; returns their number. */
static int or_children(const int32_t* par, int n, int v, int* out) {
    int m = 0;
    for (int c = v + 1; c < n; c++)
        if (par[c - 1] == v) out[m++] = c;
    return m;
}

static int or_tree_row(const void* target, const void* draft, int dtype, int K, int V,
                       int64_t t_stride, int64_t d_stride, int b, const int32_t* tok,
                       const int32_t* par, int n_cand, const or_params* prm, const float* u,
                       int32_t* out_tok, int32_t* out_path, double* diag, or_scratch* s,
                       int* kids) {
    for (int k = 0; k <= K; k++) out_tok[k] = -1;
    if (out_path)
        for (int k = 0; k <= K; k++) out_path[k] = -1;
    if (diag) or_fill_nan(diag, 4 * (K + 1));
    const double T = (double)prm->temperature;
    const double top_p = (double)prm->top_p;
    if (!(T >= 0.0) || !(T < INFINITY) || !(top_p > 0.0)) return -1;
    if (n_cand < 0 || n_cand > K) return -1;
    const int n = n_cand + 1;
    for (int c = 1; c < n; c++)
        if (par[c - 1] < 0 || par[c - 1] >= c || tok[c - 1] < 0 || tok[c - 1] >= V) return -1;
    const size_t trow0 = (size_t)b * (size_t)(K + 1);
    const size_t drow0 = (size_t)b * (size_t)K;
    int v = 0, depth = 0;
    for (;;) {
        const int m = or_children(par, n, v, kids);
        or_load_row(target, dtype, (trow0 + (size_t)v) * (size_t)t_stride, V, s->logit);
        if (T == 0.0) { /* R20 */
            const int g = or_argmax(s->logit, V);
            int next = -1;
            for (int i = 0; i < m && next < 0; i++)
                if (tok[kids[i] - 1] == g) next = kids[i];
            if (next < 0) {
                out_tok[depth] = g;
                return depth;
            }
            out_tok[depth] = g;
            if (out_path) out_path[depth] = next;
            depth++;
            v = next;
            continue;
        }
        double cm;
        if (or_dist(s->logit, V, T, prm->top_k, top_p, s->items, s->w, s->p, &cm) != 0) return -1;
        /* r = p_v, kept in s->r */
        for (int i = 0; i < V; i++) s->r[i] = s->p[i];
        int next = -1;
        if (m > 0) {
            or_load_row(draft, dtype, (drow0 + (size_t)v) * (size_t)d_stride, V, s->logit);
            if (or_dist(s->logit, V, T, prm->top_k, top_p, s->items, s->w, s->q, &cm) != 0)
                return -1;
            for (int i = 0; i < m && next < 0; i++) { /* R18 */
                const int c = kids[i];
                const int x = tok[c - 1];
                const double rx = s->r[x], qx = s->q[x];
                double a;
                if (qx > 0.0) {
                    a = rx / qx;
                    if (a > 1.0) a = 1.0;
                } else {
                    a = (rx > 0.0) ? 1.0 : 0.0;
                }
                const double uc = (double)u[c - 1];
                if (diag) {
                    diag[4 * (c - 1) + 0] = rx;
                    diag[4 * (c - 1) + 1] = qx;
                    diag[4 * (c - 1) + 2] = a;
                    diag[4 * (c - 1) + 3] = fabs(uc - a);
                }
                if (uc < a) {
                    next = c;
                    break;
                }
                double W = 0.0;
                for (int e = 0; e < V; e++) {
                    const double d = s->r[e] - s->q[e];
                    s->w[e] = d > 0.0 ? d : 0.0;
                    W += s->w[e];
                }
                if (W > 0.0)
                    for (int e = 0; e < V; e++) s->r[e] = s->w[e] / W;
            }
        }
        if (next >= 0) {
            out_tok[depth] = tok[next - 1];
            if (out_path) out_path[depth] = next;
            depth++;
            v = next;
            continue;
        }
        /* R19 */
        double lo, hi, mg;
        const int y = or_invcdf(s->r, V, (double)u[K], &lo, &hi, &mg);
        out_tok[depth] = y;
        if (diag) {
            double Wn = 0.0;
            for (int e = 0; e < V; e++) Wn += s->r[e];
            diag[4 * K + 0] = s->r[y] / Wn;
            diag[4 * K + 1] = lo;
            diag[4 * K + 2] = hi;
            diag[4 * K + 3] = mg;
        }
        return depth;
    }
}

/*
 * Batch entry point of the tree verify (host pointers), laid out like
 * sv_oracle_verify with K candidate nodes per row:
 *   target [B][K+1] rows (row v = node v), draft [B][K] rows (row v = node v,
 *   v < K); tok, par [B][K] (entry c-1 = node c); n_cand [B] in [0, K] or
 *   NULL (= K): nodes 1..n_cand are used; params [B]; uniforms [B][K+1]
 *   (column c-1 = the test of node c, column K = the final draw).
 *   out_tokens [B][K+1]: the accepted path's tokens, then the final token
 *   (the greedy argmax on greedy rows), then -1; out_len [B]: the accepted
 *   path's length (-1: invalid row); out_path [B][K+1] or NULL: the accepted
 *   nodes, -1 padded; diag [B][K+1][4] or NULL: slot c-1 = (r(x), q(x), a,
 *   |u - a|) of node c's test, slot K = the final draw as in
 *   sv_oracle_verify.
 * Returns the number of threads used, or -1 on a null required pointer.
 */
int sv_oracle_verify_tree(const void* target, const void* draft, int dtype, int B, int K, int V,
                          int64_t t_stride, int64_t d_stride, const int32_t* tok,
                          const int32_t* par, const int32_t* n_cand, const void* params,
                          const float* uniforms, int32_t* out_tokens, int32_t* out_len,
                          int32_t* out_path, double* diag, int nthreads) {
    if (!target || !tok || !par || !params || !uniforms || !out_tokens || !out_len) return -1;
    if (K > 0 && !draft) return -1;
    if (B <= 0 || K < 0 || V < 1 || t_stride < V || (K > 0 && d_stride < V)) return -1;
    const or_params* prm = (const or_params*)params;
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
        or_scratch s;
        s.logit = (double*)malloc(sizeof(double) * (size_t)V);
        s.items = (or_item*)malloc(sizeof(or_item) * (size_t)V);
        s.w = (double*)malloc(sizeof(double) * (size_t)V);
        s.p = (double*)malloc(sizeof(double) * (size_t)V);
        s.q = (double*)malloc(sizeof(double) * (size_t)V);
        s.r = (double*)malloc(sizeof(double) * (size_t)V);
        int* kids = (int*)malloc(sizeof(int) * (size_t)(K + 1));
#pragma omp for schedule(dynamic, 1)
        for (int b = 0; b < B; b++) {
            const int nc = n_cand ? n_cand[b] : K;
            int32_t* ot = out_tokens + (size_t)b * (size_t)(K + 1);
            int32_t* op = out_path ? out_path + (size_t)b * (size_t)(K + 1) : NULL;
            double* dg = diag ? diag + (size_t)b * 4 * (size_t)(K + 1) : NULL;
            const int d = or_tree_row(target, draft, dtype, K, V, t_stride, d_stride, b,
                                      tok + (size_t)b * (size_t)K, par + (size_t)b * (size_t)K,
                                      nc, prm + b, uniforms + (size_t)b * (size_t)(K + 1), ot, op,
                                      dg, &s, kids);
            if (d < 0) {
                for (int k = 0; k <= K; k++) ot[k] = -1;
                if (op)
                    for (int k = 0; k <= K; k++) op[k] = -1;
                if (dg) or_fill_nan(dg, 4 * (K + 1));
            }
            out_len[b] = d;
        }
        free(s.logit);
        free(s.items);
        free(s.w);
        free(s.p);
        free(s.q);
        free(s.r);
        free(kids);
    }
    return used;
}

/*
 * The tree rule's decisions along one given outcome (the tree counterpart of
 * or_explain_row): the accepted path path[0..len-1] (node indices) and the
 * final token y.  For every test the outcome implies, at node c: a_out[c-1]
 * = min(1, r(x)/q(x)) and need[c-1] = +1 (the outcome accepts c) or -1 (it
 * rejects c); need = 0 for nodes the outcome does not test.  *lo, *hi, *py:
 * y's bin in the final draw (R19) and its probability.  Returns 0, 1 for a
 * greedy row, -1 for an invalid row or an outcome that is not a path of
 * children from node 0.
 */
static int or_explain_tree_row(const void* target, const void* draft, int dtype, int K, int V,
                               int64_t t_stride, int64_t d_stride, int b, const int32_t* tok,
                               const int32_t* par, int n_cand, const or_params* prm,
                               const int32_t* path, int len, int y, double* a_out, int32_t* need,
                               double* lo, double* hi, double* py, or_scratch* s, int* kids) {
    or_fill_nan(a_out, K);
    for (int k = 0; k < K; k++) need[k] = 0;
    *lo = *hi = *py = NAN;
    const double T = (double)prm->temperature;
    const double top_p = (double)prm->top_p;
    if (!(T >= 0.0) || !(T < INFINITY) || !(top_p > 0.0)) return -1;
    if (n_cand < 0 || n_cand > K) return -1;
    const int n = n_cand + 1;
    for (int c = 1; c < n; c++)
        if (par[c - 1] < 0 || par[c - 1] >= c || tok[c - 1] < 0 || tok[c - 1] >= V) return -1;
    if (T == 0.0) return 1;
    if (len < 0 || len > K || y < 0 || y >= V) return -1;
    const size_t trow0 = (size_t)b * (size_t)(K + 1);
    const size_t drow0 = (size_t)b * (size_t)K;
    int v = 0;
    double cm;
    for (int d = 0; d <= len; d++) {
        const int m = or_children(par, n, v, kids);
        const int want = d < len ? path[d] : -1;
        or_load_row(target, dtype, (trow0 + (size_t)v) * (size_t)t_stride, V, s->logit);
        if (or_dist(s->logit, V, T, prm->top_k, top_p, s->items, s->w, s->p, &cm) != 0) return -1;
        for (int i = 0; i < V; i++) s->r[i] = s->p[i];
        int found = 0;
        if (m > 0) {
            or_load_row(draft, dtype, (drow0 + (size_t)v) * (size_t)d_stride, V, s->logit);
            if (or_dist(s->logit, V, T, prm->top_k, top_p, s->items, s->w, s->q, &cm) != 0)
                return -1;
            for (int i = 0; i < m; i++) {
                const int c = kids[i];
                const int x = tok[c - 1];
                const double rx = s->r[x], qx = s->q[x];
                double a;
                if (qx > 0.0) {
                    a = rx / qx;
                    if (a > 1.0) a = 1.0;
                } else {
                    a = (rx > 0.0) ? 1.0 : 0.0;
                }
                a_out[c - 1] = a;
                if (c == want) {
                    need[c - 1] = 1;
                    found = 1;
                    break;
                }
                need[c - 1] = -1;
                double W = 0.0;
                for (int e = 0; e < V; e++) {
                    const double dd = s->r[e] - s->q[e];
                    s->w[e] = dd > 0.0 ? dd : 0.0;
                    W += s->w[e];
                }
                if (W > 0.0)
                    for (int e = 0; e < V; e++) s->r[e] = s->w[e] / W;
            }
        }
        if (d < len) {
            if (!found) return -1;
            v = want;
            continue;
        }
        double W = 0.0, before = 0.0;
        for (int e = 0; e < V; e++) {
            if (e == y) before = W;
            W += s->r[e];
        }
        *lo = before / W;
        *hi = (before + s->r[y]) / W;
        *py = s->r[y] / W;
    }
    return 0;
}

/* Batch form: path [B][K+1] (the outcome's nodes, -1 padded), len [B], y [B];
 * a_out [B][K], need [B][K]; lo, hi, py [B]; status [B]. */
int sv_oracle_explain_tree(const void* target, const void* draft, int dtype, int B, int K, int V,
                           int64_t t_stride, int64_t d_stride, const int32_t* tok,
                           const int32_t* par, const int32_t* n_cand, const void* params,
                           const int32_t* path, const int32_t* len, const int32_t* y,
                           double* a_out, int32_t* need, double* lo, double* hi, double* py,
                           int32_t* status, int nthreads) {
    if (!target || !tok || !par || !params || !path || !len || !y || !a_out || !need || !lo ||
        !hi || !py || !status)
        return -1;
    if (K > 0 && !draft) return -1;
    if (B <= 0 || K < 0 || V < 1 || t_stride < V || (K > 0 && d_stride < V)) return -1;
    const or_params* prm = (const or_params*)params;
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
        or_scratch s;
        s.logit = (double*)malloc(sizeof(double) * (size_t)V);
        s.items = (or_item*)malloc(sizeof(or_item) * (size_t)V);
        s.w = (double*)malloc(sizeof(double) * (size_t)V);
        s.p = (double*)malloc(sizeof(double) * (size_t)V);
        s.q = (double*)malloc(sizeof(double) * (size_t)V);
        s.r = (double*)malloc(sizeof(double) * (size_t)V);
        int* kids = (int*)malloc(sizeof(int) * (size_t)(K + 1));
#pragma omp for schedule(dynamic, 1)
        for (int b = 0; b < B; b++) {
            const int nc = n_cand ? n_cand[b] : K;
            status[b] = or_explain_tree_row(
                target, draft, dtype, K, V, t_stride, d_stride, b, tok + (size_t)b * (size_t)K,
                par + (size_t)b * (size_t)K, nc, prm + b, path + (size_t)b * (size_t)(K + 1),
                len[b], y[b], a_out + (size_t)b * (size_t)K, need + (size_t)b * (size_t)K, lo + b,
                hi + b, py + b, &s, kids);
        }
        free(s.logit);
        free(s.items);
        free(s.w);
        free(s.p);
        free(s.q);
        free(s.r);
        free(kids);
    }
    return used;
}
