/*
 * Plain fp64 CPU oracle for causal grouped-query attention with rotary
 * position embedding.  TEST INFRASTRUCTURE ONLY: the tests, the smoke check
 * and the CPU-baseline leg of the benchmark call it; the library under test
 * never does.  It shares no source with the HIP path.
 *
 * Every function computes its result straight from the definition, one output
 * row at a time, in double precision, with no tiling, no online softmax and no
 * split of the key range.  Inputs may be given as fp64, fp32 or bf16 (raw
 * 16-bit patterns); every element is widened exactly to double before use.
 *
 * Sources (pages are cited by title and section):
 *  - "Grouped Query Attention (GQA)" (Ultralytics glossary), section
 *    "Cómo funciona GQA": each query head runs unchanged scaled dot-product
 *    attention against the one key/value head its group shares; the printed
 *    PyTorch example is causal and equals multi-head attention with every
 *    key/value head copied to the consecutive query heads of its group.
 *  - same page, section "Por qué GQA reduce la caché KV": during generation
 *    the whole cache of earlier keys/values is read for every new token.
 *  - "Compressed Convolutional Attention" (gist.science summary), section
 *    "Methodologie", item 4: RoPE is applied directly to the per-head q and k
 *    vectors of the (compressed) attention space.
 *  - "Latent-Condensed Transformer" (gist.science summary), section 2B: RoPE is
 *    a nonlinear function of the absolute token position.
 * The pages do not print the RoPE formula.  This oracle uses the original
 * rotary definition: channel pair (2i, 2i+1) is rotated by the angle
 * p * theta^(-2i/D), for absolute position p.
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp -shared -fPIC oracle.c -lm
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Element type of an input buffer. */
enum { OR_F64 = 0, OR_F32 = 1, OR_BF16 = 2 };

/* Widen element i of buffer p (element type dt) exactly to double. */
static double load(const void *p, size_t i, int dt)
{
    if (dt == OR_F64)
        return ((const double *)p)[i];
    if (dt == OR_F32)
        return (double)((const float *)p)[i];
    /* bf16: the 16 stored bits are the top half of an IEEE binary32. */
    uint32_t w = (uint32_t)((const uint16_t *)p)[i] << 16;
    float f;
    memcpy(&f, &w, sizeof f);
    return (double)f;
}

/* Threads an OpenMP parallel region of this library uses. */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------ */
/* Rounding to the storage types (models the dtype boundary between    */
/* separate library calls).                                            */
/* ------------------------------------------------------------------ */

/* Round a double to the nearest bf16 value, ties to even, returning the
 * 16-bit pattern.  bf16 has 8 significant bits and binary32's exponent
 * range, so a finite x is written as r * 2^k with k chosen so that r has 8
 * significant bits (or k = -133 in the subnormal range) and r is rounded to
 * an integer with rint() in the default round-to-nearest-even mode.  The
 * product r * 2^k is then exactly representable in binary32. */
static uint16_t round_bf16(double x)
{
    if (isnan(x))
        return 0x7fc0;
    float f;
    if (isinf(x)) {
        f = (float)x;
    } else if (x == 0.0) {
        f = (float)x; /* keeps the sign of zero */
    } else {
        int e;
        frexp(x, &e); /* |x| = m * 2^e, 0.5 <= m < 1 */
        int k = e - 8;
        if (k < -133)
            k = -133; /* bf16 subnormal spacing is 2^-133 */
        double r = rint(ldexp(x, -k));
        double y = ldexp(r, k);
        /* bf16 max finite is (2 - 2^-7) * 2^127 */
        if (fabs(y) >= 0x1p128)
            y = copysign(INFINITY, x);
        f = (float)y;
    }
    uint32_t w;
    memcpy(&w, &f, sizeof w);
    return (uint16_t)(w >> 16);
}

void oracle_round_bf16(uint16_t *out, const double *in, size_t n)
{
    for (size_t i = 0; i < n; ++i)
        out[i] = round_bf16(in[i]);
}

void oracle_round_f32(float *out, const double *in, size_t n)
{
    for (size_t i = 0; i < n; ++i)
        out[i] = (float)in[i]; /* C conversion rounds to nearest even */
}

/* ------------------------------------------------------------------ */
/* Rotary position embedding                                           */
/* ------------------------------------------------------------------ */

/* x: [B, H, S, D] (element type dt), out: [B, H, S, D] fp64.
 * Token s of sequence b sits at absolute position pos_offset[b] + s
 * (pos_offset may be NULL: all offsets zero).  For every head and every
 * channel pair i < D/2 the pair (x[2i], x[2i+1]) is rotated by the angle
 * p * theta^(-2i/D).  D must be even. */
void oracle_rope(double *out, const void *x, int dt, int B, int H, int S, int D,
                 const int32_t *pos_offset, double theta)
{
    /* rows are independent: one OpenMP iteration per (b, h, s) row */
#pragma omp parallel for schedule(static)
    for (long long flat = 0; flat < (long long)B * H * S; ++flat) {
        int s = (int)(flat % S);
        int b = (int)(flat / ((long long)S * H));
        long long off = pos_offset ? pos_offset[b] : 0;
        double p = (double)(off + s);
        size_t row = (size_t)flat * (size_t)D;
        for (int i = 0; i < D / 2; ++i) {
            double freq = pow(theta, -2.0 * i / D);
            double ang = p * freq;
            double c = cos(ang), sn = sin(ang);
            double x0 = load(x, row + 2 * i, dt);
            double x1 = load(x, row + 2 * i + 1, dt);
            out[row + 2 * i] = x0 * c - x1 * sn;
            out[row + 2 * i + 1] = x0 * sn + x1 * c;
        }
    }
}

/* Transpose of the rotary embedding, for gradients: the rotation of pair i at
 * position p is the 2x2 matrix [[cos a, -sin a], [sin a, cos a]] with
 * a = p * theta^(-2i/D); its transpose maps a gradient dy of the rotated pair
 * back to the gradient of the unrotated pair:
 *     out[2i] = dy[2i] cos a + dy[2i+1] sin a,
 *     out[2i+1] = -dy[2i] sin a + dy[2i+1] cos a.
 * Shapes and positions as oracle_rope. */
void oracle_rope_transpose(double *out, const void *dy, int dt, int B, int H, int S, int D,
                           const int32_t *pos_offset, double theta)
{
#pragma omp parallel for schedule(static)
    for (long long r = 0; r < (long long)B * H * S; ++r) {
        const int t = (int)(r % S);
        const int b = (int)(r / ((long long)S * H));
        const long long base = pos_offset ? pos_offset[b] : 0;
        const size_t at = (size_t)r * (size_t)D;
        for (int j = 0; j < D / 2; ++j) {
            const double a = (double)(base + t) * pow(theta, -(2.0 * j) / D);
            const double ca = cos(a), sa = sin(a);
            const double g0 = load(dy, at + 2 * j, dt), g1 = load(dy, at + 2 * j + 1, dt);
            out[at + 2 * j] = g0 * ca + g1 * sa;
            out[at + 2 * j + 1] = g1 * ca - g0 * sa;
        }
    }
}

/* ------------------------------------------------------------------ */
/* Attention                                                           */
/* ------------------------------------------------------------------ */

/* One output row of scaled dot-product attention, computed from the
 * definition:  s_t = scale * <q, k_t> for t in [0, n),  w_t = exp(s_t - max s),
 * o = sum_t w_t v_t / sum_t w_t.  Key/value rows are k_base + t*D and
 * v_base + t*D (element indices).  n == 0 gives a zero row.
 * w is caller-provided scratch of at least n doubles. */
static void attend_row(double *o, const void *q, size_t q_base, const void *k,
                       const void *v, size_t kv_base, int n, int D, int dt,
                       double scale, double *w)
{
    for (int d = 0; d < D; ++d)
        o[d] = 0.0;
    if (n <= 0)
        return;
    double m = -INFINITY;
    for (int t = 0; t < n; ++t) {
        double dot = 0.0;
        for (int d = 0; d < D; ++d)
            dot += load(q, q_base + d, dt) * load(k, kv_base + (size_t)t * D + d, dt);
        w[t] = scale * dot;
        if (w[t] > m)
            m = w[t];
    }
    double l = 0.0;
    for (int t = 0; t < n; ++t) {
        w[t] = exp(w[t] - m);
        l += w[t];
    }
    for (int t = 0; t < n; ++t)
        for (int d = 0; d < D; ++d)
            o[d] += w[t] * load(v, kv_base + (size_t)t * D + d, dt);
    for (int d = 0; d < D; ++d)
        o[d] /= l;
}

/* Causal grouped-query prefill.
 * q: [B, Hq, S, D], k, v: [B, Hkv, S, D] (element type dt), Hq % Hkv == 0.
 * Query head h reads key/value head h / (Hq/Hkv) (consecutive query heads form
 * a group, as the repeat-interleaved equivalence on the GQA page states).
 * Query i sees keys 0..i (causal, queries and keys at the same positions).
 * rows: NULL computes every row into out [B, Hq, S, D]; otherwise rows holds
 * n_rows flat row indices ((b*Hq + h)*S + i) and out is [n_rows, D].
 * Each OpenMP thread allocates its own S-double score row. */
int oracle_prefill(double *out, const void *q, const void *k, const void *v, int dt,
                   int B, int Hq, int Hkv, int S, int D, double scale,
                   const int64_t *rows, int64_t n_rows)
{
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || S <= 0 || D <= 0 || Hq % Hkv != 0)
        return 1;
    int G = Hq / Hkv;
    int64_t total = rows ? n_rows : (int64_t)B * Hq * S;
    int bad = 0;
#pragma omp parallel
    {
        double *w = (double *)malloc(sizeof(double) * (size_t)S);
        if (!w) {
#pragma omp atomic write
            bad = 2;
        } else {
#pragma omp for schedule(dynamic, 16)
            for (int64_t r = 0; r < total; ++r) {
                int64_t flat = rows ? rows[r] : r;
                if (flat < 0 || flat >= (int64_t)B * Hq * S)
                    continue;
                int i = (int)(flat % S);
                int h = (int)((flat / S) % Hq);
                int b = (int)(flat / ((int64_t)S * Hq));
                int j = h / G;
                size_t q_base = (size_t)flat * D;
                size_t kv_base = (((size_t)b * Hkv + j) * S) * (size_t)D;
                attend_row(out + (size_t)r * D, q, q_base, k, v, kv_base, i + 1, D,
                           dt, scale, w);
            }
            free(w);
        }
    }
    return bad;
}

/* Single-token decode over a contiguous cache.
 * q: [B, Hq, D]; k_cache, v_cache: [B, Hkv, S_cap, D]; seqlens[b] in
 * [0, S_cap] is the number of valid cached tokens of sequence b (the new
 * token's own key/value already included).  The new query sees all of them.
 * out: [B, Hq, D]; a sequence with no cached token gets a zero row. */
int oracle_decode(double *out, const void *q, const void *k_cache, const void *v_cache,
                  int dt, int B, int Hq, int Hkv, int S_cap, int D,
                  const int32_t *seqlens, double scale)
{
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || S_cap <= 0 || D <= 0 || Hq % Hkv != 0)
        return 1;
    int G = Hq / Hkv;
    int bad = 0;
#pragma omp parallel
    {
        double *w = (double *)malloc(sizeof(double) * (size_t)S_cap);
        if (!w) {
#pragma omp atomic write
            bad = 2;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t r = 0; r < (int64_t)B * Hq; ++r) {
                int h = (int)(r % Hq);
                int b = (int)(r / Hq);
                int j = h / G;
                int n = seqlens[b];
                if (n > S_cap)
                    n = S_cap;
                size_t kv_base = (((size_t)b * Hkv + j) * S_cap) * (size_t)D;
                attend_row(out + (size_t)r * D, q, (size_t)r * D, k_cache, v_cache,
                           kv_base, n, D, dt, scale, w);
            }
            free(w);
        }
    }
    return bad;
}

/* Single-token decode over a paged cache, optionally limited to a sliding
 * window.  "Grouped Query Attention (GQA)" glossary, section "GQA y técnicas
 * relacionadas": PagedAttention keeps the cache in fixed-size blocks, and
 * sliding-window attention bounds the cached tokens a query sees.  The pages
 * name both without further detail; this follows the plain reading:
 *  - k_pages, v_pages: [num_pages, Hkv, page_size, D];  block_table:
 *    [B, max_pages] page indices;  token t of sequence b is row t % page_size
 *    of page block_table[b][t / page_size];
 *  - window > 0: the query of sequence b sees tokens max(0, len_b - window)
 *    .. len_b - 1;  window <= 0: all len_b tokens.
 * Otherwise as oracle_decode: out [B, Hq, D], a sequence that sees no token
 * gets a zero row.  Returns 3 if a needed table entry is outside
 * [0, num_pages) or a length exceeds max_pages * page_size. */
int oracle_decode_paged(double *out, const void *q, const void *k_pages, const void *v_pages,
                        int dt, int B, int Hq, int Hkv, int page_size, int D, int num_pages,
                        const int32_t *block_table, int max_pages, const int32_t *seqlens,
                        int window, double scale)
{
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || page_size <= 0 || D <= 0 || num_pages <= 0 ||
        max_pages <= 0 || Hq % Hkv != 0)
        return 1;
    for (int b = 0; b < B; ++b) {
        const int len = seqlens[b];
        if (len < 0 || (int64_t)len > (int64_t)max_pages * page_size)
            return 3;
        const int lo = (window > 0 && len > window) ? len - window : 0;
        for (int t = lo; t < len; ++t) {
            int pg = block_table[(size_t)b * max_pages + t / page_size];
            if (pg < 0 || pg >= num_pages)
                return 3;
        }
    }
    int G = Hq / Hkv;
    int bad = 0;
#pragma omp parallel
    {
        size_t cap = (size_t)max_pages * page_size;
        double *w = (double *)malloc(sizeof(double) * cap);
        size_t *rowb = (size_t *)malloc(sizeof(size_t) * cap);
        if (!w || !rowb) {
#pragma omp atomic write
            bad = 2;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t r = 0; r < (int64_t)B * Hq; ++r) {
                int h = (int)(r % Hq);
                int b = (int)(r / Hq);
                int j = h / G;
                const int len = seqlens[b];
                const int lo = (window > 0 && len > window) ? len - window : 0;
                double *o = out + (size_t)r * D;
                for (int d = 0; d < D; ++d)
                    o[d] = 0.0;
                if (len <= lo)
                    continue;
                /* element offset of every visible token's row */
                for (int t = lo; t < len; ++t) {
                    size_t pg = (size_t)block_table[(size_t)b * max_pages + t / page_size];
                    rowb[t - lo] = ((pg * Hkv + j) * page_size + (size_t)(t % page_size)) * D;
                }
                const int cnt = len - lo;
                double m = -INFINITY;
                for (int t = 0; t < cnt; ++t) {
                    double dot = 0.0;
                    for (int d = 0; d < D; ++d)
                        dot += load(q, (size_t)r * D + d, dt) * load(k_pages, rowb[t] + d, dt);
                    w[t] = dot * scale;
                    if (w[t] > m)
                        m = w[t];
                }
                double l = 0.0;
                for (int t = 0; t < cnt; ++t) {
                    w[t] = exp(w[t] - m);
                    l += w[t];
                }
                for (int t = 0; t < cnt; ++t)
                    for (int d = 0; d < D; ++d)
                        o[d] += w[t] * load(v_pages, rowb[t] + d, dt);
                for (int d = 0; d < D; ++d)
                    o[d] = o[d] / l;
            }
        }
        free(w);
        free(rowb);
    }
    return bad;
}


/* ------------------------------------------------------------------ */
/* Training: log-normaliser of the forward and the backward pass       */
/* ------------------------------------------------------------------ */
/* The "Compressed Convolutional Attention" summary ("Resultaten") reports the
 * backward pass of the same attention; the pages give no formulas for it, so
 * what follows is the chain rule applied to the forward definition above.
 * For query row i of head h (key/value head j = h / G) with scores
 * s_t = scale * <q_i, k_t>, t <= i, and loss gradient dout_i = dL/do_i:
 *   lse_i  = log sum_{t<=i} exp(s_t)            p_t = exp(s_t - lse_i)
 *   o_i    = sum_t p_t v_t
 *   dL/dv_t  gets  p_t * dout_i                  (from o_i = sum_t p_t v_t)
 *   dp_t   = <dout_i, v_t>                        (dL/dp_t)
 *   ds_t   = p_t * (dp_t - sum_u p_u dp_u)        (softmax Jacobian)
 *   dL/dq_i  = scale * sum_t ds_t k_t
 *   dL/dk_t gets scale * ds_t * q_i
 * A key/value head's gradient collects these over every query head of its
 * group and every query that sees it (i >= t). */

/* Row statistics of causal prefill row (b, h, i) = flat row r:
 * lse = log sum_{t<=i} exp(s_t) and delta = sum_t p_t <dout_i, v_t>.
 * With dout NULL only lse is formed (delta = 0).  sc: scratch of i+1 doubles. */
static void row_lse_delta(const void *q, const void *k, const void *v, const void *dout,
                          int dt, int Hq, int Hkv, int S, int D, double scale, int64_t r,
                          double *sc, double *lse_out, double *delta_out)
{
    const int i = (int)(r % S);
    const int h = (int)((r / S) % Hq);
    const int b = (int)(r / ((int64_t)S * Hq));
    const int j = h / (Hq / Hkv);
    const size_t qrow = (size_t)r * D;
    const size_t kv0 = (((size_t)b * Hkv + j) * S) * (size_t)D;
    double top = -INFINITY;
    for (int t = 0; t <= i; ++t) {
        double acc = 0.0;
        for (int d = 0; d < D; ++d)
            acc += load(q, qrow + d, dt) * load(k, kv0 + (size_t)t * D + d, dt);
        sc[t] = acc * scale;
        if (sc[t] > top)
            top = sc[t];
    }
    double z = 0.0;
    for (int t = 0; t <= i; ++t)
        z += exp(sc[t] - top);
    const double lse = top + log(z);
    double delta = 0.0;
    if (dout) {
        for (int t = 0; t <= i; ++t) {
            double dp = 0.0;
            for (int d = 0; d < D; ++d)
                dp += load(dout, qrow + d, dt) * load(v, kv0 + (size_t)t * D + d, dt);
            delta += exp(sc[t] - lse) * dp;
        }
    }
    *lse_out = lse;
    *delta_out = delta;
}

/* Log-normaliser of causal prefill rows: lse[(b*Hq + h)*S + i] =
 * log sum_{t<=i} exp(scale * <q[b,h,i], k[b,h/G,t]>).  rows: NULL for every
 * row (lse is [B, Hq, S]); else n_rows flat row indices and lse is [n_rows]. */
int oracle_prefill_lse(double *lse, const void *q, const void *k, int dt, int B, int Hq,
                       int Hkv, int S, int D, double scale, const int64_t *rows,
                       int64_t n_rows)
{
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || S <= 0 || D <= 0 || Hq % Hkv != 0)
        return 1;
    const int64_t total = rows ? n_rows : (int64_t)B * Hq * S;
    int bad = 0;
#pragma omp parallel
    {
        double *sc = (double *)malloc(sizeof(double) * (size_t)S);
        if (!sc) {
#pragma omp atomic write
            bad = 2;
        } else {
#pragma omp for schedule(dynamic, 16)
            for (int64_t n = 0; n < total; ++n) {
                const int64_t r = rows ? rows[n] : n;
                double unused;
                if (r < 0 || r >= (int64_t)B * Hq * S)
                    continue;
                row_lse_delta(q, k, NULL, NULL, dt, Hq, Hkv, S, D, scale, r, sc, &lse[n],
                              &unused);
            }
            free(sc);
        }
    }
    return bad;
}

/* Gradients of L = sum <dout, prefill(q, k, v)> for causal grouped-query
 * prefill (shapes as oracle_prefill, dout like q).
 *   dq: [B, Hq, S, D] or, with q_rows, [n_q, D] for the listed flat query rows
 *       ((b*Hq + h)*S + i);
 *   dk, dv: [B, Hkv, S, D] or, with k_rows, [n_k, D] for the listed flat
 *       key rows ((b*Hkv + j)*S + t).
 * dq may be NULL (no query rows) and dk/dv NULL together (no key rows).
 * Row statistics (lse, delta) are formed first for every query row a result
 * needs: the listed query rows, and every row of a group that has a listed key
 * row. */
int oracle_prefill_backward(double *dq, double *dk, double *dv, const void *q, const void *k,
                            const void *v, const void *dout, int dt, int B, int Hq, int Hkv,
                            int S, int D, double scale, const int64_t *q_rows, int64_t n_q,
                            const int64_t *k_rows, int64_t n_k)
{
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || S <= 0 || D <= 0 || Hq % Hkv != 0)
        return 1;
    if ((dk == NULL) != (dv == NULL))
        return 1;
    const int G = Hq / Hkv;
    const int64_t nrows = (int64_t)B * Hq * S;
    const int64_t nq = dq ? (q_rows ? n_q : nrows) : 0;
    const int64_t nk = dk ? (k_rows ? n_k : (int64_t)B * Hkv * S) : 0;
    for (int64_t n = 0; q_rows && n < nq; ++n)
        if (q_rows[n] < 0 || q_rows[n] >= nrows)
            return 3;
    for (int64_t n = 0; k_rows && n < nk; ++n)
        if (k_rows[n] < 0 || k_rows[n] >= (int64_t)B * Hkv * S)
            return 3;

    /* which query rows need their statistics */
    double *lse = (double *)malloc(sizeof(double) * (size_t)nrows);
    double *delta = (double *)malloc(sizeof(double) * (size_t)nrows);
    unsigned char *need = (unsigned char *)calloc((size_t)nrows, 1);
    unsigned char *grp = (unsigned char *)calloc((size_t)B * Hkv, 1);
    if (!lse || !delta || !need || !grp) {
        free(lse);
        free(delta);
        free(need);
        free(grp);
        return 2;
    }
    for (int64_t n = 0; n < nq; ++n)
        need[q_rows ? q_rows[n] : n] = 1;
    for (int64_t n = 0; n < nk; ++n)
        grp[(k_rows ? k_rows[n] : n) / S] = 1;
    for (int64_t r = 0; r < nrows; ++r)
        if (grp[(r / S / Hq) * Hkv + (r / S % Hq) / G])
            need[r] = 1;

    int bad = 0;
#pragma omp parallel
    {
        double *sc = (double *)malloc(sizeof(double) * (size_t)S);
        if (!sc) {
#pragma omp atomic write
            bad = 2;
        } else {
#pragma omp for schedule(dynamic, 16)
            for (int64_t r = 0; r < nrows; ++r)
                if (need[r])
                    row_lse_delta(q, k, v, dout, dt, Hq, Hkv, S, D, scale, r, sc, &lse[r],
                                  &delta[r]);

            /* dq rows: scale * sum_{t<=i} ds_t k_t */
#pragma omp for schedule(dynamic, 16)
            for (int64_t n = 0; n < nq; ++n) {
                const int64_t r = q_rows ? q_rows[n] : n;
                const int i = (int)(r % S);
                const int h = (int)((r / S) % Hq);
                const int b = (int)(r / ((int64_t)S * Hq));
                const size_t kv0 = (((size_t)b * Hkv + h / G) * S) * (size_t)D;
                double *g = dq + (size_t)n * D;
                for (int d = 0; d < D; ++d)
                    g[d] = 0.0;
                for (int t = 0; t <= i; ++t) {
                    double s = 0.0, dp = 0.0;
                    for (int d = 0; d < D; ++d) {
                        s += load(q, (size_t)r * D + d, dt) * load(k, kv0 + (size_t)t * D + d, dt);
                        dp += load(dout, (size_t)r * D + d, dt) * load(v, kv0 + (size_t)t * D + d, dt);
                    }
                    const double p = exp(s * scale - lse[r]);
                    const double ds = p * (dp - delta[r]);
                    for (int d = 0; d < D; ++d)
                        g[d] += scale * ds * load(k, kv0 + (size_t)t * D + d, dt);
                }
            }

            /* dk, dv rows: over the group's query heads and the queries i >= t */
#pragma omp for schedule(dynamic, 4)
            for (int64_t n = 0; n < nk; ++n) {
                const int64_t kr = k_rows ? k_rows[n] : n;
                const int t = (int)(kr % S);
                const int j = (int)((kr / S) % Hkv);
                const int b = (int)(kr / ((int64_t)S * Hkv));
                const size_t krow = (size_t)kr * D;
                double *gk = dk + (size_t)n * D;
                double *gv = dv + (size_t)n * D;
                for (int d = 0; d < D; ++d)
                    gk[d] = gv[d] = 0.0;
                for (int h = j * G; h < (j + 1) * G; ++h)
                    for (int i = t; i < S; ++i) {
                        const int64_t r = ((int64_t)b * Hq + h) * S + i;
                        double s = 0.0, dp = 0.0;
                        for (int d = 0; d < D; ++d) {
                            s += load(q, (size_t)r * D + d, dt) * load(k, krow + d, dt);
                            dp += load(dout, (size_t)r * D + d, dt) * load(v, krow + d, dt);
                        }
                        const double p = exp(s * scale - lse[r]);
                        const double ds = p * (dp - delta[r]);
                        for (int d = 0; d < D; ++d) {
                            gk[d] += scale * ds * load(q, (size_t)r * D + d, dt);
                            gv[d] += p * load(dout, (size_t)r * D + d, dt);
                        }
                    }
            }
            free(sc);
        }
    }
    free(lse);
    free(delta);
    free(need);
    free(grp);
    return bad;
}


/* ------------------------------------------------------------------ */
/* CCA pre-attention operations on the compressed q, k, v              */
/* ------------------------------------------------------------------ */
/* "Compressed Convolutional Attention" summary, "Methodologie", items 2-4.
 * The summary names the operations without their sizes or exact form; this
 * oracle follows the plainest reading of it (stated item by item below).
 * Inputs are the compressed per-head vectors q~ [B, Hq, S, D], k~, v~
 * [B, Hkv, S, D]; query head h belongs to KV group h / G, G = Hq / Hkv.
 *
 *  (2a) sequence mixing: a causal depthwise convolution over the sequence, of
 *       width W, per channel c of every head:
 *           s[t, c] = sum_{i < W, t - i >= 0} conv[h, i, c] * x[t - i, c]
 *       (tap i weighs the token i steps back; tokens before the first are 0);
 *  (2b) channel mixing within a head: a dense D x D map per head,
 *           z[t, c] = sum_{c'} mix[h, c, c'] * s[t, c'];
 *  (2c) QK-mean: the mean of the pre-convolution query and key vectors of a
 *       token, shared by the group (the query heads of a group first averaged),
 *           m[t, j] = ( (1/G) sum_{h in group j} q~[t, h] + k~[t, j] ) / 2,
 *       is added to the convolved vectors: q[t, h] = z_q[t, h] + m[t, h / G],
 *       k[t, j] = z_k[t, j] + m[t, j] (a skip path of the pre-convolution
 *       values, and a component q and k of one token share);
 *  (4)  RoPE, when theta > 0, on those q and k at absolute position
 *       pos_offset[b] + t (oracle_rope, the same rotation as everywhere);
 *  (3)  value shift: each head's values come half from the current token and
 *       half from the previous one: v[t, c] = v~[t, c] for c < D/2 and
 *       v~[t - 1, c] for c >= D/2 (0 at t = 0).
 * conv_q [Hq, W, D], conv_k [Hkv, W, D] (tap-major), mix_q [Hq, D, D], mix_k [Hkv, D, D]
 * (row c of mix is output channel c) share the inputs' element type dt.
 * Outputs are fp64 [B, Hq, S, D], [B, Hkv, S, D], [B, Hkv, S, D]. */
int oracle_cca_mix(double *q_out, double *k_out, double *v_out, const void *q, const void *k,
                   const void *v, int dt, int B, int Hq, int Hkv, int S, int D,
                   const void *conv_q, const void *conv_k, int W, const void *mix_q,
                   const void *mix_k, const int32_t *pos_offset, double theta)
{
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || S <= 0 || D <= 0 || W <= 0 || Hq % Hkv != 0 || D % 2)
        return 1;
    const int G = Hq / Hkv;
    int bad = 0;
#pragma omp parallel
    {
        double *mean = (double *)malloc(sizeof(double) * (size_t)Hkv * D);
        double *conv = (double *)malloc(sizeof(double) * (size_t)D);
        if (!mean || !conv) {
#pragma omp atomic write
            bad = 2;
        } else {
#pragma omp for schedule(static)
            for (int64_t bt = 0; bt < (int64_t)B * S; ++bt) {
                const int b = (int)(bt / S), t = (int)(bt % S);
                /* (2c) the token's pre-convolution mean, per KV group */
                for (int j = 0; j < Hkv; ++j)
                    for (int c = 0; c < D; ++c) {
                        double qsum = 0.0;
                        for (int r = 0; r < G; ++r)
                            qsum += load(q, (((size_t)b * Hq + (size_t)j * G + r) * S + t) * D + c, dt);
                        const double kv = load(k, (((size_t)b * Hkv + j) * S + t) * D + c, dt);
                        mean[(size_t)j * D + c] = 0.5 * (qsum / G + kv);
                    }
                /* (2a), (2b) and the mean, for the query heads and then the key heads */
                for (int n = 0; n < Hq + Hkv; ++n) {
                    const int isq = n < Hq;
                    const int h = isq ? n : n - Hq;
                    const int H = isq ? Hq : Hkv;
                    const void *x = isq ? q : k;
                    const void *cw = isq ? conv_q : conv_k;
                    const void *mw = isq ? mix_q : mix_k;
                    const double *mrow = mean + (size_t)(isq ? h / G : h) * D;
                    double *out = (isq ? q_out : k_out) + (((size_t)b * H + h) * S + t) * D;
                    for (int c = 0; c < D; ++c) {
                        double acc = 0.0;
                        for (int i = 0; i < W; ++i) {
                            int src = t - i;
                            if (src < 0)
                                continue;
                            acc += load(cw, ((size_t)h * W + i) * D + c, dt) *
                                   load(x, (((size_t)b * H + h) * S + src) * D + c, dt);
                        }
                        conv[c] = acc;
                    }
                    for (int c = 0; c < D; ++c) {
                        double acc = 0.0;
                        for (int c2 = 0; c2 < D; ++c2)
                            acc += load(mw, ((size_t)h * D + c) * D + c2, dt) * conv[c2];
                        out[c] = acc + mrow[c];
                    }
                }
                /* (3) value shift */
                for (int j = 0; j < Hkv; ++j)
                    for (int c = 0; c < D; ++c) {
                        const size_t at = (((size_t)b * Hkv + j) * S + t) * D + c;
                        double val;
                        if (c < D / 2)
                            val = load(v, at, dt);
                        else
                            val = t > 0 ? load(v, at - (size_t)D, dt) : 0.0;
                        v_out[at] = val;
                    }
            }
        }
        free(mean);
        free(conv);
    }
    if (bad)
        return bad;
    /* (4) RoPE of the mixed q and k at their absolute positions */
    if (theta > 0.0) {
        double *tmp = (double *)malloc(sizeof(double) * (size_t)B * Hq * S * D);
        if (!tmp)
            return 2;
        memcpy(tmp, q_out, sizeof(double) * (size_t)B * Hq * S * D);
        oracle_rope(q_out, tmp, OR_F64, B, Hq, S, D, pos_offset, theta);
        memcpy(tmp, k_out, sizeof(double) * (size_t)B * Hkv * S * D);
        oracle_rope(k_out, tmp, OR_F64, B, Hkv, S, D, pos_offset, theta);
        free(tmp);
    }
    return 0;
}

/* Gradients of the CCA pre-attention operations (oracle_cca_mix) by the chain
 * rule, taken through its steps in reverse order.  Given gq = dL/dq, gk =
 * dL/dk (with respect to the rotated outputs) and gv = dL/dv:
 *   (4)  a_q = R_t^T gq, a_k = R_t^T gk (the transposed rotation at the same
 *        positions; a = g when theta == 0);
 *   (2c) the mean reaches every query head of the group and its key head, so
 *        dm[t, j] = sum_{h in group j} a_q[t, h] + a_k[t, j], and
 *        dq~[t, h] += dm[t, j] / (2 G),  dk~[t, j] += dm[t, j] / 2;
 *   (2b) z = M s:  ds[t, c'] = sum_c mix[h, c, c'] a[t, c]   (M^T a),
 *        dmix[h, c, c'] += sum_{b, t} a[t, c] s[t, c'];
 *   (2a) s[t] = sum_i conv[h, i] x[t - i]:
 *        dx[t, c] += sum_{i < W, t + i < S} conv[h, i, c] ds[t + i, c],
 *        dconv[h, i, c] += sum_{b, t >= i} ds[t, c] x[t - i, c];
 *   (3)  dv~[t, c] = gv[t, c] for c < D/2, gv[t + 1, c] for c >= D/2 (0 at
 *        the last token).
 * Weight gradients sum over the batch and every token.  Inputs (gradients,
 * latent q~, k~, weights) share the element type dt; outputs are fp64:
 * dq [B, Hq, S, D], dk and dv [B, Hkv, S, D], dconv_q [Hq, W, D], dconv_k
 * [Hkv, W, D], dmix_q [Hq, D, D], dmix_k [Hkv, D, D]. */
int oracle_cca_mix_backward(double *dq, double *dk, double *dv, double *dconv_q, double *dconv_k,
                            double *dmix_q, double *dmix_k, const void *gq, const void *gk,
                            const void *gv, const void *q, const void *k, int dt, int B, int Hq,
                            int Hkv, int S, int D, const void *conv_q, const void *conv_k, int W,
                            const void *mix_q, const void *mix_k, const int32_t *pos_offset,
                            double theta)
{
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || S <= 0 || D <= 0 || W <= 0 || Hq % Hkv != 0 || D % 2)
        return 1;
    const int G = Hq / Hkv;
    const size_t nq = (size_t)B * Hq * S * D, nk = (size_t)B * Hkv * S * D;
    /* (4) back through the rotation */
    double *aq = (double *)malloc(sizeof(double) * nq);
    double *ak = (double *)malloc(sizeof(double) * nk);
    double *dm = (double *)malloc(sizeof(double) * nk);
    if (!aq || !ak || !dm) {
        free(aq);
        free(ak);
        free(dm);
        return 2;
    }
    if (theta > 0.0) {
        oracle_rope_transpose(aq, gq, dt, B, Hq, S, D, pos_offset, theta);
        oracle_rope_transpose(ak, gk, dt, B, Hkv, S, D, pos_offset, theta);
    } else {
        for (size_t i = 0; i < nq; ++i)
            aq[i] = load(gq, i, dt);
        for (size_t i = 0; i < nk; ++i)
            ak[i] = load(gk, i, dt);
    }
    /* (2c) the mean's gradient per (b, j, t) */
    for (int b = 0; b < B; ++b)
        for (int j = 0; j < Hkv; ++j)
            for (int t = 0; t < S; ++t)
                for (int c = 0; c < D; ++c) {
                    const size_t at = (((size_t)b * Hkv + j) * S + t) * D + c;
                    double sum = ak[at];
                    for (int r = 0; r < G; ++r)
                        sum += aq[(((size_t)b * Hq + (size_t)j * G + r) * S + t) * D + c];
                    dm[at] = sum;
                }
    int bad = 0;
    /* (2b), (2a) per head: one head per thread, so each weight gradient is summed
     * by one thread in a fixed order */
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)S * D);
        double *ds = (double *)malloc(sizeof(double) * (size_t)S * D);
        if (!s || !ds) {
#pragma omp atomic write
            bad = 2;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int n = 0; n < Hq + Hkv; ++n) {
                const int isq = n < Hq;
                const int h = isq ? n : n - Hq;
                const int H = isq ? Hq : Hkv;
                const void *x = isq ? q : k;
                const void *cw = isq ? conv_q : conv_k;
                const void *mw = isq ? mix_q : mix_k;
                const double *a = isq ? aq : ak;
                double *dx = isq ? dq : dk;
                double *dconv = (isq ? dconv_q : dconv_k) + (size_t)h * W * D;
                double *dmix = (isq ? dmix_q : dmix_k) + (size_t)h * D * D;
                const int j = isq ? h / G : h;
                const double mean_w = isq ? 0.5 / G : 0.5;
                for (size_t i = 0; i < (size_t)W * D; ++i)
                    dconv[i] = 0.0;
                for (size_t i = 0; i < (size_t)D * D; ++i)
                    dmix[i] = 0.0;
                for (int b = 0; b < B; ++b) {
                    const size_t row0 = ((size_t)b * H + h) * S; /* first row of this head */
                    /* the forward's convolution output s, and ds = M^T a */
                    for (int t = 0; t < S; ++t)
                        for (int c = 0; c < D; ++c) {
                            double acc = 0.0;
                            for (int i = 0; i < W && t - i >= 0; ++i) {
                                const double tap = load(cw, ((size_t)h * W + i) * D + c, dt);
                                acc += tap * load(x, (row0 + t - i) * D + c, dt);
                            }
                            s[(size_t)t * D + c] = acc;
                            double g = 0.0;
                            for (int c2 = 0; c2 < D; ++c2)
                                g += load(mw, ((size_t)h * D + c2) * D + c, dt) *
                                     a[(row0 + t) * D + c2];
                            ds[(size_t)t * D + c] = g;
                        }
                    for (int t = 0; t < S; ++t)
                        for (int c = 0; c < D; ++c) {
                            /* mix gradient: a (output channel c) times s (input c2) */
                            const double av = a[(row0 + t) * D + c];
                            for (int c2 = 0; c2 < D; ++c2)
                                dmix[(size_t)c * D + c2] += av * s[(size_t)t * D + c2];
                            /* input gradient: the convolution's taps run forward in time */
                            double acc = 0.0;
                            for (int i = 0; i < W && t + i < S; ++i) {
                                const double tap = load(cw, ((size_t)h * W + i) * D + c, dt);
                                acc += tap * ds[(size_t)(t + i) * D + c];
                            }
                            const size_t mat = (((size_t)b * Hkv + j) * S + t) * D + c;
                            dx[(row0 + t) * D + c] = acc + mean_w * dm[mat];
                            /* tap gradient */
                            for (int i = 0; i < W && t - i >= 0; ++i)
                                dconv[(size_t)i * D + c] +=
                                    ds[(size_t)t * D + c] * load(x, (row0 + t - i) * D + c, dt);
                        }
                }
            }
        }
        free(s);
        free(ds);
    }
    /* (3) value shift */
    for (int b = 0; b < B; ++b)
        for (int j = 0; j < Hkv; ++j)
            for (int t = 0; t < S; ++t)
                for (int c = 0; c < D; ++c) {
                    const size_t at = (((size_t)b * Hkv + j) * S + t) * D + c;
                    if (c < D / 2)
                        dv[at] = load(gv, at, dt);
                    else
                        dv[at] = t + 1 < S ? load(gv, at + (size_t)D, dt) : 0.0;
                }
    free(aq);
    free(ak);
    free(dm);
    return bad;
}
