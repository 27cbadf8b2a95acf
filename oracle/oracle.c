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

