/*
 * Seeded synthetic inputs: genotype mosaic matrices, copy-model digraphs,
 * Gaussian weight vectors and BFS source sets.
 *
 * This module only draws random numbers and lays the resulting matrix out as
 * CSR (int64 row pointers, int32 columns, int8 values).  It contains none of
 * the grammar method's arithmetic; both the CPU oracle and the grammar builder
 * consume its output.
 *
 * Every random draw is a pure function of (seed, stream, counter), so any row
 * or column range can be regenerated on its own and in any order:
 *   mix64     = SplitMix64 output function (Steele, Lea, Flood, "Fast
 *               splittable pseudorandom number generators", OOPSLA 2014),
 *               applied to an additively combined key;
 *   uniform   = top 53 bits of the hash scaled by 2^-53;
 *   normal    = Box-Muller transform of two such uniforms;
 *   Beta(1/2,1/2) = sin^2(pi*u/2) (the arcsine law);
 *   geometric = inversion, 1 + floor(ln U / ln(1-r)) with U in (0,1].
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define GOLDEN 0x9E3779B97F4A7C15ULL

enum {
    ST_FREQ = 1,      /* per-site allele frequency               */
    ST_FOUNDER = 2,   /* founder allele at (founder, site)       */
    ST_SEGLEN = 3,    /* haplotype segment length                */
    ST_SEGSRC = 4,    /* haplotype segment founder               */
    ST_MUT = 5,       /* haplotype mutation gaps                 */
    ST_DEG = 11,      /* copy model: out-degree                  */
    ST_PROTO = 12,    /* copy model: prototype + window offset   */
    ST_REPL = 13,     /* copy model: replacement coin + target   */
    ST_EXTRA = 14,    /* copy model: extra uniform targets       */
    ST_NORMAL = 21,   /* Gaussian vectors                        */
    ST_SOURCE = 22,   /* BFS sources                             */
};

static inline uint64_t mix64(uint64_t z)
{
    z += GOLDEN;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

static inline uint64_t hkey(uint64_t seed, uint64_t stream, uint64_t a, uint64_t b)
{
    uint64_t h = mix64(seed ^ (stream * GOLDEN));
    h = mix64(h ^ a);
    return mix64(h ^ (b * 0xD1B54A32D192ED03ULL));
}

/* uniform in [0, 1) */
static inline double u01(uint64_t h) { return (double)(h >> 11) * 0x1.0p-53; }
/* uniform in (0, 1] */
static inline double u01_open0(uint64_t h) { return (double)((h >> 11) + 1) * 0x1.0p-53; }

/* geometric on {1, 2, ...} with success probability r (mean 1/r) */
static inline int64_t geometric(uint64_t h, double log1mr)
{
    if (log1mr == 0.0) return INT64_MAX;        /* r == 0: never */
    if (isinf(log1mr)) return 1;                /* r == 1        */
    double g = floor(log(u01_open0(h)) / log1mr);
    if (g > 4.0e18) return INT64_MAX;
    return 1 + (int64_t)g;
}

/* ------------------------------------------------------------------ */
/* genotype mosaic                                                      */
/* ------------------------------------------------------------------ */

typedef struct {
    int64_t n_rows;      /* individuals                                    */
    int64_t n_cols;      /* variants                                       */
    int32_t founders;    /* F                                              */
    int32_t pad_;
    double seg_mean;     /* mean segment length (variants)                 */
    double mu;           /* per-site flip probability                      */
    uint64_t seed;
} synth_geno_params;

/* Minor-allele frequency of site j: p ~ Beta(1/2,1/2), folded to min(p,1-p). */
double synth_site_maf(const synth_geno_params* P, int64_t j)
{
    double u = u01(hkey(P->seed, ST_FREQ, (uint64_t)j, 0));
    double s = sin(M_PI * u * 0.5);
    double p = s * s;
    return p < 1.0 - p ? p : 1.0 - p;
}

/* Founder allele table, F x ncols bytes (columns col0 .. col0+ncols-1). */
static uint8_t* founder_table(const synth_geno_params* P, int64_t col0, int64_t ncols)
{
    int64_t F = P->founders;
    uint8_t* t = (uint8_t*)malloc((size_t)(F * ncols > 0 ? F * ncols : 1));
    if (!t) return NULL;
#pragma omp parallel for schedule(static)
    for (int64_t jj = 0; jj < ncols; ++jj) {
        int64_t j = col0 + jj;
        double q = synth_site_maf(P, j);
        for (int64_t f = 0; f < F; ++f)
            t[f * ncols + jj] = u01(hkey(P->seed, ST_FOUNDER, (uint64_t)f, (uint64_t)j)) < q;
    }
    return t;
}

/* Haplotype h restricted to columns [col0, col0+ncols) into out[0..ncols). */
static void haplotype(const synth_geno_params* P, const uint8_t* ftab, int64_t h,
                      int64_t col0, int64_t ncols, uint8_t* out)
{
    const int64_t m = P->n_cols, c1 = col0 + ncols;
    const double lseg = log1p(-1.0 / P->seg_mean);
    int64_t pos = 0;
    for (uint64_t s = 0; pos < c1; ++s) {
        int64_t len = geometric(hkey(P->seed, ST_SEGLEN, (uint64_t)h, s), lseg);
        int64_t end = (len > m - pos) ? m : pos + len;
        if (end > col0) {
            int64_t f = (int64_t)(u01(hkey(P->seed, ST_SEGSRC, (uint64_t)h, s)) * P->founders);
            if (f >= P->founders) f = P->founders - 1;
            int64_t a = pos > col0 ? pos : col0, b = end < c1 ? end : c1;
            memcpy(out + (a - col0), ftab + f * ncols + (a - col0), (size_t)(b - a));
        }
        pos = end;
    }
    if (P->mu > 0.0) {
        const double lmu = log1p(-P->mu);
        int64_t j = -1;
        for (uint64_t k = 0;; ++k) {
            int64_t g = geometric(hkey(P->seed, ST_MUT, (uint64_t)h, k), lmu);
            if (g >= m - j) break;
            j += g;
            if (j >= c1) break;
            if (j >= col0) out[j - col0] ^= 1;
        }
    }
}

/*
 * Two-pass CSR generation of rows [row0, row0+nrows) restricted to columns
 * [col0, col0+ncols).  Column indices written are absolute.
 *   pass 1 (col == NULL): row_nnz[i] = nonzeros of row row0+i.
 *   pass 2: fills col/val at row_ptr[i] (row_ptr relative to this block).
 * Returns 0, or -1 on allocation failure.
 */
int synth_genotype_block(const synth_geno_params* P, int64_t row0, int64_t nrows,
                         int64_t col0, int64_t ncols, int64_t* row_nnz,
                         const int64_t* row_ptr, int32_t* col, int8_t* val)
{
    if (nrows <= 0) return 0;
    if (ncols <= 0) {
        if (!col) for (int64_t i = 0; i < nrows; ++i) row_nnz[i] = 0;
        return 0;
    }
    uint8_t* ftab = founder_table(P, col0, ncols);
    if (!ftab) return -1;
    int failed = 0;
#pragma omp parallel
    {
        uint8_t* h0 = (uint8_t*)malloc((size_t)ncols);
        uint8_t* h1 = (uint8_t*)malloc((size_t)ncols);
        if (!h0 || !h1) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 16)
            for (int64_t i = 0; i < nrows; ++i) {
                int64_t r = row0 + i;
                haplotype(P, ftab, 2 * r, col0, ncols, h0);
                haplotype(P, ftab, 2 * r + 1, col0, ncols, h1);
                if (!col) {
                    int64_t c = 0;
                    for (int64_t j = 0; j < ncols; ++j) c += (h0[j] | h1[j]) != 0;
                    row_nnz[i] = c;
                } else {
                    int64_t o = row_ptr[i];
                    for (int64_t j = 0; j < ncols; ++j) {
                        int g = h0[j] + h1[j];
                        if (g) { col[o] = (int32_t)(col0 + j); val[o] = (int8_t)g; ++o; }
                    }
                }
            }
        }
        free(h0);
        free(h1);
    }
    free(ftab);
    return failed ? -1 : 0;
}

/* ------------------------------------------------------------------ */
/* copy-model digraph                                                   */
/* ------------------------------------------------------------------ */

typedef struct {
    int64_t n;           /* nodes                                   */
    double mean_deg;     /* lognormal mean of the out-degree        */
    double sigma;        /* lognormal sigma                         */
    double p_replace;    /* per-copied-entry replacement probability */
    uint64_t seed;
} synth_graph_params;

static inline double normal_at(uint64_t seed, uint64_t stream, uint64_t i)
{
    double u1 = u01_open0(hkey(seed, stream, i, 0));
    double u2 = u01(hkey(seed, stream, i, 1));
    return sqrt(-2.0 * log(u1)) * cos(2.0 * M_PI * u2);
}

/* Target out-degree of node i (before de-duplication). */
int64_t synth_graph_degree(const synth_graph_params* G, int64_t i)
{
    double mu_ln = log(G->mean_deg) - 0.5 * G->sigma * G->sigma;
    double d = exp(mu_ln + G->sigma * normal_at(G->seed, ST_DEG, (uint64_t)i));
    double r = floor(d + 0.5);
    if (r < 1.0) r = 1.0;
    if (r > (double)G->n) r = (double)G->n;
    return (int64_t)r;
}

/* Sum of target degrees: an upper bound on the edge count. */
int64_t synth_graph_degree_sum(const synth_graph_params* G)
{
    int64_t s = 0;
#pragma omp parallel for reduction(+ : s) schedule(static)
    for (int64_t i = 0; i < G->n; ++i) s += synth_graph_degree(G, i);
    return s;
}

static int cmp_i32(const void* a, const void* b)
{
    int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
    return (x > y) - (x < y);
}

static int64_t sort_unique(int32_t* v, int64_t k)
{
    if (k <= 32) {
        for (int64_t i = 1; i < k; ++i) {
            int32_t t = v[i];
            int64_t j = i - 1;
            while (j >= 0 && v[j] > t) { v[j + 1] = v[j]; --j; }
            v[j + 1] = t;
        }
    } else {
        qsort(v, (size_t)k, sizeof(int32_t), cmp_i32);
    }
    int64_t w = 0;
    for (int64_t i = 0; i < k; ++i)
        if (w == 0 || v[i] != v[w - 1]) v[w++] = v[i];
    return w;
}

static inline int32_t uniform_node(const synth_graph_params* G, uint64_t stream, uint64_t a, uint64_t b)
{
    int64_t t = (int64_t)(u01(hkey(G->seed, stream, a, b)) * (double)G->n);
    return (int32_t)(t >= G->n ? G->n - 1 : t);
}

/*
 * Sequential generation (node i depends on an earlier prototype).  row_ptr has
 * n+1 entries; col has room for `cap` entries (synth_graph_degree_sum is
 * enough).  Returns the edge count, or -1 if cap is too small.
 */
int64_t synth_copy_graph(const synth_graph_params* G, int64_t* row_ptr, int32_t* col, int64_t cap)
{
    const int64_t n = G->n;
    row_ptr[0] = 0;
    if (n <= 0) return 0;
    int64_t nnz = 0;
    for (int64_t i = 0; i < n; ++i) {
        int64_t d = synth_graph_degree(G, i);
        if (nnz + d > cap) return -1;
        int32_t* out = col + nnz;
        int64_t k = 0;
        if (i == 0) {
            /* d distinct uniform targets */
            for (uint64_t t = 0; k < d; ++t) {
                int32_t c = uniform_node(G, ST_EXTRA, 0, t);
                int dup = 0;
                for (int64_t q = 0; q < k; ++q) dup |= out[q] == c;
                if (!dup) out[k++] = c;
            }
        } else {
            uint64_t hp = hkey(G->seed, ST_PROTO, (uint64_t)i, 0);
            int64_t p = (int64_t)(u01(hp) * (double)i);
            if (p >= i) p = i - 1;
            const int32_t* src = col + row_ptr[p];
            int64_t dp = row_ptr[p + 1] - row_ptr[p];
            int64_t take = d <= dp ? d : dp;
            int64_t off = 0;
            if (d <= dp) {
                off = (int64_t)(u01(hkey(G->seed, ST_PROTO, (uint64_t)i, 1)) * (double)(dp - d + 1));
                if (off > dp - d) off = dp - d;
            }
            for (int64_t q = 0; q < take; ++q) {
                int32_t c = src[off + q];
                if (u01(hkey(G->seed, ST_REPL, (uint64_t)i, 2 * (uint64_t)q)) < G->p_replace)
                    c = uniform_node(G, ST_REPL, (uint64_t)i, 2 * (uint64_t)q + 1);
                out[k++] = c;
            }
            for (int64_t q = take; q < d; ++q) out[k++] = uniform_node(G, ST_EXTRA, (uint64_t)i, (uint64_t)q);
        }
        k = sort_unique(out, k);
        nnz += k;
        row_ptr[i + 1] = nnz;
    }
    return nnz;
}

/* ------------------------------------------------------------------ */
/* vectors and sources                                                  */
/* ------------------------------------------------------------------ */

void synth_normal_f64(int64_t n, uint64_t seed, double* out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = normal_at(seed, ST_NORMAL, (uint64_t)i);
}

/* k distinct nodes in [0, n), in draw order; returns k or -1 if k > n. */
int64_t synth_sources(int64_t n, int64_t k, uint64_t seed, int64_t* out)
{
    if (k > n) return -1;
    int64_t got = 0;
    for (uint64_t t = 0; got < k; ++t) {
        int64_t c = (int64_t)(u01(hkey(seed, ST_SOURCE, t, 0)) * (double)n);
        if (c >= n) c = n - 1;
        int dup = 0;
        for (int64_t q = 0; q < got; ++q) dup |= out[q] == c;
        if (!dup) out[got++] = c;
    }
    return got;
}

int synth_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
