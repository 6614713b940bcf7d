/*
 * CPU oracle for the right product y = M x.  TEST INFRASTRUCTURE ONLY: this
 * file is built and called by the tests, the smoke check and the benchmark's
 * CPU-baseline leg, never by the product path.  It shares no code with the
 * grammar builder or the GPU kernels and never looks at a grammar: it works
 * from the original matrix in CSR form, as produced by the seeded generators.
 *
 * What it computes (page "Right Multiplication on Grammar-Compressed
 * Matrices", arXiv 2607.24971v1):
 *   - plus-times: y[r] = sum_j M[r][j] * x[j], the plain definition of the
 *     product the sweep evaluates (section 2, Lemma 2.2 and Theorem 2.3: the
 *     grammar sweep reaches exactly this value up to summation order);
 *   - Boolean: y[r] = OR_{j : M[r][j] != 0} x[j], the Boolean semiring
 *     (or, and) with the and of a nonzero entry and x[j] being x[j]
 *     (section 5);
 *   - BFS fixpoint: repeat f <- (M f) AND NOT visited, visited <- visited OR f
 *     until f is empty (section 5 names one Boolean pass as one frontier
 *     expansion; iterating it to the fixpoint is the plain reading);
 *   - tropical (min, +): y[r] = min_{j : M[r][j] stored} (M[r][j] + x[j]),
 *     +infinity for a row without stored entries (section 5: combine = min,
 *     leaf = +, identity +infinity; one pass is one Bellman-Ford
 *     relaxation).  Each term is a single addition in the precision of the
 *     policy (fp32: the fp32 value plus x[j], rounded to fp32), so the
 *     minimum is exact in any order.
 *
 * Plus-times sums are accumulated in fp64 with Neumaier's compensated
 * summation (Neumaier 1974, "Rundungsfehleranalyse einiger Verfahren zur
 * Summation endlicher Summen"), in column order, so the oracle is close to
 * the correctly rounded sum; absum[r] = sum_j |M[r][j] * x[j]| is the scale
 * the comparison tolerance is relative to.
 *
 * Matrix values: kind 0 = every stored entry is 1, kind 1 = int8 values,
 * kind 2 = fp64 values.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static inline double entry(int kind, const void* val, int64_t k)
{
    if (kind == 0) return 1.0;
    if (kind == 1) return (double)((const int8_t*)val)[k];
    return ((const double*)val)[k];
}

/* Compensated sum of row r; *abs_out = sum of |terms|. */
static double row_f64(int64_t r, const int64_t* row_ptr, const int32_t* col, int kind,
                      const void* val, const double* x, double* abs_out)
{
    double s = 0.0, c = 0.0, a = 0.0;
    for (int64_t k = row_ptr[r]; k < row_ptr[r + 1]; ++k) {
        double t = entry(kind, val, k) * x[col[k]];
        double u = s + t;
        if ((s >= 0 ? s : -s) >= (t >= 0 ? t : -t)) c += (s - u) + t;
        else c += (t - u) + s;
        s = u;
        a += t >= 0 ? t : -t;
    }
    *abs_out = a;
    return s + c;
}

/* All rows.  y and absum (optional) have n entries. */
void oracle_spmv_f64(int64_t n, const int64_t* row_ptr, const int32_t* col, int kind,
                     const void* val, const double* x, double* y, double* absum)
{
#pragma omp parallel for schedule(dynamic, 256)
    for (int64_t r = 0; r < n; ++r) {
        double a;
        y[r] = row_f64(r, row_ptr, col, kind, val, x, &a);
        if (absum) absum[r] = a;
    }
}

/* Selected rows: y[i] for row rows[i] (rows index the CSR's row_ptr). */
void oracle_spmv_f64_rows(const int64_t* rows, int64_t k, const int64_t* row_ptr, const int32_t* col,
                          int kind, const void* val, const double* x, double* y, double* absum)
{
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t i = 0; i < k; ++i) {
        int64_t r = rows[i];
        double aa;
        y[i] = row_f64(r, row_ptr, col, kind, val, x, &aa);
        if (absum) absum[i] = aa;
    }
}

/* Exact integer product: y[r] = sum_j M[r][j] * x[j] in int64 (kind 0 or 1). */
void oracle_spmv_i64(int64_t n, const int64_t* row_ptr, const int32_t* col, int kind,
                     const void* val, const int64_t* x, int64_t* y)
{
#pragma omp parallel for schedule(dynamic, 256)
    for (int64_t r = 0; r < n; ++r) {
        int64_t s = 0;
        for (int64_t k = row_ptr[r]; k < row_ptr[r + 1]; ++k) {
            int64_t v = kind == 0 ? 1 : (int64_t)((const int8_t*)val)[k];
            s += v * x[col[k]];
        }
        y[r] = s;
    }
}

/* Boolean product over (or, and); x and y hold 0/1 bytes. */
void oracle_spmv_bool(int64_t n, const int64_t* row_ptr, const int32_t* col,
                      const uint8_t* x, uint8_t* y)
{
#pragma omp parallel for schedule(dynamic, 1024)
    for (int64_t r = 0; r < n; ++r) {
        uint8_t b = 0;
        for (int64_t k = row_ptr[r]; k < row_ptr[r + 1] && !b; ++k) b = x[col[k]] != 0;
        y[r] = b;
    }
}

/*
 * BFS fixpoint on a square matrix: frontier f0 = visited0 = the sources;
 * f_{t+1} = (M f_t) AND NOT visited_t; visited_{t+1} = visited_t OR f_{t+1};
 * stop when f is empty.  visited: n bytes out.  new_counts[t] = |f_{t+1}| for
 * every executed pass (the last one is 0).  Returns the number of passes, or
 * -1 if max_passes was reached first.
 */
void oracle_spmv_min_plus_f32(int64_t n, const int64_t* row_ptr, const int32_t* col, int kind, const void* val,
                              const float* x, float* y)
{
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t r = 0; r < n; ++r) {
        float m = INFINITY;
        for (int64_t k = row_ptr[r]; k < row_ptr[r + 1]; ++k) {
            const float t = (float)entry(kind, val, k) + x[col[k]];
            if (t < m) m = t;
        }
        y[r] = m;
    }
}

void oracle_spmv_min_plus_f64(int64_t n, const int64_t* row_ptr, const int32_t* col, int kind, const void* val,
                              const double* x, double* y)
{
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t r = 0; r < n; ++r) {
        double m = INFINITY;
        for (int64_t k = row_ptr[r]; k < row_ptr[r + 1]; ++k) {
            const double t = entry(kind, val, k) + x[col[k]];
            if (t < m) m = t;
        }
        y[r] = m;
    }
}

int64_t oracle_bfs(int64_t n, const int64_t* row_ptr, const int32_t* col, const int64_t* sources,
                   int64_t nsrc, uint8_t* visited, int64_t* new_counts, int64_t max_passes)
{
    uint8_t* f = (uint8_t*)calloc((size_t)(n > 0 ? n : 1), 1);
    uint8_t* y = (uint8_t*)calloc((size_t)(n > 0 ? n : 1), 1);
    if (!f || !y) { free(f); free(y); return -2; }
    memset(visited, 0, (size_t)n);
    for (int64_t i = 0; i < nsrc; ++i) { f[sources[i]] = 1; visited[sources[i]] = 1; }
    int64_t passes = 0;
    for (;;) {
        if (passes == max_passes) { passes = -1; break; }
        oracle_spmv_bool(n, row_ptr, col, f, y);
        int64_t cnt = 0;
#pragma omp parallel for reduction(+ : cnt) schedule(static)
        for (int64_t r = 0; r < n; ++r) {
            uint8_t nf = y[r] && !visited[r];
            f[r] = nf;
            visited[r] |= nf;
            cnt += nf;
        }
        new_counts[passes++] = cnt;
        if (cnt == 0) break;
    }
    free(f);
    free(y);
    return passes;
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_threads(int t)
{
#ifdef _OPENMP
    if (t > 0) omp_set_num_threads(t);
#else
    (void)t;
#endif
}
