/*
 * vattn_oracle.c - plain float64 CPU reference, TEST INFRASTRUCTURE ONLY.
 *
 * Follows the docs.rs page "rullama 0.1.0",
 * src/kernels/wgsl/vision_attention_flash_sub_hpd_f16.wgsl:
 *   - the head-major offsets head*n_patches*head_dim + row*head_dim + dim
 *     used for the Q stage, the K/V tile loads and the output store;
 *   - the score as a plain dot product of a query row with a key row, with
 *     no scale (the Params uniform carries none; callers pre-scale Q);
 *   - every key tile is visited for every query (non-causal, no mask other
 *     than n_patches itself);
 *   - max-subtracted exponentials, their sum l, and the value rows weighted
 *     by the probabilities, divided by l in the epilogue.
 * The shader's f16 rounding of Q, K, V and P and its online rescale are
 * implementation choices of a fast kernel; the definition it approximates is
 * written out here directly, in float64, with no blocking or reordering.
 *
 * The optional rotary position transform of Q and K follows the docs.rs page
 * "rullama 0.2.0", src/kernels/wgsl/rope_neox_backward.wgsl: the forward
 * NeoX rotation its header comment states (pairs x[i], x[i + rope_dims/2])
 * and the angle pos * base^(-2i/rope_dims), divided by factors[i] when
 * factors are given, that its main function computes.  Here every patch
 * has its own position, pos_offset + patch index.
 *
 * Built with gcc (C99 + OpenMP); no GPU code, no shared headers with the
 * GPU library.
 */
#include "vattn_oracle.h"

#include <math.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* One query row: q_row[d] against the head's keys/values k_head, v_head
 * ([n][d] each).  s is caller scratch of n doubles.  Writes out_row[d]. */
static void attend_row(const double *q_row, const double *k_head,
                       const double *v_head, long n, long d, double *s,
                       double *out_row)
{
    /* logits s_j = q . k_j */
    for (long j = 0; j < n; ++j) {
        double acc = 0.0;
        for (long c = 0; c < d; ++c)
            acc += q_row[c] * k_head[j * d + c];
        s[j] = acc;
    }
    /* row maximum */
    double m = s[0];
    for (long j = 1; j < n; ++j)
        if (s[j] > m) m = s[j];
    /* e_j = exp(s_j - m), l = sum_j e_j */
    double l = 0.0;
    for (long j = 0; j < n; ++j) {
        s[j] = exp(s[j] - m);
        l += s[j];
    }
    /* out = (sum_j e_j v_j) / l */
    for (long c = 0; c < d; ++c) out_row[c] = 0.0;
    for (long j = 0; j < n; ++j)
        for (long c = 0; c < d; ++c)
            out_row[c] += s[j] * v_head[j * d + c];
    for (long c = 0; c < d; ++c) out_row[c] /= l;
}

static int run_rows(const double *q, const double *k, const double *v,
                    long n_heads, long n_patches, long head_dim,
                    const long *rows, long n_rows, double *out,
                    int n_threads)
{
    if (n_heads < 0 || n_patches < 0 || head_dim < 0 || n_rows < 0) return -1;
    if (n_rows == 0 || head_dim == 0) return 0;
    if (!q || !k || !v || !out) return -1;
    const long total = n_heads * n_patches;
    if (rows) {
        for (long r = 0; r < n_rows; ++r)
            if (rows[r] < 0 || rows[r] >= total) return -1;
    }
    int status = 0;
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#else
    (void)n_threads;
#endif
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)n_patches);
        if (!s) {
#pragma omp atomic write
            status = -2;
        } else {
#pragma omp for schedule(dynamic, 16)
            for (long r = 0; r < n_rows; ++r) {
                const long row = rows ? rows[r] : r;
                const long h = row / n_patches;
                const long i = row % n_patches;
                const long head_base = h * n_patches * head_dim;
                attend_row(q + head_base + i * head_dim, k + head_base,
                           v + head_base, n_patches, head_dim, s,
                           out + r * head_dim);
            }
            free(s);
        }
    }
    return status;
}

int vattn_oracle_f64(const double *q, const double *k, const double *v,
                     double *out, long n_heads, long n_patches,
                     long head_dim, int n_threads)
{
    if (n_heads < 0 || n_patches < 0 || head_dim < 0) return -1;
    return run_rows(q, k, v, n_heads, n_patches, head_dim, NULL,
                    n_heads * n_patches, out, n_threads);
}

int vattn_oracle_rows_f64(const double *q, const double *k, const double *v,
                          long n_heads, long n_patches, long head_dim,
                          const long *rows, long n_rows, double *out_rows,
                          int n_threads)
{
    if (n_rows > 0 && !rows) return -1;
    return run_rows(q, k, v, n_heads, n_patches, head_dim, rows, n_rows,
                    out_rows, n_threads);
}

int vattn_oracle_rope_f64(const double *x, double *y, long n_heads,
                          long n_patches, long head_dim, long rope_dims,
                          double base, const double *factors,
                          long pos_offset)
{
    if (n_heads < 0 || n_patches < 0 || head_dim < 0 || pos_offset < 0)
        return -1;
    if (rope_dims < 0 || rope_dims > head_dim || rope_dims % 2 != 0)
        return -1;
    if (n_heads * n_patches * head_dim == 0) return 0;
    if (!x || !y) return -1;
    const long half = rope_dims / 2;
    for (long h = 0; h < n_heads; ++h) {
        for (long n = 0; n < n_patches; ++n) {
            const double *xr = x + (h * n_patches + n) * head_dim;
            double *yr = y + (h * n_patches + n) * head_dim;
            for (long c = 0; c < head_dim; ++c) yr[c] = xr[c];
            const double pos = (double)(pos_offset + n);
            for (long i = 0; i < half; ++i) {
                double theta = pos * pow(base, -2.0 * (double)i / (double)rope_dims);
                if (factors) theta = theta / factors[i];
                const double cs = cos(theta);
                const double sn = sin(theta);
                const double a = xr[i];
                const double b = xr[i + half];
                yr[i] = a * cs - b * sn;
                yr[i + half] = a * sn + b * cs;
            }
        }
    }
    return 0;
}
