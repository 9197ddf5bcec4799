/*
 * vattn_oracle.h - plain CPU reference for head-major, non-causal attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * CPU-baseline leg of the benchmark load this library.  The GPU library
 * never links, includes or calls it, and it shares no code with it.
 *
 * What it computes (source: docs.rs page "rullama 0.1.0",
 * src/kernels/wgsl/vision_attention_flash_sub_hpd_f16.wgsl): for every head
 * h and query row i of tensors laid out [n_heads][n_patches][head_dim]
 * (the shader's offset head*n_patches*head_dim + row*head_dim + dim),
 *
 *     s_j        = sum_c q[h,i,c] * k[h,j,c]        (no scale applied)
 *     p_j        = exp(s_j - max_j s_j) / sum_j exp(s_j - max_j s_j)
 *     out[h,i,c] = sum_j p_j * v[h,j,c]
 *
 * over all j < n_patches (non-causal: the shader visits every key tile for
 * every query).  The shader reaches this with an online (running max /
 * running sum) softmax, which is algebraically the same result; this oracle
 * writes out the plain two-pass definition in float64 (float32 and float16
 * tensors are promoted exactly by the caller).
 *
 * The rotary transform (source: docs.rs page "rullama 0.2.0",
 * src/kernels/wgsl/rope_neox_backward.wgsl: the forward rotation stated in
 * its header comment and the angle its main function computes) rotates the
 * NeoX pairs (x[i], x[i + rope_dims/2]), i < rope_dims/2, of every row by
 *
 *     theta(pos, i) = pos * base^(-2i / rope_dims)   [ / factors[i] ]
 *
 *     x[i]        <- x[i] cos theta - x[i + half] sin theta
 *     x[i + half] <- x[i] sin theta + x[i + half] cos theta
 *
 * with pos = pos_offset + patch index (one position per patch); dimensions
 * from rope_dims on pass through unchanged.
 *
 * Status codes: 0 on success; -1 for a NULL pointer with work to do or a
 * negative size; -2 when scratch memory cannot be allocated.
 */
#ifndef VATTN_ORACLE_H
#define VATTN_ORACLE_H

#ifdef __cplusplus
extern "C" {
#endif

/* Full tensor.  q, k, v: host float64 [n_heads][n_patches][head_dim];
 * out: host float64, same shape, fully written.  n_threads <= 0 uses the
 * OpenMP default.  Parity unaffected by n_threads (rows are independent). */
int vattn_oracle_f64(const double *q, const double *k, const double *v,
                     double *out, long n_heads, long n_patches,
                     long head_dim, int n_threads);

/* Selected rows only.  rows[r] = h * n_patches + i names the query row;
 * out_rows is host float64 [n_rows][head_dim].  Same arithmetic per row as
 * vattn_oracle_f64.  A row index outside [0, n_heads*n_patches) gives -1. */
int vattn_oracle_rows_f64(const double *q, const double *k, const double *v,
                          long n_heads, long n_patches, long head_dim,
                          const long *rows, long n_rows, double *out_rows,
                          int n_threads);

/* Rotary transform of x (host float64 [n_heads][n_patches][head_dim]) into
 * y (same shape, fully written; may not overlap x).  rope_dims must be even
 * and in [0, head_dim]; factors is NULL or rope_dims/2 divisors of the
 * angles; pos_offset >= 0.  Bad arguments give -1. */
int vattn_oracle_rope_f64(const double *x, double *y, long n_heads,
                          long n_patches, long head_dim, long rope_dims,
                          double base, const double *factors,
                          long pos_offset);

#ifdef __cplusplus
}
#endif
#endif
