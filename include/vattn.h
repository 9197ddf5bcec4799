/*
 * vattn.h - head-major, non-causal attention over vision patches for
 * AMD Instinct MI355X (gfx950).  C ABI: plain pointers and sizes.
 *
 * The operation (docs.rs page "rullama 0.1.0", source of
 * src/kernels/wgsl/vision_attention_flash_sub_hpd_f16.wgsl: the Params
 * uniform, the storage bindings and the head-major offsets of its Q stage,
 * K/V tile loads and output store):
 *
 *   for every head h < n_heads and patch row i < n_patches
 *     out[h][i][:] = sum_j softmax_j( sum_c q[h][i][c] * k[h][j][c] ) * v[h][j][:]
 *
 * where the softmax runs over every patch j < n_patches (non-causal: the
 * shader visits every key tile for every query; no mask other than the
 * patch count).  No scale is applied inside: the caller folds any 1/sqrt(d)
 * into Q, as the shader's Params carries no scale field.
 *
 * Layout: q, k, v and out are float32 (float16 for the *_f16 entry
 * points).  vattn_forward and vattn_forward_precision take the page's
 * head-major layout, C-contiguous [n_heads][n_patches][head_dim]: element
 * (h, i, c) sits at h*n_patches*head_dim + i*head_dim + c.
 * vattn_forward_strided and the f16 / rotary entry points take any pair of
 * row strides, e.g. the patch-major [n_patches][n_heads][head_dim] layout a
 * fused QKV projection writes (the sibling of the page's head-major "HPD"
 * buffers).
 *
 * Numerics: Q, K, V are rounded to f16 (round-to-nearest-even) for the matrix
 * cores and all sums are accumulated in f32, with an online (running max /
 * running sum) softmax.  The result is not bitwise equal to a float64
 * evaluation; it is within max-abs 2e-3 and relative L2 1e-3 of it for inputs
 * whose logits fit the precision mode (see vattn_precision).  Inputs must be
 * finite with |q * log2(e)| and |k| below 65504 (the f16 range).
 */
#ifndef VATTN_H
#define VATTN_H

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point. */
typedef enum vattn_status {
    VATTN_OK = 0,
    VATTN_ERR_NULL = 1,      /* a tensor pointer is NULL while there is work  */
    VATTN_ERR_SIZE = 2,      /* negative size, strides that make rows overlap,
                                or a size the kernel's 32-bit per-head offsets
                                / grid cannot address                        */
    VATTN_ERR_HEAD_DIM = 3,  /* head_dim is not in [1, 64]                   */
    VATTN_ERR_ALIGN = 4,     /* a tensor base address is not aligned for its
                                access mode (4 elements: 16 bytes of f32 or
                                8 of f16; one element when head_dim or a
                                stride is not a multiple of 4)                */
    VATTN_ERR_ALIAS = 5,     /* out overlaps q, k, v or the rotary table     */
    VATTN_ERR_HIP = 6,       /* the HIP runtime refused the launch           */
    VATTN_ERR_ARG = 7,       /* unknown precision mode                       */
    VATTN_ERR_ROPE = 8       /* invalid rotary parameters (rope_dims, base,
                                factors, positions)                          */
} vattn_status;

/* How the logits q.k are formed on the matrix cores.
 *
 * FAST:  one f16 x f16 product per logit (f32 accumulate).  The error of a
 *        logit is at most 2^-10 sum_c |q_c k_c| (both operands rounded to
 *        f16, relative error 2^-11 each): fine for unit-variance operands
 *        scaled by 1/sqrt(head_dim); aligned operands with logits of more
 *        than ~6 log2 units (~4 nats), or large operands whose products
 *        cancel, miss the tolerance.
 * SPLIT: q = q_hi + q_lo and k = k_hi + k_lo with all four parts f16; the
 *        logit is q_hi.k_hi + q_lo.k_hi + q_hi.k_lo (three f16 products, f32
 *        accumulate), about 2^-21 relative per product, for every key.
 *        Three times the matrix-core work of FAST for the Q.K^T half.
 * AUTO:  SPLIT arithmetic on every key that can carry weight, FAST on the
 *        rest.  Keys are processed in tiles of 64 (128 for small grids);
 *        a 16-key block of a 16-query group gets the two correction
 *        products when some logit of the block lies within 20 log2 units
 *        of its query's running maximum, and on the group's first tile
 *        (before a running maximum exists).  The running maximum never
 *        exceeds the final one, so every key that weighs at least 2^-20 of
 *        the row maximum gets split-f16 logits, whatever the order of the
 *        keys or the size of the operands.  A key further below weighs
 *        less than 2^-20; there f16 P is a subnormal whose spacing (2^-24)
 *        already exceeds what an f16 logit error of ~2^-11 of the logit
 *        changes.  The decision itself uses the f16 logits, whose error is
 *        below 2^-10 sum_c |q_c k_c|: for operands with sum_c |q_c k_c|
 *        above ~4096 (log2 units) a key may be misplaced by more than four
 *        log2 units relative to the window.  With a flat softmax every
 *        block lies in the window and AUTO does SPLIT's work; with a sharp
 *        one (large logits) most blocks fall below it and AUTO skips their
 *        corrections.  Like every mode that rounds P and V to f16, the
 *        result meets max-abs 2e-3 / relative L2 1e-3 as a statistical
 *        property of the rounding, not as a worst case.
 */
typedef enum vattn_precision {
    VATTN_PRECISION_AUTO = 0,
    VATTN_PRECISION_FAST = 1,
    VATTN_PRECISION_SPLIT = 2
} vattn_precision;

/*
 * vattn_forward - enqueue out = softmax(Q K^T) V for every head.
 *
 * q, k, v : device pointers, float32 [n_heads][n_patches][head_dim], read
 *           only; they may alias one another.
 * out     : device pointer, float32, same shape; every element is written.
 *           It must not overlap q, k or v (VATTN_ERR_ALIAS).
 * n_heads, n_patches : >= 0.  If either is 0 the call returns VATTN_OK and
 *           enqueues nothing (pointers may then be NULL).
 *           (n_patches + 63) * head_dim + head_dim must stay below 2^28 (one
 *           head's bytes addressable with 32-bit offsets).
 * head_dim: 1 ... 64.  32 and 64 run the contiguous fast path; other values
 *           are zero-padded to 32 or 64 inside the kernel (the shader's own
 *           limit is head_dim <= 64).
 * stream  : hipStream_t to enqueue on (NULL = the default stream).
 *
 * Ownership: the caller owns all four buffers and keeps them alive until the
 * work on `stream` completes.  The library allocates nothing and is safe to
 * call from several threads; the only state it keeps between calls is each
 * device's compute-unit count, read once (vattn_launch_shape).
 *
 * Errors: arguments are checked synchronously; on any error nothing is
 * enqueued and `out` is untouched.  On VATTN_OK the kernel is enqueued and
 * the call returns without synchronising; faults during execution surface at
 * the caller's next synchronisation, as for any HIP kernel.
 *
 * Equivalent to vattn_forward_precision(..., VATTN_PRECISION_AUTO, stream).
 */
int vattn_forward(const float *q, const float *k, const float *v, float *out,
                  int n_heads, int n_patches, int head_dim, void *stream);

/* As vattn_forward, with an explicit vattn_precision mode (VATTN_ERR_ARG for
 * an unknown one). */
int vattn_forward_precision(const float *q, const float *k, const float *v,
                            float *out, int n_heads, int n_patches,
                            int head_dim, int precision, void *stream);

/*
 * vattn_forward_strided - as vattn_forward_precision, for tensors laid out
 * with any pair of row strides.  Element (h, i, c) of q, k, v and out sits
 * at h*stride_head + i*stride_patch + c (strides in floats, shared by the
 * four tensors; the head_dim elements of a row are contiguous).
 *
 *   head-major  [n_heads][n_patches][head_dim]:
 *       stride_head = n_patches*head_dim, stride_patch = head_dim
 *   patch-major [n_patches][n_heads][head_dim]:
 *       stride_head = head_dim,           stride_patch = n_heads*head_dim
 *
 * Rows must not overlap: stride_patch >= head_dim, stride_head >= head_dim,
 * and either stride_head >= n_patches*stride_patch (heads outermost) or
 * stride_patch >= n_heads*stride_head (patches outermost); otherwise
 * VATTN_ERR_SIZE.  Also VATTN_ERR_SIZE when (n_patches + 63)*stride_patch +
 * head_dim >= 2^28 or stride_patch >= 2^22.  Elements between rows (padding
 * when a stride exceeds the row) are neither read nor written.  Base
 * addresses must be 16-byte aligned, or 4-byte aligned when head_dim or a
 * stride is not a multiple of 4 (that case loads single floats and is
 * slower).  out must not overlap the address range of q, k or v.  Otherwise
 * the contract of vattn_forward holds: synchronous checks, nothing enqueued
 * on error, asynchronous on `stream` on success, no allocation.
 */
int vattn_forward_strided(const float *q, const float *k, const float *v,
                          float *out, int n_heads, int n_patches, int head_dim,
                          long long stride_head, long long stride_patch,
                          int precision, void *stream);

/*
 * vattn_forward_f16 - as vattn_forward_strided for IEEE binary16 (f16)
 * tensors: q, k, v and out hold f16 values (2 bytes each, passed as void
 * pointers since C has no standard half type).  No conversion is needed on
 * the way to the matrix cores and HBM traffic halves.  Products of f16
 * inputs are exact in the f32 accumulator, so the SPLIT/AUTO correction
 * only adds q_lo.k (the query is scaled by log2(e) in f32 and split into
 * two f16 parts).  The result is rounded to f16 (round-to-nearest-even).
 * Strides count f16 elements.  Vector access needs 8-byte aligned bases;
 * 2-byte alignment suffices when head_dim or a stride is not a multiple of
 * 4.  Head-major tensors: stride_head = n_patches*head_dim, stride_patch =
 * head_dim.  Errors and stream semantics as for vattn_forward_strided.
 */
int vattn_forward_f16(const void *q, const void *k, const void *v, void *out,
                      int n_heads, int n_patches, int head_dim,
                      long long stride_head, long long stride_patch,
                      int precision, void *stream);

/*
 * Rotary position transform of Q and K (NeoX pairing).  Source: docs.rs page
 * "rullama 0.2.0", src/kernels/wgsl/rope_neox_backward.wgsl - the forward
 * rotation its header comment states and the angle its main function
 * computes.  For rope_dims <= head_dim and half = rope_dims / 2, the row of
 * a patch at position pos turns its pairs (x[i], x[i + half]), i < half:
 *
 *     theta       = pos * base^(-2 i / rope_dims)  [ / factors[i] ]
 *     x[i]        <- x[i] cos theta - x[i + half] sin theta
 *     x[i + half] <- x[i] sin theta + x[i + half] cos theta
 *
 * and leaves dimensions >= rope_dims unchanged.  The page rotates the rows
 * of one position; here every patch has its own position (1-D patch order).
 */

/*
 * vattn_rope_table - enqueue the (cos, sin) table of the rotary angles.
 *
 * table       : device pointer, float32 [n_positions][rope_dims/2][2], fully
 *               written: table[n][i] = (cos theta, sin theta) for position
 *               pos = pos_offset + n and pair i.  theta, cos and sin are
 *               evaluated in float64 and rounded to float32 (nearest).
 *               16-byte aligned (VATTN_ERR_ALIGN).
 * n_positions : >= 0 (0: nothing to do, table may be NULL); with rope_dims/2
 *               entries per row, n_positions * rope_dims/2 < 2^31.
 * rope_dims   : even, 2 ... 64.
 * base        : finite and > 0 (the page's frequency base, e.g. 10000).
 * factors     : HOST pointer to rope_dims/2 finite values > 0 that divide the
 *               angles (the page's optional factors buffer), or NULL; read
 *               during the call only.
 * pos_offset  : position of row 0, >= 0; pos_offset + n_positions - 1 must fit
 *               an int.
 * Errors: VATTN_ERR_ROPE (rope_dims, base, factors, positions), VATTN_ERR_SIZE
 * (n_positions), VATTN_ERR_NULL, VATTN_ERR_ALIGN, VATTN_ERR_HIP; checked
 * synchronously, nothing enqueued on error.  No allocation.
 */
int vattn_rope_table(float *table, int n_positions, int rope_dims, float base,
                     const float *factors, int pos_offset, void *stream);

/*
 * vattn_forward_rope - vattn_forward_strided with the rotary transform
 * applied to q and k (not v) inside the kernel: out = softmax(rot(Q)
 * rot(K)^T) V, where row i of every head is rotated with table row i (the
 * position of patch i).  The rotation is done in f32 before the f16
 * rounding; the rotated tensors are never written to memory and q, k stay
 * unchanged.
 *
 * rope_dims  : multiple of 8, 8 ... head_dim (VATTN_ERR_ROPE otherwise).
 * rope_table : device pointer to a table from vattn_rope_table with the same
 *              rope_dims and at least n_patches rows (not checked), 16-byte
 *              aligned; read only.  out must not overlap its first n_patches
 *              rows (VATTN_ERR_ALIAS).
 * Every other argument, error and the stream semantics as for
 * vattn_forward_strided.  With f16 tensors the rotated K is not exact in f16,
 * so SPLIT / AUTO also correct with q_hi.k_lo, as for f32 inputs.
 */
int vattn_forward_rope(const float *q, const float *k, const float *v,
                       float *out, int n_heads, int n_patches, int head_dim,
                       long long stride_head, long long stride_patch,
                       int rope_dims, const float *rope_table, int precision,
                       void *stream);

/* vattn_forward_rope for f16 tensors (as vattn_forward_f16); the table stays
 * float32. */
int vattn_forward_rope_f16(const void *q, const void *k, const void *v,
                           void *out, int n_heads, int n_patches, int head_dim,
                           long long stride_head, long long stride_patch,
                           int rope_dims, const float *rope_table,
                           int precision, void *stream);

/* Workgroup shapes of the attention kernel (values of vattn_launch_shape). */
typedef enum vattn_shape {
    VATTN_SHAPE_SPLIT_KEYS = 1,  /* 64 query rows, 16 waves = 4 row groups x 4
                                    key chunks, states merged in LDS        */
    VATTN_SHAPE_4_WAVES = 4,     /* 64 query rows (rotary kernels only)     */
    VATTN_SHAPE_8_WAVES = 8,     /* 128 query rows                          */
    VATTN_SHAPE_16_WAVES = 16    /* 256 query rows, one workgroup per CU    */
} vattn_shape;

/*
 * vattn_launch_shape - the workgroup shape every attention entry point
 * launches for n_heads x n_patches rows (rotary: rope != 0) on a device with
 * cu_count compute units.  Host-only: touches no device.  The entry points
 * call it with the CU count of the stream's device, queried once per device
 * (hipDeviceAttributeMultiprocessorCount).  Rule, with W = n_heads *
 * ceil(n_patches / 256) and S = n_heads * ceil(n_patches / 64):
 *   16 waves  if 2W > cu_count (rotary: 2W >= cu_count);
 *   rotary:   4 waves otherwise;
 *   8 waves   if 2W >= cu_count;
 *   split-key if S <= cu_count;
 *   8 waves   otherwise.
 * head_dim (1 ... 64) does not change the shape.  Returns a vattn_shape
 * value, or -VATTN_ERR_SIZE when a size is < 1, head_dim > 64 or
 * cu_count < 1.
 */
int vattn_launch_shape(int n_heads, int n_patches, int head_dim, int rope, int cu_count);

/* Static, never-NULL description of a status code ("unknown status" for
 * values outside vattn_status). */
const char *vattn_status_string(int status);

/* HIP error code (hipError_t) behind the last VATTN_ERR_HIP returned on the
 * calling thread; 0 if none. */
int vattn_last_hip_error(void);

#ifdef __cplusplus
}
#endif
#endif /* VATTN_H */
