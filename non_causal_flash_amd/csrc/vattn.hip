// vattn.hip - C ABI of the MI355X vision-attention library: argument checks,
// precision-mode and access-mode choice and the kernel launch.  See
// include/vattn.h for the contract of every entry point.
#include "vattn.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attention_fwd.hpp"

namespace {

thread_local int g_last_hip_error = 0;

constexpr int64_t kCusPerDevice = 256;  // MI355X compute units

// AUTO precision: lo terms for key blocks within 16 log2 units (weight
// > 2^-16) of the running max, in waves whose running max exceeds 24 log2
// units in magnitude (f16 logit error ~2^-11 * |logit| > 0.01).
constexpr float kAutoWindow = 16.0f;
constexpr float kAutoGate = 24.0f;

// Largest per-head element span the kernel addresses with 32-bit byte
// offsets, with headroom below the out-of-range offset the strided loads
// use for padding columns.
constexpr int64_t kMaxSpan = (int64_t)1 << 28;

bool overlaps(uintptr_t a, uintptr_t a_bytes, uintptr_t b, uintptr_t b_bytes) {
    return a < b + b_bytes && b < a + a_bytes;
}

// Correction policy of the SPLIT kernel (see qk_tile): the lo terms go to
// key blocks within `window` (log2 units) of the running max, for waves
// whose running max exceeds `gate` in magnitude.
struct SplitPolicy {
    float window;
    float gate;
};

template <int D, int WAVES, bool SPLIT, int IO, typename T>
hipError_t launch(const T *q, const T *k, const T *v, T *out,
                  int n_heads, int n_patches, SplitPolicy pol, vattn::Io io,
                  hipStream_t stream) {
    constexpr int kBlockM = vattn::Shape<D, WAVES>::kBlockM;
    int q_blocks = (n_patches + kBlockM - 1) / kBlockM;
    int total_blocks = q_blocks * n_heads;
    void *args[] = {(void *)&q,           (void *)&k,          (void *)&v,
                    (void *)&out,         (void *)&n_patches,  (void *)&q_blocks,
                    (void *)&total_blocks, (void *)&pol.window, (void *)&pol.gate,
                    (void *)&io};
    return hipLaunchKernel(
        reinterpret_cast<const void *>(&vattn::attention_fwd_kernel<D, WAVES, SPLIT, IO, T>),
        dim3((unsigned)total_blocks), dim3(64 * WAVES), args, 0, stream);
}

// 16-wave workgroups (256 query rows) share each K/V tile among twice the
// queries, halving L2 traffic and conversion work per query; they run one per
// CU.  Use them when they still give every CU at least one workgroup.
template <int D, bool SPLIT, int IO, typename T>
hipError_t launch_any(const T *q, const T *k, const T *v, T *out,
                      int n_heads, int n_patches, SplitPolicy pol, vattn::Io io,
                      hipStream_t stream) {
    const int64_t wide_blocks =
        (int64_t)n_heads * (((int64_t)n_patches + vattn::Shape<D, 16>::kBlockM - 1) /
                            vattn::Shape<D, 16>::kBlockM);
    if (wide_blocks >= kCusPerDevice)
        return launch<D, 16, SPLIT, IO, T>(q, k, v, out, n_heads, n_patches, pol, io, stream);
    return launch<D, 8, SPLIT, IO, T>(q, k, v, out, n_heads, n_patches, pol, io, stream);
}

template <int D, int IO, typename T>
hipError_t launch_mode(const T *q, const T *k, const T *v, T *out,
                       int n_heads, int n_patches, bool split, SplitPolicy pol,
                       vattn::Io io, hipStream_t stream) {
    return split ? launch_any<D, true, IO>(q, k, v, out, n_heads, n_patches, pol, io, stream)
                 : launch_any<D, false, IO>(q, k, v, out, n_heads, n_patches, pol, io, stream);
}

template <int D, typename T>
hipError_t launch_io(const T *q, const T *k, const T *v, T *out,
                     int n_heads, int n_patches, bool split, SplitPolicy pol, vattn::Io io,
                     int mode, hipStream_t stream) {
    if (mode == vattn::kIoDense)
        return launch_mode<D, vattn::kIoDense>(q, k, v, out, n_heads, n_patches, split, pol, io, stream);
    if (mode == vattn::kIoVec4)
        return launch_mode<D, vattn::kIoVec4>(q, k, v, out, n_heads, n_patches, split, pol, io, stream);
    return launch_mode<D, vattn::kIoScalar>(q, k, v, out, n_heads, n_patches, split, pol, io, stream);
}

// Checks and dispatch shared by the f32 and f16 entry points.
template <typename T>
int forward_impl(const T *q, const T *k, const T *v, T *out, int n_heads, int n_patches,
                 int head_dim, long long stride_head, long long stride_patch, int precision,
                 void *stream) {
    if (n_heads < 0 || n_patches < 0) return VATTN_ERR_SIZE;
    if (head_dim < 1 || head_dim > 64) return VATTN_ERR_HEAD_DIM;
    if (precision != VATTN_PRECISION_AUTO && precision != VATTN_PRECISION_FAST &&
        precision != VATTN_PRECISION_SPLIT)
        return VATTN_ERR_ARG;
    if (n_heads == 0 || n_patches == 0) return VATTN_OK;
    if (!q || !k || !v || !out) return VATTN_ERR_NULL;

    // Strides: rows of head_dim elements that never overlap.  Either the
    // heads are outermost (stride_head covers a whole head) or the patches
    // are (stride_patch covers a whole patch of all heads).
    const int64_t sh = stride_head, sn = stride_patch, d = head_dim;
    const int64_t H = n_heads, N = n_patches;
    if (sn < d || sh < d || (sh < N * sn && sn < H * sh)) return VATTN_ERR_SIZE;
    // Per-head byte offsets (and buffer-descriptor ranges) are 32-bit inside
    // the kernel; the grid is 1-D.
    const int64_t span = (N - 1 + vattn::kTileN) * sn + d;
    const int64_t max_blocks = H * ((N + 127) / 128);
    if (span >= kMaxSpan || max_blocks >= ((int64_t)1 << 31) || sn >= ((int64_t)1 << 22))
        return VATTN_ERR_SIZE;

    const int D = head_dim <= 32 ? 32 : 64;
    int mode;
    if (head_dim == D && sn == d && sh == N * d)
        mode = vattn::kIoDense;
    else if (d % 4 == 0 && sn % 4 == 0 && sh % 4 == 0)
        mode = vattn::kIoVec4;
    else
        mode = vattn::kIoScalar;

    // Vector modes move 4-element vectors (16 bytes of f32, 8 of f16).
    const uintptr_t align = mode == vattn::kIoScalar ? sizeof(T) : 4 * sizeof(T);
    const uintptr_t mis = reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) |
                          reinterpret_cast<uintptr_t>(v) | reinterpret_cast<uintptr_t>(out);
    if (mis & (align - 1)) return VATTN_ERR_ALIGN;

    const uintptr_t bytes = (uintptr_t)(((H - 1) * sh + (N - 1) * sn + d) * (int64_t)sizeof(T));
    const uintptr_t po = reinterpret_cast<uintptr_t>(out);
    if (overlaps(po, bytes, reinterpret_cast<uintptr_t>(q), bytes) ||
        overlaps(po, bytes, reinterpret_cast<uintptr_t>(k), bytes) ||
        overlaps(po, bytes, reinterpret_cast<uintptr_t>(v), bytes))
        return VATTN_ERR_ALIAS;

    const bool split = precision != VATTN_PRECISION_FAST;
    const float inf = __builtin_inff();
    // SPLIT: every key block, every wave.  AUTO: only near-max blocks of
    // waves whose logits are large (kAutoWindow / kAutoGate).
    const SplitPolicy pol = precision == VATTN_PRECISION_SPLIT ? SplitPolicy{inf, -1.0f}
                                                               : SplitPolicy{kAutoWindow, kAutoGate};
    const vattn::Io io{stride_head, (int)stride_patch, head_dim};
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const hipError_t err =
        D == 64 ? launch_io<64>(q, k, v, out, n_heads, n_patches, split, pol, io, mode, s)
                : launch_io<32>(q, k, v, out, n_heads, n_patches, split, pol, io, mode, s);
    if (err != hipSuccess) {
        g_last_hip_error = (int)err;
        return VATTN_ERR_HIP;
    }
    return VATTN_OK;
}

}  // namespace

extern "C" const char *vattn_status_string(int status) {
    switch (status) {
        case VATTN_OK: return "ok";
        case VATTN_ERR_NULL: return "null tensor pointer";
        case VATTN_ERR_SIZE: return "invalid or too large size or stride";
        case VATTN_ERR_HEAD_DIM: return "head_dim must be in [1, 64]";
        case VATTN_ERR_ALIGN: return "tensor not aligned for its access mode";
        case VATTN_ERR_ALIAS: return "out overlaps q, k or v";
        case VATTN_ERR_HIP: return "HIP runtime error";
        case VATTN_ERR_ARG: return "unknown precision mode";
        default: return "unknown status";
    }
}

extern "C" int vattn_last_hip_error(void) { return g_last_hip_error; }

extern "C" int vattn_forward_strided(const float *q, const float *k, const float *v,
                                     float *out, int n_heads, int n_patches,
                                     int head_dim, long long stride_head,
                                     long long stride_patch, int precision, void *stream) {
    return forward_impl<float>(q, k, v, out, n_heads, n_patches, head_dim, stride_head,
                               stride_patch, precision, stream);
}

extern "C" int vattn_forward_f16(const void *q, const void *k, const void *v, void *out,
                                 int n_heads, int n_patches, int head_dim,
                                 long long stride_head, long long stride_patch,
                                 int precision, void *stream) {
    return forward_impl<_Float16>(static_cast<const _Float16 *>(q), static_cast<const _Float16 *>(k),
                                  static_cast<const _Float16 *>(v), static_cast<_Float16 *>(out),
                                  n_heads, n_patches, head_dim, stride_head, stride_patch,
                                  precision, stream);
}

extern "C" int vattn_forward_precision(const float *q, const float *k,
                                       const float *v, float *out, int n_heads,
                                       int n_patches, int head_dim,
                                       int precision, void *stream) {
    if (n_heads < 0 || n_patches < 0) return VATTN_ERR_SIZE;
    return vattn_forward_strided(q, k, v, out, n_heads, n_patches, head_dim,
                                 (long long)n_patches * head_dim, head_dim, precision, stream);
}

extern "C" int vattn_forward(const float *q, const float *k, const float *v,
                             float *out, int n_heads, int n_patches,
                             int head_dim, void *stream) {
    return vattn_forward_precision(q, k, v, out, n_heads, n_patches, head_dim,
                                   VATTN_PRECISION_AUTO, stream);
}
