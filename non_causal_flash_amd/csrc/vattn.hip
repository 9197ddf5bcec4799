// vattn.hip - C ABI of the MI355X head-major attention library: argument
// checks, precision-mode choice and the kernel launch.  See include/vattn.h
// for the contract of every entry point.
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

bool overlaps(const void *a, const void *b, size_t bytes) {
    const uintptr_t pa = reinterpret_cast<uintptr_t>(a);
    const uintptr_t pb = reinterpret_cast<uintptr_t>(b);
    return pa < pb + bytes && pb < pa + bytes;
}

// Correction policy of the SPLIT kernel (see qk_tile): the lo terms go to
// key blocks within `window` (log2 units) of the running max, for waves
// whose running max exceeds `gate` in magnitude.
struct SplitPolicy {
    float window;
    float gate;
};

template <int D, int WAVES, bool SPLIT>
hipError_t launch(const float *q, const float *k, const float *v, float *out,
                  int n_heads, int n_patches, SplitPolicy pol, hipStream_t stream) {
    constexpr int kBlockM = vattn::Shape<D, WAVES>::kBlockM;
    int q_blocks = (n_patches + kBlockM - 1) / kBlockM;
    int total_blocks = q_blocks * n_heads;
    void *args[] = {(void *)&q,        (void *)&k,          (void *)&v,
                    (void *)&out,      (void *)&n_patches,  (void *)&q_blocks,
                    (void *)&total_blocks, (void *)&pol.window, (void *)&pol.gate};
    return hipLaunchKernel(
        reinterpret_cast<const void *>(&vattn::attention_fwd_kernel<D, WAVES, SPLIT>),
        dim3((unsigned)total_blocks), dim3(64 * WAVES), args, 0, stream);
}

// 16-wave workgroups (256 query rows) share each K/V tile among twice the
// queries, halving L2 traffic and conversion work per query; they run one per
// CU.  Use them when they still give every CU at least one workgroup.
template <int D, bool SPLIT>
hipError_t launch_any(const float *q, const float *k, const float *v, float *out,
                      int n_heads, int n_patches, SplitPolicy pol, hipStream_t stream) {
    const int64_t wide_blocks =
        (int64_t)n_heads * (((int64_t)n_patches + vattn::Shape<D, 16>::kBlockM - 1) /
                            vattn::Shape<D, 16>::kBlockM);
    if (wide_blocks >= kCusPerDevice)
        return launch<D, 16, SPLIT>(q, k, v, out, n_heads, n_patches, pol, stream);
    return launch<D, 8, SPLIT>(q, k, v, out, n_heads, n_patches, pol, stream);
}

}  // namespace

extern "C" const char *vattn_status_string(int status) {
    switch (status) {
        case VATTN_OK: return "ok";
        case VATTN_ERR_NULL: return "null tensor pointer";
        case VATTN_ERR_SIZE: return "invalid or too large size";
        case VATTN_ERR_HEAD_DIM: return "head_dim must be 32 or 64";
        case VATTN_ERR_ALIGN: return "tensor not 16-byte aligned";
        case VATTN_ERR_ALIAS: return "out overlaps q, k or v";
        case VATTN_ERR_HIP: return "HIP runtime error";
        case VATTN_ERR_ARG: return "unknown precision mode";
        default: return "unknown status";
    }
}

extern "C" int vattn_last_hip_error(void) { return g_last_hip_error; }

extern "C" int vattn_forward_precision(const float *q, const float *k,
                                       const float *v, float *out, int n_heads,
                                       int n_patches, int head_dim,
                                       int precision, void *stream) {
    if (n_heads < 0 || n_patches < 0) return VATTN_ERR_SIZE;
    if (head_dim != 32 && head_dim != 64) return VATTN_ERR_HEAD_DIM;
    if (precision != VATTN_PRECISION_AUTO && precision != VATTN_PRECISION_FAST &&
        precision != VATTN_PRECISION_SPLIT)
        return VATTN_ERR_ARG;
    if (n_heads == 0 || n_patches == 0) return VATTN_OK;
    if (!q || !k || !v || !out) return VATTN_ERR_NULL;

    // Per-head byte offsets (and buffer-descriptor ranges) are 32-bit signed
    // inside the kernel; the grid is 1-D (at most 128-row blocks).
    const int64_t per_head = (int64_t)n_patches * head_dim;
    const int64_t max_blocks = (int64_t)n_heads * (((int64_t)n_patches + 127) / 128);
    if (per_head * (int64_t)sizeof(float) >= ((int64_t)1 << 31) ||
        max_blocks >= ((int64_t)1 << 31))
        return VATTN_ERR_SIZE;

    const uintptr_t mis = reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) |
                          reinterpret_cast<uintptr_t>(v) | reinterpret_cast<uintptr_t>(out);
    if (mis & 15u) return VATTN_ERR_ALIGN;

    const size_t bytes = (size_t)per_head * (size_t)n_heads * sizeof(float);
    if (overlaps(out, q, bytes) || overlaps(out, k, bytes) || overlaps(out, v, bytes))
        return VATTN_ERR_ALIAS;

    const bool split = precision != VATTN_PRECISION_FAST;
    const float inf = __builtin_inff();
    // SPLIT: every key block, every wave.  AUTO: only near-max blocks of
    // waves whose logits are large (kAutoWindow / kAutoGate).
    const SplitPolicy pol = precision == VATTN_PRECISION_SPLIT ? SplitPolicy{inf, -1.0f}
                                                               : SplitPolicy{kAutoWindow, kAutoGate};
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    hipError_t err;
    if (head_dim == 64)
        err = split ? launch_any<64, true>(q, k, v, out, n_heads, n_patches, pol, s)
                    : launch_any<64, false>(q, k, v, out, n_heads, n_patches, pol, s);
    else
        err = split ? launch_any<32, true>(q, k, v, out, n_heads, n_patches, pol, s)
                    : launch_any<32, false>(q, k, v, out, n_heads, n_patches, pol, s);
    if (err != hipSuccess) {
        g_last_hip_error = (int)err;
        return VATTN_ERR_HIP;
    }
    return VATTN_OK;
}

extern "C" int vattn_forward(const float *q, const float *k, const float *v,
                             float *out, int n_heads, int n_patches,
                             int head_dim, void *stream) {
    return vattn_forward_precision(q, k, v, out, n_heads, n_patches, head_dim,
                                   VATTN_PRECISION_AUTO, stream);
}
