// vattn.hip - C ABI of the MI355X vision-attention library: argument checks,
// precision-mode and access-mode choice and the kernel launch.  See
// include/vattn.h for the contract of every entry point.
#include "vattn.h"

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <atomic>

#include "attention_fwd.hpp"

namespace vattn {

// Rotary table: angles pos * w[i], w[i] = base^(-2i/rope_dims) / factors[i]
// (computed on the host in double precision).
struct RopeFreqs {
    double w[32];
};

// One thread per (position, pair): cos and sin of the float64 angle,
// rounded to float32, stored as one float2 (vector store).
__global__ void __launch_bounds__(256)
rope_table_kernel(float *table, int n_positions, int half, int pos_offset, RopeFreqs f) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (int64_t)n_positions * half) return;
    const int n = (int)(idx / half);
    const int i = (int)(idx - (int64_t)n * half);
    const double theta = (double)(pos_offset + n) * f.w[i];
    double sn, cs;
    sincos(theta, &sn, &cs);
    reinterpret_cast<float2_t *>(table)[idx] = (float2_t){(float)cs, (float)sn};
}

}  // namespace vattn

namespace {

thread_local int g_last_hip_error = 0;

// AUTO policy (vattn::AutoPolicy): split-f16 logits for every 16-key block
// that holds a logit within 20 log2 units of its query's running max.  A
// key further below weighs less than 2^-20 of the row maximum; there f16
// P is a subnormal whose spacing (2^-24) already exceeds what the f16
// logit error (~2^-11 of the logit) changes.
constexpr float kAutoWindow = 20.0f;

// Largest per-head element span the kernel addresses with 32-bit byte
// offsets, with headroom below the out-of-range offset the strided loads
// use for padding columns.
constexpr int64_t kMaxSpan = (int64_t)1 << 28;

bool overlaps(uintptr_t a, uintptr_t a_bytes, uintptr_t b, uintptr_t b_bytes) {
    return a < b + b_bytes && b < a + a_bytes;
}

// Everything a launch needs besides the tensor pointers.
struct LaunchArgs {
    int n_heads;
    int n_patches;
    vattn::AutoPolicy pol;
    vattn::Io io;
    vattn::Rope rope;
    hipStream_t stream;
};

template <int D, int WAVES, int PREC, int IO, typename T, bool ROPE>
hipError_t launch(const T *q, const T *k, const T *v, T *out, const LaunchArgs &a) {
    constexpr int kBlockM = vattn::Shape<D, WAVES>::kBlockM;
    int n_patches = a.n_patches;
    int q_blocks = (n_patches + kBlockM - 1) / kBlockM;
    int total_blocks = q_blocks * a.n_heads;
    vattn::AutoPolicy pol = a.pol;
    vattn::Io io = a.io;
    vattn::Rope rope = a.rope;
    void *args[] = {(void *)&q,         (void *)&k,        (void *)&v,
                    (void *)&out,       (void *)&n_patches, (void *)&q_blocks,
                    (void *)&total_blocks, (void *)&pol,   (void *)&io,
                    (void *)&rope};
    return hipLaunchKernel(
        reinterpret_cast<const void *>(&vattn::attention_fwd_kernel<D, WAVES, PREC, IO, T, ROPE>),
        dim3((unsigned)total_blocks), dim3(64 * WAVES), args, 0, a.stream);
}

template <int D, int PREC, int IO, typename T>
hipError_t launch_split_keys(const T *q, const T *k, const T *v, T *out, const LaunchArgs &a) {
    int n_patches = a.n_patches;
    int q_blocks = (n_patches + vattn::kSplitBlockM - 1) / vattn::kSplitBlockM;
    int total_blocks = q_blocks * a.n_heads;
    vattn::AutoPolicy pol = a.pol;
    vattn::Io io = a.io;
    void *args[] = {(void *)&q,         (void *)&k,         (void *)&v,
                    (void *)&out,       (void *)&n_patches, (void *)&q_blocks,
                    (void *)&total_blocks, (void *)&pol,    (void *)&io};
    return hipLaunchKernel(
        reinterpret_cast<const void *>(&vattn::attention_fwd_split_kernel<D, PREC, IO, T>),
        dim3((unsigned)total_blocks), dim3(1024), args, 0, a.stream);
}

// Compute units of the device that owns `stream` (NULL: the current
// device), queried once per device.
constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];

hipError_t device_cu_count(hipStream_t stream, int *cus) {
    int dev = 0;
    hipError_t err = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev >= 0 && dev < kMaxDevices) {
        const int cached = g_cu_count[dev].load(std::memory_order_relaxed);
        if (cached > 0) {
            *cus = cached;
            return hipSuccess;
        }
    }
    int n = 0;
    err = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (err != hipSuccess) return err;
    if (n < 1) n = 1;
    if (dev >= 0 && dev < kMaxDevices) g_cu_count[dev].store(n, std::memory_order_relaxed);
    *cus = n;
    return hipSuccess;
}

}  // namespace

// Workgroup shape (see vattn_launch_shape in vattn.h).  16 waves (256 query
// rows) share each K/V tile among the most queries (least L2 traffic and
// conversion work per query) and run one per CU: used when there are more
// of them than half the CUs.  Then 8-wave blocks would put two workgroups
// on some CUs, whose 256 rows match the 16-wave block's, but convert each
// K/V tile twice (AUTO 5-10% slower at 144-204 blocks on 256 CUs).  With
// at most half as many, 8-wave blocks (128 rows) give each CU one
// workgroup: used while there are as many of them as CUs.  Below that,
// the split-key kernel over 64-row blocks (16 waves, 4 per SIMD) while
// there is at most one such block per CU.  The grids left over (more
// 64-row blocks than CUs, hence more than a quarter of the CUs in wide
// blocks) run 8-wave blocks on fewer CUs, which beats 64-row 4-wave blocks
// at one wave per SIMD (3-6% on 20-40 heads of 600-1000 patches).  The
// rotary kernels skip the 8-wave (it would spill) and split-key steps: 16
// waves from half as many blocks as CUs, 4-wave blocks below.
extern "C" int vattn_launch_shape(int n_heads, int n_patches, int head_dim, int rope,
                                  int cu_count) {
    if (n_heads < 1 || n_patches < 1 || head_dim < 1 || head_dim > 64 || cu_count < 1)
        return -VATTN_ERR_SIZE;
    const int64_t cus = cu_count;
    const int64_t wide_blocks = (int64_t)n_heads * (((int64_t)n_patches + 255) / 256);
    if (rope ? 2 * wide_blocks >= cus : 2 * wide_blocks > cus) return VATTN_SHAPE_16_WAVES;
    if (rope) return VATTN_SHAPE_4_WAVES;
    if (2 * wide_blocks >= cus) return VATTN_SHAPE_8_WAVES;
    const int64_t small_blocks = (int64_t)n_heads * (((int64_t)n_patches + 63) / 64);
    if (small_blocks <= cus) return VATTN_SHAPE_SPLIT_KEYS;
    return VATTN_SHAPE_8_WAVES;
}

namespace {

template <int D, int PREC, int IO, typename T, bool ROPE>
hipError_t launch_any(const T *q, const T *k, const T *v, T *out, int cus, const LaunchArgs &a) {
    static_assert(vattn::Shape<D, 16>::kBlockM == 256 && vattn::kSplitBlockM == 64,
                  "vattn_launch_shape counts 256- and 64-row blocks");
    const int shape = vattn_launch_shape(a.n_heads, a.n_patches, a.io.head_dim, ROPE, cus);
    if (shape == VATTN_SHAPE_16_WAVES) return launch<D, 16, PREC, IO, T, ROPE>(q, k, v, out, a);
    if constexpr (ROPE) {
        return launch<D, 4, PREC, IO, T, ROPE>(q, k, v, out, a);
    } else {
        if (shape == VATTN_SHAPE_SPLIT_KEYS)
            return launch_split_keys<D, PREC, IO, T>(q, k, v, out, a);
        return launch<D, 8, PREC, IO, T, ROPE>(q, k, v, out, a);
    }
}

template <int D, int IO, typename T, bool ROPE>
hipError_t launch_mode(const T *q, const T *k, const T *v, T *out, int precision, int cus,
                       const LaunchArgs &a) {
    if (precision == VATTN_PRECISION_FAST)
        return launch_any<D, vattn::kPrecFast, IO, T, ROPE>(q, k, v, out, cus, a);
    if (precision == VATTN_PRECISION_SPLIT)
        return launch_any<D, vattn::kPrecSplit, IO, T, ROPE>(q, k, v, out, cus, a);
    return launch_any<D, vattn::kPrecAuto, IO, T, ROPE>(q, k, v, out, cus, a);
}

template <int D, typename T, bool ROPE>
hipError_t launch_io(const T *q, const T *k, const T *v, T *out, int precision, int mode,
                     int cus, const LaunchArgs &a) {
    if (mode == vattn::kIoDense)
        return launch_mode<D, vattn::kIoDense, T, ROPE>(q, k, v, out, precision, cus, a);
    if (mode == vattn::kIoVec4)
        return launch_mode<D, vattn::kIoVec4, T, ROPE>(q, k, v, out, precision, cus, a);
    return launch_mode<D, vattn::kIoScalar, T, ROPE>(q, k, v, out, precision, cus, a);
}

template <typename T, bool ROPE>
hipError_t launch_dim(const T *q, const T *k, const T *v, T *out, int precision, int mode,
                      int D, int cus, const LaunchArgs &a) {
    return D == 64 ? launch_io<64, T, ROPE>(q, k, v, out, precision, mode, cus, a)
                   : launch_io<32, T, ROPE>(q, k, v, out, precision, mode, cus, a);
}

// Checks and dispatch shared by every attention entry point.  rope_dims = 0
// (and no table): no rotary transform.
template <typename T>
int forward_impl(const T *q, const T *k, const T *v, T *out, int n_heads, int n_patches,
                 int head_dim, long long stride_head, long long stride_patch, int precision,
                 int rope_dims, const float *rope_table, void *stream) {
    if (n_heads < 0 || n_patches < 0) return VATTN_ERR_SIZE;
    if (head_dim < 1 || head_dim > 64) return VATTN_ERR_HEAD_DIM;
    if (precision != VATTN_PRECISION_AUTO && precision != VATTN_PRECISION_FAST &&
        precision != VATTN_PRECISION_SPLIT)
        return VATTN_ERR_ARG;
    const bool rope = rope_dims != 0;
    // Rotary pairs move in 4-column vectors: half = rope_dims/2 must be a
    // multiple of 4 so no vector straddles half or rope_dims.
    if (rope && (rope_dims < 8 || rope_dims % 8 != 0 || rope_dims > head_dim))
        return VATTN_ERR_ROPE;
    if (n_heads == 0 || n_patches == 0) return VATTN_OK;
    if (!q || !k || !v || !out || (rope && !rope_table)) return VATTN_ERR_NULL;

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
    if (rope && (reinterpret_cast<uintptr_t>(rope_table) & 15)) return VATTN_ERR_ALIGN;

    const uintptr_t bytes = (uintptr_t)(((H - 1) * sh + (N - 1) * sn + d) * (int64_t)sizeof(T));
    const uintptr_t po = reinterpret_cast<uintptr_t>(out);
    if (overlaps(po, bytes, reinterpret_cast<uintptr_t>(q), bytes) ||
        overlaps(po, bytes, reinterpret_cast<uintptr_t>(k), bytes) ||
        overlaps(po, bytes, reinterpret_cast<uintptr_t>(v), bytes))
        return VATTN_ERR_ALIAS;
    if (rope && overlaps(po, bytes, reinterpret_cast<uintptr_t>(rope_table),
                         (uintptr_t)(N * (rope_dims / 2) * 8)))
        return VATTN_ERR_ALIAS;

    const vattn::AutoPolicy pol{kAutoWindow};
    const hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    const LaunchArgs a{n_heads, n_patches, pol, vattn::Io{stride_head, (int)stride_patch, head_dim},
                       vattn::Rope{rope_table, rope_dims / 2}, hs};
    int cus = 0;
    hipError_t err = device_cu_count(hs, &cus);
    if (err == hipSuccess)
        err = rope ? launch_dim<T, true>(q, k, v, out, precision, mode, D, cus, a)
                   : launch_dim<T, false>(q, k, v, out, precision, mode, D, cus, a);
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
        case VATTN_ERR_ALIAS: return "out overlaps q, k, v or the rotary table";
        case VATTN_ERR_HIP: return "HIP runtime error";
        case VATTN_ERR_ARG: return "unknown precision mode";
        case VATTN_ERR_ROPE: return "invalid rotary parameters";
        default: return "unknown status";
    }
}

extern "C" int vattn_last_hip_error(void) { return g_last_hip_error; }

extern "C" int vattn_forward_strided(const float *q, const float *k, const float *v,
                                     float *out, int n_heads, int n_patches,
                                     int head_dim, long long stride_head,
                                     long long stride_patch, int precision, void *stream) {
    return forward_impl<float>(q, k, v, out, n_heads, n_patches, head_dim, stride_head,
                               stride_patch, precision, 0, nullptr, stream);
}

extern "C" int vattn_forward_f16(const void *q, const void *k, const void *v, void *out,
                                 int n_heads, int n_patches, int head_dim,
                                 long long stride_head, long long stride_patch,
                                 int precision, void *stream) {
    return forward_impl<_Float16>(static_cast<const _Float16 *>(q), static_cast<const _Float16 *>(k),
                                  static_cast<const _Float16 *>(v), static_cast<_Float16 *>(out),
                                  n_heads, n_patches, head_dim, stride_head, stride_patch,
                                  precision, 0, nullptr, stream);
}

extern "C" int vattn_forward_rope(const float *q, const float *k, const float *v, float *out,
                                  int n_heads, int n_patches, int head_dim,
                                  long long stride_head, long long stride_patch, int rope_dims,
                                  const float *rope_table, int precision, void *stream) {
    if (rope_dims == 0) return VATTN_ERR_ROPE;
    return forward_impl<float>(q, k, v, out, n_heads, n_patches, head_dim, stride_head,
                               stride_patch, precision, rope_dims, rope_table, stream);
}

extern "C" int vattn_forward_rope_f16(const void *q, const void *k, const void *v, void *out,
                                      int n_heads, int n_patches, int head_dim,
                                      long long stride_head, long long stride_patch,
                                      int rope_dims, const float *rope_table, int precision,
                                      void *stream) {
    if (rope_dims == 0) return VATTN_ERR_ROPE;
    return forward_impl<_Float16>(static_cast<const _Float16 *>(q), static_cast<const _Float16 *>(k),
                                  static_cast<const _Float16 *>(v), static_cast<_Float16 *>(out),
                                  n_heads, n_patches, head_dim, stride_head, stride_patch,
                                  precision, rope_dims, rope_table, stream);
}

extern "C" int vattn_rope_table(float *table, int n_positions, int rope_dims, float base,
                                const float *factors, int pos_offset, void *stream) {
    if (rope_dims < 2 || rope_dims > 64 || rope_dims % 2 != 0) return VATTN_ERR_ROPE;
    if (!(base > 0.0f) || !isfinite(base)) return VATTN_ERR_ROPE;
    if (pos_offset < 0) return VATTN_ERR_ROPE;
    if (n_positions < 0) return VATTN_ERR_SIZE;
    const int half = rope_dims / 2;
    if ((int64_t)pos_offset + n_positions - 1 > (int64_t)INT32_MAX) return VATTN_ERR_ROPE;
    if ((int64_t)n_positions * half >= ((int64_t)1 << 31)) return VATTN_ERR_SIZE;
    vattn::RopeFreqs f{};
    for (int i = 0; i < half; ++i) {
        double w = pow((double)base, -2.0 * (double)i / (double)rope_dims);
        if (factors) {
            const float fi = factors[i];
            if (!(fi > 0.0f) || !isfinite(fi)) return VATTN_ERR_ROPE;
            w /= (double)fi;
        }
        f.w[i] = w;
    }
    if (n_positions == 0) return VATTN_OK;
    if (!table) return VATTN_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(table) & 15) return VATTN_ERR_ALIGN;
    const int64_t total = (int64_t)n_positions * half;
    void *args[] = {(void *)&table, (void *)&n_positions, (void *)&half, (void *)&pos_offset,
                    (void *)&f};
    const hipError_t err = hipLaunchKernel(reinterpret_cast<const void *>(&vattn::rope_table_kernel),
                                           dim3((unsigned)((total + 255) / 256)), dim3(256), args,
                                           0, reinterpret_cast<hipStream_t>(stream));
    if (err != hipSuccess) {
        g_last_hip_error = (int)err;
        return VATTN_ERR_HIP;
    }
    return VATTN_OK;
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
