// attention_fwd.hpp - head-major, non-causal flash attention forward for
// gfx950 (MI355X): f32 or f16 tensors in HBM, f16 operands on the matrix
// cores, f32 accumulation, online softmax in registers.
//
// Operation (docs.rs page "rullama 0.1.0", source of
// src/kernels/wgsl/vision_attention_flash_sub_hpd_f16.wgsl): per head,
// out = softmax(Q K^T) V over every patch, no scale inside, tensors
// [n_heads][n_patches][head_dim].  The page's shader tiles keys in blocks,
// stages them as f16 in workgroup memory, keeps a running max / running sum
// per query in f32 and rescales the partial output when the max grows (its
// key-tile loop and online-softmax update).  These kernels keep those ideas
// and re-plan the rest for CDNA4:
//
//  * attention_fwd_kernel: one workgroup = WAVES waves (4, 8 or 16) of one
//    head; each wave owns 16 query rows, so a wave's state is small enough
//    for 4 waves per SIMD (the vector ALUs only reach full issue rate with
//    several waves).  The whole workgroup shares each converted K/V tile, so
//    16 waves (256 rows) cut the K/V traffic from L2 and the conversion work
//    per query; 8 and 4 waves give more workgroups for smaller grids.
//  * attention_fwd_split_kernel (small grids): 16 waves = 4 row groups x 4
//    key chunks over 64 rows, each wave on a quarter of every tile's keys,
//    the chunks' softmax states merged through LDS at the end.
//  * Keys stream through LDS in tiles.  The next tile is loaded into
//    registers with buffer loads (the hardware range check zero-fills rows
//    past n_patches), converted to f16 with round-to-nearest-even and
//    stored to a free LDS buffer while the current tile is consumed: two
//    buffers and one barrier per tile, or (one 16-wave workgroup per CU,
//    no rotary) four buffers, tiles stored two steps ahead and one barrier
//    per two tiles.
//  * Scores are produced transposed, S^T = K Q^T, with
//    v_mfma_f32_16x16x32_f16: the key fragment (A operand) comes from LDS,
//    the query fragment (B operand) stays in registers.  In the 16x16
//    accumulator a lane holds 4 keys of ONE query, so the max test and the
//    row sum are in-lane; the query's max across its 4 lane groups (two
//    permlane swaps) is only needed when the running max is raised, and the
//    row sum's only once at the end.  The accumulator starts at -m (running
//    max), so the matrix core also does the max subtraction.
//  * The probabilities P^T leave the accumulator as the B operand of
//    O^T = V^T P^T without data movement.  V stays row-major in LDS, like K;
//    the V^T operand is gathered with the gfx950 LDS transpose load
//    (ds_read_b64_tr_b16) in the key order the S accumulator hands out.
//  * log2(e) is folded into Q, so each exponential is one v_exp_f32 (2^x).
//    The running max is only raised when a tile's max exceeds it by more than
//    kRescaleSlack (P <= 2^8 is harmless in f16 and f32); the O/l rescale is
//    a wave-uniform branch.
//  * The row sum l accumulates the f16-rounded P (v_dot2_f32_f16 against
//    1.0), i.e. exactly the weights the P.V product uses.
//  * A 32-key half of a tile whose scores all lie more than 26 log2 units
//    below the reference max holds only probabilities that round to 0 in
//    f16: its exponentials, row-sum terms and P.V products are skipped
//    (the result is bit for bit the same).  Sharp softmax rows skip about
//    half of them.
//  * SPLIT precision: q = q_hi + q_lo, k = k_hi + k_lo (all f16); the score
//    adds q_lo.k_hi and q_hi.k_lo to q_hi.k_hi in the f32 accumulator, for
//    every block (SPLIT) or only the blocks where it can matter (AUTO).
//  * Workgroup ids are remapped so that the query blocks of one head land
//    on one XCD (dispatch is round-robin over the 8 XCDs), keeping that
//    head's K/V in one L2.
//  * Tensor access (IO): element (h, n, c) sits at h*stride_head +
//    n*stride_patch + c.  kIoDense is the contiguous head-major layout with
//    head_dim == D (the fast path: whole-row vector loads).  The strided
//    modes cover any stride pair (e.g. the patch-major [n][h][c] layout a
//    QKV projection writes) and any head_dim <= D: columns c >= head_dim are
//    zero in every operand (their loads point past the buffer range, which
//    the hardware returns as 0), so they add nothing to Q.K^T and the
//    matching output columns are simply not stored.  kIoVec4 moves 4- (or
//    2-) element vectors (head_dim and strides multiples of 4), kIoScalar
//    single elements.
//  * Optional NeoX rotary transform of Q and K (ROPE; docs.rs page "rullama
//    0.2.0", src/kernels/wgsl/rope_neox_backward.wgsl, the forward rotation
//    of its header comment): pairs (x[i], x[i + half]), i < half =
//    rope_dims/2, of the row of patch n turn by the angle whose cos/sin the
//    table row n holds.  The rotation is applied in f32 to the Q fragment
//    when it is loaded and to every K tile on its way into LDS, before the
//    f16 rounding (and the hi/lo split), so rotated K never goes to HBM.
//    A tile thread holds the columns it loaded; the other half of each pair
//    sits in a lane of the same row (half/width lanes away) and is fetched
//    with ds_bpermute.  Each wave copies the cos/sin rows its own lanes
//    rotate (one contiguous piece of the table, at most 1 KB per load)
//    global -> LDS with a buffer load that has an LDS destination, one tile
//    ahead like K and V: no registers, and no other wave waits for it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vattn {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr int kIoDense = 0;   // head-major, contiguous, head_dim == D
constexpr int kIoVec4 = 1;    // strided, head_dim and strides multiples of 4
constexpr int kIoScalar = 2;  // strided, any head_dim <= D

// Strides (elements) and true head_dim of all four tensors.
struct Io {
    long long stride_head;
    int stride_patch;
    int head_dim;
};

// Rotary table: row n (patch n) holds rope_dims/2 pairs (cos theta, sin
// theta) as f32, theta = position(n) * frequency(i); half = rope_dims / 2,
// a multiple of 4.
struct Rope {
    const float *cs;
    int half;
};

// A byte offset past any buffer range: raw buffer loads there return 0.
constexpr int kOutOfRange = 0x7ffffff0;

constexpr int kRowsPerWave = 16;         // one 16-row MFMA block per wave
constexpr int kTileN = 64;               // keys per LDS tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleSlack = 8.0f;    // log2 units

// How the logits q.k are formed (template parameter PREC).
constexpr int kPrecFast = 0;   // one f16 x f16 product per logit
constexpr int kPrecSplit = 1;  // split-f16 logits (q_hi k_hi + q_lo k_hi + q_hi k_lo) everywhere
constexpr int kPrecAuto = 2;   // split-f16 logits on the key blocks whose f16 error can matter

// AUTO policy, in log2 units (q is pre-multiplied by log2 e): a 16-key
// block gets the split-f16 correction when some logit in it lies within
// `window` of its query's running maximum (the running max never exceeds
// the final one, so every key that can weigh 2^-window or more relative to
// the row maximum is corrected).
struct AutoPolicy {
    float window;
};

// LDS tile layout (the same for every workgroup size).
template <int D>
struct Lds {
    static_assert(D == 32 || D == 64, "head_dim must be 32 or 64");
    // Row pad in halves.  ds_read_b128 of the MFMA fragments (lane l reads
    // row l%16, column 16*(l/16) bytes) is free of bank conflicts on gfx950
    // when the row pitch in 16-byte units is 2 mod 4 (measured: 96 and 160
    // bytes are conflict-free, 80/112/144/176 bytes cost 4 extra cycles).
    static constexpr int kPad = 16;
    static constexpr int kKRow = D + kPad;           // K and V row pitch (halves)
    static constexpr int kKSteps = D / 32;           // 32-wide k-steps of Q.K^T
    static constexpr int kDBlocks = D / 16;          // 16-row blocks of O^T
};

// How the threads of a WAVES-wave workgroup share one K/V tile of TN keys.
template <int D, int WAVES, int TN = kTileN>
struct Shape {
    static_assert(WAVES == 4 || WAVES == 8 || WAVES == 16, "4, 8 or 16 waves per workgroup");
    static constexpr int kThreads = 64 * WAVES;
    static constexpr int kBlockM = kRowsPerWave * WAVES;      // query rows per workgroup
    static constexpr int kTileElems = TN * D / kThreads;      // K (and V) elements per thread
    static constexpr int kKWidth = kTileElems < 4 ? kTileElems : 4;  // elements per load
    static constexpr int kKVec = kTileElems / kKWidth;        // loads per thread per tensor
    static_assert(kKWidth == 2 || kKWidth == 4, "tile/thread shape");
};

// Dispatch places workgroup b on XCD b % 8.  Give each XCD a contiguous run
// of logical blocks (head-major), so one head's blocks share an L2.
__device__ __forceinline__ int xcd_remap(int b, int n) {
    const int q = n >> 3, r = n & 7;
    const int xcd = b & 7, idx = b >> 3;
    return xcd < r ? xcd * (q + 1) + idx : r * (q + 1) + (xcd - r) * q + idx;
}

__device__ __forceinline__ half2_t cvt2(float a, float b) {
    return __builtin_convertvector((float2_t){a, b}, half2_t);  // v_cvt_pk_f16_f32, RNE
}

__device__ __forceinline__ half4_t cvt4(float4_t x) {
    return __builtin_convertvector(x, half4_t);
}

__device__ __forceinline__ float4_t zero4() { return (float4_t){0.f, 0.f, 0.f, 0.f}; }

// Max / sum over the 4 lanes {l, l^16, l^32, l^48}, which hold one query's
// keys.  v_permlane16_swap / v_permlane32_swap exchange 16-lane rows /
// 32-lane halves between two registers; applied to two copies of x they put
// the paired rows side by side.
__device__ __forceinline__ float max_lane_groups(float x) {
    const unsigned u = __builtin_bit_cast(unsigned, x);
    const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    x = fmaxf(__builtin_bit_cast(float, (unsigned)a[0]), __builtin_bit_cast(float, (unsigned)a[1]));
    const unsigned w = __builtin_bit_cast(unsigned, x);
    const auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
    return fmaxf(__builtin_bit_cast(float, (unsigned)b[0]), __builtin_bit_cast(float, (unsigned)b[1]));
}

__device__ __forceinline__ float sum_lane_groups(float x) {
    const unsigned u = __builtin_bit_cast(unsigned, x);
    const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    x = __builtin_bit_cast(float, (unsigned)a[0]) + __builtin_bit_cast(float, (unsigned)a[1]);
    const unsigned w = __builtin_bit_cast(unsigned, x);
    const auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
    return __builtin_bit_cast(float, (unsigned)b[0]) + __builtin_bit_cast(float, (unsigned)b[1]);
}

// ---------------------------------------------------------------- tile I/O
// Buffer descriptor over rows [key0, n_patches) of one head's K or V: loads
// past the last row return 0 (hardware range check), so ragged tiles need no
// guards and no address clamping in the vector ALUs.
constexpr int kBufferFlags = 0x00020000;  // raw 32-bit data, gfx9 descriptor layout

// Element type of the tensors in HBM: float (converted to f16 on the way
// into LDS) or _Float16 (copied as is).
template <typename T, int N>
struct VecOf {
    typedef T type __attribute__((ext_vector_type(N)));
};

template <int D, int IO, typename T>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const T *head, int key0,
                                                            int n_patches, const Io &io) {
    const int rows = max(n_patches - key0, 0);
    if constexpr (IO == kIoDense)
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<T *>(head + (size_t)key0 * D),
                                                 (short)0, rows * D * (int)sizeof(T),
                                                 kBufferFlags);
    else
        return __builtin_amdgcn_make_buffer_rsrc(
            const_cast<T *>(head + (size_t)key0 * io.stride_patch), (short)0,
            rows > 0 ? ((rows - 1) * io.stride_patch + io.head_dim) * (int)sizeof(T) : 0,
            kBufferFlags);
}

template <typename T, int N>
__device__ __forceinline__ typename VecOf<T, N>::type buf_load_vec(__amdgpu_buffer_rsrc_t r,
                                                                   int byte_off) {
    typedef typename VecOf<T, N>::type V;
    constexpr int kBytes = (int)sizeof(T) * N;
    if constexpr (kBytes == 16)
        return __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
    else if constexpr (kBytes == 8)
        return __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b64(r, byte_off, 0, 0));
    else
        return __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, 0));
}

template <typename T>
__device__ __forceinline__ T buf_load_one(__amdgpu_buffer_rsrc_t r, int byte_off) {
    if constexpr (sizeof(T) == 4)
        return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, 0));
    else
        return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b16(r, byte_off, 0, 0));
}

// Per-thread part of the tile layout (the same for every tile): load u of
// the thread covers f = tid + kThreads*u of the tile in units of kKWidth
// elements, row f / (D/kKWidth), columns kKWidth*(f % ..), so a wave reads
// whole rows.  K and V share the mapping.
template <int D, int WAVES, int TN = kTileN>
struct TileMap {
    using S = Shape<D, WAVES, TN>;
    static constexpr int kPerRow = D / S::kKWidth;           // loads per row
    static constexpr int kRowStep = S::kThreads / kPerRow;   // rows between u and u+1
    int row0, col;
    __device__ __forceinline__ explicit TileMap(int tid) {
        row0 = tid / kPerRow;
        col = (tid % kPerRow) * S::kKWidth;
    }
};

// One tile's K and V elements of a thread, in flight from HBM to LDS.
template <int D, int WAVES, typename T, int TN = kTileN>
struct TileRegs {
    using S = Shape<D, WAVES, TN>;
    typename VecOf<T, S::kKWidth>::type k[S::kKVec];
    typename VecOf<T, S::kKWidth>::type v[S::kKVec];
};

// Vector of N elements at columns [col, col+N) of a row (row_off = the
// row's element offset): the strided modes move columns >= head_dim out of
// the buffer range (read as 0).
template <typename T, int N, int IO>
__device__ __forceinline__ typename VecOf<T, N>::type load_cols(__amdgpu_buffer_rsrc_t r,
                                                                int row_off, int col,
                                                                const Io &io,
                                                                bool enable = true) {
    constexpr int kSz = (int)sizeof(T);
    if constexpr (IO == kIoScalar) {
        typename VecOf<T, N>::type x;
#pragma unroll
        for (int j = 0; j < N; ++j)
            x[j] = buf_load_one<T>(r, enable && col + j < io.head_dim ? (row_off + col + j) * kSz
                                                                      : kOutOfRange);
        return x;
    } else {
        const bool in = enable && (IO == kIoDense || col < io.head_dim);
        return buf_load_vec<T, N>(r, in ? (row_off + col) * kSz : kOutOfRange);
    }
}

// Buffer descriptor over table rows [row0, n_patches) of the rotary table.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rope_rsrc(const Rope &rope, int row0,
                                                            int n_patches) {
    const int rows = max(n_patches - row0, 0);
    return __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float *>(rope.cs + (size_t)row0 * rope.half * 2), (short)0,
        rows * rope.half * 8, kBufferFlags);
}

// (cos, sin) of pairs [i, i + 4) of table row `row` (relative to the
// descriptor), interleaved.
__device__ __forceinline__ void load_cs4(__amdgpu_buffer_rsrc_t r, int row, int i, int half,
                                         float4_t (&cs)[2]) {
    const int off = (row * half + i) * 8;
    cs[0] = buf_load_vec<float, 4>(r, off);
    cs[1] = buf_load_vec<float, 4>(r, off + 16);
}

// LDS copy of the cos/sin rows of one key tile: kTileN rows of half
// (cos, sin) pairs, as in the table.
template <int D>
struct CsTile {
    static constexpr int kFloats = kTileN * (D / 2) * 2;
};

// Issue the copy of the table rows this wave's lanes rotate in the tile at
// key0 into `dst` (LDS, same [row][pair] layout as the table): for each
// load u, the wave's lanes cover 64 / (D/width) consecutive rows starting at
// its first lane's row, at most 1 KB of (cos, sin) pairs, copied by one
// buffer load with an LDS destination (lane l moves 16 bytes to byte 16 l).
// Each wave reads only rows it copied, so a wait on its own vector-memory
// counter (wait_vmem) makes them visible; no barrier is involved.  Rows past
// n_patches read 0.
template <int D, int WAVES>
__device__ __forceinline__ void copy_cs_rows(const Rope &rope, int key0, int n_patches,
                                             float *dst, int wave, int lane) {
    using M = TileMap<D, WAVES>;
    constexpr int kRows = 64 / M::kPerRow;  // rows per wave and load
    const __amdgpu_buffer_rsrc_t r = rope_rsrc(rope, key0, n_patches);
    const int lanes = kRows * rope.half / 2;  // 16-byte pieces: <= 64
    // The LDS destination (M0) must be wave-uniform.
    const int w = __builtin_amdgcn_readfirstlane(wave);
#pragma unroll
    for (int u = 0; u < Shape<D, WAVES>::kKVec; ++u) {
        const int row = w * kRows + u * M::kRowStep;
        if (lane < lanes)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                r, (__attribute__((address_space(3))) void *)(dst + row * rope.half * 2), 16,
                row * rope.half * 8 + 16 * lane, 0, 0, 0);
    }
}

// All vector-memory loads of this wave have landed, LDS copies included.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0f70); }  // vmcnt(0)

// NeoX rotation of 4 columns of one side of the pairs: x holds this side, y
// the other side of the same pairs, cs their (cos, sin) interleaved.  First
// halves: x c - y s; second halves: y s + x c.
__device__ __forceinline__ float4_t rotate4(const float4_t &x, const float4_t &y,
                                            const float4_t (&cs)[2], bool first) {
    float4_t r;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float c = cs[j / 2][2 * (j % 2)];
        const float sn = first ? -cs[j / 2][2 * (j % 2) + 1] : cs[j / 2][2 * (j % 2) + 1];
        r[j] = x[j] * c + y[j] * sn;
    }
    return r;
}

// Value of `x` in lane `src` of the wave (ds_bpermute, all lanes active).
__device__ __forceinline__ float lane_fetch(float x, int src) {
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src << 2, __builtin_bit_cast(int, x)));
}

template <int D, int WAVES, int IO, typename T, int TN>
__device__ __forceinline__ void load_tile(const T *kg, const T *vg, int key0,
                                          int n_patches, const TileMap<D, WAVES, TN> &m,
                                          TileRegs<D, WAVES, T, TN> &r, const Io &io) {
    using S = Shape<D, WAVES, TN>;
    const __amdgpu_buffer_rsrc_t rk = tile_rsrc<D, IO>(kg, key0, n_patches, io);
    const __amdgpu_buffer_rsrc_t rv = tile_rsrc<D, IO>(vg, key0, n_patches, io);
    const int pitch = IO == kIoDense ? D : io.stride_patch;
#pragma unroll
    for (int u = 0; u < S::kKVec; ++u) {
        const int row_off = (m.row0 + u * TileMap<D, WAVES, TN>::kRowStep) * pitch;
        r.k[u] = load_cols<T, S::kKWidth, IO>(rk, row_off, m.col, io);
        r.v[u] = load_cols<T, S::kKWidth, IO>(rv, row_off, m.col, io);
    }
}

// Registers -> LDS, both row-major [key][dim] in f16 (RNE from f32); with
// f32 inputs SPLIT and AUTO also store k_lo = f16(k - f32(f16(k))).  f16
// inputs are exact in f16 (no k_lo).

template <int D, int WAVES, int PREC, typename T, bool ROPE, int TN>
__device__ __forceinline__ void store_tile(const TileRegs<D, WAVES, T, TN> &r,
                                           _Float16 (*kh)[Lds<D>::kKRow],
                                           _Float16 (*kl)[Lds<D>::kKRow],
                                           _Float16 (*vh)[Lds<D>::kKRow],
                                           const TileMap<D, WAVES, TN> &m, const Rope &rope,
                                           const float *cs_lds, int lane) {
    using S = Shape<D, WAVES, TN>;
    typedef typename VecOf<float, S::kKWidth>::type Vec;
    typedef typename VecOf<_Float16, S::kKWidth>::type Half;
    constexpr bool KLO = PREC != kPrecFast;
    // f32 K (or rotated K) -> f16 hi, and with SPLIT lo = f16(k - f32(hi)).
    auto put_k = [&](int row, int col, const Vec &x) __attribute__((always_inline)) {
        const Half hi = __builtin_convertvector(x, Half);
        *reinterpret_cast<Half *>(&kh[row][col]) = hi;
        if constexpr (KLO) {
            // x - f32(hi) is exact in f32; fma(hi, -1, x) lets the f16
            // operand enter without a separate conversion (v_fma_mix_f32).
            Vec lo;
#pragma unroll
            for (int j = 0; j < S::kKWidth; ++j)
                lo[j] = __builtin_fmaf((float)hi[j], -1.0f, x[j]);
            *reinterpret_cast<Half *>(&kl[row][col]) = __builtin_convertvector(lo, Half);
        }
    };
    // ROPE: this lane's columns [col, col + width) are first halves
    // (col < half), second halves (col < 2 half) or unrotated; the other
    // half of its pairs is in the lane half/width away in the same row.
    bool first = false, rotated = false;
    int partner = lane, pair_i = 0;
    if constexpr (ROPE) {
        wait_vmem();  // this wave's cos/sin copies (and the tile's loads) have landed
        first = m.col < rope.half;
        rotated = m.col < 2 * rope.half;
        const int shift = rope.half / S::kKWidth;
        partner = first ? lane + shift : (rotated ? lane - shift : lane);
        pair_i = first ? m.col : m.col - rope.half;
    }
#pragma unroll
    for (int u = 0; u < S::kKVec; ++u) {
        const int row = m.row0 + u * TileMap<D, WAVES, TN>::kRowStep;
        if constexpr (ROPE) {
            const Vec x = __builtin_convertvector(r.k[u], Vec);
            Vec y, k_rot;
#pragma unroll
            for (int j = 0; j < S::kKWidth; ++j) y[j] = lane_fetch(x[j], partner);
            if (rotated) {
                const float *c = cs_lds + 2 * (row * rope.half + pair_i);
                if constexpr (S::kKWidth == 4) {
                    const float4_t cs[2] = {*reinterpret_cast<const float4_t *>(c),
                                            *reinterpret_cast<const float4_t *>(c + 4)};
                    k_rot = rotate4(x, y, cs, first);
                } else {
                    const float4_t cs[2] = {*reinterpret_cast<const float4_t *>(c), zero4()};
                    const float4_t rr = rotate4((float4_t){x[0], x[1], 0.f, 0.f},
                                                (float4_t){y[0], y[1], 0.f, 0.f}, cs, first);
                    k_rot = (Vec){rr[0], rr[1]};
                }
            } else {
                k_rot = x;
            }
            put_k(row, m.col, k_rot);
        } else if constexpr (sizeof(T) == 4) {
            put_k(row, m.col, r.k[u]);
        } else {
            // f16 inputs are exact in f16: copied, no lo part.
            *reinterpret_cast<Half *>(&kh[row][m.col]) = r.k[u];
        }
        *reinterpret_cast<Half *>(&vh[row][m.col]) = __builtin_convertvector(r.v[u], Half);
    }
}

__device__ __forceinline__ float4_t mfma16(half8_t a, half8_t b, float4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// q_lo.k_hi (+ q_hi.k_lo) added to the scores of 16-key block kb, in the
// block's accumulator.  KLO = false (f16 inputs: k is exact in f16) drops
// the q_hi.k_lo product.
template <int D, bool KLO, int KB>
__device__ __forceinline__ void qk_correct(const _Float16 (*kh)[Lds<D>::kKRow],
                                           const _Float16 (*kl)[Lds<D>::kKRow],
                                           const half8_t (&qh)[Lds<D>::kKSteps],
                                           const half8_t (&ql)[Lds<D>::kKSteps],
                                           float4_t (&s)[KB], int kb, int l16, int g4) {
#pragma unroll
    for (int st = 0; st < Lds<D>::kKSteps; ++st) {
        const half8_t a = *reinterpret_cast<const half8_t *>(&kh[16 * kb + l16][32 * st + 8 * g4]);
        s[kb] = mfma16(a, ql[st], s[kb]);
        if constexpr (KLO) {
            const half8_t al = *reinterpret_cast<const half8_t *>(
                &kl[16 * kb + l16][32 * st + 8 * g4]);
            s[kb] = mfma16(al, qh[st], s[kb]);
        }
    }
}

// In-lane maxima of the scores: per 16-key block (bmax), per 32-key half
// (mxh) and over the tile (mx).
template <int KB>
__device__ __forceinline__ void tile_maxima(const float4_t (&s)[KB], float (&bmax)[KB],
                                            float (&mxh)[KB / 2], float &mx) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
        bmax[kb] = fmaxf(fmaxf(fmaxf(s[kb][0], s[kb][1]), s[kb][2]), s[kb][3]);
#pragma unroll
    for (int ks = 0; ks < KB / 2; ++ks) mxh[ks] = fmaxf(bmax[2 * ks], bmax[2 * ks + 1]);
    mx = mxh[0];
#pragma unroll
    for (int ks = 1; ks < KB / 2; ++ks) mx = fmaxf(mx, mxh[ks]);
}

// S'^T = K Q^T + C for one tile of 16*KB keys and the wave's 16 queries.
// `c0` starts every key block's accumulator at -m_ref, so the matrix core
// already subtracts the running max from each logit.  Keys at or past
// key_lim (the ragged last tile) are set to -inf before anything looks at
// the scores.  bmax, mxh and mx receive the lane's maxima (tile_maxima)
// before any correction: a correction moves a score by ~2^-11 of its size,
// which matters for no reference-max, window or dead-half decision.
//
// Returns the wave-uniform mask of the blocks that need the split-f16
// correction (apply_corrections): none for FAST, all for SPLIT, and for
// AUTO the blocks with a logit inside the window of the running max
// (AutoPolicy).  On a wave's first tile (`first`) there is no running max:
// every block counts as inside the window.
template <int D, int PREC, int KB = 4>
__device__ __forceinline__ unsigned qk_tile(const _Float16 (*kh)[Lds<D>::kKRow],
                                            const half8_t (&qh)[Lds<D>::kKSteps], float4_t c0,
                                            float4_t (&s)[KB], float (&bmax)[KB],
                                            float (&mxh)[KB / 2], float &mx, int l16, int g4,
                                            int key_lim, const AutoPolicy &pol, bool first) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int st = 0; st < Lds<D>::kKSteps; ++st) {
            const half8_t a = *reinterpret_cast<const half8_t *>(
                &kh[16 * kb + l16][32 * st + 8 * g4]);
            s[kb] = mfma16(a, qh[st], st == 0 ? c0 : s[kb]);
        }
    }
    if (key_lim < 16 * KB) {  // wave-uniform: only the ragged last tile
        // Key 16 kb + 4 g4 + i of the tile is past the end when 16 kb + i >=
        // key_lim - 4 g4 (compile-time constants against one lane value).
        const int lim = key_lim - 4 * g4;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (16 * kb + i >= lim) s[kb][i] = -__builtin_inff();
    }
    tile_maxima(s, bmax, mxh, mx);
    constexpr unsigned kAll = (1u << KB) - 1;
    if constexpr (PREC == kPrecSplit) {
        return kAll;
    } else if constexpr (PREC == kPrecAuto) {
        if (first) return kAll;
        unsigned mask = 0;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
            if (__ballot(bmax[kb] > -pol.window)) mask |= 1u << kb;
        return mask;
    } else {
        return 0;
    }
}

// q_lo.k_hi (+ q_hi.k_lo) added to the blocks of `mask` (SPLIT: to every
// block, unconditionally).  AUTO at d = 32 (one k-step per block) reads the
// k_lo fragments of all KB blocks before the per-block branches, so their
// LDS latency overlaps instead of being waited out inside each branch; the
// reads for blocks left uncorrected only cost LDS bandwidth.  (Measured:
// +2 to +4.5% on flat d = 32 inputs, +1.6% on sharp ones; at d = 64 the
// eight fragments cost more than they save.)
template <int D, int PREC, bool KLO, int KB>
__device__ __forceinline__ void apply_corrections(const _Float16 (*kh)[Lds<D>::kKRow],
                                                  const _Float16 (*kl)[Lds<D>::kKRow],
                                                  const half8_t (&qh)[Lds<D>::kKSteps],
                                                  const half8_t (&ql)[Lds<D>::kKSteps],
                                                  float4_t (&s)[KB], unsigned mask, int l16,
                                                  int g4) {
    if constexpr (PREC == kPrecAuto && KLO && D == 32) {
        half8_t al[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
            al[kb] = *reinterpret_cast<const half8_t *>(&kl[16 * kb + l16][8 * g4]);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            if (mask & (1u << kb)) {
                const half8_t a = *reinterpret_cast<const half8_t *>(&kh[16 * kb + l16][8 * g4]);
                s[kb] = mfma16(a, ql[0], s[kb]);
                s[kb] = mfma16(al[kb], qh[0], s[kb]);
            }
        }
    } else {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            if constexpr (PREC == kPrecSplit)
                qk_correct<D, KLO, KB>(kh, kl, qh, ql, s, kb, l16, g4);
            else if (mask & (1u << kb))
                qk_correct<D, KLO, KB>(kh, kl, qh, ql, s, kb, l16, g4);
        }
    }
}

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4_t lds_short4_t;

__device__ __forceinline__ half4_t read_tr16(const _Float16 *p) {
    return __builtin_bit_cast(half4_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t *)p));
}

// A probability below 2^-26 is 0 once rounded to f16 (the smallest f16
// subnormal is 2^-24 and round-to-nearest-even sends everything up to 2^-25
// to 0), so a score more than 26 log2 units below the reference max adds
// exactly nothing to l or O.
constexpr float kDeadBelow = -26.0f;

// Exponentials, row sum and O^T += V^T P^T for one tile, in 32-key halves
// (two 16-key blocks, one 16x16x32 MFMA k-step each).  A half whose scores
// all lie below kDeadBelow (a wave-uniform test on the lanes' maxima mxh)
// contributes exactly 0 and is skipped; sharp softmax rows have many such
// halves.  Per half: P = 2^s in f16 (RNE), l += the f16-rounded P
// (v_dot2_f32_f16 against 1.0, i.e. exactly the weights P.V uses), and the
// P.V product.  The A operand (16 dims x 32 keys) is two
// ds_read_b64_tr_b16 of row-major V: in each 16-lane group, lane s points
// at 4 consecutive dims of one key row and output lane j receives dim j of
// the 4 keys addressed by lanes j/4, j/4+4, j/4+8, j/4+12.  Lane s of group
// g addresses key 4g + s/4 (+16 for the second read) at dims 4*(s%4)..+3 of
// the block, which yields, for lane 16g+j, dim j of keys {4g..4g+3} and
// {16+4g..16+4g+3}: the keys the P operand of that lane holds, in the same
// order.  The order of every accumulation is the same whether or not other
// halves are skipped.
template <int D, int KB>
__device__ __forceinline__ void exp_pv_live(const float4_t (&s)[KB], const float (&mxh)[KB / 2],
                                            float &l_run, float4_t (&o)[Lds<D>::kDBlocks],
                                            const _Float16 (*vh)[Lds<D>::kKRow], int l16,
                                            int g4) {
    const half2_t ones = {(_Float16)1.0f, (_Float16)1.0f};
    const int key = 4 * g4 + (l16 >> 2);
    const int dim = 4 * (l16 & 3);
#pragma unroll
    for (int ks = 0; ks < KB / 2; ++ks) {
        if (__ballot(mxh[ks] > kDeadBelow)) {
            half2_t h[4];
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const float4_t x = s[2 * ks + hf];
                h[2 * hf] = cvt2(__builtin_amdgcn_exp2f(x[0]), __builtin_amdgcn_exp2f(x[1]));
                h[2 * hf + 1] = cvt2(__builtin_amdgcn_exp2f(x[2]), __builtin_amdgcn_exp2f(x[3]));
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) l_run = __builtin_amdgcn_fdot2(h[j], ones, l_run, false);
            const half8_t p = {h[0][0], h[0][1], h[1][0], h[1][1],
                               h[2][0], h[2][1], h[3][0], h[3][1]};
#pragma unroll
            for (int db = 0; db < Lds<D>::kDBlocks; ++db) {
                const half4_t a0 = read_tr16(&vh[32 * ks + key][16 * db + dim]);
                const half4_t a1 = read_tr16(&vh[32 * ks + 16 + key][16 * db + dim]);
                const half8_t a = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
                o[db] = mfma16(a, p, o[db]);
            }
        }
    }
}

// Online softmax and P.V for one tile whose scores s hold s_true - m_run
// (the QK accumulator started at c0 = -m_run; before the first tile
// m_run = -inf and c0 = 0; keys past n_patches already hold -inf).  The
// running max is raised only when the tile's
// max exceeds it by more than kRescaleSlack: then o and l are scaled by
// 2^(m_old - m_new), s is rebased and c0 follows.  That branch is
// wave-uniform and only rescales in place; both paths then share one copy
// of the exponentials and the P.V product (a copy per path made the
// register allocator merge two homes of o, l and s with ~20 register moves
// per tile on the common path).
// bmax, mxh, mx: qk_tile's maxima (tile_maxima).  RECOMPUTE: take them
// afresh from s instead of keeping qk_tile's across the corrections (fewer
// live registers, for kernels that are short of them).
// The wave runs this at raised issue priority: its exponentials stand
// between its scores and its P.V products, and the waves still issuing
// score MFMAs lose little by yielding to it.  (Measured: 8-wave d = 32
// blocks two to a CU +5%, the other shapes equal.)
template <int D, int KB = 4, bool RECOMPUTE = false>
__device__ __forceinline__ void softmax_pv_tile(float4_t (&s)[KB], float (&bmax)[KB],
                                                float (&mxh)[KB / 2], float mx, float4_t &c0,
                                                float &m_run, float &l_run,
                                                float4_t (&o)[Lds<D>::kDBlocks],
                                                const _Float16 (*vt)[Lds<D>::kKRow],
                                                int l16, int g4) {
    __builtin_amdgcn_s_setprio(1);
    if constexpr (RECOMPUTE) tile_maxima(s, bmax, mxh, mx);
    const float m_ref = -c0[0];
    // Some lane's own scores exceed the slack: only then is the query's
    // tile max (across its 4 lane groups) needed.
    if (__ballot(mx - c0[0] > m_run + kRescaleSlack)) {
        const float tile_max = max_lane_groups(mx) + m_ref;
        const bool raise = tile_max > m_run + kRescaleSlack;
        const float m_new = raise ? tile_max : m_run;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        const float delta = m_new - m_ref;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < Lds<D>::kDBlocks; ++db) o[db] *= alpha;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) s[kb] -= delta;
#pragma unroll
        for (int ks = 0; ks < KB / 2; ++ks) mxh[ks] -= delta;
        c0 -= delta;
        m_run = m_new;
    }
    exp_pv_live<D, KB>(s, mxh, l_run, o, vt, l16, g4);
    __builtin_amdgcn_s_setprio(0);
}

template <int V>
struct IntTag {
    static constexpr int value = V;
};

// Waves per SIMD the register budget is sized for: 4 (128 VGPRs) for the
// 8- and 16-wave workgroups; the 4-wave workgroups of small grids (one wave
// per SIMD each, four tile loads per thread) get 2 (256 VGPRs).
// Query fragment of this lane's row (B operand of S^T = K Q^T): columns
// 32 st + 8 g4 ... + 7 of each k-step st, times log2(e), as f16 (RNE) in qh
// and, with SPLIT, the remainder f16(x - f32(qh)) in ql.  Rows past the
// head read 0.  ROPE turns each pair first (in f32): columns [c, c + 4) lie
// on one side of half and of rope_dims (both multiples of 4), so they turn
// with their partner columns.
template <int D, int PREC, int IO, typename T, bool ROPE>
__device__ __forceinline__ void load_q_fragment(const T *__restrict__ qg, int row, int n_patches,
                                                const Io &io, const Rope &rope, int g4,
                                                half8_t (&qh)[Lds<D>::kKSteps],
                                                half8_t (&ql)[Lds<D>::kKSteps]) {
    __amdgpu_buffer_rsrc_t rq;
    if constexpr (IO != kIoDense) rq = tile_rsrc<D, IO>(qg, 0, n_patches, io);
    typedef typename VecOf<T, 4>::type T4;
    // Four query columns [c, c+4) of the row as f32 (0 past the head).
    auto q4 = [&](int c) __attribute__((always_inline)) {
        float4_t x = zero4();
        if (row < n_patches) {
            if constexpr (IO == kIoDense)
                x = __builtin_convertvector(*reinterpret_cast<const T4 *>(qg + row * D + c), float4_t);
            else
                x = __builtin_convertvector(load_cols<T, 4, IO>(rq, row * io.stride_patch, c, io),
                                            float4_t);
        }
        return x;
    };
    auto q4_rotated = [&](int c) __attribute__((always_inline)) {
        float4_t x = q4(c);
        if constexpr (ROPE) {
            if (c < 2 * rope.half) {
                const bool first = c < rope.half;
                const int i = first ? c : c - rope.half;
                const float4_t y = q4(first ? c + rope.half : c - rope.half);
                float4_t cs[2];
                load_cs4(rope_rsrc(rope, 0, n_patches), row, i, rope.half, cs);
                x = rotate4(x, y, cs, first);
            }
        }
        return x;
    };
#pragma unroll
    for (int st = 0; st < Lds<D>::kKSteps; ++st) {
        const int c = 32 * st + 8 * g4;
        float4_t x0 = q4_rotated(c), x1 = q4_rotated(c + 4);
        x0 *= kLog2e;
        x1 *= kLog2e;
        const half4_t h0 = cvt4(x0), h1 = cvt4(x1);
        qh[st] = (half8_t){h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
        if constexpr (PREC != kPrecFast) {
            const half4_t e0 = cvt4(x0 - __builtin_convertvector(h0, float4_t));
            const half4_t e1 = cvt4(x1 - __builtin_convertvector(h1, float4_t));
            ql[st] = (half8_t){e0[0], e0[1], e0[2], e0[3], e1[0], e1[1], e1[2], e1[3]};
        } else {
            ql[st] = qh[st];
        }
    }
}

// This lane's index in its wave, computed afresh with v_mbcnt: values
// derived from it after the tile loop are not kept alive (or spilled)
// across the loop.
__device__ __forceinline__ int fresh_lane_id() {
    int id;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(id));
    return id;
}

// Epilogue: out = O / l for the wave's 16 rows starting at row0 (inside the
// head: rows below n_patches; in the strided modes columns below
// head_dim).  O^T block db holds dims 16 db + 4 g4 .. + 3 of query l16.
template <int D, int IO, typename T>
__device__ __forceinline__ void store_rows(T *__restrict__ og, const float4_t (&o)[Lds<D>::kDBlocks],
                                           float l_run, int row0, int n_patches, const Io &io) {
    const float inv = 1.0f / sum_lane_groups(l_run);
    const int lane = fresh_lane_id();
    const int row = row0 + (lane & 15);
    const int g4 = lane >> 4;
    if (row >= n_patches) return;
    typedef typename VecOf<T, 4>::type T4;
    if constexpr (IO == kIoDense) {
#pragma unroll
        for (int db = 0; db < Lds<D>::kDBlocks; ++db)
            *reinterpret_cast<T4 *>(og + row * D + 16 * db + 4 * g4) =
                __builtin_convertvector(o[db] * inv, T4);
    } else {
        T *orow = og + (size_t)row * io.stride_patch;
#pragma unroll
        for (int db = 0; db < Lds<D>::kDBlocks; ++db) {
            const int c = 16 * db + 4 * g4;
            const T4 y = __builtin_convertvector(o[db] * inv, T4);
            if constexpr (IO == kIoVec4) {
                if (c < io.head_dim) *reinterpret_cast<T4 *>(orow + c) = y;
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (c + j < io.head_dim) orow[c + j] = y[j];
            }
        }
    }
}

template <int WAVES>
constexpr int kMinWavesPerSimd = WAVES == 4 ? 2 : 4;

// ------------------------------------------------------------------ kernel
// Per key tile t: a later tile, already in registers, is converted into a
// free LDS buffer and the loads of the tile after it are issued; then
// QK(t), softmax and PV(t) from tile t's buffer (see `step` for the buffer
// and barrier schedule).  A tile's HBM/L2 latency hides behind a whole tile
// of compute.  Matrix and vector work overlap across the waves each SIMD
// holds.  The loop is unrolled by two so that, with two buffers, LDS buffer
// addresses are immediates.
template <int D, int WAVES, int PREC, int IO, typename T, bool ROPE>
__global__ void __launch_bounds__(64 * WAVES, kMinWavesPerSimd<WAVES>)
attention_fwd_kernel(const T *__restrict__ q, const T *__restrict__ k,
                     const T *__restrict__ v, T *__restrict__ out,
                     int n_patches, int q_blocks, int total_blocks, AutoPolicy pol, Io io,
                     Rope rope) {
    using L = Lds<D>;
    using S = Shape<D, WAVES>;
    using M = TileMap<D, WAVES>;
    // k_lo tiles: f32 K, or rotated K (f16 inputs are exact in f16 only
    // before the rotation).
    constexpr bool KLO = PREC != kPrecFast && (sizeof(T) == 4 || ROPE);
    // LDS buffers of K/V tiles.  One workgroup per CU (16 waves, no rotary
    // tables) has room for four: tiles are stored two steps ahead and one
    // barrier follows every second step.  Otherwise two: one step ahead, a
    // barrier after every step.
    constexpr int NB = (WAVES == 16 && !ROPE) ? 4 : 2;
    constexpr int AHEAD = NB / 2;
    __shared__ __attribute__((aligned(16))) _Float16 kh_s[NB][kTileN][L::kKRow];
    __shared__ __attribute__((aligned(16))) _Float16 vt_s[NB][kTileN][L::kKRow];
    __shared__ __attribute__((aligned(16)))
    _Float16 kl_s[KLO ? NB : 1][KLO ? kTileN : 1][L::kKRow];
    __shared__ __attribute__((aligned(16))) float cs_s[ROPE ? 2 : 1][ROPE ? CsTile<D>::kFloats : 4];

    const int logical = xcd_remap(blockIdx.x, total_blocks);
    const int head = logical / q_blocks;
    const int qblk = logical - head * q_blocks;
    const size_t base = IO == kIoDense ? (size_t)head * (size_t)n_patches * D
                                       : (size_t)((long long)head * io.stride_head);
    const T *__restrict__ qg = q + base;
    const T *kg = k + base;
    const T *vg = v + base;
    T *__restrict__ og = out + base;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l16 = lane & 15;  // query column inside the wave's 16 rows
    const int g4 = lane >> 4;   // lane group 0..3
    const int row = qblk * S::kBlockM + wave * kRowsPerWave + l16;
    const int n_tiles = (n_patches + kTileN - 1) / kTileN;
    const M map(tid);

    // Tile 0's loads (and with ROPE its cos/sin rows) go out first, so their
    // latency overlaps the Q loads'.
    TileRegs<D, WAVES, T> regs;
    load_tile<D, WAVES, IO>(kg, vg, 0, n_patches, map, regs, io);
    if constexpr (ROPE) {
        // Zero both cos/sin buffers first (a barrier orders these stores
        // before every wave's copies), so no lane ever reads LDS the copies
        // leave unwritten; then copy tile 0's rows.
        for (int i = tid; i < 2 * CsTile<D>::kFloats / 4; i += 64 * WAVES)
            reinterpret_cast<float4_t *>(&cs_s[0][0])[i] = zero4();
        __syncthreads();
        copy_cs_rows<D, WAVES>(rope, 0, n_patches, cs_s[0], wave, lane);
    }

    // Query fragment (B operand of S^T = K Q^T), pre-multiplied by log2(e).
    half8_t qh[L::kKSteps];
    half8_t ql[L::kKSteps];
    load_q_fragment<D, PREC, IO, T, ROPE>(qg, row, n_patches, io, rope, g4, qh, ql);
    store_tile<D, WAVES, PREC, T, ROPE>(regs, kh_s[0], kl_s[0], vt_s[0], map, rope, cs_s[0], lane);
    if (n_tiles > 1) {
        load_tile<D, WAVES, IO>(kg, vg, kTileN, n_patches, map, regs, io);
        if constexpr (ROPE) copy_cs_rows<D, WAVES>(rope, kTileN, n_patches, cs_s[1], wave, lane);
    }
    if constexpr (AHEAD == 2) {
        if (n_tiles > 1) {
            store_tile<D, WAVES, PREC, T, ROPE>(regs, kh_s[1], kl_s[KLO ? 1 : 0], vt_s[1], map,
                                                rope, cs_s[0], lane);
            if (n_tiles > 2) load_tile<D, WAVES, IO>(kg, vg, 2 * kTileN, n_patches, map, regs, io);
        }
    }
    __syncthreads();

    float4_t o[L::kDBlocks];
#pragma unroll
    for (int db = 0; db < L::kDBlocks; ++db) o[db] = zero4();
    float m_run = -__builtin_inff();
    float l_run = 0.f;
    float4_t c0 = zero4();  // -(reference max) seeding every QK accumulator

    // Step t (odd_tag: t is odd).  Tile t + AHEAD (in registers since the
    // previous step) goes into LDS buffer (t + AHEAD) % NB, then the loads of
    // the tile after it are issued: they drain while this tile is computed,
    // and the stores have landed long before the next barrier.  The buffer a
    // store overwrites (tile data and bound-test bytes) was read AHEAD steps
    // earlier, before the last barrier every wave has passed; a tile stored
    // in step t is read in step t + AHEAD, after the barrier that ends the
    // group of AHEAD steps holding step t.
    auto step = [&](int t, auto odd_tag) __attribute__((always_inline)) {
        constexpr int ODD = decltype(odd_tag)::value;
        const int rb = NB == 2 ? ODD : (t & 3);          // buffer of tile t
        const int wb = NB == 2 ? ODD ^ 1 : ((t + 2) & 3);  // buffer of tile t + AHEAD
        if (t + AHEAD < n_tiles) {
            store_tile<D, WAVES, PREC, T, ROPE>(regs, kh_s[wb], kl_s[KLO ? wb : 0], vt_s[wb], map,
                                                rope, cs_s[ROPE ? wb : 0], lane);
            if (t + AHEAD + 1 < n_tiles) {
                load_tile<D, WAVES, IO>(kg, vg, (t + AHEAD + 1) * kTileN, n_patches, map, regs,
                                        io);
                // cos/sin of tile t+2 into the buffer tile t's store read.
                if constexpr (ROPE)
                    copy_cs_rows<D, WAVES>(rope, (t + 2) * kTileN, n_patches, cs_s[rb], wave,
                                           lane);
            }
        }
        float4_t s[4];
        float bmax[4], mxh[2], mx;
        const unsigned fix = qk_tile<D, PREC>(kh_s[rb], qh, c0, s, bmax, mxh, mx, l16, g4,
                                              n_patches - t * kTileN, pol, t == 0);
        if constexpr (PREC != kPrecFast)
            apply_corrections<D, PREC, KLO>(kh_s[rb], kl_s[KLO ? rb : 0], qh, ql, s, fix, l16, g4);
        softmax_pv_tile<D, 4, ROPE>(s, bmax, mxh, mx, c0, m_run, l_run, o, vt_s[rb], l16, g4);
        if (NB == 2 || ODD) __syncthreads();
    };
    for (int t = 0; t < n_tiles; t += 2) {
        step(t, IntTag<0>{});
        if (t + 1 < n_tiles) step(t + 1, IntTag<1>{});
    }

    store_rows<D, IO, T>(og, o, l_run, qblk * S::kBlockM + wave * kRowsPerWave, n_patches, io);
}

// ------------------------------------------------------- split-key kernel
// Small grids (at most one 64-row block per CU): 16 waves = 4 row groups x
// 4 key chunks.  A workgroup owns 64 query rows; the keys stream through
// LDS in tiles of 128 (two buffers, one barrier per tile) and
// key chunk c of every tile - rows [32c, 32c + 32) - goes to the waves of
// chunk c, so each wave keeps its own (m, l, o) over a quarter of the keys
// (16 rows x 32 keys per tile: two 16-key blocks).  At the end the chunks'
// states are merged through LDS with the online-softmax rule (scale each
// by 2^(m_c - m), add) and chunk 0 writes the rows.  This gives 4 waves per
// SIMD where the 64-row workgroups of the plain kernel give one.
constexpr int kSplitChunks = 4;
constexpr int kSplitTileN = 32 * kSplitChunks;  // keys per LDS tile
constexpr int kSplitBlockM = 64;                // query rows per workgroup

template <int D, int PREC, int IO, typename T>
__global__ void __launch_bounds__(1024, 4)
attention_fwd_split_kernel(const T *__restrict__ q, const T *__restrict__ k,
                           const T *__restrict__ v, T *__restrict__ out, int n_patches,
                           int q_blocks, int total_blocks, AutoPolicy pol, Io io) {
    using L = Lds<D>;
    constexpr int WAVES = 16;
    constexpr int TN = kSplitTileN;
    using M = TileMap<D, WAVES, TN>;
    constexpr bool KLO = PREC != kPrecFast && sizeof(T) == 4;
    __shared__ __attribute__((aligned(16))) _Float16 kh_s[2][TN][L::kKRow];
    __shared__ __attribute__((aligned(16))) _Float16 vt_s[2][TN][L::kKRow];
    __shared__ __attribute__((aligned(16)))
    _Float16 kl_s[KLO ? 2 : 1][KLO ? TN : 1][L::kKRow];
    // AUTO: a chunk decides its corrections from its own running max,
    // which never exceeds its row group's, so its window test keeps every
    // key within the window of the group's maximum.

    const int logical = xcd_remap(blockIdx.x, total_blocks);
    const int head = logical / q_blocks;
    const int qblk = logical - head * q_blocks;
    const size_t base = IO == kIoDense ? (size_t)head * (size_t)n_patches * D
                                       : (size_t)((long long)head * io.stride_head);
    const T *__restrict__ qg = q + base;
    const T *kg = k + base;
    const T *vg = v + base;
    T *__restrict__ og = out + base;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l16 = lane & 15;
    const int g4 = lane >> 4;
    const int rgroup = wave >> 2;  // 16-row group of the workgroup's 64 rows
    const int chunk = wave & 3;    // 32-key chunk of every tile
    const int row = qblk * kSplitBlockM + rgroup * kRowsPerWave + l16;
    const int n_tiles = (n_patches + TN - 1) / TN;
    const M map(tid);

    const Rope no_rope{nullptr, 0};
    TileRegs<D, WAVES, T, TN> regs;
    load_tile<D, WAVES, IO>(kg, vg, 0, n_patches, map, regs, io);

    // Query fragment, as in attention_fwd_kernel.
    half8_t qh[L::kKSteps];
    half8_t ql[L::kKSteps];
    load_q_fragment<D, PREC, IO, T, false>(qg, row, n_patches, io, no_rope, g4, qh, ql);
    store_tile<D, WAVES, PREC, T, false>(regs, kh_s[0], kl_s[0], vt_s[0], map, no_rope, nullptr,
                                         lane);
    if (n_tiles > 1) load_tile<D, WAVES, IO>(kg, vg, TN, n_patches, map, regs, io);
    __syncthreads();

    float4_t o[L::kDBlocks];
#pragma unroll
    for (int db = 0; db < L::kDBlocks; ++db) o[db] = zero4();
    float m_run = -__builtin_inff();
    float l_run = 0.f;
    float4_t c0 = zero4();
    const int key_off = 32 * chunk;

    auto step = [&](int t, auto buf_tag) __attribute__((always_inline)) {
        constexpr int BUF = decltype(buf_tag)::value;
        if (t + 1 < n_tiles) {
            store_tile<D, WAVES, PREC, T, false>(regs, kh_s[BUF ^ 1], kl_s[KLO ? (BUF ^ 1) : 0],
                                                 vt_s[BUF ^ 1], map, no_rope, nullptr, lane);
            if (t + 2 < n_tiles)
                load_tile<D, WAVES, IO>(kg, vg, (t + 2) * TN, n_patches, map, regs, io);
        }
        const int key_lim = n_patches - t * TN - key_off;
        // wave-uniform: a chunk past the last key does nothing
        if (key_lim > 0) {
            float4_t s[2];
            float bmax[2], mxh[1], mx;
            const unsigned fix = qk_tile<D, PREC, 2>(kh_s[BUF] + key_off, qh, c0, s, bmax, mxh,
                                                     mx, l16, g4, key_lim, pol, t == 0);
            if constexpr (PREC != kPrecFast)
                apply_corrections<D, PREC, KLO>(kh_s[BUF] + key_off,
                                          kl_s[KLO ? BUF : 0] + (KLO ? key_off : 0), qh, ql, s,
                                          fix, l16, g4);
            softmax_pv_tile<D, 2>(s, bmax, mxh, mx, c0, m_run, l_run, o, vt_s[BUF] + key_off,
                                  l16, g4);
        }
        __syncthreads();
    };
    for (int t = 0; t < n_tiles; t += 2) {
        step(t, IntTag<0>{});
        if (t + 1 < n_tiles) step(t + 1, IntTag<1>{});
    }

    // Merge chunks 1..3 into chunk 0 through the (now idle) K and V tile
    // buffers: chunk c writes its state (per row group 64 lanes x (16 o + m
    // + l) floats) to region c - 1, and after one barrier chunk 0 combines
    // the four with the online-softmax rule.
    constexpr int kState = 4 * L::kDBlocks + 2;
    constexpr int kRegion = 4 * 64 * kState;  // floats per chunk
    static_assert(2 * kRegion * 4 <= (int)sizeof(kh_s) && kRegion * 4 <= (int)sizeof(vt_s),
                  "merge buffers");
    auto region = [&](int c) __attribute__((always_inline)) {
        float *b = c < 3 ? reinterpret_cast<float *>(&kh_s[0][0][0]) + (c - 1) * kRegion
                         : reinterpret_cast<float *>(&vt_s[0][0][0]);
        return b + rgroup * 64 * kState;
    };
    if (chunk != 0) {
        float *xfer = region(chunk);
#pragma unroll
        for (int db = 0; db < L::kDBlocks; ++db)
#pragma unroll
            for (int j = 0; j < 4; ++j) xfer[(4 * db + j) * 64 + lane] = o[db][j];
        xfer[(4 * L::kDBlocks) * 64 + lane] = m_run;
        xfer[(4 * L::kDBlocks + 1) * 64 + lane] = l_run;
    }
    __syncthreads();
    if (chunk == 0) {
        float m_c[kSplitChunks];
        m_c[0] = m_run;
#pragma unroll
        for (int c = 1; c < kSplitChunks; ++c) m_c[c] = region(c)[(4 * L::kDBlocks) * 64 + lane];
        // m_new is finite: chunk 0 always holds key 0.  A chunk that never
        // saw a key has m = -inf and weight 0.
        const float m_new = fmaxf(fmaxf(m_c[0], m_c[1]), fmaxf(m_c[2], m_c[3]));
        const float a0 = __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
        for (int db = 0; db < L::kDBlocks; ++db) o[db] *= a0;
        l_run *= a0;
#pragma unroll
        for (int c = 1; c < kSplitChunks; ++c) {
            const float *xfer = region(c);
            const float ac = __builtin_amdgcn_exp2f(m_c[c] - m_new);
#pragma unroll
            for (int db = 0; db < L::kDBlocks; ++db)
#pragma unroll
                for (int j = 0; j < 4; ++j) o[db][j] += xfer[(4 * db + j) * 64 + lane] * ac;
            l_run += xfer[(4 * L::kDBlocks + 1) * 64 + lane] * ac;
        }
        store_rows<D, IO, T>(og, o, l_run, qblk * kSplitBlockM + rgroup * kRowsPerWave,
                             n_patches, io);
    }
}

}  // namespace vattn
