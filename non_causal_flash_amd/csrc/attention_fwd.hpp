// attention_fwd.hpp - head-major, non-causal flash attention forward for
// gfx950 (MI355X): f32 in HBM, f16 operands on the matrix cores, f32
// accumulation, online softmax in registers.
//
// Operation (docs.rs page "rullama 0.1.0", source of
// src/kernels/wgsl/vision_attention_flash_sub_hpd_f16.wgsl): per head,
// out = softmax(Q K^T) V over every patch, no scale inside, tensors
// [n_heads][n_patches][head_dim].  The page's shader tiles keys in blocks,
// stages them as f16 in workgroup memory, keeps a running max / running sum
// per query in f32 and rescales the partial output when the max grows (its
// key-tile loop and online-softmax update).  This kernel keeps those ideas
// and re-plans the rest for CDNA4:
//
//  * One workgroup = 4 waves = 128 query rows of one head; each wave owns 32
//    rows.  Keys stream through LDS in tiles of 64, double buffered: while a
//    tile is consumed, the next one is loaded from HBM/L2 into registers
//    (coalesced float4 loads), converted to f16 with round-to-nearest-even
//    and written to the other LDS buffer; one barrier per tile.
//  * Scores are produced transposed, S^T = K Q^T, with
//    v_mfma_f32_16x16x32_f16: the key fragment (A operand) comes from LDS,
//    the query fragment (B operand) sits in registers for the whole kernel.
//    In the 16x16 accumulator a lane then holds 4 keys of ONE query, so the
//    row max / row sum are in-lane, plus two cross-lane steps per tile.
//  * The probabilities P^T leave the accumulator as the B operand of the
//    next product O^T = V^T P^T without any data movement: the key order the
//    S accumulator hands out is matched by storing V^T in LDS with the same
//    key permutation (see vt_pos).
//  * log2(e) is folded into Q, so every exponential is one v_exp_f32
//    (2^x).  The running max is only raised when a tile's max exceeds it by
//    more than kRescaleSlack (then P <= 2^8, harmless in f16 and f32), so
//    the O/l rescale is skipped for most tiles; the result is the same
//    softmax, since any shift cancels between numerator and denominator.
//  * The row sum l accumulates the f16-rounded P (v_dot2_f32_f16 against
//    1.0), i.e. exactly the weights the P.V product uses.
//  * SPLIT precision: q = q_hi + q_lo, k = k_hi + k_lo (all f16); the score
//    adds q_lo.k_hi and q_hi.k_lo to q_hi.k_hi in the f32 accumulator.
//  * Workgroup ids are remapped so that the query blocks of one head land
//    on one XCD (dispatch is round-robin over the 8 XCDs), keeping that
//    head's K/V in one L2.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vattn {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;            // 4 waves of 64
constexpr int kWaves = kThreads / 64;
constexpr int kRowsPerWave = 32;         // two 16-row MFMA blocks
constexpr int kBlockM = kWaves * kRowsPerWave;  // 128 query rows per workgroup
constexpr int kTileN = 64;               // keys per LDS tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleSlack = 8.0f;    // log2 units

template <int D>
struct Shape {
    static_assert(D == 32 || D == 64, "head_dim must be 32 or 64");
    static constexpr int kPad = 8;                   // halves; breaks LDS bank aliasing
    static constexpr int kKRow = D + kPad;           // K row pitch in LDS (halves)
    static constexpr int kVRow = kTileN + kPad;      // V^T row pitch in LDS (halves)
    static constexpr int kKSteps = D / 32;           // 32-wide k-steps of Q.K^T
    static constexpr int kDBlocks = D / 16;          // 16-row blocks of O^T
    static constexpr int kKVec = kTileN * D / 4 / kThreads;  // K float4 per thread
    static constexpr int kVKeys = D / 16;            // keys per thread in the V transpose
    static constexpr int kVGroups = kTileN / kVKeys; // key groups per dim group
};

// Storage position of key `key` (0..63) inside a V^T row.  Within each
// 32-key group the f16 P operand of lane group g (lanes 16g..16g+15) holds
// keys {4g..4g+3} and {16+4g..16+4g+3}; the A operand of that lane group
// reads positions 8g..8g+7, so position p must hold key
// 16*bit2(p) + 8*bit4(p) + 4*bit3(p) + (p & 3).  Inverting: bits 4,3,2 of the
// position are bits 3,2,4 of the key.
__device__ __forceinline__ int vt_pos(int key) {
    return (key & 0x23) | (((key >> 3) & 1) << 4) | (((key >> 2) & 1) << 3) |
           (((key >> 4) & 1) << 2);
}

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

__device__ __forceinline__ float4_t load4(const float *p) {
    return *reinterpret_cast<const float4_t *>(p);
}

// Registers holding one K/V tile between its global load and its LDS store.
template <int D>
struct TileRegs {
    float4_t k[Shape<D>::kKVec];
    float4_t v[Shape<D>::kVKeys];
};

// Global -> registers.  Keys at or past `n_valid` read as zero (ragged
// tail); FULL tiles (n_valid == kTileN) skip the per-load guards.
template <int D, bool FULL>
__device__ __forceinline__ void load_tile_impl(const float *__restrict__ kg,
                                               const float *__restrict__ vg,
                                               int key0, int n_valid,
                                               TileRegs<D> &r, int tid) {
    using S = Shape<D>;
    constexpr int kVecPerRow = D / 4;
#pragma unroll
    for (int u = 0; u < S::kKVec; ++u) {
        const int f = tid + kThreads * u;
        const int key = f / kVecPerRow;
        const int c = (f % kVecPerRow) * 4;
        r.k[u] = (FULL || key < n_valid) ? load4(kg + (key0 + key) * D + c)
                                         : (float4_t){0.f, 0.f, 0.f, 0.f};
    }
    // V: thread owns kVKeys consecutive keys x 4 consecutive dims.  Adjacent
    // lanes take adjacent key groups so the transposed LDS store below hits
    // distinct banks.
    const int kgi = tid % S::kVGroups;
    const int c4 = tid / S::kVGroups;
#pragma unroll
    for (int e = 0; e < S::kVKeys; ++e) {
        const int key = kgi * S::kVKeys + e;
        r.v[e] = (FULL || key < n_valid) ? load4(vg + (key0 + key) * D + 4 * c4)
                                         : (float4_t){0.f, 0.f, 0.f, 0.f};
    }
}

template <int D>
__device__ __forceinline__ void load_tile(const float *__restrict__ kg,
                                          const float *__restrict__ vg,
                                          int key0, int n_valid,
                                          TileRegs<D> &r, int tid) {
    if (n_valid == kTileN)
        load_tile_impl<D, true>(kg, vg, key0, n_valid, r, tid);
    else
        load_tile_impl<D, false>(kg, vg, key0, n_valid, r, tid);
}

// Registers -> LDS: K row-major [key][dim] (hi, and lo for SPLIT), V
// transposed [dim][vt_pos(key)].
template <int D, bool SPLIT>
__device__ __forceinline__ void store_tile(const TileRegs<D> &r,
                                           _Float16 (*kh)[Shape<D>::kKRow],
                                           _Float16 (*kl)[Shape<D>::kKRow],
                                           _Float16 (*vt)[Shape<D>::kVRow],
                                           int tid) {
    using S = Shape<D>;
    constexpr int kVecPerRow = D / 4;
#pragma unroll
    for (int u = 0; u < S::kKVec; ++u) {
        const int f = tid + kThreads * u;
        const int key = f / kVecPerRow;
        const int c = (f % kVecPerRow) * 4;
        const half4_t hi = cvt4(r.k[u]);
        *reinterpret_cast<half4_t *>(&kh[key][c]) = hi;
        if constexpr (SPLIT) {
            const float4_t back = __builtin_convertvector(hi, float4_t);
            *reinterpret_cast<half4_t *>(&kl[key][c]) = cvt4(r.k[u] - back);
        }
    }
    const int kgi = tid % S::kVGroups;
    const int c4 = tid / S::kVGroups;
    const int pos = vt_pos(kgi * S::kVKeys);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if constexpr (S::kVKeys == 4) {
            const half2_t a = cvt2(r.v[0][j], r.v[1][j]);
            const half2_t b = cvt2(r.v[2][j], r.v[3][j]);
            *reinterpret_cast<half4_t *>(&vt[4 * c4 + j][pos]) =
                (half4_t){a[0], a[1], b[0], b[1]};
        } else {
            *reinterpret_cast<half2_t *>(&vt[4 * c4 + j][pos]) =
                cvt2(r.v[0][j], r.v[1][j]);
        }
    }
}

__device__ __forceinline__ float4_t mfma16(half8_t a, half8_t b, float4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

template <int D, bool SPLIT>
__global__ void __launch_bounds__(kThreads)
attention_fwd_kernel(const float *__restrict__ q, const float *__restrict__ k,
                     const float *__restrict__ v, float *__restrict__ out,
                     int n_patches, int q_blocks, int total_blocks) {
    using S = Shape<D>;
    __shared__ __attribute__((aligned(16))) _Float16 kh_s[2][kTileN][S::kKRow];
    __shared__ __attribute__((aligned(16))) _Float16 vt_s[2][D][S::kVRow];
    __shared__ __attribute__((aligned(16)))
    _Float16 kl_s[SPLIT ? 2 : 1][SPLIT ? kTileN : 1][S::kKRow];

    const int logical = xcd_remap(blockIdx.x, total_blocks);
    const int head = logical / q_blocks;
    const int qblk = logical - head * q_blocks;
    const size_t base = (size_t)head * (size_t)n_patches * D;
    const float *__restrict__ qg = q + base;
    const float *__restrict__ kg = k + base;
    const float *__restrict__ vg = v + base;
    float *__restrict__ og = out + base;

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int l16 = lane & 15;  // query column inside a 16-row block
    const int g4 = lane >> 4;   // lane group 0..3
    const int row0 = qblk * kBlockM + wave * kRowsPerWave;

    // Query fragments (B operand of S^T = K Q^T), pre-multiplied by log2(e).
    half8_t qh[2][S::kKSteps];
    half8_t ql[2][S::kKSteps];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const int row = row0 + 16 * qb + l16;
#pragma unroll
        for (int st = 0; st < S::kKSteps; ++st) {
            float4_t x0 = {0.f, 0.f, 0.f, 0.f}, x1 = x0;
            if (row < n_patches) {
                const float *p = qg + row * D + 32 * st + 8 * g4;
                x0 = load4(p) * kLog2e;
                x1 = load4(p + 4) * kLog2e;
            }
            const half4_t h0 = cvt4(x0), h1 = cvt4(x1);
            qh[qb][st] = (half8_t){h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
            if constexpr (SPLIT) {
                const half4_t e0 = cvt4(x0 - __builtin_convertvector(h0, float4_t));
                const half4_t e1 = cvt4(x1 - __builtin_convertvector(h1, float4_t));
                ql[qb][st] = (half8_t){e0[0], e0[1], e0[2], e0[3], e1[0], e1[1], e1[2], e1[3]};
            }
        }
    }

    float4_t o[2][S::kDBlocks];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int db = 0; db < S::kDBlocks; ++db) o[qb][db] = (float4_t){0.f, 0.f, 0.f, 0.f};
    float m_run[2] = {-__builtin_inff(), -__builtin_inff()};
    float l_run[2] = {0.f, 0.f};

    const int n_tiles = (n_patches + kTileN - 1) / kTileN;
    TileRegs<D> regs;
    load_tile<D>(kg, vg, 0, min(kTileN, n_patches), regs, tid);
    store_tile<D, SPLIT>(regs, kh_s[0], kl_s[0], vt_s[0], tid);
    __syncthreads();

    for (int t = 0; t < n_tiles; ++t) {
        const int buf = t & 1;
        const bool has_next = t + 1 < n_tiles;
        if (has_next)
            load_tile<D>(kg, vg, (t + 1) * kTileN,
                         min(kTileN, n_patches - (t + 1) * kTileN), regs, tid);

        // ---- S^T = K Q^T for 64 keys x 32 queries
        float4_t s[2][4];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) s[qb][kb] = (float4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
            for (int st = 0; st < S::kKSteps; ++st) {
                const half8_t a = *reinterpret_cast<const half8_t *>(
                    &kh_s[buf][16 * kb + l16][32 * st + 8 * g4]);
#pragma unroll
                for (int qb = 0; qb < 2; ++qb) s[qb][kb] = mfma16(a, qh[qb][st], s[qb][kb]);
                if constexpr (SPLIT) {
#pragma unroll
                    for (int qb = 0; qb < 2; ++qb) s[qb][kb] = mfma16(a, ql[qb][st], s[qb][kb]);
                    const half8_t al = *reinterpret_cast<const half8_t *>(
                        &kl_s[buf][16 * kb + l16][32 * st + 8 * g4]);
#pragma unroll
                    for (int qb = 0; qb < 2; ++qb) s[qb][kb] = mfma16(al, qh[qb][st], s[qb][kb]);
                }
            }
        }

        // ---- keys past n_patches (only in the last tile)
        const int key_lim = n_patches - t * kTileN;
        if (key_lim < kTileN) {
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (16 * kb + 4 * g4 + i >= key_lim) {
                        s[0][kb][i] = -__builtin_inff();
                        s[1][kb][i] = -__builtin_inff();
                    }
        }

        // ---- online softmax: running max, rescale, P = 2^(s - m)
        float m_new[2];
        bool raise_any = false;
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            float mx = s[qb][0][0];
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[qb][kb][i]);
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const bool raise = mx > m_run[qb] + kRescaleSlack;
            m_new[qb] = raise ? mx : m_run[qb];
            raise_any |= raise;
        }
        if (__any(raise_any)) {
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                const float alpha = __builtin_amdgcn_exp2f(m_run[qb] - m_new[qb]);
                l_run[qb] *= alpha;
#pragma unroll
                for (int db = 0; db < S::kDBlocks; ++db) o[qb][db] *= alpha;
                m_run[qb] = m_new[qb];
            }
        }

        half8_t p[2][2];
        const half2_t ones = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            const float m = m_run[qb];
            float lsum = 0.f;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                half2_t h[4];
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    const float4_t x = s[qb][2 * ks + half];
                    h[2 * half] = cvt2(__builtin_amdgcn_exp2f(x[0] - m),
                                       __builtin_amdgcn_exp2f(x[1] - m));
                    h[2 * half + 1] = cvt2(__builtin_amdgcn_exp2f(x[2] - m),
                                           __builtin_amdgcn_exp2f(x[3] - m));
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) lsum = __builtin_amdgcn_fdot2(h[j], ones, lsum, false);
                p[qb][ks] = (half8_t){h[0][0], h[0][1], h[1][0], h[1][1],
                                      h[2][0], h[2][1], h[3][0], h[3][1]};
            }
            l_run[qb] += lsum;
        }

        // ---- O^T += V^T P^T
#pragma unroll
        for (int db = 0; db < S::kDBlocks; ++db) {
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const half8_t a = *reinterpret_cast<const half8_t *>(
                    &vt_s[buf][16 * db + l16][32 * ks + 8 * g4]);
#pragma unroll
                for (int qb = 0; qb < 2; ++qb) o[qb][db] = mfma16(a, p[qb][ks], o[qb][db]);
            }
        }

        if (has_next)
            store_tile<D, SPLIT>(regs, kh_s[buf ^ 1], kl_s[SPLIT ? (buf ^ 1) : 0],
                                 vt_s[buf ^ 1], tid);
        __syncthreads();
    }

    // ---- epilogue: out = O / l for rows inside the head
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        float lt = l_run[qb];
        lt += __shfl_xor(lt, 16);
        lt += __shfl_xor(lt, 32);
        const float inv = 1.0f / lt;
        const int row = row0 + 16 * qb + l16;
        if (row < n_patches) {
#pragma unroll
            for (int db = 0; db < S::kDBlocks; ++db)
                *reinterpret_cast<float4_t *>(og + row * D + 16 * db + 4 * g4) = o[qb][db] * inv;
        }
    }
}

}  // namespace vattn
