// fd_device.h -- gfx950 device primitives for the decode-attention kernels:
// 16-lane DPP row reductions, 16-byte global loads, dtype unpack/pack, and the
// online-softmax state combine. Wave64 throughout.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fd_internal.h"

namespace fd {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int kHeadDim = 128;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------- DPP row ops
// A DPP "row" is 16 consecutive lanes. The controls used here permute lanes
// inside a row only, so every source lane exists.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL,
                                                                  0xF, 0xF, false));
}
constexpr int kQuadSwap1 = 0xB1;   // quad_perm [1,0,3,2]: lane ^ 1
constexpr int kQuadSwap2 = 0x4E;   // quad_perm [2,3,0,1]: lane ^ 2
constexpr int kHalfMirror = 0x141; // row_half_mirror: lane i <- 7 - i within each 8
constexpr int kRowMirror = 0x140;  // row_mirror: lane i <- 15 - i within the row

// Sum over the 16 lanes of a row; every lane of the row receives the total.
__device__ __forceinline__ float row16_sum(float x) {
    x += dpp<kQuadSwap1>(x);
    x += dpp<kQuadSwap2>(x);
    x += dpp<kHalfMirror>(x);
    x += dpp<kRowMirror>(x);
    return x;
}

__device__ __forceinline__ float row16_max(float x) {
    x = fmaxf(x, dpp<kQuadSwap1>(x));
    x = fmaxf(x, dpp<kQuadSwap2>(x));
    x = fmaxf(x, dpp<kHalfMirror>(x));
    x = fmaxf(x, dpp<kRowMirror>(x));
    return x;
}

__device__ __forceinline__ float wave_max(float x) {
    for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m, 64));
    return x;
}

__device__ __forceinline__ float wave_sum(float x) {
    for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
    return x;
}

// ---------------------------------------------------------------- math
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }  // v_exp_f32
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }   // v_log_f32

// ---------------------------------------------------------------- loads
// 16-byte loads of data read exactly once per step: marked non-temporal so the
// stream does not evict the small reused arrays (q, block table, workspace).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 load_stream16(const void *p) {
    const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return make_uint4(x.x, x.y, x.z, x.w);
}

__device__ __forceinline__ uint4 load16(const void *p) { return *reinterpret_cast<const uint4 *>(p); }

// ---------------------------------------------------------------- dtype traits
// Each lane of a 16-lane row owns 8 of the 128 head-dim elements. For 16-bit
// types they are elements [8c, 8c+8) (one 16-byte load per row). For fp32 they
// are [4c, 4c+4) and [64+4c, 64+4c+4), so each of the two 16-byte loads of a
// row covers 256 contiguous bytes across the 16 lanes.
template <typename T>
struct Elem;

template <>
struct Elem<float> {
    static constexpr int kLoads = 2;                                   // 16-byte loads per row per lane
    __device__ static int offset(int c, int piece) { return piece * 64 + 4 * c; }  // element offset of piece
    __device__ static int index(int c, int e) { return (e >> 2) * 64 + 4 * c + (e & 3); }
    __device__ static void unpack(const uint4 *x, float *f) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            f[4 * i + 0] = __builtin_bit_cast(float, x[i].x);
            f[4 * i + 1] = __builtin_bit_cast(float, x[i].y);
            f[4 * i + 2] = __builtin_bit_cast(float, x[i].z);
            f[4 * i + 3] = __builtin_bit_cast(float, x[i].w);
        }
    }
    // q . k over the lane's 8 elements (q pre-unpacked to fp32 in qf).
    __device__ static float dot(const float *qf, const uint32_t *, const uint4 *kx) {
        float k[8];
        unpack(kx, k);
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) s = __builtin_fmaf(qf[e], k[e], s);
        return s;
    }
    __device__ static float store_cast(float x) { return x; }
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

template <>
struct Elem<__bf16> {
    static constexpr int kLoads = 1;
    __device__ static int offset(int c, int) { return 8 * c; }
    __device__ static int index(int c, int e) { return 8 * c + e; }
    __device__ static void unpack(const uint4 *x, float *f) {
        const uint32_t w[4] = {x->x, x->y, x->z, x->w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = bf16_lo(w[i]);
            f[2 * i + 1] = bf16_hi(w[i]);
        }
    }
    // Packed bf16 pairs multiplied on v_dot2 with fp32 accumulation.
    __device__ static float dot(const float *, const uint32_t *qp, const uint4 *kx) {
        const uint32_t w[4] = {kx->x, kx->y, kx->z, kx->w};
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, qp[i]), __builtin_bit_cast(bf16x2, w[i]),
                                                s, false);
        return s;
    }
    __device__ static __bf16 store_cast(float x) { return (__bf16)x; }  // round to nearest even
};

template <>
struct Elem<_Float16> {
    static constexpr int kLoads = 1;
    __device__ static int offset(int c, int) { return 8 * c; }
    __device__ static int index(int c, int e) { return 8 * c + e; }
    __device__ static void unpack(const uint4 *x, float *f) {
        const uint32_t w[4] = {x->x, x->y, x->z, x->w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f16x2 h = __builtin_bit_cast(f16x2, w[i]);
            f[2 * i] = (float)h.x;
            f[2 * i + 1] = (float)h.y;
        }
    }
    __device__ static float dot(const float *, const uint32_t *qp, const uint4 *kx) {
        const uint32_t w[4] = {kx->x, kx->y, kx->z, kx->w};
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            s = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, qp[i]), __builtin_bit_cast(f16x2, w[i]), s, false);
        return s;
    }
    __device__ static _Float16 store_cast(float x) { return (_Float16)x; }  // round to nearest even
};

// ---------------------------------------------------------------- KV addressing
// Where the row of (token t, KV head kvh) lives, in bytes from the cache base:
//   contiguous [S, Hkv, D]:                 (t*Hkv + kvh) * row
//   paged [pages, page_size, Hkv, D]:       ((page(t)*page_size + t%page_size)*Hkv + kvh) * row
// with page(t) = block_table[b][t / page_size] ("FlashAttention 与推理算子",
// section "PagedAttention") and row = D * sizeof(T).
// Kernels walk tokens in 16-token blocks starting at multiples of 16. When the
// cache is contiguous, or paged with page_size >= 16, a block lies inside one
// page, so its base is the same for every lane (held in scalar registers) and
// a lane adds the 32-bit offset (t - block start) * Hkv * row. With smaller
// pages every row is looked up on its own.
template <int MODE>
struct KvAddr {
    const int *pages;       // LDS: the split's slice of the block table (paged)
    int page_first;         // table index of pages[0]
    int page_shift;
    int token_bytes;        // Hkv * row: distance between consecutive slots/tokens
    size_t head_bytes;      // kvh * row

    // Byte offset of the first row of the 16-token block starting at T.
    __device__ size_t block(int T) const {
        if constexpr (MODE == kContig) {
            return (size_t)T * token_bytes + head_bytes;
        } else {
            const int page = __builtin_amdgcn_readfirstlane(pages[(T >> page_shift) - page_first]);
            const size_t slot_row = ((size_t)page << page_shift) + (size_t)(T & ((1 << page_shift) - 1));
            return slot_row * token_bytes + head_bytes;
        }
    }
    // Byte offset of any single row (every mode).
    __device__ size_t row(int t) const {
        if constexpr (MODE == kContig) {
            return (size_t)t * token_bytes + head_bytes;
        } else {
            const int page = pages[(t >> page_shift) - page_first];
            const size_t slot_row = ((size_t)page << page_shift) + (size_t)(t & ((1 << page_shift) - 1));
            return slot_row * token_bytes + head_bytes;
        }
    }
};

template <typename T>
__device__ __forceinline__ uint4 load_stream16_at(const T *base, size_t byte_off) {
    return load_stream16(reinterpret_cast<const char *>(base) + byte_off);
}

// ---------------------------------------------------------------- softmax state
// Online-softmax state in the log2 domain: running max m (of scale*log2(e)*s),
// running sum l of 2^(s - m), and the unnormalised output. Combining two
// states rescales both to the larger max ("FlashAttention 与推理算子", section
// "FlashAttention：分块 + online softmax"). An empty state has m = -inf, l = 0.
__device__ __forceinline__ float finite_or_zero(float m) { return m == -INFINITY ? 0.f : m; }

}  // namespace fd
