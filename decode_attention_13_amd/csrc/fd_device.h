// fd_device.h -- gfx950 device primitives for the decode-attention kernels:
// 16-lane DPP row reductions, 16-byte global loads, dtype unpack/pack, and the
// online-softmax state combine. Wave64 throughout.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

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

// ---------------------------------------------------------------- lane pairs across rows
// The two values of lanes l and l ^ MASK (MASK = 16: neighbouring rows; 32: the
// two wave halves), from gfx950's v_permlane16_swap / v_permlane32_swap (VALU
// lane swaps, no LDS round trip). Both lanes of a pair receive the same two
// values in the same order (the lower row's or half's first), so any combine
// written in terms of (lo, hi) gives bit-identical results in both lanes.
struct LanePair {
    float lo, hi;
};

template <int MASK>
__device__ __forceinline__ LanePair lane_pair(float x) {
    static_assert(MASK == 16 || MASK == 32, "rows (16) or halves (32)");
    const unsigned u = __builtin_bit_cast(unsigned, x);
    unsigned r0, r1;  // copied out of the returned vector before any bit_cast
    if constexpr (MASK == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
        r0 = r[0];
        r1 = r[1];
    } else {
        const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
        r0 = r[0];
        r1 = r[1];
    }
    return {__builtin_bit_cast(float, r0), __builtin_bit_cast(float, r1)};
}

template <int MASK>
__device__ __forceinline__ float pair_max(float x) {
    const LanePair p = lane_pair<MASK>(x);
    return fmaxf(p.lo, p.hi);
}

template <int MASK>
__device__ __forceinline__ float pair_sum(float x) {
    const LanePair p = lane_pair<MASK>(x);
    return p.lo + p.hi;
}

// Max / sum over the whole wave; every lane receives the same value.
__device__ __forceinline__ float wave_max(float x) { return pair_max<32>(pair_max<16>(row16_max(x))); }

__device__ __forceinline__ float wave_sum(float x) { return pair_sum<32>(pair_sum<16>(row16_sum(x))); }

// Threads of a split-kernel workgroup (both split kernels run 4 waves); a
// constant rather than blockDim, which would cost a late kernel-argument load.
constexpr int kSplitThreads = 256;

// ---------------------------------------------------------------- thread index of an item
// threadIdx.x as a value the optimizer cannot see through. A persistent
// workgroup runs its items in a loop; offsets derived from this value are then
// recomputed for every item instead of being hoisted out of the loop, where they
// would all stay live and push the kernel into register spills.
__device__ __forceinline__ int item_tid() {
    int t = threadIdx.x;
    asm volatile("" : "+v"(t));
    return t;
}

// ---------------------------------------------------------------- kernel arguments
// Marks kernel-argument values as used at this point (an empty asm reading them
// from scalar registers). Called at kernel entry, it makes the compiler fetch
// them with the first kernel-argument load instead of sinking a second scalar
// load, a full memory round trip, behind an early-exit branch.
template <typename T>
__device__ __forceinline__ void pin_arg(const T &x) {
    asm volatile("" ::"s"(x));
}

template <typename... Ts>
__device__ __forceinline__ void pin_args(const Ts &...xs) {
    (pin_arg(xs), ...);
}

// ---------------------------------------------------------------- math
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }  // v_exp_f32
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }   // v_log_f32

// ---------------------------------------------------------------- loads
// 16-byte loads of data read exactly once per step: marked non-temporal so the
// stream does not evict the small reused arrays (q, block table, workspace).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint4 load_stream16(const void *p) {
    const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return make_uint4(x.x, x.y, x.z, x.w);
}

__device__ __forceinline__ uint4 load16(const void *p) { return *reinterpret_cast<const uint4 *>(p); }

// The same streamed loads as buffer loads from a wave-uniform base: the base
// goes into a buffer descriptor in scalar registers and each lane adds a 32-bit
// byte offset, so no 64-bit address is formed per lane. readfirstlane tells the
// compiler what the caller guarantees (the base is the same in every lane);
// without it the descriptor would be built in a loop over lanes. Descriptor:
// raw (stride 0), 2^31 - 1 bytes in range, word 3 = 0x00020000 (32-bit data
// format); policy nt (non-temporal, as load_stream16). Measured against the
// global form on the 32-head bf16 decode: 1.7% faster at 128k tokens, 1.5% at
// 4k (the nt, sc0, sc1 policy bits made no difference). Used for 16-bit rows;
// fp32 rows measured the same either way and 8-byte E4M3 rows slower, so
// those keep the global form. stream_rsrc also serves the prefill kernel's
// whole-tile fetches (temporal there: every query tile of a head re-reads them).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t stream_rsrc(const void *uniform_base) {
    const uint64_t a = reinterpret_cast<uint64_t>(uniform_base);
    const uint64_t u = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(a >> 32)) << 32) |
                       (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(u), (short)0, 0x7fffffff, 0x00020000);
}
constexpr int kCpolNt = 2;  // cache policy bits of a buffer load: nt

__device__ __forceinline__ uint4 buffer_stream16(const void *uniform_base, uint32_t off) {
    const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(stream_rsrc(uniform_base), off, 0, kCpolNt);
    return make_uint4(x.x, x.y, x.z, x.w);
}

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

// ---------------------------------------------------------------- KV rows
// load(p) reads a lane's piece at any address; load_at(base, off) reads it at
// base + off where base is the same in every lane of the wave.
// Cache element types and how a 16-lane row group reads one 128-element K/V
// row: lane c owns 8 elements. Raw is what one lane loads per row piece.
//   bf16/f16: elements [8c, 8c+8), one 16-byte load.
//   fp32:     elements [4c, 4c+4) and [64+4c, 64+4c+4), two 16-byte loads.
//   FP8 E4M3: elements [8c, 8c+8), one 8-byte load; codes are converted to fp32
//             in registers (v_cvt_pk_f32_fp8, OCP E4M3 on gfx950), which is exact.
struct fp8e4m3 {
    unsigned char bits;
};

typedef float f32x2 __attribute__((ext_vector_type(2)));

template <typename KV>
struct KvRow;

template <>
struct KvRow<float> {
    typedef uint4 Raw;
    static constexpr int kPieces = 2;
    __device__ static int offset(int c, int piece) { return piece * 64 + 4 * c; }
    __device__ static int index(int c, int e) { return (e >> 2) * 64 + 4 * c + (e & 3); }
    __device__ static Raw load(const char *p) { return load_stream16(p); }
    __device__ static Raw load_at(const char *uniform_base, uint32_t off) { return load(uniform_base + off); }
    __device__ static void unpack(const Raw *x, float *f) { Elem<float>::unpack(x, f); }
};

template <>
struct KvRow<__bf16> {
    typedef uint4 Raw;
    static constexpr int kPieces = 1;
    __device__ static int offset(int c, int) { return 8 * c; }
    __device__ static int index(int c, int e) { return 8 * c + e; }
    __device__ static Raw load(const char *p) { return load_stream16(p); }
    __device__ static Raw load_at(const char *uniform_base, uint32_t off) { return buffer_stream16(uniform_base, off); }
    __device__ static void unpack(const Raw *x, float *f) { Elem<__bf16>::unpack(x, f); }
};

template <>
struct KvRow<_Float16> {
    typedef uint4 Raw;
    static constexpr int kPieces = 1;
    __device__ static int offset(int c, int) { return 8 * c; }
    __device__ static int index(int c, int e) { return 8 * c + e; }
    __device__ static Raw load(const char *p) { return load_stream16(p); }
    __device__ static Raw load_at(const char *uniform_base, uint32_t off) { return buffer_stream16(uniform_base, off); }
    __device__ static void unpack(const Raw *x, float *f) { Elem<_Float16>::unpack(x, f); }
};

__device__ __forceinline__ void e4m3x4_to_f32(uint32_t w, float *f) {
    const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
    const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
    f[0] = lo.x;
    f[1] = lo.y;
    f[2] = hi.x;
    f[3] = hi.y;
}

template <>
struct KvRow<fp8e4m3> {
    typedef uint2 Raw;
    static constexpr int kPieces = 1;
    __device__ static int offset(int c, int) { return 8 * c; }
    __device__ static int index(int c, int e) { return 8 * c + e; }
    __device__ static Raw load(const char *p) {
        const u32x2 x = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(p));
        return make_uint2(x.x, x.y);
    }
    __device__ static Raw load_at(const char *uniform_base, uint32_t off) { return load(uniform_base + off); }
    __device__ static void unpack(const Raw *x, float *f) {
        e4m3x4_to_f32(x->x, f);
        e4m3x4_to_f32(x->y, f + 4);
    }
};

// ---------------------------------------------------------------- softmax state
// Online-softmax state in the log2 domain: running max m (of scale*log2(e)*s),
// running sum l of 2^(s - m), and the unnormalised output. Combining two
// states rescales both to the larger max ("FlashAttention 与推理算子", section
// "FlashAttention：分块 + online softmax"). An empty state has m = -inf, l = 0.
__device__ __forceinline__ float finite_or_zero(float m) { return m == -INFINITY ? 0.f : m; }

template <typename T>
struct Pair;
template <>
struct Pair<float> {
    typedef float2 type;
    __device__ static type make(float a, float b) { return make_float2(a, b); }
};
template <>
struct Pair<__bf16> {
    typedef __bf16 type __attribute__((ext_vector_type(2)));
    __device__ static type make(float a, float b) { return type{(__bf16)a, (__bf16)b}; }
};
template <>
struct Pair<_Float16> {
    typedef _Float16 type __attribute__((ext_vector_type(2)));
    __device__ static type make(float a, float b) { return type{(_Float16)a, (_Float16)b}; }
};

// Output row (b, h) elements 2*lane, 2*lane + 1, rounded to T (nearest even).
template <typename T>
__device__ __forceinline__ void store_out_pair(void *out, size_t bh, int lane, float2 v) {
    typedef typename Pair<T>::type P2;
    reinterpret_cast<P2 *>(reinterpret_cast<T *>(out) + bh * kHeadDim)[lane] = Pair<T>::make(v.x, v.y);
}

// ---------------------------------------------------------------- split boundaries
// A contiguous cache (one sequence; every split in one round of workgroups)
// has max(1, floor(L / chunk)) splits: split s covers [s*chunk, (s+1)*chunk)
// except the last, which runs to L and so also takes the remainder (chunk ..
// 2*chunk - 1 tokens), so no short split straggles behind the others.
// A paged batch has ceil(L / chunk) splits, the cut of "[CUDA 优化实战] 纯手搓
// flash decoding sm120", section "1. flash decoding": all but the last hold
// chunk tokens and the last the remainder (1 .. chunk tokens). Those short
// splits are numbered last, largest first (paged item order below), so they
// fill the end of a launch that would otherwise end on chunk-sized items.
// Either way every token is covered once and no split is empty; L = 0 has none.
template <bool PAGED>
__device__ __forceinline__ int splits_of(int L, int chunk) {
    if (L <= 0) return 0;
    return PAGED ? (L + chunk - 1) / chunk : max(1, L / chunk);
}

__device__ __forceinline__ int split_end(int split, int n, int L, int chunk) {
    return split == n - 1 ? L : (split + 1) * chunk;
}

// ---------------------------------------------------------------- split prologue
// Length of sequence b and, for a paged cache, the split's slice of its block
// table staged in LDS (entries clamped into [0, num_pages)). The table loads
// are issued together with the length load, before the length is known: the
// slice read is bounded by the table row, not by L_b, so both cost one round
// trip. Every thread of the workgroup must call this (it holds a barrier).
// Returns L_b clamped to [0, max_len]; *page_first is the table index of
// s_pages[0].
template <bool PAGED>
__device__ __forceinline__ int split_prologue(const SplitArgs &a, int b, int t_begin, int *s_pages, int *page_first) {
    if constexpr (!PAGED) {
        *page_first = 0;
        return a.max_len;
    } else {
        const int L_raw = a.seq_lens[b];
        const int first = t_begin >> a.page_shift;
        const int last = min((t_begin + a.chunk - 1) >> a.page_shift, a.max_blocks - 1);  // a split holds <= chunk tokens
        const int32_t *row = a.block_table + (size_t)b * a.max_blocks + first;
        for (int i = item_tid(); i <= last - first; i += kSplitThreads)
            s_pages[i] = min(max(row[i], 0), a.num_pages - 1);
        __syncthreads();
        *page_first = first;
        return max(0, min(L_raw, a.max_len));
    }
}

// ---------------------------------------------------------------- debug checks
// With fd_options.debug_checks a paged split records the first out-of-range
// value it meets (the kernels clamp either way, so no access leaves the cache):
// the workgroup of a sequence's last split (or of the item that writes an empty
// sequence's zeros) checks L_b against [0, max_len], and every split checks
// the table entries of the blocks it reads. The winner of the compare-and-swap
// on the kind word writes the rest.
__device__ __forceinline__ void report_bad(int *err, int kind, int b, int index, int value) {
    if (atomicCAS(err, 0, kind) == 0) {
        err[1] = b;
        err[2] = index;
        err[3] = value;
    }
}

// Every thread of the workgroup calls this (no barrier inside). The split reads
// tokens [t_begin, t_end) (t_end <= t_begin when the split is empty); owns_len
// is set for the one item of the sequence that checks its length.
__device__ __forceinline__ void check_paged_split(const SplitArgs &a, int b, int t_begin, int t_end, bool owns_len) {
    if (owns_len && item_tid() == 0) {
        const int L_raw = a.seq_lens[b];
        if (L_raw < 0 || L_raw > a.max_len) report_bad(a.err, kBadSeqLen, b, 0, L_raw);
    }
    if (t_end <= t_begin) return;
    const int first = t_begin >> a.page_shift, last = (t_end - 1) >> a.page_shift;
    const int32_t *row = a.block_table + (size_t)b * a.max_blocks;
    for (int i = first + (int)item_tid(); i <= last; i += kSplitThreads) {
        const int page = row[i];
        if (page < 0 || page >= a.num_pages) report_bad(a.err, kBadTableEntry, b, i, page);
    }
}

// ---------------------------------------------------------------- paged item order
// Sequence b of a paged batch holds f_b = floor(L_b / chunk) full splits of
// chunk tokens and, when chunk does not divide L_b, a remainder split of
// r_b = L_b - f_b * chunk tokens; an empty sequence holds one item that writes
// its zeros. Workgroups start, and persistent workgroups claim, in item
// order, and the items are numbered largest first (the longest-first rule of
// list scheduling): the full splits, sequence by sequence, then the remainder
// items by decreasing size (ties by sequence), the empty sequences last. The
// splits themselves, and so the results, do not depend on the order.
//
// build_work_list fills s_full[b] = full splits of the sequences before b
// (s_full[B] = F, their total) and s_rem[k] = the sequence of the k-th
// remainder item, and returns the item count F + R; it runs in two halves
// (list_full_splits, list_remainders) because full-split items are found
// from s_full alone. Every thread of the workgroup must call these (they hold
// barriers). B <= kMaxListSeqs.
struct WorkList {
    int full[kMaxListSeqs + 1];
    int rem[kMaxListSeqs];
    // Sort key of sequence b's remainder item: its size (0 for an empty sequence)
    // times kMaxListSeqs plus kMaxListSeqs - 1 - b, so that keys are distinct and
    // a larger key is a larger item or an as large one of an earlier sequence;
    // -1 for a sequence without a remainder item and past the batch.
    __attribute__((aligned(16))) int key[kMaxListSeqs];
    int wave[kSplitThreads / 64];
    int wave_rem[kSplitThreads / 64];
    int rem_count;
};
static_assert(kMaxListSeqs == 4 * kSplitThreads, "the work list gives each thread 4 sequences");
// A remainder is shorter than a split, which spans at most kMaxSplitPages - 2
// pages of at most 1024 tokens: its sort key fits an int.
static_assert((long long)((kMaxSplitPages - 2) * 1024 + 1) * kMaxListSeqs < (1LL << 31), "sort keys overflow");

// First half of the list: s_full and rem_count (the remainder items, R), from
// the sequence lengths. Returns F. Every thread of the workgroup must call this
// (it holds a barrier).
__device__ __forceinline__ int list_full_splits(const SplitArgs &a, WorkList &w) {
    const int t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    int cnt[4], key[4];
    int local = 0, local_r = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {  // sequences 4t .. 4t + 3
        const int bb = 4 * t + j;
        cnt[j] = 0;
        key[j] = -1;
        if (bb < a.B) {
            const int L = max(0, min(a.seq_lens[bb], a.max_len));
            cnt[j] = L / a.chunk;
            const int r = L - cnt[j] * a.chunk;
            if (r > 0 || L == 0) key[j] = r * kMaxListSeqs + (kMaxListSeqs - 1 - bb);
        }
        local += cnt[j];
        local_r += key[j] >= 0 ? 1 : 0;
    }
    *reinterpret_cast<int4 *>(&w.key[4 * t]) = make_int4(key[0], key[1], key[2], key[3]);
    int x = local, xr = local_r;  // inclusive scans over the wave
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off, 64);
        const int yr = __shfl_up(xr, off, 64);
        if (lane >= off) {
            x += y;
            xr += yr;
        }
    }
    if (lane == 63) {
        w.wave[wave] = x;
        w.wave_rem[wave] = xr;
    }
    __syncthreads();
    int base = 0;
    for (int v = 0; v < wave; ++v) base += w.wave[v];
    int excl = base + x - local;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int bb = 4 * t + j;
        if (bb < a.B) w.full[bb] = excl;
        excl += cnt[j];
    }
    if (t == kSplitThreads - 1) {  // the last thread's ends are the totals
        w.full[a.B] = excl;
        int rtot = 0;
        for (int v = 0; v < kSplitThreads / 64; ++v) rtot += w.wave_rem[v];
        w.rem_count = rtot;
    }
    __syncthreads();
    return w.full[a.B];
}

// Second half: s_rem, the remainder items in order. Rank of each: the number of
// larger keys (larger items, or as large ones of earlier sequences), read four
// keys per LDS access (every lane reads the same address: a broadcast). Up to
// kSplitThreads sequences each thread ranks one (B compares), beyond that its
// four. Every thread of the workgroup must call this, after list_full_splits
// (it holds a barrier).
__device__ __forceinline__ void list_remainders(const SplitArgs &a, WorkList &w) {
    const int t = threadIdx.x;
    const int4 *keys4 = reinterpret_cast<const int4 *>(w.key);
    const int n4 = (a.B + 3) / 4;
    if (a.B <= kSplitThreads) {
        const int k_me = t < a.B ? w.key[t] : -1;
        if (k_me >= 0) {
            int rank = 0;
            for (int i = 0; i < n4; ++i) {
                const int4 k4 = keys4[i];
                rank += (k4.x > k_me) + (k4.y > k_me) + (k4.z > k_me) + (k4.w > k_me);
            }
            w.rem[rank] = t;
        }
    } else {
        const int4 mine = keys4[t];
        const int key[4] = {mine.x, mine.y, mine.z, mine.w};
        int rank[4] = {0, 0, 0, 0};
        for (int i = 0; i < n4; ++i) {
            const int4 k4 = keys4[i];
#pragma unroll
            for (int j = 0; j < 4; ++j) rank[j] += (k4.x > key[j]) + (k4.y > key[j]) + (k4.z > key[j]) + (k4.w > key[j]);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (key[j] >= 0) w.rem[rank[j]] = 4 * t + j;
    }
    __syncthreads();
}

// The whole list; returns the item count F + R.
__device__ __forceinline__ int build_work_list(const SplitArgs &a, WorkList &w) {
    const int F = list_full_splits(a, w);
    list_remainders(a, w);
    return F + w.rem_count;
}

// The sequence of the r-th full split: the largest b with full[b] <= r. full
// does not decrease, and a sequence with no full split shares its start with
// the next one, so the largest such b is the one holding r.
__device__ __forceinline__ int find_sequence(const int *full, int B, int r) {
    int lo = 0, hi = B - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (full[mid] <= r) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// (sequence, split) of item `item` < F + R.
__device__ __forceinline__ void work_list_item(const WorkList &w, int B, int item, int &b, int &split) {
    const int F = w.full[B];
    if (item < F) {
        b = find_sequence(w.full, B, item);
        split = item - w.full[b];
    } else {
        b = w.rem[item - F];
        split = w.full[b + 1] - w.full[b];  // the remainder follows the full splits
    }
}

// When total_kv understated the batch, items past the grid have no workgroup.
// Their results become NaN instead of silently missing: the output rows of
// sequences with at most one split, and the LSE of the missing splits of the
// others (the merge then yields NaN). Run by one workgroup.
template <typename T>
__device__ void poison_unlisted(const SplitArgs &a, const WorkList &w, int items) {
    const float nan = __builtin_nanf("");
    for (int item = a.grid_items; item < items; ++item) {
        int b, split;
        work_list_item(w, a.B, item, b, split);
        const int n = splits_of<true>(max(0, min(a.seq_lens[b], a.max_len)), a.chunk);
        if (n <= 1) {
            T *o = reinterpret_cast<T *>(a.out) + (size_t)b * a.H * kHeadDim;
            for (int i = threadIdx.x; i < a.H * kHeadDim; i += kSplitThreads) o[i] = Elem<T>::store_cast(nan);
        } else {
            for (int h = threadIdx.x; h < a.H; h += kSplitThreads)
                a.ws_lse[((size_t)b * a.H + h) * a.num_splits + split] = nan;
        }
    }
}

// The item of a one-item-per-workgroup paged launch. With a work list, grid y
// is the item number in the order above; otherwise grid y is the split and
// grid z the sequence, and splits past a sequence's end are the grid's empty
// slots (the item function finds them empty). Returns false when the
// workgroup has nothing to do. Every thread of the workgroup must call this
// (the work list holds barriers).
template <typename T>
__device__ __forceinline__ bool paged_item(const SplitArgs &a, WorkList &w, int &b, int &split) {
    if (a.work_list) {
        const int items = build_work_list(a, w);
        const int item = blockIdx.y;
        if (item == a.grid_items - 1 && blockIdx.x == 0 && items > a.grid_items)
            poison_unlisted<T>(a, w, items);  // total_kv was short: fail loudly
        if (item >= items) return false;
        work_list_item(w, a.B, item, b, split);
        return true;
    }
    b = blockIdx.z;
    split = blockIdx.y;
    return true;
}

// ---------------------------------------------------------------- paged item loop
// The items of a paged workgroup, each handed to item(args, slice, b, split).
// One item per workgroup (paged_item) unless the launch is persistent
// (a separate kernel instantiation, PERSIST): then grid x is one workgroup per
// resident slot, and each numbers the items once (the work list) and takes
// units in item order, largest first; unit q is head slice q % slices of list
// item q / slices. Workgroup x starts with unit x without asking anyone; later
// units are claimed from one counter (unit gridDim.x + claim), each claim made
// when the workgroup's current unit is done. No workgroup waits for another, a
// slot never idles waiting for the dispatcher, and an XCD that streams slower
// (the XCDs of this GPU differ by up to a third on the same batch) takes fewer
// units. A claim made at the start of the unit before, to hide its round trip,
// cost more than it saved: at the end of the launch the slots still holding
// claimed units ran up to a whole unit past those that found the counter
// empty (GQA4 batch: split kernel 206 us against 196 us). Same-address device
// atomics serialize (about 11 ns apiece here), so no claim is made at the
// start, when every workgroup would make one at once, and workgroups count
// themselves out on one exit counter per XCD (x % kExitGroups); the last of a
// group counts the group out, and the last group sets every counter back to
// zero for the next call. Every thread of the workgroup must call this (it
// holds barriers).
// The kernel arguments as read back from an LDS copy for every item: the
// compiler barrier before the read keeps the optimizer from hoisting anything
// derived from them out of the item loop, and readfirstlane returns them to
// scalar registers. The pointers are taken from the kernel argument itself,
// which the compiler knows to address global memory: a pointer read back from
// LDS is generic, every load through it becomes a flat load, and a flat load
// also counts against the LDS wait counter, so each wait for an LDS access
// would wait for every K/V load in flight as well.
__device__ __forceinline__ SplitArgs reload_args(const SplitArgs &kern, const SplitArgs *s_args) {
    asm volatile("" ::: "memory");
    SplitArgs r;
    const int *src = reinterpret_cast<const int *>(s_args);
    int *dst = reinterpret_cast<int *>(&r);
#pragma unroll
    for (int i = 0; i < (int)(sizeof(SplitArgs) / 4); ++i) dst[i] = __builtin_amdgcn_readfirstlane(src[i]);
    r.q = kern.q;
    r.k = kern.k;
    r.v = kern.v;
    r.block_table = kern.block_table;
    r.seq_lens = kern.seq_lens;
    r.ws_o = kern.ws_o;
    r.ws_lse = kern.ws_lse;
    r.out = kern.out;
    r.err = kern.err;
    r.counters = kern.counters;
    return r;
}

template <typename T, bool PERSIST, typename ItemFn>
__device__ __forceinline__ void paged_items(const SplitArgs &a, ItemFn item) {
    __shared__ WorkList s_list;
    if constexpr (!PERSIST) {
        int b, split;
        if (paged_item<T>(a, s_list, b, split)) item(a, blockIdx.x, b, split);
    } else {
        __shared__ int s_claim;
        __shared__ SplitArgs s_args;
        unsigned *const claims = a.counters + kQueueBase;          // units claimed past the first round
        unsigned *const groups_done = claims + kQueueStride;       // exit groups whose workgroups are all gone
        const int grp = (int)(blockIdx.x % kExitGroups);
        unsigned *const gone = groups_done + (1 + grp) * kQueueStride;
        if (threadIdx.x == 0) s_args = a;
        // The remainder items are ranked only when the first of them is taken:
        // a workgroup whose first unit is a full split (on most batches all of
        // them) starts streaming without waiting for the ranking.
        const int F = list_full_splits(a, s_list);
        const int total = (F + s_list.rem_count) * a.slices;
        const bool claiming = total > (int)gridDim.x;  // else the first round holds every unit: no counter is used
        bool ranked = false;
        int next = (int)blockIdx.x;  // thread 0: the next unit
        for (;;) {
            if (threadIdx.x == 0) s_claim = next;
            __syncthreads();  // also ends every use of LDS by the previous item
            const int q = s_claim;
            __syncthreads();  // s_claim read by all before thread 0 writes the next one
            if (q >= total) break;
            const int u = q / a.slices;
            if (u >= F && !ranked) {  // uniform over the workgroup
                list_remainders(a, s_list);
                ranked = true;
            }
            int b, split;
            work_list_item(s_list, a.B, u, b, split);
            item(reload_args(a, &s_args), q - u * a.slices, b, split);
            if (threadIdx.x == 0) next = claiming ? (int)gridDim.x + (int)atomicAdd(claims, 1u) : total;
        }
        if (claiming && threadIdx.x == 0) {
            const unsigned members = (gridDim.x - grp + kExitGroups - 1) / kExitGroups;
            const unsigned groups = min(gridDim.x, (unsigned)kExitGroups);
            if (atomicAdd(gone, 1u) + 1u == members && atomicAdd(groups_done, 1u) + 1u == groups) {
                // every workgroup has made its last claim
                __hip_atomic_store(claims, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(groups_done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                for (int g = 0; g < kExitGroups; ++g)
                    __hip_atomic_store(groups_done + (1 + g) * kQueueStride, 0u, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
}

// ---------------------------------------------------------------- split epilogue
// Partials read by another workgroup of the same launch (fused merge) are
// written and read as device-scope relaxed atomics: on gfx950 these are plain
// vector stores and loads with the sc1 bit, which write through and read past
// the per-XCD L2 caches, so they are coherent across the chip without an L2
// writeback.
__device__ __forceinline__ void store_device(float *p, float x) {
    __hip_atomic_store(p, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_device(const float *p) {
    return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// End of a split in a fused launch ("[CUDA 优化实战] 纯手搓 flash decoding sm120",
// section "1. flash decoding": the partials of a (sequence, head) are combined
// once all of its splits are done; here the last of its workgroups does it
// instead of a second kernel). Every wave first waits until its partial stores
// have completed, then one thread counts the workgroup in on the (sequence,
// head slice) counter; the workgroup that brings it to n_b resets it to zero
// for the next call and merges the n_b partials of its nh heads by log-sum-exp
// (the merge kernel's arithmetic): w_s = e^(lse_s - max lse) / sum_s' e^(...),
// o = sum_s w_s O_s. No thread waits for another workgroup, so nothing can
// hang: the last one to arrive always finds every partial in place.
// The merging thread of output element (h, d) loads every lse_s of head h and
// every O_s[d] before it uses any, so the merge costs one round trip to memory
// (each of these loads crosses the L2 to reach the other XCDs' stores); the
// planner fuses only where nh * n_b is at most kFusedMaxRows (at most nh * n_b /
// 2 + n_b loads per thread).
template <typename T, int NS>
__device__ __forceinline__ void fused_merge_rows(const SplitArgs &a, int b, int h0, int nh, int n_b) {
    const size_t row0 = ((size_t)b * a.H + h0) * a.num_splits;
    // elements per thread and pass: 32 partial values (and as many lse values) in registers
    constexpr int kPer = (32 / NS) < 8 ? (32 / NS) : 8;
    for (int i0 = 0; i0 < nh * kHeadDim; i0 += kSplitThreads * kPer) {
        float lse[kPer][NS], x[kPer][NS];
#pragma unroll
        for (int e = 0; e < kPer; ++e) {
            const int i = min(i0 + e * kSplitThreads + (int)item_tid(), nh * kHeadDim - 1);
            const int hh = i / kHeadDim;
            const int d = i - hh * kHeadDim;
            const float *lrow = a.ws_lse + row0 + (size_t)hh * a.num_splits;
            const float *orow = a.ws_o + (row0 + (size_t)hh * a.num_splits) * kHeadDim + d;
#pragma unroll
            for (int sp = 0; sp < NS; ++sp) {
                const int s2 = min(sp, n_b - 1);
                lse[e][sp] = load_device(lrow + s2);
                x[e][sp] = load_device(orow + (size_t)s2 * kHeadDim);
            }
        }
#pragma unroll
        for (int e = 0; e < kPer; ++e) {
            const int i = i0 + e * kSplitThreads + (int)item_tid();
            if (i >= nh * kHeadDim) break;
            const int hh = i / kHeadDim;
            const int d = i - hh * kHeadDim;
            float M = -INFINITY;
#pragma unroll
            for (int sp = 0; sp < NS; ++sp)
                if (sp < n_b) M = fmaxf(M, lse[e][sp]);
            const float mu = finite_or_zero(M);
            float W = 0.f, o = 0.f;
#pragma unroll
            for (int sp = 0; sp < NS; ++sp) {
                if (sp < n_b) {
                    const float w = exp2_fast((lse[e][sp] - mu) * kLog2e);
                    W += w;
                    o = __builtin_fmaf(w, x[e][sp], o);
                }
            }
            reinterpret_cast<T *>(a.out)[((size_t)b * a.H + h0 + hh) * kHeadDim + d] =
                Elem<T>::store_cast(W > 0.f ? o / W : 0.f);
        }
    }
}

template <typename T>
__device__ void fused_merge_tail(const SplitArgs &a, int slice, int b, int h0, int nh, int n_b) {
    __shared__ int s_last;
    __builtin_amdgcn_s_waitcnt(0);  // vmcnt(0) expcnt(0) lgkmcnt(0): this wave's partial stores are done
    __syncthreads();
    if (item_tid() == 0) {
        unsigned *ctr = a.counters + (size_t)b * a.slices + slice;
        const unsigned prev = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int last = prev + 1u == (unsigned)n_b;
        if (last) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = last;
    }
    __syncthreads();
    if (!s_last) return;  // uniform over the workgroup
    // n_b rounded up to a compiled split count (at most kFusedMaxSplits)
    if (n_b <= 8) fused_merge_rows<T, 8>(a, b, h0, nh, n_b);
    else fused_merge_rows<T, 32>(a, b, h0, nh, n_b);
}

// Stores one workgroup's result for query heads h0 .. h0+nh-1 of sequence b,
// split `split` of n_b. value(hh, d, lse) returns the split's normalised
// output element and sets its natural-log lse. When n_b == 1 the split is the
// whole sequence and o is written directly; otherwise the partial goes to the
// workspace, for the merge kernel or, in a fused launch (FUSED: a kernel
// instantiation of its own, so the merge-kernel path carries none of this
// code), for the last workgroup of the sequence's head slice.
template <typename T, bool FUSED, typename ValueFn>
__device__ void finish_split(const SplitArgs &a, int slice, int b, int h0, int nh, int split, int n_b,
                             ValueFn value) {
    const bool direct = n_b == 1;
    for (int i = item_tid(); i < nh * kHeadDim; i += kSplitThreads) {
        const int hh = i / kHeadDim;
        const int d = i - hh * kHeadDim;
        float lse;
        const float o = value(hh, d, lse);
        const size_t bh = (size_t)b * a.H + h0 + hh;
        if (direct) {
            reinterpret_cast<T *>(a.out)[bh * kHeadDim + d] = Elem<T>::store_cast(o);
        } else if (FUSED) {
            const size_t row = bh * a.num_splits + split;
            store_device(a.ws_o + row * kHeadDim + d, o);
            if (d == 0) store_device(a.ws_lse + row, lse);
        } else {
            const size_t row = bh * a.num_splits + split;
            a.ws_o[row * kHeadDim + d] = o;
            if (d == 0) a.ws_lse[row] = lse;
        }
    }
    if constexpr (FUSED) {
        if (!direct) fused_merge_tail<T>(a, slice, b, h0, nh, n_b);
    }
}

}  // namespace fd
