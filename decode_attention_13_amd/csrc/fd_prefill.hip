// fd_prefill.hip -- prefill attention (many queries, optional causal mask) on
// the matrix cores (gfx950, wave64, v_mfma_f32_32x32x16_{bf16,f16}).
//
// The blocked algorithm of "FlashAttention 与推理算子", section
// "FlashAttention：分块 + online softmax": a block of queries walks the key
// blocks, keeps a running max and sum per query row and rescales its output
// accumulator; with the causal mask (same section) key blocks past the query
// block's last row are never visited and the diagonal block is masked element
// by element. The FlashAttention-2 layout the page describes (each Q block its
// own workgroup, waves split by query rows) is kept.
//
// Workgroup: 4 waves x 32 queries of one (sequence, head); key tiles of 32
// tokens shared by the 4 waves. Per wave and tile, with query columns in the
// 32-wide MFMA shape (lane l holds query l % 32):
//   S^T[key, q] = K[key, :] . Q[q, :]       one 32x32x16 MFMA chain of 8
//   online softmax per query (column), log2 domain, fp32
//   O^T[d, q] += V^T[d, key] . P^T[key, q]  four chains of two 32x32x16 MFMAs
//       (bf16: P split into two 16-bit parts, two MFMAs each, which keeps P.V
//       near fp32)
// The 32x32 shape does the same work in half as many MFMAs as the 16x16 one,
// each about 6% cheaper per flop on this chip, from the same LDS reads.
// The loop is a three-stage software pipeline: P.V of tile j and the scores of
// tile j + 2 go to the matrix cores while the VALU takes the softmax of j + 1.
// P^T needs no lane movement (the S accumulator elements of a lane are the key
// slots of its P.V operand, in an order the V^T reads follow); V^T comes from
// the LDS tile with ds_read_b64_tr_b16.
//
// K and V tiles go from global memory straight into LDS (global_load_lds,
// 16 bytes a lane, no registers on the way) through rings of four tiles each,
// so a tile is requested three iterations before it is read: the loads meet
// the latency of L2 and HBM without holding the loop. A tile is 32 unpadded
// 256-byte rows with their 16-byte chunks permuted per row (swz below), so the
// K fragment reads and the transposed V reads both spread over all banks.
//
// bf16 with a workspace takes three launches: prefill_convert_v_kernel writes
// an f16 copy of V (exact below 65536 in magnitude) and a flag per chunk of
// each sequence's V rows; prefill_kernel<bf16, f16> runs P.V on f16 MFMAs from
// that copy, P in f16, for the sequences with no flag set; and
// prefill_kernel<bf16, bf16> reruns the flagged ones with the split P. Without
// a workspace the last kernel runs alone, on every sequence.
#include "fd_device.h"
#include "fd_internal.h"

namespace fd {

namespace {

constexpr int kWaves = 4;      // waves per workgroup
constexpr int kWaveQ = 32;     // queries per wave (the MFMA's 32 columns)
constexpr int kThreads = 64 * kWaves;
constexpr int kKTile = 32;     // keys per LDS tile
constexpr int kRow = 256;      // bytes of a K or V row in LDS (128 16-bit elements)
constexpr int kTileBytes = kKTile * kRow;
constexpr int kRing = 4;       // LDS tiles per ring (K and V each)
constexpr int kDmaPerTile = kTileBytes / (kThreads * 16);  // 16-byte loads per lane and tile
constexpr int kXcds = 8;       // XCDs of the MI355X, each with its own L2
constexpr float kLazyLog2 = 8.f;  // the running max trails the true one by at most this (log2 units)

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2v __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

// IEEE 754-2019 maximum (v_maximum3_f32 on gfx950): -inf and finite inputs as
// usual, NaN propagates; unlike maxnum it needs no canonicalisation of the MFMA
// results it reads.
__device__ __forceinline__ float max2(float x, float y) { return __builtin_elementwise_maximum(x, y); }

// LDS chunk swizzle: 16-byte chunk x of tile row r is stored at x ^ swz(r),
// swz swapping the two 2-bit halves of r mod 16. 16 consecutive rows at one
// chunk (a K fragment read) land on 16 distinct chunks, and 8 rows aligned
// to 8 at 4 chunks aligned to 4 (a transposed V read) on 16 distinct chunks,
// two each: both reads move their bytes at the LDS's full width.
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

template <typename T>
struct Mma;

template <>
struct Mma<__bf16> {
    static constexpr bool kSplitP = true;  // bf16 keeps 8 bits of P: use hi + lo
    __device__ static f32x16 mma32(uint4 a, uint4 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                       c, 0, 0, 0);
    }
    __device__ static uint32_t pack2(float x, float y) {
        return __builtin_bit_cast(uint32_t, bf16x2{(__bf16)x, (__bf16)y});
    }
    // x = hi + lo: hi is x truncated to bf16 (its upper 16 bits, packed for two
    // values by one byte permute), lo the exact remainder x - hi rounded to
    // bf16, so hi + lo keeps 16 significant bits of x.
    __device__ static void split2(float x, float y, uint32_t &hi, uint32_t &lo) {
        const uint32_t xb = __builtin_bit_cast(uint32_t, x), yb = __builtin_bit_cast(uint32_t, y);
        hi = __builtin_amdgcn_perm(yb, xb, 0x07060302u);  // (y & 0xffff0000) | (x >> 16)
        lo = pack2(x - __builtin_bit_cast(float, xb & 0xffff0000u), y - __builtin_bit_cast(float, yb & 0xffff0000u));
    }
};

template <>
struct Mma<_Float16> {
    static constexpr bool kSplitP = false;  // f16 keeps 11 bits of P (P < 2^8: no overflow)
    __device__ static f32x16 mma32(uint4 a, uint4 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                      0, 0, 0);
    }
    __device__ static void split2(float x, float y, uint32_t &hi, uint32_t &lo) {
        hi = __builtin_bit_cast(uint32_t, f16x2{(_Float16)x, (_Float16)y});
        lo = 0;
    }
    // acc + the two f16 values of a packed pair
    __device__ static float sum2(uint32_t pair, float acc) {
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pair), f16x2{(_Float16)1.f, (_Float16)1.f}, acc, false);
    }
};

// One 16-byte global load per lane written straight to LDS: lane l's bytes go
// to LDS address lds + 16 * l (lds wave-uniform, in m0, which the compiler
// sets as the asm's input). Written as inline assembly so that the compiler,
// which would otherwise wait for every such load before any later LDS read,
// leaves the waits to wait_vm below; the instruction has no register result.
// The s_nop keeps the one wait state the LDS-load form needs after m0 is set.
__device__ __forceinline__ void dma16(const void *gptr, uint32_t lds) {
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(gptr), "{m0}"(__builtin_amdgcn_readfirstlane(lds))
                 : "memory");
}
// The same load from a wave-uniform base (in SGPRs) plus a 32-bit lane offset.
__device__ __forceinline__ void dma16_at(const void *sbase, uint32_t off, uint32_t lds) {
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(off), "s"(sbase), "{m0}"(__builtin_amdgcn_readfirstlane(lds))
                 : "memory");
}

// s_waitcnt on the vector-memory counter alone (expcnt and lgkmcnt left free):
// wait until at most N loads of this wave are in flight.
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt has 6 bits");
    __builtin_amdgcn_s_waitcnt(((N >> 4) << 14) | (0xf << 8) | (0x7 << 4) | (N & 0xf));
}

// Whether sequence b's V holds a value outside f16's range: the 1 KiB flag row
// of the sequence, 16 bytes a lane, entries at or past `chunks` masked off.
__device__ __forceinline__ bool v_flagged(uint4 fl, int chunks, int lane) {
    const uint32_t w[4] = {fl.x, fl.y, fl.z, fl.w};
    uint32_t any = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int cnt = min(max(chunks - (16 * lane + 4 * j), 0), 4);  // valid flag bytes in word j
        any |= w[j] & (cnt >= 4 ? 0xffffffffu : (1u << (8 * cnt)) - 1u);
    }
    return __builtin_amdgcn_ballot_w64(any != 0) != 0;
}

// TQ: type of q, k and o (the S MFMAs); TV: type of v and of P (the P.V
// MFMAs). <bf16, f16> runs on the f16 copy of V that the conversion kernel
// below writes. Two waves per SIMD (two workgroups per CU): the register
// budget is 256.
template <typename TQ, typename TV>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void prefill_kernel(PrefillArgs a) {
    using MS = Mma<TQ>;
    using M = Mma<TV>;
    constexpr int kQTile = kWaves * kWaveQ;  // queries per workgroup
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: wave-level branches stay scalar
    pin_args(a.q, a.k, a.v, a.o, a.scale_log2);
    // The 1-D grid is dealt round robin over the 8 XCDs (workgroup i runs on XCD
    // i % 8, as its (i / 8)-th). When the (sequence, head) units divide evenly,
    // each XCD takes its own eighth of them, so the query tiles of a head share
    // one L2 where the K/V tiles they all walk stay resident; within an XCD the
    // tiles go longest first (with the causal mask the last query tiles hold the
    // most keys), which balances the XCD's workgroup slots. Otherwise the whole
    // grid goes longest first.
    const int units = a.H * a.B;
    const int lin = blockIdx.x;
    int unit, qt_rev;
    if (units % kXcds == 0) {
        const int per = units / kXcds;
        const int t = lin / kXcds;
        unit = (lin % kXcds) * per + t % per;
        qt_rev = t / per;
    } else {
        unit = lin % units;
        qt_rev = lin / units;
    }
    const int qt = a.q_tiles - 1 - qt_rev;
    const int h = unit % a.H;
    const int b = unit / a.H;
    const int kvh = h / a.G;
    const int N = a.N;
    // The split-P kernel behind the f16 one runs only the sequences whose V
    // did not convert: the others leave before any tile load.
    if (a.flag_mode == kPrefillRunIfFlagged &&
        !v_flagged(load16(a.flags + (size_t)b * kPrefillFlagRow + 16 * lane), a.flag_chunks, lane))
        return;
    const int q0 = qt * kQTile + wave * kWaveQ;  // this wave's first query
    const int q_last = q0 + kWaveQ - 1;
    const int kv_end = a.causal ? min(N, (qt + 1) * kQTile) : N;
    const int ntiles = (kv_end + kKTile - 1) / kKTile;

    __shared__ __attribute__((aligned(16))) char sK[kRing][kTileBytes];
    __shared__ __attribute__((aligned(16))) char sV[kRing][kTileBytes];

    uint4 qf[8];  // the lane's query (q0 + lane % 32), head-dim slots 16k + 8 (lane / 32) .. + 8
    // sl > 0 (a zero scale arrives as the least normal float), so -inf * sl
    // stays -inf and a masked score gives exp2 = 0.
    const float sl = fabsf(a.scale_log2);

    // Tile loads: load i of a wave fills 1 KB of the tile, rows 4 * (kDmaPerTile *
    // wave + i) .. + 3, lane l the 16 bytes at l * 16 (row + l / 16, stored
    // chunk l % 16), which hold chunk (l % 16) ^ swz(row) of that key's row.
    // Keys past N re-read key N - 1 (never used: masked, or past the workgroup).
    static_assert(sizeof(TQ) == 2 && sizeof(TV) == 2, "K and V rows are 256 bytes");
    const size_t tok_bytes = (size_t)a.Hkv * kHeadDim * 2;
    const char *kg = reinterpret_cast<const char *>(a.k) + ((size_t)b * N * a.Hkv + kvh) * kHeadDim * 2;
    const char *vg = reinterpret_cast<const char *>(a.v) + ((size_t)b * N * a.Hkv + kvh) * kHeadDim * 2;
    // Lane offsets within a tile (row * token bytes + chunk; 32 rows of at most
    // 65535 * 256 bytes fit in 32 bits): a tile wholly below N is one scalar base
    // plus these, with no per-lane address arithmetic; a tile reaching past N
    // clamps its keys lane by lane.
    int dma_row[kDmaPerTile];
    uint32_t dma_col[kDmaPerTile], dma_off[kDmaPerTile];
#pragma unroll
    for (int i = 0; i < kDmaPerTile; ++i) {
        dma_row[i] = 4 * (kDmaPerTile * wave + i) + (lane >> 4);
        dma_col[i] = (uint32_t)(((lane & 15) ^ swz(dma_row[i])) * 16);
        dma_off[i] = (uint32_t)dma_row[i] * (uint32_t)tok_bytes + dma_col[i];
    }
    auto dma = [&](const char *src, char (*ring)[kTileBytes], int t) {
        char *dst = ring[t & (kRing - 1)];
        if (t * kKTile + kKTile <= N) {
            const char *base = src + (size_t)t * kKTile * tok_bytes;
#pragma unroll
            for (int i = 0; i < kDmaPerTile; ++i)
                dma16_at(base, dma_off[i], (uint32_t)(uintptr_t)(dst + (kDmaPerTile * wave + i) * 1024));
        } else {
#pragma unroll
            for (int i = 0; i < kDmaPerTile; ++i) {
                const int key = min(t * kKTile + dma_row[i], N - 1);
                const char *p = src + (size_t)key * tok_bytes + dma_col[i];
                dma16(p, (uint32_t)(uintptr_t)(dst + (kDmaPerTile * wave + i) * 1024));
            }
        }
    };

    // O^T of the lane's query: block db holds head-dim rows db*32 + 8 (i / 4) +
    // 4 (lane / 32) + i % 4 in element i (the 32x32 MFMA accumulator layout).
    f32x16 acc[4];
    float m = -INFINITY, lsum = 0.f;  // running max (same in lanes l and l ^ 32) and this lane's share of the sum
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;
    const int hb = lane >> 5;  // which half of the k slots (and of the accumulator rows) this lane holds
    const int qc = lane & 31;  // this lane's query (column) within the wave

    struct Scores {
        f32x16 v;  // element i: key 8 (i / 4) + 4 hb + i % 4 of the tile, query q0 + qc
    };
    // The lane's LDS byte offsets within a ring slot, formed once: each
    // fragment read is then the slot's base plus one of these.
    // K (S^T, k step ks of 16 head-dim slots): key row l % 32, chunk 2 ks + hb,
    // stored at that chunk ^ swz(row).
    uint32_t k_off[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) k_off[ks] = (uint32_t)(qc * kRow + (((2 * ks + hb) ^ swz(qc)) << 4));
    // V^T for head-dim block db, k step kv, lane l (group G = l / 16, c = l %
    // 16): transposed 8-byte reads of key rows 16 kv + 4 hb + c / 4 and the same
    // + 8, columns db*32 + 16 (G % 2) + 4 (c % 4) .. + 3 (chunk 4 db + 2 (G % 2)
    // + (c % 4) / 2, stored at that chunk ^ swz(row)); lane l receives column
    // db*32 + l % 32. Rows 16 apart share swz, so k step 1 is k step 0 + 4096.
    uint32_t v_off[8];  // [2 db + lh]
    {
        const int cc = lane & 15, bq = cc & 3;
        const int r0 = 4 * hb + (cc >> 2);  // row within the 8-row block, 0..7
        const int cpart = 2 * ((lane >> 4) & 1) + (bq >> 1);
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int lh = 0; lh < 2; ++lh) {
                const int r = r0 + 8 * lh;
                v_off[2 * db + lh] = (uint32_t)(r * kRow + (((4 * db + cpart) ^ swz(r)) << 4) + (bq & 1) * 8);
            }
    }

    // S^T of tile t from the K ring.
    auto scores = [&](int t, Scores &r) {
        lds_char *kt = (lds_char *)(uintptr_t)sK[t & (kRing - 1)];
#pragma unroll
        for (int i = 0; i < 16; ++i) r.v[i] = 0.f;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            const u32x4 kr = *(lds_u32x4 *)(kt + k_off[ks]);
            r.v = MS::mma32(make_uint4(kr.x, kr.y, kr.z, kr.w), qf[ks], r.v);
        }
    };

    // Masked scores become -inf, so their P is exactly 0: keys at or past N,
    // and with the causal mask keys after the query.
    auto mask_scores = [&](int j, Scores &sc) {
        const int q_me = q0 + qc;
        const int room = (a.causal ? min(q_me, N - 1) : N - 1) - j * kKTile - 4 * hb;  // key offset limit
#pragma unroll
        for (int i = 0; i < 16; ++i)
            if (8 * (i / 4) + (i % 4) > room) sc.v[i] = -INFINITY;
    };

    // Online softmax of one tile with a lazy running max: m moves only when the
    // tile's max exceeds it by more than kLazyLog2 (P then stays below
    // 2^kLazyLog2), so the accumulators are rescaled a few times per row instead
    // of on most tiles. Any subtracted constant gives the same softmax; the final
    // division uses the sum taken with the same constants. Produces P^T in the
    // MFMA operand layout (bf16: hi and lo parts) and alpha, the factor for the
    // accumulators; returns whether any row needs it. P^T for the k step kv of
    // P.V (keys 16 kv .. + 15) is accumulator elements 8 kv .. + 7 as they stand:
    // k slot 8 hb + j holds key 16 kv + 8 (j / 4) + 4 hb + j % 4, the same keys
    // the transposed V reads below put in that slot.
    struct Probs {
        uint4 hi[2], lo[2];
    };
    float alpha = 1.f;
    auto softmax = [&](const Scores &sc, Probs &pr) {
        // Raw-score max (the scale is > 0: its sign was moved into Q).
        float mt = sc.v[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) mt = max2(mt, sc.v[i]);
        const LanePair lp = lane_pair<32>(mt);
        mt = max2(lp.lo, lp.hi);
        const float mt_s = mt * sl;  // -inf stays -inf
        const float m_old = m;
        const float m_new = mt_s > m_old + kLazyLog2 ? mt_s : m_old;
        const float mu = finite_or_zero(m_new);
        alpha = exp2_fast(m_old - mu);  // 0 while m_old is -inf
        const bool rescale = m_new != m_old && m_old > -INFINITY;
        m = m_new;
        float pe[16];
        float ps = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            pe[i] = exp2_fast(__builtin_fmaf(sc.v[i], sl, -mu));
            if constexpr (M::kSplitP) ps += pe[i];
        }
#pragma unroll
        for (int kv = 0; kv < 2; ++kv) {
            uint32_t hw[4], lw[4];
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) M::split2(pe[8 * kv + 2 * e2], pe[8 * kv + 2 * e2 + 1], hw[e2], lw[e2]);
            pr.hi[kv] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
            if constexpr (M::kSplitP) pr.lo[kv] = make_uint4(lw[0], lw[1], lw[2], lw[3]);
            // f16 P: the sum is taken over the rounded values P.V uses, two per
            // v_dot2_f32_f16.
            if constexpr (!M::kSplitP)
#pragma unroll
                for (int e2 = 0; e2 < 4; ++e2) ps = M::sum2(hw[e2], ps);
        }
        lsum = __builtin_fmaf(lsum, alpha, ps);
        return __builtin_amdgcn_ballot_w64(rescale) != 0;
    };
    auto rescale_acc = [&]() {
#pragma unroll
        for (int db = 0; db < 4; ++db) acc[db] *= alpha;
    };

    // O^T += V^T . P^T for tile t from the V ring (reads at v_off above).
    auto pv = [&](int t, const Probs &pr) {
        lds_char *vt = (lds_char *)(uintptr_t)sV[t & (kRing - 1)];
#pragma unroll
        for (int db = 0; db < 4; ++db) {
#pragma unroll
            for (int kv = 0; kv < 2; ++kv) {
                const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_i16x4 *)(vt + v_off[2 * db] + kv * 16 * kRow));
                const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_i16x4 *)(vt + v_off[2 * db + 1] + kv * 16 * kRow));
                const u32x2v lo2 = __builtin_bit_cast(u32x2v, lo);
                const u32x2v hi2 = __builtin_bit_cast(u32x2v, hi);
                const uint4 va = make_uint4(lo2.x, lo2.y, hi2.x, hi2.y);
                acc[db] = M::mma32(va, pr.hi[kv], acc[db]);
                if constexpr (M::kSplitP) acc[db] = M::mma32(va, pr.lo[kv], acc[db]);
            }
        }
    };

    // Software pipeline, three tiles deep: iteration j runs P.V of tile j and the
    // scores of tile j + 2 on the matrix cores while the VALU takes the softmax
    // of tile j + 1 (none of the three waits for another). Iteration j requests
    // K(j + 5) and V(j + 3) into the ring slots that iteration j - 1 finished
    // reading, then waits for K(j + 3) and V(j + 1) (requested two iterations
    // earlier; the 8 loads of the two later iterations may still be in flight)
    // and meets the other waves at one barrier. Every iteration requests its
    // tiles, past the end too (they re-read key N - 1 and are never read), so
    // the count of loads in flight is the same on every iteration; the tiles
    // requested past the end are the last loads to wait for.
    // Tiles this wave computes: with the causal mask those after its last query
    // are skipped (the workgroup still loads them for its other waves). Scores
    // formed past a wave's last tile read whatever the K ring holds and are
    // never used.
    static_assert(kDmaPerTile == 2, "the waits below count 4 loads per iteration");
    const int n_w = a.causal ? min(ntiles, q_last / kKTile + 1) : ntiles;
    auto masked = [&](int j) { return j * kKTile + kKTile > N || (a.causal && j * kKTile + kKTile - 1 > q0); };
    // The first tiles, in the order they are needed: K0 K1 V0 K2, then the
    // query rows, one wait for all of them (so the waits the compiler places for
    // the queries count every load in flight), then V1 K3 V2; K4 shares its ring
    // slot with K0 and follows the barrier after K0 is read.
    // On the f16 copy of V, the sequence's flag row comes first, so the one wait
    // covers it too.
    uint4 vflags = make_uint4(0u, 0u, 0u, 0u);
    if (a.flag_mode == kPrefillRunIfClean) vflags = load16(a.flags + (size_t)b * kPrefillFlagRow + 16 * lane);
    dma(kg, sK, 0);
    dma(kg, sK, 1);
    dma(vg, sV, 0);
    dma(kg, sK, 2);
    // Q fragments (B operand of S): query q0 + qc, head-dim slots 16 ks + 8 hb .. + 8.
    {
        const int qr = min(q0 + qc, N - 1);
        const TQ *qrow = reinterpret_cast<const TQ *>(a.q) + (((size_t)b * N + qr) * a.H + h) * kHeadDim;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) qf[ks] = load16(qrow + ks * 16 + hb * 8);
    }
    // A negative scale is moved into Q (a sign flip is exact), so the running
    // max can be taken over the raw scores and scaled afterwards.
    if (a.scale_log2 < 0.f) {
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            qf[ks].x ^= 0x80008000u;
            qf[ks].y ^= 0x80008000u;
            qf[ks].z ^= 0x80008000u;
            qf[ks].w ^= 0x80008000u;
        }
    }

    wait_vm<0>();
    // A sequence whose V did not convert is left to the split-P kernel (every
    // wave reads the same row and leaves; no load is in flight).
    if (a.flag_mode == kPrefillRunIfClean && v_flagged(vflags, a.flag_chunks, lane)) return;
    dma(vg, sV, 1);
    dma(kg, sK, 3);
    dma(vg, sV, 2);
    __builtin_amdgcn_s_barrier();
    Scores sc0, sc1;
    scores(0, sc0);
    scores(1, sc1);  // tile 1, or discarded
    if (masked(0)) mask_scores(0, sc0);
    Probs p_cur;
    softmax(sc0, p_cur);   // m starts at -inf: nothing to rescale
    bool rescale = false;  // alpha of the last softmax applies before the next P.V
    __builtin_amdgcn_s_barrier();  // every wave has read K0 and K1
    dma(kg, sK, 4);
    for (int j = 0; j < ntiles; ++j) {
        dma(kg, sK, j + 5);
        dma(vg, sV, j + 3);
        if (rescale) {  // softmax(j) moved m: before P.V(j)
            rescale_acc();
            rescale = false;
        }
        if (j + 1 < n_w) {
            if (masked(j + 1)) mask_scores(j + 1, sc1);
            Probs p_next;
            // One block for the scheduler: P.V(j) and scores(j + 2) on the matrix
            // cores, softmax(j + 1) on the VALU.
            pv(j, p_cur);
            Scores sc2;
            scores(j + 2, sc2);
            rescale = softmax(sc1, p_next);
            // Interleave the block for the scheduler: one MFMA, then four VALU
            // instructions, for each MFMA of the block (left alone, the compiler
            // bunched the softmax); bf16, whose P.V issues two MFMAs per V
            // fragment, also takes one LDS read per group.
            constexpr int kBlockMfma = 8 + 8 * (M::kSplitP ? 2 : 1);
#pragma unroll
            for (int sg = 0; sg < kBlockMfma; ++sg) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
                if constexpr (M::kSplitP) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
                __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // VALU
            }
            sc1 = sc2;
            p_cur = p_next;
        } else if (j < n_w) {
            pv(j, p_cur);
        }
        wait_vm<8>();  // K(j + 3) and V(j + 1)
        __builtin_amdgcn_s_barrier();
    }

    wait_vm<0>();  // no load may still be writing LDS when the workgroup ends

    {
        const float ls = pair_sum<32>(lsum);
        const int q_me = q0 + qc;
        if (q_me < N) {
            const float inv = 1.f / ls;
            TQ *orow = reinterpret_cast<TQ *>(a.o) + (((size_t)b * N + q_me) * a.H + h) * kHeadDim;
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int i4 = 0; i4 < 4; ++i4) {
                    typedef typename Pair<TQ>::type P2;
                    P2 *dst = reinterpret_cast<P2 *>(orow + db * 32 + 8 * i4 + 4 * hb);
                    dst[0] = Pair<TQ>::make(acc[db][4 * i4] * inv, acc[db][4 * i4 + 1] * inv);
                    dst[1] = Pair<TQ>::make(acc[db][4 * i4 + 2] * inv, acc[db][4 * i4 + 3] * inv);
                }
        }
    }
}

// The f16 copy of a bf16 V for the f16-V prefill: one workgroup per chunk of
// rows (256-byte rows of one token and KV head) of one sequence. A bf16 value
// converts exactly when |v| < 65536 (bf16 has 8 significant bits, f16 11 and
// its exponent range; below 2^-14 f16 rounds to a multiple of 2^-24, an error
// under 2^-25). The chunk's flag byte records whether some finite value was
// 65536 or more; infinities and NaNs convert to themselves. Every flag of the
// row up to flag_chunks is written on each call, so no clearing is needed.
struct ConvertArgs {
    const void *v;   // [B, N, Hkv, 128] bf16
    void *v16;       // the same layout, f16
    uint8_t *flags;  // [B, kPrefillFlagRow]
    long long rows;  // N * Hkv, rows per sequence
    int rows_per_chunk, chunks;
};

constexpr int kConvThreads = 256;
constexpr int kConvUnroll = 8;  // 16-byte loads in flight per lane

__global__ __launch_bounds__(kConvThreads) void prefill_convert_v_kernel(ConvertArgs c) {
    const int b = blockIdx.x / c.chunks;
    const int ch = blockIdx.x - b * c.chunks;
    const long long row0 = (long long)ch * c.rows_per_chunk;
    const long long nrows = min((long long)c.rows_per_chunk, c.rows - row0);
    const long long pieces = nrows * (kHeadDim * 2 / 16);  // 16-byte pieces of the chunk
    const size_t first = ((size_t)b * c.rows + row0) * (kHeadDim * 2);  // byte offset of the chunk
    const char *src = reinterpret_cast<const char *>(c.v) + first;
    char *dst = reinterpret_cast<char *>(c.v16) + first;
    bool bad = false;
    for (long long p0 = 0; p0 < pieces; p0 += kConvThreads * kConvUnroll) {
        uint4 x[kConvUnroll];
#pragma unroll
        for (int i = 0; i < kConvUnroll; ++i) {
            const long long p = p0 + i * kConvThreads + (int)threadIdx.x;
            if (p < pieces) x[i] = load_stream16(src + (size_t)p * 16);
        }
#pragma unroll
        for (int i = 0; i < kConvUnroll; ++i) {
            const long long p = p0 + i * kConvThreads + (int)threadIdx.x;
            if (p >= pieces) continue;
            const uint32_t w[4] = {x[i].x, x[i].y, x[i].z, x[i].w};
            uint32_t o[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float lo = __builtin_bit_cast(float, w[j] << 16);
                const float hi = __builtin_bit_cast(float, w[j] & 0xffff0000u);
                o[j] = __builtin_bit_cast(uint32_t, f16x2{(_Float16)lo, (_Float16)hi});
                const float alo = fabsf(lo), ahi = fabsf(hi);  // NaN compares false, inf is not <= max
                bad |= (alo >= 65536.f && alo <= __FLT_MAX__) || (ahi >= 65536.f && ahi <= __FLT_MAX__);
            }
            *reinterpret_cast<uint4 *>(dst + (size_t)p * 16) = make_uint4(o[0], o[1], o[2], o[3]);
        }
    }
    bad = __syncthreads_or(bad);
    if (threadIdx.x == 0) c.flags[(size_t)b * kPrefillFlagRow + ch] = bad ? 1 : 0;
}

}  // namespace

size_t prefill_workspace_bytes(int B, int N, int Hkv) {
    return (size_t)B * N * Hkv * kHeadDim * 2 + (size_t)B * kPrefillFlagRow;
}

hipError_t launch_prefill(fd_dtype dtype, const PrefillArgs &a, void *ws, hipStream_t st, hipEvent_t e0,
                          hipEvent_t e1) {
    PrefillArgs arg = a;
    arg.q_tiles = (a.N + kWaves * kWaveQ - 1) / (kWaves * kWaveQ);
    arg.flags = nullptr;
    arg.flag_chunks = 0;
    arg.flag_mode = kPrefillNoFlags;
    LaunchShape s{dim3(arg.q_tiles * a.H * a.B), dim3(kThreads)};
    void *args[] = {&arg};
    if (dtype == FD_DTYPE_F16)
        return launch_timed(reinterpret_cast<const void *>(&prefill_kernel<_Float16, _Float16>), s, args, st, e0, e1);
    if (dtype != FD_DTYPE_BF16) return hipErrorInvalidValue;
    if (!ws)
        return launch_timed(reinterpret_cast<const void *>(&prefill_kernel<__bf16, __bf16>), s, args, st, e0, e1);
    // At most kPrefillFlagRow chunks per sequence, of at least
    // kPrefillConvMinRows rows each.
    ConvertArgs c{};
    c.v = a.v;
    c.v16 = ws;
    c.rows = (long long)a.N * a.Hkv;
    const long long per = (c.rows + kPrefillFlagRow - 1) / kPrefillFlagRow;
    c.rows_per_chunk = (int)(per > kPrefillConvMinRows ? per : kPrefillConvMinRows);
    c.chunks = (int)((c.rows + c.rows_per_chunk - 1) / c.rows_per_chunk);
    c.flags = reinterpret_cast<uint8_t *>(ws) + (size_t)a.B * a.N * a.Hkv * kHeadDim * 2;
    void *cargs[] = {&c};
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(&prefill_convert_v_kernel),
                                   dim3((unsigned)a.B * c.chunks), dim3(kConvThreads), cargs, 0, st);
    if (e != hipSuccess) return e;
    arg.v = ws;
    arg.flags = c.flags;
    arg.flag_chunks = c.chunks;
    arg.flag_mode = kPrefillRunIfClean;
    e = launch_timed(reinterpret_cast<const void *>(&prefill_kernel<__bf16, _Float16>), s, args, st, e0, e1);
    if (e != hipSuccess) return e;
    arg.v = a.v;
    arg.flag_mode = kPrefillRunIfFlagged;
    return hipLaunchKernel(reinterpret_cast<const void *>(&prefill_kernel<__bf16, __bf16>), s.grid, s.block, args, 0,
                           st);
}

}  // namespace fd
