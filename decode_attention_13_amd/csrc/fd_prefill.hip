// fd_prefill.hip -- prefill attention (many queries, optional causal mask) on
// the matrix cores (gfx950, wave64, v_mfma_f32_16x16x32_{bf16,f16}).
//
// The blocked algorithm of "FlashAttention 与推理算子", section
// "FlashAttention：分块 + online softmax": a block of queries walks the key
// blocks, keeps a running max and sum per query row and rescales its output
// accumulator; with the causal mask (same section) key blocks past the query
// block's last row are never visited and the diagonal block is masked element
// by element. The FlashAttention-2 layout the page describes (each Q block its
// own workgroup, waves split by query rows) is kept.
//
// Workgroup: 4 waves x 16 * QB queries of one (sequence, head); key tiles of 32
// tokens shared by the 4 waves. Per wave, 16-query block and tile, the
// matrix-core work is that of the decode kernel with query rows in place of
// query heads:
//   S^T[key, q] = K[key, :] . Q[q, :]       two 16x16x32 MFMA chains of 4
//   online softmax per query (column), log2 domain, fp32
//   O^T[d, q] += V^T[d, key] . P^T[key, q]  eight 16x16x32 MFMAs (bf16: P split
//       into two 16-bit parts, two MFMAs each, which keeps P.V near fp32)
// The loop is a three-stage software pipeline: P.V of tile j and the scores of
// tile j + 2 go to the matrix cores while the VALU takes the softmax of j + 1.
// P^T needs no lane movement (key slot (l/16)*8 + j holds key
// (j/4)*16 + (l/16)*4 + j%4, the keys of that lane's S accumulators); V^T comes
// from the LDS tile with ds_read_b64_tr_b16.
//
// K and V tiles go from global memory straight into LDS (global_load_lds,
// 16 bytes a lane, no registers on the way) through rings of four tiles each,
// so a tile is requested three iterations before it is read: the loads meet
// the latency of L2 and HBM without holding the loop. A tile is 32 unpadded
// 256-byte rows; 16-byte chunk x of row r is stored at chunk x ^ (r % 16), so
// the K fragment reads (16 rows, one chunk) and the transposed V reads (4 rows,
// 2 chunks, per 16 lanes) both spread over all banks.
#include "fd_device.h"
#include "fd_internal.h"

namespace fd {

namespace {

constexpr int kWaves = 4;      // waves per workgroup, 16 * QB queries each
constexpr int kThreads = 64 * kWaves;
constexpr int kKTile = 32;     // keys per LDS tile
constexpr int kRow = 256;      // bytes of a K or V row in LDS (128 16-bit elements)
constexpr int kTileBytes = kKTile * kRow;
constexpr int kRing = 4;       // LDS tiles per ring (K and V each)
constexpr int kDmaPerTile = kTileBytes / (kThreads * 16);  // 16-byte loads per lane and tile
constexpr int kXcds = 8;       // XCDs of the MI355X, each with its own L2
constexpr float kLazyLog2 = 8.f;  // the running max trails the true one by at most this (log2 units)

typedef float f32x4 __attribute__((ext_vector_type(4)));
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

template <typename T>
struct Mma;

template <>
struct Mma<__bf16> {
    static constexpr bool kSplitP = true;  // bf16 keeps 8 bits of P: use hi + lo
    __device__ static f32x4 mma(uint4 a, uint4 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
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
    __device__ static f32x4 mma(uint4 a, uint4 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                      0, 0, 0);
    }
    __device__ static void split2(float x, float y, uint32_t &hi, uint32_t &lo) {
        hi = __builtin_bit_cast(uint32_t, f16x2{(_Float16)x, (_Float16)y});
        lo = 0;
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

// QB: blocks of 16 queries per wave. Every K and V fragment read from LDS
// feeds QB MFMA column blocks, so LDS traffic per flop falls as 1 / QB.
template <typename T, int QB>
__global__ __launch_bounds__(kThreads) void prefill_kernel(PrefillArgs a) {
    using M = Mma<T>;
    constexpr int kQTile = kWaves * 16 * QB;  // queries per workgroup
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: wave-level branches stay scalar
    const int g = lane >> 4;
    const int c = lane & 15;
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
    const int q0 = qt * kQTile + wave * 16 * QB;  // this wave's first query
    const int q_last = q0 + 16 * QB - 1;
    const int kv_end = a.causal ? min(N, (qt + 1) * kQTile) : N;
    const int ntiles = (kv_end + kKTile - 1) / kKTile;

    __shared__ __attribute__((aligned(16))) char sK[kRing][kTileBytes];
    __shared__ __attribute__((aligned(16))) char sV[kRing][kTileBytes];

    uint4 qf[QB][4];  // the wave's queries, loaded with the first tiles below
    // sl > 0 (a zero scale arrives as the least normal float), so -inf * sl
    // stays -inf and a masked score gives exp2 = 0.
    const float sl = fabsf(a.scale_log2);

    // Tile loads: load i of a wave fills 1 KB of the tile, rows 4 * (kDmaPerTile *
    // wave + i) .. + 3, lane l the 16 bytes at l * 16 (row + l / 16, stored
    // chunk l % 16), which hold chunk (l % 16) ^ (row % 16) of that key's row.
    // Keys past N re-read key N - 1 (never used: masked, or past the workgroup).
    const size_t tok_bytes = (size_t)a.Hkv * kHeadDim * sizeof(T);
    const char *kg = reinterpret_cast<const char *>(a.k) + ((size_t)b * N * a.Hkv + kvh) * kHeadDim * sizeof(T);
    const char *vg = reinterpret_cast<const char *>(a.v) + ((size_t)b * N * a.Hkv + kvh) * kHeadDim * sizeof(T);
    // Lane offsets within a tile (row * token bytes + chunk; 32 rows of at most
    // 65535 * 256 bytes fit in 32 bits): a tile wholly below N is one scalar base
    // plus these, with no per-lane address arithmetic; a tile reaching past N
    // clamps its keys lane by lane.
    int dma_row[kDmaPerTile];
    uint32_t dma_col[kDmaPerTile], dma_off[kDmaPerTile];
#pragma unroll
    for (int i = 0; i < kDmaPerTile; ++i) {
        dma_row[i] = 4 * (kDmaPerTile * wave + i) + (lane >> 4);
        dma_col[i] = (uint32_t)(((lane & 15) ^ (dma_row[i] & 15)) * 16);
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

    f32x4 acc[QB][8];
    float m[QB], lsum[QB];  // running max (same in the 4 lane groups) and this lane's share of the sum
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        m[qb] = -INFINITY;
        lsum[qb] = 0.f;
#pragma unroll
        for (int db = 0; db < 8; ++db) acc[qb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    struct Scores {
        f32x4 v[QB][2];
    };
    // S^T of tile t from the K ring: lane (g, c) reads key row sb * 16 + c,
    // chunk kk * 4 + g, stored at chunk (kk * 4 + g) ^ c.
    auto scores = [&](int t) {
        lds_char *kt = (lds_char *)(uintptr_t)sK[t & (kRing - 1)];
        Scores r;
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) r.v[qb][sb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const u32x4 kr = *(lds_u32x4 *)(kt + (sb * 16 + c) * kRow + (((kk * 4 + g) ^ c) << 4));
                const uint4 ka = make_uint4(kr.x, kr.y, kr.z, kr.w);
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) r.v[qb][sb] = M::mma(ka, qf[qb][kk], r.v[qb][sb]);
            }
        }
        return r;
    };

    // Masked scores become -inf, so their P is exactly 0: keys at or past N,
    // and with the causal mask keys after the query.
    auto mask_scores = [&](int j, Scores &sc) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const int q_me = q0 + 16 * qb + c;
            const int room = (a.causal ? min(q_me, N - 1) : N - 1) - j * kKTile - g * 4;  // key offset limit
#pragma unroll
            for (int sb = 0; sb < 2; ++sb)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (sb * 16 + i > room) sc.v[qb][sb][i] = -INFINITY;
        }
    };

    // Online softmax of one tile with a lazy running max: m moves only when the
    // tile's max exceeds it by more than kLazyLog2 (P then stays below
    // 2^kLazyLog2), so the accumulators are rescaled a few times per row instead
    // of on most tiles. Any subtracted constant gives the same softmax; the final
    // division uses the sum taken with the same constants. Produces P^T in the
    // MFMA operand layout (bf16: hi and lo parts) and alpha, the factor for the
    // accumulators; returns whether any row needs it.
    struct Probs {
        uint4 hi[QB], lo[QB];
    };
    float alpha[QB];
    auto softmax = [&](const Scores &sc, Probs &pr) {
        bool rescale = false;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const f32x4 s0 = sc.v[qb][0], s1 = sc.v[qb][1];
            // Raw-score max (the scale is > 0: its sign was moved into Q).
            float mt = max2(max2(max2(s0[0], s0[1]), max2(s0[2], s0[3])), max2(max2(s1[0], s1[1]), max2(s1[2], s1[3])));
            LanePair lp = lane_pair<16>(mt);
            mt = max2(lp.lo, lp.hi);
            lp = lane_pair<32>(mt);
            mt = max2(lp.lo, lp.hi);
            const float mt_s = mt * sl;  // -inf stays -inf
            const float m_old = m[qb];
            const float m_new = mt_s > m_old + kLazyLog2 ? mt_s : m_old;
            const float mu = finite_or_zero(m_new);
            alpha[qb] = exp2_fast(m_old - mu);  // 0 while m_old is -inf
            rescale |= m_new != m_old && m_old > -INFINITY;
            m[qb] = m_new;
            float pe[8];
            float ps = 0.f;
#pragma unroll
            for (int sb = 0; sb < 2; ++sb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    pe[sb * 4 + i] = exp2_fast(__builtin_fmaf(sc.v[qb][sb][i], sl, -mu));
                    ps += pe[sb * 4 + i];
                }
            lsum[qb] = __builtin_fmaf(lsum[qb], alpha[qb], ps);
            uint32_t hw[4], lw[4];
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) M::split2(pe[2 * e2], pe[2 * e2 + 1], hw[e2], lw[e2]);
            pr.hi[qb] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
            if constexpr (M::kSplitP) pr.lo[qb] = make_uint4(lw[0], lw[1], lw[2], lw[3]);
        }
        return __builtin_amdgcn_ballot_w64(rescale) != 0;
    };
    auto rescale_acc = [&]() {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int db = 0; db < 8; ++db) acc[qb][db] *= alpha[qb];
    };

    // O^T += V^T . P^T for tile t from the V ring: lane (g, c) reads 8 bytes of
    // key rows g*4 + c/4 and 16 + g*4 + c/4 (columns db*16 + (c%4)*4 .. + 3:
    // chunk db*2 + (c%4)/2, stored at that chunk ^ (g*4 + c/4)), transposed.
    auto pv = [&](int t, const Probs &pr) {
        lds_char *vt = (lds_char *)(uintptr_t)sV[t & (kRing - 1)];
        const int e = c >> 2, bq = c & 3;
        const int rl = g * 4 + e;
#pragma unroll
        for (int db = 0; db < 8; ++db) {
            const int off = (((db * 2 + (bq >> 1)) ^ rl) << 4) + (bq & 1) * 8;
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(vt + rl * kRow + off));
            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(vt + (16 + rl) * kRow + off));
            const u32x2v lo2 = __builtin_bit_cast(u32x2v, lo);
            const u32x2v hi2 = __builtin_bit_cast(u32x2v, hi);
            const uint4 va = make_uint4(lo2.x, lo2.y, hi2.x, hi2.y);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                acc[qb][db] = M::mma(va, pr.hi[qb], acc[qb][db]);
                if constexpr (M::kSplitP) acc[qb][db] = M::mma(va, pr.lo[qb], acc[qb][db]);
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
    dma(kg, sK, 0);
    dma(kg, sK, 1);
    dma(vg, sV, 0);
    dma(kg, sK, 2);
    // Q fragments (B operand of S): query q0 + 16*qb + c, head-dim slots kk*32 + g*8 .. +8.
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int qr = min(q0 + 16 * qb + c, N - 1);
        const T *qrow = reinterpret_cast<const T *>(a.q) + (((size_t)b * N + qr) * a.H + h) * kHeadDim;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) qf[qb][kk] = load16(qrow + kk * 32 + g * 8);
    }
    // A negative scale is moved into Q (a sign flip is exact), so the running
    // max can be taken over the raw scores and scaled afterwards.
    if (a.scale_log2 < 0.f) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                qf[qb][kk].x ^= 0x80008000u;
                qf[qb][kk].y ^= 0x80008000u;
                qf[qb][kk].z ^= 0x80008000u;
                qf[qb][kk].w ^= 0x80008000u;
            }
    }

    wait_vm<0>();
    dma(vg, sV, 1);
    dma(kg, sK, 3);
    dma(vg, sV, 2);
    __builtin_amdgcn_s_barrier();
    Scores sc0 = scores(0);
    Scores sc1 = scores(1);  // tile 1, or discarded
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
            const Scores sc2 = scores(j + 2);
            rescale = softmax(sc1, p_next);
            // Interleave the block for the scheduler: one MFMA, then three VALU
            // instructions, for each MFMA of the block (left alone, the compiler
            // bunched the softmax); bf16, whose P.V issues two MFMAs per V
            // fragment, also takes one LDS read per group (1.5% on the bf16
            // workload, 3% slower for f16).
            constexpr int kBlockMfma = QB * (8 + 8 * (M::kSplitP ? 2 : 1));
#pragma unroll
            for (int sg = 0; sg < kBlockMfma; ++sg) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
                if constexpr (M::kSplitP) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
                __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // VALU
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

#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const float ls = pair_sum<32>(pair_sum<16>(lsum[qb]));
        const int q_me = q0 + 16 * qb + c;
        if (q_me < N) {
            const float inv = 1.f / ls;
            T *orow = reinterpret_cast<T *>(a.o) + (((size_t)b * N + q_me) * a.H + h) * kHeadDim;
#pragma unroll
            for (int db = 0; db < 8; ++db) {
                typedef typename Pair<T>::type P2;
                P2 *dst = reinterpret_cast<P2 *>(orow + db * 16 + g * 4);
                dst[0] = Pair<T>::make(acc[qb][db][0] * inv, acc[qb][db][1] * inv);
                dst[1] = Pair<T>::make(acc[qb][db][2] * inv, acc[qb][db][3] * inv);
            }
        }
    }
}

}  // namespace

constexpr int kQueryBlocks = 2;  // 16-query blocks per wave: each K / V fragment read from LDS feeds two

hipError_t launch_prefill(fd_dtype dtype, const PrefillArgs &a, hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
    PrefillArgs arg = a;
    arg.q_tiles = (a.N + 16 * kWaves * kQueryBlocks - 1) / (16 * kWaves * kQueryBlocks);
    LaunchShape s{dim3(arg.q_tiles * a.H * a.B), dim3(kThreads)};
    void *args[] = {&arg};
    switch (dtype) {
        case FD_DTYPE_F16:
            return launch_timed(reinterpret_cast<const void *>(&prefill_kernel<_Float16, kQueryBlocks>), s, args, st,
                                e0, e1);
        case FD_DTYPE_BF16:
            return launch_timed(reinterpret_cast<const void *>(&prefill_kernel<__bf16, kQueryBlocks>), s, args, st,
                                e0, e1);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace fd
