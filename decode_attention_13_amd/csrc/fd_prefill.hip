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
// tokens staged in LDS (two K and two V buffers) and shared by the 4 waves.
// Per wave, 16-query block and tile, the matrix-core work is that of the decode
// kernel with query rows in place of query heads:
//   S^T[key, q] = K[key, :] . Q[q, :]       two 16x16x32 MFMA chains of 4
//   online softmax per query (column), log2 domain, fp32
//   O^T[d, q] += V^T[d, key] . P^T[key, q]  eight 16x16x32 MFMAs (bf16: P split
//       into two 16-bit parts, two MFMAs each, which keeps P.V near fp32)
// The loop is a three-stage software pipeline: P.V of tile j and the scores of
// tile j + 2 go to the matrix cores while the VALU takes the softmax of j + 1.
// P^T needs no lane movement (key slot (l/16)*8 + j holds key
// (j/4)*16 + (l/16)*4 + j%4, the keys of that lane's S accumulators); V^T comes
// from the LDS tile with ds_read_b64_tr_b16.
#include "fd_device.h"
#include "fd_internal.h"

namespace fd {

namespace {

constexpr int kWaves = 4;      // waves per workgroup, 16 * QB queries each
constexpr int kThreads = 64 * kWaves;
constexpr int kKTile = 32;     // keys per LDS tile
constexpr int kPieces = kKTile * 16 / kThreads;  // 16-byte pieces (16 per 256-B row) of a tile per thread
constexpr int kKPad = 272;     // LDS bytes per K row (256 + 16)
constexpr int kVPad = 288;     // LDS bytes per V row (256 + 32, as for the transposed reads)
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

__device__ __forceinline__ float max2(float x, float y) { return __builtin_amdgcn_fmed3f(x, y, INFINITY); }

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
    __device__ static float lo_of(uint32_t w) { return bf16_lo(w); }
    __device__ static float hi_of(uint32_t w) { return bf16_hi(w); }
};

template <>
struct Mma<_Float16> {
    static constexpr bool kSplitP = false;  // f16 keeps 11 bits of P (P < 2^8: no overflow)
    __device__ static f32x4 mma(uint4 a, uint4 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                      0, 0, 0);
    }
    __device__ static uint32_t pack2(float x, float y) {
        return __builtin_bit_cast(uint32_t, f16x2{(_Float16)x, (_Float16)y});
    }
    __device__ static float lo_of(uint32_t w) { return (float)__builtin_bit_cast(f16x2, w).x; }
    __device__ static float hi_of(uint32_t w) { return (float)__builtin_bit_cast(f16x2, w).y; }
};

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

    __shared__ __attribute__((aligned(16))) char sK[2][kKTile * kKPad];
    __shared__ __attribute__((aligned(16))) char sV[2][kKTile * kVPad];

    // Q fragments (B operand of S): query q0 + 16*qb + c, head-dim slots kk*32 + g*8 .. +8.
    uint4 qf[QB][4];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int qr = min(q0 + 16 * qb + c, N - 1);
        const T *qrow = reinterpret_cast<const T *>(a.q) + (((size_t)b * N + qr) * a.H + h) * kHeadDim;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) qf[qb][kk] = load16(qrow + kk * 32 + g * 8);
    }
    // A negative scale is moved into Q (a sign flip is exact), so the running
    // max can be taken over the raw scores and scaled afterwards.
    // sl > 0 (a zero scale arrives as the least normal float), so -inf * sl
    // stays -inf and a masked score gives exp2 = 0.
    const float sl = fabsf(a.scale_log2);
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

    // Tile staging: thread t moves 16-byte pieces t + i * kThreads of a K or V tile
    // (piece p: row p / 16, bytes (p % 16) * 16); rows past N re-read row N - 1.
    const size_t tok_bytes = (size_t)a.Hkv * kHeadDim * sizeof(T);
    const char *kg = reinterpret_cast<const char *>(a.k) + ((size_t)b * N * a.Hkv + kvh) * kHeadDim * sizeof(T);
    const char *vg = reinterpret_cast<const char *>(a.v) + ((size_t)b * N * a.Hkv + kvh) * kHeadDim * sizeof(T);
    // A whole tile: a wave-uniform tile base plus a fixed 32-bit offset per lane.
    uint32_t lane_off[kPieces];
#pragma unroll
    for (int i = 0; i < kPieces; ++i) {
        const int p = threadIdx.x + i * kThreads;
        lane_off[i] = (uint32_t)(p >> 4) * (uint32_t)tok_bytes + (p & 15) * 16;
    }
    auto fetch = [&](const char *src, int j, uint4 (&st)[kPieces]) {
        if (j * kKTile + kKTile <= N) {
            // buffer loads from the uniform tile base (2% on the f16 GQA workload)
            const __amdgpu_buffer_rsrc_t r = stream_rsrc(src + (size_t)j * kKTile * tok_bytes);
#pragma unroll
            for (int i = 0; i < kPieces; ++i) {
                const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(r, lane_off[i], 0, 0);
                st[i] = make_uint4(x.x, x.y, x.z, x.w);
            }
        } else {
#pragma unroll
            for (int i = 0; i < kPieces; ++i) {
                const int p = threadIdx.x + i * kThreads;
                const int key = min(j * kKTile + (p >> 4), N - 1);
                st[i] = load16(src + (size_t)key * tok_bytes + (p & 15) * 16);
            }
        }
    };
    auto put = [&](char *dst, int pad, const uint4 (&st)[kPieces]) {
#pragma unroll
        for (int i = 0; i < kPieces; ++i) {
            const int p = threadIdx.x + i * kThreads;
            *(lds_u32x4 *)(uintptr_t)(dst + (p >> 4) * pad + (p & 15) * 16) = u32x4{st[i].x, st[i].y, st[i].z, st[i].w};
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
    // S^T of one tile from the K buffer.
    auto scores = [&](int kbuf) {
        lds_char *kt = (lds_char *)(uintptr_t)sK[kbuf];
        Scores r;
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) r.v[qb][sb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const u32x4 kr = *(lds_u32x4 *)(kt + (sb * 16 + c) * kKPad + kk * 64 + g * 16);
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
            // Raw-score max (the scale is > 0: its sign was moved into Q); med3
            // with +inf is a max that needs no NaN canonicalisation of its inputs.
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
            for (int e2 = 0; e2 < 4; ++e2) {
                hw[e2] = M::pack2(pe[2 * e2], pe[2 * e2 + 1]);
                if constexpr (M::kSplitP)
                    lw[e2] = M::pack2(pe[2 * e2] - M::lo_of(hw[e2]), pe[2 * e2 + 1] - M::hi_of(hw[e2]));
            }
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

    // O^T += V^T . P^T from a V buffer.
    auto pv = [&](int vbuf, const Probs &pr) {
        lds_char *vt = (lds_char *)(uintptr_t)sV[vbuf];
        const int e = c >> 2, bq = c & 3;
#pragma unroll
        for (int db = 0; db < 8; ++db) {
            const int col_bytes = (db * 16 + bq * 4) * 2;
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_i16x4 *)(vt + (g * 4 + e) * kVPad + col_bytes));
            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_i16x4 *)(vt + (16 + g * 4 + e) * kVPad + col_bytes));
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
    // of tile j + 1 (none of the three waits for another). K runs two tiles ahead
    // of V: iteration j fetches K(j + 3) and V(j + 1) from global memory and
    // stores them, after its own LDS reads, into the buffers that iteration
    // j - 1 finished reading; one barrier per tile.
    // Tiles this wave computes: with the causal mask those after its last query
    // are skipped (the workgroup still stages them for its other waves). Scores
    // formed past a wave's last tile read whatever the K buffer holds and are
    // never used.
    const int n_w = a.causal ? min(ntiles, q_last / kKTile + 1) : ntiles;
    auto masked = [&](int j) { return j * kKTile + kKTile > N || (a.causal && j * kKTile + kKTile - 1 > q0); };
    uint4 kst[kPieces], vst[kPieces], k2st[kPieces];
    fetch(kg, 0, kst);
    fetch(vg, 0, vst);
    if (ntiles > 2) fetch(kg, 2, k2st);
    put(sK[0], kKPad, kst);
    put(sV[0], kVPad, vst);
    if (ntiles > 1) {
        fetch(kg, 1, kst);
        put(sK[1], kKPad, kst);
    }
    __syncthreads();
    Scores sc0 = scores(0);
    Scores sc1 = scores(1);  // tile 1, or discarded
    __syncthreads();         // every wave has read K buffer 0
    if (ntiles > 2) put(sK[0], kKPad, k2st);
    if (masked(0)) mask_scores(0, sc0);
    Probs p_cur;
    softmax(sc0, p_cur);  // m starts at -inf: nothing to rescale
    bool rescale = false;  // alpha of the last softmax applies before the next P.V
    __syncthreads();
    for (int j = 0; j < ntiles; ++j) {
        const bool more_k = j + 3 < ntiles;
        const bool more_v = j + 1 < ntiles;
        if (more_k) fetch(kg, j + 3, kst);
        if (more_v) fetch(vg, j + 1, vst);
        if (rescale) {  // softmax(j) moved m: before P.V(j)
            rescale_acc();
            rescale = false;
        }
        if (j + 1 < n_w) {
            if (masked(j + 1)) mask_scores(j + 1, sc1);
            Probs p_next;
            // One block for the scheduler: P.V(j) and scores(j + 2) on the matrix
            // cores, softmax(j + 1) on the VALU.
            pv(j & 1, p_cur);
            const Scores sc2 = scores(j & 1);
            rescale = softmax(sc1, p_next);
            // Interleave the block for the scheduler: one MFMA, then three VALU
            // instructions, for each MFMA of the block (left alone, the compiler
            // bunched the softmax; this ordering ran the bf16 workload 3% and
            // the f16 one 1.5% faster).
            constexpr int kBlockMfma = QB * (8 + 8 * (M::kSplitP ? 2 : 1));
#pragma unroll
            for (int sg = 0; sg < kBlockMfma; ++sg) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
                __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // VALU
            }
            sc1 = sc2;
            p_cur = p_next;
        } else if (j < n_w) {
            pv(j & 1, p_cur);
        }
        if (more_k) put(sK[(j + 1) & 1], kKPad, kst);
        if (more_v) put(sV[(j + 1) & 1], kVPad, vst);
        __syncthreads();
    }

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
