// fd_split_mfma.hip -- split kernel on the matrix cores for grouped-query heads
// (gfx950, wave64, v_mfma_f32_16x16x32_{bf16,f16}).
//
// When G query heads share one KV head, one workgroup reads each K/V row once
// and serves all G heads ("FlashAttention 与推理算子", exercise 3: one block per
// (sequence, KV head) computing every query head of the group). From G = 3 the
// per-row work (G dot products and G axpys over 128 elements) runs here on the
// matrix cores, G padded to the 16 columns of the tile. Measured on the GQA4
// batch's lengths with 16, 24 and 32 query heads on 8 KV heads, split kernel
// time on the vector ALUs against the matrix cores: G = 2 192.1 / 195.4 us,
// G = 3 505 / 196.0 us (the vector kernel's head groups are powers of two, so
// it reads every row three times), G = 4 202.3 / 196.0 us.
//
// Per wave and tile of 32 tokens:
//   S^T[token, head] = K[token, :] . Q[head, :]    two 16x16x32 MFMA chains of 4
//       A = K rows straight from 16-byte global loads (lane: token = lane%16,
//       head-dim slot group lane/16), B = Q (loaded once).
//   online softmax per head (column) in the log2 domain, fp32;
//   O^T[d, head] += V^T[d, token] . P[token, head]  eight 16x16x32 MFMAs
//       B = P converted to the input type, taken from the S accumulators with
//       no lane movement: token slot (lane/16)*8 + j holds token
//       (j/4)*16 + (lane/16)*4 + j%4, exactly the tokens the S accumulator of
//       that lane holds. A = V^T, read from a padded LDS copy of the V tile with
//       ds_read_b64_tr_b16 (within 16 lanes: source lane 4e+b supplies 4
//       elements of row e; result lane c receives column c of rows 0..3).
// The contraction order inside an MFMA is free, so the head-dim slot order of
// K and Q only has to agree with itself; it is chosen so that the four lanes
// of a row load 64 contiguous bytes per instruction.
//
// The wave's next tile of K and V is loaded into registers while the current
// one is computed. The four waves' states are merged once at the end through
// LDS.
//
// FP8 E4M3 caches: K and V codes are converted to the query type in registers
// (v_cvt_scalef32_pk_{bf16,f16}_fp8 with unit scale; every E4M3 value is exact
// in bf16 and in f16) and the same 16-bit MFMAs run. The per-tensor scales are
// applied in fp32: k_scale inside the folded softmax scale, v_scale on the
// normalised output.
#include <type_traits>

#include "fd_device.h"
#include "fd_internal.h"

namespace fd {

namespace {

constexpr int kThreads = kSplitThreads;
constexpr int kWaves = 4;
constexpr int kTile = 32;                // tokens per wave tile
constexpr int kRowPad = 288;             // LDS bytes per V row: 256 + 32 keeps 8 rows on disjoint banks
constexpr int kVRegion = kTile * kRowPad;  // LDS bytes per wave
constexpr int kMaxHeads = 16;            // MFMA tile columns

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) char lds_char;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

template <typename T>
struct Mfma;

template <>
struct Mfma<__bf16> {
    __device__ static f32x4 mma(uint4 a, uint4 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                       c, 0, 0, 0);
    }
    __device__ static uint32_t pack2(float x, float y) {  // round to nearest even
        return __builtin_bit_cast(uint32_t, bf16x2{(__bf16)x, (__bf16)y});
    }
    __device__ static float lo_of(uint32_t w) { return bf16_lo(w); }
    __device__ static float hi_of(uint32_t w) { return bf16_hi(w); }
    template <bool HI>  // E4M3 codes in bytes 2*HI, 2*HI+1 of w -> two bf16
    __device__ static uint32_t from_e4m3(uint32_t w) {
        return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
    }
};

template <>
struct Mfma<_Float16> {
    __device__ static f32x4 mma(uint4 a, uint4 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                      0, 0, 0);
    }
    __device__ static uint32_t pack2(float x, float y) {
        return __builtin_bit_cast(uint32_t, f16x2{(_Float16)x, (_Float16)y});
    }
    __device__ static float lo_of(uint32_t w) { return (float)__builtin_bit_cast(f16x2, w).x; }
    __device__ static float hi_of(uint32_t w) { return (float)__builtin_bit_cast(f16x2, w).y; }
    template <bool HI>
    __device__ static uint32_t from_e4m3(uint32_t w) {
        return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI));
    }
};

// How one lane holds its share of K and V for query type T and cache type KV.
//   K: lane (g, c) holds, for token c of a 16-token block, the 32 head-dim
//      slots of its group; kk-th MFMA operand = 8 of them. Q uses the same
//      slot order (q_slot).
//   V: lane c of group g loads the elements [8c, 8c+8) of one row; v_lds
//      gives them as 8 values of T for the LDS copy.
template <typename T, typename KV>
struct KvFrag {  // 16-bit cache of the query type
    static constexpr int kKRegs = 4;  // uint4 per lane and 16-token block
    typedef uint4 VRaw;
    // slot d = kk*32 + g*8 + j: the 4 lanes of a row read 64 contiguous bytes per load
    __device__ static int q_slot(int g, int kk) { return kk * 32 + g * 8; }
    template <typename Off>
    __device__ static void load_k(const char *base, Off off, int g, uint4 (&kx)[kKRegs]) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) kx[kk] = load16(base + off + g * 16 + kk * 64);
    }
    __device__ static uint4 k_operand(const uint4 (&kx)[kKRegs], int kk) { return kx[kk]; }
    template <typename Off>
    __device__ static VRaw load_v(const char *base, Off off, int c) {
        return load_stream16(base + off + c * 16);
    }
    __device__ static u32x4 v_lds(VRaw v) { return u32x4{v.x, v.y, v.z, v.w}; }
};

template <typename T>
struct KvFrag<T, fp8e4m3> {
    static constexpr int kKRegs = 2;
    typedef u32x2 VRaw;
    // slot d = (kk/2)*64 + g*16 + (kk%2)*8 + j: one 16-byte load per half row,
    // again 64 contiguous bytes per row and load
    __device__ static int q_slot(int g, int kk) { return (kk >> 1) * 64 + g * 16 + (kk & 1) * 8; }
    template <typename Off>
    __device__ static void load_k(const char *base, Off off, int g, uint4 (&kx)[kKRegs]) {
#pragma unroll
        for (int h = 0; h < 2; ++h) kx[h] = load16(base + off + g * 16 + h * 64);
    }
    __device__ static uint4 k_operand(const uint4 (&kx)[kKRegs], int kk) {
        const uint32_t w0 = (kk & 1) ? kx[kk >> 1].z : kx[kk >> 1].x;
        const uint32_t w1 = (kk & 1) ? kx[kk >> 1].w : kx[kk >> 1].y;
        return make_uint4(Mfma<T>::template from_e4m3<false>(w0), Mfma<T>::template from_e4m3<true>(w0),
                          Mfma<T>::template from_e4m3<false>(w1), Mfma<T>::template from_e4m3<true>(w1));
    }
    template <typename Off>
    __device__ static VRaw load_v(const char *base, Off off, int c) {
        return __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(base + off + c * 8));
    }
    __device__ static u32x4 v_lds(VRaw v) {
        return u32x4{Mfma<T>::template from_e4m3<false>(v.x), Mfma<T>::template from_e4m3<true>(v.x),
                     Mfma<T>::template from_e4m3<false>(v.y), Mfma<T>::template from_e4m3<true>(v.y)};
    }
};

template <typename T, typename KV, int MODE, bool FUSED>
__device__ __forceinline__ void split_mfma_item(const SplitArgs &a, const int slice, const int b, const int split) {
    constexpr bool PAGED = MODE != kContig;
    using M = Mfma<T>;
    using F = KvFrag<T, KV>;
    constexpr int KR = F::kKRegs;
    using E = Elem<T>;
    const int tid = item_tid();
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int g = lane >> 4;   // 16-lane group
    const int c = lane & 15;   // row/column inside the 16x16 tile
    const int G = a.G;
    const int per_kv = G / a.heads_per_wg;
    const int kvh = slice / per_kv;
    const int h0 = kvh * G + (slice - kvh * per_kv) * a.heads_per_wg;
    const int nh = a.heads_per_wg;  // heads of this workgroup (<= 16)

    __shared__ int s_pages[PAGED ? kMaxSplitPages : 1];
    __shared__ __attribute__((aligned(16))) char s_buf[kWaves * kVRegion];
    __shared__ float s_m[kWaves][kMaxHeads];
    __shared__ float s_l[kWaves][kMaxHeads];

    const int t_begin = split * a.chunk;
    int page_first = 0;
    const int L = split_prologue<PAGED>(a, b, t_begin, s_pages, &page_first);
    const int n_b = splits_of<PAGED>(L, a.chunk);
    if constexpr (PAGED) {
        if (a.err != nullptr)
            check_paged_split(a, b, t_begin, split < n_b ? split_end(split, n_b, L, a.chunk) : t_begin,
                              split == max(n_b - 1, 0));
    }
    if (split >= n_b) {  // uniform over the workgroup
        if (split == 0) {  // empty sequence: o = 0
            T *o = reinterpret_cast<T *>(a.out) + ((size_t)b * a.H + h0) * kHeadDim;
            for (int i = tid; i < nh * kHeadDim; i += kThreads) o[i] = E::store_cast(0.f);
        }
        return;
    }
    const int t_end = split_end(split, n_b, L, a.chunk);

    const char *kbase = reinterpret_cast<const char *>(a.k);
    const char *vbase = reinterpret_cast<const char *>(a.v);
    KvAddr<MODE> A{s_pages, page_first, a.page_shift, a.Hkv * kHeadDim * (int)sizeof(KV),
                   (size_t)kvh * kHeadDim * sizeof(KV)};

    // B operand of S: 8 head-dim slots of q[h0 + c] per kk, zero for padded heads.
    uint4 qb[4];
    {
        const T *qrow = reinterpret_cast<const T *>(a.q) + ((size_t)b * a.H + h0 + min(c, nh - 1)) * kHeadDim;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            qb[kk] = load16(qrow + F::q_slot(g, kk));
            if (c >= nh) qb[kk] = make_uint4(0, 0, 0, 0);
        }
    }

    f32x4 acc[8];
#pragma unroll
    for (int db = 0; db < 8; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY;  // running max of head c (same in the 4 lane groups)
    float lsum = 0.f;     // this lane's share of the running sum of head c

    // LDS pointer of this wave's V region (the low 32 bits of a generic LDS
    // address are its LDS offset).
    lds_char *vreg = (lds_char *)(uintptr_t)(s_buf + wave * kVRegion);
    const int ntiles = (t_end - t_begin + kTile - 1) / kTile;

    // A tile is two 16-token blocks. When the second block holds no valid token
    // its rows are clamped into the first, so both are addressed from block 0.
    auto block_start = [&](int t0, int h) { return (h == 0 || t0 + 16 < t_end) ? t0 + 16 * h : t0; };
    auto load_k = [&](int j, uint4 (&kx)[2][KR]) {
        const int t0 = t_begin + j * kTile;
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
            const int tok = min(t0 + sb * 16 + c, t_end - 1);
            if constexpr (MODE == kPagedRow) {
                F::load_k(kbase, A.row(tok), g, kx[sb]);
            } else {
                const int B = block_start(t0, sb);
                F::load_k(kbase + A.block(B), (uint32_t)(tok - B) * (uint32_t)A.token_bytes, g, kx[sb]);
            }
        }
    };
    auto load_v = [&](int j, typename F::VRaw (&vx)[8]) {
        const int t0 = t_begin + j * kTile;
        size_t base[2] = {0, 0};
        if constexpr (MODE != kPagedRow) {
            base[0] = A.block(block_start(t0, 0));
            base[1] = A.block(block_start(t0, 1));
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int tok = min(t0 + 4 * i + g, t_end - 1);
            if constexpr (MODE == kPagedRow) {
                vx[i] = F::load_v(vbase, A.row(tok), c);
            } else {
                const int h = i >> 2;
                vx[i] = F::load_v(vbase + base[h], (uint32_t)(tok - block_start(t0, h)) * (uint32_t)A.token_bytes, c);
            }
        }
    };

    // K: one register set, refilled with the wave's next tile as soon as the S
    // MFMAs have consumed it. V: two register sets used as a ring, so the V rows
    // of the next two tiles are in flight while this tile is computed.
    uint4 kx[2][KR];
    typename F::VRaw vA[8], vB[8];
    // REFILL_V / REFILL_K (std::bool_constant) say at compile time whether this
    // tile refills the V set with tile j + 2*kWaves and K with tile j + kWaves,
    // so the loads are not under a branch and the compiler's waits count only
    // the loads a value really depends on.
    auto tile = [&](int j, typename F::VRaw (&vcur)[8], auto refill_v, auto refill_k) {
        const int t0 = t_begin + j * kTile;
        // V tile -> LDS (row r = token t0 + r, padded rows), then refill the set
        // with the tile after next.
#pragma unroll
        for (int i = 0; i < 8; ++i)
            *(lds_u32x4 *)(vreg + (4 * i + g) * kRowPad + c * 16) = F::v_lds(vcur[i]);
        if constexpr (decltype(refill_v)::value) load_v(j + 2 * kWaves, vcur);
        // S^T tiles: s[sb][i] = score of token t0 + sb*16 + g*4 + i for head c
        f32x4 s[2];
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
            s[sb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) s[sb] = M::mma(F::k_operand(kx[sb], kk), qb[kk], s[sb]);
        }
        if constexpr (decltype(refill_k)::value) load_k(j + kWaves, kx);
        float x[8];
        float mt = -INFINITY;
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool valid = t0 + sb * 16 + g * 4 + i < t_end;
                x[sb * 4 + i] = valid ? s[sb][i] * a.scale_log2 : -INFINITY;
                mt = fmaxf(mt, x[sb * 4 + i]);
            }
        mt = pair_max<32>(pair_max<16>(mt));
        const float m_new = fmaxf(m, mt);
        const float mu = finite_or_zero(m_new);
        const float alpha = exp2_fast(m - mu);
        m = m_new;
        float p[8];
        float ps = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            p[e] = exp2_fast(x[e] - mu);
            ps += p[e];
        }
        lsum = lsum * alpha + ps;
        // P in two 16-bit parts, p = hi + lo (+ 2^-16 p): two MFMAs per block
        // keep P.V close to fp32 precision.
        uint4 ph, pl;
        {
            uint32_t hw[4], lw[4];
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) {
                hw[e2] = M::pack2(p[2 * e2], p[2 * e2 + 1]);
                const float h0v = M::lo_of(hw[e2]), h1v = M::hi_of(hw[e2]);
                lw[e2] = M::pack2(p[2 * e2] - h0v, p[2 * e2 + 1] - h1v);
            }
            ph = make_uint4(hw[0], hw[1], hw[2], hw[3]);
            pl = make_uint4(lw[0], lw[1], lw[2], lw[3]);
        }
        // Rescale only when some head's running max moved (alpha == 1 is exact).
        if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
            for (int db = 0; db < 8; ++db) acc[db] *= alpha;
        }
        // O^T[d, head] += V^T[d, token slot] . P[token slot, head]
        const int e = c >> 2, bq = c & 3;
#pragma unroll
        for (int db = 0; db < 8; ++db) {
            const int col_bytes = (db * 16 + bq * 4) * 2;
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                reinterpret_cast<lds_i16x4 *>(vreg + (g * 4 + e) * kRowPad + col_bytes));
            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                reinterpret_cast<lds_i16x4 *>(vreg + (16 + g * 4 + e) * kRowPad + col_bytes));
            const u32x2 lo2 = __builtin_bit_cast(u32x2, lo);
            const u32x2 hi2 = __builtin_bit_cast(u32x2, hi);
            const uint4 va = make_uint4(lo2.x, lo2.y, hi2.x, hi2.y);
            acc[db] = M::mma(va, ph, acc[db]);
            acc[db] = M::mma(va, pl, acc[db]);
        }
    };
    using Yes = std::true_type;
    using No = std::false_type;
    int j = wave;
    if (j + 3 * kWaves < ntiles) {
        // Steady state, two tiles per trip: both refill, so every trip issues the
        // same loads and the loop carries an exact count of loads in flight.
        load_k(j, kx);
        load_v(j, vA);
        load_v(j + kWaves, vB);
        do {
            tile(j, vA, Yes{}, Yes{});
            tile(j + kWaves, vB, Yes{}, Yes{});
            j += 2 * kWaves;
        } while (j + 3 * kWaves < ntiles);
    } else if (j < ntiles) {
        load_k(j, kx);
        load_v(j, vA);
        if (j + kWaves < ntiles) load_v(j + kWaves, vB);
    }
    // At most three tiles of this wave remain (V sets vA, vB, vA).
    auto last_tiles = [&](int jj, typename F::VRaw (&vset)[8]) {
        if (jj + 2 * kWaves < ntiles) {
            tile(jj, vset, Yes{}, Yes{});
        } else if (jj + kWaves < ntiles) {
            tile(jj, vset, No{}, Yes{});
        } else {
            tile(jj, vset, No{}, No{});
        }
    };
    if (j < ntiles) last_tiles(j, vA);
    if (j + kWaves < ntiles) last_tiles(j + kWaves, vB);
    if (j + 2 * kWaves < ntiles) last_tiles(j + 2 * kWaves, vA);

    // Head c's running sum over the wave: the four lane groups hold disjoint tokens.
    lsum = pair_sum<32>(pair_sum<16>(lsum));

    __syncthreads();  // every wave is done with its V region; reuse it for the merge
    float *s_acc = reinterpret_cast<float *>(s_buf);  // [wave][head][d]
    if (c < nh) {
#pragma unroll
        for (int db = 0; db < 8; ++db)
            *reinterpret_cast<f32x4 *>(&s_acc[(wave * kMaxHeads + c) * kHeadDim + db * 16 + g * 4]) = acc[db];
        if (g == 0) {
            s_m[wave][c] = m;
            s_l[wave][c] = lsum;
        }
    }
    __syncthreads();
    finish_split<T, FUSED>(a, slice, b, h0, nh, split, n_b, [&](int hh, int d, float &lse) {
        float Mx = s_m[0][hh];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) Mx = fmaxf(Mx, s_m[w][hh]);
        const float mu = finite_or_zero(Mx);
        float l = 0.f, o = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float wgt = exp2_fast(s_m[w][hh] - mu);
            l = __builtin_fmaf(wgt, s_l[w][hh], l);
            o = __builtin_fmaf(wgt, s_acc[(w * kMaxHeads + hh) * kHeadDim + d], o);
        }
        lse = (Mx + log2_fast(l)) * kLn2;
        return a.v_scale * (o / l);
    });
}

// Contiguous: one workgroup per (head slice, split). Paged batches take their
// (sequence, split) items largest first, the last split of every sequence
// before the others, one per workgroup or, in a persistent launch, claimed by
// one workgroup per resident slot (paged_items).
template <typename T, typename KV, int MODE, bool PERSIST, bool FUSED>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void split_mfma_kernel(SplitArgs a) {
    pin_args(a.q, a.k, a.v, a.ws_o, a.ws_lse, a.scale_log2);
    if constexpr (MODE == kContig) {
        split_mfma_item<T, KV, MODE, FUSED>(a, blockIdx.x, 0, blockIdx.y);
    } else {
        paged_items<T, PERSIST>(a, [&](const SplitArgs &ai, int x, int b, int split) {
            split_mfma_item<T, KV, MODE, false>(ai, x, b, split);
        });
    }
}

template <typename T, typename KV, int MODE, bool PERSIST, bool FUSED = false>
hipError_t launch_one(const LaunchShape &s, const SplitArgs &a, hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
    SplitArgs arg = a;
    void *args[] = {&arg};
    return launch_timed(reinterpret_cast<const void *>(&split_mfma_kernel<T, KV, MODE, PERSIST, FUSED>), s, args, st,
                        e0, e1);
}

template <typename T, typename KV>
hipError_t launch_mode(int mode, bool persist, bool fused, const LaunchShape &s, const SplitArgs &a, hipStream_t st,
                       hipEvent_t e0, hipEvent_t e1) {
    if (fused && mode != kContig) return hipErrorInvalidValue;
    switch (mode) {
        case kContig:
            return fused ? launch_one<T, KV, kContig, false, true>(s, a, st, e0, e1)
                         : launch_one<T, KV, kContig, false, false>(s, a, st, e0, e1);
        case kPagedBlock:
            return persist ? launch_one<T, KV, kPagedBlock, true>(s, a, st, e0, e1)
                           : launch_one<T, KV, kPagedBlock, false>(s, a, st, e0, e1);
        case kPagedRow:
            return persist ? launch_one<T, KV, kPagedRow, true>(s, a, st, e0, e1)
                           : launch_one<T, KV, kPagedRow, false>(s, a, st, e0, e1);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_split_mfma(fd_dtype dtype, int gt, int mode, bool persist, bool fused, const LaunchShape &s,
                             const SplitArgs &a, hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
    if (gt < 1 || gt > kMaxHeads) return hipErrorInvalidValue;
    switch (dtype) {
        case FD_DTYPE_F16: return launch_mode<_Float16, _Float16>(mode, persist, fused, s, a, st, e0, e1);
        case FD_DTYPE_BF16: return launch_mode<__bf16, __bf16>(mode, persist, fused, s, a, st, e0, e1);
        case FD_DTYPE_F16_KV_E4M3: return launch_mode<_Float16, fp8e4m3>(mode, persist, fused, s, a, st, e0, e1);
        case FD_DTYPE_BF16_KV_E4M3: return launch_mode<__bf16, fp8e4m3>(mode, persist, fused, s, a, st, e0, e1);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace fd
