// fd_split_valu.hip -- split kernel on the vector ALUs (gfx950, wave64).
//
// One workgroup of 4 waves computes one (sequence b, KV split, group of GT
// query heads sharing KV head kvh). It streams the split's K/V rows straight
// into registers with 16-byte loads: a 16-lane DPP row owns one 256-byte bf16
// row (512-byte fp32 row as two loads), so a wave covers four rows per load
// instruction and every load fills whole 128-byte lines. Each wave walks the
// split in tiles of 16 tokens (4 rows per 16-lane group), interleaved with the
// other waves, and prefetches its next tile's K and V into a second register
// set before computing the current one (a register double buffer; no LDS is
// needed because every lane consumes exactly the bytes it loaded).
//
// The cache element type KV may differ from the query/output type T: an FP8
// E4M3 cache (8-byte loads, codes converted to fp32 in registers) is read with
// f16/bf16 queries; its per-tensor scales are folded into the score scale
// (k_scale) and the stored output (v_scale).
//
// Per row: q.k on v_dot2 (16-bit) or FMA (fp32, FP8) over the lane's 8 elements,
// a 4-step DPP butterfly across the row, then the online-softmax update in
// the log2 domain ("FlashAttention 与推理算子", section "FlashAttention：分块 +
// online softmax"; the exp2 form with scale*log2(e) folded into the scores as
// in "[CUDA 优化实战] 纯手搓 flash decoding sm120", section "2. kernel 实现细节")
// and the P.V accumulation in fp32. The 16 per-group states of a workgroup
// are merged once at the end (lane swaps across rows inside a wave, LDS
// across waves) and written as a normalised partial plus its natural-log lse, or,
// when one split covers the sequence, as the final output.
#include <type_traits>

#include "fd_device.h"
#include "fd_internal.h"

namespace fd {

namespace {

constexpr int kThreads = kSplitThreads;  // 4 waves
constexpr int kRows = 4;               // load instructions per K (and V) per wave tile
constexpr int kWaves = kThreads / 64;

// GT: query heads per KV head computed by the workgroup (they share its rows).
// HP: adjacent KV heads per workgroup (MHA only, GT = 1). A wave's load
// instruction covers 4 / HP consecutive tokens and, for each, the HP heads'
// rows, which are contiguous in the cache: 4 rows of 256 B scattered by the
// token stride stream markedly slower than the same bytes in 512-B runs
// (measured with a plain read kernel on the 32-head layout: 12.7 against 10.8 us
// for 64 MB).
template <typename T, typename KV, int GT, int HP, int MODE, bool FUSED>
__device__ __forceinline__ void split_valu_item(const SplitArgs &a, const int slice, const int b, const int split) {
    static_assert(HP == 1 || GT == 1, "packed KV heads are for MHA");
    constexpr bool PAGED = MODE != kContig;
    using E = Elem<T>;
    using R = KvRow<KV>;
    using Raw = typename R::Raw;
    constexpr int NL = R::kPieces;
    // Packed 16-bit q.k on v_dot2 when the cache holds the query's own type.
    constexpr bool kPackedDot = std::is_same<T, KV>::value && !std::is_same<T, float>::value;
    constexpr int kTok = 4 / HP;              // tokens per load instruction
    constexpr int kWaveTile = kRows * kTok;   // tokens per wave tile
    constexpr int NH = HP * GT;               // query heads of the workgroup
    const int tid = item_tid();
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int grp = lane >> 4;
    const int c = lane & 15;
    const int hs = grp % HP;  // this group's KV head within the workgroup
    const int ts = grp / HP;  // this group's token within a load instruction
    int kvh, h0;
    if constexpr (HP > 1) {  // G = 1: query head = KV head
        kvh = slice * HP;
        h0 = kvh;
    } else {
        const int per_kv = a.G / GT;
        kvh = slice / per_kv;
        h0 = kvh * a.G + (slice - kvh * per_kv) * GT;
    }

    __shared__ int s_pages[PAGED ? kMaxSplitPages : 1];
    __shared__ float s_m[kWaves][NH];
    __shared__ float s_l[kWaves][NH];
    __shared__ float s_acc[kWaves][NH][kHeadDim];

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
            for (int i = tid; i < NH * kHeadDim; i += kThreads) o[i] = E::store_cast(0.f);
        }
        return;
    }
    const int t_end = split_end(split, n_b, L, a.chunk);

    const char *kbase = reinterpret_cast<const char *>(a.k);
    const char *vbase = reinterpret_cast<const char *>(a.v);
    KvAddr<MODE> A{s_pages, page_first, a.page_shift, a.Hkv * kHeadDim * (int)sizeof(KV),
                   (size_t)kvh * kHeadDim * sizeof(KV)};
    const int row_off = hs * kHeadDim * (int)sizeof(KV);  // this group's KV head within a token

    // q fragments of the group's GT heads, on the lane's elements R::index(c, e):
    // packed pairs for the v_dot2 path, fp32 otherwise.
    float qf[GT][8];
    uint32_t qp[GT][4];
    const T *qbase = reinterpret_cast<const T *>(a.q) + ((size_t)b * a.H + h0 + hs * GT) * kHeadDim;
#pragma unroll
    for (int gi = 0; gi < GT; ++gi) {
        uint4 x[E::kLoads];
#pragma unroll
        for (int pc = 0; pc < E::kLoads; ++pc) x[pc] = load16(qbase + gi * kHeadDim + E::offset(c, pc));
        if constexpr (kPackedDot) {
            qp[gi][0] = x[0].x;
            qp[gi][1] = x[0].y;
            qp[gi][2] = x[0].z;
            qp[gi][3] = x[0].w;
        } else {
            E::unpack(x, qf[gi]);
        }
    }

    float m[GT], l[GT], acc[GT][8];
#pragma unroll
    for (int gi = 0; gi < GT; ++gi) {
        m[gi] = -INFINITY;
        l[gi] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[gi][e] = 0.f;
    }

    const int ntiles = (t_end - t_begin + kWaveTile - 1) / kWaveTile;

    // Tile j covers [tb, tb + kWaveTile), tb = t_begin + kWaveTile j, inside one
    // 16-token block; load r reads tokens tb + r*kTok .. + kTok - 1 (group ts takes
    // tb + r*kTok + ts). Rows past t_end re-read the last valid row and are masked.
    auto load_tile = [&](int j, Raw (&kx)[kRows][NL], Raw (&vx)[kRows][NL]) {
        const int tb = t_begin + j * kWaveTile;
        const int t0 = tb + ts;
        if constexpr (MODE == kPagedRow) {
#pragma unroll
            for (int r = 0; r < kRows; ++r) {
                const size_t off = A.row(min(t0 + r * kTok, t_end - 1)) + row_off;
#pragma unroll
                for (int pc = 0; pc < NL; ++pc) {
                    kx[r][pc] = R::load(kbase + off + R::offset(c, pc) * sizeof(KV));
                    vx[r][pc] = R::load(vbase + off + R::offset(c, pc) * sizeof(KV));
                }
            }
        } else {
            const size_t base = A.block(tb);
            const char *kb = kbase + base;
            const char *vb = vbase + base;
#pragma unroll
            for (int r = 0; r < kRows; ++r) {
                const uint32_t off =
                    (uint32_t)(min(t0 + r * kTok, t_end - 1) - tb) * (uint32_t)A.token_bytes + (uint32_t)row_off;
#pragma unroll
                for (int pc = 0; pc < NL; ++pc) {
                    kx[r][pc] = R::load_at(kb, off + R::offset(c, pc) * sizeof(KV));
                    vx[r][pc] = R::load_at(vb, off + R::offset(c, pc) * sizeof(KV));
                }
            }
        }
    };

    auto dot = [&](int gi, const Raw *kr) -> float {
        if constexpr (kPackedDot) {
            return E::dot(qf[gi], qp[gi], reinterpret_cast<const uint4 *>(kr));
        } else {
            float kf[8];
            R::unpack(kr, kf);
            float s = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) s = __builtin_fmaf(qf[gi][e], kf[e], s);
            return s;
        }
    };

    auto compute_tile = [&](int j, const Raw (&kx)[kRows][NL], const Raw (&vx)[kRows][NL]) {
        const int t0 = t_begin + j * kWaveTile + ts;
        float p[GT][kRows];
#pragma unroll
        for (int r = 0; r < kRows; ++r) {
            const bool valid = t0 + r * kTok < t_end;
#pragma unroll
            for (int gi = 0; gi < GT; ++gi) {
                const float d = row16_sum(dot(gi, kx[r]));
                p[gi][r] = valid ? d * a.scale_log2 : -INFINITY;
            }
        }
#pragma unroll
        for (int gi = 0; gi < GT; ++gi) {
            float mt = p[gi][0];
#pragma unroll
            for (int r = 1; r < kRows; ++r) mt = fmaxf(mt, p[gi][r]);
            const float m_new = fmaxf(m[gi], mt);
            const float mu = finite_or_zero(m_new);
            const float alpha = exp2_fast(m[gi] - mu);
            l[gi] *= alpha;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[gi][e] *= alpha;
#pragma unroll
            for (int r = 0; r < kRows; ++r) {
                p[gi][r] = exp2_fast(p[gi][r] - mu);
                l[gi] += p[gi][r];
            }
            m[gi] = m_new;
        }
#pragma unroll
        for (int r = 0; r < kRows; ++r) {
            float vf[8];
            R::unpack(vx[r], vf);
#pragma unroll
            for (int gi = 0; gi < GT; ++gi)
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[gi][e] = __builtin_fmaf(p[gi][r], vf[e], acc[gi][e]);
        }
    };

    // The compute of a tile sits in both arms of the prefetch branch, so the
    // compiler's wait before it counts only the current tile's loads (a single
    // copy after the branch would wait for the prefetched tile as well).
    Raw kA[kRows][NL], vA[kRows][NL], kB[kRows][NL], vB[kRows][NL];
    int j = wave;
    if (j < ntiles) load_tile(j, kA, vA);
    while (j < ntiles) {
        if (j + kWaves < ntiles) {
            load_tile(j + kWaves, kB, vB);
            compute_tile(j, kA, vA);
        } else {
            compute_tile(j, kA, vA);
        }
        j += kWaves;
        if (j >= ntiles) break;
        if (j + kWaves < ntiles) {
            load_tile(j + kWaves, kA, vA);
            compute_tile(j, kB, vB);
        } else {
            compute_tile(j, kB, vB);
        }
        j += kWaves;
    }

    // Merge the 16-lane groups of each wave that hold the same KV head (their
    // lanes c own the same head-dim elements): with one head per workgroup rows
    // pair up first (lane ^ 16), then halves (lane ^ 32); with two, groups g and
    // g ^ 2 (lane ^ 32); with four there is nothing to merge. Both lanes of a
    // pair compute the same merged state.
    auto merge_groups = [&](auto pair) {
#pragma unroll
        for (int gi = 0; gi < GT; ++gi) {
            const LanePair pm = pair(m[gi]);
            const LanePair pl = pair(l[gi]);
            const float M = fmaxf(pm.lo, pm.hi);
            const float mu = finite_or_zero(M);
            const float a_lo = exp2_fast(pm.lo - mu);
            const float a_hi = exp2_fast(pm.hi - mu);
            l[gi] = a_lo * pl.lo + a_hi * pl.hi;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const LanePair px = pair(acc[gi][e]);
                acc[gi][e] = a_lo * px.lo + a_hi * px.hi;
            }
            m[gi] = M;
        }
    };
    if constexpr (HP == 1) merge_groups([](float x) { return lane_pair<16>(x); });
    if constexpr (HP <= 2) merge_groups([](float x) { return lane_pair<32>(x); });
    if (ts == 0) {
#pragma unroll
        for (int gi = 0; gi < GT; ++gi) {
            const int hh = hs * GT + gi;
#pragma unroll
            for (int e = 0; e < 8; ++e) s_acc[wave][hh][R::index(c, e)] = acc[gi][e];
            if (c == 0) {
                s_m[wave][hh] = m[gi];
                s_l[wave][hh] = l[gi];
            }
        }
    }
    __syncthreads();

    // Merge the waves, then store the split (or the merged output).
    finish_split<T, FUSED>(a, slice, b, h0, NH, split, n_b, [&](int gi, int d, float &lse) {
        float M = s_m[0][gi];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) M = fmaxf(M, s_m[w][gi]);
        const float mu = finite_or_zero(M);
        float lsum = 0.f, o = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float wgt = exp2_fast(s_m[w][gi] - mu);
            lsum = __builtin_fmaf(wgt, s_l[w][gi], lsum);
            o = __builtin_fmaf(wgt, s_acc[w][gi][d], o);
        }
        lse = (M + log2_fast(lsum)) * kLn2;
        return a.v_scale * (o / lsum);
    });
}

// Contiguous: one workgroup per (head slice, split). Paged batches take their
// (sequence, split) items largest first, the last split of every sequence
// before the others, one per workgroup or, in a persistent launch, claimed by
// one workgroup per resident slot (paged_items).
template <typename T, typename KV, int GT, int HP, int MODE, bool PERSIST, bool FUSED>
__global__ __launch_bounds__(kThreads) void split_valu_kernel(SplitArgs a) {
    pin_args(a.q, a.k, a.v, a.ws_o, a.ws_lse, a.scale_log2);
    if constexpr (MODE == kContig) {
        split_valu_item<T, KV, GT, HP, MODE, FUSED>(a, blockIdx.x, 0, blockIdx.y);
    } else {
        paged_items<T, PERSIST>(a, [&](const SplitArgs &ai, int x, int b, int split) {
            split_valu_item<T, KV, GT, HP, MODE, false>(ai, x, b, split);
        });
    }
}

template <typename T, typename KV, int GT, int HP, int MODE, bool PERSIST, bool FUSED = false>
hipError_t launch_one(const LaunchShape &s, const SplitArgs &a, hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
    SplitArgs arg = a;
    void *args[] = {&arg};
    return launch_timed(reinterpret_cast<const void *>(&split_valu_kernel<T, KV, GT, HP, MODE, PERSIST, FUSED>), s,
                        args, st, e0, e1);
}

template <typename T, typename KV, int MODE, bool PERSIST, bool FUSED = false>
hipError_t launch_gt(int gt, int hp, const LaunchShape &s, const SplitArgs &a, hipStream_t st, hipEvent_t e0,
                     hipEvent_t e1) {
    if (hp == 2 && gt == 1) return launch_one<T, KV, 1, 2, MODE, PERSIST, FUSED>(s, a, st, e0, e1);
    if (hp == 4 && gt == 1) return launch_one<T, KV, 1, 4, MODE, PERSIST, FUSED>(s, a, st, e0, e1);
    if (hp != 1) return hipErrorInvalidValue;
    switch (gt) {
        case 1: return launch_one<T, KV, 1, 1, MODE, PERSIST, FUSED>(s, a, st, e0, e1);
        case 2: return launch_one<T, KV, 2, 1, MODE, PERSIST, FUSED>(s, a, st, e0, e1);
        case 4: return launch_one<T, KV, 4, 1, MODE, PERSIST, FUSED>(s, a, st, e0, e1);
        case 8:
            // fp32 rows stop at 4 heads per workgroup (the planner never asks for 8)
            if constexpr (std::is_same<T, float>::value) return hipErrorInvalidValue;
            else return launch_one<T, KV, 8, 1, MODE, PERSIST, FUSED>(s, a, st, e0, e1);
        default: return hipErrorInvalidValue;
    }
}

template <typename T, typename KV>
hipError_t launch_mode(int mode, bool persist, bool fused, int gt, int hp, const LaunchShape &s, const SplitArgs &a,
                       hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
    if (fused && mode != kContig) return hipErrorInvalidValue;
    switch (mode) {
        case kContig:
            return fused ? launch_gt<T, KV, kContig, false, true>(gt, hp, s, a, st, e0, e1)
                         : launch_gt<T, KV, kContig, false, false>(gt, hp, s, a, st, e0, e1);
        case kPagedBlock:
            return persist ? launch_gt<T, KV, kPagedBlock, true>(gt, hp, s, a, st, e0, e1)
                           : launch_gt<T, KV, kPagedBlock, false>(gt, hp, s, a, st, e0, e1);
        case kPagedRow:
            return persist ? launch_gt<T, KV, kPagedRow, true>(gt, hp, s, a, st, e0, e1)
                           : launch_gt<T, KV, kPagedRow, false>(gt, hp, s, a, st, e0, e1);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_split_valu(fd_dtype dtype, int gt, int hp, int mode, bool persist, bool fused, const LaunchShape &s,
                             const SplitArgs &a, hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
    switch (dtype) {
        case FD_DTYPE_F32: return launch_mode<float, float>(mode, persist, fused, gt, hp, s, a, st, e0, e1);
        case FD_DTYPE_F16: return launch_mode<_Float16, _Float16>(mode, persist, fused, gt, hp, s, a, st, e0, e1);
        case FD_DTYPE_BF16: return launch_mode<__bf16, __bf16>(mode, persist, fused, gt, hp, s, a, st, e0, e1);
        case FD_DTYPE_F16_KV_E4M3: return launch_mode<_Float16, fp8e4m3>(mode, persist, fused, gt, hp, s, a, st, e0, e1);
        case FD_DTYPE_BF16_KV_E4M3: return launch_mode<__bf16, fp8e4m3>(mode, persist, fused, gt, hp, s, a, st, e0, e1);
    }
    return hipErrorInvalidValue;
}

}  // namespace fd
