// fd_merge.hip -- log-sum-exp merge of the split partials (gfx950, wave64).
//
// One workgroup per (sequence b, query head h). Split s holds a normalised output
// O_s and the natural-log log-sum-exp lse_s of its scores. With
// M = max_s lse_s, w_s = exp(lse_s - M):  o = sum_s w_s O_s / sum_s w_s, which
// is the merge of "[CUDA 优化实战] 纯手搓 flash decoding sm120", section "2. kernel
// 实现细节" (weights exp(lse_s - global lse)) and equals the (m, l) form of
// "FlashAttention 与推理算子", section "decode 阶段的并行：Flash-Decoding 与
// split-K", since lse_s = m_s + ln l_s. Only the splits sequence b has are read
// (splits_of: ceil(L_b / chunk) for a paged batch, max(1, floor(S / chunk)) for a
// contiguous cache).
// Each lane owns two adjacent output elements, so a split's 512-byte partial
// row is one coalesced 8-byte-per-lane load. Sequences with one split (or no
// token) were written directly by the split kernel and are skipped here.
#include "fd_device.h"
#include "fd_internal.h"

namespace fd {

namespace {

constexpr int kMergeWaves = 4;
constexpr int kMergeBatch = 32;  // splits whose rows one wave loads before using any

// Running merge state of one wave, relative to the largest lse seen so far (m,
// natural log): the lane's share of sum_s e^(lse_s - m) and the lane's two
// output sums sum_s e^(lse_s - m) O_s[2 lane], O_s[2 lane + 1]. Raising m
// rescales the sums by e^(m_old - m_new), the same step as the online softmax
// ("FlashAttention 与推理算子", section "FlashAttention：分块 + online softmax").
// Empty: m = -inf, sums 0.
struct MergeAcc {
    float m = -INFINITY;
    float w = 0.f;
    float o0 = 0.f, o1 = 0.f;
};

// Adds splits [s_lo, s_hi) to st, kMergeBatch at a time. A batch's lse values
// and partial rows are all loaded before any is used, so it costs one round
// trip to memory (no separate pass for the max). Rows past the batch re-read
// its last row (a valid address) and get weight 0; lane i holds split s0 + i's
// lse and weight, and readlane broadcasts the weights.
__device__ __forceinline__ void merge_span(const float *ws_o_row, const float *lse_row, int s_lo, int s_hi, int lane,
                                           MergeAcc &st) {
    // Uniform base plus 32-bit lane offsets (a row has at most 4096 splits of 512 bytes).
    const char *src = reinterpret_cast<const char *>(ws_o_row);
    for (int s0 = s_lo; s0 < s_hi; s0 += kMergeBatch) {
        const int cnt = min(kMergeBatch, s_hi - s0);
        const float lse = lane < cnt ? lse_row[s0 + lane] : -INFINITY;
        float2 x[kMergeBatch];
#pragma unroll
        for (int u = 0; u < kMergeBatch; ++u)
            x[u] = *reinterpret_cast<const float2 *>(
                src + ((uint32_t)(s0 + min(u, cnt - 1)) * (uint32_t)(kHeadDim * sizeof(float)) + (uint32_t)lane * 8u));
        const float m_new = fmaxf(st.m, wave_max(lse));
        const float mu = finite_or_zero(m_new);
        const float alpha = exp2_fast((st.m - mu) * kLog2e);
        const float w = exp2_fast((lse - mu) * kLog2e);
        st.w = __builtin_fmaf(st.w, alpha, w);
        float o0 = st.o0 * alpha, o1 = st.o1 * alpha;
#pragma unroll
        for (int u = 0; u < kMergeBatch; ++u) {
            const float wu = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), u));
            o0 = __builtin_fmaf(wu, x[u].x, o0);
            o1 = __builtin_fmaf(wu, x[u].y, o1);
        }
        st.o0 = o0;
        st.o1 = o1;
        st.m = m_new;
    }
}

// One workgroup of 4 waves per (sequence b, query head h). Up to kMergeBatch
// splits are merged by wave 0 alone; beyond that each wave takes a contiguous
// quarter of the splits and the four states are combined through LDS, each
// rescaled to the common max.
template <typename T, bool PAGED>
__global__ __launch_bounds__(64 * kMergeWaves) void merge_kernel(MergeArgs a) {
    int h = blockIdx.x;
    if (a.xcd_group > 0) {  // a bijection of [0, H): workgroup i on XCD i mod 8 takes a head split there
        const int c = h & 7, k = h >> 3;
        h = (c + 8 * (k / a.xcd_group)) * a.xcd_group + k % a.xcd_group;
    }
    const int b = blockIdx.y;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    pin_args(a.ws_o, a.ws_lse, a.out, a.H);
    int L = a.max_len;
    if (PAGED) L = max(0, min(a.seq_lens[b], a.max_len));
    const int n = min(splits_of<PAGED>(L, a.chunk), a.num_splits);
    if (n <= 1) return;  // the split kernel wrote this row directly (zeros when L = 0)
    const size_t bh = (size_t)b * a.H + h;
    const float *ws_o_row = a.ws_o + bh * a.num_splits * kHeadDim;
    const float *lse_row = a.ws_lse + bh * a.num_splits;
    MergeAcc st;
    if (n <= kMergeBatch) {
        if (wave != 0) return;
        merge_span(ws_o_row, lse_row, 0, n, lane, st);
        const float wsum = wave_sum(st.w);
        const float inv = wsum > 0.f ? 1.f / wsum : 0.f;  // n == 0: o = 0
        store_out_pair<T>(a.out, bh, lane, make_float2(st.o0 * inv, st.o1 * inv));
        return;
    }
    __shared__ float s_m[kMergeWaves];
    __shared__ float s_w[kMergeWaves];
    __shared__ float2 s_o[kMergeWaves][64];
    const int per = (n + kMergeWaves - 1) / kMergeWaves;
    const int lo = min(n, wave * per), hi = min(n, lo + per);
    merge_span(ws_o_row, lse_row, lo, hi, lane, st);
    const float wsum = wave_sum(st.w);
    s_o[wave][lane] = make_float2(st.o0, st.o1);
    if (lane == 0) {
        s_m[wave] = st.m;
        s_w[wave] = wsum;
    }
    __syncthreads();
    if (wave == 0) {
        float M = s_m[0];
#pragma unroll
        for (int w = 1; w < kMergeWaves; ++w) M = fmaxf(M, s_m[w]);
        const float mu = finite_or_zero(M);
        float o0 = 0.f, o1 = 0.f, wt = 0.f;
#pragma unroll
        for (int w = 0; w < kMergeWaves; ++w) {
            const float f = exp2_fast((s_m[w] - mu) * kLog2e);
            o0 = __builtin_fmaf(f, s_o[w][lane].x, o0);
            o1 = __builtin_fmaf(f, s_o[w][lane].y, o1);
            wt = __builtin_fmaf(f, s_w[w], wt);
        }
        const float inv = wt > 0.f ? 1.f / wt : 0.f;
        store_out_pair<T>(a.out, bh, lane, make_float2(o0 * inv, o1 * inv));
    }
}

template <typename T, bool PAGED>
hipError_t launch_one(int B, const MergeArgs &a, hipStream_t st) {
    MergeArgs arg = a;
    void *args[] = {&arg};
    return hipLaunchKernel(reinterpret_cast<const void *>(&merge_kernel<T, PAGED>), dim3(a.H, B), dim3(64 * kMergeWaves), args, 0,
                           st);
}

}  // namespace

hipError_t launch_merge(fd_dtype dtype, bool paged, int B, const MergeArgs &a, hipStream_t st) {
    switch (dtype) {
        case FD_DTYPE_F32: return paged ? launch_one<float, true>(B, a, st) : launch_one<float, false>(B, a, st);
        case FD_DTYPE_F16: return paged ? launch_one<_Float16, true>(B, a, st) : launch_one<_Float16, false>(B, a, st);
        case FD_DTYPE_BF16: return paged ? launch_one<__bf16, true>(B, a, st) : launch_one<__bf16, false>(B, a, st);
        default: break;  // callers pass the query dtype
    }
    return hipErrorInvalidValue;
}

}  // namespace fd
