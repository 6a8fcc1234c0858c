// fd_merge.hip -- log-sum-exp merge of the split partials (gfx950, wave64).
//
// One workgroup per (sequence b, query head h). Split s holds a normalised output
// O_s and the natural-log log-sum-exp lse_s of its scores. With
// M = max_s lse_s, w_s = exp(lse_s - M):  o = sum_s w_s O_s / sum_s w_s, which
// is the merge of "[CUDA 优化实战] 纯手搓 flash decoding sm120", section "2. kernel
// 实现细节" (weights exp(lse_s - global lse)) and equals the (m, l) form of
// "FlashAttention 与推理算子", section "decode 阶段的并行：Flash-Decoding 与
// split-K", since lse_s = m_s + ln l_s. Only the ceil(L_b / chunk) splits that
// hold tokens are read; a sequence with no token gets o = 0. Each lane owns two
// adjacent output elements, so a split's 512-byte partial row is one coalesced
// 8-byte-per-lane load. Sequences that fit one split were written directly by
// the split kernel and are skipped here.
#include "fd_device.h"
#include "fd_internal.h"

namespace fd {

namespace {

constexpr int kMergeWaves = 4;

// One workgroup of 4 waves per (sequence b, query head h). Up to kMergeBatch
// splits are merged by wave 0 alone (one round trip); beyond that each wave
// takes a contiguous quarter of the splits against the common max, and the
// four partial sums are added through LDS.
template <typename T, bool PAGED>
__global__ __launch_bounds__(64 * kMergeWaves) void merge_kernel(MergeArgs a) {
    const int h = blockIdx.x;
    const int b = blockIdx.y;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    int L = a.max_len;
    if (PAGED) L = max(0, min(a.seq_lens[b], a.max_len));
    const int n = min((L + a.chunk - 1) / a.chunk, a.num_splits);
    if (n == 1) return;  // the split kernel wrote this row directly
    const size_t bh = (size_t)b * a.H + h;
    const float *ws_o_row = a.ws_o + bh * a.num_splits * kHeadDim;
    const float *lse_row = a.ws_lse + bh * a.num_splits;
    if (n <= kMergeBatch) {
        if (wave == 0) store_out_pair<T>(a.out, bh, lane, merge_partials(ws_o_row, lse_row, n, lane));
        return;
    }
    __shared__ float s_red[kMergeWaves];
    __shared__ float2 s_o[kMergeWaves][64];
    __shared__ float s_w[kMergeWaves];
    float mx = -INFINITY;
    for (int s = threadIdx.x; s < n; s += 64 * kMergeWaves) mx = fmaxf(mx, lse_row[s]);
    mx = wave_max(mx);
    if (lane == 0) s_red[wave] = mx;
    __syncthreads();
    float m_all = s_red[0];
#pragma unroll
    for (int w = 1; w < kMergeWaves; ++w) m_all = fmaxf(m_all, s_red[w]);
    const float mu = finite_or_zero(m_all);
    const int per = (n + kMergeWaves - 1) / kMergeWaves;
    const int lo = min(n, wave * per), hi = min(n, lo + per);
    float wpart = 0.f;
    const float2 o = merge_range(ws_o_row, lse_row, lo, hi, mu, lane, &wpart);
    const float wsum = wave_sum(wpart);
    s_o[wave][lane] = o;
    if (lane == 0) s_w[wave] = wsum;
    __syncthreads();
    if (wave == 0) {
        float o0 = 0.f, o1 = 0.f, wt = 0.f;
#pragma unroll
        for (int w = 0; w < kMergeWaves; ++w) {
            o0 += s_o[w][lane].x;
            o1 += s_o[w][lane].y;
            wt += s_w[w];
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
